"""Python binding of the C ABI in include/proj.h and include/proj_bench.h.

Argument marshalling only: every step of a projection runs in the HIP
library. Torch tensors supply device pointers and streams. If the library is
not built, loading fails with an error; there is no fallback path.
"""

import ctypes
import os

from . import layers as _layers

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libgdproj.so")

PROJ_OK = 0
STATUS = {
    0: "PROJ_OK",
    -1: "PROJ_ERR_LAYER",
    -2: "PROJ_ERR_M",
    -3: "PROJ_ERR_NULL",
    -4: "PROJ_ERR_ALIGN",
    -5: "PROJ_ERR_NOT_PREPARED",
    -6: "PROJ_ERR_UNSUPPORTED",
    -7: "PROJ_ERR_HIP",
    -8: "PROJ_ERR_DEVICE",
    -9: "PROJ_ERR_SCRATCH",
}


class ProjError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        name = STATUS.get(status, str(status))
        msg = "%s: %s (%s)" % (what, name, proj_strerror(status))
        if status == -7:
            msg += " hipError=%d" % _lib().proj_last_hip_error()
        super().__init__(msg)


class ProjConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("kind", "nt", "rb", "waves", "spw", "ksplit", "flags", "grid",
                                            "block")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}

    @classmethod
    def make(cls, kind=0, nt=1, rb=1, waves=8, spw=4, ksplit=1, flags=0):
        return cls(kind, nt, rb, waves, spw, ksplit, flags, 0, 0)


_LIB = None


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "HIP library %s is not built; run `python -m gemv_decode_projections_amd.build` "
            "(or __graft_entry__.build()) first" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    i, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    ip = ctypes.POINTER(ctypes.c_int)
    cp = ctypes.POINTER(ProjConfig)
    sig = {
        "proj_prepare": ([i, vp], i),
        "proj_run": ([i, vp, i, vp, vp], i),
        "proj_run_noalloc": ([i, vp, i, vp, vp], i),
        "proj_out_cols": ([i, i], i),
        "proj_layer_dims": ([i, ip, ip, ip, ip], i),
        "proj_release": ([i], i),
        "proj_compressed": ([i], i),
        "proj_split_giveups": ([i, i], i),
        "proj_strerror": ([i], ctypes.c_char_p),
        "proj_last_hip_error": ([], i),
        "proj_plan": ([i, i, cp], i),
        "proj_run_config": ([i, vp, i, vp, vp, cp], i),
        "proj_num_variants": ([], i),
        "proj_variant": ([i, ip, cp], i),
        "proj_bench_flush": ([vp, sz, vp, i, vp], i),
        "proj_bench_read_floor": ([vp, sz, vp, vp, i, i, i, i, vp, vp], i),
        "proj_bench_stamp": ([vp, i, vp], i),
        "proj_bench_wallclock_khz": ([ip], i),
        "proj_run_timed": ([i, vp, i, vp, vp, cp, vp, vp], i),
        "proj_bench_event_create": ([ctypes.POINTER(vp)], i),
        "proj_bench_event_destroy": ([vp], i),
        "proj_bench_event_elapsed": ([vp, vp, ctypes.POINTER(ctypes.c_float)], i),
        "proj_bench_empty": ([vp], i),
        "proj_bench_copy": ([vp, vp, sz, vp], i),
        "proj_bench_mfma_layout": ([vp, vp, vp, vp], i),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _LIB = lib
    return lib


def library_path():
    return LIB_PATH


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    if stream is None:
        import torch

        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc, what):
    if rc != PROJ_OK:
        raise ProjError(rc, what)
    return rc


# ---------------------------------------------------------------- C ABI mirror

def proj_strerror(status):
    return _lib().proj_strerror(int(status)).decode()


def proj_out_cols(layer, m):
    rc = _lib().proj_out_cols(_layers.layer_id(layer), int(m))
    return _check(rc, "proj_out_cols") if rc < 0 else rc


def proj_layer_dims(layer):
    n, k, wb, ob = (ctypes.c_int() for _ in range(4))
    _check(_lib().proj_layer_dims(_layers.layer_id(layer), ctypes.byref(n), ctypes.byref(k),
                                  ctypes.byref(wb), ctypes.byref(ob)), "proj_layer_dims")
    return n.value, k.value, wb.value, ob.value


def proj_prepare(layer, W):
    """Repack weights `W` (device tensor, N x K, bfloat16 / uint16 bits, float32 for the router)."""
    lid = _layers.layer_id(layer)
    n, k, wb, _ = proj_layer_dims(lid)
    if tuple(W.shape) != (n, k) or W.element_size() != wb or not W.is_contiguous() or not W.is_cuda:
        raise ValueError("%s: W must be a contiguous device tensor %dx%d of %d-byte elements"
                         % (_layers.layer_name(lid), n, k, wb))
    _check(_lib().proj_prepare(lid, _ptr(W)), "proj_prepare(%s)" % _layers.layer_name(lid))


_BF16_LIKE = ("torch.bfloat16", "torch.int16", "torch.uint16")


def _check_io(layer, x, m, out):
    """Host-side check of the tensors a launch will read and write: the C ABI
    takes raw pointers, so a tensor of the wrong shape would become an
    out-of-bounds GPU access. Raises ValueError before anything is launched."""
    m = int(m)
    if m < 1:
        return    # the library reports PROJ_ERR_M
    name = _layers.layer_name(layer)
    _, k, _, ob = _layers.DIMS[name]
    cols = _layers.n_eff(name, m)
    for what, t, width, dtypes in (("x", x, k, _BF16_LIKE),
                                   ("out", out, cols, ("torch.float32",) if ob == 4 else _BF16_LIKE)):
        if t is None or not hasattr(t, "data_ptr"):
            raise ValueError("%s(m=%d): %s must be a device tensor" % (name, m, what))
        if str(t.dtype) not in dtypes:
            raise ValueError("%s(m=%d): %s has dtype %s, expected one of %s" % (name, m, what, t.dtype, dtypes))
        if t.dim() != 2 or t.shape[1] != width or t.shape[0] < m:
            raise ValueError("%s(m=%d): %s has shape %s, expected (>= %d, %d)"
                             % (name, m, what, tuple(t.shape), m, width))
        if not t.is_contiguous():
            raise ValueError("%s(m=%d): %s must be contiguous (row-major)" % (name, m, what))
    for what, t in (("x", x), ("out", out)):
        if not t.is_cuda:
            raise ValueError("%s(m=%d): %s is on %s, not a GPU" % (name, m, what, t.device))
    if x.device != out.device:
        raise ValueError("%s(m=%d): x on %s, out on %s" % (name, m, x.device, out.device))


def proj_run(layer, x, m, out, stream=None):
    """out[:m] = x[:m] @ W^T, launched on `stream` (default: torch's current stream)."""
    _check_io(layer, x, m, out)
    _check(_lib().proj_run(_layers.layer_id(layer), _ptr(x), int(m), _ptr(out), _stream(stream)),
           "proj_run(%s, m=%d)" % (_layers.layer_name(layer), m))


def proj_run_noalloc(layer, x, m, out, stream=None):
    """proj_run with the split-K scratch in the library's fixed device array (allocates nothing)."""
    _check_io(layer, x, m, out)
    _check(_lib().proj_run_noalloc(_layers.layer_id(layer), _ptr(x), int(m), _ptr(out), _stream(stream)),
           "proj_run_noalloc(%s, m=%d)" % (_layers.layer_name(layer), m))


def proj_run_config(layer, x, m, out, cfg, stream=None):
    _check_io(layer, x, m, out)
    _check(_lib().proj_run_config(_layers.layer_id(layer), _ptr(x), int(m), _ptr(out), _stream(stream),
                                  ctypes.byref(cfg)),
           "proj_run_config(%s, m=%d, %s)" % (_layers.layer_name(layer), m, cfg.as_dict()))


def proj_split_giveups(layer, reset=False):
    """Give-ups of the layer's polled split-K reducers since prepare or the last
    reset; reset=True also restores the workspace's empty marks (synchronizes)."""
    rc = _lib().proj_split_giveups(_layers.layer_id(layer), 1 if reset else 0)
    return _check(rc, "proj_split_giveups") if rc < 0 else rc


def proj_compressed(layer):
    """Correction slots per row of the layer's 12-bit form, or -1 if it has none."""
    rc = _lib().proj_compressed(_layers.layer_id(layer))
    if rc < -1:
        _check(rc, "proj_compressed")
    return rc


def proj_release(layer):
    _check(_lib().proj_release(_layers.layer_id(layer)), "proj_release")


def proj_plan(layer, m):
    cfg = ProjConfig()
    _check(_lib().proj_plan(_layers.layer_id(layer), int(m), ctypes.byref(cfg)), "proj_plan")
    return cfg


def proj_num_variants():
    return _lib().proj_num_variants()


def proj_variant(i):
    f32 = ctypes.c_int()
    cfg = ProjConfig()
    _check(_lib().proj_variant(int(i), ctypes.byref(f32), ctypes.byref(cfg)), "proj_variant")
    return bool(f32.value), cfg


FLUSH_NT, FLUSH_PLAIN = 0, 1


def proj_bench_flush(buf, sink, stream=None, mode=FLUSH_NT, nbytes=None):
    """Read `nbytes` (default: all) of `buf`; mode FLUSH_NT (non-temporal) or FLUSH_PLAIN."""
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    if n > buf.numel() * buf.element_size():
        raise ValueError("flush of %d bytes from a %d-byte buffer" % (n, buf.numel() * buf.element_size()))
    _check(_lib().proj_bench_flush(_ptr(buf), n, _ptr(sink), int(mode), _stream(stream)), "proj_bench_flush")


def proj_bench_read_floor(buf, nbytes, sink, grid=0, waves=0, unroll=4, stream=None, events=None, mode=FLUSH_NT):
    if int(nbytes) > buf.numel() * buf.element_size():
        raise ValueError("read floor of %d bytes from a %d-byte buffer" % (nbytes, buf.numel() * buf.element_size()))
    if sink.numel() * sink.element_size() < 4 * max(int(grid) or 1024, 4096):
        raise ValueError("sink too small for grid %d" % grid)
    ev0, ev1 = (events.start, events.stop) if events is not None else (None, None)
    _check(_lib().proj_bench_read_floor(_ptr(buf), int(nbytes), _ptr(sink), _stream(stream),
                                        int(grid), int(waves), int(unroll), int(mode), ev0, ev1),
           "proj_bench_read_floor")


def proj_bench_stamp(buf, idx, stream=None):
    """Write the GPU wall clock to buf[idx] (buf: int64 device tensor)."""
    if not 0 <= int(idx) < buf.numel() or buf.element_size() != 8:
        raise ValueError("stamp index %d outside a %d-word buffer" % (idx, buf.numel()))
    _check(_lib().proj_bench_stamp(_ptr(buf), int(idx), _stream(stream)), "proj_bench_stamp")


def proj_bench_wallclock_khz():
    khz = ctypes.c_int()
    _check(_lib().proj_bench_wallclock_khz(ctypes.byref(khz)), "proj_bench_wallclock_khz")
    return khz.value


class KernelTimer:
    """A pair of HIP events stamped at the start and end of one kernel's execution."""

    def __init__(self):
        a, b = ctypes.c_void_p(), ctypes.c_void_p()
        _check(_lib().proj_bench_event_create(ctypes.byref(a)), "event_create")
        _check(_lib().proj_bench_event_create(ctypes.byref(b)), "event_create")
        self.start, self.stop = a, b

    def elapsed_us(self):
        ms = ctypes.c_float()
        _check(_lib().proj_bench_event_elapsed(self.start, self.stop, ctypes.byref(ms)), "event_elapsed")
        return ms.value * 1000.0

    def close(self):
        if self.start is not None:
            _lib().proj_bench_event_destroy(self.start)
            _lib().proj_bench_event_destroy(self.stop)
            self.start = self.stop = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def proj_run_timed(layer, x, m, out, timer, cfg=None, stream=None):
    """proj_run / proj_run_config launched with `timer` bracketing the kernel itself."""
    _check_io(layer, x, m, out)
    _check(_lib().proj_run_timed(_layers.layer_id(layer), _ptr(x), int(m), _ptr(out), _stream(stream),
                                 ctypes.byref(cfg) if cfg is not None else None, timer.start, timer.stop),
           "proj_run_timed(%s, m=%d)" % (_layers.layer_name(layer), m))


def proj_bench_copy(src, dst, nbytes, stream=None):
    _check(_lib().proj_bench_copy(_ptr(src), _ptr(dst), int(nbytes), _stream(stream)), "proj_bench_copy")


def proj_bench_empty(stream=None):
    _check(_lib().proj_bench_empty(_stream(stream)), "proj_bench_empty")


def proj_bench_mfma_layout(A, B, C, stream=None):
    _check(_lib().proj_bench_mfma_layout(_ptr(A), _ptr(B), _ptr(C), _stream(stream)),
           "proj_bench_mfma_layout")


# ------------------------------------------------------------- conveniences

def out_dtype(layer):
    import torch

    return torch.float32 if _layers.DIMS[_layers.layer_name(layer)][3] == 4 else torch.bfloat16


def new_out(layer, m, device="cuda"):
    """Output tensor for (layer, m): m x proj_out_cols rows, BF16 (router FP32)."""
    import torch

    return torch.empty((m, proj_out_cols(layer, m)), dtype=out_dtype(layer), device=device)


def linear(layer, x, stream=None):
    """Allocate out and run one projection of the BF16 activations `x` (m x K)."""
    m = x.shape[0]
    out = new_out(layer, m, device=x.device)
    proj_run(layer, x, m, out, stream)
    return out
