"""Host check of the skinny kernel's split-K reducer choice (csrc/common.h,
reducing_split): the reducer must be the tile's split with the highest
hardware workgroup id, so that every split it waits for is dispatched before
it. The walk is compiled for the host and compared with a brute-force
inverse of the XCD remap (logical id = (hw % 8) * (G / 8) + hw / 8)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SRC = r'''
#include "%s/gemv_decode_projections_amd/csrc/common.h"
#include <cstdio>
#include <vector>

int main()
{
    long cases = 0, bad = 0;
    for (int n_rt = 1; n_rt <= 40; ++n_rt)
        for (int n_tt = 1; n_tt <= 9; ++n_tt)
            for (int ks = 2; ks <= 16; ++ks) {
                const int G = n_rt * n_tt * ks;
                for (int remap = 0; remap < 2; ++remap) {
                    if (remap && G %% 8 != 0)
                        continue;
                    std::vector<int> hw_of(G);
                    for (int h = 0; h < G; ++h) {
                        const int l = remap ? (h %% 8) * (G / 8) + h / 8 : h;
                        hw_of[l] = h;
                    }
                    for (int rt = 0; rt < n_rt; ++rt)
                        for (int tt = 0; tt < n_tt; ++tt) {
                            // the skinny kernel's logical ids of one tile's splits
                            int want = 0;
                            for (int s = 1; s < ks; ++s)
                                if (hw_of[(rt * ks + s) * n_tt + tt] > hw_of[(rt * ks + want) * n_tt + tt])
                                    want = s;
                            const int got = gdp::reducing_split(rt * ks * n_tt + tt, n_tt, ks, G, remap != 0);
                            ++cases;
                            if (got != want && bad++ < 5)
                                std::printf("mismatch n_rt %%d n_tt %%d ks %%d remap %%d rt %%d tt %%d: %%d vs %%d\n",
                                            n_rt, n_tt, ks, remap, rt, tt, got, want);
                        }
                }
            }
    std::printf("cases %%ld bad %%ld\n", cases, bad);
    return bad != 0;
}
'''


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("g++") is None, reason="needs hipcc")
def test_reducer_is_the_last_dispatched_split(tmp_path):
    src = tmp_path / "split_order.hip"
    src.write_text(SRC % ROOT)
    exe = tmp_path / "split_order"
    subprocess.run([HIPCC, "-O1", "-std=c++17", "--offload-arch=gfx950", "-o", str(exe), str(src)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bad 0" in r.stdout and int(r.stdout.split("cases ")[1].split()[0]) > 100000
