// Registry of compiled kernel variants (host side).
#pragma once

#include <hip/hip_runtime.h>

namespace gdp {

struct SkinnyVariant {
    int nt;
    int rb;
    int waves;
    int spw;
    int f32w;
    const void *fn;   // __global__ void (SkinnyArgs)
    int z;            // 1: reads the 12-bit weights (one extra wave per workgroup)
    int xp;           // 4 or 8: activations preloaded per wave (at most that many tokens); 0: loaded per k-step
    int skm;          // 1: stream partition (skinny_kernel's SKM; rb is 1 in the configuration)
};

// Tiled (large-m) kernel variants: BMB x BNB blocks of 16 per workgroup, WR waves
// splitting the rows (KG = 1: every wave takes every k-step).
struct TiledVariant {
    int bmb;
    int bnb;
    int wr;
    int kg;
    int depth;        // prefetch distance in k-steps
    int f32w;
    const void *fn;   // __global__ void (TiledArgs)
};

// Row-dot (few tokens, few rows) kernel variants.
struct RowVariant {
    int mcap;         // largest token count
    int r;            // rows per workgroup
    int kit;          // 2048-wide k chunks per row
    int f32w;
    const void *fn;   // __global__ void (RowArgs)
};

// Wide-tile (large-m, split-K) kernel variants: BMB = 4*RBW row blocks x BNB
// token blocks per workgroup of 4 waves.
struct WideVariant {
    int bmb;
    int bnb;
    int depth;        // weight prefetch distance in k-steps
    int f32w;
    int waves;        // 4 or 8
    const void *fn;          // __global__ void (WideArgs): one tile per workgroup
    const void *fn_stream;   // the same kernel in stream mode
    int xdma;                // 1: activations by LDS DMA (wide_kernel's XDMA)
};

// Each part is defined in its own translation unit so the variants compile in parallel.
extern const SkinnyVariant kSkinnyPartBf16Nt1[];
extern const int kSkinnyPartBf16Nt1Count;
extern const SkinnyVariant kSkinnyPartBf16Nt2[];
extern const int kSkinnyPartBf16Nt2Count;
extern const SkinnyVariant kSkinnyPartF32[];
extern const int kSkinnyPartF32Count;
extern const SkinnyVariant kSkinnyPartZ[];
extern const int kSkinnyPartZCount;
extern const SkinnyVariant kSkinnyPartStream[];
extern const int kSkinnyPartStreamCount;
extern const TiledVariant kTiledVariants[];
extern const int kTiledVariantCount;
extern const WideVariant kWideVariants[];
extern const int kWideVariantCount;
extern const WideVariant kWideDmaVariants[];
extern const int kWideDmaVariantCount;
extern const RowVariant kRowVariants[];
extern const int kRowVariantCount;

// (waves, spw) pairs compiled for every (nt, rb, f32w) combination.
#define GDP_WAVES_SPW(X, NT, RB, F32W)                                                   \
    X(NT, RB, 4, 2, F32W) X(NT, RB, 4, 4, F32W) X(NT, RB, 4, 8, F32W)                       \
    X(NT, RB, 4, 16, F32W) X(NT, RB, 4, 32, F32W) X(NT, RB, 8, 2, F32W)                     \
    X(NT, RB, 8, 4, F32W) X(NT, RB, 8, 8, F32W) X(NT, RB, 8, 16, F32W)                      \
    X(NT, RB, 8, 32, F32W) X(NT, RB, 16, 2, F32W) X(NT, RB, 16, 4, F32W)                    \
    X(NT, RB, 16, 8, F32W) X(NT, RB, 16, 16, F32W)

}  // namespace gdp
