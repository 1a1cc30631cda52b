// Skinny variants reading the 12-bit weights (one or two 16-token sub-tiles).
#include "skinny.h"
#include "variants.h"

namespace gdp {

#define GDP_ENTRY(NT, RB, W, S, F) \
    {NT, RB, W, S, F, reinterpret_cast<const void *>(&skinny_kernel<NT, RB, W, S, false, true>), 1},

// (waves, k-steps per wave) for one and two row blocks; at most 8 streaming
// waves, since the correction wave makes the workgroup one wave larger.
#define GDP_Z_SET(RB)                                                                                        \
    GDP_ENTRY(1, RB, 4, 2, 0) GDP_ENTRY(1, RB, 4, 4, 0) GDP_ENTRY(1, RB, 4, 8, 0) GDP_ENTRY(1, RB, 4, 16, 0) \
    GDP_ENTRY(1, RB, 4, 32, 0) GDP_ENTRY(1, RB, 8, 2, 0) GDP_ENTRY(1, RB, 8, 4, 0) GDP_ENTRY(1, RB, 8, 8, 0)  \
    GDP_ENTRY(1, RB, 8, 16, 0) GDP_ENTRY(1, RB, 8, 32, 0)

// Two 16-token sub-tiles (17-32 tokens in one pass over the weights).
#define GDP_Z_SET2(RB)                                                                                       \
    GDP_ENTRY(2, RB, 4, 8, 0) GDP_ENTRY(2, RB, 4, 16, 0) GDP_ENTRY(2, RB, 4, 32, 0) GDP_ENTRY(2, RB, 8, 8, 0) \
    GDP_ENTRY(2, RB, 8, 16, 0) GDP_ENTRY(2, RB, 8, 32, 0)

const SkinnyVariant kSkinnyPartZ[] = {
    GDP_Z_SET(1)
    GDP_Z_SET(2)
    GDP_Z_SET2(1)
    GDP_Z_SET2(2)
    GDP_ENTRY(1, 4, 4, 8, 0) GDP_ENTRY(1, 4, 4, 16, 0) GDP_ENTRY(1, 4, 8, 8, 0) GDP_ENTRY(2, 4, 4, 8, 0)
    // activations preloaded per wave (at most 4 / 8 tokens)
    {1, 1, 8, 32, 0, reinterpret_cast<const void *>(&skinny_kernel<1, 1, 8, 32, false, true, 4>), 1, 4},
    {1, 1, 8, 32, 0, reinterpret_cast<const void *>(&skinny_kernel<1, 1, 8, 32, false, true, 8>), 1, 8},
};
const int kSkinnyPartZCount = sizeof(kSkinnyPartZ) / sizeof(kSkinnyPartZ[0]);

}  // namespace gdp
