// Wide-tile kernel variants: (row blocks per wave, token blocks, weight
// prefetch depth D in k-steps, FP32 weights[, waves]). A workgroup tile is
// (16*W*RBW) x (16*BNB) with W = 4 waves (8 for GDP_WIDE_W(..., 8)); activations
// move in super-steps of 2 k-steps, or of 4 with the depth-16 prefetch (the
// pipeline keeps at most 4 super-steps of weights ahead).
#include "variants.h"
#include "wide.h"

namespace gdp {

#define GDP_WIDE_W(RBW, BNB, D, F, W)                                                                  \
    {RBW * W, BNB, D, F, W,                                                                            \
     reinterpret_cast<const void *>(&wide_kernel<RBW, BNB, D, wide_superstep(D), (F != 0), false, W>), \
     reinterpret_cast<const void *>(&wide_kernel<RBW, BNB, D, wide_superstep(D), (F != 0), true, W>)},
#define GDP_WIDE(RBW, BNB, D, F) GDP_WIDE_W(RBW, BNB, D, F, 4)

const WideVariant kWideVariants[] = {
    GDP_WIDE(1, 2, 8, 0)
    GDP_WIDE(1, 1, 16, 0)
    GDP_WIDE(1, 2, 16, 0)
    GDP_WIDE(1, 4, 8, 0)
    GDP_WIDE(1, 8, 8, 0)
    GDP_WIDE(2, 2, 8, 0)
    GDP_WIDE(2, 4, 4, 0)
    GDP_WIDE(2, 4, 8, 0)
    GDP_WIDE(2, 4, 16, 0)
    GDP_WIDE(1, 4, 16, 0)
    GDP_WIDE(2, 8, 4, 0)
    GDP_WIDE(2, 8, 8, 0)
    GDP_WIDE(4, 4, 4, 0)
    GDP_WIDE(1, 2, 4, 1)
    GDP_WIDE(1, 2, 8, 1)
    GDP_WIDE(1, 4, 4, 1)
    GDP_WIDE(1, 8, 4, 1)
    GDP_WIDE_W(1, 4, 8, 0, 8)
    GDP_WIDE_W(1, 4, 16, 0, 8)
    GDP_WIDE_W(1, 4, 4, 0, 8)
    GDP_WIDE_W(1, 8, 8, 0, 8)
    GDP_WIDE_W(2, 4, 8, 0, 8)
    GDP_WIDE_W(2, 4, 16, 0, 8)
    GDP_WIDE_W(2, 8, 8, 0, 8)
};
const int kWideVariantCount = sizeof(kWideVariants) / sizeof(kWideVariants[0]);

}  // namespace gdp
