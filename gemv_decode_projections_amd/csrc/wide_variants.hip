// Wide-tile kernel variants: (row blocks per wave, token blocks, weight
// prefetch depth D in k-steps, FP32 weights). A workgroup tile is
// (64*RBW) x (16*BNB); activations move in super-steps of 2 k-steps.
#include "variants.h"
#include "wide.h"

namespace gdp {

#define GDP_WIDE(RBW, BNB, D, F) \
    {RBW * 4, BNB, D, F, reinterpret_cast<const void *>(&wide_kernel<RBW, BNB, D, 2, (F != 0)>)},

const WideVariant kWideVariants[] = {
    GDP_WIDE(1, 2, 8, 0)
    GDP_WIDE(1, 4, 8, 0)
    GDP_WIDE(1, 8, 8, 0)
    GDP_WIDE(2, 2, 8, 0)
    GDP_WIDE(2, 4, 4, 0)
    GDP_WIDE(2, 4, 8, 0)
    GDP_WIDE(2, 8, 4, 0)
    GDP_WIDE(2, 8, 8, 0)
    GDP_WIDE(4, 4, 4, 0)
    GDP_WIDE(1, 2, 4, 1)
    GDP_WIDE(1, 2, 8, 1)
    GDP_WIDE(1, 4, 4, 1)
    GDP_WIDE(1, 8, 4, 1)
};
const int kWideVariantCount = sizeof(kWideVariants) / sizeof(kWideVariants[0]);

}  // namespace gdp
