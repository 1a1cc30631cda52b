// Wide-tile kernel variants with activations moved by LDS DMA (XDMA): the
// BF16 variants of wide_variants.hip, same parameters.
#include "variants.h"
#include "wide.h"

namespace gdp {

#define GDP_WIDE_DMA(RBW, BNB, D, W)                                                                         \
    {RBW * W, BNB, D, 0, W,                                                                                  \
     reinterpret_cast<const void *>(&wide_kernel<RBW, BNB, D, wide_superstep(D), false, false, W, true>),    \
     reinterpret_cast<const void *>(&wide_kernel<RBW, BNB, D, wide_superstep(D), false, true, W, true>), 1},

const WideVariant kWideDmaVariants[] = {
    GDP_WIDE_DMA(1, 2, 8, 4)
    GDP_WIDE_DMA(1, 1, 16, 4)
    GDP_WIDE_DMA(1, 2, 16, 4)
    GDP_WIDE_DMA(1, 4, 8, 4)
    GDP_WIDE_DMA(1, 8, 8, 4)
    GDP_WIDE_DMA(2, 2, 8, 4)
    GDP_WIDE_DMA(2, 4, 4, 4)
    GDP_WIDE_DMA(2, 4, 8, 4)
    GDP_WIDE_DMA(2, 4, 16, 4)
    GDP_WIDE_DMA(1, 4, 16, 4)
    GDP_WIDE_DMA(2, 8, 4, 4)
    GDP_WIDE_DMA(2, 8, 8, 4)
    GDP_WIDE_DMA(4, 4, 4, 4)
    GDP_WIDE_DMA(1, 4, 8, 8)
    GDP_WIDE_DMA(1, 4, 16, 8)
    GDP_WIDE_DMA(1, 4, 4, 8)
    GDP_WIDE_DMA(1, 8, 8, 8)
    GDP_WIDE_DMA(2, 4, 8, 8)
    GDP_WIDE_DMA(2, 8, 8, 8)
    GDP_WIDE_DMA(2, 4, 16, 8)
};
const int kWideDmaVariantCount = sizeof(kWideDmaVariants) / sizeof(kWideDmaVariants[0]);

}  // namespace gdp
