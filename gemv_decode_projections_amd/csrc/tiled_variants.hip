// Tiled (large-m) kernel variants: (rows per wave in 16-row blocks, token
// blocks, waves, prefetch depth D in k-steps, FP32 weights). A workgroup tile
// is (WAVES*RBW*16) x (BNB*16); activations move in super-steps of
// S = min(4, D/2) k-steps.
#include "tiled.h"
#include "variants.h"

namespace gdp {

#define GDP_TILED(RBW, BNB, W, D, F) \
    {RBW * W, BNB, W, 1, D, F,       \
     reinterpret_cast<const void *>(&tiled_kernel<RBW, BNB, W, ((D) / 2 < 4 ? (D) / 2 : 4), D, (F != 0)>)},

const TiledVariant kTiledVariants[] = {
    GDP_TILED(1, 4, 4, 4, 0)
    GDP_TILED(1, 4, 4, 8, 0)
    GDP_TILED(2, 4, 4, 4, 0)
    GDP_TILED(2, 4, 4, 8, 0)
    GDP_TILED(2, 4, 4, 16, 0)
    GDP_TILED(1, 2, 4, 8, 0)
    GDP_TILED(2, 2, 4, 8, 0)
    GDP_TILED(1, 2, 4, 16, 0)
    GDP_TILED(1, 4, 4, 4, 1)
    GDP_TILED(1, 2, 4, 4, 1)
    GDP_TILED(1, 2, 4, 8, 1)
};
const int kTiledVariantCount = sizeof(kTiledVariants) / sizeof(kTiledVariants[0]);

}  // namespace gdp
