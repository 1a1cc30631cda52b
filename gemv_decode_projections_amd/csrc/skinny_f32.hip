// FP32-weight (router) skinny variants: one or two 16-token sub-tiles, one or
// two 16-row blocks per workgroup.
#include "skinny.h"
#include "variants.h"

namespace gdp {

#define GDP_ENTRY(NT, RB, W, S, F) {NT, RB, W, S, F, reinterpret_cast<const void *>(&skinny_kernel<NT, RB, W, S, (F != 0)>)},

const SkinnyVariant kSkinnyPartF32[] = {
    GDP_WAVES_SPW(GDP_ENTRY, 1, 1, 1)
    GDP_WAVES_SPW(GDP_ENTRY, 2, 1, 1)
    GDP_WAVES_SPW(GDP_ENTRY, 1, 2, 1)
    GDP_WAVES_SPW(GDP_ENTRY, 2, 2, 1)
};
const int kSkinnyPartF32Count = sizeof(kSkinnyPartF32) / sizeof(kSkinnyPartF32[0]);

}  // namespace gdp
