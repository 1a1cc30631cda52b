// BF16-weight skinny variants with two 16-token sub-tiles.
#include "skinny.h"
#include "variants.h"

namespace gdp {

#define GDP_ENTRY(NT, RB, W, S, F) {NT, RB, W, S, F, reinterpret_cast<const void *>(&skinny_kernel<NT, RB, W, S, (F != 0)>)},

const SkinnyVariant kSkinnyPartBf16Nt2[] = {
    GDP_WAVES_SPW(GDP_ENTRY, 2, 1, 0)
    GDP_WAVES_SPW(GDP_ENTRY, 2, 2, 0)
    GDP_ENTRY(2, 4, 4, 8, 0) GDP_ENTRY(2, 4, 4, 16, 0) GDP_ENTRY(2, 4, 8, 8, 0)
};
const int kSkinnyPartBf16Nt2Count = sizeof(kSkinnyPartBf16Nt2) / sizeof(kSkinnyPartBf16Nt2[0]);

}  // namespace gdp
