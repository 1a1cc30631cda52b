// BF16-weight skinny variants with one 16-token sub-tile.
#include "skinny.h"
#include "variants.h"

namespace gdp {

#define GDP_ENTRY(NT, RB, W, S, F) {NT, RB, W, S, F, reinterpret_cast<const void *>(&skinny_kernel<NT, RB, W, S, (F != 0)>)},

const SkinnyVariant kSkinnyPartBf16Nt1[] = {
    GDP_WAVES_SPW(GDP_ENTRY, 1, 1, 0)
    GDP_WAVES_SPW(GDP_ENTRY, 1, 2, 0)
    GDP_ENTRY(1, 4, 4, 8, 0) GDP_ENTRY(1, 4, 4, 16, 0) GDP_ENTRY(1, 4, 8, 8, 0) GDP_ENTRY(1, 4, 8, 16, 0)
    // activations preloaded per wave (at most 4 / 8 tokens)
    {1, 1, 8, 32, 0, reinterpret_cast<const void *>(&skinny_kernel<1, 1, 8, 32, false, false, 4>), 0, 4},
    {1, 1, 8, 32, 0, reinterpret_cast<const void *>(&skinny_kernel<1, 1, 8, 32, false, false, 8>), 0, 8},
    {1, 1, 4, 8, 0, reinterpret_cast<const void *>(&skinny_kernel<1, 1, 4, 8, false, false, 4>), 0, 4},
    {1, 1, 4, 8, 0, reinterpret_cast<const void *>(&skinny_kernel<1, 1, 4, 8, false, false, 8>), 0, 8},
};
const int kSkinnyPartBf16Nt1Count = sizeof(kSkinnyPartBf16Nt1) / sizeof(kSkinnyPartBf16Nt1[0]);

}  // namespace gdp
