// Skinny kernel variants with the stream partition (SKM): WAVES x SPW
// (row block, k-step) units per workgroup, one or two 16-token blocks, BF16
// or 12-bit weights. 144 units per workgroup deal qkv_gate's 144 row blocks
// x 256 k-steps to exactly 256 workgroups.
#include "skinny.h"
#include "variants.h"

namespace gdp {

#define GDP_SK(NT, W, S, Z) \
    {NT, 1, W, S, 0, reinterpret_cast<const void *>(&skinny_kernel<NT, 2, W, S, false, (Z != 0), 0, true>), Z, 0, 1},

const SkinnyVariant kSkinnyPartStream[] = {
    GDP_SK(1, 4, 36, 0) GDP_SK(1, 6, 24, 0) GDP_SK(1, 9, 16, 0) GDP_SK(1, 12, 12, 0)
    GDP_SK(1, 4, 36, 1) GDP_SK(1, 6, 24, 1) GDP_SK(1, 9, 16, 1) GDP_SK(1, 12, 12, 1)
    GDP_SK(2, 6, 24, 0) GDP_SK(2, 9, 16, 0) GDP_SK(2, 6, 24, 1) GDP_SK(2, 9, 16, 1)
    GDP_SK(1, 2, 72, 1) GDP_SK(1, 3, 48, 1) GDP_SK(2, 4, 36, 1) GDP_SK(2, 3, 48, 1) GDP_SK(2, 2, 72, 1)
};
const int kSkinnyPartStreamCount = sizeof(kSkinnyPartStream) / sizeof(kSkinnyPartStream[0]);

}  // namespace gdp
