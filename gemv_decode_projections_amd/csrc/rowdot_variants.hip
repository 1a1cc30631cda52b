// Row-dot kernel variants: (token capacity, rows per workgroup, 2048-wide k
// chunks per row, FP32 weights). FP32 variants serve the router's 8192-wide
// rows (4 chunks), BF16 ones the unpooler's 4096-wide rows (2 chunks).
#include "rowdot.h"
#include "variants.h"

namespace gdp {

#define GDP_ROW(M, R, KIT, F) {M, R, KIT, F, reinterpret_cast<const void *>(&rowdot_kernel<M, R, KIT, (F != 0)>)},

const RowVariant kRowVariants[] = {
    GDP_ROW(1, 1, 4, 1) GDP_ROW(2, 1, 4, 1) GDP_ROW(4, 1, 4, 1) GDP_ROW(8, 1, 4, 1)
    GDP_ROW(1, 2, 4, 1) GDP_ROW(2, 2, 4, 1) GDP_ROW(4, 2, 4, 1) GDP_ROW(8, 2, 4, 1)
    GDP_ROW(1, 1, 2, 0) GDP_ROW(2, 1, 2, 0) GDP_ROW(4, 1, 2, 0) GDP_ROW(8, 1, 2, 0)
    GDP_ROW(1, 2, 2, 0) GDP_ROW(2, 2, 2, 0) GDP_ROW(4, 2, 2, 0) GDP_ROW(8, 2, 2, 0)
    GDP_ROW(1, 4, 2, 0) GDP_ROW(2, 4, 2, 0) GDP_ROW(4, 4, 2, 0) GDP_ROW(8, 4, 2, 0)
};
const int kRowVariantCount = sizeof(kRowVariants) / sizeof(kRowVariants[0]);

}  // namespace gdp
