// kern_32x256_bf16.hip -- bf16 kernels of the 32 x 256 macro-tile (1 x 4 wavefronts).
#include "tile_tables.hpp"

namespace mgemm {
DenseFn dense_fn_32x256_bf16(bool ak, bool bk, int out) { return dense_table<32, 256, 1, 4, IN_BF16, false>(ak, bk, out); }
GroupedFn grouped_fn_32x256_bf16(bool bk, int out, int epi) { return grouped_table<32, 256, 1, 4, IN_BF16>(bk, out, epi); }
}  // namespace mgemm
