// kern_256x256_bf16.hip -- bf16 kernels of the 256 x 256 macro-tile (2 x 2 wavefronts).
#include "tile_tables.hpp"

namespace mgemm {
DenseFn dense_fn_256x256_bf16(bool ak, bool bk, int out) { return dense_table<256, 256, 2, 2, IN_BF16, true>(ak, bk, out); }
GroupedFn grouped_fn_256x256_bf16(bool bk, int out, int epi) { return grouped_table<256, 256, 2, 2, IN_BF16>(bk, out, epi); }
}  // namespace mgemm
