// kern_64x256_f16.hip -- f16 kernels of the 64 x 256 macro-tile (1 x 4 wavefronts).
#include "tile_tables.hpp"

namespace mgemm {
DenseFn dense_fn_64x256_f16(bool ak, bool bk, int out) { return dense_table<64, 256, 1, 4, IN_F16, false>(ak, bk, out); }
GroupedFn grouped_fn_64x256_f16(bool bk, int out, int epi) { return grouped_table<64, 256, 1, 4, IN_F16>(bk, out, epi); }
}  // namespace mgemm
