// kern_256x256_f16.hip -- f16 kernels of the 256 x 256 macro-tile (2 x 2 wavefronts).
#include "tile_tables.hpp"

namespace mgemm {
DenseFn dense_fn_256x256_f16(bool ak, bool bk, int out) { return dense_table<256, 256, 2, 2, IN_F16, true>(ak, bk, out); }
GroupedFn grouped_fn_256x256_f16(bool bk, int out, int epi) { return grouped_table<256, 256, 2, 2, IN_F16>(bk, out, epi); }
}  // namespace mgemm
