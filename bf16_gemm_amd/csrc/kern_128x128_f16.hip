// kern_128x128_f16.hip -- f16 kernels of the 128 x 128 macro-tile (2 x 2 wavefronts).
#include "tile_tables.hpp"

namespace mgemm {
DenseFn dense_fn_128x128_f16(bool ak, bool bk, int out) { return dense_table<128, 128, 2, 2, IN_F16, true>(ak, bk, out); }
GroupedFn grouped_fn_128x128_f16(bool bk, int out, int epi) { return grouped_table<128, 128, 2, 2, IN_F16>(bk, out, epi); }
}  // namespace mgemm
