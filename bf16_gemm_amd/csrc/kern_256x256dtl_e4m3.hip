// kern_256x256dtl_e4m3.hip -- E4M3 kernels of the direct-to-LDS 256 x 256 macro-tile.
#include "tile_tables.hpp"

namespace mgemm {
DenseFn dense_fn_256x256dtl_e4m3(bool ak, bool bk, int out) { return dense_e4m3_table(ak, bk, out); }
DenseFn dense_block_fn_256x256dtl_e4m3(bool ak, bool bk, int out) { return dense_e4m3_block_table(ak, bk, out); }
GroupedFn grouped_fn_256x256dtl_e4m3(bool bk, int out, int epi) { return grouped_e4m3_table(bk, out, epi); }
GroupedFn grouped_block_fn_256x256dtl_e4m3(bool bk, int out, int epi) { return grouped_e4m3_block_table(bk, out, epi); }
}  // namespace mgemm
