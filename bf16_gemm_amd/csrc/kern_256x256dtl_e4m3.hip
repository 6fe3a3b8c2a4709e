// kern_256x256dtl_e4m3.hip -- E4M3 kernels of the direct-to-LDS 256 x 256 macro-tile.
#include "tile_tables.hpp"

namespace mgemm {
DenseFn dense_fn_256x256dtl_e4m3(bool ak, bool bk, int out) { return dense_e4m3_table(ak, bk, out); }
}  // namespace mgemm
