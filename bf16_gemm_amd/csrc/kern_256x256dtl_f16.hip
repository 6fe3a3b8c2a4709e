// kern_256x256dtl_f16.hip -- f16 kernels of the direct-to-LDS 256 x 256 macro-tile.
#include "tile_tables.hpp"

namespace mgemm {
DenseFn dense_fn_256x256dtl_f16(bool ak, bool bk, int out) { return dense_dtl_table<IN_F16>(ak, bk, out); }
GroupedFn grouped_fn_256x256dtl_f16(bool bk, int out, int epi) { return grouped_dtl_table<IN_F16>(bk, out, epi); }
DenseFn dense_sk_fn_256x256dtl_f16(bool bk, int out) { return dense_sk_table<IN_F16>(bk, out); }
}  // namespace mgemm
