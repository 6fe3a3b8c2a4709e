// kern_narrow64_f16.hip -- f16 kernels of the few-token tile, 64 columns wide.
#include "tile_tables.hpp"

namespace mgemm {
DenseFn dense_fn_narrow64_f16(bool ak, bool bk, int out) { return dense_narrow_table<IN_F16, 64>(ak, bk, out); }
GroupedFn grouped_fn_narrow64_f16(bool bk, int out, int epi) { return grouped_narrow_table<IN_F16, 64>(bk, out, epi); }
}  // namespace mgemm
