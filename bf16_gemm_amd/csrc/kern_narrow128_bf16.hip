// kern_narrow128_bf16.hip -- bf16 kernels of the few-token tile, 128 columns wide.
#include "tile_tables.hpp"

namespace mgemm {
DenseFn dense_fn_narrow128_bf16(bool ak, bool bk, int out) { return dense_narrow_table<IN_BF16, 128>(ak, bk, out); }
GroupedFn grouped_fn_narrow128_bf16(bool bk, int out, int epi) { return grouped_narrow_table<IN_BF16, 128>(bk, out, epi); }
}  // namespace mgemm
