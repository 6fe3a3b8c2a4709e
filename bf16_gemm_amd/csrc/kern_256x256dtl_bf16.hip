// kern_256x256dtl_bf16.hip -- bf16 kernels of the direct-to-LDS 256 x 256 macro-tile.
#include "tile_tables.hpp"

namespace mgemm {
DenseFn dense_fn_256x256dtl_bf16(bool ak, bool bk, int out) { return dense_dtl_table<IN_BF16>(ak, bk, out); }
GroupedFn grouped_fn_256x256dtl_bf16(bool bk, int out, int epi) { return grouped_dtl_table<IN_BF16>(bk, out, epi); }
DenseFn dense_sk_fn_256x256dtl_bf16(bool bk, int out) { return dense_sk_table<IN_BF16>(bk, out); }
}  // namespace mgemm
