// tile_tables.hpp -- instantiate every kernel of one macro-tile shape and
// return launchers by (layout, dtype, epilogue).  Included once by each
// per-tile translation unit so the shapes compile in parallel.
#pragma once

#include "internal.hpp"

namespace mgemm {

template <class T, bool AK, bool BK, int IN, int OUT>
hipError_t launch_dense_tile(const DenseArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((dense_kernel<T, AK, BK, IN, OUT>), dim3(grid), dim3(T::NT), 0, s, a);
    return hipGetLastError();
}

// Register staging sets per tile.  Two for every shape: four sets on the
// narrow tiles (whose sets are only ~40 VGPRs) measured no faster on
// weight-streaming MoE experts or the decode shape.
template <int BM, int BN>
constexpr int staging_sets() { return 2; }

template <int BM, int BN, int WM, int WN, bool AK, bool BK, int IN>
using TileOf = Tile<BM, BN, WM, WN, AK, BK, IN, staging_sets<BM, BN>()>;

template <int BM, int BN, int WM, int WN, bool AK, bool BK, int IN, int OUT>
hipError_t launch_dense(const DenseArgs &a, int grid, hipStream_t s)
{
    return launch_dense_tile<TileOf<BM, BN, WM, WN, AK, BK, IN>, AK, BK, IN, OUT>(a, grid, s);
}

// Grouped launches of the register-staged tiles (task table in LDS).
template <int BM, int BN, int WM, int WN, bool BK, int IN, int OUT, int EPI>
hipError_t launch_grouped(const GroupedArgs &a, int grid, hipStream_t s)
{
    using T = TileOf<BM, BN, WM, WN, true, BK, IN>;
    hipLaunchKernelGGL((grouped_kernel<T, BK, IN, OUT, EPI>), dim3(grid), dim3(T::NT), 0, s, a);
    return hipGetLastError();
}

// Output types compiled: fp32, and the 16-bit type of the inputs.
template <int IN>
constexpr int same16() { return IN == IN_BF16 ? OUT_BF16 : OUT_F16; }

// ALL_A: also compile the row-contiguous (column-major) A loader.
template <int BM, int BN, int WM, int WN, int IN, bool ALL_A>
DenseFn dense_table(bool ak, bool bk, int out)
{
    if (out != OUT_F32 && out != same16<IN>())
        return nullptr;
    const bool f32 = out == OUT_F32;
#define MG_D(AKV, BKV) (f32 ? launch_dense<BM, BN, WM, WN, AKV, BKV, IN, OUT_F32> \
                            : launch_dense<BM, BN, WM, WN, AKV, BKV, IN, same16<IN>()>)
    if (ak)
        return bk ? MG_D(true, true) : MG_D(true, false);
    if constexpr (ALL_A)
        return bk ? MG_D(false, true) : MG_D(false, false);
    return nullptr;
#undef MG_D
}

// The direct-to-LDS 256 x 256 engine for dense plans: row-major
// (k-contiguous) A, B either way, on four waves of 128 x 128 (DtlTile4).
template <int IN>
DenseFn dense_dtl_table(bool ak, bool bk, int out)
{
    if (!ak || (out != OUT_F32 && out != same16<IN>()))
        return nullptr;
    if (bk)
        return out == OUT_F32 ? launch_dense_tile<DtlTile4<IN, true>, true, true, IN, OUT_F32>
                              : launch_dense_tile<DtlTile4<IN, true>, true, true, IN, same16<IN>()>;
    return out == OUT_F32 ? launch_dense_tile<DtlTile4<IN, false>, true, false, IN, OUT_F32>
                          : launch_dense_tile<DtlTile4<IN, false>, true, false, IN, same16<IN>()>;
}

// Stream-K launch of the four-wave direct-to-LDS tile (row-major A).
template <bool BK, int IN, int OUT>
hipError_t launch_dense_sk(const DenseArgs &a, int grid, hipStream_t s)
{
    using T = DtlTile4<IN, BK>;
    hipLaunchKernelGGL((dense_sk_kernel<T, BK, IN, OUT>), dim3(grid), dim3(T::NT), 0, s, a);
    return hipGetLastError();
}
template <int IN>
DenseFn dense_sk_table(bool bk, int out)
{
    if (out != OUT_F32 && out != same16<IN>())
        return nullptr;
    if (bk)
        return out == OUT_F32 ? launch_dense_sk<true, IN, OUT_F32> : launch_dense_sk<true, IN, same16<IN>()>;
    return out == OUT_F32 ? launch_dense_sk<false, IN, OUT_F32> : launch_dense_sk<false, IN, same16<IN>()>;
}

// E4M3 inputs: A row-major and B column-major only (both k-contiguous).
template <int OUT>
hipError_t launch_dense_e4m3(const DenseArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((dense_e4m3_kernel<OUT>), dim3(grid), dim3(DtlTile4E4M3::NT), 0, s, a);
    return hipGetLastError();
}
inline DenseFn dense_e4m3_table(bool ak, bool bk, int out)
{
    if (!ak || !bk)
        return nullptr;
    switch (out) {
    case OUT_F32: return launch_dense_e4m3<OUT_F32>;
    case OUT_BF16: return launch_dense_e4m3<OUT_BF16>;
    case OUT_F16: return launch_dense_e4m3<OUT_F16>;
    default: return nullptr;
    }
}

// The blockwise-scaled E4M3 product (E8M0 block scales in DenseArgs).
template <int OUT>
hipError_t launch_dense_e4m3_block(const DenseArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((dense_e4m3_block_kernel<OUT>), dim3(grid), dim3(DtlTile4E4M3::NT), 0, s, a);
    return hipGetLastError();
}
inline DenseFn dense_e4m3_block_table(bool ak, bool bk, int out)
{
    if (!ak || !bk)
        return nullptr;
    switch (out) {
    case OUT_F32: return launch_dense_e4m3_block<OUT_F32>;
    case OUT_BF16: return launch_dense_e4m3_block<OUT_BF16>;
    case OUT_F16: return launch_dense_e4m3_block<OUT_F16>;
    default: return nullptr;
    }
}

template <int OUT>
hipError_t launch_grouped_e4m3(const GroupedArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((grouped_e4m3_kernel<OUT>), dim3(grid), dim3(DtlTile4E4M3::NT), 0, s, a);
    return hipGetLastError();
}
template <int OUT>
hipError_t launch_grouped_e4m3_block(const GroupedArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((grouped_e4m3_block_kernel<OUT>), dim3(grid), dim3(DtlTile4E4M3::NT), 0, s, a);
    return hipGetLastError();
}
inline GroupedFn grouped_e4m3_block_table(bool bk, int out, int epi)
{
    if (!bk || epi != EPI_NONE)
        return nullptr;
    switch (out) {
    case OUT_F32: return launch_grouped_e4m3_block<OUT_F32>;
    case OUT_BF16: return launch_grouped_e4m3_block<OUT_BF16>;
    case OUT_F16: return launch_grouped_e4m3_block<OUT_F16>;
    }
    return nullptr;
}
inline GroupedFn grouped_e4m3_table(bool bk, int out, int epi)
{
    if (!bk || epi != EPI_NONE)
        return nullptr;
    switch (out) {
    case OUT_F32: return launch_grouped_e4m3<OUT_F32>;
    case OUT_BF16: return launch_grouped_e4m3<OUT_BF16>;
    case OUT_F16: return launch_grouped_e4m3<OUT_F16>;
    default: return nullptr;
    }
}

// Grouped launches of the direct-to-LDS tile: its rings fill the LDS, so
// the task list lives in registers (grouped_kernel_wt).
template <bool BK, int IN, int OUT, int EPI>
hipError_t launch_grouped_dtl(const GroupedArgs &a, int grid, hipStream_t s)
{
    using T = DtlTile<IN, BK>;
    hipLaunchKernelGGL((grouped_kernel_wt<T, BK, IN, OUT, EPI>), dim3(grid), dim3(T::NT), 0, s, a);
    return hipGetLastError();
}

template <int IN>
GroupedFn grouped_dtl_table(bool bk, int out, int epi)
{
    if (out != OUT_F32 && out != same16<IN>())
        return nullptr;
    const bool f32 = out == OUT_F32;
#define MG_G(BKV, OUTV) (epi == EPI_NONE ? launch_grouped_dtl<BKV, IN, OUTV, EPI_NONE> \
                                         : launch_grouped_dtl<BKV, IN, OUTV, EPI_SILU_GATE>)
    if (bk)
        return f32 ? MG_G(true, OUT_F32) : MG_G(true, same16<IN>());
    return f32 ? MG_G(false, OUT_F32) : MG_G(false, same16<IN>());
#undef MG_G
}

// The few-token tile (BN columns): row-major (k-contiguous) A, B either way.
template <bool BK, int IN, int OUT, int BN>
hipError_t launch_dense_narrow(const DenseArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((narrow_dense_kernel<BK, IN, OUT, BN>), dim3(grid), dim3(NarrowTile<IN, BK, BN>::NT), 0, s, a);
    return hipGetLastError();
}
template <int IN, int BN>
DenseFn dense_narrow_table(bool ak, bool bk, int out)
{
    if (!ak || (out != OUT_F32 && out != same16<IN>()))
        return nullptr;
    if (bk)
        return out == OUT_F32 ? launch_dense_narrow<true, IN, OUT_F32, BN> : launch_dense_narrow<true, IN, same16<IN>(), BN>;
    return out == OUT_F32 ? launch_dense_narrow<false, IN, OUT_F32, BN> : launch_dense_narrow<false, IN, same16<IN>(), BN>;
}
template <bool BK, int IN, int OUT, int EPI, int BN>
hipError_t launch_grouped_narrow(const GroupedArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((narrow_grouped_kernel<BK, IN, OUT, EPI, BN>), dim3(grid), dim3(NarrowTile<IN, BK, BN>::NT), 0, s,
                       a);
    return hipGetLastError();
}
template <int IN, int BN>
GroupedFn grouped_narrow_table(bool bk, int out, int epi)
{
    if (out != OUT_F32 && out != same16<IN>())
        return nullptr;
    const bool f32 = out == OUT_F32;
#define MG_G(BKV, OUTV) (epi == EPI_NONE ? launch_grouped_narrow<BKV, IN, OUTV, EPI_NONE, BN> \
                                         : launch_grouped_narrow<BKV, IN, OUTV, EPI_SILU_GATE, BN>)
    if (bk)
        return f32 ? MG_G(true, OUT_F32) : MG_G(true, same16<IN>());
    return f32 ? MG_G(false, OUT_F32) : MG_G(false, same16<IN>());
#undef MG_G
}

template <int BM, int BN, int WM, int WN, int IN>
GroupedFn grouped_table(bool bk, int out, int epi)
{
    if (out != OUT_F32 && out != same16<IN>())
        return nullptr;
    const bool f32 = out == OUT_F32;
#define MG_G(BKV, OUTV) (epi == EPI_NONE ? launch_grouped<BM, BN, WM, WN, BKV, IN, OUTV, EPI_NONE> \
                                         : launch_grouped<BM, BN, WM, WN, BKV, IN, OUTV, EPI_SILU_GATE>)
    if (bk)
        return f32 ? MG_G(true, OUT_F32) : MG_G(true, same16<IN>());
    return f32 ? MG_G(false, OUT_F32) : MG_G(false, same16<IN>());
#undef MG_G
}

}  // namespace mgemm
