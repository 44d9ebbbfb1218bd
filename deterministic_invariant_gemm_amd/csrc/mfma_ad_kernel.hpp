// MFMA kernel with the A operand read straight from global memory into MFMA
// fragment registers ("A-direct"), for operands whose reduction index is
// contiguous: linear forward (A = X), dX (A = dY), grouped forward and dinput.
//
// Same arithmetic as mfma_gemm_kernel (mfma_kernel.hpp): every output element
// receives one v_mfma_f32_32x32x16_{bf16,f16} per 16-deep reduction step, in
// ascending order from +0, with the B fragment as the first operand and each
// lane holding the same 8 reduction values of its row -- so both kernels, and
// every tile shape of either, give identical bits.
//
// Why: at full MFMA rate a wave computing FM x FN blocks of 32x32 needs about
// 128*(FM+FN)/(FM*FN) bytes per clock per CU of operand fragments.  Reading
// every fragment from LDS (as mfma_gemm_kernel does) saturates LDS for the
// tile shapes these problem sizes allow.  Here A fragments (16 contiguous
// bytes per lane) come through the vector L1/L2 path instead and only B is
// staged through LDS, splitting the fragment traffic over two paths and
// removing A's LDS writes.
//
// Pipeline per 64-deep slice s: A fragments of slice s+1 are loaded into the
// second register set while slice s is multiplied from the first; B slice s+1
// (in registers since slice s-1) is written to the other LDS buffer and B
// slice s+2 is fetched.  One workgroup barrier per slice.  The loop is
// unrolled by two so both register sets are addressed statically.
#pragma once

#include "mfma_kernel.hpp"

namespace bi {
namespace mfma {

template <int FM, int WTM>
struct DirectA {
    // per 64-deep slice: 4 steps x FM fragments of 8 values per lane
    u32x4 f[2][BK / 16][FM];
    const uint16_t *rowp[FM];  // row base (row clamped into range) + lane's k offset

    __device__ __forceinline__ void init(const uint16_t *pa, int64_t lda, int64_t row0,
                                         int64_t row_end, int wm, int lrow, int lkg) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            int64_t r = row0 + wm * WTM + 32 * i + lrow;
            if (r > row_end - 1) r = row_end - 1;  // rows past the end: never stored
            rowp[i] = pa + r * lda + 8 * lkg;
        }
    }

    // slice at reduction offset rk into set S; `full`: the whole slice is in
    // range and rows are 16-byte aligned
    template <int S>
    __device__ __forceinline__ void load(int64_t rk, int64_t r_end, bool full, int lkg) {
        if (full) {
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    f[S][kk][i] = *reinterpret_cast<const u32x4 *>(rowp[i] + rk + 16 * kk);
        } else {
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                const int64_t k0 = rk + 16 * kk + 8 * lkg;
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    uint32_t e[8];
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        const int64_t k = k0 + x;
                        const int64_t kc = k < r_end ? k : r_end - 1;
                        // rowp already includes the lane's k offset (8*lkg)
                        const uint32_t v = rowp[i][kc - 8 * lkg];
                        e[x] = k < r_end ? v : 0u;
                    }
                    f[S][kk][i] = pack8(e);
                }
            }
        }
    }
};

template <int DT, bool B_RC, int BM, int BN, int WGM, int WGN, int EPI, int MODE>
__global__ __launch_bounds__(NT) void mfma_ad_kernel(MfmaArgs p) {
    static_assert(WGM * WGN == 4, "four waves");
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    static_assert(FM * 32 == WTM && FN * 32 == WTN, "wave tile must be a multiple of 32");
    constexpr int STAGE_SLOTS = 2 * KG * BN;
    constexpr int SLAB_SLOTS = slab_bytes<EPI, WTN>() / 16;
    constexpr int LDS_SLOTS = STAGE_SLOTS > SLAB_SLOTS ? STAGE_SLOTS : SLAB_SLOTS;

    __shared__ u32x4 lds_raw[LDS_SLOTS];
    __shared__ __align__(16) float lds_bias[BN];
    auto lds_b = [&](int b) { return lds_raw + b * (KG * BN); };

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int lrow = lane & 31, lkg = lane >> 5;

    const TileInfo ti = decode_tile<MODE, BM, BN>(p, t);
    if (ti.skip) return;
    const int64_t row0 = ti.row0, row_end = ti.row_end, col0 = ti.col0;
    const float bias_v = fetch_bias<DT, EPI, BN>(p, col0, t);
    const int64_t r_begin = ti.r_begin, r_end = ti.r_end;
    const uint16_t *pb = static_cast<const uint16_t *>(p.b) + ti.b_off;

    DirectA<FM, WTM> da;
    da.init(static_cast<const uint16_t *>(p.a), p.lda, row0, row_end, wm, lrow, lkg);
    Stage<BN, B_RC> sb;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const bool vec_a = p.vec_a != 0;
    const bool int_b = p.vec_b != 0 && col0 + BN <= p.cols;
    const int64_t nst = (r_end - r_begin + BK - 1) / BK;
    auto full = [&](int64_t rk) { return vec_a && rk + BK <= r_end; };

    // one slice: multiply slice s (A in set S, B in LDS buffer s&1) while
    // staging B slice s+1, fetching B slice s+2 and A slice s+1
    auto slice = [&](auto set_tag, int64_t s) {
        constexpr int S = decltype(set_tag)::value;
        const int cur = (int)(s & 1);
        const u32x4 *lb = lds_b(cur);
        u32x4 fb[2][FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[0][j] = lb[lkg * BN + swz(wn * WTN + 32 * j + lrow, lkg)];
        if (s + 1 < nst) {
            sb.store(lds_b(cur ^ 1), t);
            if (s + 2 < nst)
                sb.load(pb, p.ldb, col0, p.cols, r_begin + (s + 2) * BK, r_end, int_b, t);
            const int64_t rk = r_begin + (s + 1) * BK;
            da.template load<S ^ 1>(rk, r_end, full(rk), lkg);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = kk & 1;
            if (kk + 1 < BK / 16) {
                const int kg = 2 * (kk + 1) + lkg;
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    fb[c ^ 1][j] = lb[kg * BN + swz(wn * WTN + 32 * j + lrow, kg)];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = mfma_step<DT>(fb[c][j], da.f[S][kk][i], acc[i][j]);
        }
        __syncthreads();
    };

    if (nst > 0) {
        da.template load<0>(r_begin, r_end, full(r_begin), lkg);
        sb.load(pb, p.ldb, col0, p.cols, r_begin, r_end, int_b, t);
        sb.store(lds_b(0), t);
        if (nst > 1) sb.load(pb, p.ldb, col0, p.cols, r_begin + BK, r_end, int_b, t);
        __syncthreads();
    }
    int64_t s = 0;
    for (; s + 1 < nst; s += 2) {
        slice(std::integral_constant<int, 0>{}, s);
        slice(std::integral_constant<int, 1>{}, s + 1);
    }
    if (s < nst) slice(std::integral_constant<int, 0>{}, s);

    static_assert(SLAB_SLOTS <= LDS_SLOTS, "slabs fit");
    write_tile<DT, EPI, WTM, WTN, FM, FN, BN>(p, ti, acc, reinterpret_cast<char *>(lds_raw),
                                              lds_bias, bias_v, wave, wm, wn, lane);
}

template <int DT, bool BRC, int EPI, int MODE, int ID>
hipError_t launch_ad_tile(const MfmaArgs &p, int64_t grid, hipStream_t s) {
    using T = TileOf<ID>;
    hipLaunchKernelGGL((mfma_ad_kernel<DT, BRC, T::BM, T::BN, T::WGM, T::WGN, EPI, MODE>),
                       dim3(grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

// tile ids 20 + base id select the A-direct kernel with base tile `id`
template <int DT, bool BRC, int EPI, int MODE, int... IDS>
hipError_t launch_ad_among(const MfmaArgs &p, int tile_id, int64_t grid, hipStream_t s) {
    hipError_t r = hipErrorInvalidValue;
    ((tile_id == 20 + IDS ? (void)(r = launch_ad_tile<DT, BRC, EPI, MODE, IDS>(p, grid, s))
                          : (void)0),
     ...);
    return r;
}

}  // namespace mfma
}  // namespace bi
