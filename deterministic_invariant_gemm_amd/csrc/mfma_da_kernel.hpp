// MFMA kernel with the A operand loaded from global memory straight into MFMA
// fragment registers and only B staged in LDS ("direct-A" family), for A
// operands whose reduction index is contiguous (linear forward, dX, grouped
// forward and dinput).
//
// Same arithmetic as every other MFMA kernel here (mfma_kernel.hpp,
// mfma_dl_kernel.hpp): one v_mfma_f32_32x32x16_{bf16,f16} per 16-deep
// reduction step per output element, ascending from +0 over 64-deep stages
// that start at the first index of the element's reduction range, zeros past
// its end, B fragment first -- so all families and tile shapes give identical
// bits (sgemm-bi PyPI page, "Determinism contracts").
//
// Why: a CU moves about 128 bytes per clock through LDS and 64 through its
// vector cache.  With both operands staged in LDS, the fragment re-reads of an
// 8-wave 256x192 tile need more LDS bandwidth than the MFMAs leave time for.
// Here the waves are stacked along M (layout WGM x 1), so every wave owns
// distinct A rows and reads each A byte exactly once, through the vector cache;
// LDS carries only the B stage copies and the B fragment reads.
//
// Pipeline (stage s = 64 reduction values):
//   * A fragments: a ring of three register sets; set s%3 holds stage s, the
//     load of stage s+2 is issued at the start of stage s.
//   * B: a ring of three LDS stages filled by buffer_load ... lds (see
//     mfma_dl_kernel.hpp), stage s+3 issued at the barrier inside stage s.
//   * Per stage: steps 0..2 read the B fragments of the next step and multiply
//     the current one; then wait for B stage s+1, barrier, issue the copies,
//     read step 0 of stage s+1 and multiply step 3.
//   The copies into LDS are invisible to the compiler, so the kernel counts
//   every vector-memory instruction it issues and waits for exactly the ones a
//   B stage needs.
#pragma once

#include "mfma_dl_kernel.hpp"

namespace bi {
namespace mfma {

// s_waitcnt vmcnt(n) for a run-time n (clamped to 63, which only waits longer)
template <int N = 0>
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
    if constexpr (N >= 63) {
        wait_vmcnt<63>();
    } else {
        if (n <= N) wait_vmcnt<N>();
        else wait_vmcnt_dyn<N + 1>(n);
    }
}

// A fragments of one wave: FM blocks of 32 rows, 16 reduction values per step.
template <int FM>
struct AFrag {
    uint32_t off[FM];  // byte offset of this lane's 16 bytes at stage 0, step 0
    int kl;            // reduction offset of this lane inside a 16-deep step

    __device__ __forceinline__ void init(int64_t lda, int64_t row0, int64_t r_begin, int lane) {
        kl = 8 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < FM; ++i)
            off[i] = (uint32_t)(((row0 + 32 * i + (lane & 31)) * lda + r_begin + kl) * 2);
    }
    // stage s into `dst`; reduction indices >= rem (counted from the stage
    // start) read as zeros.  Branch-free, so the compiler sees one straight
    // sequence of loads.
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, u32x4 (&dst)[BK / 16][FM],
                                         int s, int64_t rem) const {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                uint32_t o = off[i] + (uint32_t)s * 128u + 32u * kk;
                if (16 * kk + kl >= rem) o = kOutOfRange;
                dst[kk][i] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)o, 0, 0));
            }
    }
};

template <int DT, bool B_RC, int BM, int BN, int WGM, int WGN, int EPI, int MODE>
__global__ __launch_bounds__(64 * WGM * WGN) void mfma_da_kernel(MfmaArgs p) {
    static_assert(WGN == 1, "waves are stacked along M so each reads distinct A rows");
    constexpr int NW = WGM;
    constexpr int WTM = BM / WGM, WTN = BN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    static_assert(FM * 32 == WTM && FN * 32 == WTN, "wave tile must be a multiple of 32");
    constexpr int SB = 128 * BN;  // bytes of one B stage
    constexpr int NS = 3;
    constexpr int LDS_BYTES = NS * SB > slab_bytes<EPI, WTN, NW>() ? NS * SB
                                                                   : slab_bytes<EPI, WTN, NW>();
    static_assert(LDS_BYTES + 4 * BN <= 160 * 1024, "fits in LDS");

    __shared__ __align__(1024) char lds_raw[LDS_BYTES];
    __shared__ __align__(16) float lds_bias[BN];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave;

    const TileInfo ti = decode_tile<MODE, BM, BN, 64 * NW>(p, t);
    if (ti.skip) return;
    const int64_t row0 = ti.row0, col0 = ti.col0;
    const float bias_v = fetch_bias<DT, EPI, BN>(p, col0, t);
    const int64_t r_begin = ti.r_begin, r_end = ti.r_end;

    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(p.a), (short)0, (int)p.a_bytes, 0x00020000);
    const i32x4 rsb = make_rsrc(static_cast<const uint16_t *>(p.b) + ti.b_off,
                                p.b_bytes - 2 * ti.b_off);
    using LB = DLoad<BN, B_RC, NW>;
    LB lb;
    lb.init(p.ldb, col0, r_begin, wave, lane);
    AFrag<FM> af;
    af.init(p.lda, row0 + wm * WTM, r_begin, lane);
    typename FragOf<B_RC, BN>::type rb;
    rb.init(lane);

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const int64_t red = r_end - r_begin;
    const int nst = (int)((red + BK - 1) / BK);
    BI_LDS char *ring = (BI_LDS char *)lds_raw;

    u32x4 ra[3][BK / 16][FM];  // A fragment ring
    u32x4 fb[2][FN];
    int issued = 0;            // vector-memory instructions issued by this wave
    int mark[NS];              // `issued` right after B stage x (slot x % NS)

    auto issue_b = [&](int s, int slot) {
        BI_LDS char *db = ring + slot * SB;
        const int64_t rem = red - (int64_t)BK * s;
        if (rem >= BK) lb.template issue<false>(rsb, db, s, rem, wave);
        else lb.template issue<true>(rsb, db, s, rem, wave);
        issued += LB::NQ;
        mark[slot] = issued;
    };
    auto load_a = [&](auto set_tag, int s) {
        constexpr int S = decltype(set_tag)::value;
        af.load(rsa, ra[S], s, red - (int64_t)BK * s);
        issued += (BK / 16) * FM;
    };
    auto read_b = [&](const BI_LDS char *st, int kk, int set) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            if constexpr (B_RC) fb[set][j] = rb.read(st, 32 * j, kk);
            else fb[set][j] = rb.read(st, j, kk);
        }
    };
    auto mfmas = [&](const u32x4 (&a)[FM], int set) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma_step<DT>(fb[set][j], a[i], acc[i][j]);
    };

    // one stage; S = s % 3 selects the A set and the B slot
    auto stage = [&](auto s_tag, int s) {
        constexpr int S = decltype(s_tag)::value;
        constexpr int S1 = (S + 1) % 3, S2 = (S + 2) % 3;
        const BI_LDS char *cur = ring + S * SB;
        // A stage s+2 into the set stage s-1 used; issued even past the last
        // stage (then every lane reads zeros without touching memory) so the
        // compiler always sees the same loads outstanding
        load_a(std::integral_constant<int, S2>{}, s + 2);
#pragma unroll
        for (int kk = 0; kk < BK / 16 - 1; ++kk) {
            read_b(cur, kk + 1, (kk + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
            mfmas(ra[S][kk], kk & 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (s + 1 < nst) {
            wait_vmcnt_dyn(issued - mark[S1]);  // B stage s+1 is in (this wave's share)
            __syncthreads();                     // ... every share; B stage s is free
            if (s + 3 < nst) issue_b(s + 3, S);
            read_b(ring + S1 * SB, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfmas(ra[S][BK / 16 - 1], 1);
        __builtin_amdgcn_sched_barrier(0);
    };

    load_a(std::integral_constant<int, 0>{}, 0);
    load_a(std::integral_constant<int, 1>{}, 1);
#pragma unroll
    for (int x = 0; x < NS; ++x)
        if (x < nst) issue_b(x, x);
    if (nst > 0) {
        // everything of the prologue is in (a clean start for the compiler's
        // own bookkeeping of the A loads inside the loop)
        wait_vmcnt<0>();
        __syncthreads();
        read_b(ring, 0, 0);
    }
    int s = 0;
    for (; s + 3 <= nst; s += 3) {
        stage(std::integral_constant<int, 0>{}, s);
        stage(std::integral_constant<int, 1>{}, s + 1);
        stage(std::integral_constant<int, 2>{}, s + 2);
    }
    if (s < nst) stage(std::integral_constant<int, 0>{}, s);
    if (s + 1 < nst) stage(std::integral_constant<int, 1>{}, s + 1);

    write_tile<DT, EPI, WTM, WTN, FM, FN, BN>(p, ti, acc, reinterpret_cast<char *>(lds_raw),
                                              lds_bias, bias_v, wave, wm, 0, lane);
}

template <int DT, bool BRC, int EPI, int MODE, int ID>
hipError_t launch_da_tile(const MfmaArgs &p, int64_t grid, hipStream_t s) {
    using T = TileOf<ID>;
    hipLaunchKernelGGL((mfma_da_kernel<DT, BRC, T::BM, T::BN, T::WGM, T::WGN, EPI, MODE>),
                       dim3(grid), dim3(64 * T::WGM * T::WGN), 0, s, p);
    return hipGetLastError();
}

// tile ids 60 + base id select the direct-A kernel with base tile `id`
template <int DT, bool BRC, int EPI, int MODE, int... IDS>
hipError_t launch_da_among(const MfmaArgs &p, int tile_id, int64_t grid, hipStream_t s) {
    hipError_t r = hipErrorInvalidValue;
    ((tile_id == 60 + IDS ? (void)(r = launch_da_tile<DT, BRC, EPI, MODE, IDS>(p, grid, s))
                          : (void)0),
     ...);
    return r;
}

}  // namespace mfma
}  // namespace bi
