// MFMA kernel with eight waves in two alternating groups ("ping-pong"), both
// operands copied global -> LDS as in the direct-load family
// (mfma_dl_kernel.hpp).
//
// Same arithmetic as every other MFMA kernel here: one
// v_mfma_f32_32x32x16_{bf16,f16} per 16-deep reduction step per output element,
// ascending from +0 over 64-deep stages starting at the first index of the
// element's reduction range, zeros past its end, B fragment first -- so all
// families and tile shapes give identical bits (sgemm-bi PyPI page,
// "Determinism contracts").
//
// Why: with two waves per SIMD doing the same mix of LDS reads and MFMAs, the
// older wave of each SIMD runs ahead and then waits at the stage barrier, and
// the younger one finishes the stage alone, unable to hide its own LDS
// latency behind MFMAs.  Here waves 0..NW/2-1 (group 0) and NW/2..NW-1
// (group 1) -- one of each on every SIMD -- take turns: between two workgroup
// barriers one group only issues MFMAs (all fragments of the stage already in
// registers) while the other only reads the fragments of its next stage from
// LDS.  The MFMA unit of each SIMD is fed by one wave at a time, the LDS
// traffic of the other wave overlaps it.
//
// Slots (each ends with a workgroup barrier), stage s of NST:
//   slot 2s   : group 0 reads stage s;     group 1 multiplies stage s-1
//   slot 2s+1 : group 0 multiplies stage s; group 1 reads stage s
// Before slot 2s every wave has waited for its share of the copy of stage s;
// after slot 2s+1 stage s is no longer read, and at the start of slot 2s+2
// its LDS buffer receives stage s+NS.
#pragma once

#include "mfma_dl_kernel.hpp"

namespace bi {
namespace mfma {

template <int DT, bool A_RC, bool B_RC, int BM, int BN, int WGM, int WGN, int EPI, int MODE>
__global__ __launch_bounds__(64 * WGM * WGN) void mfma_pp_kernel(MfmaArgs p) {
    constexpr int NW = WGM * WGN;
    static_assert(NW == 8 && WGM % 2 == 0, "eight waves, each group a half of the wave rows");
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    static_assert(FM * 32 == WTM && FN * 32 == WTN, "wave tile must be a multiple of 32");
    constexpr int SA = 128 * BM, SB = 128 * BN;  // bytes of one stage of A / B
    constexpr int NS = dl_stages(BM, BN);
    static_assert(NS >= 2 && NS <= 4, "two to four stages");
    static_assert(slab_bytes<EPI, WTN, NW>() <= NS * (SA + SB), "epilogue slabs fit in the stages");
    constexpr int KS = BK / 16;  // 16-deep steps per stage

    __shared__ __align__(1024) char lds_raw[NS * (SA + SB)];
    __shared__ __align__(16) float lds_bias[BN];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int grp = wm < WGM / 2 ? 0 : 1;  // waves 0..3 / 4..7: one of each per SIMD

    const TileInfo ti = decode_tile<MODE, BM, BN, 64 * NW>(p, t);
    if (ti.skip) return;
    const int64_t row0 = ti.row0, col0 = ti.col0;
    const float bias_v = fetch_bias<DT, EPI, BN>(p, col0, t);
    const int64_t r_begin = ti.r_begin, r_end = ti.r_end;

    const i32x4 rsa = make_rsrc(p.a, p.a_bytes);
    const i32x4 rsb = make_rsrc(static_cast<const uint16_t *>(p.b) + ti.b_off,
                                p.b_bytes - 2 * ti.b_off);
    using LA = DLoad<BM, A_RC, NW>;
    using LB = DLoad<BN, B_RC, NW>;
    LA la;
    LB lb;
    la.init(p.lda, row0, r_begin, wave, lane);
    lb.init(p.ldb, col0, r_begin, wave, lane);
    typename FragOf<A_RC, BM>::type ra;
    typename FragOf<B_RC, BN>::type rb;
    ra.init(lane);
    rb.init(lane);

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const int64_t red = r_end - r_begin;
    const int nst = (int)((red + BK - 1) / BK);
    BI_LDS char *ring = (BI_LDS char *)lds_raw;

    auto issue = [&](int s) {
        BI_LDS char *da = ring + (s % NS) * (SA + SB);
        BI_LDS char *db = da + SA;
        const int64_t rem = red - (int64_t)BK * s;
        if (rem >= BK) {
            la.template issue<false>(rsa, da, s, rem, wave);
            lb.template issue<false>(rsb, db, s, rem, wave);
        } else {
            la.template issue<true>(rsa, da, s, rem, wave);
            lb.template issue<true>(rsb, db, s, rem, wave);
        }
    };

    // all fragments of one stage
    u32x4 fa[KS][FM], fb[KS][FN];
    auto read_stage = [&](int s) {
        const BI_LDS char *st = ring + (s % NS) * (SA + SB);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                if constexpr (A_RC) fa[kk][i] = ra.read(st, wm * WTM + 32 * i, kk);
                else fa[kk][i] = ra.read(st, (wm * WTM) / 32 + i, kk);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if constexpr (B_RC) fb[kk][j] = rb.read(st + SA, wn * WTN + 32 * j, kk);
                else fb[kk][j] = rb.read(st + SA, (wn * WTN) / 32 + j, kk);
            }
        }
    };
    auto multiply_stage = [&]() {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = mfma_step<DT>(fb[kk][j], fa[kk][i], acc[i][j]);
    };

#pragma unroll
    for (int s = 0; s < NS; ++s)
        if (s < nst) issue(s);
    if (nst > 0) {
        // issued: stages 0 .. min(NS-1, nst-1); wait for stage 0
        const int later = nst - 1 < NS - 1 ? nst - 1 : NS - 1;
        wait_vmcnt_stages<LA::NQ + LB::NQ>(later);
    }
    __syncthreads();

    // Each group runs its own loop so that fragments are produced and consumed
    // inside one iteration; both loops pass the same 2*nst+1 barriers.
    // stage s+1 must be in before slot 2s+2; issued by then: stages
    // 0 .. min(s+NS-1, nst-1)
    auto wait_next = [&](int s) {
        if (s + 1 < nst) {
            const int later = nst - 2 - s < NS - 2 ? nst - 2 - s : NS - 2;
            wait_vmcnt_stages<LA::NQ + LB::NQ>(later);
        }
    };
    if (grp == 0) {
        for (int s = 0; s < nst; ++s) {
            // slot 2s: stage s-1 is read by both groups, its buffer takes stage s-1+NS
            if (s >= 1 && s - 1 + NS < nst) issue(s - 1 + NS);
            read_stage(s);
            __syncthreads();
            // slot 2s+1
            multiply_stage();
            wait_next(s);
            __syncthreads();
        }
        __syncthreads();  // slot 2*nst: group 1 multiplies the last stage
    } else {
        __syncthreads();  // slot 0: group 0 reads stage 0
        for (int s = 0; s < nst; ++s) {
            // slot 2s+1
            read_stage(s);
            wait_next(s);
            __syncthreads();
            // slot 2s+2
            if (s + NS < nst) issue(s + NS);
            multiply_stage();
            __syncthreads();
        }
    }

    write_tile<DT, EPI, WTM, WTN, FM, FN, BN>(p, ti, acc, reinterpret_cast<char *>(lds_raw),
                                              lds_bias, bias_v, wave, wm, wn, lane);
}

template <int DT, bool ARC, bool BRC, int EPI, int MODE, int ID>
hipError_t launch_pp_tile(const MfmaArgs &p, int64_t grid, hipStream_t s) {
    using T = TileOf<ID>;
    hipLaunchKernelGGL((mfma_pp_kernel<DT, ARC, BRC, T::BM, T::BN, T::WGM, T::WGN, EPI, MODE>),
                       dim3(grid), dim3(64 * T::WGM * T::WGN), 0, s, p);
    return hipGetLastError();
}

// tile ids 80 + base id select the ping-pong kernel with base tile `id`
template <int DT, bool ARC, bool BRC, int EPI, int MODE, int... IDS>
hipError_t launch_pp_among(const MfmaArgs &p, int tile_id, int64_t grid, hipStream_t s) {
    hipError_t r = hipErrorInvalidValue;
    ((tile_id == 80 + IDS ? (void)(r = launch_pp_tile<DT, ARC, BRC, EPI, MODE, IDS>(p, grid, s))
                          : (void)0),
     ...);
    return r;
}

}  // namespace mfma
}  // namespace bi
