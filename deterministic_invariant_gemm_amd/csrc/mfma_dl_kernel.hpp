// MFMA kernel with both operands copied from global memory straight into LDS
// ("direct-load" family) for gfx950.
//
// Same arithmetic as mfma_gemm_kernel (mfma_kernel.hpp): every output element
// receives one v_mfma_f32_32x32x16_{bf16,f16} per 16-deep reduction step, in
// ascending order from +0 over 64-deep stages starting at the first index of
// its reduction range, reduction indices past the end contributing exact
// zeros, and the B fragment is the first MFMA operand.  fp8 e4m3 operands are
// staged as bytes (128 per stage row) and, on the exact path, widened to bf16
// in registers for the same bf16 instruction per 16-deep step; the fast path
// issues one v_mfma_scale_f32_32x32x64_f8f6f4 per 64-deep step instead.  Every tile shape of
// this family, and of the other kernel families, therefore gives identical
// bits (sgemm-bi PyPI page, "Determinism contracts": bit-identical tile
// families; the forward is batch-invariant because no tile reads M).
//
// Data movement:
//   * buffer_load_dwordx4 ... lds: each lane copies 16 bytes from global memory
//     into LDS at (instruction base + 16 * lane), without passing through
//     registers, while earlier stages are being multiplied.  Lanes are assigned so that one instruction reads whole
//     128-byte lines.  A lane whose chunk lies past the end of the reduction
//     range is given an offset beyond the buffer, which makes the hardware
//     return zeros; operand rows or columns past the matrix edge are read from
//     whatever lies there (or zero beyond the allocation) and only feed output
//     elements that are never stored.
//   * Reduction-contiguous operands are kept as [rows][64] (128-byte rows);
//     each MFMA fragment (8 consecutive reduction values of one row per lane)
//     is one ds_read_b128.  The 16-byte chunks of a row are XOR-permuted by
//     (row >> 1) & 7 so the 16 rows read in one LDS pass hit distinct banks.
//   * Row-contiguous operands (reduction index strided in memory) are kept as
//     [64][rows] and read with two ds_read_b64_tr_b16, which hand each lane
//     4 consecutive reduction values of one row; the chunks of each reduction
//     row are XOR-permuted so the 4 rows read together hit distinct banks.
//   * A ring of NS LDS stages (as many as fit, at most 4): the copies of the
//     next stages are in flight while one stage is multiplied; one workgroup
//     barrier per stage.  MFMA fragments are read three 16-deep steps ahead of
//     their use (a ring of four register sets), spread between the MFMAs.
#pragma once

#include "mfma_kernel.hpp"

#define BI_LDS __attribute__((address_space(3)))

namespace bi {
namespace mfma {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// byte offset that is past every operand buffer (operands are < 2^30 bytes)
constexpr uint32_t kOutOfRange = 0x80000000u;

// s_waitcnt with vmcnt = N and the other counters left alone
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// vmcnt(n * Q) for a run-time n in [0, 15] (a count above 63 is lowered to 63,
// which only waits longer)
template <int Q, int I = 0>
__device__ __forceinline__ void wait_vmcnt_stages(int n) {
    constexpr int C = I * Q < 63 ? I * Q : 63;
    if constexpr (I >= 15) {
        wait_vmcnt<C>();
    } else {
        if (n <= I) wait_vmcnt<C>();
        else wait_vmcnt_stages<Q, I + 1>(n);
    }
}

// LDS stages (sr = 128 bytes of every tile row each, or 256 for the
// double-depth variants of small tiles) for a BM x BN tile: as many as fit in
// 160 KB next to the bias row, at most 4 -- at most 8 for small tiles and 16
// for the 32 x 32 tile, whose stages are short and which need more of them in
// flight to keep memory busy (small-M shapes stream the whole of B through a
// few rows of A)
constexpr int dl_stages(int bm, int bn, int sr = 128) {
    const int per = sr * (bm + bn), avail = 160 * 1024 - 4 * bn;
    const int cap = bm + bn <= 64 ? 16 : bm + bn <= 128 ? 8 : 4;
    return avail / per >= cap ? cap : avail / per;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: 48-bit base, stride 0, `bytes` readable; loads at
// offsets >= bytes return zeros without touching memory.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, int64_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    return i32x4{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// buffer_load_dwordx4 ... lds: 16 bytes at `voff` of the buffer into LDS at
// `lds_addr` + 16 * lane.  Written as inline assembly so that the compiler does
// not treat it as an LDS store and wait for it before every later LDS read;
// the kernel orders these copies itself (s_waitcnt vmcnt + barrier).  M0
// carries the LDS address and is set right here; nothing else in the kernels
// keeps a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(i32x4 rs, uint32_t voff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(lds_addr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// XOR of the 16-byte chunk index inside a row of a reduction-contiguous tile
// (SR bytes per stage row).  A fragment read takes one chunk from each of 32
// consecutive rows; any 8 (and any 16) of those rows that the LDS serves
// together land on distinct banks (256-byte rows all start on bank 0, so the
// chunk turns with every row).  Depends on row & 15 only, so it is a per-lane
// constant for fragment reads.
template <int SR = 128>
__device__ __forceinline__ int rc_xor(int row) {
    if constexpr (SR >= 256) return row & 15;
    else return (row ^ ((row >> 3) & 1)) & 7;
}

// XOR of the 16-byte chunk index inside reduction row k of a row-contiguous
// tile of R columns.  A transposed fragment read takes 32 bytes (16 lanes) or
// 64 bytes (32 lanes) from each of 4 consecutive reduction rows; the XOR
// spreads those rows over distinct banks for either grouping, and it keeps
// the chunk inside the row (R/8 chunks: a multiple of 16 when R % 128 == 0,
// of 8 when R % 64 == 0).  When R is an odd multiple of 32 the row pitch is an
// odd multiple of 64 bytes, so 4 consecutive rows already start in the 4
// distinct 64-byte quarters of the 256-byte bank space: no XOR.  Depends on
// k & 3 only.
template <int R>
__device__ __forceinline__ int rs_xor(int k) {
    static_assert(R % 32 == 0, "row-contiguous tiles need a multiple of 32 columns");
    const int t = k & 3;
    if constexpr (R % 128 == 0) return 4 * t + 2 * (t >> 1);
    else if constexpr (R % 64 == 0) return 2 * t;
    else return 0;
}

// Per data type: bytes per element, reduction values per MFMA step and the
// MFMA fragment of one lane as read from LDS; a stage row of SR bytes (a
// reduction-contiguous tile row; SR / 2 reduction rows of a row-contiguous one)
// holds KPS = SR / ESZ reduction values, STEPS = KPS / STEPK steps.
template <int DT>
struct DlType {  // bf16 / f16: v_mfma_f32_32x32x16_{bf16,f16}, 16 values per step
    static constexpr int ESZ = 2, STEPK = 16;
    using Frag = u32x4;
};
// fp8 e4m3 codes of the exact path: one lane's 16 codes (one 16-byte LDS read)
struct E4m3x16 {
    u32x4 v;
};
// ... widened exactly to bf16: the operands of two MFMA steps
struct Bf16x8Pair {
    u32x4 lo, hi;
};
template <>
struct DlType<DT_E4M3> {  // fp8 e4m3 codes widened exactly to bf16: two
    // v_mfma_f32_32x32x16_bf16 per 32-deep step.  Lane half h reads the 16
    // codes 32t + 16h .. 32t + 16h + 15 of step t; the first MFMA takes codes
    // 0..7 of each half (reduction indices 32t + 0..7 and 32t + 16..23), the
    // second codes 8..15 (32t + 8..15 and 32t + 24..31)
    static constexpr int ESZ = 1, STEPK = 32;
    using Frag = E4m3x16;
};
template <>
struct DlType<DT_E4M3_FAST> {  // fp8 e4m3: v_mfma_scale_f32_32x32x64_f8f6f4, 64 per step
    static constexpr int ESZ = 1, STEPK = 64;
    using Frag = i32x8;
};

// One MFMA step, B fragment first (each lane then holds 4 consecutive output
// columns of one row).  e4m3 fragments of the exact path arrive here already
// widened to bf16 (a pair: two MFMA steps, first codes 0..7 of each lane, then
// codes 8..15).
template <int DT>
__device__ __forceinline__ f32x16 dl_mfma(u32x4 b, u32x4 a, f32x16 c) {
    return mfma_step<DT>(b, a, c);
}
template <int DT>
__device__ __forceinline__ f32x16 dl_mfma(Bf16x8Pair b, Bf16x8Pair a, f32x16 c) {
    c = mfma_step<DT_BF16>(b.lo, a.lo, c);
    return mfma_step<DT_BF16>(b.hi, a.hi, c);
}
template <int DT>
__device__ __forceinline__ f32x16 dl_mfma(i32x8 b, i32x8 a, f32x16 c) {
    // format codes 0 / 0: both operands OCP fp8 e4m3; no block scales
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 0, 0, 0, 0, 0, 0);
}
// fragment as the MFMA takes it: e4m3 codes of the exact path widened to bf16
__device__ __forceinline__ Bf16x8Pair dl_operand(E4m3x16 f) {
    return Bf16x8Pair{e4m3x8_to_bf16x8(u32x2{f.v[0], f.v[1]}),
                      e4m3x8_to_bf16x8(u32x2{f.v[2], f.v[3]})};
}
__device__ __forceinline__ u32x4 dl_operand(u32x4 f) { return f; }
__device__ __forceinline__ i32x8 dl_operand(i32x8 f) { return f; }

// Global -> LDS copy of one operand tile per stage (SR bytes of each row or,
// row-contiguous, SR / 2 reduction rows): R * SR / 1024 instructions of 1 KB,
// spread evenly over the NW waves.  ESZ: bytes per element.
template <int R, bool RC, int NW, int ESZ = 2, int SR = 128>
struct DLoad {
    static constexpr int NQ = R * SR / 1024 / NW;
    static constexpr int CPR = SR / 16;  // 16-byte chunks per reduction-contiguous row
    static_assert(NQ >= 1 && NQ * 1024 * NW == R * SR, "tile rows must spread evenly over the waves");
    uint32_t off[NQ];  // byte offset of this lane's chunk in stage 0
    int kin[NQ];       // reduction index of the chunk within its stage
    uint32_t sstride;  // bytes between consecutive stages

    // `o0`: first row (RC) or column (row-contiguous) of the tile
    __device__ __forceinline__ void init(int64_t ld, int64_t o0, int64_t r_begin, int wave,
                                         int lane) {
#pragma unroll
        for (int p = 0; p < NQ; ++p) {
            const int s = 64 * (wave + NW * p) + lane;  // chunk slot within the stage
            if constexpr (RC) {
                const int row = s / CPR, kg = (s % CPR) ^ rc_xor<SR>(row);
                off[p] = (uint32_t)(((o0 + row) * ld + r_begin) * ESZ + 16 * kg);
                kin[p] = (16 / ESZ) * kg;
            } else {
                static_assert(RC || ESZ == 2, "row-contiguous tiles are 16-bit");
                const int k = s / (R / 8), c = (s % (R / 8)) ^ rs_xor<R>(k);
                off[p] = (uint32_t)(((r_begin + k) * ld + o0 + 8 * c) * 2);
                kin[p] = k;
            }
        }
        sstride = RC ? (uint32_t)SR : (uint32_t)(SR / 2 * ld * 2);
    }

    // copy stage s into `stage`; with MASK, chunks at reduction index >= rem
    // (counted from the stage start) read as zeros
    template <bool MASK>
    __device__ __forceinline__ void issue(i32x4 rs, BI_LDS char *stage, int s, int64_t rem,
                                          int wave) const {
#pragma unroll
        for (int p = 0; p < NQ; ++p) {
            uint32_t o = off[p] + (uint32_t)s * sstride;
            if (MASK && kin[p] >= rem) o = kOutOfRange;
            lds_dma16(rs, o, (uint32_t)reinterpret_cast<uintptr_t>(stage + 1024 * (wave + NW * p)));
        }
    }

    // copy p (< NQ) of stage s alone, masked as above
    __device__ __forceinline__ void issue_one(i32x4 rs, BI_LDS char *stage, int s, int64_t rem,
                                              int wave, int p) const {
        uint32_t o = off[p] + (uint32_t)s * sstride;
        if (kin[p] >= rem) o = kOutOfRange;
        lds_dma16(rs, o, (uint32_t)reinterpret_cast<uintptr_t>(stage + 1024 * (wave + NW * p)));
    }
};

// MFMA fragment reads from a reduction-contiguous stage ([rows][SR bytes]).
// 16-bit: lane l takes 16 bytes (8 values) of row l & 31 at value 8 * (l >> 5)
// of the 16-deep step; e4m3 (exact path): 16 bytes (16 codes) at value
// 16 * (l >> 5) of the 32-deep step; e4m3 (fast path): 32 bytes (two chunks)
// at value 32 * (l >> 5) of the 64-deep step.
template <int DT, int SR = 128>
struct RcFrag {
    static constexpr int CH = DT == DT_E4M3_FAST ? 2 : 1;  // reads per lane and step
    static constexpr int STEPS = SR / DlType<DT>::ESZ / DlType<DT>::STEPK;  // steps per stage
    uint32_t koff[STEPS][CH];  // lane's byte offsets inside a 32-row block

    __device__ __forceinline__ void init(int lane) {
        const int r = lane & 31, hi = lane >> 5;
#pragma unroll
        for (int kk = 0; kk < STEPS; ++kk)
#pragma unroll
            for (int c = 0; c < CH; ++c)
                koff[kk][c] =
                    (uint32_t)(r * SR + 16 * ((2 * CH * kk + CH * hi + c) ^ rc_xor<SR>(r)));
    }
    // rows base .. base+31 (base a multiple of 32)
    __device__ __forceinline__ auto read(const BI_LDS char *stage, int base, int kk) const {
        const BI_LDS char *row = stage + base * SR;
        if constexpr (DT == DT_E4M3) {
            return E4m3x16{*reinterpret_cast<const BI_LDS u32x4 *>(row + koff[kk][0])};
        } else if constexpr (CH == 1) {
            return *reinterpret_cast<const BI_LDS u32x4 *>(row + koff[kk][0]);
        } else {
            const u32x4 lo = *reinterpret_cast<const BI_LDS u32x4 *>(row + koff[kk][0]);
            const u32x4 hi = *reinterpret_cast<const BI_LDS u32x4 *>(row + koff[kk][1]);
            return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    }
};

// MFMA fragment reads from a row-contiguous stage ([64][R]) with transposed
// LDS reads: lane l gets row (l & 31), reduction values 8*(l >> 5) + 0..7.
template <int R>
struct RsFrag {
    static constexpr int PITCH = 2 * R;
    uint32_t lane_off;
    int hq;  // XOR of the 32-column block index for this lane's reduction rows

    __device__ __forceinline__ void init(int lane) {
        const int g = lane >> 4, j = lane & 15;
        const int kr = 8 * (g >> 1) + (j >> 2);      // first reduction row of the lane
        const int cl = 2 * (g & 1) + ((j & 3) >> 1);  // 16-byte chunk inside the 32 columns
        // physical chunk (4F + cl) ^ h = 4 (F ^ (h >> 2)) + (cl ^ (h & 3))
        const int h = rs_xor<R>(kr);
        hq = h >> 2;
        lane_off = (uint32_t)(kr * PITCH + 16 * (cl ^ (h & 3)) + 8 * (j & 1));
    }
    // columns 32F .. 32F+31
    __device__ __forceinline__ u32x4 read(const BI_LDS char *stage, int F, int kk) const {
        const BI_LDS char *a = stage + lane_off + kk * 16 * PITCH + 64 * (F ^ hq);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BI_LDS s16x4 *)a);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BI_LDS s16x4 *)(a + 4 * PITCH));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    }
};

template <bool RC, int R, int DT, int SR>
struct FragOf {
    using type = RsFrag<R>;
};
template <int R, int DT, int SR>
struct FragOf<true, R, DT, SR> {
    using type = RcFrag<DT, SR>;
};

// Tiles of one to four MFMA waves (burst copies) get DL_NPW extra waves that
// issue all the copies: the MFMA waves then only read fragments, multiply and
// meet at the stage barriers, and the copies of a stage are split over four
// waves, so four times as many stages can be in flight under each wave's
// 63-load counter.  A copy wave that shares a SIMD with an MFMA wave halves that
// wave's register budget, so four-MFMA-wave tiles qualify only with wave tiles
// of at most 96 accumulator registers (e.g. 64x96); eight-wave tiles keep their
// copies for the same reason.
constexpr bool dl_producer(int nw, bool spread, int wtm, int wtn) {
    return !spread && nw >= 1 && nw <= 4 && (nw < 4 || wtm * wtn / 64 <= 96);
}
constexpr int DL_NPW = 4;
constexpr int dl_threads(int nw, bool spread, int wtm, int wtn) {
    return 64 * (nw + (dl_producer(nw, spread, wtm, wtn) ? DL_NPW : 0));
}

// Segment-anchored tile grid (MODE_SEGMENTS) of BM x BNB tiles whose slots from
// s1 on run as two BM x (BNB / 2) column halves each: half-tile workgroup u
// takes half (u / 8) & 1 of slot s1 + 8 * (u / 16) + u % 8, so both halves of
// a slot run on that slot's XCD (s1 a multiple of 8).  A half past the last
// column, or of a slot past the grid, has nothing to do.
template <int MODE, int BM, int BNB, int NTH>
__host__ __device__ __forceinline__ TileInfo decode_half_tile(const MfmaArgs &p, int t, int64_t u,
                                                              int64_t s1) {
    static_assert(MODE == MODE_SEGMENTS, "column halves of the segment grid");
    constexpr int BNH = BNB / 2;
    const int64_t xcd = u % 8, v = u / 8, h = v & 1;
    TileInfo ti = decode_tile_at<MODE, BM, BNB, NTH>(p, t, s1 + 8 * (v >> 1) + xcd, 0, h * BNH, BNH);
    if (!ti.skip) {
        ti.col0 += h * BNH;
        if (ti.col0 >= p.cols) ti.skip = true;
    }
    return ti;
}

// First workgroup of the column halves in a split launch of `nslots` segment
// slots over `cus` workgroups per round, for `work` working slots (expert row
// tiles x column tiles): F = work rounded down to whole rounds when the work
// left over is more than none and at most half a round, else nslots (every
// slot whole).
__host__ __device__ constexpr int64_t split_first_half(int64_t work, int64_t nslots, int64_t cus) {
    return work / cus > 0 && work % cus > 0 && 2 * (work % cus) <= cus ? work / cus * cus
                                                                        : nslots;
}

// LDS ring bytes of a BM x BN tile with ns stages (0: dl_stages) of sr-byte
// rows; the epilogue reuses them
constexpr int dl_lds_bytes(int bm, int bn, int ns = 0, int sr = 128) {
    return (ns > 0 ? ns : dl_stages(bm, bn, sr)) * sr * (bm + bn);
}

// One workgroup's tile: workgroup `blk` of `nblk`, LDS ring `lds_raw`
// (dl_lds_bytes(BM, BN, NSV)) and bias row `lds_bias` ([BN]) owned by the
// caller, threadIdx.x below dl_threads(...).  NSV: ring stages (0: as many as
// fit, dl_stages); fewer leave room for a second workgroup on the CU.
// HALF_OF > 0: the tile is a column half of the BM x HALF_OF segment grid
// (decode_half_tile, with `blk` the half-tile index and `nblk` the first split
// slot).
template <int DT, bool A_RC, bool B_RC, int BM, int BN, int WGM, int WGN, int EPI, int MODE,
          bool SPREAD, int NSV = 0, int SR = 128, int HALF_OF = 0>
__device__ __forceinline__ void dl_body(const MfmaArgs &p, char *lds_raw, float *lds_bias,
                                        int64_t blk, int64_t nblk) {
    constexpr int NW = WGM * WGN;
    constexpr bool PROD = dl_producer(NW, SPREAD, BM / WGM, BN / WGN);
    constexpr int NTH = dl_threads(NW, SPREAD, BM / WGM, BN / WGN);
    constexpr int NWC = PROD ? DL_NPW : NW;  // waves that issue the copies
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    static_assert(FM * 32 == WTM && FN * 32 == WTN, "wave tile must be a multiple of 32");
    constexpr int SA = SR * BM, SB = SR * BN;  // bytes of one stage of A / B
    constexpr int NS = NSV > 0 ? NSV : dl_stages(BM, BN, SR);
    static_assert(NS >= 2 && NS <= 16, "two to sixteen stages");
    using TY = DlType<DT>;
    constexpr int KPS = SR / TY::ESZ, STEPS = KPS / TY::STEPK;
    static_assert(SR == 128 || SR == 256 || SR == 512, "stage rows of 128, 256 or 512 bytes");
    static_assert(STEPS >= 2, "two or more MFMA steps per stage");
    using Frag = typename TY::Frag;
    constexpr bool FP8 = DT == DT_E4M3 || DT == DT_E4M3_FAST;
    static_assert(!FP8 || (A_RC && B_RC), "fp8 operands are reduction-contiguous");
    static_assert(slab_bytes<EPI, WTN, NW>() <= NS * (SA + SB), "epilogue slabs fit in the stages");
    static_assert((EPI != EPI_ROUND && EPI != EPI_SCALE) || BN <= 64 * NW,
                  "one thread per bias column");

    const int t = threadIdx.x;
    const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WGN, wn = wave % WGN;

    static_assert(HALF_OF == 0 || HALF_OF == 2 * BN, "halves of a tile twice as wide");
    TileInfo ti;
    if constexpr (HALF_OF > 0) ti = decode_half_tile<MODE, BM, HALF_OF, NTH>(p, t, blk, nblk);
    else ti = decode_tile_at<MODE, BM, BN, NTH>(p, t, blk, nblk);
    const bool is_prod = PROD && wave >= NW;
    // index of this wave among the copying waves
    const int cwave = PROD ? (is_prod ? wave - NW : 0) : wave;
    if (ti.skip) return;
    const int64_t row0 = ti.row0, col0 = ti.col0;
    const float bias_v = fetch_bias<DT, EPI, BN>(p, col0, t);
    const int64_t r_begin = ti.r_begin, r_end = ti.r_end;

    const i32x4 rsa = make_rsrc(p.a, p.a_bytes);
    const i32x4 rsb = make_rsrc(static_cast<const uint16_t *>(p.b) + ti.b_off, p.b_bytes - 2 * ti.b_off);
    using LA = DLoad<BM, A_RC, NWC, TY::ESZ, SR>;
    using LB = DLoad<BN, B_RC, NWC, TY::ESZ, SR>;
    LA la;
    LB lb;
    la.init(p.lda, row0, r_begin, cwave, lane);
    lb.init(p.ldb, col0, r_begin, cwave, lane);
    typename FragOf<A_RC, BM, DT, SR>::type ra;
    typename FragOf<B_RC, BN, DT, SR>::type rb;
    ra.init(lane);
    rb.init(lane);

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const int64_t red = r_end - r_begin;
    const int nst = (int)((red + KPS - 1) / KPS);
    BI_LDS char *ring = (BI_LDS char *)lds_raw;

    auto issue = [&](int s) {
        BI_LDS char *da = ring + (s % NS) * (SA + SB);
        BI_LDS char *db = da + SA;
        const int64_t rem = red - (int64_t)KPS * s;
        if (rem >= KPS) {
            la.template issue<false>(rsa, da, s, rem, cwave);
            lb.template issue<false>(rsb, db, s, rem, cwave);
        } else {
            la.template issue<true>(rsa, da, s, rem, cwave);
            lb.template issue<true>(rsb, db, s, rem, cwave);
        }
    };
    auto frag_a = [&](const BI_LDS char *st, int i, int kk) {
        if constexpr (A_RC) return ra.read(st, wm * WTM + 32 * i, kk);
        else return ra.read(st, (wm * WTM) / 32 + i, kk);
    };
    auto frag_b = [&](const BI_LDS char *st, int j, int kk) {
        if constexpr (B_RC) return rb.read(st, wn * WTN + 32 * j, kk);
        else return rb.read(st, (wn * WTN) / 32 + j, kk);
    };

    // Fragment ring: set kk holds the fragments of step kk of the stage being
    // multiplied or of the next one.  Fragments are read STEPS - 1 steps ahead
    // of their MFMAs, interleaved with the MFMAs of the current step.
    Frag fa[STEPS][FM], fb[STEPS][FN];
    auto read_step = [&](const BI_LDS char *st, int kk, int set) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[set][i] = frag_a(st, i, kk);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[set][j] = frag_b(st + SA, j, kk);
    };
    // every fragment of a set as the MFMA takes it (e4m3 codes of the exact path
    // are widened once per fragment, not once per MFMA)
    using Op = decltype(dl_operand(Frag{}));
    auto mfma_step_all = [&](int set) {
        Op ob[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) ob[j] = dl_operand(fb[set][j]);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const Op oa = dl_operand(fa[set][i]);
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = dl_mfma<DT>(ob[j], oa, acc[i][j]);
        }
    };
    constexpr int RCR = DT == DT_E4M3_FAST ? 2 : 1;  // LDS reads per reduction-contiguous fragment
    constexpr int NREAD = FM * (A_RC ? RCR : 2) + FN * (B_RC ? RCR : 2);  // per step
    constexpr int NMFMA = FM * FN;
    constexpr int MPC = DT == DT_E4M3 ? 2 : 1;  // MFMA instructions per dl_mfma
    // LDS reads of `sets` steps spread between the MFMAs of one step
    auto interleave = [&](auto sets_tag) {
        constexpr int PER = (decltype(sets_tag)::value * NREAD + NMFMA - 1) / NMFMA;
#pragma unroll
        for (int q = 0; q < NMFMA; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, MPC, 0);  // one dl_mfma
            __builtin_amdgcn_sched_group_barrier(0x100, PER, 0);  // then LDS reads
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // Schedule per stage s (buffer s % NS).  The workgroup barrier that hands
    // buffer s to the copies of stage s+NS and makes stage s+1 visible comes
    // after MFMA step BAR; the last reads of buffer s (step STEPS-1, issued at
    // step 0) then have a step of MFMAs to complete before the barrier waits
    // for them.
    //   step 0:             read step STEPS-1 of stage s, multiply step 0
    //   steps 1..BAR:       multiply
    //   barrier:            wait until stage s+1 has landed; barrier; copies of
    //                       stage s+NS into buffer s
    //   steps BAR+1..:      read steps 0..STEPS-2 of stage s+1 (step kk reads
    //                       sets first(kk) .. first(kk+1)-1), multiply step kk
    // The reads of stage s+1 are issued also after the last stage (from a
    // buffer holding older data, never used) so that they need no branch and
    // interleave freely with the MFMAs.  SPREAD: per MFMA of steps BAR+1..,
    // its share of the reads, the MFMA, its share of the copies of stage s+NS
    // (a burst of copy instructions can hold up the wave's MFMA issue while
    // the memory pipeline takes them in).
    constexpr int BAR = STEPS >= 4 ? 1 : 0;
    auto first_set = [](int kk) { return kk <= BAR + 1 ? 0 : kk - 1; };
    constexpr int NC = LA::NQ + LB::NQ;                 // copies per wave per stage
    constexpr int NSLOT = (STEPS - 1 - BAR) * NMFMA;     // MFMAs after the barrier
    constexpr int CPS = (NC + NSLOT - 1) / NSLOT;        // copies after each of them
    auto copy_one = [&](int cs, int c) {
        BI_LDS char *da = ring + (cs % NS) * (SA + SB);
        const int64_t rem = red - (int64_t)KPS * cs;
        if (c < LA::NQ) la.issue_one(rsa, da, cs, rem, cwave, c);
        else lb.issue_one(rsb, da + SA, cs, rem, cwave, c - LA::NQ);
    };

    if (!PROD || is_prod) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
            if (s < nst) issue(s);
    }
    if (nst > 0) {
        // issued: stages 0 .. min(NS-1, nst-1); wait for stage 0
        const int later = nst - 1 < NS - 1 ? nst - 1 : NS - 1;
        if (!PROD || is_prod) wait_vmcnt_stages<LA::NQ + LB::NQ>(later);
        __syncthreads();
        if (!is_prod) {
#pragma unroll
            for (int kk = 0; kk < STEPS - 1; ++kk) read_step(ring, kk, kk);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (is_prod) {
        // the copy wave: one barrier per stage, like the MFMA waves, and the
        // epilogue's barrier
        for (int s = 0; s + 1 < nst; ++s) {
            const int later = nst - 2 - s < NS - 2 ? nst - 2 - s : NS - 2;
            wait_vmcnt_stages<LA::NQ + LB::NQ>(later);
            __syncthreads();
            if (s + NS < nst) issue(s + NS);
        }
        __syncthreads();
        return;
    }
    for (int s = 0; s < nst; ++s) {
        const BI_LDS char *cur = ring + (s % NS) * (SA + SB);
        const BI_LDS char *nxt = ring + ((s + 1) % NS) * (SA + SB);
        read_step(cur, STEPS - 1, STEPS - 1);
        mfma_step_all(0);
        interleave(std::integral_constant<int, 1>{});
#pragma unroll
        for (int kk = 1; kk <= BAR; ++kk) {
            mfma_step_all(kk);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (s + 1 < nst) {
            // issued so far: stages 0 .. min(s+NS-1, nst-1); stage s+1 has
            // landed once only the copies of the stages after it are pending
            const int later = nst - 2 - s < NS - 2 ? nst - 2 - s : NS - 2;
            if (!PROD) wait_vmcnt_stages<LA::NQ + LB::NQ>(later);
            __syncthreads();
            if (!PROD && !SPREAD && s + NS < nst) issue(s + NS);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!SPREAD || PROD) {
#pragma unroll
            for (int kk = BAR + 1; kk < STEPS; ++kk) {
#pragma unroll
                for (int x = first_set(kk); x < first_set(kk + 1); ++x) read_step(nxt, x, x);
                mfma_step_all(kk);
                if (kk == BAR + 1) interleave(std::integral_constant<int, BAR + 1>{});
                else interleave(std::integral_constant<int, 1>{});
            }
        } else {
            const bool copies = s + NS < nst;
#pragma unroll
            for (int kk = BAR + 1; kk < STEPS; ++kk) {
                const int x0 = first_set(kk), nx = first_set(kk + 1) - x0;
                Op oa[FM], ob[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i) oa[i] = dl_operand(fa[kk][i]);
#pragma unroll
                for (int j = 0; j < FN; ++j) ob[j] = dl_operand(fb[kk][j]);
#pragma unroll
                for (int q = 0; q < NMFMA; ++q) {
                    // fragments (set x0 + f / (FM+FN), index f % (FM+FN)) with f = q mod NMFMA
#pragma unroll
                    for (int f = q; f < nx * (FM + FN); f += NMFMA) {
                        const int x = x0 + f / (FM + FN), g = f % (FM + FN);
                        if (g < FM) fa[x][g] = frag_a(nxt, g, x);
                        else fb[x][g - FM] = frag_b(nxt + SA, g - FM, x);
                    }
                    acc[q / FN][q % FN] =
                        dl_mfma<DT>(ob[q % FN], oa[q / FN], acc[q / FN][q % FN]);
                    if (copies) {
                        const int c0 = ((kk - BAR - 1) * NMFMA + q) * CPS;
#pragma unroll
                        for (int c = c0; c < c0 + CPS; ++c)
                            if (c < NC) copy_one(s + NS, c);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }

    write_tile<DT, EPI, WTM, WTN, FM, FN, BN>(p, ti, acc, lds_raw, lds_bias, bias_v, wave, wm, wn,
                                              lane);
}

template <int DT, bool A_RC, bool B_RC, int BM, int BN, int WGM, int WGN, int EPI, int MODE,
          bool SPREAD, int SR = 128>
__global__ __launch_bounds__(dl_threads(WGM * WGN, SPREAD, BM / WGM, BN / WGN)) void mfma_dl_kernel(
    MfmaArgs p) {
    // NS stages of [A | B]; reused by the epilogue
    __shared__ __align__(1024) char lds_raw[dl_lds_bytes(BM, BN, 0, SR)];
    __shared__ __align__(16) float lds_bias[BN];
    dl_body<DT, A_RC, B_RC, BM, BN, WGM, WGN, EPI, MODE, SPREAD, 0, SR>(p, lds_raw, lds_bias,
                                                                         blockIdx.x, gridDim.x);
}

template <int DT, bool ARC, bool BRC, int EPI, int MODE, int ID, bool SPREAD, int SR = 128>
hipError_t launch_dl_tile(const MfmaArgs &p, int64_t grid, hipStream_t s) {
    using T = TileOf<ID>;
    hipLaunchKernelGGL(
        (mfma_dl_kernel<DT, ARC, BRC, T::BM, T::BN, T::WGM, T::WGN, EPI, MODE, SPREAD, SR>),
        dim3(grid), dim3(dl_threads(T::WGM * T::WGN, SPREAD, T::BM / T::WGM, T::BN / T::WGN)), 0, s, p);
    return hipGetLastError();
}

// tile id of the direct-load kernel on base tile `base`: 40 + base for bases
// 1..19, 100 + base for bases 20..39
constexpr int dl_id(int base) { return base < 20 ? 40 + base : 100 + base; }

// tile ids dl_id(base) select the direct-load kernel with base tile `base`
template <int DT, bool ARC, bool BRC, int EPI, int MODE, int... IDS>
hipError_t launch_dl_among(const MfmaArgs &p, int tile_id, int64_t grid, hipStream_t s) {
    hipError_t r = hipErrorInvalidValue;
    ((tile_id == dl_id(IDS)
          ? (void)(r = launch_dl_tile<DT, ARC, BRC, EPI, MODE, IDS, false>(p, grid, s))
          : (void)0),
     ...);
    return r;
}

// tile ids 100 + base id (bases 1..19): the same kernel with the copies spread
// between MFMAs
template <int DT, bool ARC, bool BRC, int EPI, int MODE, int... IDS>
hipError_t launch_dls_among(const MfmaArgs &p, int tile_id, int64_t grid, hipStream_t s) {
    static_assert(((IDS < 20) && ...), "spread variants exist for bases 1..19");
    hipError_t r = hipErrorInvalidValue;
    ((tile_id == 100 + IDS
          ? (void)(r = launch_dl_tile<DT, ARC, BRC, EPI, MODE, IDS, true>(p, grid, s))
          : (void)0),
     ...);
    return r;
}

// tile ids 200 + base id (SR = 256) and 300 + base id (SR = 512), bases
// 20..39: the direct-load kernel with double- and quadruple-depth stages (256-
// and 512-byte stage rows), a half and a quarter as many stage barriers per
// reduction -- for the small tiles of small batches, whose time per stage is
// mostly fixed cost
template <int DT, bool ARC, bool BRC, int EPI, int MODE, int SR, int... IDS>
hipError_t launch_dld_among(const MfmaArgs &p, int tile_id, int64_t grid, hipStream_t s) {
    static_assert(((IDS >= 20) && ...), "deep-stage variants exist for bases 20..39");
    static_assert(SR == 256 || SR == 512, "double- or quadruple-depth stages");
    constexpr int OFF = SR == 256 ? 200 : 300;
    hipError_t r = hipErrorInvalidValue;
    ((tile_id == OFF + IDS
          ? (void)(r = launch_dl_tile<DT, ARC, BRC, EPI, MODE, IDS, false, SR>(p, grid, s))
          : (void)0),
     ...);
    return r;
}

}  // namespace mfma
}  // namespace bi
