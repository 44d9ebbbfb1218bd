// MFMA tier for bf16 / f16 operands on gfx950 (sgemm-bi PyPI page,
// "Determinism contracts": tensor-core tier with f32 accumulation, bit-identical
// across runs, forward strictly batch-invariant across all M, several tile
// families giving the same bits).
//
// One kernel template serves the linear forward, dX, dW (and pass 1 of the
// chunked dW), and the grouped forward / dinput / dweights (rublas
// tensor_grouped/mod.rs).  It computes C(i,j) = sum_r A(i,r) B(j,r) with:
//   * v_mfma_f32_32x32x16_{bf16,f16} as the only arithmetic on the reduction:
//     each output element's accumulator starts at +0 and receives one MFMA per
//     16-deep reduction step, steps in ascending order from the start of the
//     reduction range.  Neither the tile shape nor the element's position in
//     its tile changes that sequence, so all tile shapes give the same bits and
//     a row's bits never depend on the number of rows (M).
//   * 64-deep reduction slices staged global -> registers -> LDS with two LDS
//     buffers: while slice s is multiplied out of one buffer, slice s+1 (loaded
//     one slice earlier) is written to the other and slice s+2 is fetched from
//     global memory.  One workgroup barrier per slice.
//   * Interior tiles with full slices take a branch-free path of 16-byte vector
//     loads; edge tiles and the last partial slice take a branch-free masked
//     path (clamped addresses, zero-selected values), so no load waits on
//     another.
//   * LDS layout "k-grouped": for every group of 8 consecutive reduction
//     indices, each tile row owns one 16-byte slot holding those 8 values, so
//     an MFMA operand (8 consecutive reduction values of one row per lane) is a
//     single ds_read_b128.  Slots are XOR-swizzled within groups of 8 rows so
//     that the reads, the direct writes and the transposed writes spread over
//     the banks.
//   * Operands whose reduction index is contiguous in memory are copied as
//     16-byte vectors; operands whose reduction index is strided (W in the
//     forward, X and dY in dW, ...) are loaded as 8x8 element blocks and
//     transposed in registers before the LDS write.
//   * The MFMA is issued with the B fragment as its first operand, so each lane
//     ends up holding 4 consecutive output columns of one row: the epilogue
//     stores 8 bytes (bf16/f16) or 16 bytes (f32) per instruction.
//   * Workgroup ids are remapped so that the 32 CUs of one XCD work on one
//     compact block of output tiles and share operand rows in that XCD's L2.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace bi {

namespace mfma {

constexpr int BK = 64;      // reduction slice per LDS stage
constexpr int KG = BK / 8;  // 8-element groups per slice
constexpr int NT = 256;     // threads per workgroup (4 waves)

enum Mode : int { MODE_PLAIN = 0, MODE_SEGMENTS = 1, MODE_EXPERT_RED = 2 };
// EPI_SCALE: fp8 operands, RNE_bf16((acc * scale_a) * scale_b [+ bias])
enum Epi : int { EPI_ROUND = 0, EPI_PARTIAL = 1, EPI_F32 = 2, EPI_SCALE = 3 };

__device__ __forceinline__ int swz(int row, int kg) {
    return (row & ~7) | ((row ^ (row >> 3) ^ kg) & 7);
}

template <int DT>
__device__ __forceinline__ f32x16 mfma_step(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (DT == DT_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 pack8(const uint32_t e[8]) {
    return u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                 e[6] | (e[7] << 16)};
}

// Transpose an 8x8 block of 16-bit elements: in[r] holds row r (8 elements),
// out[c] receives column c (8 elements, row 0 in the low half of word 0).
__device__ __forceinline__ void transpose8x8(const u32x4 *in, u32x4 *out) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t lo = in[2 * d][c >> 1], hi = in[2 * d + 1][c >> 1];
            out[c][d] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                : ((lo & 0xffffu) | (hi << 16));
        }
    }
}

// Staging of one operand tile of R rows x BK reduction values.
//   RC = true : element (row, r) at p[row*ld + r]  (reduction-contiguous)
//   RC = false: element (row, r) at p[r*ld + row]  (row-contiguous)
template <int R, bool RC, int NTH = NT>
struct Stage {
    static constexpr int DIRECT = R * KG / NTH;              // RC: 16-byte chunks per thread
    static constexpr int UNITS = KG * (R / 8);              // !RC: 8x8 blocks per tile
    static constexpr int UNITS_PER_THREAD = (UNITS + NTH - 1) / NTH;
    static constexpr int NREG = RC ? DIRECT : UNITS_PER_THREAD * 8;
    static_assert(!RC || (R * KG) % NTH == 0, "tile rows must fill the workgroup");

    u32x4 reg[NREG];

    // All rows of the tile in range, the whole slice in range, 16-byte aligned
    // rows: unconditional vector loads.
    __device__ __forceinline__ void load_fast(const uint16_t *p, int64_t ld, int64_t row0,
                                              int64_t rk, int t) {
        if constexpr (RC) {
#pragma unroll
            for (int q = 0; q < DIRECT; ++q) {
                const int c = t + NTH * q;
                const int row = c / KG, kg = c % KG;
                reg[q] = *reinterpret_cast<const u32x4 *>(p + (row0 + row) * ld + rk + 8 * kg);
            }
        } else {
#pragma unroll
            for (int q = 0; q < UNITS_PER_THREAD; ++q) {
                int u = t + NTH * q;
                if (UNITS % NTH != 0 && u >= UNITS) u = UNITS - 1;  // duplicate, never stored
                const int kg = u / (R / 8), ib = u % (R / 8);
                const uint16_t *src = p + (rk + 8 * kg) * ld + row0 + 8 * ib;
#pragma unroll
                for (int rr = 0; rr < 8; ++rr)
                    reg[q * 8 + rr] = *reinterpret_cast<const u32x4 *>(src + rr * ld);
            }
        }
    }

    // Masked variant: rows [row0, row_end), reduction [rk, r_end); elements
    // outside are zero.  Addresses are clamped into range, so every load is
    // valid and none depends on a branch.
    __device__ __forceinline__ void load_masked(const uint16_t *p, int64_t ld, int64_t row0,
                                                int64_t row_end, int64_t rk, int64_t r_end,
                                                int t) {
        if constexpr (RC) {
#pragma unroll
            for (int q = 0; q < DIRECT; ++q) {
                const int c = t + NTH * q;
                const int row = c / KG, kg = c % KG;
                const int64_t gi = row0 + row;
                const int64_t gic = gi < row_end ? gi : row_end - 1;
                uint32_t e[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const int64_t gr = rk + 8 * kg + x;
                    const int64_t grc = gr < r_end ? gr : r_end - 1;
                    const uint32_t v = p[gic * ld + grc];
                    e[x] = (gi < row_end && gr < r_end) ? v : 0u;
                }
                reg[q] = pack8(e);
            }
        } else {
#pragma unroll
            for (int q = 0; q < UNITS_PER_THREAD; ++q) {
                int u = t + NTH * q;
                if (UNITS % NTH != 0 && u >= UNITS) u = UNITS - 1;
                const int kg = u / (R / 8), ib = u % (R / 8);
#pragma unroll
                for (int rr = 0; rr < 8; ++rr) {
                    const int64_t gr = rk + 8 * kg + rr;
                    const int64_t grc = gr < r_end ? gr : r_end - 1;
                    uint32_t e[8];
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        const int64_t gi = row0 + 8 * ib + x;
                        const int64_t gic = gi < row_end ? gi : row_end - 1;
                        const uint32_t v = p[grc * ld + gic];
                        e[x] = (gi < row_end && gr < r_end) ? v : 0u;
                    }
                    reg[q * 8 + rr] = pack8(e);
                }
            }
        }
    }

    __device__ __forceinline__ void load(const uint16_t *p, int64_t ld, int64_t row0,
                                         int64_t row_end, int64_t rk, int64_t r_end,
                                         bool interior, int t) {
        if (interior && rk + BK <= r_end) load_fast(p, ld, row0, rk, t);
        else load_masked(p, ld, row0, row_end, rk, r_end, t);
    }

    __device__ __forceinline__ void store(u32x4 *lds, int t) const {
        if constexpr (RC) {
#pragma unroll
            for (int q = 0; q < DIRECT; ++q) {
                const int c = t + NTH * q;
                const int row = c / KG, kg = c % KG;
                lds[kg * R + swz(row, kg)] = reg[q];
            }
        } else {
#pragma unroll
            for (int q = 0; q < UNITS_PER_THREAD; ++q) {
                const int u = t + NTH * q;
                if (UNITS % NTH != 0 && u >= UNITS) continue;
                const int kg = u / (R / 8), ib = u % (R / 8);
                u32x4 tr[8];
                transpose8x8(&reg[q * 8], tr);
#pragma unroll
                for (int c = 0; c < 8; ++c) lds[kg * R + swz(8 * ib + c, kg)] = tr[c];
            }
        }
    }
};

// Fast loads for interior tiles and full slices: a uniform (scalar) base
// pointer per slice plus one 32-bit byte offset per thread and load, fixed for
// the whole reduction, so address arithmetic stays out of the main loop.
template <int R, bool RC, int NTH = NT>
struct FastAddr {
    static constexpr int NOFF = RC ? Stage<R, RC, NTH>::DIRECT : Stage<R, RC, NTH>::UNITS_PER_THREAD;
    uint32_t off[NOFF];

    __device__ __forceinline__ void init(int64_t ld, int t) {
#pragma unroll
        for (int q = 0; q < NOFF; ++q) {
            if constexpr (RC) {
                const int c = t + NTH * q;
                off[q] = (uint32_t)(((c / KG) * ld + 8 * (c % KG)) * 2);
            } else {
                int u = t + NTH * q;
                if (Stage<R, RC, NTH>::UNITS % NTH != 0 && u >= Stage<R, RC, NTH>::UNITS)
                    u = Stage<R, RC, NTH>::UNITS - 1;
                const int kg = u / (R / 8), ib = u % (R / 8);
                off[q] = (uint32_t)(((int64_t)8 * kg * ld + 8 * ib) * 2);
            }
        }
    }
    // slice base: element (row0, rk) for RC, element (rk, row0) otherwise
    __device__ __forceinline__ void load(Stage<R, RC, NTH> &st, const uint16_t *p, int64_t ld,
                                         int64_t row0, int64_t rk) const {
        if constexpr (RC) {
            const char *base = reinterpret_cast<const char *>(p + row0 * ld + rk);
#pragma unroll
            for (int q = 0; q < NOFF; ++q)
                st.reg[q] = *reinterpret_cast<const u32x4 *>(base + off[q]);
        } else {
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const char *base = reinterpret_cast<const char *>(p + (rk + rr) * ld + row0);
#pragma unroll
                for (int q = 0; q < NOFF; ++q)
                    st.reg[q * 8 + rr] = *reinterpret_cast<const u32x4 *>(base + off[q]);
            }
        }
    }
};

// 32-bit offsets cover the whole tile of one slice
template <int R, bool RC>
__device__ __forceinline__ bool offsets_fit(int64_t ld) {
    const int64_t span = RC ? ((int64_t)(R - 1) * ld + BK) * 2 : ((int64_t)(BK - 1) * ld + R) * 2;
    return span < ((int64_t)1 << 31);
}

template <int DT, int BM, int BN, int WTM, int WTN, int FM, int FN>
struct Compute {
    u32x4 fa[2][FM], fb[2][FN];

    // fragments of the first 16-deep step of a slice
    __device__ __forceinline__ void first(const u32x4 *la, const u32x4 *lb, int wm, int wn,
                                          int lrow, int lkg) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[0][i] = la[lkg * BM + swz(wm * WTM + 32 * i + lrow, lkg)];
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[0][j] = lb[lkg * BN + swz(wn * WTN + 32 * j + lrow, lkg)];
    }

    // multiply one LDS slice into the accumulators (first() already issued):
    // four 16-deep steps in ascending order; the fragments of step kk+1 are
    // read while step kk's MFMAs run
    __device__ __forceinline__ void rest(const u32x4 *la, const u32x4 *lb, f32x16 (&acc)[FM][FN],
                                         int wm, int wn, int lrow, int lkg) {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int cur = kk & 1;
            if (kk + 1 < BK / 16) {
                const int kg = 2 * (kk + 1) + lkg;
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    fa[cur ^ 1][i] = la[kg * BM + swz(wm * WTM + 32 * i + lrow, kg)];
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    fb[cur ^ 1][j] = lb[kg * BN + swz(wn * WTN + 32 * j + lrow, kg)];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = mfma_step<DT>(fb[cur][j], fa[cur][i], acc[i][j]);
        }
    }

    __device__ __forceinline__ void run(const u32x4 *la, const u32x4 *lb, f32x16 (&acc)[FM][FN],
                                        int wm, int wn, int lrow, int lkg) {
        first(la, lb, wm, wn, lrow, lkg);
        rest(la, lb, acc, wm, wn, lrow, lkg);
    }
};

// Position of one workgroup's tile: output rows [row0, row_end), columns from
// col0, reduction range [r_begin, r_end), dW chunk index, offset of the output
// (grouped dweights) and of B (grouped expert).  `skip` = nothing to multiply
// (beyond the last segment tile, or a padding tile that was zero-filled here).
struct TileInfo {
    int64_t row0, row_end, col0, r_begin, r_end, chunk, c_off, b_off;
    bool skip;
};

// Workgroup `blk` of `nblk` (blockIdx.x and gridDim.x for a launch of its own;
// an offset index where one launch carries the tiles of two products).  A
// padding tile of MODE_SEGMENTS zero-fills columns col0 + fill_off ..
// col0 + fill_off + fill_w - 1 (fill_w < 0: the whole tile width).
template <int MODE, int BM, int BN, int NTH = NT>
__host__ __device__ __forceinline__ TileInfo decode_tile_at(const MfmaArgs &p, int t, int64_t blk,
                                                   int64_t nblk, int64_t fill_off = 0,
                                                   int64_t fill_w = -1) {
    TileInfo ti{};
    ti.skip = false;
    if constexpr (MODE == MODE_PLAIN) {
        const int64_t tiles = p.tiles_i * p.tiles_j;
        const int64_t bid = xcd_remap(blk, nblk);
        ti.chunk = bid / tiles;
        const int64_t tile = bid % tiles;
        // groups of 4 row-tiles, column-major inside a group
        constexpr int64_t GROUP = 4;
        const int64_t per_group = GROUP * p.tiles_j;
        const int64_t g = tile / per_group, first = g * GROUP;
        const int64_t gsz = p.tiles_i - first < GROUP ? p.tiles_i - first : GROUP;
        const int64_t in_g = tile % per_group;
        ti.row0 = (first + in_g % gsz) * BM;
        ti.col0 = (in_g / gsz) * BN;
        ti.row_end = p.rows;
        ti.r_begin = ti.chunk * p.chunk;
        ti.r_end = ti.r_begin + p.chunk < p.red ? ti.r_begin + p.chunk : p.red;
    } else if constexpr (MODE == MODE_SEGMENTS) {
        // Row tiles in groups of SEG_GROUP, each group with all its column
        // tiles on one XCD (workgroups go to XCD blk % 8), column-major inside
        // the group, groups dealt to the XCDs in turn: a group's row tiles of
        // the input are fetched once into that XCD's L2 and shared by its
        // column tiles, and the tiles past the last segment, whose count only
        // the device knows, skip evenly on every XCD.  The grid covers
        // seg_tiles rounded up to whole rounds of 8 groups (seg_grid_rows).
        const int64_t xcd = blk % 8, j = blk / 8, per = SEG_GROUP * p.tiles_j;
        const int64_t grp = (j / per) * 8 + xcd, q = j % per;
        const int64_t tt0 = grp * SEG_GROUP + q % SEG_GROUP;
        ti.col0 = (q / SEG_GROUP) * BN;
        if (tt0 >= p.seg_tiles) {
            ti.skip = true;
            return ti;
        }
        int64_t tt = tt0;
        int64_t x = 0;
        ti.row0 = -1;
        ti.row_end = 0;
        for (; x <= p.n_experts; ++x) {
            int64_t s = p.offsets[x < p.n_experts ? x : p.n_experts];
            int64_t e = x < p.n_experts ? (int64_t)p.offsets[x + 1] : p.rows;
            if (e > p.rows) e = p.rows;
            if (s > e) s = e;
            const int64_t cnt = (e - s + BM - 1) / BM;
            if (tt < cnt) {
                ti.row0 = s + tt * BM;
                ti.row_end = e;
                break;
            }
            tt -= cnt;
        }
        if (ti.row0 < 0) {  // beyond the last segment tile (whole workgroup)
            ti.skip = true;
            return ti;
        }
        if (x == p.n_experts) {
            // padding rows: exact +0 (rublas: ids outside [0,E) give zero rows)
            const int64_t r1 = ti.row0 + BM < ti.row_end ? ti.row0 + BM : ti.row_end;
            const int64_t fw = fill_w < 0 ? BN : fill_w, c0 = ti.col0 + fill_off;
            uint16_t *pc = static_cast<uint16_t *>(p.c);
            for (int64_t idx = t; idx < (r1 - ti.row0) * fw; idx += NTH) {
                const int64_t i = ti.row0 + idx / fw, j = c0 + idx % fw;
                if (j < p.cols) pc[i * p.ldc + j] = 0;
            }
            ti.skip = true;
            return ti;
        }
        ti.b_off = x * p.b_expert_stride;
        ti.r_begin = 0;
        ti.r_end = p.red;
    } else {  // MODE_EXPERT_RED
        // consecutive tiles (one expert's, in groups of 4 row tiles,
        // column-major inside a group) on one XCD, as for MODE_PLAIN
        const int64_t per_x = p.tiles_i * p.tiles_j;
        const int64_t bid = xcd_remap(blk, nblk);
        const int64_t x = bid / per_x;
        const int64_t tile = bid % per_x;
        constexpr int64_t GROUP = 4;
        const int64_t per_group = GROUP * p.tiles_j;
        const int64_t g = tile / per_group, first = g * GROUP;
        const int64_t gsz = p.tiles_i - first < GROUP ? p.tiles_i - first : GROUP;
        const int64_t in_g = tile % per_group;
        ti.row0 = (first + in_g % gsz) * BM;
        ti.col0 = (in_g / gsz) * BN;
        ti.row_end = p.rows;
        ti.r_end = p.red_offsets[x + 1];
        ti.r_begin = p.red_offsets[x];
        if (ti.r_end > p.red) ti.r_end = p.red;
        if (ti.r_begin > ti.r_end) ti.r_begin = ti.r_end;
        ti.c_off = x * p.c_expert_stride;
    }
    return ti;
}

template <int MODE, int BM, int BN, int NTH = NT>
__device__ __forceinline__ TileInfo decode_tile(const MfmaArgs &p, int t) {
    return decode_tile_at<MODE, BM, BN, NTH>(p, t, blockIdx.x, gridDim.x);
}

// The bias of this tile's columns as f32: thread t < BN fetches column t
// (clamped to the last column).  Fetched early into a register, written to
// LDS by the epilogue (write_tile), so its latency hides behind the K loop.
template <int DT, int EPI, int BN>
__device__ __forceinline__ float fetch_bias(const MfmaArgs &p, int64_t col0, int t) {
    if constexpr (EPI == EPI_ROUND || EPI == EPI_SCALE) {
        if (p.bias && t < BN) {
            const int64_t j = col0 + t < p.cols ? col0 + t : p.cols - 1;
            const uint16_t b = static_cast<const uint16_t *>(p.bias)[j];
            // the bias has the output's 16-bit type (bf16 for fp8 operands)
            return DT == DT_F16 ? f16_bits_to_f32(b) : bf16_bits_to_f32(b);
        }
    }
    return 0.0f;
}

// LDS bytes the epilogue needs (four waves, one 32-row slab each)
template <int EPI, int WTN, int NW = 4>
constexpr int slab_bytes() {
    return NW * 32 * (WTN * (EPI == EPI_ROUND || EPI == EPI_SCALE ? 2 : 4) + 16);
}

// Epilogue.  For block (i, j) a lane holds row (lane & 31) and, for
// accumulator elements 4g..4g+3, the 4 consecutive columns 8g + 4*(lane/32) +
// 0..3.  Each wave converts one 32-row slab of its tile at a time into a
// private LDS area (row-major), then writes it out as whole contiguous row
// segments, 16 bytes per lane.  Starts with a workgroup barrier, after which
// the stage buffers (`lds`) are free.
template <int DT, int EPI, int WTM, int WTN, int FM, int FN, int BN>
__device__ __forceinline__ void write_tile(const MfmaArgs &p, const TileInfo &ti,
                                           f32x16 (&acc)[FM][FN], char *lds, float *bias_l,
                                           float bias_v, int wave, int wm, int wn, int lane) {
    const int lrow = lane & 31, lkg = lane >> 5;
    const int64_t row0 = ti.row0, row_end = ti.row_end, col0 = ti.col0;
    const int64_t chunk = ti.chunk, c_off = ti.c_off;
    using OutT =
        typename std::conditional<EPI == EPI_ROUND || EPI == EPI_SCALE, uint16_t, float>::type;
    constexpr int OSZ = (int)sizeof(OutT);
    constexpr int ROWB = WTN * OSZ;           // bytes of one slab row
    constexpr int ROWP = ROWB + 16;           // padded LDS row pitch (spreads banks)
    constexpr int CPR = ROWB / 16;            // 16-byte chunks per slab row
    static_assert(ROWB % 16 == 0, "slab rows are whole 16-byte chunks");
    char *slab = lds + wave * 32 * ROWP;
    const bool vec_c = p.vec_c != 0;
    if constexpr (EPI == EPI_ROUND || EPI == EPI_SCALE) {
        const int t = wave * 64 + lane;
        if (p.bias && t < BN) bias_l[t] = bias_v;
    }
    __syncthreads();  // bias visible; every wave done with the stage buffers
    float scale_a = 0.0f, scale_b = 0.0f;
    if constexpr (EPI == EPI_SCALE) scale_a = p.scale_a[0], scale_b = p.scale_b[0];
    // this lane's bias columns, read from LDS once for all row slabs
    f32x4 bias_r[FN][4];
    if constexpr (EPI == EPI_ROUND || EPI == EPI_SCALE) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                bias_r[j][g] = *reinterpret_cast<const f32x4 *>(
                    bias_l + wn * WTN + 32 * j + 8 * g + 4 * lkg);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int cl = 32 * j + 8 * g + 4 * lkg;  // column inside the wave tile
                float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                              acc[i][j][4 * g + 3]};
                char *dst = slab + lrow * ROWP + cl * OSZ;
                if constexpr (EPI == EPI_ROUND) {
                    if (p.bias) {
#pragma unroll
                        for (int x = 0; x < 4; ++x) v[x] = v[x] + bias_r[j][g][x];
                    }
                    *reinterpret_cast<u32x2 *>(dst) =
                        u32x2{pack2_rne<DT>(v[0], v[1]), pack2_rne<DT>(v[2], v[3])};
                } else if constexpr (EPI == EPI_SCALE) {
#pragma unroll
                    for (int x = 0; x < 4; ++x) v[x] = (v[x] * scale_a) * scale_b;
                    if (p.bias) {
#pragma unroll
                        for (int x = 0; x < 4; ++x) v[x] = v[x] + bias_r[j][g][x];
                    }
                    *reinterpret_cast<u32x2 *>(dst) = u32x2{pack2_rne<DT_BF16>(v[0], v[1]),
                                                            pack2_rne<DT_BF16>(v[2], v[3])};
                } else {
                    *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0], v[1], v[2], v[3]};
                }
            }
        }
        // The slab is private to this wave and a wave's LDS operations execute
        // in program order, so the reads below see the writes above and the
        // next slab's writes cannot overtake these reads: no workgroup barrier
        // (which would also wait for every outstanding global store).
        // write the slab: rows gi0 + 0..31, columns gj0 + 0..WTN-1
        const int64_t gi0 = row0 + wm * WTM + 32 * i;
        const int64_t gj0 = col0 + wn * WTN;
        OutT *base = EPI == EPI_PARTIAL
                         ? reinterpret_cast<OutT *>(p.ws + chunk * p.rows * p.cols)
                         : reinterpret_cast<OutT *>(static_cast<char *>(p.c) + c_off * OSZ);
        const int64_t ld = EPI == EPI_PARTIAL ? p.cols : p.ldc;
#pragma unroll
        for (int q = 0; q < (32 * CPR + 63) / 64; ++q) {
            const int idx = lane + 64 * q;
            if (idx < 32 * CPR) {
                const int r = idx / CPR, c = idx % CPR;
                const int64_t gi = gi0 + r;
                const int64_t gj = gj0 + c * (16 / OSZ);
                const u32x4 val = *reinterpret_cast<const u32x4 *>(slab + r * ROWP + c * 16);
                if (gi < row_end) {
                    OutT *dst = base + gi * ld + gj;
                    if (vec_c && gj + 16 / OSZ <= p.cols) {
                        // streaming store: the output is not re-read by this
                        // kernel, and lines written this way need no write-back
                        // when the kernel ends
                        __builtin_nontemporal_store(val, reinterpret_cast<u32x4 *>(dst));
                    } else {
                        const OutT *e = reinterpret_cast<const OutT *>(&val);
#pragma unroll
                        for (int x = 0; x < 16 / OSZ; ++x)
                            if (gj + x < p.cols) dst[x] = e[x];
                    }
                }
            }
        }
    }
}

template <int DT, bool A_RC, bool B_RC, int BM, int BN, int WGM, int WGN, int EPI, int MODE>
__global__ __launch_bounds__(64 * WGM * WGN) void mfma_gemm_kernel(MfmaArgs p) {
    constexpr int NW = WGM * WGN;       // waves: 4 (one per SIMD) or 8 (two per SIMD)
    constexpr int NTH = 64 * NW;
    static_assert(NW == 4 || NW == 8, "four or eight waves");
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    static_assert(FM * 32 == WTM && FN * 32 == WTN, "wave tile must be a multiple of 32");
    using Comp = Compute<DT, BM, BN, WTM, WTN, FM, FN>;

    // stage buffers: A slices [2][KG*BM], then B slices [2][KG*BN] (16-byte
    // slots); reused by the epilogue
    __shared__ u32x4 lds_raw[2 * KG * (BM + BN)];
    __shared__ __align__(16) float lds_bias[BN];
    auto lds_a = [&](int b) { return lds_raw + b * (KG * BM); };
    auto lds_b = [&](int b) { return lds_raw + 2 * KG * BM + b * (KG * BN); };

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    const TileInfo ti = decode_tile<MODE, BM, BN, NTH>(p, t);
    if (ti.skip) return;
    const int64_t row0 = ti.row0, row_end = ti.row_end, col0 = ti.col0;
    const int64_t r_begin = ti.r_begin, r_end = ti.r_end;
    const uint16_t *pa = static_cast<const uint16_t *>(p.a);
    const uint16_t *pb = static_cast<const uint16_t *>(p.b) + ti.b_off;

    const float bias_v = fetch_bias<DT, EPI, BN>(p, col0, t);

    Stage<BM, A_RC, NTH> sa;
    Stage<BN, B_RC, NTH> sb;
    Comp comp;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // interior: every row of the operand tile exists and rows are 16-byte
    // aligned (the same value on every thread of the workgroup)
    const bool int_a = p.vec_a != 0 && row0 + BM <= row_end;
    const bool int_b = p.vec_b != 0 && col0 + BN <= p.cols;
    const int lrow = lane & 31, lkg = lane >> 5;
    const int64_t nst = (r_end - r_begin + BK - 1) / BK;
    const int64_t nfull = (r_end - r_begin) / BK;

    int64_t s = 0;
    if (int_a && int_b && offsets_fit<BM, A_RC>(p.lda) && offsets_fit<BN, B_RC>(p.ldb)) {
        // ---- lean main loop over full slices ----------------------------------
        FastAddr<BM, A_RC, NTH> fa_addr;
        FastAddr<BN, B_RC, NTH> fb_addr;
        fa_addr.init(p.lda, t);
        fb_addr.init(p.ldb, t);
        if (nfull >= 2) {
            fa_addr.load(sa, pa, p.lda, row0, r_begin);
            fb_addr.load(sb, pb, p.ldb, col0, r_begin);
            sa.store(lds_a(0), t);
            sb.store(lds_b(0), t);
            fa_addr.load(sa, pa, p.lda, row0, r_begin + BK);
            fb_addr.load(sb, pb, p.ldb, col0, r_begin + BK);
            __syncthreads();
            // slices s+1 in registers, s in LDS buffer s&1; loads run 2 ahead
            for (; s + 2 < nfull; ++s) {
                const int cur = (int)(s & 1);
                // order pinned for the scheduler: first fragments of slice s,
                // LDS writes of slice s+1, global loads of slice s+2, then the
                // MFMAs of slice s (the loads stay in flight for a whole slice)
                comp.first(lds_a(cur), lds_b(cur), wm, wn, lrow, lkg);
                sa.store(lds_a(cur ^ 1), t);
                sb.store(lds_b(cur ^ 1), t);
                const int64_t rk = r_begin + (s + 2) * BK;
                fa_addr.load(sa, pa, p.lda, row0, rk);
                fb_addr.load(sb, pb, p.ldb, col0, rk);
                __builtin_amdgcn_sched_barrier(0);
                comp.rest(lds_a(cur), lds_b(cur), acc, wm, wn, lrow, lkg);
                __syncthreads();
            }
            // here s + 2 == nfull: slice s in LDS, slice s+1 in registers
        } else {
            s = -1;  // nothing staged yet
        }
    } else {
        s = -1;
    }

    // ---- generic loop (edge tiles, partial slices, pipeline drain) -----------
    // invariant at loop entry: slice s is in LDS buffer s&1 (s >= 0) and slice
    // s+1 is in registers (if it exists); s = -1 means nothing is staged.
    if (s < 0 && nst > 0) {
        sa.load(pa, p.lda, row0, row_end, r_begin, r_end, int_a, t);
        sb.load(pb, p.ldb, col0, p.cols, r_begin, r_end, int_b, t);
        sa.store(lds_a(0), t);
        sb.store(lds_b(0), t);
        if (nst > 1) {
            sa.load(pa, p.lda, row0, row_end, r_begin + BK, r_end, int_a, t);
            sb.load(pb, p.ldb, col0, p.cols, r_begin + BK, r_end, int_b, t);
        }
        __syncthreads();
        s = 0;
    }
    for (; s >= 0 && s < nst; ++s) {
        const int cur = (int)(s & 1);
        if (s + 1 < nst) {
            sa.store(lds_a(cur ^ 1), t);
            sb.store(lds_b(cur ^ 1), t);
            if (s + 2 < nst) {
                const int64_t rk = r_begin + (s + 2) * BK;
                sa.load(pa, p.lda, row0, row_end, rk, r_end, int_a, t);
                sb.load(pb, p.ldb, col0, p.cols, rk, r_end, int_b, t);
            }
        }
        comp.run(lds_a(cur), lds_b(cur), acc, wm, wn, lrow, lkg);
        __syncthreads();
    }

    static_assert(slab_bytes<EPI, WTN, NW>() <= 2 * KG * (BM + BN) * 16, "slabs fit in the stage buffers");
    write_tile<DT, EPI, WTM, WTN, FM, FN, BN>(p, ti, acc, reinterpret_cast<char *>(lds_raw),
                                              lds_bias, bias_v, wave, wm, wn, lane);
}

}  // namespace mfma

}  // namespace bi

namespace bi {
namespace mfma {

// Tile shapes (id -> BM x BN, wave layout).  All issue the same MFMA sequence
// per output element; they differ only in how work is spread over the chip.
template <int ID> struct TileOf;
template <> struct TileOf<1> { static constexpr int BM = 256, BN = 256, WGM = 2, WGN = 2; };
template <> struct TileOf<2> { static constexpr int BM = 256, BN = 192, WGM = 2, WGN = 2; };
template <> struct TileOf<3> { static constexpr int BM = 256, BN = 128, WGM = 2, WGN = 2; };
template <> struct TileOf<4> { static constexpr int BM = 128, BN = 128, WGM = 2, WGN = 2; };
template <> struct TileOf<5> { static constexpr int BM = 128, BN = 96, WGM = 4, WGN = 1; };
template <> struct TileOf<6> { static constexpr int BM = 64, BN = 64, WGM = 2, WGN = 2; };
template <> struct TileOf<7> { static constexpr int BM = 128, BN = 256, WGM = 2, WGN = 2; };
// three waves (direct-load kernel only): 256 tiles of a 768 x 3072 output
template <> struct TileOf<8> { static constexpr int BM = 96, BN = 96, WGM = 3, WGN = 1; };
template <> struct TileOf<9> { static constexpr int BM = 128, BN = 192, WGM = 2, WGN = 2; };
template <> struct TileOf<10> { static constexpr int BM = 256, BN = 96, WGM = 4, WGN = 1; };
// eight waves, two per SIMD
template <> struct TileOf<11> { static constexpr int BM = 256, BN = 192, WGM = 4, WGN = 2; };
template <> struct TileOf<12> { static constexpr int BM = 256, BN = 256, WGM = 4, WGN = 2; };
template <> struct TileOf<13> { static constexpr int BM = 256, BN = 128, WGM = 4, WGN = 2; };
template <> struct TileOf<14> { static constexpr int BM = 128, BN = 256, WGM = 2, WGN = 4; };
template <> struct TileOf<15> { static constexpr int BM = 128, BN = 128, WGM = 2, WGN = 4; };
// three waves side by side (direct-load kernel only)
// eight waves of 96x64: 2 x 4 tiles of 1408 x 2048 per expert (grouped dweights)
template <> struct TileOf<16> { static constexpr int BM = 192, BN = 256, WGM = 2, WGN = 4; };
template <> struct TileOf<17> { static constexpr int BM = 96, BN = 96, WGM = 1, WGN = 3; };
// small-M shapes (direct-load kernel only, tile ids 120 and 121): many narrow
// column tiles; 121 (one MFMA wave, a sixteen-stage ring) for the fp8 GEMM
template <> struct TileOf<20> { static constexpr int BM = 64, BN = 32, WGM = 2, WGN = 1; };
template <> struct TileOf<21> { static constexpr int BM = 32, BN = 32, WGM = 1, WGN = 1; };

template <int DT, bool ARC, bool BRC, int EPI, int MODE, int ID>
hipError_t launch_tile(const MfmaArgs &p, int64_t grid, hipStream_t s) {
    using T = TileOf<ID>;
    hipLaunchKernelGGL((mfma_gemm_kernel<DT, ARC, BRC, T::BM, T::BN, T::WGM, T::WGN, EPI, MODE>),
                       dim3(grid), dim3(64 * T::WGM * T::WGN), 0, s, p);
    return hipGetLastError();
}

// dispatch over a compile-time list of tile ids
template <int DT, bool ARC, bool BRC, int EPI, int MODE, int... IDS>
hipError_t launch_among(const MfmaArgs &p, int tile_id, int64_t grid, hipStream_t s) {
    hipError_t r = hipErrorInvalidValue;
    ((tile_id == IDS ? (void)(r = launch_tile<DT, ARC, BRC, EPI, MODE, IDS>(p, grid, s)) : (void)0),
     ...);
    return r;
}

}  // namespace mfma
}  // namespace bi
