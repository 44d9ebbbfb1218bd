// MFMA tier for bf16 / f16 operands on gfx950 (sgemm-bi PyPI page,
// "Determinism contracts": tensor-core tier with f32 accumulation, bit-identical
// across runs, forward strictly batch-invariant across all M, several tile
// families giving the same bits).
//
// One kernel template serves the linear forward, dX, dW (both passes' pass 1),
// and the grouped forward / dinput / dweights (rublas tensor_grouped/mod.rs).
// It computes C(i,j) = sum_r A(i,r) B(j,r) with:
//   * v_mfma_f32_32x32x16_{bf16,f16} as the only arithmetic on the reduction:
//     each output element's accumulator starts at +0 and receives one MFMA per
//     16-deep reduction step, steps in ascending order from the start of the
//     reduction range.  Neither the tile shape nor the position of the element
//     inside its tile changes that sequence, so all tile shapes give the same
//     bits and a row's bits never depend on the number of rows (M).
//   * 64-deep reduction slices staged global -> registers -> LDS, the next
//     slice's global loads in flight while the current slice is multiplied.
//   * LDS layout "k-grouped": for every group of 8 consecutive reduction
//     indices, each tile row owns one 16-byte slot holding those 8 values, so
//     an MFMA operand (8 consecutive reduction values of one row per lane) is a
//     single ds_read_b128.  Slots are XOR-swizzled within groups of 8 rows so
//     that the reads, the direct writes and the transposed writes all spread
//     over the 32 banks.
//   * Operands whose reduction index is contiguous in memory are copied as
//     16-byte vectors; operands whose reduction index is strided (W in the
//     forward, X and dY in dW, ...) are loaded as 8x8 element blocks and
//     transposed in registers before the LDS write.
//   * Workgroup ids are remapped so that the 32 CUs of one XCD work on one
//     compact block of output tiles and share operand rows in that XCD's L2.
#include "device_common.hpp"
#include "kernels.hpp"

namespace bi {

namespace {

constexpr int BK = 64;      // reduction slice per LDS stage
constexpr int KG = BK / 8;  // 8-element groups per slice
constexpr int NT = 256;     // threads per workgroup (4 waves)

enum Mode : int { MODE_PLAIN = 0, MODE_SEGMENTS = 1, MODE_EXPERT_RED = 2 };
enum Epi : int { EPI_ROUND = 0, EPI_PARTIAL = 1, EPI_F32 = 2 };

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

// 8 consecutive 16-bit elements starting at p[0], zero beyond `count`.
__device__ __forceinline__ u32x4 load8(const uint16_t *p, int count, bool vec) {
    if (count >= 8 && vec) return *reinterpret_cast<const u32x4 *>(p);
    uint32_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = i < count ? p[i] : 0u;
    u32x4 r;
    r[0] = e[0] | (e[1] << 16);
    r[1] = e[2] | (e[3] << 16);
    r[2] = e[4] | (e[5] << 16);
    r[3] = e[6] | (e[7] << 16);
    return r;
}

// Transpose an 8x8 block of 16-bit elements: in[r] holds row r (8 elements),
// out[c] receives column c (8 elements, row 0 in the low half of word 0).
__device__ __forceinline__ void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
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
template <int R, bool RC>
struct Stage {
    static constexpr int DIRECT_PER_THREAD = R * KG / NT;             // RC
    static constexpr int UNITS = KG * (R / 8);                        // !RC, 8x8 blocks
    static constexpr int UNITS_PER_THREAD = (UNITS + NT - 1) / NT;
    static constexpr int NREG = RC ? DIRECT_PER_THREAD : UNITS_PER_THREAD * 8;
    static_assert(!RC || (R * KG) % NT == 0, "tile rows must fill the workgroup");

    u32x4 reg[NREG];

    // rows [row0, row_end) of the operand; reduction [rk, r_end)
    __device__ __forceinline__ void load(const uint16_t *p, int64_t ld, int64_t row0,
                                         int64_t row_end, int64_t rk, int64_t r_end, bool vec,
                                         int t) {
        if constexpr (RC) {
#pragma unroll
            for (int q = 0; q < DIRECT_PER_THREAD; ++q) {
                const int c = t + NT * q;
                const int row = c / KG, kg = c % KG;
                const int64_t gi = row0 + row, gr = rk + 8 * kg;
                int cnt = gi < row_end ? (int)(r_end - gr < 8 ? r_end - gr : 8) : 0;
                if (cnt < 0) cnt = 0;
                reg[q] = cnt > 0 ? load8(p + gi * ld + gr, cnt, vec) : u32x4{0u, 0u, 0u, 0u};
            }
        } else {
#pragma unroll
            for (int q = 0; q < UNITS_PER_THREAD; ++q) {
                const int u = t + NT * q;
                const int kg = u / (R / 8), ib = u % (R / 8);
                const int64_t gi = row0 + 8 * ib;
                int cnt = (int)(row_end - gi < 8 ? row_end - gi : 8);
                if (cnt < 0 || u >= UNITS) cnt = 0;
#pragma unroll
                for (int rr = 0; rr < 8; ++rr) {
                    const int64_t gr = rk + 8 * kg + rr;
                    reg[q * 8 + rr] = (cnt > 0 && gr < r_end) ? load8(p + gr * ld + gi, cnt, vec)
                                                              : u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    }

    __device__ __forceinline__ void store(u32x4 *lds, int t) const {
        if constexpr (RC) {
#pragma unroll
            for (int q = 0; q < DIRECT_PER_THREAD; ++q) {
                const int c = t + NT * q;
                const int row = c / KG, kg = c % KG;
                lds[kg * R + swz(row, kg)] = reg[q];
            }
        } else {
#pragma unroll
            for (int q = 0; q < UNITS_PER_THREAD; ++q) {
                const int u = t + NT * q;
                if (u >= UNITS) continue;
                const int kg = u / (R / 8), ib = u % (R / 8);
                u32x4 tr[8];
                transpose8x8(&reg[q * 8], tr);
#pragma unroll
                for (int c = 0; c < 8; ++c) lds[kg * R + swz(8 * ib + c, kg)] = tr[c];
            }
        }
    }
};

template <int DT, bool A_RC, bool B_RC, int BM, int BN, int WGM, int WGN, int EPI, int MODE>
__global__ __launch_bounds__(NT) void mfma_gemm_kernel(MfmaArgs p) {
    static_assert(WGM * WGN == 4, "four waves");
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    static_assert(FM * 32 == WTM && FN * 32 == WTN, "wave tile must be a multiple of 32");

    __shared__ u32x4 lds_a[KG * BM];
    __shared__ u32x4 lds_b[KG * BN];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    // ---- which tile, which rows, which reduction range --------------------
    int64_t row0, row_end, col0, r_begin, r_end, chunk = 0;
    const uint16_t *pa = static_cast<const uint16_t *>(p.a);
    const uint16_t *pb = static_cast<const uint16_t *>(p.b);
    int64_t c_off = 0;
    if constexpr (MODE == MODE_PLAIN) {
        const int64_t tiles = p.tiles_i * p.tiles_j;
        const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
        chunk = bid / tiles;
        const int64_t tile = bid % tiles;
        // groups of 4 row-tiles, column-major inside a group
        constexpr int64_t GROUP = 4;
        const int64_t per_group = GROUP * p.tiles_j;
        const int64_t g = tile / per_group, first = g * GROUP;
        const int64_t gsz = p.tiles_i - first < GROUP ? p.tiles_i - first : GROUP;
        const int64_t in_g = tile % per_group;
        row0 = (first + in_g % gsz) * BM;
        col0 = (in_g / gsz) * BN;
        row_end = p.rows;
        r_begin = chunk * p.chunk;
        r_end = r_begin + p.chunk < p.red ? r_begin + p.chunk : p.red;
    } else if constexpr (MODE == MODE_SEGMENTS) {
        const int64_t ti = blockIdx.x / p.tiles_j;
        col0 = (blockIdx.x % p.tiles_j) * BN;
        int64_t tt = ti;
        int64_t x = 0;
        row0 = -1;
        row_end = 0;
        for (; x <= p.n_experts; ++x) {
            int64_t s = p.offsets[x < p.n_experts ? x : p.n_experts];
            int64_t e = x < p.n_experts ? (int64_t)p.offsets[x + 1] : p.rows;
            if (e > p.rows) e = p.rows;
            if (s > e) s = e;
            const int64_t cnt = (e - s + BM - 1) / BM;
            if (tt < cnt) {
                row0 = s + tt * BM;
                row_end = e;
                break;
            }
            tt -= cnt;
        }
        if (row0 < 0) return;  // beyond the last segment tile (whole workgroup)
        if (x == p.n_experts) {
            // padding rows: exact +0 (rublas: ids outside [0,E) give zero rows)
            const int64_t r1 = row0 + BM < row_end ? row0 + BM : row_end;
            uint16_t *pc = static_cast<uint16_t *>(p.c);
            for (int64_t idx = t; idx < (r1 - row0) * BN; idx += NT) {
                const int64_t i = row0 + idx / BN, j = col0 + idx % BN;
                if (j < p.cols) pc[i * p.ldc + j] = 0;
            }
            return;
        }
        pb += x * p.b_expert_stride;
        r_begin = 0;
        r_end = p.red;
    } else {  // MODE_EXPERT_RED
        const int64_t per_x = p.tiles_i * p.tiles_j;
        const int64_t x = blockIdx.x / per_x;
        const int64_t tile = blockIdx.x % per_x;
        row0 = (tile / p.tiles_j) * BM;
        col0 = (tile % p.tiles_j) * BN;
        row_end = p.rows;
        r_end = p.red_offsets[x + 1];
        r_begin = p.red_offsets[x];
        if (r_end > p.red) r_end = p.red;
        if (r_begin > r_end) r_begin = r_end;
        c_off = x * p.c_expert_stride;
    }

    Stage<BM, A_RC> sa;
    Stage<BN, B_RC> sb;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const bool va = p.vec_a != 0, vb = p.vec_b != 0;
    if (r_begin < r_end) {
        sa.load(pa, p.lda, row0, row_end, r_begin, r_end, va, t);
        sb.load(pb, p.ldb, col0, p.cols, r_begin, r_end, vb, t);
    }
    const int lrow = lane & 31, lkg = lane >> 5;
    for (int64_t rk = r_begin; rk < r_end; rk += BK) {
        sa.store(lds_a, t);
        sb.store(lds_b, t);
        __syncthreads();
        if (rk + BK < r_end) {
            sa.load(pa, p.lda, row0, row_end, rk + BK, r_end, va, t);
            sb.load(pb, p.ldb, col0, p.cols, rk + BK, r_end, vb, t);
        }
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int kg = 2 * kk + lkg;
            u32x4 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[i] = lds_a[kg * BM + swz(wm * WTM + 32 * i + lrow, kg)];
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[j] = lds_b[kg * BN + swz(wn * WTN + 32 * j + lrow, kg)];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma_step<DT>(fa[i], fb[j], acc[i][j]);
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds column (lane & 31) of each 32x32 block, rows
    // 8*(v/4) + 4*(lane/32) + (v%4) for accumulator element v ------------------
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t gj = col0 + wn * WTN + 32 * j + lrow;
        if (gj >= p.cols) continue;
        float bias = 0.0f;
        bool has_bias = false;
        if constexpr (EPI == EPI_ROUND) {
            if (p.bias) {
                has_bias = true;
                bias = DT == DT_BF16 ? bf16_bits_to_f32(static_cast<const uint16_t *>(p.bias)[gj])
                                     : f16_bits_to_f32(static_cast<const uint16_t *>(p.bias)[gj]);
            }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t gi = row0 + wm * WTM + 32 * i + 8 * (v >> 2) + 4 * lkg + (v & 3);
                if (gi >= row_end) continue;
                float val = acc[i][j][v];
                if constexpr (EPI == EPI_ROUND) {
                    if (has_bias) val = val + bias;
                    store_elem<DT>(p.c, gi * p.ldc + gj, val);
                } else if constexpr (EPI == EPI_PARTIAL) {
                    p.ws[(chunk * p.rows + gi) * p.cols + gj] = val;
                } else {
                    static_cast<float *>(p.c)[c_off + gi * p.ldc + gj] = val;
                }
            }
        }
    }
}

// ---- tile table -------------------------------------------------------------

struct TileCfg {
    int id, bm, bn, wgm, wgn;
};

constexpr TileCfg kTiles[] = {
    {1, 256, 256, 2, 2},
    {2, 256, 192, 2, 2},
    {3, 256, 128, 2, 2},
    {4, 128, 128, 2, 2},
    {5, 128, 96, 4, 1},
    {6, 64, 64, 2, 2},
    {7, 128, 256, 2, 2},
};

template <int DT, bool ARC, bool BRC, int EPI, int MODE, int BM, int BN, int WGM, int WGN>
hipError_t launch_one(const MfmaArgs &p, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((mfma_gemm_kernel<DT, ARC, BRC, BM, BN, WGM, WGN, EPI, MODE>), dim3(grid),
                       dim3(NT), 0, s, p);
    return hipGetLastError();
}

template <int DT, bool ARC, bool BRC, int EPI, int MODE>
hipError_t launch_tiles(const MfmaArgs &p, int tile_id, int64_t grid, hipStream_t s) {
    switch (tile_id) {
    case 1: return launch_one<DT, ARC, BRC, EPI, MODE, 256, 256, 2, 2>(p, grid, s);
    case 2: return launch_one<DT, ARC, BRC, EPI, MODE, 256, 192, 2, 2>(p, grid, s);
    case 3: return launch_one<DT, ARC, BRC, EPI, MODE, 256, 128, 2, 2>(p, grid, s);
    case 4: return launch_one<DT, ARC, BRC, EPI, MODE, 128, 128, 2, 2>(p, grid, s);
    case 5: return launch_one<DT, ARC, BRC, EPI, MODE, 128, 96, 4, 1>(p, grid, s);
    case 6: return launch_one<DT, ARC, BRC, EPI, MODE, 64, 64, 2, 2>(p, grid, s);
    case 7: return launch_one<DT, ARC, BRC, EPI, MODE, 128, 256, 2, 2>(p, grid, s);
    }
    return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_dt(const MfmaArgs &p, int tile_id, int layout, int epi, int mode,
                     int64_t grid, hipStream_t s) {
    // the (layout, epilogue, mode) combinations the library uses
    if (mode == MODE_PLAIN && layout == 1 && epi == EPI_ROUND)  // forward
        return launch_tiles<DT, true, false, EPI_ROUND, MODE_PLAIN>(p, tile_id, grid, s);
    if (mode == MODE_PLAIN && layout == 3 && epi == EPI_ROUND)  // dX
        return launch_tiles<DT, true, true, EPI_ROUND, MODE_PLAIN>(p, tile_id, grid, s);
    if (mode == MODE_PLAIN && layout == 0 && epi == EPI_ROUND)  // dW, one chunk
        return launch_tiles<DT, false, false, EPI_ROUND, MODE_PLAIN>(p, tile_id, grid, s);
    if (mode == MODE_PLAIN && layout == 0 && epi == EPI_PARTIAL)  // dW pass 1
        return launch_tiles<DT, false, false, EPI_PARTIAL, MODE_PLAIN>(p, tile_id, grid, s);
    if (mode == MODE_SEGMENTS && layout == 3 && epi == EPI_ROUND)  // grouped forward
        return launch_tiles<DT, true, true, EPI_ROUND, MODE_SEGMENTS>(p, tile_id, grid, s);
    if (mode == MODE_SEGMENTS && layout == 1 && epi == EPI_ROUND)  // grouped dinput
        return launch_tiles<DT, true, false, EPI_ROUND, MODE_SEGMENTS>(p, tile_id, grid, s);
    if (mode == MODE_EXPERT_RED && layout == 0 && epi == EPI_F32)  // grouped dweights
        return launch_tiles<DT, false, false, EPI_F32, MODE_EXPERT_RED>(p, tile_id, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace

const TileShape *mfma_tile(int id) {
    static TileShape shapes[sizeof(kTiles) / sizeof(kTiles[0])];
    for (size_t i = 0; i < sizeof(kTiles) / sizeof(kTiles[0]); ++i) {
        if (kTiles[i].id == id) {
            shapes[i] = TileShape{kTiles[i].id, kTiles[i].bm, kTiles[i].bn};
            return &shapes[i];
        }
    }
    return nullptr;
}

hipError_t launch_mfma_gemm(const MfmaArgs &p, int tile_id, int dt, int layout, int epi,
                            hipStream_t s) {
    const int mode = p.offsets ? MODE_SEGMENTS : (p.red_offsets ? MODE_EXPERT_RED : MODE_PLAIN);
    int64_t grid;
    if (mode == MODE_PLAIN) grid = p.tiles_i * p.tiles_j * p.nchunks;
    else if (mode == MODE_SEGMENTS) grid = p.seg_tiles * p.tiles_j;
    else grid = p.n_experts * p.tiles_i * p.tiles_j;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (dt == DT_BF16) return launch_dt<DT_BF16>(p, tile_id, layout, epi, mode, grid, s);
    if (dt == DT_F16) return launch_dt<DT_F16>(p, tile_id, layout, epi, mode, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace bi
