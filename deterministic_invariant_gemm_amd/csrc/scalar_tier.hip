// Scalar FMA tier (sgemm-bi PyPI page, "Determinism contracts": the f32 /
// typed scalar tier, bit-identical across runs, bf16/f16 equal to "upcast ->
// f32 kernel -> RNE downcast", full shape coverage).
//
// Every output element is ONE f32 chain
//     acc = +0;  for r ascending over the reduction range: acc = fmaf(a_r, b_r, acc)
// followed by the epilogue (+bias in f32, or the two fp8 scale multiplies, or
// the f32 partial store) and a single rounding to the output type.  Inputs are
// widened exactly to f32 when staged, so the bf16/f16 instantiations execute
// the very same f32 instruction sequence as the f32 one on the upcast values.
// This file is compiled with -ffp-contract=off: the only fused operations are
// the explicit fmaf calls.
//
// Layout: a generic strided formulation C(i,j) = sum_r A(i,r) B(r,j) with
// A(i,r) = a[i*a_is + r*a_rs] and B(r,j) = b[r*b_rs + j*b_js] covers forward,
// dX, dW and fp8.  A workgroup of 256 threads computes a TM x 64 tile (TM = 64,
// 32 or 16: the tallest that still gives the chip 256 workgroups), each thread
// TM/16 rows (stride 16) by 4 adjacent columns, staging 32-deep reduction
// slices through LDS; the next slice is loaded into registers while the
// current one is multiplied.  A is staged row by row ([TM][RK]) and B one
// reduction index per row ([RK][64]), so one 16-byte LDS read gives a thread
// four reduction values of a row of A, or its four columns of B at one
// reduction index; full slices run unrolled on those reads, the last partial
// slice one reduction index at a time up to the end of the range (an fmaf on
// padding zeros could turn a chain's -0, reached by underflow, into +0).
// Neither the tile height nor the slice depth changes any element's fmaf
// chain, so every tile gives the same bits.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace bi {

namespace {

constexpr int ST = 64;  // tile columns

enum ScalarEpi : int { EPI_ROUND = 0, EPI_PARTIAL = 1, EPI_FP8 = 2 };

template <int DT_IN, int DT_OUT, int EPI, int TM>
__global__ __launch_bounds__(256) void scalar_gemm_kernel(ScalarGemmArgs p) {
    constexpr int RK = 32;             // reduction slice staged per step
    constexpr int MA = TM / 16;        // output rows per thread
    constexpr int NA = TM * RK / 256;  // A elements staged per thread per slice
    constexpr int NB = RK * ST / 256;  // B elements staged per thread per slice
    // rows padded by 4 floats: 16-byte aligned, and rows of A four banks apart
    __shared__ __align__(16) float As[TM][RK + 4];
    __shared__ __align__(16) float Bs[RK][ST + 4];

    const int t = threadIdx.x;
    const int tx = t & 15, ty = t >> 4;
    const int64_t tiles = p.tiles_i * p.tiles_j;
    const int64_t bid = blockIdx.x;
    const int64_t chunk = bid / tiles;
    const int64_t tile = bid % tiles;
    const int64_t i0 = (tile / p.tiles_j) * TM;
    const int64_t j0 = (tile % p.tiles_j) * ST;
    const int64_t r_begin = chunk * p.chunk;
    const int64_t r_end = r_begin + p.chunk < p.red ? r_begin + p.chunk : p.red;

    float acc[MA][4];
#pragma unroll
    for (int a = 0; a < MA; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;

    const bool a_r_contig = p.a_rs == 1;
    const bool b_j_contig = p.b_js == 1;

    // slice at rk into registers (exact f32), zeros outside the matrices and
    // past the end of the reduction range
    float ra[NA], rb[NB];
    auto load = [&](int64_t rk) {
#pragma unroll
        for (int q = 0; q < NA; ++q) {
            const int idx = t + 256 * q;
            int row, rr;
            if (a_r_contig) { row = idx / RK; rr = idx % RK; }
            else            { row = idx % TM; rr = idx / TM; }
            const int64_t gi = i0 + row, gr = rk + rr;
            ra[q] = (gi < p.rows && gr < r_end) ? load_elem<DT_IN>(p.a, gi * p.a_is + gr * p.a_rs)
                                                : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int idx = t + 256 * q;
            int col, rr;
            if (b_j_contig) { col = idx % ST; rr = idx / ST; }
            else            { col = idx / RK; rr = idx % RK; }
            const int64_t gj = j0 + col, gr = rk + rr;
            rb[q] = (gj < p.cols && gr < r_end) ? load_elem<DT_IN>(p.b, gr * p.b_rs + gj * p.b_js)
                                                : 0.0f;
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int q = 0; q < NA; ++q) {
            const int idx = t + 256 * q;
            if (a_r_contig) As[idx / RK][idx % RK] = ra[q];
            else            As[idx % TM][idx / TM] = ra[q];
        }
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int idx = t + 256 * q;
            if (b_j_contig) Bs[idx / ST][idx % ST] = rb[q];
            else            Bs[idx % RK][idx / RK] = rb[q];
        }
    };

    if (r_begin < r_end) load(r_begin);
    for (int64_t rk = r_begin; rk < r_end; rk += RK) {
        store();
        __syncthreads();
        if (rk + RK < r_end) load(rk + RK);  // in flight while this slice is multiplied
        if (r_end - rk >= RK) {
#pragma unroll
            for (int r4 = 0; r4 < RK; r4 += 4) {
                f32x4 av[MA], bv[4];
#pragma unroll
                for (int a = 0; a < MA; ++a)
                    av[a] = *reinterpret_cast<const f32x4 *>(&As[ty + 16 * a][r4]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    bv[q] = *reinterpret_cast<const f32x4 *>(&Bs[r4 + q][4 * tx]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int a = 0; a < MA; ++a)
#pragma unroll
                        for (int b = 0; b < 4; ++b)
                            acc[a][b] = __builtin_fmaf(av[a][q], bv[q][b], acc[a][b]);
            }
        } else {
            const int valid = (int)(r_end - rk);
            for (int rr = 0; rr < valid; ++rr) {
                float av[MA];
#pragma unroll
                for (int a = 0; a < MA; ++a) av[a] = As[ty + 16 * a][rr];
                const f32x4 bv = *reinterpret_cast<const f32x4 *>(&Bs[rr][4 * tx]);
#pragma unroll
                for (int a = 0; a < MA; ++a)
#pragma unroll
                    for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(av[a], bv[b], acc[a][b]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int a = 0; a < MA; ++a) {
        const int64_t gi = i0 + ty + 16 * a;
        if (gi >= p.rows) continue;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t gj = j0 + 4 * tx + b;
            if (gj >= p.cols) continue;
            float v = acc[a][b];
            if constexpr (EPI == EPI_PARTIAL) {
                p.ws[(chunk * p.rows + gi) * p.cols + gj] = v;
            } else {
                if constexpr (EPI == EPI_FP8) {
                    v = v * p.scale_a[0];
                    v = v * p.scale_b[0];
                    if (p.bias) v = v + load_elem<DT_OUT>(p.bias, gj);  // bf16 bias
                } else {
                    if (p.bias) v = v + load_elem<DT_IN>(p.bias, gj);
                }
                store_elem<DT_OUT>(p.c, gi * p.ldc + gj, v);
            }
        }
    }
}

// Narrow outputs (at most 64 columns, such as a 48-wide layer) whose rows of A
// are not contiguous along the reduction, or not 16-byte aligned (dW, where A
// is contiguous across rows instead).  The tiled kernel above would leave the
// columns past the output's width idle in every 64-column tile and make few
// tiles; here a lane owns ONE row and CW adjacent columns (CW = 4, or 2 when
// that gives too few workgroups), a workgroup 256 consecutive rows (one per
// lane of its four waves) of the same columns.  The B values of a reduction
// index are the same for every lane: they are staged per slice into LDS and
// read back as one broadcast LDS read per reduction index; each lane's A
// values come straight from memory into registers, one value per reduction
// index (coalesced across lanes when A is contiguous along its rows, as in
// dW).  The next slice's A and B are loaded while the current one is
// multiplied; a partial last slice loads each value as it multiplies it.  Each
// output is the same chain as in the tiled kernel: fmaf over the reduction
// indices of its range in ascending order from +0, nothing past the range.

template <int DT>
__device__ __forceinline__ float vec_elem(const u32x4 &v, int q) {
    if constexpr (DT == DT_F32) {
        return __uint_as_float(v[q]);
    } else if constexpr (DT == DT_BF16 || DT == DT_F16) {
        const uint32_t h = (v[q >> 1] >> (16 * (q & 1))) & 0xffffu;
        return DT == DT_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
    } else {
        return e4m3_bits_to_f32((v[q >> 2] >> (8 * (q & 3))) & 0xffu);
    }
}

template <int DT_IN, int DT_OUT, int EPI, int CW>
__global__ __launch_bounds__(256) void scalar_narrow_kernel(ScalarGemmArgs p) {
    constexpr int NR_SL = 64;  // reduction indices per staged slice
    constexpr int NBS = (NR_SL * CW + 255) / 256;  // B values staged per thread
    using BV = typename std::conditional<CW == 4, f32x4, f32x2>::type;
    __shared__ __align__(16) float Bs[2][NR_SL][CW];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t rgroups = (p.rows + 255) / 256, cgroups = (p.cols + CW - 1) / CW;
    const int64_t per_chunk = rgroups * cgroups;
    const int64_t bid = blockIdx.x;
    const int64_t chunk = bid / per_chunk, rem = bid % per_chunk;
    const int64_t cg = rem / rgroups, rg = rem % rgroups;
    const int64_t i = rg * 256 + wave * 64 + lane;
    const int64_t j0 = cg * CW;
    const int64_t r_begin = chunk * p.chunk;
    const int64_t r_end = r_begin + p.chunk < p.red ? r_begin + p.chunk : p.red;
    // rows past the end load the last row (their outputs are not stored)
    const int64_t ic = i < p.rows ? i : p.rows - 1;

    float acc[CW];
#pragma unroll
    for (int c = 0; c < CW; ++c) acc[c] = 0.0f;

    // thread t stages B(rs + e / CW, j0 + e % CW) for e = t + 256 u < NR_SL * CW;
    // +0 outside
    float b_next[NBS];
    auto load_b = [&](int64_t rs) {
#pragma unroll
        for (int u = 0; u < NBS; ++u) {
            const int e = t + 256 * u;
            if (e < NR_SL * CW) {
                const int64_t r = rs + e / CW, j = j0 + e % CW;
                b_next[u] = (r < r_end && j < p.cols)
                                ? load_elem<DT_IN>(p.b, r * p.b_rs + j * p.b_js)
                                : 0.0f;
            }
        }
    };
    // this lane's A values of a whole slice
    float as_next[NR_SL], as_cur[NR_SL];
    auto load_a = [&](int64_t rs) {
#pragma unroll
        for (int q = 0; q < NR_SL; ++q)
            as_next[q] = load_elem<DT_IN>(p.a, ic * p.a_is + (rs + q) * p.a_rs);
    };

    if (r_begin < r_end) {
        load_b(r_begin);
        if (r_begin + NR_SL <= r_end) load_a(r_begin);
    }
    int buf = 0;
    for (int64_t rs = r_begin; rs < r_end; rs += NR_SL, buf ^= 1) {
#pragma unroll
        for (int u = 0; u < NBS; ++u) {
            const int e = t + 256 * u;
            if (e < NR_SL * CW) Bs[buf][e / CW][e % CW] = b_next[u];
        }
        const bool full = rs + NR_SL <= r_end;
        if (full) {
#pragma unroll
            for (int q = 0; q < NR_SL; ++q) as_cur[q] = as_next[q];
        }
        __syncthreads();
        if (rs + NR_SL < r_end) {  // in flight while this slice is multiplied
            load_b(rs + NR_SL);
            if (rs + 2 * NR_SL <= r_end) load_a(rs + NR_SL);
        }
        if (full) {
            // 16 bytes of B per LDS read: one reduction index of four columns or
            // two of two
            constexpr int RPR = 4 / CW;
#pragma unroll
            for (int r0 = 0; r0 < NR_SL; r0 += RPR) {
                const f32x4 b = *reinterpret_cast<const f32x4 *>(&Bs[buf][r0][0]);
#pragma unroll
                for (int u = 0; u < RPR; ++u) {
                    const float a = as_cur[r0 + u];
#pragma unroll
                    for (int c = 0; c < CW; ++c) acc[c] = __builtin_fmaf(a, b[u * CW + c], acc[c]);
                }
            }
        } else {
            const int n = (int)(r_end - rs);
            for (int rr = 0; rr < n; ++rr) {
                const float a = load_elem<DT_IN>(p.a, ic * p.a_is + (rs + rr) * p.a_rs);
                const BV b = *reinterpret_cast<const BV *>(&Bs[buf][rr][0]);
#pragma unroll
                for (int c = 0; c < CW; ++c) acc[c] = __builtin_fmaf(a, b[c], acc[c]);
            }
        }
    }

    if (i >= p.rows) return;
#pragma unroll
    for (int c = 0; c < CW; ++c) {
        const int64_t j = j0 + c;
        if (j >= p.cols) continue;
        float v = acc[c];
        if constexpr (EPI == EPI_PARTIAL) {
            p.ws[(chunk * p.rows + i) * p.cols + j] = v;
        } else {
            if constexpr (EPI == EPI_FP8) {
                v = v * p.scale_a[0];
                v = v * p.scale_b[0];
                if (p.bias) v = v + load_elem<DT_OUT>(p.bias, j);  // bf16 bias
            } else {
                if (p.bias) v = v + load_elem<DT_IN>(p.bias, j);
            }
            store_elem<DT_OUT>(p.c, i * p.ldc + j, v);
        }
    }
}

// Narrow outputs whose rows of A are contiguous along the reduction (forward,
// dX, fp8; 16-byte aligned rows): a workgroup owns 64 rows (one per lane) and
// CB = waves x CW adjacent columns (CW per wave), so each slice of A (64 rows x 128 bytes) is
// loaded once per workgroup, in coalesced 16-byte row pieces, into LDS (rows
// padded by 16 bytes so that the lanes' 16-byte reads of their own rows fall
// in distinct banks) instead of once per column group straight into each
// lane's registers.  B is staged per slice as f32 columns ([c][r]) and read as
// broadcast 16-byte reads of four reduction indices.  The next full slice is
// loaded into registers while the current one is multiplied (two LDS buffers,
// one barrier per slice); a partial last slice is staged element by element
// and multiplied one reduction index at a time up to the end of the range.
// Each output is the same chain as in the kernels above.
constexpr int RB_SLB = 128;  // bytes of a row of A per slice
constexpr int64_t RB_WGS = 256;  // workgroups the launcher aims for

template <int DT>
__device__ __forceinline__ float lds_elem(const char *row, int q) {
    if constexpr (DT == DT_F32) return *reinterpret_cast<const float *>(row + 4 * q);
    else if constexpr (DT == DT_BF16)
        return bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(row + 2 * q));
    else if constexpr (DT == DT_F16)
        return f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(row + 2 * q));
    else return e4m3_bits_to_f32(*reinterpret_cast<const uint8_t *>(row + q));
}

template <int DT>
__device__ __forceinline__ void copy_elem(char *dst, const void *src, int64_t i) {
    if constexpr (DT == DT_F32) *reinterpret_cast<float *>(dst) = static_cast<const float *>(src)[i];
    else if constexpr (DT == DT_BF16 || DT == DT_F16)
        *reinterpret_cast<uint16_t *>(dst) = static_cast<const uint16_t *>(src)[i];
    else *reinterpret_cast<uint8_t *>(dst) = static_cast<const uint8_t *>(src)[i];
}

// blockDim.x = 64 x (4 .. 8 waves); cblocks column blocks of CB columns
template <int DT_IN, int DT_OUT, int EPI, int CW>
__global__ __launch_bounds__(512) void scalar_rowblock_kernel(ScalarGemmArgs p, int64_t cblocks) {
    constexpr int ESZ = DT_IN == DT_F32 ? 4 : DT_IN == DT_E4M3 ? 1 : 2;
    constexpr int RB_KS = RB_SLB / ESZ;       // reduction indices per slice
    constexpr int AV = 16 / ESZ;              // A values per 16-byte piece
    constexpr int PPR = RB_KS * ESZ / 16;     // 16-byte pieces per row and slice
    constexpr int APITCH = RB_KS * ESZ + 16;  // LDS bytes per row of A
    constexpr int NAP = 64 * PPR / 256;       // pieces per thread (at least four waves)
    constexpr int NBT = (CW * RB_KS + 63) / 64;  // B values per thread (at most)
    constexpr int BP = RB_KS + 4;             // LDS floats per column of B
    static_assert(NAP >= 1 && (64 * PPR) % 256 == 0, "whole pieces per thread");
    __shared__ __align__(16) char As[2][64 * APITCH];
    __shared__ __align__(16) float Bs[2][8 * CW * BP];

    const int nth = blockDim.x, t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int cb = (nth >> 6) * CW;  // columns of this workgroup
    const int64_t rblocks = (p.rows + 63) / 64;
    const int64_t per_chunk = rblocks * cblocks;
    const int64_t bid = blockIdx.x;
    const int64_t chunk = bid / per_chunk, rem = bid % per_chunk;
    // workgroups next to each other share their rows of A
    const int64_t i0 = (rem / cblocks) * 64, j0 = (rem % cblocks) * cb;
    const int64_t r_begin = chunk * p.chunk;
    const int64_t r_end = r_begin + p.chunk < p.red ? r_begin + p.chunk : p.red;
    const bool b_cols_contig = p.b_js == 1;

    // staging registers of the next full slice: A pieces e = t + nth u (row
    // e / PPR, piece e % PPR; rows past the end re-read the last row), B values
    // e = t + nth u of the cb x RB_KS block (column-fastest when B's columns
    // are contiguous, reduction-fastest otherwise; +0 outside)
    u32x4 a_next[NAP];
    float b_next[NBT];
    auto b_index = [&](int e, int &c, int &q) {
        if (b_cols_contig) { c = e % cb; q = e / cb; }
        else { c = e / RB_KS; q = e % RB_KS; }
    };
    auto stage_full = [&](int64_t rs) {
#pragma unroll
        for (int u = 0; u < NAP; ++u) {
            const int e = t + nth * u;
            if (e < 64 * PPR) {
                int64_t i = i0 + e / PPR;
                if (i >= p.rows) i = p.rows - 1;
                a_next[u] = *reinterpret_cast<const u32x4 *>(
                    static_cast<const char *>(p.a) + (i * p.a_is + rs) * ESZ + 16 * (e % PPR));
            }
        }
#pragma unroll
        for (int u = 0; u < NBT; ++u) {
            const int e = t + nth * u;
            if (e < cb * RB_KS) {
                int c, q;
                b_index(e, c, q);
                const int64_t j = j0 + c;
                b_next[u] = j < p.cols ? load_elem<DT_IN>(p.b, (rs + q) * p.b_rs + j * p.b_js) : 0.0f;
            }
        }
    };

    float acc[CW];
#pragma unroll
    for (int c = 0; c < CW; ++c) acc[c] = 0.0f;
    const int wc = wave * CW;  // this wave's first column in the workgroup

    if (r_begin < r_end && r_begin + RB_KS <= r_end) stage_full(r_begin);
    int buf = 0;
    for (int64_t rs = r_begin; rs < r_end; rs += RB_KS, buf ^= 1) {
        const int n = r_end - rs < RB_KS ? (int)(r_end - rs) : RB_KS;
        char *as = As[buf];
        float *bs = Bs[buf];
        if (n == RB_KS) {
#pragma unroll
            for (int u = 0; u < NAP; ++u) {
                const int e = t + nth * u;
                if (e < 64 * PPR)
                    *reinterpret_cast<u32x4 *>(as + (e / PPR) * APITCH + 16 * (e % PPR)) = a_next[u];
            }
#pragma unroll
            for (int u = 0; u < NBT; ++u) {
                const int e = t + nth * u;
                if (e < cb * RB_KS) {
                    int c, q;
                    b_index(e, c, q);
                    bs[c * BP + q] = b_next[u];
                }
            }
        } else {
            // the partial last slice, element by element (nothing past r_end is read)
            for (int e = t; e < 64 * RB_KS; e += nth) {
                const int row = e / RB_KS, q = e % RB_KS;
                int64_t i = i0 + row;
                if (i >= p.rows) i = p.rows - 1;
                if (q < n) copy_elem<DT_IN>(as + row * APITCH + q * ESZ, p.a, i * p.a_is + rs + q);
            }
            for (int e = t; e < cb * RB_KS; e += nth) {
                int c, q;
                b_index(e, c, q);
                const int64_t j = j0 + c;
                bs[c * BP + q] = (q < n && j < p.cols)
                                     ? load_elem<DT_IN>(p.b, (rs + q) * p.b_rs + j * p.b_js)
                                     : 0.0f;
            }
        }
        __syncthreads();
        if (rs + 2 * RB_KS <= r_end) stage_full(rs + RB_KS);  // in flight during this slice
        const char *arow = as + lane * APITCH;
        const float *bcol = bs + wc * BP;
        if (n == RB_KS) {
            // one 16-byte piece of this lane's row: AV reduction indices
            auto piece = [&](int kk) {
                const u32x4 av = *reinterpret_cast<const u32x4 *>(arow + kk * ESZ);
#pragma unroll
                for (int j = 0; j < AV; j += 4) {
                    f32x4 b[CW];
#pragma unroll
                    for (int c = 0; c < CW; ++c)
                        b[c] = *reinterpret_cast<const f32x4 *>(bcol + c * BP + kk + j);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float a = vec_elem<DT_IN>(av, j + u);
#pragma unroll
                        for (int c = 0; c < CW; ++c) acc[c] = __builtin_fmaf(a, b[c][u], acc[c]);
                    }
                }
            };
            // two pieces per loop iteration (fully unrolled, the slice's LDS
            // reads would be hoisted into more registers than two waves per
            // SIMD have)
#pragma unroll 2
            for (int kk = 0; kk < RB_KS; kk += AV) piece(kk);
        } else {
            for (int q = 0; q < n; ++q) {
                const float a = lds_elem<DT_IN>(arow, q);
#pragma unroll
                for (int c = 0; c < CW; ++c) acc[c] = __builtin_fmaf(a, bcol[c * BP + q], acc[c]);
            }
        }
    }

    const int64_t i = i0 + lane;
    if (i >= p.rows) return;
#pragma unroll
    for (int c = 0; c < CW; ++c) {
        const int64_t j = j0 + wc + c;
        if (j >= p.cols) continue;
        float v = acc[c];
        if constexpr (EPI == EPI_PARTIAL) {
            p.ws[(chunk * p.rows + i) * p.cols + j] = v;
        } else {
            if constexpr (EPI == EPI_FP8) {
                v = v * p.scale_a[0];
                v = v * p.scale_b[0];
                if (p.bias) v = v + load_elem<DT_OUT>(p.bias, j);  // bf16 bias
            } else {
                if (p.bias) v = v + load_elem<DT_IN>(p.bias, j);
            }
            store_elem<DT_OUT>(p.c, i * p.ldc + j, v);
        }
    }
}

// Pass 2 of the chunked dW and of the bias gradient: out = RNE( ((P0 + P1) +
// P2) + ... ) per element, chunks in ascending order.  Loads are issued CS_UN
// at a time so their latencies overlap; the additions stay in chunk order.
constexpr int CS_UN = 16;

template <int DT_OUT>
__global__ __launch_bounds__(64) void chunk_sum_kernel(const float *__restrict__ ws,
                                                        void *out, int64_t count,
                                                        int64_t nchunks) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        float s = ws[i];
        int64_t c = 1;
        for (; c + CS_UN <= nchunks; c += CS_UN) {
            float v[CS_UN];
#pragma unroll
            for (int u = 0; u < CS_UN; ++u) v[u] = ws[(c + u) * count + i];
#pragma unroll
            for (int u = 0; u < CS_UN; ++u) s = s + v[u];
        }
        for (; c < nchunks; ++c) s = s + ws[c * count + i];
        store_elem<DT_OUT>(out, i, s);
    }
}

// Grouped scalar tier (rublas tensor_grouped/mod.rs: one thread per output
// element, FP32 accumulation, one output rounding).
template <int DT>
__global__ __launch_bounds__(256) void grouped_fwd_scalar_kernel(GroupedScalarArgs p) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= p.m * p.n) return;
    const int64_t row = idx / p.n, col = idx % p.n;
    const uint32_t ex = p.row_experts[row];
    if ((int64_t)ex < p.e) {
        float acc = 0.0f;
        const int64_t wb = ((int64_t)ex * p.n + col) * p.k;
        for (int64_t r = 0; r < p.k; ++r)
            acc = __builtin_fmaf(load_elem<DT>(p.input, row * p.k + r),
                                 load_elem<DT>(p.weights, wb + r), acc);
        store_elem<DT>(p.out, idx, acc);
    } else {
        if constexpr (DT == DT_F32) static_cast<uint32_t *>(p.out)[idx] = 0u;
        else static_cast<uint16_t *>(p.out)[idx] = 0u;
    }
}

template <int DT>
__global__ __launch_bounds__(256) void grouped_dinput_scalar_kernel(GroupedScalarArgs p) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= p.m * p.k) return;
    const int64_t row = idx / p.k, col = idx % p.k;
    const uint32_t ex = p.row_experts[row];
    if ((int64_t)ex < p.e) {
        float acc = 0.0f;
        const int64_t wb = (int64_t)ex * p.n * p.k + col;
        for (int64_t r = 0; r < p.n; ++r)
            acc = __builtin_fmaf(load_elem<DT>(p.grad_out, row * p.n + r),
                                 load_elem<DT>(p.weights, wb + r * p.k), acc);
        store_elem<DT>(p.out, idx, acc);
    } else {
        if constexpr (DT == DT_F32) static_cast<uint32_t *>(p.out)[idx] = 0u;
        else static_cast<uint16_t *>(p.out)[idx] = 0u;
    }
}

template <int DT>
__global__ __launch_bounds__(256) void grouped_dweights_scalar_kernel(GroupedScalarArgs p) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= p.e * p.n * p.k) return;
    const int64_t ex = idx / (p.n * p.k);
    const int64_t col_n = (idx / p.k) % p.n, col_k = idx % p.k;
    // offsets are a caller invariant; clamping keeps a violated invariant from
    // reading outside the operands (the result is then simply wrong)
    int64_t r1 = p.offsets[ex + 1], r0 = p.offsets[ex];
    if (r1 > p.m) r1 = p.m;
    if (r0 > r1) r0 = r1;
    float acc = 0.0f;
    for (int64_t r = r0; r < r1; ++r)
        acc = __builtin_fmaf(load_elem<DT>(p.grad_out, r * p.n + col_n),
                             load_elem<DT>(p.input, r * p.k + col_k), acc);
    p.dweights[idx] = acc;
}

}  // namespace

#define BI_LAUNCH(kern, grid, block, stream, ...)                                   \
    do {                                                                             \
        hipLaunchKernelGGL(kern, dim3(grid), dim3(block), 0, stream, __VA_ARGS__);   \
    } while (0)

// narrow outputs with aligned rows of A contiguous along the reduction: 64-row
// workgroups of 4 to 8 waves, CW columns per wave (four while that still
// gives 1024 waves, else two, else one)
static hipError_t launch_scalar_rowblock(const ScalarGemmArgs &p, int dt_in, int dt_out,
                                         int epi, hipStream_t s) {
    const int64_t rblocks = (p.rows + 63) / 64;
    int cw = 1;
    for (int cand : {4, 2}) {
        // (e4m3: at most two, four columns' conversions spill)
        if (cand == 4 && dt_in == DT_E4M3) continue;
        if (rblocks * ((p.cols + cand - 1) / cand) * p.nchunks >= 1024) {
            cw = cand;
            break;
        }
    }
    // one wave per CW columns, split into enough column blocks of 4 to 8
    // waves to give the chip RB_WGS workgroups where the columns allow
    const int64_t waves = (p.cols + cw - 1) / cw;
    const int64_t rows_chunks = rblocks * p.nchunks;
    int64_t want = (RB_WGS + rows_chunks - 1) / rows_chunks;
    if (want < (waves + 7) / 8) want = (waves + 7) / 8;
    int64_t nw = (waves + want - 1) / want;
    nw = nw < 4 ? 4 : nw > 8 ? 8 : nw;
    const int64_t cblocks = (waves + nw - 1) / nw;
    const int64_t grid = rows_chunks * cblocks;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int nth = (int)(64 * nw);
#define RCASE(DI, DO, E)                                                                          \
    if (dt_in == DI && dt_out == DO && epi == E) {                                                \
        if (cw == 4) BI_LAUNCH((scalar_rowblock_kernel<DI, DO, E, 4>), grid, nth, s, p, cblocks);  \
        else if (cw == 2) BI_LAUNCH((scalar_rowblock_kernel<DI, DO, E, 2>), grid, nth, s, p, cblocks); \
        else BI_LAUNCH((scalar_rowblock_kernel<DI, DO, E, 1>), grid, nth, s, p, cblocks);          \
        return hipGetLastError();                                                                 \
    }
    RCASE(DT_F32, DT_F32, EPI_ROUND)
    RCASE(DT_BF16, DT_BF16, EPI_ROUND)
    RCASE(DT_F16, DT_F16, EPI_ROUND)
    RCASE(DT_F32, DT_F32, EPI_PARTIAL)
    RCASE(DT_BF16, DT_F32, EPI_PARTIAL)
    RCASE(DT_F16, DT_F32, EPI_PARTIAL)
#undef RCASE
    if (dt_in == DT_E4M3 && dt_out == DT_BF16 && epi == EPI_FP8) {
        if (cw == 2) BI_LAUNCH((scalar_rowblock_kernel<DT_E4M3, DT_BF16, EPI_FP8, 2>), grid, nth, s, p, cblocks);
        else BI_LAUNCH((scalar_rowblock_kernel<DT_E4M3, DT_BF16, EPI_FP8, 1>), grid, nth, s, p, cblocks);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

// narrow outputs (at most 64 columns): one row per lane
static hipError_t launch_scalar_narrow(const ScalarGemmArgs &p, int dt_in, int dt_out,
                                       int epi, hipStream_t s) {
    const int64_t rgroups = (p.rows + 255) / 256;
    // four columns per lane while that gives the chip 256 workgroups, else two
    const int cw = rgroups * ((p.cols + 3) / 4) * p.nchunks >= 256 ? 4 : 2;
    const int64_t grid = rgroups * ((p.cols + cw - 1) / cw) * p.nchunks;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int esz = dt_in == DT_F32 ? 4 : dt_in == DT_E4M3 ? 1 : 2;
    // rows of A contiguous along the reduction, 16-byte aligned, and so are
    // the chunk starts: the row-block kernel
    const bool vec = p.a_rs == 1 && reinterpret_cast<uintptr_t>(p.a) % 16 == 0 &&
                     (p.a_is * esz) % 16 == 0 && (p.nchunks == 1 || (p.chunk * esz) % 16 == 0);
    if (vec) return launch_scalar_rowblock(p, dt_in, dt_out, epi, s);
#define NCASE(DI, DO, E)                                                                    \
    if (dt_in == DI && dt_out == DO && epi == E) {                                          \
        if (cw == 4) BI_LAUNCH((scalar_narrow_kernel<DI, DO, E, 4>), grid, 256, s, p);      \
        else BI_LAUNCH((scalar_narrow_kernel<DI, DO, E, 2>), grid, 256, s, p);              \
        return hipGetLastError();                                                           \
    }
    NCASE(DT_F32, DT_F32, EPI_ROUND)
    NCASE(DT_BF16, DT_BF16, EPI_ROUND)
    NCASE(DT_F16, DT_F16, EPI_ROUND)
    NCASE(DT_F32, DT_F32, EPI_PARTIAL)
    NCASE(DT_BF16, DT_F32, EPI_PARTIAL)
    NCASE(DT_F16, DT_F32, EPI_PARTIAL)
    NCASE(DT_E4M3, DT_BF16, EPI_FP8)
#undef NCASE
    return hipErrorInvalidValue;
}

hipError_t launch_scalar_gemm(const ScalarGemmArgs &p, int dt_in, int dt_out, int epi,
                              hipStream_t s) {
    if (p.cols <= 64) return launch_scalar_narrow(p, dt_in, dt_out, epi, s);
    const int64_t tiles_j = (p.cols + ST - 1) / ST;
    // the tallest tile that gives at least 256 workgroups (the first that does
    // not fall below it), 16 rows if none does
    int tm = 16;
    for (int cand : {64, 32}) {
        if ((p.rows + cand - 1) / cand * tiles_j * p.nchunks >= 256) {
            tm = cand;
            break;
        }
    }
    ScalarGemmArgs a = p;
    a.tiles_i = (p.rows + tm - 1) / tm;
    a.tiles_j = tiles_j;
    const int64_t grid = a.tiles_i * a.tiles_j * a.nchunks;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
#define CASE(DI, DO, E)                                                                   \
    if (dt_in == DI && dt_out == DO && epi == E) {                                        \
        if (tm == 64) BI_LAUNCH((scalar_gemm_kernel<DI, DO, E, 64>), grid, 256, s, a);   \
        else if (tm == 32) BI_LAUNCH((scalar_gemm_kernel<DI, DO, E, 32>), grid, 256, s, a); \
        else BI_LAUNCH((scalar_gemm_kernel<DI, DO, E, 16>), grid, 256, s, a);            \
        return hipGetLastError();                                                         \
    }
    CASE(DT_F32, DT_F32, EPI_ROUND)
    CASE(DT_BF16, DT_BF16, EPI_ROUND)
    CASE(DT_F16, DT_F16, EPI_ROUND)
    CASE(DT_F32, DT_F32, EPI_PARTIAL)
    CASE(DT_BF16, DT_F32, EPI_PARTIAL)
    CASE(DT_F16, DT_F32, EPI_PARTIAL)
    CASE(DT_E4M3, DT_BF16, EPI_FP8)
#undef CASE
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_sum(const float *ws, void *out, int64_t count, int64_t nchunks,
                            int dt_out, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    // one-wave workgroups: short rows of partials still spread over many CUs
    int64_t grid = (count + 63) / 64;
    if (grid > (1 << 20)) grid = 1 << 20;
    if (dt_out == DT_F32) BI_LAUNCH(chunk_sum_kernel<DT_F32>, grid, 64, s, ws, out, count, nchunks);
    else if (dt_out == DT_BF16) BI_LAUNCH(chunk_sum_kernel<DT_BF16>, grid, 64, s, ws, out, count, nchunks);
    else if (dt_out == DT_F16) BI_LAUNCH(chunk_sum_kernel<DT_F16>, grid, 64, s, ws, out, count, nchunks);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_grouped_scalar(const GroupedScalarArgs &p, int op, int dt, hipStream_t s) {
    int64_t count = op == 0 ? p.m * p.n : (op == 1 ? p.m * p.k : p.e * p.n * p.k);
    if (count <= 0) return hipSuccess;
    const int64_t grid = (count + 255) / 256;
#define GCASE(D)                                                                           \
    if (dt == D) {                                                                         \
        if (op == 0) BI_LAUNCH(grouped_fwd_scalar_kernel<D>, grid, 256, s, p);             \
        else if (op == 1) BI_LAUNCH(grouped_dinput_scalar_kernel<D>, grid, 256, s, p);     \
        else BI_LAUNCH(grouped_dweights_scalar_kernel<D>, grid, 256, s, p);                \
        return hipGetLastError();                                                          \
    }
    GCASE(DT_F32)
    GCASE(DT_BF16)
    GCASE(DT_F16)
#undef GCASE
    return hipErrorInvalidValue;
}

}  // namespace bi
