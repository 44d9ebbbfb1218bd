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

// Narrow outputs (at most 64 columns, such as a 48-wide layer).  The tiled
// kernel above would leave the columns past the output's width idle in every
// 64-column tile and make few tiles; here a lane owns ONE row and CW adjacent
// columns (CW = 4, or 2 when that gives too few workgroups), a workgroup 256
// consecutive rows (one per lane of its four waves) of the same columns.  The
// B values of a reduction index are the same for every lane: they are staged
// per slice into LDS and read back as one broadcast LDS read per reduction
// index; each lane's A values come straight from memory into
// registers, 16 bytes at a time along the reduction when rows are contiguous
// and aligned (VEC), one value per reduction index otherwise (coalesced across
// lanes when A is contiguous along its rows, as in dW).  The next slice's A and
// B are loaded while the current one is multiplied; a partial last slice loads
// each value as it multiplies it.  Each output is the same chain as in the
// tiled kernel: fmaf over the reduction indices of its range in ascending
// order from +0, nothing past the range.

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

template <int DT_IN, int DT_OUT, int EPI, int CW, bool VEC>
__global__ __launch_bounds__(256) void scalar_narrow_kernel(ScalarGemmArgs p) {
    constexpr int ESZ = DT_IN == DT_F32 ? 4 : DT_IN == DT_E4M3 ? 1 : 2;
    // reduction indices per staged slice: 256 bytes of each lane's A row when
    // it is loaded 16 bytes at a time, 64 values otherwise
    constexpr int NR_SL = VEC ? 256 / ESZ : 64;
    constexpr int NBS = (NR_SL * CW + 255) / 256;  // B values staged per thread
    constexpr int AV = 16 / ESZ;      // A values per 16-byte load
    constexpr int NV = NR_SL / AV;    // 16-byte loads per lane and slice
    constexpr int NA = VEC ? 1 : NR_SL;
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
    u32x4 av_next[VEC ? NV : 1], av_cur[VEC ? NV : 1];
    float as_next[NA], as_cur[NA];
    auto load_a = [&](int64_t rs) {
        if constexpr (VEC) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(
                static_cast<const char *>(p.a) + (ic * p.a_is + rs) * ESZ);
#pragma unroll
            for (int v = 0; v < NV; ++v) av_next[v] = src[v];
        } else {
#pragma unroll
            for (int q = 0; q < NR_SL; ++q)
                as_next[q] = load_elem<DT_IN>(p.a, ic * p.a_is + (rs + q) * p.a_rs);
        }
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
            if constexpr (VEC) {
#pragma unroll
                for (int v = 0; v < NV; ++v) av_cur[v] = av_next[v];
            } else {
#pragma unroll
                for (int q = 0; q < NR_SL; ++q) as_cur[q] = as_next[q];
            }
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
                    const int rr = r0 + u;
                    float a;
                    if constexpr (VEC) a = vec_elem<DT_IN>(av_cur[rr / AV], rr % AV);
                    else a = as_cur[rr];
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
    // 16-byte loads of A along the reduction: contiguous, aligned rows and
    // chunk starts
    const bool vec = p.a_rs == 1 && reinterpret_cast<uintptr_t>(p.a) % 16 == 0 &&
                     (p.a_is * esz) % 16 == 0 && (p.nchunks == 1 || (p.chunk * esz) % 16 == 0);
#define NCASE(DI, DO, E)                                                                    \
    if (dt_in == DI && dt_out == DO && epi == E) {                                          \
        if (cw == 4 && vec) BI_LAUNCH((scalar_narrow_kernel<DI, DO, E, 4, true>), grid, 256, s, p);  \
        else if (cw == 4) BI_LAUNCH((scalar_narrow_kernel<DI, DO, E, 4, false>), grid, 256, s, p);   \
        else if (vec) BI_LAUNCH((scalar_narrow_kernel<DI, DO, E, 2, true>), grid, 256, s, p);        \
        else BI_LAUNCH((scalar_narrow_kernel<DI, DO, E, 2, false>), grid, 256, s, p);                \
        return hipGetLastError();                                                           \
    }
    NCASE(DT_F32, DT_F32, EPI_ROUND)
    NCASE(DT_BF16, DT_BF16, EPI_ROUND)
    NCASE(DT_F16, DT_F16, EPI_ROUND)
    NCASE(DT_F32, DT_F32, EPI_PARTIAL)
    NCASE(DT_BF16, DT_F32, EPI_PARTIAL)
    NCASE(DT_F16, DT_F32, EPI_PARTIAL)
#undef NCASE
    // e4m3 codes one at a time (16-byte loads of 16 codes cost registers the
    // conversions need)
    if (dt_in == DT_E4M3 && dt_out == DT_BF16 && epi == EPI_FP8) {
        if (cw == 4) BI_LAUNCH((scalar_narrow_kernel<DT_E4M3, DT_BF16, EPI_FP8, 4, false>), grid, 256, s, p);
        else BI_LAUNCH((scalar_narrow_kernel<DT_E4M3, DT_BF16, EPI_FP8, 2, false>), grid, 256, s, p);
        return hipGetLastError();
    }
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
