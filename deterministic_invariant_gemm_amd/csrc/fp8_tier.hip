// fp8 e4m3fn GEMM with per-tensor dequantisation scales and bf16 output
// (AstrAI fp8_mm.cu: fp8_mm on e4m3fn a[M,K] and b[N,K] giving bf16 [M,N];
// fp8_gemm_into: per-tensor f32 scales applied inside the GEMM,
// D = A_SCALE * B_SCALE * A * B, f32 compute type).
//
//   y[m,n] = RNE_bf16( ((sum_k a[m,k] * bt[n,k]) * scale_a) * scale_b )
//
// MFMA tier, f32 accumulation, each output element's accumulator starting at
// +0, reduction steps in ascending k:
//   * default (FAST = false): every e4m3 code is widened exactly to bf16 in
//     registers and each 32-deep step is two v_mfma_f32_32x32x16_bf16, which
//     add the exact products at f32 precision: lane half h holds the 16 codes
//     32t + 16h .. + 15 of step t, the first MFMA takes codes 0..7 of each
//     half, the second codes 8..15 (so each lane reads 16 bytes of LDS);
//   * FAST = true (opt-in): each 64-deep step is one
//     v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in the OCP e4m3
//     format (format code 0), which aligns the products of each group of 8
//     reduction indices to the group's largest before adding them.
// Every tile shape, here and in the direct-load kernel (fp8_dl.hip), issues the
// same sequence for a path, so tile shape and M never change the bits.  Both operands are k-contiguous, so staging is a
// straight 16-byte copy into a k-grouped, XOR-swizzled LDS layout (16 fp8
// values per slot); an operand fragment of one lane is two adjacent slots.
// Pipeline: two LDS buffers, one slice in registers ahead, one barrier per
// slice; branch-free vector loads for interior tiles, masked loads at edges.
#include "device_common.hpp"
#include "kernels.hpp"

namespace bi {

namespace {

constexpr int BK = 128;      // reduction slice per LDS stage (bytes = values)
constexpr int KG = BK / 16;  // 16-value groups per slice
constexpr int NT = 256;

__device__ __forceinline__ int swz(int row, int kg) {
    return (row & ~7) | ((row ^ (row >> 3) ^ kg) & 7);
}

template <int R>
struct Stage8 {
    static constexpr int PER_THREAD = R * KG / NT;
    static_assert((R * KG) % NT == 0, "tile rows must fill the workgroup");
    u32x4 reg[PER_THREAD];

    // whole tile and slice in range, 16-byte aligned rows: vector loads
    __device__ __forceinline__ void load_fast(const uint8_t *p, int64_t ld, int64_t row0,
                                              int64_t rk, int t) {
#pragma unroll
        for (int q = 0; q < PER_THREAD; ++q) {
            const int c = t + NT * q;
            const int row = c / KG, kg = c % KG;
            reg[q] = *reinterpret_cast<const u32x4 *>(p + (row0 + row) * ld + rk + 16 * kg);
        }
    }
    // masked: clamped addresses, zero outside [row0,row_end) x [rk,r_end)
    __device__ __forceinline__ void load_masked(const uint8_t *p, int64_t ld, int64_t row0,
                                                int64_t row_end, int64_t rk, int64_t r_end,
                                                int t) {
#pragma unroll
        for (int q = 0; q < PER_THREAD; ++q) {
            const int c = t + NT * q;
            const int row = c / KG, kg = c % KG;
            const int64_t gi = row0 + row;
            const int64_t gic = gi < row_end ? gi : row_end - 1;
            uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const int64_t gr = rk + 16 * kg + x;
                const int64_t grc = gr < r_end ? gr : r_end - 1;
                const uint32_t v = p[gic * ld + grc];
                w[x >> 2] |= ((gi < row_end && gr < r_end) ? v : 0u) << (8 * (x & 3));
            }
            reg[q] = u32x4{w[0], w[1], w[2], w[3]};
        }
    }
    __device__ __forceinline__ void load(const uint8_t *p, int64_t ld, int64_t row0,
                                         int64_t row_end, int64_t rk, int64_t r_end,
                                         bool interior, int t) {
        if (interior && rk + BK <= r_end) load_fast(p, ld, row0, rk, t);
        else load_masked(p, ld, row0, row_end, rk, r_end, t);
    }
    __device__ __forceinline__ void store(u32x4 *lds, int t) const {
#pragma unroll
        for (int q = 0; q < PER_THREAD; ++q) {
            const int c = t + NT * q;
            const int row = c / KG, kg = c % KG;
            lds[kg * R + swz(row, kg)] = reg[q];
        }
    }
};

template <int BM, int BN, int WGM, int WGN, bool FAST>
__global__ __launch_bounds__(NT) void fp8_gemm_kernel(Fp8Args p) {
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    static_assert(WGM * WGN == 4 && FM * 32 == WTM && FN * 32 == WTN, "wave tiling");

    __shared__ u32x4 lds_a[2][KG * BM];
    __shared__ u32x4 lds_b[2][KG * BN];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    const int64_t tile = xcd_remap(blockIdx.x, gridDim.x);
    constexpr int64_t GROUP = 4;
    const int64_t per_group = GROUP * p.tiles_j;
    const int64_t g = tile / per_group, first = g * GROUP;
    const int64_t gsz = p.tiles_i - first < GROUP ? p.tiles_i - first : GROUP;
    const int64_t in_g = tile % per_group;
    const int64_t row0 = (first + in_g % gsz) * BM;
    const int64_t col0 = (in_g / gsz) * BN;

    Stage8<BM> sa;
    Stage8<BN> sb;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const bool int_a = p.vec != 0 && row0 + BM <= p.m;
    const bool int_b = p.vec != 0 && col0 + BN <= p.n;
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int64_t nst = (p.k + BK - 1) / BK;

    if (nst > 0) {
        sa.load(p.a, p.k, row0, p.m, 0, p.k, int_a, t);
        sb.load(p.bt, p.k, col0, p.n, 0, p.k, int_b, t);
        sa.store(lds_a[0], t);
        sb.store(lds_b[0], t);
        if (nst > 1) {
            sa.load(p.a, p.k, row0, p.m, BK, p.k, int_a, t);
            sb.load(p.bt, p.k, col0, p.n, BK, p.k, int_b, t);
        }
        __syncthreads();
    }
    for (int64_t s = 0; s < nst; ++s) {
        const int cur = (int)(s & 1);
        if (s + 1 < nst) {
            sa.store(lds_a[cur ^ 1], t);
            sb.store(lds_b[cur ^ 1], t);
            if (s + 2 < nst) {
                sa.load(p.a, p.k, row0, p.m, (s + 2) * BK, p.k, int_a, t);
                sb.load(p.bt, p.k, col0, p.n, (s + 2) * BK, p.k, int_b, t);
            }
        }
        const u32x4 *la = lds_a[cur];
        const u32x4 *lb = lds_b[cur];
        if constexpr (FAST) {
#pragma unroll
            for (int kk = 0; kk < BK / 64; ++kk) {
                // this lane's 32 reduction values of the step: groups kg0, kg0 + 1
                const int kg0 = 4 * kk + 2 * lhalf;
                i32x8 fa[FM], fb[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int row = wm * WTM + 32 * i + lrow;
                    const u32x4 lo = la[kg0 * BM + swz(row, kg0)];
                    const u32x4 hi = la[(kg0 + 1) * BM + swz(row, kg0 + 1)];
                    fa[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                }
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int row = wn * WTN + 32 * j + lrow;
                    const u32x4 lo = lb[kg0 * BN + swz(row, kg0)];
                    const u32x4 hi = lb[(kg0 + 1) * BN + swz(row, kg0 + 1)];
                    fb[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        // B fragment first: the lane then holds 4 consecutive output
                        // columns of one row.  Format codes 0/0: both operands OCP
                        // fp8 e4m3; no block scales.
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fb[j], fa[i], acc[i][j], 0, 0, 0, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < BK / 32; ++kk) {
                // 32-deep step kk: this lane's 16 codes, group 2 kk + lhalf, widened
                // exactly to bf16; the first MFMA takes codes 0..7 of each lane
                // half, the second codes 8..15 (the direct-load kernel's order)
                const int g = 2 * kk + lhalf;
                u32x4 fa[2][FM], fb[2][FN];
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int row = wm * WTM + 32 * i + lrow;
                    const u32x4 w = la[g * BM + swz(row, g)];
                    fa[0][i] = e4m3x8_to_bf16x8(u32x2{w[0], w[1]});
                    fa[1][i] = e4m3x8_to_bf16x8(u32x2{w[2], w[3]});
                }
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int row = wn * WTN + 32 * j + lrow;
                    const u32x4 w = lb[g * BN + swz(row, g)];
                    fb[0][j] = e4m3x8_to_bf16x8(u32x2{w[0], w[1]});
                    fb[1][j] = e4m3x8_to_bf16x8(u32x2{w[2], w[3]});
                }
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(bf16x8, fb[h][j]),
                                __builtin_bit_cast(bf16x8, fa[h][i]), acc[i][j], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    const float sa_v = p.scale_a[0], sb_v = p.scale_b[0];
    const bool vec_c = p.vec_c != 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t gi = row0 + wm * WTM + 32 * i + lrow;
        if (gi >= p.m) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int64_t gj = col0 + wn * WTN + 32 * j + 8 * g4 + 4 * lhalf;
                if (gj >= p.n) continue;
                uint32_t h[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    float v = acc[i][j][4 * g4 + x] * sa_v;
                    v = v * sb_v;
                    if (p.bias && gj + x < p.n) v = v + bf16_bits_to_f32(p.bias[gj + x]);
                    h[x] = f32_to_bf16_bits(v);
                }
                uint16_t *pc = p.c + gi * p.n + gj;
                if (vec_c && gj + 4 <= p.n) {
                    *reinterpret_cast<u32x2 *>(pc) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
                } else {
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        if (gj + x < p.n) pc[x] = (uint16_t)h[x];
                }
            }
        }
    }
}

}  // namespace

template <bool FAST>
hipError_t launch_fp8_tile(const Fp8Args &p, int tile_id, int64_t grid, hipStream_t s) {
    switch (tile_id) {
    case 1: hipLaunchKernelGGL((fp8_gemm_kernel<256, 256, 2, 2, FAST>), dim3(grid), dim3(NT), 0, s, p); break;
    case 4: hipLaunchKernelGGL((fp8_gemm_kernel<128, 128, 2, 2, FAST>), dim3(grid), dim3(NT), 0, s, p); break;
    case 6: hipLaunchKernelGGL((fp8_gemm_kernel<64, 64, 2, 2, FAST>), dim3(grid), dim3(NT), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_fp8_gemm(const Fp8Args &p, int tile_id, bool fast, hipStream_t s) {
    const int64_t grid = p.tiles_i * p.tiles_j;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return fast ? launch_fp8_tile<true>(p, tile_id, grid, s) : launch_fp8_tile<false>(p, tile_id, grid, s);
}

}  // namespace bi
