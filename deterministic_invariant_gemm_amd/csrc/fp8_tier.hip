// fp8 e4m3fn GEMM with per-tensor dequantisation scales and bf16 output
// (AstrAI fp8_mm.cu: fp8_mm on e4m3fn a[M,K] and b[N,K] giving bf16 [M,N];
// fp8_gemm_into: per-tensor f32 scales applied inside the GEMM,
// D = A_SCALE * B_SCALE * A * B, f32 compute type).
//
//   y[m,n] = RNE_bf16( ((sum_k a[m,k] * bt[n,k]) * scale_a) * scale_b )
//
// MFMA tier: v_mfma_f32_32x32x64_f8f6f4 with both operands in the OCP e4m3
// format (format code 0), f32 accumulation.  Each output element's accumulator
// starts at +0 and receives one MFMA per 64-deep reduction step, steps in
// ascending k; every tile shape issues the same sequence, so tile shape and M
// never change the bits.  Both operands are k-contiguous, so staging is a
// straight 16-byte copy into a k-grouped, XOR-swizzled LDS layout (16 fp8
// values per slot); an operand fragment of one lane is two adjacent slots.
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

// 16 consecutive fp8 codes from p[0], zero beyond `count`.
__device__ __forceinline__ u32x4 load16(const uint8_t *p, int count, bool vec) {
    if (count >= 16 && vec) return *reinterpret_cast<const u32x4 *>(p);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (i < count) w[i >> 2] |= (uint32_t)p[i] << (8 * (i & 3));
    return u32x4{w[0], w[1], w[2], w[3]};
}

template <int R>
struct Stage8 {
    static constexpr int PER_THREAD = R * KG / NT;
    static_assert((R * KG) % NT == 0, "tile rows must fill the workgroup");
    u32x4 reg[PER_THREAD];

    __device__ __forceinline__ void load(const uint8_t *p, int64_t ld, int64_t row0,
                                         int64_t row_end, int64_t rk, int64_t r_end, bool vec,
                                         int t) {
#pragma unroll
        for (int q = 0; q < PER_THREAD; ++q) {
            const int c = t + NT * q;
            const int row = c / KG, kg = c % KG;
            const int64_t gi = row0 + row, gr = rk + 16 * kg;
            int cnt = gi < row_end ? (int)(r_end - gr < 16 ? r_end - gr : 16) : 0;
            if (cnt < 0) cnt = 0;
            reg[q] = cnt > 0 ? load16(p + gi * ld + gr, cnt, vec) : u32x4{0u, 0u, 0u, 0u};
        }
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

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(NT) void fp8_gemm_kernel(Fp8Args p) {
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    static_assert(WGM * WGN == 4 && FM * 32 == WTM && FN * 32 == WTN, "wave tiling");

    __shared__ u32x4 lds_a[KG * BM];
    __shared__ u32x4 lds_b[KG * BN];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    const int64_t tiles = p.tiles_i * p.tiles_j;
    const int64_t tile = xcd_remap(blockIdx.x, gridDim.x);
    constexpr int64_t GROUP = 4;
    const int64_t per_group = GROUP * p.tiles_j;
    const int64_t g = tile / per_group, first = g * GROUP;
    const int64_t gsz = p.tiles_i - first < GROUP ? p.tiles_i - first : GROUP;
    const int64_t in_g = tile % per_group;
    const int64_t row0 = (first + in_g % gsz) * BM;
    const int64_t col0 = (in_g / gsz) * BN;
    (void)tiles;

    Stage8<BM> sa;
    Stage8<BN> sb;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const bool vec = p.vec != 0;
    if (p.k > 0) {
        sa.load(p.a, p.k, row0, p.m, 0, p.k, vec, t);
        sb.load(p.bt, p.k, col0, p.n, 0, p.k, vec, t);
    }
    const int lrow = lane & 31, lhalf = lane >> 5;
    for (int64_t rk = 0; rk < p.k; rk += BK) {
        sa.store(lds_a, t);
        sb.store(lds_b, t);
        __syncthreads();
        if (rk + BK < p.k) {
            sa.load(p.a, p.k, row0, p.m, rk + BK, p.k, vec, t);
            sb.load(p.bt, p.k, col0, p.n, rk + BK, p.k, vec, t);
        }
#pragma unroll
        for (int kk = 0; kk < BK / 64; ++kk) {
            // this lane's 32 reduction values of the step: groups kg0, kg0 + 1
            const int kg0 = 4 * kk + 2 * lhalf;
            i32x8 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * WTM + 32 * i + lrow;
                const u32x4 lo = lds_a[kg0 * BM + swz(row, kg0)];
                const u32x4 hi = lds_a[(kg0 + 1) * BM + swz(row, kg0 + 1)];
                fa[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * WTN + 32 * j + lrow;
                const u32x4 lo = lds_b[kg0 * BN + swz(row, kg0)];
                const u32x4 hi = lds_b[(kg0 + 1) * BN + swz(row, kg0 + 1)];
                fb[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    // format codes 0/0: both operands OCP fp8 e4m3; no block scales
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[i], fb[j], acc[i][j], 0, 0, 0, 0, 0, 0);
        }
        __syncthreads();
    }

    const float sa_v = p.scale_a[0], sb_v = p.scale_b[0];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t gj = col0 + wn * WTN + 32 * j + lrow;
        if (gj >= p.n) continue;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t gi = row0 + wm * WTM + 32 * i + 8 * (v >> 2) + 4 * lhalf + (v & 3);
                if (gi >= p.m) continue;
                float val = acc[i][j][v] * sa_v;
                val = val * sb_v;
                p.c[gi * p.n + gj] = (uint16_t)f32_to_bf16_bits(val);
            }
        }
    }
}

}  // namespace

hipError_t launch_fp8_gemm(const Fp8Args &p, int tile_id, hipStream_t s) {
    const int64_t grid = p.tiles_i * p.tiles_j;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    switch (tile_id) {
    case 1: hipLaunchKernelGGL((fp8_gemm_kernel<256, 256, 2, 2>), dim3(grid), dim3(NT), 0, s, p); break;
    case 4: hipLaunchKernelGGL((fp8_gemm_kernel<128, 128, 2, 2>), dim3(grid), dim3(NT), 0, s, p); break;
    case 6: hipLaunchKernelGGL((fp8_gemm_kernel<64, 64, 2, 2>), dim3(grid), dim3(NT), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace bi
