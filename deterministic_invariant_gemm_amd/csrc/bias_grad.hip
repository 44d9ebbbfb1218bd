// Bias gradient of the training linear (ViperLLM ffma.py, _FFMAAddmm.backward:
// the bias gradient is the column sum of the output gradient, accumulated in
// f32 and cast back to the bias dtype once).  The sum runs over the batch, so
// it is deterministic for a fixed m but not batch-invariant; the order is fixed
// by m alone:
//   * rows are cut into chunks of BG_CHUNK rows (the same for every shape);
//   * inside a chunk, thread row t (0..63) adds rows t, t+64, ... in ascending
//     order; the eight thread rows of a wave are combined by a butterfly over
//     lane distances 8, 16, 32 (lanes 0..7 keep the result), then the eight
//     waves' sums are added in ascending wave order;
//   * with one chunk the sum is rounded and stored here; otherwise each chunk
//     writes an f32 partial and the chunk-sum kernel adds the partials in
//     ascending chunk order and rounds once.
// HBM-bound: dY is read once; the partials add 4 bytes per 256 elements.
#include "device_common.hpp"
#include "kernels.hpp"

namespace bi {

namespace {

constexpr int BG_T = 512;                  // threads per workgroup (eight waves)
constexpr int BG_VEC = 8;                  // columns per thread
constexpr int BG_TPR = 8;                  // threads per row: 128 contiguous bytes of bf16
constexpr int BG_COLS = BG_TPR * BG_VEC;   // columns per workgroup
constexpr int BG_ROWS = BG_T / BG_TPR;     // thread rows (rows read in parallel)
constexpr int BG_PER = BG_CHUNK / BG_ROWS; // rows per thread per chunk

template <int DT>
__device__ __forceinline__ void load8(const void *base, int64_t idx, float v[BG_VEC]) {
    if constexpr (DT == DT_F32) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const float *>(base) + idx);
        const u32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(w[j]);
    } else {
        const u32x4 a = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + idx));
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (DT == DT_BF16) {
                v[2 * j] = bf16_bits_to_f32(w[j] & 0xffffu);
                v[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
            } else {
                v[2 * j] = f16_bits_to_f32(w[j] & 0xffffu);
                v[2 * j + 1] = f16_bits_to_f32(w[j] >> 16);
            }
        }
    }
}

// VEC: dy 16-byte aligned and n % 8 == 0 (a thread's 8 columns are in one or
// two 16-byte pieces, all inside the row).  The element path adds the same
// values in the same order, so both give the same bits.
template <int DT, bool VEC>
__global__ __launch_bounds__(BG_T) void bias_grad_kernel(const void *__restrict__ dy, int64_t m,
                                                         int64_t n, int64_t nchunks,
                                                         float *__restrict__ ws, void *out) {
    __shared__ float red[BG_T / 64][BG_COLS];
    const int tr = threadIdx.x / BG_TPR, tc = threadIdx.x % BG_TPR;
    const int64_t ncb = (n + BG_COLS - 1) / BG_COLS;
    for (int64_t b = blockIdx.x; b < nchunks * ncb; b += gridDim.x) {
        const int64_t cb = b % ncb, chunk = b / ncb;
        const int64_t col = cb * BG_COLS + tc * BG_VEC;
        const int64_t row0 = chunk * BG_CHUNK + tr;
        float acc[BG_VEC];
#pragma unroll
        for (int j = 0; j < BG_VEC; ++j) acc[j] = 0.0f;
        if (VEC && col < n) {
            float v[BG_PER][BG_VEC];
#pragma unroll
            for (int r = 0; r < BG_PER; ++r) {
                const int64_t row = row0 + (int64_t)r * BG_ROWS;
                if (row < m) load8<DT>(dy, row * n + col, v[r]);
            }
#pragma unroll
            for (int r = 0; r < BG_PER; ++r) {
                if (row0 + (int64_t)r * BG_ROWS < m) {
#pragma unroll
                    for (int j = 0; j < BG_VEC; ++j) acc[j] = acc[j] + v[r][j];
                }
            }
        } else if (!VEC) {
            for (int r = 0; r < BG_PER; ++r) {
                const int64_t row = row0 + (int64_t)r * BG_ROWS;
                if (row >= m) break;
#pragma unroll
                for (int j = 0; j < BG_VEC; ++j)
                    if (col + j < n) acc[j] = acc[j] + load_elem<DT>(dy, row * n + col + j);
            }
        }
#pragma unroll
        for (int j = 0; j < BG_VEC; ++j) {
#pragma unroll
            for (int d = BG_TPR; d < 64; d *= 2) acc[j] = acc[j] + __shfl_xor(acc[j], d, 64);
        }
        if ((threadIdx.x & 63) < BG_TPR) {
#pragma unroll
            for (int j = 0; j < BG_VEC; ++j) red[threadIdx.x / 64][tc * BG_VEC + j] = acc[j];
        }
        __syncthreads();
        const int64_t c = cb * BG_COLS + threadIdx.x;
        if (threadIdx.x < BG_COLS && c < n) {
            float s = red[0][threadIdx.x];
#pragma unroll
            for (int w = 1; w < BG_T / 64; ++w) s = s + red[w][threadIdx.x];
            if (nchunks == 1) store_elem<DT>(out, c, s);
            else ws[chunk * n + c] = s;
        }
        __syncthreads();
    }
}

template <int DT>
hipError_t launch_bias_grad_dt(const void *dy, int64_t m, int64_t n, int64_t nchunks, float *ws,
                               void *out, bool vec, hipStream_t s) {
    const int64_t blocks = nchunks * ((n + BG_COLS - 1) / BG_COLS);
    const int64_t grid = blocks < (1 << 20) ? blocks : (1 << 20);
    if (vec)
        hipLaunchKernelGGL((bias_grad_kernel<DT, true>), dim3(grid), dim3(BG_T), 0, s, dy, m, n,
                           nchunks, ws, out);
    else
        hipLaunchKernelGGL((bias_grad_kernel<DT, false>), dim3(grid), dim3(BG_T), 0, s, dy, m,
                           n, nchunks, ws, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bias_grad(const void *dy, int64_t m, int64_t n, int64_t nchunks, float *ws,
                            void *out, int dt, bool vec, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipError_t e;
    if (dt == DT_F32) e = launch_bias_grad_dt<DT_F32>(dy, m, n, nchunks, ws, out, vec, s);
    else if (dt == DT_BF16) e = launch_bias_grad_dt<DT_BF16>(dy, m, n, nchunks, ws, out, vec, s);
    else if (dt == DT_F16) e = launch_bias_grad_dt<DT_F16>(dy, m, n, nchunks, ws, out, vec, s);
    else return hipErrorInvalidValue;
    if (e != hipSuccess || nchunks <= 1) return e;
    return launch_chunk_sum(ws, out, n, nchunks, dt, s);
}

}  // namespace bi
