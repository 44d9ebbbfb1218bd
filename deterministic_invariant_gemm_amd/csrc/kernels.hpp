// Internal interface between the C ABI (bi_api.cpp) and the kernel files.
// Every launch_* function enqueues on the given stream and returns the HIP
// status of the launch; none of them allocates or synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

// Generic strided scalar GEMM  C(i,j) = sum_r A(i,r) B(r,j)  over the rows of
// one reduction chunk [chunk*c, min((chunk+1)*c, red)).
struct ScalarGemmArgs {
    const void *a;
    int64_t a_is, a_rs;  // A(i,r) = a[i*a_is + r*a_rs]
    const void *b;
    int64_t b_rs, b_js;  // B(r,j) = b[r*b_rs + j*b_js]
    const void *bias;    // [cols] of the input dtype, or null
    const float *scale_a, *scale_b;  // fp8 dequantisation scales (device)
    void *c;
    int64_t ldc;
    float *ws;  // f32 chunk partials [nchunks][rows][cols] (EPI_PARTIAL)
    int64_t rows, cols, red;
    int64_t chunk, nchunks;
    int64_t tiles_i, tiles_j;
};

struct GroupedScalarArgs {
    const void *input, *weights, *grad_out;
    const uint32_t *row_experts, *offsets;
    void *out;        // y [m,n] or dinput [m,k]
    float *dweights;  // [e,n,k]
    int64_t m, k, n, e;
};

// MFMA tier (bf16 / f16): C(i,j) = sum_r A(i,r) B(j,r).
//   A "reduction-contiguous":  A(i,r) = a[i*lda + r];  else A(i,r) = a[r*lda + i]
//   B "reduction-contiguous":  B(j,r) = b[j*ldb + r];  else B(j,r) = b[r*ldb + j]
// Grouped mode (offsets != null): the row range of C is cut into expert
// segments [offsets[x], offsets[x+1]); tiles are anchored at segment starts,
// B is advanced by x*b_expert_stride, rows in [offsets[e], rows) are written as
// +0.  Expert-reduction mode (red_offsets != null): tile z = expert x reduces
// over r in [red_offsets[x], red_offsets[x+1]), A/B rows are global, C is
// advanced by x*c_expert_stride.
struct MfmaArgs {
    const void *a;
    int64_t lda;
    const void *b;
    int64_t ldb;
    void *c;
    int64_t ldc;
    const void *bias;  // [cols] of the operand dtype or null
    float *ws;         // f32 partials [nchunks][rows][cols]
    int64_t rows, cols, red;
    int64_t chunk, nchunks;
    int64_t tiles_i, tiles_j;
    // grouped forward / dinput
    const uint32_t *offsets;
    int64_t n_experts;
    int64_t b_expert_stride;
    int64_t seg_tiles;  // tiles_i bound: ceil(rows/BM) + n_experts
    // grouped dweights
    const uint32_t *red_offsets;
    int64_t c_expert_stride;
    int vec_a, vec_b;  // 16-byte vector loads allowed for A / B
    int vec_c;         // 8-byte (16-bit outputs) / 16-byte (f32) vector stores allowed
    // bytes readable from a / b (direct-load kernels: reads past them return zero)
    int64_t a_bytes, b_bytes;
    // fp8: per-tensor dequantisation scales (device f32 scalars)
    const float *scale_a, *scale_b;
};

// Row tiles per XCD group of a segment-anchored launch (grouped forward and
// dinput), and the row tiles its grid covers: seg_tiles rounded up to whole
// rounds of 8 groups, one group per XCD.
constexpr int64_t SEG_GROUP = 4;
__host__ __device__ constexpr int64_t seg_grid_rows(int64_t seg_tiles) {
    return (seg_tiles + 8 * SEG_GROUP - 1) / (8 * SEG_GROUP) * (8 * SEG_GROUP);
}

struct Fp8Args {
    const uint8_t *a;   // [m,k]
    const uint8_t *bt;  // [n,k]
    uint16_t *c;        // [m,n] bf16
    const float *scale_a, *scale_b;
    const uint16_t *bias;  // [n] bf16 or null, added after the scales
    int64_t m, n, k;
    int64_t tiles_i, tiles_j;
    int vec;    // 16-byte vector loads allowed
    int vec_c;  // 8-byte vector stores allowed
};

hipError_t launch_scalar_gemm(const ScalarGemmArgs &p, int dt_in, int dt_out, int epi,
                              hipStream_t s);
hipError_t launch_chunk_sum(const float *ws, void *out, int64_t count, int64_t nchunks,
                            int dt_out, hipStream_t s);
hipError_t launch_grouped_scalar(const GroupedScalarArgs &p, int op, int dt, hipStream_t s);

// Tile shapes of the MFMA tier.  All use v_mfma_f32_32x32x16_{bf16,f16} with
// the same ascending 16-deep reduction steps, so they give identical bits.
struct TileShape {
    int id, bm, bn;
};
const TileShape *mfma_tile(int id);  // null for an unknown id

// layout: bit 0 = A reduction-contiguous, bit 1 = B reduction-contiguous.
// epi: 0 round to dtype (+bias), 1 f32 partial into ws, 2 f32 into c (dweights).
hipError_t launch_mfma_gemm(const MfmaArgs &p, int tile_id, int dt, int layout, int epi,
                            hipStream_t s);

// dX (px: both operands reduction-contiguous, rounded) and dW (pw: both
// strided, rounded, one chunk) of one linear layer in one launch, for the
// direct-load tile pairs mfma_backward_pair() accepts (bf16 / f16); bits equal
// those of the two launches.  hipErrorNotSupported (nothing launched) otherwise.
bool mfma_backward_pair(int tile_x, int tile_w, int dt);
hipError_t launch_mfma_backward(const MfmaArgs &px, int tile_x, const MfmaArgs &pw, int tile_w,
                                int dt, hipStream_t s);

// Grouped dinput (pd: segment-anchored rows) and f32 dweights (pw: expert-local
// reduction) in one launch, for the direct-load tile pair
// mfma_grouped_backward_pair() accepts (bf16 / f16); bits equal those of the
// two launches.  hipErrorNotSupported (nothing launched) otherwise.
bool mfma_grouped_backward_pair(int tile_d, int tile_w, int dt);
hipError_t launch_mfma_grouped_backward(const MfmaArgs &pd, int tile_d, const MfmaArgs &pw,
                                        int tile_w, int dt, hipStream_t s);

// Grouped forward on tile 112 (256x256, segment-anchored rows) when its grid
// has more slots than one round of kGroupedSplitCUs workgroups: in one launch,
// the slots of the whole rounds run as 256x256 tiles and, if the work left
// over (counted on the device from the offsets) fills at most half a round,
// the remaining slots as two 256x128 column halves each, so that the last
// round takes about half as long.  Same bits as the plain launch.
// hipErrorNotSupported (nothing launched) for other tiles, dtypes or grids.
constexpr int64_t kGroupedSplitCUs = 256;
bool mfma_grouped_split(int tile, int dt);
hipError_t launch_mfma_grouped_split(const MfmaArgs &p, int tile, int dt, hipStream_t s);

// fp8 e4m3 GEMM on the register-staged kernel (tile ids 1, 4, 6) and on the
// direct-load kernel (tile ids 40 + base, 100 + base):
// C(i,j) = RNE_bf16((sum_r A(i,r) B(j,r)) * scale_a * scale_b), both operands
// reduction-contiguous e4m3 bytes.  fast = false: codes widened exactly to bf16,
// one bf16 MFMA per 16-deep step; fast = true: one f8f6f4 MFMA per 64-deep step.
hipError_t launch_fp8_gemm(const Fp8Args &p, int tile_id, bool fast, hipStream_t s);
hipError_t launch_fp8_dl(const MfmaArgs &p, int tile_id, bool fast, hipStream_t s);
// fp8 quantisation (quant.hip): fmt DT_E4M3 or DT_E5M2; amax (nullable)
// receives max(*amax, max |src|).  quantize: n elements; transpose_quantize:
// src [rows, cols] -> dst [cols, rows].
hipError_t launch_quantize(const void *src, const float *scale_inv, void *dst, float *amax,
                           int64_t n, int fmt, hipStream_t s);
// dst_rows (nullable) also receives the untransposed codes from the same read.
hipError_t launch_transpose_quantize(const void *src, const float *scale_inv, void *dst,
                                     void *dst_rows, float *amax, int64_t rows, int64_t cols,
                                     int fmt, hipStream_t s);
// Bias gradient (bias_grad.hip): out[n] = RNE(column sums of dy [m, n]) in a
// fixed order; rows in chunks of BG_CHUNK, nchunks = max(1, ceil(m / BG_CHUNK));
// with more than one chunk ws holds nchunks * n f32 partials.  vec: dy 16-byte
// aligned and n % 8 == 0.
constexpr int64_t BG_CHUNK = 256;
hipError_t launch_bias_grad(const void *dy, int64_t m, int64_t n, int64_t nchunks, float *ws,
                            void *out, int dt, bool vec, hipStream_t s);
// *a = *b = *c = +0 (null pointers skipped), one tiny kernel
hipError_t launch_zero3(float *a, float *b, float *c, hipStream_t s);

}  // namespace bi
