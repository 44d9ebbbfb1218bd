// Instantiations of the direct-load MFMA kernel for the fp8 e4m3 GEMM
// (AstrAI fp8_mm.cu: fp8_mm / fp8_gemm_into, e4m3fn a[M,K] and b[N,K], f32
// compute, per-tensor scales inside the GEMM, bf16 output):
//   y[m,n] = RNE_bf16(((sum_k a[m,k] * bt[n,k]) * scale_a) * scale_b)
// Each 128-byte stage row holds 128 reduction values.
//   * Default (exact products, f32 accumulation): every code is widened exactly
//     to bf16 in registers and each 16-deep step is one
//     v_mfma_f32_32x32x16_bf16, ascending from +0 -- the accumulation of the
//     bf16 path, on the same values.
//   * Opt-in fast path: each 64-deep step is one
//     v_mfma_scale_f32_32x32x64_f8f6f4, which aligns the products of each group
//     of 8 reduction indices to the group's largest before adding them.
// Zeros past the end of the reduction; the register-staged fp8 kernel
// (fp8_tier.hip) issues the same per-element sequence for either path, so every
// tile gives the same bits.
#include "mfma_dl_kernel.hpp"

namespace bi {

hipError_t launch_fp8_dl(const MfmaArgs &p, int tile_id, bool fast, hipStream_t s) {
    using namespace mfma;
    const int64_t grid = p.tiles_i * p.tiles_j;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (fast) {
        if (tile_id >= 300)
            return launch_dld_among<DT_E4M3_FAST, true, true, EPI_SCALE, MODE_PLAIN, 512, 21>(p, tile_id, grid, s);
        if (tile_id >= 200)
            return launch_dld_among<DT_E4M3_FAST, true, true, EPI_SCALE, MODE_PLAIN, 256, 20>(p, tile_id, grid, s);
        if (tile_id >= 120)
            return launch_dl_among<DT_E4M3_FAST, true, true, EPI_SCALE, MODE_PLAIN, 20, 21>(p, tile_id, grid, s);
        if (tile_id >= 100)
            return launch_dls_among<DT_E4M3_FAST, true, true, EPI_SCALE, MODE_PLAIN, 11, 12, 15>(
                p, tile_id, grid, s);
        return launch_dl_among<DT_E4M3_FAST, true, true, EPI_SCALE, MODE_PLAIN, 1, 4, 6, 11, 12, 15>(
            p, tile_id, grid, s);
    }
    if (tile_id >= 300)
        return launch_dld_among<DT_E4M3, true, true, EPI_SCALE, MODE_PLAIN, 512, 21>(p, tile_id, grid, s);
    if (tile_id >= 200)
        return launch_dld_among<DT_E4M3, true, true, EPI_SCALE, MODE_PLAIN, 256, 20>(p, tile_id, grid, s);
    if (tile_id >= 120)
        return launch_dl_among<DT_E4M3, true, true, EPI_SCALE, MODE_PLAIN, 20, 21>(p, tile_id, grid, s);
    if (tile_id >= 100)
        return launch_dls_among<DT_E4M3, true, true, EPI_SCALE, MODE_PLAIN, 11, 12, 14, 15>(
            p, tile_id, grid, s);
    return launch_dl_among<DT_E4M3, true, true, EPI_SCALE, MODE_PLAIN, 1, 4, 6, 11, 12, 14, 15>(
        p, tile_id, grid, s);
}

}  // namespace bi
