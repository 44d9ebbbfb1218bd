// Instantiations of the MFMA kernels for the grouped GEMM: forward and dinput (segment-anchored row tiles) and f32 dweights (expert-local reduction).
#include "mfma_dl_kernel.hpp"

namespace bi {

hipError_t launch_mfma_grouped(const MfmaArgs &p, int tile_id, int dt, int epi, int64_t grid, hipStream_t s) {
    using namespace mfma;
    // epi selects the op: 0 forward, 1 dinput, 2 dweights
    if (tile_id >= 100) {
        if (dt == DT_BF16 && epi == 0) return launch_dls_among<DT_BF16, true, true, EPI_ROUND, MODE_SEGMENTS, 11, 12, 15>(p, tile_id, grid, s);
        if (dt == DT_F16 && epi == 0) return launch_dls_among<DT_F16, true, true, EPI_ROUND, MODE_SEGMENTS, 11, 12, 15>(p, tile_id, grid, s);
        if (dt == DT_BF16 && epi == 1) return launch_dls_among<DT_BF16, true, false, EPI_ROUND, MODE_SEGMENTS, 11, 12, 15>(p, tile_id, grid, s);
        if (dt == DT_F16 && epi == 1) return launch_dls_among<DT_F16, true, false, EPI_ROUND, MODE_SEGMENTS, 11, 12, 15>(p, tile_id, grid, s);
        if (dt == DT_BF16 && epi == 2) return launch_dls_among<DT_BF16, false, false, EPI_F32, MODE_EXPERT_RED, 11, 15, 16>(p, tile_id, grid, s);
        if (dt == DT_F16 && epi == 2) return launch_dls_among<DT_F16, false, false, EPI_F32, MODE_EXPERT_RED, 11, 15, 16>(p, tile_id, grid, s);
        return hipErrorInvalidValue;
    }
    if (tile_id >= 40) {
        if (dt == DT_BF16 && epi == 0) return launch_dl_among<DT_BF16, true, true, EPI_ROUND, MODE_SEGMENTS, 1, 4, 6, 11, 12, 15>(p, tile_id, grid, s);
        if (dt == DT_F16 && epi == 0) return launch_dl_among<DT_F16, true, true, EPI_ROUND, MODE_SEGMENTS, 1, 4, 6, 11, 12, 15>(p, tile_id, grid, s);
        if (dt == DT_BF16 && epi == 1) return launch_dl_among<DT_BF16, true, false, EPI_ROUND, MODE_SEGMENTS, 1, 4, 6, 11, 12, 15>(p, tile_id, grid, s);
        if (dt == DT_F16 && epi == 1) return launch_dl_among<DT_F16, true, false, EPI_ROUND, MODE_SEGMENTS, 1, 4, 6, 11, 12, 15>(p, tile_id, grid, s);
        if (dt == DT_BF16 && epi == 2) return launch_dl_among<DT_BF16, false, false, EPI_F32, MODE_EXPERT_RED, 1, 4, 6, 11, 15, 16>(p, tile_id, grid, s);
        if (dt == DT_F16 && epi == 2) return launch_dl_among<DT_F16, false, false, EPI_F32, MODE_EXPERT_RED, 1, 4, 6, 11, 15, 16>(p, tile_id, grid, s);
        return hipErrorInvalidValue;
    }
    if (dt == DT_BF16 && epi == 0) return launch_among<DT_BF16, true, true, EPI_ROUND, MODE_SEGMENTS, 1, 4, 6>(p, tile_id, grid, s);
    if (dt == DT_F16 && epi == 0) return launch_among<DT_F16, true, true, EPI_ROUND, MODE_SEGMENTS, 1, 4, 6>(p, tile_id, grid, s);
    if (dt == DT_BF16 && epi == 1) return launch_among<DT_BF16, true, false, EPI_ROUND, MODE_SEGMENTS, 1, 4, 6>(p, tile_id, grid, s);
    if (dt == DT_F16 && epi == 1) return launch_among<DT_F16, true, false, EPI_ROUND, MODE_SEGMENTS, 1, 4, 6>(p, tile_id, grid, s);
    if (dt == DT_BF16 && epi == 2) return launch_among<DT_BF16, false, false, EPI_F32, MODE_EXPERT_RED, 1, 4, 6>(p, tile_id, grid, s);
    if (dt == DT_F16 && epi == 2) return launch_among<DT_F16, false, false, EPI_F32, MODE_EXPERT_RED, 1, 4, 6>(p, tile_id, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace bi
