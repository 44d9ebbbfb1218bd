// Instantiations of the MFMA kernels for dW (both operands row-contiguous), rounded or as f32 chunk partials.
#include "mfma_dl_kernel.hpp"

namespace bi {

hipError_t launch_mfma_dw(const MfmaArgs &p, int tile_id, int dt, int epi, int64_t grid, hipStream_t s) {
    using namespace mfma;
    if (tile_id >= 100) {
        if (dt == DT_BF16 && epi == EPI_ROUND) return launch_dls_among<DT_BF16, false, false, EPI_ROUND, MODE_PLAIN, 4, 5, 8, 15>(p, tile_id, grid, s);
        if (dt == DT_F16 && epi == EPI_ROUND) return launch_dls_among<DT_F16, false, false, EPI_ROUND, MODE_PLAIN, 4, 5, 8, 15>(p, tile_id, grid, s);
        if (dt == DT_BF16 && epi == EPI_PARTIAL) return launch_dls_among<DT_BF16, false, false, EPI_PARTIAL, MODE_PLAIN, 4, 5, 8, 15>(p, tile_id, grid, s);
        if (dt == DT_F16 && epi == EPI_PARTIAL) return launch_dls_among<DT_F16, false, false, EPI_PARTIAL, MODE_PLAIN, 4, 5, 8, 15>(p, tile_id, grid, s);
        return hipErrorInvalidValue;
    }
    if (tile_id >= 40) {
        if (dt == DT_BF16 && epi == EPI_ROUND) return launch_dl_among<DT_BF16, false, false, EPI_ROUND, MODE_PLAIN, 1, 3, 4, 5, 6, 7, 8, 13, 14, 15, 17>(p, tile_id, grid, s);
        if (dt == DT_F16 && epi == EPI_ROUND) return launch_dl_among<DT_F16, false, false, EPI_ROUND, MODE_PLAIN, 1, 3, 4, 5, 6, 7, 8, 13, 14, 15, 17>(p, tile_id, grid, s);
        if (dt == DT_BF16 && epi == EPI_PARTIAL) return launch_dl_among<DT_BF16, false, false, EPI_PARTIAL, MODE_PLAIN, 1, 3, 4, 5, 6, 7, 8, 13, 14, 15, 17>(p, tile_id, grid, s);
        if (dt == DT_F16 && epi == EPI_PARTIAL) return launch_dl_among<DT_F16, false, false, EPI_PARTIAL, MODE_PLAIN, 1, 3, 4, 5, 6, 7, 8, 13, 14, 15, 17>(p, tile_id, grid, s);
        return hipErrorInvalidValue;
    }
    if (dt == DT_BF16 && epi == EPI_ROUND) return launch_among<DT_BF16, false, false, EPI_ROUND, MODE_PLAIN, 1, 3, 4, 5, 6, 7, 10, 13, 14, 15>(p, tile_id, grid, s);
    if (dt == DT_F16 && epi == EPI_ROUND) return launch_among<DT_F16, false, false, EPI_ROUND, MODE_PLAIN, 1, 3, 4, 5, 6, 7, 10, 13, 14, 15>(p, tile_id, grid, s);
    if (dt == DT_BF16 && epi == EPI_PARTIAL) return launch_among<DT_BF16, false, false, EPI_PARTIAL, MODE_PLAIN, 1, 3, 4, 5, 6, 7, 10, 13, 14, 15>(p, tile_id, grid, s);
    if (dt == DT_F16 && epi == EPI_PARTIAL) return launch_among<DT_F16, false, false, EPI_PARTIAL, MODE_PLAIN, 1, 3, 4, 5, 6, 7, 10, 13, 14, 15>(p, tile_id, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace bi
