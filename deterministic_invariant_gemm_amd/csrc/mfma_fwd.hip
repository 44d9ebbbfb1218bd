// Instantiations of the MFMA kernels for the linear forward (A reduction-contiguous, B = W row-contiguous).
#include "mfma_dl_kernel.hpp"

namespace bi {

hipError_t launch_mfma_fwd(const MfmaArgs &p, int tile_id, int dt, int epi, int64_t grid, hipStream_t s) {
    using namespace mfma;
    (void)epi;
    if (tile_id >= 300) {
        if (dt == DT_BF16) return launch_dld_among<DT_BF16, true, false, EPI_ROUND, MODE_PLAIN, 512, 21>(p, tile_id, grid, s);
        if (dt == DT_F16) return launch_dld_among<DT_F16, true, false, EPI_ROUND, MODE_PLAIN, 512, 21>(p, tile_id, grid, s);
        return hipErrorInvalidValue;
    }
    if (tile_id >= 200) {
        if (dt == DT_BF16) return launch_dld_among<DT_BF16, true, false, EPI_ROUND, MODE_PLAIN, 256, 20>(p, tile_id, grid, s);
        if (dt == DT_F16) return launch_dld_among<DT_F16, true, false, EPI_ROUND, MODE_PLAIN, 256, 20>(p, tile_id, grid, s);
        return hipErrorInvalidValue;
    }
    if (tile_id >= 120) {
        if (dt == DT_BF16) return launch_dl_among<DT_BF16, true, false, EPI_ROUND, MODE_PLAIN, 20>(p, tile_id, grid, s);
        if (dt == DT_F16) return launch_dl_among<DT_F16, true, false, EPI_ROUND, MODE_PLAIN, 20>(p, tile_id, grid, s);
        return hipErrorInvalidValue;
    }
    if (tile_id >= 100) {
        if (dt == DT_BF16) return launch_dls_among<DT_BF16, true, false, EPI_ROUND, MODE_PLAIN, 11, 15>(p, tile_id, grid, s);
        if (dt == DT_F16) return launch_dls_among<DT_F16, true, false, EPI_ROUND, MODE_PLAIN, 11, 15>(p, tile_id, grid, s);
        return hipErrorInvalidValue;
    }
    if (tile_id >= 40) {
        if (dt == DT_BF16) return launch_dl_among<DT_BF16, true, false, EPI_ROUND, MODE_PLAIN, 1, 2, 3, 4, 6, 7, 9, 11, 12, 13, 14, 15>(p, tile_id, grid, s);
        if (dt == DT_F16) return launch_dl_among<DT_F16, true, false, EPI_ROUND, MODE_PLAIN, 1, 2, 3, 4, 6, 7, 9, 11, 12, 13, 14, 15>(p, tile_id, grid, s);
        return hipErrorInvalidValue;
    }
    if (dt == DT_BF16) return launch_among<DT_BF16, true, false, EPI_ROUND, MODE_PLAIN, 1, 2, 3, 4, 6, 7, 9, 11, 12, 13, 14>(p, tile_id, grid, s);
    if (dt == DT_F16) return launch_among<DT_F16, true, false, EPI_ROUND, MODE_PLAIN, 1, 2, 3, 4, 6, 7, 9, 11, 12, 13, 14>(p, tile_id, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace bi
