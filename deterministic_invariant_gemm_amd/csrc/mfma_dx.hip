// Instantiations of the MFMA kernels for dX (both operands reduction-contiguous).
#include "mfma_dl_kernel.hpp"

namespace bi {

hipError_t launch_mfma_dx(const MfmaArgs &p, int tile_id, int dt, int epi, int64_t grid, hipStream_t s) {
    using namespace mfma;
    (void)epi;
    if (tile_id >= 120) {
        if (dt == DT_BF16) return launch_dl_among<DT_BF16, true, true, EPI_ROUND, MODE_PLAIN, 20>(p, tile_id, grid, s);
        if (dt == DT_F16) return launch_dl_among<DT_F16, true, true, EPI_ROUND, MODE_PLAIN, 20>(p, tile_id, grid, s);
        return hipErrorInvalidValue;
    }
    if (tile_id >= 100) {
        if (dt == DT_BF16) return launch_dls_among<DT_BF16, true, true, EPI_ROUND, MODE_PLAIN, 5, 11, 15>(p, tile_id, grid, s);
        if (dt == DT_F16) return launch_dls_among<DT_F16, true, true, EPI_ROUND, MODE_PLAIN, 5, 11, 15>(p, tile_id, grid, s);
        return hipErrorInvalidValue;
    }
    if (tile_id >= 40) {
        if (dt == DT_BF16) return launch_dl_among<DT_BF16, true, true, EPI_ROUND, MODE_PLAIN, 2, 3, 4, 5, 6, 10, 11, 13, 15>(p, tile_id, grid, s);
        if (dt == DT_F16) return launch_dl_among<DT_F16, true, true, EPI_ROUND, MODE_PLAIN, 2, 3, 4, 5, 6, 10, 11, 13, 15>(p, tile_id, grid, s);
        return hipErrorInvalidValue;
    }
    if (dt == DT_BF16) return launch_among<DT_BF16, true, true, EPI_ROUND, MODE_PLAIN, 1, 2, 3, 4, 5, 6, 7, 9, 10, 11, 13, 15>(p, tile_id, grid, s);
    if (dt == DT_F16) return launch_among<DT_F16, true, true, EPI_ROUND, MODE_PLAIN, 1, 2, 3, 4, 5, 6, 7, 9, 10, 11, 13, 15>(p, tile_id, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace bi
