// A linear layer's dX and dW in one launch of the direct-load kernel: the first
// workgroups compute dX tiles, the others dW tiles, each running the tile code
// of its own launch (the same MFMA sequence per output element, so the same
// bits).  The two tiles get shorter LDS rings than in their own launches (dX
// two stages, dW three) and at most 128 VGPRs, so that a dX and a dW
// workgroup share each CU: while one waits at a stage barrier, the other's
// MFMAs run.
#include "mfma_dl_kernel.hpp"

namespace bi {
namespace mfma {
namespace {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// dX tile 128x96 (four MFMA waves along M plus four copy waves), dW tile 96x96
// (three MFMA waves along N plus four copy waves): tile ids 45 and 57
constexpr int kTileX = 45, kTileW = 57;
constexpr int kBaseX = kTileX - 40, kBaseW = kTileW - 40;
constexpr int kStagesX = 2, kStagesW = 3;
using TX = TileOf<kBaseX>;
using TW = TileOf<kBaseW>;
constexpr int kThX = dl_threads(TX::WGM * TX::WGN, false, TX::BM / TX::WGM, TX::BN / TX::WGN);
constexpr int kThW = dl_threads(TW::WGM * TW::WGN, false, TW::BM / TW::WGM, TW::BN / TW::WGN);
constexpr int kTh = cmax(kThX, kThW);
constexpr int kLds = cmax(dl_lds_bytes(TX::BM, TX::BN, kStagesX), dl_lds_bytes(TW::BM, TW::BN, kStagesW));
constexpr int kBiasN = cmax(TX::BN, TW::BN);
static_assert(2 * (kLds + 4 * kBiasN) <= 160 * 1024, "two workgroups per CU");
// waves per SIMD with two workgroups on a CU (the register budget follows)
constexpr int kWavesPerSimd = 2 * kTh / 64 / 4;

// Workgroups [0, nbx): dX tiles; [nbx, offw): nothing (offw is nbx rounded up
// to a multiple of 8, so that dW tile b runs on the same XCD as in a launch of
// its own); [offw, offw + nbw): dW tiles.  Waves beyond a tile's own count end
// at once; a workgroup barrier then waits only for the waves still running.
template <int DT>
__global__ __launch_bounds__(kTh, kWavesPerSimd) void mfma_dl_backward_kernel(
    MfmaArgs px, MfmaArgs pw, int64_t nbx, int64_t offw, int64_t nbw) {
    __shared__ __align__(1024) char lds_raw[kLds];
    __shared__ __align__(16) float lds_bias[kBiasN];
    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    if (b < offw) {
        if (b >= nbx || t >= kThX) return;
        dl_body<DT, true, true, TX::BM, TX::BN, TX::WGM, TX::WGN, EPI_ROUND, MODE_PLAIN, false,
                kStagesX>(px, lds_raw, lds_bias, b, nbx);
    } else {
        if (t >= kThW) return;
        dl_body<DT, false, false, TW::BM, TW::BN, TW::WGM, TW::WGN, EPI_ROUND, MODE_PLAIN, false,
                kStagesW>(pw, lds_raw, lds_bias, b - offw, nbw);
    }
}

}  // namespace
}  // namespace mfma

bool mfma_backward_pair(int tile_x, int tile_w, int dt) {
    return (dt == DT_BF16 || dt == DT_F16) && tile_x == mfma::kTileX && tile_w == mfma::kTileW;
}

hipError_t launch_mfma_backward(const MfmaArgs &px, int tile_x, const MfmaArgs &pw, int tile_w,
                                int dt, hipStream_t s) {
    if (!mfma_backward_pair(tile_x, tile_w, dt) || pw.nchunks != 1 || px.nchunks != 1)
        return hipErrorNotSupported;
    // grids from the tiles this kernel runs
    MfmaArgs ax = px, aw = pw;
    ax.tiles_i = (ax.rows + mfma::TX::BM - 1) / mfma::TX::BM;
    ax.tiles_j = (ax.cols + mfma::TX::BN - 1) / mfma::TX::BN;
    aw.tiles_i = (aw.rows + mfma::TW::BM - 1) / mfma::TW::BM;
    aw.tiles_j = (aw.cols + mfma::TW::BN - 1) / mfma::TW::BN;
    const int64_t nbx = ax.tiles_i * ax.tiles_j, nbw = aw.tiles_i * aw.tiles_j;
    const int64_t offw = (nbx + 7) / 8 * 8;
    if (nbx <= 0 || nbw <= 0) return hipErrorNotSupported;
    if (offw + nbw > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (dt == DT_BF16)
        hipLaunchKernelGGL(mfma::mfma_dl_backward_kernel<DT_BF16>, dim3(offw + nbw),
                           dim3(mfma::kTh), 0, s, ax, aw, nbx, offw, nbw);
    else
        hipLaunchKernelGGL(mfma::mfma_dl_backward_kernel<DT_F16>, dim3(offw + nbw),
                           dim3(mfma::kTh), 0, s, ax, aw, nbx, offw, nbw);
    return hipGetLastError();
}

}  // namespace bi
