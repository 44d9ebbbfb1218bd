// The grouped GEMM's dinput and dweights (rublas tensor_grouped, the segmented
// backward: dinput = dY W_e per row of expert e, dweights_e = dY_e^T X_e in
// f32) in one launch of the direct-load kernel: the first workgroups compute
// dinput tiles (segment-anchored 256x256, eight waves), the others dweights
// tiles (expert-local 192x256, eight waves, copies spread), each running the
// tile code of its own launch with its own full LDS ring (the same MFMA
// sequence per output element, so the same bits).  One workgroup fits a CU
// either way; in one launch the CUs that the dinput tiles' last, partial round
// leaves idle start dweights tiles instead of waiting for the launch to end.
#include "mfma_dl_kernel.hpp"

namespace bi {
namespace mfma {
namespace {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

constexpr int kTileD = 52, kTileW = 116;  // dinput 256x256, dweights 192x256 spread
using TD = TileOf<kTileD - 40>;
using TW = TileOf<kTileW - 100>;
constexpr int kThD = dl_threads(TD::WGM * TD::WGN, false, TD::BM / TD::WGM, TD::BN / TD::WGN);
constexpr int kThW = dl_threads(TW::WGM * TW::WGN, true, TW::BM / TW::WGM, TW::BN / TW::WGN);
constexpr int kTh = cmax(kThD, kThW);
constexpr int kLds = cmax(dl_lds_bytes(TD::BM, TD::BN), dl_lds_bytes(TW::BM, TW::BN));
constexpr int kBiasN = cmax(TD::BN, TW::BN);
static_assert(kLds + 4 * kBiasN <= 160 * 1024, "one workgroup per CU");

// Workgroups [0, nbd): dinput tiles (the segment grid, padding slots included);
// [nbd, offw): nothing (offw is nbd rounded up to a multiple of 8, so that
// dweights tile b runs on the same XCD as in a launch of its own);
// [offw, offw + nbw): dweights tiles.  Threads past a tile's own count end at
// once.
template <int DT>
__global__ __launch_bounds__(kTh) void mfma_dl_grouped_backward_kernel(MfmaArgs pd, MfmaArgs pw,
                                                                       int64_t nbd, int64_t offw,
                                                                       int64_t nbw) {
    __shared__ __align__(1024) char lds_raw[kLds];
    __shared__ __align__(16) float lds_bias[kBiasN];
    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    if (b < offw) {
        if (b >= nbd || t >= kThD) return;
        dl_body<DT, true, false, TD::BM, TD::BN, TD::WGM, TD::WGN, EPI_ROUND, MODE_SEGMENTS, false>(
            pd, lds_raw, lds_bias, b, nbd);
    } else {
        if (t >= kThW) return;
        dl_body<DT, false, false, TW::BM, TW::BN, TW::WGM, TW::WGN, EPI_F32, MODE_EXPERT_RED, true>(
            pw, lds_raw, lds_bias, b - offw, nbw);
    }
}

}  // namespace
}  // namespace mfma

bool mfma_grouped_backward_pair(int tile_d, int tile_w, int dt) {
    return (dt == DT_BF16 || dt == DT_F16) && tile_d == mfma::kTileD && tile_w == mfma::kTileW;
}

hipError_t launch_mfma_grouped_backward(const MfmaArgs &pd, int tile_d, const MfmaArgs &pw,
                                        int tile_w, int dt, hipStream_t s) {
    if (!mfma_grouped_backward_pair(tile_d, tile_w, dt) || pd.offsets == nullptr ||
        pw.red_offsets == nullptr)
        return hipErrorNotSupported;
    // the grids of the two launches (segment grid for dinput, expert x tiles
    // for dweights)
    const int64_t nbd = seg_grid_rows(pd.seg_tiles) * pd.tiles_j;
    const int64_t nbw = pw.n_experts * pw.tiles_i * pw.tiles_j;
    const int64_t offw = (nbd + 7) / 8 * 8;
    if (nbd <= 0 || nbw <= 0) return hipErrorNotSupported;
    if (offw + nbw > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (dt == DT_BF16)
        hipLaunchKernelGGL(mfma::mfma_dl_grouped_backward_kernel<DT_BF16>, dim3(offw + nbw),
                           dim3(mfma::kTh), 0, s, pd, pw, nbd, offw, nbw);
    else
        hipLaunchKernelGGL(mfma::mfma_dl_grouped_backward_kernel<DT_F16>, dim3(offw + nbw),
                           dim3(mfma::kTh), 0, s, pd, pw, nbd, offw, nbw);
    return hipGetLastError();
}

}  // namespace bi
