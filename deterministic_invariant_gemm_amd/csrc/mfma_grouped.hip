// Instantiations of the MFMA kernels for the grouped GEMM: forward and dinput (segment-anchored row tiles) and f32 dweights (expert-local reduction).
#include "mfma_dl_kernel.hpp"

namespace bi {
namespace mfma {
namespace {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// The split launch of the grouped forward: 256x256 tiles (eight waves of
// 64x128, copies spread: tile 112) and their 256x128 column halves (eight
// waves of 64x64, copies spread).
using TBig = TileOf<12>;
using THalf = TileOf<13>;
static_assert(TBig::BM == THalf::BM && TBig::BN == 2 * THalf::BN, "column halves");
constexpr int kThSplit =
    cmax(dl_threads(TBig::WGM * TBig::WGN, true, TBig::BM / TBig::WGM, TBig::BN / TBig::WGN),
         dl_threads(THalf::WGM * THalf::WGN, true, THalf::BM / THalf::WGM, THalf::BN / THalf::WGN));
constexpr int kLdsSplit = cmax(dl_lds_bytes(TBig::BM, TBig::BN), dl_lds_bytes(THalf::BM, THalf::BN));
static_assert(kLdsSplit + 4 * TBig::BN <= 160 * 1024, "one workgroup per CU");
static_assert(kGroupedSplitCUs % 8 == 0, "split slots keep their XCD");

// Row tiles of BM rows that the experts' segments take (the padding segment
// left out), as the segment decode counts them; the 64 lanes of the calling
// wave load 64 experts' offsets at a time.  The same value in every lane.
template <int BM>
__device__ __forceinline__ int expert_row_tiles(const MfmaArgs &p, int lane) {
    int tot = 0;
    for (int64_t x0 = 0; x0 < p.n_experts; x0 += 64) {
        const int64_t x = x0 + lane;
        int c = 0;
        if (x < p.n_experts) {
            int64_t s = p.offsets[x], e = p.offsets[x + 1];
            if (e > p.rows) e = p.rows;
            if (s > e) s = e;
            c = (int)((e - s + BM - 1) / BM);
        }
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) c += __shfl_xor(c, d, 64);
        tot += c;
    }
    return __builtin_amdgcn_readfirstlane(tot);
}

// Workgroups [0, kGroupedSplitCUs) take the grid's first slots whole.  The
// others first count the work slots W (expert row tiles x column tiles): with
// F = W rounded down to whole rounds and 0 < W - F <= half a round, workgroups
// [kGroupedSplitCUs, F) take slots whole and workgroups F + u the column
// halves of decode_half_tile(u, F); otherwise workgroup b takes slot b.
// Workgroups past their layout's end have nothing to do.
template <int DT>
__global__ __launch_bounds__(kThSplit) void mfma_dl_grouped_split_kernel(MfmaArgs p,
                                                                         int64_t nslots) {
    __shared__ __align__(1024) char lds_raw[kLdsSplit];
    __shared__ __align__(16) float lds_bias[TBig::BN];
    const int64_t b = blockIdx.x;
    int64_t first_half = nslots;  // first workgroup of the half tiles
    if (b >= kGroupedSplitCUs)
        first_half = split_first_half(
            (int64_t)expert_row_tiles<TBig::BM>(p, threadIdx.x & 63) * p.tiles_j, nslots,
            kGroupedSplitCUs);
    if (b < first_half) {
        if (b >= nslots) return;
        dl_body<DT, true, true, TBig::BM, TBig::BN, TBig::WGM, TBig::WGN, EPI_ROUND,
                MODE_SEGMENTS, true>(p, lds_raw, lds_bias, b, nslots);
    } else {
        dl_body<DT, true, true, THalf::BM, THalf::BN, THalf::WGM, THalf::WGN, EPI_ROUND,
                MODE_SEGMENTS, true, 0, 128, TBig::BN>(p, lds_raw, lds_bias, b - first_half,
                                                        first_half);
    }
}

}  // namespace
}  // namespace mfma

bool mfma_grouped_split(int tile, int dt) {
    return tile == 112 && (dt == DT_BF16 || dt == DT_F16);
}

hipError_t launch_mfma_grouped_split(const MfmaArgs &p, int tile, int dt, hipStream_t s) {
    if (!mfma_grouped_split(tile, dt) || p.offsets == nullptr) return hipErrorNotSupported;
    const int64_t nslots = seg_grid_rows(p.seg_tiles) * p.tiles_j;
    if (nslots <= kGroupedSplitCUs) return hipErrorNotSupported;
    // enough workgroups for either layout: nslots whole, or F whole and
    // 2 (nslots - F) halves with F >= kGroupedSplitCUs
    const int64_t grid = 2 * nslots - kGroupedSplitCUs;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (dt == DT_BF16)
        hipLaunchKernelGGL(mfma::mfma_dl_grouped_split_kernel<DT_BF16>, dim3(grid),
                           dim3(mfma::kThSplit), 0, s, p, nslots);
    else
        hipLaunchKernelGGL(mfma::mfma_dl_grouped_split_kernel<DT_F16>, dim3(grid),
                           dim3(mfma::kThSplit), 0, s, p, nslots);
    return hipGetLastError();
}

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
