// Host-side check of the MFMA kernels' tile decode (the same source the
// kernels use: decode_tile_at, decode_half_tile, split_first_half, compiled
// here for the host only).  For each mode and a set of shapes it walks every
// workgroup index of a launch and checks that the tiles cover the output
// exactly once:
//   * plain grid: every (row tile, column tile, chunk) once (xcd_remap is a
//     permutation of the grid);
//   * segment grid (grouped forward / dinput): every row of every expert's
//     segment in exactly one tile, tiles anchored at the segment start and
//     inside it, every 32-column block of such a row once, the padding rows
//     (ids outside the experts) zero-filled over every column and no other
//     row written; the same for the split launch (whole slots, then column
//     halves) under the layout split_first_half picks;
//   * expert-local reduction grid (grouped dweights): every (expert, row tile,
//     column tile) once, reduction range = the expert's segment.
// Prints "decode ok" and exits 0, or names the first failure and exits 1.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mfma_dl_kernel.hpp"

using namespace bi;
using namespace bi::mfma;

static int g_fail = 0;
#define CHECK(c, ...)                                                   \
    do {                                                                \
        if (!(c)) {                                                     \
            if (!g_fail) std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
            if (!g_fail) std::printf(__VA_ARGS__);                      \
            if (!g_fail) std::printf("\n");                             \
            g_fail = 1;                                                 \
        }                                                               \
    } while (0)

// seeded 64-bit LCG (Knuth's MMIX constants), test data only
struct Lcg {
    uint64_t s;
    uint64_t next() { return s = s * 6364136223846793005ULL + 1442695040888963407ULL; }
    int64_t below(int64_t n) { return (int64_t)((next() >> 33) % (uint64_t)n); }
};

// offsets[0..e] of m rows: each row's expert uniform over [0, e) except the
// `empty` expert (if >= 0), `pad` rows of padding at the end
static std::vector<uint32_t> routing(int64_t m, int64_t e, int64_t pad, int64_t empty, uint64_t seed) {
    Lcg g{seed};
    std::vector<int64_t> cnt(e, 0);
    for (int64_t r = 0; r < m - pad; ++r) {
        int64_t x = g.below(e);
        if (x == empty) x = (x + 1) % e;
        ++cnt[x];
    }
    std::vector<uint32_t> off(e + 1, 0);
    for (int64_t x = 0; x < e; ++x) off[x + 1] = off[x] + (uint32_t)cnt[x];
    return off;
}

template <int BM, int BN>
static void check_plain(int64_t rows, int64_t cols, int64_t nchunks) {
    MfmaArgs p{};
    p.rows = rows; p.cols = cols; p.red = 1000; p.chunk = 1000; p.nchunks = nchunks;
    p.tiles_i = (rows + BM - 1) / BM; p.tiles_j = (cols + BN - 1) / BN;
    const int64_t grid = p.tiles_i * p.tiles_j * nchunks;
    std::vector<int> seen(grid, 0);
    for (int64_t b = 0; b < grid; ++b) {
        const TileInfo ti = decode_tile_at<MODE_PLAIN, BM, BN>(p, 0, b, grid);
        CHECK(!ti.skip, "plain tile %lld skipped", (long long)b);
        CHECK(ti.row0 % BM == 0 && ti.col0 % BN == 0 && ti.row0 < rows && ti.col0 < cols,
              "plain tile %lld at %lld,%lld", (long long)b, (long long)ti.row0, (long long)ti.col0);
        const int64_t id = (ti.chunk * p.tiles_i + ti.row0 / BM) * p.tiles_j + ti.col0 / BN;
        CHECK(id >= 0 && id < grid, "plain tile id %lld", (long long)id);
        if (id >= 0 && id < grid) ++seen[id];
    }
    for (int64_t i = 0; i < grid; ++i) CHECK(seen[i] == 1, "plain slot %lld covered %d times", (long long)i, seen[i]);
}

// one launch over the segment grid: whole slots below first_half (of the
// BM x BNB tile), column halves from there on when split
template <int BM, int BNB>
static void check_segments(int64_t m, int64_t n, int64_t e, int64_t pad, int64_t empty,
                           uint64_t seed, bool split) {
    std::vector<uint32_t> off = routing(m, e, pad, empty, seed);
    std::vector<uint16_t> out((size_t)(m * n), 0xffff);
    MfmaArgs p{};
    p.rows = m; p.cols = n; p.red = 64; p.ldc = n; p.c = out.data(); p.offsets = off.data();
    p.n_experts = e; p.tiles_j = (n + BNB - 1) / BNB; p.seg_tiles = (m + BM - 1) / BM + e;
    const int64_t nslots = seg_grid_rows(p.seg_tiles) * p.tiles_j;
    int64_t work_rows = 0;
    for (int64_t x = 0; x < e; ++x) work_rows += ((int64_t)off[x + 1] - off[x] + BM - 1) / BM;
    const int64_t cus = kGroupedSplitCUs;
    int64_t first_half = nslots, grid = nslots;
    if (split && nslots > cus) {
        first_half = split_first_half(work_rows * p.tiles_j, nslots, cus);
        grid = 2 * nslots - cus;
    }
    constexpr int NB = 32;  // column blocks of 32
    const int64_t ncb = (n + NB - 1) / NB;
    std::vector<int> cover((size_t)(m * ncb), 0);
    auto take = [&](const TileInfo &ti, int64_t width) {
        if (ti.skip) return;
        int64_t x = 0;
        while (x < e && !((int64_t)off[x] <= ti.row0 && ti.row0 < (int64_t)off[x + 1])) ++x;
        CHECK(x < e, "tile at row %lld outside every segment", (long long)ti.row0);
        if (x >= e) return;
        CHECK((ti.row0 - off[x]) % BM == 0, "tile at row %lld not anchored at segment %lld", (long long)ti.row0, (long long)x);
        CHECK(ti.row_end == (int64_t)off[x + 1], "tile row_end %lld for segment end %u", (long long)ti.row_end, off[x + 1]);
        CHECK(ti.b_off == x * p.b_expert_stride, "expert offset");
        const int64_t r1 = ti.row0 + BM < ti.row_end ? ti.row0 + BM : ti.row_end;
        for (int64_t r = ti.row0; r < r1; ++r)
            for (int64_t c = ti.col0; c < ti.col0 + width && c < n; c += NB) ++cover[r * ncb + c / NB];
    };
    for (int64_t b = 0; b < grid; ++b) {
        if (b < first_half) {
            if (b >= nslots) continue;
            take(decode_tile_at<MODE_SEGMENTS, BM, BNB, 256>(p, 0, b, nslots), BNB);
        } else {
            // every thread index of the workgroup, as the padding fill spreads over them
            TileInfo ti{};
            for (int t = 0; t < 512; ++t) ti = decode_half_tile<MODE_SEGMENTS, BM, BNB, 512>(p, t, b - first_half, first_half);
            take(ti, BNB / 2);
        }
    }
    // whole slots fill padding with thread t = 0 only above: run every thread
    for (int64_t b = 0; b < (first_half < nslots ? first_half : nslots); ++b)
        for (int t = 1; t < 256; ++t) decode_tile_at<MODE_SEGMENTS, BM, BNB, 256>(p, t, b, nslots);
    const int64_t pad0 = off[e];
    for (int64_t r = 0; r < m; ++r) {
        for (int64_t cb = 0; cb < ncb; ++cb) {
            const int want = r < pad0 ? 1 : 0;
            CHECK(cover[r * ncb + cb] == want, "segments m=%lld n=%lld e=%lld split=%d: row %lld block %lld covered %d times",
                  (long long)m, (long long)n, (long long)e, (int)split, (long long)r, (long long)cb, cover[r * ncb + cb]);
        }
        for (int64_t c = 0; c < n; ++c) {
            const uint16_t want = r < pad0 ? 0xffff : 0;
            CHECK(out[r * n + c] == want, "segments m=%lld n=%lld e=%lld split=%d: output %lld,%lld is %04x",
                  (long long)m, (long long)n, (long long)e, (int)split, (long long)r, (long long)c, out[r * n + c]);
        }
    }
    if (split) std::printf("segments m=%lld n=%lld e=%lld: %lld slots, %s\n", (long long)m, (long long)n,
                           (long long)e, (long long)nslots,
                           first_half < nslots ? "split" : "whole slots");
}

template <int BM, int BN>
static void check_expert_red(int64_t rows, int64_t cols, int64_t m, int64_t e, uint64_t seed) {
    std::vector<uint32_t> off = routing(m, e, m / 20, 1, seed);
    MfmaArgs p{};
    p.rows = rows; p.cols = cols; p.red = m; p.red_offsets = off.data(); p.n_experts = e;
    p.c_expert_stride = rows * cols;
    p.tiles_i = (rows + BM - 1) / BM; p.tiles_j = (cols + BN - 1) / BN;
    const int64_t grid = e * p.tiles_i * p.tiles_j;
    std::vector<int> seen(grid, 0);
    for (int64_t b = 0; b < grid; ++b) {
        const TileInfo ti = decode_tile_at<MODE_EXPERT_RED, BM, BN>(p, 0, b, grid);
        const int64_t x = ti.c_off / p.c_expert_stride;
        CHECK(x >= 0 && x < e, "expert %lld", (long long)x);
        if (x < 0 || x >= e) continue;
        CHECK(ti.r_begin == (int64_t)off[x] && ti.r_end == (int64_t)off[x + 1], "reduction range of expert %lld", (long long)x);
        const int64_t id = (x * p.tiles_i + ti.row0 / BM) * p.tiles_j + ti.col0 / BN;
        if (id >= 0 && id < grid) ++seen[id];
    }
    for (int64_t i = 0; i < grid; ++i) CHECK(seen[i] == 1, "expert slot %lld covered %d times", (long long)i, seen[i]);
}

int main() {
    check_plain<256, 192>(4096, 3072, 1);
    check_plain<128, 96>(4096, 768, 1);
    check_plain<96, 96>(768, 3072, 3);
    check_plain<64, 32>(128, 4096, 1);
    check_plain<256, 256>(1000, 1000, 1);
    // segment grids: plain launches of several tiles, and the split launch of
    // the 256x256 tile (config-5-like shapes give both layouts)
    check_segments<256, 256>(700, 200, 5, 37, 3, 11, false);
    check_segments<128, 128>(2600, 264, 37, 100, 5, 12, false);
    check_segments<256, 192>(3000, 1408, 8, 150, -1, 13, false);
    check_segments<256, 256>(16384, 1408, 8, 819, -1, 14, true);
    check_segments<256, 256>(12000, 1408, 8, 300, 2, 15, true);
    check_segments<256, 256>(20000, 1408, 16, 500, -1, 16, true);
    check_segments<256, 256>(9000, 4096, 3, 70, -1, 17, true);
    check_segments<256, 256>(10000, 2048, 8, 0, -1, 18, true);
    check_segments<256, 256>(5000, 4096, 4, 33, 1, 19, true);
    check_segments<256, 256>(64, 64, 4, 64, -1, 20, true);
    check_expert_red<192, 256>(1408, 2048, 16384, 8, 21);
    check_expert_red<128, 128>(200, 136, 700, 5, 22);
    if (g_fail) return 1;
    std::printf("decode ok\n");
    return 0;
}
