// C ABI of the deterministic GEMM library: argument validation, the shape-only
// tier / tile plan, and kernel launches.  Nothing here allocates, synchronises
// or keeps state between calls.
#include "../../include/bi.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace {

using namespace bi;

constexpr int64_t kMaxElems = (int64_t)1 << 40;
constexpr int64_t kNoSplit = (int64_t)1 << 62;  // "one chunk for any m"

enum Op : int { OP_FWD = 0, OP_DX = 1, OP_DW = 2, OP_FP8 = 3, OP_GFWD = 4, OP_GDIN = 5, OP_GDW = 6 };

bool dtype_ok(int dt) { return dt == BI_F32 || dt == BI_BF16 || dt == BI_F16; }

// product of non-negative dims within kMaxElems, else -1
int64_t checked_elems(int64_t a, int64_t b, int64_t c = 1) {
    if (a < 0 || b < 0 || c < 0) return -1;
    __int128 p = (__int128)a * b * c;
    return p > kMaxElems ? -1 : (int64_t)p;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned8(const void *p) { return ((uintptr_t)p & 7u) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- the plan: tier, tile and chunk from (op, dtype, tc, k, n) only ----------

struct Plan {
    int tile;       // 0 = scalar tier, else MFMA tile id
    int64_t chunk;  // dW: reduction rows per chunk
};

// non-M output dims of each op: the scalar tier takes over when one is < 64
bool mfma_eligible(int op, int dt, int tc, int64_t k, int64_t n) {
    if (!tc) return false;
    if (op != OP_FP8 && dt == BI_F32) return false;
    switch (op) {
    case OP_FWD: case OP_FP8: case OP_GFWD: return n >= 64;
    case OP_DX: case OP_GDIN: return k >= 64;
    case OP_DW: case OP_GDW: return k >= 64 && n >= 64;
    }
    return false;
}

// tc = 2 asks for the MFMA tier explicitly (rublas grouped_matmul_nt: an
// explicit tensor-core strategy fails when that path is unavailable instead of
// falling back); tc = 1 is the automatic choice, tc = 0 the scalar tier.
// tc = 3 (fp8 GEMMs only) chooses the tier like tc = 1 and multiplies on the
// MFMA tier with the fp8 matrix instruction instead of the exact widened path.
constexpr int kTcRequired = 2;
constexpr int kTcFp8Fast = 3;

// Testing builds only (BI_TESTING, libbi_testing.so): tc = 16 + id forces MFMA
// tile `id` when the op is on the MFMA tier (plus kFastBit: the fp8 fast path on
// tile `id`; plus (16 + id2) << 16: tile id2 for the dweights of a grouped
// backward, whose dinput takes `id`), for the tile-identity tests and tile
// tuning.  Tiles do not change results.  Production builds reject every other
// tc with BI_ERR_UNSUPPORTED.
constexpr int kForceBase = 16;
constexpr int kFastBit = 4096;
constexpr int kGdwShift = 16;
#ifdef BI_TESTING
constexpr bool kForceHook = true;
#else
constexpr bool kForceHook = false;
#endif

bool tc_known(int op, int tc) {
    if (tc >= 0 && tc <= kTcRequired) return true;
    if (tc == kTcFp8Fast) return op == OP_FP8;
    if (kForceHook && tc > 0) {
        const int lo = tc & (kFastBit - 1), hi = tc >> kGdwShift;
        const bool hi_ok = hi == 0 || (hi >= kForceBase && (op == OP_GDIN || op == OP_GDW));
        if (lo >= kForceBase && (tc & ((1 << kGdwShift) - 1) & ~(2 * kFastBit - 1)) == 0 && hi_ok)
            return op == OP_FP8 || !(tc & kFastBit);
    }
    return false;
}

// testing builds: the tile a forcing tc asks for on `op`
int forced_tile(int op, int tc) {
    const int hi = tc >> kGdwShift;
    if (op == OP_GDW && hi) return hi - kForceBase;
    return (tc & (kFastBit - 1)) - kForceBase;
}

// fp8 GEMMs: the fp8 matrix instruction was asked for
bool fp8_fast(int tc) { return tc == kTcFp8Fast || (kForceHook && tc >= kForceBase && (tc & kFastBit)); }

int tier_check(int op, int dt, int tc, int64_t k, int64_t n) {
    if (!tc_known(op, tc)) return BI_ERR_UNSUPPORTED;
    if (tc == kTcRequired && !mfma_eligible(op, dt, tc, k, n)) return BI_ERR_UNSUPPORTED;
    return BI_OK;
}

// Tile per op from the non-M output dims only (the kernel's column count is N
// for forward / fp8 / grouped forward, K for dX / grouped dinput; dW tiles its
// [K, N] output).  Every tile issues the same MFMA sequence per element, so
// this choice affects speed only.  Ids 40 + i are the direct-load kernel on
// shape i and 100 + i the same with its copies spread between MFMAs (both used
// when operands are aligned, see direct_tile; fp8 otherwise runs its
// register-staged kernel on 256x256, 128x128 or 64x64).
int pick_tile(int op, int64_t k, int64_t n, bool fast) {
    const int64_t cols = (op == OP_DX || op == OP_GDIN) ? k : n;
    switch (op) {
    case OP_FP8:
        if (fast) {
            // 256x256, eight waves, copies spread; 128x128 eight waves below
            if (cols >= 2048) return 112;
            return cols >= 128 ? 115 : 46;
        }
        // exact path: 256x256 with four waves of 128x128 (one per SIMD, its
        // accumulators in the AGPRs); the eight-wave 256x256 tile needs more
        // registers than two waves per SIMD have once fragments are widened
        if (cols >= 2048) return 41;
        return cols >= 128 ? 115 : 46;
    case OP_FWD:
        // 256x192, 8 waves, copies spread; 256x256, 8 waves
        if (cols >= 2048 && cols % 192 == 0 && cols / 192 <= 16) return 111;
        if (cols >= 2048) return 52;
        return cols >= 128 ? 44 : 46;
    case OP_DX:
        if (cols % 96 == 0 && cols <= 1536) return 45;  // 128x96, four waves along M
        if (cols >= 2048) return 111;                   // 256x192, eight waves, spread
        return cols >= 128 ? 115 : 46;                  // 128x128, eight waves, spread
    case OP_DW:
        // 96x96 with three MFMA waves side by side along N (one per SIMD on
        // three SIMDs, plus the copy waves) while that makes at most one tile
        // per CU and fills at least half of them
        if (k >= 96 && n >= 96 && cdiv(k, 96) * cdiv(n, 96) <= 256 &&
            cdiv(k, 96) * cdiv(n, 96) >= 128)
            return 57;
        // 128x128, four MFMA waves and four copy waves
        return (k >= 128 && n >= 128) ? 44 : 46;
    case OP_GFWD: case OP_GDIN:
        // dinput over whole 256-column tiles: 256x256, eight waves (its weights
        // are row-contiguous, read transposed); else 256x192 / 128x128, eight
        // waves, copies spread
        if (op == OP_GDIN && cols >= 2048 && cols % 256 == 0) return 52;
        if (cols >= 1024) return 111;
        return cols >= 128 ? 115 : 46;
    case OP_GDW:
        // large expert weights: 192x256, eight waves of 96x64, copies spread
        // (config 5: 8 x 8 tiles per expert, two rounds of the CUs); else
        // 128x128, four MFMA waves and four copy waves
        if (n >= 768 && k >= 1024) return 116;
        return (k >= 128 && n >= 128) ? 44 : 46;
    }
    return 44;
}

Plan make_plan(int op, int dt, int tc, int64_t k, int64_t n) {
    Plan pl{0, kNoSplit};
    if (mfma_eligible(op, dt, tc, k, n)) pl.tile = pick_tile(op, k, n, op == OP_FP8 && fp8_fast(tc));
    if (op == OP_DW) {
        // the chunk length follows from the default tile of (k, n), so a
        // forced tile below never changes the reduction order
        if (pl.tile) {
            const TileShape *ts = mfma_tile(pl.tile);
            const int64_t tiles = cdiv(k, ts->bm) * cdiv(n, ts->bn);
            pl.chunk = tiles >= 128 ? kNoSplit : 1024;
        } else {
            // scalar tier: same rule for every dtype (bf16/f16 == upcast f32)
            const int64_t tiles = cdiv(k, 64) * cdiv(n, 64);
            pl.chunk = tiles >= 128 ? kNoSplit : 256;
        }
    }
    if (kForceHook && pl.tile && tc >= kForceBase) {
        const int id = forced_tile(op, tc);
        if (mfma_tile(id)) pl.tile = id;
    }
    return pl;
}

// Launch-time model of the forward, dX and fp8 tiles.  A launch of W workgroups
// (one per CU: every candidate's LDS ring takes most of a CU's LDS) runs in
// R = ceil(W / 256) rounds; a round costs the tile's fixed time f (prologue,
// epilogue, dispatch) plus p per output element and 64-deep stage, and a
// partial round of w workgroups less in proportion to how few CUs it occupies
// (they share L2 and memory bandwidth with fewer others):
//   t = f R + p S E ((R - 1) + a + (1 - a) w / 256)
// with S = ceil(reduction / 64) stages and E = BM BN elements per tile.  f, p
// and a are least-squares fits to forced-tile timings on one MI355X (M 4096
// and 16384, reductions 512 to 4096, output widths 1024 to 5120; the choices
// at the fitted shapes are within 2 % (forward) and 11 % (dX, 0.5 % on
// average) of the fastest candidate, against 11-15 % on average and up to
// 36-56 % for a fixed tile per (k, n)).  Tiles change speed only, never bits.
struct TileCost {
    int id;
    double f_us, p_ps;
};
constexpr TileCost kFwdCost[] = {{111, 6.59, 24.06}, {52, 7.69, 23.28}, {53, 4.13, 30.52},
                                 {44, 3.25, 28.36}};
constexpr double kFwdShare = 0.65;
constexpr TileCost kDxCost[] = {{45, 3.02, 31.58}, {50, 4.98, 26.34}, {53, 4.12, 30.29},
                                {55, 2.29, 35.68}, {111, 6.75, 25.55}};
constexpr double kDxShare = 0.35;
// fp8 (A [m,k] and B^T [n,k] both reduction-contiguous): the exact path
// (codes widened to bf16) and the fp8-instruction path, fitted the same way at
// 28 shapes each (M 2048-16384, K and N 1024-8192): leave-one-out within 0.2 %
// (exact) and 0.03 % (fast) of the fastest candidate on average, 3.5 % and
// 0.6 % at worst, against 9 % and 4 % on average, up to 35 % and 48 %, for the
// default tile of (k, n)
constexpr TileCost kFp8Cost[] = {{52, 10.06, 23.26}, {111, 8.18, 22.96}, {54, 4.55, 27.03},
                                 {44, 3.72, 25.98}};
constexpr double kFp8Share = 0.40;
constexpr TileCost kFp8FastCost[] = {{112, 7.96, 10.51}, {111, 7.33, 11.43}, {41, 10.3, 13.08},
                                     {44, 3.35, 13.65}, {115, 2.58, 15.68}};
constexpr double kFp8FastShare = 0.35;
// grouped forward (segment-anchored rows: ceil(m / BM) + e row tiles), fitted
// at 16 shapes (M 2048-65536, K 1024-4096, N 512-4096, 4-64 experts): in-sample
// within 8 % of the fastest candidate at every shape, where the default tile
// of (k, n) was 25 % slower on average and up to 2x
constexpr TileCost kGfwdCost[] = {{112, 4.35, 22.95}, {111, 7.24, 22.5}, {44, 4.08, 26.06}};
constexpr double kGfwdShare = 0.85;
// grouped dinput (same segments, output width k, reduction n): 256x256 (eight
// waves, which shares a launch with the default dweights tile, so the launch's
// tail fills with dweights tiles) unless 128x128 with copy waves is modelled
// 10 % faster, both priced with the forward's fit; forced-tile timings of the
// backward at 10 shapes put this choice at the best dinput tile or within 2 %
// of it (up to 30 % faster than the tile of (k, n))
constexpr TileCost kGdinWide = {52, 4.35, 22.95}, kGdinNarrow = {44, 4.08, 26.06};
constexpr int64_t kCUs = 256;

// Modelled time of tile c (extra: row tiles beyond ceil(m / BM), the grouped
// GEMM's one partial tile per expert segment)
double model_us(const TileCost &c, double a, int64_t m, int64_t cols, int64_t red,
                int64_t extra = 0) {
    const TileShape *ts = mfma_tile(c.id);
    const int64_t w = (cdiv(m, ts->bm) + extra) * cdiv(cols, ts->bn);
    const int64_t r = cdiv(w, kCUs), last = w - kCUs * (r - 1);
    const double stage = c.p_ps * 1e-6 * (double)ts->bm * (double)ts->bn;
    return c.f_us * (double)r + stage * (double)cdiv(red, 64) *
                                    ((double)(r - 1) + a + (1.0 - a) * (double)last / (double)kCUs);
}

template <size_t N>
int model_tile(const TileCost (&tab)[N], double a, int64_t m, int64_t cols, int64_t red,
               int64_t extra = 0) {
    int best = tab[0].id;
    double best_t = 0.0;
    for (size_t i = 0; i < N; ++i) {
        const double t = model_us(tab[i], a, m, cols, red, extra);
        if (i == 0 || t < best_t) {
            best = tab[i].id;
            best_t = t;
        }
    }
    return best;
}

// Tile for the batch at hand (forward, dX, fp8; cols = the output width,
// red = the reduction length).  Small batches (128x128 tiles would fill under
// three quarters of the CUs) stream B through a few rows of A: one round (at
// most 256 workgroups) of a narrow tile spreads that stream over the most
// workgroups, and their time goes mostly to the fixed cost of each LDS stage,
// so the forward and fp8 take the deep-stage variants (32x32 with 512-byte
// stage rows while it fits one round, else 64x32 with 256-byte rows) and dX
// the 64x32 tile.  Otherwise the candidate the launch model above finds
// fastest.  The tile may follow m because every tile issues the same MFMA
// sequence per element (the bits do not change); the tier never follows m.
// Forced tiles are kept.
int batch_tile(int op, const Plan &pl, int tc, int64_t m, int64_t cols, int64_t red) {
    if (pl.tile < 40 || (kForceHook && tc >= kForceBase)) return pl.tile;
    auto wgs = [&](int id) {
        const TileShape *ts = mfma_tile(id);
        return cdiv(m, ts->bm) * cdiv(cols, ts->bn);
    };
    const bool deep = op == OP_FWD || op == OP_FP8;
    if (wgs(115) < 192) {
        if (deep && wgs(321) <= 256) return 321;
        if (deep && wgs(220) <= 256) return 220;
        if (wgs(120) <= 256) return 120;
    }
    // outputs narrower than 128 columns keep the 64x64 default (the model's
    // candidates are 128 to 256 columns wide)
    if (cols < 128) return pl.tile;
    if (op == OP_FWD) return model_tile(kFwdCost, kFwdShare, m, cols, red);
    if (op == OP_DX) return model_tile(kDxCost, kDxShare, m, cols, red);
    if (op == OP_FP8)
        return fp8_fast(tc) ? model_tile(kFp8FastCost, kFp8FastShare, m, cols, red)
                            : model_tile(kFp8Cost, kFp8Share, m, cols, red);
    return pl.tile;
}

int64_t dw_chunks(const Plan &pl, int64_t m) { return m <= 0 ? 1 : cdiv(m, pl.chunk); }

// Grouped forward and dinput tiles for m rows routed to e experts (forced
// tiles kept; outputs narrower than 128 columns keep the default)
int grouped_fwd_tile(const Plan &pl, int tc, int64_t m, int64_t k, int64_t n, int64_t e) {
    if (pl.tile < 40 || (kForceHook && tc >= kForceBase) || n < 128) return pl.tile;
    return model_tile(kGfwdCost, kGfwdShare, m, n, k, e);
}
int grouped_din_tile(const Plan &pl, int tc, int64_t m, int64_t k, int64_t n, int64_t e) {
    if (pl.tile < 40 || (kForceHook && tc >= kForceBase) || k < 128) return pl.tile;
    const double wide = model_us(kGdinWide, kGfwdShare, m, k, n, e);
    const double narrow = model_us(kGdinNarrow, kGfwdShare, m, k, n, e);
    return narrow < 0.9 * wide ? kGdinNarrow.id : kGdinWide.id;
}

int hip_status(hipError_t e) { return e == hipSuccess ? BI_OK : BI_ERR_HIP; }

// The tile that runs, its operand extents and its grid.  The direct-load family
// (ids 40, 100, 200 and 300 + base) needs 16-byte-aligned rows whose length is a
// multiple of 8 elements and operands below 2^30 bytes; otherwise the register-staged kernel
// runs on the tile every op instantiates that is closest in shape: 256x256,
// 128x128 or 64x64 (same bits either way).  The grid (tiles_i or seg_tiles,
// and tiles_j, over rows x cols) is set here from the shape that actually runs.
constexpr int64_t kDirectMaxBytes = (int64_t)1 << 30;
int direct_tile(MfmaArgs &a, int tile, int64_t a_bytes, int64_t b_bytes) {
    a.a_bytes = a_bytes;
    a.b_bytes = b_bytes;
    int t = tile;
    if (tile >= 40) {
        const bool ok =
            a.vec_a && a.vec_b && a_bytes <= kDirectMaxBytes && b_bytes <= kDirectMaxBytes;
        if (!ok) {
            const TileShape *ts = mfma_tile(tile);
            t = ts->bm >= 256 && ts->bn >= 256 ? 1 : ts->bm <= 64 && ts->bn <= 64 ? 6 : 4;
        }
    }
    const TileShape *ts = mfma_tile(t);
    if (a.offsets) a.seg_tiles = cdiv(a.rows, ts->bm) + a.n_experts;
    else a.tiles_i = cdiv(a.rows, ts->bm);
    a.tiles_j = cdiv(a.cols, ts->bn);
    return t;
}

// MFMA-tier arguments of dX = dY W^T ([m,k] from dy [m,n], w [k,n]) on tile
// `tile` (before the alignment check) and the tile that runs.
int dx_mfma_args(MfmaArgs &a, void *dx, const void *dy, const void *w, int64_t m, int64_t k,
                 int64_t n, int tile) {
    a.a = dy; a.lda = n; a.b = w; a.ldb = n; a.c = dx; a.ldc = k;
    a.rows = m; a.cols = k; a.red = n; a.chunk = kNoSplit; a.nchunks = 1;
    a.vec_a = aligned16(dy) && n % 8 == 0;
    a.vec_b = aligned16(w) && n % 8 == 0;
    a.vec_c = aligned8(dx) && k % 4 == 0;
    return direct_tile(a, tile, 2 * m * n, 2 * k * n);
}

// MFMA-tier arguments of dW = X^T dY ([k,n] from x [m,k], dy [m,n]; f32 chunk
// partials into the workspace when chunks > 1) and the tile that runs.
int dw_mfma_args(MfmaArgs &a, void *dw, const void *x, const void *dy, int64_t m, int64_t k,
                 int64_t n, const Plan &pl, int64_t chunks, void *workspace) {
    a.a = x; a.lda = k; a.b = dy; a.ldb = n; a.c = dw; a.ldc = n;
    a.ws = static_cast<float *>(workspace);
    a.rows = k; a.cols = n; a.red = m; a.chunk = pl.chunk; a.nchunks = chunks;
    a.vec_a = aligned16(x) && k % 8 == 0;
    a.vec_b = aligned16(dy) && n % 8 == 0;
    a.vec_c = chunks > 1 ? (aligned16(workspace) && n % 4 == 0) : (aligned8(dw) && n % 4 == 0);
    return direct_tile(a, pl.tile, 2 * m * k, 2 * m * n);
}

}  // namespace

extern "C" {

const char *bi_status_string(int status) {
    switch (status) {
    case BI_OK: return "BI_OK: success";
    case BI_ERR_NULL: return "BI_ERR_NULL: a required pointer is NULL";
    case BI_ERR_DTYPE: return "BI_ERR_DTYPE: unsupported dtype";
    case BI_ERR_SHAPE: return "BI_ERR_SHAPE: invalid dimension";
    case BI_ERR_TOO_LARGE: return "BI_ERR_TOO_LARGE: a tensor exceeds 2^40 elements";
    case BI_ERR_WORKSPACE: return "BI_ERR_WORKSPACE: workspace missing or too small";
    case BI_ERR_HIP: return "BI_ERR_HIP: a HIP launch failed";
    case BI_ERR_UNSUPPORTED: return "BI_ERR_UNSUPPORTED: no tier for this dtype/tc";
    }
    return "unknown bi status";
}

int bi_plan(int op, int dtype, int tc, int64_t k, int64_t n, int64_t *chunk_rows) {
    if (op < OP_FWD || op > OP_GDW) return BI_ERR_UNSUPPORTED;
    if (op != OP_FP8 && !dtype_ok(dtype)) return BI_ERR_DTYPE;
    if (k < 0 || n < 0) return BI_ERR_SHAPE;
    const int ts = tier_check(op, op == OP_FP8 ? BI_BF16 : dtype, tc, k, n);
    if (ts != BI_OK) return ts;
    Plan pl = make_plan(op, op == OP_FP8 ? BI_BF16 : dtype, tc, k, n);
    if (chunk_rows) *chunk_rows = pl.chunk;
    return pl.tile;
}

int bi_plan_batch(int op, int dtype, int tc, int64_t m, int64_t k, int64_t n, int64_t e) {
    const int t = bi_plan(op, dtype, tc, k, n, nullptr);
    if (t <= 0) return t;
    if (m < 0 || e < 0) return BI_ERR_SHAPE;
    if (m == 0) return t;
    const Plan pl = make_plan(op, op == OP_FP8 ? BI_BF16 : dtype, tc, k, n);
    if (op == OP_FWD || op == OP_FP8) return batch_tile(op, pl, tc, m, n, k);
    if (op == OP_DX) return batch_tile(op, pl, tc, m, k, n);
    if (op == OP_GFWD) return grouped_fwd_tile(pl, tc, m, k, n, e);
    if (op == OP_GDIN) return grouped_din_tile(pl, tc, m, k, n, e);
    return t;
}

int bi_forward(void *y, const void *x, const void *w, const void *bias, int64_t m, int64_t k,
               int64_t n, int dtype, hipStream_t stream, int tc) {
    if (!dtype_ok(dtype)) return BI_ERR_DTYPE;
    if (m < 0 || k < 0 || n < 0) return BI_ERR_SHAPE;
    if (checked_elems(m, k) < 0 || checked_elems(k, n) < 0 || checked_elems(m, n) < 0)
        return BI_ERR_TOO_LARGE;
    { const int ts = tier_check(OP_FWD, dtype, tc, k, n); if (ts != BI_OK) return ts; }
    if (m == 0 || n == 0) return BI_OK;
    if (!y || (k > 0 && (!x || !w))) return BI_ERR_NULL;
    const Plan pl = make_plan(OP_FWD, dtype, tc, k, n);
    if (pl.tile == 0) {
        ScalarGemmArgs a{};
        a.a = x; a.a_is = k; a.a_rs = 1;
        a.b = w; a.b_rs = n; a.b_js = 1;
        a.bias = bias; a.c = y; a.ldc = n;
        a.rows = m; a.cols = n; a.red = k; a.chunk = kNoSplit; a.nchunks = 1;
        a.tiles_i = cdiv(m, 64); a.tiles_j = cdiv(n, 64);
        return hip_status(launch_scalar_gemm(a, dtype, dtype, 0, stream));
    }
    MfmaArgs a{};
    a.a = x; a.lda = k; a.b = w; a.ldb = n; a.c = y; a.ldc = n; a.bias = bias;
    a.rows = m; a.cols = n; a.red = k; a.chunk = kNoSplit; a.nchunks = 1;
    a.vec_a = aligned16(x) && k % 8 == 0;
    a.vec_b = aligned16(w) && n % 8 == 0;
    a.vec_c = aligned8(y) && n % 4 == 0;
    const int tile = direct_tile(a, batch_tile(OP_FWD, pl, tc, m, n, k), 2 * m * k, 2 * k * n);
    return hip_status(launch_mfma_gemm(a, tile, dtype, /*layout A rc, B strided*/ 1, 0, stream));
}

int bi_backward_dx(void *dx, const void *dy, const void *w, int64_t m, int64_t k, int64_t n,
                   int dtype, hipStream_t stream, int tc) {
    if (!dtype_ok(dtype)) return BI_ERR_DTYPE;
    if (m < 0 || k < 0 || n < 0) return BI_ERR_SHAPE;
    if (checked_elems(m, k) < 0 || checked_elems(k, n) < 0 || checked_elems(m, n) < 0)
        return BI_ERR_TOO_LARGE;
    { const int ts = tier_check(OP_DX, dtype, tc, k, n); if (ts != BI_OK) return ts; }
    if (m == 0 || k == 0) return BI_OK;
    if (!dx || (n > 0 && (!dy || !w))) return BI_ERR_NULL;
    const Plan pl = make_plan(OP_DX, dtype, tc, k, n);
    if (pl.tile == 0) {
        ScalarGemmArgs a{};
        a.a = dy; a.a_is = n; a.a_rs = 1;
        a.b = w; a.b_rs = 1; a.b_js = n;
        a.c = dx; a.ldc = k;
        a.rows = m; a.cols = k; a.red = n; a.chunk = kNoSplit; a.nchunks = 1;
        a.tiles_i = cdiv(m, 64); a.tiles_j = cdiv(k, 64);
        return hip_status(launch_scalar_gemm(a, dtype, dtype, 0, stream));
    }
    MfmaArgs a{};
    const int tile = dx_mfma_args(a, dx, dy, w, m, k, n, batch_tile(OP_DX, pl, tc, m, k, n));
    return hip_status(launch_mfma_gemm(a, tile, dtype, /*both rc*/ 3, 0, stream));
}

size_t bi_backward_dw_workspace_bytes(int64_t m, int64_t k, int64_t n, int dtype, int tc) {
    if (!dtype_ok(dtype) || m < 0 || k < 0 || n < 0) return 0;
    if (checked_elems(m, k) < 0 || checked_elems(m, n) < 0 || checked_elems(k, n) < 0) return 0;
    if (tier_check(OP_DW, dtype, tc, k, n) != BI_OK) return 0;
    const Plan pl = make_plan(OP_DW, dtype, tc, k, n);
    const int64_t chunks = dw_chunks(pl, m);
    if (chunks <= 1) return 0;
    return (size_t)chunks * (size_t)k * (size_t)n * sizeof(float);
}

int bi_backward_dw(void *dw, const void *x, const void *dy, int64_t m, int64_t k, int64_t n,
                   int dtype, void *workspace, size_t workspace_bytes, hipStream_t stream,
                   int tc) {
    if (!dtype_ok(dtype)) return BI_ERR_DTYPE;
    if (m < 0 || k < 0 || n < 0) return BI_ERR_SHAPE;
    if (checked_elems(m, k) < 0 || checked_elems(k, n) < 0 || checked_elems(m, n) < 0)
        return BI_ERR_TOO_LARGE;
    { const int ts = tier_check(OP_DW, dtype, tc, k, n); if (ts != BI_OK) return ts; }
    if (k == 0 || n == 0) return BI_OK;
    if (!dw || (m > 0 && (!x || !dy))) return BI_ERR_NULL;
    const Plan pl = make_plan(OP_DW, dtype, tc, k, n);
    const int64_t chunks = dw_chunks(pl, m);
    const size_t need = chunks > 1 ? (size_t)chunks * (size_t)k * (size_t)n * sizeof(float) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need)) return BI_ERR_WORKSPACE;
    const int epi = chunks > 1 ? 1 : 0;
    hipError_t e;
    if (pl.tile == 0) {
        ScalarGemmArgs a{};
        a.a = x; a.a_is = 1; a.a_rs = k;
        a.b = dy; a.b_rs = n; a.b_js = 1;
        a.c = dw; a.ldc = n; a.ws = static_cast<float *>(workspace);
        a.rows = k; a.cols = n; a.red = m; a.chunk = pl.chunk; a.nchunks = chunks;
        a.tiles_i = cdiv(k, 64); a.tiles_j = cdiv(n, 64);
        e = launch_scalar_gemm(a, dtype, epi ? BI_F32 : dtype, epi, stream);
    } else {
        MfmaArgs a{};
        const int tile = dw_mfma_args(a, dw, x, dy, m, k, n, pl, chunks, workspace);
        e = launch_mfma_gemm(a, tile, dtype, /*both strided*/ 0, epi, stream);
    }
    if (e != hipSuccess) return BI_ERR_HIP;
    if (chunks > 1)
        e = launch_chunk_sum(static_cast<const float *>(workspace), dw, k * n, chunks, dtype,
                             stream);
    return hip_status(e);
}

int bi_linear_backward(void *dx, void *dw, const void *dy, const void *x, const void *w,
                       int64_t m, int64_t k, int64_t n, int dtype, void *workspace,
                       size_t workspace_bytes, hipStream_t stream, int tc) {
    if (!dx && !dw) {
        // nothing requested: valid only when both outputs, dx [m,k] and dw
        // [k,n], are empty (callers may pass NULL for an empty tensor)
        if (!dtype_ok(dtype)) return BI_ERR_DTYPE;
        if (m < 0 || k < 0 || n < 0) return BI_ERR_SHAPE;
        return (k == 0 || (m == 0 && n == 0)) ? BI_OK : BI_ERR_NULL;
    }
    if (!dw) return bi_backward_dx(dx, dy, w, m, k, n, dtype, stream, tc);
    if (!dx) return bi_backward_dw(dw, x, dy, m, k, n, dtype, workspace, workspace_bytes, stream, tc);
    // every check of the two calls, before anything is enqueued
    if (!dtype_ok(dtype)) return BI_ERR_DTYPE;
    if (m < 0 || k < 0 || n < 0) return BI_ERR_SHAPE;
    if (checked_elems(m, k) < 0 || checked_elems(k, n) < 0 || checked_elems(m, n) < 0)
        return BI_ERR_TOO_LARGE;
    { const int ts = tier_check(OP_DX, dtype, tc, k, n); if (ts != BI_OK) return ts; }
    { const int ts = tier_check(OP_DW, dtype, tc, k, n); if (ts != BI_OK) return ts; }
    if (m > 0 && k > 0 && n > 0 && (!dy || !w || !x)) return BI_ERR_NULL;
    const Plan px = make_plan(OP_DX, dtype, tc, k, n), pw = make_plan(OP_DW, dtype, tc, k, n);
    const int64_t chunks = dw_chunks(pw, m);
    const size_t need = chunks > 1 ? (size_t)chunks * (size_t)k * (size_t)n * sizeof(float) : 0;
    if (k > 0 && n > 0 && need > 0 && (!workspace || workspace_bytes < need))
        return BI_ERR_WORKSPACE;
    if (m > 0 && k > 0 && n > 0 && px.tile != 0 && pw.tile != 0 && chunks == 1) {
        MfmaArgs ax{}, aw{};
        // the pair runs the (k, n) default dX tile (128x96 where it applies)
        const int tx = dx_mfma_args(ax, dx, dy, w, m, k, n, px.tile);
        const int tw = dw_mfma_args(aw, dw, x, dy, m, k, n, pw, 1, nullptr);
        // one launch pays off while the dX tiles alone fill most CUs; with fewer,
        // the dX tiles (on the critical path, with the shorter ring of the
        // shared launch) are faster in a launch of their own
        if (mfma_backward_pair(tx, tw, dtype) && ax.tiles_i * ax.tiles_j >= 192)
            return hip_status(launch_mfma_backward(ax, tx, aw, tw, dtype, stream));
    }
    const int st = bi_backward_dx(dx, dy, w, m, k, n, dtype, stream, tc);
    if (st != BI_OK) return st;
    return bi_backward_dw(dw, x, dy, m, k, n, dtype, workspace, workspace_bytes, stream, tc);
}

size_t bi_bias_grad_workspace_bytes(int64_t m, int64_t n, int dtype) {
    if (!dtype_ok(dtype) || m < 0 || n < 0 || checked_elems(m, n) < 0) return 0;
    const int64_t chunks = m <= 0 ? 1 : cdiv(m, BG_CHUNK);
    return chunks > 1 ? (size_t)chunks * (size_t)n * sizeof(float) : 0;
}

int bi_bias_grad(void *db, const void *dy, int64_t m, int64_t n, int dtype, void *workspace,
                 size_t workspace_bytes, hipStream_t stream) {
    if (!dtype_ok(dtype)) return BI_ERR_DTYPE;
    if (m < 0 || n < 0) return BI_ERR_SHAPE;
    if (checked_elems(m, n) < 0) return BI_ERR_TOO_LARGE;
    if (n == 0) return BI_OK;
    if (!db || (m > 0 && !dy)) return BI_ERR_NULL;
    const int64_t chunks = m <= 0 ? 1 : cdiv(m, BG_CHUNK);
    const size_t need = chunks > 1 ? (size_t)chunks * (size_t)n * sizeof(float) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 3u)))
        return BI_ERR_WORKSPACE;
    const bool vec = aligned16(dy) && n % 8 == 0;
    return hip_status(launch_bias_grad(dy, m, n, chunks, static_cast<float *>(workspace), db,
                                       dtype, vec, stream));
}

}  // extern "C"

namespace {

// Y = RNE_bf16((A B^T) * a_dequant * b_dequant [+ bias]): the fp8 GEMM behind
// bi_fp8_mm and the scaled fp8 linear.  Validates like bi_fp8_mm.
int fp8_gemm(void *y, const void *a, const void *bt, const float *a_dequant,
             const float *b_dequant, const void *bias, int64_t m, int64_t k, int64_t n,
             hipStream_t stream, int tc) {
    if (m < 0 || k < 0 || n < 0) return BI_ERR_SHAPE;
    if (checked_elems(m, k) < 0 || checked_elems(n, k) < 0 || checked_elems(m, n) < 0)
        return BI_ERR_TOO_LARGE;
    { const int ts = tier_check(OP_FP8, BI_BF16, tc, k, n); if (ts != BI_OK) return ts; }
    if (m == 0 || n == 0) return BI_OK;
    if (!y || !a_dequant || !b_dequant || (k > 0 && (!a || !bt))) return BI_ERR_NULL;
    const Plan pl = make_plan(OP_FP8, BI_BF16, tc, k, n);
    if (pl.tile == 0) {
        ScalarGemmArgs s{};
        s.a = a; s.a_is = k; s.a_rs = 1;
        s.b = bt; s.b_rs = 1; s.b_js = k;
        s.scale_a = a_dequant; s.scale_b = b_dequant;
        s.bias = bias;
        s.c = y; s.ldc = n;
        s.rows = m; s.cols = n; s.red = k; s.chunk = kNoSplit; s.nchunks = 1;
        s.tiles_i = cdiv(m, 64); s.tiles_j = cdiv(n, 64);
        return hip_status(launch_scalar_gemm(s, 3 /*e4m3*/, BI_BF16, 2, stream));
    }
    const bool vec = aligned16(a) && aligned16(bt) && k % 16 == 0;
    const bool fast = fp8_fast(tc);
    if (pl.tile >= 40 && vec && m * k <= kDirectMaxBytes && n * k <= kDirectMaxBytes) {
        MfmaArgs d{};
        d.a = a; d.lda = k; d.b = bt; d.ldb = k; d.c = y; d.ldc = n;
        d.rows = m; d.cols = n; d.red = k; d.chunk = kNoSplit; d.nchunks = 1;
        d.vec_a = d.vec_b = 1;
        d.vec_c = aligned8(y) && n % 4 == 0;
        d.scale_a = a_dequant; d.scale_b = b_dequant;
        d.bias = bias;
        const int tile = direct_tile(d, batch_tile(OP_FP8, pl, tc, m, n, k), m * k, n * k);
        return hip_status(launch_fp8_dl(d, tile, fast, stream));
    }
    // register-staged fp8 kernel: 256x256, 128x128 or 64x64 tiles
    const TileShape *ts = mfma_tile(pl.tile);
    int tile = pl.tile;
    if (tile >= 40) tile = ts->bm >= 256 && ts->bn >= 256 ? 1 : ts->bm <= 64 ? 6 : 4;
    ts = mfma_tile(tile);
    Fp8Args f{};
    f.a = static_cast<const uint8_t *>(a);
    f.bt = static_cast<const uint8_t *>(bt);
    f.c = static_cast<uint16_t *>(y);
    f.scale_a = a_dequant; f.scale_b = b_dequant;
    f.bias = static_cast<const uint16_t *>(bias);
    f.m = m; f.n = n; f.k = k;
    f.tiles_i = cdiv(m, ts->bm); f.tiles_j = cdiv(n, ts->bn);
    f.vec = vec;
    f.vec_c = aligned8(y) && n % 4 == 0;
    return hip_status(launch_fp8_gemm(f, tile, fast, stream));
}

}  // namespace

extern "C" {

int bi_fp8_mm(void *y, const void *a, const void *bt, const float *a_dequant,
              const float *b_dequant, int64_t m, int64_t k, int64_t n, hipStream_t stream,
              int tc) {
    return fp8_gemm(y, a, bt, a_dequant, b_dequant, nullptr, m, k, n, stream, tc);
}

static bool fp8_fmt_ok(int fmt) { return fmt == BI_FP8_E4M3 || fmt == BI_FP8_E5M2; }
static size_t align256(int64_t bytes) { return (size_t)((bytes + 255) / 256 * 256); }

int bi_fp8_quantize(void *dst, const void *src, const float *scale_inv, float *amax, int64_t n,
                    int fmt, hipStream_t stream) {
    if (!fp8_fmt_ok(fmt)) return BI_ERR_DTYPE;
    if (n < 0) return BI_ERR_SHAPE;
    if (n > kMaxElems) return BI_ERR_TOO_LARGE;
    if (n == 0) return BI_OK;
    if (!dst || !src || !scale_inv) return BI_ERR_NULL;
    return hip_status(launch_quantize(src, scale_inv, dst, amax, n, fmt, stream));
}

int bi_fp8_transpose_quantize(void *dst, const void *src, const float *scale_inv, float *amax,
                              int64_t rows, int64_t cols, int fmt, hipStream_t stream) {
    if (!fp8_fmt_ok(fmt)) return BI_ERR_DTYPE;
    if (rows < 0 || cols < 0) return BI_ERR_SHAPE;
    if (checked_elems(rows, cols) < 0 || rows > (int64_t)65535 * 64) return BI_ERR_TOO_LARGE;
    if (rows == 0 || cols == 0) return BI_OK;
    if (!dst || !src || !scale_inv) return BI_ERR_NULL;
    return hip_status(launch_transpose_quantize(src, scale_inv, dst, nullptr, amax, rows, cols, fmt,
                                                stream));
}

size_t bi_fp8_linear_workspace_bytes(int64_t m, int64_t k, int64_t n) {
    if (m < 0 || k < 0 || n < 0) return 0;
    if (checked_elems(m, k) < 0 || checked_elems(n, k) < 0 || checked_elems(m, n) < 0) return 0;
    const size_t fwd = align256(m * k) + align256(n * k);
    const size_t bwd = align256(m * n) + align256(k * n) + align256(n * m) + align256(k * m) + 256;
    return fwd > bwd ? fwd : bwd;
}

int bi_fp8_linear_forward(void *y, const void *x, const void *w, const void *bias,
                          const float *sx, const float *sw, const float *sx_inv,
                          const float *sw_inv, float *amax_x, float *amax_w, int64_t m,
                          int64_t k, int64_t n, void *workspace, size_t workspace_bytes,
                          hipStream_t stream, int tc) {
    if (m < 0 || k < 0 || n < 0) return BI_ERR_SHAPE;
    if (checked_elems(m, k) < 0 || checked_elems(n, k) < 0 || checked_elems(m, n) < 0 ||
        m > (int64_t)65535 * 64 || n > (int64_t)65535 * 64)
        return BI_ERR_TOO_LARGE;
    { const int ts = tier_check(OP_FP8, BI_BF16, tc, k, n); if (ts != BI_OK) return ts; }
    if (!sx || !sw || !sx_inv || !sw_inv) return BI_ERR_NULL;
    if ((m > 0 && n > 0 && !y) || (m * k > 0 && !x) || (n * k > 0 && !w)) return BI_ERR_NULL;
    const size_t need = align256(m * k) + align256(n * k);
    if (need > 0 && (!workspace || workspace_bytes < need)) return BI_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    void *x8 = ws, *w8 = ws + align256(m * k);
    if (amax_x || amax_w)
        if (launch_zero3(amax_x, amax_w, nullptr, stream) != hipSuccess) return BI_ERR_HIP;
    int st = bi_fp8_quantize(x8, x, sx_inv, amax_x, m * k, BI_FP8_E4M3, stream);
    if (st != BI_OK) return st;
    st = bi_fp8_quantize(w8, w, sw_inv, amax_w, n * k, BI_FP8_E4M3, stream);
    if (st != BI_OK) return st;
    return fp8_gemm(y, x8, w8, sx, sw, bias, m, k, n, stream, tc);
}

int bi_fp8_linear_backward(void *dx, void *dw, const void *g, const void *x, const void *w,
                           const float *sg, const float *sw, const float *sx,
                           const float *sg_inv, const float *sw_inv, const float *sx_inv,
                           float *amax_g, int64_t m, int64_t k, int64_t n, void *workspace,
                           size_t workspace_bytes, hipStream_t stream, int tc) {
    if (m < 0 || k < 0 || n < 0) return BI_ERR_SHAPE;
    if (checked_elems(m, k) < 0 || checked_elems(n, k) < 0 || checked_elems(m, n) < 0 ||
        m > (int64_t)65535 * 64 || n > (int64_t)65535 * 64)
        return BI_ERR_TOO_LARGE;
    // dX GEMM: reduction n, columns k; dW GEMM: reduction m, columns k
    if (dx) { const int ts = tier_check(OP_FP8, BI_BF16, tc, n, k); if (ts != BI_OK) return ts; }
    if (dw) { const int ts = tier_check(OP_FP8, BI_BF16, tc, m, k); if (ts != BI_OK) return ts; }
    if (!sg || !sw || !sx || !sg_inv || !sw_inv || !sx_inv) return BI_ERR_NULL;
    if ((m * n > 0 && !g) || (dx && n * k > 0 && !w) || (dw && m * k > 0 && !x))
        return BI_ERR_NULL;
    const size_t o_wt = align256(m * n), o_gt = o_wt + align256(k * n);
    const size_t o_xt = o_gt + align256(n * m), o_amax = o_xt + align256(k * m);
    const size_t need = o_amax + 256;
    if (!workspace || workspace_bytes < need) return BI_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    const bool need_dx = dx && m > 0 && k > 0, need_dw = dw && n > 0 && k > 0;
    if (launch_zero3(amax_g, nullptr, nullptr, stream) != hipSuccess) return BI_ERR_HIP;
    // g is read once: with dW wanted, the transposing quantiser writes gt8 and
    // (when dX is wanted too) g8 from the same read and folds amax_g; the
    // transposed copies of w and x fold no max-abs (the page keeps theirs in a
    // scratch value that nothing reads)
    hipError_t e;
    if (need_dw)
        e = launch_transpose_quantize(g, sg_inv, ws + o_gt, need_dx ? ws : nullptr, amax_g, m, n,
                                      BI_FP8_E4M3, stream);
    else
        e = launch_quantize(g, sg_inv, ws, amax_g, m * n, BI_FP8_E4M3, stream);
    if (e != hipSuccess) return BI_ERR_HIP;
    int st;
    if (need_dx) {
        // dX[m,k] = (g8[m,n] . wt8[k,n]^T) * sg * sw
        e = launch_transpose_quantize(w, sw_inv, ws + o_wt, nullptr, nullptr, n, k, BI_FP8_E4M3,
                                      stream);
        if (e != hipSuccess) return BI_ERR_HIP;
        st = fp8_gemm(dx, ws, ws + o_wt, sg, sw, nullptr, m, n, k, stream, tc);
        if (st != BI_OK) return st;
    }
    if (need_dw) {
        // dW[n,k] = (gt8[n,m] . xt8[k,m]^T) * sg * sx
        e = launch_transpose_quantize(x, sx_inv, ws + o_xt, nullptr, nullptr, m, k, BI_FP8_E4M3,
                                      stream);
        if (e != hipSuccess) return BI_ERR_HIP;
        st = fp8_gemm(dw, ws + o_gt, ws + o_xt, sg, sx, nullptr, n, m, k, stream, tc);
        if (st != BI_OK) return st;
    }
    return BI_OK;
}

static int grouped_validate(int64_t m, int64_t k, int64_t n, int64_t e, int dtype) {
    if (!dtype_ok(dtype)) return BI_ERR_DTYPE;
    if (m < 0 || k <= 0 || n <= 0 || e <= 0) return BI_ERR_SHAPE;
    if (checked_elems(m, k) < 0 || checked_elems(m, n) < 0 || checked_elems(e, n, k) < 0)
        return BI_ERR_TOO_LARGE;
    if (m > 0xffffffffLL) return BI_ERR_TOO_LARGE;  // row indices are uint32 offsets
    return BI_OK;
}

int bi_grouped_nt(void *y, const void *input, const void *weights, const uint32_t *row_experts,
                  const uint32_t *offsets, int64_t m, int64_t k, int64_t n, int64_t e, int dtype,
                  hipStream_t stream, int tc) {
    int st = grouped_validate(m, k, n, e, dtype);
    if (st != BI_OK) return st;
    { const int ts = tier_check(OP_GFWD, dtype, tc, k, n); if (ts != BI_OK) return ts; }
    if (m == 0) return BI_OK;
    if (!y || !input || !weights || !row_experts) return BI_ERR_NULL;
    const Plan pl = make_plan(OP_GFWD, dtype, tc, k, n);
    if (pl.tile == 0) {
        GroupedScalarArgs g{};
        g.input = input; g.weights = weights; g.row_experts = row_experts; g.offsets = offsets;
        g.out = y; g.m = m; g.k = k; g.n = n; g.e = e;
        return hip_status(launch_grouped_scalar(g, 0, dtype, stream));
    }
    if (!offsets) return BI_ERR_NULL;
    MfmaArgs a{};
    a.a = input; a.lda = k; a.b = weights; a.ldb = k; a.c = y; a.ldc = n;
    a.rows = m; a.cols = n; a.red = k; a.chunk = kNoSplit; a.nchunks = 1;
    a.offsets = offsets; a.n_experts = e; a.b_expert_stride = n * k;
    a.vec_a = aligned16(input) && k % 8 == 0;
    a.vec_b = aligned16(weights) && k % 8 == 0;
    a.vec_c = aligned8(y) && n % 4 == 0;
    const int tile = direct_tile(a, grouped_fwd_tile(pl, tc, m, k, n, e), 2 * m * k, 2 * e * n * k);
    // more slots than one round: the split launch (same bits; forced tiles run
    // the plain launch)
    if (!(kForceHook && tc >= kForceBase) && mfma_grouped_split(tile, dtype) &&
        seg_grid_rows(a.seg_tiles) * a.tiles_j > kGroupedSplitCUs)
        return hip_status(launch_mfma_grouped_split(a, tile, dtype, stream));
    return hip_status(launch_mfma_gemm(a, tile, dtype, 3, 0, stream));
}

int bi_grouped_nt_backward(void *dinput, float *dweights, const void *input, const void *weights,
                           const void *grad_out, const uint32_t *row_experts,
                           const uint32_t *offsets, int64_t m, int64_t k, int64_t n, int64_t e,
                           int dtype, hipStream_t stream, int tc) {
    int st = grouped_validate(m, k, n, e, dtype);
    if (st != BI_OK) return st;
    { const int ts = tier_check(OP_GDIN, dtype, tc, k, n); if (ts != BI_OK) return ts; }
    { const int ts = tier_check(OP_GDW, dtype, tc, k, n); if (ts != BI_OK) return ts; }
    if (!dweights || !offsets) return BI_ERR_NULL;
    if (m > 0 && (!dinput || !input || !weights || !grad_out || !row_experts)) return BI_ERR_NULL;
    // dinput (skipped for an empty batch): the scalar tier launches here, the
    // MFMA tier below (with dweights in one launch where the tile pair allows)
    MfmaArgs ad{};
    int tile_d = 0;
    if (m > 0) {
        const Plan pl = make_plan(OP_GDIN, dtype, tc, k, n);
        if (pl.tile == 0) {
            GroupedScalarArgs g{};
            g.grad_out = grad_out; g.weights = weights; g.row_experts = row_experts;
            g.out = dinput; g.m = m; g.k = k; g.n = n; g.e = e;
            if (launch_grouped_scalar(g, 1, dtype, stream) != hipSuccess) return BI_ERR_HIP;
        } else {
            ad.a = grad_out; ad.lda = n; ad.b = weights; ad.ldb = k; ad.c = dinput; ad.ldc = k;
            ad.rows = m; ad.cols = k; ad.red = n; ad.chunk = kNoSplit; ad.nchunks = 1;
            ad.offsets = offsets; ad.n_experts = e; ad.b_expert_stride = n * k;
            ad.vec_a = aligned16(grad_out) && n % 8 == 0;
            ad.vec_b = aligned16(weights) && k % 8 == 0;
            ad.vec_c = aligned8(dinput) && k % 4 == 0;
            tile_d = direct_tile(ad, grouped_din_tile(pl, tc, m, k, n, e), 2 * m * n, 2 * e * n * k);
        }
    }
    // dweights (always written, so experts without rows get +0)
    const Plan pw = make_plan(OP_GDW, dtype, tc, k, n);
    if (pw.tile == 0 || m == 0) {
        if (tile_d && launch_mfma_gemm(ad, tile_d, dtype, 1, 0, stream) != hipSuccess)
            return BI_ERR_HIP;
        GroupedScalarArgs g{};
        g.input = input; g.grad_out = grad_out; g.offsets = offsets; g.dweights = dweights;
        g.m = m; g.k = k; g.n = n; g.e = e;
        return hip_status(launch_grouped_scalar(g, 2, dtype, stream));
    }
    MfmaArgs a{};
    a.a = grad_out; a.lda = n; a.b = input; a.ldb = k; a.c = dweights; a.ldc = k;
    a.rows = n; a.cols = k; a.red = m; a.chunk = kNoSplit; a.nchunks = 1;
    a.red_offsets = offsets; a.n_experts = e; a.c_expert_stride = n * k;
    a.vec_a = aligned16(grad_out) && n % 8 == 0;
    a.vec_b = aligned16(input) && k % 8 == 0;
    a.vec_c = aligned16(dweights) && k % 4 == 0;
    const int tile = direct_tile(a, pw.tile, 2 * m * n, 2 * m * k);
    if (tile_d && mfma_grouped_backward_pair(tile_d, tile, dtype))
        return hip_status(launch_mfma_grouped_backward(ad, tile_d, a, tile, dtype, stream));
    if (tile_d && launch_mfma_gemm(ad, tile_d, dtype, 1, 0, stream) != hipSuccess) return BI_ERR_HIP;
    return hip_status(launch_mfma_gemm(a, tile, dtype, 0, 2, stream));
}

}  // extern "C"
