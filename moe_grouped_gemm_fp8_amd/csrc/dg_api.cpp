// C ABI of the FP8 GEMM library: argument validation (pure host code, no HIP call before it
// passes), the tile-configuration heuristic, the split-K workspace, and the launches.
#include <hip/hip_runtime_api.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <mutex>
#include <set>
#include <string>
#include <tuple>

#include "../../include/dg.h"
#include "dg_internal.h"
#include "dg_tiles.h"

namespace {

thread_local char g_err[512] = "";
int g_num_cus_cap = 0;

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok()
{
    g_err[0] = '\0';
    return DG_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape and pointer checks shared by every entry point; `rows` is the number of A rows per
// group (m, m_total or m_max).  With zero rows A, sfa and D may be null (empty tensors).
int check_common(const void *a, const float *sfa, int64_t ld_sfa, const void *b,
                 const float *sfb, const void *d, int64_t rows, int n, int k)
{
    if (!b || !sfb || (rows > 0 && (!a || !sfa || !d)))
        return fail(DG_ERR_INVALID_ARG, "null tensor pointer");
    if (rows < 0 || n <= 0 || k <= 0)
        return fail(DG_ERR_INVALID_ARG, "sizes must be positive (rows=%lld n=%d k=%d)",
                    (long long)rows, n, k);
    if (k % 128 != 0)
        return fail(DG_ERR_UNSUPPORTED, "k=%d is not a multiple of 128", k);
    if (n % 16 != 0)
        return fail(DG_ERR_UNSUPPORTED, "n=%d is not a multiple of 16", n);
    if (ld_sfa < rows)
        return fail(DG_ERR_INVALID_ARG, "ld_sfa=%lld is smaller than the row count %lld",
                    (long long)ld_sfa, (long long)rows);
    if (ld_sfa % 4 != 0)
        return fail(DG_ERR_MISALIGNED, "ld_sfa=%lld is not a multiple of 4", (long long)ld_sfa);
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 16))
        return fail(DG_ERR_MISALIGNED, "A, B and D must be 16-byte aligned");
    // the A scales are copied 16 bytes (four rows) at a time from sfa + row
    if (!aligned(sfa, 16))
        return fail(DG_ERR_MISALIGNED, "sfa must be 16-byte aligned");
    if (!aligned(sfb, 4))
        return fail(DG_ERR_MISALIGNED, "sfb must be 4-byte aligned");
    return DG_OK;
}

int device_cus(int *out)
{
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return fail(DG_ERR_HIP, "no HIP device available");
    std::lock_guard<std::mutex> lk(mu);
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess ||
            cus <= 0)
            return fail(DG_ERR_HIP, "cannot query the compute-unit count");
        cached[dev] = cus;
    }
    *out = cached[dev];
    if (g_num_cus_cap > 0 && g_num_cus_cap < *out)
        *out = g_num_cus_cap;
    return DG_OK;
}

// Library-owned device workspaces (the split-K partial tiles of the streaming kernel, the
// transposed operands of the dense NN/TN/TT layouts): one per (device, stream, purpose), so that
// calls on different streams never share one.  A workspace is allocated on the first call that
// needs it on its stream while that stream is not being captured, and replaced by a larger one
// (at least twice the size) when a call needs more; a replaced one is never freed, since graphs
// captured earlier keep its address and may still be replayed.  A captured call that finds no
// large enough workspace for its stream gets none (*out = nullptr) and takes a path without it.
// A graph keeps using the workspace of the stream it was captured on, wherever it is replayed.
enum WsKind { WS_SPLITK = 0, WS_LAYOUT = 1 };

int stream_workspace(int kind, hipStream_t stream, size_t need, void **out)
{
    static std::mutex mu;
    static std::map<std::tuple<int, uintptr_t, int>, std::pair<void *, size_t>> table;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(DG_ERR_HIP, "no HIP device available");
    std::lock_guard<std::mutex> lk(mu);
    std::pair<void *, size_t> &e = table[std::make_tuple(dev, (uintptr_t)stream, kind)];
    if (e.first && e.second >= need) {
        *out = e.first;
        return DG_OK;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
        *out = nullptr;
        return DG_OK;
    }
    constexpr size_t kUnit = (size_t)4 << 20;
    size_t bytes = e.second * 2 > need ? e.second * 2 : need;
    bytes = (bytes + kUnit - 1) / kUnit * kUnit;
    void *p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess)
        return fail(DG_ERR_HIP, "workspace allocation of %zu bytes failed", bytes);
    e = std::make_pair(p, bytes);  // the previous buffer stays allocated (see above)
    *out = p;
    return DG_OK;
}

int forced_config()
{
    const char *s = getenv("DG_FORCE_CONFIG");
    if (!s || !*s)
        return -1;
    for (int c = 0; c < dg::CFG_COUNT; ++c)
        if (strcmp(s, dg::kTiles[c].name) == 0)
            return c;
    return -1;
}

// Workgroups a persistent tile configuration may launch: one per CU.  DG_NO_PERSIST=1
// launches one per tile (for comparisons); DG_PERSIST_WGS=n caps them at n (tests: many
// tiles per workgroup on small problems).
int persistent_wgs(int cus)
{
    const char *s = getenv("DG_NO_PERSIST");
    if (s && *s && *s != '0')
        return 0;
    const char *w = getenv("DG_PERSIST_WGS");
    if (w && *w && atoi(w) > 0)
        return atoi(w);
    return cus;
}

int forced_splits()
{
    const char *s = getenv("DG_FORCE_SPLITS");
    return (s && *s) ? atoi(s) : 0;
}

void print_config(const char *what, int m, int n, int k, int g, int cfg, int splits,
                  int expected_m = -1, int tail = 0)
{
    static std::mutex mu;
    static std::set<std::tuple<std::string, int, int, int, int, int>> seen;
    const char *env = getenv("DG_PRINT_CONFIGS");
    if (!env || !*env || *env == '0')
        return;
    std::lock_guard<std::mutex> lk(mu);
    if (!seen.insert(std::make_tuple(std::string(what), m, n, k, g, expected_m)).second)
        return;
    char hint[32] = "";
    if (expected_m >= 0)
        snprintf(hint, sizeof(hint), " expected_m=%d", expected_m);
    char tl[64] = "";
    if (tail > 0)
        snprintf(tl, sizeof(tl), ", tail up to %d tiles in 128-row tiles", tail);
    fprintf(stderr, "[dg] %s m=%d n=%d k=%d groups=%d%s -> tile %s (%dx%d), splits=%d%s\n", what,
            m, n, k, g, hint, dg::kTiles[cfg].name, dg::kTiles[cfg].bm, dg::kTiles[cfg].bn,
            splits, tl);
}

// Estimated cost of a tile choice: waves of workgroups over the CUs times the work of one
// tile, with a small per-tile overhead term that favours larger tiles on ties.
double tile_cost(int bm, int bn, int64_t tiles, int cus)
{
    int64_t waves = (tiles + cus - 1) / cus;
    return (double)waves * ((double)bm * bn + 64.0 * (bm + bn));
}

int launch(int mode, int cfg, dg::GemmArgs &args, hipStream_t stream)
{
    int64_t grid = dg::grid_size(mode, cfg, args);
    if (grid <= 0 || grid > 0x7fffffff)
        return fail(DG_ERR_UNSUPPORTED, "problem too large for one launch (%lld workgroups)",
                    (long long)grid);
    hipError_t e = dg::launch_gemm(mode, cfg, args, stream);
    if (e != hipSuccess)
        return fail(DG_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}



int gemm_nt(int sf_fmt, const void *a, const float *sfa, int64_t ld_sfa, const void *b,
            const float *sfb, const float *c, void *d, int m, int n, int k, void *stream,
            bool noalloc = false);

// The tail of the contiguous forms' 256 x 256 tiles (args.straddle_rows already set).  These
// tiles run one workgroup each, and the last ones dispatched can form a last partial wave that
// leaves most CUs idle.  Where that wave could hold between an eighth and a quarter of the CUs'
// worth of busy workgroups (for some count of served straddles; the kernel counts the actual
// ones from the group indices), the launch gets workgroups of 128-row tiles after the others,
// which run the tiles of those last workgroups over two or four times as many CUs.
// DG_TAIL_TILES=n (tests) leaves n tiles to them whatever the wave, 0 never.  Sets the tail
// fields of args; returns the most tiles the tail may take (0: no tail).
int plan_contig_tail(dg::GemmArgs &args, int m_total, int n, int cus)
{
    const char *e = getenv("DG_TAIL_TILES");
    const int force = (e && *e) ? atoi(e) : -1;
    const int tm = (m_total + 255) / 256, tn = (n + 255) / 256;
    const int64_t tiles = (int64_t)tm * tn;
    int tail_max = 0;
    if (force > 0) {
        tail_max = (int)(force < tiles - 1 ? force : tiles - 1);
    } else if (force < 0) {
        for (int s = 0; s <= args.straddle_rows && tail_max == 0; ++s)
            if (dg::tail_count(tiles + (int64_t)s * tn, tiles, cus) > 0)
                tail_max = cus / 4;
    }
    if (tail_max > 0) {
        args.tail_cus = cus;
        args.tail_force = force > 0 ? force : 0;
        args.tail_tm = tm;
        args.tail_tn = tn;
        args.tail_max = tail_max;
    }
    return tail_max;
}

int launch_with_tail(int mode, const dg::GemmArgs &args, hipStream_t stream)
{
    const int64_t grid = dg::contig_tail_grid(mode, args);
    if (grid <= 0 || grid > 0x7fffffff)
        return fail(DG_ERR_UNSUPPORTED, "problem too large for one launch (%lld workgroups)",
                    (long long)grid);
    const hipError_t e = dg::launch_contig_tail(mode, args, stream);
    if (e != hipSuccess)
        return fail(DG_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

bool layout_native_forced()
{
    const char *s = getenv("DG_LAYOUT_NATIVE");
    return s && *s && *s != '0';
}

// The dense NN, TN and TT layouts (operands stored MN-major on one or both sides).  By default
// each MN-major operand is transposed into a workspace (a byte transpose moves it once through
// HBM) and the NT path runs; under graph capture before the workspace exists, or with
// DG_LAYOUT_NATIVE=1, the layout kernel reads the MN-major operands directly.
int gemm_layout(int layout, const void *a, const float *sfa, int64_t ld_sfa, const void *b,
                const float *sfb, const float *c, void *d, int m, int n, int k, void *stream)
{
    int rc = check_common(a, sfa, ld_sfa, b, sfb, d, m, n, k);
    if (rc != DG_OK)
        return rc;
    if (m == 0)
        return ok();  // empty problem: nothing to write
    const bool a_mn = layout == dg::LAYOUT_TN || layout == dg::LAYOUT_TT;
    if (a_mn && m % 16 != 0)
        return fail(DG_ERR_UNSUPPORTED, "m=%d must be a multiple of 16 when A is stored [K, M]",
                    m);
    if ((int64_t)k * (m > n ? m : n) > 0x7fffffffLL)
        return fail(DG_ERR_UNSUPPORTED, "k * max(m, n) exceeds 2^31 bytes");
    if (!aligned(sfa, 16))
        return fail(DG_ERR_MISALIGNED, "sfa must be 16-byte aligned");
    if (c && !aligned(c, 16))
        return fail(DG_ERR_MISALIGNED, "C must be 16-byte aligned");
    if (c && (const void *)c == d)
        return fail(DG_ERR_INVALID_ARG, "C and D must not alias");
    const bool b_mn = layout == dg::LAYOUT_NN || layout == dg::LAYOUT_TN;
    hipStream_t s = (hipStream_t)stream;
    if (!layout_native_forced()) {
        const size_t a_bytes = a_mn ? ((size_t)m * k + 255) / 256 * 256 : 0;
        const size_t b_bytes = b_mn ? (size_t)n * k : 0;
        void *ws = nullptr;
        if ((rc = stream_workspace(WS_LAYOUT, s, a_bytes + b_bytes, &ws)) != DG_OK)
            return rc;
        if (ws) {
            // A stored [k][m] -> [m][k] and B stored [k][n] -> [n][k], in one launch
            const void *a_nt = a_mn ? ws : a;
            const void *b_nt = b_mn ? (const void *)((const uint8_t *)ws + a_bytes) : b;
            const hipError_t e = dg::launch_transpose_u8(
                a_mn ? a : nullptr, ws, k, m, b_mn ? b : nullptr, (uint8_t *)ws + a_bytes, k, n,
                s);
            if (e != hipSuccess)
                return fail(DG_ERR_HIP, "transpose launch failed: %s", hipGetErrorString(e));
            return gemm_nt(dg::SF_FP32, a_nt, sfa, ld_sfa, b_nt, sfb, c, d, m, n, k, stream);
        }
    }
    dg::LayoutArgs args;
    memset(&args, 0, sizeof(args));
    args.a = (const uint8_t *)a;
    args.sfa = sfa;
    args.ld_sfa = ld_sfa;
    args.b = (const uint8_t *)b;
    args.sfb = sfb;
    args.c = c;
    args.d = d;
    args.m = m;
    args.n = n;
    args.k = k;
    args.num_groups = 1;
    hipError_t e = dg::launch_layout(layout, args, s);
    if (e != hipSuccess)
        return fail(DG_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// The three forms, for either scale format (UE8M0: the scale pointers hold int32 words).
// noalloc: the split-K partials go to the static scratch array (dg_stream.hip) instead of a
// per-stream workspace, and nothing is allocated.
int gemm_nt(int sf_fmt, const void *a, const float *sfa, int64_t ld_sfa, const void *b,
            const float *sfb, const float *c, void *d, int m, int n, int k, void *stream,
            bool noalloc)
{
    int rc = check_common(a, sfa, ld_sfa, b, sfb, d, m, n, k);
    if (rc != DG_OK)
        return rc;
    if (m == 0)
        return ok();  // empty problem: nothing to write
    if (c && !aligned(c, 16))
        return fail(DG_ERR_MISALIGNED, "C must be 16-byte aligned");
    if (c && (const void *)c == d)
        return fail(DG_ERR_INVALID_ARG, "C and D must not alias");
    int cus = 0;
    if ((rc = device_cus(&cus)) != DG_OK)
        return rc;
    hipStream_t s = (hipStream_t)stream;

    const int kb = k / 128;
    dg::GemmArgs args{};
    args.a = (const uint8_t *)a;
    args.sfa = sfa;
    args.ld_sfa = ld_sfa;
    args.b = (const uint8_t *)b;
    args.sfb = sfb;
    args.c = c;
    args.d = (uint16_t *)d;
    args.m = m;
    args.n = n;
    args.k = k;
    args.num_groups = 1;
    args.splits = 1;
    args.max_wgs = persistent_wgs(cus);
    args.sf_fmt = sf_fmt;

    // Pipelined tiles for shapes that fill the CUs; the split-K streaming kernel for skinny M
    // and for shapes whose big tiles would leave most CUs idle.
    int cfg = forced_config();
    if (cfg < 0) {
        const int cands[] = {dg::CFG_256x224, dg::CFG_128x256w8, dg::CFG_128x128};
        const int ncands = 3;
        double best = 0;
        int64_t best_tiles = 0;
        for (int ci = 0; ci < ncands; ++ci) {
            const int cnd = cands[ci];
            const dg::TileInfo &t = dg::kTiles[cnd];
            int64_t tiles = (int64_t)((m + t.bm - 1) / t.bm) * ((n + t.bn - 1) / t.bn);
            double cost = tile_cost(t.bm, t.bn, tiles, cus);
            if (cfg < 0 || cost < best) {
                best = cost;
                cfg = cnd;
                best_tiles = tiles;
            }
        }
        if (m <= 64 || 2 * best_tiles < cus)
            cfg = dg::CFG_STREAM64;
    }
    if (cfg == dg::CFG_STREAM64) {
        // one workgroup per (64x64 tile, split): enough splits to cover the CUs, never more
        // than stream_max_kblocks() K blocks in one split, every split non-empty.  When all of
        // K fits one split, one: a workgroup requests its whole share at once, so its time is
        // set by the load latency more than by its block count, and one split needs no second
        // launch (128 x 256 x 512: 5.5 against 6.6 us with four splits and the reduction)
        const int64_t tiles = (int64_t)((m + 63) / 64) * ((n + 63) / 64);
        const int maxkb = dg::stream_max_kblocks();
        const int min_splits = (kb + maxkb - 1) / maxkb;
        int want = (int)(kb <= maxkb || tiles >= cus ? 1 : cus / tiles);
        const int fs = forced_splits();
        if (fs > 0)
            want = fs;
        want = want < min_splits ? min_splits : (want > kb ? kb : want);
        const int kbs = (kb + want - 1) / want;
        args.splits = (kb + kbs - 1) / kbs;
        if (args.splits > 1) {
            void *w = nullptr;
            const size_t need = (size_t)dg::stream_workspace_bytes(tiles, args.splits);
            if (noalloc) {
                float *sp = nullptr;
                size_t floats = 0;
                const hipError_t e = dg::static_scratch(&sp, &floats);
                if (e != hipSuccess)
                    return fail(DG_ERR_HIP, "static scratch lookup failed: %s",
                                hipGetErrorString(e));
                if (need > floats * sizeof(float))
                    return fail(DG_ERR_UNSUPPORTED,
                                "split-K partials need %zu bytes, more than the %zu-byte static "
                                "scratch of the no-allocation call",
                                need, floats * sizeof(float));
                w = sp;
            } else if ((rc = stream_workspace(WS_SPLITK, s, need, &w)) != DG_OK) {
                return rc;
            }
            if (w) {
                args.ws = (float *)w;
            } else {
                // no workspace for this stream (a call made under graph capture before any
                // outside it): the pipelined kernel without split-K is slower here but needs none
                cfg = dg::CFG_64x32;
                args.splits = 1;
            }
        }
    }
    print_config("fp8_gemm_nt", m, n, k, 1, cfg, args.splits);
    return launch(dg::MODE_DENSE, cfg, args, s);
}

int grouped_contiguous(int sf_fmt, const void *a, const float *sfa, int64_t ld_sfa,
                       const void *b, const float *sfb, void *d, const int32_t *m_indices,
                       int m_total, int n, int k, int num_groups, void *stream)
{
    int rc = check_common(a, sfa, ld_sfa, b, sfb, d, m_total, n, k);
    if (rc != DG_OK)
        return rc;
    if (!m_indices)
        return fail(DG_ERR_INVALID_ARG, "null m_indices");
    if (num_groups <= 0)
        return fail(DG_ERR_INVALID_ARG, "num_groups=%d must be positive", num_groups);
    if (m_total % 128 != 0)
        return fail(DG_ERR_UNSUPPORTED, "m_total=%d is not a multiple of 128", m_total);
    if (!aligned(m_indices, 4))
        return fail(DG_ERR_MISALIGNED, "m_indices must be 4-byte aligned");
    if (m_total == 0)
        return ok();
    int cus = 0;
    if ((rc = device_cus(&cus)) != DG_OK)
        return rc;
    // A tile takes one group's B.  Tiles of up to 128 rows hold one group (the alignment);
    // a 256-row tile, one workgroup per tile, runs twice where it holds two groups, about
    // half of the (num_groups - 1) group boundaries for padded expert blocks.
    int cfg = forced_config();
    if (cfg >= 0 && (cfg == dg::CFG_STREAM64 ||
                     (128 % dg::kTiles[cfg].bm != 0 &&
                      (dg::kTiles[cfg].bm != 256 || dg::kTiles[cfg].persistent))))
        cfg = -1;
    if (cfg < 0) {
        // 256 x 256 (scales in registers) when N % 256 == 0: its cost is weighted by its
        // measured per-tile efficiency against 256 x 224 (0.92 with FP32 scales: one scale
        // product per row and block, fewer copy bytes per MFMA; better still with UE8M0)
        const int cands[] = {dg::CFG_256x256, dg::CFG_256x224, dg::CFG_128x256w8, dg::CFG_128x128};
        double best = 0;
        for (int cnd : cands) {
            const dg::TileInfo &t = dg::kTiles[cnd];
            if ((cnd == dg::CFG_128x256w8 || cnd == dg::CFG_256x256) && n % 256 != 0)
                continue;
            int64_t rows = (m_total + t.bm - 1) / t.bm;
            if (t.bm > 128)
                rows += (num_groups - 1) / 2;
            const double cost = tile_cost(t.bm, t.bn, rows * ((n + t.bn - 1) / t.bn), cus) *
                                (cnd == dg::CFG_256x256 ? 0.92 : 1.0);
            if (cfg < 0 || cost < best) {
                best = cost;
                cfg = cnd;
            }
        }
    }
    dg::GemmArgs args{};
    args.a = (const uint8_t *)a;
    args.sfa = sfa;
    args.ld_sfa = ld_sfa;
    args.b = (const uint8_t *)b;
    args.sfb = sfb;
    args.d = (uint16_t *)d;
    args.grp = m_indices;
    args.m = m_total;
    args.n = n;
    args.k = k;
    args.num_groups = num_groups;
    args.splits = 1;
    args.max_wgs = persistent_wgs(cus);
    args.sf_fmt = sf_fmt;
    if (dg::kTiles[cfg].bm > 128) {
        // second groups of straddling 256-row tiles on workgroups of their own: as many
        // tile-rows as group boundaries (groups laid out in order), for up to 256 tile-rows
        const int tiles_m = (m_total + 255) / 256;
        args.straddle_rows = tiles_m <= 256 ? (num_groups - 1 < tiles_m ? num_groups - 1 : tiles_m) : 0;
        const char *e = getenv("DG_STRADDLE_ROWS");  // tests: fewer served slots
        if (e && *e && atoi(e) >= 0 && atoi(e) < args.straddle_rows)
            args.straddle_rows = atoi(e);
    }
    const int tail_max = cfg == dg::CFG_256x256 ? plan_contig_tail(args, m_total, n, cus) : 0;
    print_config("m_grouped_contiguous", m_total, n, k, num_groups, cfg, 1, -1, tail_max);
    if (tail_max == 0)
        return launch(dg::MODE_CONTIG, cfg, args, (hipStream_t)stream);
    return launch_with_tail(dg::MODE_CONTIG, args, (hipStream_t)stream);
}

// The contiguous form with the activation step fused into the epilogue: B is [G, 2I, K] with
// the gate rows first; the tile writes the 1x128 FP8 cast of SwiGLU(gate, up) instead of D.
int grouped_contiguous_swiglu(const void *a, const float *sfa, int64_t ld_sfa, const void *b,
                              const float *sfb, void *q, float *sfq, int64_t ld_sfq,
                              const int32_t *m_indices, int m_total, int n, int k,
                              int num_groups, void *stream)
{
    int rc = check_common(a, sfa, ld_sfa, b, sfb, q, m_total, n, k);
    if (rc != DG_OK)
        return rc;
    if (!m_indices)
        return fail(DG_ERR_INVALID_ARG, "null m_indices");
    if (num_groups <= 0)
        return fail(DG_ERR_INVALID_ARG, "num_groups=%d must be positive", num_groups);
    if (m_total % 128 != 0)
        return fail(DG_ERR_UNSUPPORTED, "m_total=%d is not a multiple of 128", m_total);
    if (n % 256 != 0)
        return fail(DG_ERR_UNSUPPORTED, "n=%d: the gate and up halves must be multiples of 128",
                    n);
    if (!aligned(m_indices, 4))
        return fail(DG_ERR_MISALIGNED, "m_indices must be 4-byte aligned");
    if (m_total > 0 && !sfq)
        return fail(DG_ERR_INVALID_ARG, "null sfq");
    if (ld_sfq < m_total)
        return fail(DG_ERR_INVALID_ARG, "ld_sfq=%lld is smaller than m_total=%d",
                    (long long)ld_sfq, m_total);
    if (ld_sfq % 4 != 0 || !aligned(sfq, 16))
        return fail(DG_ERR_MISALIGNED, "sfq must be 16-byte aligned with ld_sfq %% 4 == 0");
    if (m_total == 0)
        return ok();
    int cus = 0;
    if ((rc = device_cus(&cus)) != DG_OK)
        return rc;
    dg::GemmArgs args{};
    args.a = (const uint8_t *)a;
    args.sfa = sfa;
    args.ld_sfa = ld_sfa;
    args.b = (const uint8_t *)b;
    args.sfb = sfb;
    args.grp = m_indices;
    args.m = m_total;
    args.n = n;
    args.k = k;
    args.num_groups = num_groups;
    args.splits = 1;
    args.max_wgs = persistent_wgs(cus);
    args.sf_fmt = dg::SF_FP32;
    args.q = (uint8_t *)q;
    args.sfq = sfq;
    args.ld_sfq = ld_sfq;
    // one tile per 128-column segment of h, (128 gate + 128 up columns): 256 rows (straddling
    // tiles run once per group, as in the contiguous form; weighted by the same measured
    // per-tile efficiency) or 128 rows, persistent
    int cfg = forced_config();
    if (cfg != dg::CFG_128x256w8 && cfg != dg::CFG_256x256) {
        const int64_t rows256 = (m_total + 255) / 256 + (num_groups - 1) / 2;
        const int64_t rows128 = (m_total + 127) / 128;
        const double c256 = tile_cost(256, 256, rows256 * (n / 256), cus) * 0.92;
        const double c128 = tile_cost(128, 256, rows128 * (n / 256), cus);
        cfg = c256 < c128 ? dg::CFG_256x256 : dg::CFG_128x256w8;
    }
    if (cfg == dg::CFG_256x256) {
        const int tiles_m = (m_total + 255) / 256;
        args.straddle_rows = tiles_m <= 256 ? (num_groups - 1 < tiles_m ? num_groups - 1 : tiles_m) : 0;
        const char *e = getenv("DG_STRADDLE_ROWS");  // tests: fewer served slots
        if (e && *e && atoi(e) >= 0 && atoi(e) < args.straddle_rows)
            args.straddle_rows = atoi(e);
    }
    const int tail_max = cfg == dg::CFG_256x256 ? plan_contig_tail(args, m_total, n, cus) : 0;
    print_config("m_grouped_contiguous_swiglu", m_total, n, k, num_groups, cfg, 1, -1, tail_max);
    if (tail_max == 0)
        return launch(dg::MODE_CONTIG_SWIGLU, cfg, args, (hipStream_t)stream);
    return launch_with_tail(dg::MODE_CONTIG_SWIGLU, args, (hipStream_t)stream);
}

int grouped_masked(int sf_fmt, const void *a, const float *sfa, int64_t ld_sfa, const void *b,
                   const float *sfb, void *d, const int32_t *masked_m, int num_groups, int m_max,
                   int n, int k, int expected_m, void *stream)
{
    int rc = check_common(a, sfa, ld_sfa, b, sfb, d, m_max, n, k);
    if (rc != DG_OK)
        return rc;
    if (!masked_m)
        return fail(DG_ERR_INVALID_ARG, "null masked_m");
    if (num_groups <= 0)
        return fail(DG_ERR_INVALID_ARG, "num_groups=%d must be positive", num_groups);
    if (!aligned(masked_m, 4))
        return fail(DG_ERR_MISALIGNED, "masked_m must be 4-byte aligned");
    if (m_max == 0)
        return ok();
    int cus = 0;
    if ((rc = device_cus(&cus)) != DG_OK)
        return rc;
    // The valid rows per group are known only on the device; the caller's expected count (<= 0:
    // half of m_max) is the pages' hint for the tile choice.  Measured on the MI355X (16 groups,
    // N = 7168, K = 2048, masked_m uniform in [0, 2e]), 256-row tiles are the fastest at every
    // expected count from e = 8 to 128, ahead of 128-row tiles by 25-50%: a group's rows past
    // masked_m skip their MFMAs and read zeros, so the taller tile costs little, and it reads
    // each B column block once where two 128-row tiles may read it twice.  So the choice depends
    // on m_max (one 256-row tile per N tile when the groups can exceed 128 rows) and not on the
    // hint, which is printed with the choice.  Of the 256-row widths, the one with less column
    // padding, the wider on a tie (each N tile re-reads the group's A from L2, so fewer, wider
    // tiles read less); 256 columns with FP32 scales only (measured 67.0 against 68.0 us for
    // 224 on the shape above).
    const int e = expected_m > 0 ? (expected_m < m_max ? expected_m : m_max) : (m_max + 1) / 2;
    int cfg = forced_config();
    if (cfg < 0 || cfg == dg::CFG_STREAM64) {
        if (m_max > 128) {
            const int64_t pad224 = (int64_t)((n + 223) / 224) * 224 - n;
            const int64_t pad128 = (int64_t)((n + 127) / 128) * 128 - n;
            cfg = pad224 <= pad128 ? dg::CFG_256x224 : dg::CFG_256x128;
            if (sf_fmt == dg::SF_FP32 && n % 256 == 0)
                cfg = dg::CFG_256x256;  // no padding: as little as either, and the widest
        } else {
            cfg = dg::CFG_128x128;
        }
    }
    dg::GemmArgs args{};
    args.a = (const uint8_t *)a;
    args.sfa = sfa;
    args.ld_sfa = ld_sfa;
    args.b = (const uint8_t *)b;
    args.sfb = sfb;
    args.d = (uint16_t *)d;
    args.grp = masked_m;
    args.m = m_max;
    args.n = n;
    args.k = k;
    args.num_groups = num_groups;
    args.splits = 1;
    args.max_wgs = persistent_wgs(cus);
    args.sf_fmt = sf_fmt;
    print_config("m_grouped_masked", m_max, n, k, num_groups, cfg, 1, e);
    return launch(dg::MODE_MASKED, cfg, args, (hipStream_t)stream);
}

}  // namespace

extern "C" {

int dg_fp8_gemm_nt(const void *a, const float *sfa, int64_t ld_sfa, const void *b,
                   const float *sfb, const float *c, void *d, int m, int n, int k, void *stream)
{
    return gemm_nt(dg::SF_FP32, a, sfa, ld_sfa, b, sfb, c, d, m, n, k, stream);
}

int dg_fp8_gemm_nt_noalloc(const void *a, const float *sfa, int64_t ld_sfa, const void *b,
                           const float *sfb, const float *c, void *d, int m, int n, int k,
                           void *stream)
{
    return gemm_nt(dg::SF_FP32, a, sfa, ld_sfa, b, sfb, c, d, m, n, k, stream, true);
}

int dg_m_grouped_fp8_gemm_nt_contiguous(const void *a, const float *sfa, int64_t ld_sfa,
                                        const void *b, const float *sfb, void *d,
                                        const int32_t *m_indices, int m_total, int n, int k,
                                        int num_groups, void *stream)
{
    return grouped_contiguous(dg::SF_FP32, a, sfa, ld_sfa, b, sfb, d, m_indices, m_total, n, k,
                              num_groups, stream);
}

int dg_m_grouped_fp8_gemm_nt_contiguous_swiglu(const void *a, const float *sfa,
                                               int64_t ld_sfa, const void *b, const float *sfb,
                                               void *q, float *sfq, int64_t ld_sfq,
                                               const int32_t *m_indices, int m_total, int n,
                                               int k, int num_groups, void *stream)
{
    return grouped_contiguous_swiglu(a, sfa, ld_sfa, b, sfb, q, sfq, ld_sfq, m_indices, m_total,
                                     n, k, num_groups, stream);
}

int dg_m_grouped_fp8_gemm_nt_masked(const void *a, const float *sfa, int64_t ld_sfa,
                                    const void *b, const float *sfb, void *d,
                                    const int32_t *masked_m, int num_groups, int m_max, int n,
                                    int k, int expected_m, void *stream)
{
    return grouped_masked(dg::SF_FP32, a, sfa, ld_sfa, b, sfb, d, masked_m, num_groups, m_max, n,
                          k, expected_m, stream);
}

int dg_fp8_gemm_nn(const void *a, const float *sfa, int64_t ld_sfa, const void *b,
                   const float *sfb, const float *c, void *d, int m, int n, int k, void *stream)
{
    return gemm_layout(dg::LAYOUT_NN, a, sfa, ld_sfa, b, sfb, c, d, m, n, k, stream);
}

int dg_fp8_gemm_tn(const void *a, const float *sfa, int64_t ld_sfa, const void *b,
                   const float *sfb, const float *c, void *d, int m, int n, int k, void *stream)
{
    return gemm_layout(dg::LAYOUT_TN, a, sfa, ld_sfa, b, sfb, c, d, m, n, k, stream);
}

int dg_fp8_gemm_tt(const void *a, const float *sfa, int64_t ld_sfa, const void *b,
                   const float *sfb, const float *c, void *d, int m, int n, int k, void *stream)
{
    return gemm_layout(dg::LAYOUT_TT, a, sfa, ld_sfa, b, sfb, c, d, m, n, k, stream);
}

// UE8M0 scales: int32 words of four biased exponents, 4-byte elements like the FP32 scales
int dg_fp8_gemm_nt_ue8m0(const void *a, const int32_t *sfa, int64_t ld_sfa, const void *b,
                         const int32_t *sfb, const float *c, void *d, int m, int n, int k,
                         void *stream)
{
    return gemm_nt(dg::SF_UE8M0, a, reinterpret_cast<const float *>(sfa), ld_sfa, b,
                   reinterpret_cast<const float *>(sfb), c, d, m, n, k, stream);
}

int dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const void *a, const int32_t *sfa, int64_t ld_sfa,
                                              const void *b, const int32_t *sfb, void *d,
                                              const int32_t *m_indices, int m_total, int n,
                                              int k, int num_groups, void *stream)
{
    return grouped_contiguous(dg::SF_UE8M0, a, reinterpret_cast<const float *>(sfa), ld_sfa, b,
                              reinterpret_cast<const float *>(sfb), d, m_indices, m_total, n, k,
                              num_groups, stream);
}

int dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const void *a, const int32_t *sfa, int64_t ld_sfa,
                                          const void *b, const int32_t *sfb, void *d,
                                          const int32_t *masked_m, int num_groups, int m_max,
                                          int n, int k, int expected_m, void *stream)
{
    return grouped_masked(dg::SF_UE8M0, a, reinterpret_cast<const float *>(sfa), ld_sfa, b,
                          reinterpret_cast<const float *>(sfb), d, masked_m, num_groups, m_max,
                          n, k, expected_m, stream);
}

int dg_k_grouped_fp8_gemm_tn_contiguous(const void *a, const float *sfa, const void *b,
                                        const float *sfb, const float *c, float *d,
                                        const int32_t *ks, int num_groups, int m, int n,
                                        int k_total, void *stream)
{
    if (!ks)
        return fail(DG_ERR_INVALID_ARG, "null group extents");
    if (num_groups < 1 || num_groups > dg::KG_MAX_GROUPS)
        return fail(DG_ERR_UNSUPPORTED, "num_groups=%d outside [1, %d]", num_groups,
                    dg::KG_MAX_GROUPS);
    if (m <= 0 || n <= 0 || k_total < 0)
        return fail(DG_ERR_INVALID_ARG, "sizes must be positive (m=%d n=%d k_total=%d)", m, n,
                    k_total);
    if (m % 16 != 0 || n % 16 != 0)
        return fail(DG_ERR_UNSUPPORTED, "m=%d and n=%d must be multiples of 16", m, n);
    if (k_total % 128 != 0)
        return fail(DG_ERR_UNSUPPORTED, "k_total=%d is not a multiple of 128", k_total);
    if (!d || (k_total > 0 && (!a || !sfa || !b || !sfb)))
        return fail(DG_ERR_INVALID_ARG, "null tensor pointer");
    // byte offsets inside one operand are 32-bit
    if ((int64_t)k_total * (m > n ? m : n) > 0x7fffffffLL)
        return fail(DG_ERR_UNSUPPORTED, "k_total * max(m, n) exceeds 2^31 bytes");
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 16) || !aligned(c, 16))
        return fail(DG_ERR_MISALIGNED, "A, B, C and D must be 16-byte aligned");
    if (!aligned(sfa, 16) || !aligned(sfb, 16))
        return fail(DG_ERR_MISALIGNED, "scale pointers must be 16-byte aligned");
    // C may be D itself (accumulate in place), but must not overlap it otherwise
    const int64_t d_bytes = (int64_t)num_groups * m * n * 4;
    if (c && c != d) {
        const char *cb = (const char *)c, *db = (const char *)d;
        if (cb < db + d_bytes && db < cb + d_bytes)
            return fail(DG_ERR_INVALID_ARG, "C overlaps D without being D");
    }
    dg::LayoutArgs args;
    memset(&args, 0, sizeof(args));
    args.a = (const uint8_t *)a;
    args.sfa = sfa;
    args.ld_sfa = m;
    args.b = (const uint8_t *)b;
    args.sfb = sfb;
    args.c = c;
    args.d = d;
    args.m = m;
    args.n = n;
    args.k = k_total;
    args.num_groups = num_groups;
    int64_t kb = 0;
    for (int g = 0; g < num_groups; ++g) {
        if (ks[g] < 0 || ks[g] % 128 != 0)
            return fail(DG_ERR_UNSUPPORTED, "ks[%d]=%d is not a non-negative multiple of 128", g,
                        ks[g]);
        args.kb_start[g] = (int)kb;
        kb += ks[g] / 128;
    }
    if (kb * 128 != k_total)
        return fail(DG_ERR_INVALID_ARG, "the group extents sum to %lld, not k_total=%d",
                    (long long)(kb * 128), k_total);
    args.kb_start[num_groups] = (int)kb;
    hipError_t e = dg::launch_layout(dg::LAYOUT_KGROUPED_TN, args, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(DG_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int dg_swiglu_fp8_quant(const void *x, void *q, float *sfa, int64_t ld_sfa, int m, int i,
                        void *stream)
{
    if (m < 0 || i <= 0)
        return fail(DG_ERR_INVALID_ARG, "sizes must be positive (m=%d i=%d)", m, i);
    if (i % 128 != 0)
        return fail(DG_ERR_UNSUPPORTED, "i=%d is not a multiple of 128", i);
    if (m == 0)
        return ok();
    if (!x || !q || !sfa)
        return fail(DG_ERR_INVALID_ARG, "null tensor pointer");
    if (ld_sfa < m)
        return fail(DG_ERR_INVALID_ARG, "ld_sfa=%lld is smaller than m=%d", (long long)ld_sfa, m);
    if (!aligned(x, 16) || !aligned(q, 8) || !aligned(sfa, 4))
        return fail(DG_ERR_MISALIGNED, "X must be 16-byte, q 8-byte and sfa 4-byte aligned");
    hipError_t e = dg::launch_swiglu_quant(x, q, sfa, ld_sfa, m, i, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(DG_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int dg_get_mk_alignment_for_contiguous_layout(void) { return 128; }

int64_t dg_get_sf_aligned_m(int64_t m) { return m <= 0 ? 0 : (m + 3) / 4 * 4; }

int dg_set_num_cus(int n)
{
    int prev = g_num_cus_cap;
    g_num_cus_cap = n > 0 ? n : 0;
    return prev;
}

int dg_get_num_cus(void)
{
    int cus = 0;
    int rc = device_cus(&cus);
    return rc == DG_OK ? cus : rc;
}

const char *dg_last_error(void) { return g_err; }

}  // extern "C"
