// api.cpp -- C ABI of libw4a16: host-side validation, planning, scratch
// management and dispatch.  Every argument is checked before the first HIP
// call, so invalid calls return a status without touching the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "w4a16.h"
#include "kernels.h"

namespace w4a16 {
int gemv_words_for_m(int64_t M);
}

namespace {

using namespace w4a16;

thread_local std::string g_last_error;

int fail(int status, const std::string &msg) {
    g_last_error = msg;
    return status;
}

int ok() {
    g_last_error.clear();
    return W4A16_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void *p, size_t pn, const void *q, size_t qn) {
    if (!p || !q || pn == 0 || qn == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + pn;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(q), b1 = b0 + qn;
    return a0 < b1 && b0 < a1;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- tuning ---
// Plan knobs, overridable for tuning sweeps: "key=value,..." from the
// environment variable W4A16_TUNE at first use, or from w4a16_set_tuning().
struct Tune {
    int64_t gemv_target_waves = 1600;  // M <= 2: aim for about this many GEMV waves (see plan_gemm)
    int64_t gemv_waves = 8;            // waves per GEMV workgroup (4 or 8)
    int64_t gemv_splits = 0;           // force the GEMV K-split count
    int64_t gemv_fold = -1;            // bias/zero removed per chunk: 1 always, 0 never, -1 symmetric M <= 2
    int64_t gemv_max_m = 8;            // largest M sent to the GEMV path (at most 8)
    int64_t gemv_mma = 1;              // GEMV k-reduction on the matrix cores (0: the dot2 GEMV)
    int64_t gemv_mma_words = 0;        // matrix-core GEMV words per lane: 2 (256-column tiles), 4 (512, M <= 2), 0 by fill
    int64_t mfma_target_waves = 2048;  // aim for about this many MFMA-path waves
    int64_t mfma_splits = 0;           // force the MFMA split count
    int64_t mfma_cfg = 0;  // force (mt, waves, kwaves): 1..6 = (1,2,4) (2,2,4) (4,2,2) (2,1,8) (4,2,4) (4,1,8)
    int64_t mfma_mgroup = 0;           // force the MFMA row-tile group (0: by estimated L2 traffic)
    int64_t max_partial_bytes = 64ll << 20;
    int64_t decode_fuse = 1;           // 0: decode-step glue as separate kernels
    int64_t decode_swiglu_m = 3;       // GEMV route: from this M on, SwiGLU + row-norm as a kernel of its own
};

// Returns false on an unknown key or a malformed entry (nothing applied).
bool parse_tune(const char *spec, Tune *out) {
    Tune v;
    std::string s(spec ? spec : "");
    size_t pos = 0;
    while (pos < s.size()) {
        size_t end = s.find(',', pos);
        if (end == std::string::npos) end = s.size();
        const std::string kv = s.substr(pos, end - pos);
        pos = end + 1;
        if (kv.empty()) continue;
        const size_t eq = kv.find('=');
        if (eq == std::string::npos) return false;
        const std::string k = kv.substr(0, eq);
        char *tail = nullptr;
        const long long val = std::strtoll(kv.c_str() + eq + 1, &tail, 10);
        if (tail == kv.c_str() + eq + 1 || *tail != '\0') return false;
        if (k == "gemv_target_waves") v.gemv_target_waves = val;
        else if (k == "gemv_waves") v.gemv_waves = val;
        else if (k == "gemv_splits") v.gemv_splits = val;
        else if (k == "gemv_fold") v.gemv_fold = val;
        else if (k == "gemv_max_m") v.gemv_max_m = val;
        else if (k == "gemv_mma") v.gemv_mma = val;
        else if (k == "gemv_mma_words") v.gemv_mma_words = val;

        else if (k == "mfma_target_waves") v.mfma_target_waves = val;
        else if (k == "mfma_splits") v.mfma_splits = val;
        else if (k == "mfma_cfg") v.mfma_cfg = val;
        else if (k == "mfma_mgroup") v.mfma_mgroup = val;
        else if (k == "max_partial_bytes") v.max_partial_bytes = val;
        else if (k == "decode_fuse") v.decode_fuse = val;
        else if (k == "decode_swiglu_m") v.decode_swiglu_m = val;
        else return false;
    }
    *out = v;
    return true;
}

// The active knobs: an immutable snapshot, replaced whole by w4a16_set_tuning
// (earlier snapshots are kept alive, so a plan being computed concurrently
// keeps a valid view).
std::atomic<const Tune *> g_tune{nullptr};

const Tune &tune() {
    const Tune *t = g_tune.load(std::memory_order_acquire);
    if (t) return *t;
    static const Tune *from_env = [] {
        Tune *v = new Tune();
        if (!parse_tune(std::getenv("W4A16_TUNE"), v)) *v = Tune();
        return v;
    }();
    const Tune *expect = nullptr;
    g_tune.compare_exchange_strong(expect, from_env, std::memory_order_acq_rel);
    return *g_tune.load(std::memory_order_acquire);
}

// ---------------------------------------------------------- validation ---
int validate_sizes(int64_t M, int64_t K, int64_t N, int64_t G) {
    if (M < 0) return fail(W4A16_ERR_INVALID_ARG, "M must be >= 0");
    if (K <= 0 || N <= 0 || G <= 0) return fail(W4A16_ERR_INVALID_ARG, "K, N and G must be > 0");
    if (N % 8 != 0) return fail(W4A16_ERR_INVALID_ARG, "N must be a multiple of 8");
    if (K % G != 0) return fail(W4A16_ERR_INVALID_ARG, "K must be a multiple of G");
    if (G % 32 != 0) return fail(W4A16_ERR_UNSUPPORTED, "G must be a multiple of 32");
    // Every tensor must fit a buffer resource (byte extent < 2^32).
    if (M > (1ll << 20) || K > (1ll << 26) || N > (1ll << 26) || M * N >= (1ll << 31) ||
        M * K >= (1ll << 31) || K * (N / 8) >= (1ll << 30))
        return fail(W4A16_ERR_UNSUPPORTED, "problem too large for 32-bit kernel indexing");
    return W4A16_OK;
}

}  // namespace

namespace w4a16 {

GemmPlan plan_gemm(int64_t M, int64_t K, int64_t N, int64_t G, bool allow_mma, bool allow_wide) {
    const Tune &t = tune();
    GemmPlan p;
    const int64_t N8 = N / 8;
    if (M <= std::min<int64_t>(8, t.gemv_max_m) && N % 32 == 0) {
        // 256-column tiles (one 128-byte line of every weight row per
        // workgroup); K-splits to fill one round of the 256 CUs (below).
        p.path = kPathGemv;
        p.words = gemv_words_for_m(M);
        // The folded form drops one packed subtract per weight pair; measured
        // on MI355X it pays where the dot products are few (M <= 2, where the
        // exact form also runs out of registers at M = 2).  By default only
        // with a symmetric zero point, where it keeps all-zp columns exactly 0.
        p.fold = t.gemv_fold < 0 ? M <= 2 : t.gemv_fold != 0;
        p.fold_asym = t.gemv_fold > 0;
        const int64_t CL = 32 / p.words, RL = 64 / CL;
        p.tiles_n = cdiv(N8, 32);
        const int64_t nchunks = K / 16;
        p.waves = t.gemv_waves == 4 ? 4 : 8;
        int64_t splits;
        if (t.gemv_splits > 0) {
            splits = t.gemv_splits;
        } else {
            // Measured on MI355X: as many splits as one round of workgroups
            // holds (one 8-wave workgroup per CU) is fastest, except at M <= 2,
            // where the stream is purely bandwidth-bound and fewer splits (less
            // fixed-point slot traffic, longer per-wave streams) win as long as
            // they still give 3/4 of the CUs a workgroup: about
            // gemv_target_waves waves, each workgroup's row lanes kept at
            // least half busy.  Splits keep at least 8 chunks each.
            const int64_t per_cu = 8 / p.waves;
            splits = std::max<int64_t>(1, 256 * per_cu / p.tiles_n);
            splits = std::min<int64_t>(splits, std::max<int64_t>(1, nchunks / 8));  // >= 128 rows per split
            if (M <= 2) {
                int64_t fewer = cdiv(t.gemv_target_waves, p.tiles_n * p.waves);
                fewer = std::min<int64_t>(fewer, std::max<int64_t>(1, nchunks / (p.waves * RL / 2)));
                if (fewer < splits && 4 * fewer * p.tiles_n >= 3 * 256 * per_cu) splits = fewer;
            }
        }
        splits = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(splits, 32), nchunks));
        p.split_len = cdiv(nchunks, splits);
        p.splits = (int)cdiv(nchunks, p.split_len);
        p.tiles_m = 1;
        // The matrix-core GEMV (gemv_mma_kernel) needs far fewer vector-ALU
        // instructions per weight than the dot2 form; its products are summed
        // less finely (about 1e-4 of the output: subnormal-encoded weights on
        // the matrix core) but far inside the tolerance.  Measured on MI355X,
        // with one round of workgroups (256 / tiles splits, waves of a split
        // taking unequal chunk counts where they do not divide): the headline
        // M = 1 K = 4096 N = 12800 8.57 -> 7.94 us, K = 12800 N = 4096
        // 9.50 -> 7.88 us, K = 8192 N = 8192 11.9 -> 9.0 us, and 40-53% less
        // time at M = 8.  Rounding the splits down to equal chunk counts per
        // wave (one round fewer workgroups) was slower at M <= 2 (headline
        // 8.56 us).
        if (allow_mma && p.waves == 8 && t.gemv_mma != 0) {
            // 512-column tiles (16-byte loads) measured slower wherever 256-column
            // tiles fill the chip (headline 8.22 -> 8.57 us, M = 8 by 40-60%), but
            // faster where those leave CUs idle: K = 4096 N = 25600 at M = 1 runs
            // 100 tiles x 2 splits = 200 workgroups against 50 x 5 = 250,
            // 13.72 -> 12.27 us.  So at M <= 2, when 256-column tiles fill under
            // 85% of the CUs and 512-column ones at least 10% more.
            auto fill = [](int64_t tiles) { return tiles * std::max<int64_t>(1, std::min<int64_t>(32, 256 / tiles)); };
            const int64_t t2 = cdiv(N8, 32), t4 = cdiv(N8, 64);
            const bool wide = t.gemv_mma_words == 4 ||
                              (t.gemv_mma_words == 0 && fill(t2) < 218 && fill(t4) >= fill(t2) + 26);
            p.words = 2;
            if (allow_wide && M <= 2 && wide) {
                p.words = 4;
                p.tiles_n = t4;
            }
            const int64_t mchunks = K / kMmaChunkRows;
            int64_t ms = t.gemv_splits > 0 ? t.gemv_splits : std::max<int64_t>(1, 256 / p.tiles_n);
            ms = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(ms, 32), mchunks));
            p.split_len = cdiv(mchunks, ms);
            p.splits = (int)cdiv(mchunks, p.split_len);
            p.mma = true;
            p.fold = p.fold_asym = false;
        }
    } else {
        // MFMA: wave tile (16*mt rows) x 128 columns; `waves` along N and
        // `kwaves` along K per workgroup (one workgroup per CU); K-splits
        // across workgroups until the grid has about mfma_target_waves waves
        // (the last workgroup of a tile sums the splits' fp32 partials).
        // Measured on MI355X: at M = 32 the 128-column, 8-K-wave shape beats
        // 256-column tiles on the 8B-class decode shapes (fewer splits, less
        // partial traffic).  Above M = 32, 64-row wave tiles (below).
        p.path = kPathMfma;
        auto fill = [&](int mt, int waves, int kwaves) {
            p.mt = mt;
            p.waves = waves;
            p.kwaves = kwaves;
            p.tiles_n = cdiv(N8, 16 * p.waves);
            p.tiles_m = cdiv(M, 16 * p.mt);
            const int64_t nsteps = K / 32;
            const int64_t wg_waves = (int64_t)p.waves * p.kwaves;
            const int64_t tiles = p.tiles_n * p.tiles_m;
            const int64_t target = t.mfma_target_waves > 0 ? t.mfma_target_waves : 2048;
            // Round down: these workgroups hold one per CU, and a grid past one
            // round of the chip would run its last workgroups as a second wave.
            int64_t splits = t.mfma_splits > 0 ? t.mfma_splits : target / (tiles * wg_waves);
            // at least two 32-row steps per K-wave, bounded partials
            splits = std::min<int64_t>(splits, std::max<int64_t>(1, nsteps / (2 * p.kwaves)));
            splits = std::min<int64_t>(splits, std::max<int64_t>(1, t.max_partial_bytes / std::max<int64_t>(1, M * N * 4)));
            splits = std::min<int64_t>(splits, mfma_max_splits(p.mt, p.waves, p.kwaves));
            splits = std::max<int64_t>(1, splits);
            p.split_len = cdiv(nsteps, splits);
            p.splits = (int)cdiv(nsteps, p.split_len);
        };
        static const int kCfg[6][3] = {{1, 2, 4}, {2, 2, 4}, {4, 2, 2}, {2, 1, 8}, {4, 2, 4}, {4, 1, 8}};
        if (t.mfma_cfg >= 1 && t.mfma_cfg <= 6) {
            fill(kCfg[t.mfma_cfg - 1][0], kCfg[t.mfma_cfg - 1][1], kCfg[t.mfma_cfg - 1][2]);
        } else if (M <= 16) {
            // One 16-row tile.  Measured on MI355X at M = 9..16: the 256-column
            // shape wins from N = 8192 on; below, the 128-column 8-K-wave shape
            // (twice the column tiles, fewer split partials): K = 12800
            // N = 4096 19.5 -> 15.4 us, K = 4096 N = 4096 10.9 -> 9.3 us,
            // N = 6144 within 0.1 us at M = 9 and 0.7 us better at M = 16.
            if (cdiv(N8, 32) <= 24) fill(2, 1, 8);
            else fill(1, 2, 4);
        } else if (M <= 32) {
            fill(2, 1, 8);
        } else {
            // 64-row wave tiles: 256 columns with 2 or 4 K-waves, or 128 columns
            // with 8 K-waves (twice the tiles, so half the K-splits, or a full
            // chip where 256-column tiles leave CUs idle).  Measured on MI355X:
            // prefer the shape that keeps the most CUs busy per round of
            // workgroups, then the fewest K-splits (split partials go through
            // memory), then the fewest workgroups.
            static const int kBig[3][3] = {{4, 2, 2}, {4, 2, 4}, {4, 1, 8}};
            int best = -1;
            double best_eff = -1;
            int best_splits = 0;
            int64_t best_grid = 0;
            for (int c = 0; c < 3; ++c) {
                fill(kBig[c][0], kBig[c][1], kBig[c][2]);
                const int64_t grid = p.tiles_n * p.tiles_m * p.splits;
                const int64_t rounds = cdiv(grid, 256);
                const double eff = (double)grid / (double)(rounds * 256);
                const bool better = best < 0 || eff > best_eff + 1e-9 ||
                                    (eff > best_eff - 1e-9 && (p.splits < best_splits ||
                                                               (p.splits == best_splits && grid < best_grid)));
                if (better) {
                    best = c;
                    best_eff = eff;
                    best_splits = p.splits;
                    best_grid = grid;
                }
            }
            fill(kBig[best][0], kBig[best][1], kBig[best][2]);
        }
        // Row-tile group: the 32 workgroups an XCD holds at once (one per CU)
        // are consecutive logical indices; walking g row tiles per column tile
        // makes them read about ceil(32/g) column tiles of weights and g row
        // tiles of activations through that XCD's L2.  Pick the g with the
        // fewest such bytes (the smallest g on ties).
        const int64_t krows = p.split_len * 32;
        const int64_t cols = 16 * 8 * (int64_t)p.waves;
        const double wcol = (double)krows * (double)cols * 0.5 + (double)(krows / G) * (double)cols * 2.5;
        const double arow = (double)(16 * p.mt) * (double)krows * 2.0;
        const int64_t resident = std::max<int64_t>(1, std::min<int64_t>(32, cdiv(p.tiles_n * p.tiles_m * p.splits, 8)));
        int64_t gbest = 1;
        double cbest = -1;
        for (int64_t g = 1; g <= std::min<int64_t>(p.tiles_m, resident); ++g) {
            const double cost = (double)std::min<int64_t>(cdiv(resident, g), p.tiles_n) * wcol +
                                (double)std::min<int64_t>(g, resident) * arow;
            if (cbest < 0 || cost < cbest - 1e-6 * cbest) {
                cbest = cost;
                gbest = g;
            }
        }
        if (t.mfma_mgroup > 0) gbest = std::min<int64_t>(t.mfma_mgroup, p.tiles_m);
        p.m_group = (int)gbest;
    }
    p.grid = p.tiles_n * p.tiles_m * p.splits;
    p.grid = cdiv(p.grid, 8) * 8;  // XCD-aware index mapping needs a multiple of 8
    if (p.path == kPathGemv) {
        // one 64-bit fixed-point slot per output (two counter words)
        p.partial_floats = 0;
        p.counters = p.splits > 1 ? (size_t)(2 * M * N) : 0;
    } else {
        p.partial_floats = p.splits > 1 ? (size_t)(p.splits * M * N) : 0;
        p.counters = p.splits > 1 ? (size_t)(p.tiles_n * p.tiles_m) : 0;
    }
    return p;
}

}  // namespace w4a16

namespace {

// ------------------------------------------------- library-owned scratch ---
// Split-K partials and arrival counters / fixed-point slots, one set per
// (device, stream).  The counter words are zeroed once at allocation; the
// last arrival at each counter or slot zeroes it again, so they are zero
// whenever the stream is idle.
struct Scratch {
    float *partials = nullptr;
    size_t partial_cap = 0;  // floats
    uint32_t *counters = nullptr;
    size_t counter_cap = 0;  // words
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Scratch> g_scratch;

int get_scratch(hipStream_t stream, const GemmPlan &plan, float **partials, uint32_t **counters) {
    *partials = nullptr;
    *counters = nullptr;
    if (plan.splits <= 1) return W4A16_OK;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_mu);
    Scratch &s = g_scratch[{dev, stream}];
    if (s.partial_cap < plan.partial_floats || s.counter_cap < plan.counters) {
        // Growing: the old buffers may still be read by queued kernels.
        if (s.partials || s.counters) {
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return fail(W4A16_ERR_HIP, std::string("hipStreamSynchronize: ") + hipGetErrorString(e));
            (void)hipFree(s.partials);
            (void)hipFree(s.counters);
            s = Scratch();
        }
        const size_t pcap = std::max<size_t>(plan.partial_floats, (size_t)1 << 20);
        const size_t ccap = std::max<size_t>(plan.counters, (size_t)1 << 14);
        e = hipMalloc((void **)&s.partials, pcap * sizeof(float));
        if (e != hipSuccess) { s = Scratch(); return fail(W4A16_ERR_WORKSPACE, "hipMalloc of split-K partials failed"); }
        e = hipMalloc((void **)&s.counters, ccap * sizeof(uint32_t));
        if (e != hipSuccess) {
            (void)hipFree(s.partials);
            s = Scratch();
            return fail(W4A16_ERR_WORKSPACE, "hipMalloc of split-K counters failed");
        }
        e = hipMemsetAsync(s.counters, 0, ccap * sizeof(uint32_t), stream);
        if (e != hipSuccess) return fail(W4A16_ERR_HIP, std::string("hipMemsetAsync: ") + hipGetErrorString(e));
        s.partial_cap = pcap;
        s.counter_cap = ccap;
    }
    *partials = s.partials;
    *counters = s.counters;
    return W4A16_OK;
}

int validate_gemm(const uint16_t *a, const int32_t *b, const uint16_t *s, const int32_t *qz,
                  int64_t M, int64_t K, int64_t N, int64_t G, int32_t zp, const uint16_t *out) {
    if (!b || !s) return fail(W4A16_ERR_INVALID_ARG, "b_packed and scales must be non-NULL");
    if (M != 0 && (!a || !out)) return fail(W4A16_ERR_INVALID_ARG, "a and out must be non-NULL when M > 0");
    int rc = validate_sizes(M, K, N, G);
    if (rc != W4A16_OK) return rc;
    if (!qz && (zp < 0 || zp > 15)) return fail(W4A16_ERR_INVALID_ARG, "zp_bias must be in [0, 15]");
    const size_t out_b = (size_t)M * N * 2;
    if (overlaps(out, out_b, a, (size_t)M * K * 2) || overlaps(out, out_b, b, (size_t)K * (N / 8) * 4) ||
        overlaps(out, out_b, s, (size_t)(K / G) * N * 2) ||
        overlaps(out, out_b, qz, (size_t)(K / G) * (N / 8) * 4))
        return fail(W4A16_ERR_INVALID_ARG, "out overlaps an input");
    if (!aligned16(a) || !aligned16(b) || !aligned16(s) || !aligned16(out) || (qz && !aligned16(qz)))
        return fail(W4A16_ERR_UNSUPPORTED, "a, b_packed, scales, qzeros and out must be 16-byte aligned");
    return W4A16_OK;
}

// exact_form: the dot2 GEMV keeping (q - z) exact per weight (no folded zero
// correction, no matrix cores).  The decode step's separate-kernel route uses
// it for every linear (the oracle's roundings).
int run_gemm(const uint16_t *a, const int32_t *b, const uint16_t *s, const int32_t *qz, int64_t M,
             int64_t K, int64_t N, int64_t G, int32_t zp, uint16_t *out, hipStream_t stream,
             bool exact_form = false) {
    if (M == 0) return ok();
    GemmPlan plan = plan_gemm(M, K, N, G, !exact_form);
    if (exact_form) plan.fold = plan.fold_asym = false;
    GemmArgs args{a, b, s, qz, M, K, N, G, zp, out, nullptr, nullptr};
    int rc = get_scratch(stream, plan, &args.partials, &args.counters);
    if (rc != W4A16_OK) return rc;
    hipError_t e = plan.path == kPathGemv ? launch_gemv(args, plan, stream) : launch_mfma(args, plan, stream);
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return ok();
}

// GEMV whose activations are the glue transform (act 1: row-norm, act 2:
// SwiGLU + row-norm) of `src` (row stride ld), for the decode step.
int run_gemm_act(int act, const uint16_t *src, int64_t ld, const w4a16_linear &L, int64_t M, int64_t K, int64_t N,
                 uint16_t *out, hipStream_t stream) {
    GemmPlan plan = plan_gemm(M, K, N, L.G, true, act != 2);
    if (plan.path == kPathMfma) {
        if (act != 1) return fail(W4A16_ERR_UNSUPPORTED, "the MFMA path folds the row-norm only");
        plan.partial_floats += mfma_rn_extra_floats(plan);
    }
    GemmArgs args{nullptr, L.b_packed, L.scales, L.qzeros, M, K, N, L.G, L.zp_bias, out, nullptr, nullptr};
    int rc = get_scratch(stream, plan, &args.partials, &args.counters);
    if (rc != W4A16_OK) return rc;
    hipError_t e = plan.path == kPathMfma ? launch_mfma_rn(args, plan, true, src, ld, stream)
                                          : launch_gemv_act(args, plan, act, src, ld, stream);
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return ok();
}

// A glue step folds into the GEMV that consumes it when that GEMV runs the
// default shape (M <= 8, 8 waves).
bool fusable(const GemmPlan &p) { return p.path == kPathGemv && p.waves == 8; }

// Decode-step workspace layout: two buffers of M x maxN fp16 (maxN = the
// widest linear output), each 256-byte aligned.
struct DecodeShape {
    int64_t H = 0, NQ = 0, I = 0, maxN = 0, maxK = 0;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_stack(const w4a16_linear *lin, int64_t n_layers, DecodeShape *sh) {
    if (!lin || n_layers <= 0) return fail(W4A16_ERR_INVALID_ARG, "empty stack");
    const int64_t H = lin[0].K;
    DecodeShape d;
    d.H = H;
    for (int64_t l = 0; l < n_layers; ++l) {
        const w4a16_linear *L = lin + 4 * l;
        const int64_t I = L[2].N / 2;
        if (L[0].K != H || L[0].N < H || L[1].K != H || L[1].N != H || L[2].K != H || L[2].N % 2 != 0 ||
            L[3].K != I || L[3].N != H)
            return fail(W4A16_ERR_INVALID_ARG, "stack shapes do not chain (qkv, o, gate_up, down)");
        for (int j = 0; j < 4; ++j) {
            if (!L[j].b_packed || !L[j].scales)
                return fail(W4A16_ERR_INVALID_ARG, "stack linear with NULL weights or scales");
            int rc = validate_sizes(1, L[j].K, L[j].N, L[j].G);
            if (rc != W4A16_OK) return rc;
            if (!L[j].qzeros && (L[j].zp_bias < 0 || L[j].zp_bias > 15))
                return fail(W4A16_ERR_INVALID_ARG, "zp_bias must be in [0, 15]");
            if (!aligned16(L[j].b_packed) || !aligned16(L[j].scales) || (L[j].qzeros && !aligned16(L[j].qzeros)))
                return fail(W4A16_ERR_UNSUPPORTED, "stack tensors must be 16-byte aligned");
            d.maxN = std::max(d.maxN, L[j].N);
        }
        if (H % 8 != 0 || I % 8 != 0 || H > kGlueMaxWidth || I > kGlueMaxWidth)
            return fail(W4A16_ERR_UNSUPPORTED, "decode step needs H and I multiples of 8 and at most 32768");
        d.I = std::max(d.I, I);
        d.NQ = std::max(d.NQ, L[0].N);
    }
    d.maxK = std::max(d.H, d.I);
    *sh = d;
    return W4A16_OK;
}

}  // namespace

extern "C" {

const char *w4a16_status_string(int status) {
    switch (status) {
        case W4A16_OK: return "W4A16_OK";
        case W4A16_ERR_INVALID_ARG: return "W4A16_ERR_INVALID_ARG";
        case W4A16_ERR_UNSUPPORTED: return "W4A16_ERR_UNSUPPORTED";
        case W4A16_ERR_HIP: return "W4A16_ERR_HIP";
        case W4A16_ERR_WORKSPACE: return "W4A16_ERR_WORKSPACE";
        default: return "W4A16_ERR_UNKNOWN";
    }
}

const char *w4a16_last_error(void) { return g_last_error.c_str(); }

int w4a16_repack(const int32_t *src_nk8, int32_t *dst_kn8, int64_t K, int64_t N, hipStream_t stream) {
    if (!src_nk8 || !dst_kn8) return fail(W4A16_ERR_INVALID_ARG, "src and dst must be non-NULL");
    if (K <= 0 || N <= 0 || K % 8 != 0 || N % 8 != 0)
        return fail(W4A16_ERR_INVALID_ARG, "K and N must be positive multiples of 8");
    if (K * (N / 8) > (1ll << 31)) return fail(W4A16_ERR_UNSUPPORTED, "repack too large for 32-bit indexing");
    const size_t bytes = (size_t)K * (N / 8) * 4;
    if (overlaps(src_nk8, bytes, dst_kn8, bytes)) return fail(W4A16_ERR_INVALID_ARG, "dst overlaps src");
    hipError_t e = launch_repack(src_nk8, dst_kn8, K, N, stream);
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, std::string("repack launch: ") + hipGetErrorString(e));
    return ok();
}

int w4a16_repack_scales(const uint16_t *src_ng, uint16_t *dst_gn, int64_t Gn, int64_t N, hipStream_t stream) {
    if (!src_ng || !dst_gn) return fail(W4A16_ERR_INVALID_ARG, "src and dst must be non-NULL");
    if (Gn <= 0 || N <= 0 || N % 8 != 0)
        return fail(W4A16_ERR_INVALID_ARG, "Gn must be positive and N a positive multiple of 8");
    if (Gn * N >= (1ll << 31) || N >= (1ll << 30))
        return fail(W4A16_ERR_UNSUPPORTED, "scales too large for 32-bit indexing");
    const size_t bytes = (size_t)Gn * N * 2;
    if (overlaps(src_ng, bytes, dst_gn, bytes)) return fail(W4A16_ERR_INVALID_ARG, "dst overlaps src");
    hipError_t e = launch_repack_scales(src_ng, dst_gn, Gn, N, stream);
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, std::string("scale repack launch: ") + hipGetErrorString(e));
    return ok();
}

int w4a16_gemm(const uint16_t *a, const int32_t *b_packed, const uint16_t *scales, const int32_t *qzeros,
               int64_t M, int64_t K, int64_t N, int64_t G, int32_t zp_bias, uint16_t *out,
               hipStream_t stream) {
    int rc = validate_gemm(a, b_packed, scales, qzeros, M, K, N, G, zp_bias, out);
    if (rc != W4A16_OK) return rc;
    return run_gemm(a, b_packed, scales, qzeros, M, K, N, G, zp_bias, out, stream);
}

int w4a16_gemm_plan(int64_t M, int64_t K, int64_t N, int64_t G, int32_t *path, int32_t *splits,
                    int64_t *grid) {
    int rc = validate_sizes(M, K, N, G);
    if (rc != W4A16_OK) return rc;
    const GemmPlan p = plan_gemm(std::max<int64_t>(M, 1), K, N, G);
    if (path) *path = p.mma ? 3 : p.path;
    if (splits) *splits = p.splits;
    if (grid) *grid = p.grid;
    return ok();
}

size_t w4a16_decode_workspace_bytes(int64_t M, const w4a16_linear *lin, int64_t n_layers) {
    DecodeShape d;
    if (M <= 0 || check_stack(lin, n_layers, &d) != W4A16_OK) return 0;
    return 2 * align256((size_t)M * d.maxN * 2);
}

int w4a16_decode_step(const w4a16_linear *lin, int64_t n_layers, const uint16_t *x_in, uint16_t *x_out,
                      int64_t M, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!x_in || !x_out || !workspace) return fail(W4A16_ERR_INVALID_ARG, "x_in, x_out and workspace must be non-NULL");
    if (M < 1 || M > 8192) return fail(W4A16_ERR_INVALID_ARG, "M must be in [1, 8192]");
    DecodeShape d;
    int rc = check_stack(lin, n_layers, &d);
    if (rc != W4A16_OK) return rc;
    const size_t buf_bytes = align256((size_t)M * d.maxN * 2);
    const size_t need = 2 * buf_bytes;
    if (workspace_bytes < need) return fail(W4A16_ERR_INVALID_ARG, "workspace smaller than w4a16_decode_workspace_bytes()");
    if (M * d.maxN >= (1ll << 31)) return fail(W4A16_ERR_UNSUPPORTED, "decode step too large for 32-bit kernel indexing");
    if (!aligned16(x_in) || !aligned16(x_out) || !aligned16(workspace))
        return fail(W4A16_ERR_UNSUPPORTED, "x_in, x_out and workspace must be 16-byte aligned");
    const size_t x_b = (size_t)M * d.H * 2;
    if (overlaps(workspace, need, x_in, x_b) || overlaps(workspace, need, x_out, x_b))
        return fail(W4A16_ERR_INVALID_ARG, "workspace overlaps x_in or x_out");
    // Two buffers, each M x maxN: every kernel reads one and writes the other.
    uint16_t *A = static_cast<uint16_t *>(workspace);
    uint16_t *B = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) + buf_bytes);
    auto other = [&](const uint16_t *p) { return p == A ? B : A; };
    auto glue = [](hipError_t e) {
        return e == hipSuccess ? W4A16_OK
                               : fail(W4A16_ERR_HIP, std::string("glue launch: ") + hipGetErrorString(e));
    };
    const bool fuse = tune().decode_fuse != 0;
    const uint16_t *x = x_in;  // the layer input, row-normed (when pend is null)
    uint16_t *pend = nullptr;  // or: the previous layer's down output, its row-norm not yet applied
    for (int64_t l = 0; l < n_layers; ++l) {
        const w4a16_linear *L = lin + 4 * l;
        const int64_t H = d.H, NQ = L[0].N, I = L[2].N / 2;
        const GemmPlan pq = plan_gemm(M, H, NQ, L[0].G), po = plan_gemm(M, H, H, L[1].G),
                       pg = plan_gemm(M, H, 2 * I, L[2].G), pd = plan_gemm(M, I, H, L[3].G);
        // GEMV route (M <= 8): every glue step runs inside the GEMV that consumes
        // it.  MFMA route: the row-norms run inside the MFMA GEMMs that consume
        // them; SwiGLU + row-norm stays a kernel of its own.
        const bool gemv_route = fuse && fusable(po) && fusable(pg) && fusable(pd);
        const bool mfma_route = fuse && !gemv_route && po.path == kPathMfma && pg.path == kPathMfma;
        const bool qkv_rn = pend && ((gemv_route && fusable(pq)) || (mfma_route && pq.path == kPathMfma));
        if (pend && !qkv_rn) {
            if ((rc = glue(launch_rownorm(pend, M, H, H, x_out, stream)))) return rc;
            x = x_out;
            pend = nullptr;
        }
        uint16_t *q = pend ? other(pend) : A;
        uint16_t *o = other(q);
        if ((rc = qkv_rn ? run_gemm_act(1, pend, H, L[0], M, H, NQ, q, stream)
                         : run_gemm(x, L[0].b_packed, L[0].scales, L[0].qzeros, M, H, NQ, L[0].G, L[0].zp_bias,
                                    q, stream, !fuse)))
            return rc;
        if (gemv_route && M < tune().decode_swiglu_m) {
            // q -> o (O), o -> q (gate+up), q -> o (down)
            if ((rc = run_gemm_act(1, q, NQ, L[1], M, H, H, o, stream)) ||
                (rc = run_gemm_act(1, o, H, L[2], M, H, 2 * I, q, stream)) ||
                (rc = run_gemm_act(2, q, 2 * I, L[3], M, I, H, o, stream)))
                return rc;
            pend = o;
        } else if (gemv_route) {
            // SwiGLU folded into the down GEMV costs every workgroup M x I
            // SwiGLUs for its row sums; from decode_swiglu_m rows on it runs
            // as a kernel of its own.  q -> o (O), o -> q (gate+up),
            // q -> o (SwiGLU + row-norm), o -> q (down)
            if ((rc = run_gemm_act(1, q, NQ, L[1], M, H, H, o, stream)) ||
                (rc = run_gemm_act(1, o, H, L[2], M, H, 2 * I, q, stream)) ||
                (rc = glue(launch_swiglu_rownorm(q, M, I, o, stream))) ||
                (rc = run_gemm(o, L[3].b_packed, L[3].scales, L[3].qzeros, M, I, H, L[3].G, L[3].zp_bias, q,
                               stream)))
                return rc;
            pend = q;
        } else if (mfma_route) {
            // q -> o (O), o -> q (gate+up), q -> o (SwiGLU + row-norm), o -> q (down)
            if ((rc = run_gemm_act(1, q, NQ, L[1], M, H, H, o, stream)) ||
                (rc = run_gemm_act(1, o, H, L[2], M, H, 2 * I, q, stream)) ||
                (rc = glue(launch_swiglu_rownorm(q, M, I, o, stream))) ||
                (rc = run_gemm(o, L[3].b_packed, L[3].scales, L[3].qzeros, M, I, H, L[3].G, L[3].zp_bias, q,
                               stream, true)))
                return rc;
            pend = q;
        } else {
            // every glue step a kernel of its own
            if ((rc = glue(launch_rownorm(q, M, NQ, H, o, stream))) ||
                (rc = run_gemm(o, L[1].b_packed, L[1].scales, L[1].qzeros, M, H, H, L[1].G, L[1].zp_bias, q, stream, true)) ||
                (rc = glue(launch_rownorm(q, M, H, H, o, stream))) ||
                (rc = run_gemm(o, L[2].b_packed, L[2].scales, L[2].qzeros, M, H, 2 * I, L[2].G, L[2].zp_bias, q, stream, true)) ||
                (rc = glue(launch_swiglu_rownorm(q, M, I, o, stream))) ||
                (rc = run_gemm(o, L[3].b_packed, L[3].scales, L[3].qzeros, M, I, H, L[3].G, L[3].zp_bias, q, stream, true)) ||
                (rc = glue(launch_rownorm(q, M, H, H, x_out, stream))))
                return rc;
            x = x_out;
        }
    }
    if (pend && (rc = glue(launch_rownorm(pend, M, d.H, d.H, x_out, stream)))) return rc;
    return ok();
}

int w4a16_set_tuning(const char *spec) {
    Tune *v = new Tune();
    if (!parse_tune(spec, v)) {
        delete v;
        return fail(W4A16_ERR_INVALID_ARG, "malformed tuning spec or unknown key");
    }
    tune();  // the environment's snapshot is taken first, then replaced
    g_tune.store(v, std::memory_order_release);
    return ok();
}

int w4a16_release(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    int rc = W4A16_OK;
    for (auto &kv : g_scratch) {
        int cur = 0;
        (void)hipGetDevice(&cur);
        if (hipSetDevice(kv.first.first) != hipSuccess) rc = W4A16_ERR_HIP;
        if (hipStreamSynchronize(kv.first.second) != hipSuccess) rc = W4A16_ERR_HIP;
        if (kv.second.partials) (void)hipFree(kv.second.partials);
        if (kv.second.counters) (void)hipFree(kv.second.counters);
        (void)hipSetDevice(cur);
    }
    g_scratch.clear();
    if (rc != W4A16_OK) return fail(rc, "synchronising a stream during release failed");
    return ok();
}

}  // extern "C"
