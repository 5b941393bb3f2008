// cp_chain.cpp -- host side of the C ABI declared in include/cp_chain.h:
// argument validation, the dependency-table builder, plan-owned device state,
// the three execution modes, and the invariant read-back.
//
// Method: CTA-Pipelining (arXiv 2607.07862).  The dependency structure --
// dependency arrays, scoreboards and work-queues (§III-A) -- is built here
// from the static tile dataflow of the GEMM chain: in the two-layer running
// example (§III-B) a tile (i, j) of the second GEMM reads row-block i of the
// first GEMM's output across all its columns, so it depends on every tile
// (i, k) of that row-block.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "cp_chain.h"
#include "cp_device.h"

namespace {

// detail of the last failure on this thread: a fixed buffer, so that error
// paths allocate nothing either
thread_local char g_last_error[512];

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_last_error[0] = 0; }

#define CP_HIP(call)                                                                     \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess)                                                            \
            return fail(e_ == hipErrorOutOfMemory ? CP_ERR_OOM : CP_ERR_HIP, "%s: %s (%s:%d)", \
                        #call, hipGetErrorString(e_), __FILE__, __LINE__);               \
    } while (0)

// Tile graph of a chain: flat work-item IDs, in-degree template and CSR
// out-edges.  Without split-K an item is a tile; with nsplit[l] > 1 each
// tile of layer l is nsplit[l] consecutive items over disjoint k ranges.
struct TileGraph {
    int32_t T = 0, P1 = 0, E = 0;
    std::vector<int32_t> layer_off, nbn, nsplit, indeg, dep_off, dep_ids;
};

int check_shape(int64_t M, int32_t L, const int64_t *widths, int32_t tile_m, int32_t tile_n,
                int32_t k_step) {
    if (L < 1 || L > CP_MAX_LAYERS) return fail(CP_ERR_INVALID_ARG, "n_layers %d not in [1, %d]", L, CP_MAX_LAYERS);
    if (!widths) return fail(CP_ERR_INVALID_ARG, "widths is NULL");
    if (tile_m <= 0 || tile_n <= 0) return fail(CP_ERR_INVALID_ARG, "tile %dx%d", tile_m, tile_n);
    if (M <= 0) return fail(CP_ERR_SHAPE, "M = %lld must be positive", (long long)M);
    if (M % tile_m) return fail(CP_ERR_SHAPE, "M = %lld is not a multiple of tile_m = %d", (long long)M, tile_m);
    int64_t tiles = 0;
    for (int l = 0; l <= L; ++l) {
        if (widths[l] <= 0) return fail(CP_ERR_SHAPE, "widths[%d] = %lld must be positive", l, (long long)widths[l]);
        if (widths[l] > (int64_t)1 << 22)
            return fail(CP_ERR_SHAPE, "widths[%d] = %lld exceeds 2^22 (tile-relative 32-bit offsets)", l,
                        (long long)widths[l]);
        if (l < L && k_step > 0 && widths[l] % k_step)
            return fail(CP_ERR_SHAPE, "contraction length widths[%d] = %lld is not a multiple of %d", l,
                        (long long)widths[l], k_step);
        if (l > 0) {
            if (widths[l] % tile_n)
                return fail(CP_ERR_SHAPE, "N_%d = %lld is not a multiple of tile_n = %d", l, (long long)widths[l], tile_n);
            tiles += (M / tile_m) * (widths[l] / tile_n);
        }
    }
    if (M > (int64_t)1 << 30) return fail(CP_ERR_SHAPE, "M too large");
    if (tiles >= (int64_t)0x7FFFFFF0) return fail(CP_ERR_SHAPE, "too many tiles");
    return CP_OK;
}

// Sizes of the tile graph in 64-bit arithmetic, before anything is built:
// items T = sum_l nrb nbn_l nsplit_l, edges E = sum_l nrb nbn_l nbn_{l+1}
// (a producer tile has one edge per consumer tile of its row-block, split
// or not).  The graph holds them in int32 arrays (dep_off has T + 1
// entries and its last one is E), so both, and T + E, must stay below
// 2^31.
int check_graph_size(int64_t M, int32_t L, const int64_t *widths, int32_t tile_m, int32_t tile_n,
                     const int32_t *nsplit) {
    const int64_t nrb = M / tile_m, lim = (int64_t)0x7FFFFFF0;
    int64_t T = 0, E = 0;
    for (int l = 0; l < L; ++l) {
        const int64_t nbn = widths[l + 1] / tile_n, ns = nsplit ? nsplit[l] : 1;
        T += nrb * nbn * ns;  // each factor < 2^31, nbn * ns <= 2^22 * 2^22 when ns divides K0
        if (l + 1 < L) E += nrb * nbn * (widths[l + 2] / tile_n);
        if (T > lim || E > lim) break;
    }
    if (T > lim || E > lim || T + E > lim)
        return fail(CP_ERR_SHAPE, "tile graph too large: %lld work items and %lld dependency edges "
                    "(the table is indexed with 32-bit integers)", (long long)T, (long long)E);
    return CP_OK;
}

// Dependency table (§III-A): tile (l+1, i, j) waits on all N_l / tile_n tiles
// (l, i, k) of row-block i, because its A operand is that whole row-block.
// With split-K, item s of tile (l+1, i, j) reads only columns
// [s N_l / ns, (s + 1) N_l / ns) of that row-block, so it waits on just the
// producer tiles of those columns.  A producer tile's out-edges sit on its
// first item: whichever of its items completes the tile releases them.
void build_graph(int64_t M, int32_t L, const int64_t *widths, int32_t tile_m, int32_t tile_n,
                 const int32_t *nsplit, TileGraph &g) {
    const int32_t nrb = (int32_t)(M / tile_m);
    g.layer_off.assign(L + 1, 0);
    g.nbn.assign(L, 0);
    g.nsplit.assign(L, 1);
    for (int l = 0; l < L; ++l) {
        g.nbn[l] = (int32_t)(widths[l + 1] / tile_n);
        g.nsplit[l] = nsplit ? nsplit[l] : 1;
        g.layer_off[l + 1] = g.layer_off[l] + nrb * g.nbn[l] * g.nsplit[l];
    }
    g.T = g.layer_off[L];
    g.P1 = g.layer_off[1];
    g.indeg.assign(g.T, 0);
    g.dep_off.assign(g.T + 1, 0);
    for (int l = 0; l < L; ++l)
        for (int32_t t = g.layer_off[l]; t < g.layer_off[l + 1]; ++t) {
            const int32_t split = (t - g.layer_off[l]) % g.nsplit[l];
            if (l > 0) g.indeg[t] = g.nbn[l - 1] / g.nsplit[l];
            g.dep_off[t + 1] = g.dep_off[t] + (l + 1 < L && split == 0 ? g.nbn[l + 1] : 0);
        }
    g.E = g.dep_off[g.T];
    g.dep_ids.assign(g.E, 0);
    for (int l = 0; l + 1 < L; ++l) {
        const int32_t per_split = g.nbn[l] / g.nsplit[l + 1];  // producer tiles per consumer k range
        for (int32_t i = 0; i < nrb; ++i)
            for (int32_t k = 0; k < g.nbn[l]; ++k) {
                const int32_t p = g.layer_off[l] + (i * g.nbn[l] + k) * g.nsplit[l];
                int32_t e = g.dep_off[p];
                for (int32_t j = 0; j < g.nbn[l + 1]; ++j)
                    g.dep_ids[e++] = g.layer_off[l + 1] + (i * g.nbn[l + 1] + j) * g.nsplit[l + 1] + k / per_split;
            }
    }
}

// Split-K factor per layer: a layer with fewer tiles than the persistent grid
// holds is split into power-of-two k ranges until it fills the grid, keeping
// at least 16 k steps per bf16 item (4 slabs of 32 k per fp32 item) and
// (beyond layer 0) k ranges that are whole producer tiles.
void choose_splits(int64_t M, int32_t L, const int64_t *widths, int32_t tile_m, int32_t tile_n, int32_t dtype,
                   int32_t k_step, int32_t capacity, bool allow, int32_t *ns) {
    const int64_t nrb = M / tile_m;
    for (int l = 0; l < L; ++l) {
        ns[l] = 1;
        if (!allow) continue;
        // an item keeps at least 16 k steps of the tile body (bf16: 64 k, or
        // 128 k for 256x256 tiles) or 4 steps of 32 k (fp32: its small tiles
        // leave most of the device idle otherwise; on the 128x512x512x512
        // chain 4 steps ran 21.8 us, 2 steps 23.5 us, 8 steps 26.5 us)
        const int64_t min_slabs = dtype == CP_BF16 ? 16 : 4;
        const int64_t tiles = nrb * (widths[l + 1] / tile_n), slabs = widths[l] / k_step;
        const int64_t prod_tiles = l > 0 ? widths[l] / tile_n : 0;
        while (tiles * 2 * ns[l] <= capacity && slabs % (2 * ns[l]) == 0 && slabs / (2 * ns[l]) >= min_slabs &&
               (l == 0 || prod_tiles % (2 * ns[l]) == 0))
            ns[l] *= 2;
    }
}

}  // namespace

struct cp_chain {
    int64_t M = 0;
    int32_t L = 0;
    int64_t widths[CP_MAX_LAYERS + 1] = {};
    int32_t dtype = 0, tile_m = 0, tile_n = 0;
    int32_t acts[CP_MAX_LAYERS] = {};
    uint32_t flags = 0;
    int device = 0;
    const cp::Variant *var = nullptr;
    TileGraph g;
    int n_workers = 0;                 // pipelined mode's persistent grid
    // Queue layouts: kXcd (pipelined mode) has one queue per XCD, a tile in
    // the queue of its column panel mod 8, and worker b serves queue b mod 8;
    // kLayer (spatial mode) has one queue per layer, served by that layer's
    // own launch.
    struct Layout {
        int nq = 1;
        int32_t qbase[cp::kMaxQueues] = {}, qsize[cp::kMaxQueues] = {}, qfirst[cp::kMaxQueues] = {};
        int32_t qworkers[cp::kMaxQueues] = {};
        int32_t first_formula = 0;     // pre-filled slots follow cp::first_item
        uint32_t *d_qinit = nullptr;   // initial queue image
    } lay[2];
    int copy_layout[2] = {0, 0};       // layout each per-run state copy was reset for
    int last_layout = 0;
    // spatial mode: two disjoint CU sets, layer l on set l mod 2, each set
    // with its own CU-masked stream (made on first use)
    int n_sets = 1;
    uint32_t cu_mask[2][8] = {};
    int sp_workers[CP_MAX_LAYERS] = {};
    int sp_cus[2] = {};
    hipStream_t sp_stream[2] = {};
    hipEvent_t sp_join[2] = {};
    bool coop = false;                 // cooperative launch of the persistent grid
    // device state (one allocation) and intermediates.  The per-run state
    // (scoreboard, queues, counters, debug counts, trace) has two copies: a
    // pipelined run uses copy `cur` and its workers reset the other one,
    // which the next run uses, so no reset launch precedes the worker grid.
    char *state = nullptr;
    int32_t *d_indeg = nullptr, *d_dep_off = nullptr, *d_dep_ids = nullptr;
    int32_t *d_score[2] = {};
    uint32_t *d_arrive[3] = {};        // split-K arrival counts: run copies 0, 1 and the baselines'
    int32_t nsplit[CP_MAX_LAYERS] = {};
    float *ws[CP_MAX_LAYERS] = {};     // split-K partial tiles per split layer
    uint32_t *d_queue[2] = {}, *d_ctl[2] = {}, *d_deq[2] = {};
    uint64_t *d_trace[2] = {};
    int cur = 0;                       // copy of the next pipelined run
    int last_copy = 0;                 // copy of the last pipelined run
    void *inter[CP_MAX_LAYERS] = {};
    size_t inter_bytes[CP_MAX_LAYERS] = {};
    // CP_FLAG_LAMPORT: two sentinel-filled copies of the intermediates for the
    // pipelined runs (copy c with per-run state copy c); `lam_clean[c]` says
    // copy c holds only the sentinel (filled at plan time, or by the workers
    // of the previous run); the baselines keep using `inter`
    bool lamport = false;
    void *lam[2][CP_MAX_LAYERS] = {};
    bool lam_clean[2] = {false, false};
    int inter_src = -1;                // intermediates of the last run: -1 `inter`, else lam copy
    hipStream_t side[2] = {nullptr, nullptr};
    hipStream_t cap = nullptr;         // origin stream of graph captures
    hipEvent_t ev_fork = nullptr, ev_join[2] = {nullptr, nullptr};
    // replayable sequential / micro-batched runs, keyed by mode, chunk and pointers
    struct Replay {
        int32_t mode = 0;
        int64_t mb = 0;
        const void *X = nullptr, *W[CP_MAX_LAYERS] = {};
        void *Y = nullptr;
        hipGraph_t graph = nullptr;
        hipGraphExec_t exec = nullptr;
    };
    std::vector<Replay> replays;       // most recently used last
    hipEvent_t ev_start = nullptr, ev_kernel = nullptr, ev_stop = nullptr;  // CP_FLAG_TIMING
    hipStream_t last_stream = nullptr; // stream of the last run
    bool timed = false;                // the last run recorded timing events
    bool fenced = false;               // release protocol: fence (true) or write-through
    uint64_t timeout_ticks = 200000000ull;  // 2 s at 100 MHz
    int32_t last_mode = -1;
    bool ran = false;
};

namespace {

constexpr size_t kMaxReplays = 16;

void drop_replay(cp_chain::Replay &r) {
    if (r.exec) (void)hipGraphExecDestroy(r.exec);
    if (r.graph) (void)hipGraphDestroy(r.graph);
    r.exec = nullptr;
    r.graph = nullptr;
}

void release(cp_chain *p) {
    if (!p) return;
    for (auto &r : p->replays) drop_replay(r);
    for (auto &s : p->side)
        if (s) (void)hipStreamDestroy(s);
    if (p->cap) (void)hipStreamDestroy(p->cap);
    for (auto &st : p->sp_stream)
        if (st) (void)hipStreamDestroy(st);
    for (auto &e : p->sp_join)
        if (e) (void)hipEventDestroy(e);
    if (p->ev_fork) (void)hipEventDestroy(p->ev_fork);
    for (auto &e : p->ev_join)
        if (e) (void)hipEventDestroy(e);
    if (p->ev_start) (void)hipEventDestroy(p->ev_start);
    if (p->ev_kernel) (void)hipEventDestroy(p->ev_kernel);
    if (p->ev_stop) (void)hipEventDestroy(p->ev_stop);
    for (auto &b : p->inter)
        if (b) (void)hipFree(b);
    for (auto &c : p->lam)
        for (auto &b : c)
            if (b) (void)hipFree(b);
    for (auto &b : p->ws)
        if (b) (void)hipFree(b);
    if (p->state) (void)hipFree(p->state);
    delete p;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

cp::ChainArgs make_args(const cp_chain *p, const void *X, const void *const *W, void *Y, int copy,
                        int32_t mode = CP_MODE_PIPELINED, int layout = 0, int fixed_queue = -1) {
    cp::ChainArgs a;
    memset(&a, 0, sizeof a);
    for (int l = 0; l < p->L; ++l) {
        cp::LayerDesc &d = a.layer[l];
        d.A = l == 0 ? X : p->inter[l - 1];
        d.W = W ? W[l] : nullptr;
        d.C = l + 1 == p->L ? Y : p->inter[l];
        d.K = (int32_t)p->widths[l];
        d.N = (int32_t)p->widths[l + 1];
        d.nbn = p->g.nbn[l];
        d.act = p->acts[l];
        d.coherent = ((mode == CP_MODE_PIPELINED || mode == CP_MODE_SPATIAL) && l + 1 < p->L &&
                      !p->fenced) ? 1 : 0;
        if (p->lamport && mode == CP_MODE_PIPELINED) {
            if (l > 0) d.A = p->lam[copy][l - 1];
            if (l + 1 < p->L) d.C = p->lam[copy][l];
            d.lam_in = l > 0 ? 1 : 0;
            d.lam_out = l + 1 < p->L ? 1 : 0;
            // early dispatch: the arrival counter also counts starts
            d.arrive_shift = (p->flags & CP_FLAG_EARLY_DISPATCH) && l + 1 < p->L && p->g.nsplit[l] > 1 ? 16 : 0;
        }
        d.tile_off = p->g.layer_off[l];
        d.ntiles = p->g.layer_off[l + 1] - p->g.layer_off[l];
        d.nsplit = p->g.nsplit[l];
        d.ws = p->ws[l];
    }
    a.L = p->L;
    a.T = p->g.T;
    // the kernels read the release protocol the plan chose from the flags
    a.flags = (p->flags & ~(uint32_t)CP_FLAG_FENCE_RELEASE) | (p->fenced ? CP_FLAG_FENCE_RELEASE : 0u);
    const cp_chain::Layout &ly = p->lay[layout];
    a.nq = ly.nq;
    a.nworkers = fixed_queue >= 0 ? p->sp_workers[fixed_queue] : p->n_workers;
    a.fixed_queue = fixed_queue;
    a.queue_by_layer = layout == 1 ? 1 : 0;
    for (int q = 0; q < cp::kMaxQueues; ++q) {
        a.qbase[q] = ly.qbase[q];
        a.qsize[q] = ly.qsize[q];
        a.qfirst[q] = ly.qfirst[q];
        a.qworkers[q] = ly.qworkers[q];
    }
    a.first_formula = fixed_queue < 0 ? ly.first_formula : 0;
    a.qinit = ly.d_qinit;
    const int c = copy, n = copy ^ 1;
    a.queue = p->d_queue[c];
    a.ctl = p->d_ctl[c];
    a.score = p->d_score[c];
    const bool protocol = mode == CP_MODE_PIPELINED || mode == CP_MODE_SPATIAL;
    a.arrive = protocol ? p->d_arrive[c] : p->d_arrive[2];
    a.nxt_arrive = p->d_arrive[n];
    a.nxt_queue = p->d_queue[n];
    a.nxt_ctl = p->d_ctl[n];
    a.nxt_score = p->d_score[n];
    a.dep_off = p->d_dep_off;
    a.dep_ids = p->d_dep_ids;
    a.indeg = p->d_indeg;
    a.deq_count = (p->flags & CP_FLAG_DEBUG) ? p->d_deq[c] : nullptr;
    a.trace = (p->flags & CP_FLAG_TRACE) ? p->d_trace[c] : nullptr;
    a.nxt_deq_count = (p->flags & CP_FLAG_DEBUG) ? p->d_deq[n] : nullptr;
    a.nxt_trace = (p->flags & CP_FLAG_TRACE) ? p->d_trace[n] : nullptr;
    a.timeout_ticks = p->timeout_ticks;
    if (p->lamport && mode == CP_MODE_PIPELINED) {
        // this run's workers fill the other copy for the next run
        for (int l = 0; l + 1 < p->L; ++l) {
            a.lam_fill[l] = p->lam[copy ^ 1][l];
            a.lam_fill_bytes[l] = p->inter_bytes[l];
        }
        a.lam_pattern = cp::lamport_pattern(p->dtype);
    }
    return a;
}

}  // namespace

extern "C" {

const char *cp_chain_error_string(int code) {
    switch (code) {
        case CP_OK: return "ok";
        case CP_ERR_INVALID_ARG: return "invalid argument";
        case CP_ERR_SHAPE: return "shape not supported (not a multiple of the tile or k step)";
        case CP_ERR_UNSUPPORTED: return "unsupported dtype / tile combination";
        case CP_ERR_OOM: return "out of device memory";
        case CP_ERR_HIP: return "HIP runtime error";
        case CP_ERR_TIMEOUT: return "a queue wait exceeded the watchdog (dependency never satisfied)";
        case CP_ERR_NO_DEVICE: return "no HIP device available";
        case CP_ERR_INVARIANT: return "scoreboard / queue invariant violated";
        default: return "unknown status";
    }
}

const char *cp_chain_last_error(void) { return g_last_error; }

int cp_chain_tile_graph(int64_t M, int32_t n_layers, const int64_t *widths, int32_t tile_m,
                        int32_t tile_n, int32_t *n_tiles, int32_t *n_edges, int32_t *layer_off,
                        int32_t *indeg, int32_t *dep_off, int32_t *dep_ids) {
    return cp_chain_tile_graph_split(M, n_layers, widths, tile_m, tile_n, nullptr, n_tiles, n_edges, layer_off,
                                     indeg, dep_off, dep_ids);
}

int cp_chain_tile_graph_split(int64_t M, int32_t n_layers, const int64_t *widths, int32_t tile_m,
                              int32_t tile_n, const int32_t *nsplit, int32_t *n_tiles, int32_t *n_edges,
                              int32_t *layer_off, int32_t *indeg, int32_t *dep_off, int32_t *dep_ids) {
    clear_error();
    int rc = check_shape(M, n_layers, widths, tile_m, tile_n, 0);
    if (rc) return rc;
    if (nsplit)
        for (int l = 0; l < n_layers; ++l) {
            const int64_t div = l == 0 ? widths[0] : widths[l] / tile_n;
            if (nsplit[l] < 1 || div % nsplit[l])
                return fail(CP_ERR_SHAPE, "nsplit[%d] = %d must be >= 1 and divide %lld", l, nsplit[l],
                            (long long)div);
        }
    rc = check_graph_size(M, n_layers, widths, tile_m, tile_n, nsplit);
    if (rc) return rc;
    TileGraph g;
    try {
        build_graph(M, n_layers, widths, tile_m, tile_n, nsplit, g);
    } catch (const std::bad_alloc &) {
        return fail(CP_ERR_OOM, "host allocation failed");
    }
    if (n_tiles) *n_tiles = g.T;
    if (n_edges) *n_edges = g.E;
    if (layer_off) std::copy(g.layer_off.begin(), g.layer_off.end(), layer_off);
    if (indeg) std::copy(g.indeg.begin(), g.indeg.end(), indeg);
    if (dep_off) std::copy(g.dep_off.begin(), g.dep_off.end(), dep_off);
    if (dep_ids) std::copy(g.dep_ids.begin(), g.dep_ids.end(), dep_ids);
    return CP_OK;
}

int cp_chain_plan(cp_chain **out, int64_t M, int32_t n_layers, const int64_t *widths,
                  int32_t dtype, int32_t tile_m, int32_t tile_n, const int32_t *acts,
                  uint32_t flags) {
    clear_error();
    if (!out) return fail(CP_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (dtype != CP_F32 && dtype != CP_BF16) return fail(CP_ERR_INVALID_ARG, "dtype %d", dtype);
    const cp::Variant *var = cp::find_variant(dtype, tile_m, tile_n);
    if (!var)
        return fail(CP_ERR_UNSUPPORTED, "no %s kernel for tile %dx%d", dtype == CP_BF16 ? "bf16" : "fp32",
                    tile_m, tile_n);
    int rc = check_shape(M, n_layers, widths, tile_m, tile_n, var->k_step);
    if (rc) return rc;
    rc = check_graph_size(M, n_layers, widths, tile_m, tile_n, nullptr);  // again once splits are chosen
    if (rc) return rc;
    if (acts)
        for (int l = 0; l < n_layers; ++l)
            if (acts[l] != CP_ACT_NONE && acts[l] != CP_ACT_GELU_TANH)
                return fail(CP_ERR_INVALID_ARG, "acts[%d] = %d", l, acts[l]);
    const uint32_t known = CP_FLAG_DEBUG | CP_FLAG_TRACE | CP_FLAG_POISON | CP_FLAG_DELAY_INJECT | CP_FLAG_STARVE_LAST |
                           CP_FLAG_EAGER | CP_FLAG_COOPERATIVE | CP_FLAG_FENCE_RELEASE | CP_FLAG_TIMING |
                           CP_FLAG_NO_SPLIT | CP_FLAG_LAMPORT | CP_FLAG_EARLY_DISPATCH;
    if (flags & ~known) return fail(CP_ERR_INVALID_ARG, "unknown flags 0x%x", flags & ~known);
    if ((flags & CP_FLAG_STARVE_LAST) && n_layers < 2)
        return fail(CP_ERR_INVALID_ARG, "CP_FLAG_STARVE_LAST needs at least two layers");
    if ((flags & CP_FLAG_LAMPORT) && (flags & CP_FLAG_FENCE_RELEASE))
        return fail(CP_ERR_INVALID_ARG, "CP_FLAG_LAMPORT and CP_FLAG_FENCE_RELEASE are two different release protocols");
    if ((flags & CP_FLAG_EARLY_DISPATCH) && !(flags & CP_FLAG_LAMPORT))
        return fail(CP_ERR_INVALID_ARG, "CP_FLAG_EARLY_DISPATCH needs CP_FLAG_LAMPORT (consumers started before "
                                        "their producers finish must find the sentinel in the data)");

    int ndev = 0;
    const hipError_t de = hipGetDeviceCount(&ndev);
    if (de != hipSuccess || ndev <= 0)
        return fail(CP_ERR_NO_DEVICE, "no HIP device visible (hipGetDeviceCount: %s, count %d)",
                    hipGetErrorString(de), ndev);

    cp_chain *p = new (std::nothrow) cp_chain();
    if (!p) return fail(CP_ERR_OOM, "host allocation failed");
    p->M = M;
    p->L = n_layers;
    for (int l = 0; l <= n_layers; ++l) p->widths[l] = widths[l];
    p->dtype = dtype;
    p->tile_m = tile_m;
    p->tile_n = tile_n;
    for (int l = 0; l < n_layers; ++l) p->acts[l] = acts ? acts[l] : CP_ACT_NONE;
    p->flags = flags;
    p->var = var;
    auto bail = [&](int code) {
        release(p);
        return code;
    };
    if (hipGetDevice(&p->device) != hipSuccess) return bail(fail(CP_ERR_NO_DEVICE, "hipGetDevice failed"));
    int per_cu = 0, cus = 0;
    if (var->occupancy(&per_cu, (flags & CP_FLAG_LAMPORT) != 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device) != hipSuccess)
        return bail(fail(CP_ERR_HIP, "occupancy / CU count query failed"));
    if (per_cu < 1) return bail(fail(CP_ERR_UNSUPPORTED, "kernel cannot be resident (occupancy 0)"));
    choose_splits(M, n_layers, widths, tile_m, tile_n, dtype, var->k_step, per_cu * cus,
                  !(flags & CP_FLAG_NO_SPLIT), p->nsplit);
    if (int rc3 = check_graph_size(M, n_layers, widths, tile_m, tile_n, p->nsplit)) return bail(rc3);
    try {
        build_graph(M, n_layers, widths, tile_m, tile_n, p->nsplit, p->g);
    } catch (const std::bad_alloc &) {
        return bail(fail(CP_ERR_OOM, "host allocation failed"));
    }
    if (flags & CP_FLAG_STARVE_LAST) p->g.indeg[p->g.T - 1] += 1;
    const TileGraph &g = p->g;

    // one device allocation for all protocol state
    const size_t T = (size_t)g.T, E = (size_t)std::max(g.E, 1);
    size_t off = 0;
    size_t o_ctl[2], o_score[2], o_queue[2], o_deq[2], o_trace[2], o_arrive[3];
    for (int c = 0; c < 3; ++c) {
        o_arrive[c] = off; off = align_up(off + T * 4, 256);  // two run copies + the baselines'
    }
    for (int c = 0; c < 2; ++c) {
        o_ctl[c] = off;   off = align_up(off + cp::kCtlWords * 4, 256);
        o_score[c] = off; off = align_up(off + T * 4, 256);
        o_queue[c] = off; off = align_up(off + T * 4, 256);
        o_deq[c] = off;   off = align_up(off + T * 4, 256);
        o_trace[c] = off; off = align_up(off + ((flags & CP_FLAG_TRACE) ? T * 8 * cp::kTraceWords : 0), 256);
    }
    const size_t o_indeg = off;   off = align_up(off + T * 4, 256);
    const size_t o_doff = off;    off = align_up(off + (T + 1) * 4, 256);
    const size_t o_dids = off;    off = align_up(off + E * 4, 256);
    const size_t o_qinit = off;   off = align_up(off + T * 4, 256);
    const size_t o_qinit2 = off;  off = align_up(off + T * 4, 256);
    int rc2 = [&]() -> int {
        CP_HIP(hipMalloc(&p->state, off));
        for (int c = 0; c < 2; ++c) {
            p->d_ctl[c] = reinterpret_cast<uint32_t *>(p->state + o_ctl[c]);
            p->d_score[c] = reinterpret_cast<int32_t *>(p->state + o_score[c]);
            p->d_queue[c] = reinterpret_cast<uint32_t *>(p->state + o_queue[c]);
            p->d_deq[c] = reinterpret_cast<uint32_t *>(p->state + o_deq[c]);
            p->d_trace[c] = (flags & CP_FLAG_TRACE) ? reinterpret_cast<uint64_t *>(p->state + o_trace[c]) : nullptr;
        }
        for (int c = 0; c < 3; ++c) p->d_arrive[c] = reinterpret_cast<uint32_t *>(p->state + o_arrive[c]);
        p->d_indeg = reinterpret_cast<int32_t *>(p->state + o_indeg);
        p->d_dep_off = reinterpret_cast<int32_t *>(p->state + o_doff);
        p->d_dep_ids = reinterpret_cast<int32_t *>(p->state + o_dids);
        p->lay[0].d_qinit = reinterpret_cast<uint32_t *>(p->state + o_qinit);
        p->lay[1].d_qinit = reinterpret_cast<uint32_t *>(p->state + o_qinit2);
        CP_HIP(hipMemset(p->state, 0, off));
        CP_HIP(hipMemcpy(p->d_indeg, g.indeg.data(), T * 4, hipMemcpyHostToDevice));
        CP_HIP(hipMemcpy(p->d_dep_off, g.dep_off.data(), (T + 1) * 4, hipMemcpyHostToDevice));
        if (g.E) CP_HIP(hipMemcpy(p->d_dep_ids, g.dep_ids.data(), (size_t)g.E * 4, hipMemcpyHostToDevice));
        const size_t es = dtype == CP_BF16 ? 2 : 4;
        for (int l = 0; l + 1 < n_layers; ++l) {
            p->inter_bytes[l] = (size_t)M * (size_t)widths[l + 1] * es;
            CP_HIP(hipMalloc(&p->inter[l], p->inter_bytes[l]));
        }
        p->lamport = (flags & CP_FLAG_LAMPORT) != 0;
        if (p->lamport) {
            for (int c = 0; c < 2; ++c)
                for (int l = 0; l + 1 < n_layers; ++l) {
                    CP_HIP(hipMalloc(&p->lam[c][l], p->inter_bytes[l]));
                    CP_HIP(cp::launch_fill(p->lam[c][l], p->inter_bytes[l], cp::lamport_pattern(dtype), nullptr));
                }
            CP_HIP(hipDeviceSynchronize());
            p->lam_clean[0] = p->lam_clean[1] = true;
        }
        for (int l = 0; l < n_layers; ++l)  // split-K partials: one fp32 tile per item
            if (p->nsplit[l] > 1)
                CP_HIP(hipMalloc(&p->ws[l], (size_t)(g.layer_off[l + 1] - g.layer_off[l]) * tile_m * tile_n * 4));
        CP_HIP(hipEventCreateWithFlags(&p->ev_fork, hipEventDisableTiming));
        for (auto &e : p->ev_join) CP_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
        CP_HIP(hipEventCreate(&p->ev_start));
        CP_HIP(hipEventCreate(&p->ev_kernel));
        CP_HIP(hipEventCreate(&p->ev_stop));
        p->n_workers = std::max(1, std::min(per_cu * cus, g.T));
        // Release protocol (both exact): write-through unless the fence is
        // asked for.  Interleaved steady-state measurements on one MI355X
        // favoured write-through on every shape tried (C3 413 vs 418 us,
        // C4 512 vs 548, M = 4096 803 vs 815, M = 16384 3168 vs 3211).
        p->fenced = (flags & CP_FLAG_FENCE_RELEASE) != 0;
        if (flags & CP_FLAG_COOPERATIVE) {
            int coop_ok = 0;
            if (hipDeviceGetAttribute(&coop_ok, hipDeviceAttributeCooperativeLaunch, p->device) != hipSuccess)
                coop_ok = 0;
            if (!coop_ok) return fail(CP_ERR_UNSUPPORTED, "device has no cooperative launch");
            p->coop = true;
        }
        // one queue per XCD; a tile belongs to the queue of its column panel
        int xcds = 8;
        cp_chain::Layout &lx = p->lay[0];
        lx.nq = std::max(1, std::min({cp::kMaxQueues, xcds, p->n_workers}));
        std::vector<std::vector<uint32_t>> first(lx.nq);
        std::vector<int32_t> size(lx.nq, 0);
        for (int l = 0; l < n_layers; ++l)
            for (int32_t t = g.layer_off[l]; t < g.layer_off[l + 1]; ++t) {
                cp::LayerDesc d;
                memset(&d, 0, sizeof d);
                d.tile_off = g.layer_off[l];
                d.nbn = g.nbn[l];
                d.nsplit = g.nsplit[l];
                const int q = cp::owner_queue(d, t, lx.nq);
                ++size[q];
                if (l == 0) first[q].push_back((uint32_t)t);  // row-block-major (then item order)
            }
        std::vector<uint32_t> qinit((size_t)g.T, cp::kEmpty);
        int32_t base = 0;
        for (int q = 0; q < lx.nq; ++q) {
            lx.qbase[q] = base;
            lx.qsize[q] = size[q];
            lx.qfirst[q] = (int32_t)first[q].size();
            lx.qworkers[q] = (p->n_workers - q + lx.nq - 1) / lx.nq;
            std::copy(first[q].begin(), first[q].end(), qinit.begin() + base);
            base += size[q];
        }
        // the kernel computes a worker's pre-filled first slot instead of
        // reading it; use that only where the formula reproduces the image
        lx.first_formula = 1;
        for (int q = 0; q < lx.nq && lx.first_formula; ++q)
            for (size_t r = 0; r < first[q].size(); ++r)
                if (cp::first_item(g.nbn[0] * g.nsplit[0], lx.nq, q, (uint32_t)r) != first[q][r]) {
                    lx.first_formula = 0;
                    break;
                }
        CP_HIP(hipMemcpy(lx.d_qinit, qinit.data(), T * 4, hipMemcpyHostToDevice));
        // spatial layout: queue l holds layer l's tiles (layer 0 pre-filled,
        // row-block-major).  Layer l runs on CU set l mod 2, so every layer's
        // CUs are disjoint from those of the layers it feeds and consumes;
        // the sets are sized by the flops of their layers.  The driver
        // accepts a mask only in whole groups of 8 CUs (measured: 4-CU runs
        // and every-other-CU masks are refused), so each 32-CU word of the
        // mask is cut into two contiguous runs of whole octets.  Only two
        // CU-masked streams are used: each takes a hardware queue of its own,
        // and a process has few.
        cp_chain::Layout &ll = p->lay[1];
        ll.nq = n_layers;
        p->n_sets = n_layers > 1 ? 2 : 1;
        double fl[2] = {0.0, 0.0};
        for (int l = 0; l < n_layers; ++l) fl[l % 2] += (double)widths[l] * (double)widths[l + 1];
        for (int w = 0; w < 8 && 32 * w < cus; ++w) {
            const int octs = std::min(32, cus - 32 * w) / 8;
            int o0 = octs;
            if (p->n_sets == 2) {
                if (octs < 2) return fail(CP_ERR_UNSUPPORTED, "spatial mode: too few CUs per mask word");
                o0 = std::min(octs - 1, std::max(1, (int)(fl[0] / (fl[0] + fl[1]) * octs + 0.5)));
            }
            for (int b = 0; b < 8 * octs; ++b) {
                const int set = b < 8 * o0 ? 0 : 1;
                p->cu_mask[set][w] |= 1u << b;
                ++p->sp_cus[set];
            }
        }
        for (int l = 0; l < n_layers; ++l) {
            const int32_t nt = g.layer_off[l + 1] - g.layer_off[l];
            p->sp_workers[l] = std::max(1, std::min(per_cu * p->sp_cus[l % 2], nt));
            ll.qbase[l] = g.layer_off[l];
            ll.qsize[l] = nt;
            ll.qfirst[l] = l == 0 ? nt : 0;
            ll.qworkers[l] = p->sp_workers[l];
        }
        std::vector<uint32_t> qinit2((size_t)g.T, cp::kEmpty);
        for (int32_t t = 0; t < g.P1; ++t) qinit2[t] = (uint32_t)t;
        CP_HIP(hipMemcpy(ll.d_qinit, qinit2.data(), T * 4, hipMemcpyHostToDevice));
        for (auto &s : p->side) CP_HIP(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
        CP_HIP(hipStreamCreateWithFlags(&p->cap, hipStreamNonBlocking));
        // both copies of the per-run state start reset
        for (int c = 0; c < 2; ++c) CP_HIP(cp::launch_reset(make_args(p, nullptr, nullptr, nullptr, c), p->cap));
        CP_HIP(hipStreamSynchronize(p->cap));
        int clk_khz = 0;
        if (hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeWallClockRate, p->device) == hipSuccess &&
            clk_khz > 0)
            p->timeout_ticks = (uint64_t)clk_khz * 1000ull * 2ull;  // 2 s
        if (flags & CP_FLAG_STARVE_LAST) p->timeout_ticks = (uint64_t)std::max(clk_khz, 1) * 50ull;  // 50 ms
        return CP_OK;
    }();
    if (rc2) return bail(rc2);
    *out = p;
    return CP_OK;
}

namespace {

// The layer launches of the sequential and micro-batched modes.  Micro-batched:
// chunk c of microbatch_rows rows runs its whole chain on side stream c mod 2,
// forked from and joined back into `s`.
int enqueue_layers(cp_chain *p, const cp::ChainArgs &a, int32_t mode, int64_t microbatch_rows,
                   hipStream_t s) {
    if (mode == CP_MODE_SEQUENTIAL) {
        const int nrb = (int)(p->M / p->tile_m);
        for (int l = 0; l < p->L; ++l) CP_HIP(p->var->launch_layer(a, l, 0, nrb, s));
        return CP_OK;
    }
    const int chunk_rb = (int)(microbatch_rows / p->tile_m);
    const int nchunks = (int)(p->M / microbatch_rows);
    CP_HIP(hipEventRecord(p->ev_fork, s));
    for (auto &side : p->side) CP_HIP(hipStreamWaitEvent(side, p->ev_fork, 0));
    for (int c = 0; c < nchunks; ++c) {
        hipStream_t cs = p->side[c & 1];
        for (int l = 0; l < p->L; ++l) CP_HIP(p->var->launch_layer(a, l, c * chunk_rb, chunk_rb, cs));
    }
    for (int k = 0; k < 2; ++k) {
        CP_HIP(hipEventRecord(p->ev_join[k], p->side[k]));
        CP_HIP(hipStreamWaitEvent(s, p->ev_join[k], 0));
    }
    return CP_OK;
}

// The executable graph of a sequential / micro-batched run on these pointers:
// captured from the plan's own origin stream on first use, then replayed.
int find_replay(cp_chain *p, const cp::ChainArgs &a, const void *X, const void *const *W, void *Y,
                int32_t mode, int64_t mb, hipGraphExec_t *out) {
    if (mode != CP_MODE_MICROBATCH) mb = 0;
    for (size_t i = 0; i < p->replays.size(); ++i) {
        cp_chain::Replay &r = p->replays[i];
        bool hit = r.mode == mode && r.mb == mb && r.X == X && r.Y == Y;
        for (int l = 0; hit && l < p->L; ++l) hit = r.W[l] == W[l];
        if (!hit) continue;
        std::rotate(p->replays.begin() + i, p->replays.begin() + i + 1, p->replays.end());
        *out = p->replays.back().exec;
        return CP_OK;
    }
    cp_chain::Replay r;
    r.mode = mode;
    r.mb = mb;
    r.X = X;
    r.Y = Y;
    for (int l = 0; l < p->L; ++l) r.W[l] = W[l];
    CP_HIP(hipStreamBeginCapture(p->cap, hipStreamCaptureModeThreadLocal));
    int rc = enqueue_layers(p, a, mode, mb, p->cap);
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(p->cap, &graph);
    if (rc) {
        if (graph) (void)hipGraphDestroy(graph);
        return rc;
    }
    CP_HIP(e);
    r.graph = graph;
    const hipError_t ei = hipGraphInstantiate(&r.exec, graph, nullptr, nullptr, 0);
    if (ei != hipSuccess) {
        drop_replay(r);
        CP_HIP(ei);
    }
    if (p->replays.size() >= kMaxReplays) {
        drop_replay(p->replays.front());
        p->replays.erase(p->replays.begin());
    }
    p->replays.push_back(r);
    *out = r.exec;
    return CP_OK;
}

}  // namespace

namespace {

// Spatial mode: layer l's persistent grid on CU set l mod 2 (a CU-masked
// stream), forked from and joined back into `s`.  Layer l's workers serve
// only queue l; producers push consumers into the next layer's queue.
// Disjoint CU sets make it deadlock-free: a consumer grid spinning on its
// queue never holds its producer's CUs.
int enqueue_spatial(cp_chain *p, const void *X, const void *const *W, void *Y, hipStream_t s) {
    for (int k = 0; k < p->n_sets; ++k) {
        if (p->sp_stream[k]) continue;
        const hipError_t e = hipExtStreamCreateWithCUMask(&p->sp_stream[k], 8, p->cu_mask[k]);  // 8 words
        if (e != hipSuccess) {
            p->sp_stream[k] = nullptr;
            return fail(CP_ERR_UNSUPPORTED, "spatial mode: the runtime refused a CU-masked stream (%s); "
                        "each needs a hardware queue of its own", hipGetErrorString(e));
        }
        CP_HIP(hipEventCreateWithFlags(&p->sp_join[k], hipEventDisableTiming));
    }
    CP_HIP(hipEventRecord(p->ev_fork, s));
    for (int k = 0; k < p->n_sets; ++k) CP_HIP(hipStreamWaitEvent(p->sp_stream[k], p->ev_fork, 0));
    // in layer order: a layer only ever queues behind an earlier layer on its
    // set, which never waits on it, so the in-order streams cannot deadlock
    for (int l = 0; l < p->L; ++l) {
        const cp::ChainArgs a = make_args(p, X, W, Y, p->cur, CP_MODE_SPATIAL, 1, l);
        const hipError_t e = p->var->launch_worker(a, p->sp_workers[l], false, p->sp_stream[l % 2]);
        if (e == hipErrorCooperativeLaunchTooLarge)
            return fail(CP_ERR_UNSUPPORTED, "spatial grid of layer %d (%d workers) exceeds what the device holds "
                        "at once", l, p->sp_workers[l]);
        CP_HIP(e);
    }
    for (int k = 0; k < p->n_sets; ++k) {
        CP_HIP(hipEventRecord(p->sp_join[k], p->sp_stream[k]));
        CP_HIP(hipStreamWaitEvent(s, p->sp_join[k], 0));
    }
    return CP_OK;
}

}  // namespace

int cp_chain_run(cp_chain *p, const void *X, const void *const *W, void *Y, void *stream,
                 int32_t mode, int64_t microbatch_rows) {
    clear_error();
    if (!p) return fail(CP_ERR_INVALID_ARG, "plan is NULL");
    if (!X || !W || !Y) return fail(CP_ERR_INVALID_ARG, "X, W or Y is NULL");
    for (int l = 0; l < p->L; ++l)
        if (!W[l]) return fail(CP_ERR_INVALID_ARG, "W[%d] is NULL", l);
    if (mode != CP_MODE_PIPELINED && mode != CP_MODE_SEQUENTIAL && mode != CP_MODE_MICROBATCH &&
        mode != CP_MODE_SPATIAL)
        return fail(CP_ERR_INVALID_ARG, "mode %d", mode);
    if (mode == CP_MODE_MICROBATCH) {
        if (microbatch_rows <= 0 || microbatch_rows % p->tile_m || p->M % microbatch_rows)
            return fail(CP_ERR_SHAPE, "microbatch_rows = %lld must be a positive multiple of tile_m = %d dividing M = %lld",
                        (long long)microbatch_rows, p->tile_m, (long long)p->M);
    }
    int cur = -1;
    CP_HIP(hipGetDevice(&cur));
    if (cur != p->device) return fail(CP_ERR_INVALID_ARG, "current device %d differs from the plan's %d", cur, p->device);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const cp::ChainArgs a = make_args(p, X, W, Y, p->cur, mode);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    CP_HIP(hipStreamIsCapturing(s, &cs));
    if (cs != hipStreamCaptureStatusNone) {
        // recorded into the caller's graph: kernels only, no timing events
        if (mode == CP_MODE_PIPELINED || mode == CP_MODE_SPATIAL)
            return fail(CP_ERR_UNSUPPORTED, "pipelined and spatial modes cannot be captured into a graph (their per-run state alternates between two copies)");
        if (p->flags & CP_FLAG_POISON)
            for (int l = 0; l + 1 < p->L; ++l) CP_HIP(cp::launch_poison(p->inter[l], p->inter_bytes[l], p->dtype, s));
        return enqueue_layers(p, a, mode, microbatch_rows, s);
    }

    // Timing events stall the stream for a few microseconds each, so they
    // are recorded only when the plan asks for them.
    const bool timed = (p->flags & CP_FLAG_TIMING) != 0;
    if (timed) CP_HIP(hipEventRecord(p->ev_start, s));
    if (p->flags & CP_FLAG_POISON)
        for (int l = 0; l + 1 < p->L; ++l) CP_HIP(cp::launch_poison(p->inter[l], p->inter_bytes[l], p->dtype, s));
    if (mode == CP_MODE_SPATIAL && p->lamport)
        return fail(CP_ERR_UNSUPPORTED, "spatial mode has no Lamport-sentinel release (plan built with CP_FLAG_LAMPORT)");
    if (mode == CP_MODE_PIPELINED || mode == CP_MODE_SPATIAL) {
        // The state copy must have been reset for this mode's queue layout
        // (the previous run's workers reset it for their own layout).
        const int layout = mode == CP_MODE_SPATIAL ? 1 : 0;
        if (p->copy_layout[p->cur] != layout)
            CP_HIP(cp::launch_reset(make_args(p, nullptr, nullptr, nullptr, p->cur, mode, layout), s));
        if (timed && (p->flags & CP_FLAG_POISON)) CP_HIP(hipEventRecord(p->ev_kernel, s));
        if (mode == CP_MODE_PIPELINED && p->lamport && !p->lam_clean[p->cur]) {
            // this copy was not refilled by a previous run's workers
            for (int l = 0; l + 1 < p->L; ++l)
                CP_HIP(cp::launch_fill(p->lam[p->cur][l], p->inter_bytes[l], cp::lamport_pattern(p->dtype), s));
        }
        if (mode == CP_MODE_PIPELINED) {
            if (p->lamport) p->lam_clean[0] = p->lam_clean[1] = false;  // until the launch is in
            const hipError_t e = p->var->launch_worker(a, p->n_workers, p->coop, s);
            if (e == hipErrorCooperativeLaunchTooLarge)
                return fail(CP_ERR_UNSUPPORTED, "persistent grid of %d workers exceeds what the device holds at once "
                            "for the launched kernel (every worker must be resident)", p->n_workers);
            CP_HIP(e);
            if (p->lamport) p->lam_clean[p->cur ^ 1] = true;  // this run's workers fill it
        } else {
            int rc = enqueue_spatial(p, X, W, Y, s);
            if (rc) return rc;
        }
        p->copy_layout[p->cur] = layout;
        p->copy_layout[p->cur ^ 1] = layout;  // reset by this run's workers
        p->last_layout = layout;
        p->last_copy = p->cur;
        p->inter_src = (p->lamport && mode == CP_MODE_PIPELINED) ? p->cur : -1;
        p->cur ^= 1;
    } else {
        p->inter_src = -1;
        if (p->flags & CP_FLAG_EAGER) {
            int rc = enqueue_layers(p, a, mode, microbatch_rows, s);
            if (rc) return rc;
        } else {
            hipGraphExec_t exec = nullptr;
            int rc = find_replay(p, a, X, W, Y, mode, microbatch_rows, &exec);
            if (rc) return rc;
            CP_HIP(hipGraphLaunch(exec, s));
        }
    }
    if (timed) CP_HIP(hipEventRecord(p->ev_stop, s));
    p->timed = timed;
    p->last_stream = s;
    p->last_mode = mode;
    p->ran = true;
    return CP_OK;
}

namespace {

// Wait for the plan's last run: its stop event when timed, else its stream.
int wait_last(cp_chain *p) {
    if (!p->ran) return CP_OK;
    if (p->timed) CP_HIP(hipEventSynchronize(p->ev_stop));
    else CP_HIP(hipStreamSynchronize(p->last_stream));
    return CP_OK;
}

}  // namespace

int cp_chain_stats(cp_chain *p, cp_chain_stats_t *out) {
    clear_error();
    if (!p || !out) return fail(CP_ERR_INVALID_ARG, "plan or out is NULL");
    memset(out, 0, sizeof *out);
    out->mode = p->last_mode;
    out->n_tiles = p->g.T;
    out->n_first = p->g.P1;
    out->n_edges = p->g.E;
    out->n_workers = p->n_workers;
    out->n_queues = p->lay[0].nq;
    out->tile_m = p->tile_m;
    out->tile_n = p->tile_n;
    out->bad_dequeues = -1;
    out->order_violations = -1;
    out->fenced = p->fenced ? 1 : 0;
    out->lamport = p->lamport ? 1 : 0;
    out->lamport_rereads = -1;
    for (int l = 0; l < CP_MAX_LAYERS; ++l) out->nsplit[l] = l < p->L ? p->g.nsplit[l] : 0;
    out->last_run_ms = -1.0;
    out->last_kernel_ms = -1.0;
    if (!p->ran) return CP_OK;
    int rc = wait_last(p);
    if (rc) return rc;
    if (p->timed) {
        float ms = 0.f;
        CP_HIP(hipEventElapsedTime(&ms, p->ev_start, p->ev_stop));
        out->last_run_ms = ms;
        out->last_kernel_ms = ms;
        if (p->last_mode == CP_MODE_PIPELINED && (p->flags & CP_FLAG_POISON)) {
            CP_HIP(hipEventElapsedTime(&ms, p->ev_kernel, p->ev_stop));
            out->last_kernel_ms = ms;
        }
    }
    if (p->last_mode != CP_MODE_PIPELINED && p->last_mode != CP_MODE_SPATIAL) return CP_OK;

    const size_t T = (size_t)p->g.T;
    uint32_t ctl[cp::kCtlWords];
    std::vector<int32_t> score(T);
    std::vector<uint32_t> queue(T);
    const int c = p->last_copy;
    CP_HIP(hipMemcpy(ctl, p->d_ctl[c], sizeof ctl, hipMemcpyDeviceToHost));
    CP_HIP(hipMemcpy(score.data(), p->d_score[c], T * 4, hipMemcpyDeviceToHost));
    CP_HIP(hipMemcpy(queue.data(), p->d_queue[c], T * 4, hipMemcpyDeviceToHost));
    out->status = (int32_t)ctl[cp::kCtlStatus];
    out->lamport_rereads = (p->lamport && (p->flags & CP_FLAG_DEBUG)) ? (int32_t)ctl[cp::kCtlRereads] : -1;
    const cp_chain::Layout &ly = p->lay[p->last_layout];
    out->n_queues = ly.nq;
    out->queues_drained = 1;
    for (int q = 0; q < ly.nq; ++q) {
        const uint32_t h = ctl[cp::ctl_head(q)], t = ctl[cp::ctl_tail(q)];
        out->head += h;
        out->tail += t;
        if (t != (uint32_t)ly.qsize[q] || h < (uint32_t)ly.qsize[q]) out->queues_drained = 0;
    }
    int32_t nz = 0;
    for (size_t t = 0; t < T; ++t) nz += score[t] != 0;
    out->nonzero_scores = nz;
    std::vector<uint32_t> arr(T);
    CP_HIP(hipMemcpy(arr.data(), p->d_arrive[c], T * 4, hipMemcpyDeviceToHost));
    nz = 0;
    for (size_t t = 0; t < T; ++t) nz += arr[t] != 0;
    out->nonzero_arrivals = nz;
    std::vector<uint8_t> seen(T, 0);
    bool perm = true;
    for (size_t t = 0; t < T; ++t) {
        if (queue[t] >= T || seen[queue[t]]) {
            perm = false;
            break;
        }
        seen[queue[t]] = 1;
    }
    out->queue_is_perm = perm ? 1 : 0;
    if (p->flags & CP_FLAG_DEBUG) {
        std::vector<uint32_t> deq(T);
        CP_HIP(hipMemcpy(deq.data(), p->d_deq[c], T * 4, hipMemcpyDeviceToHost));
        int32_t bad = 0;
        for (size_t t = 0; t < T; ++t) bad += deq[t] != 1;
        out->bad_dequeues = bad;
    }
    if (p->flags & CP_FLAG_TRACE) {
        std::vector<uint64_t> tr(T * cp::kTraceWords);
        CP_HIP(hipMemcpy(tr.data(), p->d_trace[c], T * 8 * cp::kTraceWords, hipMemcpyDeviceToHost));
        int32_t viol = 0;
        for (size_t pr = 0; pr < T; ++pr)
            for (int32_t e = p->g.dep_off[pr]; e < p->g.dep_off[pr + 1]; ++e) {
                const size_t c = (size_t)p->g.dep_ids[e];
                if (tr[cp::kTraceWords * c + 1] < tr[cp::kTraceWords * pr + 3]) ++viol;  // consumer dequeued before producer released
            }
        out->order_violations = viol;
    }
    if (out->status != 0) return fail(out->status, "device status %d: %s", out->status, cp_chain_error_string(out->status));
    return CP_OK;
}

int cp_chain_trace(cp_chain *p, uint64_t *out, int64_t capacity) {
    clear_error();
    if (!p || !out) return fail(CP_ERR_INVALID_ARG, "plan or out is NULL");
    if (!(p->flags & CP_FLAG_TRACE)) return fail(CP_ERR_INVALID_ARG, "plan was built without CP_FLAG_TRACE");
    if (capacity < cp::kTraceWords * (int64_t)p->g.T)
        return fail(CP_ERR_INVALID_ARG, "capacity %lld < %d*T", (long long)capacity, cp::kTraceWords);
    int rc = wait_last(p);
    if (rc) return rc;
    CP_HIP(hipMemcpy(out, p->d_trace[p->last_copy], (size_t)p->g.T * 8 * cp::kTraceWords, hipMemcpyDeviceToHost));
    return CP_OK;
}

int cp_chain_intermediate(cp_chain *p, int32_t layer, void *dst, int64_t capacity) {
    clear_error();
    if (!p || !dst) return fail(CP_ERR_INVALID_ARG, "plan or dst is NULL");
    if (layer < 1 || layer >= p->L)
        return fail(CP_ERR_INVALID_ARG, "layer %d: a %d-layer chain has intermediates C_1 .. C_%d", layer, p->L,
                    p->L - 1);
    const size_t bytes = p->inter_bytes[layer - 1];
    if (capacity < 0 || (uint64_t)capacity < bytes)
        return fail(CP_ERR_INVALID_ARG, "capacity %lld < %zu bytes of C_%d", (long long)capacity, bytes, layer);
    int rc = wait_last(p);
    if (rc) return rc;
    const void *src = p->inter_src >= 0 ? p->lam[p->inter_src][layer - 1] : p->inter[layer - 1];
    CP_HIP(hipMemcpy(dst, src, bytes, hipMemcpyDefault));
    return CP_OK;
}

int cp_chain_destroy(cp_chain *p) {
    clear_error();
    if (!p) return CP_OK;
    if (p->ran) (void)hipDeviceSynchronize();  // the last run's stream may be gone
    for (auto &s : p->side)
        if (s) (void)hipStreamSynchronize(s);
    release(p);
    return CP_OK;
}


// ----------------------------------------------------------------------------
// Allocation-free pipelined run: every piece of device state a pipelined run
// needs (dependency table, queue image, two per-run state copies,
// intermediates, split-K partials) lives in one file-scope device array, and
// the dependency table is written on the device from its closed form, so a
// call allocates neither device nor host memory.
// ----------------------------------------------------------------------------
namespace {

constexpr size_t kStaticScratchBytes = (size_t)64 << 20;  // 64 MiB per device
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kStaticMaxDevices = 64;

// Host-side bookkeeping per device: the scratch array's device address (the
// array's name is only a host-side stand-in), the resident capacity of the
// variant last used, and the shape whose tables the scratch holds, with the
// state copy the next run of that shape uses.
struct StaticDevice {
    bool ready = false;
    char *ptr = nullptr;
    int cus = 0;
    // tables in the scratch are valid for this shape
    bool have_shape = false;
    int64_t M = 0;
    int32_t L = 0, dtype = 0, tile_m = 0, tile_n = 0;
    int64_t widths[CP_MAX_LAYERS + 1] = {};
    int cur = 0;
};
StaticDevice g_static[kStaticMaxDevices];
std::mutex g_static_mu;

// Layout of one chain's state inside the scratch array (byte offsets).
struct StaticLayout {
    cp::GraphDims g;
    int nq = 1, n_workers = 0;
    int32_t qbase[cp::kMaxQueues] = {}, qsize[cp::kMaxQueues] = {}, qfirst[cp::kMaxQueues] = {},
            qworkers[cp::kMaxQueues] = {};
    size_t o_ctl[2] = {}, o_score[2] = {}, o_queue[2] = {}, o_arrive[2] = {};
    size_t o_indeg = 0, o_doff = 0, o_dids = 0, o_qinit = 0;
    size_t o_inter[CP_MAX_LAYERS] = {}, o_ws[CP_MAX_LAYERS] = {};
    size_t total = 0;
};

// Items of one row-block whose position p satisfies p mod nq == q.
int32_t per_queue(int32_t per, int nq, int q) { return per > q ? (per - q + nq - 1) / nq : 0; }

void static_layout(int64_t M, int32_t L, const int64_t *widths, int32_t dtype, int32_t tile_m, int32_t tile_n,
                   const int32_t *nsplit, int n_workers, StaticLayout &s) {
    cp::GraphDims &g = s.g;
    memset(&g, 0, sizeof g);
    g.L = L;
    g.nrb = (int32_t)(M / tile_m);
    for (int l = 0; l < L; ++l) {
        g.nbn[l] = (int32_t)(widths[l + 1] / tile_n);
        g.nsplit[l] = nsplit[l];
        g.layer_off[l + 1] = g.layer_off[l] + g.nrb * g.nbn[l] * g.nsplit[l];
        g.edge_off[l + 1] = g.edge_off[l] + (l + 1 < L ? g.nrb * g.nbn[l] * (int32_t)(widths[l + 2] / tile_n) : 0);
    }
    g.T = g.layer_off[L];
    g.E = g.edge_off[L];
    s.n_workers = n_workers;
    s.nq = std::max(1, std::min({cp::kMaxQueues, 8, n_workers}));
    int32_t base = 0;
    for (int q = 0; q < s.nq; ++q) {
        int32_t size = 0;
        for (int l = 0; l < L; ++l) size += g.nrb * per_queue(g.nbn[l] * g.nsplit[l], s.nq, q);
        s.qbase[q] = base;
        s.qsize[q] = size;
        s.qfirst[q] = g.nrb * per_queue(g.nbn[0] * g.nsplit[0], s.nq, q);
        s.qworkers[q] = (n_workers - q + s.nq - 1) / s.nq;
        base += size;
    }
    const size_t T = (size_t)g.T, E = (size_t)std::max(g.E, 1);
    size_t off = 0;
    for (int c = 0; c < 2; ++c) {
        s.o_ctl[c] = off;    off = align_up(off + cp::kCtlWords * 4, 256);
        s.o_score[c] = off;  off = align_up(off + T * 4, 256);
        s.o_queue[c] = off;  off = align_up(off + T * 4, 256);
        s.o_arrive[c] = off; off = align_up(off + T * 4, 256);
    }
    s.o_indeg = off; off = align_up(off + T * 4, 256);
    s.o_doff = off;  off = align_up(off + (T + 1) * 4, 256);
    s.o_dids = off;  off = align_up(off + E * 4, 256);
    s.o_qinit = off; off = align_up(off + T * 4, 256);
    const size_t es = dtype == CP_BF16 ? 2 : 4;
    for (int l = 0; l + 1 < L; ++l) {
        s.o_inter[l] = off;
        off = align_up(off + (size_t)M * (size_t)widths[l + 1] * es, 256);
    }
    for (int l = 0; l < L; ++l)
        if (nsplit[l] > 1) {
            s.o_ws[l] = off;
            off = align_up(off + (size_t)(g.layer_off[l + 1] - g.layer_off[l]) * tile_m * tile_n * 4, 256);
        }
    s.total = off;
}

}  // namespace

int cp_chain_run_noalloc(int64_t M, int32_t n_layers, const int64_t *widths, int32_t dtype, int32_t tile_m,
                         int32_t tile_n, const int32_t *acts, const void *X, const void *const *W, void *Y,
                         void *stream, int32_t *status) {
    clear_error();
    if (status) *status = CP_OK;
    if (dtype != CP_F32 && dtype != CP_BF16) return fail(CP_ERR_INVALID_ARG, "dtype %d", dtype);
    const cp::Variant *var = cp::find_variant(dtype, tile_m, tile_n);
    if (!var)
        return fail(CP_ERR_UNSUPPORTED, "no %s kernel for tile %dx%d", dtype == CP_BF16 ? "bf16" : "fp32", tile_m,
                    tile_n);
    int rc = check_shape(M, n_layers, widths, tile_m, tile_n, var->k_step);
    if (rc) return rc;
    rc = check_graph_size(M, n_layers, widths, tile_m, tile_n, nullptr);
    if (rc) return rc;
    if (acts)
        for (int l = 0; l < n_layers; ++l)
            if (acts[l] != CP_ACT_NONE && acts[l] != CP_ACT_GELU_TANH)
                return fail(CP_ERR_INVALID_ARG, "acts[%d] = %d", l, acts[l]);
    if (!X || !W || !Y) return fail(CP_ERR_INVALID_ARG, "X, W or Y is NULL");
    for (int l = 0; l < n_layers; ++l)
        if (!W[l]) return fail(CP_ERR_INVALID_ARG, "W[%d] is NULL", l);
    int dev = -1;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return fail(CP_ERR_NO_DEVICE, "no HIP device visible");
    CP_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kStaticMaxDevices) return fail(CP_ERR_UNSUPPORTED, "device %d beyond %d", dev, kStaticMaxDevices);
    hipStream_t s = static_cast<hipStream_t>(stream);

    std::lock_guard<std::mutex> lock(g_static_mu);
    StaticDevice &sd = g_static[dev];
    if (!sd.ready) {
        // once per device, with that device current: the array's device
        // address; kernels and copies use this, never the array's name
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(CP_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        CP_HIP(hipDeviceGetAttribute(&sd.cus, hipDeviceAttributeMultiprocessorCount, dev));
        sd.ptr = static_cast<char *>(ptr);
        sd.ready = true;
    }
    int per_cu = 0;
    CP_HIP(var->occupancy(&per_cu, false));
    if (per_cu < 1) return fail(CP_ERR_UNSUPPORTED, "kernel cannot be resident (occupancy 0)");
    // the split factors and grid of cp_chain_plan for this shape
    int32_t nsplit[CP_MAX_LAYERS] = {};
    choose_splits(M, n_layers, widths, tile_m, tile_n, dtype, var->k_step, per_cu * sd.cus, true, nsplit);
    rc = check_graph_size(M, n_layers, widths, tile_m, tile_n, nsplit);
    if (rc) return rc;
    int64_t T = 0;
    for (int l = 0; l < n_layers; ++l) T += (M / tile_m) * (widths[l + 1] / tile_n) * nsplit[l];
    const int n_workers = (int)std::max<int64_t>(1, std::min<int64_t>((int64_t)per_cu * sd.cus, T));
    StaticLayout ly;
    static_layout(M, n_layers, widths, dtype, tile_m, tile_n, nsplit, n_workers, ly);
    if (ly.total > kStaticScratchBytes)
        return fail(CP_ERR_OOM, "this chain needs %zu bytes of device state; the allocation-free entry point "
                    "holds %zu (use cp_chain_plan / cp_chain_run)", ly.total, kStaticScratchBytes);

    bool same = sd.have_shape && sd.M == M && sd.L == n_layers && sd.dtype == dtype && sd.tile_m == tile_m &&
                sd.tile_n == tile_n;
    for (int l = 0; same && l <= n_layers; ++l) same = sd.widths[l] == widths[l];

    char *base = sd.ptr;
    cp::ChainArgs a;
    memset(&a, 0, sizeof a);
    for (int l = 0; l < n_layers; ++l) {
        cp::LayerDesc &d = a.layer[l];
        d.A = l == 0 ? X : static_cast<const void *>(base + ly.o_inter[l - 1]);
        d.W = W[l];
        d.C = l + 1 == n_layers ? Y : static_cast<void *>(base + ly.o_inter[l]);
        d.K = (int32_t)widths[l];
        d.N = (int32_t)widths[l + 1];
        d.nbn = ly.g.nbn[l];
        d.act = acts ? acts[l] : CP_ACT_NONE;
        d.coherent = l + 1 < n_layers ? 1 : 0;  // write-through release
        d.tile_off = ly.g.layer_off[l];
        d.ntiles = ly.g.layer_off[l + 1] - ly.g.layer_off[l];
        d.nsplit = nsplit[l];
        d.ws = nsplit[l] > 1 ? reinterpret_cast<float *>(base + ly.o_ws[l]) : nullptr;
    }
    a.L = n_layers;
    a.T = ly.g.T;
    a.flags = 0;
    a.nq = ly.nq;
    a.nworkers = n_workers;
    a.fixed_queue = -1;
    a.queue_by_layer = 0;
    for (int q = 0; q < cp::kMaxQueues; ++q) {
        a.qbase[q] = ly.qbase[q];
        a.qsize[q] = ly.qsize[q];
        a.qfirst[q] = ly.qfirst[q];
        a.qworkers[q] = ly.qworkers[q];
    }
    a.first_formula = 1;
    a.indeg = reinterpret_cast<const int32_t *>(base + ly.o_indeg);
    a.dep_off = reinterpret_cast<const int32_t *>(base + ly.o_doff);
    a.dep_ids = reinterpret_cast<const int32_t *>(base + ly.o_dids);
    a.qinit = reinterpret_cast<const uint32_t *>(base + ly.o_qinit);
    int clk_khz = 0;
    if (hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || clk_khz <= 0)
        clk_khz = 100000;
    a.timeout_ticks = (uint64_t)clk_khz * 1000ull * 2ull;  // 2 s
    auto point = [&](cp::ChainArgs &x, int c) {
        const int n = c ^ 1;
        x.ctl = reinterpret_cast<uint32_t *>(base + ly.o_ctl[c]);
        x.score = reinterpret_cast<int32_t *>(base + ly.o_score[c]);
        x.queue = reinterpret_cast<uint32_t *>(base + ly.o_queue[c]);
        x.arrive = reinterpret_cast<uint32_t *>(base + ly.o_arrive[c]);
        x.nxt_ctl = reinterpret_cast<uint32_t *>(base + ly.o_ctl[n]);
        x.nxt_score = reinterpret_cast<int32_t *>(base + ly.o_score[n]);
        x.nxt_queue = reinterpret_cast<uint32_t *>(base + ly.o_queue[n]);
        x.nxt_arrive = reinterpret_cast<uint32_t *>(base + ly.o_arrive[n]);
    };
    if (!same) {
        // a new shape: write its tables and reset both state copies
        sd.have_shape = false;
        point(a, 0);
        CP_HIP(cp::launch_graph_setup(a, ly.g, s));
        sd.cur = 0;
    }
    point(a, sd.cur);
    const hipError_t e = var->launch_worker(a, n_workers, false, s);
    if (e != hipSuccess) {
        sd.have_shape = false;  // the copies' state is unknown: set up again next time
        if (e == hipErrorCooperativeLaunchTooLarge)
            return fail(CP_ERR_UNSUPPORTED, "persistent grid of %d workers exceeds what the device holds at once",
                        n_workers);
        return fail(CP_ERR_HIP, "worker launch: %s", hipGetErrorString(e));
    }
    const int used = sd.cur;
    sd.cur ^= 1;  // this run's workers reset the other copy
    sd.have_shape = true;
    sd.M = M;
    sd.L = n_layers;
    sd.dtype = dtype;
    sd.tile_m = tile_m;
    sd.tile_n = tile_n;
    for (int l = 0; l <= n_layers; ++l) sd.widths[l] = widths[l];
    if (status) {
        // synchronise and read the run's device status (CP_OK or CP_ERR_TIMEOUT)
        uint32_t st = 0;
        CP_HIP(hipMemcpyAsync(&st, base + ly.o_ctl[used] + (size_t)cp::kCtlStatus * 4, 4, hipMemcpyDeviceToHost, s));
        CP_HIP(hipStreamSynchronize(s));
        *status = (int32_t)st;
        if (st != 0) return fail((int)(int32_t)st, "device status %d: %s", (int)(int32_t)st,
                                 cp_chain_error_string((int)(int32_t)st));
    }
    return CP_OK;
}

}  // extern "C"
