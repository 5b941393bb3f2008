// cp_protocol_sim.cpp -- CPU model of the tile-pipelined chain's queue
// protocol, for ThreadSanitizer.  TEST INFRASTRUCTURE: built and run by
// tests/test_protocol_sim.py, never by the library.
//
// Each std::thread plays one persistent workgroup of the worker kernel and
// takes the kernel's steps in the kernel's order (CTA-Pipelining: the
// dependency structure of §III-A and the prologue / epilogue of Fig. 2):
//   first slot (static, computed with cp::first_item when the queue image
//   follows it) -> wait for a slot's tile ID -> acquire -> decode -> tile
//   body -> claim the next ticket (the scheduler lane does it during the
//   epilogue) -> split-K arrival (the last item sums the partials) -> store
//   -> publish: one decrement per out-edge in batches of 64 "lanes", ready
//   consumers claim slots of their owner queues (cp::owner_queue) with one
//   tail atomic per queue and store their IDs -> loop; on exit every worker
//   resets its share of the other per-run state copy.
// Runs are separated by joining every thread (the kernel boundary) and
// alternate between the two state copies, as consecutive launches do.  The
// dependency table is the library's own (written to a file by the test from
// cp_chain_tile_graph_split); the control-word layout, queue ownership and
// first-slot formula come from the library's cp_device.h.
//
// Memory orders.  On the GPU the release is either a per-tile agent-scope
// fence before relaxed decrements (CP_FLAG_FENCE_RELEASE) or store
// completion before relaxed decrements (write-through); the consumer
// acquires its own counter after reading the slot.  ThreadSanitizer does not
// model standalone fences, so a producer's decrements are release RMWs here
// (the counter's final value is then read by the consumer's acquire load
// through the release sequence of every producer's decrement, as with the
// fence).  Split-K arrivals are acq_rel RMWs.  Tile data and partials are
// plain memory, so any read of a producer's output that is not ordered
// after its write is a data race TSan reports.
//
// Checks after every run: status, every counter 0, every arrival count 0,
// the queue a permutation of all items, every queue filled to its size and
// fully taken, every item dequeued once, no consumer started before one of
// its producers released, and the outputs equal a sequential evaluation of
// the same integer chain (mod 2^64).  --starve raises the last item's
// in-degree by one: the run must end through the watchdog with
// CP_ERR_TIMEOUT, every worker exiting, and only that item never dequeued.
//
// --early models CP_FLAG_EARLY_DISPATCH of Lamport plans: a producer tile's
// consumers are queued once every item of the tile has been dequeued (the
// low half of the tile's arrival word counts starts, the high half
// completions), and a consumer waits, per producer tile it reads, until the
// tile is stored.  On the GPU the wait is the sentinel check and re-read of
// the data after an agent-scope acquire; here it is a per-copy "stored" word
// per tile, written with release after the tile's data and polled with
// acquire (with the watchdog) before the data is read, so TSan still reports
// any read of a tile not ordered after its write.  The order check then
// requires every consumer to start after every item of each of its producer
// tiles started, and few workers (down to one) must still finish.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "cp_device.h"

namespace {

using cp::kCtlWords;
using cp::kDone;
using cp::kEmpty;
using cp::kMaxQueues;

[[noreturn]] void die(const char *fmt, const char *a = "", long long b = 0, long long c = 0) {
    std::fprintf(stderr, "FAIL: ");
    std::fprintf(stderr, fmt, a, b, c);
    std::fprintf(stderr, "\n");
    std::exit(1);
}

struct Graph {
    int L = 0, nrb = 0, T = 0, E = 0;
    std::vector<int> nbn, nsplit, layer_off, indeg, dep_off, dep_ids;
};

Graph read_graph(const char *path) {
    FILE *f = std::fopen(path, "r");
    if (!f) die("cannot open %s", path);
    Graph g;
    auto rd = [&](int &x) {
        if (std::fscanf(f, "%d", &x) != 1) die("short graph file %s", path);
    };
    rd(g.L);
    rd(g.nrb);
    g.nbn.resize(g.L);
    g.nsplit.resize(g.L);
    g.layer_off.resize(g.L + 1);
    for (auto &x : g.nbn) rd(x);
    for (auto &x : g.nsplit) rd(x);
    for (auto &x : g.layer_off) rd(x);
    rd(g.T);
    rd(g.E);
    g.indeg.resize(g.T);
    g.dep_off.resize(g.T + 1);
    g.dep_ids.resize(g.E);
    for (auto &x : g.indeg) rd(x);
    for (auto &x : g.dep_off) rd(x);
    for (auto &x : g.dep_ids) rd(x);
    std::fclose(f);
    return g;
}

// one copy of the per-run state, as the plan allocates it twice
struct State {
    std::vector<std::atomic<uint32_t>> queue, arrive, deq, stored;
    std::vector<std::atomic<int32_t>> score;
    std::atomic<uint32_t> ctl[kCtlWords];
    std::vector<uint64_t> start_seq, release_seq;  // order check (the kernel's trace stamps)
    explicit State(int T) : queue(T), arrive(T), deq(T), stored(T), score(T), start_seq(T), release_seq(T) {}
};

struct Config {
    int nworkers = 16, nq = 8, runs = 4;
    bool spatial = false, starve = false, early = false;
    uint64_t seed = 1;
    int delay_us = 20;        // upper bound of an injected delay
    int delay_pct = 25;       // chance of a delay at each delay point
    int timeout_ms = 2000;    // watchdog on one slot wait
    // a planted mistake (tests of the simulator itself): 1 consumer load
    // relaxed instead of acquire, 2 producer decrements relaxed instead of
    // release, 3 split-K arrival relaxed, 4 exit-time reset skipped, 5 first
    // slots computed one item off, 6 (early dispatch) consumers queued when
    // the first item of a split producer tile starts, not the last
    int plant = 0;
};

struct Sim {
    Graph g;
    Config cfg;
    // queue layout (cp_chain_plan's kXcd layout, or the spatial kLayer one)
    int nq = 1;
    int32_t qbase[kMaxQueues] = {}, qsize[kMaxQueues] = {}, qfirst[kMaxQueues] = {}, qworkers[kMaxQueues] = {};
    bool first_formula = false;
    std::vector<uint32_t> qinit;
    std::vector<int> indeg;                 // in-degree template (starve: last + 1)
    std::vector<cp::LayerDesc> layer;       // tile_off, nbn, nsplit, ntiles for cp::owner_queue
    std::vector<int> worker_queue, worker_first_ticket;
    // data: C[l][i * nbn + j] outputs, P[l][item] split partials
    std::vector<std::vector<uint64_t>> C, P;
    std::atomic<uint64_t> seq{1};
    State *st[2];

    static uint64_t mix(uint64_t x) {
        x += 0x9E3779B97F4A7C15ull;
        x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
        x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
        return x ^ (x >> 31);
    }
    static uint64_t weight(int l, int k, int j) { return mix(((uint64_t)l << 48) ^ ((uint64_t)k << 24) ^ j) | 1; }

    void layout() {
        layer.resize(g.L);
        for (int l = 0; l < g.L; ++l) {
            cp::LayerDesc &d = layer[l];
            std::memset(&d, 0, sizeof d);
            d.tile_off = g.layer_off[l];
            d.nbn = g.nbn[l];
            d.nsplit = g.nsplit[l];
            d.ntiles = g.layer_off[l + 1] - g.layer_off[l];
        }
        indeg = g.indeg;
        if (cfg.starve) indeg[g.T - 1] += 1;
        qinit.assign(g.T, kEmpty);
        worker_queue.resize(cfg.nworkers);
        worker_first_ticket.resize(cfg.nworkers);
        if (!cfg.spatial) {
            nq = std::max(1, std::min(std::min(kMaxQueues, cfg.nq), cfg.nworkers));
            std::vector<std::vector<uint32_t>> first(nq);
            std::vector<int32_t> size(nq, 0);
            for (int l = 0; l < g.L; ++l)
                for (int t = g.layer_off[l]; t < g.layer_off[l + 1]; ++t) {
                    const int q = cp::owner_queue(layer[l], t, nq);
                    ++size[q];
                    if (l == 0) first[q].push_back((uint32_t)t);
                }
            int32_t base = 0;
            for (int q = 0; q < nq; ++q) {
                qbase[q] = base;
                qsize[q] = size[q];
                qfirst[q] = (int32_t)first[q].size();
                qworkers[q] = (cfg.nworkers - q + nq - 1) / nq;
                for (size_t r = 0; r < first[q].size(); ++r) qinit[base + r] = first[q][r];
                base += size[q];
            }
            first_formula = true;
            for (int q = 0; q < nq; ++q)
                for (size_t r = 0; r < first[q].size(); ++r)
                    if (cp::first_item(g.nbn[0] * g.nsplit[0], nq, q, (uint32_t)r) != first[q][r])
                        first_formula = false;
            for (int w = 0; w < cfg.nworkers; ++w) {
                worker_queue[w] = w % nq;
                worker_first_ticket[w] = w / nq;
            }
        } else {
            // one queue per layer, each served by its own group of workers
            if (g.L > kMaxQueues) die("spatial model: %s%lld layers", "", g.L);
            nq = g.L;
            for (int l = 0; l < g.L; ++l) {
                qbase[l] = g.layer_off[l];
                qsize[l] = g.layer_off[l + 1] - g.layer_off[l];
                qfirst[l] = l == 0 ? qsize[l] : 0;
            }
            for (int t = 0; t < g.layer_off[1]; ++t) qinit[t] = (uint32_t)t;
            std::vector<int> cnt(g.L, 0);
            for (int w = 0; w < cfg.nworkers; ++w) {
                const int l = w % g.L;
                worker_queue[w] = l;
                worker_first_ticket[w] = cnt[l]++;
            }
            for (int l = 0; l < g.L; ++l) qworkers[l] = cnt[l];
            first_formula = false;
        }
        C.assign(g.L, {});
        P.assign(g.L, {});
        for (int l = 0; l < g.L; ++l) {
            C[l].assign((size_t)g.nrb * g.nbn[l], 0);
            P[l].assign((size_t)(g.layer_off[l + 1] - g.layer_off[l]), 0);
        }
    }

    // per-run state reset of one copy: worker w's share (the kernel's
    // grid-stride loop), plus the control words by worker 0
    void reset_share(State &s, int w, int nw) {
        for (int t = w; t < g.T; t += nw) {
            s.score[t].store(indeg[t], std::memory_order_relaxed);
            s.queue[t].store(qinit[t], std::memory_order_relaxed);
            s.arrive[t].store(0, std::memory_order_relaxed);
            s.deq[t].store(0, std::memory_order_relaxed);
            s.stored[t].store(0, std::memory_order_relaxed);
        }
        if (w == 0) {
            for (int i = 0; i < kCtlWords; ++i) s.ctl[i].store(0, std::memory_order_relaxed);
            for (int q = 0; q < kMaxQueues; ++q) {
                s.ctl[cp::ctl_head(q)].store(q < nq ? (uint32_t)qworkers[q] : 0u, std::memory_order_relaxed);
                s.ctl[cp::ctl_tail(q)].store(q < nq ? (uint32_t)qfirst[q] : 0u, std::memory_order_relaxed);
            }
            s.ctl[cp::kCtlStatus].store(0, std::memory_order_relaxed);
        }
    }

    struct Rng {
        std::mt19937_64 r;
        int pct, us;
        void delay() {
            if ((int)(r() % 100) >= pct) return;
            const int d = (int)(r() % (uint64_t)(us + 1));
            if (d == 0) std::this_thread::yield();
            else std::this_thread::sleep_for(std::chrono::microseconds(d));
        }
    };

    uint32_t take_ticket(State &s, int q) {
        if (s.ctl[cp::kCtlStatus].load(std::memory_order_relaxed) != 0) return kDone;
        return s.ctl[cp::ctl_head(q)].fetch_add(1, std::memory_order_relaxed);
    }

    void dequeued(State &s, uint32_t id) {
        s.deq[id].fetch_add(1, std::memory_order_relaxed);
        // relaxed: the order check must not itself synchronise producer and
        // consumer; the modification order of `seq` still respects
        // happens-before (coherence), so a correct protocol gives
        // start > release on every edge
        s.start_seq[id] = seq.fetch_add(1, std::memory_order_relaxed);
    }

    uint32_t wait_slot(State &s, int q, uint32_t t) {
        if (t >= (uint32_t)qsize[q]) return kDone;
        const auto t0 = std::chrono::steady_clock::now();
        uint32_t id;
        uint32_t polls = 0;
        while ((id = s.queue[qbase[q] + t].load(std::memory_order_relaxed)) == kEmpty) {
            std::this_thread::yield();
            if ((++polls & 63) == 0) {
                if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(cfg.timeout_ms)) {
                    s.ctl[cp::kCtlStatus].store((uint32_t)cp::kStatusTimeout, std::memory_order_relaxed);
                    return kDone;
                }
                if (s.ctl[cp::kCtlStatus].load(std::memory_order_relaxed) != 0) return kDone;
            }
        }
        // consumer acquire: the counter's final value, written by the last
        // producer's decrement (release sequence of every producer's)
        if (id >= (uint32_t)layer[0].ntiles)
            (void)s.score[id].load(cfg.plant == 1 ? std::memory_order_relaxed : std::memory_order_acquire);
        dequeued(s, id);
        return id;
    }

    uint32_t first_slot(State &s, int q, uint32_t t) {
        if (!first_formula || t >= (uint32_t)qfirst[q]) return wait_slot(s, q, t);
        const uint32_t id = cp::first_item(g.nbn[0] * g.nsplit[0], nq, q, t) + (cfg.plant == 5 && t > 0 ? 1 : 0);
        dequeued(s, id);
        return id;
    }

    void decode(uint32_t id, int &l, int &i, int &j, int &split) {
        l = 0;
        while (l + 1 < g.L && (int)id >= g.layer_off[l + 1]) ++l;
        const int loc = (int)id - g.layer_off[l];
        const int tile = loc / g.nsplit[l];
        split = loc - tile * g.nsplit[l];
        i = tile / g.nbn[l];
        j = tile - i * g.nbn[l];
    }

    // early dispatch: wait until producer tile (l, i, k) is stored (the
    // sentinel check); false if the watchdog ended the run
    bool wait_stored(State &s, int l, int i, int k) {
        const uint32_t t = (uint32_t)(g.layer_off[l] + (i * g.nbn[l] + k) * g.nsplit[l]);  // its first item
        const auto t0 = std::chrono::steady_clock::now();
        uint32_t polls = 0;
        while (s.stored[t].load(std::memory_order_acquire) == 0) {
            std::this_thread::yield();
            if ((++polls & 63) == 0) {
                if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(cfg.timeout_ms)) {
                    s.ctl[cp::kCtlStatus].store((uint32_t)cp::kStatusTimeout, std::memory_order_relaxed);
                    return false;
                }
                if (s.ctl[cp::kCtlStatus].load(std::memory_order_relaxed) != 0) return false;
            }
        }
        return true;
    }

    // the tile body: item (l, i, j, split) over its k range; layer 0 reads
    // the (constant) input, later layers the producers' outputs (plain reads)
    uint64_t body(State &s, int l, int i, int j, int split) {
        if (l == 0) return mix(((uint64_t)i << 40) ^ ((uint64_t)j << 20) ^ (uint64_t)split);
        const int per = g.nbn[l - 1] / g.nsplit[l];
        uint64_t acc = 0;
        for (int k = split * per; k < (split + 1) * per; ++k) {
            if (cfg.early && !wait_stored(s, l - 1, i, k)) return 0;
            acc += C[l - 1][(size_t)i * g.nbn[l - 1] + k] * weight(l, k, j);
        }
        return acc;
    }

    // producer epilogue: one decrement per out-edge, 64 edges per batch (the
    // publisher wave's lanes); ready consumers claim slots of their owner
    // queues with one tail atomic per queue and store their IDs
    void publish(State &s, uint32_t id, int l, Rng &rng) {
        s.release_seq[id] = seq.fetch_add(1, std::memory_order_relaxed);
        const cp::LayerDesc &next = layer[l + 1];
        const int beg = g.dep_off[id], end = g.dep_off[id + 1];
        for (int e0 = beg; e0 < end; e0 += 64) {
            bool ready[64] = {};
            uint32_t c[64] = {};
            int cq[64] = {};
            bool any = false;
            for (int lane = 0; lane < 64 && e0 + lane < end; ++lane) {
                c[lane] = (uint32_t)g.dep_ids[e0 + lane];
                const int old = s.score[c[lane]].fetch_sub(
                    1, cfg.plant == 2 ? std::memory_order_relaxed : std::memory_order_release);
                ready[lane] = old == 1;
                any |= ready[lane];
                cq[lane] = cfg.spatial ? l + 1 : cp::owner_queue(next, (int)c[lane], nq);
                if (old < 1) die("counter of item %s%lld went below zero (was %lld)", "", c[lane], old);
            }
            if (!any) continue;
            rng.delay();  // between the decrements and the pushes
            uint32_t cnt[kMaxQueues] = {}, rank[64] = {}, base[kMaxQueues] = {};
            for (int lane = 0; lane < 64; ++lane)
                if (ready[lane]) rank[lane] = cnt[cq[lane]]++;
            for (int q = 0; q < nq; ++q)
                if (cnt[q]) base[q] = s.ctl[cp::ctl_tail(q)].fetch_add(cnt[q], std::memory_order_relaxed);
            for (int lane = 0; lane < 64; ++lane)
                if (ready[lane]) {
                    const uint32_t slot = base[cq[lane]] + rank[lane];
                    if (slot >= (uint32_t)qsize[cq[lane]]) die("queue %s%lld overflows at slot %lld", "", cq[lane], slot);
                    s.queue[qbase[cq[lane]] + slot].store(c[lane], std::memory_order_relaxed);
                }
        }
    }

    void worker(int w, State &s, State &nxt) {
        Rng rng{std::mt19937_64(mix(cfg.seed * 1000003ull + (uint64_t)w)), cfg.delay_pct, cfg.delay_us};
        const int q = worker_queue[w];
        uint32_t ticket = (uint32_t)worker_first_ticket[w];
        bool first = true;
        for (;;) {
            rng.delay();
            const uint32_t id = first ? first_slot(s, q, ticket) : wait_slot(s, q, ticket);
            first = false;
            if (id >= (uint32_t)g.T) break;
            int l, i, j, split;
            decode(id, l, i, j, split);
            const uint32_t first_item_id = id - (uint32_t)split;
            const int ns = g.nsplit[l];
            // early dispatch: the last item of the tile to start queues its
            // consumers (the GPU does it once its first loads are issued)
            const int shift = cfg.early && l + 1 < g.L && ns > 1 ? 16 : 0;
            if (cfg.early && l + 1 < g.L) {
                bool last_start = true;
                if (ns > 1) {
                    const uint32_t old = s.arrive[first_item_id].fetch_add(1, std::memory_order_relaxed);
                    last_start = (old & 0xFFFFu) == (uint32_t)(cfg.plant == 6 ? 0 : ns - 1);
                }
                if (last_start) publish(s, first_item_id, l, rng);
            }
            uint64_t acc = body(s, l, i, j, split);
            ticket = take_ticket(s, q);  // the scheduler lane, during the epilogue
            rng.delay();
            bool done = true;
            if (g.nsplit[l] > 1) {
                P[l][id - g.layer_off[l]] = acc;
                const uint32_t old = s.arrive[first_item_id].fetch_add(
                    1u << shift, cfg.plant == 3 ? std::memory_order_relaxed : std::memory_order_acq_rel) >> shift;
                if (old != (uint32_t)g.nsplit[l] - 1) {
                    done = false;
                } else {
                    s.arrive[first_item_id].store(0, std::memory_order_relaxed);
                    acc = 0;
                    for (int k = 0; k < g.nsplit[l]; ++k) acc += P[l][first_item_id - g.layer_off[l] + k];
                }
            }
            if (done) C[l][(size_t)i * g.nbn[l] + j] = acc;
            if (done && cfg.early) s.stored[first_item_id].store(1, std::memory_order_release);
            rng.delay();
            if (done && l + 1 < g.L && !cfg.early) publish(s, first_item_id, l, rng);
        }
        if (cfg.plant != 4) reset_share(nxt, w, cfg.nworkers);
    }

    std::vector<uint64_t> reference() {
        std::vector<std::vector<uint64_t>> R(g.L);
        for (int l = 0; l < g.L; ++l) {
            R[l].assign((size_t)g.nrb * g.nbn[l], 0);
            for (int i = 0; i < g.nrb; ++i)
                for (int j = 0; j < g.nbn[l]; ++j) {
                    uint64_t acc = 0;
                    for (int s = 0; s < g.nsplit[l]; ++s) {
                        if (l == 0) {
                            acc += mix(((uint64_t)i << 40) ^ ((uint64_t)j << 20) ^ (uint64_t)s);
                        } else {
                            const int per = g.nbn[l - 1] / g.nsplit[l];
                            for (int k = s * per; k < (s + 1) * per; ++k)
                                acc += R[l - 1][(size_t)i * g.nbn[l - 1] + k] * weight(l, k, j);
                        }
                    }
                    R[l][(size_t)i * g.nbn[l] + j] = acc;
                }
        }
        return R[g.L - 1];
    }

    int run_all() {
        State a(g.T), b(g.T);
        st[0] = &a;
        st[1] = &b;
        for (int w = 0; w < cfg.nworkers; ++w) {  // both copies start reset (the plan's reset launch)
            reset_share(a, w, cfg.nworkers);
            reset_share(b, w, cfg.nworkers);
        }
        const std::vector<uint64_t> ref = cfg.starve ? std::vector<uint64_t>() : reference();
        int cur = 0;
        for (int r = 0; r < cfg.runs; ++r) {
            State &s = *st[cur], &nxt = *st[cur ^ 1];
            for (int l = 0; l < g.L; ++l) std::fill(C[l].begin(), C[l].end(), 0xDEADull);  // poison
            std::vector<std::thread> th;
            th.reserve(cfg.nworkers);
            for (int w = 0; w < cfg.nworkers; ++w) th.emplace_back([this, w, &s, &nxt] { worker(w, s, nxt); });
            for (auto &t : th) t.join();  // the kernel boundary
            check(s, ref, r);
            cur ^= 1;
        }
        return 0;
    }

    void check(State &s, const std::vector<uint64_t> &ref, int r) {
        const uint32_t status = s.ctl[cp::kCtlStatus].load();
        uint64_t heads = 0, tails = 0;
        bool drained = true;
        for (int q = 0; q < nq; ++q) {
            const uint32_t h = s.ctl[cp::ctl_head(q)].load(), t = s.ctl[cp::ctl_tail(q)].load();
            heads += h;
            tails += t;
            if (t != (uint32_t)qsize[q] || h < (uint32_t)qsize[q]) drained = false;
        }
        int nz = 0, nza = 0, bad_deq = 0, never = -1;
        for (int t = 0; t < g.T; ++t) {
            nz += s.score[t].load() != 0;
            nza += s.arrive[t].load() != 0;
            const uint32_t d = s.deq[t].load();
            if (d != 1) {
                ++bad_deq;
                if (d == 0) never = t;
            }
        }
        std::vector<char> seen(g.T, 0);
        bool perm = true;
        for (int t = 0; t < g.T; ++t) {
            const uint32_t v = s.queue[t].load();
            if (v >= (uint32_t)g.T || seen[v]) perm = false;
            else seen[v] = 1;
        }
        if (cfg.starve) {
            if (status != (uint32_t)cp::kStatusTimeout) die("run %s%lld: expected a watchdog timeout, status %lld", "", r, status);
            if (tails != (uint64_t)g.T - 1) die("run %s%lld: %lld slots filled, expected T - 1", "", r, (long long)tails);
            if (bad_deq != 1 || never != g.T - 1) die("run %s%lld: %lld items not dequeued once (expected only the last)", "", r, bad_deq);
            std::printf("run %d: starved item %d timed out, all %d workers exited, %" PRIu64 " slots filled\n", r,
                        g.T - 1, cfg.nworkers, tails);
            return;
        }
        if (status != 0) die("run %s%lld: device status %lld", "", r, (int32_t)status);
        if (nz) die("run %s%lld: %lld counters not at 0", "", r, nz);
        if (nza) die("run %s%lld: %lld arrival counts not at 0", "", r, nza);
        if (!perm) die("run %s%lld: queue is not a permutation of the items", "", r);
        if (!drained || tails != (uint64_t)g.T) die("run %s%lld: queues not drained (%lld slots filled)", "", r, (long long)tails);
        if (bad_deq) die("run %s%lld: %lld items not dequeued exactly once", "", r, bad_deq);
        int viol = 0;
        for (int p = 0; p < g.T; ++p)
            for (int e = g.dep_off[p]; e < g.dep_off[p + 1]; ++e) {
                if (!cfg.early) {
                    viol += s.start_seq[g.dep_ids[e]] < s.release_seq[p];
                } else {
                    // every item of producer tile p (p is its first item) started first
                    int l = 0;
                    while (l + 1 < g.L && p >= g.layer_off[l + 1]) ++l;
                    for (int k = 0; k < g.nsplit[l]; ++k) viol += s.start_seq[g.dep_ids[e]] < s.start_seq[p + k];
                }
            }
        if (viol)
            die(cfg.early ? "run %s%lld: %lld consumers started before a producer item started"
                          : "run %s%lld: %lld consumers started before a producer released", "", r, viol);
        const std::vector<uint64_t> &y = C[g.L - 1];
        for (size_t k = 0; k < y.size(); ++k)
            if (y[k] != ref[k]) die("run %s%lld: output element %lld differs from the sequential chain", "", r, (long long)k);
        std::printf("run %d: ok, %d items, %d edges, %d workers, %d queues, heads %" PRIu64 "\n", r, g.T, g.E,
                    cfg.nworkers, nq, heads);
    }
};

}  // namespace

int main(int argc, char **argv) {
    if (argc < 2) {
        std::fprintf(stderr, "usage: %s GRAPH [--workers N] [--queues N] [--runs N] [--seed S] [--delay-us D] "
                             "[--delay-pct P] [--spatial] [--starve] [--early] [--timeout-ms T]\n", argv[0]);
        return 2;
    }
    Sim sim;
    sim.g = read_graph(argv[1]);
    for (int a = 2; a < argc; ++a) {
        const std::string k = argv[a];
        auto val = [&]() -> long long {
            if (a + 1 >= argc) die("missing value for %s", k.c_str());
            return std::atoll(argv[++a]);
        };
        if (k == "--workers") sim.cfg.nworkers = (int)val();
        else if (k == "--queues") sim.cfg.nq = (int)val();
        else if (k == "--runs") sim.cfg.runs = (int)val();
        else if (k == "--seed") sim.cfg.seed = (uint64_t)val();
        else if (k == "--delay-us") sim.cfg.delay_us = (int)val();
        else if (k == "--delay-pct") sim.cfg.delay_pct = (int)val();
        else if (k == "--timeout-ms") sim.cfg.timeout_ms = (int)val();
        else if (k == "--spatial") sim.cfg.spatial = true;
        else if (k == "--starve") sim.cfg.starve = true;
        else if (k == "--early") sim.cfg.early = true;
        else if (k == "--plant") sim.cfg.plant = (int)val();
        else die("unknown option %s", k.c_str());
    }
    if (sim.cfg.nworkers < 1 || (sim.cfg.spatial && sim.cfg.nworkers < sim.g.L)) die("too few workers%s", "");
    sim.layout();
    return sim.run_all();
}
