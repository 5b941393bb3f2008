// cp_device.h -- structures shared by the host side and the kernels of the
// tile-pipelined GEMM chain.  Internal to the library (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cp_chain.h"

namespace cp {

constexpr int kMaxLayers = 8;
constexpr int kThreads = 256;              // 4 wave64 per workgroup
constexpr uint32_t kEmpty = 0xFFFFFFFFu;   // queue slot not yet filled
constexpr uint32_t kDone = 0xFFFFFFFEu;    // prologue: no more work

// Work-queues.  The paper keeps one workqueue per consumer device; here the
// unit with a private cache is the XCD (8 per MI355X, each with its own L2),
// so there is one queue per XCD.  A tile belongs to the queue of its column
// panel (j mod nq): the weight panel it reads then stays in one XCD's L2.
constexpr int kMaxQueues = 8;
// trace words per tile: ticket taken, dequeued, body done, released (100 MHz
// wall clock), then the shader clock counter at dequeue and at body done
constexpr int kTraceWords = CP_TRACE_WORDS;

// Control words, each on its own 128-byte line: per queue a ticket counter
// (head) and a push counter (tail), then the run status.
constexpr int kCtlLine = 32;                               // words per line
__host__ __device__ constexpr int ctl_head(int q) { return (2 * q) * kCtlLine; }
__host__ __device__ constexpr int ctl_tail(int q) { return (2 * q + 1) * kCtlLine; }
constexpr int kCtlStatus = 2 * kMaxQueues * kCtlLine;      // 0 = ok, else a CP_ERR_* code
constexpr int kCtlRereads = kCtlStatus + 1;                // Lamport debug: sentinel re-reads
constexpr int kCtlWords = kCtlStatus + kCtlLine;

constexpr int32_t kStatusTimeout = -6;  // == CP_ERR_TIMEOUT

// One GEMM of the chain: C[M][N] = act(A[M][K] . W[K][N]), row-major.
struct LayerDesc {
    const void *A;
    const void *W;
    void *C;
    int32_t K, N;
    int32_t nbn;       // N / tile_n: tiles per row-block
    int32_t act;       // CP_ACT_*
    int32_t tile_off;  // flat ID of this layer's first tile
    int32_t ntiles;    // work items of this layer: (M / tile_m) * nbn * nsplit
    int32_t coherent;  // store C at agent scope (write-through of the XCD's L2)
    int32_t nsplit;    // split-K: items per output tile (1 = no split); item s of a
                       // tile covers k in [s K / nsplit, (s + 1) K / nsplit)
    float *ws;         // nsplit > 1: fp32 partial tiles, one per item
    // Lamport-sentinel release (CP_FLAG_LAMPORT, pipelined mode):
    int32_t lam_out;   // C is an intermediate pre-filled with the sentinel -0.0: stored
                       // values have -0.0 replaced by +0.0, and the release does not wait
                       // for the stores to complete
    int32_t lam_in;    // A is such an intermediate: every A fragment is checked for the
                       // sentinel before use and re-read from memory until it holds none
    // Split-K arrival counter of a tile (nsplit > 1): an item's completion adds
    // 1 << arrive_shift, and the item that sees nsplit - 1 earlier completions
    // is the last.  16 with CP_FLAG_EARLY_DISPATCH when the tile has in-run
    // consumers: the low 16 bits then count the tile's items as they are
    // dequeued (the one that sees nsplit - 1 earlier starts queues the
    // consumers), the high 16 bits their completions.
    int32_t arrive_shift;
};

// Everything one launch needs, passed by value as the kernel argument.
struct ChainArgs {
    LayerDesc layer[kMaxLayers];
    int32_t L;           // layers
    int32_t T;           // tiles over all layers
    uint32_t flags;      // CP_FLAG_*
    int32_t nq;          // queues in use (1..kMaxQueues)
    int32_t nworkers;    // persistent workers (grid size)
    int32_t fixed_queue;     // >= 0: every worker of this launch serves that queue (spatial
                             // mode), else worker b serves queue b mod nq
    int32_t queue_by_layer;  // 1: a tile's queue is its layer (spatial); 0: column panel mod nq
    int32_t qworkers[kMaxQueues];  // workers serving each queue; they own its first slots
    int32_t qbase[kMaxQueues];   // first slot of each queue in `queue`
    int32_t qsize[kMaxQueues];   // tiles owned by each queue
    int32_t qfirst[kMaxQueues];  // of which first-layer tiles (pre-filled)
    int32_t first_formula;   // 1: slot r < qfirst[q] of queue q holds first_item(q, r), so a
                             // worker's static first slot needs no queue read (checked at plan)
    uint32_t *queue;     // [T] slots of all queues (kEmpty until pushed)
    uint32_t *ctl;       // [kCtlWords] per-queue head / tail, status
    int32_t *score;      // [T] remaining producers per tile
    const int32_t *dep_off;  // [T+1] CSR producer -> consumers
    const int32_t *dep_ids;  // [E]
    const int32_t *indeg;    // [T] initial scoreboard (reset source)
    const uint32_t *qinit;   // [T] initial queue contents (reset source)
    uint32_t *deq_count;     // [T] debug: dequeues per tile, or null
    uint64_t *trace;         // [kTraceWords T] timestamps, or null
    uint32_t *arrive;        // [T] split-K: items of a tile that finished (at its first item's
                             // index); the last one sums the partials and resets it to 0
    // the other copy of the per-run state (queue, ctl, score, deq_count,
    // trace), used by the next pipelined run; this run's workers reset it
    uint32_t *nxt_queue, *nxt_ctl;
    int32_t *nxt_score;
    uint32_t *nxt_deq_count;
    uint32_t *nxt_arrive;
    uint64_t *nxt_trace;
    uint64_t timeout_ticks;  // watchdog on a queue wait, 100 MHz ticks
    // Lamport plans: the other copy of the intermediates, which this run's
    // workers fill with the sentinel for the next run (null: nothing to fill)
    void *lam_fill[kMaxLayers];
    uint64_t lam_fill_bytes[kMaxLayers];  // multiples of 16
    uint32_t lam_pattern;                 // sentinel word: two bf16 -0.0, or fp32 -0.0
};

// Queue that owns work item `id` of layer `l`: (column panel x nsplit +
// split) modulo nq, so the items of one tile spread over the queues.
__host__ __device__ inline int owner_queue(const LayerDesc &d, int id, int nq) {
    return ((id - d.tile_off) % (d.nbn * d.nsplit)) % nq;
}

// The r-th pre-filled (first-layer) item of queue q, r < qfirst[q]: the
// queue image lists, row-block by row-block, the items whose position in
// the row-block (column panel x nsplit + split, `per` of them) is q modulo
// nq.  Row-block i holds ceil((per - q) / nq) of them.
__host__ __device__ inline uint32_t first_item(int per, int nq, int q, uint32_t r) {
    const uint32_t in_rb = (uint32_t)((per - q + nq - 1) / nq);
    const uint32_t i = r / in_rb, k = r - i * in_rb;
    return i * (uint32_t)per + (uint32_t)q + k * (uint32_t)nq;
}

// Closed-form description of a chain's tile graph and queue layout, from
// which a device kernel writes the dependency table, the queue image and
// both per-run state copies (the allocation-free entry point builds no host
// tables).  The table is the one the host builder makes.
struct GraphDims {
    int32_t L;
    int32_t nrb;                   // row-blocks
    int32_t nbn[kMaxLayers];       // tiles per row-block of each layer
    int32_t nsplit[kMaxLayers];    // items per tile of each layer
    int32_t layer_off[kMaxLayers + 1];  // first item of each layer, then T
    int32_t edge_off[kMaxLayers + 1];   // first edge of each layer's producers, then E
    int32_t T, E;
};

// A compiled kernel variant (element type x tile shape).
struct Variant {
    int dtype, tile_m, tile_n, k_step;
    int lds_bytes;
    hipError_t (*launch_worker)(const ChainArgs &, int grid, bool cooperative, hipStream_t);
    hipError_t (*launch_layer)(const ChainArgs &, int layer, int rb0, int nrb, hipStream_t);
    // workgroups of the persistent worker per compute unit, smallest over the
    // instantiations a plan may launch (with or without split-K; Lamport or not)
    hipError_t (*occupancy)(int *blocks_per_cu, bool lamport);
};

const Variant *find_variant(int dtype, int tile_m, int tile_n);
const Variant *variant_list(int *count);

hipError_t launch_reset(const ChainArgs &a, hipStream_t s);
// Writes indeg, dep_off, dep_ids and qinit of `a` from `g`, and resets both
// per-run state copies (a.queue/ctl/score/arrive and a.nxt_*).
hipError_t launch_graph_setup(const ChainArgs &a, const GraphDims &g, hipStream_t s);
hipError_t launch_poison(void *p, size_t bytes, int dtype, hipStream_t s);
// Fill with a 32-bit pattern (the Lamport sentinel), written through to memory.
hipError_t launch_fill(void *p, size_t bytes, uint32_t pattern, hipStream_t s);
// Sentinel word of the Lamport release for an element type: -0.0 in every element.
constexpr uint32_t lamport_pattern(int dtype) { return dtype == CP_BF16 ? 0x80008000u : 0x80000000u; }

}  // namespace cp
