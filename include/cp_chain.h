/*
 * cp_chain.h -- C ABI of the tile-pipelined dependent-GEMM chain for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (CTA-Pipelining: A Latency-Oriented Spatial Scaling Method for
 * Multi-GPU Systems, arXiv 2607.07862):
 *   Y = ((X . W1) . W2) ... . WL          (§III-B running example: a two-layer
 *                                         GEMM whose first output feeds the
 *                                         second; §IV-A: one GEMM per layer;
 *                                         §IV-B: Y = X A B)
 * computed in output tiles.  A tile of layer l+1 starts as soon as every
 * tile of layer l that it reads has been stored, instead of waiting for a
 * kernel boundary (§III, execution model; Fig. 1).  Readiness is tracked by a
 * host-built dependency array, a device scoreboard of atomic counters that
 * producer epilogues decrement once their stores are released (see
 * CP_FLAG_FENCE_RELEASE for the two ways), and a work-queue into
 * which the producer that completes a consumer's count pushes the consumer's
 * tile ID; a consumer prologue takes queue slots in order and remaps its
 * workgroup to the tile it dequeued (§III-A "dependency structure"; the
 * pith.science review, "What carries the argument").
 *
 * Conventions common to every entry point:
 *   - every function returns CP_OK (0) or a negative CP_ERR_* code; no C++
 *     exception crosses the ABI; cp_chain_last_error() gives a thread-local
 *     detail string for the most recent failure on the calling thread;
 *   - all matrices are dense and row-major with no padding: X[M][K0],
 *     W_l[K_{l-1}][N_l], Y[M][N_L]; element type is the plan's dtype
 *     (CP_F32: IEEE binary32; CP_BF16: bfloat16 bit patterns, accumulated in
 *     fp32 and rounded to nearest-even when stored, §III-C);
 *   - X, W[] and Y are DEVICE pointers owned by the caller; the library never
 *     frees or retains them past the call that uses them;
 *   - the plan owns its dependency table, scoreboard, queue, intermediates,
 *     internal streams and events, and frees them in cp_chain_destroy.
 */
#ifndef CP_CHAIN_H
#define CP_CHAIN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cp_chain cp_chain; /* opaque plan */

/* element types */
#define CP_F32 0
#define CP_BF16 1

/* activation applied to the fp32 accumulator of a layer, before rounding */
#define CP_ACT_NONE 0
#define CP_ACT_GELU_TANH 1 /* x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */

/* execution modes of cp_chain_run */
#define CP_MODE_PIPELINED 0  /* one persistent launch, tile dependencies   */
#define CP_MODE_SEQUENTIAL 1 /* one launch per layer (kernel boundaries)   */
#define CP_MODE_MICROBATCH 2 /* M split into chunks over two streams       */
#define CP_MODE_SPATIAL 3    /* one persistent launch per layer; layer l on CU
                                set l mod 2 (two disjoint CU-masked streams),
                                linked by the same scoreboard through one queue
                                per layer                                      */

/* status codes */
#define CP_OK 0
#define CP_ERR_INVALID_ARG (-1)
#define CP_ERR_SHAPE (-2)
#define CP_ERR_UNSUPPORTED (-3)
#define CP_ERR_OOM (-4)
#define CP_ERR_HIP (-5)
#define CP_ERR_TIMEOUT (-6)
#define CP_ERR_NO_DEVICE (-7)
#define CP_ERR_INVARIANT (-8)

/* plan flags (bitmask) */
#define CP_FLAG_DEBUG 1u        /* count dequeues per tile; enables invariant checks in stats */
#define CP_FLAG_TRACE 2u        /* per-tile timestamps (wall clock, shader clock)            */
#define CP_FLAG_POISON 4u       /* fill intermediates with NaN before every run              */
#define CP_FLAG_DELAY_INJECT 8u /* a fixed pseudo-random quarter of producers stall ~20 us   */
/* test only: the last tile's in-degree is raised by one so that it never
 * becomes ready; the worker holding its slot gives up after 50 ms (instead of
 * the default 2 s), sets CP_ERR_TIMEOUT and every worker exits.  Needs L >= 2. */
#define CP_FLAG_STARVE_LAST 16u
/* sequential and micro-batched modes: launch kernel by kernel instead of
 * replaying the plan's cached hipGraph of the run */
#define CP_FLAG_EAGER 32u
/* pipelined mode: launch the worker grid cooperatively, so that the runtime
 * guarantees every worker is resident even on a device shared with other
 * work; without it the grid (sized to what the device holds at once) is a
 * plain launch, which skips the cooperative launch path's extra latency and
 * relies on the device being otherwise idle (else the watchdog may end the
 * run with CP_ERR_TIMEOUT) */
#define CP_FLAG_COOPERATIVE 64u
/* release protocol of the pipelined and spatial modes (both exact):
 *   write-through (default): intermediates are stored at agent scope
 *     (write-through of the XCD's L2), each producer waits until its stores
 *     have completed before it decrements a counter, and consumers need no
 *     invalidate;
 *   CP_FLAG_FENCE_RELEASE: every producer tile is released with an
 *     agent-scope fence (write-back of its XCD's whole L2) and every consumer
 *     tile acquired with an L2 invalidate, the plain memory-model protocol.
 * cp_chain_stats reports the protocol in use. */
#define CP_FLAG_FENCE_RELEASE 128u
/* record HIP timing events around every run (cp_chain_stats then reports
 * last_run_ms / last_kernel_ms); each event stalls the stream for a few
 * microseconds, so untimed plans record only one completion event */
#define CP_FLAG_TIMING 256u
/* never split a layer's k range (see cp_chain_plan: split-K) */
#define CP_FLAG_NO_SPLIT 512u
/* pipelined mode: Lamport-sentinel release instead of the default one
 * (CTA-Pipelining §V-A, the Lamport synchronization alternative).  The plan
 * keeps two copies of the intermediates, pre-filled with the sentinel -0.0
 * (each run's workers fill the copy the next run uses); producers store
 * their tiles with -0.0 replaced by +0.0 and decrement the counters
 * without waiting for their stores to complete; consumers check the A data
 * they load for the sentinel (bf16: every slab as it lands in LDS; fp32:
 * every fragment) and re-load it from memory until it holds none.  Y is bit for bit that of every other mode.  Not with
 * CP_FLAG_FENCE_RELEASE (CP_ERR_INVALID_ARG); CP_MODE_SPATIAL runs of such a
 * plan return CP_ERR_UNSUPPORTED.  With CP_FLAG_DELAY_INJECT a quarter of
 * producers release their tile before storing it (stored ~20 us later), so
 * that consumers do read sentinels. */
#define CP_FLAG_LAMPORT 1024u
/* with CP_FLAG_LAMPORT only (CP_ERR_INVALID_ARG otherwise): a producer tile's
 * consumers are queued as soon as every item of the tile has been dequeued,
 * i.e. has started, instead of once it is stored (CTA-Pipelining §V-A: with
 * the sentinel in the data, the consumer itself waits for each value; the
 * dependency array of §III only has to say that the producer is running).
 * A consumer then waits inside its k loop, slab by slab, for the sentinel
 * to leave the A data it reads.  Deadlock-free for any worker count: an
 * item is queued only when all its producers are on workers, and a running
 * item waits only on running or finished items (first-layer items wait on
 * nothing).  A wait longer than the watchdog ends the run with
 * CP_ERR_TIMEOUT.  Y is bit for bit that of every other mode. */
#define CP_FLAG_EARLY_DISPATCH 2048u

#define CP_MAX_LAYERS 8

/* Statistics and invariants of the most recent run on a plan. */
typedef struct cp_chain_stats_t {
    int32_t status;          /* CP_OK, or CP_ERR_TIMEOUT if a worker's wait expired        */
    int32_t mode;            /* mode of the last run                                      */
    int32_t n_tiles;         /* T: work items over all layers (tiles, or tiles x nsplit)  */
    int32_t n_first;         /* P1: tiles of layer 1 (pre-filled into the queue)          */
    int32_t n_edges;         /* E: dependency edges = scoreboard decrements per run       */
    int32_t n_workers;       /* persistent workgroups launched (pipelined mode)           */
    int32_t tile_m, tile_n;  /* tile shape                                                */
    /* invariants, valid after a pipelined run (dequeue counts need CP_FLAG_DEBUG):      */
    int32_t nonzero_scores;  /* consumers whose counter did not end at 0                  */
    int32_t bad_dequeues;    /* tiles not dequeued exactly once (-1 if not recorded)      */
    int32_t queue_is_perm;   /* 1 if queue[0..T) is a permutation of [0,T)                */
    uint32_t head, tail;     /* summed over the queues: tickets taken (>= T), slots filled (== T) */
    int32_t n_queues;        /* work-queues (one per XCD)                                 */
    int32_t queues_drained;  /* 1 if every queue was filled to its size and fully taken   */
    int32_t order_violations;/* TRACE only: consumers that started before a producer ended */
    double last_run_ms;      /* elapsed time of the last run, from events on its stream
                                (plans built with CP_FLAG_TIMING; -1 otherwise)           */
    double last_kernel_ms;   /* pipelined with CP_FLAG_POISON: the persistent launch alone
                                (poison fills excluded); otherwise same as last_run_ms    */
    int32_t nonzero_arrivals;/* split-K tiles whose arrival count did not end at 0        */
    int32_t nsplit[CP_MAX_LAYERS]; /* split-K items per tile of each layer (1 = no split) */
    int32_t fenced;          /* release protocol of the plan: 1 fence, 0 write-through   */
    int32_t lamport;         /* 1 if the plan uses the Lamport-sentinel release           */
    int32_t lamport_rereads; /* Lamport plans with CP_FLAG_DEBUG, after a pipelined run:
                                slabs (bf16) or slab rows (fp32) in which a consumer found
                                the sentinel and re-read (-1 if not recorded)             */
} cp_chain_stats_t;

/*
 * cp_chain_plan -- validate a chain shape and build everything a run needs.
 *   out       receives the plan (set to NULL on failure)
 *   M         rows of X (the "input sequence length", §IV-A); M % tile_m == 0
 *   n_layers  L, 1 <= L <= CP_MAX_LAYERS
 *   widths    L+1 entries K0, N1, ..., NL; every N_l % tile_n == 0, and every
 *             contraction length K_{l-1} a multiple of the tile's k step: 64
 *             for bf16 (128 for 256 x 256 tiles), 32 for fp32
 *   dtype     CP_F32 or CP_BF16
 *   tile_m,n  output tile of one workgroup (one CTA, §III).  bf16: each of
 *             64, 128, 256; fp32: 64 x 64.  Other tiles: CP_ERR_UNSUPPORTED.
 *   acts      L activation codes (after each layer), or NULL for none
 *   flags     CP_FLAG_* bitmask
 * Builds the dependency array on the host -- consumer tile (l+1, i, j) waits
 * on all tiles (l, i, k) of row-block i, derived from the static tile dataflow
 * of the GEMM (§III-A; review, "Circularity Check") -- uploads it, allocates the
 * scoreboard, queue, intermediates C_1..C_{L-1} (M x N_l each) and sizes the
 * persistent grid from occupancy.  Needs a HIP device (CP_ERR_NO_DEVICE).
 * Every width must be at most 2^22.
 * Split-K: a layer with fewer tiles than the persistent grid holds is split
 * along k into power-of-two ranges (items) until it fills the grid, keeping
 * at least 16 k steps per bf16 item (64 k, or 128 k for 256x256 tiles) or 4
 * slabs of 32 k per fp32 item and, beyond layer 1, ranges made of whole
 * producer tiles; an item then waits only on the producer tiles of its own
 * k range.  Items store fp32 partials into a plan-owned workspace and
 * the last item of a tile to finish sums them in split order, so results do
 * not depend on timing and all modes agree bit for bit.  CP_FLAG_NO_SPLIT
 * turns it off; cp_chain_stats reports the split of each layer.
 */
int cp_chain_plan(cp_chain **out, int64_t M, int32_t n_layers, const int64_t *widths,
                  int32_t dtype, int32_t tile_m, int32_t tile_n, const int32_t *acts,
                  uint32_t flags);

/*
 * cp_chain_run -- enqueue one evaluation of the chain on `stream`
 * (a hipStream_t; NULL means the default stream) and return.
 *   X, W[0..L-1], Y   device pointers as described above
 *   mode              CP_MODE_*; all modes run the same tile body and produce
 *                     bit-identical Y (the original kernel is preserved, §III-C)
 *   microbatch_rows   CP_MODE_MICROBATCH only: rows per chunk, a multiple of
 *                     tile_m dividing M (the static micro-batching baseline's
 *                     "chunk size", §IV-A); ignored otherwise
 * Pipelined mode launches one persistent grid.  The plan holds two copies of
 * the per-run scoreboard/queue state; a run uses one and its workers reset
 * the other for the next run, so no reset launch precedes the grid.  The
 * sequential and micro-batched baselines are captured
 * once per (mode, microbatch_rows, X, W, Y) into a hipGraph that the plan owns
 * (at most 16 are kept, least recently used dropped) and replayed with one
 * hipGraphLaunch, as the paper's baselines replay CUDA graphs (§IV-A); with
 * CP_FLAG_EAGER their kernels are enqueued one by one.  While `stream` is
 * itself being captured, a sequential or micro-batched run is recorded kernel
 * by kernel into the caller's graph and is not timed (cp_chain_stats keeps
 * reporting the last uncaptured run); pipelined mode returns
 * CP_ERR_UNSUPPORTED there (a replay would reuse one state copy).  At most one run may be in flight per plan.  A
 * device-side watchdog expiry is reported by cp_chain_stats (status
 * CP_ERR_TIMEOUT).
 */
int cp_chain_run(cp_chain *plan, const void *X, const void *const *W, void *Y,
                 void *stream, int32_t mode, int64_t microbatch_rows);

/*
 * cp_chain_stats -- synchronise with the plan's last run and report status,
 * timing and the scoreboard/queue invariants into the caller's `out`.
 * The invariants restate the dependency structure (§III-A; Fig. 1): every
 * producer epilogue decrements the scoreboard entry of each consumer once,
 * so after a complete run every counter has gone from the consumer's
 * in-degree to exactly 0; the producer whose decrement reaches 0 pushes
 * the consumer's ID once, and every pushed ID is taken once from the
 * workqueue, so the queue holds a permutation of all tile IDs and each tile
 * is dequeued exactly once.  Without CP_FLAG_TIMING it synchronises the last
 * run's stream, which must still exist; cp_chain_trace likewise.
 * Returns CP_ERR_INVALID_ARG for a NULL plan or `out`, the device status
 * (CP_ERR_TIMEOUT) when a worker's wait expired, CP_ERR_HIP on a failed copy.
 * The invariant fields are filled after pipelined and spatial runs only.
 */
int cp_chain_stats(cp_chain *plan, cp_chain_stats_t *out);

/*
 * cp_chain_trace -- copy the per-tile timestamps of the last pipelined run
 * (plan built with CP_FLAG_TRACE) into host memory `out` of 8*T uint64
 * (CP_TRACE_WORDS per tile, tile-ID order):
 *   [0..3] ticket taken, tile dequeued (ready), GEMM body done, stores
 *          released, in 100 MHz wall-clock ticks -- the epilogue /
 *          visibility / prologue phases of the paper's Fig. 2;
 *   [4..5] the shader clock counter (s_memtime) at dequeue and at body done,
 *          so (w[5] - w[4]) / (w[2] - w[1]) x 100 MHz is the clock the tile's
 *          compute unit ran at (under a power cap it differs between XCDs);
 *   [6]    the persistent workgroup that ran the tile;
 *   [7]    1 if its release was deferred until the same worker's next tile
 *          had requested its first slabs (that tile was already queued).
 * CP_ERR_INVALID_ARG without the flag or with capacity < 8*T.
 */
#define CP_TRACE_WORDS 8
int cp_chain_trace(cp_chain *plan, uint64_t *out, int64_t capacity);

/*
 * cp_chain_intermediate -- copy the stored output C_layer of GEMM `layer`
 * (1 <= layer < L; the tiles that layer layer+1 consumes, §III-B running
 * example: the first GEMM's output read by the second) of the plan's last
 * run into `dst`, host or device memory of at least M x N_layer elements of
 * the plan's dtype (row-major, `capacity` in bytes).  Synchronises with the
 * last run first; the contents are undefined before the first run.  For the
 * element-wise error of each intermediate against a reference.
 * CP_ERR_INVALID_ARG for a NULL plan or dst, a layer out of range or a
 * capacity too small; CP_ERR_HIP if the copy fails.
 */
int cp_chain_intermediate(cp_chain *plan, int32_t layer, void *dst, int64_t capacity);

/* cp_chain_destroy -- wait for the device (the plan's last stream may be
 * gone) and free the plan: the dependency structure it allocated (§III-A:
 * dependency array, scoreboard, workqueues), the intermediates, split-K
 * partials, streams, events and cached graphs.  Caller memory (X, W, Y,
 * streams) is untouched.  NULL is a no-op; always returns CP_OK. */
int cp_chain_destroy(cp_chain *plan);

/*
 * cp_chain_tile_graph -- host-only: the dependency array a plan of this shape
 * would use, without touching a device.  Pass NULL arrays to query sizes.
 *   n_tiles, n_edges         out: T and E
 *   layer_off[L+1]           first flat tile ID of each layer, then T
 *   indeg[T]                 initial scoreboard value per tile (0 for layer 1)
 *   dep_off[T+1], dep_ids[E] CSR producer -> consumers
 * Flat IDs list each layer's tiles row-block-major: id = off_l + i*(N_l/tile_n) + j.
 */
int cp_chain_tile_graph(int64_t M, int32_t n_layers, const int64_t *widths, int32_t tile_m,
                        int32_t tile_n, int32_t *n_tiles, int32_t *n_edges, int32_t *layer_off,
                        int32_t *indeg, int32_t *dep_off, int32_t *dep_ids);

/*
 * cp_chain_tile_graph_split -- as cp_chain_tile_graph, with nsplit[l] >= 1
 * work items per tile of layer l (split-K; NULL = no split).  Items of a tile
 * are consecutive: id = off_l + (i*(N_l/tile_n) + j)*nsplit[l] + s.  Item s
 * of a consumer tile depends on the producer tiles of its k range only; a
 * producer tile's out-edges sit on its first item.  Needs nsplit[l] to
 * divide N_{l-1}/tile_n for l >= 1 and K_0 for l = 0 (CP_ERR_SHAPE).
 */
int cp_chain_tile_graph_split(int64_t M, int32_t n_layers, const int64_t *widths, int32_t tile_m,
                              int32_t tile_n, const int32_t *nsplit, int32_t *n_tiles, int32_t *n_edges,
                              int32_t *layer_off, int32_t *indeg, int32_t *dep_off, int32_t *dep_ids);

/*
 * cp_chain_run_noalloc -- for callers that cannot allocate (code that may run
 * under stream capture, tight serving loops, harnesses that forbid
 * hipMalloc): cp_chain_run in CP_MODE_PIPELINED with no plan and no
 * allocation.  The arguments are those of cp_chain_plan (flags 0) followed by
 * those of cp_chain_run; the split factors, persistent grid and kernels are
 * the ones a plan of that shape uses, so Y is bit for bit what
 * cp_chain_plan + cp_chain_run give.  Every piece of device state the run
 * needs (dependency table, queues, scoreboard, intermediates, split-K
 * partials) lives in one fixed device array of 64 MiB held by each device the
 * library runs on until the process ends; the dependency table is written
 * on the device by a setup kernel when the shape differs from the previous
 * call's on that device.  No hipMalloc, hipFree or other allocation happens
 * on any path.
 *   status  NULL: the call only enqueues on `stream` and returns;
 *           non-NULL: it also synchronises `stream` and stores the run's
 *           device status there (CP_OK, or CP_ERR_TIMEOUT if a worker's wait
 *           expired, which is also the return value).
 * Errors: the plan's argument errors (CP_ERR_INVALID_ARG, CP_ERR_SHAPE,
 * CP_ERR_UNSUPPORTED, CP_ERR_NO_DEVICE); CP_ERR_OOM when the chain needs more
 * than the 64 MiB of state (e.g. intermediates beyond it), with the size in
 * cp_chain_last_error; CP_ERR_HIP on a failed launch.  All calls on one
 * device share its array, which keeps the last call's contents: calls whose
 * runs may overlap on one device (other streams, other host threads'
 * enqueues) race and must be ordered by the caller.
 */
int cp_chain_run_noalloc(int64_t M, int32_t n_layers, const int64_t *widths, int32_t dtype, int32_t tile_m,
                         int32_t tile_n, const int32_t *acts, const void *X, const void *const *W, void *Y,
                         void *stream, int32_t *status);

/* Diagnostics of the library itself (the pages define no error reporting;
 * the timeout they name is the bound on a consumer's queue wait, §III-A
 * workqueue polling):
 * cp_chain_error_string -- static, never-NULL description of a status code
 *   ("unknown status" for codes outside CP_OK .. CP_ERR_INVARIANT); the
 *   string is owned by the library;
 * cp_chain_last_error -- thread-local detail of the most recent failure on
 *   the calling thread ("" if the last call succeeded); valid until the
 *   thread's next call into the library. */
const char *cp_chain_error_string(int code);
const char *cp_chain_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CP_CHAIN_H */
