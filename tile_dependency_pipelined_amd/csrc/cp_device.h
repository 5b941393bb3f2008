// cp_device.h -- structures shared by the host side and the kernels of the
// tile-pipelined GEMM chain.  Internal to the library (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cp {

constexpr int kMaxLayers = 8;
constexpr int kThreads = 256;              // 4 wave64 per workgroup
constexpr uint32_t kEmpty = 0xFFFFFFFFu;   // queue slot not yet filled
constexpr uint32_t kDone = 0xFFFFFFFEu;    // prologue: no more work

// Control words, each on its own 128-byte line so that the ticket counter,
// the push counter and the status flag do not share a cache line.
constexpr int kCtlHead = 0;     // next ticket (slot) to hand out
constexpr int kCtlTail = 32;    // next free queue slot for a push
constexpr int kCtlStatus = 64;  // 0 = ok, else a CP_ERR_* code
constexpr int kCtlWords = 96;

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
    int32_t ntiles;    // (M / tile_m) * nbn
};

// Everything one launch needs, passed by value as the kernel argument.
struct ChainArgs {
    LayerDesc layer[kMaxLayers];
    int32_t L;           // layers
    int32_t T;           // tiles over all layers
    uint32_t flags;      // CP_FLAG_*
    int32_t pad0;
    uint32_t *queue;     // [T] tile IDs in dequeue order (kEmpty until pushed)
    uint32_t *ctl;       // [kCtlWords] head / tail / status
    int32_t *score;      // [T] remaining producers per tile
    const int32_t *dep_off;  // [T+1] CSR producer -> consumers
    const int32_t *dep_ids;  // [E]
    const int32_t *indeg;    // [T] initial scoreboard (reset source)
    uint32_t *deq_count;     // [T] debug: dequeues per tile, or null
    uint64_t *trace;         // [4T] timestamps, or null
    uint64_t timeout_ticks;  // watchdog on a queue wait, 100 MHz ticks
};

// A compiled kernel variant (element type x tile shape).
struct Variant {
    int dtype, tile_m, tile_n, k_step;
    int lds_bytes;
    hipError_t (*launch_worker)(const ChainArgs &, int grid, hipStream_t);
    hipError_t (*launch_layer)(const ChainArgs &, int layer, int rb0, int nrb, hipStream_t);
    hipError_t (*occupancy)(int *blocks_per_cu);
};

const Variant *find_variant(int dtype, int tile_m, int tile_n);
const Variant *variant_list(int *count);

hipError_t launch_reset(const ChainArgs &a, int n_first, hipStream_t s);
hipError_t launch_poison(void *p, size_t bytes, int dtype, hipStream_t s);

}  // namespace cp
