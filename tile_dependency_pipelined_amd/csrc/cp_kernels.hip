// cp_kernels.hip -- device code of the tile-pipelined GEMM chain for gfx950.
//
// Method: CTA-Pipelining: A Latency-Oriented Spatial Scaling Method for
// Multi-GPU Systems (arXiv 2607.07862).  A workgroup plays the role of the
// paper's CTA: it consumes input tiles and produces exactly one output tile
// (§III, execution model).  The GEMM tile body is left unchanged; only a
// prologue (take a queue slot, wait until it holds a ready tile ID, remap the
// workgroup to that tile) and an epilogue (store, release, decrement the
// scoreboard of every consumer, push consumers that became ready) are added
// around it (§III-A "dependency structure"; §III-C; Fig. 2).  The same body is
// launched without prologue/epilogue for the sequential and micro-batched
// baselines, so all modes produce bit-identical results.
//
// gfx950 mapping (MI355X): 4 wave64 per workgroup (8 for 256 x 256 tiles);
// bf16 tiles use fp32-accumulating MFMAs, v_mfma_f32_16x16x32_bf16 for
// 256 x 256 tiles and v_mfma_f32_32x32x16_bf16 for the others; fp32 tiles
// v_mfma_f32_32x32x2_f32.  The paper's system-wide threadfence becomes, on
// one GPU, agent scope: by default the producer writes intermediate tiles
// with agent-scope (L2 write-through) stores and waits for their completion
// before it touches a counter; with CP_FLAG_FENCE_RELEASE it is one
// agent-scope release fence per tile (write-back of the XCD-private L2) and
// the consumer's read of its counter an agent-scope acquire.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "cp_chain.h"
#include "cp_device.h"

namespace cp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// ----------------------------------------------------------------------------
// Element conversion and activation (applied to the fp32 accumulator).
// ----------------------------------------------------------------------------

// fp32 -> bf16, round to nearest even (inputs here are finite; NaN is kept NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float act_apply(float x, int act) {
    if (act == CP_ACT_GELU_TANH) {
        // x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
        const float k0 = 0.7978845608028654f;
        float u = k0 * (x + 0.044715f * x * x * x);
        return 0.5f * x * (1.0f + tanhf(u));
    }
    return x;
}

// wait until at most N vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int U>
using ic = std::integral_constant<int, U>;

// Lamport-sentinel checks.  A bf16 word holds two elements; either one equal
// to the sentinel -0.0 (0x8000) marks data not yet stored in this run.
__device__ __forceinline__ uint32_t has_sentinel_bf16x2(uint32_t w) {
    return ((w & 0xFFFFu) == 0x8000u) | ((w >> 16) == 0x8000u);
}
__device__ __forceinline__ uint32_t has_sentinel_f32(float f) { return __float_as_uint(f) == 0x80000000u; }

// Where a Lamport consumer reports a sentinel wait that exceeded the watchdog.
struct LamWatch {
    uint32_t *status;   // the run's status word, or null (baseline launches)
    uint64_t timeout;   // 100 MHz ticks
    uint32_t *rereads;  // CP_FLAG_DEBUG: count of fragments that found the sentinel, or null
};

// Re-read loop of a Lamport consumer: `n` 8-byte words at `src` (device
// memory another XCD stores into), re-read after an agent-scope acquire
// (which invalidates this XCD's L2, so a line read while it still held the
// sentinel is not served again) until `clean` holds for every lane, or the
// watchdog expires (the run's status becomes CP_ERR_TIMEOUT).
template <int N, class Clean>
__device__ __forceinline__ void lamport_reread(const uint64_t *src, uint64_t (&v)[N], const LamWatch &w,
                                            Clean &&clean) {
    const uint64_t t0 = wall_clock64();
    if (w.rereads && (threadIdx.x & 63) == 0)
        __hip_atomic_fetch_add(w.rereads, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t naps = 1;  // back-off, as in the bf16 re-load rounds
    for (;;) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
        for (int e = 0; e < N; ++e) v[e] = __hip_atomic_load(src + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!__ballot(!clean(v))) return;
        if (wall_clock64() - t0 > w.timeout) {
            if (w.status)
                __hip_atomic_store(w.status, (uint32_t)kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        for (uint32_t n = 0; n < naps; ++n) __builtin_amdgcn_s_sleep(8);
        if (naps < 16) ++naps;
    }
}

// A pointer every lane holds the same value of, in scalar registers (an
// out-of-line function receives its arguments in vector registers).  The
// builtin returns a signed int: each half goes through uint32_t before it is
// widened, or a low half with bit 31 set would fill the high half with ones.
template <class T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<T *>(((uint64_t)hi << 32) | lo);
}

// Fourth word of a raw (stride 0) buffer resource on gfx9-family parts:
// 32-bit data format, so untyped dword loads are in range.
constexpr int kRsrcWord3 = 0x00020000;

// 16-byte direct load (buffer_load_dwordx4 ... lds): each lane's 16 bytes at
// byte `voff` of the resource go to LDS at `lds` + 16 * lane (`lds`
// wave-uniform).  Inline asm, so that the compiler's wait insertion does not
// track it: the compiler cannot tell which LDS array a direct load writes,
// and before every later LDS read it waits for ALL direct loads in flight,
// which leaves a multi-stage pipeline one slab in flight.  Every read of
// data loaded this way therefore follows an explicit wait_vmcnt (and a
// barrier where other waves loaded it).  The asm writes no VGPR (the data
// goes to LDS) and restores M0, which the compiler does not let an asm
// clobber; the compiler's own waits for its loads only get stricter, since
// these count in vmcnt too.  The memory clobber keeps LDS reads on their
// side of it (the compiler does not otherwise know that it writes LDS).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const void *lds, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t *)lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0), "v"(voff), "s"(r)
        : "memory");
}

// Four LDS words of a Lamport consumer: flags of the last three slabs'
// checks and of a re-load round (zeroed at worker start and after each tile).
__device__ __forceinline__ uint32_t *lamport_flags() {
    __shared__ uint32_t flags[4];
    return flags;
}

// ----------------------------------------------------------------------------
// bf16 tile body: C[BM x BN] tile (i, j) of A[M][K] . W[K][N], slabs of BK
// (32 or 64) k, S-stage LDS pipeline.
//
// Both operands travel HBM -> LDS by 16-byte direct loads (global_load_lds):
// lane l of a load lands at LDS base + 16 l, so no VGPR staging and no LDS
// store instructions are needed; the swizzle below is applied by choosing
// which global 16-byte chunk each lane fetches.
//   A tile [BM][BK] bf16.  BK = 64: 128-byte rows, chunk c of row r stored at
//     chunk position c ^ fa(r).  BK = 32: rows 2L and 2L+1 share the
//     128-byte line L, chunk c of row r at position (4 (r & 1) + c) ^ fl(L),
//     fl(L) = (L ^ (L >> 2)) & 3.  The MFMA A fragment (8 consecutive k of
//     one row) is one ds_read_b128, and a 128-bit LDS read is served in
//     pairs of 8-lane groups, lanes l .. l+7 with lanes l+32 .. l+39 (these
//     16 reads must fall on distinct 16-byte bank groups of a 256-byte
//     window), as well as in plain 16-lane groups.  With 32x32x16 blocks,
//     lanes l and l+32 read chunks c and c+1 of one row; fa(r) =
//     (r ^ (r >> 3)) & 7 keeps both groupings conflict-free.  With 16x16x32
//     blocks they read chunks c and c+2, where that fa collides; there
//     fa(r) = r1 | r3 << 1 | r2 << 2 (ri = bit i of r) is conflict-free in
//     both groupings.
//   W tile [64][BN] bf16 in its natural n-contiguous layout, chunk c of row k
//     stored at c ^ fb(k), fb = {0, 6, 10, 12}[k mod 4] (BN >= 128): the 4
//     rows x 2 chunks read by 16 lanes are distinct modulo 128 bytes and the
//     4 rows x 4 chunks read by 32 lanes distinct modulo 256 bytes.  With
//     16x16x32 blocks, 32 lanes read rows k .. k+3 and k+8 .. k+11 x 2
//     chunks; there fb also flips chunk bit 1 with bit 3 of k, which keeps
//     those 16 chunks distinct modulo 256 bytes.
//     The B fragment (8 consecutive k of one column)
//     is read by two ds_read_b64_tr_b16: within a group of 16 lanes, result
//     lane i, element j is element (i mod 4) of the 8 bytes addressed by lane
//     4 j + i / 4, so lane s addresses row k0 + s/4, columns n0 + 4 (s mod 4)
//     and lane i receives W[k0 .. k0+3][n0 + i].
// Pipeline: S-1 slabs are in flight while one is multiplied; a stage is
// refilled as soon as every wave holds the fragments of its last k step.
// Every stage is its own __shared__ array and every stage index a
// compile-time constant (no dynamic LDS addressing).  With more than two
// stages the direct loads are hidden from the compiler's wait insertion
// (dma16), so the explicit waits below alone decide how many slabs stay in
// flight.  Past the last slab the prefetch re-reads the last slab into a
// stage that is no longer read, which keeps the number of loads in flight,
// and so the wait, constant.
// ----------------------------------------------------------------------------
template <int BM_, int BN_, int S_, int WGM_ = 2, int WGN_ = 2, int BK_ = 64, int MI_ = 32>
struct Bf16Body {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_;
    static constexpr int WGM = WGM_, WGN = WGN_;     // wave grid
    static constexpr int NW = WGM * WGN, NT = 64 * NW;
    static constexpr int WM = BM / WGM, WN = BN / WGN;  // per-wave sub-tile
    // MFMA block: MI = 32 is v_mfma_f32_32x32x16_bf16 (16 k per step, 16
    // accumulators per lane), MI = 16 is v_mfma_f32_16x16x32_bf16 (32 k per
    // step, 4 accumulators per lane: half the accumulator traffic per flop)
    static constexpr int MI = MI_;
    static constexpr int KM = MI == 32 ? 16 : 32;    // k per MFMA step
    static constexpr int ACC = MI * MI / 64;         // fp32 accumulators per lane per block
    static constexpr int FM = WM / MI, FN = WN / MI; // MFMA blocks per wave
    // k granularity the plan guarantees per item (its k step): one slab, or
    // for the 16x16x32 body S slabs, so that its k loop needs no remainder
    // step (a remainder keeps the loop's addresses live past it, which the
    // persistent worker of that body can only afford by spilling them)
    static constexpr int KQ = MI == 16 ? BK * S : BK;
    static constexpr int RB = BN * 2;                // bytes per W row in LDS
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * RB;
    static constexpr int A_PW = A_BYTES / 1024 / NW;  // 1 KiB direct loads per wave (A)
    static constexpr int B_PW = B_BYTES / 1024 / NW;  // (W)
    static constexpr int PER = A_PW + B_PW;          // loads per wave per slab
    static constexpr int STAGE = A_BYTES + B_BYTES;  // bytes of one LDS stage
    // Direct loads through dma16 where more than one slab is meant to be in
    // flight; with one (two stages) the compiler's own waits are the
    // pipeline's, and the builtin leaves it more freedom to schedule.
    static constexpr bool ASM_DMA = S > 2;
    __device__ __forceinline__ static void dma(__amdgpu_buffer_rsrc_t r, char *lds, uint32_t voff) {
        if constexpr (ASM_DMA) dma16(r, lds, voff);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds, 16, voff, 0, 0, 0);
    }
    static_assert(BM >= 64 && BN >= 64 && BM <= 256 && BN <= 256, "tile");
    static_assert(MI == 32 || MI == 16, "MFMA block");
    static_assert(WM >= 32 && WN >= 32 && WM % 32 == 0 && WN % 32 == 0, "wave sub-tile");
    static_assert(A_PW >= 1 && B_PW >= 1 && A_PW * NW * 1024 == A_BYTES && B_PW * NW * 1024 == B_BYTES,
                  "loads per wave");
    static_assert(BK == 32 || BK == 64, "k slab");
    static_assert(S >= 2 && S <= 5 && (S - 1) * PER < 64, "stages");

    // A swizzle for BK = 64 (header comment): chunk position of chunk 0 of row r
    __device__ static int fa(int r) {
        if constexpr (MI == 32) return (r ^ (r >> 3)) & 7;
        else return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r >> 2) & 1) << 2);
    }
    // byte offset of 16-byte chunk c (0 .. BK/8-1) of A row r within the A tile
    __device__ static int a_at(int r, int c) {
        if constexpr (BK == 64) return r * 128 + ((c ^ fa(r)) << 4);
        else {
            const int L = r >> 1;
            return L * 128 + ((((r & 1) << 2 | c) ^ ((L ^ (L >> 2)) & 3)) << 4);
        }
    }
    // W swizzle.  The 16x16x32 B fragment reads rows k, k+8, k+16, k+24 (+0..3)
    // in one instruction, so there bit 3 of k also moves the chunk.
    __device__ static int fb(int k) {
        if constexpr (MI == 32) {
            if constexpr (BN >= 128) return (0xCA60 >> ((k & 3) * 4)) & 15;  // 0, 6, 10, 12
            else return (k & 3) << 1;
        } else {
            if constexpr (BN >= 128) return ((0xCA60 >> ((k & 3) * 4)) & 15) ^ (((k >> 3) & 1) << 1);
            else return ((k & 3) << 1) ^ ((k >> 3) & 1);  // stays below 8 chunks
        }
    }

    // The rare path of a bf16 Lamport consumer (every thread of the workgroup):
    // some wave found the sentinel in the A part of the slab at `src` (bytes
    // from the tile's first A row, `bytes` in range).  Each wave re-loads the A
    // chunks it loads into LDS `As`, after an agent-scope acquire (which drops
    // lines this XCD read while they still held the sentinel), and checks them
    // again, until no wave finds a sentinel; three barriers per round, so that
    // the vote word (flags[3]) is cleared before any wave marks it and read by
    // every wave before it is cleared.  The watchdog is a round count, the same
    // in every wave, so that all leave together.  Out of line: none of its
    // state is live in the k loop.
    struct LaneOffsets {
        uint32_t v[A_PW];
    };
    __device__ __noinline__ static void lamport_reload_slab(char *As, char *src, uint32_t bytes, LaneOffsets a_off,
                                                            LamWatch lw) {
        uint32_t *lflag = lamport_flags();
        const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const uint64_t rounds = lw.timeout / 100 + 1;  // a round takes well over 1 us
        if (lw.rereads && tid == 0) __hip_atomic_fetch_add(lw.rereads, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (uint64_t round = 0;; ++round) {
            __syncthreads();  // every wave has read the flags
            if (tid == 0) lflag[3] = 0u;
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
                uniform_ptr(src), 0, (int)__builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
#pragma unroll
            for (int q = 0; q < A_PW; ++q) dma(ra, As + (q * NW + wave) * 1024, a_off.v[q]);
            wait_vmcnt<0>();
            __syncthreads();  // lflag[3] cleared before any wave marks it
            uint32_t bad = 0;
#pragma unroll
            for (int q = 0; q < A_PW; ++q) {
                const uint4 v = *reinterpret_cast<const uint4 *>(As + (q * NW + wave) * 1024 + lane * 16);
                bad |= has_sentinel_bf16x2(v.x) | has_sentinel_bf16x2(v.y) | has_sentinel_bf16x2(v.z) |
                       has_sentinel_bf16x2(v.w);
            }
            if (__ballot(bad) != 0 && lane == 0) lflag[3] = 1u;
            __syncthreads();
            if (__builtin_amdgcn_readfirstlane(lflag[3]) == 0) break;
            if (round >= rounds) {
                if (lw.status && tid == 0)
                    __hip_atomic_store(lw.status, (uint32_t)kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            // back off: every round's acquire invalidates this XCD's L2 under
            // the workgroups still computing; a consumer started before its
            // producers finished (early dispatch) may wait a whole tile here
            const uint64_t naps = round < 16 ? round + 1 : 16;
            for (uint64_t n = 0; n < naps; ++n) __builtin_amdgcn_s_sleep(8);
        }
        __syncthreads();
    }

    // `before_epilogue` runs in every thread once the main loop is done (the
    // worker takes its next ticket there).  Split-K (d.nsplit > 1): this
    // item multiplies k in [split K / nsplit, (split + 1) K / nsplit) and
    // stores an fp32 partial; the last item of the tile to arrive sums all
    // partials in split order and runs the epilogue.  Returns whether this
    // call completed the tile (stored C).
    // SPLIT = false compiles the split-K path out (plans without a split
    // layer use that instantiation: the extra live state would cost the
    // persistent worker its scalar registers).
    //
    // LAM (Lamport consumer, d.lam_in): every A fragment is checked for the
    // sentinel before the MFMAs that use it; a wave that finds one re-reads
    // that step's A fragments from memory (lamport_reread), leaving the LDS
    // copy alone, so the product never sees a sentinel and the result is
    // the same bits as in every other mode.  `before_store` runs in every
    // thread right before the tile's global stores.
    // `after_issue` runs in every thread once the tile's first slabs are
    // requested, while they are in flight (the worker releases a previous
    // tile there).
    template <bool SPLIT, bool LAM, class Hook, class StoreHook, class IssueHook>
    __device__ __forceinline__ static bool run(const LayerDesc &d, int i, int j, int split, uint32_t *arrive,
                                               char *const *stg, Hook &&before_epilogue, StoreHook &&before_store,
                                               IssueHook &&after_issue, const LamWatch &lw) {
        const uint16_t *__restrict__ A = static_cast<const uint16_t *>(d.A);
        const uint16_t *__restrict__ W = static_cast<const uint16_t *>(d.W);
        uint16_t *__restrict__ C = static_cast<uint16_t *>(d.C);
        const int K = d.K, N = d.N;
        const int row0 = i * BM, col0 = j * BN;
        // Per-lane addresses derive from tid; the empty asm makes them
        // opaque to the compiler, so a persistent worker recomputes them per
        // tile instead of keeping them live across its tile loop (which
        // would exceed the register budget and spill).
        int tid = threadIdx.x;
        __asm__ volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wave / WGN, wn = wave % WGN;

        using AccT = std::conditional_t<MI == 32, f32x16_t, f32x4_t>;
        AccT acc[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int r = 0; r < ACC; ++r) acc[fm][fn][r] = 0.0f;

        // per-lane source offsets (elements) of this wave's direct loads
        // Direct loads are buffer loads: a wave-uniform buffer resource (in
        // SGPRs; base = the tile's first A row, or W row k0, advanced per
        // slab, size = the bytes the slab may touch) plus a 32-bit per-lane
        // byte offset that is fixed for the whole tile.  No 64-bit per-lane
        // address arithmetic, half the address registers, and a lane outside
        // the resource reads zeros instead of faulting.  Offsets stay below
        // 2^32 because rows are at most 2^22 elements (checked at plan time).
        uint32_t a_off[A_PW], b_off[B_PW];
#pragma unroll
        for (int q = 0; q < A_PW; ++q) {
            const int o = (q * NW + wave) * 1024 + lane * 16;  // byte in the A region
            int r, c;
            if constexpr (BK == 64) {
                r = o >> 7;
                c = ((o >> 4) & 7) ^ fa(r);
            } else {  // inverse of a_at for 64-byte rows
                const int L = o >> 7, v = ((o >> 4) & 7) ^ ((L ^ (L >> 2)) & 3);
                r = 2 * L + (v >> 2);
                c = v & 3;
            }
            a_off[q] = (uint32_t)r * (uint32_t)K * 2u + (uint32_t)c * 16u;
        }
#pragma unroll
        for (int q = 0; q < B_PW; ++q) {
            const int o = (q * NW + wave) * 1024 + lane * 16;  // byte in the W region
            const int k = o / RB, c = ((o % RB) >> 4) ^ fb(o / RB);
            b_off[q] = (uint32_t)k * (uint32_t)N * 2u + (uint32_t)c * 16u;
        }
        // this item's k range; integer division runs on the vector ALU, so
        // say that the results are uniform (they feed the buffer resources)
        const int kspan = SPLIT ? __builtin_amdgcn_readfirstlane(K / d.nsplit) : K;
        const int kbeg = SPLIT ? __builtin_amdgcn_readfirstlane(split * kspan) : 0;
        char *const a_base = reinterpret_cast<char *>(const_cast<uint16_t *>(A) + (size_t)row0 * K + kbeg);
        char *const w_base = reinterpret_cast<char *>(const_cast<uint16_t *>(W) + (size_t)kbeg * N + col0);
        const uint32_t a_bytes = (uint32_t)BM * (uint32_t)K * 2u - 2u * kbeg;  // the tile's A rows from kbeg
        const uint32_t w_bytes = (uint32_t)(BK - 1) * (uint32_t)N * 2u + BN * 2u;  // one W slab

        auto issue = [&](char *As, int k0) {
            char *Bs = As + A_BYTES;
            const __amdgpu_buffer_rsrc_t ra =
                __builtin_amdgcn_make_buffer_rsrc(a_base + (size_t)k0 * 2, 0, (int)(a_bytes - 2u * k0), kRsrcWord3);
#pragma unroll
            for (int q = 0; q < A_PW; ++q) dma(ra, As + (q * NW + wave) * 1024, a_off[q]);
            const __amdgpu_buffer_rsrc_t rw =
                __builtin_amdgcn_make_buffer_rsrc(w_base + (size_t)k0 * N * 2, 0, (int)w_bytes, kRsrcWord3);
#pragma unroll
            for (int q = 0; q < B_PW; ++q) dma(rw, Bs + (q * NW + wave) * 1024, b_off[q]);
        };

        // fragment addresses that do not depend on the stage or k step
        // MI = 32: lanes 32..63 hold the second 8 k of a 16-k step, and a
        // transpose group of 16 lanes covers 16 of a block's 32 columns.
        // MI = 16: lane group lane/16 holds k 8 (lane/16) .. +7 of a 32-k step,
        // and a transpose group covers the block's 16 columns.
        const int g = MI == 32 ? lane >> 5 : lane >> 4;  // k group of the fragment
        const int s4 = (lane & 15) >> 2;          // row within a transpose group
        const int nb = MI == 32 ? 16 * ((lane >> 4) & 1) + 4 * (lane & 3) : 4 * (lane & 3);
        // fragments of one k step (16 k) of the wave's sub-tile
        struct Frags {
            bf16x8_t a[FM], b[FN];
        };
        auto load = [&](const char *As, int kk, Frags &f) {
            const char *Bs = As + A_BYTES;
            const int c = kk * (KM / 8) + g;       // 16-byte chunk of the A row
            auto load_a = [&] {
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int r = wm * WM + fm * MI + (lane & (MI - 1));
                    f.a[fm] = *reinterpret_cast<const bf16x8_t *>(As + a_at(r, c));
                }
            };
            // MI = 16 reads W first: the A fragments of the next step then
            // land in the registers of the current step's A fragments, each
            // read once that fragment's MFMAs are issued
            if constexpr (MI == 32) load_a();
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int n = wn * WN + fn * MI + nb;
                const int k = kk * KM + 8 * g + s4;
                const int cn = n >> 3, half = ((n >> 2) & 1) * 8;
                const char *p0 = Bs + k * RB + ((cn ^ fb(k)) << 4) + half;
                const char *p1 = Bs + (k + 4) * RB + ((cn ^ fb(k + 4)) << 4) + half;
                const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)p0);
                const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)p1);
                const v4i16_t both[2] = {lo, hi};
                f.b[fn] = *reinterpret_cast<const bf16x8_t *>(both);
            }
            if constexpr (MI == 16) load_a();
        };
        // W fragment as the first operand: the result holds, per lane, output
        // row m = lane mod MI and four consecutive output columns.
        auto mma = [&](const Frags &f) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    if constexpr (MI == 32)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[fn], f.a[fm], acc[fm][fn],
                                                                              0, 0, 0);
                    else
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[fn], f.a[fm], acc[fm][fn],
                                                                              0, 0, 0);
        };
        // Software pipeline over k steps that crosses slab boundaries: the
        // fragment reads of k step kk+1 are issued between the MFMAs of k step
        // kk, including the reads of the next slab's first step, which ride on
        // the MFMAs of this slab's last step.  The workgroup barrier therefore
        // sits before that last step: by then every wave has read all of this
        // slab (its last-step fragments are in registers), so the stage can be
        // refilled, and the next slab has landed.  The scheduling barriers pin
        // the interleaving (the compiler would otherwise group each step's
        // reads right before its own MFMAs).
        constexpr int KS = BK / KM;                // k steps per slab
        constexpr int RD = FM + 2 * FN;            // LDS reads per k step
        constexpr int MF = FM * FN;                // MFMAs per k step
        constexpr bool TWO_PER_READ = MI == 16 && MF == 2 * RD;
        static_assert(KS % 2 == 0, "fragment double buffer parity");
        Frags f[2];
        auto head = [&](const char *As) {          // k steps 0 .. KS-2 of a slab
#pragma unroll
            for (int kk = 0; kk + 1 < KS; ++kk) {
                load(As, kk + 1, f[(kk + 1) & 1]);
                mma(f[kk & 1]);
            }
            constexpr int PAIRS = RD < MF ? RD : MF;
#pragma unroll
            for (int kk = 0; kk + 1 < KS; ++kk) {
                if constexpr (TWO_PER_READ) {
                    // two MFMAs per read: the next step's A fragment fm is
                    // read after the last MFMA of this step's fragment fm
#pragma unroll
                    for (int r = 0; r < RD; ++r) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one read of step kk+1
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < PAIRS; ++r) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one read of step kk+1
                    }
                    if constexpr (RD > PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, RD - PAIRS, 0);
                    if constexpr (MF > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, MF - PAIRS, 0);
                }
            }
        };
        // last k step of a slab, the refill of its stage and the first reads
        // of the next slab, interleaved MFMA / read / direct load
        auto tail = [&](char *refill, int k0, const char *Anext) {
            issue(refill, k0);
            load(Anext, 0, f[0]);
            mma(f[(KS - 1) & 1]);
            if constexpr (TWO_PER_READ) {
#pragma unroll
                for (int r = 0; r < RD; ++r) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    if (r % 2 == 0 && r / 2 < PER) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
                if constexpr (PER > RD / 2) __builtin_amdgcn_sched_group_barrier(0x020, PER - RD / 2, 0);
            } else {
                constexpr int R = MF > RD ? (MF > PER ? MF : PER) : (RD > PER ? RD : PER);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (r < MF) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (r < RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    if (r < PER) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
            }
        };

        const int nk = __builtin_amdgcn_readfirstlane(kspan / BK);
        // one pipeline step on the slab in stage u: slabs slab+1 .. slab+S-1
        // are in flight into the other stages; after the barrier stage u is
        // refilled with slab+S
        // Lamport consumer: each wave checks the A chunks it loaded itself as
        // soon as its own loads of the slab have landed (before the slab's
        // barrier), and marks flag (slab mod 3) in LDS if one holds the
        // sentinel; after the barrier every wave reads the flag, so the
        // whole workgroup agrees without a barrier of its own.  A marked
        // slab's A part is re-loaded after an agent-scope acquire (which
        // drops lines this XCD read while they still held the sentinel)
        // until no wave finds one, before any fragment of it is read.  Flag
        // (slab mod 3) is cleared by thread 0 after the next barrier, when
        // every wave has read it and two barriers before it is set again.
        uint32_t *lflag = lamport_flags();
        // The 8-wave bodies hold 128 accumulators per lane and have no
        // registers to spare: there the chunks are read one at a time (the
        // scheduling barrier keeps the compiler from batching the reads);
        // the others read them all at once, one LDS round trip.
        auto scan_own = [&](const char *As) -> bool {
            uint32_t bad = 0;
#pragma unroll
            for (int q = 0; q < A_PW; ++q) {
                const uint4 v = *reinterpret_cast<const uint4 *>(As + (q * NW + wave) * 1024 + lane * 16);
                bad |= has_sentinel_bf16x2(v.x) | has_sentinel_bf16x2(v.y) | has_sentinel_bf16x2(v.z) |
                       has_sentinel_bf16x2(v.w);
                if constexpr (NW == 8) __builtin_amdgcn_sched_barrier(0);
            }
            return __ballot(bad) != 0;
        };
        auto mark = [&](const char *As, int v) {
            if constexpr (LAM)
                if (scan_own(As) && lane == 0) lflag[v % 3] = 1u;
        };
        auto settle = [&](char *As, int v, int k0) {  // after the barrier that follows mark(As, v)
            if constexpr (LAM) {
                if (__builtin_amdgcn_readfirstlane(lflag[v % 3]) != 0) {
                    LaneOffsets o;
#pragma unroll
                    for (int q = 0; q < A_PW; ++q) o.v[q] = a_off[q];
                    lamport_reload_slab(As, a_base + (size_t)k0 * 2, a_bytes - 2u * k0, o, lw);
                }
                if (tid == 0) lflag[(v + 2) % 3] = 0u;  // read by every wave before this barrier
            }
        };
        auto step = [&](auto U, int slab) {
            constexpr int u = decltype(U)::value;
            head(stg[u]);
            wait_vmcnt<(S - 2) * PER>();
            const bool more = slab + 1 < nk;      // stage u+1 holds slab + 1
            if (more) mark(stg[(u + 1) % S], slab + 1);
            __syncthreads();
            if (more) settle(stg[(u + 1) % S], slab + 1, (slab + 1) * BK);
            const int pre = slab + S < nk ? slab + S : nk - 1;
            tail(stg[u], pre * BK, stg[(u + 1) % S]);
        };
#pragma unroll
        for (int u = 0; u < S; ++u) issue(stg[u], (u < nk ? u : nk - 1) * BK);
        after_issue();
        wait_vmcnt<(S - 1) * PER>();
        mark(stg[0], 0);
        __syncthreads();
        settle(stg[0], 0, 0);
        load(stg[0], 0, f[0]);
        int slab = 0;
        for (; slab + S <= nk; slab += S) {
            step(ic<0>{}, slab);
            step(ic<1>{}, slab + 1);
            if constexpr (S > 2) step(ic<2 % S>{}, slab + 2);
            if constexpr (S > 3) step(ic<3 % S>{}, slab + 3);
            if constexpr (S > 4) step(ic<4 % S>{}, slab + 4);
        }
        if constexpr (KQ % (BK * S) != 0) {
            if (slab < nk) step(ic<0>{}, slab++);
            if constexpr (S > 2) if (slab < nk) step(ic<1 % S>{}, slab++);
            if constexpr (S > 3) if (slab < nk) step(ic<2 % S>{}, slab++);
            if constexpr (S > 4) if (slab < nk) step(ic<3 % S>{}, slab++);
        }
        wait_vmcnt<0>();  // the trailing prefetches must land before the LDS is reused
        __syncthreads();
        if constexpr (LAM)
            if (tid == 0) lflag[0] = lflag[1] = lflag[2] = lflag[3] = 0u;  // for the next tile
        before_epilogue();
        const LayerDesc *dp = &d;

        if (SPLIT && dp->nsplit > 1) {
            // Partial tile, fragment-native layout [wave][fm][fn][h][lane][2]
            // (h < ACC / 2)
            // floats: every 8-byte store instruction writes 512 contiguous
            // bytes.  Stored at agent scope (write-through of this XCD's L2);
            // each wave waits for its stores before the barrier, so all of
            // them are in memory before the arrival count is raised.
            const int tile = i * dp->nbn + j;
            float *ws = dp->ws + (size_t)(tile * dp->nsplit + split) * (BM * BN);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int h = 0; h < ACC / 2; ++h) {
                        const uint64_t v = (uint64_t)__float_as_uint(acc[fm][fn][2 * h]) |
                                           ((uint64_t)__float_as_uint(acc[fm][fn][2 * h + 1]) << 32);
                        float *dst = ws + ((((wave * FM + fm) * FN + fn) * (ACC / 2) + h) * 64 + lane) * 2;
                        __hip_atomic_store(reinterpret_cast<uint64_t *>(dst), v, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    }
            wait_vmcnt<0>();
            __syncthreads();
            volatile uint32_t *word = reinterpret_cast<volatile uint32_t *>(stg[0]) + 1;
            if (tid == 0)
                *word = __hip_atomic_fetch_add(arrive, 1u << dp->arrive_shift, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) >> dp->arrive_shift;
            __syncthreads();
            const bool last = *word == (uint32_t)(dp->nsplit - 1);
            __syncthreads();  // everyone has read the word before the LDS is reused
            if (!last) return false;
            // Last to arrive: every item's partial, this one's included, is in
            // memory.  Reset the count for the next run and sum the partials in
            // split order (the same order whichever item arrives last), reading
            // them at agent scope so that no cached line can be stale.  With
            // more than four partials the loads of up to four partials of one
            // block are all issued before any of them is used: one memory
            // round trip per block and group of four, instead of one per
            // partial and 8-byte pair.
            if (tid == 0) __hip_atomic_store(arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const float *ws0 = dp->ws + (size_t)(tile * dp->nsplit) * (BM * BN);
            const int ns = dp->nsplit;
            constexpr int G = 4;                   // partials loaded per group
            auto part = [&](int k, int fm, int fn, int h) -> uint64_t {
                const size_t o = ((((size_t)wave * FM + fm) * FN + fn) * (ACC / 2)) * 128 + lane * 2;
                return __hip_atomic_load(
                    reinterpret_cast<const uint64_t *>(ws0 + (size_t)k * (BM * BN) + o + h * 128),
                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            };
            // Two or four partials (the common splits): the reduction runs
            // over units of HC 8-byte pairs of one block, and the loads of the
            // next unit are issued before the current one is summed, so the
            // wave waits for about one memory round trip in all rather than
            // one per block.  Two units of loads in flight hold 64 VGPRs, as
            // the one group of the general loop below does.
            auto reduce_pipelined = [&](auto nsc) {
                constexpr int NS = decltype(nsc)::value;
                constexpr int HC = 16 / NS < ACC / 2 ? 16 / NS : ACC / 2;
                constexpr int UPB = (ACC / 2) / HC;  // units per block
                constexpr int NU = FM * FN * UPB;
                uint64_t v[2][NS][HC];
                auto issue_unit = [&](int u, uint64_t (&dst)[NS][HC]) {
                    const int blk = u / UPB, h0 = (u % UPB) * HC;
#pragma unroll
                    for (int k = 0; k < NS; ++k)
#pragma unroll
                        for (int h = 0; h < HC; ++h) dst[k][h] = part(k, blk / FN, blk % FN, h0 + h);
                };
                issue_unit(0, v[0]);
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    if (u + 1 < NU) issue_unit(u + 1, v[(u + 1) & 1]);
                    const int blk = u / UPB, h0 = (u % UPB) * HC;
#pragma unroll
                    for (int h = 0; h < HC; ++h) {
                        float s0 = __uint_as_float((uint32_t)v[u & 1][0][h]);
                        float s1 = __uint_as_float((uint32_t)(v[u & 1][0][h] >> 32));
#pragma unroll
                        for (int k = 1; k < NS; ++k) {
                            s0 = s0 + __uint_as_float((uint32_t)v[u & 1][k][h]);
                            s1 = s1 + __uint_as_float((uint32_t)(v[u & 1][k][h] >> 32));
                        }
                        acc[blk / FN][blk % FN][2 * (h0 + h)] = s0;
                        acc[blk / FN][blk % FN][2 * (h0 + h) + 1] = s1;
                    }
                    __builtin_amdgcn_sched_barrier(0);  // no unit's loads move above an earlier unit's sums
                }
            };
            if (ns == 2) {
                reduce_pipelined(ic<2>{});
            } else if (ns == 4) {
                reduce_pipelined(ic<4>{});
            } else {
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        const size_t o = ((((size_t)wave * FM + fm) * FN + fn) * (ACC / 2)) * 128 + lane * 2;
                        AccT sum;
                        for (int k0 = 0; k0 < ns; k0 += G) {
                            uint64_t v[G][ACC / 2];
#pragma unroll
                            for (int g = 0; g < G; ++g) {
                                const int k = k0 + g < ns ? k0 + g : ns - 1;  // in range; unused past ns
#pragma unroll
                                for (int h = 0; h < ACC / 2; ++h)
                                    v[g][h] = __hip_atomic_load(
                                        reinterpret_cast<const uint64_t *>(ws0 + (size_t)k * (BM * BN) + o + h * 128),
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            }
#pragma unroll
                            for (int g = 0; g < G; ++g) {
                                if (k0 + g >= ns) break;
#pragma unroll
                                for (int h = 0; h < ACC / 2; ++h) {
                                    const float v0 = __uint_as_float((uint32_t)v[g][h]);
                                    const float v1 = __uint_as_float((uint32_t)(v[g][h] >> 32));
                                    sum[2 * h] = k0 + g == 0 ? v0 : sum[2 * h] + v0;
                                    sum[2 * h + 1] = k0 + g == 0 ? v1 : sum[2 * h + 1] + v1;
                                }
                            }
                        }
                        acc[fm][fn] = sum;
                    }
            }
        }

        // Epilogue: activation on the fp32 accumulator, RNE to bf16, then the
        // tile goes through the (now idle) LDS stages so that every store
        // instruction writes whole contiguous rows (64 lanes x 8 bytes):
        // full 128-byte lines, which write-through stores need to run at
        // full speed.  LDS layout: row r in stage r / RPS, 16-byte chunk c
        // at position c ^ (r mod CPR), which spreads the 32 rows written by
        // one fragment store over distinct bank groups.
        constexpr int CPR = BN / 8;                // 16-byte chunks per row
        constexpr int RPS0 = STAGE / (BN * 2);     // tile rows one stage holds
        constexpr int RPS = RPS0 >= BM ? BM : RPS0;  // tile rows per stage used
        constexpr int UPR = BN / 4;                // 8-byte units per row
        constexpr int NUSE = (BM + RPS - 1) / RPS;  // stages the tile needs
        static_assert(RPS % 32 == 0 && NUSE <= S && NT % UPR == 0 && RPS % (NT / UPR) == 0,
                      "epilogue staging");
        // k uniform; selects among the stages the tile needs only (a select
        // over more of them became an indexed array in private memory)
        auto stage_of = [&](int k) -> char * {
            char *p = stg[0];
            if constexpr (NUSE > 1) p = k == 1 ? stg[1] : p;
            if constexpr (NUSE > 2) p = k == 2 ? stg[2] : p;
            if constexpr (NUSE > 3) p = k == 3 ? stg[3] : p;
            if constexpr (NUSE > 4) p = k == 4 ? stg[4] : p;
            return p;
        };
        const int act = dp->act;
        // Lamport intermediates never hold the sentinel: -0.0 is stored as
        // +0.0 (no stored bf16 equals 0xFFFFFFFF, so other layers keep theirs)
        const uint32_t canon = dp->lam_out ? 0x8000u : 0xFFFFFFFFu;
        // A lane holds, per block, output row m = lane mod MI and groups of
        // four consecutive columns: MI = 32, column 8 gq + 4 (lane / 32) of
        // the block for accumulators 4 gq .. 4 gq + 3; MI = 16, column
        // 4 (lane / 16) for its four accumulators.
        const int h8 = MI == 32 ? (lane >> 5) * 8 : ((lane >> 4) & 1) * 8;  // byte half of a chunk
        const int cl = MI == 32 ? 0 : (lane >> 5);                       // chunk within the block
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int rb = wm * WM + fm * MI;      // first row of this fragment block (uniform)
            const int r = rb + (lane & (MI - 1));
            char *rowp = stage_of(rb / RPS) + (r % RPS) * (BN * 2) + h8;
            const int key = r % CPR;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int c0 = (wn * WN + fn * MI) / 8 + cl;
                const AccT &v = acc[fm][fn];
#pragma unroll
                for (int gq = 0; gq < ACC / 4; ++gq) {
                    uint32_t b0 = f32_to_bf16_rne(act_apply(v[4 * gq + 0], act));
                    uint32_t b1 = f32_to_bf16_rne(act_apply(v[4 * gq + 1], act));
                    uint32_t b2 = f32_to_bf16_rne(act_apply(v[4 * gq + 2], act));
                    uint32_t b3 = f32_to_bf16_rne(act_apply(v[4 * gq + 3], act));
                    b0 = b0 == canon ? 0u : b0;
                    b1 = b1 == canon ? 0u : b1;
                    b2 = b2 == canon ? 0u : b2;
                    b3 = b3 == canon ? 0u : b3;
                    *reinterpret_cast<uint2 *>(rowp + (((c0 + gq) ^ key) << 4)) =
                        make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
                }
            }
        }
        __syncthreads();
        // An intermediate consumed by other XCDs while the run goes on is
        // stored at agent scope, which writes through this XCD's L2.
        before_store();
        constexpr int RPI = NT / UPR;              // rows per store instruction
        constexpr int NI = BM / RPI;               // store instructions per lane
        const int t = tid / UPR, u = tid % UPR;
        const int lds_u = (u & 1) * 8;
        uint64_t *dst = reinterpret_cast<uint64_t *>(C + (size_t)(row0 + t) * N + col0 + u * 4);
        auto lds_at = [&](int it) {
            const int r = it * RPI + t;
            return reinterpret_cast<const uint64_t *>(stage_of((it * RPI) / RPS) + (r % RPS) * (BN * 2) +
                                                      (((u >> 1) ^ (r % CPR)) << 4) + lds_u);
        };
        if (__builtin_amdgcn_readfirstlane(dp->coherent)) {
#pragma unroll
            for (int it = 0; it < NI; ++it)
                __hip_atomic_store(dst + (size_t)it * RPI * N / 4, *lds_at(it), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        } else {
#pragma unroll
            for (int it = 0; it < NI; ++it) dst[(size_t)it * RPI * N / 4] = *lds_at(it);
        }
        return true;
    }
};

// ----------------------------------------------------------------------------
// fp32 tile body (64 x 64, BK = 32) on v_mfma_f32_32x32x2_f32, two LDS
// stages fed from a ring of four register-staged slabs.  Small chains only; A is transposed into LDS ([k][m],
// padded) so that both fragment reads are lane-contiguous.
// ----------------------------------------------------------------------------
struct F32Body {
    static constexpr int BM = 64, BN = 64, BK = 32, S = 2, NT = 256;
    static constexpr int AP = BM + 1;  // padded A row ([k][m])
    static constexpr int BP = BN + 4;  // padded W row ([k][n]), keeps 16-byte alignment
    static constexpr int STAGE = (BK * AP + BK * BP) * 4;

    // `before_epilogue` and split-K as in Bf16Body: with d.nsplit > 1 this
    // item multiplies k in [split K / nsplit, (split + 1) K / nsplit), stores
    // an fp32 partial, and the last item of the tile to arrive sums all
    // partials in split order and runs the epilogue.  Returns whether this
    // call completed the tile.
    // LAM: the A values of every slab are checked for the sentinel -0.0 when
    // they move from registers to LDS and re-read from memory until they
    // hold none (see Bf16Body); `before_store` as in Bf16Body.
    template <bool SPLIT, bool LAM, class Hook, class StoreHook, class IssueHook>
    __device__ __forceinline__ static bool run(const LayerDesc &d, int i, int j, int split, uint32_t *arrive,
                                               char *const *stg, Hook &&before_epilogue, StoreHook &&before_store,
                                               IssueHook &&after_issue, const LamWatch &lw) {
        const int K = d.K, N = d.N;
        const int kspan = SPLIT ? __builtin_amdgcn_readfirstlane(K / d.nsplit) : K;
        const int kbeg = SPLIT ? __builtin_amdgcn_readfirstlane(split * kspan) : 0;
        const float *__restrict__ A = static_cast<const float *>(d.A) + kbeg;
        const float *__restrict__ W = static_cast<const float *>(d.W) + (size_t)kbeg * N;
        float *__restrict__ C = static_cast<float *>(d.C);
        const int row0 = i * BM, col0 = j * BN;
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int wm = wave >> 1, wn = wave & 1;

        f32x16_t acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

        // Register ring of D slabs: the global loads of slabs ks+1 .. ks+D-1
        // are in flight while slab ks is multiplied out of LDS, so a tile pays
        // the load latency about once instead of once per slab.
        // The ring is four named slabs chosen at compile time (no array), so
        // that every slab stays in registers.
        constexpr int D = 4;
        struct Slab {
            float4 a0, a1, b0, b1;
        };
        Slab r0, r1, r2, r3;
        auto ring = [&](auto U) -> Slab & {
            constexpr int u = decltype(U)::value;
            if constexpr (u == 0) return r0;
            else if constexpr (u == 1) return r1;
            else if constexpr (u == 2) return r2;
            else return r3;
        };
        auto gload = [&](int k0, Slab &sl) {
            const int r = tid >> 3, c4 = tid & 7;
            sl.a0 = *reinterpret_cast<const float4 *>(A + (size_t)(row0 + r) * K + k0 + c4 * 4);
            sl.a1 = *reinterpret_cast<const float4 *>(A + (size_t)(row0 + 32 + r) * K + k0 + c4 * 4);
            const int k = tid >> 4, n4 = tid & 15;
            sl.b0 = *reinterpret_cast<const float4 *>(W + (size_t)(k0 + k) * N + col0 + n4 * 4);
            sl.b1 = *reinterpret_cast<const float4 *>(W + (size_t)(k0 + 16 + k) * N + col0 + n4 * 4);
        };
        // Lamport consumer: the slab at k0 (relative to kbeg) holds no
        // sentinel in its A values once this returns
        auto validate = [&](Slab &sl, int k0) {
            const uint32_t bad = has_sentinel_f32(sl.a0.x) | has_sentinel_f32(sl.a0.y) | has_sentinel_f32(sl.a0.z) |
                                 has_sentinel_f32(sl.a0.w) | has_sentinel_f32(sl.a1.x) | has_sentinel_f32(sl.a1.y) |
                                 has_sentinel_f32(sl.a1.z) | has_sentinel_f32(sl.a1.w);
            if (__builtin_expect(__ballot(bad) != 0, 0)) {
                const int r = tid >> 3, c4 = tid & 7;
                auto clean = [](const uint64_t(&x)[2]) {
                    return !(has_sentinel_f32(__uint_as_float((uint32_t)x[0])) |
                             has_sentinel_f32(__uint_as_float((uint32_t)(x[0] >> 32))) |
                             has_sentinel_f32(__uint_as_float((uint32_t)x[1])) |
                             has_sentinel_f32(__uint_as_float((uint32_t)(x[1] >> 32))));
                };
                uint64_t v[2];
                lamport_reread(reinterpret_cast<const uint64_t *>(A + (size_t)(row0 + r) * K + k0 + c4 * 4), v, lw, clean);
                sl.a0 = *reinterpret_cast<const float4 *>(v);
                lamport_reread(reinterpret_cast<const uint64_t *>(A + (size_t)(row0 + 32 + r) * K + k0 + c4 * 4), v, lw,
                               clean);
                sl.a1 = *reinterpret_cast<const float4 *>(v);
            }
        };
        auto lstore = [&](char *st, const Slab &sl) {
            float *As = reinterpret_cast<float *>(st);
            float *Bs = As + BK * AP;
            const int r = tid >> 3, c4 = tid & 7;
            As[(c4 * 4 + 0) * AP + r] = sl.a0.x;
            As[(c4 * 4 + 1) * AP + r] = sl.a0.y;
            As[(c4 * 4 + 2) * AP + r] = sl.a0.z;
            As[(c4 * 4 + 3) * AP + r] = sl.a0.w;
            As[(c4 * 4 + 0) * AP + 32 + r] = sl.a1.x;
            As[(c4 * 4 + 1) * AP + 32 + r] = sl.a1.y;
            As[(c4 * 4 + 2) * AP + 32 + r] = sl.a1.z;
            As[(c4 * 4 + 3) * AP + 32 + r] = sl.a1.w;
            const int k = tid >> 4, n4 = tid & 15;
            *reinterpret_cast<float4 *>(Bs + k * BP + n4 * 4) = sl.b0;
            *reinterpret_cast<float4 *>(Bs + (16 + k) * BP + n4 * 4) = sl.b1;
        };
        auto compute = [&](const char *st) {
            const float *As = reinterpret_cast<const float *>(st);
            const float *Bs = As + BK * AP;
#pragma unroll
            for (int kk = 0; kk < BK / 2; ++kk) {
                const int k = kk * 2 + (lane >> 5);
                const float a = As[k * AP + wm * 32 + (lane & 31)];
                const float b = Bs[k * BP + wn * 32 + (lane & 31)];
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(b, a, acc, 0, 0, 0);
            }
        };

        const int nk = kspan / BK;
        // slabs past the last one re-load the last slab (in bounds, unused)
        gload(0, r0);
        after_issue();  // with one slab in registers, not four
        gload((1 < nk ? 1 : nk - 1) * BK, r1);
        gload((2 < nk ? 2 : nk - 1) * BK, r2);
        gload((3 < nk ? 3 : nk - 1) * BK, r3);
        if constexpr (LAM) validate(r0, 0);
        lstore(stg[0], r0);
        __syncthreads();
        // slab ks sits in LDS stage ks mod 2 and its ring slot u = ks mod D is
        // free again: refill it with slab ks + D, multiply slab ks, move slab
        // ks + 1 from its ring slot into the other stage
        auto step = [&](auto U, int ks) {
            constexpr int u = decltype(U)::value, un = (u + 1) % D;
            char *cur = (ks & 1) ? stg[1] : stg[0], *nxt = (ks & 1) ? stg[0] : stg[1];  // no dynamic indexing
            gload((ks + D < nk ? ks + D : nk - 1) * BK, ring(ic<u>{}));
            compute(cur);
            if (ks + 1 < nk) {
                if constexpr (LAM) validate(ring(ic<un>{}), (ks + 1) * BK);
                lstore(nxt, ring(ic<un>{}));
            }
            __syncthreads();
        };
        int ks = 0;
        for (; ks + D <= nk; ks += D) {
            step(ic<0>{}, ks);
            step(ic<1>{}, ks + 1);
            step(ic<2>{}, ks + 2);
            step(ic<3>{}, ks + 3);
        }
        if (ks < nk) step(ic<0>{}, ks++);
        if (ks < nk) step(ic<1>{}, ks++);
        if (ks < nk) step(ic<2>{}, ks++);
        before_epilogue();

        if (SPLIT && d.nsplit > 1) {
            // Partial tile in fragment-native layout [wave][h][lane][2]
            // floats, stored at agent scope (write-through); every wave waits
            // for its stores before the barrier, so they are all in memory
            // before the arrival count is raised.
            const int tile = i * d.nbn + j;
            float *ws = d.ws + (size_t)(tile * d.nsplit + split) * (BM * BN);
#pragma unroll
            for (int h = 0; h < 8; ++h) {
                const uint64_t v = (uint64_t)__float_as_uint(acc[2 * h]) |
                                   ((uint64_t)__float_as_uint(acc[2 * h + 1]) << 32);
                __hip_atomic_store(reinterpret_cast<uint64_t *>(ws + ((wave * 8 + h) * 64 + lane) * 2), v,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            wait_vmcnt<0>();
            __syncthreads();
            volatile uint32_t *word = reinterpret_cast<volatile uint32_t *>(stg[0]) + 1;
            if (tid == 0)
                *word = __hip_atomic_fetch_add(arrive, 1u << d.arrive_shift, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) >> d.arrive_shift;
            __syncthreads();
            const bool last = *word == (uint32_t)(d.nsplit - 1);
            __syncthreads();  // everyone has read the word before the LDS is reused
            if (!last) return false;
            // Last to arrive: reset the count for the next run and sum all
            // partials (its own included, read back) in split order, at
            // agent scope, up to four partials' loads in flight at once.
            if (tid == 0) __hip_atomic_store(arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const float *ws0 = d.ws + (size_t)(tile * d.nsplit) * (BM * BN) + ((size_t)wave * 8 * 64 + lane) * 2;
            const int ns = d.nsplit;
            constexpr int G = 4;
            for (int k0 = 0; k0 < ns; k0 += G) {
                uint64_t v[G][8];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int k = k0 + g < ns ? k0 + g : ns - 1;  // in range; unused past ns
#pragma unroll
                    for (int h = 0; h < 8; ++h)
                        v[g][h] = __hip_atomic_load(
                            reinterpret_cast<const uint64_t *>(ws0 + (size_t)k * (BM * BN) + h * 128),
                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    if (k0 + g >= ns) break;
#pragma unroll
                    for (int h = 0; h < 8; ++h) {
                        const float v0 = __uint_as_float((uint32_t)v[g][h]);
                        const float v1 = __uint_as_float((uint32_t)(v[g][h] >> 32));
                        acc[2 * h] = k0 + g == 0 ? v0 : acc[2 * h] + v0;
                        acc[2 * h + 1] = k0 + g == 0 ? v1 : acc[2 * h + 1] + v1;
                    }
                }
            }
        }

        const int act = d.act;
        const int m = row0 + wm * 32 + (lane & 31);
        float *crow = C + (size_t)m * N + col0 + wn * 32;
        // Lamport intermediates never hold the sentinel: -0.0 is stored as +0.0
        const uint32_t canon = d.lam_out ? 0x80000000u : 0u;
        auto cf = [&](float x) { return __float_as_uint(x) == canon && canon ? 0.0f : x; };
        before_store();
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = g * 8 + (lane >> 5) * 4;
            const float4 v = make_float4(cf(act_apply(acc[4 * g + 0], act)), cf(act_apply(acc[4 * g + 1], act)),
                                         cf(act_apply(acc[4 * g + 2], act)), cf(act_apply(acc[4 * g + 3], act)));
            if (d.coherent) {  // agent scope: writes through this XCD's L2
                const uint64_t lo = (uint64_t)__float_as_uint(v.x) | ((uint64_t)__float_as_uint(v.y) << 32);
                const uint64_t hi = (uint64_t)__float_as_uint(v.z) | ((uint64_t)__float_as_uint(v.w) << 32);
                __hip_atomic_store(reinterpret_cast<uint64_t *>(crow + n), lo, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(reinterpret_cast<uint64_t *>(crow + n + 2), hi, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            } else {
                *reinterpret_cast<float4 *>(crow + n) = v;
            }
        }
        return true;
    }
};

// LDS stages of a body: one __shared__ array per stage (see Bf16Body).
template <class Body, int S = Body::S>
struct Stages;
template <class Body>
struct Stages<Body, 2> {
    __device__ __forceinline__ static void get(char **p) {
        __shared__ __attribute__((aligned(1024))) char s0[Body::STAGE];
        __shared__ __attribute__((aligned(1024))) char s1[Body::STAGE];
        p[0] = s0; p[1] = s1; p[2] = s0; p[3] = s1; p[4] = s0;
    }
};
template <class Body>
struct Stages<Body, 3> {
    __device__ __forceinline__ static void get(char **p) {
        __shared__ __attribute__((aligned(1024))) char s0[Body::STAGE];
        __shared__ __attribute__((aligned(1024))) char s1[Body::STAGE];
        __shared__ __attribute__((aligned(1024))) char s2[Body::STAGE];
        p[0] = s0; p[1] = s1; p[2] = s2; p[3] = s0; p[4] = s1;
    }
};
template <class Body>
struct Stages<Body, 5> {
    __device__ __forceinline__ static void get(char **p) {
        __shared__ __attribute__((aligned(1024))) char s0[Body::STAGE];
        __shared__ __attribute__((aligned(1024))) char s1[Body::STAGE];
        __shared__ __attribute__((aligned(1024))) char s2[Body::STAGE];
        __shared__ __attribute__((aligned(1024))) char s3[Body::STAGE];
        __shared__ __attribute__((aligned(1024))) char s4[Body::STAGE];
        p[0] = s0; p[1] = s1; p[2] = s2; p[3] = s3; p[4] = s4;
    }
};
template <class Body>
struct Stages<Body, 4> {
    __device__ __forceinline__ static void get(char **p) {
        __shared__ __attribute__((aligned(1024))) char s0[Body::STAGE];
        __shared__ __attribute__((aligned(1024))) char s1[Body::STAGE];
        __shared__ __attribute__((aligned(1024))) char s2[Body::STAGE];
        __shared__ __attribute__((aligned(1024))) char s3[Body::STAGE];
        p[0] = s0; p[1] = s1; p[2] = s2; p[3] = s3; p[4] = s0;
    }
};

// ----------------------------------------------------------------------------
// Protocol: prologue (consumer side) and publish (producer side).
// Every helper that takes the kernel's ChainArgs by reference is inlined:
// an out-of-line call needs the argument's address, and the compiler then
// copies the whole by-value kernel argument (about 800 bytes) into private
// memory at kernel start, which also costs the registers it stages through.
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Scheduler lane only.  take_ticket claims the next slot (ticket) of this
// worker's queue q; wait_slot waits until a tile ID has been pushed into a
// claimed slot and, with CP_FLAG_FENCE_RELEASE, makes the producers' stores
// of that tile's inputs visible.  wait_slot returns the tile ID, or kDone
// when the queue is exhausted or the run has failed.  A worker claims its
// next slot while its current tile's epilogue runs, so the claim's round
// trip is hidden and a slot waits at most one epilogue for its worker.
//
// Forward progress: slots of a queue are handed out in order and pushes
// claim slots in order, so if some tile is ready, every slot of its queue
// below it is claimed and filled without waiting.  Take an unfinished tile
// of lowest layer: its producers are finished, so it has been pushed, and
// the workers of its queue reach it (a worker holding that slot is at worst
// finishing a tile whose own inputs are complete).  Every queue has workers
// and all workers are resident (the grid fits the device at once), so no
// wait lasts forever for a well-formed dependency table; if the device is
// shared and some workers are not resident, the watchdog ends the run with
// a timeout.
__device__ __forceinline__ uint32_t take_ticket(const ChainArgs &a, int q) {
    if (ld_relaxed(a.ctl + kCtlStatus) != 0) return kDone;  // >= any queue size
    return __hip_atomic_fetch_add(a.ctl + ctl_head(q), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Debug and trace bookkeeping of a dequeue: count it, stamp it.
__device__ __forceinline__ void dequeued(const ChainArgs &a, uint32_t id, uint64_t t0) {
    if (a.deq_count)
        __hip_atomic_fetch_add(a.deq_count + id, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a.trace) {
        a.trace[kTraceWords * (size_t)id + 0] = t0;
        a.trace[kTraceWords * (size_t)id + 1] = wall_clock64();
        a.trace[kTraceWords * (size_t)id + 4] = clock64();
        a.trace[kTraceWords * (size_t)id + 6] = blockIdx.x;
    }
}

__device__ __forceinline__ uint32_t wait_slot(const ChainArgs &a, int q, uint32_t t) {
    if (t >= (uint32_t)a.qsize[q]) return kDone;
    const uint32_t *slot = a.queue + a.qbase[q] + t;
    const uint64_t t0 = wall_clock64();
    uint32_t id;
    uint32_t polls = 0;
    while ((id = ld_relaxed(slot)) == kEmpty) {
        __builtin_amdgcn_s_sleep(1);
        if ((++polls & 63) == 0) {
            if (wall_clock64() - t0 > a.timeout_ticks) {
                __hip_atomic_store(a.ctl + kCtlStatus, (uint32_t)kStatusTimeout, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                return kDone;
            }
            if (ld_relaxed(a.ctl + kCtlStatus) != 0) return kDone;
        }
    }
    if (id >= (uint32_t)a.layer[0].ntiles && (a.flags & CP_FLAG_FENCE_RELEASE)) {
        // Every producer of `id` released its stores before decrementing
        // score[id]; acquiring the final value (0) of that counter orders this
        // workgroup's subsequent loads after all of those stores (and
        // invalidates this XCD's L2).  With write-through release (default)
        // no invalidate is needed: the run's reads of an intermediate
        // row-block all come after its producers finished, the caches held
        // none of its lines at kernel start, and the producers' agent-scope
        // stores reached memory before any counter was decremented.
        (void)__hip_atomic_load(a.score + id, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    }
    dequeued(a, id, t0);
    return id;
}

// A worker's first slot is its own (no ticket atomic) and, for the
// pre-filled first-layer slots, its content is known: compute it instead
// of reading it, which saves the first tile a memory round trip.
__device__ __forceinline__ uint32_t first_slot(const ChainArgs &a, int q, uint32_t t) {
    if (!a.first_formula || t >= (uint32_t)a.qfirst[q]) return wait_slot(a, q, t);
    const uint64_t t0 = a.trace ? wall_clock64() : 0;
    const uint32_t id = first_item(a.layer[0].nbn * a.layer[0].nsplit, a.nq, q, t);
    dequeued(a, id, t0);
    return id;
}

// All threads.  Called after the tile's stores.  Release, two ways:
//   write-through (default): the tile was stored at agent scope, which
//     writes through this XCD's L2; every wave waits until its stores have
//     completed (vmcnt 0) before the barrier, so all of them are in memory
//     before wave 0 touches a counter.  No L2 write-back is needed.
//   CP_FLAG_FENCE_RELEASE: the barrier makes every wave's (write-back)
//     stores happen-before wave 0's agent-scope release fence, which writes
//     back this XCD's whole L2.
// Wave 0 then decrements the counter of every consumer (all in layer l+1),
// one edge per lane, and pushes the consumers whose counter reached zero into
// their owner queues, one tail atomic per queue.
//   Lamport (the tile's layer has lam_out): no wait at all; consumers check
//     the data itself for the sentinel and re-read it until it has landed.
//
// release_stores: every thread, once its stores are issued (the completion
// wait and the barrier); publish_edges: wave 0 only, any time after it (the
// fence, the decrements and the pushes); publish: both at once.
__device__ __forceinline__ void release_stores(const ChainArgs &a, int l) {
    const bool fenced = (a.flags & CP_FLAG_FENCE_RELEASE) != 0;
    if (!fenced && !a.layer[l].lam_out) wait_vmcnt<0>();
    __syncthreads();
}

__device__ __forceinline__ void publish_edges(const ChainArgs &a, uint32_t id, int l) {
    const bool fenced = (a.flags & CP_FLAG_FENCE_RELEASE) != 0;
    const int lane = threadIdx.x & 63;
    if (fenced) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if ((a.flags & CP_FLAG_DELAY_INJECT) && ((id * 2654435761u) >> 30) == 0) {
        const uint64_t s = wall_clock64();
        while (wall_clock64() - s < 2000) __builtin_amdgcn_s_sleep(8);  // ~20 us
    }
    if (a.trace && lane == 0) a.trace[kTraceWords * (size_t)id + 3] = wall_clock64();
    const LayerDesc &next = a.layer[l + 1];
    const int beg = a.dep_off[id], end = a.dep_off[id + 1];
    for (int e0 = beg; e0 < end; e0 += 64) {
        const int e = e0 + lane;
        bool ready = false;
        uint32_t c = 0;
        int cq = 0;
        if (e < end) {
            c = (uint32_t)a.dep_ids[e];
            const int old = __hip_atomic_fetch_sub(a.score + c, 1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            ready = (old == 1);
            cq = a.queue_by_layer ? l + 1 : owner_queue(next, (int)c, a.nq);
        }
        if (!__ballot(ready)) continue;
        // Lane q counts this batch's ready consumers of queue q and every
        // ready lane its rank among them; then lanes 0 .. nq-1 claim their
        // queues' slots in one atomic instruction (one round trip for all
        // queues), and each ready lane stores its ID into its claimed slot.
        const uint64_t below = (1ull << lane) - 1ull;
        uint32_t cnt = 0, rank = 0;
        for (int q = 0; q < a.nq; ++q) {
            const uint64_t m = __ballot(ready && cq == q);
            if (lane == q) cnt = (uint32_t)__popcll(m);
            if (cq == q) rank = (uint32_t)__popcll(m & below);
        }
        uint32_t base = 0;
        if (lane < a.nq && cnt)
            base = __hip_atomic_fetch_add(a.ctl + ctl_tail(lane), cnt, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        base = __shfl(base, cq);
        if (ready)
            __hip_atomic_store(a.queue + a.qbase[cq] + base + rank, c, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

__device__ __forceinline__ void publish(const ChainArgs &a, uint32_t id, int l) {
    release_stores(a, l);
    if (threadIdx.x < 64) publish_edges(a, id, l);
}

__device__ __forceinline__ void decode(const ChainArgs &a, uint32_t id, int &l, int &i, int &j, int &split) {
    l = 0;
    while (l + 1 < a.L && (int)id >= a.layer[l + 1].tile_off) ++l;
    const LayerDesc &d = a.layer[l];
    const int loc = (int)id - d.tile_off;
    const int tile = __builtin_amdgcn_readfirstlane(loc / d.nsplit);
    split = __builtin_amdgcn_readfirstlane(loc - tile * d.nsplit);
    i = __builtin_amdgcn_readfirstlane(tile / d.nbn);
    j = __builtin_amdgcn_readfirstlane(tile - i * d.nbn);
}

// ----------------------------------------------------------------------------
// Kernels
// ----------------------------------------------------------------------------

// Per-run state reset of one copy: scoreboard from the in-degree template,
// queues from their initial image (each pre-filled with its first-layer
// tiles in row-block-major order, EMPTY after), per-queue head = 0,
// tail = pre-filled, status OK.  Grid-stride over the calling grid.
__device__ __forceinline__ void reset_copy(const ChainArgs &a, uint32_t *queue, uint32_t *ctl, int32_t *score,
                           uint32_t *deq_count, uint64_t *trace, uint32_t *arrive) {
    const int stride = gridDim.x * blockDim.x;
    // opaque thread index: a persistent worker calls this on its way out,
    // and nothing of it should be computed early and held across its tiles
    int tx = threadIdx.x;
    __asm__ volatile("" : "+v"(tx));
    for (int t = blockIdx.x * blockDim.x + tx; t < a.T; t += stride) {
        score[t] = a.indeg[t];
        queue[t] = a.qinit[t];
        arrive[t] = 0;
        if (deq_count) deq_count[t] = 0;
        if (trace)
            for (int w = 0; w < kTraceWords; ++w) trace[kTraceWords * (size_t)t + w] = 0;
    }
    if (blockIdx.x == 0 && tx < kMaxQueues) {
        const int q = tx;
        // slots 0 .. (workers of queue q) - 1 are handed out statically
        ctl[ctl_head(q)] = q < a.nq ? (uint32_t)a.qworkers[q] : 0u;
        ctl[ctl_tail(q)] = q < a.nq ? (uint32_t)a.qfirst[q] : 0u;
        if (q == 0) {
            ctl[kCtlStatus] = 0;
            ctl[kCtlRereads] = 0;
        }
    }
}

// Lane 0 of wave 0: the worker's scheduler (takes tickets, peeks and polls
// slots).  Wave 0 is also the publisher, so the wave that knows whether the
// next tile is already there is the one that decides when to release.
constexpr int kSchedLane = 0;

// Lamport plans: this worker's share of the sentinel fill of the other copy
// of the intermediates (used by the next run), 16-byte stores written
// through to memory.
__device__ __forceinline__ void lamport_fill_share(const ChainArgs &a, int nt) {
    const uint64_t pat = (uint64_t)a.lam_pattern | ((uint64_t)a.lam_pattern << 32);
    const size_t stride = (size_t)a.nworkers * nt;
    for (int l = 0; l < kMaxLayers && a.lam_fill[l]; ++l) {
        uint64_t *p = static_cast<uint64_t *>(a.lam_fill[l]);
        const size_t n = a.lam_fill_bytes[l] / 16;
        for (size_t c = (size_t)blockIdx.x * nt + threadIdx.x; c < n; c += stride) {
            __hip_atomic_store(p + 2 * c, pat, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(p + 2 * c + 1, pat, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Persistent worker: loop prologue -> tile body -> publish until its queue
// (blockIdx.x mod nq, so that workgroups dispatched round-robin over the
// XCDs serve the queue of their own XCD) is exhausted.  The grid is the
// number of workgroups the device holds at once, so on an otherwise idle
// device every worker is resident (a cooperative launch guarantees it).
// On the way out the workers reset the other copy of the per-run state for
// the next run (nothing of this run reads it; the kernel boundary publishes
// it).  The tile ID is broadcast through the first word of stage 0; the
// second barrier guarantees every thread has read it before the body's
// loads reuse stage 0.
//
// LAM (Lamport plans): consumers check their A data for the sentinel; each
// worker, once its first tile is done, fills its share of the other copy of
// the intermediates with the sentinel for the next run; with
// CP_FLAG_DELAY_INJECT a fixed quarter of producers release their tile
// BEFORE storing it and store it ~20 us later, so that consumers do read
// sentinels (a test of the re-read path that the other protocols could not
// survive).
template <class Body, bool SPLIT, bool LAM>
__device__ __forceinline__ void worker_loop(ChainArgs &a) {
    char *stg[5];
    Stages<Body>::get(stg);
    volatile uint32_t *slot = reinterpret_cast<volatile uint32_t *>(stg[0]);
    const int q = a.fixed_queue >= 0 ? a.fixed_queue : (int)(blockIdx.x % (unsigned)a.nq);
    const bool sched = threadIdx.x == kSchedLane;
    // first slot without an atomic: the r-th worker of queue q owns slot r
    // (the reset set each head past the workers' count)
    uint32_t ticket = a.fixed_queue >= 0 ? blockIdx.x : blockIdx.x / (unsigned)a.nq;
    bool first = true;
    bool filled = !LAM;
    const LamWatch lw{a.ctl + kCtlStatus, a.timeout_ticks, a.deq_count ? a.ctl + kCtlRereads : nullptr};
    // Deferred release (wave roles, Fig. 2(b)): when the scheduler lane finds
    // its next slot already filled as the tile body ends, wave 0 does not
    // release the finished tile before the next one starts; it does so once
    // the next tile's first slabs are requested, while they are in flight.
    // The MFMA waves thus start the next tile without waiting for the
    // decrements and pushes.  Only a tile that is already there (its inputs
    // complete) is started before the release, so no wait can depend on the
    // deferred release.
    uint32_t pending = kEmpty;  // deferred tile (wave 0's view; uniform in wave 0)
    int pending_l = 0;
    uint32_t peek = 0;          // scheduler lane: the next slot held a tile
    // wave 0 by a wave-uniform test, so that the deferral state stays in
    // scalar registers
    const bool wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
    auto release_pending = [&] {
        if (wave0 && pending != kEmpty) {
            publish_edges(a, pending, pending_l);
            pending = kEmpty;
        }
    };
    if (LAM && threadIdx.x < 4) lamport_flags()[threadIdx.x] = 0u;  // before the loop's first barrier
    for (;;) {
        if (sched) *slot = first ? first_slot(a, q, ticket) : wait_slot(a, q, ticket);
        first = false;
        __syncthreads();
        // the broadcast ID is uniform; saying so keeps the layer descriptor
        // and the buffer resources derived from it in scalar registers
        const uint32_t id = __builtin_amdgcn_readfirstlane(*slot);
        __syncthreads();
        if (id >= (uint32_t)a.T) break;
        int l, i, j, split;
        decode(a, id, l, i, j, split);
        const uint32_t first_item_id = id - (uint32_t)split;  // the tile's first item carries its edges
        bool released = false;
        // Early dispatch (Lamport plans with CP_FLAG_EARLY_DISPATCH): a
        // tile's consumers are queued once all its items have started, not
        // when it is stored.  Each item counts its start in the low half of
        // the tile's arrival counter; the one that completes the count
        // queues the consumers (wave 0, right after this item's first loads
        // are requested).  The tile is then not released when it is stored.
        const bool early = LAM && (a.flags & CP_FLAG_EARLY_DISPATCH) != 0;
        bool start_publish = false;
        if (early && l + 1 < a.L && wave0) {
            const int ns = a.layer[l].nsplit;
            if (ns == 1) {
                start_publish = true;
            } else {
                uint32_t old = 0;
                if (threadIdx.x == 0)
                    old = __hip_atomic_fetch_add(a.arrive + first_item_id, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
                start_publish = (__builtin_amdgcn_readfirstlane(old) & 0xFFFFu) == (uint32_t)(ns - 1);
            }
        }
        auto after_issue = [&] {
            release_pending();
            if (start_publish) publish_edges(a, first_item_id, l);
        };
        auto next_ticket = [&] {
            if (sched) {
                ticket = take_ticket(a, q);
                // the load's round trip overlaps the epilogue
                peek = ticket < (uint32_t)a.qsize[q] ? (ld_relaxed(a.queue + a.qbase[q] + ticket) != kEmpty) : 0u;
            }
        };

        auto store_hook = [&] {
            if constexpr (LAM) {
                if ((a.flags & CP_FLAG_DELAY_INJECT) && l + 1 < a.L && ((first_item_id * 2654435761u) >> 30) == 0) {
                    if (!early) {  // (early dispatch: the consumers are queued already)
                        publish(a, first_item_id, l);  // release first ...
                        released = true;
                    }
                    const uint64_t s0 = wall_clock64();
                    while (wall_clock64() - s0 < 2000) __builtin_amdgcn_s_sleep(8);  // ... store ~20 us later
                }
            }
        };
        // Only a layer whose A is a Lamport intermediate checks it for the
        // sentinel (the first layer's A is the caller's X, whose -0.0 is
        // data); the other layers run the plain body.
        bool done;
        if (LAM && a.layer[l].lam_in)
            done = Body::template run<SPLIT, true>(a.layer[l], i, j, split, a.arrive + first_item_id, stg, next_ticket,
                                                   store_hook, after_issue, lw);
        else
            done = Body::template run<SPLIT, false>(a.layer[l], i, j, split, a.arrive + first_item_id, stg,
                                                    next_ticket, store_hook, after_issue, lw);
        if (a.trace && threadIdx.x == 0) {
            a.trace[kTraceWords * (size_t)id + 2] = wall_clock64();
            a.trace[kTraceWords * (size_t)id + 5] = clock64();
        }
        // a split-K item that did not complete its tile has nothing to
        // release; a completed one is released now, or, if the next tile is
        // already there, right after that tile's first loads are requested
        if (done && l + 1 < a.L && !released && !early) {
            release_stores(a, l);
            if (wave0) {
                if (__builtin_amdgcn_readfirstlane(peek)) {
                    pending = first_item_id;
                    pending_l = l;
                    if (a.trace && threadIdx.x == 0) a.trace[kTraceWords * (size_t)first_item_id + 7] = 1;
                } else {
                    publish_edges(a, first_item_id, l);
                }
            }
        } else {
            __syncthreads();
        }
        if (LAM && !filled) {
            filled = true;
            lamport_fill_share(a, Body::NT);
        }
    }
    release_pending();  // (never pending here: a deferred release always has a next tile)
    if (LAM && !filled) lamport_fill_share(a, Body::NT);  // a worker that got no tile
    // Reset the other copy of the per-run state for the next run: nothing of
    // this run reads it, and the kernel boundary publishes it.  Done on the
    // way out, where a worker has nothing left to wait for, rather than
    // ahead of its first tile.
    reset_copy(a, a.nxt_queue, a.nxt_ctl, a.nxt_score, a.nxt_deq_count, a.nxt_trace, a.nxt_arrive);
}

// Waves per SIMD the LDS of a body allows (at most 2): the register budget
// the Lamport worker is held to, so that its checks and re-read path never
// cost it the occupancy of the plain worker.
template <class Body>
constexpr int lds_waves_per_simd() {
    const int wgs = (160 * 1024) / (Body::S * Body::STAGE);
    const int w = wgs * (Body::NT / 64) / 4;
    return w < 1 ? 1 : (w > 2 ? 2 : w);
}

template <class Body, bool SPLIT, bool LAM>
__global__ void __launch_bounds__(Body::NT) worker_kernel(ChainArgs a) {
    static_assert(!LAM, "Lamport workers are lamport_worker_kernel");
    worker_loop<Body, SPLIT, false>(a);
}

template <class Body, bool SPLIT>
__global__ void __launch_bounds__(Body::NT, lds_waves_per_simd<Body>()) lamport_worker_kernel(ChainArgs a) {
    worker_loop<Body, SPLIT, true>(a);
}

// The kernel of a (SPLIT, LAM) instantiation.
template <class Body, bool SPLIT, bool LAM>
constexpr auto worker_fn() {
    if constexpr (LAM) return lamport_worker_kernel<Body, SPLIT>;
    else return worker_kernel<Body, SPLIT, false>;
}

// One layer, one tile per workgroup, row-blocks [rb0, rb0 + nrb): the plain
// kernel-boundary execution used by the sequential and micro-batched modes.
template <class Body, bool SPLIT>
__global__ void __launch_bounds__(Body::NT) layer_kernel(ChainArgs a, int l, int rb0) {
    char *stg[5];
    Stages<Body>::get(stg);
    const LayerDesc &d = a.layer[l];
    const int per_rb = d.nbn * d.nsplit;  // items per row-block
    const int t = blockIdx.x;
    const int i = __builtin_amdgcn_readfirstlane(rb0 + t / per_rb), rem = t % per_rb;
    const int j = __builtin_amdgcn_readfirstlane(rem / d.nsplit), split = __builtin_amdgcn_readfirstlane(rem % d.nsplit);
    (void)Body::template run<SPLIT, false>(d, i, j, split, a.arrive + d.tile_off + (i * d.nbn + j) * d.nsplit,
                                           stg, [] {}, [] {}, [] {}, LamWatch{nullptr, 0, nullptr});
}

// Reset of the current copy (at plan time, for both copies).
__global__ void reset_kernel(ChainArgs a) {
    reset_copy(a, a.queue, a.ctl, a.score, a.deq_count, a.trace, a.arrive);
}

// The dependency table, queue image and both state copies, computed from
// the closed form of the tile graph (the same table the host builder makes):
//   indeg   item of layer l > 0: N_{l-1} / tile_n producer tiles over its
//           layer's split, 0 in layer 0;
//   dep_off producers are the first items of layers 0 .. L-2, each with one
//           edge per consumer tile of its row-block, in item order;
//   dep_ids edge e of producer tile (i, k) of layer l goes to consumer tile
//           (i, j) of layer l+1, item k / (producer tiles per k range);
//   qinit   queue q holds its first-layer items, cp::first_item order, then
//           empty slots.
// Grid-stride over items, edges and queue slots; no thread reads what
// another writes.
__global__ void graph_setup_kernel(ChainArgs a, GraphDims g) {
    const int stride = gridDim.x * blockDim.x;
    const int t0 = blockIdx.x * blockDim.x + threadIdx.x;
    int32_t *indeg = const_cast<int32_t *>(a.indeg);
    int32_t *dep_off = const_cast<int32_t *>(a.dep_off);
    int32_t *dep_ids = const_cast<int32_t *>(a.dep_ids);
    uint32_t *qinit = const_cast<uint32_t *>(a.qinit);
    for (int t = t0; t < g.T; t += stride) {
        int l = 0;
        while (l + 1 < g.L && t >= g.layer_off[l + 1]) ++l;
        const int loc = t - g.layer_off[l], ns = g.nsplit[l];
        const int32_t d = l > 0 ? g.nbn[l - 1] / ns : 0;
        indeg[t] = d;
        a.score[t] = d;
        a.nxt_score[t] = d;
        a.arrive[t] = 0;
        a.nxt_arrive[t] = 0;
        dep_off[t] = g.edge_off[l] + (l + 1 < g.L ? ((loc + ns - 1) / ns) * g.nbn[l + 1] : 0);
        // queue slot t
        int q = 0;
        while (q + 1 < a.nq && t >= a.qbase[q + 1]) ++q;
        const int r = t - a.qbase[q];
        const uint32_t v = r < a.qfirst[q]
                               ? first_item(g.nbn[0] * g.nsplit[0], a.nq, q, (uint32_t)r)
                               : kEmpty;
        qinit[t] = v;
        a.queue[t] = v;
        a.nxt_queue[t] = v;
    }
    if (t0 == 0) dep_off[g.T] = g.E;
    for (int e = t0; e < g.E; e += stride) {
        int l = 0;
        while (l + 2 < g.L && e >= g.edge_off[l + 1]) ++l;
        const int le = e - g.edge_off[l];
        const int nc = g.nbn[l + 1];
        const int ptile = le / nc, j = le - ptile * nc;
        const int i = ptile / g.nbn[l], k = ptile - i * g.nbn[l];
        const int per_split = g.nbn[l] / g.nsplit[l + 1];
        dep_ids[e] = g.layer_off[l + 1] + (i * nc + j) * g.nsplit[l + 1] + k / per_split;
    }
    if (t0 < kMaxQueues) {
        const int q = t0;
        // slots 0 .. (workers of queue q) - 1 are handed out statically
        const uint32_t head = q < a.nq ? (uint32_t)a.qworkers[q] : 0u;
        const uint32_t tail = q < a.nq ? (uint32_t)a.qfirst[q] : 0u;
        a.ctl[ctl_head(q)] = head;
        a.ctl[ctl_tail(q)] = tail;
        a.nxt_ctl[ctl_head(q)] = head;
        a.nxt_ctl[ctl_tail(q)] = tail;
        if (q == 0) {
            a.ctl[kCtlStatus] = 0;
            a.nxt_ctl[kCtlStatus] = 0;
            a.ctl[kCtlRereads] = 0;
            a.nxt_ctl[kCtlRereads] = 0;
        }
    }
}

// Fill an intermediate with quiet NaN so that a premature read is visible.
__global__ void poison_kernel(uint32_t *p, size_t words, uint32_t pattern) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t w = (size_t)blockIdx.x * blockDim.x + threadIdx.x; w < words; w += stride)
        p[w] = pattern;
}

// ----------------------------------------------------------------------------
// Launchers and the variant table
// ----------------------------------------------------------------------------
// Workgroups of this instantiation the current device holds at once (its
// occupancy times the compute units), computed once per process.
template <class Body, bool SPLIT, bool LAM>
int resident_capacity() {
    static const int cap = [] {
        int occ = 0, dev = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, worker_fn<Body, SPLIT, LAM>(), Body::NT, 0) !=
                hipSuccess ||
            hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        return occ * cus;
    }();
    return cap;
}

// The queue protocol's forward progress needs every worker resident, so a
// grid larger than the launched instantiation's capacity is refused
// (hipErrorCooperativeLaunchTooLarge) instead of launched.
template <class Body, bool SPLIT, bool LAM>
hipError_t launch_worker_s(const ChainArgs &a, int grid, bool cooperative, hipStream_t s) {
    if (grid > resident_capacity<Body, SPLIT, LAM>()) return hipErrorCooperativeLaunchTooLarge;
    if (!cooperative) {
        hipLaunchKernelGGL((worker_fn<Body, SPLIT, LAM>()), dim3(grid), dim3(Body::NT), 0, s, a);
        return hipGetLastError();
    }
    ChainArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(worker_fn<Body, SPLIT, LAM>()), dim3(grid),
                                      dim3(Body::NT), args, 0, s);
}

// A plan with a split layer launches the split-K instantiation, a Lamport
// plan the Lamport one.
template <class Body>
hipError_t launch_worker_t(const ChainArgs &a, int grid, bool cooperative, hipStream_t s) {
    bool split = false, lam = false;
    for (int l = 0; l < a.L; ++l) {
        split |= a.layer[l].nsplit > 1;
        lam |= a.layer[l].lam_in != 0;
    }
    if (lam) {
        if (split) return launch_worker_s<Body, true, true>(a, grid, cooperative, s);
        return launch_worker_s<Body, false, true>(a, grid, cooperative, s);
    }
    if (split) return launch_worker_s<Body, true, false>(a, grid, cooperative, s);
    return launch_worker_s<Body, false, false>(a, grid, cooperative, s);
}

template <class Body>
hipError_t launch_layer_t(const ChainArgs &a, int l, int rb0, int nrb, hipStream_t s) {
    const int grid = nrb * a.layer[l].nbn * a.layer[l].nsplit;
    if (grid <= 0) return hipSuccess;
    if (a.layer[l].nsplit > 1) {
        hipLaunchKernelGGL((layer_kernel<Body, true>), dim3(grid), dim3(Body::NT), 0, s, a, l, rb0);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((layer_kernel<Body, false>), dim3(grid), dim3(Body::NT), 0, s, a, l, rb0);
    return hipGetLastError();
}

// Workgroups of the persistent worker one compute unit holds at once.  A
// plan sizes its grid before it knows whether it will launch the split-K
// instantiation, whose register use differs, so this is the smaller of the
// two instantiations' figures (Lamport plans: of the two Lamport ones):
// every worker of either is then resident, which the queue protocol's
// forward progress relies on.
template <class Body>
hipError_t occupancy_t(int *blocks, bool lamport) {
    int plain = 0, split = 0;
    hipError_t e = lamport
                       ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&plain, worker_fn<Body, false, true>(),
                                                                      Body::NT, 0)
                       : hipOccupancyMaxActiveBlocksPerMultiprocessor(&plain, worker_fn<Body, false, false>(),
                                                                      Body::NT, 0);
    if (e != hipSuccess) return e;
    e = lamport ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&split, worker_fn<Body, true, true>(), Body::NT, 0)
                : hipOccupancyMaxActiveBlocksPerMultiprocessor(&split, worker_fn<Body, true, false>(), Body::NT, 0);
    if (e != hipSuccess) return e;
    *blocks = split < plain ? split : plain;
    return hipSuccess;
}

// LDS stages per tile shape: as many as fit the occupancy each shape aims for
// (64x128: four stages, one workgroup per CU; on 512 x 4096 x 4096 x 4096
// its 256 tiles per layer then run unsplit, 55.3 us on 4 waves against
// 59.1 us for 128x64 tiles on three stages, two per CU, split two ways)
#ifndef CP_S_256x256
#define CP_S_256x256 2
#endif
#ifndef CP_S_256x128
#define CP_S_256x128 3
#endif
#ifndef CP_S_128x256
#define CP_S_128x256 3
#endif
#ifndef CP_S_128x128
#define CP_S_128x128 2
#endif
#ifndef CP_S_256x64
#define CP_S_256x64 2
#endif
#ifndef CP_S_64x256
#define CP_S_64x256 2
#endif
#ifndef CP_S_128x64
#define CP_S_128x64 3
#endif
#ifndef CP_S_64x128
#define CP_S_64x128 4
#endif
#ifndef CP_S_64x64
#define CP_S_64x64 4
#endif

// wave grid (waves along M x along N) per tile shape.  The one-workgroup-
// per-CU shapes take 8 waves (two per SIMD, which cover each other's barrier
// and LDS waits); 256x128 and 128x256 on 4 x 2 waves of 64 x 64 (or 32 x
// 128): on 256 x 8192 x 28672 x 8192 with tanh-GeLU, 256x128 tiles ran the
// pipelined chain in 280.3 us against 302.8 us for 128x128 tiles, 2 x 4
// waves 286.5 us, 2 x 2 waves 319.8 us.  64x128 on 2 x 4 waves of 32 x 32:
// 512 x 4096 x 4096 x 4096 in 54.7 us against 58.4 us on 2 x 2 waves.
#ifndef CP_W_256x256
#define CP_W_256x256 2, 4
#endif
#ifndef CP_W_256x128
#define CP_W_256x128 4, 2
#endif
#ifndef CP_W_128x256
#define CP_W_128x256 4, 2
#endif
#ifndef CP_W_128x128
#define CP_W_128x128 2, 2
#endif
#ifndef CP_W_256x64
#define CP_W_256x64 2, 2
#endif
#ifndef CP_W_64x256
#define CP_W_64x256 2, 2
#endif
#ifndef CP_W_128x64
#define CP_W_128x64 2, 2
#endif
#ifndef CP_W_64x128
#define CP_W_64x128 2, 4
#endif
#ifndef CP_W_64x64
#define CP_W_64x64 2, 2
#endif

// k slab per tile shape
#ifndef CP_K_256x256
#define CP_K_256x256 64
#endif
#ifndef CP_K_256x128
#define CP_K_256x128 64
#endif
#ifndef CP_K_128x256
#define CP_K_128x256 64
#endif
#ifndef CP_K_128x128
#define CP_K_128x128 64
#endif
#ifndef CP_K_256x64
#define CP_K_256x64 64
#endif
#ifndef CP_K_64x256
#define CP_K_64x256 64
#endif
#ifndef CP_K_128x64
#define CP_K_128x64 64
#endif
#ifndef CP_K_64x128
#define CP_K_64x128 64
#endif
#ifndef CP_K_64x64
#define CP_K_64x64 64
#endif

// MFMA block per tile shape (32: 32x32x16, 16: 16x16x32)
#ifndef CP_MI_256x256
#define CP_MI_256x256 16
#endif
#ifndef CP_MI_256x128
#define CP_MI_256x128 32
#endif
#ifndef CP_MI_128x256
#define CP_MI_128x256 32
#endif
#ifndef CP_MI_128x128
#define CP_MI_128x128 32
#endif
#ifndef CP_MI_256x64
#define CP_MI_256x64 32
#endif
#ifndef CP_MI_64x256
#define CP_MI_64x256 32
#endif
#ifndef CP_MI_128x64
#define CP_MI_128x64 32
#endif
#ifndef CP_MI_64x128
#define CP_MI_64x128 32
#endif
#ifndef CP_MI_64x64
#define CP_MI_64x64 32
#endif

#define CP_BODY(bm, bn) \
    Bf16Body<bm, bn, CP_S_##bm##x##bn, CP_W_##bm##x##bn, CP_K_##bm##x##bn, CP_MI_##bm##x##bn>
#define CP_BF16_VARIANT(bm, bn)                                                                  \
    {CP_BF16, bm, bn, CP_BODY(bm, bn)::KQ, CP_S_##bm##x##bn * CP_BODY(bm, bn)::STAGE,                         \
     launch_worker_t<CP_BODY(bm, bn)>, launch_layer_t<CP_BODY(bm, bn)>, occupancy_t<CP_BODY(bm, bn)>}

static const Variant kVariants[] = {
    {CP_F32, 64, 64, 32, 2 * F32Body::STAGE, launch_worker_t<F32Body>, launch_layer_t<F32Body>,
     occupancy_t<F32Body>},
    CP_BF16_VARIANT(256, 256), CP_BF16_VARIANT(256, 128), CP_BF16_VARIANT(128, 256),
    CP_BF16_VARIANT(128, 128), CP_BF16_VARIANT(256, 64),  CP_BF16_VARIANT(64, 256),
    CP_BF16_VARIANT(128, 64),  CP_BF16_VARIANT(64, 128),  CP_BF16_VARIANT(64, 64),
};

const Variant *find_variant(int dtype, int tile_m, int tile_n) {
    for (const Variant &v : kVariants)
        if (v.dtype == dtype && v.tile_m == tile_m && v.tile_n == tile_n) return &v;
    return nullptr;
}

const Variant *variant_list(int *count) {
    *count = (int)(sizeof(kVariants) / sizeof(kVariants[0]));
    return kVariants;
}

hipError_t launch_reset(const ChainArgs &a, hipStream_t s) {
    int grid = (a.T + kThreads - 1) / kThreads;
    if (grid > 1024) grid = 1024;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(reset_kernel, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_graph_setup(const ChainArgs &a, const GraphDims &g, hipStream_t s) {
    const int n = g.T > g.E ? g.T : g.E;
    int grid = (n + kThreads - 1) / kThreads;
    if (grid > 1024) grid = 1024;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(graph_setup_kernel, dim3(grid), dim3(kThreads), 0, s, a, g);
    return hipGetLastError();
}

// Sentinel fill of a Lamport intermediate, written through to memory.
__global__ void fill_kernel(uint64_t *p, size_t n16, uint32_t pattern) {
    const uint64_t pat = (uint64_t)pattern | ((uint64_t)pattern << 32);
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < n16; c += stride) {
        __hip_atomic_store(p + 2 * c, pat, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p + 2 * c + 1, pat, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

hipError_t launch_fill(void *p, size_t bytes, uint32_t pattern, hipStream_t s) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    size_t grid = (n16 + kThreads - 1) / kThreads;
    if (grid > 2048) grid = 2048;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, static_cast<uint64_t *>(p), n16,
                       pattern);
    return hipGetLastError();
}

hipError_t launch_poison(void *p, size_t bytes, int dtype, hipStream_t s) {
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    const uint32_t pattern = dtype == CP_BF16 ? 0x7FC07FC0u : 0x7FC00000u;
    size_t grid = (words + kThreads - 1) / kThreads;
    if (grid > 2048) grid = 2048;
    hipLaunchKernelGGL(poison_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s,
                       static_cast<uint32_t *>(p), words, pattern);
    return hipGetLastError();
}

}  // namespace cp
