// bf16 GEMM on CDNA4 matrix cores (gfx950) for the SP-TP linear layer.
//
// C[M, N] = A[M, K] @ B[K, N], bf16 operands, fp32 accumulation, bf16 (nearest-even) or fp32
// stores.  This one kernel serves both the column-parallel chunk GEMMs of the chunked
// all-gather + matmul and the row-parallel partial-sum GEMM ("Potential Solution" of the
// AReaL async-TP issue; "partial output" in the delayed-TP abstract).
//
// Two kernels, chosen per call (resolve()):
//   * the ring kernel (gemm_ring_kernel, described at its definition): 256 x 256 tiles,
//     v_mfma_f32_16x16x32_bf16, direct-to-LDS loads into a ring of stages.  Its four-wave form
//     runs every 256 x 256 GEMM with K >= 2048 (one workgroup per tile); its eight-wave form
//     runs shorter K (persistent, with the next tile's first stages prefetched);
//   * the register-staged kernel (gemm_bf16_kernel, described next): 128 x 128 tiles for
//     GEMMs too small to fill the chip with 256 x 256 tiles or chunks of 128-row multiples,
//     and the other measured configurations.
//
// Register-staged kernel, design for gfx950:
//   * A workgroup owns a BM x BN output tile; its WGM x WGN wave64s each own a (BM/WGM) x
//     (BN/WGN) block made of 32 x 32 blocks of v_mfma_f32_32x32x16_bf16.
//   * K is walked in stages of 64.  A stage of A ([BM][64]) and B ([64][BN]) sits in LDS,
//     double buffered.  Global loads are buffer loads (one scalar descriptor per operand,
//     32-bit lane offsets, out-of-range offsets read as zero, which handles every ragged
//     edge), staged in registers: the next stage's loads are issued at the top of a stage
//     and written to the other LDS buffer at its end, so one barrier per stage suffices.
//   * A is read as 8 consecutive k per lane (ds_read_b128).  B keeps the weight's [k][n]
//     layout in LDS and is read with the gfx950 transposing LDS read, so no thread ever
//     transposes data in registers.
//   * The instruction order inside a stage is pinned: the stage's global loads, the first
//     step's fragment reads, then each MFMA followed by one fragment read of the next step.
//   * Workgroups are dispatched round-robin over the 8 XCDs; the tile order gives each XCD a
//     contiguous run of tiles so that neighbouring tiles share that XCD's L2.
//   * Every tile configuration uses the same MFMA instruction and visits K in the same
//     ascending order, with no split-K, so the result bits do not depend on tiling or
//     chunking.
//
// ds_read_b64_tr_b16, per group of 16 lanes: source lane r supplies the address of 4
// consecutive bf16; result lane i element j is element (i % 4) of source lane 4 j + i / 4.
// With source lane r pointing at B[kb + r / 4][nb + 4 (r % 4)], result lane i holds
// B[kb + 0..3][nb + i]: four consecutive k of one column, half of an MFMA B operand.
//
// LDS layouts (bytes):
//   A stage: BM rows of 128 bytes (64 k); 16-byte chunk c of row r is stored at
//            c ^ ((r ^ r >> 3) & 7).
//   B stage: 64 rows (k) of 2 BN bytes; 32-byte unit u (16 columns) of row k is stored at
//            u ^ ((k & 3) << 1).  The LDS serves 32 lanes (256 bytes, all 64 banks) per
//            cycle; a transposing read by lanes 0..31 touches rows kb..kb+3 at units u
//            (lanes 0..15) and u + 1 (lanes 16..31), u even, which this map sends to 8
//            distinct 32-byte bank groups.
#include <atomic>
#include <cstdlib>
#include <cstring>

#include "sptl_internal.h"
#include "sptl_tilemap.h"

namespace sptl {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBK = 64;                   // K depth of one LDS stage
constexpr int kRsrcFlags = 0x00020000;    // raw buffer, 32-bit data format
constexpr int kOutOfRange = 0x7ffffff0;   // an offset past any num_records used here

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// The ring kernel's chunk swizzle of a 64-byte row form (A, or an n-major B): 16-byte chunk c of
// row r sits at chunk c ^ ring_aswz(r).  Both the direct-to-LDS loads and the fragment reads use it.
__device__ __forceinline__ int ring_aswz(int r) { return (r >> 1) & 3; }

// The ring kernel's swizzle of a k-major stage (32 rows of 512 bytes): 16-byte piece h of row k
// sits at piece h ^ ring_kswz(k, is_b).  Bits 2-3 take k & 3 and one more bit takes bit 3 of k:
// bit 0 for B (whose fragment reads follow ring_bcol), bit 1 for a k-major A (plain column order).
// Either way the transposing fragment reads of the two lane groups that the LDS serves together
// (rows 8 g .. 8 g + 3, g = 0, 1) fall on different banks: no conflict cycles in a read probe
// (SQ_LDS_BANK_CONFLICT), where the permuted B reads with A's form took 2 per instruction.
__device__ __forceinline__ int ring_kswz(int k, bool is_b) {
    return ((k & 3) << 2) | (((k >> 3) & 1) << (is_b ? 0 : 1));
}

// The ring kernel's B column order.  Block j (16 columns) of a wave's 16 x 16 blocks carries, in
// its MFMA column c, the wave's output column ring_bcol(j, c).  Columns come in runs of 4 (the
// transposing read gives each group of 4 result lanes 4 consecutive columns), and lane group
// g = c / 4 of blocks 2 s and 2 s + 1 together holds the 8 consecutive columns 32 s + 8 g .. + 7,
// which the tile store writes as one 16-byte vector per lane.  Which block of the pair holds the
// first 4 alternates with g, so that a fragment read uses both halves of every 16-byte piece.
__device__ __forceinline__ int ring_bcol(int j, int c) {
    const int g = c >> 2;
    return 32 * (j >> 1) + 8 * g + 4 * ((j + g) & 1) + (c & 3);
}

constexpr int kWaitVmcnt0 = (7 << 4) | (15 << 8);  // s_waitcnt vmcnt(0); expcnt, lgkmcnt not waited

// Release fences whose L2 write-back (buffer_wbl2) has completed before the caller's next memory
// operation is issued.  The compiler follows the write-back with a wait only when some other
// memory operation is still outstanding, so the count or flag store that publishes the data
// could otherwise be performed while the write-back is still running.
__device__ __forceinline__ void release_system() {
    __atomic_thread_fence(__ATOMIC_RELEASE);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
}
__device__ __forceinline__ void release_agent() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
}

// Bounded spins on SDMA completion signals: `words` lists the value words of one chunk's copy
// pieces (n <= 64), each 1 until its piece lands and then <= 0.  The waits are run by one whole
// wave, lane l watching piece l, so one vector load checks every piece.  On timeout a wait sets
// *plan.err and returns, so every wave exits.  The polls are relaxed (coherent loads that bypass
// the caches, no cache invalidation); one acquire fence follows the last poll, so a waiting
// workgroup does not invalidate its L2 while others stream through it.
// A timed-out wait also records the launch's epoch in plan.timedout: the copies it gave up on
// may still be in flight after the launch ends, and the stager drains them before it re-arms
// their signals.  The fence completes that store before this workgroup counts itself done,
// so the host sees it no later than the launch's end word.
__device__ __forceinline__ bool timed_out(uint64_t t0, const ChunkPlan &plan) {
    if (wall_clock64() - t0 <= plan.timeout_ticks) return false;
    __hip_atomic_store(plan.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (plan.timedout) __hip_atomic_store(plan.timedout, plan.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    release_system();
    return true;
}

__device__ __forceinline__ void poll_pause(const ChunkPlan &plan) {
    __builtin_amdgcn_s_sleep(32);
    for (int i = 0; i < plan.poll_sleep; ++i) __builtin_amdgcn_s_sleep(127);
}

// Whether every piece has landed; the same answer in every lane of the calling wave.
__device__ __forceinline__ bool pieces_landed(const int64_t *const *words, int n) {
    const int lane = threadIdx.x & 63;
    const bool mine = lane >= n || __hip_atomic_load(words[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) <= 0;
    return __all(mine);
}

// Called by a whole wave.
__device__ __forceinline__ void wait_ready(const int64_t *const *words, int n, const ChunkPlan &plan) {
    if (!words) return;
    const uint64_t t0 = wall_clock64();
    while (!pieces_landed(words, n)) {
        if (timed_out(t0, plan)) break;
        poll_pause(plan);
    }
    __atomic_thread_fence(__ATOMIC_ACQUIRE);  // system scope: the copied rows are visible
}

// Wait of workgroup `bid` for chunk `chunk` through the replicated landed flags (see
// ChunkPlan), run by the workgroup's first wave; falls back to wait_ready when the launch has
// no flags.
constexpr unsigned kSignalPollEvery = 16;
static_assert(kFlagReplicas <= 64, "one lane per flag replica");

__device__ __forceinline__ void wait_chunk(const ChunkPlan &plan, int chunk, int bid) {
    const int64_t *const *words = plan.ready[chunk];
    if (!words || plan.copy_out) return;
    const int n = plan.ready_n[chunk];
    if (!plan.flags) return wait_ready(words, n, plan);
    const int lane = threadIdx.x & 63;
    uint64_t *mine = plan.flags + (size_t)(bid % kFlagReplicas) * kFlagStride + chunk;
    const uint64_t t0 = wall_clock64();
    for (unsigned it = (unsigned)bid;; ++it) {
        if (__hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == plan.flag_epoch) break;
        if (it % kSignalPollEvery == 0 && pieces_landed(words, n)) {
            __atomic_thread_fence(__ATOMIC_ACQ_REL);  // the flags are set after the landing was seen
            if (lane < kFlagReplicas)
                __hip_atomic_store(plan.flags + (size_t)lane * kFlagStride + chunk, plan.flag_epoch, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_SYSTEM);
            break;
        }
        if (timed_out(t0, plan)) break;
        poll_pause(plan);
    }
    __atomic_thread_fence(__ATOMIC_ACQUIRE);
}

// Lead chunks copied by the launch's own workgroups (ChunkPlan::cu_n), run by the whole
// workgroup: take blocks of the copies until none is left; once the workgroup's stores have
// completed, count its blocks done with an agent-scope release (its XCD's L2 is written back
// first); then wait, with the first wave, until every block is done, and invalidate the caches
// (agent-scope acquire).  A workgroup waits only after the grab counter has run out, so every
// block has been taken by a running workgroup that copies it without waiting for anything: the
// wait ends whatever number of workgroups is resident.
// The workgroup whose count completes the total sets one landed flag for all lead chunks (the
// flag slot of the first of them), and the waiters poll their own replica of it (checking the
// counter itself every kSignalPollEvery polls): up to one wave per CU polling the counter's line
// would slow the counts and grabs next to it.
__device__ __forceinline__ bool cu_copies_done(const ChunkPlan &plan) {
    const int64_t per_chunk = (plan.cu_chunk_bytes + kCuBlockBytes - 1) / kCuBlockBytes;
    return __hip_atomic_load(plan.wg_count + (size_t)kCuDoneLine * kEndLine, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT) >= (uint64_t)(per_chunk * plan.cu_n);
}

__device__ __forceinline__ uint64_t *cu_flag(const ChunkPlan &plan, int replica) {
    return plan.flags + (size_t)replica * kFlagStride + __builtin_ctzll(plan.cu_mask);
}

__device__ __forceinline__ bool cu_flag_set(const ChunkPlan &plan, int bid) {
    return plan.flags &&
           __hip_atomic_load(cu_flag(plan, bid % kFlagReplicas), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) ==
               plan.flag_epoch;
}

__device__ void cu_copy_and_wait(const ChunkPlan &plan, int bid) {
    __shared__ uint64_t grabbed;
    typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
    uint64_t *grab = plan.wg_count + (size_t)kCuGrabLine * kEndLine;
    uint64_t *done = plan.wg_count + (size_t)kCuDoneLine * kEndLine;
    const int64_t per_chunk = (plan.cu_chunk_bytes + kCuBlockBytes - 1) / kCuBlockBytes;
    const uint64_t total = (uint64_t)(per_chunk * plan.cu_n);
    uint64_t mine = 0;
    for (;;) {
        if (threadIdx.x == 0) grabbed = __hip_atomic_fetch_add(grab, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const uint64_t b = grabbed;
        __syncthreads();
        if (b >= total) break;
        const int i = (int)(b / (uint64_t)per_chunk);
        const int64_t off = (int64_t)(b % (uint64_t)per_chunk) * kCuBlockBytes;
        const int64_t len = plan.cu_chunk_bytes - off < kCuBlockBytes ? plan.cu_chunk_bytes - off : kCuBlockBytes;
        const char *src = static_cast<const char *>(plan.cu_src[i]) + off;
        char *dst = static_cast<char *>(plan.cu_dst[i]) + off;
        // a pass issues all of its loads before its stores (8 x 16 bytes per thread: 4 was slower by
        // about 1 us per call at M = 8192, 16 no faster; neither spills in the four-wave form), so
        // each pass waits for memory once
        constexpr int kU = 8;
        const int64_t step = (int64_t)blockDim.x * 16;
        for (int64_t e0 = (int64_t)threadIdx.x * 16; e0 < len; e0 += step * kU) {
            v4u32 v[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (e0 + u * step < len) v[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u32 *>(src + e0 + u * step));
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (e0 + u * step < len)
                    __builtin_nontemporal_store(v[u], reinterpret_cast<v4u32 *>(dst + e0 + u * step));
        }
        ++mine;
    }
    if (mine) {
        // vmcnt(0): this thread's stores have reached the L2 (the barrier's workgroup-scope fence
        // does not wait for them); the release then writes the XCD's L2 back before the count
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
    }
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int completed = 0;
        if (mine && lane == 0) {
            release_agent();
            completed = __hip_atomic_fetch_add(done, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + mine == total;
        }
        if (__shfl(completed, 0, 64) && plan.flags) {
            // this count read every other workgroup's, each made after its release: acquire them,
            // then publish the flags
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            release_agent();
            if (lane < kFlagReplicas)
                __hip_atomic_store(cu_flag(plan, lane), plan.flag_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        const uint64_t t0 = wall_clock64();
        for (unsigned it = (unsigned)bid;; ++it) {
            if (cu_flag_set(plan, bid)) break;
            if ((!plan.flags || it % kSignalPollEvery == 0) && cu_copies_done(plan)) break;
            if (timed_out(t0, plan)) break;
            poll_pause(plan);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

// Non-blocking form of wait_chunk, run by a whole wave: whether chunk `chunk` has landed now
// (setting the landed flags when this wave is the first to see it).  When it returns true the
// copied rows are visible to the workgroup's later loads (after a barrier).
__device__ __forceinline__ bool chunk_ready_now(const ChunkPlan &plan, int chunk, int bid) {
    if ((plan.cu_mask >> chunk) & 1) {
        const bool ok = cu_flag_set(plan, bid) || cu_copies_done(plan);
        if (ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        return ok;
    }
    const int64_t *const *words = plan.ready[chunk];
    if (!words || plan.copy_out) return true;
    const int n = plan.ready_n[chunk];
    bool ok;
    if (plan.flags &&
        __hip_atomic_load(plan.flags + (size_t)(bid % kFlagReplicas) * kFlagStride + chunk, __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_SYSTEM) == plan.flag_epoch) {
        ok = true;
    } else {
        ok = pieces_landed(words, n);
        if (ok && plan.flags) {
            __atomic_thread_fence(__ATOMIC_ACQ_REL);
            const int lane = threadIdx.x & 63;
            if (lane < kFlagReplicas)
                __hip_atomic_store(plan.flags + (size_t)lane * kFlagStride + chunk, plan.flag_epoch, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
    if (ok) __atomic_thread_fence(__ATOMIC_ACQUIRE);
    return ok;
}

// Output tile of this workgroup and, for a chunk-ordered launch, the wait for its chunk.
struct TileOrigin {
    int64_t m0, n0;          // output tile origin
    const uint16_t *a_tile;  // first row of this tile's A rows
    int rows_valid;
    int chunk;               // chunk-ordered launches: the tile's chunk, else -1
};

// Origin of tile `bid` (the workgroup index of a one-tile-per-workgroup launch).
template <int BM, int BN, bool CHUNKED>
__device__ __forceinline__ void tile_origin(const GemmProblem &p, int tiles_m, int tiles_n, TileOrigin &o, int bid) {
    const ChunkPlan &plan = p.plan;
    int64_t &m0 = o.m0, &n0 = o.n0;
    const uint16_t *&a_tile = o.a_tile;
    int &rows_valid = o.rows_valid;
    int &chunk = o.chunk;
    chunk = -1;
    if constexpr (!CHUNKED) {
        // XCD-aware tile order (plain_tile, sptl_tilemap.h)
        int tm, tn;
        plain_tile(tiles_m, tiles_n, bid, tm, tn);
        m0 = (int64_t)tm * BM;
        n0 = (int64_t)tn * BN;
        a_tile = p.a + m0 * p.lda;
        rows_valid = (int)((p.m - m0) < BM ? (p.m - m0) : BM);
    } else {
        // Chunk-ordered: on every XCD the tiles of chunks that land first come first (chunk_tile,
        // sptl_tilemap.h, with the layout chunk_layout chose).  A chunk is a whole number of
        // tile rows.
        int pos, sub, tn;
        chunk_tile(plan.chunk_rows / BM, tiles_n, plan.xcd_group, plan.chunk_band, bid, pos, sub, tn);
        chunk = plan.order[pos];
        m0 = (int64_t)chunk * plan.chunk_rows + (int64_t)sub * BM;
        n0 = (int64_t)tn * BN;
        rows_valid = BM;
        const int own_idx = chunk - plan.own_first;
        a_tile = (own_idx >= 0 && own_idx < plan.own_count)
                     ? plan.own_a + ((int64_t)own_idx * plan.chunk_rows + (int64_t)sub * BM) * p.lda
                     : p.a + m0 * p.lda;
    }
}

// Chunk-ordered launches: the wait of tile `bid` for its chunk (first wave), then a barrier.
template <bool CHUNKED>
__device__ __forceinline__ void tile_wait(const GemmProblem &p, const TileOrigin &o, int bid) {
    if constexpr (CHUNKED) {
        const ChunkPlan &plan = p.plan;
        const int tid = threadIdx.x;
        // the launch has started, so every earlier operation on its stream has completed: the
        // staging worker may start the copies (ForkWait::Started)
        if (plan.started && bid == 0 && tid == 0)
            __hip_atomic_store(plan.started, plan.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        // the timeline's origin: the earliest tile start of the launch (every tile takes part, so
        // no landing can be seen before it)
        if (plan.ts && tid == 0)
            atomicMin(reinterpret_cast<unsigned long long *>(plan.ts + 3 * plan.n_chunks),
                      (unsigned long long)wall_clock64());
        const bool cu = (plan.cu_mask >> o.chunk) & 1;
        if (cu) cu_copy_and_wait(plan, bid);  // the chunk is copied by the launch's own workgroups
        if (tid < 64) {
            if (!cu) wait_chunk(plan, o.chunk, bid);  // this chunk's copy pieces have landed
            if (plan.ts && tid == 0) {
                const unsigned long long now = wall_clock64();
                atomicMin(reinterpret_cast<unsigned long long *>(plan.ts + o.chunk), now);
                atomicMin(reinterpret_cast<unsigned long long *>(plan.ts + plan.n_chunks + o.chunk), now);
            }
        }
        __syncthreads();
    }
}

template <int BM, int BN, bool CHUNKED>
__device__ __forceinline__ void tile_begin(const GemmProblem &p, int tiles_m, int tiles_n, TileOrigin &o) {
    tile_origin<BM, BN, CHUNKED>(p, tiles_m, tiles_n, o, blockIdx.x);
    tile_wait<CHUNKED>(p, o, blockIdx.x);
}

// The end count of workgroup bid (lane 0): its end group's counter value before the count, low 32
// bits (a call's counts on a set lie within 2^32 below grp_last, so they compare exactly).
__device__ __forceinline__ uint32_t end_count(const ChunkPlan &plan, int bid) {
    return (uint32_t)__hip_atomic_fetch_add(plan.wg_count + (bid % kEndGroups) * kEndLine, 1ull, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
}

// EARLY: the workgroup counted itself already (end_count's value grp_v, wave-uniform).
template <bool CHUNKED, bool EARLY = false>
__device__ __forceinline__ void tile_finish(const GemmProblem &p, const TileOrigin &o, int bid, uint32_t grp_v = 0);

// Stores the tile's accumulators (32 x 32 MFMA result layout) and, for a chunk-ordered launch,
// records the tile's end and completes the call when this is its last tile.
template <int BM, int BN, int WGM, int WGN, bool OUT_F32, bool CHUNKED>
__device__ __forceinline__ void tile_end(const GemmProblem &p, const TileOrigin &o,
                                         const f32x16_t (&acc)[BM / WGM / 32][BN / WGN / 32], int bid) {
    constexpr int TM = BM / WGM / 32, TN = BN / WGN / 32;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm0 = (wave / WGN) * (BM / WGM), wn0 = (wave % WGN) * (BN / WGN);
    const int64_t m0 = o.m0, n0 = o.n0;
    // 32 x 32 MFMA result layout: lane l holds column l % 32; register r holds row
    // 8 (r / 4) + 4 (l / 32) + r % 4.
    if constexpr (OUT_F32) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t col = n0 + wn0 + j * 32 + (lane & 31);
                if (col >= p.n) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = m0 + wm0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                    if (row < p.m) static_cast<float *>(p.c)[row * p.ldc + col] = acc[i][j][r];
                }
            }
        }
    } else {
        // bf16: lanes 2 q and 2 q + 1 hold adjacent columns.  One DPP swap per pair of values
        // gives the even lane both columns of rows r = 0..7 and the odd lane both columns of
        // rows r = 8..15, so every store writes two columns (4 bytes; N is a multiple of 8, so
        // the pair is whole).  The conversion is the native nearest-even one, two values at a
        // time.
        const bool odd = lane & 1;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t col = n0 + wn0 + j * 32 + (lane & 31 & ~1);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float send = odd ? acc[i][j][k] : acc[i][j][k + 8];
                    const float recv = __builtin_bit_cast(
                        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, false));
                    const float mine = odd ? acc[i][j][k + 8] : acc[i][j][k];
                    const int r = odd ? k + 8 : k;
                    const int64_t row = m0 + wm0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                    bf16x2_t v;
                    v[0] = (__bf16)(odd ? recv : mine);
                    v[1] = (__bf16)(odd ? mine : recv);
                    if (row < p.m && col < p.n)
                        *reinterpret_cast<bf16x2_t *>(static_cast<uint16_t *>(p.c) + row * p.ldc + col) = v;
                }
            }
        }
    }
    tile_finish<CHUNKED>(p, o, bid);
}

// Chunk-ordered launches: records the tile's end and completes the call when this is its last
// tile.
template <bool CHUNKED, bool EARLY>
__device__ __forceinline__ void tile_finish(const GemmProblem &p, const TileOrigin &o, int bid, uint32_t grp_v) {
    if (CHUNKED && p.plan.copy_out && p.plan.ready[o.chunk]) {
        // A slice that is copied out (see ChunkPlan): every wave waits until its stores of the
        // tile have reached the L2 (vmcnt 0: the barrier's workgroup-scope fence does not wait
        // for them); then the first thread counts the tile, and the XCD's last tile of the slice
        // writes the L2 back (system-scope release: the copy engines read memory, not the L2).
        // The slice is released once slice_last + 1 XCDs have each counted slice_xcd_last + 1
        // tiles, which is every tile of the slice: so each tile's rows were written back after
        // its stores, wherever it ran.  Any other placement ends in the report below or in the
        // bounded wait for the copies, never in a release before a write-back.
        const ChunkPlan &plan = p.plan;
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (threadIdx.x == 0) {
            uint64_t *line = plan.slice_count + (size_t)o.chunk * kEndLine;
            bool last = true;
            if (plan.flush_each_tile) {
                release_system();  // this tile's rows, from its own L2
            } else {
                // counted under the XCD it runs on (the hardware's XCC id): the host's per-XCD share
                // holds for any rotation of the round-robin placement
                unsigned xcc;
                asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(xcc));
                const uint64_t v = __hip_atomic_fetch_add(line + 1 + (xcc & 7), 1ull, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
                if (v > (uint64_t)plan.slice_xcd_last[o.chunk])  // more tiles on this XCD than counted
                    __hip_atomic_store(plan.err + 2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                last = v == (uint64_t)plan.slice_xcd_last[o.chunk];
                if (last) release_system();  // every tile of the slice that ran here
            }
            // The count that completes the slice reads every other XCD's count, each made after
            // that XCD's release: an acquire here makes their rows happen before the ready store.
            if (last && __hip_atomic_fetch_add(line, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                            plan.slice_last[o.chunk]) {
                __atomic_thread_fence(__ATOMIC_ACQUIRE);
                release_system();
                __hip_atomic_store(plan.slice_ready + 16 * (size_t)o.chunk, plan.epoch, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_SYSTEM);
            }
        }
    }
    if (CHUNKED && threadIdx.x < 64) {
        const ChunkPlan &plan = p.plan;
        const int chunk = o.chunk;
        // The last workgroup to finish waits for every copy of the call (own slot included),
        // so the kernel ends only after all of them, then reports the call done.  The counts
        // are relaxed: a workgroup counts itself after its chunk wait has returned, so a full
        // count means that no workgroup of the call still reads the set's signals or flags,
        // which is all the report promises (the outputs are ordered by the kernel's end).  A
        // release or acquire per workgroup would write back or invalidate its L2 each time.
        // Lane 0 counts; the first wave then waits for the join together.
        int last = 0;
        if (threadIdx.x == 0) {
            if (plan.ts)
                atomicMax(reinterpret_cast<unsigned long long *>(plan.ts + 2 * plan.n_chunks + chunk),
                          (unsigned long long)wall_clock64());
            const int g = bid % kEndGroups;
            const uint32_t v = EARLY ? grp_v : end_count(plan, bid);
            last = v == (uint32_t)plan.grp_last[g] &&
                   __hip_atomic_fetch_add(plan.wg_count + kEndGroups * kEndLine, 1ull, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == plan.all_last;
        }
        if (__shfl(last, 0, 64)) {
            wait_ready(plan.join, plan.join_n, plan);
            if (plan.copy_out)
                for (int c = 0; c < plan.n_chunks; ++c) wait_ready(plan.ready[c], plan.ready_n[c], plan);
            if (threadIdx.x == 0) {
                if (plan.cu_n) {  // every tile has taken its last block: the set's next call starts at zero
                    __hip_atomic_store(plan.wg_count + (size_t)kCuGrabLine * kEndLine, 0ull, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(plan.wg_count + (size_t)kCuDoneLine * kEndLine, 0ull, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
                release_system();
                __hip_atomic_store(plan.finished, plan.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            }
        }
    }
}

// Stores the accumulators of a ring-kernel tile, then as tile_end.  The ring kernel computes each
// 16 x 16 block transposed (B's fragment is the MFMA's first operand: the same products, summed
// over the same k, so the same bits), and in the 16 x 16 result layout lane l then holds output
// row 16 i + l % 16 of block row i, register e of block j its column ring_bcol(j, 4 (l / 16) + e).
// So lane group g = l / 16 holds, over blocks 2 s and 2 s + 1, the 8 consecutive columns
// 32 s + 8 g .. + 7 of its row: one 16-byte store per lane (two for fp32) writes 64 contiguous
// bytes of each of 16 rows, a quarter of the store instructions of one 4-byte store per
// adjacent pair of columns.  Block 2 s + (g & 1) holds the first 4 of them.
template <int BM, int BN, int WGM, int WGN, bool OUT_F32, bool CHUNKED, bool EARLY = false>
__device__ __forceinline__ void tile_end16(const GemmProblem &p, const TileOrigin &o,
                                           const f32x4_t (&acc)[BM / WGM / 16][BN / WGN / 16], int bid,
                                           uint32_t grp_v = 0) {
    constexpr int TM = BM / WGM / 16, TN = BN / WGN / 16;
    static_assert(TN % 2 == 0, "column pairs of blocks");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm0 = (wave / WGN) * (BM / WGM), wn0 = (wave % WGN) * (BN / WGN);
    const int g = lane >> 4;
    const bool second = g & 1;  // the pair's second block holds the first 4 columns
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t row = o.m0 + wm0 + i * 16 + (lane & 15);
#pragma unroll
        for (int s = 0; s < TN / 2; ++s) {
            const int64_t col = o.n0 + wn0 + 32 * s + 8 * g;  // N is a multiple of 8: all 8 or none
            f32x4_t lo, hi;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lo[e] = second ? acc[i][2 * s + 1][e] : acc[i][2 * s][e];
                hi[e] = second ? acc[i][2 * s][e] : acc[i][2 * s + 1][e];
            }
            if (row < p.m && col < p.n) {
                if constexpr (OUT_F32) {
                    float *c = static_cast<float *>(p.c) + row * p.ldc + col;
                    *reinterpret_cast<f32x4_t *>(c) = lo;
                    *reinterpret_cast<f32x4_t *>(c + 4) = hi;
                } else {
                    bf16x8_t v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[e] = (__bf16)lo[e];
                        v[4 + e] = (__bf16)hi[e];
                    }
                    *reinterpret_cast<bf16x8_t *>(static_cast<uint16_t *>(p.c) + row * p.ldc + col) = v;
                }
            }
        }
    }
    tile_finish<CHUNKED, EARLY>(p, o, bid, grp_v);
}

template <int BM, int BN, int WGM, int WGN, int BK>
struct Cfg {
    static constexpr int THREADS = 64 * WGM * WGN;
    static constexpr int WM = BM / WGM, WN = BN / WGN;      // one wave's block
    static constexpr int TM = WM / 32, TN = WN / 32;        // 32 x 32 MFMA blocks per wave
    static constexpr int A_ROW = BK * 2;                    // bytes per A row in LDS
    static constexpr int CPR = BK / 8;                      // 16-byte chunks per A row
    static constexpr int A_STAGE = BM * A_ROW;              // bytes
    static constexpr int B_STAGE = BN * 2 * BK;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int B_ROW = BN * 2;                    // bytes per B row in LDS
    static constexpr int A_VEC = BM * BK / 8 / THREADS;     // 16-byte A vectors per thread
    static constexpr int B_VEC = BN * BK / 8 / THREADS;
    // transposed-B staging: one thread per 8 k x 8 n block of B, the other threads A only
    static constexpr int BT_B_THREADS = (BK / 8) * (BN / 8);
    static constexpr int BT_VEC = 8;                          // 16-byte loads per thread
    static_assert(BK == 64 || BK == 32, "stage depth");
    static_assert(TM >= 1 && TN >= 1 && A_VEC >= 1 && B_VEC >= 1, "tile shape");
    static_assert(BN >= 128, "B swizzle needs at least 8 units of 32 bytes per row");
    // A chunk swizzle: 64-k rows (8 chunks) use c ^ ((r ^ r >> 3) & 7); 32-k rows (4 chunks)
    // use c ^ ((r >> 2) & 3).  Either way 16 lanes reading one chunk of 16 consecutive rows
    // hit 16 distinct 16-byte bank groups.
    static __device__ __forceinline__ int aswz(int r) { return BK == 64 ? swz(r) : (r >> 2) & 3; }
};

// BT: B is transposed on its way into LDS (see load_stage), so that B fragments, like A
// fragments, are single ds_read_b128s of 8 consecutive k.  On gfx950 the LDS issues about one
// instruction per 4-5 clocks per CU whatever its width, so this cuts the LDS instructions per
// MFMA from 1.5 to 1.0.  The fragments, the MFMA instruction and the K order are unchanged,
// so the result bits are the same.
// LSPREAD: 0 issues a stage's global loads before its first MFMA; n > 0 issues one load after
// every n-th MFMA instead, so that the CU's vector-memory queue sees a steady stream rather
// than every wave's loads at once.
template <int BM, int BN, int WGM, int WGN, bool OUT_F32, bool CHUNKED, int BK = kBK, int WPE = 1, bool BT = false,
          int LSPREAD = 0>
__global__ void __launch_bounds__(64 * WGM * WGN, WPE)
gemm_bf16_kernel(GemmProblem p, int tiles_m, int tiles_n) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer resources exist only in the device pass
    using T = Cfg<BM, BN, WGM, WGN, BK>;
    constexpr int A_VEC = BT ? T::BT_VEC : T::A_VEC, B_VEC = BT ? 0 : T::B_VEC;
    static_assert(!BT || (T::THREADS == 2 * T::BT_B_THREADS && BK == 64), "transposed-B thread split");
    __shared__ __attribute__((aligned(1024))) char smem[2 * T::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // BT: the first half of the waves stage B blocks, the second half A rows (wave-uniform)
    const bool b_role = BT && __builtin_amdgcn_readfirstlane(wave) < T::BT_B_THREADS / 64;
    const int wm0 = (wave / WGN) * T::WM;
    const int wn0 = (wave % WGN) * T::WN;

    TileOrigin o;
    tile_begin<BM, BN, CHUNKED>(p, tiles_m, tiles_n, o);
    const int64_t m0 = o.m0, n0 = o.n0;
    const uint16_t *a_tile = o.a_tile;
    const int rows_valid = o.rows_valid;

    // Global -> register staging.  Thread t loads A vectors q = t + THREADS i (row q / CPR,
    // 16-byte chunk q % CPR) and B vectors q = t + THREADS i (row q / (BN / 8), columns
    // 8 (q % (BN / 8)) ..).
    //
    // BT: thread t < BT_B_THREADS owns the 8 x 8 block of k rows 8 (t / (BN / 8)) .. + 7 and
    // columns 8 (t % (BN / 8)) .. + 7: it loads the block's 8 rows (A_VEC loads of 16 bytes),
    // transposes it in registers and writes 8 columns of 8 consecutive k.  LDS then holds B
    // as BN rows (n) of BK k, with the A layout and swizzle.  The other threads load A
    // vectors q = (t - BT_B_THREADS) + (THREADS - BT_B_THREADS) i.
    //   Offsets are kept per role as one base plus a stride: load i of a B thread reads k row
    //   8 rg + i (stride ldb), load i of an A thread reads row r0 + 32 i (stride 32 lda); the
    //   LDS address of B column cb 8 + j is (bt_lds ^ (j << 4)) + 128 j (the swizzle of column
    //   8 cb + j is rg ^ cb ^ j), of A row r0 + 32 i is bt_lds + 4096 i with the row's swizzle,
    //   which alternates with i.
    int a_voff[BT ? 1 : A_VEC], a_kc[BT ? 1 : A_VEC], a_lds[BT ? 2 : A_VEC];
    int bt_stride = 0;
    if constexpr (BT) {
        const int cb = tid % (BN / 8), rg = (tid / (BN / 8)) & 7;
        const int bq = (tid - T::BT_B_THREADS) & (T::THREADS - T::BT_B_THREADS - 1);
        const int r0 = bq / T::CPR, c = bq % T::CPR;  // A: rows r0 + 32 i, chunk c
        const int64_t n = n0 + cb * 8;
        bt_stride = b_role ? (int)(p.ldb * 2) : (int)(32 * p.lda * 2);
        a_kc[0] = c * 8;
        a_voff[0] = b_role ? (n < p.n ? (int)((rg * 8 * p.ldb + n) * 2) : kOutOfRange) : (int)((r0 * p.lda + c * 8) * 2);
        a_lds[0] = b_role ? T::A_STAGE + cb * 8 * T::A_ROW + (((rg ^ cb) & 7) << 4)
                          : r0 * T::A_ROW + ((c ^ T::aswz(r0)) << 4);
        a_lds[1] = r0 * T::A_ROW + ((c ^ T::aswz(r0 + 32)) << 4);  // A rows r0 + 32 (odd i)
    } else {
#pragma unroll
        for (int i = 0; i < A_VEC; ++i) {
            const int q = tid + i * T::THREADS;
            const int row = q / T::CPR, c = q % T::CPR;
            a_kc[i] = c * 8;
            a_voff[i] = (int)((row * p.lda + c * 8) * 2);
            a_lds[i] = row * T::A_ROW + ((c ^ T::aswz(row)) << 4);
        }
    }
    int b_voff[B_VEC > 0 ? B_VEC : 1], b_lds[B_VEC > 0 ? B_VEC : 1];
#pragma unroll
    for (int i = 0; i < B_VEC; ++i) {
        const int q = tid + i * T::THREADS;
        const int row = q / (BN / 8), piece = q % (BN / 8);
        const int64_t n = n0 + piece * 8;
        b_voff[i] = n < p.n ? (int)((row * p.ldb + n) * 2) : kOutOfRange;
        b_lds[i] = row * T::B_ROW + (((piece >> 1) ^ ((row & 3) << 1)) << 5) + ((piece & 1) << 4);
    }
    u32x4_t ra[A_VEC], rb[B_VEC > 0 ? B_VEC : 1];

    const int nk = (int)((p.k + BK - 1) / BK);
    // Loads stage kt into registers.  Stages past the end (kt >= nk) get an empty buffer
    // range and read zeros, which keeps the loop free of branches.
    auto load_stage = [&](int kt) {
        const bool live = kt < nk;
        const int64_t k0 = live ? (int64_t)kt * BK : 0;
        const int64_t a_bytes = live ? ((int64_t)rows_valid * p.lda - k0) * 2 : 0;
        __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a_tile + k0), (short)0, (int)a_bytes, kRsrcFlags);
        const bool k_tail = k0 + BK > p.k;
        const int64_t k_rows = !live ? 0 : (p.k - k0) < BK ? (p.k - k0) : BK;
        __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(p.b + k0 * p.ldb), (short)0, (int)(k_rows * p.ldb * 2), kRsrcFlags);
        if constexpr (BT) {
            // one descriptor per wave: B rows past K lie beyond br's range and read zero
            const __amdgpu_buffer_rsrc_t r = b_role ? br : ar;
            // A chunk past K, or B columns past N: every load of the thread reads zero
            // (kOutOfRange + 7 strides stays below 2^32, so it stays out of range)
            const int base = !b_role && k_tail && k0 + a_kc[0] >= p.k ? kOutOfRange : a_voff[0];
#pragma unroll
            for (int i = 0; i < A_VEC; ++i)
                ra[i] = __builtin_bit_cast(u32x4_t,
                                           __builtin_amdgcn_raw_buffer_load_b128(r, base + i * bt_stride, 0, 0));
        } else {
#pragma unroll
            for (int i = 0; i < A_VEC; ++i) {
                const int off = (k_tail && k0 + a_kc[i] >= p.k) ? kOutOfRange : a_voff[i];
                ra[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ar, off, 0, 0));
            }
#pragma unroll
            for (int i = 0; i < B_VEC; ++i)
                rb[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(br, b_voff[i], 0, 0));
        }
    };
    auto store_stage = [&](char *dst) {
        if constexpr (BT) {
            if (b_role) {
                // 8 x 8 transpose of 16-bit elements: ra[i] holds k row i (columns 0..7, two per
                // word); column j's word w takes element j of rows 2 w and 2 w + 1.  Each column
                // is stored as soon as it is formed.
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    u32x4_t t;
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        t[w] = __builtin_amdgcn_perm(ra[2 * w + 1][j >> 1], ra[2 * w][j >> 1],
                                                     (j & 1) ? 0x07060302u : 0x05040100u);
                    *reinterpret_cast<u32x4_t *>(dst + ((a_lds[0] ^ (j << 4)) + j * T::A_ROW)) = t;
                }
            } else {
#pragma unroll
                for (int i = 0; i < A_VEC; ++i)
                    *reinterpret_cast<u32x4_t *>(dst + a_lds[i & 1] + i * 32 * T::A_ROW) = ra[i];
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < A_VEC; ++i) *reinterpret_cast<u32x4_t *>(dst + a_lds[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_VEC; ++i) *reinterpret_cast<u32x4_t *>(dst + T::A_STAGE + b_lds[i]) = rb[i];
    };

    // fragment read offsets
    const int a_hi = lane >> 5;
    int a_row_off[T::TM], a_swz[T::TM];
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
        const int r = wm0 + i * 32 + (lane & 31);
        a_row_off[i] = r * T::A_ROW;
        a_swz[i] = T::aswz(r);
    }
    const int rr = lane & 15;
    const int b_k0 = 8 * (lane >> 5) + (rr >> 2);  // k within a 16-k step, first half
    int b_col_off[T::TN], bt_row_off[T::TN], bt_swz[T::TN];
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
        const int n = wn0 + j * 32 + 16 * ((lane >> 4) & 1) + 4 * (rr & 3);
        b_col_off[j] = (((n >> 4) ^ ((b_k0 & 3) << 1)) << 5) + (n & 15) * 2;
        const int nt = wn0 + j * 32 + (lane & 31);  // BT: lane l reads column l % 32
        bt_row_off[j] = nt * T::A_ROW;
        bt_swz[j] = T::aswz(nt);
    }

    f32x16_t acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto load_frags = [&](const char *as, const char *bs, int s, bf16x8_t *af, bf16x8_t *bfr) {
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            const int ch = (2 * s + a_hi) ^ a_swz[i];
            af[i] = *reinterpret_cast<const bf16x8_t *>(as + a_row_off[i] + ch * 16);
        }
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            if constexpr (BT) {
                const int ch = (2 * s + a_hi) ^ bt_swz[j];
                bfr[j] = *reinterpret_cast<const bf16x8_t *>(bs + bt_row_off[j] + ch * 16);
            } else {
                const char *base = bs + (s * 16 + b_k0) * T::B_ROW + b_col_off[j];
                bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(base));
                bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(base + 4 * T::B_ROW));
                bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
    };

    // MFMAs of one stage on `cur`, with the fragments of step s + 1 read during step s.
    auto compute_stage = [&](const char *cur) {
        const char *as = cur;
        const char *bs = cur + T::A_STAGE;
        bf16x8_t af[2][T::TM], bfr[2][T::TN];
        load_frags(as, bs, 0, af[0], bfr[0]);
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            if (s + 1 < BK / 16) load_frags(as, bs, s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][i], bfr[s & 1][j],
                                                                        acc[i][j], 0, 0, 0);
        }
    };
    // Instruction order of a stage (see the file comment).
    auto pin_schedule = [&]() {
        constexpr int kDsPerStep = T::TM + (BT ? 1 : 2) * T::TN;
        constexpr int kMfmaPerStep = T::TM * T::TN;
        constexpr int kSteps = BK / 16;
        constexpr int kLoads = A_VEC + B_VEC;
        if (LSPREAD == 0) __builtin_amdgcn_sched_group_barrier(0x020, kLoads, 0);  // global loads first
        __builtin_amdgcn_sched_group_barrier(0x100, kDsPerStep, 0);
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
#pragma unroll
            for (int m = 0; m < kMfmaPerStep; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (s + 1 < kSteps && m < kDsPerStep) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                const int q = s * kMfmaPerStep + m;
                if (LSPREAD > 0 && q % (LSPREAD > 0 ? LSPREAD : 1) == 0 && q / (LSPREAD > 0 ? LSPREAD : 1) < kLoads)
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
    };

    load_stage(0);
    store_stage(smem);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        char *cur = smem + (kt & 1) * T::STAGE;
        char *nxt = smem + ((kt & 1) ^ 1) * T::STAGE;
        load_stage(kt + 1);
        compute_stage(cur);
        pin_schedule();
        store_stage(nxt);
        __syncthreads();
    }

    tile_end<BM, BN, WGM, WGN, OUT_F32, CHUNKED>(p, o, acc, blockIdx.x);
#endif
}

// A raw buffer descriptor (V#) for `bytes` bytes from `base`: 32-bit data format, no
// stride, so out-of-range lane offsets read zero.
__device__ __forceinline__ u32x4_t buffer_desc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    u32x4_t d;
    d.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
    d.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
    d.z = __builtin_amdgcn_readfirstlane(bytes);
    d.w = (uint32_t)kRsrcFlags;
    return d;
}

__device__ __forceinline__ uint32_t lds_addr(const char *p) {
    return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char *)p);
}

// buffer_load_dwordx4 ... lds: lane l's 16 bytes land at LDS byte lds + 16 l.  Written as
// inline assembly so that the compiler, which cannot tell which ring slot a load writes,
// does not wait for every load before each LDS read; the kernel waits explicitly.
__device__ __forceinline__ void load_to_lds(u32x4_t desc, uint32_t lds, int voffset) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voffset), "s"(desc), "{m0}"(lds) : "memory");
}

constexpr int kDmaBK = 32;
constexpr int kDmaSlotBytes = 256 * kDmaBK * 2;  // 16 KB per operand per stage

// s_waitcnt with only the vector-memory count set (expcnt and lgkmcnt at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Ring kernel: the 256 x 256 tile with WGM x WGN waves, K walked in 32-deep stages held in a
// ring of SLOTS LDS slots that direct-to-LDS buffer loads fill (64 lanes x 16 bytes = 1 KB per
// instruction, lane l at byte 16 l), so no register staging and no LDS store instructions are
// needed.  Stage kt + 1 is made visible (own loads waited for, then a barrier) at the top of
// stage kt, and its fragments are read during stage kt, one stage (32 MFMAs per wave) before
// their use, which covers the LDS latency of a CU whose 8 waves all read at once.  Two fragment
// register sets alternate, so the loop is unrolled twice.
//
// MFMA: v_mfma_f32_16x16x32_bf16, one per 16 x 16 block and 32-deep stage.  Its products and
// sums are those of two v_mfma_f32_32x32x16_bf16 steps over the same 32 k (bit-identical
// results, checked against every other configuration), and it moves less accumulator data per
// flop, which at the chip's power limit lets the clock run higher (about 10 % more GEMM
// throughput with random operands).  Each block is computed transposed, B's fragment as the
// first operand, and B's columns are taken in the order ring_bcol: a lane then ends the tile
// holding runs of 8 consecutive output columns of one row, which it stores as 16-byte vectors
// (tile_end16).
//
// Four waves (WGM = WGN = 2): each wave owns 128 x 128 (8 x 8 blocks), so a stage's fragment
// reads are a third fewer bytes per MFMA than with eight waves of 64 x 128.  Its 256
// accumulator registers per lane live in the AGPRs: the MFMAs are written as inline assembly
// with the accumulator tied to an AGPR operand (with the builtin, the register allocator
// permutes the accumulators between AGPRs and VGPRs at the loop head every iteration).  With
// one wave per SIMD, each stage interleaves its work so that the matrix core always has MFMAs
// queued: the barrier comes after the first column block of MFMAs (which need only registers),
// and after each column block follow one of the stage's global loads and the next stage's
// fragment reads for that block (the A fragments, all of which the next stage's first block
// needs, in the first half).
//
// Persistent: workgroup b takes tiles b, b + G, b + 2 G, ... (G = gridDim.x, a multiple of 8,
// so every tile keeps the XCD of a one-tile-per-workgroup launch).  The ring runs on across
// tiles: SLOTS - 1 stages before the end of a tile its first wave checks, without waiting,
// whether the next tile's chunk has landed; if it has, the ring's next SLOTS - 1 stages are
// the next tile's first stages, so the next tile starts with its data in LDS.  If it has not,
// those stages read zeros and the next tile waits and loads as the first one does.
//
// The per-lane global addresses apply the LDS swizzles in reverse:
//   A slot: 256 rows of 64 bytes; 16-byte chunk c of row r at c ^ ((r >> 1) & 3): a fragment
//           read (16 rows x 4 chunks per ds_read_b128) then runs without bank conflicts, 4 LDS
//           cycles per instruction (measured by SQ_LDS_BANK_CONFLICT; c ^ ((r >> 2) & 3) and
//           the other row-bit swizzles took 8, half of them conflict stalls);
//   B slot: 32 rows (k) of 512 bytes; 16-byte piece h of row k at h ^ ring_kswz(k) (the
//           transposing reads of a fragment take rows 8 g .. 8 g + 3 in lane group g; bit 3 of k
//           keeps groups 0 and 1, which the LDS serves together, on different banks).
// Same K order as every other configuration.
//
// Operand layouts (LAYOUT, GemmProblem::layout): kLayoutRowMajor as above; kLayoutAKMajor, A
// stored k-major (element (i, k) at a[k lda + i], the transposed activation of a weight
// gradient): its stage is staged and read exactly like B's (32 k rows of 256 values, transposing
// fragment reads); kLayoutBNMajor, B stored n-major (element (k, j) at b[j ldb + k], the
// transposed weight of an input gradient): its stage is staged and read like A's (256 rows of 32
// k, one ds_read_b128 per fragment).  The MFMA sees the same fragments either way, so the K
// order, and every product and sum, are those of the row-major form.
template <int WGM, int WGN, int SLOTS, bool OUT_F32, bool CHUNKED, int LAYOUT = kLayoutRowMajor>
__global__ void __launch_bounds__(64 * WGM * WGN)
gemm_ring_kernel(GemmProblem p, int tiles_m, int tiles_n) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr bool A_KM = LAYOUT == kLayoutAKMajor, B_NM = LAYOUT == kLayoutBNMajor;
    static_assert(!CHUNKED || LAYOUT == kLayoutRowMajor, "chunk-ordered launches are row-major");
    constexpr int BM = 256, BN = 256, TM = BM / WGM / 16, TN = BN / WGN / 16;  // 16 x 16 blocks per wave
    constexpr int NBLK = 16 / (WGM * WGN);   // 1 KB blocks per operand per wave per stage
    constexpr bool kFour = WGM * WGN == 4;   // the four-wave form (AGPR accumulators)
    static_assert(NBLK * WGM * WGN == 16 && SLOTS >= 4 && SLOTS * 2 * kDmaSlotBytes <= 160 * 1024, "shape");
    static_assert(!kFour || (TN == 2 * NBLK && TM % 2 == 0 && TM / 2 <= TN), "four-wave stage layout");
    // The four-wave form keeps its accumulators in AGPRs; naming one here makes the compiler
    // allocate them (it assumes none are used otherwise).
    if constexpr (kFour) asm volatile("; agprs in use" ::: "a0");
    constexpr int B_ROW = BN * 2;
    constexpr int SLOT = 2 * kDmaSlotBytes;  // ring slot: A (16 KB) then B (16 KB)
    __shared__ __attribute__((aligned(1024))) char smem[SLOTS * SLOT];
    __shared__ int next_ok_lds;              // the first wave's prefetch decision

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm0 = (wave / WGN) * (BM / WGM);
    const int wn0 = (wave % WGN) * (BN / WGN);
    const int nt = tiles_m * tiles_n;
    const int nk = (int)((p.k + kDmaBK - 1) / kDmaBK);

    // Per-lane offsets of this wave's NBLK row-form blocks (16 rows of 32 k each) of a stage,
    // relative to the operand tile's origin (A, or with B_NM the n-major B); the k-major form's
    // blocks (2 k-rows each) are addressed in load_kmajor.
    int a_off[NBLK], b_off[B_NM ? NBLK : 1], r_kc[NBLK];
#pragma unroll
    for (int t = 0; t < NBLK; ++t) {
        const int blk = wave * NBLK + t;
        const int row = blk * 16 + (lane >> 2);
        const int c = (lane & 3) ^ ring_aswz(row);
        r_kc[t] = c * 8;
        a_off[t] = (int)((row * p.lda + c * 8) * 2);
        if constexpr (B_NM) b_off[t] = (int)((row * p.ldb + c * 8) * 2);
    }
    const uint32_t lds0 = lds_addr(smem) + (uint32_t)(wave * NBLK) * 1024;  // this wave's first block
    // Load t of a stage's row-form blocks (16 rows, one 16-byte piece of k per lane).
    auto load_rows = [&](const u32x4_t &r, uint32_t l, int t, bool k_tail, int64_t k0, const int *off)
        __attribute__((always_inline)) {
        load_to_lds(r, l + t * 1024, (k_tail && k0 + r_kc[t] >= p.k) ? kOutOfRange : off[t]);
    };
    // Load t of a stage's k-major blocks: k-rows 2 blk, 2 blk + 1 (lane / 32); lane q writes
    // 16-byte piece q of that row, which holds piece q ^ ring_kswz(k) of the operand's row
    // (recomputed here rather than kept in registers across the tiles).  x0: the tile's first
    // column (of B, or with A_KM the tile's first row of the output), x_end: the operand's column
    // count, ld: its row stride.
    auto load_kmajor = [&](const u32x4_t &r, uint32_t l, int t, int64_t x0, int64_t x_end, int64_t ld, bool is_b)
        __attribute__((always_inline)) {
        const int krow = (wave * NBLK + t) * 2 + (lane >> 5);
        const int q = lane & 31;
        const int64_t x = x0 + 8 * (q ^ ring_kswz(krow, is_b));
        load_to_lds(r, l + t * 1024, x < x_end ? (int)((krow * ld + x) * 2) : kOutOfRange);
    };
    auto load_a = [&](const u32x4_t &ar, uint32_t la, int t, bool k_tail, int64_t k0, const TileOrigin &o)
        __attribute__((always_inline)) {
        if constexpr (A_KM) load_kmajor(ar, la, t, o.m0, p.m, p.lda, false);
        else load_rows(ar, la, t, k_tail, k0, a_off);
    };
    auto load_b = [&](const u32x4_t &br, uint32_t lb, int t, bool k_tail, int64_t k0, const TileOrigin &o)
        __attribute__((always_inline)) {
        if constexpr (B_NM) load_rows(br, lb, t, k_tail, k0, b_off);
        else load_kmajor(br, lb, t, o.n0, p.n, p.ldb, true);
    };
    // Buffer ranges of stage k0 (k_rows of its 32 k exist; 0 for an empty stage).  Row form:
    // from the tile's first row at k0 to the end of its last valid row (rows and k past the end
    // read zeros).  k-major form: the stage's k_rows rows of the whole operand.
    auto a_desc = [&](const TileOrigin &o, bool live, int64_t k0, int64_t k_rows) __attribute__((always_inline)) {
        if constexpr (A_KM) return buffer_desc(p.a + k0 * p.lda, (uint32_t)(k_rows * p.lda * 2));
        else return buffer_desc(o.a_tile + k0, (uint32_t)(live ? ((int64_t)o.rows_valid * p.lda - k0) * 2 : 0));
    };
    auto b_desc = [&](const TileOrigin &o, bool live, int64_t k0, int64_t k_rows) __attribute__((always_inline)) {
        if constexpr (B_NM) {
            const int64_t cols = (p.n - o.n0) < BN ? (p.n - o.n0) : BN;
            return buffer_desc(p.b + o.n0 * p.ldb + k0, (uint32_t)(live ? (cols * p.ldb - k0) * 2 : 0));
        } else {
            return buffer_desc(p.b + k0 * p.ldb, (uint32_t)(k_rows * p.ldb * 2));
        }
    };

    // Stage kt of the tile at `o` into ring slot `slot`; live = false (or kt >= nk) reads an
    // empty range (zeros), so every stage issues exactly 2 NBLK loads per wave and the wait
    // counts stay fixed.
    auto issue = [&](const TileOrigin &o, bool live_tile, int kt, int slot) {
        const bool live = live_tile && kt < nk;
        const int64_t k0 = live ? (int64_t)kt * kDmaBK : 0;
        const bool k_tail = k0 + kDmaBK > p.k;
        const int64_t k_rows = !live ? 0 : (p.k - k0) < kDmaBK ? (p.k - k0) : kDmaBK;
        const u32x4_t ar = a_desc(o, live, k0, k_rows);
        const u32x4_t br = b_desc(o, live, k0, k_rows);
        const uint32_t la = lds0 + (uint32_t)(slot * SLOT), lb = la + kDmaSlotBytes;
#pragma unroll
        for (int t = 0; t < NBLK; ++t) load_a(ar, la, t, k_tail, k0, o);
#pragma unroll
        for (int t = 0; t < NBLK; ++t) load_b(br, lb, t, k_tail, k0, o);
    };

    // Fragment read addresses within a slot.  A block i (16 rows): lane l reads row
    // wm0 + 16 i + l % 16, k 8 (l / 16) .. + 7 (one ds_read_b128).  B block j (16 columns): lane
    // l holds column wn0 + ring_bcol(j, l % 16), k 8 (l / 16) .. + 7, from two transposing reads;
    // per 16 lanes source lane s supplies row kb + s / 4 at columns x + 0 .. 3, x = the column of
    // result lanes 4 (s % 4) .. + 3, and result lane i gets B[kb .. kb + 3][x + i % 4], with
    // kb = 8 (l / 16) and 8 (l / 16) + 4.
    // Row form, at `half`: lane l reads row r (its block's row or column for lane l % 16) at
    // k 8 (l / 16) .. + 7.  k-major form: source lane group s % 4 points at column x.
    const int rr = lane & 15;
    const int b_k0 = 8 * (lane >> 4) + (rr >> 2);
    auto row_addr = [&](int half, int r) {
        return half + r * (kDmaBK * 2) + (((lane >> 4) ^ ring_aswz(r)) << 4);
    };
    auto kmajor_addr = [&](int half, int x, bool is_b) {
        return half + b_k0 * B_ROW + (((x >> 3) ^ ring_kswz(b_k0, is_b)) << 4) + (x & 7) * 2;
    };
    int a_addr[TM], b_addr[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
        a_addr[i] = A_KM ? kmajor_addr(0, wm0 + i * 16 + 4 * (rr & 3), false) : row_addr(0, wm0 + i * 16 + rr);
#pragma unroll
    for (int j = 0; j < TN; ++j)
        b_addr[j] = B_NM ? row_addr(kDmaSlotBytes, wn0 + ring_bcol(j, rr))
                         : kmajor_addr(kDmaSlotBytes, wn0 + ring_bcol(j, 4 * (rr & 3)), true);
    auto read_rows = [&](const char *at) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8_t *>(at);
    };
    auto read_kmajor = [&](const char *at) __attribute__((always_inline)) {
        bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(at));
        bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(at + 4 * B_ROW));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto read_a = [&](const char *slot, int i) __attribute__((always_inline)) {
        if constexpr (A_KM) return read_kmajor(slot + a_addr[i]);
        else return read_rows(slot + a_addr[i]);
    };
    auto read_b = [&](const char *slot, int j) __attribute__((always_inline)) {
        if constexpr (B_NM) return read_rows(slot + b_addr[j]);
        else return read_kmajor(slot + b_addr[j]);
    };
    constexpr int kReadsA = A_KM ? 2 : 1, kReadsB = B_NM ? 1 : 2;  // LDS reads per fragment

    f32x4_t acc[TM][TN];
    auto load_frags = [&](const char *slot, bf16x8_t *af, bf16x8_t *bfr) {
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = read_a(slot, i);
#pragma unroll
        for (int j = 0; j < TN; ++j) bfr[j] = read_b(slot, j);
    };
    constexpr int kMf = TM * TN;
    // Column block major: B fragment j of the stage is dead after its TM MFMAs, so the next
    // stage's B fragment j (read right then) can take its registers; only the A fragments of
    // two stages are live at once.
    auto mfmas = [&](const bf16x8_t *af, const bf16x8_t *bfr) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    };
    // Order within a stage: the next stage's A fragment reads after the first TM MFMAs, its B
    // fragment j's two reads after the last MFMA of column block j, and the stage's global loads
    // after every TM-th MFMA.
    auto pin = [&]() {
#pragma unroll
        for (int m = 0; m < kMf; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (m < TM) __builtin_amdgcn_sched_group_barrier(0x100, kReadsA, 0);
            if (m % TM == TM - 1) {
                __builtin_amdgcn_sched_group_barrier(0x100, kReadsB, 0);
                if (m / TM < 2 * NBLK) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
    };
    auto slot_of = [&](int s) { return s % SLOTS; };

    bf16x8_t fa[2][TM], fb[2][TN];
    int slot0 = 0;            // ring slot of the current tile's stage 0
    bool prefetched = false;  // the current tile's stages 0 .. SLOTS - 2 are already in flight
    const int kt_check = nk - SLOTS;  // the next tile's chunk is checked at about this stage
    for (int vb = blockIdx.x; vb < nt; vb = kFour ? nt : vb + (int)gridDim.x) {
        TileOrigin o, on;
        tile_origin<BM, BN, CHUNKED>(p, tiles_m, tiles_n, o, vb);
        const int vn = vb + (int)gridDim.x;
        // the four-wave form runs one tile per workgroup (its launch has a workgroup per tile),
        // which leaves out the next tile's state and keeps its registers within the VGPRs
        const bool has_next = !kFour && vn < nt && kt_check >= 0;
        if (has_next) tile_origin<BM, BN, CHUNKED>(p, tiles_m, tiles_n, on, vn);
        else on = o;  // never loaded from (its stages are issued with an empty range)
        tile_wait<CHUNKED>(p, o, vb);  // at once when prefetched: the chunk was seen landed
        if (!prefetched) {
#pragma unroll
            for (int st = 0; st < SLOTS - 1; ++st) issue(o, true, st, slot_of(slot0 + st));
        }
        // The four-wave form reads none of the set's signals or flags after its one chunk wait,
        // so it counts itself for the call's end here, behind its first stages' loads: the
        // count's round trip then overlaps their latency (the wait for its value also waits for
        // stages 1 and 2, issued with stage 0) instead of holding the workgroup, and its CU's
        // next tile, at the tile's end.
        uint32_t grp_v = 0;
        if constexpr (kFour && CHUNKED) {
            uint32_t v = 0;
            if (threadIdx.x == 0) v = end_count(p.plan, vb);
            grp_v = __builtin_amdgcn_readfirstlane(v);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
        // stage 0 landed (stages 1 .. SLOTS - 2 may be in flight; so may the previous tile's
        // stores, which only makes this wait longer)
        wait_vmcnt<2 * NBLK * (SLOTS - 2)>();
        __syncthreads();
        load_frags(smem + slot_of(slot0) * SLOT, fa[0], fb[0]);
        bool next_ok = false;
        // Stage kt: fragment set S0 holds stage kt.  Wait for this wave's loads of stage kt + 1
        // and make every wave's visible (the barrier also retires the slot of stage kt - 1,
        // whose fragments were read during stage kt - 2); start stage kt + SLOTS - 1 (of the next
        // tile past the end) into that slot; read stage kt + 1 into S1 during the MFMAs.
        // Four-wave stage kt (see above): column block j of the MFMAs, then (after block 0) the
        // wait and barrier of the eight-wave stage, then global load j of stage kt + SLOTS - 1
        // (past the tile's end, an empty range, as the eight-wave stage issues with no next
        // tile), then the next stage's fragment reads for block j.  Empty asm statements with a
        // memory clobber keep the reads and loads between the blocks they were written between.
        auto stage4 = [&](int kt, int S0, int S1) __attribute__((always_inline)) {
            const int nslot = slot_of(slot0 + kt + 1);
            const int fslot = slot_of(slot0 + kt + SLOTS - 1);
            const int g = kt + SLOTS - 1;
            const bool live = g < nk;
            const int64_t k0 = live ? (int64_t)g * kDmaBK : 0;
            const bool k_tail = k0 + kDmaBK > p.k;
            const int64_t k_rows = !live ? 0 : (p.k - k0) < kDmaBK ? (p.k - k0) : kDmaBK;
            const u32x4_t ar = a_desc(o, live, k0, k_rows);
            const u32x4_t br = b_desc(o, live, k0, k_rows);
            const uint32_t la = lds0 + (uint32_t)(fslot * SLOT), lb = la + kDmaSlotBytes;
            const char *ns = smem + nslot * SLOT;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                                 : "+a"(acc[i][j])
                                 : "v"(fb[S0][j]), "v"(fa[S0][i]));
                asm volatile("" ::: "memory");
                if (j == 0) {
                    wait_vmcnt<2 * NBLK * (SLOTS - 3)>();  // SLOTS - 3 later stages may stay in flight
                    __syncthreads();
                }
                if (j < NBLK) load_a(ar, la, j, k_tail, k0, o);
                else load_b(br, lb, j - NBLK, k_tail, k0, o);
                if (2 * j < TM) {
                    fa[S1][2 * j] = read_a(ns, 2 * j);
                    fa[S1][2 * j + 1] = read_a(ns, 2 * j + 1);
                }
                fb[S1][j] = read_b(ns, j);
                asm volatile("" ::: "memory");
            }
        };
        auto stage = [&](int kt, int S0, int S1) {
            const int nslot = slot_of(slot0 + kt + 1);
            const int fslot = slot_of(slot0 + kt + SLOTS - 1);
            wait_vmcnt<2 * NBLK * (SLOTS - 3)>();  // SLOTS - 3 later stages may stay in flight
            __syncthreads();
            if (has_next && kt == kt_check + 1) next_ok = __builtin_amdgcn_readfirstlane(next_ok_lds) != 0;
            const int g = kt + SLOTS - 1;
            if (g < nk) issue(o, true, g, fslot);
            else issue(on, next_ok, g - nk, fslot);
            load_frags(smem + nslot * SLOT, fa[S1], fb[S1]);
            mfmas(fa[S0], fb[S0]);
            pin();
        };
        int kt = 0;
        while (kt + 2 <= nk) {
            // The check falls in this pair of stages (kt_check = nk - SLOTS always lies below
            // the last full pair); the barrier of a later stage publishes the decision before
            // stage kt_check + 1 reads it.
            if (kt <= kt_check && kt_check < kt + 2 && wave == 0) {
                const bool ok = has_next && (!CHUNKED || chunk_ready_now(p.plan, on.chunk, vn));
                if (lane == 0) next_ok_lds = ok ? 1 : 0;
            }
            if constexpr (kFour) {
                stage4(kt, 0, 1);
                stage4(kt + 1, 1, 0);
            } else {
                stage(kt, 0, 1);
                stage(kt + 1, 1, 0);
            }
            kt += 2;
        }
        if (kt < nk) {
            if constexpr (kFour) stage4(kt, 0, 1);
            else stage(kt, 0, 1);
        }
        // the accumulators are read next; the compiler does not know the inline-assembly MFMAs
        // wrote them, so their result latency is waited out here (32 wait states)
        if constexpr (kFour) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        tile_end16<BM, BN, WGM, WGN, OUT_F32, CHUNKED, kFour && CHUNKED>(p, o, acc, vb, grp_v);
        prefetched = has_next && next_ok;
        slot0 = slot_of(slot0 + nk);
    }
    // no load may still be writing this workgroup's LDS when it exits
    wait_vmcnt<0>();
#endif
}

// Closes a staged call whose copies no GEMM tile waits for (the re-gather of agmm_backward,
// consumed by a later launch on the stream): one wave, counted in the call's end counters like a
// GEMM's only workgroup, waits for every piece of the call, then reports the call done.  The
// launches after it on the stream see the copied rows (their start invalidates the caches).
__global__ void __launch_bounds__(64) stage_join_kernel(ChunkPlan plan) {
    int last = 0;
    if (threadIdx.x == 0)
        last = __hip_atomic_fetch_add(plan.wg_count, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   plan.grp_last[0] &&
               __hip_atomic_fetch_add(plan.wg_count + kEndGroups * kEndLine, 1ull, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == plan.all_last;
    if (__shfl(last, 0, 64)) {
        for (int c = 0; c < plan.n_chunks; ++c) wait_ready(plan.ready[c], plan.ready_n[c], plan);
        wait_ready(plan.join, plan.join_n, plan);
        if (threadIdx.x == 0) {
            release_system();
            __hip_atomic_store(plan.finished, plan.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
}

__global__ void fill_u64_kernel(uint64_t *p, int64_t n, uint64_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

template <int BM, int BN, int WGM, int WGN, int BK = kBK, int WPE = 1, bool BT = false, int LSPREAD = 0>
hipError_t launch_cfg(const GemmProblem &p, hipStream_t stream) {
    const int64_t tm = (p.m + BM - 1) / BM, tn = (p.n + BN - 1) / BN;
    const int64_t nt = tm * tn;
    if (nt == 0) return hipSuccess;
    if (nt > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nt), block(64 * WGM * WGN);
    const bool chunked = p.plan.chunk_rows != 0;
    if (p.c_f32 && chunked)
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, true, true, BK, WPE, BT, LSPREAD>), grid, block, 0, stream, p, (int)tm, (int)tn);
    else if (p.c_f32)
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, true, false, BK, WPE, BT, LSPREAD>), grid, block, 0, stream, p, (int)tm, (int)tn);
    else if (chunked)
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, false, true, BK, WPE, BT, LSPREAD>), grid, block, 0, stream, p, (int)tm, (int)tn);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, false, false, BK, WPE, BT, LSPREAD>), grid, block, 0, stream, p, (int)tm, (int)tn);
    return hipGetLastError();
}

// CUs of the current device, rounded down to a multiple of 8 (so that workgroup b of a grid of
// that size runs on XCD b mod 8, as in any larger grid).
int device_cus8() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int g = cached[dev].load(std::memory_order_relaxed);
    if (g == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) cus = 256;
        g = cus & ~7;
        cached[dev].store(g, std::memory_order_relaxed);
    }
    return g;
}

// Workgroups of a persistent launch on the current device: one per CU (device_cus8).
int persistent_grid() {
    // SPTL_GEMM_PERSIST=0 launches one workgroup per tile instead (measurement aid)
    static const bool off = [] {
        const char *e = getenv("SPTL_GEMM_PERSIST");
        return e && !strcmp(e, "0");
    }();
    return off ? 0x7fffffff : device_cus8();
}

template <int WGM, int WGN, int SLOTS>
hipError_t launch_ring(const GemmProblem &p, hipStream_t stream) {
    const int64_t tm = (p.m + 255) / 256, tn = (p.n + 255) / 256;
    const int64_t nt = tm * tn;
    if (nt == 0) return hipSuccess;
    if (nt > 0x7fffffff) return hipErrorInvalidValue;
    // one workgroup per CU, each taking several tiles; the four-wave form one workgroup per tile
    const int64_t g = WGM * WGN == 4 ? nt : persistent_grid();
    const dim3 grid((unsigned)(nt < g ? nt : g)), block(64 * WGM * WGN);
    if (p.layout != kLayoutRowMajor) {
        if (p.plan.chunk_rows != 0) return hipErrorInvalidValue;
#define SPTL_RING_LAYOUT(L)                                                                                         \
    do {                                                                                                            \
        if (p.c_f32)                                                                                                \
            hipLaunchKernelGGL((gemm_ring_kernel<WGM, WGN, SLOTS, true, false, L>), grid, block, 0, stream, p,      \
                               (int)tm, (int)tn);                                                                   \
        else                                                                                                        \
            hipLaunchKernelGGL((gemm_ring_kernel<WGM, WGN, SLOTS, false, false, L>), grid, block, 0, stream, p,     \
                               (int)tm, (int)tn);                                                                   \
    } while (0)
        if (p.layout == kLayoutAKMajor) SPTL_RING_LAYOUT(kLayoutAKMajor);
        else if (p.layout == kLayoutBNMajor) SPTL_RING_LAYOUT(kLayoutBNMajor);
        else return hipErrorInvalidValue;
#undef SPTL_RING_LAYOUT
        return hipGetLastError();
    }
    const bool chunked = p.plan.chunk_rows != 0;
    if (p.c_f32 && chunked)
        hipLaunchKernelGGL((gemm_ring_kernel<WGM, WGN, SLOTS, true, true>), grid, block, 0, stream, p, (int)tm, (int)tn);
    else if (p.c_f32)
        hipLaunchKernelGGL((gemm_ring_kernel<WGM, WGN, SLOTS, true, false>), grid, block, 0, stream, p, (int)tm, (int)tn);
    else if (chunked)
        hipLaunchKernelGGL((gemm_ring_kernel<WGM, WGN, SLOTS, false, true>), grid, block, 0, stream, p, (int)tm, (int)tn);
    else
        hipLaunchKernelGGL((gemm_ring_kernel<WGM, WGN, SLOTS, false, false>), grid, block, 0, stream, p, (int)tm, (int)tn);
    return hipGetLastError();
}

// Tile configurations.  All share the MFMA instruction and the K order.
enum Config { k256x256w2x2, k256x256w2x4, k256x256w4x2, k256x128w4x2, k256x128w4x1, k128x128w2x2, k256x256ring,
              k128x256w2x2k32, k256x256w4x2k32, k256x256bt, k256x256il2, k256x256il4, k256x256btil2, k256x256ring4,
              kNumConfigs };

const char *config_name(int c) {
    switch (c) {
        case k256x256w2x2: return "256x256w2x2";
        case k256x256w2x4: return "256x256w2x4";
        case k256x256w4x2: return "256x256w4x2";
        case k256x128w4x2: return "256x128w4x2";
        case k256x128w4x1: return "256x128w4x1";
        case k256x256ring: return "256x256ring";
        case k128x256w2x2k32: return "128x256w2x2k32";
        case k256x256w4x2k32: return "256x256w4x2k32";
        case k256x256bt: return "256x256bt";
        case k256x256il2: return "256x256il2";
        case k256x256il4: return "256x256il4";
        case k256x256btil2: return "256x256btil2";
        case k256x256ring4: return "256x256ring4";
        default: return "128x128w2x2";
    }
}

constexpr int64_t kFourWaveMinK = 2048;

int config_rows(int c) { return c == k128x128w2x2 || c == k128x256w2x2k32 ? 128 : 256; }
int config_cols(int c) { return c == k256x128w4x2 || c == k256x128w4x1 || c == k128x128w2x2 ? 128 : 256; }

// Chunk-ordered tile layout (chunk_layout_choice, sptl_tilemap.h): plan.xcd_group holds a
// forced group size or 0 on entry and the chosen one on return; each XCD runs one workgroup per
// CU at once.
void chunk_layout(ChunkPlan &plan, int bm, int64_t tiles_n) {
    plan.xcd_group = chunk_layout_choice(plan.chunk_rows / bm, tiles_n, plan.n_chunks, plan.xcd_group,
                                         device_cus8() / 8, &plan.chunk_band);
}

// SPTL_GEMM_CFG=<name> forces one configuration for every GEMM (measurement aid).
int forced_config() {
    static const int forced = [] {
        const char *e = getenv("SPTL_GEMM_CFG");
        if (!e) return -1;
        for (int c = 0; c < kNumConfigs; ++c)
            if (!strcmp(e, config_name(c))) return c;
        return -1;
    }();
    return forced;
}

int resolve(const GemmProblem &p, GemmTile t) {
    if (p.layout != kLayoutRowMajor)  // the other layouts exist on the ring kernels only
        return p.k >= kFourWaveMinK ? k256x256ring4 : k256x256ring;
    if (p.plan.chunk_rows) {  // chunk-ordered: the tile height must divide the chunk
        if (forced_config() >= 0 && p.plan.chunk_rows % config_rows(forced_config()) == 0)
            return forced_config();
        if (p.plan.chunk_rows % 256) return k128x128w2x2;
        // measured at 8192 x 4096 x 4096: 907-920 against 880-891 TFLOP/s for the eight-wave
        // persistent kernel (whose next-tile prefetch the four-wave form does not have)
        return p.k >= kFourWaveMinK ? k256x256ring4 : k256x256ring;
    }
    if (forced_config() >= 0) return forced_config();
    // 256 x 256 tiles: the four-wave form when K is long enough to carry its per-tile start (it
    // runs one tile per workgroup, with no next-tile prefetch); gemm_partial measured +1 to +3 %
    // at K = 3584 and 4096, -9 % at K = 768
    const int wide = p.k >= kFourWaveMinK ? k256x256ring4 : k256x256ring;
    if (t == GemmTile::T256x256) return wide;
    if (t == GemmTile::T128x128) return k128x128w2x2;
    // One wave of 256 x 256 tiles needs about one workgroup per CU (256 on MI355X); below
    // that, 128 x 128 tiles keep every CU busy.
    const int64_t big = ((p.m + 255) / 256) * ((p.n + 255) / 256);
    return big >= 240 ? wide : k128x128w2x2;
}

}  // namespace

int chunk_tile_rows(int64_t chunk_rows) {
    if (chunk_rows > 0 && chunk_rows % 256 == 0) return 256;
    if (chunk_rows > 0 && chunk_rows % 128 == 0) return 128;
    return 0;
}

hipError_t launch_stage_join(const ChunkPlan &plan, hipStream_t stream) {
    hipLaunchKernelGGL(stage_join_kernel, dim3(1), dim3(64), 0, stream, plan);
    return hipGetLastError();
}

hipError_t launch_fill_u64(uint64_t *p, int64_t n, uint64_t v, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_u64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n, v);
    return hipGetLastError();
}

void chunk_xcd_tiles(const GemmProblem &problem, int64_t *tiles) {
    const int c = resolve(problem, GemmTile::Auto);
    ChunkPlan plan = problem.plan;
    const int bm = config_rows(c), bn = config_cols(c);
    const int64_t tiles_n = (problem.n + bn - 1) / bn;
    chunk_layout(plan, bm, tiles_n);
    const int tpc = plan.chunk_rows / bm;
    const int64_t nt = tiles_n * tpc * plan.n_chunks;
    for (int64_t i = 0; i < (int64_t)plan.n_chunks * 8; ++i) tiles[i] = 0;
    for (int64_t b = 0; b < nt; ++b) {
        int pos, sub, tn;
        chunk_tile(tpc, (int)tiles_n, plan.xcd_group, plan.chunk_band, (int)b, pos, sub, tn);
        tiles[(int64_t)plan.order[pos] * 8 + (b & 7)]++;
    }
}

int64_t gemm_workgroups(const GemmProblem &p, GemmTile tile) {
    const int c = resolve(p, tile);
    const int64_t bm = config_rows(c), bn = config_cols(c);
    return ((p.m + bm - 1) / bm) * ((p.n + bn - 1) / bn);
}

hipError_t launch_gemm(const GemmProblem &problem, hipStream_t stream, GemmTile tile) {
    const int c = resolve(problem, tile);
    GemmProblem p = problem;
    if (p.plan.chunk_rows) chunk_layout(p.plan, config_rows(c), (p.n + config_cols(c) - 1) / config_cols(c));
    switch (c) {
        case k256x256w2x2: return launch_cfg<256, 256, 2, 2>(p, stream);
        case k256x256w2x4: return launch_cfg<256, 256, 2, 4>(p, stream);
        case k256x256w4x2: return launch_cfg<256, 256, 4, 2>(p, stream);
        case k256x128w4x2: return launch_cfg<256, 128, 4, 2>(p, stream);
        case k256x128w4x1: return launch_cfg<256, 128, 4, 1>(p, stream);
        case k256x256ring: return launch_ring<4, 2, 4>(p, stream);
        case k256x256ring4: return launch_ring<2, 2, 4>(p, stream);
        case k128x256w2x2k32: return launch_cfg<128, 256, 2, 2, 32, 2>(p, stream);
        case k256x256w4x2k32: return launch_cfg<256, 256, 4, 2, 32>(p, stream);
        case k256x256bt: return launch_cfg<256, 256, 4, 2, kBK, 1, true>(p, stream);
        case k256x256il2: return launch_cfg<256, 256, 4, 2, kBK, 1, false, 2>(p, stream);
        case k256x256il4: return launch_cfg<256, 256, 4, 2, kBK, 1, false, 4>(p, stream);
        case k256x256btil2: return launch_cfg<256, 256, 4, 2, kBK, 1, true, 2>(p, stream);
        default: return launch_cfg<128, 128, 2, 2>(p, stream);
    }
}

}  // namespace sptl
