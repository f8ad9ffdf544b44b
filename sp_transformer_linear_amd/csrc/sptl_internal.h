// Internal interfaces between the C-ABI layer, the SDMA stager and the HIP kernels of
// libsptl.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sptl {

constexpr int kMaxPlanChunks = 64;  // chunks of one chunk-ordered GEMM launch
constexpr int kEndGroups = 8;       // end-counter groups (workgroup index mod 8)
constexpr int kEndLine = 32;        // 64-bit words between end counters (256 bytes)
constexpr int kEndCounters = kEndGroups + 1;
// A call's counter block (kCallCountLines lines of kEndLine words): the end counters, then the
// grab and done counters of the lead chunks its own workgroups copy (ChunkPlan::cu_n).
constexpr int kCuGrabLine = kEndCounters, kCuDoneLine = kEndCounters + 1;
constexpr int kCallCountLines = kEndCounters + 2;
constexpr int kMaxCuChunks = 16;         // lead chunks a launch's workgroups may copy
constexpr int64_t kCuBlockBytes = 65536;  // one grab of such a copy

// Landed flags of a chunk-ordered launch: kFlagReplicas copies per chunk, 4 KiB apart so that
// they fall on different memory channels; replica r of chunk c is word r * kFlagStride + c.
constexpr int kFlagReplicas = 16;
constexpr int kFlagStride = 512;                                   // 64-bit words
constexpr size_t kFlagSetWords = (size_t)kFlagReplicas * kFlagStride;

// Chunk-ordered GEMM over a gathered activation (the column GEMM of the chunked all-gather +
// matmul).  Row tiles are processed in `order` (own chunks first, then the peers' chunks in
// arrival order); the workgroups of a tile of chunk c wait, with a bounded spin, until every
// word of ready[c][0 .. ready_n[c]) is <= 0 (the SDMA completion signals of the chunk's copy
// pieces, one per piece) before reading its rows.  Rows of chunks [own_first, own_first + own_count) are read from own_a
// (this rank's shard), all others from GemmProblem::a (the gathered buffer).
struct ChunkPlan {
    int chunk_rows;                          // rows per chunk, a multiple of the tile height
    int n_chunks;                            // <= kMaxPlanChunks
    int own_first, own_count;
    int order[kMaxPlanChunks];               // processing position -> chunk
    const int64_t *const *ready[kMaxPlanChunks];  // per chunk: piece signal words; nullptr: no wait
    int ready_n[kMaxPlanChunks];
    const int64_t *const *join;              // waited for by the last workgroup to finish
    int join_n;
    const uint16_t *own_a;
    int *err;                                // set to 1 when a wait times out
    uint64_t timeout_ticks;                  // wall-clock ticks of the bounded waits
    int poll_sleep;                          // extra s_sleep 127 per poll (0: ~1 us between polls)
    int xcd_group;                           // XCDs per chunk: a forced value or 0 (choose) on entry
                                             // to launch_gemm; the kernel sees the chosen one (0: plain
                                             // chunk order)
    int chunk_band;                          // tile rows per band inside a chunk (set by launch_gemm)
    uint64_t *flags;                         // landed flags (kFlagSetWords words), or nullptr
    uint64_t flag_epoch;                     // value a landed flag holds for this launch (unique
                                             // among the launches that share the flags)
    uint64_t epoch;                          // value the end words take for this launch
    uint64_t *finished;                      // pinned host word: epoch once the launch is done
    uint64_t *timedout;                      // pinned host word: epoch if a wait of the launch timed out
    uint64_t *started;                       // pinned host word (or null): tile 0 stores epoch at its start
    uint64_t *wg_count;                      // the call's counter block (kCallCountLines lines)
    uint64_t grp_last[kEndGroups];           // group counter value seen by a group's last workgroup
    uint64_t all_last;                       // final counter value seen by the last group
    uint64_t *ts;                            // optional per-chunk timestamps (see below)
    // Copy-out mode (the reduce-scatter mirror): the chunks are output slices and no tile waits
    // for input.  ready[c] then lists the completion words of slice c's outgoing copies (null: the
    // slice stays).  The copy engines read memory, so a slice is released only once every XCD
    // that ran some of its tiles has written its L2 back after their stores: each such tile waits
    // for its stores and counts itself in the counter of the XCD it runs on (line c of
    // slice_count, kEndLine words: word 1 + x for XCC x), and the XCD's last tile of the slice (it
    // sees slice_xcd_last[c], the per-XCD share less one) writes the XCD's L2 back and counts the
    // XCD in word 0; the last XCD (it sees slice_last[c], the XCDs holding the slice less one)
    // stores epoch to slice_ready[16 c] (pinned host memory, where the copies are released from).
    // A count past the share sets err[2].  The counters are zeroed by the call before the launch.
    // flush_each_tile: every tile writes back and counts in word 0 (slice_last[c] then counts
    // tiles), for layouts whose XCDs hold unequal shares of a slice.  The launch's last workgroup
    // waits for every copy before reporting the end.
    // Lead chunks copied by the launch's own workgroups: when the own chunks do not fill the
    // first round of tiles, the tiles of the first peer chunks would sit idle until the copy
    // engines land them; instead each such tile takes kCuBlockBytes blocks of those chunks' copies
    // (from the grab counter, line kCuGrabLine of wg_count) until none is left, with agent-scope
    // stores (written through its XCD's L2), and once they have completed adds its blocks to the
    // done counter (line kCuDoneLine);
    // then it waits (bounded) for done to reach every block and invalidates its caches.  Any
    // resident workgroup can do any block, so the copies finish whichever tiles run.  cu_mask has
    // bit c set for such a chunk c; the i-th of the cu_n copies goes from cu_src[i] to cu_dst[i]
    // (cu_chunk_bytes each).  The launch's last workgroup resets both counters.
    int cu_n;
    uint64_t cu_mask;
    int64_t cu_chunk_bytes;
    const void *cu_src[kMaxCuChunks];
    void *cu_dst[kMaxCuChunks];
    bool copy_out;
    bool flush_each_tile;
    uint64_t *slice_ready;
    uint64_t *slice_count;
    uint64_t slice_last[kMaxPlanChunks];
    uint32_t slice_xcd_last[kMaxPlanChunks];
};
// Waiting: a workgroup of chunk c polls its replica of c's landed flag about every
// microsecond and, once every 16 polls (phase set by its index), c's completion words
// themselves.  The first workgroup to see them all reach zero sets every replica to `flag_epoch`.  Spreading
// the polls over replicas keeps a few hundred waiting workgroups from hammering the one
// memory line the copy engines update.
// End: workgroup b counts itself in group counter b % kEndGroups (line g of wg_count, 256
// bytes apart) when done; the last of a group (it sees grp_last[g]) counts the group in the
// final counter (line kEndGroups), and the last group's workgroup (it sees all_last) waits for
// the join, then stores epoch to *finished.  Spreading the counting keeps the last round's
// workgroups from queueing on one atomic (one counter cost about 15 us per launch).  Every
// counter is cumulative over the launches of a set; groups with no workgroup are skipped.
// ts layout (wall-clock ticks, n = n_chunks): ts[c] = first time a tile of chunk c found it
// ready (min), ts[n + c] = first tile start of chunk c (min), ts[2 n + c] = last tile end of
// chunk c (max), ts[3 n] = start of workgroup 0.

// C[M, N] = A[M, K] @ B[K, N]; bf16 inputs, fp32 accumulation, bf16 or fp32 output.
// Row-major with leading dimensions lda, ldb, ldc (elements).  K and N multiples of 8,
// pointers 16-byte aligned.  Every tile configuration uses the same MFMA instruction and
// the same ascending K order, so the result bits do not depend on the tiling.
// Operand layouts of a GEMM C[m, n] = sum_k A(i, k) B(k, j):
//   kLayoutRowMajor  A(i, k) = a[i lda + k], B(k, j) = b[k ldb + j]
//   kLayoutAKMajor   A(i, k) = a[k lda + i] (a weight gradient's transposed activation)
//   kLayoutBNMajor   B(k, j) = b[j ldb + k] (an input gradient's transposed weight)
// The layouts other than row-major run on the 256 x 256 ring kernels only, never chunk-ordered.
constexpr int kLayoutRowMajor = 0, kLayoutAKMajor = 1, kLayoutBNMajor = 2;

struct GemmProblem {
    const uint16_t *a;
    const uint16_t *b;
    void *c;
    int64_t m, n, k;
    int64_t lda, ldb, ldc;
    bool c_f32;
    ChunkPlan plan;   // plan.chunk_rows == 0: plain GEMM
    int layout = kLayoutRowMajor;
};

enum class GemmTile { T256x256, T128x128, Auto };

// Picks a tile shape for the problem (Auto) and launches.  Returns the HIP error of the
// launch.
hipError_t launch_gemm(const GemmProblem &p, hipStream_t stream, GemmTile tile = GemmTile::Auto);

// Per chunk of a chunk-ordered launch of p: the tiles each of the 8 XCDs runs under round-robin
// placement (tiles[8 c + x], x = tile index mod 8), from the same tile map the kernel uses.
void chunk_xcd_tiles(const GemmProblem &p, int64_t *tiles);

// Workgroups launch_gemm(p, stream, tile) launches.
int64_t gemm_workgroups(const GemmProblem &p, GemmTile tile = GemmTile::Auto);

// Tile height a chunk-ordered launch of `p` would use (0: chunk_rows fits no tile height).
int chunk_tile_rows(int64_t chunk_rows);

// Fills n 64-bit words with v on `stream` (a kernel, so it is safe inside graph capture).
hipError_t launch_fill_u64(uint64_t *p, int64_t n, uint64_t v, hipStream_t stream);

// Launches the one-wave kernel that waits for every copy of a staged call (plan: n_chunks, ready,
// join, the end counters and words of the call) and then reports the call done.
hipError_t launch_stage_join(const ChunkPlan &plan, hipStream_t stream);

// dst = src ([rows, cols] bf16, cols % 8 == 0) with rows (dim 0: dst[i, :] = src[perm[i], :]) or
// columns (dim 1: dst[:, j] = src[:, perm[j]]) permuted; an index out of range gives zeros and
// sets *err to 1 (sptl_copy.hip).
hipError_t launch_permute(const void *src, void *dst, int64_t rows, int64_t cols, int dim, const int32_t *perm,
                          int *err, hipStream_t stream);

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) with a kernel on the compute
// units: `workgroups` workgroups of 256 threads, or a grid sized to the copy when 0 (sptl_copy.hip).
hipError_t launch_blit(void *dst, const void *src, size_t bytes, int workgroups, hipStream_t stream);

constexpr int kMaxEpilogueInputs = 17;  // residual + 16 partials

// h = in[0] + in[1] + ... + in[n_in - 1] (fp32, in this order); y = RMSNorm(h) * gamma.
// h_out / y_out may be null (then not written; with y_out null no norm is taken).
struct EpilogueProblem {
    const uint16_t *in[kMaxEpilogueInputs];
    int n_in;
    const uint16_t *gamma;
    uint16_t *h_out;
    uint16_t *y_out;
    int64_t rows;
    int64_t hidden;  // multiple of 8
    float eps;
};

hipError_t launch_epilogue(const EpilogueProblem &p, hipStream_t stream);

}  // namespace sptl
