/*
 * sptl.h - C ABI of libsptl.so: one GPU's share of the sequence-parallel tensor-parallel
 * (SP-TP) linear layer on AMD Instinct MI355X (gfx950).
 *
 * The layer (sources are web pages; each call below names the passage it implements):
 *   [AReaL] "[Feature] Async Tensor Parallelism for Archon Engine" (AReaL issue),
 *           sections "TP Communication Is on Activations, Not Weights" and
 *           "Potential Solution".
 *   [DTP]   "Affinity-Aware Sharding for Delayed Tensor Parallelism" (arXiv abstract).
 *   [MLM]   "Add forward all-gather overlap" (Megatron-LM pull request #5513),
 *           sections "Summary", "Notes from the review meeting", "Observations" and
 *           "Recommendations".
 *
 * Conventions for every call
 *   - Tensors are row-major with the last dimension contiguous and no padding.  bf16 is
 *     IEEE bfloat16 (upper half of a binary32); results are rounded to nearest-even.
 *   - Every tensor pointer is a DEVICE pointer on the context's device and must be 16-byte
 *     aligned.  Pointer arrays (shard_src, partials, delayed_peers) are HOST arrays of
 *     device pointers; the library reads them during the call only.
 *   - Streams are hipStream_t values passed as void*; NULL means the null stream.
 *   - Ownership: the caller owns every buffer and stream.  The library never allocates,
 *     frees or retains caller memory.  A context owns its own resources only: HIP events,
 *     a few small device buffers (an error word, chunk timestamps, 256 KiB of landed
 *     flags), an SDMA stager (4160 HSA completion signals, about 40 KiB of device counters
 *     and tables, one page of pinned host memory and one worker thread), all created with
 *     the context, and the copy stream of the per-chunk path, created on its first use.
 *     The library also holds one 67 KiB device array per GPU (agmm_chunked_noalloc).
 *     Inputs must stay valid until the stream work of the call completes.
 *   - Every call is asynchronous (stream-ordered) and returns an sptl_status.  All
 *     arguments are validated BEFORE anything is enqueued: on any non-OK status nothing
 *     was enqueued and sptl_last_error() holds a message.  HIP failures after validation
 *     return SPTL_E_HIP with the HIP error text.  No call aborts or throws.
 *   - ctx may be NULL: the call then uses a per-device default context for the current
 *     device, created on first use.  Argument validation happens before that, so a call
 *     with invalid arguments makes no HIP call at all.
 *   - Sizes are element counts.  Empty work (seq_len == 0) is valid and enqueues nothing.
 *   - A context serves one host thread at a time; different contexts (and the default
 *     contexts of different devices) may be used from different threads concurrently.
 *   - Calls on one context may be issued on different compute streams and run at the same time
 *     on the GPU: each staged call has a signal set of its own (4 per context), and the per-chunk
 *     paths share the context's copy stream.  The exceptions: two timed calls (timing != 0) on
 *     one context must not overlap (they share its timestamps), nor may two agmm_chunked_noalloc
 *     calls on one GPU (they share its scratch array).
 */
#ifndef SPTL_H
#define SPTL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sptl_ctx sptl_ctx;

typedef enum { SPTL_BF16 = 0, SPTL_F32 = 1 } sptl_dtype;

typedef enum {
    SPTL_OK = 0,
    SPTL_E_NULL = 1,         /* a required pointer is NULL                                */
    SPTL_E_SHAPE = 2,        /* a size is negative, zero where it must be positive, or
                                exceeds a documented limit                               */
    SPTL_E_DIVISIBILITY = 3, /* seq_len % n_chunks, n_chunks % tp, or a size not a
                                multiple of 8 (16-byte rows)                             */
    SPTL_E_ALIGN = 4,        /* a device pointer is not 16-byte aligned                   */
    SPTL_E_DTYPE = 5,        /* dtype not in sptl_dtype                                   */
    SPTL_E_RANGE = 6,        /* rank, tp, delta or module index out of range, or a pointer
                                given/omitted against the delayed-TP schedule            */
    SPTL_E_HIP = 7,          /* a HIP runtime call failed                                 */
    SPTL_E_UNSUPPORTED = 8,  /* valid request the library does not handle                */
    SPTL_E_ASYNC = 9         /* an asynchronous failure was recorded (see sptl_ctx_check)  */
} sptl_status;

/* Limits. */
#define SPTL_MAX_PARTIALS 16   /* partials per reduce call; also bounds dtp_accumulate's tp */
#define SPTL_MAX_TP 64         /* TP degree of agmm_chunked                              */
#define SPTL_MAX_CHUNKS 512    /* chunk count of agmm_chunked                            */
#define SPTL_MAX_K 2097152     /* GEMM reduction size (hidden of agmm_chunked, k_local)  */
#define SPTL_MAX_N 8388608     /* GEMM output width (n_local, hidden of gemm_partial)    */
#define SPTL_MAX_HEAD_LAYOUTS 67108864LL /* head layouts dtp_affinity_layout tries per round */

/* Create a context on HIP device `device`: events, small device buffers and the SDMA stager
 * are created now (the copy stream of the per-chunk path on its first use), together with the
 * set-up of agmm_chunked_noalloc for the device.  *out receives the
 * context.  Returns SPTL_E_NULL if out is NULL, SPTL_E_RANGE for a bad device, SPTL_E_HIP on
 * runtime failure.  Environment read here: SPTL_STAGING=events forces the per-chunk path;
 * SPTL_WAIT_TIMEOUT_US=1..10000000 sets the bound on one chunk wait (default 10 s). */
int sptl_create(sptl_ctx **out, int device);

/* Destroy a context created by sptl_create: waits (bounded) for its staged calls and its copy
 * stream, stops its worker thread, then releases everything it owns.  NULL is accepted and
 * ignored. */
int sptl_destroy(sptl_ctx *ctx);

/* Text describing the last non-OK status returned on the calling thread ("" if none).
 * The pointer stays valid until the next sptl call on this thread. */
const char *sptl_last_error(void);

/* ABI version (major * 100 + minor). */
int sptl_version(void);

/* Waits (bounded, 30 s per wait) until every staged agmm_chunked call made on ctx has
 * completed on the GPU, including the copies of a call whose chunk wait timed out (those may
 * still write that call's x_gathered after its kernel has ended; once this returns they have
 * landed), then reports asynchronous failures recorded since the last check: SPTL_E_ASYNC if
 * a staging wait timed out (the affected call's y is invalid; a chunk wait gives up after
 * 10 s unless sptl_ctx_set_wait_timeout_us says otherwise), a staging copy could not be
 * submitted (the staged path is then disabled for ctx) or the copies of a timed-out call did
 * not complete within the bound; SPTL_OK otherwise.  Clears the recorded state. */
int sptl_ctx_check(sptl_ctx *ctx);

/* Sets the bound on one chunk wait inside the staged GEMM of later agmm_chunked calls on ctx,
 * in microseconds: 1..10000000, or 0 for the default (10 s).  A wait that runs out lets its
 * workgroups go on with whatever the chunk's rows hold; the call is then reported by
 * sptl_ctx_check (SPTL_E_ASYNC).  Meant for failure-path tests and for callers that prefer an
 * early error over a long stall.  SPTL_E_NULL for a NULL ctx, SPTL_E_RANGE otherwise. */
int sptl_ctx_set_wait_timeout_us(sptl_ctx *ctx, int64_t us);

/* How the staging copies of agmm_chunked (copy == NULL), reduce_norm_agmm_chunked and
 * gemm_rs_chunked run on ctx.  [MLM "Observations"]: a gather that runs on the compute units
 * (the ring all-gather's CTAs) contends with the GEMM, while the copy-engine gather does not;
 * the modes other than the default exist to measure that and to give a capturable path.
 *   SPTL_COPY_STAGED  the default: the copy engines driven by the context's worker thread,
 *                     one chunk-ordered GEMM launch that waits for each chunk on the GPU.
 *                     Falls back to SPTL_COPY_EVENTS where it does not apply (no copy engines,
 *                     chunk heights that fit no chunk tile, a stream under graph capture).
 *   SPTL_COPY_EVENTS  one SDMA-class hipMemcpyAsync per chunk on the context's copy stream with
 *                     an event each, one GEMM launch per chunk after its event.  Under graph
 *                     capture the copies are recorded as device-to-device copy nodes.
 *   SPTL_COPY_BLIT    as SPTL_COPY_EVENTS, but each copy is a copy kernel on the compute units
 *                     (blit_workgroups workgroups of 256 threads; 0 = sized to the copy).
 *   SPTL_COPY_SERIAL  no overlap: every copy on the compute stream, then one GEMM launch over
 *                     all rows (agmm_chunked), or the GEMM then the copies (gemm_rs_chunked).
 * Every mode gives bit-identical outputs.  agmm_chunked_noalloc always stages (the mode does not
 * apply to it).  SPTL_E_NULL for a NULL ctx; SPTL_E_RANGE for a mode outside the enum or
 * blit_workgroups outside [0, 65535]. */
typedef enum { SPTL_COPY_STAGED = 0, SPTL_COPY_EVENTS = 1, SPTL_COPY_BLIT = 2, SPTL_COPY_SERIAL = 3 } sptl_copy_mode;
int sptl_ctx_set_copy_mode(sptl_ctx *ctx, int mode, int blit_workgroups);

/* Chunk order and link model of agmm_chunked's gather on ctx.  [AReaL "Potential Solution"]:
 * each chunk's matmul starts as soon as the chunk has arrived, so chunks are processed in the
 * order in which they are meant to arrive.
 *   order  SPTL_ORDER_RING (the default): this rank's sub-chunks, then all of peer rank+1's, then
 *          rank+2's, ...: the order in which a ring all-gather delivers them.
 *          SPTL_ORDER_INTERLEAVED: this rank's sub-chunks, then sub-chunk 0 of peers rank+1,
 *          rank+2, ..., then sub-chunk 1 of each, ...: the order in which a direct gather over
 *          point-to-point links (one per peer, all streaming at once) delivers them.  The same
 *          as the ring order when n_chunks == tp.
 *   engines_per_peer  0 (the default): the staged path spreads the copies over all copy
 *          engines.  k >= 1: the link model.  Each peer's copies run only on k copy engines of
 *          their own, engines (p*k + j) mod E for the p-th peer after this rank.  They stand in
 *          for one link per peer with a bandwidth of its own (one engine streams about 47 GB/s).
 *          The launch's own workgroups then copy no lead chunks, and the own slot is spread over
 *          all engines.  The staged path only; the event paths ignore it.
 * Both apply to agmm_chunked, reduce_norm_agmm_chunked, agmm_chunked_noalloc and gemm_rs_chunked
 * (its send order; each peer sub-slice pushed on its peer's engines); the link model also to the
 * staged path of agmm_backward (the re-gather).  Every setting gives bit-identical outputs.  SPTL_E_NULL for a
 * NULL ctx; SPTL_E_RANGE for an order outside the enum or engines_per_peer outside [0, 16]. */
typedef enum { SPTL_ORDER_RING = 0, SPTL_ORDER_INTERLEAVED = 1 } sptl_chunk_order;
int sptl_ctx_set_staging(sptl_ctx *ctx, int order, int engines_per_peer);

/* Short text naming how agmm_chunked stages chunks on ctx with copy == NULL (copy engines
 * driven directly with a chunk-ordered GEMM, or one copy and one GEMM launch per chunk) and,
 * for the latter, why.  Owned by ctx; valid until ctx is destroyed.  Diagnostic only. */
const char *sptl_ctx_info(sptl_ctx *ctx);

/*
 * (1) Chunked sequence all-gather + column-parallel GEMM, this rank's share.
 *
 * [AReaL "Potential Solution", intra-layer overlap]: the all-gather + matmul is split into
 * chunked, pipelined pieces, and each chunk's matmul starts as soon as the chunk has
 * arrived.  [AReaL "TP Communication Is on Activations, Not Weights"]: the gather is over
 * the sequence dimension of the activations.  [MLM "Observations", "Recommendations"]:
 * the gather runs on its own stream and must not take compute units from the GEMM, so the
 * staging copies go to the copy engines (SDMA) rather than to a copy kernel; [MLM "Notes
 * from the review meeting"]: all copies are enqueued before the GEMMs.
 *
 *   seq_len  M: gathered sequence length (rows of x_gathered and y)
 *   hidden   K: hidden size (columns of x_gathered, rows of w); multiple of 8
 *   n_local  N: this rank's column-shard width (columns of w and y); multiple of 8
 *   tp       TP degree, 1 <= tp <= SPTL_MAX_TP
 *   n_chunks chunk count, n_chunks % tp == 0, seq_len % n_chunks == 0,
 *            n_chunks <= SPTL_MAX_CHUNKS.  Rank q's shard is split into n_chunks/tp
 *            contiguous sub-chunks of seq_len/n_chunks rows.
 *   rank     this rank, 0 <= rank < tp
 *   shard_src  host array [tp] of device pointers; shard_src[q] is rank q's sequence shard
 *            [seq_len/tp, hidden] bf16.  shard_src[rank] may point at this rank's slot of
 *            x_gathered (then it is not copied).  For q != rank it stands in for the
 *            peer's buffer and is read only by the staging copies: the copy engines and, for
 *            the lead chunks of a first round that the own chunks do not fill, the launch's own
 *            workgroups.
 *   x_gathered [seq_len, hidden] bf16 output: rank-major concatenation of the shards.
 *   w        [hidden, n_local] bf16 weight shard (logical [in, out]).
 *   y, y_dtype  [seq_len, n_local] output, SPTL_BF16 or SPTL_F32; y = x_gathered @ w with
 *            fp32 accumulation in a fixed order, so every chunking gives identical bits.
 *   compute  stream that runs the GEMMs; the call is ordered after earlier work on it,
 *            and later work on it sees x_gathered and y complete.
 *   copy     NULL: staged path (below).  Otherwise a stream for the per-chunk path.
 *   timing   0: no timing; 1: record per-chunk landing and GEMM timestamps, read
 *            afterwards with sptl_agmm_timeline().  SPTL_E_UNSUPPORTED with the serial copy
 *            mode and on a stream under graph capture.
 * Staged path (copy == NULL and the context's copy mode is SPTL_COPY_STAGED, the default;
 * used when the device's SDMA engines can be driven through HSA, seq_len / n_chunks is a
 * multiple of 128, n_chunks <= 64 and `compute` is not under graph capture; else the per-chunk
 * path runs on the context's own copy stream, see sptl_ctx_set_copy_mode):
 *   - Every peer chunk is split into pieces for the SDMA copy engines.  The peer chunks that
 *     the GEMM's first round of tiles needs (one tile per compute unit, the round sized for
 *     an output at least `hidden` wide) are split together, one piece per engine, so that
 *     they land together.  The later copies are split together in groups large enough that
 *     every engine's piece is at least 2 MiB (a chunk that large on its own is striped over
 *     all engines), a short last group joining the one before.  The pieces are
 *     submitted by the context's worker thread as soon as an event recorded on `compute` at
 *     the call's position has completed, so the copies never overwrite x_gathered while
 *     earlier work on `compute` still reads it.  Copy order: chunks of ranks rank+1, ...,
 *     rank+tp-1 (mod tp), then this rank's own slot unless shard_src[rank] aliases it.
 *   - ONE GEMM launch on `compute` processes row tiles in chunk order: this rank's chunks
 *     first (read straight from shard_src[rank]), then the peers' chunks in copy order;
 *     each tile waits on the GPU for its own chunk's pieces to land.  The launch has one
 *     workgroup per tile, except with 256-row tiles at hidden < 2048: then one workgroup per
 *     compute unit, each taking its tiles in that order.
 *     The launch ends only after every copy of the call (own slot included) has landed.
 *   - The waiting tiles depend on the context's worker thread: the copies start only once it
 *     has seen the call's fork (the GEMM's start, or an event recorded before it when a tile of
 *     the first round waits for an engine copy) and submitted them.  A worker kept off the CPU for longer than
 *     the wait bound (sptl_ctx_set_wait_timeout_us) makes the waits time out; the call's
 *     results are then invalid and sptl_ctx_check reports SPTL_E_ASYNC.  Until then the
 *     waiting workgroups hold their compute units.
 *   - Up to 4 staged calls per context may be in flight; a fifth blocks the calling thread
 *     until the oldest has finished on the GPU (and, if a wait of that call timed out, until
 *     its copies have landed; SPTL_E_ASYNC if they do not within 30 s).
 * Per-chunk path (copy != NULL): for each peer chunk, one SDMA-class hipMemcpyAsync on
 * `copy` (forked from `compute`) and an event; then one GEMM launch per chunk on `compute`
 * after that chunk's event, own chunks first; `compute` joins `copy` at the end.
 * Both paths give bit-identical x_gathered and y.
 */
int agmm_chunked(sptl_ctx *ctx, int64_t seq_len, int64_t hidden, int64_t n_local,
                 int tp, int n_chunks, int rank,
                 const void *const *shard_src, void *x_gathered, const void *w,
                 void *y, int y_dtype, void *compute, void *copy, int timing);

/*
 * (1') agmm_chunked for callers that cannot allocate device memory (code that must not call
 * hipMalloc: tight serving loops, harnesses that forbid it).  The same staged path and kernels
 * as agmm_chunked with copy == NULL and timing == 0, with the same arguments otherwise and the
 * same bits in x_gathered and y; the call itself calls no hipMalloc, hipFree or other
 * allocating routine.
 *   ctx      required (not NULL): sptl_create does this call's set-up, once per device (it
 *            resolves the device's scratch array) and once per context (its copy engines).
 *   The chunk-ordered GEMM keeps its state (landed flags, end and lead-copy counters, error
 *   word) in a fixed 67 KiB device array (at most 80 KiB), one per GPU, held until the process
 *   ends; the counters are zeroed by a small kernel on `compute` before each launch (no memset).
 * Limits: n_chunks <= 64 (the chunks the scratch holds: SPTL_E_SHAPE beyond) and
 * seq_len / n_chunks a multiple of 128 (SPTL_E_UNSUPPORTED otherwise); SPTL_E_UNSUPPORTED also
 * when the context has no working copy engines.  Every call on a GPU shares that GPU's
 * scratch: calls whose GPU work overlaps in time (on different streams, or on contexts used
 * from different threads) race and must not be made; calls ordered on one stream are safe.
 * Timed-out waits are reported by sptl_ctx_check(ctx) as for agmm_chunked.
 */
int agmm_chunked_noalloc(sptl_ctx *ctx, int64_t seq_len, int64_t hidden, int64_t n_local,
                         int tp, int n_chunks, int rank,
                         const void *const *shard_src, void *x_gathered, const void *w,
                         void *y, int y_dtype, void *compute);

/* Per-chunk timeline of the last agmm_chunked call on ctx that had timing = 1.  Blocks
 * until that call's work is done.  out (host) receives n_chunks rows of 4 doubles in
 * milliseconds: copy start, copy end, GEMM start, GEMM end.  Staged path: times from the
 * start of the GEMM launch's first workgroup (device wall clock); copy start is 0 (all
 * copies are queued at the fork), copy end is when the first tile of the chunk saw it
 * landed, GEMM start/end are the chunk's first tile start and last tile end.  Per-chunk path:
 * event times from the call's fork point.  Chunks with no copy have copy start = copy end =
 * -1.  Returns SPTL_E_RANGE if n_chunks differs from the recorded call or no timed call was
 * made. */
int sptl_agmm_timeline(sptl_ctx *ctx, double *out, int n_chunks);

/*
 * (2) Row-parallel GEMM producing this rank's partial sum: partial = a @ w.
 *
 * [DTP abstract] ("partial output" of a tensor-parallel module); [AReaL "Potential
 * Solution"] (the partial sums are reduce-scattered at the end of a sub-layer).
 *   a        [seq_len, k_local] bf16;  k_local multiple of 8
 *   w        [k_local, hidden]  bf16;  hidden multiple of 8
 *   partial  [seq_len, hidden], out_dtype SPTL_BF16 (the layer's form) or SPTL_F32;
 *            fp32 accumulation, same fixed order as agmm_chunked.
 */
int gemm_partial(sptl_ctx *ctx, int64_t seq_len, int64_t k_local, int64_t hidden,
                 const void *a, const void *w, void *partial, int out_dtype, void *stream);

/*
 * (2') Row-parallel GEMM with the reduce-scatter's sends overlapped: the mirror of agmm_chunked.
 *
 * [AReaL "Potential Solution"]: the partial sums of a row-parallel linear are reduce-scattered
 * at the end of the sub-layer (each rank keeps the sum over ranks of its own sequence slice);
 * [MLM "Scope"] leaves that half of the overlap out.  Here the partial is computed sub-slice by
 * sub-slice in send order, and each peer's sub-slice is copied out by the SDMA copy engines as
 * soon as its rows are written, while the following sub-slices are computed.
 *   seq_len, k_local, hidden, a, w: as gemm_partial; slice q is rows
 *            [q seq_len/tp, (q+1) seq_len/tp) of partial
 *   n_chunks sub-slice count: n_chunks % tp == 0, seq_len % n_chunks == 0, n_chunks <= 64.  Each
 *            slice is n_chunks/tp sub-slices of seq_len/n_chunks rows.  Send order: the peers'
 *            sub-slices in the context's chunk order (sptl_ctx_set_staging; the ring order takes
 *            all of rank+1's, then rank+2's, ...; the interleaved order takes sub-slice 0 of
 *            every peer, then sub-slice 1, ...), then this rank's own.  n_chunks == tp: one
 *            slice at a time, peers rank+1, ..., rank+tp-1, then the own.
 *   partial  [seq_len, hidden] bf16: this rank's whole partial sum, the same bits as gemm_partial
 *   dst      host array [tp] of device pointers: dst[q] ([seq_len/tp, hidden] bf16) receives slice q
 *            for q != rank (it stands in for rank q's receive buffer); dst[rank] is not used and
 *            may be NULL.  A dst[q] that is slice q of partial itself is left as is.
 *   tp in [1, 64].  One GEMM launch on `compute`; the launch ends after every copy has landed, so
 *   later work on `compute` sees partial and every dst complete.  The copies are released by the
 *   context's worker thread as the kernel reports each sub-slice done.  Sub-slices of a height
 *   that fits no chunk tile (a multiple of 128 rows), a context without copy engines or a stream
 *   under capture: one GEMM launch per sub-slice in send order, each peer sub-slice copied on the
 *   context's copy stream after its event.
 * Errors: SPTL_E_NULL (a, w, partial, dst or a peer's dst[q] NULL), SPTL_E_RANGE (tp, n_chunks,
 * rank), SPTL_E_SHAPE / SPTL_E_DIVISIBILITY (sizes, n_chunks % tp, seq_len % n_chunks),
 * SPTL_E_ALIGN (any pointer not 16-byte aligned), SPTL_E_ASYNC (an earlier call's copies timed
 * out and are still draining); nothing is launched then.  The kernel's bounded wait for the
 * copies reports through sptl_ctx_check.
 */
int gemm_rs_chunked(sptl_ctx *ctx, int64_t seq_len, int64_t k_local, int64_t hidden, int tp, int n_chunks, int rank,
                    const void *a, const void *w, void *partial, void *const *dst, void *compute);

/*
 * (1') Backward of the chunked all-gather + column-parallel GEMM, with the re-gather overlapped.
 *
 * [MLM "Scope"]: the backward pass gathers again (the weight gradient needs the gathered
 * activation, of which each rank keeps only its shard), and that gather was left without
 * overlap.  Here it runs on the copy engines while the input-gradient GEMM, which does not read
 * the activation, computes; the weight-gradient GEMM follows.  For y = x_gathered @ w (agmm_chunked):
 *   x_gathered = rank-major concatenation of the shards (as agmm_chunked)
 *   dx = dy @ w^T   [seq_len, hidden] bf16: this rank's partial sum of the input gradient (its
 *                   sequence slices are reduce-scattered over the ranks, as gemm_rs_chunked does)
 *   dw = x_gathered^T @ dy   [hidden, n_local], dw_dtype SPTL_F32 or SPTL_BF16
 * Both GEMMs accumulate in fp32, over n_local ascending (dx) and seq_len ascending (dw).
 *   seq_len, hidden, n_local, tp, rank, shard_src, x_gathered, w: as agmm_chunked
 *            (seq_len % tp == 0; hidden and n_local multiples of 8; tp <= 64)
 *   dy       [seq_len, n_local] bf16, the gradient of y
 *   compute  stream; the call is ordered after earlier work on it, and later work on it sees
 *            x_gathered, dx and dw complete.
 * Staged (the context's copy mode SPTL_COPY_STAGED, copy engines available, no graph capture):
 * every copy goes to the SDMA engines at the call's position on `compute`; the dx GEMM, a
 * one-wave kernel that waits (bounded, as the chunk waits of agmm_chunked) for every copy, and
 * the dw GEMM follow on `compute`.  Otherwise the copies run on the context's copy stream
 * (events mode, blit mode or graph capture) or on `compute` before the GEMMs (serial mode).
 * Every path gives the same bits.  Errors as agmm_chunked (SPTL_E_DTYPE for dw_dtype).
 */
int agmm_backward(sptl_ctx *ctx, int64_t seq_len, int64_t hidden, int64_t n_local, int tp, int rank,
                  const void *const *shard_src, void *x_gathered, const void *w, const void *dy,
                  void *dx, void *dw, int dw_dtype, void *compute);

/*
 * (3) Fused reduce + residual + RMSNorm at a sub-layer boundary.
 *
 * [AReaL "Potential Solution", sub-layer boundary overlap]: between a sub-layer's
 * reduce-scatter and the next all-gather sit the residual add and an RMSNorm that reduces
 * over the hidden dimension.
 *   h = residual + partials[0] + ... + partials[tp-1]    (fp32, added in this order)
 *   y = h / sqrt(mean_j h_j^2 + eps) * gamma             (from the unrounded fp32 h)
 *   tp        number of partials, 0 <= tp <= SPTL_MAX_PARTIALS (0: plain residual norm)
 *   partials  host array [tp] of device pointers, each [seq_len, hidden] bf16
 *   residual  [seq_len, hidden] bf16;  hidden multiple of 8
 *   gamma     [hidden] bf16;  eps >= 0
 *   residual_out [seq_len, hidden] bf16 receives h; may equal residual (in place);
 *            NULL = do not write h
 *   y         [seq_len, hidden] bf16; may point at this rank's own slot of the next layer's
 *            x_gathered, which agmm_chunked then reads in place when shard_src[rank] is
 *            the same pointer (no own-slot copy)
 */
int reduce_residual_rmsnorm(sptl_ctx *ctx, int64_t seq_len, int64_t hidden, int tp,
                            const void *const *partials, const void *residual,
                            const void *gamma, float eps, void *residual_out, void *y,
                            void *stream);

/*
 * (3+1) Sub-layer boundary overlap: reduce + residual + RMSNorm of this rank's rows fused with the
 * next sub-layer's chunked all-gather + column GEMM.
 *
 * [AReaL "Potential Solution", sub-layer boundary overlap]: the norm reduces over the hidden
 * dimension and the gather runs over the sequence, so gathering before the norm gives the same
 * result and lets the gather start earlier.  Here the peers' rows (the other ranks' already
 * normalised shards) start staging at the call's position, before this rank's boundary epilogue
 * runs; the epilogue writes this rank's normalised rows straight into its slot of x_gathered, and
 * the chunk-ordered GEMM follows on `compute`.  The results are bit for bit those of
 *   reduce_residual_rmsnorm(rows = seq_len / tp, partials, residual, gamma, eps, residual_out,
 *                           y = this rank's slot of x_gathered)
 *   agmm_chunked(shard_src with entry `rank` = that slot, ..., copy = NULL, timing = 0)
 * on the same stream; only the peers' copies start earlier (they overlap the epilogue).
 *   n_partials, partials, residual, gamma, eps, residual_out: as reduce_residual_rmsnorm for the
 *            seq_len / tp rows of this rank (hidden columns); residual_out may be NULL
 *   seq_len .. y_dtype, compute: as agmm_chunked; shard_src[rank] is not used (may be NULL)
 * Work on `compute` before the call must be done with x_gathered (the copies start at the call's
 * position, as in agmm_chunked).  Without copy engines the pair runs unfused on `compute`.
 */
int reduce_norm_agmm_chunked(sptl_ctx *ctx, int n_partials, const void *const *partials,
                             const void *residual, const void *gamma, float eps, void *residual_out,
                             int64_t seq_len, int64_t hidden, int64_t n_local, int tp, int n_chunks,
                             int rank, const void *const *shard_src, void *x_gathered,
                             const void *w, void *y, int y_dtype, void *compute);

/*
 * (4) Delayed tensor parallelism: residual update of module `module_idx`.
 *
 * [DTP abstract]: each device adds its own partial output to its residual stream at once
 * and adds the other devices' partials delta modules later.
 *   x <- x + own_partial + [module_idx >= delta] * (peers[0] + ... + peers[tp-2])
 *   y  = x / sqrt(mean_j x_j^2 + eps) * gamma        (from the unrounded fp32 x)
 * Summation order (fp32): x, own, then peers in the given order, so delta = 0 gives the
 * same bits as reduce_residual_rmsnorm with partials [own, peers...].
 *   residual      [seq_len, hidden] bf16, updated in place
 *   own_partial   this rank's partial of module module_idx; NULL marks a flush call (after
 *                 the last module: adds the outstanding peer partials, takes no norm)
 *   delayed_peers host array [tp-1] of device pointers: the peers' partials of module
 *                 module_idx - delta.  Must be NULL when module_idx < delta and non-NULL
 *                 (with non-NULL entries) otherwise.  The caller owns the delay line.
 *   gamma, eps    RMSNorm gain [hidden] bf16 and epsilon; gamma may be NULL when y is NULL
 *   y             [seq_len, hidden] bf16 normalised output; required unless a flush call,
 *                 where it must be NULL.
 *   tp in [1, SPTL_MAX_PARTIALS], delta >= 0, module_idx >= 0.
 */
int dtp_accumulate(sptl_ctx *ctx, int64_t seq_len, int64_t hidden, int tp, int delta,
                   int module_idx, void *residual, const void *own_partial,
                   const void *const *delayed_peers, const void *gamma, float eps,
                   void *y, void *stream);

/*
 * (5) Affinity-aware sharding for delayed TP: the layout of KV heads and FFN neurons over the
 * devices, and the permutation of the dense weights before sharding.
 *
 * [DTP abstract]: delayed TP breaks the permutation symmetry of FFN neurons and of KV heads, so
 * which heads and neurons share a device matters.  The layout maximises the co-located affinity
 *     score = sum over devices d, heads h on d, neurons j on d of affinity[h][j]
 * (affinity[h][j]: how much neuron j's output depends on head h, a first-order estimate the
 * caller computes from a trained model), with n_heads / tp heads and n_neurons / tp neurons per
 * device, by coordinate ascent: each round assigns the neurons exactly for the current heads (a
 * balanced assignment), then tries every head layout for those neurons and keeps the best;
 * it stops after a round that does not raise the score.  Host code; no GPU is used.
 *   affinity      HOST [n_heads, n_neurons] float64, row-major, finite
 *   head_device   HOST [n_heads] int: in, the starting layout (n_heads / tp heads per device, e.g.
 *                 the contiguous one or a seeded random one); out, the optimised one
 *   neuron_device HOST [n_neurons] int, out
 *   score         out: the co-located affinity of the result;  rounds: out, may be NULL
 *   n_heads % tp == 0, n_neurons % tp == 0, 1 <= tp <= 64, max_rounds >= 1.  Ties go to the
 *   first layout in the order the search takes (lower device numbers for lower indices).
 * SPTL_E_UNSUPPORTED when a round would try more than SPTL_MAX_HEAD_LAYOUTS head layouts
 * (n_heads! / ((n_heads / tp)!)^tp); SPTL_E_RANGE for a starting layout that is not balanced.
 */
int dtp_affinity_layout(const double *affinity, int n_heads, int n_neurons, int tp, int max_rounds,
                        int *head_device, int *neuron_device, double *score, int *rounds);

/* The co-located affinity of a given layout (definition above).  Every device index must lie
 * in [0, tp); the layout need not be balanced. */
int dtp_colocated_affinity(const double *affinity, int n_heads, int n_neurons, int tp,
                           const int *head_device, const int *neuron_device, double *score);

/* The permutation that shards a layout: perm lists the items of device 0 in ascending order,
 * then those of device 1, and so on, each item i expanded to the `group` consecutive indices
 * i*group .. i*group + group - 1 (e.g. a KV head's head_dim columns).  HOST arrays: layout [n],
 * perm [n * group] (out).  Device d's shard is then the d-th block of the permuted tensor when
 * the layout is balanced. */
int dtp_layout_permutation(const int *layout, int n, int tp, int group, int32_t *perm);

/* [DTP abstract] "permuting the dense model before sharding": dst = src with its rows (dim 0:
 * dst[i, :] = src[perm[i], :]) or its columns (dim 1: dst[:, j] = src[:, perm[j]]) permuted.
 *   src, dst [rows, cols] bf16, distinct, 16-byte aligned; cols % 8 == 0
 *   perm     DEVICE int32 array [rows] (dim 0) or [cols] (dim 1), 4-byte aligned
 * An index out of range gives zeros in its place; sptl_ctx_check then reports SPTL_E_ASYNC. */
int permute_bf16(sptl_ctx *ctx, const void *src, void *dst, int64_t rows, int64_t cols, int dim,
                 const int32_t *perm, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPTL_H */
