// C ABI of libsptl.so: argument validation, contexts, and the copy/compute scheduler of the
// chunked all-gather + column-parallel GEMM.  The declarations, with argument meaning,
// layout, ownership and error behaviour, are in include/sptl.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "sptl.h"
#include "sptl_affinity.h"
#include "sptl_internal.h"
#include "sptl_noalloc.h"
#include "sptl_stager.h"

struct sptl_ctx {
    int device = 0;
    // SDMA stager (chunk-ordered path); created on first use, null if unavailable
    sptl::SdmaStager *stager = nullptr;
    bool stager_tried = false;
    bool events_only = false;           // SPTL_STAGING=events: no stager, copy mode SPTL_COPY_EVENTS
    int copy_mode = SPTL_COPY_STAGED;   // sptl_ctx_set_copy_mode
    int blit_wgs = 0;                   // workgroups of a blit-mode copy (0: sized to the copy)
    int chunk_order = SPTL_ORDER_RING;  // sptl_ctx_set_staging
    int engines_per_peer = 0;           // sptl_ctx_set_staging (0: every copy over all engines)
    std::string staging_info;           // how agmm_chunked stages chunks, and why
    int *err_dev = nullptr;             // device flag set by a timed-out staging wait
    uint64_t *ts_dev = nullptr;         // [3 * kMaxPlanChunks + 1] chunk timestamps
    uint64_t *flags_dev = nullptr;      // landed flags, kFlagSetWords per stager set
    int wallclock_khz = 100000;
    int64_t cus = 256;                  // compute units of the device
    uint64_t wait_timeout_us = 10000000;  // bound on one chunk wait inside the GEMM (default 10 s)
    int t_mode = 0;                     // 0: event timeline, 1: chunk-ordered timeline
    int t_rank_first = 0, t_rank_count = 0;
    int t_set = -1;                     // stager set and epoch of the last timed chunk-ordered call
    uint64_t t_epoch = 0;
    hipStream_t copy_stream = nullptr;  // created on first use
    hipEvent_t fork = nullptr;          // compute stream -> copy stream
    hipEvent_t join = nullptr;          // copy stream -> compute stream
    std::vector<hipEvent_t> ready;      // per chunk: its staging copy has landed
    // timeline of the last timed agmm_chunked call
    hipEvent_t t_base = nullptr;
    std::vector<hipEvent_t> t_copy_start, t_gemm_start, t_gemm_end;
    std::vector<char> t_has_copy;
    int t_chunks = -1;
};

namespace {

constexpr uint64_t kDefaultWaitUs = 10000000;  // default bound on one chunk wait (10 s)
thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(SPTL_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define SPTL_HIP(call)                                  \
    do {                                                \
        hipError_t e_ = (call);                         \
        if (e_ != hipSuccess) return hip_fail(e_, #call); \
    } while (0)

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Switches to the context's device for the duration of a call.
struct DeviceGuard {
    int prev = -1;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev) {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
        else if (err == hipSuccess) prev = -1;
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

int make_event(hipEvent_t *e) {
    SPTL_HIP(hipEventCreate(e));
    return SPTL_OK;
}

int grow_events(std::vector<hipEvent_t> &v, size_t n) {
    while (v.size() < n) {
        hipEvent_t e;
        int rc = make_event(&e);
        if (rc) return rc;
        v.push_back(e);
    }
    return SPTL_OK;
}

// Creates the context's SDMA stager (at context creation, with the context's device current);
// without one, agmm_chunked takes the per-chunk event path.
void make_stager(sptl_ctx *ctx) {
    ctx->stager_tried = true;
    if (ctx->events_only) return;
    std::string why;
    ctx->stager = sptl::stager_create(ctx->device, &why);
    ctx->staging_info = ctx->stager ? "sdma-striped over " + std::to_string(sptl::stager_engine_count(ctx->stager)) +
                                          " engines, chunk-ordered GEMM"
                                    : "per-chunk events (copy engines unavailable: " + why + ")";
}

int create_ctx(sptl_ctx **out, int device) {
    int count = 0;
    SPTL_HIP(hipGetDeviceCount(&count));
    if (device < 0 || device >= count)
        return fail(SPTL_E_RANGE, "device %d out of range [0, %d)", device, count);
    DeviceGuard g(device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    auto *c = new (std::nothrow) sptl_ctx;
    if (!c) return fail(SPTL_E_HIP, "out of host memory");
    c->device = device;
    int rc = SPTL_OK;
    if (!rc) rc = make_event(&c->fork);
    if (!rc) rc = make_event(&c->join);
    if (!rc) rc = make_event(&c->t_base);
    if (!rc) rc = grow_events(c->ready, 64);
    if (!rc && hipMalloc(&c->err_dev, 256) != hipSuccess) rc = fail(SPTL_E_HIP, "hipMalloc of the error flag failed");
    if (!rc && hipMalloc(&c->ts_dev, sizeof(uint64_t) * (3 * sptl::kMaxPlanChunks + 8)) != hipSuccess)
        rc = fail(SPTL_E_HIP, "hipMalloc of the timestamp buffer failed");
    if (!rc && hipMalloc(&c->flags_dev, sizeof(uint64_t) * sptl::kFlagSetWords * sptl::kStageSets) != hipSuccess)
        rc = fail(SPTL_E_HIP, "hipMalloc of the landed flags failed");
    if (!rc && (hipMemset(c->err_dev, 0, 256) != hipSuccess ||
                hipMemset(c->flags_dev, 0, sizeof(uint64_t) * sptl::kFlagSetWords * sptl::kStageSets) != hipSuccess ||
                hipDeviceSynchronize() != hipSuccess))
        rc = fail(SPTL_E_HIP, "hipMemset failed");
    if (!rc) {
        (void)hipDeviceGetAttribute(&c->wallclock_khz, hipDeviceAttributeWallClockRate, device);
        if (c->wallclock_khz <= 0) c->wallclock_khz = 100000;
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess && cus > 0)
            c->cus = cus;
        const char *e = getenv("SPTL_STAGING");
        c->events_only = e && !strcmp(e, "events");
        if (c->events_only) c->copy_mode = SPTL_COPY_EVENTS;
        // SPTL_WAIT_TIMEOUT_US shortens the bound on a chunk wait (failure-path tests)
        if (const char *t = getenv("SPTL_WAIT_TIMEOUT_US")) {
            const long long us = strtoll(t, nullptr, 10);
            if (us >= 1 && us <= 10000000) c->wait_timeout_us = (uint64_t)us;
        }
        // set-up for agmm_chunked_noalloc: the device's scratch array and this context's
        // copy engines, so that the call itself allocates nothing
        std::string why;
        if (sptl::noalloc_setup(device, &why)) rc = fail(SPTL_E_HIP, "sptl_create: %s", why.c_str());
        if (!rc) make_stager(c);
    }
    if (rc) {
        sptl_destroy(c);
        return rc;
    }
    *out = c;
    return SPTL_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_default_mu;
sptl_ctx *g_default[kMaxDevices] = {};

// Resolves a NULL ctx to the current device's default context.
int resolve_ctx(sptl_ctx *&ctx) {
    if (ctx) return SPTL_OK;
    int dev = 0;
    SPTL_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(SPTL_E_RANGE, "device %d unsupported", dev);
    std::lock_guard<std::mutex> lk(g_default_mu);
    if (!g_default[dev]) {
        int rc = create_ctx(&g_default[dev], dev);
        if (rc) return rc;
    }
    ctx = g_default[dev];
    return SPTL_OK;
}

int copy_stream_of(sptl_ctx *ctx, hipStream_t *out) {
    if (!ctx->copy_stream) SPTL_HIP(hipStreamCreateWithFlags(&ctx->copy_stream, hipStreamNonBlocking));
    *out = ctx->copy_stream;
    return SPTL_OK;
}

int check_gemm_dims(int64_t m, int64_t k, int64_t n) {
    if (m < 0 || k <= 0 || n <= 0)
        return fail(SPTL_E_SHAPE, "bad GEMM sizes m=%lld k=%lld n=%lld", (long long)m, (long long)k,
                    (long long)n);
    if (k % 8 || n % 8)
        return fail(SPTL_E_DIVISIBILITY, "k=%lld and n=%lld must be multiples of 8", (long long)k,
                    (long long)n);
    // the kernels address a tile's A rows and B rows with 32-bit byte offsets
    if (k > SPTL_MAX_K || n > SPTL_MAX_N)
        return fail(SPTL_E_SHAPE, "k=%lld or n=%lld above the limits %d and %d", (long long)k, (long long)n,
                    SPTL_MAX_K, SPTL_MAX_N);
    // grid of 128 x 128 tiles must fit a 32-bit dimension
    if (((m + 127) / 128) * ((n + 127) / 128) > 0x7fffffffLL)
        return fail(SPTL_E_SHAPE, "GEMM too large for one launch");
    return SPTL_OK;
}

// SPTL_POLL_SLEEP=0..64: extra s_sleep 127 per poll of a bounded wait (measurement aid).
int poll_sleep_setting() {
    static const int v = [] {
        const char *e = getenv("SPTL_POLL_SLEEP");
        const long x = e ? strtol(e, nullptr, 10) : 0;
        return (int)(x >= 0 && x <= 64 ? x : 0);
    }();
    return v;
}

// Whether stream s is being captured into a graph (a failed query counts as captured: the
// per-chunk path is correct either way, the staged one needs its worker thread at run time).
bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(s, &st) != hipSuccess || st != hipStreamCaptureStatusNone;
}

// Whether the chunk-ordered path (SDMA stager + one chunk-ordered GEMM) can serve this call on
// compute stream cs.
bool staged_path(sptl_ctx *ctx, int64_t rows_c, int n_chunks, hipStream_t cs) {
    if (ctx->copy_mode != SPTL_COPY_STAGED || n_chunks > sptl::kMaxPlanChunks || !sptl::chunk_tile_rows(rows_c))
        return false;
    return ctx->stager && !sptl::stager_failed(ctx->stager) && !capturing(cs);
}

// One staging copy of the per-chunk and serial paths on stream s: a copy-engine (SDMA-class)
// copy, recorded as a plain device-to-device copy node under graph capture, or in blit mode a
// copy kernel on the compute units.
hipError_t stage_copy(const sptl_ctx *ctx, void *dst, const void *src, size_t bytes, hipStream_t s, bool cap) {
    if (ctx->copy_mode == SPTL_COPY_BLIT) return sptl::launch_blit(dst, src, bytes, ctx->blit_wgs, s);
    return hipMemcpyAsync(dst, src, bytes, cap ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToDeviceNoCU, s);
}

// The peers' chunks of agmm_chunked in processing (and arrival) order under ctx's chunk order:
// ring, peer by peer (rank+1's sub-chunks, then rank+2's, ...), or interleaved, sub-chunk by
// sub-chunk (sub-chunk 0 of rank+1, rank+2, ..., then sub-chunk 1 of each, ...).
std::vector<int> peer_chunk_order(const sptl_ctx *ctx, int rank, int tp, int cpr) {
    std::vector<int> out;
    out.reserve((size_t)(tp - 1) * (size_t)cpr);
    if (ctx->chunk_order == SPTL_ORDER_INTERLEAVED) {
        for (int s = 0; s < cpr; ++s)
            for (int d = 1; d < tp; ++d) out.push_back(((rank + d) % tp) * cpr + s);
    } else {
        for (int d = 1; d < tp; ++d)
            for (int s = 0; s < cpr; ++s) out.push_back(((rank + d) % tp) * cpr + s);
    }
    return out;
}

// Chunk-ordered agmm: all staging copies go to the SDMA stager (striped over the copy
// engines, released at the fork point), and one GEMM launch processes the row tiles in
// chunk order, each tile waiting for its chunk's completion signal.  Arguments validated.
// na: null for the context's own state (landed flags, error word, the stager's cumulative end
// counters), or the device scratch of agmm_chunked_noalloc (timing is then 0).  pre: an epilogue
// launched on cs between the fork point and the GEMM (the sub-layer boundary of
// reduce_norm_agmm_chunked; it writes the own slot, which shard_src[rank] then aliases).
int agmm_staged(sptl_ctx *ctx, int64_t seq_len, int64_t hidden, int64_t n_local, int tp, int n_chunks,
                int rank, const void *const *shard_src, uint16_t *xg, const void *w, void *y, int y_dtype,
                hipStream_t cs, int timing, const sptl::NoallocScratch *na = nullptr,
                const sptl::EpilogueProblem *pre = nullptr) {
    const int cpr = n_chunks / tp;
    const int64_t rows_c = seq_len / n_chunks;
    const size_t chunk_elems = (size_t)rows_c * (size_t)hidden;
    const size_t chunk_bytes = chunk_elems * 2;
    auto src_chunk = [&](int q, int s) {
        return static_cast<const uint16_t *>(shard_src[q]) + (size_t)s * chunk_elems;
    };
    const bool own_aliased = shard_src[rank] == xg + (size_t)rank * cpr * chunk_elems;

    // copies in arrival order (the peers' chunks in the context's chunk order), then this rank's
    // own slot; link: each copy's peer (0 for rank+1, ...), -1 for the own slot
    std::vector<sptl::CopyPiece> copies;
    std::vector<int> link;
    sptl::GemmProblem gp{};
    sptl::ChunkPlan &plan = gp.plan;
    int pos = 0;
    for (int s = 0; s < cpr; ++s) plan.order[pos++] = rank * cpr + s;
    for (const int c : peer_chunk_order(ctx, rank, tp, cpr)) {
        const int q = c / cpr;
        plan.order[pos++] = c;
        copies.push_back({xg + (size_t)c * chunk_elems, src_chunk(q, c % cpr), chunk_bytes, c});
        link.push_back((q - rank + tp) % tp - 1);
    }
    if (!own_aliased) {
        copies.push_back({xg + (size_t)rank * cpr * chunk_elems, shard_src[rank], chunk_bytes * cpr, sptl::kJoinChunk});
        link.push_back(-1);
    }
    const int n = n_chunks;
    gp.a = xg;
    gp.b = static_cast<const uint16_t *>(w);
    gp.c = y;
    gp.m = seq_len;
    gp.n = n_local;
    gp.k = hidden;
    gp.lda = hidden;
    gp.ldb = n_local;
    gp.ldc = n_local;
    gp.c_f32 = y_dtype == SPTL_F32;
    plan.chunk_rows = (int)rows_c;
    plan.n_chunks = n;
    plan.own_first = rank * cpr;
    plan.own_count = cpr;
    plan.own_a = static_cast<const uint16_t *>(shard_src[rank]);
    plan.err = na ? na->err : ctx->err_dev;
    plan.timeout_ticks = (uint64_t)ctx->wallclock_khz * ctx->wait_timeout_us / 1000u;
    plan.poll_sleep = poll_sleep_setting();
    // SPTL_CHUNK_XCDS=g (1, 2, 4 or 8) spreads every chunk's tiles over g XCDs (measurement aid)
    static const int xcd_group = [] {
        const char *e = getenv("SPTL_CHUNK_XCDS");
        const long v = e ? strtol(e, nullptr, 10) : 0;
        return (int)(v == 1 || v == 2 || v == 4 || v == 8 ? v : 0);
    }();
    plan.xcd_group = xcd_group;
    plan.ts = timing ? ctx->ts_dev : nullptr;

    // The GEMM's first round of tiles (one per CU) spans the own chunks and the first `lead`
    // peer chunks; those peers are staged together so that the round starts complete as early
    // as the engines allow.  The round is sized for an output at least `hidden` wide, so that a
    // narrower weight stages its chunks the same way as a full-width one.
    const int64_t wgs = sptl::gemm_workgroups(gp);
    sptl::GemmProblem wide = gp;
    wide.n = std::max(gp.n, gp.k);
    const int64_t per_chunk = std::max<int64_t>(1, sptl::gemm_workgroups(wide) / n);
    const int64_t first_round = (ctx->cus + per_chunk - 1) / per_chunk;
    const int lead = (int)std::max<int64_t>(1, std::min<int64_t>(first_round - cpr, (int64_t)(n - cpr)));
    // When the own chunks do not fill the first round, the lead chunks' tiles are resident from
    // the start and would wait for the engines: they copy the lead chunks themselves (ChunkPlan,
    // cu_n), and the engines take the later chunks.  Not under the link model, whose point is a
    // rate per peer.  SPTL_CU_LEAD=0 leaves every chunk to the engines (measurement aid).
    static const bool cu_lead_on = [] {
        const char *e = getenv("SPTL_CU_LEAD");
        return !(e && !strcmp(e, "0"));
    }();
    const bool links = ctx->engines_per_peer > 0;
    const int cu = cu_lead_on && !links && first_round > cpr ? std::min(lead, sptl::kMaxCuChunks) : 0;
    plan.cu_n = cu;
    plan.cu_mask = 0;
    plan.cu_chunk_bytes = (int64_t)chunk_bytes;
    for (int i = 0; i < cu; ++i) {
        plan.cu_src[i] = copies[(size_t)i].src;
        plan.cu_dst[i] = copies[(size_t)i].dst;
        plan.cu_mask |= 1ull << copies[(size_t)i].chunk;
    }
    copies.erase(copies.begin(), copies.begin() + cu);
    std::vector<sptl::CopyPiece> pieces =
        links ? sptl::stager_plan_links(ctx->stager, copies, link, ctx->engines_per_peer)
              : sptl::stager_plan(ctx->stager, copies, std::max(1, lead - cu));

    sptl::StageCall call;
    std::string why;
    if (int rc = sptl::stager_begin(ctx->stager, pieces, wgs, &call, &why, na ? na->counts : nullptr))
        return fail(rc == -2 ? SPTL_E_ASYNC : SPTL_E_HIP, "agmm_chunked: %s", why.c_str());
    for (int c = 0; c < n; ++c) {
        plan.ready[c] = call.ready[c];
        plan.ready_n[c] = call.ready_n[c];
    }
    for (int s = 0; s < cpr; ++s) plan.ready[rank * cpr + s] = nullptr;  // read from the source
    plan.join = call.join;
    plan.join_n = call.join_n;
    plan.flags = na ? na->flags : ctx->flags_dev + (size_t)call.set * sptl::kFlagSetWords;
    plan.epoch = call.epoch;
    plan.flag_epoch = na ? na->flag_epoch : call.epoch;  // the context's flags are the set's own
    plan.finished = call.finished;
    plan.timedout = call.timedout;
    plan.wg_count = call.wg_count;
    for (int g = 0; g < sptl::kEndGroups; ++g) plan.grp_last[g] = call.grp_last[g];
    plan.all_last = call.all_last;
    hipError_t he = hipSuccess;
    if (na) he = sptl::launch_fill_u64(na->counts, na->count_words, 0ull, cs);  // a kernel, not a memset
    if (he == hipSuccess && timing) {
        // first landings and tile starts (minima), last tile ends (maxima), the origin (a minimum)
        he = sptl::launch_fill_u64(ctx->ts_dev, 2 * n, ~0ull, cs);
        if (he == hipSuccess) he = sptl::launch_fill_u64(ctx->ts_dev + 2 * n, n, 0ull, cs);
        if (he == hipSuccess) he = sptl::launch_fill_u64(ctx->ts_dev + 3 * n, 1, ~0ull, cs);
    }
    // The copies start once every earlier operation on the stream has completed.  When no tile
    // of the GEMM's first round waits for an engine copy (the own chunks fill the round, or the
    // launch's own workgroups copy its peer chunks), they start at the GEMM's start, which its
    // tile 0 reports: the worker sees that a little later than a fork event, but the event's
    // marker on the stream costs several microseconds of GPU time before the launch.  Otherwise
    // (and ahead of an epilogue launched before the GEMM, `pre`, whose run the copies overlap)
    // at a fork event recorded before the launch.
    const int first_peers = (int)std::max<int64_t>(0, std::min<int64_t>(first_round - cpr, (int64_t)(n - cpr)));
    const bool by_start = !pre && cu >= first_peers;
    plan.started = by_start ? call.started : nullptr;
    if (he == hipSuccess && !by_start) he = hipEventRecord(call.fork, cs);
    if (he == hipSuccess && pre) he = sptl::launch_epilogue(*pre, cs);  // the copies run meanwhile
    if (he == hipSuccess) he = sptl::launch_gemm(gp, cs);
    if (he != hipSuccess) {
        sptl::stager_cancel(ctx->stager, call);
        return hip_fail(he, "agmm_chunked: kernel launch");
    }
    if (sptl::stager_submit(ctx->stager, call, std::move(pieces), &why, false,
                            by_start ? sptl::ForkWait::Started : sptl::ForkWait::Event))
        return fail(SPTL_E_HIP, "agmm_chunked: %s", why.c_str());
    if (timing) {
        ctx->t_mode = 1;
        ctx->t_chunks = n;
        ctx->t_set = call.set;
        ctx->t_epoch = call.epoch;
        ctx->t_rank_first = rank * cpr;
        ctx->t_rank_count = cpr;
    }
    return SPTL_OK;
}

}  // namespace

extern "C" {

int sptl_version(void) { return 100; }

const char *sptl_ctx_info(sptl_ctx *ctx) {
    if (resolve_ctx(ctx)) return "";
    if (ctx->events_only) return "per-chunk events (forced by SPTL_STAGING=events)";
    if (ctx->copy_mode == SPTL_COPY_EVENTS) return "per-chunk events (copy mode)";
    if (ctx->copy_mode == SPTL_COPY_BLIT) return "per-chunk events with copy kernels (blit copy mode)";
    if (ctx->copy_mode == SPTL_COPY_SERIAL) return "copies, then the GEMM (serial copy mode)";
    if (!ctx->stager_tried) return "no copy engines set up";
    return ctx->staging_info.c_str();
}

int sptl_ctx_check(sptl_ctx *ctx) {
    if (int rc = resolve_ctx(ctx)) return rc;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    if (ctx->stager)
        if (int rc = sptl::stager_wait_idle(ctx->stager))
            return fail(rc == -2 ? SPTL_E_ASYNC : SPTL_E_HIP,
                        rc == -2 ? "sptl_ctx_check: the copies of a timed-out call did not complete"
                                 : "sptl_ctx_check: waiting for staged calls failed");
    // [0]: a staging wait timed out; [1]: a permutation index was out of range; [2]: a copy-out
    // tile ran on another XCD than the one its slice's release counted it on
    int flag[3] = {0, 0, 0};
    SPTL_HIP(hipMemcpy(flag, ctx->err_dev, sizeof flag, hipMemcpyDeviceToHost));
    if (flag[0] || flag[1] || flag[2]) SPTL_HIP(hipMemset(ctx->err_dev, 0, sizeof flag));
    if (flag[1]) return fail(SPTL_E_ASYNC, "permute_bf16: an index was out of range (zeros written there)");
    if (flag[2])
        return fail(SPTL_E_ASYNC, "gemm_rs_chunked: an XCD ran more tiles of a slice than counted for it; the "
                                  "copied slices of that call may hold stale rows");
    if (flag[0]) {
        if (ctx->stager) (void)sptl::stager_take_timeouts(ctx->stager);  // the same report
        return fail(SPTL_E_ASYNC, "a staging wait timed out; the affected agmm_chunked results are invalid");
    }
    if (ctx->stager && sptl::stager_take_timeouts(ctx->stager))
        return fail(SPTL_E_ASYNC, "a staging wait timed out; the affected agmm_chunked results are invalid");
    if (ctx->stager && sptl::stager_failed(ctx->stager))
        return fail(SPTL_E_ASYNC, "a staging copy could not be submitted; the staged path is now disabled");
    return SPTL_OK;
}

const char *sptl_last_error(void) { return g_err.c_str(); }

int sptl_ctx_set_wait_timeout_us(sptl_ctx *ctx, int64_t us) {
    if (!ctx) return fail(SPTL_E_NULL, "sptl_ctx_set_wait_timeout_us: ctx is NULL");
    if (us < 0 || us > 10000000)
        return fail(SPTL_E_RANGE, "sptl_ctx_set_wait_timeout_us: us=%lld not in [0, 10000000]", (long long)us);
    ctx->wait_timeout_us = us ? (uint64_t)us : kDefaultWaitUs;
    return SPTL_OK;
}

int sptl_ctx_set_copy_mode(sptl_ctx *ctx, int mode, int blit_workgroups) {
    if (!ctx) return fail(SPTL_E_NULL, "sptl_ctx_set_copy_mode: ctx is NULL");
    if (mode < SPTL_COPY_STAGED || mode > SPTL_COPY_SERIAL)
        return fail(SPTL_E_RANGE, "sptl_ctx_set_copy_mode: mode=%d", mode);
    if (blit_workgroups < 0 || blit_workgroups > 65535)
        return fail(SPTL_E_RANGE, "sptl_ctx_set_copy_mode: blit_workgroups=%d not in [0, 65535]", blit_workgroups);
    ctx->copy_mode = mode;
    ctx->blit_wgs = blit_workgroups;
    return SPTL_OK;
}

int sptl_ctx_set_staging(sptl_ctx *ctx, int order, int engines_per_peer) {
    if (!ctx) return fail(SPTL_E_NULL, "sptl_ctx_set_staging: ctx is NULL");
    if (order != SPTL_ORDER_RING && order != SPTL_ORDER_INTERLEAVED)
        return fail(SPTL_E_RANGE, "sptl_ctx_set_staging: order=%d", order);
    if (engines_per_peer < 0 || engines_per_peer > sptl::kMaxPieces)
        return fail(SPTL_E_RANGE, "sptl_ctx_set_staging: engines_per_peer=%d not in [0, %d]", engines_per_peer,
                    sptl::kMaxPieces);
    ctx->chunk_order = order;
    ctx->engines_per_peer = engines_per_peer;
    return SPTL_OK;
}

int sptl_create(sptl_ctx **out, int device) {
    if (!out) return fail(SPTL_E_NULL, "out is NULL");
    *out = nullptr;
    return create_ctx(out, device);
}

int sptl_destroy(sptl_ctx *ctx) {
    if (!ctx) return SPTL_OK;
    DeviceGuard g(ctx->device);
    if (ctx->stager) sptl::stager_destroy(ctx->stager);
    if (ctx->err_dev) (void)hipFree(ctx->err_dev);
    if (ctx->ts_dev) (void)hipFree(ctx->ts_dev);
    if (ctx->flags_dev) (void)hipFree(ctx->flags_dev);
    if (ctx->copy_stream) {
        (void)hipStreamSynchronize(ctx->copy_stream);
        (void)hipStreamDestroy(ctx->copy_stream);
    }
    for (hipEvent_t e : {ctx->fork, ctx->join, ctx->t_base})
        if (e) (void)hipEventDestroy(e);
    for (auto *v : {&ctx->ready, &ctx->t_copy_start, &ctx->t_gemm_start, &ctx->t_gemm_end})
        for (hipEvent_t e : *v) (void)hipEventDestroy(e);
    {
        std::lock_guard<std::mutex> lk(g_default_mu);
        for (int d = 0; d < kMaxDevices; ++d)
            if (g_default[d] == ctx) g_default[d] = nullptr;
    }
    delete ctx;
    return SPTL_OK;
}

}  // extern "C"

namespace {

// Argument checks shared by agmm_chunked and agmm_chunked_noalloc (fn names the call).
int check_agmm_args(const char *fn, int64_t seq_len, int64_t hidden, int64_t n_local, int tp, int n_chunks,
                    int rank, const void *const *shard_src, const void *x_gathered, const void *w, const void *y,
                    int y_dtype) {
    if (!shard_src || !x_gathered || !w || !y) return fail(SPTL_E_NULL, "%s: NULL pointer argument", fn);
    if (seq_len < 0 || hidden <= 0 || n_local <= 0)
        return fail(SPTL_E_SHAPE, "%s: bad sizes seq_len=%lld hidden=%lld n_local=%lld", fn, (long long)seq_len,
                    (long long)hidden, (long long)n_local);
    if (tp < 1 || tp > SPTL_MAX_TP) return fail(SPTL_E_RANGE, "%s: tp=%d not in [1, %d]", fn, tp, SPTL_MAX_TP);
    if (n_chunks < 1 || n_chunks > SPTL_MAX_CHUNKS)
        return fail(SPTL_E_RANGE, "%s: n_chunks=%d not in [1, %d]", fn, n_chunks, SPTL_MAX_CHUNKS);
    if (rank < 0 || rank >= tp) return fail(SPTL_E_RANGE, "%s: rank=%d not in [0, %d)", fn, rank, tp);
    if (n_chunks % tp) return fail(SPTL_E_DIVISIBILITY, "%s: n_chunks=%d not a multiple of tp=%d", fn, n_chunks, tp);
    if (seq_len % n_chunks)
        return fail(SPTL_E_DIVISIBILITY, "%s: seq_len=%lld not a multiple of n_chunks=%d", fn, (long long)seq_len,
                    n_chunks);
    if (y_dtype != SPTL_BF16 && y_dtype != SPTL_F32) return fail(SPTL_E_DTYPE, "%s: y_dtype=%d", fn, y_dtype);
    if (int rc = check_gemm_dims(seq_len / n_chunks, hidden, n_local)) return rc;
    for (int q = 0; q < tp; ++q) {
        if (!shard_src[q]) return fail(SPTL_E_NULL, "%s: shard_src[%d] is NULL", fn, q);
        if (!aligned16(shard_src[q])) return fail(SPTL_E_ALIGN, "%s: shard_src[%d] not 16-byte aligned", fn, q);
    }
    if (!aligned16(x_gathered) || !aligned16(w) || !aligned16(y))
        return fail(SPTL_E_ALIGN, "%s: x_gathered, w and y must be 16-byte aligned", fn);
    return SPTL_OK;
}

}  // namespace

extern "C" {

int agmm_chunked(sptl_ctx *ctx, int64_t seq_len, int64_t hidden, int64_t n_local, int tp,
                 int n_chunks, int rank, const void *const *shard_src, void *x_gathered,
                 const void *w, void *y, int y_dtype, void *compute, void *copy, int timing) {
    // ---- validation: nothing is enqueued on failure ------------------------------------
    if (int rc = check_agmm_args("agmm_chunked", seq_len, hidden, n_local, tp, n_chunks, rank, shard_src, x_gathered,
                                 w, y, y_dtype))
        return rc;
    if (timing != 0 && timing != 1) return fail(SPTL_E_RANGE, "agmm_chunked: timing=%d", timing);
    if (seq_len == 0) return SPTL_OK;
    if (int rc = resolve_ctx(ctx)) return rc;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");

    hipStream_t cs = static_cast<hipStream_t>(compute);
    const bool cap = capturing(cs);
    const bool serial = !copy && ctx->copy_mode == SPTL_COPY_SERIAL;
    if (timing && (cap || serial))
        return fail(SPTL_E_UNSUPPORTED, "agmm_chunked: timing with %s", cap ? "a stream under graph capture"
                                                                              : "the serial copy mode");
    if (!copy && staged_path(ctx, seq_len / n_chunks, n_chunks, cs)) {
        ctx->t_chunks = -1;
        return agmm_staged(ctx, seq_len, hidden, n_local, tp, n_chunks, rank, shard_src,
                           static_cast<uint16_t *>(x_gathered), w, y, y_dtype, cs, timing);
    }
    if (serial) {
        // no overlap (the baseline the overlap is measured against): every copy on `compute`,
        // then one GEMM over all gathered rows
        if (int rc = check_gemm_dims(seq_len, hidden, n_local)) return rc;
        ctx->t_chunks = -1;
        auto *xg = static_cast<uint16_t *>(x_gathered);
        const size_t shard_elems = (size_t)(seq_len / tp) * (size_t)hidden;
        for (int d = 1; d <= tp; ++d) {
            const int q = (rank + d) % tp;
            if (shard_src[q] != xg + (size_t)q * shard_elems)
                SPTL_HIP(stage_copy(ctx, xg + (size_t)q * shard_elems, shard_src[q], shard_elems * 2, cs, cap));
        }
        sptl::GemmProblem gp{};
        gp.a = xg;
        gp.b = static_cast<const uint16_t *>(w);
        gp.c = y;
        gp.m = seq_len;
        gp.n = n_local;
        gp.k = hidden;
        gp.lda = hidden;
        gp.ldb = n_local;
        gp.ldc = n_local;
        gp.c_f32 = y_dtype == SPTL_F32;
        SPTL_HIP(sptl::launch_gemm(gp, cs));
        return SPTL_OK;
    }
    // ---- event path: one copy per chunk on a copy stream, one GEMM launch per chunk ----
    hipStream_t ps = static_cast<hipStream_t>(copy);
    if (!ps)
        if (int rc = copy_stream_of(ctx, &ps)) return rc;
    if (int rc = grow_events(ctx->ready, n_chunks)) return rc;
    if (timing) {
        for (auto *v : {&ctx->t_copy_start, &ctx->t_gemm_start, &ctx->t_gemm_end})
            if (int rc = grow_events(*v, n_chunks)) return rc;
        ctx->t_has_copy.assign(n_chunks, 0);
        ctx->t_chunks = -1;
    }

    const int cpr = n_chunks / tp;                    // chunks per rank
    const int64_t rows_c = seq_len / n_chunks;        // rows per chunk
    const size_t chunk_elems = (size_t)rows_c * (size_t)hidden;
    const size_t chunk_bytes = chunk_elems * 2;
    auto *xg = static_cast<uint16_t *>(x_gathered);
    auto src_chunk = [&](int q, int s) {
        return static_cast<const uint16_t *>(shard_src[q]) + (size_t)s * chunk_elems;
    };
    const bool own_aliased = shard_src[rank] == xg + (size_t)rank * cpr * chunk_elems;

    // ---- fork: copies start only after earlier work on the compute stream -------------
    if (timing) SPTL_HIP(hipEventRecord(ctx->t_base, cs));
    SPTL_HIP(hipEventRecord(ctx->fork, cs));
    SPTL_HIP(hipStreamWaitEvent(ps, ctx->fork, 0));

    // ---- copy stream: every staging copy is enqueued before any GEMM ------------------
    // Peers in the context's chunk order (ring by default: rank+1, rank+2, ..., the order of
    // arrival in a real ring).  hipMemcpyDeviceToDeviceNoCU keeps the copies on the SDMA engines
    // (a plain device-to-device copy may run as a copy kernel on the compute units); the blit
    // mode runs them as a copy kernel on purpose.
    const std::vector<int> peers = peer_chunk_order(ctx, rank, tp, cpr);
    for (const int c : peers) {
        if (timing) {
            SPTL_HIP(hipEventRecord(ctx->t_copy_start[c], ps));
            ctx->t_has_copy[c] = 1;
        }
        SPTL_HIP(stage_copy(ctx, xg + (size_t)c * chunk_elems, src_chunk(c / cpr, c % cpr), chunk_bytes, ps, cap));
        SPTL_HIP(hipEventRecord(ctx->ready[c], ps));
    }
    if (!own_aliased) {
        // this rank's own slot; its GEMMs read the source directly and do not wait for it
        const int c0 = rank * cpr;
        if (timing) {
            SPTL_HIP(hipEventRecord(ctx->t_copy_start[c0], ps));
            for (int s = 0; s < cpr; ++s) ctx->t_has_copy[c0 + s] = 1;
        }
        SPTL_HIP(stage_copy(ctx, xg + (size_t)c0 * chunk_elems, shard_src[rank], chunk_bytes * cpr, ps, cap));
        SPTL_HIP(hipEventRecord(ctx->ready[c0], ps));
        for (int s = 1; s < cpr; ++s) {
            if (timing) SPTL_HIP(hipEventRecord(ctx->t_copy_start[c0 + s], ps));
            SPTL_HIP(hipEventRecord(ctx->ready[c0 + s], ps));
        }
    }
    SPTL_HIP(hipEventRecord(ctx->join, ps));

    // ---- compute stream: own chunks first, then each chunk once its copy has landed ----
    sptl::GemmProblem gp{};
    gp.b = static_cast<const uint16_t *>(w);
    gp.m = rows_c;
    gp.n = n_local;
    gp.k = hidden;
    gp.lda = hidden;
    gp.ldb = n_local;
    gp.ldc = n_local;
    gp.c_f32 = y_dtype == SPTL_F32;
    const size_t esz = gp.c_f32 ? 4 : 2;
    auto run_chunk = [&](int c, const uint16_t *a) -> int {
        gp.a = a;
        gp.c = static_cast<char *>(y) + (size_t)c * (size_t)rows_c * (size_t)n_local * esz;
        if (timing) SPTL_HIP(hipEventRecord(ctx->t_gemm_start[c], cs));
        SPTL_HIP(sptl::launch_gemm(gp, cs));
        if (timing) SPTL_HIP(hipEventRecord(ctx->t_gemm_end[c], cs));
        return SPTL_OK;
    };
    for (int s = 0; s < cpr; ++s)
        if (int rc = run_chunk(rank * cpr + s, src_chunk(rank, s))) return rc;
    for (const int c : peers) {
        SPTL_HIP(hipStreamWaitEvent(cs, ctx->ready[c], 0));
        if (int rc = run_chunk(c, xg + (size_t)c * chunk_elems)) return rc;
    }
    // ---- join: later work on the compute stream sees x_gathered complete ---------------
    SPTL_HIP(hipStreamWaitEvent(cs, ctx->join, 0));
    if (timing) {
        ctx->t_mode = 0;
        ctx->t_chunks = n_chunks;
    }
    return SPTL_OK;
}

int agmm_chunked_noalloc(sptl_ctx *ctx, int64_t seq_len, int64_t hidden, int64_t n_local, int tp, int n_chunks,
                         int rank, const void *const *shard_src, void *x_gathered, const void *w, void *y,
                         int y_dtype, void *compute) {
    static const char *fn = "agmm_chunked_noalloc";
    if (!ctx) return fail(SPTL_E_NULL, "%s: ctx is NULL (its set-up happens in sptl_create)", fn);
    if (int rc = check_agmm_args(fn, seq_len, hidden, n_local, tp, n_chunks, rank, shard_src, x_gathered, w, y,
                                 y_dtype))
        return rc;
    if (n_chunks > sptl::kMaxPlanChunks)
        return fail(SPTL_E_SHAPE, "%s: n_chunks=%d exceeds the %d chunks its device scratch holds", fn, n_chunks,
                    sptl::kMaxPlanChunks);
    if (!sptl::chunk_tile_rows(seq_len / n_chunks))
        return fail(SPTL_E_UNSUPPORTED, "%s: rows per chunk (%lld) must be a multiple of 128", fn,
                    (long long)(seq_len / n_chunks));
    if (seq_len == 0) return SPTL_OK;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    if (!ctx->stager || sptl::stager_failed(ctx->stager))
        return fail(SPTL_E_UNSUPPORTED, "%s: the context has no working copy engines (%s)", fn,
                    ctx->staging_info.c_str());
    if (capturing(static_cast<hipStream_t>(compute)))
        return fail(SPTL_E_UNSUPPORTED, "%s: the staged copies cannot be captured into a graph", fn);
    sptl::NoallocScratch na;
    if (!sptl::noalloc_scratch(ctx->device, &na))
        return fail(SPTL_E_HIP, "%s: the device scratch was not set up", fn);
    ctx->t_chunks = -1;
    return agmm_staged(ctx, seq_len, hidden, n_local, tp, n_chunks, rank, shard_src,
                       static_cast<uint16_t *>(x_gathered), w, y, y_dtype, static_cast<hipStream_t>(compute), 0, &na);
}

int sptl_agmm_timeline(sptl_ctx *ctx, double *out, int n_chunks) {
    if (!out) return fail(SPTL_E_NULL, "sptl_agmm_timeline: out is NULL");
    if (int rc = resolve_ctx(ctx)) return rc;
    if (ctx->t_chunks < 0 || n_chunks != ctx->t_chunks)
        return fail(SPTL_E_RANGE, "sptl_agmm_timeline: no timed call with n_chunks=%d", n_chunks);
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    if (ctx->t_mode == 1) {
        // chunk-ordered call: timestamps taken by the GEMM's workgroups (wall clock)
        const int n = n_chunks;
        std::vector<uint64_t> ts(3 * n + 1);
        if (!ctx->stager || sptl::stager_wait_call(ctx->stager, ctx->t_set, ctx->t_epoch))
            return fail(SPTL_E_HIP, "sptl_agmm_timeline: the timed call did not finish");
        SPTL_HIP(hipMemcpy(ts.data(), ctx->ts_dev, ts.size() * sizeof(uint64_t), hipMemcpyDeviceToHost));
        const double per_ms = (double)ctx->wallclock_khz;
        const uint64_t t0 = ts[3 * n];
        auto ms = [&](uint64_t t) { return ((double)(int64_t)(t - t0)) / per_ms; };
        for (int c = 0; c < n; ++c) {
            double *row = out + 4 * c;
            const bool own = c >= ctx->t_rank_first && c < ctx->t_rank_first + ctx->t_rank_count;
            row[0] = own ? -1.0 : 0.0;          // every copy is queued at the fork point
            row[1] = own ? -1.0 : ms(ts[c]);    // first tile of the chunk found it landed
            row[2] = ms(ts[n + c]);
            row[3] = ms(ts[2 * n + c]);
        }
        return SPTL_OK;
    }
    SPTL_HIP(hipEventSynchronize(ctx->join));
    for (int c = 0; c < n_chunks; ++c) {
        float t = 0.0f;
        double *row = out + 4 * c;
        if (ctx->t_has_copy[c]) {
            SPTL_HIP(hipEventSynchronize(ctx->ready[c]));
            SPTL_HIP(hipEventElapsedTime(&t, ctx->t_base, ctx->t_copy_start[c]));
            row[0] = t;
            SPTL_HIP(hipEventElapsedTime(&t, ctx->t_base, ctx->ready[c]));
            row[1] = t;
        } else {
            row[0] = row[1] = -1.0;
        }
        SPTL_HIP(hipEventSynchronize(ctx->t_gemm_end[c]));
        SPTL_HIP(hipEventElapsedTime(&t, ctx->t_base, ctx->t_gemm_start[c]));
        row[2] = t;
        SPTL_HIP(hipEventElapsedTime(&t, ctx->t_base, ctx->t_gemm_end[c]));
        row[3] = t;
    }
    return SPTL_OK;
}

int gemm_partial(sptl_ctx *ctx, int64_t seq_len, int64_t k_local, int64_t hidden, const void *a,
                 const void *w, void *partial, int out_dtype, void *stream) {
    if (!a || !w || !partial) return fail(SPTL_E_NULL, "gemm_partial: NULL pointer argument");
    if (out_dtype != SPTL_BF16 && out_dtype != SPTL_F32) return fail(SPTL_E_DTYPE, "gemm_partial: out_dtype=%d", out_dtype);
    if (int rc = check_gemm_dims(seq_len, k_local, hidden)) return rc;
    if (!aligned16(a) || !aligned16(w) || !aligned16(partial))
        return fail(SPTL_E_ALIGN, "gemm_partial: pointers must be 16-byte aligned");
    if (seq_len == 0) return SPTL_OK;
    if (int rc = resolve_ctx(ctx)) return rc;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    sptl::GemmProblem gp{};
    gp.a = static_cast<const uint16_t *>(a);
    gp.b = static_cast<const uint16_t *>(w);
    gp.c = partial;
    gp.m = seq_len;
    gp.n = hidden;
    gp.k = k_local;
    gp.lda = k_local;
    gp.ldb = hidden;
    gp.ldc = hidden;
    gp.c_f32 = out_dtype == SPTL_F32;
    SPTL_HIP(sptl::launch_gemm(gp, static_cast<hipStream_t>(stream)));
    return SPTL_OK;
}

int gemm_rs_chunked(sptl_ctx *ctx, int64_t seq_len, int64_t k_local, int64_t hidden, int tp, int n_chunks,
                    int rank, const void *a, const void *w, void *partial, void *const *dst, void *compute) {
    static const char *fn = "gemm_rs_chunked";
    if (!a || !w || !partial || !dst) return fail(SPTL_E_NULL, "%s: NULL pointer argument", fn);
    if (tp < 1 || tp > sptl::kMaxPlanChunks)
        return fail(SPTL_E_RANGE, "%s: tp=%d not in [1, %d]", fn, tp, sptl::kMaxPlanChunks);
    if (n_chunks < 1 || n_chunks > sptl::kMaxPlanChunks)
        return fail(SPTL_E_RANGE, "%s: n_chunks=%d not in [1, %d]", fn, n_chunks, sptl::kMaxPlanChunks);
    if (rank < 0 || rank >= tp) return fail(SPTL_E_RANGE, "%s: rank=%d not in [0, %d)", fn, rank, tp);
    if (n_chunks % tp) return fail(SPTL_E_DIVISIBILITY, "%s: n_chunks=%d not a multiple of tp=%d", fn, n_chunks, tp);
    if (seq_len < 0) return fail(SPTL_E_SHAPE, "%s: seq_len=%lld", fn, (long long)seq_len);
    if (seq_len % n_chunks)
        return fail(SPTL_E_DIVISIBILITY, "%s: seq_len=%lld not a multiple of n_chunks=%d", fn, (long long)seq_len,
                    n_chunks);
    const int64_t R = seq_len / tp;
    const int sub = n_chunks / tp;              // sub-slices per slice
    const int64_t Rc = seq_len / n_chunks;      // rows per sub-slice
    if (int rc = check_gemm_dims(R, k_local, hidden)) return rc;
    for (int q = 0; q < tp; ++q) {
        if (q != rank && !dst[q]) return fail(SPTL_E_NULL, "%s: dst[%d] is NULL", fn, q);
        if (dst[q] && !aligned16(dst[q])) return fail(SPTL_E_ALIGN, "%s: dst[%d] not 16-byte aligned", fn, q);
    }
    if (!aligned16(a) || !aligned16(w) || !aligned16(partial))
        return fail(SPTL_E_ALIGN, "%s: a, w and partial must be 16-byte aligned", fn);
    if (seq_len == 0) return SPTL_OK;
    if (int rc = resolve_ctx(ctx)) return rc;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    hipStream_t cs = static_cast<hipStream_t>(compute);
    auto *pb = static_cast<uint16_t *>(partial);
    const size_t slice_elems = (size_t)R * (size_t)hidden;
    const size_t slice_bytes = slice_elems * 2;
    const size_t sub_elems = (size_t)Rc * (size_t)hidden;
    const size_t sub_bytes = sub_elems * 2;
    sptl::GemmProblem gp{};
    gp.a = static_cast<const uint16_t *>(a);
    gp.b = static_cast<const uint16_t *>(w);
    gp.c = partial;
    gp.m = seq_len;
    gp.n = hidden;
    gp.k = k_local;
    gp.lda = k_local;
    gp.ldb = hidden;
    gp.ldc = hidden;
    gp.c_f32 = false;
    auto in_place = [&](int q) { return q == rank || dst[q] == pb + (size_t)q * slice_elems; };
    // sub-slice c (rows [c Rc, (c+1) Rc) of partial) is sub-slice c % sub of slice c / sub
    auto sub_dst = [&](int c) {
        return static_cast<uint16_t *>(dst[c / sub]) + (size_t)(c % sub) * sub_elems;
    };
    // send order: the peers' sub-slices in the context's chunk order (copied out while later
    // sub-slices compute), this rank's own last
    std::vector<int> order = peer_chunk_order(ctx, rank, tp, sub);
    for (int j = 0; j < sub; ++j) order.push_back(rank * sub + j);
    if (ctx->copy_mode == SPTL_COPY_SERIAL) {
        // no overlap (the baseline the overlap is measured against): the GEMM, then the copies
        const bool cap = capturing(cs);
        SPTL_HIP(sptl::launch_gemm(gp, cs));
        for (int d = 1; d < tp; ++d) {
            const int q = (rank + d) % tp;
            if (!in_place(q)) SPTL_HIP(stage_copy(ctx, dst[q], pb + (size_t)q * slice_elems, slice_bytes, cs, cap));
        }
        return SPTL_OK;
    }
    if (!staged_path(ctx, Rc, n_chunks, cs)) {
        // per-sub-slice events: one GEMM launch per sub-slice on `compute` in send order, each
        // peer sub-slice then copied on the copy stream after its event while the next compute
        const bool cap = capturing(cs);
        hipStream_t ps;
        if (int rc = copy_stream_of(ctx, &ps)) return rc;
        if (int rc = grow_events(ctx->ready, n_chunks)) return rc;
        sptl::GemmProblem sp = gp;
        sp.m = Rc;
        bool copied = false;
        for (const int c : order) {
            sp.a = gp.a + (size_t)c * (size_t)Rc * (size_t)k_local;
            sp.c = pb + (size_t)c * sub_elems;
            SPTL_HIP(sptl::launch_gemm(sp, cs));
            if (in_place(c / sub)) continue;
            SPTL_HIP(hipEventRecord(ctx->ready[c], cs));
            SPTL_HIP(hipStreamWaitEvent(ps, ctx->ready[c], 0));
            SPTL_HIP(stage_copy(ctx, sub_dst(c), pb + (size_t)c * sub_elems, sub_bytes, ps, cap));
            copied = true;
        }
        if (copied) {
            // later work on `compute` sees every destination complete
            SPTL_HIP(hipEventRecord(ctx->join, ps));
            SPTL_HIP(hipStreamWaitEvent(cs, ctx->join, 0));
        }
        return SPTL_OK;
    }
    std::vector<sptl::CopyPiece> copies;
    std::vector<int> link;  // each sub-slice's peer (0 for rank+1, ...), for the link model
    sptl::ChunkPlan &plan = gp.plan;
    for (int i = 0; i < n_chunks; ++i) {
        const int c = order[(size_t)i], q = c / sub;
        plan.order[i] = c;
        if (in_place(q)) continue;  // stays in place
        copies.push_back({sub_dst(c), pb + (size_t)c * sub_elems, sub_bytes, c});
        link.push_back((q - rank + tp) % tp - 1);
    }
    plan.chunk_rows = (int)Rc;
    plan.n_chunks = n_chunks;
    plan.own_first = 0;
    plan.own_count = 0;
    plan.own_a = gp.a;
    plan.err = ctx->err_dev;
    plan.timeout_ticks = (uint64_t)ctx->wallclock_khz * ctx->wait_timeout_us / 1000u;
    plan.copy_out = true;
    std::vector<sptl::CopyPiece> pieces = ctx->engines_per_peer > 0
                                              ? sptl::stager_plan_links(ctx->stager, copies, link, ctx->engines_per_peer)
                                              : sptl::stager_plan(ctx->stager, copies, 1, 1);
    const int64_t wgs = sptl::gemm_workgroups(gp);
    // The release of a slice (see ChunkPlan): the XCD's last tile of the slice writes its L2
    // back, which needs every XCD's share of a copied slice to be equal; else every tile does.
    static const bool each_tile = [] {
        const char *e = getenv("SPTL_RS_FLUSH");  // "tile": every tile writes back (measurement aid)
        return e && !strcmp(e, "tile");
    }();
    static const int share_skew = [] {
        const char *e = getenv("SPTL_RS_SHARE_SKEW");  // under-counted share (test aid: the report)
        return e ? (int)(strtol(e, nullptr, 10) & 1) : 0;
    }();
    std::vector<int64_t> xt((size_t)n_chunks * 8);
    sptl::chunk_xcd_tiles(gp, xt.data());
    plan.flush_each_tile = each_tile;
    for (const sptl::CopyPiece &pc : copies) {
        int64_t share = 0, groups = 0;
        for (int x = 0; x < 8; ++x) {
            const int64_t t = xt[(size_t)pc.chunk * 8 + x];
            if (!t) continue;
            if (share && t != share) plan.flush_each_tile = true;
            share = t;
            ++groups;
        }
        plan.slice_xcd_last[pc.chunk] = (uint32_t)(share - 1 - (share > 1 ? share_skew : 0));
        plan.slice_last[pc.chunk] = (uint64_t)(groups - 1);
    }
    if (plan.flush_each_tile)
        for (const sptl::CopyPiece &pc : copies) {
            int64_t tiles = 0;
            for (int x = 0; x < 8; ++x) tiles += xt[(size_t)pc.chunk * 8 + x];
            plan.slice_last[pc.chunk] = (uint64_t)(tiles - 1);
        }
    sptl::StageCall call;
    std::string why;
    if (int rc = sptl::stager_begin(ctx->stager, pieces, wgs, &call, &why))
        return fail(rc == -2 ? SPTL_E_ASYNC : SPTL_E_HIP, "%s: %s", fn, why.c_str());
    for (int c = 0; c < n_chunks; ++c) {
        plan.ready[c] = call.ready[c];  // copy-out: the sub-slice's outgoing copies
        plan.ready_n[c] = call.ready_n[c];
    }
    plan.slice_ready = call.slice_ready;
    plan.slice_count = call.slice_count;
    plan.join = nullptr;
    plan.join_n = 0;
    plan.flags = nullptr;
    plan.epoch = call.epoch;
    plan.flag_epoch = call.epoch;
    plan.finished = call.finished;
    plan.timedout = call.timedout;
    plan.wg_count = call.wg_count;
    for (int gi = 0; gi < sptl::kEndGroups; ++gi) plan.grp_last[gi] = call.grp_last[gi];
    plan.all_last = call.all_last;
    // the call's slice counters start at zero (a fill kernel rather than a memset; the set's
    // previous call has finished, stager_begin saw to that)
    // (no fork event: the copies are released slice by slice by the kernel itself)
    hipError_t he = sptl::launch_fill_u64(call.slice_count, (int64_t)n_chunks * sptl::kEndLine, 0ull, cs);
    if (he == hipSuccess) he = sptl::launch_gemm(gp, cs);
    if (he != hipSuccess) {
        sptl::stager_cancel(ctx->stager, call);
        return hip_fail(he, "gemm_rs_chunked: kernel launch");
    }
    if (sptl::stager_submit(ctx->stager, call, std::move(pieces), &why, true))
        return fail(SPTL_E_HIP, "%s: %s", fn, why.c_str());
    return SPTL_OK;
}

int agmm_backward(sptl_ctx *ctx, int64_t seq_len, int64_t hidden, int64_t n_local, int tp, int rank,
                  const void *const *shard_src, void *x_gathered, const void *w, const void *dy, void *dx, void *dw,
                  int dw_dtype, void *compute) {
    static const char *fn = "agmm_backward";
    if (!shard_src || !x_gathered || !w || !dy || !dx || !dw) return fail(SPTL_E_NULL, "%s: NULL pointer argument", fn);
    if (seq_len < 0 || hidden <= 0 || n_local <= 0)
        return fail(SPTL_E_SHAPE, "%s: bad sizes seq_len=%lld hidden=%lld n_local=%lld", fn, (long long)seq_len,
                    (long long)hidden, (long long)n_local);
    if (tp < 1 || tp > sptl::kMaxPlanChunks)
        return fail(SPTL_E_RANGE, "%s: tp=%d not in [1, %d]", fn, tp, sptl::kMaxPlanChunks);
    if (rank < 0 || rank >= tp) return fail(SPTL_E_RANGE, "%s: rank=%d not in [0, %d)", fn, rank, tp);
    if (seq_len % tp)
        return fail(SPTL_E_DIVISIBILITY, "%s: seq_len=%lld not a multiple of tp=%d", fn, (long long)seq_len, tp);
    if (dw_dtype != SPTL_BF16 && dw_dtype != SPTL_F32) return fail(SPTL_E_DTYPE, "%s: dw_dtype=%d", fn, dw_dtype);
    // dx = dy w^T: m = seq_len, k = n_local, n = hidden; dw = x^T dy: m = hidden, k = seq_len (the row
    // index of both operands, so any length), n = n_local
    if (int rc = check_gemm_dims(seq_len, n_local, hidden)) return rc;
    if (int rc = check_gemm_dims(hidden, 8, n_local)) return rc;
    for (int q = 0; q < tp; ++q) {
        if (!shard_src[q]) return fail(SPTL_E_NULL, "%s: shard_src[%d] is NULL", fn, q);
        if (!aligned16(shard_src[q])) return fail(SPTL_E_ALIGN, "%s: shard_src[%d] not 16-byte aligned", fn, q);
    }
    if (!aligned16(x_gathered) || !aligned16(w) || !aligned16(dy) || !aligned16(dx) || !aligned16(dw))
        return fail(SPTL_E_ALIGN, "%s: x_gathered, w, dy, dx and dw must be 16-byte aligned", fn);
    if (seq_len == 0) return SPTL_OK;
    if (int rc = resolve_ctx(ctx)) return rc;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    hipStream_t cs = static_cast<hipStream_t>(compute);
    auto *xg = static_cast<uint16_t *>(x_gathered);
    const size_t shard_elems = (size_t)(seq_len / tp) * (size_t)hidden;
    sptl::GemmProblem gx{}, gw{};
    gx.a = static_cast<const uint16_t *>(dy);  // dx[m, k] = sum_j dy[m, j] w[k, j]
    gx.b = static_cast<const uint16_t *>(w);
    gx.c = dx;
    gx.m = seq_len;
    gx.n = hidden;
    gx.k = n_local;
    gx.lda = n_local;
    gx.ldb = n_local;
    gx.ldc = hidden;
    gx.c_f32 = false;
    gx.layout = sptl::kLayoutBNMajor;
    gw.a = xg;  // dw[k, j] = sum_m x[m, k] dy[m, j]
    gw.b = static_cast<const uint16_t *>(dy);
    gw.c = dw;
    gw.m = hidden;
    gw.n = n_local;
    gw.k = seq_len;
    gw.lda = hidden;
    gw.ldb = n_local;
    gw.ldc = n_local;
    gw.c_f32 = dw_dtype == SPTL_F32;
    gw.layout = sptl::kLayoutAKMajor;
    // the copies, peers in arrival order (rank+1, rank+2, ...) then the own slot unless aliased
    std::vector<sptl::CopyPiece> copies;
    std::vector<int> link;  // each copy's peer (0 for rank+1, ...; -1 for the own slot), for the link model
    for (int d = 1; d <= tp; ++d) {
        const int q = (rank + d) % tp;
        if (shard_src[q] != xg + (size_t)q * shard_elems) {
            copies.push_back({xg + (size_t)q * shard_elems, shard_src[q], shard_elems * 2, q});
            link.push_back(q == rank ? -1 : d - 1);
        }
    }
    const bool cap = capturing(cs);
    if (ctx->copy_mode == SPTL_COPY_SERIAL) {
        for (const sptl::CopyPiece &c : copies) SPTL_HIP(stage_copy(ctx, c.dst, c.src, c.bytes, cs, cap));
        SPTL_HIP(sptl::launch_gemm(gx, cs));
        SPTL_HIP(sptl::launch_gemm(gw, cs));
        return SPTL_OK;
    }
    if (copies.empty()) {
        SPTL_HIP(sptl::launch_gemm(gx, cs));
        SPTL_HIP(sptl::launch_gemm(gw, cs));
        return SPTL_OK;
    }
    const bool staged = ctx->copy_mode == SPTL_COPY_STAGED && ctx->stager && !sptl::stager_failed(ctx->stager) && !cap;
    if (!staged) {
        // per-copy events on the context's copy stream; dw waits for all of them
        hipStream_t ps;
        if (int rc = copy_stream_of(ctx, &ps)) return rc;
        SPTL_HIP(hipEventRecord(ctx->fork, cs));
        SPTL_HIP(hipStreamWaitEvent(ps, ctx->fork, 0));
        for (const sptl::CopyPiece &c : copies) SPTL_HIP(stage_copy(ctx, c.dst, c.src, c.bytes, ps, cap));
        SPTL_HIP(hipEventRecord(ctx->join, ps));
        SPTL_HIP(sptl::launch_gemm(gx, cs));
        SPTL_HIP(hipStreamWaitEvent(cs, ctx->join, 0));
        SPTL_HIP(sptl::launch_gemm(gw, cs));
        return SPTL_OK;
    }
    // staged: the copy engines take the re-gather at the fork point, dx's GEMM runs meanwhile (it
    // does not read x), a one-wave kernel then waits for every piece, and dw's GEMM follows it
    std::vector<sptl::CopyPiece> pieces = ctx->engines_per_peer > 0
                                              ? sptl::stager_plan_links(ctx->stager, copies, link, ctx->engines_per_peer)
                                              : sptl::stager_plan(ctx->stager, copies, 1, 1);
    sptl::StageCall call;
    std::string why;
    if (int rc = sptl::stager_begin(ctx->stager, pieces, 1, &call, &why))
        return fail(rc == -2 ? SPTL_E_ASYNC : SPTL_E_HIP, "%s: %s", fn, why.c_str());
    sptl::ChunkPlan jp{};
    jp.n_chunks = tp;
    for (int c = 0; c < tp; ++c) {
        jp.ready[c] = call.ready[c];
        jp.ready_n[c] = call.ready_n[c];
    }
    jp.join = call.join;
    jp.join_n = call.join_n;
    jp.err = ctx->err_dev;
    jp.timeout_ticks = (uint64_t)ctx->wallclock_khz * ctx->wait_timeout_us / 1000u;
    jp.poll_sleep = poll_sleep_setting();
    jp.epoch = call.epoch;
    jp.flag_epoch = call.epoch;
    jp.finished = call.finished;
    jp.timedout = call.timedout;
    jp.wg_count = call.wg_count;
    for (int gi = 0; gi < sptl::kEndGroups; ++gi) jp.grp_last[gi] = call.grp_last[gi];
    jp.all_last = call.all_last;
    hipError_t he = hipEventRecord(call.fork, cs);
    if (he == hipSuccess) he = sptl::launch_gemm(gx, cs);
    if (he == hipSuccess) he = sptl::launch_stage_join(jp, cs);
    if (he != hipSuccess) {
        sptl::stager_cancel(ctx->stager, call);
        return hip_fail(he, "agmm_backward: kernel launch");
    }
    he = sptl::launch_gemm(gw, cs);
    if (sptl::stager_submit(ctx->stager, call, std::move(pieces), &why))
        return fail(SPTL_E_HIP, "%s: %s", fn, why.c_str());
    if (he != hipSuccess) return hip_fail(he, "agmm_backward: dw kernel launch");
    return SPTL_OK;
}

int dtp_colocated_affinity(const double *affinity, int n_heads, int n_neurons, int tp, const int *head_device,
                           const int *neuron_device, double *score) {
    static const char *fn = "dtp_colocated_affinity";
    if (!affinity || !head_device || !neuron_device || !score) return fail(SPTL_E_NULL, "%s: NULL pointer argument", fn);
    if (n_heads <= 0 || n_neurons <= 0) return fail(SPTL_E_SHAPE, "%s: n_heads=%d n_neurons=%d", fn, n_heads, n_neurons);
    if (tp < 1) return fail(SPTL_E_RANGE, "%s: tp=%d", fn, tp);
    for (int h = 0; h < n_heads; ++h)
        if (head_device[h] < 0 || head_device[h] >= tp) return fail(SPTL_E_RANGE, "%s: head_device[%d]", fn, h);
    for (int j = 0; j < n_neurons; ++j)
        if (neuron_device[j] < 0 || neuron_device[j] >= tp) return fail(SPTL_E_RANGE, "%s: neuron_device[%d]", fn, j);
    *score = sptl::colocated_affinity(affinity, n_heads, n_neurons, head_device, neuron_device);
    return SPTL_OK;
}

int dtp_affinity_layout(const double *affinity, int n_heads, int n_neurons, int tp, int max_rounds, int *head_device,
                        int *neuron_device, double *score, int *rounds) {
    static const char *fn = "dtp_affinity_layout";
    if (!affinity || !head_device || !neuron_device || !score) return fail(SPTL_E_NULL, "%s: NULL pointer argument", fn);
    if (n_heads <= 0 || n_neurons <= 0) return fail(SPTL_E_SHAPE, "%s: n_heads=%d n_neurons=%d", fn, n_heads, n_neurons);
    if (tp < 1 || tp > 64) return fail(SPTL_E_RANGE, "%s: tp=%d not in [1, 64]", fn, tp);
    if (n_heads % tp || n_neurons % tp)
        return fail(SPTL_E_DIVISIBILITY, "%s: n_heads=%d and n_neurons=%d must be multiples of tp=%d", fn, n_heads,
                    n_neurons, tp);
    if (max_rounds < 1) return fail(SPTL_E_RANGE, "%s: max_rounds=%d", fn, max_rounds);
    if (sptl::head_layout_count(n_heads, tp) > SPTL_MAX_HEAD_LAYOUTS)
        return fail(SPTL_E_UNSUPPORTED, "%s: %d heads over %d devices have more than %lld layouts to search", fn,
                    n_heads, tp, (long long)SPTL_MAX_HEAD_LAYOUTS);
    std::vector<int> per(tp, 0);
    for (int h = 0; h < n_heads; ++h) {
        if (head_device[h] < 0 || head_device[h] >= tp) return fail(SPTL_E_RANGE, "%s: head_device[%d]", fn, h);
        per[head_device[h]]++;
    }
    for (int d = 0; d < tp; ++d)
        if (per[d] != n_heads / tp)
            return fail(SPTL_E_RANGE, "%s: the starting head layout puts %d heads on device %d (not %d)", fn, per[d], d,
                        n_heads / tp);
    for (int64_t i = 0; i < (int64_t)n_heads * n_neurons; ++i)
        if (!std::isfinite(affinity[i])) return fail(SPTL_E_RANGE, "%s: affinity[%lld] is not finite", fn, (long long)i);
    const int r = sptl::affinity_layout(affinity, n_heads, n_neurons, tp, max_rounds, head_device, neuron_device, score);
    if (rounds) *rounds = r;
    return SPTL_OK;
}

int dtp_layout_permutation(const int *layout, int n, int tp, int group, int32_t *perm) {
    static const char *fn = "dtp_layout_permutation";
    if (!layout || !perm) return fail(SPTL_E_NULL, "%s: NULL pointer argument", fn);
    if (n <= 0 || group <= 0 || (int64_t)n * group > 0x7fffffff)
        return fail(SPTL_E_SHAPE, "%s: n=%d group=%d", fn, n, group);
    if (tp < 1) return fail(SPTL_E_RANGE, "%s: tp=%d", fn, tp);
    for (int i = 0; i < n; ++i)
        if (layout[i] < 0 || layout[i] >= tp) return fail(SPTL_E_RANGE, "%s: layout[%d]=%d", fn, i, layout[i]);
    int64_t o = 0;
    for (int d = 0; d < tp; ++d)
        for (int i = 0; i < n; ++i)
            if (layout[i] == d)
                for (int e = 0; e < group; ++e) perm[o++] = (int32_t)((int64_t)i * group + e);
    return SPTL_OK;
}

int permute_bf16(sptl_ctx *ctx, const void *src, void *dst, int64_t rows, int64_t cols, int dim, const int32_t *perm,
                 void *stream) {
    static const char *fn = "permute_bf16";
    if (!src || !dst || !perm) return fail(SPTL_E_NULL, "%s: NULL pointer argument", fn);
    if (rows < 0 || cols <= 0 || rows > 0x7fffffff || cols > 0x7fffffff)
        return fail(SPTL_E_SHAPE, "%s: rows=%lld cols=%lld", fn, (long long)rows, (long long)cols);
    if (cols % 8) return fail(SPTL_E_DIVISIBILITY, "%s: cols=%lld not a multiple of 8", fn, (long long)cols);
    if (dim != 0 && dim != 1) return fail(SPTL_E_RANGE, "%s: dim=%d", fn, dim);
    if (src == dst) return fail(SPTL_E_RANGE, "%s: src and dst must not be the same buffer", fn);
    if (!aligned16(src) || !aligned16(dst)) return fail(SPTL_E_ALIGN, "%s: src and dst must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(perm) & 3u) != 0) return fail(SPTL_E_ALIGN, "%s: perm not 4-byte aligned", fn);
    if (rows == 0) return SPTL_OK;
    if (int rc = resolve_ctx(ctx)) return rc;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    SPTL_HIP(sptl::launch_permute(src, dst, rows, cols, dim, perm, ctx->err_dev + 1, static_cast<hipStream_t>(stream)));
    return SPTL_OK;
}

}  // extern "C"

namespace {

int check_epilogue_common(const char *fn, int64_t seq_len, int64_t hidden, float eps) {
    if (seq_len < 0 || hidden <= 0)
        return fail(SPTL_E_SHAPE, "%s: bad sizes seq_len=%lld hidden=%lld", fn, (long long)seq_len,
                    (long long)hidden);
    if (hidden % 8) return fail(SPTL_E_DIVISIBILITY, "%s: hidden=%lld not a multiple of 8", fn, (long long)hidden);
    if (seq_len > 0x7fffffffLL) return fail(SPTL_E_SHAPE, "%s: seq_len too large", fn);
    if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(SPTL_E_RANGE, "%s: eps must be finite and >= 0", fn);
    return SPTL_OK;
}

// Validates the arguments of a reduce + residual + RMSNorm over `rows` rows and fills *ep
// (everything but the launch).  fn names the calling entry point.
int build_reduce(const char *fn, int64_t rows, int64_t hidden, int tp, const void *const *partials,
                 const void *residual, const void *gamma, float eps, void *residual_out, void *y,
                 sptl::EpilogueProblem *ep) {
    if (!residual || !gamma || !y) return fail(SPTL_E_NULL, "%s: NULL pointer argument", fn);
    if (tp < 0 || tp > SPTL_MAX_PARTIALS) return fail(SPTL_E_RANGE, "%s: tp=%d not in [0, %d]", fn, tp, SPTL_MAX_PARTIALS);
    if (tp > 0 && !partials) return fail(SPTL_E_NULL, "%s: partials is NULL", fn);
    if (int rc = check_epilogue_common(fn, rows, hidden, eps)) return rc;
    *ep = sptl::EpilogueProblem{};
    ep->in[0] = static_cast<const uint16_t *>(residual);
    for (int p = 0; p < tp; ++p) {
        if (!partials[p]) return fail(SPTL_E_NULL, "%s: partials[%d] is NULL", fn, p);
        ep->in[1 + p] = static_cast<const uint16_t *>(partials[p]);
    }
    ep->n_in = 1 + tp;
    for (int i = 0; i < ep->n_in; ++i)
        if (!aligned16(ep->in[i])) return fail(SPTL_E_ALIGN, "%s: input %d not 16-byte aligned", fn, i);
    if (!aligned16(gamma) || !aligned16(y) || !aligned16(residual_out))
        return fail(SPTL_E_ALIGN, "%s: gamma, y, residual_out must be 16-byte aligned", fn);
    ep->gamma = static_cast<const uint16_t *>(gamma);
    ep->h_out = static_cast<uint16_t *>(residual_out);
    ep->y_out = static_cast<uint16_t *>(y);
    ep->rows = rows;
    ep->hidden = hidden;
    ep->eps = eps;
    return SPTL_OK;
}

}  // namespace

extern "C" {

int reduce_residual_rmsnorm(sptl_ctx *ctx, int64_t seq_len, int64_t hidden, int tp,
                            const void *const *partials, const void *residual, const void *gamma,
                            float eps, void *residual_out, void *y, void *stream) {
    sptl::EpilogueProblem ep;
    if (int rc = build_reduce("reduce_residual_rmsnorm", seq_len, hidden, tp, partials, residual, gamma, eps,
                              residual_out, y, &ep))
        return rc;
    if (seq_len == 0) return SPTL_OK;
    if (int rc = resolve_ctx(ctx)) return rc;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    SPTL_HIP(sptl::launch_epilogue(ep, static_cast<hipStream_t>(stream)));
    return SPTL_OK;
}

int reduce_norm_agmm_chunked(sptl_ctx *ctx, int n_partials, const void *const *partials, const void *residual,
                             const void *gamma, float eps, void *residual_out, int64_t seq_len, int64_t hidden,
                             int64_t n_local, int tp, int n_chunks, int rank, const void *const *shard_src,
                             void *x_gathered, const void *w, void *y, int y_dtype, void *compute) {
    static const char *fn = "reduce_norm_agmm_chunked";
    if (!shard_src || !x_gathered) return fail(SPTL_E_NULL, "%s: NULL pointer argument", fn);
    if (tp < 1 || tp > SPTL_MAX_TP) return fail(SPTL_E_RANGE, "%s: tp=%d not in [1, %d]", fn, tp, SPTL_MAX_TP);
    if (rank < 0 || rank >= tp) return fail(SPTL_E_RANGE, "%s: rank=%d not in [0, %d)", fn, rank, tp);
    if (seq_len < 0 || hidden <= 0)
        return fail(SPTL_E_SHAPE, "%s: bad sizes seq_len=%lld hidden=%lld", fn, (long long)seq_len, (long long)hidden);
    // the own rows' normalised output goes to this rank's slot of x_gathered, which the GEMM then
    // reads in place (shard_src[rank] is not used)
    const int64_t own_rows = seq_len / tp;
    auto *own_slot = static_cast<uint16_t *>(x_gathered) + (size_t)rank * (size_t)own_rows * (size_t)hidden;
    std::vector<const void *> src(shard_src, shard_src + tp);
    src[(size_t)rank] = own_slot;
    if (int rc = check_agmm_args(fn, seq_len, hidden, n_local, tp, n_chunks, rank, src.data(), x_gathered, w, y,
                                 y_dtype))
        return rc;
    sptl::EpilogueProblem ep;
    if (int rc = build_reduce(fn, own_rows, hidden, n_partials, partials, residual, gamma, eps, residual_out,
                              own_slot, &ep))
        return rc;
    if (seq_len == 0) return SPTL_OK;
    if (int rc = resolve_ctx(ctx)) return rc;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    hipStream_t cs = static_cast<hipStream_t>(compute);
    if (staged_path(ctx, seq_len / n_chunks, n_chunks, cs)) {
        ctx->t_chunks = -1;
        return agmm_staged(ctx, seq_len, hidden, n_local, tp, n_chunks, rank, src.data(),
                           static_cast<uint16_t *>(x_gathered), w, y, y_dtype, cs, 0, nullptr, &ep);
    }
    // not staged (see sptl_ctx_set_copy_mode): the unfused pair (the copies start after the epilogue)
    SPTL_HIP(sptl::launch_epilogue(ep, cs));
    return agmm_chunked(ctx, seq_len, hidden, n_local, tp, n_chunks, rank, src.data(), x_gathered, w, y, y_dtype,
                        compute, nullptr, 0);
}

int dtp_accumulate(sptl_ctx *ctx, int64_t seq_len, int64_t hidden, int tp, int delta, int module_idx,
                   void *residual, const void *own_partial, const void *const *delayed_peers,
                   const void *gamma, float eps, void *y, void *stream) {
    if (!residual) return fail(SPTL_E_NULL, "dtp_accumulate: residual is NULL");
    if (tp < 1 || tp > SPTL_MAX_PARTIALS)
        return fail(SPTL_E_RANGE, "dtp_accumulate: tp=%d not in [1, %d]", tp, SPTL_MAX_PARTIALS);
    if (delta < 0) return fail(SPTL_E_RANGE, "dtp_accumulate: delta=%d < 0", delta);
    if (module_idx < 0) return fail(SPTL_E_RANGE, "dtp_accumulate: module_idx=%d < 0", module_idx);
    const bool flush = own_partial == nullptr;
    const bool peers_due = module_idx >= delta && tp > 1;
    if (module_idx < delta && delayed_peers)
        return fail(SPTL_E_RANGE, "dtp_accumulate: module %d < delta %d has no delayed peers; pass NULL",
                    module_idx, delta);
    if (peers_due && !delayed_peers)
        return fail(SPTL_E_NULL, "dtp_accumulate: module %d needs the peers' partials of module %d",
                    module_idx, module_idx - delta);
    if (flush && !peers_due)
        return fail(SPTL_E_RANGE, "dtp_accumulate: flush call (own_partial NULL) with nothing to add");
    if (flush && y) return fail(SPTL_E_RANGE, "dtp_accumulate: flush calls take no norm; y must be NULL");
    if (!flush && !y) return fail(SPTL_E_NULL, "dtp_accumulate: y is NULL");
    if (y && !gamma) return fail(SPTL_E_NULL, "dtp_accumulate: gamma is NULL");
    if (int rc = check_epilogue_common("dtp_accumulate", seq_len, hidden, eps)) return rc;
    sptl::EpilogueProblem ep{};
    ep.in[0] = static_cast<const uint16_t *>(residual);
    ep.n_in = 1;
    if (!flush) ep.in[ep.n_in++] = static_cast<const uint16_t *>(own_partial);
    if (peers_due)
        for (int q = 0; q < tp - 1; ++q) {
            if (!delayed_peers[q]) return fail(SPTL_E_NULL, "dtp_accumulate: delayed_peers[%d] is NULL", q);
            ep.in[ep.n_in++] = static_cast<const uint16_t *>(delayed_peers[q]);
        }
    for (int i = 0; i < ep.n_in; ++i)
        if (!aligned16(ep.in[i])) return fail(SPTL_E_ALIGN, "dtp_accumulate: input %d not 16-byte aligned", i);
    if (!aligned16(gamma) || !aligned16(y)) return fail(SPTL_E_ALIGN, "dtp_accumulate: gamma and y must be 16-byte aligned");
    if (seq_len == 0) return SPTL_OK;
    if (int rc = resolve_ctx(ctx)) return rc;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    ep.gamma = static_cast<const uint16_t *>(gamma);
    ep.h_out = static_cast<uint16_t *>(residual);
    ep.y_out = static_cast<uint16_t *>(y);
    ep.rows = seq_len;
    ep.hidden = hidden;
    ep.eps = eps;
    SPTL_HIP(sptl::launch_epilogue(ep, static_cast<hipStream_t>(stream)));
    return SPTL_OK;
}

}  // extern "C"
