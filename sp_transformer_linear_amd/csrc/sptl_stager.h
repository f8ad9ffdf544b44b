// SDMA chunk stager: drives the GPU's copy engines directly through HSA for the chunk staging
// of agmm_chunked.  Internal to libsptl.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "sptl_internal.h"
#include "sptl_plan.h"

namespace sptl {

// One staging copy: `bytes` from src to dst, piece `piece` of chunk `chunk` (kJoinChunk for
// copies that only the end of the call waits for).
struct CopyPiece {
    void *dst;
    const void *src;
    size_t bytes;
    int chunk;
    int piece;
    int engine = 0;  // index into the stager's engines (set by stager_plan)
};
constexpr int kJoinChunk = kMaxPlanChunks;
constexpr int kStageSets = 4;   // calls that can be in flight on one stager
static_assert(kMaxPieces <= 64, "the GEMM watches a chunk's pieces with one lane each");

// One call's view of its completion-signal set.  ready[c] is a device array of the value
// words of chunk c's ready_n[c] piece signals (null: chunk c has no piece); each word goes from
// 1 to <= 0 when its piece has landed.  join / join_n likewise for the kJoinChunk pieces.  One
// signal per copy, not one signal per chunk counted down by its pieces: under a tool that
// intercepts the copies (rocprofv3 --memory-copy-trace), a signal shared by several copies
// read as complete before all of them had landed, while a signal of one copy stays exact.  `fork`, when
// the caller records it on the compute stream right before the consuming kernel, completes
// once every earlier operation on the stream has, so the copies may overwrite the gathered
// buffer; `started` says the same from the kernel's start (ForkWait).  The kernel
// reports its own end through a word of pinned host memory: the end counters at wg_count
// count finished workgroups in groups (see ChunkPlan), and the workgroup that completes the
// count waits for the join and then stores `epoch` to *finished.  (No marker follows the
// kernel on the stream: each marker costs several microseconds of GPU time.)
struct StageCall {
    int set = -1;               // in [0, kStageSets)
    const int64_t *const *ready[kMaxPlanChunks] = {};
    int ready_n[kMaxPlanChunks] = {};
    const int64_t *const *join = nullptr;
    int join_n = 0;
    hipEvent_t fork = nullptr;
    uint64_t epoch = 0;
    uint64_t *finished = nullptr;
    uint64_t *timedout = nullptr;   // pinned host word: the kernel stores epoch here if a wait timed out
    uint64_t *started = nullptr;    // pinned host word: the consuming kernel's tile 0 stores epoch here first
    uint64_t *wg_count = nullptr;
    uint64_t grp_last[kEndGroups] = {};
    uint64_t all_last = 0;
    uint64_t grp_first[kEndGroups] = {};  // the set's totals before this call (for a cancel)
    uint64_t all_first = 0;
    // copy-out calls: the set's slice-ready words (pinned host, 16 apart) and slice counter lines
    // (device, kEndLine words apart, zeroed by the call before its launch); see ChunkPlan
    uint64_t *slice_ready = nullptr;
    uint64_t *slice_count = nullptr;
};

class SdmaStager;

// nullptr (with *err set) when the copy engines cannot be driven on `device`.
SdmaStager *stager_create(int device, std::string *err);
void stager_destroy(SdmaStager *s);
int stager_engine_count(const SdmaStager *s);

// Splits the chunk copies into pieces with an engine each (plan_pieces, sptl_plan.h) and returns
// them in submission order with their chunk and piece ids, which is what stager_begin and
// stager_submit expect; each engine takes its pieces in submission order.
// group > 0 overrides the grouping of the later copies (1: each striped over all engines).
std::vector<CopyPiece> stager_plan(const SdmaStager *s, const std::vector<CopyPiece> &copies, int lead = 1,
                                   int group = 0);

// The link model (plan_pieces_links, sptl_plan.h): link[i] is copy i's peer (0, 1, ... after this
// rank; -1 for a copy that crosses no link), and each peer's copies run only on `per` engines of
// their own.  Returned in submission order with chunk and piece ids, like stager_plan.
std::vector<CopyPiece> stager_plan_links(const SdmaStager *s, const std::vector<CopyPiece> &copies,
                                         const std::vector<int> &link, int per);

// Reserves a completion-signal set for one call whose consuming kernel has `workgroups`
// workgroups, and arms it with the number of pieces per chunk.  Blocks (bounded) while the
// set's previous call is still running and, if a wait of that call timed out, until its copies
// have completed.  Returns 0, -1 (the previous call did not finish; bad pieces) or -2 (the
// copies of a timed-out call did not complete within the bound).  fresh_counts: null to count
// the kernel's workgroups in the set's own cumulative counters, or kEndCounters lines of
// counters (kEndLine words apart) that the caller zeroes on the stream before the launch.
int stager_begin(SdmaStager *s, const std::vector<CopyPiece> &pieces, int64_t workgroups, StageCall *out,
                 std::string *err, uint64_t *fresh_counts = nullptr);

// Whether a call whose chunk wait timed out has been seen (on reuse of its set, on an idle wait or
// now, for calls that have ended) since the last time this returned true.
bool stager_take_timeouts(SdmaStager *s);

// What the worker waits for before a call's first piece: the fork event recorded on the compute
// stream (Event), or the consuming kernel's start (Started: its tile 0 stores the call's epoch
// to call.started before anything else; the kernel starts only once every earlier operation on
// the stream has completed, as the event would).
enum class ForkWait { Event, Started };

// Queues the pieces; a worker thread submits them to the engines once the fork (`fork`) has been
// seen (bounded: after 30 s the stager fails and releases the call's waiters).  gated: a copy-out
// call, whose pieces of chunk c are submitted only once the kernel has stored the call's epoch to
// call.slice_ready[16 c] (bounded wait: 10 s); it waits for no fork, because a slice is ready
// only once the kernel runs.
int stager_submit(SdmaStager *s, const StageCall &call, std::vector<CopyPiece> pieces, std::string *err,
                  bool gated = false, ForkWait fork = ForkWait::Event);

// Gives back a set reserved by stager_begin whose kernel was never launched.
void stager_cancel(SdmaStager *s, const StageCall &call);

// True once a submission failed; the stager is then not used again.
bool stager_failed(const SdmaStager *s);

// Blocks (bounded) until the kernel of the call (set, epoch) has finished.
int stager_wait_call(SdmaStager *s, int set, uint64_t epoch);

// Blocks (bounded) until every call begun on the stager has completed on the GPU and the copies
// of any call whose waits timed out have completed: 0, -1 (a kernel did not finish) or -2 (copies
// of a timed-out call did not complete).
int stager_wait_idle(SdmaStager *s);

}  // namespace sptl
