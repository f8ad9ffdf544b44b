// SDMA chunk stager: drives the GPU's copy engines directly through HSA for the chunk staging
// of agmm_chunked.  Internal to libsptl.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "sptl_internal.h"

namespace sptl {

// One staging copy: `bytes` from src to dst, counted against chunk `chunk` (kJoinChunk for
// copies that only the end of the call waits for).
struct CopyPiece {
    void *dst;
    const void *src;
    size_t bytes;
    int chunk;
};
constexpr int kJoinChunk = kMaxPlanChunks;
constexpr int kStageSets = 4;  // calls that can be in flight on one stager

// Device-side view of one call's completion words: ready[c] reaches <= 0 once every piece of
// chunk c has landed; join likewise for the kJoinChunk pieces.
struct StageCall {
    int set = -1;               // in [0, kStageSets)
    const int64_t *ready[kMaxPlanChunks] = {};
    const int64_t *join = nullptr;
    hipEvent_t fork = nullptr;  // record on the compute stream before the consuming GEMM
    hipEvent_t done = nullptr;  // record on the compute stream after it
};

class SdmaStager;

// nullptr (with *err set) when the copy engines cannot be driven on `device`.
SdmaStager *stager_create(int device, std::string *err);
void stager_destroy(SdmaStager *s);
int stager_engine_count(const SdmaStager *s);

// Splits every chunk copy into pieces striped over the engines (`chunk_bytes` per chunk in
// submission order) and returns them with their chunk ids; the result is what
// stager_submit expects.
std::vector<CopyPiece> stager_plan(const SdmaStager *s, const std::vector<CopyPiece> &copies);

// Reserves a completion-signal set for one call and arms it with the number of pieces per
// chunk.  Blocks while the set's previous call is still running.
int stager_begin(SdmaStager *s, const std::vector<CopyPiece> &pieces, StageCall *out, std::string *err);

// Queues the pieces; a worker thread submits them to the engines as soon as `call.fork`
// has completed (so the copies never overwrite data that earlier stream work still reads).
int stager_submit(SdmaStager *s, const StageCall &call, std::vector<CopyPiece> pieces, std::string *err);

// True once a submission failed; the stager is then not used again.
bool stager_failed(const SdmaStager *s);

// Blocks until every call begun on the stager has completed on the GPU.
int stager_wait_idle(SdmaStager *s);

}  // namespace sptl
