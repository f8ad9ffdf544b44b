// SDMA chunk stager for agmm_chunked (see sptl_stager.h).
//
// Why: the sequence all-gather must not take compute units from the GEMM (Megatron-LM pull
// request #5513, "Observations" and "Recommendations": only the copy-engine gather helped).
// On MI355X one SDMA engine moves ~57 GB/s device to device and a HIP copy stream uses one
// engine at a time, so a chunk is striped over all available engines (14 on MI355X), driven
// through HSA, each piece completing a signal of its own.  The signals are GPU-only HSA
// signals, whose values live in device memory where the chunk-ordered GEMM polls them.
//
// Ordering: copies must not overwrite the gathered buffer while earlier work on the compute
// stream still reads it, nor read sources that work still writes.  A worker thread submits the
// pieces, with no HSA dependencies, once it has seen the call's fork: either a HIP event
// recorded on the stream right before the consuming kernel, or that kernel's start, which its
// tile 0 reports by storing the call's epoch to a pinned host word before anything else (the
// kernel starts only once every earlier operation on the stream has completed).  The event
// completes earlier (the command processor signals it while the kernel is being dispatched; the
// kernel's store queues behind its own loads, about 20 us later), but the marker it adds costs
// several microseconds of GPU time before the launch.  So the start is used where no tile of the
// first round waits for an engine copy (M = 8192 with the lead copy: agmm 33-34 against 37-40 us
// over the pre-staged GEMM), the event where one does, ahead of an epilogue launched between the
// fork and the GEMM, and under the backward's GEMMs.  A copy-out call's pieces wait for the
// kernel's slice words, which imply its start.  (A dependency on a signal written by a kernel is
// resolved by the runtime's host thread with millisecond latency, because a kernel store raises
// no interrupt: so the worker polls the word itself.)
//
// Reuse: completion-signal sets form a ring; a set is re-armed only after the kernel that
// waited on it has reported its end through a pinned host word.  By then every piece of the
// set has landed, unless a wait of that kernel timed out: the kernel then records the call's
// epoch in a second pinned word, and the set is drained first (the worker has handled the
// call's job and every armed signal has reached zero), because a late copy would otherwise
// complete a re-armed signal of the next call.  No marker follows the kernel on the stream.
#include "sptl_stager.h"

#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <chrono>
#include <condition_variable>
#include <deque>
#include <mutex>
#include <thread>

namespace sptl {

namespace {
constexpr int kSets = kStageSets;

struct FindAgent {
    uint32_t bdf;
    uint32_t domain;
    hsa_agent_t agent;
    bool found;
};

hsa_status_t find_agent(hsa_agent_t a, void *data) {
    auto *f = static_cast<FindAgent *>(data);
    hsa_device_type_t t;
    if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &t) != HSA_STATUS_SUCCESS || t != HSA_DEVICE_TYPE_GPU)
        return HSA_STATUS_SUCCESS;
    uint32_t bdf = 0, dom = 0;
    hsa_agent_get_info(a, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_BDFID, &bdf);
    hsa_agent_get_info(a, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_DOMAIN, &dom);
    if ((bdf & ~7u) == (f->bdf & ~7u) && dom == f->domain) {
        f->agent = a;
        f->found = true;
        return HSA_STATUS_INFO_BREAK;
    }
    return HSA_STATUS_SUCCESS;
}
}  // namespace

// Pinned host words: set s finished at word 16 * s (one 128-byte line each).  Device
// counters: set s's kEndCounters end counters from word kSetCountWords * s, kEndLine apart.
constexpr int kHostWords = 16 * kStageSets;
constexpr int kSetCountWords = kCallCountLines * kEndLine;
constexpr int kCountWords = kSetCountWords * kStageSets;
constexpr double kReuseWaitSeconds = 30.0;  // longest a call waits for a set to come free

constexpr int kSetSignals = (kMaxPlanChunks + 1) * kMaxPieces;
// slice-ready words (16 apart) and slice counters (kEndLine apart) of copy-out calls, per set
constexpr int kSliceSetWords = kMaxPlanChunks * (kEndLine > 16 ? kEndLine : 16);
constexpr int kSliceWords = kSliceSetWords * kStageSets;

struct SignalSet {
    hsa_signal_t sig[kMaxPlanChunks + 1][kMaxPieces] = {};
    int64_t **words = nullptr;  // device: value word of sig[c][p] at words[c * kMaxPieces + p]
    hipEvent_t fork = nullptr;
    uint64_t epoch = 0;       // of the last call begun on the set (0: never used)
    int armed[kMaxPlanChunks + 1] = {};   // pieces per chunk armed by that call
    std::atomic<uint64_t> handled{0};     // epoch of the last job the worker has handled
    uint64_t grp_total[kEndGroups] = {};  // workgroups counted per group, all calls on the set
    uint64_t all_total = 0;               // groups counted, all calls on the set
};

struct Job {
    int set;
    uint64_t epoch;
    hipEvent_t fork;
    std::vector<CopyPiece> pieces;
    const volatile uint64_t *gates = nullptr;  // copy-out: chunk c's pieces wait for gates[16 c] == epoch
    ForkWait wait = ForkWait::Event;
    const volatile uint64_t *started = nullptr;  // ForkWait::Started: the kernel stores epoch here
    bool fork_wait = true;                       // false for a gated call (its slice words imply the kernel ran)
};
constexpr double kStartWaitSeconds = 30.0;
constexpr double kGateWaitSeconds = 10.0;

// Spins (with pauses, yielding now and then) until *word == value; false after `seconds`.
bool spin_until(const volatile uint64_t *word, uint64_t value, double seconds) {
    const auto t0 = std::chrono::steady_clock::now();
    for (unsigned i = 1;; ++i) {
        if (__atomic_load_n(word, __ATOMIC_ACQUIRE) == value) return true;
        __builtin_ia32_pause();
        if ((i & 1023) == 0) {
            if (std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count() > seconds) return false;
            std::this_thread::yield();
        }
    }
}

class SdmaStager {
  public:
    int device = 0;
    hsa_agent_t agent{};
    std::vector<uint32_t> engines;  // hsa_amd_sdma_engine_id_t bits
    SignalSet sets[kSets];
    int next_set = 0;
    std::mutex mu;                  // guards next_set and the queue
    std::condition_variable cv;
    std::deque<Job> queue;
    bool stop = false;
    std::atomic<int> queued{0};        // jobs in the queue (polled without the lock)
    bool wake = false;                 // a call has begun: leave the blocking wait (guarded by mu)
    std::atomic<bool> stop_flag{false};
    static constexpr auto kIdleSpin = std::chrono::milliseconds(2);
    std::thread worker;
    std::atomic<bool> failed{false};
    void *scratch = nullptr;        // 8 KB for the engine checks
    uint64_t *host_words = nullptr; // pinned, kHostWords
    uint64_t *counts = nullptr;     // device, kCountWords
    uint64_t *slice_words = nullptr;   // pinned: per set, kMaxPlanChunks slice-ready words 16 apart
    uint64_t *slice_counts = nullptr;  // device: per set, kMaxPlanChunks slice counters kEndLine apart

    volatile uint64_t *finished(int set) const { return host_words + 16 * set; }
    volatile uint64_t *started(int set) const { return host_words + 16 * set + 4; }
    volatile uint64_t *timedout(int set) const { return host_words + 16 * set + 8; }

    // Whether the last call begun on `set` may have left copies in flight: a wait of its
    // kernel timed out, or a submission failed (the failure path released its waiters).
    // Only meaningful once that kernel has reported its end.
    bool tainted(int set) {
        const uint64_t e = sets[set].epoch;
        const bool timed_out = e && __atomic_load_n(timedout(set), __ATOMIC_ACQUIRE) == e;
        if (timed_out && timeout_noted[set] != e) {
            timeout_noted[set] = e;
            timeout_pending = true;
        }
        return e && (timed_out || failed.load());
    }
    uint64_t timeout_noted[kSets] = {};  // per set: epoch of the last timed-out call noted
    bool timeout_pending = false;        // a timed-out call was noted since the last report

    // Bounded wait until every copy of the last call on `set` is done: the worker has handled
    // its job (submitted every piece or given up) and every armed piece signal reads <= 0.
    bool drain(int set, double seconds) {
        SignalSet &ss = sets[set];
        const auto t0 = std::chrono::steady_clock::now();
        auto expired = [&] {
            return std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count() > seconds;
        };
        while (ss.handled.load(std::memory_order_acquire) < ss.epoch) {
            if (expired()) return false;
            std::this_thread::yield();
        }
        for (int c = 0; c <= kMaxPlanChunks; ++c)
            for (int q = 0; q < ss.armed[c]; ++q)
                for (unsigned i = 1; hsa_signal_load_scacquire(ss.sig[c][q]) > 0; ++i) {
                    __builtin_ia32_pause();
                    if ((i & 1023) == 0 && expired()) return false;
                }
        return true;
    }

    // The copies should start the moment the fork completes: a blocking event wait wakes
    // up tens of microseconds late, which delays every chunk by as much.  So the worker
    // polls while a call is pending (the host usually runs ahead of the GPU by a few
    // calls, i.e. up to a few milliseconds), and only blocks after kForkSpin.
    static constexpr auto kForkSpin = std::chrono::milliseconds(50);
    static bool wait_fork(hipEvent_t fork) {
        const auto t0 = std::chrono::steady_clock::now();
        for (unsigned i = 1;; ++i) {
            const hipError_t q = hipEventQuery(fork);
            if (q == hipSuccess) return true;
            if (q != hipErrorNotReady) return false;
            if ((i & 255) == 0 && std::chrono::steady_clock::now() - t0 > kForkSpin)
                return hipEventSynchronize(fork) == hipSuccess;
        }
    }

    void run() {
        (void)hipSetDevice(device);
        for (;;) {
            Job job;
            // A call usually follows the last one within a millisecond; waking a blocked
            // thread takes tens of microseconds, which would delay every chunk of that call.
            // So poll for a while before blocking.
            const auto idle0 = std::chrono::steady_clock::now();
            for (unsigned i = 1; queued.load(std::memory_order_acquire) == 0 && !stop_flag.load(); ++i) {
                __builtin_ia32_pause();
                if ((i & 1023) == 0 && std::chrono::steady_clock::now() - idle0 > kIdleSpin) break;
            }
            {
                std::unique_lock<std::mutex> lk(mu);
                cv.wait(lk, [&] { return stop || !queue.empty() || wake; });
                wake = false;
                if (queue.empty()) {
                    if (stop) return;  // stop requested and nothing left
                    continue;          // woken ahead of a call: poll for its job
                }
                job = std::move(queue.front());
                queue.pop_front();
                queued.fetch_sub(1, std::memory_order_relaxed);
            }
            submit(job);
        }
    }

    // A kernel start (ForkWait::Started) is seen by polling its word, as the fork event is: spin
    // for kForkSpin, then poll with short sleeps, up to kStartWaitSeconds.
    static bool wait_started(const volatile uint64_t *word, uint64_t epoch) {
        const auto t0 = std::chrono::steady_clock::now();
        for (unsigned i = 1;; ++i) {
            if (__atomic_load_n(word, __ATOMIC_ACQUIRE) == epoch) return true;
            __builtin_ia32_pause();
            if ((i & 255) == 0) {
                const auto dt = std::chrono::steady_clock::now() - t0;
                if (dt > kForkSpin) {
                    if (std::chrono::duration<double>(dt).count() > kStartWaitSeconds) return false;
                    std::this_thread::sleep_for(std::chrono::microseconds(20));
                }
            }
        }
    }

    // Submits a job's pieces once its fork has been seen, then records the job handled.
    void submit(const Job &job) {
        SignalSet &ss = sets[job.set];
        static const bool trace = getenv("SPTL_STAGER_TRACE") != nullptr;
        const auto tq = std::chrono::steady_clock::now();
        bool ok = !job.fork_wait               ? true
                  : job.wait == ForkWait::Event ? wait_fork(job.fork)
                                                : wait_started(job.started, job.epoch);
        const auto tf = std::chrono::steady_clock::now();
        int last_chunk = -2;
        for (const CopyPiece &pc : job.pieces) {
            if (ok && job.gates && pc.chunk != last_chunk) {
                // copy-out: the slice's rows are written and visible once the kernel says so
                const volatile uint64_t *g = job.gates + 16 * (size_t)pc.chunk;
                ok = spin_until(g, job.epoch, kGateWaitSeconds);
            }
            if (trace && pc.chunk != last_chunk)
                fprintf(stderr, "[stager] chunk %d submit at +%.1f us after fork (fork wait %.1f us)\n", pc.chunk,
                        std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - tf).count(),
                        std::chrono::duration<double, std::micro>(tf - tq).count());
            last_chunk = pc.chunk;
            const uint32_t eng = engines[(size_t)pc.engine % engines.size()];
            if (ok)
                ok = hsa_amd_memory_async_copy_on_engine(pc.dst, agent, pc.src, agent, pc.bytes, 0, nullptr,
                                                         ss.sig[pc.chunk][pc.piece],
                                                         (hsa_amd_sdma_engine_id_t)eng, true) == HSA_STATUS_SUCCESS;
            if (!ok) {
                // release every waiter of this call; the call's results are invalid and the
                // failure is reported through stager_failed
                failed = true;
                for (int c = 0; c <= kMaxPlanChunks; ++c)
                    for (int q = 0; q < kMaxPieces; ++q) hsa_signal_store_screlease(ss.sig[c][q], 0);
                break;
            }
        }
        ss.handled.store(job.epoch, std::memory_order_release);
    }
};

SdmaStager *stager_create(int device, std::string *err) {
    if (hsa_init() != HSA_STATUS_SUCCESS) {
        *err = "hsa_init failed";
        return nullptr;
    }
    int bus = 0, dev = 0, dom = 0;
    if (hipDeviceGetAttribute(&bus, hipDeviceAttributePciBusId, device) != hipSuccess ||
        hipDeviceGetAttribute(&dev, hipDeviceAttributePciDeviceId, device) != hipSuccess ||
        hipDeviceGetAttribute(&dom, hipDeviceAttributePciDomainID, device) != hipSuccess) {
        *err = "cannot read the device's PCI location";
        hsa_shut_down();
        return nullptr;
    }
    FindAgent f{(uint32_t)((bus << 8) | (dev << 3)), (uint32_t)dom, {}, false};
    hsa_iterate_agents(find_agent, &f);
    if (!f.found) {
        *err = "no HSA agent matches the HIP device";
        hsa_shut_down();
        return nullptr;
    }
    // Candidate engines: what the runtime reports free for device-to-device copies; some
    // runtime versions report none for a same-device copy, then the agent's xGMI-class
    // engines (else its plain SDMA engines) are the candidates.  Every candidate is checked
    // with a small copy below, and only engines that complete it are used.
    uint32_t mask = 0;
    if (hsa_amd_memory_copy_engine_status(f.agent, f.agent, &mask) != HSA_STATUS_SUCCESS || mask == 0) {
        uint32_t n_sdma = 0, n_xgmi = 0;
        hsa_agent_get_info(f.agent, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_NUM_SDMA_ENG, &n_sdma);
        hsa_agent_get_info(f.agent, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_NUM_SDMA_XGMI_ENG, &n_xgmi);
        const uint32_t first = n_xgmi ? n_sdma : 0, count = n_xgmi ? n_xgmi : n_sdma;
        mask = 0;
        for (uint32_t b = first; b < first + count && b < 16; ++b) mask |= 1u << b;
    }
    if (mask == 0) {
        *err = "the agent reports no SDMA engine";
        hsa_shut_down();
        return nullptr;
    }
    auto *s = new SdmaStager;
    s->device = device;
    s->agent = f.agent;
    if (hipMalloc(&s->scratch, 8192) != hipSuccess || hipMemset(s->scratch, 0, 8192) != hipSuccess ||
        hipMalloc(&s->counts, kCountWords * sizeof(uint64_t)) != hipSuccess ||
        hipMemset(s->counts, 0, kCountWords * sizeof(uint64_t)) != hipSuccess ||
        hipHostMalloc(&s->host_words, kHostWords * sizeof(uint64_t), hipHostMallocMapped | hipHostMallocCoherent) !=
            hipSuccess ||
        hipHostMalloc(&s->slice_words, kSliceWords * sizeof(uint64_t), hipHostMallocMapped | hipHostMallocCoherent) !=
            hipSuccess ||
        hipMalloc(&s->slice_counts, kSliceWords * sizeof(uint64_t)) != hipSuccess ||
        hipMemset(s->slice_counts, 0, kSliceWords * sizeof(uint64_t)) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        *err = "cannot allocate the engine-check buffer, counters or pinned progress words";
        (void)hipGetLastError();
        stager_destroy(s);
        return nullptr;
    }
    {
        hsa_signal_t probe;
        if (hsa_signal_create(1, 0, nullptr, &probe) != HSA_STATUS_SUCCESS) {
            *err = "hsa_signal_create failed";
            stager_destroy(s);
            return nullptr;
        }
        for (int b = 0; b < 16; ++b) {
            if (!(mask & (1u << b))) continue;
            hsa_signal_store_screlease(probe, 1);
            char *sc = static_cast<char *>(s->scratch);
            if (hsa_amd_memory_async_copy_on_engine(sc + 4096, f.agent, sc, f.agent, 256, 0, nullptr, probe,
                                                    (hsa_amd_sdma_engine_id_t)(1u << b), true) != HSA_STATUS_SUCCESS)
                continue;
            // bounded wait (200 ms); an engine that does not finish is left out
            bool done = false;
            for (int i = 0; i < 200 && !done; ++i)
                done = hsa_signal_wait_scacquire(probe, HSA_SIGNAL_CONDITION_LT, 1, 1000000, HSA_WAIT_STATE_ACTIVE) < 1;
            if (done) s->engines.push_back(1u << b);
            else break;  // a copy may still be pending on `probe`: stop using it
        }
        if (hsa_signal_load_scacquire(probe) < 1) hsa_signal_destroy(probe);  // else leak it safely
    }
    // tuning knob: SPTL_SDMA_ENGINES=n keeps only the first n working engines
    if (const char *e = getenv("SPTL_SDMA_ENGINES")) {
        const long n = strtol(e, nullptr, 10);
        if (n > 0 && (size_t)n < s->engines.size()) s->engines.resize((size_t)n);
    }
    if (s->engines.empty()) {
        *err = "no SDMA engine completed a device-to-device check copy";
        stager_destroy(s);
        return nullptr;
    }
    bool ok = true;
    std::string why;
    for (int i = 0; i < kHostWords; ++i) s->host_words[i] = 0;
    for (int i = 0; i < kSliceWords; ++i) s->slice_words[i] = 0;
    {
        // the kernels write these words through the device address of the pinned block
        void *dp = nullptr, *dq = nullptr;
        if (hipHostGetDevicePointer(&dp, s->host_words, 0) != hipSuccess || dp != (void *)s->host_words ||
            hipHostGetDevicePointer(&dq, s->slice_words, 0) != hipSuccess || dq != (void *)s->slice_words) {
            *err = "pinned progress words have no identical device address";
            (void)hipGetLastError();
            stager_destroy(s);
            return nullptr;
        }
    }
    for (SignalSet &ss : s->sets) {
        int64_t *host_words[kSetSignals];
        for (int i = 0; i < kSetSignals && ok; ++i) {
            hsa_signal_t &sg = ss.sig[i / kMaxPieces][i % kMaxPieces];
            hsa_status_t st = hsa_amd_signal_create(0, 0, nullptr, HSA_AMD_SIGNAL_AMD_GPU_ONLY, &sg);
            if (st != HSA_STATUS_SUCCESS) {
                why = "hsa_amd_signal_create(GPU_ONLY) status " + std::to_string((int)st);
                ok = false;
                break;
            }
            volatile hsa_signal_value_t *vp = nullptr;
            st = hsa_amd_signal_value_pointer(sg, &vp);
            if (st != HSA_STATUS_SUCCESS || !vp) {
                why = "hsa_amd_signal_value_pointer status " + std::to_string((int)st);
                ok = false;
                break;
            }
            // the GEMM polls this word: it must be device memory the kernels can read
            hipPointerAttribute_t pa;
            const hipError_t he = hipPointerGetAttributes(&pa, (void *)vp);
            if (he != hipSuccess || pa.type != hipMemoryTypeDevice) {
                why = std::string("signal value is not known device memory (") + hipGetErrorString(he) +
                      ", type " + std::to_string(he == hipSuccess ? (int)pa.type : -1) + ")";
                ok = false;
                break;
            }
            host_words[i] = (int64_t *)vp;
        }
        if (ok && (hipMalloc(&ss.words, sizeof host_words) != hipSuccess ||
                   hipMemcpy(ss.words, host_words, sizeof host_words, hipMemcpyHostToDevice) != hipSuccess)) {
            why = "cannot store the signal word table";
            ok = false;
        }
        if (ok && hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess) {
            why = "hipEventCreate failed";
            ok = false;
        }
        if (!ok) break;
    }
    (void)hipGetLastError();
    if (!ok) {
        *err = "cannot create device-memory completion signals: " + why;
        stager_destroy(s);
        return nullptr;
    }
    s->worker = std::thread([s] { s->run(); });
    return s;
}

void stager_destroy(SdmaStager *s) {
    if (!s) return;
    {
        std::lock_guard<std::mutex> lk(s->mu);
        s->stop = true;
        s->stop_flag.store(true);
    }
    s->cv.notify_all();
    if (s->worker.joinable()) s->worker.join();  // the worker submits every queued job first
    // A kernel that has not reported its end may still use the counters, tables and host words,
    // and copies still in flight still complete their signals: whatever may still be in use is
    // leaked rather than freed.
    bool kernels_done = true;
    for (int set = 0; set < kSets; ++set) {
        SignalSet &ss = s->sets[set];
        if (ss.epoch && s->host_words && !spin_until(s->finished(set), ss.epoch, kReuseWaitSeconds)) {
            kernels_done = false;
            continue;
        }
        if (ss.epoch && s->host_words && s->tainted(set) && !s->drain(set, kReuseWaitSeconds)) continue;
        for (int c = 0; c <= kMaxPlanChunks; ++c)
            for (int q = 0; q < kMaxPieces; ++q)
                if (ss.sig[c][q].handle) hsa_signal_destroy(ss.sig[c][q]);
        if (ss.words) (void)hipFree(ss.words);
        if (ss.fork) (void)hipEventDestroy(ss.fork);
    }
    if (kernels_done) {
        if (s->scratch) (void)hipFree(s->scratch);
        if (s->counts) (void)hipFree(s->counts);
        if (s->host_words) (void)hipHostFree(s->host_words);
        if (s->slice_words) (void)hipHostFree(s->slice_words);
        if (s->slice_counts) (void)hipFree(s->slice_counts);
        delete s;
        hsa_shut_down();
    }
}

int stager_engine_count(const SdmaStager *s) { return s ? (int)s->engines.size() : 0; }

bool stager_failed(const SdmaStager *s) { return s && s->failed.load(); }

int stager_wait_call(SdmaStager *s, int set, uint64_t epoch) {
    if (set < 0 || set >= kSets) return -1;
    return spin_until(s->finished(set), epoch, kReuseWaitSeconds) ? 0 : -1;
}

int stager_wait_idle(SdmaStager *s) {
    for (int set = 0; set < kSets; ++set) {
        if (!s->sets[set].epoch) continue;
        if (!spin_until(s->finished(set), s->sets[set].epoch, kReuseWaitSeconds)) return -1;
        if (s->tainted(set) && !s->drain(set, kReuseWaitSeconds)) return -2;
    }
    return 0;
}

std::vector<CopyPiece> stager_plan(const SdmaStager *s, const std::vector<CopyPiece> &copies, int lead, int group_in) {
    // tuning knob: SPTL_SDMA_SPLIT=p stripes a chunk into up to p pieces per engine
    static const size_t split = [] {
        const char *e = getenv("SPTL_SDMA_SPLIT");
        const long v = e ? strtol(e, nullptr, 10) : 1;
        return (size_t)(v >= 1 && v <= 16 ? v : 1);
    }();
    // tuning knob: SPTL_SDMA_GROUP=g splits the later copies together in groups of g (0: by size)
    static const int forced_group = [] {
        const char *e = getenv("SPTL_SDMA_GROUP");
        const long v = e ? strtol(e, nullptr, 10) : 0;
        return (int)(v >= 1 && v <= 64 ? v : 0);
    }();
    std::vector<PlanCopy> pc;
    pc.reserve(copies.size());
    for (const CopyPiece &c : copies) pc.push_back({c.bytes, c.chunk});
    const int engines = (int)s->engines.size();
    const int group = group_in > 0     ? group_in
                      : forced_group ? forced_group
                                     : later_group(engines, copies.empty() ? 0 : copies[0].bytes);
    // the own slot's copies (kJoinChunk), which only the end of the call waits for, come last on
    // their own; SPTL_SDMA_JOIN_GROUPED=1 groups them with the peers' chunks (measurement aid)
    static const bool join_grouped = [] {
        const char *e = getenv("SPTL_SDMA_JOIN_GROUPED");
        return e && !strcmp(e, "1");
    }();
    int trailing = 0;
    for (size_t i = copies.size(); !join_grouped && i > 0 && copies[i - 1].chunk == kJoinChunk; --i) ++trailing;
    std::vector<CopyPiece> out;
    for (const PlanPiece &q : plan_pieces(pc, lead, engines, split, group, trailing)) {
        const CopyPiece &c = copies[(size_t)q.copy];
        CopyPiece piece{static_cast<char *>(c.dst) + q.offset, static_cast<const char *>(c.src) + q.offset, q.bytes,
                        q.chunk, q.piece};
        piece.engine = q.engine;
        out.push_back(piece);
    }
    return out;
}

std::vector<CopyPiece> stager_plan_links(const SdmaStager *s, const std::vector<CopyPiece> &copies,
                                         const std::vector<int> &link, int per) {
    std::vector<PlanCopy> pc;
    pc.reserve(copies.size());
    for (const CopyPiece &c : copies) pc.push_back({c.bytes, c.chunk});
    std::vector<CopyPiece> out;
    for (const PlanPiece &q : plan_pieces_links(pc, link, (int)s->engines.size(), per)) {
        const CopyPiece &c = copies[(size_t)q.copy];
        CopyPiece piece{static_cast<char *>(c.dst) + q.offset, static_cast<const char *>(c.src) + q.offset, q.bytes,
                        q.chunk, q.piece};
        piece.engine = q.engine;
        out.push_back(piece);
    }
    return out;
}

bool stager_take_timeouts(SdmaStager *s) {
    for (int set = 0; set < kSets; ++set)
        if (s->sets[set].epoch && __atomic_load_n(s->finished(set), __ATOMIC_ACQUIRE) == s->sets[set].epoch)
            (void)s->tainted(set);
    const bool r = s->timeout_pending;
    s->timeout_pending = false;
    return r;
}

int stager_begin(SdmaStager *s, const std::vector<CopyPiece> &pieces, int64_t workgroups, StageCall *out,
                 std::string *err, uint64_t *fresh_counts) {
    int count[kMaxPlanChunks + 1] = {};
    for (const CopyPiece &p : pieces) {
        if (p.chunk < 0 || p.chunk > kMaxPlanChunks || p.piece != count[p.chunk] || p.piece >= kMaxPieces) {
            *err = "copy pieces out of order or too many per chunk";
            return -1;
        }
        count[p.chunk]++;
    }
    int set;
    {
        std::lock_guard<std::mutex> lk(s->mu);
        set = s->next_set;
        s->next_set = (s->next_set + 1) % kSets;
        s->wake = true;
    }
    // A blocked worker takes tens of microseconds to wake up: wake it now, so that it is
    // polling by the time this call's job is queued (after the kernel launch).
    s->cv.notify_one();
    SignalSet &ss = s->sets[set];
    if (ss.epoch && !spin_until(s->finished(set), ss.epoch, kReuseWaitSeconds)) {
        *err = "an earlier staged call did not finish";
        return -1;
    }
    // After a timed-out wait the set's copies may still be in flight (or not yet submitted):
    // a late one would complete a signal re-armed for this call.
    if (s->tainted(set) && !s->drain(set, kReuseWaitSeconds)) {
        *err = "the copies of an earlier timed-out call did not complete";
        return -2;
    }
    for (int c = 0; c <= kMaxPlanChunks; ++c) {
        for (int q = 0; q < count[c]; ++q) hsa_signal_store_screlease(ss.sig[c][q], 1);
        ss.armed[c] = count[c];
    }
    out->set = set;
    for (int c = 0; c < kMaxPlanChunks; ++c) {
        out->ready[c] = count[c] ? ss.words + (size_t)c * kMaxPieces : nullptr;
        out->ready_n[c] = count[c];
    }
    out->join = count[kJoinChunk] ? ss.words + (size_t)kJoinChunk * kMaxPieces : nullptr;
    out->join_n = count[kJoinChunk];
    out->epoch = ++ss.epoch;
    out->fork = ss.fork;
    out->finished = const_cast<uint64_t *>(s->finished(set));
    out->timedout = const_cast<uint64_t *>(s->timedout(set));
    out->started = const_cast<uint64_t *>(s->started(set));
    // Cumulative counters of the set, or counters the caller zeroes before the launch.
    out->wg_count = fresh_counts ? fresh_counts : s->counts + (size_t)kSetCountWords * set;
    int groups = 0;
    for (int g = 0; g < kEndGroups; ++g) {
        const int64_t n = workgroups > g ? (workgroups - g + kEndGroups - 1) / kEndGroups : 0;
        const uint64_t base = fresh_counts ? 0 : ss.grp_total[g];
        out->grp_first[g] = ss.grp_total[g];
        out->grp_last[g] = n ? base + (uint64_t)n - 1 : ~0ull;
        if (!fresh_counts) ss.grp_total[g] += (uint64_t)n;
        groups += n ? 1 : 0;
    }
    const uint64_t all_base = fresh_counts ? 0 : ss.all_total;
    out->all_first = ss.all_total;
    out->all_last = all_base + (uint64_t)groups - 1;
    if (!fresh_counts) ss.all_total += (uint64_t)groups;
    // copy-out calls: the set's slice-ready words (pinned) and slice counters (device; the call
    // zeroes the ones it uses on its stream before the launch)
    out->slice_ready = s->slice_words + (size_t)kSliceSetWords * set;
    out->slice_count = s->slice_counts + (size_t)kSliceSetWords * set;
    return 0;
}

int stager_submit(SdmaStager *s, const StageCall &call, std::vector<CopyPiece> pieces, std::string *err,
                  bool gated, ForkWait fork) {
    (void)err;
    {
        std::lock_guard<std::mutex> lk(s->mu);
        s->queue.push_back(Job{call.set, call.epoch, call.fork, std::move(pieces), gated ? call.slice_ready : nullptr,
                               fork, call.started, !gated});
        s->queued.fetch_add(1, std::memory_order_release);
    }
    s->cv.notify_one();
    return 0;
}

void stager_cancel(SdmaStager *s, const StageCall &call) {
    // nothing ran on the set: mark the call finished and handled (no job was queued) and take
    // back its workgroup count
    SignalSet &ss = s->sets[call.set];
    for (int g = 0; g < kEndGroups; ++g) ss.grp_total[g] = call.grp_first[g];
    ss.all_total = call.all_first;
    for (int c = 0; c <= kMaxPlanChunks; ++c) ss.armed[c] = 0;
    ss.handled.store(call.epoch, std::memory_order_release);
    __atomic_store_n(s->host_words + 16 * call.set, call.epoch, __ATOMIC_RELEASE);
}

}  // namespace sptl
