// Device scratch of agmm_chunked_noalloc (sptl_noalloc.hip).  Internal to libsptl.so.
#pragma once

#include <stdint.h>

#include <string>

namespace sptl {

// Where a chunk-ordered launch of agmm_chunked_noalloc keeps its state, inside the device's
// scratch array.  flags: kFlagSetWords landed flags (never cleared: flag_epoch is new for every
// call on the device, and the array starts at zero); counts: count_words end-counter words that
// the call zeroes on its stream before the launch; err: the word a timed-out wait sets.
struct NoallocScratch {
    uint64_t *flags;
    uint64_t *counts;
    int64_t count_words;
    int *err;
    uint64_t flag_epoch;
};

// Set-up, once per device, with `device` current: resolves the address of this device's copy
// of the scratch array.  0, or -1 with *err set.
int noalloc_setup(int device, std::string *err);

// The scratch of `device` for one call (false if noalloc_setup has not run for it).
bool noalloc_scratch(int device, NoallocScratch *out);

}  // namespace sptl
