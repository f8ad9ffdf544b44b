// Launch planning of the register-resident epilogue: how many workgroups may share a CU.
// Plain host code, internal to libsptl.so.
//
// Every workgroup keeps all of its row's loads in flight, so the workgroups resident on a CU
// set how many rows HBM serves at once.  At 8192 rows of 9 inputs and 4096 columns, as many as
// the registers allow (5 per CU: 368 KiB of loads) streamed about 4 % slower than 3 per CU.
// The launch therefore caps the workgroups per CU through an unused LDS allocation, so that
// about kInflightBytes of loads are in flight per CU, for launches of at most kCapRowsPerCu
// rows per CU: at 64 rows per CU the cap was neutral and at 256 it cost about 2 %.  The result
// bits do not depend on it.
#pragma once

#include <stdint.h>

namespace sptl {

constexpr int64_t kInflightBytes = 192 * 1024;
constexpr int64_t kCapRowsPerCu = 48;

// Dynamic LDS bytes that cap a launch of `rows` workgroups, each with `bytes_per_wg` bytes of
// loads in flight, at the workgroups per CU that keep about `target` bytes in flight (0: no
// cap).  `forced`: the target was set explicitly and applies at any row count.  lds_per_cu,
// lds_per_block, cus: the device's limits.  A 1 KiB margin is left for the kernel's own LDS,
// and the allocation is a whole number of KiB.
inline int64_t epilogue_cap_lds(int64_t bytes_per_wg, int64_t rows, int64_t target, bool forced, int64_t lds_per_cu,
                                int64_t lds_per_block, int64_t cus) {
    if (target <= 0 || bytes_per_wg <= 0 || cus <= 0 || lds_per_cu <= 0) return 0;
    if (!forced && rows > kCapRowsPerCu * cus) return 0;
    int64_t wgs = (target + bytes_per_wg / 2) / bytes_per_wg;
    if (wgs < 1) wgs = 1;
    const int64_t dyn = (lds_per_cu / wgs - 1024) / 1024 * 1024;
    if (dyn <= 0 || dyn > lds_per_block - 1024) return 0;
    return dyn;
}

}  // namespace sptl
