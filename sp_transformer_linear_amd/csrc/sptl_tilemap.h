// Tile orders of the GEMM launches: which output tile a workgroup index takes, and the
// host-side choice of the chunk-ordered layout.  Plain index arithmetic, shared by the kernels
// (device) and the launch planning (host); internal to libsptl.so.
//
// Workgroup b of a launch runs on XCD b mod 8, and each XCD runs its workgroups in index
// order.  The orders below give each XCD contiguous runs of a banded tile order (bands of a
// few tile rows, column-major inside a band), so the workgroups an XCD runs at once share a
// few A and B panels in its L2.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SPTL_HD __host__ __device__ __forceinline__
#else
#define SPTL_HD inline
#endif

namespace sptl {

constexpr int kBand = 4;  // tile rows per band of the plain tile order

// Plain launches over tiles_m x tiles_n tiles: workgroup bid takes tile (tm, tn).  XCD x takes
// the x-th eighth (rounded) of the banded order.
SPTL_HD void plain_tile(int tiles_m, int tiles_n, int bid, int &tm, int &tn) {
    const int nt = tiles_m * tiles_n;
    const int per = nt >> 3, rem = nt & 7;
    const int xcd = bid & 7, slot = bid >> 3;
    const int t = xcd * per + (xcd < rem ? xcd : rem) + slot;
    const int band = t / (kBand * tiles_n), in_band = t - band * (kBand * tiles_n);
    const int band_rows = tiles_m - band * kBand < kBand ? tiles_m - band * kBand : kBand;
    tm = band * kBand + in_band % band_rows;
    tn = in_band / band_rows;
}

// Chunk-ordered launches: chunks of tpc tile rows, taken in processing position order.
// Workgroup bid takes tile row `sub` and column `tn` of the chunk at position `pos`.
//   g > 0: a chunk's tiles go to a group of g XCDs and 8 / g chunks run side by side; each
//          XCD's share of a chunk is a contiguous run of the chunk's banded order with kb
//          tile rows per band;
//   g = 0: chunk after chunk, row-major inside a chunk.
// Either way every XCD meets the chunks in position order.
SPTL_HD void chunk_tile(int tpc, int tiles_n, int g, int kb, int bid, int &pos, int &sub, int &tn) {
    const int per_chunk = tpc * tiles_n;
    if (g) {
        const int x = bid & 7, slot = bid >> 3, share = per_chunk / g;
        pos = (slot / share) * (8 / g) + x / g;
        const int t = (x % g) * share + slot % share;
        const int band = t / (kb * tiles_n), in_band = t - band * (kb * tiles_n);
        const int band_rows = tpc - band * kb < kb ? tpc - band * kb : kb;
        sub = band * kb + in_band % band_rows;
        tn = in_band / band_rows;
    } else {
        pos = bid / per_chunk;
        const int local = bid - pos * per_chunk;
        sub = local / tiles_n;
        tn = local - sub * tiles_n;
    }
}

// Host: the chunk-ordered layout for chunks of tpc x tiles_n tiles, n_chunks of them, when each
// XCD runs `conc` workgroups at once.  Returns g, the XCDs per chunk: `forced` if it divides
// evenly, else the most of 8, 4, 2, 1 that divide a chunk's tiles (with 8 / g dividing the
// chunk count), so that a chunk that has landed while others have not is spread over the
// whole chip; 0 when none does.  *band gets the band height: the concurrent workgroups of an
// XCD hold one band x ceil(share / band) block in each of the chunks they span, at the same
// columns, and the band minimises the A plus B panels they read (ties: the band nearest
// kBand).
inline int chunk_layout_choice(int64_t tpc, int64_t tiles_n, int n_chunks, int forced, int64_t conc, int *band) {
    const int64_t per_chunk = tpc * tiles_n;
    auto fits = [&](int c) { return per_chunk % c == 0 && n_chunks % (8 / c) == 0; };
    int g = (forced == 1 || forced == 2 || forced == 4 || forced == 8) && fits(forced) ? forced : 0;
    for (int c = 8; c >= 1 && !g; c /= 2)
        if (fits(c)) g = c;
    *band = kBand;
    if (!g) return 0;
    const int64_t share = per_chunk / g;
    const int64_t width = share < conc ? share : conc, chunks = (conc + share - 1) / share;
    int64_t best = -1;
    for (int b = 1; b <= 8 && b <= tpc; b *= 2) {
        const int64_t panels = chunks * b + (width + b - 1) / b;
        const int dist = b > kBand ? b - kBand : kBand - b;
        const int best_dist = *band > kBand ? *band - kBand : kBand - *band;
        if (best < 0 || panels < best || (panels == best && dist < best_dist)) {
            best = panels;
            *band = b;
        }
    }
    return g;
}

}  // namespace sptl
