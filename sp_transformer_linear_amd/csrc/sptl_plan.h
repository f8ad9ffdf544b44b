// Piece planning of the SDMA chunk stager: how each staging copy of agmm_chunked is split into
// copy pieces and which engine takes each piece.  Plain host code (no HIP or HSA), internal to
// libsptl.so.
//
// The chunked all-gather is the communication half of the chunked all-gather + matmul
// ("Potential Solution" of the AReaL async-TP issue); the copies run on copy engines rather
// than compute units ("Observations" of Megatron-LM pull request 5513).  Each copy engine
// spends a fixed time per piece beyond its streaming rate, so pieces are as large as the
// pipeline allows:
//   * the first `lead` copies (the peer chunks that the GEMM's first round of tiles needs) are
//     split together, about one piece per engine in proportion to their sizes, so that they
//     land at about the same time, as early as the engines allow;
//   * every later copy is striped over all engines (piece p on engine p), at most kMaxPieces
//     pieces and no piece below kMinPiece / split bytes;
//   * pieces are equal and rounded up to 256 bytes; the last piece of a copy takes the rest.
// Each engine takes its pieces in the order returned.
#pragma once

#include <stddef.h>

#include <vector>

namespace sptl {

constexpr int kMaxPieces = 16;               // copy pieces per chunk, each with a completion signal
constexpr size_t kMinPiece = 512 * 1024;     // below this, striping costs more than it gains

struct PlanCopy {
    size_t bytes;
    int chunk;
};

struct PlanPiece {
    int copy;       // index into the copies
    size_t offset;  // byte offset within the copy
    size_t bytes;
    int chunk;
    int piece;      // index within the copy, from 0
    int engine;     // in [0, engines)
};

// `split` (>= 1) allows up to split pieces per engine and copy; `engines` >= 1.
inline std::vector<PlanPiece> plan_pieces(const std::vector<PlanCopy> &copies, int lead, int engines, size_t split) {
    std::vector<PlanPiece> out;
    size_t E = (size_t)engines * split;
    if (E > (size_t)kMaxPieces) E = kMaxPieces;
    // equal pieces of copy i rounded to 256 bytes (the last takes the remainder, so at most n
    // pieces), on engines first, first + 1, ...
    auto cut = [&](int i, size_t n, int first) {
        const PlanCopy &c = copies[(size_t)i];
        const size_t step = ((c.bytes / n) + 255) & ~(size_t)255;
        size_t off = 0;
        int piece = 0;
        while (off < c.bytes) {
            const size_t b = c.bytes - off < step ? c.bytes - off : step;
            out.push_back({i, off, b, c.chunk, piece, (first + piece) % engines});
            off += b;
            ++piece;
        }
    };
    if (lead > (int)copies.size()) lead = (int)copies.size();
    if (lead > engines) lead = engines;
    if (lead < 1) lead = 1;
    size_t lead_bytes = 0;
    for (int i = 0; i < lead; ++i) lead_bytes += copies[(size_t)i].bytes;
    int first = 0;
    for (int i = 0; i < lead && lead > 1; ++i) {
        const int rest = lead - 1 - i;  // copies after this one, each needs an engine
        size_t n = lead_bytes ? (size_t)(((double)copies[(size_t)i].bytes / (double)lead_bytes) * engines + 0.5) : 1;
        if (n < 1) n = 1;
        if ((int)n > engines - first - rest) n = (size_t)(engines - first - rest);
        if (i == lead - 1) n = (size_t)(engines - first);
        if (n > (size_t)kMaxPieces) n = kMaxPieces;
        const size_t by_size = copies[(size_t)i].bytes / (kMinPiece / split);
        if (n > by_size) n = by_size < 1 ? 1 : by_size;
        cut(i, n, first);
        first += (int)n;
    }
    for (size_t i = lead > 1 ? (size_t)lead : 0; i < copies.size(); ++i) {
        size_t n = copies[i].bytes / (kMinPiece / split);
        n = n < 1 ? 1 : n > E ? E : n;
        cut((int)i, n, 0);
    }
    return out;
}

}  // namespace sptl
