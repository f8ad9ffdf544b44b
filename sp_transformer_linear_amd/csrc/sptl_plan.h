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
//   * the later copies are split together in groups, like the leading group, with enough
//     copies per group that every engine's piece is at least kGroupPiece bytes (a copy engine
//     streams a small piece at about half its rate); copies large enough for that on their own
//     are striped over all engines one after another (piece p on engine p), at most
//     kMaxPieces pieces and no piece below kMinPiece / split bytes;
//   * the trailing copies that no tile waits for (this rank's own slot, which only the end of
//     the call waits for) join the peers' last group only when they add at most a quarter of
//     its bytes; otherwise they come last, striped over the engines in pieces of at least
//     kGroupPiece bytes, so they do not hold back chunks that tiles wait for;
//   * pieces are equal and rounded up to 256 bytes; the last piece of a copy takes the rest.
// Each engine takes its pieces in the order returned.
//
// plan_pieces_links is the link model: each peer's copies run on engines of their own, as each
// peer's chunks would come over a point-to-point link of their own on a node.
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

// Group size for the later copies of `chunk_bytes` each: the fewest copies that give every
// engine a piece of at least kGroupPiece bytes (1 when a striped copy already does).
constexpr size_t kGroupPiece = 2 * 1024 * 1024;

inline int later_group(int engines, size_t chunk_bytes) {
    if (engines < 1 || chunk_bytes == 0) return 1;
    const size_t want = (size_t)engines * kGroupPiece;
    const size_t g = (want + chunk_bytes - 1) / chunk_bytes;
    return g < 1 ? 1 : g > (size_t)engines ? engines : (int)g;
}

// Appends copy i cut into equal pieces rounded to 256 bytes (the last takes the remainder, so
// at most n pieces), on engines first, first + 1, ... (mod engines).
inline void cut_copy(std::vector<PlanPiece> &out, const std::vector<PlanCopy> &copies, int i, size_t n, int first,
                     int engines) {
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
}

// `split` (>= 1) allows up to split pieces per engine and copy; `engines` >= 1.  `group` (>= 1)
// splits the later copies together in successive groups of `group` copies, like the leading
// group (1: each later copy striped over all engines on its own); a last group shorter than
// `group` is merged into the one before when both fit on the engines.  The last `trailing`
// copies join the last group when they add at most a quarter of its bytes and all fit on the
// engines; otherwise they are striped one after another, in pieces of at least kGroupPiece bytes.
inline std::vector<PlanPiece> plan_pieces(const std::vector<PlanCopy> &copies, int lead, int engines, size_t split,
                                          int group = 1, int trailing = 0) {
    std::vector<PlanPiece> out;
    size_t E = (size_t)engines * split;
    if (E > (size_t)kMaxPieces) E = kMaxPieces;
    auto cut = [&](int i, size_t n, int first) { cut_copy(out, copies, i, n, first, engines); };
    // copies [b, e) (e - b <= engines) split together: each takes a run of distinct engines, about
    // in proportion to its size, and the runs cover every engine
    auto joint = [&](int b, int e) {
        size_t bytes = 0;
        for (int i = b; i < e; ++i) bytes += copies[(size_t)i].bytes;
        int first = 0;
        for (int i = b; i < e; ++i) {
            const int rest = e - 1 - i;  // copies after this one, each needs an engine
            size_t n = bytes ? (size_t)(((double)copies[(size_t)i].bytes / (double)bytes) * engines + 0.5) : 1;
            if (n < 1) n = 1;
            if ((int)n > engines - first - rest) n = (size_t)(engines - first - rest);
            if (i == e - 1) n = (size_t)(engines - first);
            if (n > (size_t)kMaxPieces) n = kMaxPieces;
            const size_t by_size = copies[(size_t)i].bytes / (kMinPiece / split);
            if (n > by_size) n = by_size < 1 ? 1 : by_size;
            cut(i, n, first);
            first += (int)n;
        }
    };
    const int total = (int)copies.size();
    if (trailing < 0) trailing = 0;
    if (trailing > total) trailing = total;
    const int count = total - trailing;  // the copies that tiles wait for
    if (lead > count) lead = count;
    if (lead > engines) lead = engines;
    if (lead < 1) lead = 1;
    if (group > engines) group = engines;
    if (group < 1) group = 1;
    if (lead > 1) joint(0, lead);
    auto bytes_of = [&](int b, int e) {
        size_t n = 0;
        for (int i = b; i < e; ++i) n += copies[(size_t)i].bytes;
        return n;
    };
    bool merged = false;  // the trailing copies went into the last group
    for (int i = lead > 1 ? lead : 0; i < count;) {
        if (group > 1) {
            int e = i + group < count ? i + group : count;
            // a short last group joins this one when they fit on the engines together, so no
            // copy is left to run alone at the end
            if (e < count && count - e < group && count - i <= engines) e = count;
            // the trailing copies join the last group when they add at most a quarter of its bytes
            // (its chunks then land at most a quarter later, and no copy runs on alone while the
            // tiles of the next chunks compute)
            if (e == count && trailing && total - i <= engines && 4 * bytes_of(count, total) <= bytes_of(i, e)) {
                e = total;
                merged = true;
            }
            joint(i, e);
            i = e;
        } else {
            size_t n = copies[(size_t)i].bytes / (kMinPiece / split);
            n = n < 1 ? 1 : n > E ? E : n;
            cut(i, n, 0);
            ++i;
        }
    }
    for (int i = merged ? total : count; i < total; ++i) {  // pieces of at least kGroupPiece
        size_t n = copies[(size_t)i].bytes / kGroupPiece;
        n = n < 1 ? 1 : n > E ? E : n;
        cut(i, n, 0);
    }
    return out;
}

// Link model.  link[i] is the peer of copy i (0 for the first peer after this rank, 1 for the
// next, ...; -1 for a copy that crosses no link, such as this rank's own slot).  Peer p's copies
// run only on its `per` engines (p * per + j) mod engines, j < per, each copy striped over them in
// the order given (no piece below kMinPiece unless the copy is smaller); the other copies are
// striped over every engine.  Each engine takes its pieces in the order returned, so a peer's
// copies land in their order, at the rate of its engines alone.
inline std::vector<PlanPiece> plan_pieces_links(const std::vector<PlanCopy> &copies, const std::vector<int> &link,
                                                int engines, int per) {
    std::vector<PlanPiece> out;
    if (per < 1) per = 1;
    if (per > engines) per = engines;
    for (int i = 0; i < (int)copies.size(); ++i) {
        const bool peer = link[(size_t)i] >= 0;
        size_t n = (size_t)(peer ? per : engines);
        if (n > (size_t)kMaxPieces) n = kMaxPieces;
        const size_t by_size = copies[(size_t)i].bytes / kMinPiece;
        if (n > by_size) n = by_size < 1 ? 1 : by_size;
        cut_copy(out, copies, i, n, peer ? (int)(((size_t)link[(size_t)i] * (size_t)per) % (size_t)engines) : 0,
                 engines);
    }
    return out;
}

}  // namespace sptl
