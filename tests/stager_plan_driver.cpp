// Prints the stager's copy-piece plan (sptl_plan.h) for the arguments
//   engines split lead bytes_0 bytes_1 ...
// one piece per line: copy offset bytes chunk piece engine.  Built and run by
// test_stager_plan.py on the CPU.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "sptl_plan.h"

int main(int argc, char **argv) {
    if (argc < 5) return 2;
    const int engines = atoi(argv[1]);
    const size_t split = (size_t)strtoull(argv[2], nullptr, 10);
    const int lead = atoi(argv[3]);
    std::vector<sptl::PlanCopy> copies;
    for (int i = 4; i < argc; ++i) copies.push_back({(size_t)strtoull(argv[i], nullptr, 10), i - 4});
    for (const sptl::PlanPiece &p : sptl::plan_pieces(copies, lead, engines, split))
        printf("%d %zu %zu %d %d %d\n", p.copy, p.offset, p.bytes, p.chunk, p.piece, p.engine);
    return 0;
}
