// Prints the stager's copy-piece plan (sptl_plan.h) for the arguments
//   engines split lead group bytes_0 bytes_1 ...
// (group 0: the size rule, later_group): first "group g", then one piece per line: copy offset
// bytes chunk piece engine.  Built and run by test_stager_plan.py on the CPU.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "sptl_plan.h"

int main(int argc, char **argv) {
    if (argc < 6) return 2;
    const int engines = atoi(argv[1]);
    const size_t split = (size_t)strtoull(argv[2], nullptr, 10);
    const int lead = atoi(argv[3]);
    int group = atoi(argv[4]);
    std::vector<sptl::PlanCopy> copies;
    for (int i = 5; i < argc; ++i) copies.push_back({(size_t)strtoull(argv[i], nullptr, 10), i - 5});
    if (group == 0) group = sptl::later_group(engines, copies[0].bytes);
    printf("group %d\n", group);
    for (const sptl::PlanPiece &p : sptl::plan_pieces(copies, lead, engines, split, group))
        printf("%d %zu %zu %d %d %d\n", p.copy, p.offset, p.bytes, p.chunk, p.piece, p.engine);
    return 0;
}
