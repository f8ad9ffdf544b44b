// Prints the stager's copy-piece plan (sptl_plan.h) for the arguments
//   engines split lead group[:trailing] bytes_0 bytes_1 ...
// (group 0: the size rule, later_group; trailing: the last copies kept out of the groups): first
// "group g", then one piece per line: copy offset bytes chunk piece engine.  With the arguments
//   links engines per bytes_0:link_0 bytes_1:link_1 ...
// it prints the link model's plan (plan_pieces_links) the same way, after "group 0".  Built and
// run by test_stager_plan.py on the CPU.
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "sptl_plan.h"

int main(int argc, char **argv) {
    if (argc >= 5 && std::string(argv[1]) == "links") {
        const int engines = atoi(argv[2]);
        const int per = atoi(argv[3]);
        std::vector<sptl::PlanCopy> copies;
        std::vector<int> link;
        for (int i = 4; i < argc; ++i) {
            char *end = nullptr;
            copies.push_back({(size_t)strtoull(argv[i], &end, 10), i - 4});
            link.push_back(end && *end == ':' ? atoi(end + 1) : -1);
        }
        printf("group 0\n");
        for (const sptl::PlanPiece &p : sptl::plan_pieces_links(copies, link, engines, per))
            printf("%d %zu %zu %d %d %d\n", p.copy, p.offset, p.bytes, p.chunk, p.piece, p.engine);
        return 0;
    }
    if (argc < 6) return 2;
    const int engines = atoi(argv[1]);
    const size_t split = (size_t)strtoull(argv[2], nullptr, 10);
    const int lead = atoi(argv[3]);
    char *tail = nullptr;
    int group = (int)strtol(argv[4], &tail, 10);
    const int trailing = tail && *tail == ':' ? atoi(tail + 1) : 0;
    std::vector<sptl::PlanCopy> copies;
    for (int i = 5; i < argc; ++i) copies.push_back({(size_t)strtoull(argv[i], nullptr, 10), i - 5});
    if (group == 0) group = sptl::later_group(engines, copies[0].bytes);
    printf("group %d\n", group);
    for (const sptl::PlanPiece &p : sptl::plan_pieces(copies, lead, engines, split, group, trailing))
        printf("%d %zu %zu %d %d %d\n", p.copy, p.offset, p.bytes, p.chunk, p.piece, p.engine);
    return 0;
}
