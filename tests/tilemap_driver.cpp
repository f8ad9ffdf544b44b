// Checks the GEMM tile orders of csrc/sptl_tilemap.h on the CPU.  Built and run by
// test_tilemap.py.
//   plain tiles_m tiles_n                  -> "ok" if the workgroups cover every tile once
//   chunk tpc tiles_n n_chunks forced conc -> "g band ok" if the chunk-ordered workgroups cover
//                                             every tile of every chunk once and each XCD
//                                             meets the chunks in position order
// Any failure prints "FAIL ..." and exits with status 1.
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "sptl_tilemap.h"

static int fail(const char *what, int a, int b) {
    printf("FAIL %s %d %d\n", what, a, b);
    return 1;
}

int main(int argc, char **argv) {
    if (argc < 2) return 2;
    const std::string mode = argv[1];
    if (mode == "plain" && argc == 4) {
        const int tm_n = atoi(argv[2]), tn_n = atoi(argv[3]);
        std::vector<int> seen((size_t)tm_n * tn_n, 0);
        for (int b = 0; b < tm_n * tn_n; ++b) {
            int tm, tn;
            sptl::plain_tile(tm_n, tn_n, b, tm, tn);
            if (tm < 0 || tm >= tm_n || tn < 0 || tn >= tn_n) return fail("range", b, tm);
            if (seen[(size_t)tm * tn_n + tn]++) return fail("twice", tm, tn);
        }
        printf("ok\n");
        return 0;
    }
    if (mode == "chunk" && argc == 7) {
        const int tpc = atoi(argv[2]), tiles_n = atoi(argv[3]), n_chunks = atoi(argv[4]);
        const int forced = atoi(argv[5]), conc = atoi(argv[6]);
        int band = 0;
        const int g = sptl::chunk_layout_choice(tpc, tiles_n, n_chunks, forced, conc, &band);
        if (band < 1) return fail("band", band, 0);
        const int per_chunk = tpc * tiles_n, total = per_chunk * n_chunks;
        std::vector<int> seen((size_t)total, 0);
        std::vector<int> last_pos(8, -1);
        for (int b = 0; b < total; ++b) {
            int pos, sub, tn;
            sptl::chunk_tile(tpc, tiles_n, g, band, b, pos, sub, tn);
            if (pos < 0 || pos >= n_chunks || sub < 0 || sub >= tpc || tn < 0 || tn >= tiles_n)
                return fail("range", b, pos);
            if (seen[((size_t)pos * tpc + sub) * tiles_n + tn]++) return fail("twice", b, pos);
            // workgroup b runs on XCD b mod 8, which runs its workgroups in index order
            if (pos < last_pos[b & 7]) return fail("order", b, pos);
            last_pos[b & 7] = pos;
        }
        printf("%d %d ok\n", g, band);
        return 0;
    }
    return 2;
}
