// Prints the epilogue's cap allocation (sptl_epilogue_plan.h) for each line of stdin:
//   bytes_per_wg rows target forced lds_per_cu lds_per_block cus
// one dynamic-LDS byte count per line.  Built and run by test_epilogue_plan.py on the CPU.
#include <cstdio>

#include "sptl_epilogue_plan.h"

int main() {
    long long b, r, t, f, lc, lb, c;
    while (scanf("%lld %lld %lld %lld %lld %lld %lld", &b, &r, &t, &f, &lc, &lb, &c) == 7)
        printf("%lld\n", (long long)sptl::epilogue_cap_lds(b, r, t, f != 0, lc, lb, c));
    printf("target %lld rows_per_cu %lld\n", (long long)sptl::kInflightBytes, (long long)sptl::kCapRowsPerCu);
    return 0;
}
