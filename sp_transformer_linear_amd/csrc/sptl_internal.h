// Internal interfaces between the C-ABI layer and the HIP kernels of libsptl.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sptl {

// C[M, N] = A[M, K] @ B[K, N]; bf16 inputs, fp32 accumulation, bf16 or fp32 output.
// Row-major with leading dimensions lda, ldb, ldc (elements).  K and N multiples of 8,
// pointers 16-byte aligned.  Every tile configuration uses the same MFMA instruction and
// the same ascending K order, so the result bits do not depend on the tiling.
struct GemmProblem {
    const uint16_t *a;
    const uint16_t *b;
    void *c;
    int64_t m, n, k;
    int64_t lda, ldb, ldc;
    bool c_f32;
};

enum class GemmTile { T256x256, T128x128, Auto };

// Picks a tile shape for the problem (Auto) and launches.  Returns the HIP error of the
// launch.
hipError_t launch_gemm(const GemmProblem &p, hipStream_t stream, GemmTile tile = GemmTile::Auto);

// Number of workgroups the launch of `p` uses with tile `t` (Auto resolved).
int64_t gemm_workgroups(const GemmProblem &p, GemmTile t = GemmTile::Auto);

constexpr int kMaxEpilogueInputs = 17;  // residual + 16 partials

// h = in[0] + in[1] + ... + in[n_in - 1] (fp32, in this order); y = RMSNorm(h) * gamma.
// h_out / y_out may be null (then not written; with y_out null no norm is taken).
struct EpilogueProblem {
    const uint16_t *in[kMaxEpilogueInputs];
    int n_in;
    const uint16_t *gamma;
    uint16_t *h_out;
    uint16_t *y_out;
    int64_t rows;
    int64_t hidden;  // multiple of 8
    float eps;
};

hipError_t launch_epilogue(const EpilogueProblem &p, hipStream_t stream);

}  // namespace sptl
