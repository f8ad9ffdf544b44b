// Copy kernel of the blit copy mode: the staging copies run on the compute units, as a ring
// all-gather's copies do, instead of on the copy engines.  Only used for the comparison of the
// two ("Add forward all-gather overlap", "Observations": a gather that runs on SMs takes them
// from the GEMM); the default path never launches it.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "sptl_internal.h"

namespace sptl {
namespace {

typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

constexpr int kBlitThreads = 256;
constexpr int kBlitUnroll = 4;  // 16-byte vectors per thread per pass

// dst[i] = src[i] for n 16-byte vectors.  Grid-stride: any grid size covers every vector; each
// pass issues kBlitUnroll independent loads before their stores.
__global__ void __launch_bounds__(kBlitThreads) blit_kernel(v4u32 *__restrict__ dst, const v4u32 *__restrict__ src,
                                                            int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kBlitThreads;
    int64_t i = (int64_t)blockIdx.x * kBlitThreads + threadIdx.x;
    for (; i + (kBlitUnroll - 1) * stride < n; i += kBlitUnroll * stride) {
        v4u32 v[kBlitUnroll];
#pragma unroll
        for (int u = 0; u < kBlitUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kBlitUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
    for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Permutation before sharding ("Affinity-Aware Sharding for Delayed Tensor Parallelism",
// abstract: the dense model is permuted, then sharded), bf16 [rows, cols] row-major.
// Rows: dst row i = src row perm[i], 16-byte vectors (cols % 8 == 0).  An index out of range
// gives a zero row and sets *err.
__global__ void __launch_bounds__(kBlitThreads) permute_rows_kernel(const v4u32 *__restrict__ src,
                                                                    v4u32 *__restrict__ dst,
                                                                    const int32_t *__restrict__ perm, int64_t rows,
                                                                    int64_t vec_per_row, int *err) {
    const int64_t n = rows * vec_per_row;
    for (int64_t i = (int64_t)blockIdx.x * kBlitThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlitThreads) {
        const int64_t r = i / vec_per_row, v = i - r * vec_per_row;
        const int32_t q = perm[r];
        v4u32 x = {0u, 0u, 0u, 0u};
        if (q >= 0 && q < rows) x = __builtin_nontemporal_load(src + (int64_t)q * vec_per_row + v);
        else if (v == 0) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_nontemporal_store(x, dst + i);
    }
}

// Columns: dst[r, j] = src[r, perm[j]].  A workgroup takes 8 columns x 256 rows: each thread
// gathers 8 elements of one row (the row's bytes are then in the caches for its neighbours)
// and stores them as one 16-byte vector (cols % 8 == 0).  An index out of range gives zeros and
// sets *err.
__global__ void __launch_bounds__(kBlitThreads) permute_cols_kernel(const uint16_t *__restrict__ src,
                                                                    v4u32 *__restrict__ dst,
                                                                    const int32_t *__restrict__ perm, int64_t rows,
                                                                    int64_t cols, int *err) {
    const int64_t vpr = cols / 8;
    const int64_t n = rows * vpr;
    for (int64_t i = (int64_t)blockIdx.x * kBlitThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlitThreads) {
        const int64_t r = i / vpr, v = i - r * vpr;
        const uint16_t *row = src + r * cols;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int32_t q0 = perm[v * 8 + 2 * e], q1 = perm[v * 8 + 2 * e + 1];
            const bool ok0 = q0 >= 0 && q0 < cols, ok1 = q1 >= 0 && q1 < cols;
            if (!(ok0 && ok1)) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t lo = ok0 ? row[q0] : 0u, hi = ok1 ? row[q1] : 0u;
            w[e] = lo | (hi << 16);
        }
        __builtin_nontemporal_store(v4u32{w[0], w[1], w[2], w[3]}, dst + i);
    }
}

}  // namespace

hipError_t launch_permute(const void *src, void *dst, int64_t rows, int64_t cols, int dim, const int32_t *perm,
                          int *err, hipStream_t stream) {
    const int64_t n = rows * (cols / 8);
    if (n <= 0) return hipSuccess;
    const int64_t g = std::min<int64_t>((n + kBlitThreads - 1) / kBlitThreads, 8192);
    if (dim == 0)
        hipLaunchKernelGGL(permute_rows_kernel, dim3((unsigned)g), dim3(kBlitThreads), 0, stream,
                           static_cast<const v4u32 *>(src), static_cast<v4u32 *>(dst), perm, rows, cols / 8, err);
    else
        hipLaunchKernelGGL(permute_cols_kernel, dim3((unsigned)g), dim3(kBlitThreads), 0, stream,
                           static_cast<const uint16_t *>(src), static_cast<v4u32 *>(dst), perm, rows, cols, err);
    return hipGetLastError();
}

hipError_t launch_blit(void *dst, const void *src, size_t bytes, int workgroups, hipStream_t stream) {
    const int64_t n = (int64_t)(bytes / 16);
    if (n <= 0) return hipSuccess;
    // default: enough workgroups for one unrolled pass, at most 8 per compute unit of the chip
    int64_t g = workgroups > 0 ? workgroups : (n + kBlitThreads * kBlitUnroll - 1) / (kBlitThreads * kBlitUnroll);
    if (workgroups <= 0 && g > 2048) g = 2048;
    hipLaunchKernelGGL(blit_kernel, dim3((unsigned)g), dim3(kBlitThreads), 0, stream, static_cast<v4u32 *>(dst),
                       static_cast<const v4u32 *>(src), n);
    return hipGetLastError();
}

}  // namespace sptl
