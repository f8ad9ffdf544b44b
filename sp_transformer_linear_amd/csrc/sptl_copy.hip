// Copy kernel of the blit copy mode: the staging copies run on the compute units, as a ring
// all-gather's copies do, instead of on the copy engines.  Only used for the comparison of the
// two ("Add forward all-gather overlap", "Observations": a gather that runs on SMs takes them
// from the GEMM); the default path never launches it.
#include <hip/hip_runtime.h>

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

}  // namespace

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
