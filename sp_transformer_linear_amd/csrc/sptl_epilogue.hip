// Fused reduce + residual + RMSNorm epilogue for the SP-TP linear layer (gfx950).
//
// h = in[0] + in[1] + ... + in[n-1]            (fp32, added in this order)
// y = h / sqrt(mean_j h_j^2 + eps) * gamma      (from the unrounded fp32 h)
// The sub-layer boundary of the AReaL async-TP issue ("Potential Solution": residual add and
// an RMSNorm over the hidden dimension between a reduce-scatter and the next all-gather) and
// the residual update of delayed TP (delayed-TP abstract: own partial now, peers' partials
// delta modules later) are both this kernel with different input lists.
//
// The kernel is HBM-bound: (n + 2) * hidden * 2 bytes move per row for ~(n + 4) * hidden flops.
// Design:
//   * one workgroup per row (rows are independent, so any split of the rows gives identical
//     bits); each thread owns VPT 16-byte vectors (8 bf16) of the row, strided by the block
//     size so that every load instruction of a wave covers 1 KB of contiguous memory;
//   * every input vector of the thread is loaded before any is used (NIN x VPT 16-byte loads
//     in flight per thread) with non-temporal hints: each byte is read exactly once;
//   * the sum of squares is reduced with wave64 butterfly shuffles, then across waves in LDS
//     in a fixed order;
//   * h and y are rounded to bf16 (nearest-even) and stored with 16-byte non-temporal stores
//     (streamed out rather than kept in the caches: ~11 % more bandwidth on cold inputs).
#include "sptl_internal.h"
#include "sptl_epilogue_plan.h"

#include <algorithm>
#include <atomic>
#include <cstdlib>

namespace sptl {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxThreads = 256;

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return f32_to_bf16(a) | (f32_to_bf16(b) << 16);
}

__device__ __forceinline__ void unpack8(const u32x4_t v, float *f) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        f[2 * w] = lo_bf16(v[w]);
        f[2 * w + 1] = hi_bf16(v[w]);
    }
}

__device__ __forceinline__ u32x4_t pack8(const float *f) {
    u32x4_t v;
    v.x = pack2(f[0], f[1]);
    v.y = pack2(f[2], f[3]);
    v.z = pack2(f[4], f[5]);
    v.w = pack2(f[6], f[7]);
    return v;
}

// Sum of `v` over the workgroup, the same value in every thread.  Fixed order: butterfly
// within each wave, then waves 0, 1, 2, ... in LDS.
__device__ __forceinline__ float block_sum(float v, float *red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float t = red[0];
    for (int w = 1; w < nwaves; ++w) t += red[w];
    return t;
}

template <int NIN, int VPT>
__global__ void __launch_bounds__(kMaxThreads) epilogue_kernel(EpilogueProblem p) {
    __shared__ float red[kMaxThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * p.hidden;
    const int nv = (int)(p.hidden >> 3);
    const u32x4_t zero = {0u, 0u, 0u, 0u};

    u32x4_t raw[NIN][VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int v = threadIdx.x + j * blockDim.x;
#pragma unroll
        for (int i = 0; i < NIN; ++i)
            raw[i][j] = v < nv ? __builtin_nontemporal_load(
                                     reinterpret_cast<const u32x4_t *>(p.in[i] + base) + v)
                               : zero;
    }

    float h[VPT][8];
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        unpack8(raw[0][j], h[j]);
#pragma unroll
        for (int i = 1; i < NIN; ++i) {
            float f[8];
            unpack8(raw[i][j], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) h[j][e] += f[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += h[j][e] * h[j][e];
    }

    if (p.h_out) {
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = threadIdx.x + j * blockDim.x;
            if (v < nv) __builtin_nontemporal_store(pack8(h[j]), reinterpret_cast<u32x4_t *>(p.h_out + base) + v);
        }
    }
    if (!p.y_out) return;  // uniform over the grid

    const float total = block_sum(ss, red);
    const float rstd = 1.0f / sqrtf(total / (float)p.hidden + p.eps);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int v = threadIdx.x + j * blockDim.x;
        if (v >= nv) continue;
        float g[8], y[8];
        unpack8(reinterpret_cast<const u32x4_t *>(p.gamma)[v], g);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = h[j][e] * rstd * g[e];
        __builtin_nontemporal_store(pack8(y), reinterpret_cast<u32x4_t *>(p.y_out + base) + v);
    }
}

// Rows too wide for the register-resident kernel: two passes over the inputs (the first
// only reads, the second recomputes h with the same order and writes h and y).
__global__ void __launch_bounds__(kMaxThreads) epilogue_wide_kernel(EpilogueProblem p) {
    __shared__ float red[kMaxThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * p.hidden;
    const int nv = (int)(p.hidden >> 3);
    auto row_sum = [&](int v, float *h) {
        unpack8(reinterpret_cast<const u32x4_t *>(p.in[0] + base)[v], h);
        for (int i = 1; i < p.n_in; ++i) {
            float f[8];
            unpack8(reinterpret_cast<const u32x4_t *>(p.in[i] + base)[v], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] += f[e];
        }
    };
    float rstd = 0.0f;
    if (p.y_out) {
        float ss = 0.0f;
        for (int v = threadIdx.x; v < nv; v += blockDim.x) {
            float h[8];
            row_sum(v, h);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += h[e] * h[e];
        }
        const float total = block_sum(ss, red);
        rstd = 1.0f / sqrtf(total / (float)p.hidden + p.eps);
        __syncthreads();  // every thread has read the inputs before any in-place write
    }
    for (int v = threadIdx.x; v < nv; v += blockDim.x) {
        float h[8];
        row_sum(v, h);
        if (p.h_out) reinterpret_cast<u32x4_t *>(p.h_out + base)[v] = pack8(h);
        if (p.y_out) {
            float g[8], y[8];
            unpack8(reinterpret_cast<const u32x4_t *>(p.gamma)[v], g);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = h[e] * rstd * g[e];
            reinterpret_cast<u32x4_t *>(p.y_out + base)[v] = pack8(y);
        }
    }
}

// Register-resident variant: NIN x VPT 16-byte vectors live per thread.  Kept to at most
// kMaxLiveVectors (4 VGPRs each) so the kernel does not spill; wider cases take the
// two-pass kernel.
constexpr int kMaxLiveVectors = 36;

// Workgroups per CU of the register-resident kernel: epilogue_cap_lds (sptl_epilogue_plan.h).

struct DeviceLimits {
    int lds_per_cu = 0, lds_per_block = 0, cus = 0;
};

DeviceLimits device_limits() {
    constexpr int kDevices = 64;
    static std::atomic<int> per_cu[kDevices], per_block[kDevices], cus[kDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return {};
    DeviceLimits l{per_cu[dev].load(std::memory_order_relaxed), per_block[dev].load(std::memory_order_relaxed),
                   cus[dev].load(std::memory_order_relaxed)};
    if (l.cus == 0) {
        int a = 0, b = 0, c = 0;
        if (hipDeviceGetAttribute(&a, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
            hipDeviceGetAttribute(&b, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
            return {};
        per_cu[dev].store(a, std::memory_order_relaxed);
        per_block[dev].store(b, std::memory_order_relaxed);
        cus[dev].store(c, std::memory_order_relaxed);
        l = {a, b, c};
    }
    return l;
}

// Dynamic LDS bytes of a launch of `rows` workgroups with `bytes_per_wg` bytes of loads each
// (0: no cap).  SPTL_EPI_INFLIGHT_KIB overrides the in-flight target and applies it at any row
// count (0: never cap; a measurement aid).
size_t inflight_cap_lds(int64_t bytes_per_wg, int64_t rows) {
    static const int64_t forced = [] {
        const char *e = getenv("SPTL_EPI_INFLIGHT_KIB");
        const long v = e ? strtol(e, nullptr, 10) : -1;
        return v >= 0 && v <= 65536 ? (int64_t)v * 1024 : (int64_t)-1;
    }();
    if (forced == 0) return 0;
    const DeviceLimits l = device_limits();
    return (size_t)epilogue_cap_lds(bytes_per_wg, rows, forced > 0 ? forced : kInflightBytes, forced > 0,
                                    l.lds_per_cu, l.lds_per_block, l.cus);
}

template <int N, int VPT>
bool launch_nin(const EpilogueProblem &p, int threads, hipStream_t s) {
    if constexpr (N * VPT <= kMaxLiveVectors) {
        if (p.n_in == N) {
            const size_t lds = inflight_cap_lds((int64_t)threads * VPT * N * 16, p.rows);
            hipLaunchKernelGGL((epilogue_kernel<N, VPT>), dim3((unsigned)p.rows),
                               dim3((unsigned)threads), lds, s, p);
            return true;
        }
    }
    if constexpr (N < kMaxEpilogueInputs) return launch_nin<N + 1, VPT>(p, threads, s);
    return false;
}

}  // namespace

hipError_t launch_epilogue(const EpilogueProblem &p, hipStream_t stream) {
    if (p.rows == 0) return hipSuccess;
    if (p.rows > 0x7fffffff || p.n_in < 1 || p.n_in > kMaxEpilogueInputs || (p.hidden & 7))
        return hipErrorInvalidValue;
    const int64_t nv = p.hidden >> 3;
    auto threads_for = [&](int vpt) {
        const int64_t t = (nv + vpt - 1) / vpt;
        return (int)((t + 63) / 64 * 64);
    };
    bool done = false;
    if (nv <= 256) done = launch_nin<1, 1>(p, threads_for(1), stream);
    else if (nv <= 512) done = launch_nin<1, 2>(p, threads_for(2), stream);
    else if (nv <= 1024) done = launch_nin<1, 4>(p, threads_for(4), stream);
    if (!done)
        hipLaunchKernelGGL(epilogue_wide_kernel, dim3((unsigned)p.rows), dim3(kMaxThreads), 0,
                           stream, p);
    return hipGetLastError();
}

}  // namespace sptl
