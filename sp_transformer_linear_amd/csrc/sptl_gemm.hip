// bf16 GEMM on CDNA4 matrix cores (gfx950) for the SP-TP linear layer.
//
// C[M, N] = A[M, K] @ B[K, N], bf16 operands, fp32 accumulation, bf16 (nearest-even) or fp32
// stores.  This one kernel serves both the column-parallel chunk GEMMs of the chunked
// all-gather + matmul and the row-parallel partial-sum GEMM ("Potential Solution" of the
// AReaL async-TP issue; "partial output" in the delayed-TP abstract).
//
// Design for gfx950:
//   * 256 threads = 4 wave64s in a 2 x 2 grid over a BM x BN output tile; each wave owns a
//     (BM/2) x (BN/2) block made of 32 x 32 blocks of v_mfma_f32_32x32x16_bf16.
//   * K is walked in stages of 64.  Each stage of A ([BM][64]) and of B, stored transposed as
//     [BN][64] so both MFMA operands read 8 consecutive k per lane, sits in LDS, double
//     buffered (256 x 256 tile: 2 x 64 KB of the 160 KB LDS).  The next stage's global loads
//     are issued before the current stage's MFMAs and written to the other buffer after them,
//     so one barrier per stage suffices.
//   * B arrives N-contiguous ([in, out] weight layout); each thread loads an 8 x 8 block
//     (8 rows of 16 bytes) and transposes it in registers before its 16-byte LDS writes.
//   * LDS rows are 128 bytes (8 chunks of 16 bytes); chunk c of row r is stored at
//     c ^ ((r ^ r >> 3) & 7), which keeps both the fragment reads (8 consecutive rows, same
//     chunk) and the transposed B writes (rows 8 apart, same chunk) free of bank conflicts.
//   * Workgroups are dispatched round-robin over the 8 XCDs; the tile order gives each XCD a
//     contiguous run of tiles so that neighbouring tiles share that XCD's L2.
//   * Every tile shape uses the same MFMA instruction and visits K in the same ascending
//     order, with no split-K, so the result bits do not depend on tiling or chunking.
#include "sptl_internal.h"

namespace sptl {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;        // K depth of one LDS stage
constexpr int kThreads = 256;  // 4 waves in a 2 x 2 grid

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int BM, int BN>
struct Tile {
    static constexpr int WM = BM / 2, WN = BN / 2;          // one wave's block
    static constexpr int TM = WM / 32, TN = WN / 32;        // 32 x 32 MFMA blocks per wave
    static constexpr int A_VEC = BM * kBK / 8 / kThreads;   // 16-byte A vectors per thread
    static constexpr int B_BLK = (kBK / 8) * (BN / 8);      // 8 x 8 B blocks per stage
    static constexpr int LDS_A = BM * kBK / 8;              // 16-byte chunks per A stage
    static constexpr int LDS_B = BN * kBK / 8;
    static_assert(A_VEC >= 1 && B_BLK <= kThreads, "tile shape");
};

template <int BM, int BN, bool OUT_F32>
__global__ void __launch_bounds__(kThreads)
gemm_bf16_kernel(GemmProblem p, int tiles_m, int tiles_n) {
    using T = Tile<BM, BN>;
    __shared__ u32x4_t smem[2 * (T::LDS_A + T::LDS_B)];
    u32x4_t *As = smem;                  // [2][BM][8 chunks]
    u32x4_t *Bs = smem + 2 * T::LDS_A;   // [2][BN][8 chunks], B transposed

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave >> 1) * T::WM;
    const int wn0 = (wave & 1) * T::WN;

    // XCD-aware tile order: workgroup b runs on XCD b % 8; XCD x takes a contiguous run.
    const int nt = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int per = nt >> 3, rem = nt & 7;
    const int xcd = bid & 7, slot = bid >> 3;
    const int t = xcd * per + (xcd < rem ? xcd : rem) + slot;
    const int tm = t / tiles_n, tn = t - tm * tiles_n;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    const u32x4_t zero = {0u, 0u, 0u, 0u};
    u32x4_t ra[T::A_VEC];
    u32x4_t rb[8];

    const int b_kb = tid / (BN / 8), b_nb = tid % (BN / 8);
    const bool b_active = tid < T::B_BLK;

    auto load_stage = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < T::A_VEC; ++i) {
            const int q = tid + i * kThreads;
            const int r = q >> 3, c = q & 7;
            const int64_t gm = m0 + r, gk = k0 + c * 8;
            ra[i] = (gm < p.m && gk < p.k)
                        ? *reinterpret_cast<const u32x4_t *>(p.a + gm * p.lda + gk) : zero;
        }
        if (b_active) {
            const int64_t gn = n0 + b_nb * 8;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t gk = k0 + b_kb * 8 + j;
                rb[j] = (gk < p.k && gn < p.n)
                            ? *reinterpret_cast<const u32x4_t *>(p.b + gk * p.ldb + gn) : zero;
            }
        }
    };

    auto store_stage = [&](int buf) {
        u32x4_t *as = As + buf * T::LDS_A;
#pragma unroll
        for (int i = 0; i < T::A_VEC; ++i) {
            const int q = tid + i * kThreads;
            const int r = q >> 3, c = q & 7;
            as[r * 8 + (c ^ swz(r))] = ra[i];
        }
        if (b_active) {
            u32x4_t *bs = Bs + buf * T::LDS_B;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                // column c of the 8 x 8 block: k = 0..7 of output feature b_nb * 8 + c
                const int w = c >> 1, sh = (c & 1) * 16;
                u32x4_t o;
                o.x = ((rb[0][w] >> sh) & 0xffffu) | (((rb[1][w] >> sh) & 0xffffu) << 16);
                o.y = ((rb[2][w] >> sh) & 0xffffu) | (((rb[3][w] >> sh) & 0xffffu) << 16);
                o.z = ((rb[4][w] >> sh) & 0xffffu) | (((rb[5][w] >> sh) & 0xffffu) << 16);
                o.w = ((rb[6][w] >> sh) & 0xffffu) | (((rb[7][w] >> sh) & 0xffffu) << 16);
                const int n = b_nb * 8 + c;
                bs[n * 8 + (b_kb ^ swz(n))] = o;
            }
        }
    };

    f32x16_t acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto compute_stage = [&](int buf) {
        const u32x4_t *as = As + buf * T::LDS_A;
        const u32x4_t *bs = Bs + buf * T::LDS_B;
#pragma unroll
        for (int s = 0; s < kBK / 16; ++s) {
            const int ch = 2 * s + (lane >> 5);  // 16-byte chunk holding k = 16 s + 8 (lane / 32) ..
            bf16x8_t af[T::TM], bfr[T::TN];
#pragma unroll
            for (int i = 0; i < T::TM; ++i) {
                const int r = wm0 + i * 32 + (lane & 31);
                af[i] = __builtin_bit_cast(bf16x8_t, as[r * 8 + (ch ^ swz(r))]);
            }
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const int n = wn0 + j * 32 + (lane & 31);
                bfr[j] = __builtin_bit_cast(bf16x8_t, bs[n * 8 + (ch ^ swz(n))]);
            }
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j],
                                                                        0, 0, 0);
        }
    };

    const int nk = (int)((p.k + kBK - 1) / kBK);
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) load_stage((int64_t)(kt + 1) * kBK);
        compute_stage(cur);
        if (more) store_stage(cur ^ 1);
        __syncthreads();
    }

    // 32 x 32 MFMA result layout: lane l holds column l % 32; register r holds row
    // 8 (r / 4) + 4 (l / 32) + r % 4.
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int64_t col = n0 + wn0 + j * 32 + (lane & 31);
            if (col >= p.n) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (row < p.m) {
                    if constexpr (OUT_F32)
                        static_cast<float *>(p.c)[row * p.ldc + col] = acc[i][j][r];
                    else
                        static_cast<uint16_t *>(p.c)[row * p.ldc + col] = f32_to_bf16(acc[i][j][r]);
                }
            }
        }
    }
}

template <int BM, int BN>
hipError_t launch_tile(const GemmProblem &p, hipStream_t stream) {
    const int64_t tm = (p.m + BM - 1) / BM, tn = (p.n + BN - 1) / BN;
    const int64_t nt = tm * tn;
    if (nt == 0) return hipSuccess;
    if (nt > 0x7fffffff) return hipErrorInvalidValue;
    if (p.c_f32)
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, true>), dim3((unsigned)nt), dim3(kThreads), 0,
                           stream, p, (int)tm, (int)tn);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, false>), dim3((unsigned)nt), dim3(kThreads), 0,
                           stream, p, (int)tm, (int)tn);
    return hipGetLastError();
}

GemmTile resolve(const GemmProblem &p, GemmTile t) {
    if (t != GemmTile::Auto) return t;
    // One wave of 256 x 256 tiles needs about one workgroup per CU (256 on MI355X); below
    // that, 128 x 128 tiles keep every CU busy.
    const int64_t big = ((p.m + 255) / 256) * ((p.n + 255) / 256);
    return big >= 240 ? GemmTile::T256x256 : GemmTile::T128x128;
}

}  // namespace

int64_t gemm_workgroups(const GemmProblem &p, GemmTile t) {
    const int s = resolve(p, t) == GemmTile::T256x256 ? 256 : 128;
    return ((p.m + s - 1) / s) * ((p.n + s - 1) / s);
}

hipError_t launch_gemm(const GemmProblem &p, hipStream_t stream, GemmTile tile) {
    switch (resolve(p, tile)) {
        case GemmTile::T256x256: return launch_tile<256, 256>(p, stream);
        default: return launch_tile<128, 128>(p, stream);
    }
}

}  // namespace sptl
