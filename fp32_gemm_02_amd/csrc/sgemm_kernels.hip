// gfx950 (CDNA4) kernels for C <- alpha*A*B + beta*C in fp32.
//
// The GEMM kernel is the single-GPU leaf of the Phobos pages: one workgroup
// owns one BM x BN tile of C and walks K in chunks of BK, accumulating
// acc += A_tile * B_tile ("Show HN: Phobos", section "Matrix
// Multiplication"), then stores alpha*acc + beta*C.  The techniques the blog
// lists in "GPU Performance" (coalescing, a shared-memory tile per CTA, a
// per-warp register micro-tile free of bank conflicts, the matrix units) and
// the ping-pong buffering of "Are we cuBLAS yet?" map onto CDNA4 as:
//   - global -> LDS with 128-bit loads, consecutive lanes on consecutive
//     addresses; one stage in flight in registers while the other is used;
//   - two LDS stages (double buffering), one barrier per K chunk;
//   - each 64-lane wavefront owns a TWM x TWN sub-tile made of MB x NB blocks
//     of 32 x 32, accumulated by v_mfma_f32_32x32x2_f32 in registers for the
//     whole K loop;
//   - LDS rows of A padded so that the MFMA operand reads are conflict free.
//
// MFMA 32x32x2 f32 operand layout (one block, 64 lanes, l = lane):
//   src A: lane l holds A'[l % 32][l / 32]      (32 x 2)
//   src B: lane l holds B'[l / 32][l % 32]      (2 x 32)
//   acc  : lane l, register r holds D[8*(r/4) + 4*(l/32) + r%4][l % 32]
// Two free choices make the LDS reads wide:
//   - k order: within a BK chunk, lane half h = l/32 takes the k values
//     h*BK/2 + kk for kk = 0..BK/2-1, so a lane reads 4 consecutive k of its
//     A row with one ds_read_b128 (four MFMA steps' worth).
//   - column order: block bn of a wave holds the columns NB*j + bn
//     (j = 0..31), so one NB-wide LDS read of B feeds all NB blocks, and the
//     epilogue writes NB consecutive columns of C with one vector store.
// Any permutation of k leaves the sum's terms unchanged (only their order,
// which the fp32 result may depend on within the error bound).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgemm_internal.h"

namespace phobos {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int BM, int BN, int BK, int WM, int WN>
struct TileShape {
    static constexpr int NT = 64 * WM * WN;      // threads per workgroup
    static constexpr int TWM = BM / WM;          // wave tile rows
    static constexpr int TWN = BN / WN;          // wave tile columns
    static constexpr int MB = TWM / 32;          // 32x32 blocks per wave, rows
    static constexpr int NB = TWN / 32;          // 32x32 blocks per wave, columns
    static constexpr int LDA_S = BK + 4;         // A row stride in LDS (floats)
    static constexpr int LDB_S = BN;             // B row stride in LDS (floats)
    static constexpr int A_FLOATS = BM * LDA_S;
    static constexpr int B_FLOATS = BK * LDB_S;
    static constexpr int STAGE = A_FLOATS + B_FLOATS;
    static constexpr int LDS_BYTES = 2 * STAGE * 4;
    static constexpr int QA = BK / 4;            // float4 per A tile row
    static constexpr int LA = BM * QA / NT;      // float4 of A per thread per stage
    static constexpr int QB = BN / 4;            // float4 per B tile row
    static constexpr int LB = BK * QB / NT;      // float4 of B per thread per stage
    static_assert(BM % WM == 0 && BN % WN == 0, "wave grid must divide the tile");
    static_assert(TWM % 32 == 0 && TWN % 32 == 0, "wave tile is whole 32x32 blocks");
    static_assert(NB == 1 || NB == 2 || NB == 4, "B reads are 1, 2 or 4 floats wide");
    static_assert(BK % 8 == 0, "BK/2 must be a multiple of 4 (b128 A reads)");
    static_assert((BM * QA) % NT == 0 && (BK * QB) % NT == 0, "whole loads per thread");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS of one CU");
};

// Map the workgroup to its output tile.  Workgroups are handed to the 8 XCDs
// of the chip round robin (id % 8); with xcd_remap the ids an XCD receives
// become one contiguous run of the raster order, so tiles that share rows of
// A and columns of B sit in the same L2.  The raster walks group_m tile rows
// at a time, column by column, to keep the A panels of a group hot.
__device__ __forceinline__ void tile_of(const GemmArgs& p, int& tm, int& tn) {
    int bid = blockIdx.x;
    if (p.xcd_remap) {
        const int per = (p.tiles_m * p.tiles_n) >> 3;
        bid = (bid & 7) * per + (bid >> 3);
    }
    const int group = p.group_m * p.tiles_n;
    const int g = bid / group;
    const int first = g * p.group_m;
    const int gsz = min(p.tiles_m - first, p.group_m);
    const int r = bid - g * group;
    tm = first + r % gsz;
    tn = r / gsz;
}

// Load 4 consecutive floats src[0..3] whose positions are valid while
// e < nvalid (nvalid <= 0: all zero).  VEC: src is 16-byte aligned.
template <bool VEC>
__device__ __forceinline__ f32x4 load4(const float* src, int nvalid) {
    f32x4 v;
    if (VEC && nvalid >= 4) {
        v = *reinterpret_cast<const f32x4*>(src);
    } else {
        v[0] = nvalid > 0 ? src[0] : 0.0f;
        v[1] = nvalid > 1 ? src[1] : 0.0f;
        v[2] = nvalid > 2 ? src[2] : 0.0f;
        v[3] = nvalid > 3 ? src[3] : 0.0f;
    }
    return v;
}

template <int BM, int BN, int BK, int WM, int WN, bool VEC>
__global__ __launch_bounds__(64 * WM * WN) void sgemm_mfma_kernel(GemmArgs p) {
    using T = TileShape<BM, BN, BK, WM, WN>;
    __shared__ __attribute__((aligned(16))) float smem[2 * T::STAGE];

    int tm, tn;
    tile_of(p, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int l32 = lane & 31;
    const int h = lane >> 5;

    // ---- global -> register staging (one K chunk) ----
    f32x4 ra[T::LA], rb[T::LB];
    auto load_stage = [&](int k0) {
#pragma unroll
        for (int i = 0; i < T::LA; ++i) {
            const int idx = tid + i * T::NT;
            const int row = idx / T::QA;
            const int kq = (idx % T::QA) * 4;
            const int grow = m0 + row;
            const int gk = k0 + kq;
            const int nvalid = (grow < p.M) ? (p.K - gk) : 0;
            const float* src = p.A + (int64_t)(grow < p.M ? grow : 0) * p.lda + gk;
            ra[i] = load4<VEC>(src, nvalid);
        }
#pragma unroll
        for (int i = 0; i < T::LB; ++i) {
            const int idx = tid + i * T::NT;
            const int kr = idx / T::QB;
            const int nq = (idx % T::QB) * 4;
            const int gk = k0 + kr;
            const int gn = n0 + nq;
            const int nvalid = (gk < p.K) ? (p.N - gn) : 0;
            const float* src = p.B + (int64_t)(gk < p.K ? gk : 0) * p.ldb + gn;
            rb[i] = load4<VEC>(src, nvalid);
        }
    };
    auto store_stage = [&](int s) {
        float* As = smem + s * T::STAGE;
        float* Bs = As + T::A_FLOATS;
#pragma unroll
        for (int i = 0; i < T::LA; ++i) {
            const int idx = tid + i * T::NT;
            const int row = idx / T::QA;
            const int kq = (idx % T::QA) * 4;
            *reinterpret_cast<f32x4*>(As + row * T::LDA_S + kq) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < T::LB; ++i) {
            const int idx = tid + i * T::NT;
            const int kr = idx / T::QB;
            const int nq = (idx % T::QB) * 4;
            *reinterpret_cast<f32x4*>(Bs + kr * T::LDB_S + nq) = rb[i];
        }
    };

    f32x16 acc[T::MB][T::NB];
#pragma unroll
    for (int i = 0; i < T::MB; ++i)
#pragma unroll
        for (int j = 0; j < T::NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Per-lane LDS offsets of the MFMA operands inside one stage.
    const int a_off = (wm * T::TWM + l32) * T::LDA_S + h * (BK / 2);
    const int b_off = T::A_FLOATS + h * (BK / 2) * T::LDB_S + wn * T::TWN + T::NB * l32;

    auto compute_stage = [&](int s) {
        const float* base = smem + s * T::STAGE;
#pragma unroll
        for (int c = 0; c < BK / 8; ++c) {
            f32x4 a[T::MB];
#pragma unroll
            for (int i = 0; i < T::MB; ++i)
                a[i] = *reinterpret_cast<const f32x4*>(base + a_off + i * 32 * T::LDA_S + 4 * c);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float* bp = base + b_off + (4 * c + j) * T::LDB_S;
                float b[T::NB];
                if constexpr (T::NB == 4) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(bp);
                    b[0] = v[0]; b[1] = v[1]; b[2] = v[2]; b[3] = v[3];
                } else if constexpr (T::NB == 2) {
                    const f32x2 v = *reinterpret_cast<const f32x2*>(bp);
                    b[0] = v[0]; b[1] = v[1];
                } else {
                    b[0] = bp[0];
                }
#pragma unroll
                for (int i = 0; i < T::MB; ++i)
#pragma unroll
                    for (int n = 0; n < T::NB; ++n)
                        acc[i][n] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][j], b[n],
                                                                         acc[i][n], 0, 0, 0);
            }
        }
    };

    const int nk = (p.K + BK - 1) / BK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) load_stage((kt + 1) * BK);
        compute_stage(cur);
        if (more) store_stage(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: C <- alpha*acc + beta*C (beta == 0: C not read) ----
    const float alpha = p.alpha, beta = p.beta;
    const int col = n0 + wn * T::TWN + T::NB * l32;
    const int ncols = p.N - col;
#pragma unroll
    for (int i = 0; i < T::MB; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * T::TWM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (row >= p.M || ncols <= 0) continue;
            float* dst = p.C + (int64_t)row * p.ldc + col;
            float v[T::NB];
#pragma unroll
            for (int n = 0; n < T::NB; ++n) v[n] = alpha * acc[i][n][r];
            if (VEC && ncols >= T::NB) {
                if (beta != 0.0f) {
                    if constexpr (T::NB == 4) {
                        const f32x4 c = *reinterpret_cast<const f32x4*>(dst);
                        v[0] += beta * c[0]; v[1] += beta * c[1];
                        v[2] += beta * c[2]; v[3] += beta * c[3];
                    } else if constexpr (T::NB == 2) {
                        const f32x2 c = *reinterpret_cast<const f32x2*>(dst);
                        v[0] += beta * c[0]; v[1] += beta * c[1];
                    } else {
                        v[0] += beta * dst[0];
                    }
                }
                if constexpr (T::NB == 4) {
                    f32x4 o = {v[0], v[1], v[2], v[3]};
                    *reinterpret_cast<f32x4*>(dst) = o;
                } else if constexpr (T::NB == 2) {
                    f32x2 o = {v[0], v[1]};
                    *reinterpret_cast<f32x2*>(dst) = o;
                } else {
                    dst[0] = v[0];
                }
            } else {
#pragma unroll
                for (int n = 0; n < T::NB; ++n) {
                    if (n < ncols) {
                        float o = v[n];
                        if (beta != 0.0f) o += beta * dst[n];
                        dst[n] = o;
                    }
                }
            }
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN, bool VEC>
hipError_t launch_gemm(const GemmArgs& p, hipStream_t stream) {
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
    const dim3 block(64 * WM * WN);
    hipLaunchKernelGGL((sgemm_mfma_kernel<BM, BN, BK, WM, WN, VEC>), grid, block, 0, stream, p);
    return hipGetLastError();
}

#define PHOBOS_CFG(BM, BN, BK, WM, WN)                                                  \
    KernelEntry{sgemm_config{BM, BN, BK, WM, WN}, 64 * WM * WN,                        \
                TileShape<BM, BN, BK, WM, WN>::LDS_BYTES,                               \
                &launch_gemm<BM, BN, BK, WM, WN, true>,                                 \
                &launch_gemm<BM, BN, BK, WM, WN, false>}

// The compiled configurations.  A host function holds the table so that the
// device pass never sees the host launch functions it points to.
const KernelEntry* kernel_table(int* count) {
    static const KernelEntry table[] = {
        PHOBOS_CFG(256, 256, 16, 2, 2),
        PHOBOS_CFG(256, 256, 32, 2, 2),
        PHOBOS_CFG(256, 256, 16, 4, 2),
        PHOBOS_CFG(256, 128, 16, 2, 2),
        PHOBOS_CFG(128, 256, 16, 2, 2),
        PHOBOS_CFG(128, 128, 16, 2, 2),
        PHOBOS_CFG(128, 128, 32, 2, 2),
        PHOBOS_CFG(128, 128, 8, 2, 2),
        PHOBOS_CFG(128, 64, 16, 2, 1),
        PHOBOS_CFG(64, 128, 16, 1, 2),
        PHOBOS_CFG(64, 64, 16, 1, 1),
        PHOBOS_CFG(32, 32, 16, 1, 1),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

// ---------------------------------------------------------------------------
// Init leaf: C <- beta*C, or C <- 0 without reading C when beta == 0.
// HBM-bound: each thread handles one float4 of a row; rows are strided over
// gridDim.y so any M fits the grid limits.
template <bool ZERO, bool VEC>
__global__ __launch_bounds__(256) void init_leaf_kernel(int64_t M, int64_t N, float beta,
                                                        float* C, int64_t ldc) {
    const int64_t col = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (col >= N) return;
    const int64_t left = N - col;
    for (int64_t row = blockIdx.y; row < M; row += gridDim.y) {
        float* p = C + row * ldc + col;
        if (VEC && left >= 4) {
            f32x4 v;
            if (ZERO) {
                v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            } else {
                v = *reinterpret_cast<const f32x4*>(p);
                v[0] *= beta; v[1] *= beta; v[2] *= beta; v[3] *= beta;
            }
            *reinterpret_cast<f32x4*>(p) = v;
        } else {
            for (int e = 0; e < 4 && e < left; ++e) p[e] = ZERO ? 0.0f : beta * p[e];
        }
    }
}

hipError_t launch_init_leaf(int64_t M, int64_t N, float beta, float* C, int64_t ldc,
                            hipStream_t stream) {
    const int64_t quads = (N + 3) / 4;
    const dim3 grid((unsigned)((quads + 255) / 256), (unsigned)(M < 65535 ? M : 65535));
    const dim3 block(256);
    const bool vec = ((uintptr_t)C % 16 == 0) && (ldc % 4 == 0);
    if (beta == 0.0f) {
        if (vec)
            hipLaunchKernelGGL((init_leaf_kernel<true, true>), grid, block, 0, stream, M, N, beta, C, ldc);
        else
            hipLaunchKernelGGL((init_leaf_kernel<true, false>), grid, block, 0, stream, M, N, beta, C, ldc);
    } else {
        if (vec)
            hipLaunchKernelGGL((init_leaf_kernel<false, true>), grid, block, 0, stream, M, N, beta, C, ldc);
        else
            hipLaunchKernelGGL((init_leaf_kernel<false, false>), grid, block, 0, stream, M, N, beta, C, ldc);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tuner scratch fill: a 32-bit integer hash of (index, seed) mapped to [-1, 1).
__global__ __launch_bounds__(256) void fill_pattern_kernel(float* p, int64_t n, uint32_t seed) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * 256) {
        uint32_t x = (uint32_t)i * 0x9E3779B1u ^ seed;
        x ^= x >> 16;
        x *= 0x85EBCA6Bu;
        x ^= x >> 13;
        x *= 0xC2B2AE35u;
        x ^= x >> 16;
        p[i] = (float)(x >> 8) * (1.0f / 8388608.0f) - 1.0f;
    }
}

hipError_t launch_fill_pattern(float* p, int64_t n, uint32_t seed, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_pattern_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, seed);
    return hipGetLastError();
}

}  // namespace phobos
