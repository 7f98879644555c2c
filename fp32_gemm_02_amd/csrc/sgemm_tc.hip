// gfx950 kernels for the matrix-core variant of C <- alpha*A*B + beta*C:
// A, B and C are fp32 in memory; every element of A and B is rounded to a
// 16-bit format (binary16 or bfloat16, round to nearest even) as it is
// loaded, the products are accumulated by the 16-bit matrix instructions
// into fp32 accumulators, and the epilogue is the fp32 one ("Show HN:
// Phobos", section "Are we cuBLAS yet?", the side-quest that casts to fp16
// before the tensor cores and keeps an fp32 accumulator).
//
// One workgroup owns a BM x BN tile of C and walks K in chunks of 32:
//   - global -> registers: 128-bit fp32 loads (bounds-checked, zero fill at
//     the edges), issued one chunk ahead so they overlap the MFMAs;
//   - registers -> LDS: converted with gfx950's packed converts
//     (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32, round to nearest even) and
//     stored as 16-bit values, halving LDS traffic against fp32.  A is stored
//     row-major (k contiguous); B is stored transposed (n-major, k
//     contiguous), which the register pass makes free: a thread holds 8 (or
//     4) rows of k for 4 columns and writes each column's k run at once;
//   - each 64-lane wave owns a TWM x TWN sub-tile of MB x NB blocks of
//     32 x 32, accumulated by v_mfma_f32_32x32x16_{f16,bf16};
//   - two LDS stages, one barrier per chunk.
//
// MFMA 32x32x16 16-bit operand layout (checked on the GPU with an in-bounds
// probe; l = lane, h = l / 32):
//   src A: lane l holds A'[l % 32][8h + e], e = 0..7  (one 16-byte LDS read)
//   src B: lane l holds B'[8h + e][l % 32], e = 0..7  (one 16-byte LDS read of
//          the transposed tile)
//   acc  : lane l, register r holds D[8*(r/4) + 4h + r%4][l % 32]
// LDS rows are 32 halves = 64 bytes = 4 pieces of 16 bytes, XOR-swizzled by
// row (swz<4>) so the 32-row operand reads are free of bank conflicts.  As in
// the fp32 kernel, block nb of a wave holds the columns NB*j + nb (j =
// 0..31): the B tile's LDS rows are written in that interleaved order, and
// the epilogue stores NB consecutive columns of C at once.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgemm_device.h"
#include "sgemm_internal.h"

namespace phobos {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int FMT> struct TcFmt;

template <> struct TcFmt<SGEMM_TC_F16> {
    typedef _Float16 x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 x8 __attribute__((ext_vector_type(8)));
    // lo -> bits 0..15 (the lower k), hi -> bits 16..31
    static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
        const x2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(x8, a),
                                                      __builtin_bit_cast(x8, b), c, 0, 0, 0);
    }
};

template <> struct TcFmt<SGEMM_TC_BF16> {
    typedef __bf16 x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 x8 __attribute__((ext_vector_type(8)));
    static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
        const x2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(x8, a),
                                                       __builtin_bit_cast(x8, b), c, 0, 0, 0);
    }
};

template <int BM, int BN, int WM, int WN>
struct TcShape {
    static constexpr int NT = 64 * WM * WN;      // threads
    static constexpr int BK = 32;                // k per chunk: two MFMA k-steps
    static constexpr int TWM = BM / WM, TWN = BN / WN;
    static constexpr int MB = TWM / 32, NB = TWN / 32;
    static constexpr int ROWB = BK * 2;          // bytes of one LDS row (16-bit values)
    static constexpr int UA = BM * 4 / NT;       // A units (8 k of one row) per thread
    static constexpr int KB = (BN % NT == 0) ? 8 : 4;   // k rows of one B unit
    static constexpr int QB = BN / 4;            // column quads of the tile
    static constexpr int UB = QB * (BK / KB) / NT;      // B units per thread
    static constexpr int STAGE = (BM + BN) * ROWB;
    static constexpr int LDS_BYTES = 2 * STAGE;
    static_assert(TWM % 32 == 0 && TWN % 32 == 0, "whole 32 x 32 blocks per wave");
    static_assert(NB == 1 || NB == 2 || NB == 4, "NB-wide epilogue stores");
    static_assert(UA >= 1 && UA * NT == BM * 4, "whole A units per thread");
    static_assert(UB >= 1 && UB * NT == QB * (BK / KB), "whole B units per thread");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS of one CU");
};

template <int FMT, int BM, int BN, int WM, int WN, bool VEC>
__global__ __launch_bounds__(64 * WM * WN) void sgemm_tc_kernel(GemmArgs p) {
    using F = TcFmt<FMT>;
    using T = TcShape<BM, BN, WM, WN>;
    constexpr int NT = T::NT, BK = T::BK, ROWB = T::ROWB, UA = T::UA, UB = T::UB, KB = T::KB,
                  QB = T::QB, MB = T::MB, NB = T::NB, TWM = T::TWM, TWN = T::TWN;
    __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31, h = lane >> 5;
    int tm, tn;
    tile_of(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = (p.K + BK - 1) / BK;

    f32x4 ra[UA][2];    // A: 8 consecutive k of one row per unit
    f32x4 rb[UB][KB];   // B: KB rows of k, 4 consecutive columns per unit

    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < UA; ++i) {
            const int u = t + i * NT, row = u >> 2, oct = u & 3;
            const int gr = m0 + row, gk = k0 + 8 * oct;
            if (gr < p.M) {
                const float* src = p.A + (int64_t)gr * p.lda + gk;
                ra[i][0] = load4<VEC>(src, p.K - gk);
                ra[i][1] = load4<VEC>(src + 4, p.K - gk - 4);
            } else {
                ra[i][0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                ra[i][1] = ra[i][0];
            }
        }
#pragma unroll
        for (int i = 0; i < UB; ++i) {
            const int u = t + i * NT, q = u % QB, grp = u / QB;
            const int gc = n0 + 4 * q, gk = k0 + KB * grp;
            const int ncols = p.N - gc;
#pragma unroll
            for (int r = 0; r < KB; ++r) {
                const int k = gk + r;
                rb[i][r] = (k < p.K) ? load4<VEC>(p.B + (int64_t)k * p.ldb + gc, ncols)
                                     : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
    };

    auto store = [&](int stage) {
        char* sa = lds + stage * T::STAGE;
        char* sb = sa + BM * ROWB;
#pragma unroll
        for (int i = 0; i < UA; ++i) {
            const int u = t + i * NT, row = u >> 2, oct = u & 3;
            const u32x4 v = {F::pack(ra[i][0][0], ra[i][0][1]), F::pack(ra[i][0][2], ra[i][0][3]),
                             F::pack(ra[i][1][0], ra[i][1][1]), F::pack(ra[i][1][2], ra[i][1][3])};
            *reinterpret_cast<u32x4*>(sa + row * ROWB + 16 * (oct ^ swz<4>(row))) = v;
        }
#pragma unroll
        for (int i = 0; i < UB; ++i) {
            const int u = t + i * NT, q = u % QB, grp = u / QB;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                // tile column 4q + c lands on the interleaved LDS row of its wave
                const int col = 4 * q + c, wcol = col % TWN;
                const int lrow = (col - wcol) + (wcol % NB) * 32 + wcol / NB;
                char* rowp = sb + lrow * ROWB;
                if constexpr (KB == 8) {
                    const u32x4 v = {F::pack(rb[i][0][c], rb[i][1][c]), F::pack(rb[i][2][c], rb[i][3][c]),
                                     F::pack(rb[i][4][c], rb[i][5][c]), F::pack(rb[i][6][c], rb[i][7][c])};
                    *reinterpret_cast<u32x4*>(rowp + 16 * (grp ^ swz<4>(lrow))) = v;
                } else {
                    const u32x2 v = {F::pack(rb[i][0][c], rb[i][1][c]), F::pack(rb[i][2][c], rb[i][3][c])};
                    *reinterpret_cast<u32x2*>(rowp + 16 * ((grp >> 1) ^ swz<4>(lrow)) + 8 * (grp & 1)) = v;
                }
            }
        }
    };

    // lane l's operand of block row `row` (A) or interleaved row `row` (B) at
    // MFMA k-step s of the chunk: 8 values at k = 16s + 8h
    auto frag = [&](const char* base, int row, int s) -> u32x4 {
        return *reinterpret_cast<const u32x4*>(base + row * ROWB + 16 * ((2 * s + h) ^ swz<4>(row)));
    };

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    load(0);
    store(0);
    __syncthreads();
    for (int c = 0; c < nk; ++c) {
        const bool more = c + 1 < nk;
        if (more) load((c + 1) * BK);   // in flight during this chunk's MFMAs
        const char* sa = lds + (c & 1) * T::STAGE;
        const char* sb = sa + BM * ROWB;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            u32x4 fa[MB], fb[NB];
#pragma unroll
            for (int i = 0; i < MB; ++i) fa[i] = frag(sa, wm * TWM + i * 32 + l32, s);
#pragma unroll
            for (int j = 0; j < NB; ++j) fb[j] = frag(sb, wn * TWN + j * 32 + l32, s);
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j) acc[i][j] = F::mma(fa[i], fb[j], acc[i][j]);
        }
        // the other stage was last read before the previous barrier
        if (more) store((c + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: C <- alpha*acc + beta*C (beta == 0: C not read) ----
    const float alpha = p.alpha, beta = p.beta;
    const int col = n0 + wn * TWN + NB * l32;
    const int ncols = p.N - col;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * TWM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (row >= p.M || ncols <= 0) continue;
            float* dst = p.C + (int64_t)row * p.ldc + col;
            float v[NB];
#pragma unroll
            for (int n = 0; n < NB; ++n) v[n] = alpha * acc[i][n][r];
            if (VEC && ncols >= NB) {
                if constexpr (NB == 4) {
                    if (beta != 0.0f) {
                        const f32x4 cv = *reinterpret_cast<const f32x4*>(dst);
                        v[0] += beta * cv[0]; v[1] += beta * cv[1];
                        v[2] += beta * cv[2]; v[3] += beta * cv[3];
                    }
                    *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
                } else if constexpr (NB == 2) {
                    if (beta != 0.0f) {
                        const f32x2 cv = *reinterpret_cast<const f32x2*>(dst);
                        v[0] += beta * cv[0]; v[1] += beta * cv[1];
                    }
                    *reinterpret_cast<f32x2*>(dst) = f32x2{v[0], v[1]};
                } else {
                    if (beta != 0.0f) v[0] += beta * dst[0];
                    dst[0] = v[0];
                }
            } else {
#pragma unroll
                for (int n = 0; n < NB; ++n) {
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

template <int FMT, int BM, int BN, int WM, int WN, bool VEC>
hipError_t launch_tc(const GemmArgs& p, hipStream_t stream) {
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
    const dim3 block(64 * WM * WN);
    hipLaunchKernelGGL((sgemm_tc_kernel<FMT, BM, BN, WM, WN, VEC>), grid, block, 0, stream, p);
    return hipGetLastError();
}

#define PHOBOS_TC_CFG(FMT, BM, BN, WM, WN)                                              \
    KernelEntry{sgemm_config{BM, BN, 32, WM, WN}, 64 * WM * WN,                        \
                TcShape<BM, BN, WM, WN>::LDS_BYTES,                                     \
                &launch_tc<FMT, BM, BN, WM, WN, true>,                                  \
                &launch_tc<FMT, BM, BN, WM, WN, false>}

#define PHOBOS_TC_TABLE(FMT)                                                            \
    {                                                                                   \
        PHOBOS_TC_CFG(FMT, 256, 256, 2, 2), PHOBOS_TC_CFG(FMT, 256, 256, 4, 2),         \
            PHOBOS_TC_CFG(FMT, 256, 128, 2, 2), PHOBOS_TC_CFG(FMT, 128, 256, 2, 2),     \
            PHOBOS_TC_CFG(FMT, 128, 128, 2, 2), PHOBOS_TC_CFG(FMT, 128, 64, 2, 1),      \
            PHOBOS_TC_CFG(FMT, 64, 64, 1, 1),                                           \
    }

// The compiled configurations of the matrix-core variant, per input format
// (bk is always 32); nullptr for an unknown format.
const KernelEntry* tc_kernel_table(int fmt, int* count) {
    static const KernelEntry f16[] = PHOBOS_TC_TABLE(SGEMM_TC_F16);
    static const KernelEntry bf16[] = PHOBOS_TC_TABLE(SGEMM_TC_BF16);
    *count = (int)(sizeof(f16) / sizeof(f16[0]));
    if (fmt == SGEMM_TC_F16) return f16;
    if (fmt == SGEMM_TC_BF16) return bf16;
    *count = 0;
    return nullptr;
}

}  // namespace phobos
