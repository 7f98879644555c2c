// gfx950 kernels for the matrix-core variant of C <- alpha*A*B + beta*C:
// A, B and C are fp32 in memory; every element of A and B is rounded to a
// 16-bit format (binary16 or bfloat16, round to nearest even) as it is
// loaded, the products are accumulated by the 16-bit matrix instructions
// into fp32 accumulators, and the epilogue is the fp32 one ("Show HN:
// Phobos", section "Are we cuBLAS yet?", the side-quest that casts to fp16
// before the tensor cores and keeps an fp32 accumulator).
//
// One workgroup owns a BM x BN tile of C and walks K in chunks of BK (32 or
// 64, i.e. 2 or 4 MFMA k-steps):
//   - global -> registers: 128-bit fp32 loads (bounds-checked, zero fill at
//     the edges), issued a whole chunk ahead so they overlap the MFMAs;
//   - registers -> LDS: converted with gfx950's packed converts
//     (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32, round to nearest even) and
//     stored as 16-bit values, halving LDS traffic against fp32.  A is stored
//     row-major (k contiguous); B is stored transposed (n-major, k
//     contiguous), which the register pass makes free: a thread holds 8 (or
//     4) rows of k for 4 columns and writes each column's k run at once;
//   - each 64-lane wave owns a TWM x TWN sub-tile of MB x NB blocks of
//     32 x 32, accumulated by v_mfma_f32_32x32x16_{f16,bf16};
//   - two LDS stages, one barrier per chunk, placed before the last k-step's
//     MFMAs so that those overlap the barrier and the next chunk's first
//     operand reads; operands are read one k-step ahead of their MFMAs.
//
// MFMA 32x32x16 16-bit operand layout (checked on the GPU with an in-bounds
// probe; l = lane, h = l / 32):
//   src A: lane l holds A'[l % 32][8h + e], e = 0..7  (one 16-byte LDS read)
//   src B: lane l holds B'[8h + e][l % 32], e = 0..7  (one 16-byte LDS read of
//          the transposed tile)
//   acc  : lane l, register r holds D[8*(r/4) + 4h + r%4][l % 32]
// LDS rows are BK halves = 4 or 8 pieces of 16 bytes, XOR-swizzled by row
// (swz<4> / swz<8>) so the 32-row operand reads are free of bank conflicts.  As in
// the fp32 kernel, block nb of a wave holds the columns NB*j + nb (j =
// 0..31): the B tile's LDS rows are written in that interleaved order, and
// the epilogue stores NB consecutive columns of C at once.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "sgemm_device.h"
#include "sgemm_internal.h"

// The staged form's 16-bit workspace for callers that cannot allocate
// (sgemm_tc_noalloc): a static device array of SGEMM_TC_SCRATCH_BYTES that
// every GPU the library runs on holds from the module's load until the
// process ends.  Host code never uses this name as an address (on the host
// it is only a stand-in for the symbol): tc_scratch() below looks up its
// device address once per device and hands that out.
static __device__ __align__(256) uint16_t scratch[SGEMM_TC_SCRATCH_BYTES / sizeof(uint16_t)];

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

template <int BM, int BN, int BK_, int WM, int WN>
struct TcShape {
    static constexpr int NT = 64 * WM * WN;      // threads
    static constexpr int BK = BK_;               // k per chunk: BK/16 MFMA k-steps
    static constexpr int KS = BK / 16;
    static constexpr int TWM = BM / WM, TWN = BN / WN;
    static constexpr int MB = TWM / 32, NB = TWN / 32;
    static constexpr int ROWB = BK * 2;          // bytes of one LDS row (16-bit values)
    static constexpr int PR = ROWB / 16;         // 16-byte pieces per LDS row
    static constexpr int OA = BK / 8;            // A units (8 k of one row) per row
    static constexpr int UA = BM * OA / NT;      // A units per thread
    static constexpr int QB = BN / 4;            // column quads of the tile
    static constexpr int KB = (QB * (BK / 8)) % NT == 0 ? 8 : 4;   // k rows of one B unit
    static constexpr int UB = QB * (BK / KB) / NT;                 // B units per thread
    static constexpr int STAGE = (BM + BN) * ROWB;
    static constexpr int LDS_BYTES = 2 * STAGE;
    static_assert(BK == 32 || BK == 64, "4 or 8 pieces per LDS row");
    static_assert(TWM % 32 == 0 && TWN % 32 == 0, "whole 32 x 32 blocks per wave");
    static_assert(NB == 1 || NB == 2 || NB == 4, "NB-wide epilogue stores");
    static_assert(UA >= 1 && UA * NT == BM * OA, "whole A units per thread");
    static_assert(UB >= 1 && UB * NT == QB * (BK / KB), "whole B units per thread");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS of one CU");
};

template <int FMT, int BM, int BN, int BK_, int WM, int WN, int PF, bool VEC>
__global__ __launch_bounds__(64 * WM * WN) void sgemm_tc_kernel(GemmArgs p) {
    using F = TcFmt<FMT>;
    using T = TcShape<BM, BN, BK_, WM, WN>;
    constexpr int NT = T::NT, BK = T::BK, KS = T::KS, ROWB = T::ROWB, PR = T::PR, OA = T::OA,
                  UA = T::UA, UB = T::UB, KB = T::KB, QB = T::QB, MB = T::MB, NB = T::NB,
                  TWM = T::TWM, TWN = T::TWN;
    __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31, h = lane >> 5;
    int tm, tn;
    tile_of(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = (p.K + BK - 1) / BK;

    // PF sets of staging registers: chunk j >= 1 is loaded into set (j-1) % PF
    f32x4 ra[PF][UA][2];    // A: 8 consecutive k of one row per unit
    f32x4 rb[PF][UB][KB];   // B: KB rows of k, 4 consecutive columns per unit

    // Interior chunks (the whole tile inside M and N, the chunk inside K,
    // 16-byte aligned operands) load without bounds checks through pointers
    // set up once; the checked path below serves the edges.  The test is
    // uniform over the workgroup, so the choice is a scalar branch.
    const bool tile_inside = VEC && m0 + BM <= p.M && n0 + BN <= p.N;
    const float* pa[UA];
    const float* pb[UB];
#pragma unroll
    for (int i = 0; i < UA; ++i) {
        const int u = t + i * NT;
        pa[i] = p.A + (int64_t)(m0 + u / OA) * p.lda + 8 * (u % OA);
    }
#pragma unroll
    for (int i = 0; i < UB; ++i) {
        const int u = t + i * NT;
        pb[i] = p.B + (int64_t)(KB * (u / QB)) * p.ldb + n0 + 4 * (u % QB);
    }

    auto load = [&](int k0, auto set) {
        if (tile_inside && k0 + BK <= p.K) {
#pragma unroll
            for (int i = 0; i < UA; ++i) {
                ra[set][i][0] = *reinterpret_cast<const f32x4*>(pa[i] + k0);
                ra[set][i][1] = *reinterpret_cast<const f32x4*>(pa[i] + k0 + 4);
            }
#pragma unroll
            for (int i = 0; i < UB; ++i) {
                const float* src = pb[i] + (int64_t)k0 * p.ldb;
#pragma unroll
                for (int r = 0; r < KB; ++r)
                    rb[set][i][r] = *reinterpret_cast<const f32x4*>(src + (int64_t)r * p.ldb);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < UA; ++i) {
            const int u = t + i * NT, row = u / OA, oct = u % OA;
            const int gr = m0 + row, gk = k0 + 8 * oct;
            if (gr < p.M) {
                const float* src = p.A + (int64_t)gr * p.lda + gk;
                ra[set][i][0] = load4<VEC>(src, p.K - gk);
                ra[set][i][1] = load4<VEC>(src + 4, p.K - gk - 4);
            } else {
                ra[set][i][0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                ra[set][i][1] = ra[set][i][0];
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
                rb[set][i][r] = (k < p.K) ? load4<VEC>(p.B + (int64_t)k * p.ldb + gc, ncols)
                                          : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
    };

    auto store = [&](int stage, auto set) {
        char* sa = lds + stage * T::STAGE;
        char* sb = sa + BM * ROWB;
#pragma unroll
        for (int i = 0; i < UA; ++i) {
            const int u = t + i * NT, row = u / OA, oct = u % OA;
            const f32x4 a0 = ra[set][i][0], a1 = ra[set][i][1];
            const u32x4 v = {F::pack(a0[0], a0[1]), F::pack(a0[2], a0[3]), F::pack(a1[0], a1[1]),
                             F::pack(a1[2], a1[3])};
            *reinterpret_cast<u32x4*>(sa + row * ROWB + 16 * (oct ^ swz<PR>(row))) = v;
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
                const auto& b = rb[set][i];
                if constexpr (KB == 8) {
                    const u32x4 v = {F::pack(b[0][c], b[1][c]), F::pack(b[2][c], b[3][c]),
                                     F::pack(b[4][c], b[5][c]), F::pack(b[6][c], b[7][c])};
                    *reinterpret_cast<u32x4*>(rowp + 16 * (grp ^ swz<PR>(lrow))) = v;
                } else {
                    const u32x2 v = {F::pack(b[0][c], b[1][c]), F::pack(b[2][c], b[3][c])};
                    *reinterpret_cast<u32x2*>(rowp + 16 * ((grp >> 1) ^ swz<PR>(lrow)) + 8 * (grp & 1)) = v;
                }
            }
        }
    };

    // lane l's operand of block row `row` (A) or interleaved row `row` (B) at
    // MFMA k-step s of the chunk: 8 values at k = 16s + 8h
    auto frag = [&](const char* base, int row, int s) -> u32x4 {
        return *reinterpret_cast<const u32x4*>(base + row * ROWB + 16 * ((2 * s + h) ^ swz<PR>(row)));
    };
    u32x4 fa[2][MB], fb[2][NB];
    auto read_step = [&](int stage, int s, int buf) {
        const char* sa = lds + stage * T::STAGE;
        const char* sb = sa + BM * ROWB;
#pragma unroll
        for (int i = 0; i < MB; ++i) fa[buf][i] = frag(sa, wm * TWM + i * 32 + l32, s);
#pragma unroll
        for (int j = 0; j < NB; ++j) fb[buf][j] = frag(sb, wn * TWN + j * 32 + l32, s);
    };

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Pipeline: while chunk c is computed from LDS, the registers hold (or
    // are receiving) chunks c+1 .. c+PF.  At the last k-step of chunk c the
    // set holding chunk c+1 goes to the other LDS stage, the barrier follows,
    // the loads of chunk c+1+PF are issued into the set just emptied and the
    // first operands of chunk c+1 are read; only then are the last k-step's
    // MFMAs issued, so they overlap all of that.  Loads thus have PF whole
    // chunks to land.  The stage written at chunk c was last read during
    // chunk c-1, before that chunk's barrier.
    using S0 = std::integral_constant<int, 0>;
    load(0, S0{});
    store(0, S0{});
    if (nk > 1) load(BK, S0{});
    if constexpr (PF == 2) {
        if (nk > 2) load(2 * BK, std::integral_constant<int, 1>{});
    }
    __syncthreads();
    read_step(0, 0, 0);
    auto chunk = [&](int c, auto set) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s + 1 < KS) {
                read_step(c & 1, s + 1, (s + 1) & 1);
            } else if (c + 1 < nk) {
                store((c + 1) & 1, set);
                __syncthreads();
                if (c + 1 + PF < nk) load((c + 1 + PF) * BK, set);
                read_step((c + 1) & 1, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j) acc[i][j] = F::mma(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int c = 0; c < nk; c += PF) {
        chunk(c, S0{});
        if constexpr (PF == 2) {
            if (c + 1 < nk) chunk(c + 1, std::integral_constant<int, 1>{});
        }
    }

    // ---- epilogue: C <- alpha*acc + beta*C (beta == 0: C not read) ----
    // Every tile through edge_block_epilogue: several rows of C per block
    // read before any is written, with unguarded reads clamped into C.
    const float alpha = p.alpha, beta = p.beta;
    const int col = n0 + wn * TWN + NB * l32;
    constexpr int RB = MB * NB * 16 >= 256 ? 4 : 16;   // rows per batch
#pragma unroll
    for (int i = 0; i < MB; ++i)
        edge_block_epilogue<NB, RB>(p.C, p.ldc, p.M, p.N, m0 + wm * TWM + i * 32 + 4 * h, col, alpha,
                                    beta, [&](int n, int r) { return acc[i][n][r]; });
}

template <int FMT, int BM, int BN, int BK, int WM, int WN, int PF, bool VEC>
hipError_t launch_tc(const GemmArgs& p, hipStream_t stream) {
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
    const dim3 block(64 * WM * WN);
    hipLaunchKernelGGL((sgemm_tc_kernel<FMT, BM, BN, BK, WM, WN, PF, VEC>), grid, block, 0,
                       stream, p);
    return hipGetLastError();
}

#ifndef PHOBOS_TC_PF
#define PHOBOS_TC_PF 1
#endif

#define PHOBOS_TC_CFG(FMT, BM, BN, BK, WM, WN)                                          \
    KernelEntry{sgemm_config{BM, BN, BK, WM, WN}, 64 * WM * WN,                        \
                TcShape<BM, BN, BK, WM, WN>::LDS_BYTES,                                 \
                &launch_tc<FMT, BM, BN, BK, WM, WN, PHOBOS_TC_PF, true>,                \
                &launch_tc<FMT, BM, BN, BK, WM, WN, PHOBOS_TC_PF, false>}

#define PHOBOS_TC_TABLE(FMT)                                                            \
    {                                                                                   \
        PHOBOS_TC_CFG(FMT, 256, 256, 32, 2, 2), PHOBOS_TC_CFG(FMT, 256, 256, 32, 4, 2), \
            PHOBOS_TC_CFG(FMT, 256, 128, 32, 2, 2), PHOBOS_TC_CFG(FMT, 128, 256, 32, 2, 2), \
            PHOBOS_TC_CFG(FMT, 128, 128, 32, 2, 2), PHOBOS_TC_CFG(FMT, 128, 128, 64, 2, 2), \
            PHOBOS_TC_CFG(FMT, 128, 64, 32, 2, 1), PHOBOS_TC_CFG(FMT, 64, 64, 32, 1, 1),  \
    }

// ---------------------------------------------------------------------------
// Staged form of the variant: the rounding is done once, by a cast pass, into
// a 16-bit workspace laid out for the GEMM (A row-major, B transposed, both k
// contiguous, zero-padded to whole tiles and whole K chunks); the GEMM then
// streams 16-bit operands straight into LDS with direct loads.  Each element
// is rounded by the same conversion as in the fused form, so the products
// and their order are the same.

// A16[i][k] = round(A[i][k]) for i < M, k < K, 0 elsewhere in Mp x Kp.  One
// thread per 8 consecutive k of a row (two 16-byte loads, one 16-byte store).
template <int FMT, bool VEC>
__global__ __launch_bounds__(256) void tc_cast_rows_kernel(const float* A, int64_t lda, int M,
                                                           int K, uint16_t* out, int Mp, int Kp) {
    using F = TcFmt<FMT>;
    const int64_t per_row = Kp / 8, total = (int64_t)Mp * per_row;
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < total;
         u += (int64_t)gridDim.x * 256) {
        const int i = (int)(u / per_row), k = 8 * (int)(u % per_row);
        f32x4 a0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, a1 = a0;
        if (i < M) {
            const float* src = A + (int64_t)i * lda + k;
            a0 = load4<VEC>(src, K - k);
            a1 = load4<VEC>(src + 4, K - k - 4);
        }
        const u32x4 v = {F::pack(a0[0], a0[1]), F::pack(a0[2], a0[3]), F::pack(a1[0], a1[1]),
                         F::pack(a1[2], a1[3])};
        *reinterpret_cast<u32x4*>(out + (int64_t)i * Kp + k) = v;
    }
}

// B16[n][k] = round(B[k][n]) for k < K, n < N, 0 elsewhere in Np x Kp: a
// 64 (k) x 128 (n) transpose through LDS per workgroup step, tiles taken n
// first.  Reads take 512 contiguous bytes of a row of B, writes 128 bytes of
// a row of B16, both 16 bytes per lane.  (64 x 64 tiles ran 12% slower at
// 16384 x 16384; taller tiles or banded tile orders did not help either.)
// The tile sits in LDS unpadded, as 16-byte pieces; piece q of row r is kept
// at q ^ ((r >> 3) & 7).  A column read (8 rows o..o+7 of one n per lane, o
// a multiple of 8, 8 n per wave, 4-byte reads) is served 32 lanes at a time
// from 32 banks of 4 bytes, as the counters show: the 32 lanes of a half
// wave (rows 8m+i for m = 0..7, four consecutive n) then take 8 different
// pieces mod 8 and 4 words of each, 32 different banks.  (The swizzle
// 2*((r >> 3) & 7) gave 64 different words mod 256 bytes per wave but put
// rows m and m ^ 4 of a half wave on the same banks: half of the read cycles
// were conflicts.)  A tile wholly inside B (16-byte aligned rows, offsets in 32
// bits) comes in by direct global-to-LDS loads: each wave's load fills 64
// consecutive 16-byte slots, two rows, the swizzle applied to the global
// address of each slot.  Edge tiles go through registers with bounds checks
// and zero fill and are stored with one 16-byte write per lane.  (Stored
// through registers, every tile spent a third of its LDS cycles in bank
// conflicts on those writes, at 8 conflict cycles per 16-byte write of a
// wave; the direct loads write no LDS through the LDS pipe.)
template <int FMT, bool VEC>
__global__ __launch_bounds__(256) void tc_cast_cols_kernel(const float* B, int64_t ldb, int K,
                                                           int N, uint16_t* out, int Np, int Kp) {
    using F = TcFmt<FMT>;
    constexpr int TK = 64, TN = 128;
    constexpr int LPR = TN / 4, RPP = 256 / LPR, UPR = TK / 8;   // lanes per row, rows per pass
    constexpr int DL = TK * LPR / 256;                           // direct loads per wave
    static_assert(kTcPadMN % TN == 0 && kTcPadK % TK == 0, "whole tiles of the padded B16");
    static_assert(DL * 256 == TK * LPR, "whole direct loads per wave");
    __shared__ __attribute__((aligned(16))) f32x4 t[TK][TN / 4];
    const float* tf = reinterpret_cast<const float*>(&t[0][0]);
    auto piece = [](int r, int q) { return q ^ ((r >> 3) & 7); };
    auto at = [&](int r, int n) { return tf[r * TN + 4 * piece(r, n >> 2) + (n & 3)]; };
    const int tn = Np / TN, tk = Kp / TK;
    const int64_t tiles = (int64_t)tn * tk;
    const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
    const bool narrow = ((int64_t)(TK - 1) * ldb + TN) * 4 <= (int64_t)UINT32_MAX;
    for (int64_t b = blockIdx.x; b < tiles; b += gridDim.x) {
        const int n0 = (int)(b % tn) * TN, k0 = (int)(b / tn) * TK;
        if (VEC && narrow && k0 + TK <= K && n0 + TN <= N) {
            // slot u = (j*4 + wave)*64 + lane holds row u / LPR, stored piece
            // u % LPR, i.e. logical piece (u % LPR) ^ swizzle(row)
            const float* base = B + (int64_t)k0 * ldb + n0;
#pragma unroll
            for (int j = 0; j < DL; ++j) {
                const int u = (j * 4 + wave) * 64 + lane, r = u / LPR;
                const uint32_t off = ((uint32_t)r * (uint32_t)ldb + 4u * (uint32_t)piece(r, u % LPR)) * 4u;
                dma16s(base, off, reinterpret_cast<char*>(&t[0][0]) + (j * 4 + wave) * 1024);
            }
            __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
        } else {
#pragma unroll
            for (int pass = 0; pass < TK / RPP; ++pass) {
                const int kr = RPP * pass + (int)threadIdx.x / LPR, q = (int)threadIdx.x % LPR;
                const int k = k0 + kr, n = n0 + 4 * q;
                t[kr][piece(kr, q)] = (k < K) ? load4<VEC>(B + (int64_t)k * ldb + n, N - n)
                                              : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < TN * UPR / 256; ++j) {
            const int u = (int)threadIdx.x + 256 * j, n = u / UPR, o = 8 * (u % UPR);
            const u32x4 v = {F::pack(at(o, n), at(o + 1, n)), F::pack(at(o + 2, n), at(o + 3, n)),
                             F::pack(at(o + 4, n), at(o + 5, n)), F::pack(at(o + 6, n), at(o + 7, n))};
            *reinterpret_cast<u32x4*>(out + (int64_t)(n0 + n) * Kp + k0 + o) = v;
        }
        __syncthreads();
    }
}

template <int BM, int BN, int BK, int NS, int WM, int WN>
struct Tc16Shape {
    static constexpr int NW = WM * WN, NT = 64 * NW;
    static constexpr int KS = BK / 16;           // MFMA k-steps per chunk
    static constexpr int TWM = BM / WM, TWN = BN / WN;
    static constexpr int MB = TWM / 32, NB = TWN / 32;
    static constexpr int ROWB = BK * 2, PR = ROWB / 16;
    static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB, STAGE = A_BYTES + B_BYTES;
    // NS == 5: a ring of five one-operand slots (A and B of a chunk apart)
    static constexpr bool SPLIT = NS == 5;
    static constexpr int LDS_BYTES = SPLIT ? 5 * A_BYTES : NS * STAGE;
    static constexpr int DA = A_BYTES / 1024 / NW, DB = B_BYTES / 1024 / NW;   // per wave
    static constexpr int D = DA + DB;
    static_assert(BK == 32 || BK == 64, "4 or 8 pieces per LDS row");
    static_assert(KS % 2 == 0, "operand double buffer returns to slot 0 each chunk");
    static_assert(NS >= 2 && NS <= 5, "ring depth");
    static_assert(!SPLIT || A_BYTES == B_BYTES, "one slot size");
    static_assert(DA * 1024 * NW == A_BYTES && DB * 1024 * NW == B_BYTES, "whole loads per wave");
    static_assert(TWM % 32 == 0 && TWN % 32 == 0 && (NB == 1 || NB == 2 || NB == 4), "wave tile");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS of one CU");
    static_assert((SPLIT ? DA : (NS - 2) * D) <= 63, "s_waitcnt vmcnt range");
};

// s_waitcnt for at most n outstanding direct loads (n a multiple of d, at
// most 2d) and every LDS access, then the workgroup barrier.  The barrier is
// issued as assembly with a memory clobber: the compiler's own barrier would
// first wait for every outstanding load, draining the ring.
template <int D>
__device__ __forceinline__ void wait_loads_and_barrier(int later) {
    if (later <= 0)
        __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
    else if (later == 1)
        __builtin_amdgcn_s_waitcnt(kWaitVm<D>);
    else
        __builtin_amdgcn_s_waitcnt(kWaitVm<2 * D>);
    asm volatile("s_barrier" ::: "memory");
}

template <int FMT, int BM, int BN, int BK, int NS, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void tc16_kernel(Tc16Args p) {
    using F = TcFmt<FMT>;
    using T = Tc16Shape<BM, BN, BK, NS, WM, WN>;
    constexpr int NW = T::NW, KS = T::KS, ROWB = T::ROWB, PR = T::PR, MB = T::MB, NB = T::NB,
                  TWM = T::TWM, TWN = T::TWN, DA = T::DA, DB = T::DB;
    __shared__ __attribute__((aligned(1024))) char lds[T::LDS_BYTES];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31, h = lane >> 5;
    int tm, tn;
    tile_of(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = p.K / BK;   // K is padded to whole chunks

    // Direct load j of this wave fills the 64 consecutive 16-byte slots
    // (j*NW + wave)*64 .. +63 of the tile; slot g holds row g / PR, stored
    // piece g % PR, i.e. logical piece (g % PR) ^ swz(row) (8 k values).  B's
    // LDS rows are in the interleaved column order of the epilogue.
    // Byte offsets from the chunk's first row (A) or column (B) of the tile;
    // the host checks that (BM-1)*ld + BK and (BN-1)*ld + BK 16-bit values
    // fit in 32-bit byte offsets.
    uint32_t da[DA], db[DB];
#pragma unroll
    for (int j = 0; j < DA; ++j) {
        const int g = (j * NW + wave) * 64 + lane, row = g / PR;
        da[j] = (uint32_t)(((int64_t)row * p.ld + 8 * ((g % PR) ^ swz<PR>(row))) * 2);
    }
#pragma unroll
    for (int j = 0; j < DB; ++j) {
        const int g = (j * NW + wave) * 64 + lane, lr = g / PR;
        const int u = lr % TWN, n = (lr - u) + NB * (u % 32) + u / 32;
        db[j] = (uint32_t)(((int64_t)n * p.ld + 8 * ((g % PR) ^ swz<PR>(lr))) * 2);
    }
    auto issue = [&](int kc, int buf) {
        char* As = lds + buf * T::STAGE;
        char* Bs = As + T::A_BYTES;
        const int64_t k0 = (int64_t)kc * BK;
        const uint16_t* a0 = p.A + (int64_t)m0 * p.ld + k0;
        const uint16_t* b0 = p.B + (int64_t)n0 * p.ld + k0;
#pragma unroll
        for (int j = 0; j < DA; ++j) dma16s(a0, da[j], As + (j * NW + wave) * 1024);
#pragma unroll
        for (int j = 0; j < DB; ++j) dma16s(b0, db[j], Bs + (j * NW + wave) * 1024);
    };

    u32x4 fa[2][MB], fb[2][NB];
    auto frag = [&](const char* base, int row, int s) -> u32x4 {
        return *reinterpret_cast<const u32x4*>(base + row * ROWB + 16 * ((2 * s + h) ^ swz<PR>(row)));
    };
    auto read_step = [&](int buf, int s, int slot) {
        const char* As = lds + buf * T::STAGE;
        const char* Bs = As + T::A_BYTES;
#pragma unroll
        for (int i = 0; i < MB; ++i) fa[slot][i] = frag(As, wm * TWM + i * 32 + l32, s);
#pragma unroll
        for (int j = 0; j < NB; ++j) fb[slot][j] = frag(Bs, wn * TWN + j * 32 + l32, s);
    };

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // NS of 2 to 4: a ring of NS buffers of whole chunks (NS == 5 is the
    // split ring below); chunk c lives in buffer c % NS.  Chunk c+NS-1 is
    // loaded during chunk c into the buffer chunk c-1 used (every wave
    // finished reading it before the barrier that ended chunk c-1).  The
    // barrier that ends chunk c comes after the first MFMA of its last
    // k-step, once chunk c+1 has landed: loads complete in issue order, so it
    // is enough that at most the loads of the chunks issued after c+1 are
    // still outstanding.
    //
    // Between MFMAs: each MFMA is followed by at most one fragment read (for
    // the next k-step), one direct load (the chunk's loads follow its first
    // MFMAs, as early as possible) and, at the last k-step, the barrier.
    // Each is issued while the MFMA before it runs, and the stage loop is
    // straight-line code, so the compiler's LDS waits are exact.
    constexpr int MF = MB * NB;                      // MFMAs per k-step
    constexpr int GAP = 1;                           // loads as early as possible
    static_assert(T::D * GAP <= (KS - 1) * MF, "a chunk's loads are issued before its barrier");
    static_assert(MB + NB <= MF, "the next k-step's reads fit between this one's MFMAs");
    if constexpr (T::SPLIT) {
        // Five slots of one operand chunk each: A of chunk c in slot 2c mod 5,
        // B in slot 2c+1 mod 5.  While chunk c is computed, B of chunk c+1 and
        // then A of chunk c+2 are loaded into the two slots chunk c-1 used, so
        // half of every chunk is in flight for two chunks' time and the
        // barrier that ends chunk c waits only for the loads issued before A
        // of c+2.  A two-stage ring of whole chunks makes that barrier wait
        // for all 64 KB issued at the start of the chunk, and the loads'
        // latency at that depth, not their rate, bounds the loop.
        constexpr int SLOT = T::A_BYTES;
        auto mod5 = [](int x) { return x >= 5 ? x - 5 : x; };
        auto load_a = [&](int c, int slot, int j) {
            dma16s(p.A + (int64_t)m0 * p.ld + (int64_t)c * BK, da[j],
                   lds + slot * SLOT + (j * NW + wave) * 1024);
        };
        auto load_b = [&](int c, int slot, int j) {
            dma16s(p.B + (int64_t)n0 * p.ld + (int64_t)c * BK, db[j],
                   lds + slot * SLOT + (j * NW + wave) * 1024);
        };
        auto frag2 = [&](const char* As, const char* Bs, int s, int slot, int r) {
            if (r < MB)
                fa[slot][r] = frag(As, wm * TWM + r * 32 + l32, s);
            else
                fb[slot][r - MB] = frag(Bs, wn * TWN + (r - MB) * 32 + l32, s);
        };
#pragma unroll
        for (int j = 0; j < DA; ++j) load_a(0, 0, j);
#pragma unroll
        for (int j = 0; j < DB; ++j) load_b(0, 1, j);
        if (nk > 1) {
#pragma unroll
            for (int j = 0; j < DA; ++j) load_a(1, 2, j);
            __builtin_amdgcn_s_waitcnt(kWaitVm<DA>);
        } else {
            __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
        }
        asm volatile("s_barrier" ::: "memory");
#pragma unroll
        for (int r = 0; r < MB + NB; ++r) frag2(lds, lds + SLOT, 0, 0, r);
        int sa = 0;   // slot of A of the chunk being computed
        // One chunk.  MORE: a chunk follows (B of c+1 is loaded during this
        // one); LA: A of c+2 is loaded too.
        auto chunk2 = [&](int c, auto more_tag, auto la_tag) {
            constexpr bool MORE = decltype(more_tag)::value, LA = decltype(la_tag)::value;
            const char* As = lds + sa * SLOT;
            const char* Bs = lds + mod5(sa + 1) * SLOT;
            const int sa_n = mod5(sa + 2);
            const char* As_n = lds + sa_n * SLOT;
            const char* Bs_n = lds + mod5(sa + 3) * SLOT;
            const int sb_load = mod5(sa + 3), sa_load = mod5(sa + 4);   // chunk c-1's slots
#pragma unroll
            for (int s = 0; s < KS; ++s) {
#pragma unroll
                for (int m = 0; m < MF; ++m) {
                    const int i = m / NB, j = m % NB;
                    acc[i][j] = F::mma(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (s + 1 < KS) {
                        if (m < MB + NB) frag2(As, Bs, s + 1, (s + 1) & 1, m);
                    } else if (MORE) {
                        if (m == 0) {
                            __builtin_amdgcn_s_waitcnt(kWaitVm<LA ? DA : 0>);
                            asm volatile("s_barrier" ::: "memory");
                        }
                        if (m < MB + NB) frag2(As_n, Bs_n, 0, 0, m);
                    }
                    const int g = s * MF + m;
                    if (MORE && g < DB) load_b(c + 1, sb_load, g);
                    if (LA && g >= DB && g < DB + DA) load_a(c + 2, sa_load, g - DB);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            sa = sa_n;
        };
        using T1 = std::true_type;
        using F0 = std::false_type;
        for (int c = 0; c + 2 < nk; ++c) chunk2(c, T1{}, T1{});
        if (nk >= 2) chunk2(nk - 2, T1{}, F0{});
        chunk2(nk - 1, F0{}, F0{});
    } else {
#pragma unroll
        for (int c = 0; c < NS - 1; ++c)
            if (c < nk) issue(c, c);
        wait_loads_and_barrier<T::D>(min(NS - 2, nk - 1));
        read_step(0, 0, 0);
        int cur = 0;
        auto frag_one = [&](int buf, int s, int slot, int r) {
            const char* As = lds + buf * T::STAGE;
            const char* Bs = As + T::A_BYTES;
            if (r < MB)
                fa[slot][r] = frag(As, wm * TWM + r * 32 + l32, s);
            else
                fb[slot][r - MB] = frag(Bs, wn * TWN + (r - MB) * 32 + l32, s);
        };
        // One chunk.  LOAD: chunk kt+NS-1 is loaded during it; MORE: a chunk
        // follows; LATER: loads that may still be in flight at its barrier.
        auto chunk = [&](int kt, auto more_tag, auto load_tag, auto later_tag) {
            constexpr bool MORE = decltype(more_tag)::value, LOAD = decltype(load_tag)::value;
            constexpr int LATER = decltype(later_tag)::value;
            const int nxt = (cur + 1 == NS) ? 0 : cur + 1;
            const int lbuf = (cur == 0) ? NS - 1 : cur - 1;
            char* As = lds + lbuf * T::STAGE;
            char* Bs = As + T::A_BYTES;
            const int64_t k0 = (int64_t)(kt + NS - 1) * BK;
            const uint16_t* a0 = p.A + (int64_t)m0 * p.ld + k0;
            const uint16_t* b0 = p.B + (int64_t)n0 * p.ld + k0;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
#pragma unroll
                for (int m = 0; m < MF; ++m) {
                    const int i = m / NB, j = m % NB;
                    acc[i][j] = F::mma(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (s + 1 < KS) {
                        if (m < MB + NB) frag_one(cur, s + 1, (s + 1) & 1, m);
                    } else if (MORE) {
                        if (m == 0) {
                            __builtin_amdgcn_s_waitcnt(kWaitVm<LATER * T::D>);
                            asm volatile("s_barrier" ::: "memory");
                        }
                        if (m < MB + NB) frag_one(nxt, 0, 0, m);
                    }
                    const int g = s * MF + m;
                    if (LOAD && g % GAP == 0 && g / GAP < T::D) {
                        const int d = g / GAP;
                        if (d < DA)
                            dma16s(a0, da[d], As + (d * NW + wave) * 1024);
                        else
                            dma16s(b0, db[d - DA], Bs + ((d - DA) * NW + wave) * 1024);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            cur = nxt;
        };
        using T1 = std::true_type;
        using F0 = std::false_type;
        if (nk >= NS) {
            for (int kt = 0; kt + NS - 1 < nk; ++kt) chunk(kt, T1{}, T1{}, std::integral_constant<int, NS - 2>{});
            if constexpr (NS >= 4) chunk(nk - 3, T1{}, F0{}, std::integral_constant<int, 1>{});
            if constexpr (NS >= 3) chunk(nk - 2, T1{}, F0{}, std::integral_constant<int, 0>{});
            chunk(nk - 1, F0{}, F0{}, std::integral_constant<int, 0>{});
        } else {
            // fewer chunks than ring stages: the prologue issued all of them, and
            // each barrier waits for every load still in flight
            for (int kt = 0; kt + 1 < nk; ++kt) chunk(kt, T1{}, F0{}, std::integral_constant<int, 0>{});
            chunk(nk - 1, F0{}, F0{}, std::integral_constant<int, 0>{});
        }
    }

    // ---- epilogue: C <- alpha*acc + beta*C (beta == 0: C not read) ----
    const float alpha = p.alpha, beta = p.beta;
    const int col = n0 + wn * TWN + NB * l32;
    if constexpr (NB == 4) {
        if (p.vec_c && m0 + BM <= p.M && n0 + BN <= p.N) {
            // Whole tile inside C: the 16 rows of C of a 32-row block are read
            // before any is written, one memory round trip per block rather
            // than one per row.
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                float* base = p.C + (int64_t)(m0 + wm * TWM + i * 32 + 4 * h) * p.ldc + col;
                auto row_ptr = [&](int r) { return base + (int64_t)(8 * (r >> 2) + (r & 3)) * p.ldc; };
                f32x4 cv[16];
                if (beta != 0.0f) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) cv[r] = *reinterpret_cast<const f32x4*>(row_ptr(r));
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    f32x4 o;
#pragma unroll
                    for (int n = 0; n < 4; ++n) {
                        float v = alpha * acc[i][n][r];
                        if (beta != 0.0f) v += beta * cv[r][n];
                        o[n] = v;
                    }
                    *reinterpret_cast<f32x4*>(row_ptr(r)) = o;
                }
            }
            return;
        }
    }
    // A tile at an edge of C (or C rows not 16-byte aligned): several rows
    // per block read before any is written, with unguarded reads clamped
    // into C (edge_block_epilogue).
    constexpr int RB = MB * NB * 16 >= 256 ? 4 : 16;   // rows per batch
#pragma unroll
    for (int i = 0; i < MB; ++i)
        edge_block_epilogue<NB, RB>(p.C, p.ldc, p.M, p.N, m0 + wm * TWM + i * 32 + 4 * h, col, alpha,
                                    beta, [&](int n, int r) { return acc[i][n][r]; });
}

template <int FMT, int BM, int BN, int BK, int NS, int WM, int WN>
hipError_t launch_tc16(const Tc16Args& p, hipStream_t stream) {
    hipLaunchKernelGGL((tc16_kernel<FMT, BM, BN, BK, NS, WM, WN>),
                       dim3((unsigned)(p.tiles_m * p.tiles_n)), dim3(64 * WM * WN), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_tc_cast(int fmt, const float* A, int64_t lda, bool vec_a, const float* B,
                          int64_t ldb, bool vec_b, int M, int N, int K, uint16_t* A16,
                          uint16_t* B16, int Mp, int Np, int Kp, hipStream_t stream) {
    const int64_t units = (int64_t)Mp * (Kp / 8);
    const unsigned ga = (unsigned)std::min<int64_t>((units + 255) / 256, 1 << 20);
    const int64_t tiles = (int64_t)(Np / 128) * (Kp / 64);
    const unsigned gb = (unsigned)std::min<int64_t>(tiles, 1 << 20);
#define PHOBOS_CAST(F)                                                                         \
    do {                                                                                       \
        if (vec_a)                                                                             \
            hipLaunchKernelGGL((tc_cast_rows_kernel<F, true>), dim3(ga), dim3(256), 0, stream, \
                               A, lda, M, K, A16, Mp, Kp);                                     \
        else                                                                                   \
            hipLaunchKernelGGL((tc_cast_rows_kernel<F, false>), dim3(ga), dim3(256), 0, stream,\
                               A, lda, M, K, A16, Mp, Kp);                                     \
        if (vec_b)                                                                             \
            hipLaunchKernelGGL((tc_cast_cols_kernel<F, true>), dim3(gb), dim3(256), 0, stream, \
                               B, ldb, K, N, B16, Np, Kp);                                     \
        else                                                                                   \
            hipLaunchKernelGGL((tc_cast_cols_kernel<F, false>), dim3(gb), dim3(256), 0, stream,\
                               B, ldb, K, N, B16, Np, Kp);                                     \
    } while (0)
    if (fmt == SGEMM_TC_F16)
        PHOBOS_CAST(SGEMM_TC_F16);
    else
        PHOBOS_CAST(SGEMM_TC_BF16);
#undef PHOBOS_CAST
    return hipGetLastError();
}

void* tc_scratch(hipError_t* err) {
    // device -> address of `scratch` there; looked up with that device current
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    *err = hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *err = e;
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return nullptr;
        }
        addr[dev] = p;
    }
    return addr[dev];
}

#define PHOBOS_TC16_CFG(FMT, BM, BN, BK, NS, WM, WN)                                        \
    Tc16Entry{sgemm_config{BM, BN, BK, WM, WN}, NS, 64 * WM * WN,                          \
              Tc16Shape<BM, BN, BK, NS, WM, WN>::LDS_BYTES,                                 \
              &launch_tc16<FMT, BM, BN, BK, NS, WM, WN>}

#define PHOBOS_TC16_TABLE(FMT)                                                              \
    {                                                                                       \
        PHOBOS_TC16_CFG(FMT, 256, 256, 32, 4, 2, 2), PHOBOS_TC16_CFG(FMT, 256, 256, 32, 4, 4, 2), \
            PHOBOS_TC16_CFG(FMT, 256, 256, 64, 5, 2, 2), PHOBOS_TC16_CFG(FMT, 256, 256, 64, 5, 4, 2), \
            PHOBOS_TC16_CFG(FMT, 256, 128, 32, 4, 2, 2), PHOBOS_TC16_CFG(FMT, 128, 128, 64, 2, 2, 2), \
    }

const Tc16Entry* tc16_kernel_table(int fmt, int* count) {
    static const Tc16Entry f16[] = PHOBOS_TC16_TABLE(SGEMM_TC_F16);
    static const Tc16Entry bf16[] = PHOBOS_TC16_TABLE(SGEMM_TC_BF16);
    *count = (int)(sizeof(f16) / sizeof(f16[0]));
    if (fmt == SGEMM_TC_F16) return f16;
    if (fmt == SGEMM_TC_BF16) return bf16;
    *count = 0;
    return nullptr;
}

// The compiled configurations of the matrix-core variant, per input format;
// nullptr for an unknown format.
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
