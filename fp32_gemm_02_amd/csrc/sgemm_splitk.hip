// gfx950 (CDNA4) split-K GEMM kernel: the product C <- alpha*A*B + beta*C in
// fp32 of "Show HN: Phobos", section "Matrix Multiplication", for products
// with too few tiles to give every SIMD work.  The waves of one workgroup
// share a tile of C; the K sum is split over them and their parts are added
// in a fixed order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgemm_device.h"
#include "sgemm_internal.h"

namespace phobos {

// ---------------------------------------------------------------------------
// Split-K within one workgroup, for products with few tiles (a single wave
// per small tile leaves most SIMDs idle and waits out every chunk's load
// latency alone): KS waves share one TL x TL tile of C (TL = 32 or 64), each
// holding the whole tile's accumulators.  Wave w takes the chunks w, w + KS,
// w + 2KS, ... of BK k each and accumulates its own partial tile with
// v_mfma_f32_32x32x2_f32 (operand layout as in sgemm_mfma_kernel with one
// wave over TL/32 x TL/32 blocks), through two LDS stages of its own: each
// wave loads and reads only its own stages, so the K loop has no barrier,
// only the wave's own wait for its loads.  The partial tiles are then added
// in wave order 0, 1, ..., KS-1 through LDS, each wave finishing 16/KS of the
// 16 rows of every block of every lane, and stored as alpha*sum + beta*C.
// Any order of the k terms is within the error bound, and this one is fixed,
// so results repeat bit for bit.
template <int TL, int BK, int KS, bool VEC>
__global__ __launch_bounds__(64 * KS) void sgemm_splitk_kernel(GemmArgs p) {
    constexpr int QA = BK / 4;                  // 16-byte pieces per A row
    constexpr int QB = TL / 4;                  // 16-byte pieces per B row
    constexpr int MB = TL / 32, NB = TL / 32;   // 32 x 32 blocks per wave
    constexpr int A_FLOATS = TL * BK;
    constexpr int STAGE = 2 * TL * BK;          // A (TL x BK) then B (BK x TL)
    constexpr int REGION = 2 * STAGE;           // a wave's two stages
    constexpr int LA = TL * QA / 64;            // 16-byte pieces of A per lane per chunk
    constexpr int LB = BK * QB / 64;            // and of B
    constexpr int RW = 16 / KS;                 // accumulator rows each wave finishes
    using BV = typename BVec<NB>::type;
    static_assert(TL == 32 || TL == 64, "tile of 32 or 64");
    static_assert(QA == 4 || QA == 8, "BK is 16 or 32");
    static_assert(LA + LB == 4 || LA + LB == 8, "loads per chunk");
    static_assert(RW * KS == 16, "accumulator rows split evenly over the waves");
    static_assert(REGION >= MB * NB * 16 * 64, "a wave's partial tile fits its region");
    static_assert(KS * REGION * 4 <= 160 * 1024, "LDS of one CU");
    __shared__ __attribute__((aligned(16))) float smem[KS * REGION];

    int tm, tn;
    tile_of(p, tm, tn);
    const int m0 = tm * TL, n0 = tn * TL;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    float* const mine = smem + wave * REGION;
    const int nk = (p.K + BK - 1) / BK;
    const int nmine = wave < nk ? (nk - 1 - wave) / KS + 1 : 0;   // this wave's chunks

    // Direct loads (as in sgemm_mfma_kernel): A piece g of a chunk sits in
    // slot g (row g / QA, stored piece g % QA = logical piece ^ swz(row)); a
    // row past M reads row M-1, a B piece wholly past N the tile's first piece
    // (both feed only unstored results).  A chunk that holds row K-1 of B on
    // a tile at the N edge, or runs past K, comes through registers.
    const bool n_inside = n0 + TL <= p.N;
    const bool narrow = ((int64_t)(TL - 1) * p.lda + BK) * 4 <= (int64_t)UINT32_MAX &&
                        ((int64_t)(BK - 1) * p.ldb + TL) * 4 <= (int64_t)UINT32_MAX;
    uint32_t da_off[LA], db_off[LB];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        const int g = j * 64 + lane, row = g / QA;
        const int q = (g % QA) ^ swz<QA>(row);
        da_off[j] = (uint32_t)(((int64_t)(min(m0 + row, p.M - 1) - m0) * p.lda + 4 * q) * 4);
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
        const int g = j * 64 + lane, gn = n0 + 4 * (g % QB);
        db_off[j] = (uint32_t)(((int64_t)(g / QB) * p.ldb + (gn < p.N ? gn - n0 : 0)) * 4);
    }
    auto direct_ok = [&](int k0) {
        return VEC && narrow && (n_inside ? k0 + BK <= p.K : k0 + BK < p.K);
    };
    // Chunk c into stage s; true if it went direct (its loads still in flight).
    auto load_chunk = [&](int c, int s) -> bool {
        float* As = mine + s * STAGE;
        float* Bs = As + A_FLOATS;
        const int k0 = c * BK;
        if (direct_ok(k0)) {
            // every read of this stage (chunk c - 2) has returned
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int j = 0; j < LA; ++j) dma16s(p.A + (int64_t)m0 * p.lda + k0, da_off[j], As + j * 256);
#pragma unroll
            for (int j = 0; j < LB; ++j) dma16s(p.B + (int64_t)k0 * p.ldb + n0, db_off[j], Bs + j * 256);
            return true;
        }
#pragma unroll
        for (int j = 0; j < LA; ++j) {
            const int g = j * 64 + lane, row = g / QA, sp = g % QA;
            const int gk = k0 + 4 * (sp ^ swz<QA>(row)), grow = m0 + row;
            const int nvalid = grow < p.M ? p.K - gk : 0;
            const float* src = p.A + (int64_t)(grow < p.M ? grow : 0) * p.lda + gk;
            *reinterpret_cast<f32x4*>(As + 4 * g) = load4<VEC>(src, nvalid);
        }
#pragma unroll
        for (int j = 0; j < LB; ++j) {
            const int g = j * 64 + lane, gk = k0 + g / QB, gn = n0 + 4 * (g % QB);
            const int nvalid = gk < p.K ? p.N - gn : 0;
            const float* src = p.B + (int64_t)(gk < p.K ? gk : 0) * p.ldb + gn;
            *reinterpret_cast<f32x4*>(Bs + 4 * g) = load4<VEC>(src, nvalid);
        }
        return false;
    };

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][n][r] = 0.0f;
    // Operand offsets inside a stage: lane half h takes k = h*BK/2 + kk of the
    // chunk; one 16-byte read gives 4 consecutive k of an A row (block i: row
    // i*32 + l32, whose swizzle is that of l32); one NB-wide read of B gives
    // the columns NB*l32 + n of the NB blocks.
    const int a_row = l32 * BK;
    const int b_col = A_FLOATS + h * (BK / 2) * TL + NB * l32;
    bool pend = nmine > 0 && load_chunk(wave, 0);
    for (int it = 0; it < nmine; ++it) {
        const float* As = mine + (it & 1) * STAGE;
        bool next = false;
        if (it + 1 < nmine) next = load_chunk(wave + (it + 1) * KS, (it + 1) & 1);
        // chunk it has landed: only the next chunk's direct loads may remain
        if (pend) {
            if (next) {
                if constexpr (LA + LB == 8)
                    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
                else
                    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
        }
        pend = next;
#pragma unroll
        for (int c = 0; c < QA / 2; ++c) {
            f32x4 a[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i)
                a[i] = *reinterpret_cast<const f32x4*>(
                    As + a_row + i * 32 * BK + 4 * ((h * (QA / 2) + c) ^ swz<QA>(l32)));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const BV b = *reinterpret_cast<const BV*>(As + b_col + (4 * c + e) * TL);
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int n = 0; n < NB; ++n)
                        acc[i][n] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            a[i][e], BVec<NB>::get(b, n), acc[i][n], 0, 0, 0);
            }
        }
    }

    // Partial tiles into LDS (each wave over its own region, whose reads have
    // all returned), then rows r = wave*RW .. +RW-1 of every block of every
    // lane summed in wave order and stored.
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) mine[((i * NB + n) * 16 + r) * 64 + lane] = acc[i][n][r];
    __syncthreads();
    const float alpha = p.alpha, beta = p.beta;
    const int col = n0 + NB * l32;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        auto row_of = [&](int rr) {
            const int r = wave * RW + rr;
            return m0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        };
        float v[RW][NB];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            const int r = wave * RW + rr;
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                const int q = ((i * NB + n) * 16 + r) * 64 + lane;
                float sum = smem[q];
#pragma unroll
                for (int w = 1; w < KS; ++w) sum += smem[w * REGION + q];
                v[rr][n] = alpha * sum;
            }
        }
        if (beta != 0.0f) {
            // The C values of all the wave's rows, read with no branch (a row
            // past M reads row M-1, a column past N column N-1: every read
            // lies inside C and feeds only elements that are stored), then
            // one wait: a read under a per-lane bounds check made the
            // compiler wait for it before the next row.
            float c[RW][NB];
#pragma unroll
            for (int rr = 0; rr < RW; ++rr) {
                const float* src = p.C + (int64_t)min(row_of(rr), p.M - 1) * p.ldc;
#pragma unroll
                for (int n = 0; n < NB; ++n) c[rr][n] = src[min(col + n, p.N - 1)];
            }
            __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
#pragma unroll
            for (int rr = 0; rr < RW; ++rr)
#pragma unroll
                for (int n = 0; n < NB; ++n) v[rr][n] += beta * c[rr][n];
        }
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            const int row = row_of(rr);
            if (row >= p.M) continue;
            float* dst = p.C + (int64_t)row * p.ldc + col;
            if (VEC && NB == 2 && col + 1 < p.N) {
                *reinterpret_cast<f32x2*>(dst) = f32x2{v[rr][0], v[rr][NB - 1]};
            } else {
#pragma unroll
                for (int n = 0; n < NB; ++n)
                    if (col + n < p.N) dst[n] = v[rr][n];
            }
        }
    }
}

template <int TL, int BK, int KS, bool VEC>
hipError_t launch_splitk(const GemmArgs& p, hipStream_t stream) {
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
    hipLaunchKernelGGL((sgemm_splitk_kernel<TL, BK, KS, VEC>), grid, dim3(64 * KS), 0, stream, p);
    return hipGetLastError();
}

// A split-K entry is named by its TL x TL tile with wm x wn waves (wm * wn =
// KS) where 32 * wm > TL: a wave grid larger than the tile's 32 x 32 blocks,
// whose waves split K instead, each over the whole tile.
#define PHOBOS_SPLITK_CFG(TL, BK, WM, WN)                                                \
    KernelEntry{sgemm_config{TL, TL, BK, WM, WN}, 64 * WM * WN,                          \
                WM * WN * 4 * TL * BK * 4,                                               \
                &launch_splitk<TL, BK, WM * WN, true>, &launch_splitk<TL, BK, WM * WN, false>}

// The split-K configurations.  A host function holds the table so that the
// device pass never sees the host launch functions it points to.
const KernelEntry* splitk_kernel_table(int* count) {
    static const KernelEntry table[] = {
        PHOBOS_SPLITK_CFG(32, 32, 2, 2),
        PHOBOS_SPLITK_CFG(32, 32, 4, 2),
        PHOBOS_SPLITK_CFG(32, 16, 2, 2),
        PHOBOS_SPLITK_CFG(32, 16, 4, 2),
        PHOBOS_SPLITK_CFG(64, 16, 4, 1),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace phobos
