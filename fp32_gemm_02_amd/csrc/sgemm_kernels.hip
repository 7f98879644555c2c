// gfx950 (CDNA4) kernels for C <- alpha*A*B + beta*C in fp32.
//
// The GEMM kernel is the single-GPU leaf of the Phobos pages: one workgroup
// owns one BM x BN tile of C and walks K in chunks of BK, accumulating
// acc += A_tile * B_tile ("Show HN: Phobos", section "Matrix
// Multiplication"), then stores alpha*acc + beta*C.  The techniques the blog
// lists in "GPU Performance" (coalescing, a shared-memory tile per CTA, a
// per-warp register micro-tile free of bank conflicts, the matrix units) and
// the ping-pong buffering and XOR swizzling of "Are we cuBLAS yet?" map onto
// CDNA4 as:
//   - global -> LDS with 128-bit loads, consecutive lanes on consecutive
//     addresses.  Interior chunks use gfx950's direct global-to-LDS loads
//     (global_load_lds_dwordx4: each lane fetches 16 bytes, the wave writes
//     its 64 x 16 bytes contiguously into LDS, no registers in between);
//     chunks at an edge of M, N or K go through registers with per-element
//     bounds checks and zero fill;
//   - two LDS stages (double buffering), one barrier per K chunk;
//   - each 64-lane wavefront owns a TWM x TWN sub-tile made of MB x NB blocks
//     of 32 x 32, accumulated by v_mfma_f32_32x32x2_f32 in registers for the
//     whole K loop;
//   - the A tile is stored row-major without padding, its 16-byte pieces
//     XOR-swizzled within each row, so that the MFMA operand reads are free of
//     LDS bank conflicts (the swizzle is applied to the global addresses of
//     the direct loads, since those write LDS in lane order);
//   - with beta != 0, part of the C tile is loaded into LDS during the last
//     K chunk, while the matrix cores still run, so that less of C is read
//     in the burst at the end, when every workgroup of a launch reads and
//     writes its tile at once.
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

#include <type_traits>

#include "sgemm_device.h"
#include "sgemm_internal.h"

// The direct global-to-LDS loads of a stage are issued spread over its first
// PHOBOS_DMA_SPREAD k-steps when a stage has 16 k-steps or more (BK = 32), and
// all at the first k-step otherwise (a BK = 16 stage has too few k-steps left
// before its barrier for the last loads to land).
#ifndef PHOBOS_DMA_SPREAD
#define PHOBOS_DMA_SPREAD 4
#endif

// Upper bound on the LDS ring depth of the GEMM kernel (2 or 3).
#ifndef PHOBOS_MAX_STAGES
#define PHOBOS_MAX_STAGES 2
#endif

namespace phobos {


template <int BM, int BN, int BK, int WM, int WN>
struct TileShape {
    static constexpr int NT = 64 * WM * WN;      // threads per workgroup
    static constexpr int NW = WM * WN;           // waves per workgroup
    static constexpr int TWM = BM / WM;          // wave tile rows
    static constexpr int TWN = BN / WN;          // wave tile columns
    static constexpr int MB = TWM / 32;          // 32x32 blocks per wave, rows
    static constexpr int NB = TWN / 32;          // 32x32 blocks per wave, columns
    static constexpr int A_FLOATS = BM * BK;     // A tile, row-major, swizzled
    static constexpr int B_FLOATS = BK * BN;     // B tile, row-major
    static constexpr int STAGE = A_FLOATS + B_FLOATS;
    // LDS ring of NS stages: three when they fit (loads run two stages
    // ahead of the MFMAs), else two.
    static constexpr int NS = (3 * STAGE * 4 <= 160 * 1024 && PHOBOS_MAX_STAGES >= 3) ? 3 : 2;
    static constexpr int LDS_BYTES = NS * STAGE * 4;
    static constexpr int QA = BK / 4;            // 16-byte pieces per A tile row
    static constexpr int LA = BM * QA / NT;      // pieces of A per thread per stage
    static constexpr int QB = BN / 4;            // 16-byte pieces per B tile row
    static constexpr int LB = BK * QB / NT;      // pieces of B per thread per stage
    static constexpr int DA = BM * QA / 64 / NW; // direct loads of A per wave per stage
    static constexpr int DB = BK * QB / 64 / NW; // direct loads of B per wave per stage
    static_assert(BM % WM == 0 && BN % WN == 0, "wave grid must divide the tile");
    static_assert(TWM % 32 == 0 && TWN % 32 == 0, "wave tile is whole 32x32 blocks");
    static_assert(NB >= 1 && NB <= 4, "B reads are 1 to 4 floats wide");
    static_assert(QA == 4 || QA == 8, "BK is 16 or 32");
    static_assert((BM * QA) % NT == 0 && (BK * QB) % NT == 0, "whole loads per thread");
    static_assert(DA * 64 * NW == BM * QA && DB * 64 * NW == BK * QB,
                  "whole direct loads per wave");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS of one CU");
    // C prefetch for beta != 0 (8-wave tiles whose waves write 4 consecutive
    // columns per lane and hold at least 128 accumulators, so that one
    // workgroup fills its CU whatever its LDS): during the last K chunk, rows
    // of each wave's first 32-row block of C are loaded straight into LDS,
    // CPF_FREE of them into the stage buffer that chunk leaves free and
    // CPF_SPARE more into LDS beyond the ring; the epilogue takes them from
    // there instead of from memory.  Every row is 1 KiB per wave: lane l
    // holds its own 16 bytes at offset 16*l.
    static constexpr bool CPF_OK = NB == 4 && NW == 8 && MB * NB * 16 >= 128;
    static constexpr int CPF_ROW_BYTES = 64 * 16;
    static constexpr int CPF_FREE =
        CPF_OK ? (STAGE * 4 / (NW * CPF_ROW_BYTES) < 16 ? STAGE * 4 / (NW * CPF_ROW_BYTES) : 16) : 0;
    static constexpr int CPF_SPARE_MAX = (160 * 1024 - LDS_BYTES) / (NW * CPF_ROW_BYTES);
    static constexpr int CPF_SPARE =
        CPF_OK ? (CPF_SPARE_MAX < 16 - CPF_FREE ? CPF_SPARE_MAX : 16 - CPF_FREE) : 0;
    static constexpr int CPF = CPF_FREE + CPF_SPARE;   // prefetched rows per lane, <= 16
    static constexpr int SMEM_FLOATS = NS * STAGE + CPF_SPARE * NW * CPF_ROW_BYTES / 4;
    static_assert(SMEM_FLOATS * 4 <= 160 * 1024, "LDS of one CU");
};

template <int BM, int BN, int BK, int WM, int WN, bool VEC>
__global__ __launch_bounds__(64 * WM * WN) void sgemm_mfma_kernel(GemmArgs p) {
    using T = TileShape<BM, BN, BK, WM, WN>;
    __shared__ __attribute__((aligned(16))) float smem[T::SMEM_FLOATS];

    int tm, tn;
    tile_of(p, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int l32 = lane & 31;
    const int h = lane >> 5;

    // ---- register path: global -> registers -> LDS (edges of M, N, K) ----
    struct Staged {
        f32x4 a[T::LA], b[T::LB];
    };
    // Piece j (0 .. LA+LB-1) of a chunk: A's pieces first, then B's.
    auto load_piece = [&](Staged& r, int k0, int j) {
        if (j < T::LA) {
            const int idx = tid + j * T::NT;
            const int row = idx / T::QA;
            const int gk = k0 + (idx % T::QA) * 4;
            const int grow = m0 + row;
            const int nvalid = (grow < p.M) ? (p.K - gk) : 0;
            const float* src = p.A + (int64_t)(grow < p.M ? grow : 0) * p.lda + gk;
            r.a[j] = load4<VEC>(src, nvalid);
        } else {
            const int i = j - T::LA, idx = tid + i * T::NT;
            const int gk = k0 + idx / T::QB;
            const int gn = n0 + (idx % T::QB) * 4;
            const int nvalid = (gk < p.K) ? (p.N - gn) : 0;
            const float* src = p.B + (int64_t)(gk < p.K ? gk : 0) * p.ldb + gn;
            r.b[i] = load4<VEC>(src, nvalid);
        }
    };
    auto store_piece = [&](const Staged& r, int s, int j) {
        float* As = smem + s * T::STAGE;
        float* Bs = As + T::A_FLOATS;
        if (j < T::LA) {
            const int idx = tid + j * T::NT;
            const int row = idx / T::QA;
            const int q = (idx % T::QA) ^ swz<T::QA>(row);
            *reinterpret_cast<f32x4*>(As + row * BK + 4 * q) = r.a[j];
        } else {
            const int idx = tid + (j - T::LA) * T::NT;
            *reinterpret_cast<f32x4*>(Bs + 4 * idx) = r.b[j - T::LA];
        }
    };
    auto load_regs = [&](Staged& r, int k0) {
#pragma unroll
        for (int j = 0; j < T::LA + T::LB; ++j) load_piece(r, k0, j);
    };
    auto store_regs = [&](const Staged& r, int s) {
#pragma unroll
        for (int j = 0; j < T::LA + T::LB; ++j) store_piece(r, s, j);
    };

    // ---- direct path: global -> LDS, whole K chunks of aligned operands ----
    // Wave w's j-th load of A fills the 64 consecutive 16-byte slots
    // (j*NW + w)*64 .. +63 of the A tile; slot g holds row g / QA, stored
    // piece g % QA, i.e. logical piece (g % QA) ^ swz(row).  B's slots are
    // its pieces in row-major order.  Offsets are relative to the chunk's
    // first row and column inside the tile.
    // Tiles at the M or N edge load too: a row of A past M reads row M-1 and
    // a piece of B wholly past N reads the tile's first piece instead; both
    // only feed rows or columns of C that are never stored.  A piece of B
    // that straddles N reads the pad floats after column N-1 of the same row
    // (ldb is a multiple of 4 here, so they lie before the next row); for the
    // last row of B that could pass the end of the buffer, so a chunk that
    // holds row K-1 of an N-edge tile takes the register path.
    // The loads take a wave-uniform base (A: row m0, column k0; B: row k0,
    // column n0) and a 32-bit byte offset per lane, so they need
    // (BM-1)*lda + BK and (BK-1)*ldb + BN floats to fit in 32-bit byte
    // offsets; beyond that every chunk takes the register path.
    uint32_t da_off[T::DA], db_off[T::DB];
#pragma unroll
    for (int j = 0; j < T::DA; ++j) {
        const int g = (j * T::NW + wave) * 64 + lane;
        const int row = g / T::QA;
        const int q = (g % T::QA) ^ swz<T::QA>(row);
        const int grow = min(m0 + row, p.M - 1);
        da_off[j] = (uint32_t)(((int64_t)(grow - m0) * p.lda + 4 * q) * 4);
    }
#pragma unroll
    for (int j = 0; j < T::DB; ++j) {
        const int g = (j * T::NW + wave) * 64 + lane;
        const int gn = n0 + 4 * (g % T::QB);
        db_off[j] = (uint32_t)(((int64_t)(g / T::QB) * p.ldb + (gn < p.N ? gn - n0 : 0)) * 4);
    }
    const bool narrow = ((int64_t)(BM - 1) * p.lda + BK) * 4 <= (int64_t)UINT32_MAX &&
                        ((int64_t)(BK - 1) * p.ldb + BN) * 4 <= (int64_t)UINT32_MAX;
    // Direct load number j (0 .. DA+DB-1) of the chunk at k0 into buffer s.
    auto load_direct_one = [&](int k0, int s, int j) {
        float* As = smem + s * T::STAGE;
        float* Bs = As + T::A_FLOATS;
        if (j < T::DA)
            dma16s(p.A + (int64_t)m0 * p.lda + k0, da_off[j], As + (j * T::NW + wave) * 256);
        else
            dma16s(p.B + (int64_t)k0 * p.ldb + n0, db_off[j - T::DA],
                   Bs + ((j - T::DA) * T::NW + wave) * 256);
    };
    auto load_direct = [&](int k0, int s) {
#pragma unroll
        for (int j = 0; j < T::DA + T::DB; ++j) load_direct_one(k0, s, j);
    };
    // The chunk k0 .. k0+BK-1 goes direct when it lies wholly inside K, and,
    // for a tile at the N edge, does not hold the last row of B.
    const bool n_inside = n0 + BN <= p.N;
    auto direct_ok = [&](int k0) {
        return VEC && narrow && (n_inside ? k0 + BK <= p.K : k0 + BK < p.K);
    };

    f32x16 acc[T::MB][T::NB];
#pragma unroll
    for (int i = 0; i < T::MB; ++i)
#pragma unroll
        for (int j = 0; j < T::NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Per-lane LDS offsets of the MFMA operands inside one stage.  The A row
    // of a lane is wm*TWM + i*32 + l32 for block i; its swizzle is that of
    // l32 (TWM and 32 are multiples of 16).  Chunk c of the stage covers the
    // k-steps 4c..4c+3, i.e. logical piece h*QA/2 + c of the row.
    const int a_row = (wm * T::TWM + l32) * BK;
    int a_piece[T::QA / 2];
#pragma unroll
    for (int c = 0; c < T::QA / 2; ++c) a_piece[c] = 4 * ((h * (T::QA / 2) + c) ^ swz<T::QA>(l32));
    const int b_off = T::A_FLOATS + h * (BK / 2) * BN + wn * T::TWN + T::NB * l32;

    // Operand fragments, double-buffered in registers: fa holds the A values
    // of one chunk of 4 k-steps (one ds_read_b128 per 32-row block), fb the B
    // values of one k-step (one NB-wide read).  Reads for step kk+1 are issued
    // before the MFMAs of step kk, so LDS latency hides behind 64-cycle MFMAs.
    using BV = typename BVec<T::NB>::type;
    f32x4 fa[2][T::MB];
    BV fb[2];
    auto read_a = [&](const float* base, int c, f32x4* dst) {
#pragma unroll
        for (int i = 0; i < T::MB; ++i)
            dst[i] = *reinterpret_cast<const f32x4*>(base + a_row + i * 32 * BK + a_piece[c]);
    };
    auto read_b = [&](const float* base, int kk) -> BV {
        return *reinterpret_cast<const BV*>(base + b_off + kk * BN);
    };
    auto mfma_step = [&](const f32x4* a, int j, BV b) {
#pragma unroll
        for (int i = 0; i < T::MB; ++i)
#pragma unroll
            for (int n = 0; n < T::NB; ++n)
                acc[i][n] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][j], BVec<T::NB>::get(b, n),
                                                                 acc[i][n], 0, 0, 0);
    };

    // K loop over a ring of NS LDS buffers; stage kt lives in buffer kt % NS.
    // During stage kt the loads of stage kt+NS-1 are issued after the first
    // k-step's reads, into the buffer stage kt-1 used (everyone finished
    // reading it before the barrier that ended stage kt-1): direct loads land
    // in LDS by themselves; register loads are written to LDS four k-steps
    // before the end of the stage.  The barrier that ends stage kt sits before
    // its last k-step's MFMAs, after every read of the stage has returned and
    // once the loads of stage kt+1 have landed (those of later stages may
    // still be in flight), so the first reads of stage kt+1 are issued right
    // after it and overlap those MFMAs.
    constexpr int KS = BK / 2;         // k-steps per stage (2 k each)
    constexpr int NS = T::NS;
    constexpr int DIRECT_LOADS = T::DA + T::DB;   // per wave per stage
    constexpr int DMA_STEPS = (KS >= 16) ? PHOBOS_DMA_SPREAD : 1;
    constexpr int DMA_PER_STEP = (DIRECT_LOADS + DMA_STEPS - 1) / DMA_STEPS;
    static_assert(DMA_STEPS >= 1 && DMA_STEPS <= KS - 4, "loads land well before the barrier");
    const int nk = (p.K + BK - 1) / BK;
    // Wait until at most `pending` direct loads of this wave are in flight and
    // every LDS access has returned, then meet the other waves.
    auto wait_and_barrier = [&](bool pending) {
        if (NS == 3 && pending)
            __builtin_amdgcn_s_waitcnt(kWaitVm<DIRECT_LOADS>);
        else
            __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
        __syncthreads();
    };
    auto issue = [&](int stage, int buf) {       // prologue loads, register path stored at once
        if (direct_ok(stage * BK)) {
            load_direct(stage * BK, buf);
            return true;
        }
        Staged st;
        load_regs(st, stage * BK);
        store_regs(st, buf);
        return false;
    };
    // ---- fast path ----
    // With a two-stage ring, the stage loop of a tile has no data-dependent
    // branch, and the work between MFMAs is spread out: the fragment reads
    // for the next k-step, the loads of the next chunk and the stage barrier
    // are each issued right after one MFMA, while it runs, instead of as one
    // group between k-steps that leaves the matrix core idle until the group
    // has issued.  The loop body is straight-line code, so the compiler's LDS
    // waits are exact: before an MFMA it waits only for the fragments that
    // MFMA reads, not for the next stage's first reads issued after the
    // barrier.  Every chunk loads directly except, on a tile at the N edge or
    // when K is not a whole number of chunks, the last one, which holds row
    // K-1 of B: that one comes through registers with bounds checks.
    // C prefetch: whole tile, beta != 0, every chunk direct, and the lane
    // offsets of four rows of C fit in 32 bits.
    const bool whole = VEC && m0 + BM <= p.M && n_inside;
    const uint32_t c_off = (uint32_t)((4 * h * p.ldc + 4 * l32) * 4);
    auto cpf_dst = [&](int nb, int r) -> float* {
        if (r < T::CPF_FREE) return smem + nb * T::STAGE + (wave * T::CPF_FREE + r) * 256;
        return smem + NS * T::STAGE + (wave * T::CPF_SPARE + (r - T::CPF_FREE)) * 256;
    };
    int cpf_buf = 0;
    constexpr int MFMAS = T::MB * T::NB;                // MFMAs per k-step
    constexpr int DMA_AT = (MFMAS >= 10) ? 6 : MFMAS - DMA_PER_STEP;
    const bool reg_last = !n_inside || p.K % BK != 0;
    const int nk_direct = reg_last ? (p.K - 1) / BK : p.K / BK;   // chunks loaded directly
    const bool cpf = T::CPF > 0 && whole && p.beta != 0.0f && !reg_last && narrow &&
                     (4 * p.ldc + 4 * 32) * 4 <= (int64_t)UINT32_MAX;
    bool cpf_done = false;
    bool done = false;
    if constexpr (NS == 2 && T::MB + 2 <= MFMAS && DMA_AT >= 0) {
        if (VEC && narrow && nk_direct >= 1) {
            auto read_a_one = [&](const float* base, int c, f32x4* dst, int i) {
                dst[i] = *reinterpret_cast<const f32x4*>(base + a_row + i * 32 * BK + a_piece[c]);
            };
            load_direct(0, 0);
            __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
            __syncthreads();
            read_a(smem, 0, fa[0]);
            fb[0] = read_b(smem, 0);
            int cur = 0;
            // Prefetch load r (0 .. CPF-1) of C: the lane's row r of its
            // wave's first 32-row block (what the epilogue reads as cv[r]),
            // into the free stage buffer nb (r < CPF_FREE) or beyond the
            // ring.  The whole tile lies inside C, so every address is.
            auto load_c_one = [&](int nb, int r) {
                const float* row = p.C + (int64_t)(m0 + wm * T::TWM + 8 * (r >> 2) + (r & 3)) * p.ldc +
                                   n0 + wn * T::TWN;
                dma16s(row, c_off, cpf_dst(nb, r));
            };
            // One stage: the k-steps of chunk kt from buffer cur, while chunk
            // kt+1 is loaded directly into the other buffer (NEXT 1; 0: no
            // next chunk here, and with the C prefetch its rows are loaded
            // into the other buffer instead); at the last k-step, the barrier
            // and the first reads of chunk kt+1.
            auto stage = [&](int kt, auto next_tag) {
                constexpr int NEXT = decltype(next_tag)::value;
                const float* base = smem + cur * T::STAGE;
                const int nb = cur ^ 1;
                const float* nbase = smem + nb * T::STAGE;
                const int lk0 = (kt + 1) * BK;
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
                    for (int m = 0; m < MFMAS; ++m) {
                        const int i = m / T::NB, n = m % T::NB;
                        acc[i][n] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            fa[(kk / 4) & 1][i][kk % 4], BVec<T::NB>::get(fb[kk & 1], n), acc[i][n],
                            0, 0, 0);
                        __builtin_amdgcn_sched_barrier(0);
                        if (kk + 1 < KS) {
                            if (m == 0) fb[(kk + 1) & 1] = read_b(base, kk + 1);
                            if ((kk + 1) % 4 == 0 && m >= 1 && m <= T::MB)
                                read_a_one(base, (kk + 1) / 4, fa[((kk + 1) / 4) & 1], m - 1);
                        } else if (NEXT == 1) {
                            // chunk kt+1 has landed (and its register-path
                            // stores are done) everywhere, and every wave has
                            // read chunk kt's buffer for the last time (its
                            // fragments are in registers)
                            if (m == 0) {
                                __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
                                asm volatile("s_barrier" ::: "memory");
                            }
                            if (m == 1) fb[0] = read_b(nbase, 0);
                            if (m >= 2 && m < 2 + T::MB) read_a_one(nbase, 0, fa[0], m - 2);
                        }
                        if (NEXT == 1 && kk < DMA_STEPS && m >= DMA_AT && m < DMA_AT + DMA_PER_STEP) {
                            const int j = kk * DMA_PER_STEP + (m - DMA_AT);
                            if (j < DIRECT_LOADS) load_direct_one(lk0, nb, j);
                        }
                        if (NEXT == 0 && m >= DMA_AT && m < DMA_AT + DMA_PER_STEP) {
                            const int r = kk * DMA_PER_STEP + (m - DMA_AT);
                            if (r < T::CPF && cpf) load_c_one(nb, r);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                cur = nb;
            };
            using Direct = std::integral_constant<int, 1>;
            using Last = std::integral_constant<int, 0>;
            for (int kt = 0; kt + 1 < nk_direct; ++kt) stage(kt, Direct{});
            cpf_buf = cur ^ 1;
            stage(nk_direct - 1, Last{});
            if (reg_last) {
                // The last chunk through registers, into the buffer chunk
                // nk_direct-2 used (read for the last time before the barrier
                // that ended it); one barrier publishes it.
                Staged st;
                load_regs(st, nk_direct * BK);
                store_regs(st, cur);
                __syncthreads();
                read_a(smem + cur * T::STAGE, 0, fa[0]);
                fb[0] = read_b(smem + cur * T::STAGE, 0);
                stage(nk_direct, Last{});
            }
            cpf_done = cpf;
            done = true;
        }
    }

    // ---- general path: three-stage rings, unaligned operands, K below two chunks ----
    if (!done) {
        bool pend = false;
        issue(0, 0);
        if (NS == 3 && nk > 1) pend = issue(1, 1);
        wait_and_barrier(pend);
        read_a(smem, 0, fa[0]);
        fb[0] = read_b(smem, 0);
        int cur = 0;                       // buffer of stage kt
        for (int kt = 0; kt < nk; ++kt) {
            const int nxt = (cur + 1 == NS) ? 0 : cur + 1;
            const int lbuf = (cur == 0) ? NS - 1 : cur - 1;   // buffer of stage kt+NS-1
            const float* base = smem + cur * T::STAGE;
            const float* nbase = smem + nxt * T::STAGE;
            const int lk0 = (kt + NS - 1) * BK;
            const bool more = kt + 1 < nk;
            const bool load = kt + NS - 1 < nk;
            const bool direct = load && direct_ok(lk0);
            const bool staged = load && !direct;
            Staged st;   // register path only; dead outside this iteration
    #pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                if (kk + 1 < KS) {
                    if ((kk + 1) % 4 == 0) read_a(base, (kk + 1) / 4, fa[((kk + 1) / 4) & 1]);
                    fb[(kk + 1) & 1] = read_b(base, kk + 1);
                } else if (more) {
                    wait_and_barrier(direct);
                    read_a(nbase, 0, fa[0]);
                    fb[0] = read_b(nbase, 0);
                }
                if (direct) {
    #pragma unroll
                    for (int j = kk * DMA_PER_STEP; j < (kk + 1) * DMA_PER_STEP; ++j)
                        if (j < DIRECT_LOADS) load_direct_one(lk0, lbuf, j);
                }
                if (kk == 0 && staged) load_regs(st, lk0);
                if (kk == KS - 4 && staged) store_regs(st, lbuf);
                __builtin_amdgcn_sched_barrier(0);
                mfma_step(fa[(kk / 4) & 1], kk % 4, fb[kk & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            cur = nxt;
        }
    }

    // ---- epilogue: C <- alpha*acc + beta*C (beta == 0: C not read) ----
    const float alpha = p.alpha, beta = p.beta;
    const int col = n0 + wn * T::TWN + T::NB * l32;
    using CV = typename BVec<T::NB>::type;
    if (whole) {
        // Whole tile inside C: the 16 rows of a 32-row block are read before
        // any is written, so a lane waits for one memory round trip per block
        // rather than one per row.  With the C prefetch, the first CPF rows
        // of block 0 come from LDS, where the wave's own loads put them
        // during the last chunk (its vmcnt wait covers those loads).
#pragma unroll
        for (int i = 0; i < T::MB; ++i) {
            float* base = p.C + (int64_t)(m0 + wm * T::TWM + i * 32 + 4 * h) * p.ldc + col;
            auto row_ptr = [&](int r) { return base + (int64_t)(8 * (r >> 2) + (r & 3)) * p.ldc; };
            CV cv[16];
            if (beta != 0.0f) {
                if (i == 0 && T::CPF > 0 && cpf_done) {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
                    for (int r = 0; r < T::CPF; ++r)
                        cv[r] = *reinterpret_cast<const CV*>(cpf_dst(cpf_buf, r) + 4 * lane);
                } else {
#pragma unroll
                    for (int r = 0; r < T::CPF; ++r) cv[r] = *reinterpret_cast<const CV*>(row_ptr(r));
                }
#pragma unroll
                for (int r = T::CPF; r < 16; ++r) cv[r] = *reinterpret_cast<const CV*>(row_ptr(r));
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                CV o;
#pragma unroll
                for (int n = 0; n < T::NB; ++n) {
                    float v = alpha * acc[i][n][r];
                    if (beta != 0.0f) v += beta * BVec<T::NB>::get(cv[r], n);
                    BVec<T::NB>::set(o, n, v);
                }
                *reinterpret_cast<CV*>(row_ptr(r)) = o;
            }
        }
        return;
    }
    // Tile at an edge of C: as above, a lane reads the C values of several
    // rows of a block before it writes any (all 16, or 2 at a time where the
    // accumulators fill the register file), with unguarded reads clamped
    // into C (edge_block_epilogue).
    constexpr int RB = T::MB * T::NB * 16 >= 256 ? 2 : 16;   // rows per batch
#pragma unroll
    for (int i = 0; i < T::MB; ++i)
        edge_block_epilogue<T::NB, RB>(p.C, p.ldc, p.M, p.N, m0 + wm * T::TWM + i * 32 + 4 * h, col,
                                       alpha, beta, [&](int n, int r) { return acc[i][n][r]; });
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
                TileShape<BM, BN, BK, WM, WN>::SMEM_FLOATS * 4,                         \
                &launch_gemm<BM, BN, BK, WM, WN, true>,                                 \
                &launch_gemm<BM, BN, BK, WM, WN, false>}

// The compiled configurations.  A host function holds the table so that the
// device pass never sees the host launch functions it points to.
const KernelEntry* kernel_table(int* count) {
    static const KernelEntry table[] = {
        PHOBOS_CFG(256, 256, 16, 4, 2),
        PHOBOS_CFG(256, 256, 32, 4, 2),
        PHOBOS_CFG(256, 256, 16, 2, 4),
        PHOBOS_CFG(256, 256, 16, 4, 4),
        PHOBOS_CFG(256, 256, 16, 2, 2),
        PHOBOS_CFG(256, 256, 32, 2, 2),
        PHOBOS_CFG(256, 128, 16, 4, 2),
        PHOBOS_CFG(320, 192, 16, 2, 2),
        PHOBOS_CFG(256, 128, 16, 2, 2),
        PHOBOS_CFG(128, 256, 16, 2, 4),
        PHOBOS_CFG(128, 256, 16, 2, 2),
        PHOBOS_CFG(128, 128, 16, 2, 2),
        PHOBOS_CFG(128, 128, 32, 2, 2),
        PHOBOS_CFG(128, 64, 16, 2, 1),
        PHOBOS_CFG(64, 128, 16, 1, 2),
        PHOBOS_CFG(64, 64, 16, 1, 1),
        PHOBOS_CFG(32, 32, 16, 1, 1),
        PHOBOS_CFG(64, 64, 32, 1, 1),
        PHOBOS_CFG(32, 32, 32, 1, 1),
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
