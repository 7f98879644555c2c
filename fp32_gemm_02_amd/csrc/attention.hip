// gfx950 kernel for the pages' second @cluster example, flash attention
// ("@cluster" page, "The same names at two levels"): O = softmax(scale * Q K^T) V
// with a row softmax over the keys, fp32 throughout, head dimension D = 64
// (the only value the pages' @autotune lists).  The body follows the
// FlashAttention paper the pages cite: one pass over the keys per block of
// query rows, keeping a running maximum, a running sum of weights and a
// running weighted sum of value rows, rescaled whenever the maximum grows.
//
// Query rows come in super-tiles of br rows (the pages' @cluster row block;
// br = Nq for the monolithic form), each worked by ceil(br/64) workgroups of
// one launch.  One workgroup owns 64 query rows of its super-tile, 16 per
// query group; the workgroup stages 128 keys of K and V per step in rings of
// LDS stages, loaded ahead by direct global-to-LDS loads, and each group has
// four waves that take a quarter of each step's keys (two waves and halves
// on the register path) and merge their running statistics at the end.  Both products run on the FP32 matrix cores
// (v_mfma_f32_16x16x4_f32, lane layout checked on the GPU with an in-bounds
// probe; l = lane, g = l / 16, q = l % 16):
//   src A: lane l holds A'[q][g]   (16 x 4)
//   src B: lane l holds B'[g][q]   (4 x 16)
//   acc  : lane l, register r holds D[4g + r][q]
// Scores are formed transposed, S^T = K Q^T (16 keys x 16 queries per
// block), so every lane holds one query q and the keys 4g + r: the softmax
// statistics of a query live in the four lanes q, q+16, q+32, q+48.  The
// output is formed transposed too, O^T = V^T P^T: its B operand P^T[key][q] is
// exactly the score registers after the exponential (the key order of the
// contraction is permuted to match them), and its accumulator again holds
// one query per lane, so the rescaling by the running maximum is a plain
// per-lane multiply.  Within a 4-key MFMA step, lane group g supplies head
// dimension d = 16g + j (QK) or key 4g + t%4 of sub-block t/4 (PV); any such
// permutation of a contraction index leaves the sum's terms unchanged.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "sgemm_device.h"
#include "sgemm_internal.h"

// Waves per query group on the direct-load path (2 or 4).
#ifndef PHOBOS_ATT_KSPLIT
#define PHOBOS_ATT_KSPLIT 4
#endif

namespace phobos {

namespace {

constexpr int kD = 64;      // head dimension
constexpr int kBQ = 64;     // query rows per workgroup (16 per wave)
constexpr int kKI = 128;    // keys per step of the key loop
constexpr int kRowB = kD * 4;                      // bytes of one K or V row in LDS
constexpr float kLog2e = 1.4426950408889634f;

// K rows are stored with their 16-byte pieces XOR-swizzled by row.  The LDS
// serves a 128-bit read for 16 lanes per cycle, from a 256-byte bank window,
// in the lane sets {0-3, 8-11, 20-23, 28-31} and {4-7, 12-15, 16-19, 24-27}
// (and the same plus 32): those are the sets whose counter-measured conflict
// cycles match this kernel's reads.  The score reads give lane (q, g) row q
// and piece 4g + cc; with the swizzle row & 11 each of those sets touches 16
// different 16-byte bank groups, and so do the row-major stores (16 lanes per
// row).  The plain swizzle row & 15 put lanes 0-3 and 20-23 on the same groups.
__device__ __forceinline__ int kswz(int row, int piece) { return piece ^ (row & 11); }

// Maximum and sum over the four lanes l, l^16, l^32, l^48 (the lanes that hold
// one query), with the register swaps of 16- and 32-lane halves: a value
// swapped with a copy of itself leaves lane l and lane l^32 (l^16) in the
// same lane of the two registers.  No LDS permute is involved.
__device__ __forceinline__ float quad_max(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// KSPLIT waves per group of 16 queries, each taking its own 128/KSPLIT keys
// of every step of 128 (KSPLIT waves per SIMD in all); their running
// (maximum, weight sum, weighted sum) are merged at the end.  With four
// waves per SIMD instead of two (and 97 instead of 169 registers), one
// wave's softmax overlaps the others' MFMAs better: 0.5% faster.
//
// With direct loads, K has a ring of three LDS stages and V of two, and
// each wave forms the scores of the next step before the softmax of the
// current one (see the loop).  With the register path, K has two stages and V three: K
// stage it & 1 and V stage it % 3 hold the rows of step it while those of
// step it+1 are in flight.  The two waves of a query group share a SIMD
// (waves w and w+4), and the barrier that ends each step would keep them in
// the same phase, taking their exponentials at the same time while the
// matrix core idles.  So there the second wave runs half a step behind: in
// step it it takes the exponentials and output products of step it-1 (whose
// V rows the third V stage keeps), then the scores of step it, and finishes
// step ni-1 after the loop.
template <bool VEC, bool DMA, int KSPLIT>
__global__ __launch_bounds__(256 * KSPLIT) void attention_kernel(AttnArgs p) {
    constexpr int NT = 256 * KSPLIT;           // threads
    constexpr int KI = kKI;                    // keys per step
    constexpr int KW = KI / KSPLIT;            // keys per wave per step
    constexpr int NSB = KW / 16;               // sub-blocks of 16 keys per wave
    static_assert(KSPLIT == 2 || (KSPLIT == 4 && DMA), "key splits: 2, or 4 with direct loads");
    constexpr int TILE = KI * kRowB;           // bytes of the K (or V) rows of one step
    constexpr int LD = KI * 16 / NT;           // 16-byte pieces per thread per tensor
    static_assert(LD * NT == KI * 16, "whole pieces per thread");
    __shared__ __attribute__((aligned(16))) char lds[5 * TILE];
    // direct loads: K stages 0, 1, 2 and V stages 0, 1; register path: K
    // stages 0, 1 and V stages 0, 1, 2
    char* const kring = lds;
    char* const vring = lds + (DMA ? 3 : 2) * TILE;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int q = lane & 15, g = lane >> 4;
    const int wq = wave & 3, half = wave >> 2;   // query group, key part
    // super-tile of this workgroup and its rows; one launch holds the leaves
    // of every super-tile
    const int st = blockIdx.x / p.blocks_per_tile, lb = blockIdx.x - st * p.blocks_per_tile;
    const int row_end = min(p.Nq, (st + 1) * p.br);
    const int qrow = st * p.br + lb * kBQ + wq * 16 + q;   // this lane's query row
    const bool qin = qrow < row_end;
    const int ni = (p.Nk + KI - 1) / KI;

    // ---- Q operand, held for the whole key loop: c * Q[qrow][16g + j] ----
    // The scores come out in base-2 exponent units, scale * log2(e) * S0, so
    // the softmax needs no multiply per score.
    const float c = p.scale * kLog2e;
    float qv[16];
    {
        const float* src = p.Q + (int64_t)qrow * p.ldq + 16 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 v = qin ? load4<VEC>(src + 4 * j, 4) : f32x4{0.f, 0.f, 0.f, 0.f};
            qv[4 * j] = v[0] * c;
            qv[4 * j + 1] = v[1] * c;
            qv[4 * j + 2] = v[2] * c;
            qv[4 * j + 3] = v[3] * c;
        }
    }

    // ---- K / V rows of one step: thread t moves 16-byte pieces t + NT*i ----
    // DMA: direct global-to-LDS loads, no registers and no LDS stores.  The
    // wave's i-th load fills the 64 16-byte slots (i*NW + wave)*64 + lane of
    // a tile; slot u holds row u/16 and stored piece u%16, which for K is
    // logical piece (u%16) ^ swizzle(row), so the swizzle is applied to the
    // global address.  Each load takes the step's first row as a
    // wave-uniform base and a 32-bit byte offset per lane.  Rows past Nk read
    // row Nk-1 instead: their scores are masked and their weights are 0.  The
    // loads of step it+1 are issued at the start of step it and land by the
    // barrier that ends it.
    // Otherwise the rows come through registers and are stored to LDS before
    // that barrier.
    constexpr int NW = NT / 64;
    f32x4 sk[DMA ? 1 : LD], sv[DMA ? 1 : LD];
    auto issue_dma = [&](const float* src, int64_t ld, int it, char* tile, bool swizzled) {
        const int k0 = it * KI, last = p.Nk - 1 - k0;
        const float* base = src + (int64_t)k0 * ld;
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int u = (i * NW + wave) * 64 + lane, row = u >> 4, sp = u & 15;
            const int lp = swizzled ? kswz(row, sp) : sp;
            const uint32_t off = ((uint32_t)min(row, last) * (uint32_t)ld + 4 * lp) * 4;
            dma16s(base, off, tile + (i * NW + wave) * 1024);
        }
    };
    auto load_rows = [&](const float* src, int64_t ld, int it, f32x4* dst) {
        const int k0 = it * KI;
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int u = t + NT * i, row = u >> 4, piece = u & 15, key = k0 + row;
            dst[i] = key < p.Nk ? load4<VEC>(src + (int64_t)key * ld + 4 * piece, 4)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    // the loads of step it into K stage it & 1 and V stage it % 3
    auto fetch = [&](int it) {
        if constexpr (DMA) {
            issue_dma(p.K, p.ldk, it, kring + (it & 1) * TILE, true);
            issue_dma(p.V, p.ldv, it, vring + (it % 3) * TILE, false);
        } else {
            load_rows(p.K, p.ldk, it, sk);
            load_rows(p.V, p.ldv, it, sv);
        }
    };
    auto store_k = [&](int buf) {
        if constexpr (DMA) return;
        char* ks = kring + buf * TILE;
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int u = t + NT * i, row = u >> 4, piece = u & 15;
            *reinterpret_cast<f32x4*>(ks + row * kRowB + 16 * kswz(row, piece)) = sk[i];
        }
    };
    auto store_v = [&](int buf) {
        if constexpr (DMA) return;
        char* vs = vring + buf * TILE;
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int u = t + NT * i;
            *reinterpret_cast<f32x4*>(vs + (u >> 4) * kRowB + 16 * (u & 15)) = sv[i];
        }
    };
    // S^T for this wave's KW keys of a step (rows KW*half .. +KW-1 of the
    // stage), in NSB sub-blocks of 16: s[kb][r] = S[qrow][kbase + 16kb + r]
    // The sub-blocks' accumulations are interleaved, so that an MFMA never
    // waits for the result of the one just before it.
    auto scores = [&](int buf, f32x4* s) {
        const char* ks = kring + buf * TILE + half * (KW * kRowB);
#pragma unroll
        for (int kb = 0; kb < NSB; ++kb) s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // K fragments read two k-chunks ahead of the MFMAs that use them, so
        // their LDS latency hides behind MFMAs instead of stalling the wave
        f32x4 a[3][NSB];
        auto read_k = [&](int cc, f32x4* dst) {
#pragma unroll
            for (int kb = 0; kb < NSB; ++kb) {
                const int krow = 16 * kb + q;             // A' row of this lane
                // the swizzle of row KW*half + krow is that of krow (KW = 0 mod 16)
                dst[kb] = *reinterpret_cast<const f32x4*>(ks + krow * kRowB + 16 * kswz(krow, 4 * g + cc));
            }
        };
        read_k(0, a[0]);
        read_k(1, a[1]);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            if (cc + 2 < 4) read_k(cc + 2, a[(cc + 2) % 3]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int kb = 0; kb < NSB; ++kb)
                    s[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[cc % 3][kb][e], qv[4 * cc + e], s[kb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    float m = -INFINITY;                // running maximum (base 2), same in the 4 lanes of q
    float l = 0.0f;                     // this lane's part of the running weight sum
    f32x4 o[4];                         // O^T blocks: o[db][r] = O[qrow][16g + 4r + db]
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    // softmax of one step's scores s (in place) and the output products
    auto consume = [&](int it, f32x4* s, int vstage) {
        // the first two V fragments are read before the softmax, the others
        // two groups of MFMAs ahead of their use
        const char* vs = vring + vstage * TILE + half * (KW * kRowB);
        auto read_v = [&](int ts) {
            const int vrow = 16 * (ts >> 2) + 4 * g + (ts & 3);
            return *reinterpret_cast<const f32x4*>(vs + vrow * kRowB + 16 * q);
        };
        f32x4 va[3];
        va[0] = read_v(0);
        va[1] = read_v(1);
        // online softmax in base 2; keys past Nk weigh nothing (only the
        // last step can hold any)
        float bm = -INFINITY;
        if ((it + 1) * KI > p.Nk) {
            const int kbase = it * KI + half * KW + 4 * g;
#pragma unroll
            for (int kb = 0; kb < NSB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (kbase + 16 * kb + r >= p.Nk) s[kb][r] = -INFINITY;
        }
#pragma unroll
        for (int kb = 0; kb < NSB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) bm = fmaxf(bm, s[kb][r]);
        bm = quad_max(bm);
        const float mn = fmaxf(m, bm);
        const bool grew = mn > m;
        // a key half that has met no key yet keeps weight 0 (not exp2(-inf + inf))
        const float base = (mn == -INFINITY) ? 0.0f : mn;
        const float alpha = __builtin_amdgcn_exp2f(m - base);   // 0 until a key is met
        m = mn;
        // The running output and weight sum are rescaled first, so that the
        // output products need not wait for the multiplies, and only when the
        // maximum of some lane of the wave grew: otherwise alpha is exactly 1
        // (or o and l are still 0) and they would change nothing.
        if (__builtin_amdgcn_ballot_w64(grew) != 0) {
            l *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db) o[db] *= alpha;
        }
#pragma unroll
        for (int kb = 0; kb < NSB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) s[kb][r] = __builtin_amdgcn_exp2f(s[kb][r] - base);
        // the step's weights summed pairwise (short dependency chains)
        float part[NSB];
#pragma unroll
        for (int kb = 0; kb < NSB; ++kb) part[kb] = (s[kb][0] + s[kb][1]) + (s[kb][2] + s[kb][3]);
        float bl = part[0];
#pragma unroll
        for (int kb = 1; kb < NSB; ++kb) bl += part[kb];
        l += bl;

        // O^T += V^T P^T: step ts uses keys 16(ts/4) + 4g + ts%4 (lane group g)
#pragma unroll
        for (int ts = 0; ts < 4 * NSB; ++ts) {
            if (ts + 2 < 4 * NSB) va[(ts + 2) % 3] = read_v(ts + 2);
            __builtin_amdgcn_sched_barrier(0);
            const float w = s[ts >> 2][ts & 3];
#pragma unroll
            for (int db = 0; db < 4; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[ts % 3][db], w, o[db], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

  if constexpr (DMA) {
    // Scores one step ahead: in step it the wave forms the scores of step
    // it+1 (K stage (it+1) % 3) before the softmax and output products of
    // step it (V stage it & 1), so its exponentials of step it can overlap
    // its own MFMAs.  K(it+2) and V(it+1) are loaded meanwhile.  K needs three
    // stages: K(it+2) is issued at the start of step it, when K(it+1) is
    // about to be read and a wave may still be reading K(it) (the scores of
    // step 0 run before the loop, with no barrier after them).
    issue_dma(p.K, p.ldk, 0, kring, true);
    issue_dma(p.V, p.ldv, 0, vring, false);
    if (ni > 1) issue_dma(p.K, p.ldk, 1, kring + TILE, true);
    __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
    __syncthreads();
    f32x4 s[NSB];
    scores(0, s);
    int k1 = 1, k2 = 2;                  // K stages of steps it+1 and it+2
    for (int it = 0; it < ni; ++it) {
        // K stage k2 held K(it-1), read in step it-2 (or never, for it = 0);
        // V stage (it+1) & 1 held V(it-1), read in step it-1
        if (it + 2 < ni) issue_dma(p.K, p.ldk, it + 2, kring + k2 * TILE, true);
        if (it + 1 < ni) issue_dma(p.V, p.ldv, it + 1, vring + ((it + 1) & 1) * TILE, false);
        f32x4 sn[NSB];
#pragma unroll
        for (int kb = 0; kb < NSB; ++kb) sn[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (it + 1 < ni) scores(k1, sn);
        consume(it, s, it & 1);
        k1 = k2;
        k2 = (k2 == 2) ? 0 : k2 + 1;
        __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < NSB; ++kb) s[kb] = sn[kb];
    }
  } else {
    fetch(0);
    store_k(0);
    store_v(0);
    __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
    __syncthreads();
    f32x4 s[NSB];
    for (int it = 0; it < ni; ++it) {
        const bool more = it + 1 < ni;
        if (more) fetch(it + 1);
        if (half == 0) {
            scores(it & 1, s);
            consume(it, s, it % 3);
        } else {
            // half a step behind: the previous step's softmax and output
            // products first, then this step's scores
            if (it > 0) consume(it - 1, s, (it - 1) % 3);
            scores(it & 1, s);
        }
        // K stage (it+1) & 1 held K(it-1) and V stage (it+1) % 3 held
        // V(it-2): both last read before the previous barrier
        if (more) {
            store_k((it + 1) & 1);
            store_v((it + 1) % 3);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVm<0>);   // this wave's loads of step it+1
        __syncthreads();
    }
    if (half == 1) consume(ni - 1, s, (ni - 1) % 3);
  }

    {
        // merge the other key parts into the first: all hold the same lanes'
        // queries and output columns; the K ring (2 * TILE bytes, room for
        // 3 parts x 4 groups x 64 lanes x 18 floats) is free after the last
        // barrier (the last output products read the V ring).  Parts are
        // added in order 1, 2, 3, each rescaled to the larger maximum.
        static_assert((KSPLIT - 1) * 4 * 64 * 18 * 4 <= 2 * TILE, "merge area in the K ring");
        float* x = reinterpret_cast<float*>(lds) + (((half - 1) * 4 + wq) * 64 + lane) * 18;
        if (half != 0) {
            x[0] = m;
            x[1] = l;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) x[2 + 4 * db + r] = o[db][r];
        }
        __syncthreads();
        if (half != 0) return;
#pragma unroll
        for (int part = 1; part < KSPLIT; ++part) {
            const float* y = reinterpret_cast<const float*>(lds) + (((part - 1) * 4 + wq) * 64 + lane) * 18;
            const float m2 = y[0], mm = fmaxf(m, m2);
            // a part that has met no key keeps weight 0 (not exp2(-inf + inf))
            const float f1 = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mm);
            const float f2 = (m2 == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m2 - mm);
            m = mm;
            l = l * f1 + y[1] * f2;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) o[db][r] = o[db][r] * f1 + y[2 + 4 * db + r] * f2;
        }
    }

    // ---- epilogue: the weight sum over all keys, O = o / l ----
    l = quad_sum(l);
    if (!qin) return;
    const float inv = 1.0f / l;
    float* dst = p.O + (int64_t)qrow * p.ldo + 16 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const f32x4 v = {o[0][r] * inv, o[1][r] * inv, o[2][r] * inv, o[3][r] * inv};
        if (VEC) {
            *reinterpret_cast<f32x4*>(dst + 4 * r) = v;
        } else {
            dst[4 * r] = v[0];
            dst[4 * r + 1] = v[1];
            dst[4 * r + 2] = v[2];
            dst[4 * r + 3] = v[3];
        }
    }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& p, bool vec, hipStream_t stream) {
    // KS waves per query group: at 16384 queries one 16-query wave per SIMD
    // left latency exposed (87-92 TFLOP/s); two per SIMD reached 103-107
    constexpr int KS = 2;
    constexpr int KS_DMA = PHOBOS_ATT_KSPLIT;
    const int64_t tiles = (p.Nq + (int64_t)p.br - 1) / p.br;
    const dim3 grid((unsigned)(tiles * p.blocks_per_tile));
    // direct loads when 32-bit byte offsets cover the rows of one step of K
    // and of V, and the rows are 16-byte aligned
    const int64_t span = ((int64_t)(kKI - 1) * std::max(p.ldk, p.ldv) + kD) * 4;
    if (vec && span <= (int64_t)UINT32_MAX)
        hipLaunchKernelGGL((attention_kernel<true, true, KS_DMA>), grid, dim3(256 * KS_DMA), 0,
                           stream, p);
    else if (vec)
        hipLaunchKernelGGL((attention_kernel<true, false, KS>), grid, dim3(256 * KS), 0, stream, p);
    else
        hipLaunchKernelGGL((attention_kernel<false, false, KS>), grid, dim3(256 * KS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace phobos
