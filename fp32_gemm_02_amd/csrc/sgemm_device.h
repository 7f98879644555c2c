// Device helpers shared by the fp32 kernels (sgemm_kernels.hip) and the
// matrix-core variant (sgemm_tc.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgemm_internal.h"

namespace phobos {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Map the workgroup to its output tile.  Workgroups are handed to the 8 XCDs
// of the chip round robin (id % 8); with xcd_remap the ids an XCD receives
// become one contiguous run of the raster order, so tiles that share rows of
// A and columns of B sit in the same L2.  The raster walks group_m tile rows
// at a time, column by column, to keep the A panels of a group hot.
template <class Args>
__device__ __forceinline__ void tile_of(const Args& p, int& tm, int& tn) {
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

// Four floats at 4-byte alignment: one 16-byte global load all the same
// (gfx9 global memory instructions take dword-aligned addresses for wider
// accesses), where the compiler would otherwise issue four dword loads.
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x2u __attribute__((ext_vector_type(2), aligned(4)));

// Load 4 consecutive floats src[0..3] whose positions are valid while
// e < nvalid (nvalid <= 0: all zero).  VEC: src is 16-byte aligned;
// otherwise 4-byte aligned, and a piece wholly inside is still read with
// one 16-byte load.
template <bool VEC>
__device__ __forceinline__ f32x4 load4(const float* src, int nvalid) {
    f32x4 v;
    if (VEC && nvalid >= 4) {
        v = *reinterpret_cast<const f32x4*>(src);
    } else if (nvalid >= 4) {
        v = *reinterpret_cast<const f32x4u*>(src);
    } else {
        v[0] = nvalid > 0 ? src[0] : 0.0f;
        v[1] = nvalid > 1 ? src[1] : 0.0f;
        v[2] = nvalid > 2 ? src[2] : 0.0f;
        v[3] = nvalid > 3 ? src[3] : 0.0f;
    }
    return v;
}

// XOR swizzle of the 16-byte pieces of one A-tile row in LDS (QA pieces per
// row): piece q of row r is stored at position q ^ swz(r).  It depends on
// r mod 16 only.  For the MFMA reads (32 rows, one piece each) any 8
// consecutive lanes then touch 8 different 16-byte bank groups of a 128-byte
// line, and any 16 consecutive lanes 16 different groups of a 256-byte line,
// so the reads are conflict free whether the LDS serves 8 or 16 lanes of a
// 128-bit read per cycle.
template <int QA>
__device__ __forceinline__ int swz(int r) {
    if constexpr (QA == 8) return (r & 7) ^ ((r >> 3) & 1);
    else return ((r >> 1) & 3) ^ ((r >> 3) & 1);
}

// One direct global-to-LDS load: every lane fetches the 16 bytes at its `src`
// and the wave writes them to LDS at lds_dst + 16*lane (lds_dst is the same
// for the whole wave; it goes in M0).  Issued as inline assembly so that the
// compiler's wait-count analysis does not see an instruction that touches
// both memory and LDS: that would make it wait for every outstanding LDS read
// (lgkmcnt(0)) at each use, where one k-step of lookahead is intended.  The
// kernel therefore waits for these loads itself (vmcnt) before the barrier
// that publishes a stage.  Vector-memory loads complete in issue order, so
// loads the compiler does not track can only make its own waits stricter.
__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_dst;
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// The same load with a wave-uniform 64-bit base (held in scalar registers)
// and a 32-bit per-lane byte offset: lane l fetches the 16 bytes at
// base + voff.  Interleaved between MFMAs, the form with a 64-bit address per
// lane cost about 2% of the matrix-core rate in a register-only timing test
// and this form nothing measurable, so it is the one the GEMM kernels use
// wherever their offsets fit in 32 bits.
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, void* lds_dst) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_dst;
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(m0) : "memory");
}

// s_waitcnt immediate (gfx9 encoding) waiting for at most N outstanding
// vector-memory loads and for every LDS access; exports are not waited for.
template <int N>
constexpr int kWaitVm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8);
static_assert(kWaitVm<0> == 0x70 && kWaitVm<4> == 0x74, "s_waitcnt encoding");

// NB consecutive floats of B read with one LDS instruction, and element n of
// it; utype is the same NB floats at 4-byte alignment, for global accesses at
// any float position.
template <int NB> struct BVec;
template <> struct BVec<1> {
    using type = float;
    using utype = float;
    static __device__ __forceinline__ float get(float v, int) { return v; }
    static __device__ __forceinline__ void set(float& v, int, float x) { v = x; }
};
template <> struct BVec<2> {
    using type = f32x2;
    using utype = f32x2u;
    static __device__ __forceinline__ float get(f32x2 v, int n) { return v[n]; }
    static __device__ __forceinline__ void set(f32x2& v, int n, float x) { v[n] = x; }
};
// Three floats as a plain struct: an ext_vector_type of 3 is 16 bytes wide
// and 16-byte aligned, so its loads and stores would touch a fourth float.
struct f32x3s {
    float v[3];
};
template <> struct BVec<3> {
    using type = f32x3s;
    using utype = f32x3s;
    static __device__ __forceinline__ float get(const f32x3s& v, int n) { return v.v[n]; }
    static __device__ __forceinline__ void set(f32x3s& v, int n, float x) { v.v[n] = x; }
};
template <> struct BVec<4> {
    using type = f32x4;
    using utype = f32x4u;
    static __device__ __forceinline__ float get(f32x4 v, int n) { return v[n]; }
    static __device__ __forceinline__ void set(f32x4& v, int n, float x) { v[n] = x; }
};

// Epilogue of one lane's share of a 32-row block of C that may reach past
// an edge of the matrix: for r = 0..15, row = row0 + 8*(r/4) + r%4, and
// n = 0..NB-1, C[row][col+n] <- alpha*acc(n, r) + beta*C[row][col+n] where
// row < M and col+n < N (beta == 0: C not read); nothing past M or N is
// written.  RB rows form a batch: their C values are read before any of them
// is written.  The reads take no branch: a row past M reads row M-1, and a
// lane whose NB columns pass N reads the NB columns that end at column N-1
// and moves the ones it needs into place, so every read lies inside C and
// feeds only elements that are stored.  Reads under per-lane bounds checks
// made the compiler wait for every outstanding access before each row, one
// memory round trip per row.  After the batch's one wait its results are all
// formed, then its guarded stores issue back to back.  A lane whose NB
// columns lie inside C writes them with one access.  Needs M >= 1.
template <int NB, int RB, typename Acc>
__device__ __forceinline__ void edge_block_epilogue(float* C, int64_t ldc, int M, int N, int row0,
                                                    int col, float alpha, float beta, Acc acc) {
    static_assert(16 % RB == 0, "whole batches of rows");
    using CV = typename BVec<NB>::type;
    using UV = typename BVec<NB>::utype;
    const int ncols = N - col;
    auto row_of = [&](int r) { return row0 + 8 * (r >> 2) + (r & 3); };
    if (N < NB) {
        // C narrower than one lane's NB columns: element by element.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (row_of(r) >= M) continue;
            float* dst = C + (int64_t)row_of(r) * ldc + col;
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                if (n >= ncols) continue;
                float v = alpha * acc(n, r);
                if (beta != 0.0f) v += beta * dst[n];
                dst[n] = v;
            }
        }
        return;
    }
    const bool wide = ncols >= NB;   // all NB columns of the lane inside C
    // First column read by the lane and how far its wanted columns sit past
    // it (0 for a wide lane, 1..NB-1 for one that straddles N, more for a
    // lane wholly past N, whose values go unused).
    const int cs = min(col, N - NB);
    const int sh = col - cs;
#pragma unroll
    for (int rb = 0; rb < 16; rb += RB) {
        CV cv[RB];
        if (beta != 0.0f) {
#pragma unroll
            for (int e = 0; e < RB; ++e)
                cv[e] = *reinterpret_cast<const UV*>(C + (int64_t)min(row_of(rb + e), M - 1) * ldc + cs);
            __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
            if constexpr (NB > 1) {
#pragma unroll
                for (int e = 0; e < RB; ++e) {
                    const CV x = cv[e];
#pragma unroll
                    for (int n = 0; n < NB; ++n) {
                        float v = BVec<NB>::get(x, n);
#pragma unroll
                        for (int s = 1; n + s < NB; ++s) v = sh == s ? BVec<NB>::get(x, n + s) : v;
                        BVec<NB>::set(cv[e], n, v);
                    }
                }
            }
        }
#pragma unroll
        for (int e = 0; e < RB; ++e) {
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                float v = alpha * acc(n, rb + e);
                if (beta != 0.0f) v += beta * BVec<NB>::get(cv[e], n);
                BVec<NB>::set(cv[e], n, v);
            }
        }
#pragma unroll
        for (int e = 0; e < RB; ++e) {
            const int row = row_of(rb + e);
            if (row >= M || ncols <= 0) continue;
            float* dst = C + (int64_t)row * ldc + col;
            if (wide) {
                *reinterpret_cast<UV*>(dst) = cv[e];
            } else {
#pragma unroll
                for (int n = 0; n < NB; ++n)
                    if (n < ncols) dst[n] = BVec<NB>::get(cv[e], n);
            }
        }
    }
}

}  // namespace phobos

