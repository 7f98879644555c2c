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
// one launch.  One workgroup (4 waves) owns 64 query rows, 16 per wave, of
// its super-tile, and walks the keys
// in blocks of 64 staged through LDS (K and V, double-buffered, loaded one
// block ahead through registers).  Both products run on the FP32 matrix cores
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

#include "sgemm_device.h"
#include "sgemm_internal.h"

namespace phobos {

namespace {

constexpr int kD = 64;      // head dimension
constexpr int kBQ = 64;     // query rows per workgroup (16 per wave)
constexpr int kBC = 64;     // keys per block
constexpr int kRowB = kD * 4;                      // bytes of one K or V row in LDS
constexpr int kTile = kBC * kRowB;                 // bytes of one K or V tile
constexpr int kStage = 2 * kTile;                  // K and V
constexpr float kLog2e = 1.4426950408889634f;

// K rows are stored with their 16-byte pieces XOR-swizzled by row, so the
// 16 lanes that read one piece of 16 consecutive rows hit 16 different bank
// groups (and 8 consecutive lanes 8 different ones of a 128-byte line).
__device__ __forceinline__ int kswz(int row, int piece) { return piece ^ (row & 15); }

template <bool VEC>
__global__ __launch_bounds__(256) void attention_kernel(AttnArgs p) {
    __shared__ __attribute__((aligned(16))) char lds[2 * kStage];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int q = lane & 15, g = lane >> 4;
    // super-tile of this workgroup and its rows; one launch holds the leaves
    // of every super-tile
    const int st = blockIdx.x / p.blocks_per_tile, lb = blockIdx.x - st * p.blocks_per_tile;
    const int row_end = min(p.Nq, (st + 1) * p.br);
    const int qrow = st * p.br + lb * kBQ + wave * 16 + q;   // this lane's query row
    const bool qin = qrow < row_end;
    const int nb = (p.Nk + kBC - 1) / kBC;

    // ---- Q operand, held for the whole key loop: Q[qrow][16g + j] ----
    float qv[16];
    {
        const float* src = p.Q + (int64_t)qrow * p.ldq + 16 * g;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const f32x4 v = qin ? load4<VEC>(src + 4 * c, 4) : f32x4{0.f, 0.f, 0.f, 0.f};
            qv[4 * c] = v[0];
            qv[4 * c + 1] = v[1];
            qv[4 * c + 2] = v[2];
            qv[4 * c + 3] = v[3];
        }
    }

    // ---- K / V tiles: thread t moves 16-byte pieces (t + 256*i) of each ----
    f32x4 sk[4], sv[4];
    auto load = [&](int b) {
        const int k0 = b * kBC;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int u = t + 256 * i, row = u >> 4, piece = u & 15, key = k0 + row;
            const bool in = key < p.Nk;
            sk[i] = in ? load4<VEC>(p.K + (int64_t)key * p.ldk + 4 * piece, 4)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
            sv[i] = in ? load4<VEC>(p.V + (int64_t)key * p.ldv + 4 * piece, 4)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto store = [&](int buf) {
        char* ks = lds + buf * kStage;
        char* vs = ks + kTile;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int u = t + 256 * i, row = u >> 4, piece = u & 15;
            *reinterpret_cast<f32x4*>(ks + row * kRowB + 16 * kswz(row, piece)) = sk[i];
            *reinterpret_cast<f32x4*>(vs + row * kRowB + 16 * piece) = sv[i];
        }
    };

    const float c = p.scale * kLog2e;   // scores in base-2 exponent units
    float m = -INFINITY;                // running maximum (base 2), same in the 4 lanes of q
    float l = 0.0f;                     // this lane's part of the running weight sum
    f32x4 o[4];                         // O^T blocks: o[db][r] = O[qrow][16g + 4r + db]
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    load(0);
    store(0);
    __syncthreads();
    for (int b = 0; b < nb; ++b) {
        const bool more = b + 1 < nb;
        if (more) load(b + 1);
        const char* ks = lds + (b & 1) * kStage;
        const char* vs = ks + kTile;

        // S^T for the 4 sub-blocks of 16 keys: s[kb][r] = S[qrow][64b + 16kb + 4g + r]
        f32x4 s[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int krow = 16 * kb + q;                 // A' row of this lane
            const char* kr = ks + krow * kRowB;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(kr + 16 * kswz(krow, 4 * g + cc));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], qv[4 * cc + e], s[kb], 0, 0, 0);
            }
        }

        // online softmax in base 2; keys past Nk weigh nothing
        const int kbase = b * kBC + 4 * g;
        float bm = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = s[kb][r] * c;
                if (kbase + 16 * kb + r >= p.Nk) x = -INFINITY;
                s[kb][r] = x;
                bm = fmaxf(bm, x);
            }
        bm = fmaxf(bm, __shfl_xor(bm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float mn = fmaxf(m, bm);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);   // 0 on the first block
        m = mn;
        float bl = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float w = __builtin_amdgcn_exp2f(s[kb][r] - mn);
                s[kb][r] = w;
                bl += w;
            }
        l = l * alpha + bl;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;

        // O^T += V^T P^T: step ts uses keys 16(ts/4) + 4g + ts%4 (lane group g)
#pragma unroll
        for (int ts = 0; ts < 16; ++ts) {
            const int vrow = 16 * (ts >> 2) + 4 * g + (ts & 3);
            const f32x4 a = *reinterpret_cast<const f32x4*>(vs + vrow * kRowB + 16 * q);
            const float w = s[ts >> 2][ts & 3];
#pragma unroll
            for (int db = 0; db < 4; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[db], w, o[db], 0, 0, 0);
        }

        // the other buffer was last read before the previous barrier
        if (more) store((b + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: the weight sum over all keys, O = o / l ----
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
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
    const int64_t tiles = (p.Nq + (int64_t)p.br - 1) / p.br;
    const dim3 grid((unsigned)(tiles * p.blocks_per_tile)), block(256);
    if (vec)
        hipLaunchKernelGGL(attention_kernel<true>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(attention_kernel<false>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace phobos
