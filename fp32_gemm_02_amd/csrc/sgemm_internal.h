// Internal interface between the C-ABI layer (sgemm_api.cpp) and the gfx950
// kernels (sgemm_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "phobos_sgemm.h"

namespace phobos {

// Everything one GEMM launch needs.  Dimensions fit in int32 (the API layer
// rejects larger ones); element offsets are formed in 64 bits.
struct GemmArgs {
    int32_t M, N, K;
    float alpha, beta;
    const float* A;
    int64_t lda;
    const float* B;
    int64_t ldb;
    float* C;
    int64_t ldc;
    int32_t tiles_m, tiles_n;   // ceil(M/bm), ceil(N/bn)
    int32_t group_m;            // tile rows per raster group (>= 1)
    int32_t xcd_remap;          // 1: tiles_m*tiles_n % 8 == 0, spread groups per XCD
};

using GemmLaunchFn = hipError_t (*)(const GemmArgs&, hipStream_t);

struct KernelEntry {
    sgemm_config cfg;
    int32_t threads;      // 64 * wm * wn
    int32_t lds_bytes;    // static LDS of the kernel
    GemmLaunchFn vec4;    // needs 16-byte aligned A, B, C and lda, ldb, ldc % 4 == 0
    GemmLaunchFn scalar;  // any alignment
};

// The compiled configurations (count written to *count).
const KernelEntry* kernel_table(int* count);
// The split-K entries (sgemm_splitk.hip), listed after kernel_table's.
const KernelEntry* splitk_kernel_table(int* count);

// The compiled configurations of the matrix-core variant for input format
// fmt (SGEMM_TC_F16 or SGEMM_TC_BF16); nullptr and *count = 0 otherwise.
const KernelEntry* tc_kernel_table(int fmt, int* count);

// Staged form of the matrix-core variant: the 16-bit operands prepared by
// the cast pass (A16: Mp x Kp row-major; B16: B transposed, Np x Kp; both
// with row pitch Kp, zero past the real M, N, K) and the fp32 output.
struct Tc16Args {
    const uint16_t* A;
    const uint16_t* B;
    int64_t ld;                 // Kp
    int32_t M, N, K;            // real M and N; K = Kp
    float alpha, beta;
    float* C;
    int64_t ldc;
    int32_t vec_c;              // C 16-byte aligned and ldc % 4 == 0
    int32_t tiles_m, tiles_n;   // ceil(M/bm), ceil(N/bn)
    int32_t group_m, xcd_remap;
};
using Tc16LaunchFn = hipError_t (*)(const Tc16Args&, hipStream_t);
struct Tc16Entry {
    sgemm_config cfg;
    int32_t stages;       // LDS ring depth
    int32_t threads;
    int32_t lds_bytes;
    Tc16LaunchFn launch;
};
// Tiles of the staged GEMM divide 256 x 256 and chunks divide 64, so the
// cast pass pads M and N to multiples of 256 and K to a multiple of 64.
constexpr int kTcPadMN = 256, kTcPadK = 64;
const Tc16Entry* tc16_kernel_table(int fmt, int* count);
// The cast pass: A16 and B16 from A and B (vec_*: 16-byte aligned rows).
hipError_t launch_tc_cast(int fmt, const float* A, int64_t lda, bool vec_a, const float* B,
                          int64_t ldb, bool vec_b, int M, int N, int K, uint16_t* A16,
                          uint16_t* B16, int Mp, int Np, int Kp, hipStream_t stream);

// Device address of the static workspace of SGEMM_TC_SCRATCH_BYTES on the
// current device (sgemm_tc.hip), looked up on the first call on each device;
// nullptr with *err set when the lookup fails.
constexpr int kMaxDevices = 64;
void* tc_scratch(hipError_t* err);

// Attention O = softmax(scale * Q K^T) V over query rows 0 .. Nq-1 of the
// given pointers, head dimension 64 (attention.hip), as one launch holding
// the leaves of every super-tile of br rows.
struct AttnArgs {
    int32_t Nq, Nk;
    const float* Q;
    int64_t ldq;
    const float* K;
    int64_t ldk;
    const float* V;
    int64_t ldv;
    float* O;
    int64_t ldo;
    float scale;
    int32_t br;                 // query rows per super-tile (Nq: one super-tile)
    int32_t blocks_per_tile;    // ceil(br / 64) workgroups per super-tile
};
// vec: Q, K, V, O 16-byte aligned with leading dimensions % 4 == 0.
hipError_t launch_attention(const AttnArgs& p, bool vec, hipStream_t stream);

// C <- beta*C over an M x N view (beta == 0: C <- 0 without reading C).
hipError_t launch_init_leaf(int64_t M, int64_t N, float beta, float* C, int64_t ldc,
                            hipStream_t stream);

// Fill n floats with a fixed pseudo-random pattern in [-1, 1) (tuner scratch).
hipError_t launch_fill_pattern(float* p, int64_t n, uint32_t seed, hipStream_t stream);

}  // namespace phobos
