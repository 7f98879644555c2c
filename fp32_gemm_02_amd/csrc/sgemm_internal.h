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

// The compiled configurations of the matrix-core variant for input format
// fmt (SGEMM_TC_F16 or SGEMM_TC_BF16); nullptr and *count = 0 otherwise.
const KernelEntry* tc_kernel_table(int fmt, int* count);

// C <- beta*C over an M x N view (beta == 0: C <- 0 without reading C).
hipError_t launch_init_leaf(int64_t M, int64_t N, float beta, float* C, int64_t ldc,
                            hipStream_t stream);

// Fill n floats with a fixed pseudo-random pattern in [-1, 1) (tuner scratch).
hipError_t launch_fill_pattern(float* p, int64_t n, uint32_t seed, hipStream_t stream);

}  // namespace phobos
