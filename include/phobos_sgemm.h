/*
 * phobos_sgemm.h -- C ABI of the MI355X (gfx950) FP32 SGEMM library.
 *
 * The operation is C <- alpha*A*B + beta*C on 32-bit floats, as defined in
 * "Show HN: Phobos - A tiny scale-free kernel language with tile-DAG
 * support", section "Matrix Multiplication", and its two-level form with
 * super-tiles and a cluster loop over K from the Phobos "@cluster" attribute
 * page, section "What the cluster compiler accepts".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  All matrices are row-major: element (i, j) of X is X[i*ldx + j].
 *   A is M x K (lda >= max(1, K)), B is K x N (ldb >= max(1, N)),
 *   C is M x N (ldc >= max(1, N)).  Elements past the logical width of a row
 *   (the pads) are never written and never reach a result, whatever they hold
 *   (NaN and Inf included).  Some of them may be read: in the fp32 GEMM
 *   kernels, when a tile at the right edge of C loads a 16-byte piece of a
 *   row of B that straddles column N-1, the piece's floats past N-1 (at most
 *   three, always before column ldb: that load path needs ldb % 4 == 0) are
 *   read and then feed only columns of the tile that are not stored.  Rows
 *   of a tile past M read row M-1 of A instead, and are not stored either.
 *   Rows past the last one are never read.  No other kernel reads a pad.
 *   C is read (beta != 0) only inside the logical matrix: a tile at an edge
 *   of C reads row M-1 and columns up to N-1 in place of those past the
 *   edges, and those values feed only elements that are not stored.
 * Memory.  A, B and C are device pointers (hipMalloc'ed or equivalent) owned
 *   by the caller.  The library neither frees nor retains them.  They must
 *   stay valid until the work enqueued on `stream` has finished.  C must not
 *   overlap A or B (not checked).  The GEMM entry points allocate nothing.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 *   stream).  Calls are asynchronous: they enqueue kernels and return without
 *   synchronising.
 * beta == 0.  C is write-only: it is never read, so it may hold NaN or Inf,
 *   and the result is alpha*A*B exactly as if C had been zero.
 * Quick returns.  M == 0 or N == 0: nothing is enqueued.  K == 0 or
 *   alpha == 0: A and B are not read and C <- beta*C (beta == 1: nothing is
 *   enqueued; beta == 0: C <- 0).
 * Accuracy.  Products and sums are fp32 (MFMA fp32 arithmetic, sums in an
 *   order of the library's choosing), so results are within
 *   2*K*2^-24*(|alpha|*(|A||B|)ij + |beta*Cij|) + 1e-30 of the exact value,
 *   and exact whenever every partial sum is representable in fp32.
 * Errors.  0 = success.  A negative value -i = the i-th argument is invalid
 *   (numbered from 1 in the order of the prototype); every argument check
 *   runs before any HIP call, so argument errors never touch the GPU.
 *   SGEMM_ERR_* below for the other failures; 1000 + e = HIP error e was
 *   reported by the runtime (hipGetLastError after the launches).
 * Threads.  Calls on different streams may run concurrently.  The config
 *   table and the trace buffer are guarded by a mutex; sgemm_tune must not
 *   run concurrently with other calls on the same device.
 */
#ifndef PHOBOS_SGEMM_H
#define PHOBOS_SGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PHOBOS_SGEMM_VERSION 1

#define SGEMM_OK 0
#define SGEMM_ERR_NO_CONFIG 2      /* no compiled kernel matches the request   */
#define SGEMM_ERR_TOO_LARGE 3      /* a dimension exceeds 2^30, or the launch   */
                                   /* grid exceeds 2^32-1 work-items           */
#define SGEMM_ERR_ALLOC 4          /* a device allocation failed               */
#define SGEMM_ERR_BUDGET 5         /* no plan fits the device memory budget    */
#define SGEMM_ERR_IO 6             /* the tuning cache file could not be read  */
                                   /* or written                               */
#define SGEMM_ERR_SCRATCH 7        /* the product's workspace exceeds the      */
                                   /* static scratch (sgemm_tc_noalloc)        */
#define SGEMM_ERR_HIP_BASE 1000    /* 1000 + hipError_t                        */

/*
 * A compiled kernel configuration: the CTA tile bm x bn (rows x columns of
 * C one workgroup owns) stepped through K in chunks of bk, computed by
 * wm x wn wavefronts of 64 lanes (workgroup = 64*wm*wn threads).  These are
 * the TILE_M / TILE_N / TILE_K of the pages' @autotune attribute ("Show HN:
 * Phobos", sections "Introducing the Phobos Language" and "Runtime").
 * An entry whose wave grid is larger than its tile's 32x32 blocks
 * (32*wm > bm or 32*wn > bn; 32x32 tiles with 4 or 8 waves, 64x64 with 4) is
 * a split-K entry: its wm*wn waves each hold the whole bm x bn tile, each
 * taking every (wm*wn)-th chunk of bk of K, and their partial sums are added
 * in wave order before the store (a fixed order, so results repeat bit for
 * bit).
 */
typedef struct sgemm_config {
    int32_t bm, bn, bk, wm, wn;
} sgemm_config;

/*
 * sgemm: C <- alpha*A*B + beta*C in one launch (the single-GPU kernel of
 * "Show HN: Phobos", section "Matrix Multiplication"; on one GPU the
 * @cluster line is ignored, "@cluster" page, section "On one GPU").
 * Arguments: 1 M, 2 N, 3 K, 4 alpha, 5 A, 6 lda, 7 B, 8 ldb, 9 beta, 10 C,
 * 11 ldc, 12 stream.  A and B may be NULL when they are not read (M, N or K
 * zero, or alpha == 0); C may be NULL when M or N is zero.
 */
int sgemm(int64_t M, int64_t N, int64_t K, float alpha,
          const float* A, int64_t lda, const float* B, int64_t ldb,
          float beta, float* C, int64_t ldc, void* stream);

/*
 * sgemm_supertiled: the same result through the two-level decomposition of
 * the "@cluster" page ("What the cluster compiler accepts": the matmul kernel
 * with a cluster loop, split into an init leaf and a step leaf, the running
 * sum kept in C itself) and the conceptual cluster IR
 * of "Show HN: Phobos", section "The DAG Compiler".
 * For each output super-tile (pm, pn) of TM x TN, in row-major order
 * (pm outer, pn inner, as the runtime deals them out, "@cluster" page,
 * "What runs today"), it enqueues on `stream`:
 *   one init leaf:  C[pm,pn] <- beta*C[pm,pn]   (0 when beta == 0, C unread)
 *   then for kt = 0 .. ceil(K/TK)-1, one step leaf:
 *                   C[pm,pn] <- alpha*A[pm,kt]*B[kt,pn] + C[pm,pn]
 * i.e. beta is hoisted into the init leaf and every step adds onto C with
 * beta = 1 ("Show HN: Phobos", section "Clustering").  C holds the
 * fp32 partial sum between steps.  Stream order makes each super-tile's steps
 * a chain.  Edge super-tiles are clipped to the matrix (the pages' runtime
 * rejects sizes that are not whole multiples; this library accepts them).
 * Arguments: 1..11 as sgemm, 12 TM, 13 TN, 14 TK (each >= 1), 15 stream.
 */
int sgemm_supertiled(int64_t M, int64_t N, int64_t K, float alpha,
                     const float* A, int64_t lda, const float* B, int64_t ldb,
                     float beta, float* C, int64_t ldc,
                     int64_t TM, int64_t TN, int64_t TK, void* stream);

/*
 * sgemm_init_leaf: the init leaf on its own, C <- beta*C over an M x N view
 * (C <- 0 without reading C when beta == 0; nothing is enqueued when
 * beta == 1).  "@cluster" page, "What the cluster compiler accepts": the init
 * leaf prepares the output super-tile (zero, or beta times its old value).
 * Arguments: 1 M, 2 N, 3 beta, 4 C, 5 ldc, 6 stream.
 */
int sgemm_init_leaf(int64_t M, int64_t N, float beta, float* C, int64_t ldc,
                    void* stream);

/*
 * Kernel configurations.
 * sgemm_config_count / sgemm_config_at list the compiled configurations
 * (index 0 .. count-1; -1 for a bad index).
 * sgemm_get_config reports the configuration sgemm would launch for this
 * shape and these leading dimensions (a forced one, else a tuned one, else
 * the built-in default); returns 0 or a negative argument error
 * (1 M, 2 N, 3 K, 4 lda, 5 ldb, 6 ldc, 7 out).
 * sgemm_set_config forces one compiled configuration for every later call in
 * the process (NULL clears the forcing); returns SGEMM_ERR_NO_CONFIG when
 * `cfg` names no compiled configuration.  Order of precedence: a config set
 * here, then the environment variable SGEMM_FORCE_CFG="BMxBNxBKxWMxWN" (read
 * once per process; ignored with a message on stderr when malformed or not
 * compiled), then a tuned config for the exact shape, then the default:
 * among the 256x256x32 (4x2 waves), 256x128x16 (4x2), 128x128x32 (2x2) and
 * single-wave 32x32 tiles (32 deep while a CU holds at most nine of them,
 * else 16 deep; 16 deep whenever K <= 16), the one with the least estimated
 * time on 256 CUs of 4 SIMDs: with T tiles the busiest CU holds
 * ceil(T/256) of them and runs its matrix cores at full rate only with at
 * least 4 waves, and a workgroup alone on its CU (a 256x256 or 320x192
 * one, or any when ceil(T/256) == 1) pays about 64 k-steps of fixed cost
 * that a second
 * resident one would hide, so the estimate is ceil(T/256) * bm * bn *
 * (K + [alone] * 64) / (rate * min(1, ceil(T/256) * waves / 4)), `rate`
 * being the tile's measured rate (1.00, 0.98, 0.90, from K = 2048 on 1.00,
 * 0.94, 0.93, and 0.60 / 0.70 for 32x32 at depth 32 / 16), and from
 * K = 2048 on also the split-K entries
 * 32x32x16 on 2x2 waves (4 waves per tile, rate 0.79) and, for more than 2560
 * 32x32 tiles, 64x64x16 on 4x1 waves (rate 0.85), and where its chunks load
 * straight into LDS (leading dimensions multiples of 4 and 16-byte aligned
 * operands) and the rows of A are 64-byte aligned (lda a multiple of 16, A
 * 64-byte aligned; sgemm_get_config, which sees no addresses, assumes aligned
 * ones) the 320x192x16 tile on 2x2 waves (rate 0.965, alone on its CU like
 * 256x256; 16 x 16 of them cover 5120 x 3072).  When the least is a 32x32
 * tile, with T 32x32 tiles: for T <= 2560, K >= 512 (except T a
 * multiple of 1024 from 2048 on with K < 4096, where two single-wave tiles
 * per SIMD already run) the split-K entry 32x32x32 on 4x2 waves if T <= 512
 * or K >= 16384, else 32x32x16 on 2x2 waves, and for 64 <= K < 512 with
 * T <= 576 the 32x32x16 2x2 entry; for T > 2560 the split-K entry when the
 * estimate picked it; otherwise one wave per tile.  The other compiled
 * configurations are there for the tuner and for forcing.
 */
int sgemm_config_count(void);
int sgemm_config_at(int32_t index, sgemm_config* out);
int sgemm_get_config(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                     int64_t ldc, sgemm_config* out);
int sgemm_set_config(const sgemm_config* cfg);

/*
 * The tile tuner, after "Show HN: Phobos", section "Runtime": every candidate
 * tile is built ahead of time; each is timed once, the best three get a
 * longer run, and the fastest of those wins.  Before the first timing the
 * built-in choice runs for about 100 ms, so that the chip's clock has risen;
 * the short timings each cover about 1 ms of launches.  The built-in choice
 * joins the longer run, which takes five rounds of `reps` runs of each
 * contender in turn and ranks them by their median; it stays the choice
 * unless another tile is more than 0.5% faster.
 * sgemm_tune_candidates (host only, no GPU work) writes into `out` (room for
 * `cap`) the compiled configurations that survive pruning for this shape:
 * tile extents inside the @autotune ranges of the "@cluster" page's matmul
 * (TILE_M, TILE_N in [32, 256], TILE_K in [4, 32]) and no tile larger than the
 * problem needs (bm <= max(32, roundup32(M)), bn <= max(32, roundup32(N))),
 * and split-K entries only when every wave gets a chunk (ceil(K/bk) >= wm*wn).
 * Returns the number of candidates, or a negative argument error
 * (1 M, 2 N, 3 K, 4 out, 5 cap).
 * sgemm_tune times the candidates on scratch buffers it allocates and frees
 * itself (inputs filled with a fixed pseudo-random pattern), then records
 * the winner for this (M, N, K, lda, ldb, ldc) so that later sgemm calls of
 * that shape use it.  `reps` is the number of timed runs of each of the top
 * three in each round (>= 1; the pages' long probe).  `winner` (may be NULL)
 * receives the choice and `winner_ms` (may be NULL) its median time per call.
 * With SGEMM_TUNE_CACHE set, the table is then saved to that file (see the
 * tuning cache below; SGEMM_ERR_IO if the save fails).  Synchronises
 * `stream`.  Arguments: 1 M, 2 N, 3 K, 4 lda, 5 ldb, 6 ldc, 7 reps,
 * 8 stream, 9 winner, 10 winner_ms.
 */
int sgemm_tune_candidates(int64_t M, int64_t N, int64_t K, sgemm_config* out,
                          int32_t cap);
int sgemm_tune(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
               int32_t reps, void* stream, sgemm_config* winner, float* winner_ms);

/*
 * Tuning cache: the tuner's table kept between processes (the pages' tuner
 * keeps nothing; this is the library's own addition).  The file is text,
 * one JSON object per line, e.g.
 *   {"M": 4096, "N": 4096, "K": 4096, "lda": 4096, "ldb": 4096, "ldc": 4096,
 *    "bm": 256, "bn": 256, "bk": 32, "wm": 2, "wn": 2}
 * (on one line; keys in any order).  sgemm_tune_cache_load adds the file's
 * entries to the in-process table, replacing entries of the same shape; a
 * line that lacks a key, names a configuration that is not compiled or a
 * shape that sgemm would reject is skipped.  `count` (may be NULL) receives
 * the number of entries taken.  Returns SGEMM_OK, -1 for a NULL path, or
 * SGEMM_ERR_IO if the file cannot be opened or read.
 * sgemm_tune_cache_save writes the whole table to `path` through a
 * temporary file in the same directory renamed into place; `count` (may be
 * NULL) receives the number of entries written.  Returns SGEMM_OK, -1 for a
 * NULL path, or SGEMM_ERR_IO on failure (the file is then unchanged).
 * sgemm_tune_forget empties the in-process table (the file is untouched)
 * and returns the number of entries removed; it cannot fail.
 * Environment: with SGEMM_TUNE_CACHE=path the file, if it exists, is loaded
 * before the process's first configuration choice, and the table is saved
 * there after every successful sgemm_tune (which then returns SGEMM_ERR_IO
 * if that save fails; the winner is recorded and reported all the same).
 * Processes that share one file: the last save wins.  Host only; no GPU work.
 */
int sgemm_tune_cache_load(const char* path, int32_t* count);
int sgemm_tune_cache_save(const char* path, int32_t* count);
int sgemm_tune_forget(void);

/*
 * Matrix-core variant ("Show HN: Phobos", section "Are we cuBLAS yet?", the
 * side-quest that casts the fp32 data to fp16 before the tensor cores and
 * keeps an fp32 accumulator).  sgemm_tc computes
 *     C <- alpha * A' * B' + beta * C
 * where A' and B' are A and B with every element rounded to the 16-bit
 * format `fmt`: SGEMM_TC_F16 (IEEE binary16) or SGEMM_TC_BF16 (bfloat16),
 * round to nearest even, values past the format's range becoming
 * infinities.  The products of the rounded values are exact and are
 * accumulated in fp32 by the 16-bit matrix instructions
 * (v_mfma_f32_32x32x16_f16 / _bf16); alpha, beta, C and the epilogue are
 * fp32.  A, B and C stay fp32 in memory.
 *
 * Two forms compute it.  Fused: the GEMM rounds each element as it loads it
 * (rounding on load, as on the pages).  Staged: a cast pass first rounds A
 * and B once into a 16-bit workspace laid out for the GEMM (A row-major, B
 * transposed, zero-padded to multiples of 256 rows and 64 columns of k),
 * then the 16-bit GEMM streams it into LDS.  Both round with the same
 * conversion.  The workspace, (ceil256(M) + ceil256(N)) * ceil64(K) * 2
 * bytes, comes from a stream-ordered memory pool of the library's own on
 * the current device (allocated and freed on `stream`; the pool keeps freed
 * memory for later calls); when it cannot be allocated, or when a tile's
 * 256 rows of it would span more than 4 GiB (the 16-bit GEMM addresses them
 * with 32-bit byte offsets), the fused form runs instead.  Under stream
 * capture the workspace's allocation and free become nodes of the graph.
 * Large products (M, N >= 2048 and K >= 1024) take the staged form by
 * default.
 *
 * Accuracy: within 2*K*2^-24 * (|alpha| sum_k |A'[i][k]| |B'[k][j]| +
 * |beta C[i][j]|) of the exact value of the expression above.  Against the
 * fp32 product the input rounding adds at most |alpha| sum_k (|a| d(b) +
 * |b| d(a) + d(a) d(b)), with d(x) = max(2^-11 |x|, 2^-25) for binary16 and
 * |x| <= 65504, and d(x) = max(2^-8 |x|, 2^-134) for bfloat16.
 *
 * Arguments 1..11, quick returns (M or N = 0: nothing; K = 0 or alpha = 0:
 * C <- beta*C, A and B not read), streams and errors as sgemm; 12 fmt (-12
 * if unknown), 13 stream.  Tile configurations (sgemm_tc_config: the tile,
 * and `staged` 1 for the staged form): sgemm_tc_config_count and
 * sgemm_tc_config_at list those compiled for a format, sgemm_tc_get_config
 * reports the one an M x N x K call would use, and sgemm_tc_set_config
 * forces one for every later call with that format (NULL: back to the
 * built-in choice; process-wide, not thread-safe against concurrent calls).
 */
#define SGEMM_TC_F16 1
#define SGEMM_TC_BF16 2

typedef struct sgemm_tc_config {
    int32_t bm, bn, bk, wm, wn;
    int32_t staged;   /* 0: rounding on load; 1: cast pass + 16-bit GEMM */
} sgemm_tc_config;

int sgemm_tc(int64_t M, int64_t N, int64_t K, float alpha, const float* A, int64_t lda,
             const float* B, int64_t ldb, float beta, float* C, int64_t ldc, int32_t fmt,
             void* stream);
/*
 * sgemm_tc_noalloc: sgemm_tc in its staged form without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture
 * that must not record allocation nodes, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, quick returns, result and errors as
 * sgemm_tc; the staged form always runs (the tile configuration forced for
 * `fmt` by sgemm_tc_set_config when that is a staged one, else
 * 256x256x64 on 4x2 waves), with the cast pass writing the 16-bit operands
 * into a static device array of SGEMM_TC_SCRATCH_BYTES (64 MiB) instead of a
 * pool allocation.  Its results are bit for bit those of sgemm_tc with the
 * same staged configuration.  The array is the library's own, one per GPU,
 * held until the process ends; its address on a GPU is looked up on the first
 * call there.  The workspace, (ceil256(M) + ceil256(N)) * ceil64(K) * 2 bytes,
 * must fit in it: larger products return SGEMM_ERR_SCRATCH before anything is
 * enqueued (e.g. 4096^3 fits exactly; 8192 x 8192 x 2048 fits; 8192^3 does
 * not).  No hipMalloc, hipFree or allocating library call is made.  Every
 * call on a GPU shares that GPU's array and the cast pass rewrites all of the
 * part a call uses (zero padding included), so nothing carries over between
 * calls; calls that overlap in time on one GPU (different streams, or
 * different host threads) race on the array and must be ordered by the caller.
 */
#define SGEMM_TC_SCRATCH_BYTES (64 * 1024 * 1024)
int sgemm_tc_noalloc(int64_t M, int64_t N, int64_t K, float alpha, const float* A,
                     int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                     int64_t ldc, int32_t fmt, void* stream);

int sgemm_tc_config_count(int32_t fmt);
int sgemm_tc_config_at(int32_t fmt, int32_t index, sgemm_tc_config* out);
int sgemm_tc_get_config(int32_t fmt, int64_t M, int64_t N, int64_t K, sgemm_tc_config* out);
int sgemm_tc_set_config(int32_t fmt, const sgemm_tc_config* cfg);

/*
 * Attention, the pages' second @cluster example ("@cluster" page, "The same
 * names at two levels": flash_attention(Q[Nq, D], K[Nk, D], V[Nk, D],
 * O[Nq, D], scale) with D = 64; its body is not on the pages, which cite the
 * FlashAttention paper).  Computes exact, unmasked attention with a row
 * softmax over the keys, in fp32:
 *     O[i][:] = sum_j P[i][j] V[j][:],
 *     P[i][j] = exp(scale * Q[i].K[j] - max_j(...)) / sum_j exp(...)
 * in one pass over the keys per block of query rows (running maximum,
 * running weight sum, running weighted sum, rescaled as the maximum grows).
 * The scores and the weighted sum run on the FP32 matrix cores.
 *
 * flash_attention computes all Nq rows as one super-tile.  flash_attention_
 * supertiled follows the pages' cluster form: super-tiles of BR query rows
 * (the pages' @cluster BR, 1024 to 4096), each worked by its own leaf, which
 * reads all of K and V.  Super-tiles are independent, so the leaves of all of
 * them go out as one grouped launch (ceil(BR/64) workgroups of 64 rows per
 * super-tile) and run side by side; the result is bit for bit that of
 * flash_attention (every row is computed by the same code either way).
 *
 * All matrices are row-major fp32 device buffers with leading dimensions.
 * Arguments: 1 Nq, 2 Nk (>= 1), 3 D (64 only), 4 Q, 5 ldq, 6 K, 7 ldk, 8 V,
 * 9 ldv, 10 O, 11 ldo (each >= D), 12 scale, then 13 BR (super-tiled form),
 * then the stream.  Nq = 0: nothing.  Errors as sgemm (negative argument
 * index, SGEMM_ERR_TOO_LARGE above 2^30 rows, HIP status).  O must not
 * overlap Q, K or V.  Asynchronous on `stream`.
 */
int flash_attention(int64_t Nq, int64_t Nk, int64_t D, const float* Q, int64_t ldq,
                    const float* K, int64_t ldk, const float* V, int64_t ldv, float* O,
                    int64_t ldo, float scale, void* stream);
int flash_attention_supertiled(int64_t Nq, int64_t Nk, int64_t D, const float* Q, int64_t ldq,
                               const float* K, int64_t ldk, const float* V, int64_t ldv,
                               float* O, int64_t ldo, float scale, int64_t BR, void* stream);

/*
 * Host-resident super-tiled SGEMM, the single-GPU form of the pages' cluster
 * runtime ("@cluster" page, "What runs today": per node, allocate tile
 * buffers, load super-tiles, compute the init and step leaves as their inputs
 * arrive, store the outputs, free the buffers; "Show HN: Phobos", section
 * "The DAG Compiler": a super-tile is the unit that moves, and the next
 * block's loads are issued while the current one computes).  For products
 * whose operands live in host memory, e.g. larger than the GPU.
 *
 * sgemm_plan_supertiles chooses super-tile extents, device tile slots and the
 * walk order the way the pages' cluster tuner plans ("@cluster" page, "What
 * runs today", Tuning): every candidate TM x TN x TK (powers of two from 256
 * below each dimension, and the dimension itself) with A slots in {2,
 * ceil(K/TK), all of A}, B slots in {2, all of B} and two C slots, walked row
 * by row (at most one row of A super-tiles kept) or, when all of A and B are
 * kept, in growing squares (each shell brings one new row of A super-tiles
 * and one new column of B super-tiles, which spreads the loads over the run),
 * is dropped if its device buffers exceed `device_bytes`; the rest are ranked
 * by a replay of the executor's schedule: the same walk and slot
 * replacement, an in-order load stream, a store stream and the compute
 * stream, with a step leaf taking 2*m*n*k at the GEMM rate scaled by how full
 * it keeps the 256 CUs (ceil(m/256)*ceil(n/256) workgroups in waves of 256)
 * plus 15 us and its C read and write at 5 TB/s, and a copy taking its bytes
 * at the link rate plus 10 us, both directions together at most 1.7 times
 * one direction.  `model` gives the rates (NULL: 146 TFLOP/s, 55 GB/s each
 * way).  Nothing is run.  Host-only.  Arguments: 1 M, 2 N, 3 K, 4 beta (0: C
 * is only written), 5 device_bytes, 6 model, 7 out.  SGEMM_ERR_BUDGET if
 * nothing fits, SGEMM_ERR_TOO_LARGE for a dimension above 2^30; candidates
 * with more than 2^20 step launches are not considered.
 *
 * sgemm_supertiled_host computes C <- alpha*A*B + beta*C with A, B and C in
 * host memory (row-major, leading dimensions as for sgemm; pinned memory,
 * e.g. hipHostMalloc'ed, gives full link speed) using `plan`.  It allocates
 * the plan's device slots and walks the output super-tiles in the plan's
 * order: per output super-tile load C (unless beta == 0), run the init leaf
 * and the K step leaves (the same kernels as sgemm_supertiled, so the result
 * is bit for bit that of sgemm_supertiled with the same extents on the same
 * values), store C.  A and B super-tiles are loaded into the least recently
 * used slot of their kind on a load stream of its own, which runs ahead of
 * the compute (`stream`) as far as free slots allow; C stores run on a store
 * stream; events order every load after the last compute or store that used
 * its slot.  Device slot pitches are the tile widths rounded up to 4 floats,
 * each slot starting on a 256-byte boundary; slot counts above the number of
 * distinct tiles of their kind are cut to it: for a plan that
 * sgemm_plan_supertiles returned for the same M, N, K and beta, at most the
 * plan's `device_bytes` are allocated.  Synchronous: returns once C is
 * complete in host memory, after freeing everything it allocated.
 * Arguments: 1..11 as sgemm (host pointers), 12 plan, 13 stream.  Errors:
 * negative argument index as sgemm (-12: plan NULL, an extent or slot count
 * below 1, or an unknown walk), SGEMM_ERR_TOO_LARGE, SGEMM_ERR_ALLOC, or a
 * HIP status; after a failure every stream is drained and everything freed,
 * and C may hold finished super-tiles next to unchanged ones.
 */
typedef struct sgemm_plan_model {
    double gemm_tflops;   /* sustained GEMM rate of one step leaf, TFLOP/s */
    double link_gbs;      /* host<->device copy bandwidth of one direction, GB/s */
} sgemm_plan_model;

#define SGEMM_WALK_ROWS 0     /* output super-tiles row by row (the pages' order) */
#define SGEMM_WALK_SHELLS 1   /* growing squares: shell s = tiles with max(pm, pn) == s */
#define SGEMM_WALK_BLOCKS 2   /* 2 x 2 blocks of output super-tiles, row by row of blocks, the
                                 K loop outside inside a block: c_slots must cover the tiles of
                                 one block (up to 4), else -12 */

typedef struct sgemm_plan {
    int64_t TM, TN, TK;                /* super-tile extents */
    int32_t a_slots, b_slots, c_slots; /* device tile buffers of each kind */
    int32_t walk;                      /* SGEMM_WALK_ROWS, _SHELLS or _BLOCKS */
    int64_t device_bytes;              /* device memory the slots take */
    double transfer_bytes;             /* host<->device bytes of the schedule */
    double modeled_ms;                 /* modeled time of the whole product */
} sgemm_plan;

int sgemm_plan_supertiles(int64_t M, int64_t N, int64_t K, float beta, int64_t device_bytes,
                          const sgemm_plan_model* model, sgemm_plan* out);
int sgemm_supertiled_host(int64_t M, int64_t N, int64_t K, float alpha,
                          const float* A, int64_t lda, const float* B, int64_t ldb,
                          float beta, float* C, int64_t ldc, const sgemm_plan* plan,
                          void* stream);

/*
 * Launch trace.  Between sgemm_trace_begin(capacity) and sgemm_trace_end,
 * every kernel the library enqueues is bracketed by a pair of HIP events
 * recorded on the launch's own stream (up to `capacity` launches; later ones
 * are not traced).  The events are for timing only: they are created without
 * the system-scope fence (hipEventDisableSystemFence), so recording them
 * writes back and invalidates no cache.  sgemm_trace_end waits for those events, writes each
 * launch's duration in milliseconds to ms_out[i] and its kind to kind_out[i]
 * (SGEMM_KIND_*), for i < min(count, cap), stores the count in *n_out and
 * frees the events.  Arguments of begin: 1 capacity (>= 1).  Of end:
 * 1 ms_out, 2 kind_out, 3 cap, 4 n_out (the output arrays may be NULL when
 * cap is 0).
 * sgemm_trace_begin_sampled(capacity, every) traces only launches 0, every,
 * 2*every, ... of those enqueued after it (every >= 1, else -2): a pair of
 * events costs the stream some microseconds, so a long run of equal
 * launches can be timed on a sample of them without slowing the rest.
 * sgemm_trace_begin(capacity) is sgemm_trace_begin_sampled(capacity, 1).
 */
#define SGEMM_KIND_GEMM 0
#define SGEMM_KIND_INIT_LEAF 1
#define SGEMM_KIND_TC 2          /* the matrix-core GEMM (either form) */
#define SGEMM_KIND_TC_CAST 3     /* the cast pass of its staged form */
#define SGEMM_KIND_ATTENTION 4   /* one attention leaf */
int sgemm_trace_begin(int64_t capacity);
int sgemm_trace_begin_sampled(int64_t capacity, int64_t every);
int sgemm_trace_end(float* ms_out, int32_t* kind_out, int64_t cap, int64_t* n_out);

/* Human-readable text for a status code (static storage, never NULL). */
const char* sgemm_status_string(int status);

/* PHOBOS_SGEMM_VERSION of the built library. */
int sgemm_version(void);

/*
 * Dispatch log.  When on, every entry point writes one line to stderr per
 * decision it takes, each starting "phobos_sgemm: ": a quick return (empty
 * product; K == 0 or alpha == 0; an init leaf at beta == 1 that enqueues
 * nothing), the super-tile grid of a super-tiled call, and each kernel it
 * enqueues with its shape, scalars, tile and wave grid, where the tile came
 * from (forced, SGEMM_FORCE_CFG, tuned or default), the load path (vec4 or
 * scalar), the grid and the stream.  The environment variable SGEMM_LOG (a
 * non-empty value other than "0") turns it on at the first call;
 * sgemm_set_log(on) turns it on (non-zero) or off (0) for the process and
 * returns the previous state (1 on, 0 off).  Host only; cannot fail.
 * SGEMM_GROUP_M (tile rows per raster group, default 4) and SGEMM_XCD_REMAP
 * (0 turns the XCD-aware tile order off), read once per process, tune the
 * tile order of the fp32 and 16-bit GEMM kernels.
 */
int sgemm_set_log(int32_t on);

#ifdef __cplusplus
}
#endif

#endif /* PHOBOS_SGEMM_H */
