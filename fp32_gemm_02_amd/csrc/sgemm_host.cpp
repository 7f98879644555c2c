// Host-resident super-tiled SGEMM: the single-GPU form of the pages' cluster
// runtime, in which each node allocates tile buffers, loads the super-tiles
// it needs, computes the init and step leaves as their inputs arrive, stores
// its output super-tiles and frees what it no longer needs ("@cluster" page,
// "What runs today"; "Show HN: Phobos", sections "The DAG Compiler" and
// "Where Does This Fit In?").  Here A, B and C stay in host memory, the GPU
// holds a bounded set of tile slots, and loads run on a stream of their own
// that works ahead of the compute stream as far as free slots allow, stores
// on another (the link carries both directions at once).
//
// The planner picks the super-tile extents and slot counts the way the pages'
// cluster tuner does: enumerate candidates, drop those whose working set does
// not fit the device budget, rank the rest by a model of compute and transfer
// time built from figures the caller supplies.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "phobos_sgemm.h"
#include "sgemm_internal.h"

namespace phobos {
// Defined in sgemm_api.cpp: one checked GEMM launch and one init-leaf launch.
int host_launch_gemm(int64_t M, int64_t N, int64_t K, float alpha, const float* A,
                     int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                     int64_t ldc, hipStream_t stream);
int host_launch_init(int64_t M, int64_t N, float beta, float* C, int64_t ldc,
                     hipStream_t stream);
}  // namespace phobos

namespace {

constexpr double kDefaultTflops = 140.0;   // sustained step-leaf rate on MI355X
constexpr double kDefaultLinkGBs = 50.0;   // pinned host<->device copies
constexpr double kLaunchMs = 0.015;        // per-launch ramp and gap
constexpr int64_t kCtaTile = 256;          // output tile of one workgroup (large shapes)
constexpr int64_t kCUs = 256;              // compute units of an MI355X
constexpr double kHbmGBs = 5000.0;         // effective HBM rate of a step leaf's C traffic

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t up4(int64_t x) { return (x + 3) / 4 * 4; }
// Floats one device slot takes: rows x pitch (pitch rounded up to 4 floats
// for 16-byte rows), rounded up to 64 floats so every slot starts on a
// 256-byte boundary.
int64_t slot_floats(int64_t rows, int64_t cols) { return (rows * up4(cols) + 63) / 64 * 64; }

// Extents tried for one dimension: powers of two from 256 below the
// dimension, and the dimension itself.
std::vector<int64_t> extents(int64_t dim) {
    std::vector<int64_t> v;
    for (int64_t p = 256; p < dim; p *= 2) v.push_back(p);
    v.push_back(dim);
    return v;
}

struct Modeled {
    int64_t device_bytes;
    double transfer_bytes, ms;
};

Modeled model_plan(int64_t M, int64_t N, int64_t K, float beta, int64_t TM, int64_t TN,
                   int64_t TK, int32_t a_slots, int32_t b_slots, int32_t c_slots,
                   const sgemm_plan_model& m) {
    const int64_t gm = cdiv(M, TM), gn = cdiv(N, TN), nk = cdiv(K, TK);
    const int64_t a_tile = 4 * slot_floats(TM, TK), b_tile = 4 * slot_floats(TK, TN),
                  c_tile = 4 * slot_floats(TM, TN);
    Modeled r{};
    r.device_bytes = a_slots * a_tile + b_slots * b_tile + c_slots * c_tile;
    const double a_bytes = 4.0 * M * K * (a_slots >= nk ? 1 : gn);
    const double b_bytes = 4.0 * K * N * (b_slots >= nk * gn ? 1 : gm);
    const double c_in = beta != 0.0f ? 4.0 * M * N : 0.0, c_out = 4.0 * M * N;
    r.transfer_bytes = a_bytes + b_bytes + c_in + c_out;
    // a step leaf runs ceil(TM/256)*ceil(TN/256) workgroups in waves of one per
    // CU: a super-tile with fewer workgroups than CUs leaves the rest idle
    const int64_t ctas = cdiv(TM, kCtaTile) * cdiv(TN, kCtaTile);
    const double fill = (double)ctas / (double)(cdiv(ctas, kCUs) * kCUs);
    // every step leaf also reads and writes its C super-tile in device memory
    const double c_rw_ms = 2.0 * 4.0 * TM * TN / (kHbmGBs * 1e9) * 1e3;
    const double compute_ms = 2.0 * M * N * K / (m.gemm_tflops * 1e12 * fill) * 1e3 +
                              gm * gn * nk * (kLaunchMs + c_rw_ms);
    // the link is full duplex: loads and stores run on streams of their own
    const double link = m.link_gbs * 1e9;
    const double transfer_ms = std::max(a_bytes + b_bytes + c_in, c_out) / link * 1e3;
    // the first A, B (and C) tiles are loaded before any compute, the last C
    // tile is stored after it
    const double fill_ms = (a_tile + b_tile + (beta != 0.0f ? c_tile : 0) + c_tile) / link * 1e3;
    r.ms = std::max(compute_ms, transfer_ms) + fill_ms;
    return r;
}

struct Slot {
    float* dev = nullptr;
    int64_t i = -1, j = -1;        // tile coordinates held (-1: none)
    uint64_t last = 0;             // LRU stamp
    hipEvent_t ready = nullptr;    // recorded on the load stream after a load
    hipEvent_t free = nullptr;     // recorded after the slot's last use (compute, or a C store)
};

int hip_status(hipError_t e) { return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_HIP_BASE + (int)e; }

}  // namespace

extern "C" {

int sgemm_plan_supertiles(int64_t M, int64_t N, int64_t K, float beta, int64_t device_bytes,
                          const sgemm_plan_model* model, sgemm_plan* out) {
    if (M < 1) return -1;
    if (N < 1) return -2;
    if (K < 1) return -3;
    if (device_bytes < 1) return -5;
    if (out == nullptr) return -7;
    sgemm_plan_model m{kDefaultTflops, kDefaultLinkGBs};
    if (model != nullptr) {
        if (!(model->gemm_tflops > 0.0) || !(model->link_gbs > 0.0)) return -6;
        m = *model;
    }
    bool found = false;
    sgemm_plan best{};
    for (int64_t TM : extents(M))
        for (int64_t TN : extents(N))
            for (int64_t TK : extents(K)) {
                const int64_t gm = cdiv(M, TM), gn = cdiv(N, TN), nk = cdiv(K, TK);
                const int32_t c_slots = (int32_t)std::min<int64_t>(2, gm * gn);
                const int64_t a_opts[2] = {std::min<int64_t>(2, nk), nk};
                const int64_t b_opts[2] = {std::min<int64_t>(2, nk), nk * gn};
                for (int64_t na : a_opts)
                    for (int64_t nb : b_opts) {
                        if (na > (1 << 20) || nb > (1 << 20)) continue;
                        const Modeled r = model_plan(M, N, K, beta, TM, TN, TK, (int32_t)na,
                                                     (int32_t)nb, c_slots, m);
                        if (r.device_bytes > device_bytes) continue;
                        const bool better =
                            !found || r.ms < best.modeled_ms * (1 - 1e-9) ||
                            (r.ms <= best.modeled_ms * (1 + 1e-9) && r.device_bytes < best.device_bytes);
                        if (better) {
                            best = sgemm_plan{TM, TN, TK, (int32_t)na, (int32_t)nb, c_slots,
                                              r.device_bytes, r.transfer_bytes, r.ms};
                            found = true;
                        }
                    }
            }
    if (!found) return SGEMM_ERR_BUDGET;
    *out = best;
    return SGEMM_OK;
}

int sgemm_supertiled_host(int64_t M, int64_t N, int64_t K, float alpha, const float* A,
                          int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                          int64_t ldc, const sgemm_plan* plan, void* stream) {
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    if (lda < std::max<int64_t>(1, K)) return -6;
    if (ldb < std::max<int64_t>(1, N)) return -8;
    if (ldc < std::max<int64_t>(1, N)) return -11;
    if (plan == nullptr || plan->TM < 1 || plan->TN < 1 || plan->TK < 1 || plan->a_slots < 1 ||
        plan->b_slots < 1 || plan->c_slots < 1)
        return -12;
    if (M == 0 || N == 0) return SGEMM_OK;
    const bool steps = K > 0 && alpha != 0.0f;
    if (steps && A == nullptr) return -5;
    if (steps && B == nullptr) return -7;
    if (C == nullptr) return -10;
    if (M > (int64_t(1) << 30) || N > (int64_t(1) << 30) || K > (int64_t(1) << 30))
        return SGEMM_ERR_TOO_LARGE;
    if (!steps && beta == 1.0f) return SGEMM_OK;   // C unchanged

    hipStream_t comp = reinterpret_cast<hipStream_t>(stream);
    const int64_t TM = std::min(plan->TM, M), TN = std::min(plan->TN, N);
    const int64_t TK = std::min(plan->TK, std::max<int64_t>(K, 1));
    const int64_t gm = cdiv(M, TM), gn = cdiv(N, TN), nk = steps ? cdiv(K, TK) : 0;
    const int64_t lda_t = up4(TK), ldb_t = up4(TN), ldc_t = up4(TN);   // device tile pitches
    const int64_t a_tile = slot_floats(TM, TK), b_tile = slot_floats(TK, TN),
                  c_tile = slot_floats(TM, TN);
    // never more slots than distinct tiles of a kind
    const int64_t na = steps ? std::min<int64_t>(plan->a_slots, gm * nk) : 0;
    const int64_t nb = steps ? std::min<int64_t>(plan->b_slots, nk * gn) : 0;
    const int64_t nc = std::min<int64_t>(plan->c_slots, gm * gn);
    const int64_t total = na * a_tile + nb * b_tile + nc * c_tile;

    float* pool = nullptr;
    hipStream_t h2d = nullptr, d2h = nullptr;   // loads, stores
    hipEvent_t start = nullptr;
    std::vector<Slot> sa(na), sb(nb), sc(nc);
    std::vector<hipEvent_t> c_done(nc, nullptr);
    int st = SGEMM_OK;
    // runs `call` only while nothing has failed; keeps the first failure
#define PHOBOS_CHK(call)                                        \
    do {                                                        \
        if (st == SGEMM_OK) st = hip_status(call);              \
    } while (0)
    if (hipMalloc(&pool, total * sizeof(float)) != hipSuccess) {
        (void)hipGetLastError();   // a failed allocation must not fail later launches
        return SGEMM_ERR_ALLOC;
    }
    {
        float* p = pool;
        for (auto& s : sa) { s.dev = p; p += a_tile; }
        for (auto& s : sb) { s.dev = p; p += b_tile; }
        for (auto& s : sc) { s.dev = p; p += c_tile; }
    }
    PHOBOS_CHK(hipStreamCreateWithFlags(&h2d, hipStreamNonBlocking));
    PHOBOS_CHK(hipStreamCreateWithFlags(&d2h, hipStreamNonBlocking));
    PHOBOS_CHK(hipEventCreateWithFlags(&start, hipEventDisableTiming));
    for (auto* v : {&sa, &sb, &sc})
        for (auto& s : *v) {
            PHOBOS_CHK(hipEventCreateWithFlags(&s.ready, hipEventDisableTiming));
            PHOBOS_CHK(hipEventCreateWithFlags(&s.free, hipEventDisableTiming));
        }
    for (auto& e : c_done) PHOBOS_CHK(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    // everything already queued on the caller's stream comes first
    PHOBOS_CHK(hipEventRecord(start, comp));
    PHOBOS_CHK(hipStreamWaitEvent(h2d, start, 0));
    PHOBOS_CHK(hipStreamWaitEvent(d2h, start, 0));
    for (auto* v : {&sa, &sb, &sc})
        for (auto& s : *v) PHOBOS_CHK(hipEventRecord(s.free, comp));

    uint64_t clock = 0;
    // Make tile (i, j) of a host matrix resident in one of `slots`, loading it
    // on the load stream into the least recently used slot once no queued
    // compute uses that slot any more.
    auto acquire = [&](std::vector<Slot>& slots, int64_t i, int64_t j, const float* host,
                       int64_t ldh, int64_t r0, int64_t c0, int64_t rows, int64_t cols,
                       int64_t pitch) -> Slot* {
        for (auto& s : slots)
            if (s.i == i && s.j == j) {
                s.last = ++clock;
                return &s;
            }
        Slot* v = &slots[0];
        for (auto& s : slots)
            if (s.last < v->last) v = &s;
        PHOBOS_CHK(hipStreamWaitEvent(h2d, v->free, 0));
        PHOBOS_CHK(hipMemcpy2DAsync(v->dev, pitch * sizeof(float), host + r0 * ldh + c0,
                                    ldh * sizeof(float), cols * sizeof(float), rows,
                                    hipMemcpyHostToDevice, h2d));
        PHOBOS_CHK(hipEventRecord(v->ready, h2d));
        v->i = i;
        v->j = j;
        v->last = ++clock;
        return v;
    };

    int64_t ci = 0;
    for (int64_t pm = 0; pm < gm && st == SGEMM_OK; ++pm) {
        const int64_t r0 = pm * TM, rows = std::min(TM, M - r0);
        for (int64_t pn = 0; pn < gn && st == SGEMM_OK; ++pn) {
            const int64_t c0 = pn * TN, cols = std::min(TN, N - c0);
            const int64_t slot = ci++ % nc;
            Slot& cs = sc[slot];
            // cs.free is recorded after the store of the slot's previous tile
            // (or at the start): nothing overwrites the slot before that
            if (beta != 0.0f) {
                PHOBOS_CHK(hipStreamWaitEvent(h2d, cs.free, 0));
                PHOBOS_CHK(hipMemcpy2DAsync(cs.dev, ldc_t * sizeof(float), C + r0 * ldc + c0,
                                            ldc * sizeof(float), cols * sizeof(float), rows,
                                            hipMemcpyHostToDevice, h2d));
                PHOBOS_CHK(hipEventRecord(cs.ready, h2d));
                PHOBOS_CHK(hipStreamWaitEvent(comp, cs.ready, 0));
            } else {
                PHOBOS_CHK(hipStreamWaitEvent(comp, cs.free, 0));
            }
            // init leaf, then one step leaf per K chunk
            if (st == SGEMM_OK) st = phobos::host_launch_init(rows, cols, beta, cs.dev, ldc_t, comp);
            for (int64_t kt = 0; kt < nk && st == SGEMM_OK; ++kt) {
                const int64_t k0 = kt * TK, depth = std::min(TK, K - k0);
                Slot* a = acquire(sa, pm, kt, A, lda, r0, k0, rows, depth, lda_t);
                Slot* b = acquire(sb, kt, pn, B, ldb, k0, c0, depth, cols, ldb_t);
                PHOBOS_CHK(hipStreamWaitEvent(comp, a->ready, 0));
                PHOBOS_CHK(hipStreamWaitEvent(comp, b->ready, 0));
                if (st != SGEMM_OK) break;
                st = phobos::host_launch_gemm(rows, cols, depth, alpha, a->dev, lda_t, b->dev,
                                              ldb_t, 1.0f, cs.dev, ldc_t, comp);
                PHOBOS_CHK(hipEventRecord(a->free, comp));
                PHOBOS_CHK(hipEventRecord(b->free, comp));
            }
            // store the finished super-tile on the store stream
            PHOBOS_CHK(hipEventRecord(c_done[slot], comp));
            PHOBOS_CHK(hipStreamWaitEvent(d2h, c_done[slot], 0));
            PHOBOS_CHK(hipMemcpy2DAsync(C + r0 * ldc + c0, ldc * sizeof(float), cs.dev,
                                        ldc_t * sizeof(float), cols * sizeof(float), rows,
                                        hipMemcpyDeviceToHost, d2h));
            PHOBOS_CHK(hipEventRecord(cs.free, d2h));
        }
    }
#undef PHOBOS_CHK
    // the call returns with C complete in host memory; every stream is
    // drained before anything is freed, also after a failure
    auto drain = [&](hipStream_t s) {
        const hipError_t e = hipStreamSynchronize(s);
        if (st == SGEMM_OK) st = hip_status(e);
    };
    if (h2d) drain(h2d);
    if (d2h) drain(d2h);
    drain(comp);
    for (auto* v : {&sa, &sb, &sc})
        for (auto& s : *v) {
            if (s.ready) (void)hipEventDestroy(s.ready);
            if (s.free) (void)hipEventDestroy(s.free);
        }
    for (auto& e : c_done)
        if (e) (void)hipEventDestroy(e);
    if (start) (void)hipEventDestroy(start);
    if (h2d) (void)hipStreamDestroy(h2d);
    if (d2h) (void)hipStreamDestroy(d2h);
    (void)hipFree(pool);
    return st;
}

}  // extern "C"
