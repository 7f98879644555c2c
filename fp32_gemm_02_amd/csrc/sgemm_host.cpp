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
// The planner picks the super-tile extents, slot counts and walk order the
// way the pages' cluster tuner does: enumerate candidates, drop those whose
// working set does not fit the device budget, rank the rest by modeled time.
// The model is a replay of the executor's own schedule (the same walk, the
// same slot replacement, in-order load and store streams) with durations
// from a few rates, so what the planner ranks is what the executor issues.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <list>
#include <unordered_map>
#include <utility>
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

// Default model rates (MI355X, PCIe 5.0 x16 host link, pinned memory).
constexpr double kDefaultTflops = 146.0;   // sustained step-leaf rate
constexpr double kDefaultLinkGBs = 55.0;   // one direction
constexpr double kDuplex = 1.7;            // both directions at once: this many times one
constexpr double kCopyMs = 0.010;          // fixed cost of one copy call
constexpr double kLaunchMs = 0.015;        // per-launch ramp and gap
constexpr double kHbmGBs = 5000.0;         // effective HBM rate of a leaf's C traffic
constexpr int64_t kCtaTile = 256;          // output tile of one workgroup (large shapes)
constexpr int64_t kCUs = 256;              // compute units
constexpr int64_t kMaxLaunches = int64_t(1) << 20;   // larger candidates are not planned

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

// Output super-tiles (pm, pn) in the order they are computed.  Rows: the
// pages' row-major placement.  Shells: growing squares, shell s = the tiles
// with max(pm, pn) == s, first row s left of the diagonal, then column s
// above it, then (s, s); each shell brings one new row of A super-tiles and
// one new column of B super-tiles, so loads spread over the whole run
// instead of all of B arriving during the first row of outputs.
std::vector<std::pair<int64_t, int64_t>> walk_order(int64_t gm, int64_t gn, int32_t walk) {
    std::vector<std::pair<int64_t, int64_t>> v;
    v.reserve((size_t)(gm * gn));
    if (walk == SGEMM_WALK_ROWS) {
        for (int64_t pm = 0; pm < gm; ++pm)
            for (int64_t pn = 0; pn < gn; ++pn) v.emplace_back(pm, pn);
        return v;
    }
    for (int64_t s = 0; s < std::max(gm, gn); ++s) {
        if (s < gm)
            for (int64_t pn = 0; pn < std::min(s, gn); ++pn) v.emplace_back(s, pn);
        if (s < gn)
            for (int64_t pm = 0; pm < std::min(s, gm); ++pm) v.emplace_back(pm, s);
        if (s < gm && s < gn) v.emplace_back(s, s);
    }
    return v;
}

// Output super-tiles live at once in a BLOCKS walk: blocks of kBlock x kBlock.
constexpr int64_t kBlock = 2;
int64_t live_c_tiles(int64_t gm, int64_t gn, int32_t walk) {
    return walk == SGEMM_WALK_BLOCKS ? std::min(kBlock, gm) * std::min(kBlock, gn) : 1;
}

// One step of a schedule: step leaf kt of output super-tile (pm, pn) (kt = -1
// when there is no K chunk: only the init leaf runs); `first` and `last`
// mark the tile's first and last step (load or clear C before, store after).
struct Step {
    int64_t pm, pn, kt;
    bool first, last;
};

// The steps in execution order.  ROWS and SHELLS finish each output
// super-tile, all its K chunks in turn, before the next.  BLOCKS takes the
// output super-tiles in blocks of kBlock x kBlock (row by row of blocks) and
// runs the K loop outside inside a block: chunk kt of every tile of the
// block, then chunk kt+1.  A block's tiles then share each A and B chunk
// while it is resident, so the first tiles need a block row of A and a block
// column of B per chunk, rather than a whole row of A and column of B before
// the first tile can finish.
std::vector<Step> walk_steps(int64_t gm, int64_t gn, int64_t nk, int32_t walk) {
    std::vector<Step> v;
    const int64_t ks = std::max<int64_t>(nk, 1);
    v.reserve((size_t)(gm * gn * ks));
    if (walk == SGEMM_WALK_BLOCKS) {
        for (int64_t m0 = 0; m0 < gm; m0 += kBlock)
            for (int64_t n0 = 0; n0 < gn; n0 += kBlock)
                for (int64_t k = 0; k < ks; ++k)
                    for (int64_t pm = m0; pm < std::min(m0 + kBlock, gm); ++pm)
                        for (int64_t pn = n0; pn < std::min(n0 + kBlock, gn); ++pn)
                            v.push_back({pm, pn, nk > 0 ? k : -1, k == 0, k == ks - 1});
        return v;
    }
    for (const auto& t : walk_order(gm, gn, walk))
        for (int64_t k = 0; k < ks; ++k)
            v.push_back({t.first, t.second, nk > 0 ? k : -1, k == 0, k == ks - 1});
    return v;
}

// Least-recently-used assignment of tiles of one kind to a fixed set of slots.
class SlotTable {
public:
    explicit SlotTable(int64_t slots) : holds_(slots, -1), pos_(slots) {
        for (int64_t s = 0; s < slots; ++s) pos_[s] = lru_.insert(lru_.end(), s);
    }
    // Slot that holds tile `id` after the call; *load is set when the tile
    // has to be loaded into it first (the slot held another tile, or none).
    int64_t acquire(int64_t id, bool* load) {
        auto it = where_.find(id);
        int64_t s;
        if (it != where_.end()) {
            s = it->second;
            *load = false;
        } else {
            s = lru_.front();
            if (holds_[s] >= 0) where_.erase(holds_[s]);
            holds_[s] = id;
            where_[id] = s;
            *load = true;
        }
        lru_.splice(lru_.end(), lru_, pos_[s]);
        return s;
    }

private:
    std::vector<int64_t> holds_;                     // slot -> tile id, -1: empty
    std::unordered_map<int64_t, int64_t> where_;     // tile id -> slot
    std::list<int64_t> lru_;                         // slots, least recently used first
    std::vector<std::list<int64_t>::iterator> pos_;  // slot -> its place in lru_
};

struct Candidate {
    int64_t TM, TN, TK, na, nb, nc;
    int32_t walk;
    int64_t device_bytes;
    double lower_ms;   // no schedule of this candidate can be faster
};

struct Modeled {
    double ms, h2d_bytes, d2h_bytes;
};

double fill_of(int64_t rows, int64_t cols) {
    // a step leaf runs ceil(rows/256)*ceil(cols/256) workgroups in waves of
    // one per CU: a super-tile with fewer workgroups than CUs leaves the rest idle
    const int64_t ctas = cdiv(rows, kCtaTile) * cdiv(cols, kCtaTile);
    return (double)ctas / (double)(cdiv(ctas, kCUs) * kCUs);
}

// Replays the executor's schedule: the compute stream runs init and step
// leaves in walk order; the load stream runs loads in the order they are
// issued, each after the last use of its slot; the store stream stores each
// finished super-tile.  Returns the modeled time and the bytes moved.
Modeled simulate(int64_t M, int64_t N, int64_t K, float beta, const Candidate& c,
                 const sgemm_plan_model& m) {
    const int64_t gm = cdiv(M, c.TM), gn = cdiv(N, c.TN), nk = cdiv(K, c.TK);
    const double link = m.link_gbs * 1e9;
    auto copy_ms = [&](double bytes) { return bytes / link * 1e3 + kCopyMs; };
    auto step_ms = [&](int64_t rows, int64_t cols, int64_t depth) {
        return 2.0 * rows * cols * depth / (m.gemm_tflops * 1e12 * fill_of(rows, cols)) * 1e3 +
               kLaunchMs + 8.0 * rows * cols / (kHbmGBs * 1e9) * 1e3;
    };
    SlotTable ta(c.na), tb(c.nb);
    std::vector<double> a_ready(c.na, 0), a_free(c.na, 0), b_ready(c.nb, 0), b_free(c.nb, 0),
        c_free(c.nc, 0);
    std::vector<int64_t> tile_slot((size_t)(gm * gn), -1);
    double h2d = 0, d2h = 0, comp = 0, h2d_bytes = 0, d2h_bytes = 0;
    int64_t ci = 0;
    for (const Step& t : walk_steps(gm, gn, nk, c.walk)) {
        const int64_t pm = t.pm, pn = t.pn;
        const int64_t rows = std::min(c.TM, M - pm * c.TM), cols = std::min(c.TN, N - pn * c.TN);
        const double cb = 4.0 * rows * cols;
        if (t.first) {
            const int64_t slot = ci++ % c.nc;
            tile_slot[(size_t)(pm * gn + pn)] = slot;
            if (beta != 0.0f) {
                h2d = std::max(h2d, c_free[slot]) + copy_ms(cb);
                h2d_bytes += cb;
                comp = std::max(comp, h2d);
            } else {
                comp = std::max(comp, c_free[slot]);
            }
            if (beta != 1.0f) comp += kLaunchMs + (beta != 0.0f ? 2 : 1) * cb / (kHbmGBs * 1e9) * 1e3;
        }
        if (t.kt >= 0) {
            const int64_t kt = t.kt, depth = std::min(c.TK, K - kt * c.TK);
            bool load;
            const int64_t sa = ta.acquire(pm * nk + kt, &load);
            if (load) {
                h2d = std::max(h2d, a_free[sa]) + copy_ms(4.0 * rows * depth);
                h2d_bytes += 4.0 * rows * depth;
                a_ready[sa] = h2d;
            }
            const int64_t sb = tb.acquire(kt * gn + pn, &load);
            if (load) {
                h2d = std::max(h2d, b_free[sb]) + copy_ms(4.0 * depth * cols);
                h2d_bytes += 4.0 * depth * cols;
                b_ready[sb] = h2d;
            }
            comp = std::max({comp, a_ready[sa], b_ready[sb]}) + step_ms(rows, cols, depth);
            a_free[sa] = b_free[sb] = comp;
        }
        if (t.last) {
            d2h = std::max(d2h, comp) + copy_ms(cb);
            d2h_bytes += cb;
            c_free[tile_slot[(size_t)(pm * gn + pn)]] = d2h;
        }
    }
    // both directions together move at most kDuplex times one direction's rate
    const double both = (h2d_bytes + d2h_bytes) / (kDuplex * link) * 1e3;
    return Modeled{std::max({comp, d2h, both}), h2d_bytes, d2h_bytes};
}

int hip_status(hipError_t e) { return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_HIP_BASE + (int)e; }

struct Slot {
    float* dev = nullptr;
    hipEvent_t ready = nullptr;    // recorded on the load stream after a load
    hipEvent_t free = nullptr;     // recorded after the slot's last use (compute, or a C store)
};

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
    if (M > (int64_t(1) << 30) || N > (int64_t(1) << 30) || K > (int64_t(1) << 30))
        return SGEMM_ERR_TOO_LARGE;
    const double link = m.link_gbs * 1e9;
    // every element of A and B crosses the link at least once, C once each way
    const double min_h2d = 4.0 * ((double)M * K + (double)K * N + (beta != 0.0f ? (double)M * N : 0));
    const double min_d2h = 4.0 * (double)M * N;
    const double min_link_ms =
        std::max({min_h2d / link, min_d2h / link, (min_h2d + min_d2h) / (kDuplex * link)}) * 1e3;
    const double min_flop_ms = 2.0 * M * N * K / (m.gemm_tflops * 1e12) * 1e3;

    std::vector<Candidate> cands;
    for (int64_t TM : extents(M))
        for (int64_t TN : extents(N))
            for (int64_t TK : extents(K)) {
                const int64_t gm = cdiv(M, TM), gn = cdiv(N, TN), nk = cdiv(K, TK);
                if (gm * gn * nk > kMaxLaunches) continue;
                const int64_t a_all = gm * nk, b_all = nk * gn;
                const double lower = std::max(min_flop_ms + gm * gn * nk * kLaunchMs, min_link_ms);
                auto add = [&](int64_t na, int64_t nb, int64_t nc, int32_t walk) {
                    const int64_t bytes = 4 * (na * slot_floats(TM, TK) + nb * slot_floats(TK, TN) +
                                               nc * slot_floats(TM, TN));
                    if (bytes <= device_bytes)
                        cands.push_back({TM, TN, TK, na, nb, nc, walk, bytes, lower});
                };
                const int64_t a_opts[4] = {std::min<int64_t>(2, nk), nk,
                                           std::min<int64_t>(kBlock * nk, a_all), a_all};
                const int64_t b_opts[3] = {std::min<int64_t>(2, nk),
                                           std::min<int64_t>(kBlock * nk, b_all), b_all};
                for (int ia = 0; ia < 4; ++ia)
                    for (int ib = 0; ib < 3; ++ib) {
                        const int64_t na = a_opts[ia], nb = b_opts[ib];
                        bool dup = false;
                        for (int j = 0; j < ia; ++j) dup |= a_opts[j] == na;
                        for (int j = 0; j < ib; ++j) dup |= b_opts[j] == nb;
                        if (dup) continue;
                        const int64_t nc = std::min<int64_t>(2, gm * gn);
                        // row-major walks keep one row of A resident at most;
                        // shells need all of A and B resident
                        if (na <= nk && (nb == b_opts[0] || nb == b_all)) add(na, nb, nc, SGEMM_WALK_ROWS);
                        if (na == a_all && nb == b_all && gm > 1 && gn > 1)
                            add(na, nb, nc, SGEMM_WALK_SHELLS);
                        // blocks: one block's C tiles, or two blocks' (the next
                        // one's loads overlap this one's steps)
                        const int64_t live = live_c_tiles(gm, gn, SGEMM_WALK_BLOCKS);
                        if (live > 1 && na >= std::min<int64_t>(2, nk))
                            for (int64_t ncb : {live, std::min<int64_t>(2 * live, gm * gn)}) {
                                add(na, nb, ncb, SGEMM_WALK_BLOCKS);
                                if (ncb == gm * gn) break;
                            }
                    }
            }
    if (cands.empty()) return SGEMM_ERR_BUDGET;
    std::stable_sort(cands.begin(), cands.end(), [](const Candidate& x, const Candidate& y) {
        return x.lower_ms < y.lower_ms;
    });
    bool found = false;
    sgemm_plan best{};
    for (const Candidate& c : cands) {
        if (found && c.lower_ms > best.modeled_ms) break;   // no later candidate can win
        const Modeled r = simulate(M, N, K, beta, c, m);
        const bool better = !found || r.ms < best.modeled_ms * (1 - 1e-9) ||
                            (r.ms <= best.modeled_ms * (1 + 1e-9) && c.device_bytes < best.device_bytes);
        if (better) {
            best = sgemm_plan{c.TM, c.TN, c.TK, (int32_t)c.na, (int32_t)c.nb, (int32_t)c.nc,
                              c.walk, c.device_bytes, r.h2d_bytes + r.d2h_bytes, r.ms};
            found = true;
        }
    }
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
        plan->b_slots < 1 || plan->c_slots < 1 ||
        (plan->walk != SGEMM_WALK_ROWS && plan->walk != SGEMM_WALK_SHELLS &&
         plan->walk != SGEMM_WALK_BLOCKS))
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
    // every output super-tile that is live at once needs a C slot of its own
    if (nc < live_c_tiles(gm, gn, plan->walk)) return -12;
    const int64_t total = na * a_tile + nb * b_tile + nc * c_tile;

    float* pool = nullptr;
    if (hipMalloc(&pool, total * sizeof(float)) != hipSuccess) {
        (void)hipGetLastError();   // a failed allocation must not fail later launches
        return SGEMM_ERR_ALLOC;
    }
    hipStream_t h2d = nullptr, d2h = nullptr;   // loads, stores
    hipEvent_t start = nullptr;
    std::vector<Slot> sa(na), sb(nb), sc(nc);
    std::vector<hipEvent_t> c_done(nc, nullptr);
    {
        float* p = pool;
        for (auto& s : sa) { s.dev = p; p += a_tile; }
        for (auto& s : sb) { s.dev = p; p += b_tile; }
        for (auto& s : sc) { s.dev = p; p += c_tile; }
    }
    int st = SGEMM_OK;
    // runs `call` only while nothing has failed; keeps the first failure
#define PHOBOS_CHK(call)                                        \
    do {                                                        \
        if (st == SGEMM_OK) st = hip_status(call);              \
    } while (0)
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

    // Make a tile resident in one of `slots`, loading it on the load stream
    // into the least recently used slot once no queued work uses that slot.
    auto acquire = [&](SlotTable& table, std::vector<Slot>& slots, int64_t id, const float* host,
                       int64_t ldh, int64_t r0, int64_t c0, int64_t rows, int64_t cols,
                       int64_t pitch) -> Slot* {
        bool load;
        Slot* v = &slots[table.acquire(id, &load)];
        if (load) {
            PHOBOS_CHK(hipStreamWaitEvent(h2d, v->free, 0));
            PHOBOS_CHK(hipMemcpy2DAsync(v->dev, pitch * sizeof(float), host + r0 * ldh + c0,
                                        ldh * sizeof(float), cols * sizeof(float), rows,
                                        hipMemcpyHostToDevice, h2d));
            PHOBOS_CHK(hipEventRecord(v->ready, h2d));
        }
        return v;
    };

    SlotTable ta(std::max<int64_t>(na, 1)), tb(std::max<int64_t>(nb, 1));
    std::vector<int64_t> tile_slot((size_t)(gm * gn), -1);
    int64_t ci = 0;
    for (const Step& t : walk_steps(gm, gn, nk, plan->walk)) {
        if (st != SGEMM_OK) break;
        const int64_t pm = t.pm, pn = t.pn;
        const int64_t r0 = pm * TM, rows = std::min(TM, M - r0);
        const int64_t c0 = pn * TN, cols = std::min(TN, N - c0);
        if (t.first) {
            // C slots go round-robin over the output super-tiles in the order
            // they start; a walk never has more tiles live than slots
            const int64_t slot = ci++ % nc;
            tile_slot[(size_t)(pm * gn + pn)] = slot;
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
            if (st == SGEMM_OK) st = phobos::host_launch_init(rows, cols, beta, cs.dev, ldc_t, comp);
        }
        const int64_t slot = tile_slot[(size_t)(pm * gn + pn)];
        Slot& cs = sc[slot];
        if (t.kt >= 0 && st == SGEMM_OK) {
            const int64_t kt = t.kt, k0 = kt * TK, depth = std::min(TK, K - k0);
            Slot* a = acquire(ta, sa, pm * nk + kt, A, lda, r0, k0, rows, depth, lda_t);
            Slot* b = acquire(tb, sb, kt * gn + pn, B, ldb, k0, c0, depth, cols, ldb_t);
            PHOBOS_CHK(hipStreamWaitEvent(comp, a->ready, 0));
            PHOBOS_CHK(hipStreamWaitEvent(comp, b->ready, 0));
            if (st != SGEMM_OK) break;
            st = phobos::host_launch_gemm(rows, cols, depth, alpha, a->dev, lda_t, b->dev, ldb_t,
                                          1.0f, cs.dev, ldc_t, comp);
            PHOBOS_CHK(hipEventRecord(a->free, comp));
            PHOBOS_CHK(hipEventRecord(b->free, comp));
        }
        if (t.last) {
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
