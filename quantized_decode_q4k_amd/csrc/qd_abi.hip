// qd_abi.hip -- the C ABI of include/qdecode.h: argument checks, launch-shape
// choice and the split-K workspace.  Every check runs on the host before any
// HIP call, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <atomic>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "qd_internal.h"
#include "qdecode.h"

namespace {
constexpr size_t kScratchFloats = size_t(2) << 20;  // partial sums and h: 8 MiB
constexpr size_t kScratchCounterWords = (size_t(1) << 16) + 4096;
}  // namespace

// Scratch of the allocation-free entry point (qffn_decode_noalloc): one per
// GPU, held until the process ends.  Host code never uses this name as an
// address; it asks hipGetSymbolAddress for the device's copy (see
// scratch_workspace below).
static __device__ __align__(256) float scratch[kScratchFloats + kScratchCounterWords];

namespace {

using qd::Shape;

// Zero n words (a kernel rather than a memory set, so that it may sit in a
// captured graph).
__global__ void zero_words_kernel(unsigned *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

constexpr int kVersion = 10000;  // 1.0.0

int block_elems(int fmt) {
    switch (fmt) {
    case QD_Q4_K: return 256;
    case QD_Q6_K: return 256;
    case QD_Q8_0: return 32;
    default: return 0;
    }
}

int block_bytes(int fmt) {
    switch (fmt) {
    case QD_Q4_K: return 144;
    case QD_Q6_K: return 210;
    case QD_Q8_0: return 34;
    default: return 0;
    }
}

int64_t row_bytes(int fmt, int64_t K) {
    const int qk = block_elems(fmt);
    if (qk == 0 || K <= 0 || K % qk != 0) return 0;
    return (K / qk) * (int64_t)block_bytes(fmt);
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// [p, p + n) and [q, q + m) overlap?
bool overlap(const void *p, size_t n, const void *q, size_t m) {
    if (!p || !q || n == 0 || m == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + m && b < a + n;
}

// ------------------------------------------------------- launch shapes ---
std::atomic<int> g_over_pin{0}, g_over_pout{0}, g_over_nr{0}, g_over_rpg{0};

constexpr int kTargetWorkgroups = 400;   // enough to keep every CU streaming
constexpr int kWalkMinWorkgroups = 1000; // batch 1-2 row walk only with rows to spare
constexpr int kMaxTiles = 1 << 16;       // split-K counters per workspace
constexpr int64_t kStreamMinK = 8192;    // automatic use of the streaming kernel
constexpr int64_t kRegisterMinKFfnB2 = 4096;  // fused gate/up at batch 2: register kernel from this K
constexpr int kAuxWords = 4096;          // counters after the tile counters: row epilogues, FFN flags

int lds_units_max(int fmt, int batch) {
    // largest nk whose staging fits the per-workgroup LDS budget
    int nk = 1;
    while (qd::mv_lds_bytes(fmt, batch, nk + 1) <= (size_t)qd::kLdsBudgetBytes) nk++;
    return nk;
}

struct Plan {
    Shape s;
    int nk;
    int64_t tiles;
};

Plan make_plan(int fmt, int64_t N, int64_t K, int batch, bool ffn, Shape s) {
    const int nb = (int)((K + qd::kSuper - 1) / qd::kSuper);
    Plan p;
    p.s = s;
    p.nk = (nb + s.p_out - 1) / s.p_out;
    p.s.p_out = (nb + p.nk - 1) / p.nk;  // every slice non-empty
    const int rows_wg = (qd::kGroups / s.p_in) * (ffn ? 1 : s.nr) * std::max(1, s.rpg);
    p.tiles = (N + rows_wg - 1) / rows_wg;
    return p;
}

Plan choose_plan(int fmt, int64_t N, int64_t K, int batch, bool ffn) {
    const int nb = (int)((K + qd::kSuper - 1) / qd::kSuper);
    const int max_nk = lds_units_max(fmt, batch);
    const int p_lds = (nb + max_nk - 1) / max_nk;  // K-slices the LDS budget forces
    // Measured on MI355X (sweeps over p_in x p_out x nr for every workload
    // shape): two lane groups per row is the best streaming shape; small-N
    // shapes then need more K-parallelism inside the workgroup to fill the
    // chip, and only then across workgroups.
    Shape s{2, p_lds, 1};
    Plan p = make_plan(fmt, N, K, batch, ffn, s);
    // Batch 2 over rows of K >= kStreamMinK, few of them (the streaming
    // kernel takes the rest): four K-slices across workgroups and no more
    // lane groups per row (Gemma-3 down 2560 x 10240, graph replay, p_in /
    // p_out 2/4 against 2/2, 4/4, 2/8: Q6_K 15.4 against 17.8, 17.9, 17.8 us;
    // Q4_K 13.0 against 15.8, 12.6, 13.2; Q8_0 17.1 against 20.9, 16.7, 17.4).
    // The fused gate/up at batch 2 over rows of K >= 4096: one lane group per
    // row and two K-slices across workgroups (graph replay, against the
    // streaming kernel: Gemma-4 21504 x 5376 62.7-66.1 -> 54.7-57.9 us,
    // 14336 x 4096 32.9-39.3 -> 27.3-30.4 us; p_out 3 and 4 no better).
    const bool long_b2 = batch == 2 && !ffn && K >= kStreamMinK;
    const bool ffn_b2 = batch == 2 && ffn && K >= kRegisterMinKFfnB2;
    if (long_b2) p = make_plan(fmt, N, K, batch, ffn, Shape{2, std::max(p_lds, 4), 1});
    if (ffn_b2) p = make_plan(fmt, N, K, batch, ffn, Shape{1, std::max(p_lds, 2), 1});
    for (int iter = 0; iter < 16 && !long_b2 && !ffn_b2; iter++) {
        const int64_t wgs = p.tiles * p.s.p_out;
        if (wgs >= kTargetWorkgroups) break;
        Shape t = p.s;
        if (t.p_in < 16 && (p.nk + 2 * t.p_in - 1) / (2 * t.p_in) >= 1) t.p_in *= 2;
        else if (p.nk >= 2 && p.tiles <= kMaxTiles) t.p_out = p.s.p_out + 1;
        else break;
        Plan q = make_plan(fmt, N, K, batch, ffn, t);
        if (q.s.p_out == p.s.p_out && q.s.p_in == p.s.p_in) break;
        p = q;
    }
    // Row walk (measured on MI355X): where the matrix has rows to spare, lane
    // groups walk several row slots, so a workgroup stages its activation
    // slice once for more rows and its load ring runs on across rows.
    //  * batch 3..8: one lane group per row (p_in 1), two row slots each
    //    (Gemma-4-31B FFN at batch 8: gate/up 194-282 -> 114-137 us, down
    //    113 -> 85 us);
    //  * batch 1..2 plain GEMV over many rows: two rows per lane group, two
    //    row slots (lm_head 262144 x 2560: Q4_K 82 -> 71-75 us, Q8_0 155 ->
    //    144 us), four for Q8_0's longer rows and for Q4_K where the rows
    //    allow (lm_head Q4_K on activation digits, same box: batch 1
    //    78.9-82.0 -> 75.1-76.3 us, batch 2 101.7-104.6 -> 99.2-101.7 us;
    //    eight: 74.6-74.9 and 101.9-102.7 us).
    if (batch >= 3) {
        Shape t = p.s;
        t.p_in = 1;
        t.rpg = 2;
        Plan q = make_plan(fmt, N, K, batch, ffn, t);
        if (q.tiles * q.s.p_out >= kTargetWorkgroups) p = q;
    } else if (!ffn && p.s.p_in == 2) {
        Shape t = p.s;
        t.nr = 2;
        for (int rpg = fmt == qd::kQ6K ? 2 : 4; rpg >= 2; rpg /= 2) {
            t.rpg = rpg;
            Plan q = make_plan(fmt, N, K, batch, ffn, t);
            if (q.tiles * q.s.p_out >= kWalkMinWorkgroups) {
                p = q;
                break;
            }
        }
    }
    // explicit overrides (tuning sweeps)
    const int op = g_over_pin.load(), oq = g_over_pout.load(), onr = g_over_nr.load();
    if (op || oq || onr) {
        Shape t = p.s;
        t.nr = 1;   // a forced shape walks one row slot of one row unless asked
        t.rpg = 1;
        if (op) t.p_in = op;
        if (oq) t.p_out = std::max(oq, p_lds);
        if (onr && !ffn) t.nr = onr;
        p = make_plan(fmt, N, K, batch, ffn, t);
    }
    if (p.s.p_out > 1 && p.tiles > kMaxTiles) {  // fall back: no split across workgroups
        Shape t = p.s;
        t.p_out = p_lds;
        p = make_plan(fmt, N, K, batch, ffn, t);
    }
    // row slots per lane group (explicit override, tuning sweeps)
    if (const int orpg = g_over_rpg.load()) {
        Shape t = p.s;
        t.rpg = orpg;
        p = make_plan(fmt, N, K, batch, ffn, t);
    }
    return p;
}

// ---------------------------------------------------------- workspace ---
// Split-K partial sums and counters, one block per (device, stream) so that
// calls on different streams never share it.  Counters start at zero and
// every kernel that uses one resets it before it ends, so a block needs no
// reset between calls.  A block is allocated (and its counters cleared on
// the caller's stream) only by a call made while the stream is not being
// captured; a capturing call that would need a new or larger block returns
// QD_ECAPTURE with nothing enqueued.  A block that has been outgrown stays
// allocated until the process ends, so a graph captured with it stays
// valid.
struct Workspace {
    float *partials = nullptr;
    unsigned *counters = nullptr;   // [kMaxTiles] tile counters, then [kAuxWords]
    size_t partial_floats = 0;
};

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::vector<std::pair<float *, unsigned *>> g_ws_retired;

constexpr size_t kInitialPartials = size_t(8) << 20;  // 32 MiB of floats
constexpr size_t kCounterWords = (size_t)kMaxTiles + kAuxWords;
static_assert(kCounterWords == kScratchCounterWords, "the scratch holds the workspace's counters");

// True when `st` is being captured into a graph (or its state cannot be read).
bool capturing(hipStream_t st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) return true;
    return cs != hipStreamCaptureStatusNone;
}

qd_status get_workspace(hipStream_t st, size_t need_floats, Workspace *out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QD_ELAUNCH;
    std::lock_guard<std::mutex> lk(g_ws_mu);
    Workspace &w = g_ws[{dev, st}];
    if (w.partials == nullptr || w.partial_floats < need_floats) {
        if (capturing(st)) return QD_ECAPTURE;
        size_t n = std::max(kInitialPartials, need_floats);
        if (w.partials != nullptr) n = std::max(n, 2 * w.partial_floats);
        float *p = nullptr;
        unsigned *c = nullptr;
        if (hipMalloc(&p, n * sizeof(float)) != hipSuccess) return QD_ENOMEM;
        if (hipMalloc(&c, kCounterWords * sizeof(unsigned)) != hipSuccess) {
            (void)hipFree(p);
            return QD_ENOMEM;
        }
        if (hipMemsetAsync(c, 0, kCounterWords * sizeof(unsigned), st) != hipSuccess) {
            (void)hipFree(p);
            (void)hipFree(c);
            return QD_ELAUNCH;
        }
        if (w.partials != nullptr) g_ws_retired.emplace_back(w.partials, w.counters);
        w.partials = p;
        w.counters = c;
        w.partial_floats = n;
    }
    *out = w;
    return QD_OK;
}

// The workspace of a call: the stream's own (allocated on first need), or a
// fixed block the caller hands in (the allocation-free entry point's
// scratch), which is never grown: a call that needs more returns
// QD_ETOOBIG with nothing enqueued.
qd_status acquire_ws(hipStream_t st, size_t need_floats, const Workspace *fixed, Workspace *out) {
    if (fixed) {
        if (need_floats > fixed->partial_floats) return QD_ETOOBIG;
        *out = *fixed;
        return QD_OK;
    }
    return get_workspace(st, need_floats, out);
}

// The device's scratch as a fixed workspace: its address from
// hipGetSymbolAddress, asked once per device with that device current (each
// GPU holds its own copy of the array).
std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices] = {};

qd_status scratch_workspace(Workspace *out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QD_ELAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return QD_EUNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return QD_ELAUNCH;
        g_scratch_ptr[dev] = p;
    }
    float *base = static_cast<float *>(g_scratch_ptr[dev]);
    out->partials = base;
    out->counters = reinterpret_cast<unsigned *>(base + kScratchFloats);
    out->partial_floats = kScratchFloats;
    return QD_OK;
}

// Compute units of the current device (asked once per device).
int cu_count() {
    static std::mutex mu;
    static std::map<int, int> cus;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    std::lock_guard<std::mutex> lk(mu);
    auto it = cus.find(dev);
    if (it != cus.end()) return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
    return n;
}

// ------------------------------------------------ matrix-core batch path ---
// Batch 3..64 (qd_gemv_mfma.hip): the call's activation digits, then one
// launch that streams the weights once for every batch row.  Process-wide
// mode (qd_set_batch_override): 0 = automatic (matrix cores from batch 3
// on), 1 = the fp32 register kernel in launches of up to 8 batch rows.
std::atomic<int> g_batch_mode{0}, g_mq_pout{0};

size_t round64(size_t n) { return (n + 63) / 64 * 64; }

struct MqPlan {
    int ng = 1, nb = 0, nk = 1, p_out = 1;
    int64_t tiles = 0;
    size_t dig_floats = 0, part_floats = 0;
    size_t floats() const { return dig_floats + part_floats; }
};

MqPlan mq_plan(int fmt, int64_t N, int64_t K, int batch, bool ffn) {
    MqPlan p;
    p.ng = batch <= 8 ? 1 : batch <= 16 ? 2 : batch <= 32 ? 4 : 8;
    const int nb = (int)((K + qd::kSuper - 1) / qd::kSuper);
    p.nb = nb;
    p.tiles = (N + qd::mq_tile_rows(ffn) - 1) / qd::mq_tile_rows(ffn);
    // K-slices: the least work on the busiest CU.  A CU given w workgroups
    // of nk superunits runs them about two at a time, or one where only one
    // is resident (a third resident one adds little: Gemma-4-31B down at
    // batch 8, 42 tiles x 84 superunits, 12 slices = 2 workgroups on every CU
    // 42 us, 14 slices = 2 or 3 47 us), so it takes w (nk + 2) / min(w, c);
    // the fewest slices among equals (less split-K traffic)
    const int64_t cus = cu_count();
    const int64_t conc = std::min(2, qd::mq_wg_per_cu(fmt, p.ng, ffn));
    int64_t best = INT64_MAX;
    for (int po = 1; po <= nb; po++) {
        if (po > 1 && p.tiles > kMaxTiles) break;  // a counter per row tile
        const int nk = (nb + po - 1) / po;
        const int pp = (nb + nk - 1) / nk;
        if (pp != po) continue;
        // a workgroup's start (digits, first loads) costs about two
        // superunits; the last workgroup of a tile reads its slices' partial
        // sums about 8 at a time, each batch about one superunit
        const int64_t w = (p.tiles * pp + cus - 1) / cus;
        const int64_t c = std::max<int64_t>(1, std::min(w, conc));
        const int64_t cost = (2 * w * (nk + 2) + c - 1) / c + 2 * (pp > 1 ? (pp + 7) / 8 : 0);
        if (cost < best) {
            best = cost;
            p.nk = nk;
            p.p_out = pp;
        }
    }
    if (const int fo = g_mq_pout.load()) {  // tuning override
        const int po = std::min(fo, p.tiles > kMaxTiles ? 1 : nb);
        p.nk = (nb + po - 1) / po;
        p.p_out = (nb + p.nk - 1) / p.nk;
    }
    p.dig_floats = round64((size_t)p.ng * nb * qd::mq_su_bytes_host(fmt) / 4);
    p.part_floats = p.p_out > 1 ? (size_t)p.p_out * batch * (ffn ? 2 : 1) * N : 0;
    return p;
}

bool launch_forced() { return g_over_pin.load() || g_over_pout.load() || g_over_nr.load(); }
// (a Q8_0 row whose length is not a multiple of 256 has a partial last
// superunit, which the matrix kernel's whole-unit tile reads do not take)
bool use_mq(int batch, int64_t K) {
    return batch >= 3 && K % qd::kSuper == 0 && K <= qd::xdig_max_k() && g_batch_mode.load() == 0 &&
           !launch_forced();
}

// ------------------------------------------------------------- checks ---
qd_status check_shape(int fmt, int64_t N, int64_t K, int batch) {
    if (block_elems(fmt) == 0) return QD_EINVAL;
    if (N < 1 || K < 1 || batch < 1 || batch > QD_MAX_BATCH) return QD_ESHAPE;
    if (row_bytes(fmt, K) == 0) return QD_ESHAPE;
    if (N > (int64_t(1) << 31) || K > (int64_t(1) << 24)) return QD_ESHAPE;
    return QD_OK;
}

// ------------------------------------------------- streaming GEMV plan ---
constexpr int kCUs = 256;                  // MI355X compute units
constexpr size_t kLdsPerCU = 160 * 1024;    // gfx950 LDS per CU
constexpr int kStreamMaxWait = 63;          // vmcnt limit: copies in flight per wave
// tuning overrides (0 = automatic)
std::atomic<int> g_stream_wpc{0}, g_stream_depth{0}, g_stream_consumers{0}, g_stream_producers{0};
constexpr int64_t kStreamMinRowsTall = 65536;  // streaming kernel for tall Q6_K / Q8_0 matrices at batch 1
constexpr int64_t kStreamMinRowsB2 = 4096;     // ... and at batch 2 only from this many rows

// n_sel > 1: the routed slots of a MoE launch share the CUs, each slot
// taking G workgroups (at least one) over its own matrix.  g_set > 0: G
// workgroups (at most N), the matrix's share of a launch.
void stream_rows(int64_t N, int64_t K, int fmt, int wpc, const float *norm_w, qd::StreamArgs *a,
                 unsigned *grid, int n_sel = 1, int g_set = 0) {
    const int64_t rb = row_bytes(fmt, K);
    const int G = (int)std::min<int64_t>(
        N, g_set > 0 ? g_set : std::max<int64_t>(1, (int64_t)kCUs * wpc / n_sel));
    a->N = N;
    a->K = K;
    a->row_bytes = rb;
    a->mat_bytes = N * rb;
    a->nb = (int)(K / qd::kSuper);
    a->rows_base = (int)(N / G);
    a->rows_extra = (int)(N % G);
    a->units_max = (a->rows_base + (a->rows_extra > 0 ? 1 : 0)) * a->nb;
    a->norm_w = norm_w;
    a->wps = G;
    *grid = (unsigned)(G * n_sel);
}

// Producer / consumer kernel: as many ring slots as the LDS share holds (a
// multiple of the copying waves, no more than the workgroup's steps need), and
// as many steps in flight per copying wave as its vmcnt can track.  When slots
// are reused, slots >= consumers + producers * (lag - 1) keeps every wait of a
// copying wave for a free slot finite.  False if it does not fit.
bool stream_plan_pc(int fmt, bool ffn, int64_t N, int64_t K, int batch, const float *norm_w,
                    int wpc, int consumers, int producers, int lag_default, qd::StreamArgs *a,
                    unsigned *grid, size_t *lds, int n_sel = 1, int g_set = 0) {
    stream_rows(N, K, fmt, wpc, norm_w, a, grid, n_sel, g_set);
    a->consumers = consumers;
    a->producers = producers;
    const size_t budget = kLdsPerCU / wpc;
    const int copies = qd::stream_copies_per_step(fmt, ffn);
    if (copies <= 0) return false;
    const size_t fixed = qd::stream_pc_layout(fmt, batch, ffn, a->nb, a->units_max, 0, a);
    const size_t per_slot = qd::stream_pc_layout(fmt, batch, ffn, a->nb, a->units_max, 1, a) - fixed + 16;
    if (fixed >= budget) return false;
    const int steps = (a->units_max + 15) / 16;
    const int need = (steps + producers - 1) / producers * producers;
    int slots = (int)std::min<size_t>((size_t)need, (budget - fixed) / per_slot);
    slots -= slots % producers;
    while (slots >= producers && qd::stream_pc_layout(fmt, batch, ffn, a->nb, a->units_max, slots, a) > budget)
        slots -= producers;
    if (slots < producers) return false;
    *lds = qd::stream_pc_layout(fmt, batch, ffn, a->nb, a->units_max, slots, a);
    if (*lds > budget) return false;
    const int lag_max = 1 + kStreamMaxWait / copies;
    int lag = g_stream_depth.load() ? g_stream_depth.load() : lag_default;
    lag = std::min(lag, lag_max);
    if (steps > slots) lag = std::min(lag, (slots - consumers) / producers + 1);
    if (lag < 1) return false;

    a->slots = slots;
    a->lag = lag;
    return true;
}

// Launch of a streaming kernel for this shape, or false where the
// register-streaming kernel is used instead: batch > 2, Q8_0 rows of partial
// superunits, a matrix whose size is not a multiple of 16 bytes, an LDS
// layout that does not fit, and (unless overridden) plain GEMVs with K <
// 8192 other than the tall Q6_K / Q8_0 ones at batch 1.  The fused gate/up
// and the long-row GEMVs take the producer / consumer kernel.  At batch 1:
// one workgroup per CU with 8 decoding waves, 4 steps in flight per copying
// wave (fewer where the ring's slot-reuse bound asks), and 4 copying waves
// when a workgroup's rows hold 256 KB or more (2 below).  At batch 2 (8
// decoding waves spill registers): 4 decoding waves, 2 copying waves, 3
// steps in flight, one workgroup per CU when its whole row range fits in
// the ring, else two.  Measured on MI355X (graph replay, 1 GiB of rotating
// weights, after the clocks and the weight copies have warmed up), batch 1:
//   Gemma-3 gate/up 10240 x 2560:   9.9-10.0 us
//   Gemma-3 down Q6_K 2560 x 10240: 9.9-10.1 us
//   Gemma-4 gate/up 21504 x 5376:   28.9-29.3 us
//   Gemma-4 down Q6_K 5376 x 21504: 25.8-25.9 us
//   lm_head 262144 x 2560: Q8_0 127.4 us (register kernel 141.6), Q6_K
//   114.1 (123.0); Q4_K stays on the register kernel, 78-79 (88).
bool stream_plan(int fmt, bool ffn, int64_t N, int64_t K, int batch, const float *norm_w,
                 qd::StreamArgs *a, unsigned *grid, size_t *lds) {
    if (batch > 2) return false;
    if (K % qd::kSuper != 0) return false;
    if ((N * row_bytes(fmt, K)) % 16 != 0) return false;
    const int wpc = g_stream_wpc.load();
    const int cons = g_stream_consumers.load();
    constexpr int kPcLag = 3;  // steps in flight per copying wave
    if (wpc) {
        const int prod = g_stream_producers.load() ? g_stream_producers.load() : 2;
        return stream_plan_pc(fmt, ffn, N, K, batch, norm_w, wpc, cons ? cons : 8, prod, kPcLag, a, grid, lds);
    }
    // plain GEMVs: the long rows, and the tall Q6_K / Q8_0 matrices at batch
    // 1 (lm_head 262144 x 2560, graph replay: Q8_0 141.6 -> 127.4 us, Q6_K
    // 123.0 -> 114.1 us; Q4_K stays on the register kernel, 79 against 88)
    const bool tall = batch == 1 && fmt != QD_Q4_K && N >= kStreamMinRowsTall;
    if (!ffn && K < kStreamMinK && !tall) return false;
    if (batch == 1) {
        // steps in flight per copying wave (MI355X, decode FFN in graph
        // replay, medians of 6 interleaved runs; lag 3 / 4 / 5): Gemma-3
        // 20.32 / 20.26 / 20.49 us, Gemma-4-31B 56.64 / 56.86 / 56.77 us
        constexpr int kPcLag1 = 4;
        const int64_t wg_bytes = (N + kCUs - 1) / kCUs * row_bytes(fmt, K) * (ffn ? 2 : 1);
        const int prod = wg_bytes >= (int64_t(256) << 10) ? 4 : 2;
        return stream_plan_pc(fmt, ffn, N, K, batch, norm_w, 1, 8, prod, kPcLag1, a, grid, lds);
    }
    // batch 2 over few rows: the register kernel's K split across
    // workgroups fills the chip better (Gemma-3 down 2560 x 10240, graph
    // replay: Q6_K 21.5-22.0 -> 15.4 us, Q4_K 18.3-19.0 -> 13.0 us, Q8_0
    // 18.2-18.6 -> 17.1 us; 5376 x 21504 about even)
    if (!ffn && N < kStreamMinRowsB2) return false;
    // ... and the fused gate/up over rows of K >= 4096 (choose_plan)
    if (ffn && K >= kRegisterMinKFfnB2) return false;
    // 8 decoding waves spill registers at batch 2
    if (stream_plan_pc(fmt, ffn, N, K, batch, norm_w, 1, 4, 2, kPcLag, a, grid, lds) &&
        a->slots * 16 >= a->units_max)
        return true;
    return stream_plan_pc(fmt, ffn, N, K, batch, norm_w, 2, 4, 2, kPcLag, a, grid, lds);
}

// The routed experts of the MoE decode FFN on the producer / consumer kernel
// (batch 1): the slots split the CUs, each slot's workgroups a contiguous
// row range of its expert's matrix, with the batch-1 settings of the plain
// launches.  False where the register kernel is used instead (rows not of
// whole 256-weight superunits, an expert matrix not a multiple of 16 bytes,
// an LDS layout that does not fit).
bool stream_plan_moe(int fmt, bool ffn, int64_t N, int64_t K, int n_sel, const float *norm_w,
                     qd::StreamArgs *a, unsigned *grid, size_t *lds) {
    if (K % qd::kSuper != 0) return false;
    if ((N * row_bytes(fmt, K)) % 16 != 0) return false;
    const int64_t G = std::min<int64_t>(N, std::max<int64_t>(1, kCUs / n_sel));
    const int64_t wg_bytes = (N + G - 1) / G * row_bytes(fmt, K) * (ffn ? 2 : 1);
    const int prod = wg_bytes >= (int64_t(256) << 10) ? 4 : 2;
    return stream_plan_pc(fmt, ffn, N, K, 1, norm_w, 1, 8, prod, 4, a, grid, lds, n_sel);
}

// Row epilogue arguments of a plain GEMV (post-norm, residual, next norm).
struct PostArgs {
    const float *w1 = nullptr;  // post-norm weight [N]; nullptr = none
    const float *w2 = nullptr;  // next-norm weight [N] or nullptr
    float *y2 = nullptr;        // [batch][N] with w2
    float eps = 0.f;
};

// The activation digits of x (unless `dig` already holds them), then one
// matrix-core launch.  region: this call's floats of the workspace, holding
// (in order) its own digits when it forms them, the split-K partials and
// the post-norm projection.  hd: FFN only, h written as the down
// projection's digits instead of (or besides, y != nullptr) fp32.
struct HDigits {
    uint8_t *dig = nullptr;
    int nb = 0;
    int sx = 0;
};
qd_status mq_run(const MqPlan &p, int fmt, bool ffn, const void *W0, const void *W1, const float *x,
                 const uint8_t *dig, const float *norm_w, float eps, int act, float *y, float *g_out,
                 float *u_out, int64_t N, int64_t K, int batch, hipStream_t hs, const Workspace &w, float *region,
                 const float *res, const PostArgs &post, const HDigits &hd = HDigits()) {
    const bool pnorm = post.w1 != nullptr;
    float *next = region;
    if (!dig) {
        qd::XdArgs xa{};
        xa.x = x;
        xa.norm_w = norm_w;
        xa.eps = eps;
        xa.dig = reinterpret_cast<uint8_t *>(region);
        xa.K = K;
        xa.R = (int)(K / 32);
        xa.nb = p.nb;
        xa.batch = batch;
        if (qd::launch_xdig(xa, p.ng, fmt == QD_Q4_K, hs) != hipSuccess) return QD_ELAUNCH;
        dig = xa.dig;
        next += p.dig_floats;
    }
    qd::MqArgs a{};
    a.W0 = static_cast<const uint8_t *>(W0);
    a.W1 = static_cast<const uint8_t *>(W1);
    a.dig = dig;
    a.y = y;
    a.g_out = g_out;
    a.u_out = u_out;
    a.res = pnorm ? nullptr : res;
    a.partials = next;
    a.counters = w.counters;
    a.N = N;
    a.K = K;
    a.row_bytes = row_bytes(fmt, K);
    a.nb = (int)((K + qd::kSuper - 1) / qd::kSuper);
    a.nblk = (int)(K / block_elems(fmt));
    a.nk = p.nk;
    a.batch = batch;
    a.act = act;
    if (pnorm) {
        a.pn.w1 = post.w1;
        a.pn.w2 = post.w2;
        a.pn.r = res;
        a.pn.y2 = post.y2;
        a.pn.p = next + p.part_floats;
        a.pn.ctr = w.counters + kMaxTiles;  // auxiliary counter 0
        a.pn.tiles = (unsigned)p.tiles;
        a.pn.eps = post.eps;
    }
    a.hdig = hd.dig;
    a.hd_nb = hd.nb;
    a.hd_sx = hd.sx;
    const hipError_t e = qd::launch_mq(fmt, p.ng, ffn, a, (unsigned)p.tiles, (unsigned)p.p_out, hs);
    return e == hipSuccess ? QD_OK : QD_ELAUNCH;
}

qd_status run_mv(int fmt, bool ffn, const void *W0, const void *W1, const float *x,
                 const float *norm_w, float eps, int act, float *y, float *g_out, float *u_out,
                 int64_t N, int64_t K, int batch, void *stream, size_t ws_offset = 0,
                 const float *res = nullptr, const PostArgs &post = PostArgs(),
                 const Workspace *fixed = nullptr) {
    qd_status st = check_shape(fmt, N, K, batch);
    if (st != QD_OK) return st;
    if (!W0 || !x || !y || (ffn && !W1)) return QD_EINVAL;
    if (ffn && act != QD_ACT_GELU_TANH && act != QD_ACT_SILU) return QD_EINVAL;
    if (!aligned(W0, 16) || (W1 && !aligned(W1, 16)) || !aligned(x, 16)) return QD_EALIGN;
    if (norm_w && !aligned(norm_w, 16)) return QD_EALIGN;
    if (!aligned(y, 4) || (g_out && !aligned(g_out, 4)) || (u_out && !aligned(u_out, 4)))
        return QD_EALIGN;
    const bool pnorm = post.w1 != nullptr;
    if (pnorm && (ffn || !res || (post.w2 == nullptr) != (post.y2 == nullptr))) return QD_EINVAL;
    if (pnorm && (!aligned(post.w1, 4) || (post.w2 && !aligned(post.w2, 4)) || !aligned(post.y2, 4)))
        return QD_EALIGN;
    const size_t xbytes = (size_t)batch * K * 4, ybytes = (size_t)batch * N * 4;
    const size_t wbytes = (size_t)N * row_bytes(fmt, K);
    const void *outs[4] = {y, g_out, u_out, post.y2};
    for (const void *o : outs) {
        if (!o) continue;
        if (overlap(o, ybytes, x, xbytes) || overlap(o, ybytes, W0, wbytes) ||
            (W1 && overlap(o, ybytes, W1, wbytes)) || (norm_w && overlap(o, ybytes, norm_w, K * 4)) ||
            (post.w1 && overlap(o, ybytes, post.w1, N * 4)) || (post.w2 && overlap(o, ybytes, post.w2, N * 4)))
            return QD_EINVAL;
    }
    if (overlap(y, ybytes, g_out, ybytes) || overlap(y, ybytes, u_out, ybytes) ||
        overlap(g_out, ybytes, u_out, ybytes) || overlap(y, ybytes, post.y2, ybytes))
        return QD_EINVAL;
    // the residual is read at each output's own index just before that
    // output is written, so it may be y itself, but no other part of it
    if (res && (ffn || (res != y && overlap(res, ybytes, y, ybytes)))) return QD_EINVAL;
    if (res && overlap(res, ybytes, post.y2, ybytes)) return QD_EINVAL;
    if (res && !aligned(res, 4)) return QD_EALIGN;
    if (use_mq(batch, K)) {
        hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
        const MqPlan p = mq_plan(fmt, N, K, batch, ffn);
        const size_t p_floats = pnorm ? (size_t)batch * N : 0;
        Workspace w;
        st = acquire_ws(hs, ws_offset + p.floats() + p_floats, fixed, &w);
        if (st != QD_OK) return st;
        return mq_run(p, fmt, ffn, W0, W1, x, nullptr, norm_w, eps, act, y, g_out, u_out, N, K, batch, hs, w,
                      w.partials + ws_offset, res, post);
    }
    if (batch > QD_BATCH_CHUNK) {
        // successive launches of up to QD_BATCH_CHUNK columns
        for (int c0 = 0; c0 < batch; c0 += QD_BATCH_CHUNK) {
            const int nb = std::min(QD_BATCH_CHUNK, batch - c0);
            const int64_t xo = (int64_t)c0 * K, yo = (int64_t)c0 * N;
            PostArgs pc = post;
            if (pc.y2) pc.y2 += yo;
            qd_status cs = run_mv(fmt, ffn, W0, W1, x + xo, norm_w, eps, act, y + yo, g_out ? g_out + yo : nullptr,
                                  u_out ? u_out + yo : nullptr, N, K, nb, stream, ws_offset, res ? res + yo : nullptr,
                                  pc, fixed);
            if (cs != QD_OK) return cs;
        }
        return QD_OK;
    }

    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    // the row epilogue keeps the projection in the workspace, after the
    // split-K partials (if any)
    qd::PostNorm pn{};
    auto bind_post = [&](size_t p_offset, unsigned tiles, const Workspace &w) {
        pn.w1 = post.w1;
        pn.w2 = post.w2;
        pn.r = res;
        pn.y2 = post.y2;
        pn.p = w.partials + p_offset;
        pn.ctr = w.counters + kMaxTiles;  // auxiliary counter 0
        pn.tiles = tiles;
        pn.eps = post.eps;
    };
    const size_t p_floats = pnorm ? (size_t)batch * N : 0;
    if (!launch_forced()) {
        qd::StreamArgs sa{};
        unsigned grid = 0;
        size_t lds = 0;
        if (stream_plan(fmt, ffn, N, K, batch, norm_w, &sa, &grid, &lds)) {
            if (pnorm) {
                Workspace w;
                st = acquire_ws(hs, ws_offset + p_floats, fixed, &w);
                if (st != QD_OK) return st;
                bind_post(ws_offset, grid, w);
                sa.pn = pn;
            }
            sa.W0 = static_cast<const uint8_t *>(W0);
            sa.W1 = static_cast<const uint8_t *>(W1);
            sa.x = x;
            sa.y = y;
            sa.g_out = g_out;
            sa.u_out = u_out;
            sa.res = pnorm ? nullptr : res;
            sa.act = act;
            sa.eps = eps;
            hipError_t e = qd::launch_stream(fmt, batch, ffn, sa, grid, lds, hs);
            return e == hipSuccess ? QD_OK : QD_ELAUNCH;
        }
    }
    Plan p = choose_plan(fmt, N, K, batch, ffn);
    qd::MvArgs a{};
    a.W0 = static_cast<const uint8_t *>(W0);
    a.W1 = static_cast<const uint8_t *>(W1);
    a.x = x;
    a.norm_w = norm_w;
    a.y = y;
    a.g_out = g_out;
    a.u_out = u_out;
    a.res = pnorm ? nullptr : res;
    a.N = N;
    a.K = K;
    a.row_bytes = row_bytes(fmt, K);
    a.nb = (int)((K + qd::kSuper - 1) / qd::kSuper);
    a.nblk = (int)(K / block_elems(fmt));
    a.nk = p.nk;
    a.act = act;
    a.eps = eps;
    const size_t part_floats = p.s.p_out > 1 ? (size_t)p.s.p_out * batch * (ffn ? 2 : 1) * N : 0;
    if (part_floats + p_floats > 0) {
        Workspace w;
        qd_status ws = acquire_ws(hs, ws_offset + part_floats + p_floats, fixed, &w);
        if (ws != QD_OK) return ws;
        a.partials = w.partials + ws_offset;
        a.counters = w.counters;
        if (pnorm) {
            bind_post(ws_offset + part_floats, (unsigned)p.tiles, w);
            a.pn = pn;
        }
    }
    hipError_t e = qd::launch_gemv(fmt, batch, ffn, a, p.s, hs);
    return e == hipSuccess ? QD_OK : QD_ELAUNCH;
}

// y = Wd (act(Wg xn) * (Wu xn)) as the two calls qffn_gate_up_act + qgemv on
// the same stream, h in the stream's workspace unless the caller keeps it.
qd_status run_ffn_decode(int fmt_gu, const void *Wg, const void *Wu, int fmt_d, const void *Wd,
                         const float *x, const float *norm_w, float eps, int act, float *y,
                         float *h_out, int64_t N_ff, int64_t K, int batch, void *stream,
                         const float *res = nullptr, const PostArgs &post = PostArgs(),
                         const Workspace *fixed = nullptr) {
    qd_status st = check_shape(fmt_gu, N_ff, K, batch);
    if (st != QD_OK) return st;
    st = check_shape(fmt_d, K, N_ff, batch);
    if (st != QD_OK) return st;
    if (!Wg || !Wu || !Wd || !x || !y) return QD_EINVAL;
    if (act != QD_ACT_GELU_TANH && act != QD_ACT_SILU) return QD_EINVAL;
    if (!aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(Wd, 16) || !aligned(x, 16)) return QD_EALIGN;
    if ((norm_w && !aligned(norm_w, 16)) || !aligned(y, 4)) return QD_EALIGN;
    if (h_out && !aligned(h_out, 16)) return QD_EALIGN;
    const size_t xbytes = (size_t)batch * K * 4, hbytes = (size_t)batch * N_ff * 4;
    const void *ins[5] = {Wg, Wu, Wd, x, norm_w};
    const size_t insz[5] = {(size_t)N_ff * row_bytes(fmt_gu, K), (size_t)N_ff * row_bytes(fmt_gu, K),
                            (size_t)K * row_bytes(fmt_d, N_ff), xbytes, (size_t)K * 4};
    for (int i = 0; i < 5; i++) {
        if (overlap(y, xbytes, ins[i], insz[i]) || (h_out && overlap(h_out, hbytes, ins[i], insz[i])))
            return QD_EINVAL;
    }
    if (h_out && overlap(y, xbytes, h_out, hbytes)) return QD_EINVAL;
    if (res && ((res != y && overlap(res, xbytes, y, xbytes)) || (h_out && overlap(res, xbytes, h_out, hbytes))))
        return QD_EINVAL;
    if (post.y2) {
        for (int i = 0; i < 5; i++)
            if (overlap(post.y2, xbytes, ins[i], insz[i])) return QD_EINVAL;
        if (h_out && overlap(post.y2, xbytes, h_out, hbytes)) return QD_EINVAL;
    }
    if (res && !aligned(res, 4)) return QD_EALIGN;
    const bool mq = use_mq(batch, K) && use_mq(batch, N_ff);
    if (!mq && batch > QD_BATCH_CHUNK) {
        for (int c0 = 0; c0 < batch; c0 += QD_BATCH_CHUNK) {
            const int nb = std::min(QD_BATCH_CHUNK, batch - c0);
            const int64_t xo = (int64_t)c0 * K;
            PostArgs pc = post;
            if (pc.y2) pc.y2 += xo;
            qd_status cs = run_ffn_decode(fmt_gu, Wg, Wu, fmt_d, Wd, x + xo, norm_w, eps, act, y + xo,
                                          h_out ? h_out + (int64_t)c0 * N_ff : nullptr, N_ff, K, nb, stream,
                                          res ? res + xo : nullptr, pc, fixed);
            if (cs != QD_OK) return cs;
        }
        return QD_OK;
    }

    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (mq) {
        // gate/up writes h as the down projection's digits (and as fp32 only
        // when the caller keeps h): [down digits][gate/up digits + partials,
        // then down partials + post-norm projection]
        const MqPlan qa = mq_plan(fmt_gu, N_ff, K, batch, true);
        const MqPlan qb = mq_plan(fmt_d, K, N_ff, batch, false);
        const size_t need = qb.dig_floats + std::max(qa.floats(), qb.part_floats + (post.w1 ? (size_t)batch * K : 0));
        Workspace w;
        st = acquire_ws(hs, need, fixed, &w);
        if (st != QD_OK) return st;
        if (fixed) {
            hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, hs, w.counters, kCounterWords);
            if (hipGetLastError() != hipSuccess) return QD_ELAUNCH;
        }
        HDigits hd;
        hd.dig = reinterpret_cast<uint8_t *>(w.partials);
        hd.nb = qb.nb;
        hd.sx = fmt_d == QD_Q4_K;
        float *region = w.partials + qb.dig_floats;
        st = mq_run(qa, fmt_gu, true, Wg, Wu, x, nullptr, norm_w, eps, act, h_out, nullptr, nullptr, N_ff, K, batch,
                    hs, w, region, nullptr, PostArgs(), hd);
        if (st != QD_OK) return st;
        return mq_run(qb, fmt_d, false, Wd, nullptr, nullptr, hd.dig, nullptr, 0.f, 0, y, nullptr, nullptr, K, N_ff,
                      batch, hs, w, region, res, post);
    }
    const size_t h_floats = h_out ? 0 : (((size_t)batch * N_ff + 63) / 64) * 64;
    // size the workspace once for h and both calls' split-K partials, so
    // that neither call reallocates it under h
    size_t need_a = 0, need_b = post.w1 ? (size_t)batch * K : 0;
    {
        const Plan qa = choose_plan(fmt_gu, N_ff, K, batch, true);
        const Plan qb = choose_plan(fmt_d, K, N_ff, batch, false);
        need_a = qa.s.p_out > 1 ? (size_t)qa.s.p_out * batch * 2 * N_ff : 0;
        need_b += qb.s.p_out > 1 ? (size_t)qb.s.p_out * batch * K : 0;
    }
    float *h = h_out;
    if (h_floats + std::max(need_a, need_b) > 0) {
        Workspace w;
        st = acquire_ws(hs, h_floats + std::max(need_a, need_b), fixed, &w);
        if (st != QD_OK) return st;
        if (!h) h = w.partials;
        if (fixed) {
            // the scratch keeps the last call's contents: its counters start
            // this call at zero
            hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, hs, w.counters, kCounterWords);
            if (hipGetLastError() != hipSuccess) return QD_ELAUNCH;
        }
    }
    st = run_mv(fmt_gu, true, Wg, Wu, x, norm_w, eps, act, h, nullptr, nullptr, N_ff, K, batch, stream,
                h_floats, nullptr, PostArgs(), fixed);
    if (st != QD_OK) return st;
    return run_mv(fmt_d, false, Wd, nullptr, h, nullptr, 0.f, 0, y, nullptr, nullptr, K, N_ff, batch, stream,
                  h_floats, res, post, fixed);
}

// ------------------------------------------------------------ prefill ---
std::atomic<int> g_gemm_tm{0}, g_gemm_splits{0}, g_gemm_sk{0};
constexpr int kGemmTargetWorkgroups = 256;  // one resident workgroup per CU (LDS and registers)
constexpr int kGemmMinKTiles = 8;          // K-tiles per split, at least

struct GemmPlan {
    int tm, m_tiles, n_tiles, kt_total, kt_per_split, splits;
    int sk_per;  // stream-K units per workgroup (0: one tile or K-slice each)
    int64_t grid() const {
        const int64_t units = (int64_t)m_tiles * n_tiles * kt_total;
        return sk_per > 0 ? (units + sk_per - 1) / sk_per : (int64_t)m_tiles * n_tiles * splits;
    }
};

GemmPlan gemm_plan(bool ffn, int64_t M, int64_t N, int64_t K) {
    GemmPlan p;
    p.tm = g_gemm_tm.load() ? g_gemm_tm.load() : (M > 64 ? 4 : 2);
    const int64_t bm = 32 * p.tm, bn = ffn ? qd::kGemmCols / 2 : qd::kGemmCols;
    p.m_tiles = (int)((M + bm - 1) / bm);
    p.n_tiles = (int)((N + bn - 1) / bn);
    p.kt_total = (int)((K + qd::kGemmKT - 1) / qd::kGemmKT);
    const int64_t tiles = (int64_t)p.m_tiles * p.n_tiles;
    int s = 1;
    if (tiles <= kMaxTiles) {
        // split K only while the splits still fit in one round of resident
        // workgroups: a partial tile costs a write and a read of 32*tm*256
        // floats, and splits beyond one round only add that traffic
        // (measured: Gemma-4-31B down, 84 tiles: 3 splits 300 us, 4: 412, 7: 502)
        while (tiles * (s + 1) <= kGemmTargetWorkgroups && p.kt_total / (s + 1) >= kGemmMinKTiles)
            s++;
        if (g_gemm_splits.load()) s = std::min(g_gemm_splits.load(), p.kt_total);
    }
    p.kt_per_split = (p.kt_total + s - 1) / s;
    p.splits = (p.kt_total + p.kt_per_split - 1) / p.kt_per_split;  // every split non-empty
    // stream-K only on request: each workgroup an equal run of (tile,
    // K-tile) units.  Measured level with whole tiles on the Gemma-4-31B
    // gate/up (512 tokens: 672 tiles, 2.625 rounds of 256; 298-306 us either
    // way) and slower on its split-K down (247 against 176 us)
    p.sk_per = 0;
    const int sk = g_gemm_sk.load();
    if (sk > 0 && tiles <= kMaxTiles) p.sk_per = (int)std::min<int64_t>(sk, tiles * p.kt_total);
    if (p.sk_per > 0) {
        p.splits = 1;
        p.kt_per_split = p.kt_total;
    }
    return p;
}

qd_status run_gemm(int fmt, bool ffn, const void *Wg, const void *Wu, const uint16_t *X, int act,
                   float *Y, uint16_t *H, float *g_out, float *u_out, int64_t M, int64_t N,
                   int64_t K, void *stream) {
    qd_status st = check_shape(fmt, N, K, 1);
    if (st != QD_OK) return st;
    if (M < 1 || M * K > INT32_MAX) return QD_ESHAPE;
    if (!Wg || !X || (ffn ? (!Wu || !H) : !Y)) return QD_EINVAL;
    if (ffn && act != QD_ACT_GELU_TANH && act != QD_ACT_SILU) return QD_EINVAL;
    if (!aligned(Wg, 16) || (Wu && !aligned(Wu, 16)) || !aligned(X, 16)) return QD_EALIGN;
    if ((Y && !aligned(Y, 4)) || (H && !aligned(H, 2)) || (g_out && !aligned(g_out, 4)) ||
        (u_out && !aligned(u_out, 4)))
        return QD_EALIGN;
    const size_t wbytes = (size_t)N * row_bytes(fmt, K), xbytes = (size_t)M * K * 2;
    const size_t f32bytes = (size_t)M * N * 4, hbytes = (size_t)M * N * 2;
    const void *outs[4] = {ffn ? nullptr : Y, H, g_out, u_out};
    const size_t osz[4] = {f32bytes, hbytes, f32bytes, f32bytes};
    for (int i = 0; i < 4; i++) {
        if (!outs[i]) continue;
        if (overlap(outs[i], osz[i], X, xbytes) || overlap(outs[i], osz[i], Wg, wbytes) ||
            (Wu && overlap(outs[i], osz[i], Wu, wbytes)))
            return QD_EINVAL;
        for (int j = i + 1; j < 4; j++)
            if (outs[j] && overlap(outs[i], osz[i], outs[j], osz[j])) return QD_EINVAL;
    }

    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    const GemmPlan p = gemm_plan(ffn, M, N, K);
    qd::GemmArgs a{};
    a.Wg = static_cast<const uint8_t *>(Wg);
    a.Wu = static_cast<const uint8_t *>(Wu);
    a.X = X;
    a.Y = ffn ? nullptr : Y;
    a.H = H;
    a.g_out = g_out;
    a.u_out = u_out;
    a.M = M;
    a.N = N;
    a.K = K;
    a.row_bytes = row_bytes(fmt, K);
    a.nblk = (int)(K / block_elems(fmt));
    a.kt_total = p.kt_total;
    a.kt_per_split = p.kt_per_split;
    a.splits = p.splits;
    a.m_tiles = p.m_tiles;
    a.n_tiles = p.n_tiles;
    a.act = act;
    a.sk_per = p.sk_per;
    if (p.grid() <= 0 || p.grid() > 0x7FFFFFFF) return QD_ESHAPE;
    if (p.splits > 1 || p.sk_per > 0) {
        Workspace w;
        const size_t tile_f = (size_t)(32 * p.tm) * qd::kGemmCols;
        const size_t need = p.sk_per > 0 ? 2 * (size_t)p.grid() * tile_f
                                         : (size_t)p.m_tiles * p.n_tiles * p.splits * tile_f;
        st = get_workspace(hs, need, &w);
        if (st != QD_OK) return st;
        a.partials = w.partials;
        a.counters = w.counters;
    }
    hipError_t e = qd::launch_gemm(fmt, ffn, p.tm, a, hs);
    return e == hipSuccess ? QD_OK : QD_ELAUNCH;
}

// Q, K and V projections of one attention input in one launch (larql Gemma 3
// table: the input norm and the QKV projection fused into one dispatch, Q/K
// in Q4_K and V in Q6_K).  Each matrix keeps the launch shape the planner
// gives it as a plain GEMV, without a split across workgroups; where its
// activation slice does not fit one workgroup's LDS the three projections
// run as three GEMV calls instead.
qd_status run_qkv(const int fmt[3], const void *const W[3], const int64_t N[3], const float *x,
                  const float *norm_w, float eps, float *const y[3], int64_t K, int batch,
                  void *stream) {
    for (int i = 0; i < 3; i++) {
        qd_status st = check_shape(fmt[i], N[i], K, batch);
        if (st != QD_OK) return st;
        if (!W[i] || !y[i]) return QD_EINVAL;
    }
    if (!x) return QD_EINVAL;
    if (!aligned(x, 16) || (norm_w && !aligned(norm_w, 16))) return QD_EALIGN;
    for (int i = 0; i < 3; i++)
        if (!aligned(W[i], 16) || !aligned(y[i], 4)) return QD_EALIGN;
    const size_t xbytes = (size_t)batch * K * 4;
    for (int i = 0; i < 3; i++) {
        const size_t yb = (size_t)batch * N[i] * 4;
        if (overlap(y[i], yb, x, xbytes) || (norm_w && overlap(y[i], yb, norm_w, (size_t)K * 4)))
            return QD_EINVAL;
        for (int j = 0; j < 3; j++) {
            if (overlap(y[i], yb, W[j], (size_t)N[j] * row_bytes(fmt[j], K))) return QD_EINVAL;
            if (j != i && overlap(y[i], yb, y[j], (size_t)batch * N[j] * 4)) return QD_EINVAL;
        }
    }
    if (batch > QD_BATCH_CHUNK) {
        for (int c0 = 0; c0 < batch; c0 += QD_BATCH_CHUNK) {
            const int nbc = std::min(QD_BATCH_CHUNK, batch - c0);
            float *const yc[3] = {y[0] + (int64_t)c0 * N[0], y[1] + (int64_t)c0 * N[1], y[2] + (int64_t)c0 * N[2]};
            qd_status cs = run_qkv(fmt, W, N, x + (int64_t)c0 * K, norm_w, eps, yc, K, nbc, stream);
            if (cs != QD_OK) return cs;
        }
        return QD_OK;
    }
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (batch == 1 && !launch_forced() && K % qd::kSuper == 0) {
        // batch 1: the three matrices on the streaming kernel in one launch,
        // the CUs shared in proportion to their bytes (Gemma-3-4B: 115, 57
        // and 83 workgroups)
        qd::StreamQkvArgs q{};
        size_t lds = 0;
        int64_t bytes[3], total = 0;
        for (int i = 0; i < 3; i++) {
            bytes[i] = N[i] * row_bytes(fmt[i], K);
            total += bytes[i];
        }
        bool ok = true;
        for (int i = 0; i < 3 && ok; i++) {
            const int G = (int)std::max<int64_t>(1, std::min<int64_t>(N[i], kCUs * bytes[i] / total));
            const int64_t wg_bytes = (N[i] + G - 1) / G * row_bytes(fmt[i], K);
            const int prod = wg_bytes >= (int64_t(256) << 10) ? 4 : 2;
            unsigned g = 0;
            size_t l = 0;
            ok = bytes[i] % 16 == 0 &&
                 stream_plan_pc(fmt[i], false, N[i], K, 1, norm_w, 1, 8, prod, 4, &q.a[i], &g, &l, 1, G);
            if (!ok) break;
            qd::StreamArgs &a = q.a[i];
            a.W0 = static_cast<const uint8_t *>(W[i]);
            a.x = x;
            a.y = y[i];
            a.eps = eps;
            q.fmt[i] = fmt[i];
            q.wgs[i] = (int)g;
            lds = std::max(lds, l);
        }
        if (ok) {
            hipError_t e = qd::launch_stream_qkv(q, lds, hs);
            return e == hipSuccess ? QD_OK : QD_ELAUNCH;
        }
    }
    const int nb = (int)(K / qd::kSuper);
    bool fused = K % qd::kSuper == 0;
    for (int i = 0; i < 3 && fused; i++) fused = nb <= lds_units_max(fmt[i], batch);
    if (!fused) {
        for (int i = 0; i < 3; i++) {
            qd_status st = run_mv(fmt[i], false, W[i], nullptr, x, norm_w, eps, 0, y[i], nullptr,
                                  nullptr, N[i], K, batch, stream);
            if (st != QD_OK) return st;
        }
        return QD_OK;
    }
    // Lane groups per row: the fewest (from 2) that give the launch a
    // workgroup per CU.  Measured on MI355X, Gemma-3-4B Q/K/V (4096 rows over
    // K = 2560, graph replay, rotating weights): 4 per row (256 workgroups)
    // 7.4 us, 8 per row 7.4 us, 16 per row (1024 workgroups, each staging x)
    // 10.1-10.3 us; three separate GEMV launches 18.3 us.
    int p_in = 2;
    const int64_t rows = N[0] + N[1] + N[2];
    while (p_in < 16 && rows * p_in / qd::kGroups < kCUs) p_in *= 2;
    if (const int op = g_over_pin.load()) p_in = op;
    qd::QkvArgs q{};
    size_t lds = 0;
    for (int i = 0; i < 3; i++) {
        const Plan p = make_plan(fmt[i], N[i], K, batch, false, Shape{p_in, 1, 1, 1});
        qd::MvArgs &a = q.a[i];
        a.W0 = static_cast<const uint8_t *>(W[i]);
        a.x = x;
        a.norm_w = norm_w;
        a.y = y[i];
        a.N = N[i];
        a.K = K;
        a.row_bytes = row_bytes(fmt[i], K);
        a.nb = nb;
        a.nblk = (int)(K / block_elems(fmt[i]));
        a.nk = p.nk;
        a.p_in = p.s.p_in;
        a.p_out = 1;
        a.rpg = 1;
        a.eps = eps;
        q.fmt[i] = fmt[i];
        q.tiles[i] = (int)p.tiles;
        lds = std::max(lds, qd::mv_lds_bytes(fmt[i], batch, p.nk));
    }
    hipError_t e = qd::launch_qkv(q, batch, lds, hs);
    return e == hipSuccess ? QD_OK : QD_ELAUNCH;
}

// Mixture-of-experts decode FFN, batch 1: y = sum_z coef[z] * Wd[e_z] h_z,
// h_z = act(Wg[e_z] xn) * (Wu[e_z] xn), e_z = ids[z] (device arrays).
constexpr int kMoeMaxSlots = 64;

// Lane groups per row: the fewest (from 2) that give a workgroup per CU over
// all slots.
int moe_p_in(int64_t rows, int n_sel) {
    int p_in = 2;
    while (p_in < 16 && (rows * p_in / qd::kGroups) * n_sel < kCUs) p_in *= 2;
    return p_in;
}

qd_status run_moe(int fmt_gu, const void *Wg, const void *Wu, int fmt_d, const void *Wd, int n_experts,
                  const int32_t *ids, const float *coef, int n_sel, const float *x, const float *norm_w,
                  float eps, int act, float *y, float *h_out, int64_t N_ff, int64_t K, void *stream) {
    qd_status st = check_shape(fmt_gu, N_ff, K, 1);
    if (st != QD_OK) return st;
    st = check_shape(fmt_d, K, N_ff, 1);
    if (st != QD_OK) return st;
    if (n_experts < 1 || n_sel < 1 || n_sel > kMoeMaxSlots) return QD_ESHAPE;
    if (!Wg || !Wu || !Wd || !ids || !coef || !x || !y) return QD_EINVAL;
    if (act != QD_ACT_GELU_TANH && act != QD_ACT_SILU) return QD_EINVAL;
    if (!aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(Wd, 16) || !aligned(x, 16)) return QD_EALIGN;
    if ((norm_w && !aligned(norm_w, 16)) || (h_out && !aligned(h_out, 16))) return QD_EALIGN;
    if (!aligned(y, 4) || !aligned(ids, 4) || !aligned(coef, 4)) return QD_EALIGN;
    const int64_t rb_a = row_bytes(fmt_gu, K), rb_b = row_bytes(fmt_d, N_ff);
    const size_t ybytes = (size_t)K * 4, hbytes = (size_t)n_sel * N_ff * 4;
    const void *ins[7] = {Wg, Wu, Wd, x, norm_w, ids, coef};
    const size_t insz[7] = {(size_t)n_experts * N_ff * rb_a, (size_t)n_experts * N_ff * rb_a,
                            (size_t)n_experts * K * rb_b, (size_t)K * 4, (size_t)K * 4,
                            (size_t)n_sel * 4, (size_t)n_sel * 4};
    for (int i = 0; i < 7; i++)
        if (overlap(y, ybytes, ins[i], insz[i]) || (h_out && overlap(h_out, hbytes, ins[i], insz[i])))
            return QD_EINVAL;
    if (h_out && overlap(y, ybytes, h_out, hbytes)) return QD_EINVAL;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    const size_t h_floats = h_out ? 0 : (((size_t)n_sel * N_ff + 63) / 64) * 64;
    if (!launch_forced()) {
        qd::StreamArgs sa{}, sb{};
        unsigned ga = 0, gb = 0;
        size_t la = 0, lb = 0;
        if (stream_plan_moe(fmt_gu, true, N_ff, K, n_sel, norm_w, &sa, &ga, &la) &&
            stream_plan_moe(fmt_d, false, K, N_ff, n_sel, nullptr, &sb, &gb, &lb)) {
            Workspace w;
            st = get_workspace(hs, h_floats + (size_t)n_sel * K, &w);
            if (st != QD_OK) return st;
            float *h = h_out ? h_out : w.partials;
            sa.W0 = static_cast<const uint8_t *>(Wg);
            sa.W1 = static_cast<const uint8_t *>(Wu);
            sa.x = x;
            sa.y = h;
            sa.act = act;
            sa.eps = eps;
            sa.ids = ids;
            sa.n_experts = n_experts;
            sa.n_sel = n_sel;
            sa.w_estride = N_ff * rb_a;
            sa.y_sstride = N_ff;
            hipError_t e = qd::launch_stream_moe(fmt_gu, true, sa, ga, la, hs);
            if (e != hipSuccess) return QD_ELAUNCH;
            sb.W0 = static_cast<const uint8_t *>(Wd);
            sb.x = h;
            sb.y = y;
            sb.ids = ids;
            sb.coef = coef;
            sb.n_experts = n_experts;
            sb.n_sel = n_sel;
            sb.w_estride = K * rb_b;
            sb.x_sstride = N_ff;
            sb.part = w.partials + h_floats;
            sb.counters = w.counters;
            e = qd::launch_stream_moe(fmt_d, false, sb, gb, lb, hs);
            return e == hipSuccess ? QD_OK : QD_ELAUNCH;
        }
    }

    // register kernel: every slot stages its whole activation row in one
    // workgroup
    const int nb_a = (int)((K + qd::kSuper - 1) / qd::kSuper);
    const int nb_b = (int)((N_ff + qd::kSuper - 1) / qd::kSuper);
    if (nb_a > lds_units_max(fmt_gu, 1) || nb_b > lds_units_max(fmt_d, 1)) return QD_EUNSUPPORTED;
    const Plan pa = make_plan(fmt_gu, N_ff, K, 1, true, Shape{moe_p_in(N_ff, n_sel), 1, 1, 1});
    const Plan pb = make_plan(fmt_d, K, N_ff, 1, false, Shape{moe_p_in(K, n_sel), 1, 1, 1});
    if (pb.tiles > kMaxTiles) return QD_EUNSUPPORTED;
    Workspace w;
    st = get_workspace(hs, h_floats + (size_t)n_sel * K, &w);
    if (st != QD_OK) return st;
    float *h = h_out ? h_out : w.partials;

    qd::MvArgs a{};
    a.W0 = static_cast<const uint8_t *>(Wg);
    a.W1 = static_cast<const uint8_t *>(Wu);
    a.x = x;
    a.norm_w = norm_w;
    a.y = h;
    a.N = N_ff;
    a.K = K;
    a.row_bytes = rb_a;
    a.nb = nb_a;
    a.nblk = (int)(K / block_elems(fmt_gu));
    a.nk = nb_a;
    a.p_in = pa.s.p_in;
    a.p_out = 1;
    a.rpg = 1;
    a.act = act;
    a.eps = eps;
    a.ids = ids;
    a.w_estride = N_ff * rb_a;
    a.y_sstride = N_ff;
    a.n_experts = n_experts;
    hipError_t e = qd::launch_moe(fmt_gu, true, a, pa.tiles, n_sel, hs);
    if (e != hipSuccess) return QD_ELAUNCH;

    qd::MvArgs b{};
    b.W0 = static_cast<const uint8_t *>(Wd);
    b.x = h;
    b.y = y;
    b.partials = w.partials + h_floats;
    b.counters = w.counters;
    b.N = K;
    b.K = N_ff;
    b.row_bytes = rb_b;
    b.nb = nb_b;
    b.nblk = (int)(N_ff / block_elems(fmt_d));
    b.nk = nb_b;
    b.p_in = pb.s.p_in;
    b.p_out = n_sel;
    b.rpg = 1;
    b.ids = ids;
    b.coef = coef;
    b.w_estride = K * rb_b;
    b.x_sstride = N_ff;
    b.n_experts = n_experts;
    e = qd::launch_moe(fmt_d, false, b, pb.tiles, n_sel, hs);
    return e == hipSuccess ? QD_OK : QD_ELAUNCH;
}

// Q8_0 weights against int8-quantized activations (opt-in; dotLLM's CPU
// Q8_0 GEMM on pre-quantized input).
// workgroups per CU of the int8-activation GEMV: each quantizes x once and
// then takes ceil(tiles / grid) row tiles (1 to 16 time the same on the
// 262144 x 2560 lm_head)
constexpr int kQ8aWgPerCu = 4;

// Launch plan of the int8-activation GEMV.
struct Q8Plan {
    int p = 1;        // lane groups per row
    int ks = 1;       // K-slices across workgroups
    int su_per = 0;   // superunits per slice
    int chunk = 0;    // columns per launch (0: one column's slice does not fit LDS)
    int64_t tiles = 0;
};

Q8Plan q8act_plan(int64_t N, int64_t K, int batch) {
    const int nsu = (int)((K / 32 + 7) / 8);
    Q8Plan pl;
    // lane groups per row.  One column: as many as leave each at least two
    // superunits (parallelism within the row).  More columns: at most 4, and
    // at least 8 superunits each, because lane groups of different rows read
    // the same LDS codes (a broadcast) only when they walk the same
    // superunit, and each column multiplies those reads (sweep over the
    // Gemma-3/4 and lm_head shapes, batch 1-8).
    if (batch == 1)
        while (pl.p < 16 && 4 * pl.p <= nsu) pl.p *= 2;
    else
        while (pl.p < 4 && 16 * pl.p <= nsu) pl.p *= 2;
    // Several columns on a matrix with few row tiles: split K across
    // workgroups instead (one lane group per row, up to 8 slices of at least
    // two superunits, aiming at 1024 workgroups), so each stages only its
    // slice of the codes.  Gemma-3 down at batch 8: 53 -> 23 us; Gemma-4
    // down 141 -> 47 us; Gemma-3 gate 24 -> 19 us.  One column gains nothing.
    if (batch > 1) {
        const int64_t tiles1 = (N + qd::kGroups - 1) / qd::kGroups;
        const int64_t want = (1024 + tiles1 - 1) / tiles1;
        const int ks = (int)std::min<int64_t>(std::min<int64_t>(8, nsu / 2), want);
        if (ks > 1) {
            pl.p = 1;
            pl.ks = ks;
        }
    }
    if (g_over_pin.load() != 0) pl.p = g_over_pin.load();  // tuning overrides
    if (g_over_pout.load() != 0) pl.ks = g_over_pout.load();
    const int64_t rows_wg = qd::kGroups / pl.p;
    pl.tiles = (N + rows_wg - 1) / rows_wg;
    pl.ks = std::min(pl.ks, nsu);
    pl.su_per = (nsu + pl.ks - 1) / pl.ks;
    pl.ks = (nsu + pl.su_per - 1) / pl.su_per;  // every slice non-empty
    if (pl.ks > 1 && pl.tiles > kMaxTiles) {
        pl.ks = 1;
        pl.su_per = nsu;
    }
    // a column whose codes do not fit one workgroup's LDS: slices of the
    // largest superunit count that fits (when the row tiles can carry
    // counters).  su_fit only decreases, so the search ends; the slices are
    // then balanced, which never makes one larger than su_fit.
    if (pl.tiles <= kMaxTiles) {
        int su_fit = pl.su_per;
        while (su_fit > 1 && qd::q8act_lds_bytes(1, std::min<int64_t>(K, (int64_t)su_fit * qd::kSuper)) >
                                 (size_t)qd::kLdsBudgetBytes)
            su_fit--;
        if (su_fit < pl.su_per) {
            pl.ks = (nsu + su_fit - 1) / su_fit;
            pl.su_per = (nsu + pl.ks - 1) / pl.ks;
            pl.ks = (nsu + pl.su_per - 1) / pl.su_per;
        }
    }
    // columns per launch: at most QD_BATCH_CHUNK, and as many as one
    // workgroup's LDS holds quantized (its K-slice of each)
    const int64_t kslice = std::min<int64_t>(K, (int64_t)pl.su_per * qd::kSuper);
    int chunk = std::min(batch, QD_BATCH_CHUNK);
    while (chunk > 1 && qd::q8act_lds_bytes(chunk, kslice) > (size_t)qd::kLdsBudgetBytes) chunk--;
    pl.chunk = qd::q8act_lds_bytes(chunk, kslice) > (size_t)qd::kLdsBudgetBytes ? 0 : chunk;
    return pl;
}

// Partial-sum floats the plan needs in the workspace.
size_t q8act_partial_floats(const Q8Plan &pl, int64_t N) {
    return pl.ks > 1 ? (size_t)pl.ks * (size_t)pl.chunk * (size_t)N : 0;
}

// The GEMV launches on validated codes q [batch][K] and scales d [batch][K/32].
qd_status launch_q8act_chunks(const Q8Plan &pl, const void *W, const int8_t *q, const float *d, float *y,
                              int64_t N, int64_t K, int batch, float *partials, unsigned *counters,
                              hipStream_t hs) {
    const int64_t nblk = K / 32;
    const int64_t kslice = std::min<int64_t>(K, (int64_t)pl.su_per * qd::kSuper);
    for (int c0 = 0; c0 < batch; c0 += pl.chunk) {
        const int nb = std::min(pl.chunk, batch - c0);
        qd::Q8ActArgs a{};
        a.W = static_cast<const uint8_t *>(W);
        a.q = q + (int64_t)c0 * K;
        a.d = d + (int64_t)c0 * nblk;
        a.y = y + (int64_t)c0 * N;
        a.N = N;
        a.K = K;
        a.row_bytes = row_bytes(QD_Q8_0, K);
        a.p = pl.p;
        a.off_scales = (int)(((size_t)nb * kslice + 15) & ~(size_t)15);
        a.ks = pl.ks;
        a.su_per = pl.su_per;
        a.partials = partials;
        a.counters = counters;
        // split K: one row tile per workgroup; else a grid that strides over
        // the tiles, each workgroup staging the codes once
        const unsigned grid = (unsigned)(pl.ks > 1 ? pl.tiles
                                                   : std::min<int64_t>(pl.tiles, (int64_t)kQ8aWgPerCu * kCUs));
        if (qd::launch_q8act(a, nb, grid, hs) != hipSuccess) return QD_ELAUNCH;
    }
    return QD_OK;
}

qd_status run_q8quant(const float *x, int8_t *q, float *d, int64_t K, int batch, void *stream) {
    qd_status st = check_shape(QD_Q8_0, 1, K, batch);
    if (st != QD_OK) return st;
    if (!x || !q || !d) return QD_EINVAL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(d, 4)) return QD_EALIGN;
    const size_t xb = (size_t)batch * K * 4, qb = (size_t)batch * K, db = (size_t)batch * (K / 32) * 4;
    if (overlap(q, qb, x, xb) || overlap(d, db, x, xb) || overlap(q, qb, d, db)) return QD_EINVAL;
    const hipError_t e = qd::launch_q8quant(x, q, d, (int64_t)batch * (K / 32), reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? QD_OK : QD_ELAUNCH;
}

qd_status run_q8preq(const void *W, const int8_t *q, const float *d, float *y, int64_t N, int64_t K, int batch,
                     void *stream) {
    qd_status st = check_shape(QD_Q8_0, N, K, batch);
    if (st != QD_OK) return st;
    if (!W || !q || !d || !y) return QD_EINVAL;
    if (!aligned(W, 16) || !aligned(q, 16) || !aligned(d, 4) || !aligned(y, 4)) return QD_EALIGN;
    const size_t yb = (size_t)batch * N * 4;
    if (overlap(y, yb, q, (size_t)batch * K) || overlap(y, yb, d, (size_t)batch * (K / 32) * 4) ||
        overlap(y, yb, W, (size_t)N * row_bytes(QD_Q8_0, K)))
        return QD_EINVAL;
    const Q8Plan pl = q8act_plan(N, K, batch);
    if (pl.chunk == 0) return QD_EUNSUPPORTED;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    float *partials = nullptr;
    unsigned *counters = nullptr;
    if (pl.ks > 1) {
        Workspace w;
        st = get_workspace(hs, q8act_partial_floats(pl, N), &w);
        if (st != QD_OK) return st;
        partials = w.partials;
        counters = w.counters;
    }
    return launch_q8act_chunks(pl, W, q, d, y, N, K, batch, partials, counters, hs);
}

// Quantize into the stream's workspace, then the GEMV on the codes.
qd_status run_q8act(const void *W, const float *x, float *y, int64_t N, int64_t K, int batch, void *stream) {
    qd_status st = check_shape(QD_Q8_0, N, K, batch);
    if (st != QD_OK) return st;
    if (!W || !x || !y) return QD_EINVAL;
    if (!aligned(W, 16) || !aligned(x, 16)) return QD_EALIGN;
    if (!aligned(y, 4)) return QD_EALIGN;
    const size_t ybytes = (size_t)batch * N * 4;
    if (overlap(y, ybytes, x, (size_t)batch * K * 4) || overlap(y, ybytes, W, (size_t)N * row_bytes(QD_Q8_0, K)))
        return QD_EINVAL;
    const Q8Plan pl = q8act_plan(N, K, batch);
    if (pl.chunk == 0) return QD_EUNSUPPORTED;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    // codes first (batch * K bytes, rounded up to 256), then the scales,
    // then the split-K partial sums
    const size_t code_floats = (((size_t)batch * K + 255) / 256) * 64;
    const size_t scale_floats = (((size_t)batch * (K / 32) + 63) / 64) * 64;
    Workspace w;
    st = get_workspace(hs, code_floats + scale_floats + q8act_partial_floats(pl, N), &w);
    if (st != QD_OK) return st;
    int8_t *q = reinterpret_cast<int8_t *>(w.partials);
    float *d = w.partials + code_floats;
    if (qd::launch_q8quant(x, q, d, (int64_t)batch * (K / 32), hs) != hipSuccess) return QD_ELAUNCH;
    return launch_q8act_chunks(pl, W, q, d, y, N, K, batch, w.partials + code_floats + scale_floats,
                               w.counters, hs);
}

}  // namespace

extern "C" {

int qd_block_elems(qd_format fmt) { return block_elems(fmt); }
int qd_block_bytes(qd_format fmt) { return block_bytes(fmt); }
int64_t qd_row_bytes(qd_format fmt, int64_t K) { return row_bytes(fmt, K); }
int qd_version(void) { return kVersion; }

const char *qd_status_str(qd_status s) {
    switch (s) {
    case QD_OK: return "ok";
    case QD_EINVAL: return "invalid argument (null pointer, unknown enum or overlapping buffers)";
    case QD_ESHAPE: return "shape out of range (N, M, K or batch)";
    case QD_EALIGN: return "pointer not aligned as required";
    case QD_ELAUNCH: return "kernel launch failed";
    case QD_EUNSUPPORTED: return "not supported by the library";
    case QD_ENOMEM: return "workspace allocation failed";
    case QD_ECAPTURE: return "the stream is capturing a graph and the call needs a new or larger workspace";
    case QD_ETOOBIG: return "the call needs more scratch than the allocation-free entry point holds";
    default: return "unknown status";
    }
}

qd_status qgemv(qd_format fmt, const void *W, const float *x, float *y, int64_t N, int64_t K,
                int batch, void *stream) {
    return run_mv(fmt, false, W, nullptr, x, nullptr, 0.f, 0, y, nullptr, nullptr, N, K, batch,
                  stream);
}

qd_status qgemv_residual(qd_format fmt, const void *W, const float *x, const float *r, float *y,
                         int64_t N, int64_t K, int batch, void *stream) {
    if (!r) return QD_EINVAL;
    return run_mv(fmt, false, W, nullptr, x, nullptr, 0.f, 0, y, nullptr, nullptr, N, K, batch,
                  stream, 0, r);
}

qd_status qgemv_post_norm_residual(qd_format fmt, const void *W, const float *x, const float *post_w, float eps,
                                   const float *r, float *y, const float *next_w, float *y2, int64_t N, int64_t K,
                                   int batch, void *stream) {
    if (!post_w || !r || (next_w == nullptr) != (y2 == nullptr)) return QD_EINVAL;
    PostArgs pa;
    pa.w1 = post_w;
    pa.w2 = next_w;
    pa.y2 = y2;
    pa.eps = eps;
    return run_mv(fmt, false, W, nullptr, x, nullptr, 0.f, 0, y, nullptr, nullptr, N, K, batch, stream, 0, r, pa);
}

qd_status qffn_decode_post_norm_residual(qd_format fmt_gu, const void *Wg, const void *Wu, qd_format fmt_down,
                                         const void *Wd, const float *x, const float *norm_w, float eps, qd_act act,
                                         const float *post_w, const float *r, float *y, const float *next_w,
                                         float *y2, float *h_out, int64_t N_ff, int64_t K, int batch,
                                         void *stream) {
    if (!post_w || !r || (next_w == nullptr) != (y2 == nullptr)) return QD_EINVAL;
    PostArgs pa;
    pa.w1 = post_w;
    pa.w2 = next_w;
    pa.y2 = y2;
    pa.eps = eps;
    return run_ffn_decode(fmt_gu, Wg, Wu, fmt_down, Wd, x, norm_w, eps, act, y, h_out, N_ff, K, batch, stream, r,
                          pa);
}

qd_status qgemv_q8_0_q8act(const void *W, const float *x, float *y, int64_t N, int64_t K, int batch,
                          void *stream) {
    return run_q8act(W, x, y, N, K, batch, stream);
}

qd_status qquantize_q8_act(const float *x, int8_t *q, float *d, int64_t K, int batch, void *stream) {
    return run_q8quant(x, q, d, K, batch, stream);
}

qd_status qgemv_q8_0_preq(const void *W, const int8_t *q, const float *d, float *y, int64_t N, int64_t K,
                          int batch, void *stream) {
    return run_q8preq(W, q, d, y, N, K, batch, stream);
}

qd_status qgemv_q4k(const void *W, const float *x, float *y, int64_t N, int64_t K, int batch,
                    void *stream) {
    return qgemv(QD_Q4_K, W, x, y, N, K, batch, stream);
}

qd_status qgemv_q6k(const void *W, const float *x, float *y, int64_t N, int64_t K, int batch,
                    void *stream) {
    return qgemv(QD_Q6_K, W, x, y, N, K, batch, stream);
}

qd_status qgemv_q8_0(const void *W, const float *x, float *y, int64_t N, int64_t K, int batch,
                     void *stream) {
    return qgemv(QD_Q8_0, W, x, y, N, K, batch, stream);
}

qd_status qqkv_proj(qd_format fmt_q, const void *Wq, int64_t Nq, qd_format fmt_k, const void *Wk,
                    int64_t Nk, qd_format fmt_v, const void *Wv, int64_t Nv, const float *x,
                    const float *norm_w, float eps, float *q, float *k, float *v, int64_t K, int batch,
                    void *stream) {
    const int fmt[3] = {fmt_q, fmt_k, fmt_v};
    const void *const W[3] = {Wq, Wk, Wv};
    const int64_t N[3] = {Nq, Nk, Nv};
    float *const y[3] = {q, k, v};
    return run_qkv(fmt, W, N, x, norm_w, eps, y, K, batch, stream);
}

qd_status qffn_gate_up_act(qd_format fmt, const void *Wg, const void *Wu, const float *x,
                           const float *norm_w, float eps, qd_act act, float *h, float *g_out,
                           float *u_out, int64_t N_ff, int64_t K, int batch, void *stream) {
    return run_mv(fmt, true, Wg, Wu, x, norm_w, eps, act, h, g_out, u_out, N_ff, K, batch, stream);
}

qd_status qffn_decode_residual(qd_format fmt_gu, const void *Wg, const void *Wu, qd_format fmt_down,
                               const void *Wd, const float *x, const float *norm_w, float eps,
                               qd_act act, const float *r, float *y, float *h_out, int64_t N_ff,
                               int64_t K, int batch, void *stream) {
    if (!r) return QD_EINVAL;
    return run_ffn_decode(fmt_gu, Wg, Wu, fmt_down, Wd, x, norm_w, eps, act, y, h_out, N_ff, K,
                          batch, stream, r);
}

qd_status qmoe_ffn_decode(qd_format fmt_gu, const void *Wg, const void *Wu, qd_format fmt_down,
                          const void *Wd, int n_experts, const int32_t *ids, const float *coef, int n_sel,
                          const float *x, const float *norm_w, float eps, qd_act act, float *y,
                          float *h_out, int64_t N_ff, int64_t K, void *stream) {
    return run_moe(fmt_gu, Wg, Wu, fmt_down, Wd, n_experts, ids, coef, n_sel, x, norm_w, eps, act, y,
                   h_out, N_ff, K, stream);
}

qd_status qffn_decode(qd_format fmt_gu, const void *Wg, const void *Wu, qd_format fmt_down,
                      const void *Wd, const float *x, const float *norm_w, float eps, qd_act act,
                      float *y, float *h_out, int64_t N_ff, int64_t K, int batch, void *stream) {
    return run_ffn_decode(fmt_gu, Wg, Wu, fmt_down, Wd, x, norm_w, eps, act, y, h_out, N_ff, K,
                          batch, stream);
}

qd_status qffn_decode_noalloc(qd_format fmt_gu, const void *Wg, const void *Wu, qd_format fmt_down,
                              const void *Wd, const float *x, const float *norm_w, float eps, qd_act act,
                              float *y, float *h_out, int64_t N_ff, int64_t K, int batch, void *stream) {
    Workspace w;
    qd_status st = scratch_workspace(&w);
    if (st != QD_OK) return st;
    return run_ffn_decode(fmt_gu, Wg, Wu, fmt_down, Wd, x, norm_w, eps, act, y, h_out, N_ff, K, batch, stream,
                          nullptr, PostArgs(), &w);
}

qd_status qdequant(qd_format fmt, const void *W, float *out, int64_t N, int64_t K, void *stream) {
    qd_status st = check_shape(fmt, N, K, 1);
    if (st != QD_OK) return st;
    if (!W || !out) return QD_EINVAL;
    if (!aligned(W, 16)) return QD_EALIGN;
    if (!aligned(out, 4)) return QD_EALIGN;
    if (overlap(out, (size_t)N * K * 4, W, (size_t)N * row_bytes(fmt, K))) return QD_EINVAL;
    hipError_t e = qd::launch_dequant(fmt, static_cast<const uint8_t *>(W), out, nullptr, N, K,
                                      reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? QD_OK : QD_ELAUNCH;
}

qd_status qdequant_bf16(qd_format fmt, const void *W, uint16_t *out, int64_t N, int64_t K,
                        void *stream) {
    qd_status st = check_shape(fmt, N, K, 1);
    if (st != QD_OK) return st;
    if (!W || !out) return QD_EINVAL;
    if (!aligned(W, 16)) return QD_EALIGN;
    if (!aligned(out, 2)) return QD_EALIGN;
    if (overlap(out, (size_t)N * K * 2, W, (size_t)N * row_bytes(fmt, K))) return QD_EINVAL;
    hipError_t e = qd::launch_dequant(fmt, static_cast<const uint8_t *>(W), nullptr, out, N, K,
                                      reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? QD_OK : QD_ELAUNCH;
}

qd_status qgemm_prefill(qd_format fmt, const void *W, const uint16_t *X, float *Y, int64_t M,
                        int64_t N, int64_t K, void *stream) {
    return run_gemm(fmt, false, W, nullptr, X, 0, Y, nullptr, nullptr, nullptr, M, N, K, stream);
}

qd_status qgemm_prefill_gate_up_act(qd_format fmt, const void *Wg, const void *Wu,
                                    const uint16_t *X, qd_act act, uint16_t *H, float *g_out,
                                    float *u_out, int64_t M, int64_t N_ff, int64_t K,
                                    void *stream) {
    return run_gemm(fmt, true, Wg, Wu, X, act, nullptr, H, g_out, u_out, M, N_ff, K, stream);
}

qd_status qd_set_gemm_streamk(int units_per_wg) {
    if (units_per_wg < 0) return QD_EINVAL;
    g_gemm_sk.store(units_per_wg);
    return QD_OK;
}

qd_status qd_set_gemm_override(int tm, int splits) {
    if (tm != 0 && tm != 2 && tm != 4) return QD_EINVAL;
    if (splits < 0 || splits > 1024) return QD_EINVAL;
    g_gemm_tm.store(tm);
    g_gemm_splits.store(splits);
    return QD_OK;
}

qd_status qd_set_stream_override(int wg_per_cu, int depth, int consumers, int producers) {
    if (wg_per_cu < 0 || wg_per_cu > 8 || depth < 0 || depth > 32) return QD_EINVAL;
    if (consumers != 0 && consumers != 4 && consumers != 8) return QD_EINVAL;
    if (producers < 0 || producers == 3 || producers > 4) return QD_EINVAL;
    g_stream_wpc.store(wg_per_cu);
    g_stream_depth.store(depth);
    g_stream_consumers.store(consumers);
    g_stream_producers.store(producers);
    return QD_OK;
}

qd_status qd_plan_q8act(int64_t N, int64_t K, int batch, int32_t *out) {
    qd_status st = check_shape(QD_Q8_0, N, K, batch);
    if (st != QD_OK) return st;
    if (!out) return QD_EINVAL;
    const Q8Plan pl = q8act_plan(N, K, batch);
    out[0] = pl.p;
    out[1] = pl.ks;
    out[2] = pl.su_per;
    out[3] = pl.chunk;
    return QD_OK;
}

qd_status qd_set_walk_override(int rows_per_group) {
    if (rows_per_group < 0 || rows_per_group > 64) return QD_EINVAL;
    g_over_rpg.store(rows_per_group);
    return QD_OK;
}

qd_status qd_set_batch_override(int mode, int k_slices) {
    if (mode != 0 && mode != 1) return QD_EINVAL;
    if (k_slices < 0 || k_slices > 1024) return QD_EINVAL;
    g_batch_mode.store(mode);
    g_mq_pout.store(k_slices);
    return QD_OK;
}

qd_status qd_set_launch_override(int p_in, int p_out, int nr) {
    auto pow2_le16 = [](int v) { return v == 1 || v == 2 || v == 4 || v == 8 || v == 16; };
    if (p_in != 0 && !pow2_le16(p_in)) return QD_EINVAL;
    if (p_out < 0 || p_out > 256) return QD_EINVAL;
    if (nr != 0 && nr != 1 && nr != 2) return QD_EINVAL;
    g_over_pin.store(p_in);
    g_over_pout.store(p_out);
    g_over_nr.store(nr);
    return QD_OK;
}

}  // extern "C"
