// Host side of the C ABI in include/np.h: layer state, host-side validation,
// error reporting and the per-token driver (NeuroPrefetcher, sections 3.1, 3.4
// and 3.5). Every check runs before anything is enqueued, so a failing call
// leaves all state unchanged.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <utility>
#include <atomic>
#include <map>
#include <memory>
#include <mutex>
#include <condition_variable>
#include <functional>
#include <string>
#include <thread>
#include <vector>

#include "np.h"
#include "np_internal.hpp"

namespace np {
int ffn_win_max();
}

using namespace np;

// Scratch of np_sparse_ffn_noalloc: the FFN's cross-workgroup exchange words, 2 MiB per device,
// held from the library's load until the process ends. Host code never uses this name as an
// address (in host code it is a stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, once per device, when the first layer of that device is created.
namespace {
constexpr size_t kScratchWords = size_t(1) << 18;   // 64-bit (sequence, value) words: 2 MiB
constexpr size_t kScratchHWords = size_t(1) << 16;  // the first 64 Ki words: h (one per active slot)
}  // namespace
static __device__ __align__(256) uint64_t scratch[kScratchWords];

namespace {

struct DeviceScratch {
    uint64_t* ptr = nullptr;  // device address of `scratch` on that device (nullptr if unavailable)
    uint32_t seq = 0;         // sequence number of the last launch that used it
};
std::mutex g_scratch_mu;
std::map<int, DeviceScratch>& g_scratch = *new std::map<int, DeviceScratch>();

// Once per device, with that device current (called by np_layer_create).
void setup_scratch(int dev) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch.count(dev)) return;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
        (void)hipGetLastError();
        p = nullptr;  // np_sparse_ffn_noalloc then fails with NP_EHIP on this device
    }
    g_scratch[dev].ptr = static_cast<uint64_t*>(p);
}

thread_local std::string g_err;

np_status fail(np_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

#define NP_HIP(call)                                                                          \
    do {                                                                                      \
        hipError_t e_ = (call);                                                               \
        if (e_ != hipSuccess) return fail(NP_EHIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
    } while (0)

// Makes `dev` current for the scope and restores the previous device.
struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

enum LayerState { kFresh = 0, kAssigned = 1, kScattered = 2 };
constexpr size_t kCountsBytes = 8 * 4 + 2 * 8;  // int32 counts[8] + 2 x uint64 running sums (cleared by resets)
constexpr size_t kCountsAlloc = kCountsBytes + 8;  // + the device address of the host error word
constexpr int kLists = 7;                        // K-entry lists per layer

constexpr int kDefaultSlotsPerWg = 0;  // 0: one workgroup per compute unit
constexpr int kDefaultTileCols = 256;

}  // namespace

// Staging of the TokenArgs of direct token launches led by one layer: the device copy the
// launch reads and a ring of pinned host copies, each reused once its last copy to the device
// has completed. (Calls that share a leading layer are ordered, as every call on a layer is.)
struct TokenStage {
    static constexpr int kRing = 4;
    TokenArgs* dev = nullptr;
    TokenArgs* host[kRing] = {};
    hipEvent_t copied[kRing] = {};
    int next = 0;
    ~TokenStage() {
        if (dev) (void)hipFree(dev);
        for (int i = 0; i < kRing; ++i) {
            if (host[i]) (void)hipHostFree(host[i]);
            if (copied[i]) (void)hipEventDestroy(copied[i]);
        }
    }
};

// A token launch captured into a decode graph: its arguments, written once before capture.
struct TokenLaunch {
    TokenArgs* dev = nullptr;
    int grid = 0;
    FfnShape sh{};
    bool gated = false;
};

struct np_layer {
    np_layer_desc desc{};
    int W = 0, Kw = 0, n_tables = 0;
    std::vector<uint64_t> h_masks;  // copy of the centroid tables (validation, |S|)
    std::vector<uint64_t> h_res;    // host mirror of the resident set
    int32_t n_active = 0, n_in = 0;
    int64_t total_active = 0, total_in = 0;
    int state = kFresh;
    const uint16_t* store_dev = nullptr;
    bool store_is_host = false;

    uint64_t* d_masks = nullptr;
    uint16_t* buf = nullptr;
    int32_t* slot_map = nullptr;
    int32_t* owner = nullptr;
    uint64_t* res = nullptr;
    uint64_t* freeb = nullptr;
    int32_t* lists = nullptr;  // d_in | slot_in | d_out | act | act_src | mv_src | mv_dst, K each
    int32_t* counts = nullptr;  // int32 [8], the two 64-bit running sums (LayerDev::acc), the error word's address
    uint32_t* err_h = nullptr;  // pinned host word: error bits a kernel raised since the last reset
    uint64_t* ring = nullptr;   // window > 1: [window - 1][W] recent active sets
    int window = 1;
    uint64_t* levels = nullptr; // n_levels > 0: [n_levels][W] neurons per frequency level
    int n_levels = 0;
    int layout = NP_LAYOUT_SLOTS;
    int planar = 0;             // 1: one buffer per projection row instead of one bundle per slot
    int reduce = NP_REDUCE_ORDERED;  // how the FFN combines the partial sums of its workgroups
    LayerDev ldh{};             // host copy of *ldev
    uint64_t* hpair = nullptr;
    uint64_t* ppair = nullptr;
    uint32_t ffn_seq = 0;
    uint64_t version = 0;  // bumped when cached decode graphs must be rebuilt
    LayerDev* ldev = nullptr;
    hipEvent_t ev_scatter = nullptr;
    std::unique_ptr<TokenStage> tstage;  // direct token launches led by this layer

    int spw = kDefaultSlotsPerWg;
    int tw = kDefaultTileCols;
    int nt = 0;  // threads per FFN workgroup; 0 = by d_model
    int cus = 256;  // compute units of the device
    size_t ppair_words = 0;

    int32_t* d_in() const { return lists; }
    int32_t* slot_in() const { return lists + desc.k_max; }
    int32_t* d_out() const { return lists + 2 * (size_t)desc.k_max; }
    int32_t* act() const { return lists + 3 * (size_t)desc.k_max; }
    int32_t* act_src() const { return lists + 4 * (size_t)desc.k_max; }
    int32_t* mv_src() const { return lists + 5 * (size_t)desc.k_max; }
    int32_t* mv_dst() const { return lists + 6 * (size_t)desc.k_max; }
    size_t bundle_elems() const { return (size_t)desc.n_rows * desc.d_model; }
};

namespace {

// A retention rule (window or frequency levels) decides the resident set, and so |D_in|, on
// the device; without one the host knows |D_in| from its mirror of the resident set.
bool device_decides(const np_layer* L) { return L->window > 1 || L->n_levels > 0; }

int pow2_floor(int v) {
    int p = 1;
    while (p * 2 <= v) p *= 2;
    return p;
}

// 1024 threads (a whole compute unit) when x fits one 16-byte chunk per lane, else 512.
int default_threads(int d) {
    const int cpr = d / 8;
    if (cpr < 256) return 256;
    return cpr <= 512 ? 1024 : 512;
}


int q_of(const np_layer* L) { return (L->desc.d_model + L->tw - 1) / L->tw; }

// FFN launch shape for n active slots.
// fixed = true: a shape that serves every |S| <= k_max (captured decode graphs).
bool ffn_shape(const np_layer* L, int n, FfnShape* sh, bool fixed = false) {
    if (fixed) n = L->desc.k_max;
    const int d = L->desc.d_model;
    sh->nt = L->nt ? L->nt : default_threads(d);
    const int cpr = d / 8;
    const int cl = std::min(sh->nt, pow2_floor(cpr));
    sh->jx = (cpr + cl - 1) / cl;
    sh->tw = L->tw;
    sh->q = q_of(L);
    const int win = ffn_win_max();
    int p1;
    if (L->spw > 0) {
        p1 = std::max(1, (n + L->spw - 1) / L->spw);
    } else {
        // One workgroup per compute unit, so the whole grid is resident at once.
        p1 = std::max(1, L->cus - sh->q + 1);
    }
    const int per_chunk_max = win / sh->q;  // slots per chunk the window can hold
    if (per_chunk_max < 1) return false;
    p1 = std::max(p1, (n + per_chunk_max - 1) / per_chunk_max);
    if (p1 > kP1Cap) return false;
    if (!fixed) p1 = std::min(p1, std::max(1, n));
    sh->p1 = p1;
    sh->nwg = p1 + sh->q - 1;
    sh->win_max = win;
    sh->fixed = cl == 512 && sh->tw == 256 && sh->nt >= 512 ? 1 : 0;
    // 1024-thread workgroups keep x for one 16-byte chunk per lane in registers
    return sh->jx <= (sh->nt == 1024 ? 1 : 4) && sh->tw <= sh->nt;
}

np_status alloc_ffn_scratch(np_layer* L) {
    const int q = q_of(L);
    const size_t need = (size_t)(kP1Cap + q) * L->tw;
    if (L->ppair && L->ppair_words >= need) return NP_OK;
    if (L->ppair) (void)hipFree(L->ppair);
    L->ppair = nullptr;
    if (hipMalloc(&L->ppair, need * sizeof(uint64_t)) != hipSuccess) {
        (void)hipGetLastError();
        return fail(NP_ENOMEM, "cannot allocate %zu FFN partial words", need);
    }
    if (hipMemset(L->ppair, 0, need * sizeof(uint64_t)) != hipSuccess) {
        (void)hipGetLastError();
        return fail(NP_EHIP, "cannot clear FFN partial words");
    }
    L->ppair_words = need;
    return NP_OK;
}

void free_layer(np_layer* L) {
    void* ptrs[] = {L->d_masks, L->buf, L->slot_map, L->owner, L->res, L->freeb, L->lists,
                    L->counts, L->ring, L->levels, L->hpair, L->ppair, L->ldev};
    for (void* p : ptrs)
        if (p) (void)hipFree(p);
    if (L->ev_scatter) (void)hipEventDestroy(L->ev_scatter);
    if (L->err_h) (void)hipHostFree(L->err_h);
    delete L;
}

// Device state as np_layer_create leaves it (synchronous).
np_status init_state(np_layer* L) {
    const int K = L->desc.k_max, M = L->desc.d_ff;
    NP_HIP(hipMemset(L->buf, 0, (size_t)K * L->bundle_elems() * 2));
    NP_HIP(hipMemset(L->slot_map, 0xFF, (size_t)M * 4));
    NP_HIP(hipMemset(L->owner, 0xFF, (size_t)K * 4));
    NP_HIP(hipMemset(L->res, 0, (size_t)L->W * 8));
    std::vector<uint64_t> fb(L->Kw, ~0ull);
    if (K & 63) fb[L->Kw - 1] = (1ull << (K & 63)) - 1;
    NP_HIP(hipMemcpy(L->freeb, fb.data(), (size_t)L->Kw * 8, hipMemcpyHostToDevice));
    NP_HIP(hipMemset(L->lists, 0, (size_t)kLists * K * 4));
    NP_HIP(hipMemset(L->counts, 0, kCountsBytes));
    if (L->ring) NP_HIP(hipMemset(L->ring, 0, (size_t)(L->window - 1) * L->W * 8));
    NP_HIP(hipDeviceSynchronize());
    if (L->err_h) __atomic_store_n(L->err_h, 0u, __ATOMIC_RELEASE);  // no kernel of the layer is in flight
    std::fill(L->h_res.begin(), L->h_res.end(), 0ull);
    L->n_active = 0;
    L->n_in = 0;
    L->total_active = 0;
    L->total_in = 0;
    L->state = kFresh;
    return NP_OK;
}

// Host copy of the combined mask words for (gate_cid, up_cid); returns |S|.
int combine_host(const np_layer* L, int32_t g, int32_t u, uint64_t* out) {
    const uint64_t* ma = L->h_masks.data() + (size_t)g * L->W;
    const uint64_t* mb = L->h_masks.data() + ((size_t)(L->n_tables - 1) * L->desc.n_centroids + u) * L->W;
    int n = 0;
    for (int w = 0; w < L->W; ++w) {
        uint64_t s;
        switch (L->desc.mask_mode) {
            case NP_MASK_UNION: s = ma[w] | mb[w]; break;
            case NP_MASK_INTERSECT: s = ma[w] & mb[w]; break;
            default: s = ma[w]; break;
        }
        out[w] = s;
        n += __builtin_popcountll(s);
    }
    return n;
}

// Validation shared by np_delta_assign and np_decode_step.
np_status check_cids(const np_layer* L, int32_t g, int32_t u, int32_t* eff_u) {
    const int C = L->desc.n_centroids;
    if (g < 0 || g >= C) return fail(NP_EINVAL, "gate centroid id %d out of range [0, %d)", g, C);
    if (L->desc.mask_mode == NP_MASK_SINGLE) {
        *eff_u = g;
    } else {
        if (u < 0 || u >= C) return fail(NP_EINVAL, "up centroid id %d out of range [0, %d)", u, C);
        *eff_u = u;
    }
    return NP_OK;
}

int scatter_grid(int n_in) { return std::max(1, std::min(n_in, 4096)); }

// prm != nullptr: a launch captured into a decode graph (per-token values from prm).
// read_through: the slots filled by the last assignment are read from the (device) row
// store and written into the slot buffer by the FFN itself, in place of a scatter.
// y_holds_base: y already holds the value to add the FFN output to (zeros in a decode step,
// whose assign launch clears y, or the caller's value for np_sparse_ffn_acc); otherwise the
// FFN output replaces y.
// xch (optional): exchange words and sequence number to use instead of the layer's own (the
// no-allocation entry point passes its static scratch); the reduction is then the ordered one.
// Workgroups of the scatter from a host-memory row store (scatter_flat), in a launch of its
// own or as the prefetch workgroups of an FFN launch (each on a compute unit of its own; the
// FFN takes the rest): about four bundles per workgroup, at most kPrefetchWgsMax workgroups
// (48, six per XCD: on the Llama-2-7B-shaped decode, 16 to 64 keep the host link within 2 %
// of its best and 48 was the best).
constexpr int kPrefetchWgsMax = 48;
constexpr int kPrefetchBundlesPerWg = 4;
int prefetch_wgs(int n_bundles) {
    return std::max(1, std::min(kPrefetchWgsMax, (n_bundles + kPrefetchBundlesPerWg - 1) / kPrefetchBundlesPerWg));
}

struct Exchange {
    uint64_t* hpair;
    uint64_t* ppair;
    uint32_t seq;
};

// The arguments and shape of layer L's FFN launch. prm: a launch captured into a decode graph
// (fixed shape; seq, x and y from prm). Outside a graph, and without xch, this takes the
// layer's next launch sequence number.
np_status ffn_args(np_layer* L, const float* x, float* y, const DecodeParams* prm, int layer, bool read_through,
                   bool y_holds_base, const Exchange* xch, FfnArgs* out, FfnShape* out_sh) {
    FfnShape sh{};
    if (!ffn_shape(L, L->n_active, &sh, prm != nullptr))
        return fail(NP_EINVAL, "no FFN launch shape for d_model=%d n=%d tile=%d", L->desc.d_model,
                    L->n_active, L->tw);
    FfnArgs a{};
    a.buf = L->buf;
    a.act = L->act();
    a.act_src = L->act_src();
    a.store = L->store_dev;
    a.read_through = read_through ? 1 : 0;
    a.store_bytes = read_through ? (uint32_t)((size_t)L->desc.d_ff * L->bundle_elems() * 2) : 0u;
    a.counts = L->counts;
    a.x = x;
    a.y = y;
    a.hpair = xch ? xch->hpair : L->hpair;
    a.ppair = xch ? xch->ppair : L->ppair;
    a.prm = prm;
    a.layer = layer;
    if (prm) {
        a.seq = 0;
        a.n = -1;
    } else if (xch) {
        a.seq = xch->seq;
        a.n = L->n_active;
    } else {
        if (++L->ffn_seq == 0) L->ffn_seq = 1;  // 0 marks never-written words
        a.seq = L->ffn_seq;
        a.n = L->n_active;
    }
    a.buf_bytes = (uint32_t)((size_t)L->desc.k_max * L->bundle_elems() * 2);
    a.slot_stride = (uint32_t)L->ldh.stride16 * 16u;
    a.row_plane = (uint32_t)((size_t)L->ldh.plane16 * 16u);
    a.d = L->desc.d_model;
    a.K = L->desc.k_max;
    a.R = L->desc.n_rows;
    a.M = L->desc.d_ff;
    a.activation = L->desc.act;
    a.atomic_y = !xch && L->reduce == NP_REDUCE_ATOMIC ? 1 : 0;
    a.accumulate = y_holds_base ? 1 : 0;
    a.p1 = sh.p1;
    a.q = sh.q;
    a.tw = sh.tw;
    a.nwg = sh.nwg;
    *out = a;
    *out_sh = sh;
    return NP_OK;
}

// pf (optional): a layer with a host-memory row store whose last assignment is not scattered
// yet; the launch also scatters its new bundles (prefetch workgroups), pf_fixed (a captured
// launch) with a grid that does not depend on the host's count of them.
np_status enqueue_ffn(np_layer* L, const float* x, float* y, hipStream_t s, const DecodeParams* prm = nullptr,
                      int layer = 0, bool read_through = false, bool y_holds_base = false,
                      const Exchange* xch = nullptr, const np_layer* pf = nullptr, bool pf_fixed = false) {
    FfnArgs a{};
    FfnShape sh{};
    const np_status st = ffn_args(L, x, y, prm, layer, read_through, y_holds_base, xch, &a, &sh);
    if (st != NP_OK) return st;
    if (a.atomic_y && !y_holds_base)  // the atomic reduction adds into y: start from zero
        NP_HIP(hipMemsetAsync(y, 0, (size_t)L->desc.d_model * sizeof(float), s));
    if (pf) {
        a.pf = pf->ldev;
        a.pf_wgs = prefetch_wgs(pf_fixed || pf->n_in < 0 ? pf->desc.k_max : pf->n_in);
    }
    NP_HIP(launch_sparse_ffn(a, sh, L->desc.n_rows == 3, s));
    return NP_OK;
}

// ---- token launches: every layer of a decode token whose row store is pinned host memory in
// one grid per group of up to kTokenLayers layers (TokenArgs): kTokenPfWgs workgroups stream
// the layers' deltas over the host link without a break between layers, and each layer's FFN
// runs on the other compute units as soon as its delta is in place. Per-layer launches instead
// drain and refill the host link at every launch boundary (about 7 us per layer).
// kTokenPfWgs: 24 (three per XCD); on the Llama-2-7B-shaped decode 24 gave 2.81 ms per token,
// 32 2.86, 48 2.89 and 64 2.91 (the FFN keeps more units with fewer).
constexpr int kTokenPfWgs = 24;

bool staged(const np_layer* L);

// The token path applies to layers that all have pinned host row stores (not staged), equal
// row counts and the same FFN workgroup size and x chunks per lane.
bool token_eligible(np_layer* const* layers, int n, bool fixed) {
    FfnShape s0{};
    for (int l = 0; l < n; ++l) {
        const np_layer* L = layers[l];
        if (!L->store_is_host || staged(L) || L->desc.n_rows != layers[0]->desc.n_rows) return false;
        FfnShape sh{};
        if (!ffn_shape(L, L->n_active, &sh, fixed)) return false;
        if (l == 0) s0 = sh;
        else if (sh.nt != s0.nt || sh.jx != s0.jx) return false;
    }
    return true;
}

// Fills T for layers [0, n) (decode-step indices layer0 ..), returns the grid and the shape.
np_status token_args(np_layer* const* layers, int n, const float* x, float* y, const DecodeParams* prm,
                     int layer0, bool y_holds_base, TokenArgs* T, int* grid, FfnShape* sh) {
    const int d = layers[0]->desc.d_model;
    T->n_layers = n;
    T->n_pf = kTokenPfWgs;
    int tot = 0, fixed = 1;
    for (int l = 0; l < n; ++l) {
        const int gl = layer0 + l;
        const np_status st = ffn_args(layers[l], prm ? nullptr : x + (size_t)gl * d, prm ? nullptr : y + (size_t)gl * d,
                                      prm, gl, false, y_holds_base, nullptr, &T->ffn[l], sh);
        if (st != NP_OK) return st;
        T->wg0[l] = tot;
        tot += sh->nwg;
        fixed &= sh->fixed;  // the compiled lane geometry only when every layer of the launch has it
        T->src[l] = layers[l]->ldev;
    }
    sh->fixed = fixed;
    T->wg0[n] = tot;
    *grid = kTokenPfWgs + tot;
    return NP_OK;
}

size_t token_bytes(int n) { return offsetof(TokenArgs, ffn) + (size_t)n * sizeof(FfnArgs); }

// The argument staging of direct token launches led by `lead`, allocated on first use.
np_status token_stage(np_layer* lead) {
    if (lead->tstage) return NP_OK;
    auto ts = std::make_unique<TokenStage>();
    if (hipMalloc(&ts->dev, sizeof(TokenArgs)) != hipSuccess) {
        (void)hipGetLastError();
        return fail(NP_ENOMEM, "cannot allocate the token launch arguments");
    }
    for (int i = 0; i < TokenStage::kRing; ++i) {
        if (hipHostMalloc((void**)&ts->host[i], sizeof(TokenArgs), 0) != hipSuccess) {
            (void)hipGetLastError();
            return fail(NP_ENOMEM, "cannot allocate pinned token launch arguments");
        }
        NP_HIP(hipEventCreateWithFlags(&ts->copied[i], hipEventDisableTiming));
    }
    lead->tstage = std::move(ts);
    return NP_OK;
}

np_status enqueue_token_launch(np_layer* const* layers, int n, const float* x, float* y, hipStream_t s,
                               int layer0, bool y_holds_base) {
    np_layer* lead = layers[0];
    const np_status as = token_stage(lead);
    if (as != NP_OK) return as;
    TokenStage& ts = *lead->tstage;
    const int k = ts.next;
    ts.next = (k + 1) % TokenStage::kRing;
    NP_HIP(hipEventSynchronize(ts.copied[k]));  // its previous copy (a few tokens back) is done
    TokenArgs* T = ts.host[k];
    int grid = 0;
    FfnShape sh{};
    np_status st = token_args(layers, n, x, y, nullptr, layer0, y_holds_base, T, &grid, &sh);
    if (st != NP_OK) return st;
    NP_HIP(hipMemcpyAsync(ts.dev, T, token_bytes(n), hipMemcpyHostToDevice, s));
    NP_HIP(hipEventRecord(ts.copied[k], s));
    NP_HIP(launch_token(ts.dev, grid, sh, lead->desc.n_rows == 3, s));
    return NP_OK;
}

np_status enqueue_scatter(np_layer* L, hipStream_t s, bool fixed_grid = false) {
    if (L->store_is_host) {  // a few workgroups hold the host link at its ceiling
        NP_HIP(launch_scatter_flat(L->ldev, prefetch_wgs(fixed_grid || L->n_in < 0 ? L->desc.k_max : L->n_in), s));
        return NP_OK;
    }
    const int grid = fixed_grid || L->n_in < 0 ? std::max(1, std::min(L->desc.k_max, 1024)) : scatter_grid(L->n_in);
    NP_HIP(launch_scatter(L->counts, L->d_in(), L->slot_in(), L->store_dev, L->buf, L->desc.d_ff,
                          L->desc.k_max, (int32_t)L->bundle_elems(), L->ldh.row16, L->ldh.stride16, L->ldh.plane16,
                          grid, s));
    return NP_OK;
}

// The FFN reads a device row store through a buffer descriptor with 32-bit offsets, so it reads
// new bundles straight from the store (read-through) only when the store is below 4 GiB; a larger
// one is scattered into the slots first.
bool read_through_ok(const np_layer* L) {
    return !L->store_is_host && (uint64_t)L->desc.d_ff * L->bundle_elems() * 2 <= kMaxBufBytes;
}

// The FFN of a layer in a decode step: device row stores go through read-through, or, above
// 4 GiB, an explicit scatter first.
np_status enqueue_step_ffn(np_layer* L, const float* x, float* y, hipStream_t s, const DecodeParams* prm, int layer,
                           bool y_holds_base, const np_layer* pf = nullptr, bool pf_fixed = false) {
    if (!L->store_is_host && !read_through_ok(L)) {
        const np_status r = enqueue_scatter(L, s, prm != nullptr);
        if (r != NP_OK) return r;
    }
    return enqueue_ffn(L, x, y, s, prm, layer, read_through_ok(L), y_holds_base, nullptr, pf, pf_fixed);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Error bits that a kernel of the layer raised since its last reset (read without synchronizing:
// a kernel still running may add some later). Calls that enqueue work for the layer refuse it
// with NP_EDEVICE while any are set.
// x and y must be memory the layer's device can read and write: its own device memory or pinned
// host memory mapped for it. A pageable host pointer (or another device's memory) would fault the
// GPU instead of failing here.
np_status check_io_ptr(const void* p, int dev, const char* what) {
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof attr);
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return fail(NP_EINVAL, "%s is neither device memory nor pinned host memory", what);
    }
    if (attr.type == hipMemoryTypeDevice) {
        if (attr.device != dev) return fail(NP_EINVAL, "%s lives on device %d, the layer on device %d", what, attr.device, dev);
        return NP_OK;
    }
    if (attr.type == hipMemoryTypeHost && attr.devicePointer) return NP_OK;
    return fail(NP_EINVAL, "%s (memory type %d) is not device memory or mapped pinned host memory", what, (int)attr.type);
}

np_status check_device_err(const np_layer* L, int index = -1) {
    const uint32_t bits = L->err_h ? __atomic_load_n(L->err_h, __ATOMIC_ACQUIRE) : 0u;
    if (!bits) return NP_OK;
    if (index >= 0)
        return fail(NP_EDEVICE, "layer %d: a kernel reported error bits 0x%x (np_layer_read_state shows them all; "
                    "np_layer_reset clears them)", index, bits);
    return fail(NP_EDEVICE, "a kernel reported error bits 0x%x (np_layer_read_state shows them all; np_layer_reset "
                "clears them)", bits);
}

// ---- staged delta I/O (NeuroPrefetcher section 3.5: the host reads the incoming rows, sorted
// and with adjacent ones merged, into a bounded pinned staging buffer, the DMA engine copies it
// to the device and a kernel places every bundle in its slot; a delta larger than the staging
// is sent in chunks). The alternative, and the default, is the zero-copy pull by the scatter
// kernel. Used by np_decode_step for host-memory row stores of layers whose delta the host
// knows (no window, no frequency levels).

// A fixed set of worker threads that run parts 1..n-1 of a job while the caller runs part 0.
class GatherPool {
public:
    explicit GatherPool(int n) : n_(std::max(1, n)) {
        for (int i = 1; i < n_; ++i) th_.emplace_back([this, i] { loop(i); });
    }
    ~GatherPool() {
        {
            std::lock_guard<std::mutex> lk(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& t : th_) t.join();
    }
    int size() const { return n_; }
    void run(const std::function<void(int)>& f) {
        {
            std::lock_guard<std::mutex> lk(mu_);
            job_ = &f;
            pending_ = n_ - 1;
            ++gen_;
        }
        cv_.notify_all();
        f(0);
        std::unique_lock<std::mutex> lk(mu_);
        done_.wait(lk, [this] { return pending_ == 0; });
        job_ = nullptr;
    }

private:
    void loop(int i) {
        uint64_t seen = 0;
        for (;;) {
            const std::function<void(int)>* f;
            {
                std::unique_lock<std::mutex> lk(mu_);
                cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
                if (stop_) return;
                seen = gen_;
                f = job_;
            }
            (*f)(i);
            std::lock_guard<std::mutex> lk(mu_);
            if (--pending_ == 0) done_.notify_one();
        }
    }
    int n_;
    std::vector<std::thread> th_;
    std::mutex mu_;
    std::condition_variable cv_, done_;
    const std::function<void(int)>* job_ = nullptr;
    int pending_ = 0;
    uint64_t gen_ = 0;
    bool stop_ = false;
};

struct Stager {
    int dev = -1;
    size_t cap = 0;                 // bytes per half
    void* host[2] = {nullptr, nullptr};  // pinned staging (hipHostMalloc)
    void* devb[2] = {nullptr, nullptr};  // device staging
    hipEvent_t ready[2] = {nullptr, nullptr};  // the last copy out of host[h] (and its scatter) done
    int next = 0;
    std::unique_ptr<GatherPool> pool;
    ~Stager() {
        for (int h = 0; h < 2; ++h) {
            if (ready[h]) (void)hipEventSynchronize(ready[h]);
            if (ready[h]) (void)hipEventDestroy(ready[h]);
            if (host[h]) (void)hipHostFree(host[h]);
            if (devb[h]) (void)hipFree(devb[h]);
        }
    }
};

std::mutex g_stage_mu;                 // guards the settings and the stagers
size_t g_stage_bytes = 0;              // 0: zero-copy pull (default)
int g_stage_threads = 0;
// Never destroyed: at process exit the HIP runtime may already be gone, and the pool threads
// are then simply ended with the process.
std::map<int, std::unique_ptr<Stager>>& g_stagers = *new std::map<int, std::unique_ptr<Stager>>();

bool staged(const np_layer* L) { return g_stage_bytes > 0 && L->store_is_host && !device_decides(L); }

np_status get_stager(int dev, Stager** out) {
    auto& sp = g_stagers[dev];
    if (!sp) {
        auto st = std::make_unique<Stager>();
        st->dev = dev;
        st->cap = g_stage_bytes;
        for (int h = 0; h < 2; ++h) {
            if (hipHostMalloc(&st->host[h], st->cap, hipHostMallocDefault) != hipSuccess ||
                hipMalloc(&st->devb[h], st->cap) != hipSuccess ||
                hipEventCreateWithFlags(&st->ready[h], hipEventDisableTiming) != hipSuccess) {
                (void)hipGetLastError();
                return fail(NP_ENOMEM, "cannot allocate two %zu-byte staging buffers", st->cap);
            }
            NP_HIP(hipEventRecord(st->ready[h], nullptr));
        }
        st->pool = std::make_unique<GatherPool>(g_stage_threads);
        sp = std::move(st);
    }
    *out = sp.get();
    return NP_OK;
}

// Layer L's incoming bundles (d_in ascending, as the assignment lists them) through the staging
// buffers in chunks; everything on stream s, which must already follow L's assignment.
np_status enqueue_staged(np_layer* L, const std::vector<int32_t>& d_in, hipStream_t s, Stager* st) {
    const size_t bb = L->bundle_elems() * 2;
    const int per = (int)std::min<size_t>(st->cap / bb, (size_t)L->desc.k_max);
    if (per < 1) return fail(NP_EINVAL, "staging of %zu bytes holds no %zu-byte bundle", st->cap, bb);
    const char* store = static_cast<const char*>(L->desc.row_store);
    const int n = (int)d_in.size();
    std::vector<std::pair<int, int>> runs;  // (first index in the chunk, length) of adjacent IDs
    for (int first = 0; first < n; first += per) {
        const int cnt = std::min(per, n - first);
        const int h = st->next;
        st->next ^= 1;
        NP_HIP(hipEventSynchronize(st->ready[h]));  // the copy that last read host[h] is done
        runs.clear();
        for (int i = 0; i < cnt; ++i) {
            if (!runs.empty() && d_in[first + i] == d_in[first + i - 1] + 1) ++runs.back().second;
            else runs.emplace_back(i, 1);
        }
        char* dst = static_cast<char*>(st->host[h]);
        const int parts = st->pool->size();
        const std::function<void(int)> job = [&](int part) {
            // runs split over the parts by bundle count
            const int lo = (int)((int64_t)cnt * part / parts), hi = (int)((int64_t)cnt * (part + 1) / parts);
            for (const auto& r : runs) {
                const int a = std::max(lo, r.first), b = std::min(hi, r.first + r.second);
                if (a >= b) continue;
                const int32_t nid = d_in[first + r.first] + (a - r.first);
                std::memcpy(dst + (size_t)a * bb, store + (size_t)nid * bb, (size_t)(b - a) * bb);
            }
        };
        st->pool->run(job);
        NP_HIP(hipMemcpyAsync(st->devb[h], st->host[h], (size_t)cnt * bb, hipMemcpyHostToDevice, s));
        NP_HIP(launch_scatter_staged(L->counts, L->slot_in() + first, st->devb[h], L->buf, cnt, L->desc.k_max,
                                     (int32_t)L->bundle_elems(), L->ldh.row16, L->ldh.stride16, L->ldh.plane16, s));
        NP_HIP(hipEventRecord(st->ready[h], s));
    }
    return NP_OK;
}

// Staged delta I/O: the staged layers' copies and scatters go to the copy stream, and layer l's
// FFN waits only for layer l's, unless the two streams are the same (or no row store is in
// host memory): then everything goes to one queue.
bool one_queue(np_layer* const* layers, int n, hipStream_t cs, hipStream_t ps) {
    if (cs == ps) return true;
    for (int l = 0; l < n; ++l)
        if (layers[l]->store_is_host) return false;
    return true;
}

constexpr int kScatterWgsPerLayer = 64;

// One token's launches. cid: host [n][2] (gate, effective up) ids; with prm (capture into a
// decode graph) the ids, x and y come from the parameter block instead. ev: n + 2 events, used
// only on the two-stream path of staged delta I/O.
np_status enqueue_token(np_layer* const* layers, int n, const int32_t* cid, const float* x, float* y,
                        hipStream_t cs, hipStream_t ps, const DecodeParams* prm, const hipEvent_t* ev,
                        const std::vector<std::vector<int32_t>>* din = nullptr, Stager* st = nullptr,
                        const std::vector<TokenLaunch>* tok = nullptr) {
    const int d = layers[0]->desc.d_model;
    // the assign launch clears every layer's y, so the FFN launches add into zeros
    bool any_atomic = false;
    for (int l = 0; l < n; ++l) any_atomic |= layers[l]->reduce == NP_REDUCE_ATOMIC;
    for (int l0 = 0; l0 < n; l0 += kMaxLayersPerLaunch) {
        DeltaLaunch a{};
        a.n_layers = std::min(kMaxLayersPerLaunch, n - l0);
        for (int k = 0; k < a.n_layers; ++k) {
            a.layers[k] = layers[l0 + k]->ldev;
            a.cid[k][0] = cid ? cid[2 * (l0 + k)] : 0;
            a.cid[k][1] = cid ? cid[2 * (l0 + k) + 1] : 0;
        }
        a.prm = prm;
        a.layer0 = l0;
        a.zero_y = any_atomic ? 1 : 0;
        a.y = prm ? nullptr : y;
        a.d = d;
        NP_HIP(launch_delta_assign(a, cs));
    }
    // compacted layouts: the rows moved by the assignment, before anything writes new rows
    {
        ScatterLaunch ma{};
        for (int l = 0; l < n; ++l) {
            if (layers[l]->layout != NP_LAYOUT_COMPACT) continue;
            ma.layers[ma.n_layers++] = layers[l]->ldev;
            if (ma.n_layers == kMaxLayersPerLaunch) {
                NP_HIP(launch_move_all(ma, kScatterWgsPerLayer, cs));
                ma.n_layers = 0;
            }
        }
        if (ma.n_layers > 0) NP_HIP(launch_move_all(ma, kScatterWgsPerLayer, cs));
    }
    bool uses_stager = false;
    for (int l = 0; l < n && din && st; ++l) uses_stager |= staged(layers[l]);
    if (!uses_stager && token_eligible(layers, n, prm != nullptr)) {
        // Every row store in pinned host memory: one token launch per group of layers.
        if (prm) {
            if (!tok || tok->empty()) return fail(NP_EHIP, "decode graph: token launch arguments missing");
            for (const TokenLaunch& t : *tok) NP_HIP(launch_token(t.dev, t.grid, t.sh, t.gated, cs));
            return NP_OK;
        }
        for (int g0 = 0; g0 < n; g0 += kTokenLayers) {
            const np_status r = enqueue_token_launch(layers + g0, std::min(kTokenLayers, n - g0), x, y, cs, g0,
                                                     any_atomic);
            if (r != NP_OK) return r;
        }
        return NP_OK;
    }
    if (!uses_stager) {
        // Everything on compute_stream, one launch per layer. Device-memory row stores: each
        // FFN reads its new bundles from the store and writes them into their slots
        // (read-through). Host-memory row stores: layer 0's scatter runs alone, and the scatter
        // of layer l + 1 runs in layer l's FFN launch (prefetch workgroups), so the host link
        // carries the next layer's delta while this layer's FFN reads its resident rows.
        if (layers[0]->store_is_host) {
            const np_status r = enqueue_scatter(layers[0], cs, prm != nullptr);
            if (r != NP_OK) return r;
        }
        for (int l = 0; l < n; ++l) {
            const np_layer* pf = l + 1 < n && layers[l + 1]->store_is_host ? layers[l + 1] : nullptr;
            np_status r = enqueue_step_ffn(layers[l], prm ? nullptr : x + (size_t)l * d,
                                           prm ? nullptr : y + (size_t)l * d, cs, prm, l, any_atomic, pf,
                                           prm != nullptr);
            if (r != NP_OK) return r;
        }
        return NP_OK;
    }
    // Staged delta I/O for some layer: the host's gathers and DMA copies of layer l overlap
    // the device's work on earlier layers.
    if (one_queue(layers, n, cs, ps)) {
        // Device-memory row stores: each FFN reads its new bundles from the store and writes
        // them into their slots (read-through). Host-memory stores: one scatter launch first.
        ScatterLaunch sa{};
        for (int l = 0; l < n; ++l) {
            if (!layers[l]->store_is_host) continue;
            if (din && st && staged(layers[l])) {
                np_status r = enqueue_staged(layers[l], (*din)[l], cs, st);
                if (r != NP_OK) return r;
                continue;
            }
            sa.layers[sa.n_layers++] = layers[l]->ldev;
            if (sa.n_layers == kMaxLayersPerLaunch) {
                NP_HIP(launch_scatter_all(sa, kScatterWgsPerLayer, cs));
                sa.n_layers = 0;
            }
        }
        if (sa.n_layers > 0) NP_HIP(launch_scatter_all(sa, kScatterWgsPerLayer, cs));
        for (int l = 0; l < n; ++l) {
            np_status r = enqueue_step_ffn(layers[l], prm ? nullptr : x + (size_t)l * d,
                                           prm ? nullptr : y + (size_t)l * d, cs, prm, l, any_atomic);
            if (r != NP_OK) return r;
        }
        return NP_OK;
    }
    NP_HIP(hipEventRecord(ev[0], cs));
    NP_HIP(hipStreamWaitEvent(ps, ev[0], 0));
    for (int l = 0; l < n; ++l) {
        np_status r = din && st && staged(layers[l]) ? enqueue_staged(layers[l], (*din)[l], ps, st)
                                                     : enqueue_scatter(layers[l], ps, prm != nullptr);
        if (r != NP_OK) return r;
        NP_HIP(hipEventRecord(ev[2 + l], ps));
        NP_HIP(hipStreamWaitEvent(cs, ev[2 + l], 0));
        r = enqueue_ffn(layers[l], prm ? nullptr : x + (size_t)l * d, prm ? nullptr : y + (size_t)l * d, cs, prm, l,
                        false, any_atomic);
        if (r != NP_OK) return r;
    }
    NP_HIP(hipEventRecord(ev[1], ps));  // join the copy stream back to the compute stream
    NP_HIP(hipStreamWaitEvent(cs, ev[1], 0));
    return NP_OK;
}

// Events for the two-stream path of staged steps: per thread and device, grown on demand.
np_status step_events(int dev, int n, const hipEvent_t** out) {
    thread_local std::map<int, std::vector<hipEvent_t>> evs;
    auto& v = evs[dev];
    while ((int)v.size() < n + 2) {
        hipEvent_t e;
        NP_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
        v.push_back(e);
    }
    *out = v.data();
    return NP_OK;
}

// ---- decode graphs: one token's launches captured once per (layer set, streams), replayed
// with the per-token values written into a device parameter block just before.
struct DecodePlan {
    std::vector<np_layer*> layers;
    std::vector<uint64_t> versions;
    hipStream_t cs = nullptr, ps = nullptr;
    int device = 0;
    DecodeParams* prm = nullptr;
    hipGraphExec_t exec = nullptr;
    std::vector<TokenLaunch> tok;  // token launches of the captured step (host row stores)
    ~DecodePlan() {
        if (exec) (void)hipGraphExecDestroy(exec);
        for (TokenLaunch& t : tok)
            if (t.dev) (void)hipFree(t.dev);
        if (prm) (void)hipFree(prm);
    }
};

std::mutex g_plan_mu;
// Plans are shared: a caller keeps its plan alive from lookup until its graph launch is
// enqueued, even if another thread drops the plan from the cache meanwhile.
std::vector<std::shared_ptr<DecodePlan>> g_plans;  // most recently used last
std::atomic<int> g_use_graphs{0};
constexpr size_t kMaxPlans = 8;

void drop_plans_with(const np_layer* L) {
    std::lock_guard<std::mutex> lk(g_plan_mu);
    for (size_t i = 0; i < g_plans.size();) {
        auto& ls = g_plans[i]->layers;
        if (std::find(ls.begin(), ls.end(), L) != ls.end()) g_plans.erase(g_plans.begin() + i);
        else ++i;
    }
}

np_status capture_plan(DecodePlan* P) {
    const int n = (int)P->layers.size();
    NP_HIP(hipMalloc(&P->prm, sizeof(DecodeParams)));
    NP_HIP(hipMemset(P->prm, 0, sizeof(DecodeParams)));
    // Token launches (every row store in pinned host memory): their arguments are written once,
    // here; per-token values (sequence numbers, x, y, |S|) come from the parameter block.
    if (token_eligible(P->layers.data(), n, true)) {
        bool any_atomic = false;
        for (np_layer* L : P->layers) any_atomic |= L->reduce == NP_REDUCE_ATOMIC;
        auto T = std::make_unique<TokenArgs>();
        for (int g0 = 0; g0 < n; g0 += kTokenLayers) {
            const int gn = std::min(kTokenLayers, n - g0);
            TokenLaunch t{};
            const np_status ts = token_args(P->layers.data() + g0, gn, nullptr, nullptr, P->prm, g0, any_atomic,
                                            T.get(), &t.grid, &t.sh);
            if (ts != NP_OK) return ts;
            t.gated = P->layers[g0]->desc.n_rows == 3;
            NP_HIP(hipMalloc(&t.dev, token_bytes(gn)));
            P->tok.push_back(t);
            NP_HIP(hipMemcpy(t.dev, T.get(), token_bytes(gn), hipMemcpyHostToDevice));
        }
    }
    NP_HIP(hipStreamBeginCapture(P->cs, hipStreamCaptureModeRelaxed));
    // a captured step never stages, so it runs on compute_stream alone and needs no events
    const np_status st = enqueue_token(P->layers.data(), n, nullptr, nullptr, nullptr, P->cs, P->ps, P->prm,
                                       nullptr, nullptr, nullptr, &P->tok);
    hipGraph_t graph = nullptr;
    const hipError_t ee = hipStreamEndCapture(P->cs, &graph);
    if (st != NP_OK) {  // the failing call has set the message
        if (graph) (void)hipGraphDestroy(graph);
        return st;
    }
    if (ee != hipSuccess || !graph) {
        if (graph) (void)hipGraphDestroy(graph);
        return fail(NP_EHIP, "decode graph capture failed: %s", hipGetErrorString(ee));
    }
    const hipError_t ie = hipGraphInstantiate(&P->exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ie != hipSuccess) {
        P->exec = nullptr;
        return fail(NP_EHIP, "decode graph instantiation failed: %s", hipGetErrorString(ie));
    }
    return NP_OK;
}

// The cached plan for these layers and streams, captured on first use.
std::shared_ptr<DecodePlan> get_plan(np_layer* const* layers, int n, hipStream_t cs, hipStream_t ps, int dev,
                                     np_status* st) {
    std::lock_guard<std::mutex> lk(g_plan_mu);
    for (size_t i = 0; i < g_plans.size(); ++i) {
        DecodePlan* P = g_plans[i].get();
        if ((int)P->layers.size() != n || P->cs != cs || P->ps != ps) continue;
        bool same = true;
        for (int l = 0; l < n && same; ++l) same = P->layers[l] == layers[l] && P->versions[l] == layers[l]->version;
        if (!same) continue;
        auto keep = std::move(g_plans[i]);
        g_plans.erase(g_plans.begin() + i);
        g_plans.push_back(keep);
        return keep;
    }
    auto P = std::make_shared<DecodePlan>();
    P->layers.assign(layers, layers + n);
    for (int l = 0; l < n; ++l) P->versions.push_back(layers[l]->version);
    P->cs = cs;
    P->ps = ps;
    P->device = dev;
    *st = capture_plan(P.get());
    if (*st != NP_OK) return nullptr;
    if (g_plans.size() >= kMaxPlans) g_plans.erase(g_plans.begin());
    g_plans.push_back(P);
    return P;
}

}  // namespace

extern "C" {

const char* np_last_error(void) { return g_err.c_str(); }

np_status np_layer_create(const np_layer_desc* desc, np_layer** out) {
    if (!desc || !out) return fail(NP_EINVAL, "desc and out must not be NULL");
    *out = nullptr;
    const np_layer_desc& D = *desc;
    if (D.d_model < 8 || D.d_model > kMaxDModel || D.d_model % 8)
        return fail(NP_EINVAL, "d_model=%d must be a multiple of 8 in [8, %d]", D.d_model, kMaxDModel);
    if (D.d_ff < 1 || D.d_ff > kMaxDff) return fail(NP_EINVAL, "d_ff=%d must be in [1, %d]", D.d_ff, kMaxDff);
    if (D.k_max < 1 || D.k_max > std::min(D.d_ff, kMaxKmax))
        return fail(NP_EINVAL, "k_max=%d must be in [1, min(d_ff, %d)]", D.k_max, kMaxKmax);
    if (D.n_rows != 2 && D.n_rows != 3) return fail(NP_EINVAL, "n_rows=%d must be 2 or 3", D.n_rows);
    if (D.n_centroids < 1 || D.n_centroids > kMaxCentroids)
        return fail(NP_EINVAL, "n_centroids=%d must be in [1, %d]", D.n_centroids, kMaxCentroids);
    if (D.mask_mode < NP_MASK_UNION || D.mask_mode > NP_MASK_SINGLE)
        return fail(NP_EINVAL, "unknown mask_mode %d", D.mask_mode);
    if (D.act != NP_ACT_RELU && D.act != NP_ACT_SILU) return fail(NP_EINVAL, "unsupported activation %d", D.act);
    if (!D.masks || !D.row_store) return fail(NP_EINVAL, "masks and row_store must not be NULL");
    if ((uint64_t)D.k_max * D.n_rows * D.d_model * 2 > kMaxBufBytes)
        return fail(NP_EINVAL, "slot buffer k_max * n_rows * d_model * 2 bytes must stay below 4 GiB");
    if (!aligned16(D.row_store)) return fail(NP_EINVAL, "row_store must be 16-byte aligned");
    int ndev = 0;
    NP_HIP(hipGetDeviceCount(&ndev));
    if (D.device < 0 || D.device >= ndev) return fail(NP_EINVAL, "device %d out of range [0, %d)", D.device, ndev);

    np_layer* L = new np_layer();
    L->desc = D;
    L->desc.masks = nullptr;
    L->W = (D.d_ff + 63) / 64;
    L->Kw = (D.k_max + 63) / 64;
    L->n_tables = D.mask_mode == NP_MASK_SINGLE ? 1 : 2;
    const size_t mask_words = (size_t)L->n_tables * D.n_centroids * L->W;
    L->h_masks.assign(D.masks, D.masks + mask_words);
    L->h_res.assign(L->W, 0ull);
    if (D.d_ff & 63) {
        const uint64_t stray = ~((1ull << (D.d_ff & 63)) - 1);
        for (size_t m = 0; m < (size_t)L->n_tables * D.n_centroids; ++m)
            if (L->h_masks[m * L->W + L->W - 1] & stray) {
                delete L;
                return fail(NP_EINVAL, "mask %zu has bits at or above d_ff=%d", m, D.d_ff);
            }
    }

    DeviceGuard g(D.device);
    if (!g.ok) {
        delete L;
        return fail(NP_EHIP, "hipSetDevice(%d) failed", D.device);
    }
    setup_scratch(D.device);
    // Classify the row store: device memory of this device, or pinned host memory.
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof attr);
    hipError_t pe = hipPointerGetAttributes(&attr, D.row_store);
    if (pe != hipSuccess) {
        (void)hipGetLastError();
        delete L;
        return fail(NP_EINVAL, "row_store is neither device memory nor pinned host memory");
    }
    if (attr.type == hipMemoryTypeDevice) {
        if (attr.device != D.device) {
            delete L;
            return fail(NP_EINVAL, "row_store lives on device %d, layer on device %d", attr.device, D.device);
        }
        L->store_dev = static_cast<const uint16_t*>(D.row_store);
    } else if (attr.type == hipMemoryTypeHost) {
        void* dp = nullptr;
        if (hipHostGetDevicePointer(&dp, const_cast<void*>(D.row_store), 0) != hipSuccess || !dp) {
            (void)hipGetLastError();
            delete L;
            return fail(NP_EINVAL, "pinned row_store is not mapped for device access");
        }
        L->store_dev = static_cast<const uint16_t*>(dp);
        L->store_is_host = true;
    } else {
        delete L;
        return fail(NP_EINVAL, "row_store memory type %d is not supported", (int)attr.type);
    }

    const int K = D.k_max, M = D.d_ff;
    {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, D.device) == hipSuccess && cus > 0)
            L->cus = cus;
        else
            (void)hipGetLastError();
    }
    auto dmalloc = [&](void** p, size_t bytes) -> bool {
        if (hipMalloc(p, bytes) != hipSuccess) {
            (void)hipGetLastError();
            return false;
        }
        return true;
    };
    const size_t buf_bytes = (size_t)K * L->bundle_elems() * 2;
    bool ok = dmalloc((void**)&L->d_masks, mask_words * 8) && dmalloc((void**)&L->buf, buf_bytes) &&
              dmalloc((void**)&L->slot_map, (size_t)M * 4) && dmalloc((void**)&L->owner, (size_t)K * 4) &&
              dmalloc((void**)&L->res, (size_t)L->W * 8) && dmalloc((void**)&L->freeb, (size_t)L->Kw * 8) &&
              dmalloc((void**)&L->lists, (size_t)kLists * K * 4) && dmalloc((void**)&L->counts, kCountsAlloc) &&
              dmalloc((void**)&L->hpair, (size_t)K * 8) &&
              dmalloc((void**)&L->ldev, sizeof(LayerDev));
    if (!ok) {
        free_layer(L);
        return fail(NP_ENOMEM, "device allocation failed (slot buffer %zu bytes)", buf_bytes);
    }
    np_status st = alloc_ffn_scratch(L);
    if (st != NP_OK) {
        free_layer(L);
        return st;
    }
    {
        // the host error word: pinned, coherent, mapped; its device address follows the counts
        void* dp = nullptr;
        if (hipHostMalloc((void**)&L->err_h, sizeof(uint32_t),
                          hipHostMallocMapped | hipHostMallocCoherent | hipHostMallocPortable) != hipSuccess ||
            hipHostGetDevicePointer(&dp, L->err_h, 0) != hipSuccess || !dp) {
            (void)hipGetLastError();
            free_layer(L);
            return fail(NP_ENOMEM, "cannot allocate the pinned error word");
        }
        *L->err_h = 0;
        if (hipMemcpy(L->counts + kErrMirrorSlot, &dp, sizeof dp, hipMemcpyHostToDevice) != hipSuccess) {
            (void)hipGetLastError();
            free_layer(L);
            return fail(NP_EHIP, "cannot record the error word's address");
        }
    }
    LayerDev ld{};
    ld.masks = L->d_masks;
    ld.res = L->res;
    ld.freeb = L->freeb;
    ld.slot_map = L->slot_map;
    ld.owner = L->owner;
    ld.d_in = L->d_in();
    ld.slot_in = L->slot_in();
    ld.d_out = L->d_out();
    ld.act = L->act();
    ld.act_src = L->act_src();
    ld.counts = L->counts;
    ld.acc = reinterpret_cast<unsigned long long*>(L->counts + 8);
    ld.ring = nullptr;
    ld.window = 1;
    ld.levels = nullptr;
    ld.n_levels = 0;
    ld.compact = 0;
    ld.mv_src = L->mv_src();
    ld.mv_dst = L->mv_dst();
    ld.W = L->W;
    ld.Kw = L->Kw;
    ld.M = M;
    ld.K = K;
    ld.mode = D.mask_mode;
    ld.n_tables = L->n_tables;
    ld.C = D.n_centroids;
    ld.pad = 0;
    ld.store = L->store_dev;
    ld.buf = L->buf;
    ld.bundle16 = (int32_t)(L->bundle_elems() / 8);
    ld.row16 = D.d_model / 8;
    ld.stride16 = ld.bundle16;  // interleaved until np_layer_set_planar
    ld.plane16 = ld.row16;
    L->ldh = ld;
    hipError_t e = hipMemcpy(L->ldev, &ld, sizeof ld, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(L->d_masks, L->h_masks.data(), mask_words * 8, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemset(L->hpair, 0, (size_t)K * 8);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&L->ev_scatter, hipEventDisableTiming);
    if (e != hipSuccess) {
        free_layer(L);
        return fail(NP_EHIP, "layer setup failed: %s", hipGetErrorString(e));
    }
    st = init_state(L);
    if (st != NP_OK) {
        free_layer(L);
        return st;
    }
    *out = L;
    return NP_OK;
}

np_status np_layer_destroy(np_layer* L) {
    if (!L) return fail(NP_EINVAL, "layer must not be NULL");
    DeviceGuard g(L->desc.device);
    (void)hipDeviceSynchronize();
    drop_plans_with(L);
    free_layer(L);
    return NP_OK;
}

np_status np_layer_reset(np_layer* L) {
    if (!L) return fail(NP_EINVAL, "layer must not be NULL");
    DeviceGuard g(L->desc.device);
    NP_HIP(hipDeviceSynchronize());
    ++L->version;
    return init_state(L);
}

np_status np_layer_set_ffn_shape(np_layer* L, int32_t slots_per_wg, int32_t tile_cols, int32_t threads) {
    if (!L) return fail(NP_EINVAL, "layer must not be NULL");
    if (slots_per_wg && slots_per_wg != -1 && (slots_per_wg < 1 || slots_per_wg > 16))
        return fail(NP_EINVAL, "slots_per_wg=%d must be -1 or in [1, 16]", slots_per_wg);
    if (tile_cols) {
        const int ct = tile_cols / 8;
        if (tile_cols % 8 || tile_cols < 64 || tile_cols > 1024 || (ct & (ct - 1)))
            return fail(NP_EINVAL, "tile_cols=%d must be 8 * (power of two), 64..1024", tile_cols);
    }
    if (threads && threads != 256 && threads != 512 && threads != 1024)
        return fail(NP_EINVAL, "threads=%d must be 256, 512 or 1024", threads);
    DeviceGuard g(L->desc.device);
    NP_HIP(hipDeviceSynchronize());
    const int old_spw = L->spw, old_tw = L->tw, old_nt = L->nt;
    if (slots_per_wg) L->spw = slots_per_wg < 0 ? 0 : slots_per_wg;
    if (tile_cols) L->tw = tile_cols;
    if (threads) L->nt = threads;
    FfnShape sh{};
    if (!ffn_shape(L, L->desc.k_max, &sh)) {
        L->spw = old_spw;
        L->tw = old_tw;
        L->nt = old_nt;
        return fail(NP_EINVAL, "shape (%d, %d, %d) cannot cover k_max=%d", slots_per_wg, tile_cols, threads,
                    L->desc.k_max);
    }
    np_status st = alloc_ffn_scratch(L);
    if (st != NP_OK) {
        L->spw = old_spw;
        L->tw = old_tw;
        L->nt = old_nt;
    }
    ++L->version;
    return st;
}

np_status np_delta_assign(np_layer* L, int32_t gate_cid, int32_t up_cid, void* stream) {
    if (!L) return fail(NP_EINVAL, "layer must not be NULL");
    const np_status de = check_device_err(L);
    if (de != NP_OK) return de;
    if (L->state == kAssigned)
        return fail(NP_ESTATE, "previous delta not scattered: call np_scatter_rows first");
    int32_t u;
    np_status st = check_cids(L, gate_cid, up_cid, &u);
    if (st != NP_OK) return st;
    std::vector<uint64_t> S(L->W);
    const int n = combine_host(L, gate_cid, u, S.data());
    if (n > L->desc.k_max)
        return fail(NP_ECAPACITY, "|S| = %d exceeds k_max = %d", n, L->desc.k_max);
    int n_in = -1;  // with a retention rule the resident set is decided on the device
    if (!device_decides(L)) {
        n_in = 0;
        for (int w = 0; w < L->W; ++w) n_in += __builtin_popcountll(S[w] & ~L->h_res[w]);
    }
    DeviceGuard g(L->desc.device);
    DeltaLaunch a{};
    a.layers[0] = L->ldev;
    a.cid[0][0] = gate_cid;
    a.cid[0][1] = u;
    a.n_layers = 1;
    NP_HIP(launch_delta_assign(a, (hipStream_t)stream));
    if (L->layout == NP_LAYOUT_COMPACT) {
        ScatterLaunch ma{};
        ma.layers[0] = L->ldev;
        ma.n_layers = 1;
        NP_HIP(launch_move_all(ma, kScatterWgsPerLayer, (hipStream_t)stream));
    }
    L->h_res.swap(S);
    L->n_active = n;
    L->n_in = n_in;
    L->total_active += n;
    L->total_in += std::max(n_in, 0);
    L->state = kAssigned;
    return NP_OK;
}

np_status np_scatter_rows(np_layer* L, void* stream) {
    if (!L) return fail(NP_EINVAL, "layer must not be NULL");
    if (L->state != kAssigned) return fail(NP_ESTATE, "np_scatter_rows needs a preceding np_delta_assign");
    const np_status de = check_device_err(L);
    if (de != NP_OK) return de;
    DeviceGuard g(L->desc.device);
    np_status st = enqueue_scatter(L, (hipStream_t)stream);
    if (st != NP_OK) return st;
    L->state = kScattered;
    return NP_OK;
}

namespace {
np_status sparse_ffn_call(np_layer* L, const float* x, float* y, void* stream, bool acc,
                          const Exchange* xch = nullptr) {
    if (!L) return fail(NP_EINVAL, "layer must not be NULL");
    if (!x || !y || !aligned16(x) || !aligned16(y)) return fail(NP_EINVAL, "x and y must be 16-byte aligned device pointers");
    if (L->state == kFresh) return fail(NP_ESTATE, "np_sparse_ffn needs a preceding np_delta_assign");
    for (const auto& io : {std::make_pair((const void*)x, "x"), std::make_pair((const void*)y, "y")}) {
        const np_status pe = check_io_ptr(io.first, L->desc.device, io.second);
        if (pe != NP_OK) return pe;
    }
    bool read_through = L->state == kAssigned;
    if (read_through && L->store_is_host)
        return fail(NP_ESTATE, "the row store is host memory: call np_scatter_rows before np_sparse_ffn");
    const np_status de = check_device_err(L);
    if (de != NP_OK) return de;
    DeviceGuard g(L->desc.device);
    Exchange xs{};
    if (xch) {
        // the no-allocation entry point: exchange words in the device's static scratch
        FfnShape sh{};
        if (!ffn_shape(L, L->n_active, &sh))
            return fail(NP_EINVAL, "no FFN launch shape for d_model=%d n=%d", L->desc.d_model, L->n_active);
        const size_t pwords = (size_t)sh.nwg * sh.tw;
        if ((size_t)L->desc.k_max > kScratchHWords || pwords > kScratchWords - kScratchHWords)
            return fail(NP_EINVAL, "the FFN launch needs %d h words and %zu partial-sum words; the no-allocation "
                        "scratch holds %zu and %zu (use np_sparse_ffn)", L->desc.k_max, pwords, kScratchHWords,
                        kScratchWords - kScratchHWords);
        uint64_t* base = nullptr;
        uint32_t seq = 0;
        {
            std::lock_guard<std::mutex> lk(g_scratch_mu);
            auto it = g_scratch.find(L->desc.device);
            if (it != g_scratch.end()) {
                base = it->second.ptr;
                if (++it->second.seq == 0) it->second.seq = 1;  // 0: words never written
                seq = it->second.seq;
            }
        }
        if (!base) return fail(NP_EHIP, "the static scratch of device %d has no device address", L->desc.device);
        xs = Exchange{base, base + kScratchHWords, seq};
    }
    if (read_through && !read_through_ok(L)) {  // a device row store above 4 GiB: scatter first
        FfnShape sh{};
        if (!ffn_shape(L, L->n_active, &sh))  // refused before anything is enqueued
            return fail(NP_EINVAL, "no FFN launch shape for d_model=%d n=%d", L->desc.d_model, L->n_active);
        const np_status r = enqueue_scatter(L, (hipStream_t)stream);
        if (r != NP_OK) return r;
        read_through = false;
    }
    np_status st = enqueue_ffn(L, x, y, (hipStream_t)stream, nullptr, 0, read_through, acc, xch ? &xs : nullptr);
    if (st != NP_OK) return st;
    L->state = kScattered;
    return NP_OK;
}
}  // namespace

np_status np_sparse_ffn(np_layer* L, const float* x, float* y, void* stream) {
    return sparse_ffn_call(L, x, y, stream, false);
}

np_status np_sparse_ffn_acc(np_layer* L, const float* x, float* y, void* stream) {
    return sparse_ffn_call(L, x, y, stream, true);
}

np_status np_sparse_ffn_noalloc(np_layer* L, const float* x, float* y, void* stream) {
    const Exchange tag{};
    return sparse_ffn_call(L, x, y, stream, false, &tag);
}

np_status np_layer_set_ffn_reduce(np_layer* L, int32_t mode) {
    if (!L) return fail(NP_EINVAL, "layer must not be NULL");
    if (mode != NP_REDUCE_ATOMIC && mode != NP_REDUCE_ORDERED) return fail(NP_EINVAL, "unknown reduce mode %d", mode);
    DeviceGuard g(L->desc.device);
    NP_HIP(hipDeviceSynchronize());
    L->reduce = mode;
    ++L->version;  // captured decode graphs carry the mode
    return NP_OK;
}

np_status np_decode_step(np_layer* const* layers, int32_t n_layers, const int32_t* cids, const float* x,
                         float* y, void* compute_stream, void* copy_stream) {
    if (!layers || !cids || n_layers < 1) return fail(NP_EINVAL, "layers, cids and n_layers >= 1 required");
    if (!x || !y || !aligned16(x) || !aligned16(y)) return fail(NP_EINVAL, "x and y must be 16-byte aligned device pointers");
    const np_layer* L0 = layers[0];
    if (!L0) return fail(NP_EINVAL, "layer 0 is NULL");
    const int dev = L0->desc.device, d = L0->desc.d_model;
    for (const auto& io : {std::make_pair((const void*)x, "x"), std::make_pair((const void*)y, "y")}) {
        const np_status pe = check_io_ptr(io.first, dev, io.second);
        if (pe != NP_OK) return pe;
    }
    std::vector<std::vector<uint64_t>> S(n_layers);
    std::vector<int> n_act(n_layers), n_in(n_layers), u_eff(n_layers);
    std::unique_lock<std::mutex> stage_lk(g_stage_mu);  // staging settings and buffers
    const bool stage_on = g_stage_bytes > 0;
    if (!stage_on) stage_lk.unlock();
    bool any_staged = false;
    std::vector<std::vector<int32_t>> din(n_layers);
    for (int l = 0; l < n_layers; ++l) {
        const np_layer* L = layers[l];
        if (!L) return fail(NP_EINVAL, "layer %d is NULL", l);
        if (L->desc.device != dev || L->desc.d_model != d)
            return fail(NP_EINVAL, "layer %d: all layers must share device and d_model", l);
        for (int k = 0; k < l; ++k)
            if (layers[k] == L) return fail(NP_EINVAL, "layer %d appears twice", l);
        if (L->state == kAssigned) return fail(NP_ESTATE, "layer %d has an unscattered delta", l);
        const np_status de = check_device_err(L, l);
        if (de != NP_OK) return de;
        int32_t u;
        np_status st = check_cids(L, cids[2 * l], cids[2 * l + 1], &u);
        if (st != NP_OK) return fail(st, "layer %d: %s", l, g_err.c_str());
        u_eff[l] = u;
        S[l].resize(L->W);
        n_act[l] = combine_host(L, cids[2 * l], u, S[l].data());
        if (n_act[l] > L->desc.k_max)
            return fail(NP_ECAPACITY, "layer %d: |S| = %d exceeds k_max = %d", l, n_act[l], L->desc.k_max);
        int ni = -1;  // with a retention rule the resident set is decided on the device
        if (!device_decides(L)) {
            ni = 0;
            for (int w = 0; w < L->W; ++w) ni += __builtin_popcountll(S[l][w] & ~L->h_res[w]);
        }
        n_in[l] = ni;
        if (stage_on && staged(L)) {  // the host reads these rows itself (staged I/O)
            any_staged = true;
            din[l].reserve(ni);
            for (int w = 0; w < L->W; ++w)
                for (uint64_t b = S[l][w] & ~L->h_res[w]; b; b &= b - 1)
                    din[l].push_back(w * 64 + __builtin_ctzll(b));
        }
    }
    DeviceGuard g(dev);
    hipStream_t cs = (hipStream_t)compute_stream, ps = (hipStream_t)copy_stream;
    auto commit_host_state = [&]() {
        for (int l = 0; l < n_layers; ++l) {
            np_layer* L = layers[l];
            L->h_res.swap(S[l]);
            L->n_active = n_act[l];
            L->n_in = n_in[l];
            L->total_active += n_act[l];
            L->total_in += std::max(n_in[l], 0);
            L->state = kAssigned;
        }
    };

    if (g_use_graphs.load() && n_layers <= kMaxGraphLayers && cs && ps && !any_staged) {
        np_status st = NP_OK;
        const std::shared_ptr<DecodePlan> P = get_plan(layers, n_layers, cs, ps, dev, &st);
        if (P) {
            for (int l0 = 0; l0 < n_layers; l0 += kParamsPerLaunch) {
                ParamsUpdate pu{};
                pu.first = l0;
                pu.count = std::min(kParamsPerLaunch, n_layers - l0);
                for (int k = 0; k < pu.count; ++k) {
                    np_layer* L = layers[l0 + k];
                    pu.cid[k][0] = cids[2 * (l0 + k)];
                    pu.cid[k][1] = u_eff[l0 + k];
                    if (++L->ffn_seq == 0) L->ffn_seq = 1;
                    pu.seq[k] = L->ffn_seq;
                }
                pu.x = x;
                pu.y = y;
                NP_HIP(launch_set_params(pu, P->prm, cs));
            }
            NP_HIP(hipGraphLaunch(P->exec, cs));
            commit_host_state();
            for (int l = 0; l < n_layers; ++l) layers[l]->state = kScattered;
            return NP_OK;
        }
        if (st != NP_OK && st != NP_EHIP) return st;  // a real argument error, not a capture failure
        // capture unavailable: fall through to direct launches
    }

    const hipEvent_t* ev = nullptr;
    if (any_staged && !one_queue(layers, n_layers, cs, ps)) {
        np_status st = step_events(dev, n_layers, &ev);
        if (st != NP_OK) return st;
    }
    std::vector<int32_t> cid_eff(2 * n_layers);
    for (int l = 0; l < n_layers; ++l) {
        cid_eff[2 * l] = cids[2 * l];
        cid_eff[2 * l + 1] = u_eff[l];
    }
    // the direct launches size their grids from the new host counts; a launch failure leaves the
    // layers assigned-but-unscattered, so they need np_layer_reset before further use
    if (!any_staged) {
        // token launches (groups of pinned-host-store layers): their argument staging is allocated
        // before anything is enqueued, so that a failed allocation leaves every layer unchanged
        for (int g0 = 0; g0 < n_layers; g0 += kTokenLayers) {
            bool host = true;
            for (int l = g0; l < std::min(n_layers, g0 + kTokenLayers); ++l) host = host && layers[l]->store_is_host;
            if (!host) continue;
            const np_status r = token_stage(layers[g0]);
            if (r != NP_OK) return r;
        }
    }
    Stager* stg = nullptr;
    if (any_staged) {
        for (int l = 0; l < n_layers; ++l)
            if (staged(layers[l]) && g_stage_bytes < layers[l]->bundle_elems() * 2)
                return fail(NP_EINVAL, "layer %d: staging of %zu bytes holds no %zu-byte bundle", l, g_stage_bytes,
                            (size_t)layers[l]->bundle_elems() * 2);
        np_status r = get_stager(dev, &stg);
        if (r != NP_OK) return r;
    }
    commit_host_state();
    np_status st = enqueue_token(layers, n_layers, cid_eff.data(), x, y, cs, ps, nullptr, ev,
                                 any_staged ? &din : nullptr, stg);
    if (st != NP_OK) return st;
    for (int l = 0; l < n_layers; ++l) layers[l]->state = kScattered;
    return NP_OK;
}

np_status np_decode_use_graphs(int32_t enable) {
    g_use_graphs.store(enable ? 1 : 0);
    if (!enable) {
        std::lock_guard<std::mutex> lk(g_plan_mu);
        g_plans.clear();
    }
    return NP_OK;
}

np_status np_layer_read_state(const np_layer* L, int32_t* slot_map, int32_t* owner, int32_t* d_in,
                              int32_t* slot_in, int32_t* d_out, int32_t* act_slots, int32_t* counts) {
    if (!L) return fail(NP_EINVAL, "layer must not be NULL");
    DeviceGuard g(L->desc.device);
    NP_HIP(hipDeviceSynchronize());
    const size_t K = L->desc.k_max;
    if (slot_map) NP_HIP(hipMemcpy(slot_map, L->slot_map, (size_t)L->desc.d_ff * 4, hipMemcpyDeviceToHost));
    if (owner) NP_HIP(hipMemcpy(owner, L->owner, K * 4, hipMemcpyDeviceToHost));
    if (d_in) NP_HIP(hipMemcpy(d_in, L->d_in(), K * 4, hipMemcpyDeviceToHost));
    if (slot_in) NP_HIP(hipMemcpy(slot_in, L->slot_in(), K * 4, hipMemcpyDeviceToHost));
    if (d_out) NP_HIP(hipMemcpy(d_out, L->d_out(), K * 4, hipMemcpyDeviceToHost));
    if (act_slots) NP_HIP(hipMemcpy(act_slots, L->act(), K * 4, hipMemcpyDeviceToHost));
    int32_t c[4];
    NP_HIP(hipMemcpy(c, L->counts, sizeof c, hipMemcpyDeviceToHost));
    if (counts) std::memcpy(counts, c, sizeof c);
    if (c[3]) return fail(NP_EDEVICE, "device error bits 0x%x", c[3]);
    return NP_OK;
}

np_status np_layer_read_rows(const np_layer* L, const int32_t* slots, int32_t n, void* dst) {
    if (!L || !dst || n < 0) return fail(NP_EINVAL, "layer and dst must not be NULL, n >= 0");
    DeviceGuard g(L->desc.device);
    NP_HIP(hipDeviceSynchronize());
    const size_t bb = L->bundle_elems() * 2;
    if (!slots) {
        if (n != L->desc.k_max) return fail(NP_EINVAL, "slots == NULL requires n == k_max");
    } else {
        for (int i = 0; i < n; ++i)
            if (slots[i] < 0 || slots[i] >= L->desc.k_max)
                return fail(NP_EINVAL, "slot %d out of range [0, %d)", slots[i], L->desc.k_max);
    }
    if (!L->planar) {
        if (!slots) {
            NP_HIP(hipMemcpy(dst, L->buf, (size_t)n * bb, hipMemcpyDeviceToHost));
            return NP_OK;
        }
        for (int i = 0; i < n; ++i)
            NP_HIP(hipMemcpy((char*)dst + (size_t)i * bb, (const char*)L->buf + (size_t)slots[i] * bb, bb,
                             hipMemcpyDeviceToHost));
        return NP_OK;
    }
    // planar buffers: copy them whole and reassemble the bundles
    const size_t rb = (size_t)L->desc.d_model * 2, K = (size_t)L->desc.k_max;
    std::vector<char> all(K * bb);
    NP_HIP(hipMemcpy(all.data(), L->buf, K * bb, hipMemcpyDeviceToHost));
    for (int i = 0; i < n; ++i) {
        const size_t sl = slots ? (size_t)slots[i] : (size_t)i;
        for (int r = 0; r < L->desc.n_rows; ++r)
            std::memcpy((char*)dst + (size_t)i * bb + r * rb, all.data() + (r * K + sl) * rb, rb);
    }
    return NP_OK;
}

np_status np_layer_info(const np_layer* L, int32_t* out6) {
    if (!L || !out6) return fail(NP_EINVAL, "layer and out must not be NULL");
    out6[0] = L->desc.d_model;
    out6[1] = L->desc.d_ff;
    out6[2] = L->desc.k_max;
    out6[3] = L->desc.n_rows;
    out6[4] = L->n_active;
    out6[5] = L->n_in;
    if (device_decides(L) && L->state != kFresh) {  // |D_in| is decided on the device
        DeviceGuard g(L->desc.device);
        NP_HIP(hipDeviceSynchronize());
        NP_HIP(hipMemcpy(&out6[5], L->counts, 4, hipMemcpyDeviceToHost));
    }
    return NP_OK;
}

np_status np_layer_counters(const np_layer* L, int64_t* out2) {
    if (!L || !out2) return fail(NP_EINVAL, "layer and out must not be NULL");
    out2[0] = L->total_active;
    out2[1] = L->total_in;
    if (device_decides(L)) {  // |D_in| is decided on the device: its running sum lives there
        DeviceGuard g(L->desc.device);
        NP_HIP(hipDeviceSynchronize());
        unsigned long long acc[2];
        NP_HIP(hipMemcpy(acc, L->counts + 8, sizeof acc, hipMemcpyDeviceToHost));
        out2[1] = (int64_t)acc[1];
    }
    return NP_OK;
}

np_status np_layer_set_window(np_layer* L, int32_t window) {
    if (!L) return fail(NP_EINVAL, "layer must not be NULL");
    if (window < 1 || window > kMaxWindow) return fail(NP_EINVAL, "window=%d must be in [1, %d]", window, kMaxWindow);
    if (window > 1 && L->n_levels > 0) return fail(NP_EINVAL, "a window excludes frequency levels (set n_levels 0 first)");
    if (window > 1 && L->layout == NP_LAYOUT_COMPACT) return fail(NP_EINVAL, "a window needs the slot layout");
    if (L->state != kFresh) return fail(NP_ESTATE, "set the window before the first np_delta_assign (or after np_layer_reset)");
    DeviceGuard g(L->desc.device);
    NP_HIP(hipDeviceSynchronize());
    uint64_t* ring = nullptr;
    if (window > 1) {
        const size_t bytes = (size_t)(window - 1) * L->W * 8;
        if (hipMalloc(&ring, bytes) != hipSuccess) {
            (void)hipGetLastError();
            return fail(NP_ENOMEM, "cannot allocate the %zu-byte window ring", bytes);
        }
        if (hipMemset(ring, 0, bytes) != hipSuccess) {
            (void)hipFree(ring);
            return fail(NP_EHIP, "window ring clear failed");
        }
    }
    LayerDev ld = L->ldh;
    ld.ring = ring;
    ld.window = window;
    if (hipMemcpy(L->ldev, &ld, sizeof ld, hipMemcpyHostToDevice) != hipSuccess) {
        if (ring) (void)hipFree(ring);
        return fail(NP_EHIP, "layer descriptor update failed");
    }
    if (L->ring) (void)hipFree(L->ring);
    L->ring = ring;
    L->window = window;
    L->ldh = ld;
    NP_HIP(hipMemset(L->counts, 0, kCountsBytes));  // token count and running sums restart
    ++L->version;
    return NP_OK;
}

np_status np_layer_raise_error(np_layer* L, int32_t bits, void* stream) {
    if (!L) return fail(NP_EINVAL, "layer must not be NULL");
    if (bits <= 0) return fail(NP_EINVAL, "bits=%d must be positive", bits);
    DeviceGuard g(L->desc.device);
    NP_HIP(launch_raise_err(L->counts, bits, (hipStream_t)stream));
    return NP_OK;
}

// The probes run on the current device: their pointers must be memory it can access.
static np_status check_probe_ptrs(std::initializer_list<std::pair<const void*, const char*>> ptrs) {
    int dev = 0;
    NP_HIP(hipGetDevice(&dev));
    for (const auto& p : ptrs) {
        const np_status st = check_io_ptr(p.first, dev, p.second);
        if (st != NP_OK) return st;
    }
    return NP_OK;
}

np_status np_probe_read(const void* src, int64_t bytes, float* sink, void* stream) {
    if (!src || !sink || bytes <= 0 || bytes % 16 || !aligned16(src))
        return fail(NP_EINVAL, "probe_read needs 16-byte aligned src, bytes > 0 and a multiple of 16");
    const np_status pc = check_probe_ptrs({{src, "src"}, {sink, "sink"}});
    if (pc != NP_OK) return pc;
    NP_HIP(launch_probe_read(src, bytes, sink, (hipStream_t)stream));
    return NP_OK;
}

np_status np_probe_read_set(const void* const* srcs, int32_t n_srcs, int64_t bytes, int32_t passes, float* sink,
                            void* stream) {
    if (!srcs || !sink || n_srcs < 1 || n_srcs > 4096 || passes < 1 || passes > 1000 || bytes <= 0 || bytes % 16)
        return fail(NP_EINVAL, "probe_read_set needs 1..4096 sources, 1..1000 passes, bytes > 0 and a multiple of 16");
    for (int32_t i = 0; i < n_srcs; ++i) {
        if (!srcs[i] || !aligned16(srcs[i])) return fail(NP_EINVAL, "probe_read_set: source %d is NULL or misaligned", i);
        const np_status pc = check_probe_ptrs({{srcs[i], "a source"}});
        if (pc != NP_OK) return pc;
    }
    const np_status pc = check_probe_ptrs({{sink, "sink"}});
    if (pc != NP_OK) return pc;
    for (int32_t p = 0; p < passes; ++p)
        for (int32_t i = 0; i < n_srcs; ++i) NP_HIP(launch_probe_read(srcs[i], bytes, sink, (hipStream_t)stream));
    return NP_OK;
}

np_status np_probe_copy(void* dst, const void* src, int64_t bytes, void* stream) {
    if (!src || !dst || bytes <= 0 || bytes % 16 || !aligned16(src) || !aligned16(dst))
        return fail(NP_EINVAL, "probe_copy needs 16-byte aligned pointers, bytes a multiple of 16");
    const np_status pc = check_probe_ptrs({{src, "src"}, {dst, "dst"}});
    if (pc != NP_OK) return pc;
    NP_HIP(launch_probe_copy(dst, src, bytes, (hipStream_t)stream));
    return NP_OK;
}

np_status np_layer_set_levels(np_layer* L, int32_t n_levels, const uint8_t* level) {
    if (!L) return fail(NP_EINVAL, "layer must not be NULL");
    if (n_levels < 0 || n_levels > kMaxLevels) return fail(NP_EINVAL, "n_levels=%d must be in [0, %d]", n_levels, kMaxLevels);
    if (n_levels > 0 && !level) return fail(NP_EINVAL, "level must not be NULL when n_levels > 0");
    if (n_levels > 0 && L->window > 1) return fail(NP_EINVAL, "frequency levels exclude a window > 1 (set window 1 first)");
    if (n_levels > 0 && L->layout == NP_LAYOUT_COMPACT) return fail(NP_EINVAL, "frequency levels need the slot layout");
    if (L->state != kFresh) return fail(NP_ESTATE, "set the levels before the first np_delta_assign (or after np_layer_reset)");
    const int M = L->desc.d_ff, W = L->W;
    std::vector<uint64_t> masks((size_t)n_levels * W, 0ull);
    for (int i = 0; i < M && n_levels > 0; ++i) {
        if (level[i] >= n_levels) return fail(NP_EINVAL, "level[%d] = %d is not below n_levels = %d", i, level[i], n_levels);
        const int j = n_levels - 1 - level[i];  // class order: highest level first
        masks[(size_t)j * W + (i >> 6)] |= 1ull << (i & 63);
    }
    DeviceGuard g(L->desc.device);
    NP_HIP(hipDeviceSynchronize());
    uint64_t* dm = nullptr;
    if (n_levels > 0) {
        const size_t bytes = masks.size() * 8;
        if (hipMalloc(&dm, bytes) != hipSuccess) {
            (void)hipGetLastError();
            return fail(NP_ENOMEM, "cannot allocate the %zu-byte level masks", bytes);
        }
        if (hipMemcpy(dm, masks.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
            (void)hipFree(dm);
            return fail(NP_EHIP, "level mask upload failed");
        }
    }
    LayerDev ld = L->ldh;
    ld.levels = dm;
    ld.n_levels = n_levels;
    if (hipMemcpy(L->ldev, &ld, sizeof ld, hipMemcpyHostToDevice) != hipSuccess) {
        if (dm) (void)hipFree(dm);
        return fail(NP_EHIP, "layer descriptor update failed");
    }
    if (L->levels) (void)hipFree(L->levels);
    L->levels = dm;
    L->n_levels = n_levels;
    L->ldh = ld;
    NP_HIP(hipMemset(L->counts, 0, kCountsBytes));  // token count and running sums restart
    ++L->version;
    return NP_OK;
}

np_status np_layer_set_layout(np_layer* L, int32_t layout) {
    if (!L) return fail(NP_EINVAL, "layer must not be NULL");
    if (layout != NP_LAYOUT_SLOTS && layout != NP_LAYOUT_COMPACT) return fail(NP_EINVAL, "unknown layout %d", layout);
    if (layout == NP_LAYOUT_COMPACT && (L->window > 1 || L->n_levels > 0))
        return fail(NP_EINVAL, "the compacted layout holds exactly S: no window or frequency levels");
    if (L->state != kFresh) return fail(NP_ESTATE, "set the layout before the first np_delta_assign (or after np_layer_reset)");
    DeviceGuard g(L->desc.device);
    NP_HIP(hipDeviceSynchronize());
    LayerDev ld = L->ldh;
    ld.compact = layout == NP_LAYOUT_COMPACT ? 1 : 0;
    NP_HIP(hipMemcpy(L->ldev, &ld, sizeof ld, hipMemcpyHostToDevice));
    L->ldh = ld;
    L->layout = layout;
    ++L->version;
    return NP_OK;
}

np_status np_layer_read_moves(const np_layer* L, int32_t* src, int32_t* dst, int32_t* n_moves) {
    if (!L || !n_moves) return fail(NP_EINVAL, "layer and n_moves must not be NULL");
    DeviceGuard g(L->desc.device);
    NP_HIP(hipDeviceSynchronize());
    int32_t n = 0;
    if (L->layout == NP_LAYOUT_COMPACT && L->state != kFresh)
        NP_HIP(hipMemcpy(&n, L->counts + 5, 4, hipMemcpyDeviceToHost));
    n = std::max(0, std::min(n, L->desc.k_max));
    if (n && src) NP_HIP(hipMemcpy(src, L->mv_src(), (size_t)n * 4, hipMemcpyDeviceToHost));
    if (n && dst) NP_HIP(hipMemcpy(dst, L->mv_dst(), (size_t)n * 4, hipMemcpyDeviceToHost));
    *n_moves = n;
    return NP_OK;
}

np_status np_decode_set_staging(int64_t bytes, int32_t threads) {
    if (bytes < 0 || bytes > (int64_t)1 << 30) return fail(NP_EINVAL, "staging bytes=%lld must be in [0, 1 GiB]", (long long)bytes);
    if (threads < 0 || threads > 64) return fail(NP_EINVAL, "threads=%d must be in [0, 64]", threads);
    std::lock_guard<std::mutex> lk(g_stage_mu);
    g_stagers.clear();  // waits for their last copies, frees the buffers
    g_stage_bytes = (size_t)bytes;
    const int hw = (int)std::thread::hardware_concurrency();
    g_stage_threads = threads ? threads : std::max(1, std::min(8, hw));
    return NP_OK;
}

np_status np_layer_set_planar(np_layer* L, int32_t planar) {
    if (!L) return fail(NP_EINVAL, "layer must not be NULL");
    if (planar != 0 && planar != 1) return fail(NP_EINVAL, "planar=%d must be 0 or 1", planar);
    if (L->state != kFresh) return fail(NP_ESTATE, "set the arrangement before the first np_delta_assign (or after np_layer_reset)");
    DeviceGuard g(L->desc.device);
    NP_HIP(hipDeviceSynchronize());
    LayerDev ld = L->ldh;
    ld.stride16 = planar ? ld.row16 : ld.bundle16;
    ld.plane16 = planar ? (int64_t)L->desc.k_max * ld.row16 : ld.row16;
    NP_HIP(hipMemcpy(L->ldev, &ld, sizeof ld, hipMemcpyHostToDevice));
    // the buffer is zero-filled in a fresh layer: nothing to rearrange
    L->ldh = ld;
    L->planar = planar;
    drop_plans_with(L);
    ++L->version;
    return NP_OK;
}

}  // extern "C"
