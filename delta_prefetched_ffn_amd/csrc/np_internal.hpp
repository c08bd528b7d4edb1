// Internal declarations shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace np {

// Library limits (also documented in include/np.h).
constexpr int kMaxDModel = 16384;
constexpr int kMaxDff = 65536;
constexpr int kMaxKmax = 65536;
constexpr int kMaxCentroids = 65536;
constexpr int kMaxWords = kMaxDff / 64;  // mask words per set
constexpr int kMaxKWords = kMaxKmax / 64;
constexpr int kMaxLayersPerLaunch = 64;
constexpr int kMaxWindow = 16;             // residency window, tokens
constexpr int kMaxLevels = 16;             // frequency levels of the retention by frequency
constexpr int kMaxClasses = 16;            // retention classes (window ages 1..15 or levels)
constexpr uint64_t kMaxBufBytes = (1ull << 32) - 4096;  // slot buffer addressed by 32-bit offsets

// Device error bits (counts[3]).
constexpr int kErrFreeExhausted = 1;   // delta assign: no free slot for an incoming neuron
constexpr int kErrBadList = 2;         // scatter/FFN: a list entry out of range
constexpr int kErrWindow = 4;          // FFN: window larger than the LDS staging
constexpr int kErrSpin = 8;            // FFN: a wait hit its iteration limit
constexpr int kErrCount = 16;          // FFN: host and device active counts differ

// Device code: view a pointer read from memory as a global-memory pointer. Without it the
// compiler must use flat accesses, which share a wait counter with LDS, so every LDS wait
// would also wait for outstanding global loads and stores.
#define NP_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ inline NP_GLOBAL T* gmem(T* p) {
    return (NP_GLOBAL T*)p;
}

// A layer's counts block: int32 [8] (counts[3] = error bits), 2 x uint64 running sums, then
// (int32 index 12, 8-byte aligned, not cleared by resets) the device address of the layer's
// pinned host error word. A kernel that raises error bits ORs them into counts[3] and stores
// them into the host word with a system-scope store, so the host sees them at the layer's next
// call without synchronizing (the host word may miss bits that two kernels raise at once;
// counts[3] has them all).
constexpr int kErrMirrorSlot = 12;
__device__ inline void raise_err(int32_t* counts, int bits) {
    NP_GLOBAL int32_t* const c = gmem(counts);
    __hip_atomic_fetch_or(c + 3, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    auto* const m = reinterpret_cast<uint32_t*>(*reinterpret_cast<NP_GLOBAL const uintptr_t*>(c + kErrMirrorSlot));
    if (m) __hip_atomic_store(gmem(m), (uint32_t)bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Everything a kernel needs about one layer; lives in device memory.
struct LayerDev {
    const uint64_t* masks;   // [n_tables][C][W]
    uint64_t* res;           // [W]  resident set R
    uint64_t* freeb;         // [Kw] free slots
    int32_t* slot_map;       // [M]
    int32_t* owner;          // [K]
    int32_t* d_in;           // [K]
    int32_t* slot_in;        // [K]
    int32_t* d_out;          // [K]
    int32_t* act;            // [K] ascending occupied slots
    int32_t* act_src;        // [K] per act position: the neuron if its slot was filled this step, else -1
    int32_t* counts;         // [8] n_in, n_out, n_active, error bits, tokens assigned, moves,
                             // prefetch and FFN workgroups done (token launch)
    unsigned long long* acc; // [2] running sums of n_active and n_in
    uint64_t* ring;          // [window - 1][W] active sets of the last tokens (window > 1)
    int32_t W, Kw, M, K;
    int32_t mode, n_tables, C, pad;
    const uint16_t* store;   // backing row store (device address; may be mapped host memory)
    uint16_t* buf;           // [K][R][d] slot buffer
    int32_t bundle16;        // 16-byte chunks per bundle (as laid out in the row store)
    // Slot buffer arrangement, in 16-byte chunks: row r of slot s starts at
    // s * stride16 + r * plane16. Interleaved (one bundle per slot): stride16 = bundle16,
    // plane16 = row16. Planar (one buffer per projection): stride16 = row16, plane16 = K * row16.
    int32_t row16;           // 16-byte chunks per row (d_model / 8)
    int32_t stride16;
    int64_t plane16;
    int32_t window;          // residency window in tokens (1: the buffer holds exactly S)
    // Retention by frequency level (n_levels > 0, window 1): bit masks of the neurons of each
    // level, highest level first ([n_levels][W]).
    const uint64_t* levels;
    int32_t n_levels;
    // Compacted layout (compact != 0): the active rows are positions 0 .. |S|-1; the rows
    // moved this step are mv_src[k] -> mv_dst[k], k < counts[5].
    int32_t compact;
    int32_t* mv_src;         // [K]
    int32_t* mv_dst;         // [K]
};

// One launch scattering the deltas of many layers (blockIdx.y = layer).
struct ScatterLaunch {
    const LayerDev* layers[kMaxLayersPerLaunch];
    int32_t n_layers;
};

// Per-token values of a replayed decode step, in device memory: written by k_set_params
// (whose kernel arguments carry them) before the step's captured launches read them.
constexpr int kMaxGraphLayers = 256;
struct DecodeParams {
    int32_t cid[kMaxGraphLayers][2];
    uint32_t seq[kMaxGraphLayers];
    const float* x;  // [n_layers][d]
    float* y;        // [n_layers][d]
};
// What one k_set_params launch carries (kernel arguments are limited to 4 KiB).
constexpr int kParamsPerLaunch = 128;
struct ParamsUpdate {
    int32_t first, count;
    int32_t cid[kParamsPerLaunch][2];
    uint32_t seq[kParamsPerLaunch];
    const float* x;
    float* y;
};

struct DeltaLaunch {
    const LayerDev* layers[kMaxLayersPerLaunch];
    int32_t cid[kMaxLayersPerLaunch][2];
    int32_t n_layers;
    const DecodeParams* prm;  // if set, centroid IDs come from prm->cid[layer0 + i]
    int32_t layer0;
    // zero_y != 0: each workgroup also clears y[layer0 + i][0..d) (y from prm when set),
    // for FFN launches that add their partial sums into y.
    float* y;
    int32_t zero_y, d;
};

// FFN launch shape (chosen on the host from the host-known |S|).
struct FfnShape {
    int nt;        // threads per workgroup
    int p1;        // gate/up chunks (= workgroups with gate/up work)
    int q;         // column tiles of the down phase
    int tw;        // columns per tile (multiple of 8)
    int nwg;       // p1 + q - 1 workgroups
    int jx;        // 16-byte x chunks per thread (gate/up phase)
    int win_max;   // LDS window capacity (positions)
    int fixed;     // 1: rows of 512 lanes and 256-column tiles, a lane geometry fixed at compile time
};

struct TokenArgs;

struct FfnArgs {
    uint16_t* buf;          // [K][R][d]
    const int32_t* act;     // [K]
    // Read-through (read_through != 0): bundles of slots filled this step are read from the
    // row store (act_src gives the neuron) and written into their slots by this launch.
    const int32_t* act_src; // [K] (always a valid array)
    const uint16_t* store;  // [M][R][d]
    uint32_t store_bytes;   // size of store when read_through (below 4 GiB), else 0
    int32_t read_through;
    int32_t* counts;        // [4]
    const float* x;         // [d]
    float* y;               // [d]
    uint64_t* hpair;        // [K] (launch sequence, h) words
    uint64_t* ppair;        // [nwg][tw] (launch sequence, partial sum) words
    uint32_t seq;           // this launch's sequence number (never 0)
    int32_t n;              // active slots (host-known), or -1 to read counts[2]
    const DecodeParams* prm;  // if set: seq, x and y come from prm (layer `layer`), n from counts[2]
    int32_t layer;
    uint32_t buf_bytes;     // size of buf (below 4 GiB)
    uint32_t slot_stride;   // bytes from one slot's row to the next slot's same row
    uint32_t row_plane;     // bytes from a slot's row r to its row r + 1
    int32_t d, K, R, M;
    int32_t p1, q, tw, nwg;
    int32_t activation;     // 0 ReLU, 1 SiLU
    int32_t atomic_y;       // 1: every workgroup adds its tile partials into y with float atomics
    int32_t accumulate;     // ordered reduction only: y = y + FFN instead of y = FFN
    // Prefetch (pf_wgs > 0): the launch's first pf_wgs workgroups scatter the new bundles of
    // another layer (pf) from its row store into its slots; the FFN workgroups follow them.
    const LayerDev* pf;
    int32_t pf_wgs;
    // Token launch (only this field is read from the kernel argument): the whole decode token
    // of a group of layers, described by *tok in device memory.
    const TokenArgs* tok;
};

// One launch for a decode token over up to kTokenLayers layers whose row stores are pinned host
// memory. Workgroups [0, n_pf) copy every layer's new bundles (scatter_flat), layer after layer,
// and after each layer add 1 to that layer's counts[kPfDoneSlot]; workgroups
// [n_pf + wg0[l], n_pf + wg0[l + 1]) are layer l's FFN, which starts once that count reaches
// n_pf and layer l - 1's counts[kFfnDoneSlot] (one per finished FFN workgroup) reaches its
// workgroup count. The assign launch zeroes both counts. ffn is last so that a copy can stop
// after the layers in use.
constexpr int kTokenLayers = 64;
constexpr int kPfDoneSlot = 6;
constexpr int kFfnDoneSlot = 7;
struct TokenArgs {
    int32_t n_layers, n_pf;
    int32_t wg0[kTokenLayers + 1];
    const LayerDev* src[kTokenLayers];
    FfnArgs ffn[kTokenLayers];
};

// 16-byte chunk c of a bundle (rows of row16 chunks, one after the other) in slot s of the
// slot buffer: row r = c / row16 lives at s * stride16 + r * plane16 (interleaved or planar).
__device__ inline size_t slot_chunk(int s, int c, int row16, int stride16, int64_t plane16) {
    const int r = c / row16;
    return (size_t)s * stride16 + (size_t)r * plane16 + (size_t)(c - r * row16);
}

// Copies the bundles that layer L's last assignment brought in (d_in / slot_in, counts[0] of
// them) from its row store into their slots. Workgroup g of ng (NT threads) takes bundles
// g, g + ng, ...; each lane moves U 16-byte chunks per pass, all U loads issued before the
// stores.
template <int NT, int U>
__device__ inline void scatter_bundles(const LayerDev* layer, int g, int ng) {
    const NP_GLOBAL LayerDev* const L = gmem(layer);
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const int M = L->M, K = L->K, cb = L->bundle16;
    const int n_in = min(gmem(L->counts)[0], K);  // the lists hold at most K entries
    const auto* store = gmem(reinterpret_cast<const u4*>(L->store));
    auto* buf = gmem(reinterpret_cast<u4*>(L->buf));
    const auto* d_in = gmem(L->d_in);
    const auto* slot_in = gmem(L->slot_in);
    for (int i = g; i < n_in; i += ng) {
        const int n = d_in[i], s = slot_in[i];
        if ((unsigned)n >= (unsigned)M || (unsigned)s >= (unsigned)K) {
            if (threadIdx.x == 0) raise_err(L->counts, kErrBadList);
            continue;
        }
        const auto* src = store + (size_t)n * cb;
        for (int c = threadIdx.x; c < cb; c += NT * U) {
            u4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c + u * NT < cb) v[u] = src[c + u * NT];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c + u * NT < cb) buf[slot_chunk(s, c + u * NT, L->row16, L->stride16, L->plane16)] = v[u];
        }
    }
}

// The scatter for a row store in pinned host memory. A compute unit keeps only a few
// kilobytes of host-link loads in flight (about 6 GB/s per unit), so a few dozen units hold the
// link at its ceiling; more workgroups only take units from other work. Workgroup g of ng (NT
// threads) copies bundles [n_in g / ng, n_in (g + 1) / ng) of layer L's last assignment as one
// run of 16-byte chunks, kFlatU loads per lane in flight; its (neuron, slot) list goes through
// LDS (s_n, s_s: CAP entries each) in pieces.
constexpr int kFlatU = 8;
template <int NT, int CAP>
__device__ inline void scatter_flat(const LayerDev* layer, int g, int ng, int* s_n, int* s_s) {
    const NP_GLOBAL LayerDev* const L = gmem(layer);
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const int M = L->M, K = L->K, cb = L->bundle16;
    const int row16 = L->row16, stride16 = L->stride16;
    const int64_t plane16 = L->plane16;
    const int n_in = max(0, min(gmem(L->counts)[0], K));  // the lists hold at most K entries
    const auto* store = gmem(reinterpret_cast<const u4*>(L->store));
    auto* buf = gmem(reinterpret_cast<u4*>(L->buf));
    const int b0 = (int)((int64_t)n_in * g / ng), b1 = (int)((int64_t)n_in * (g + 1) / ng);
    int err = 0;
    for (int p0 = b0; p0 < b1; p0 += CAP) {
        const int np = min(CAP, b1 - p0);
        __syncthreads();  // the previous piece's list is no longer read
        for (int i = threadIdx.x; i < np; i += NT) {
            const int n = gmem(L->d_in)[p0 + i], s = gmem(L->slot_in)[p0 + i];
            const bool bad = (unsigned)n >= (unsigned)M || (unsigned)s >= (unsigned)K;
            err |= bad ? kErrBadList : 0;
            s_n[i] = bad ? -1 : n;
            s_s[i] = s;
        }
        __syncthreads();
        const int total = np * cb;  // CAP * 3 * 2048 chunks at most: fits 32 bits
        for (int k0 = threadIdx.x; k0 < total; k0 += NT * kFlatU) {
            u4 v[kFlatU];
#pragma unroll
            for (int u = 0; u < kFlatU; ++u) {
                const int k = k0 + u * NT, b = k / cb, n = k < total ? s_n[b] : -1;
                if (n >= 0) v[u] = store[(size_t)n * cb + (k - b * cb)];
            }
#pragma unroll
            for (int u = 0; u < kFlatU; ++u) {
                const int k = k0 + u * NT, b = k / cb, n = k < total ? s_n[b] : -1;
                if (n >= 0) buf[slot_chunk(s_s[b], k - b * cb, row16, stride16, plane16)] = v[u];
            }
        }
    }
    if (err) raise_err(L->counts, err);
}

// Launchers (return hipError_t from the launch).
hipError_t launch_delta_assign(const DeltaLaunch& a, hipStream_t s);
hipError_t launch_set_params(const ParamsUpdate& p, DecodeParams* dst, hipStream_t s);
hipError_t launch_raise_err(int32_t* counts, int bits, hipStream_t s);
hipError_t launch_scatter(int32_t* counts, const int32_t* d_in, const int32_t* slot_in,
                          const uint16_t* store, uint16_t* buf, int32_t M, int32_t K,
                          int32_t bundle_elems, int32_t row16, int32_t stride16, int64_t plane16, int grid,
                          hipStream_t s);
hipError_t launch_scatter_all(const ScatterLaunch& a, int wgs_per_layer, hipStream_t s);
hipError_t launch_scatter_flat(const LayerDev* L, int wgs, hipStream_t s);
hipError_t launch_move_all(const ScatterLaunch& a, int wgs_per_layer, hipStream_t s);
hipError_t launch_scatter_staged(int32_t* counts, const int32_t* slot_in, const void* stage, uint16_t* buf,
                                 int32_t cnt, int32_t K, int32_t bundle_elems, int32_t row16, int32_t stride16,
                                 int64_t plane16, hipStream_t s);
hipError_t launch_sparse_ffn(const FfnArgs& a, const FfnShape& sh, bool gated, hipStream_t s);
hipError_t launch_token(const TokenArgs* ta, int grid, const FfnShape& sh, bool gated, hipStream_t s);
hipError_t launch_probe_read(const void* src, int64_t bytes, float* sink, hipStream_t s);
hipError_t launch_probe_copy(void* dst, const void* src, int64_t bytes, hipStream_t s);

// Gate/up chunks per FFN launch are capped; the partial-sum area is sized for it.
constexpr int kP1Cap = 4096;
constexpr int kMaxTiles = kMaxDModel / 64;

}  // namespace np
