// Fused gather-GEMV sparse FFN for gfx950 (batch 1, bf16 rows, fp32 math).
//
// Computes y = sum over the resident slots s of down_s * act(gate_s . x) * (up_s . x)
// (gated bundle [gate|up|down^T]) or y = sum_s down_s * act(up_s . x) (bundle
// [up|down^T]); NeuroPrefetcher, section 3.4: each active neuron i uses row i of
// gate, up and down^T; the slot map locates the rows, whose order in the buffer
// does not matter.
//
// Batch-1 decode is a memory-bound GEMV (about 1 flop per byte), so there is no
// MFMA here. The kernel is built so that every weight byte crosses HBM once,
// every workgroup has all of its loads in flight right after it learns its slot
// list, and the cross-workgroup exchanges cost one round trip each.
//
// Decomposition (n active slots, listed in ascending slot order):
//   * The slot list is cut into P1 balanced chunks. Workgroup w < P1 computes
//     h for its chunk (phase 1): full-row dot products of the gate and up rows
//     with x (x lives in registers: each lane always covers the same 16-byte
//     column chunks), reduced across the workgroup.
//   * The down rows are cut into Q column tiles of TW columns. Workgroup w
//     (0 <= w < P1 + Q - 1) takes tile w mod Q over the window of chunks
//     [w - Q + 1, w] (phase 2). Its down-row loads are issued before phase 1,
//     so they overlap the gate/up traffic.
//   * Over the contributors of a tile (w = t, t + Q, ...) the windows cover
//     every chunk exactly once. Ordered reduction: the highest contributor of a
//     tile sums the tile's partials in ascending contributor order (fixed
//     order: results are identical run to run) and writes y. Atomic reduction:
//     every contributor adds its partial into y with float atomics, which saves
//     the second exchange but leaves the order of the additions free.
//
// Read-through: in a decode step whose row store is device memory, a slot filled this
// step is read from the row store (where its bundle already is) instead of from the slot
// buffer, and the workgroup that reads a piece of such a bundle also writes it into the
// slot. Every piece of every active bundle is read by exactly one workgroup, so the new
// rows cross HBM once for reading and once for writing, and no separate scatter runs.
//
// Prefetch: a decode step with host-memory row stores runs layer l's FFN and the scatter of
// layer l + 1's new bundles in one launch. The scatter takes the first few workgroups, so its
// loads go out on the host link first, and the FFN workgroups follow; both write disjoint
// memory (different layers), the scatter never waits, and the FFN workgroups wait only on
// FFN workgroups below them. A compute unit returns its loads in order, so an FFN workgroup
// beside a scatter workgroup would wait for the scatter's host-link loads (tens of
// microseconds) before its own: the scatter workgroups use all their waves, which with this
// kernel's register count leaves no room for an FFN workgroup on their units, and they are few
// (a handful of units keeps the host link busy). With one launch per layer on one queue, the
// next layer's FFN starts as soon as this launch ends, with no event between queues.
//
// Exchanges between workgroups carry their own validity: every h value and
// every partial sum is stored as one 64-bit word (launch sequence number,
// value) with an agent-scope store, which writes through the XCD's own L2 so
// that workgroups on the other XCDs see it, and the reader re-reads a word
// with agent-scope loads until its sequence number is this launch's. So there are no flags, no
// fences and no counters, and a reader waits only for workgroups with lower
// IDs, which the dispatcher starts first: every wait ends. A wait also gives
// up after a fixed number of polls and reports an error bit instead of hanging.
#include <type_traits>

#include "np_internal.hpp"

namespace np {
namespace {

constexpr int kWinMax = 2048;            // staged window positions per workgroup
constexpr uint32_t kSpinLimit = 1u << 20;

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float fv4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// x is held as two bf16 halves per value (x = hi + lo to 16 significant bits, relative error
// at most 2^-17), so that a gate or up row, whose weights are bf16, is dotted with x by
// v_dot2c_f32_bf16: two products and the fp32 accumulation in one instruction, with no
// unpacking of the weights. 16 bytes of weights (8 columns) take 8 such instructions.
struct XSplit {
    uint32_t hi[4], lo[4];
};
__device__ inline XSplit split_x(const fv4 a, const fv4 b, bool valid) {
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    XSplit s;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float2 f = valid ? make_float2(v[2 * k], v[2 * k + 1]) : make_float2(0.f, 0.f);
        const bf2 h = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){f.x, f.y}, bf2);
        const uint32_t hb = __builtin_bit_cast(uint32_t, h);
        const float r0 = f.x - __uint_as_float(hb << 16), r1 = f.y - __uint_as_float(hb & 0xffff0000u);
        const bf2 l = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){r0, r1}, bf2);
        s.hi[k] = hb;
        s.lo[k] = __builtin_bit_cast(uint32_t, l);
    }
    return s;
}
__device__ inline float dot2(uint32_t w, uint32_t x, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w), __builtin_bit_cast(bf2, x), c, false);
}
// Dot product of 8 bf16 weights with the 8 x values of s: the hi half first, then the lo half.
__device__ inline float dot8(const uint4 v, const XSplit& s) {
    float a = 0.f;
    a = dot2(v.x, s.hi[0], a);
    a = dot2(v.y, s.hi[1], a);
    a = dot2(v.z, s.hi[2], a);
    a = dot2(v.w, s.hi[3], a);
    a = dot2(v.x, s.lo[0], a);
    a = dot2(v.y, s.lo[1], a);
    a = dot2(v.z, s.lo[2], a);
    a = dot2(v.w, s.lo[3], a);
    return a;
}

// h of one neuron from its gate (g) and up (u) dot products: act(g) * u gated, act(u) not.
// act 1 is SiLU, g / (1 + exp(-g)) (for very negative g, exp overflows to +inf and the
// quotient is -0); act 0 is ReLU.
__device__ inline float neuron_h(float g, float u, bool gated, int act) {
    const float v = gated ? g : u;
    const float a = act == 1 ? v / (1.f + expf(-v)) : fmaxf(v, 0.f);
    return gated ? a * u : a;
}

__device__ inline void axpy8(float* acc, const float h, const uint4 v) {
    acc[0] = fmaf(h, bf_lo(v.x), acc[0]);
    acc[1] = fmaf(h, bf_hi(v.x), acc[1]);
    acc[2] = fmaf(h, bf_lo(v.y), acc[2]);
    acc[3] = fmaf(h, bf_hi(v.y), acc[3]);
    acc[4] = fmaf(h, bf_lo(v.z), acc[4]);
    acc[5] = fmaf(h, bf_hi(v.z), acc[5]);
    acc[6] = fmaf(h, bf_lo(v.w), acc[6]);
    acc[7] = fmaf(h, bf_hi(v.w), acc[7]);
}

// Cross-lane exchanges of one wave without the LDS crossbar. Lane pairing at offset OFF:
// 32 and 16 by the gfx950 lane-swap instructions (v_permlane32_swap / v_permlane16_swap
// move one operand's upper half of each 2*OFF-lane group into the other operand's lower
// half), 8 by a rotation of each 16-lane row by 8, 4 by mirroring each 8-lane half-row
// (lane i with 7 - i, which also pairs a lane that has bit 2 clear with one that has it set),
// 2 and 1 by quad permutations.
template <int OFF>
__device__ inline float lane_partner(float x) {
    static_assert(OFF == 8 || OFF == 4 || OFF == 2 || OFF == 1, "row-local offsets only");
    constexpr int ctrl = OFF == 8 ? 0x128 : OFF == 4 ? 0x141 : OFF == 2 ? 0x4E : 0xB1;
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xF, 0xF, false));
}
// Transposing exchange: lanes with the OFF bit clear return x + x(partner), lanes with it
// set return y + y(partner).
template <int OFF>
__device__ inline float lane_fold(float x, float y, int lane) {
    if constexpr (OFF == 32 || OFF == 16) {
        const auto r = OFF == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false)
                                 : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        const float sx = x + lane_partner<OFF>(x), sy = y + lane_partner<OFF>(y);
        return (lane & OFF) ? sy : sx;
    }
}

// Weight rows are read with 16-byte buffer loads at 32-bit offsets from a buffer descriptor of
// the slot buffer (or of the row store). A lane with nothing to load uses an offset past the
// end of every buffer: the hardware's range check returns zeros for it without a memory access.
// Every load is then an unconditional instruction, so the compiler waits for exactly the loads
// a computation needs, and the zeros add nothing to the sums they enter.
constexpr uint32_t kOOB = 0xFFFFF000u;  // >= every buffer's size (at most 4 GiB - 4096)
constexpr int kBufWord3 = 0x00020000;   // descriptor word 3: 32-bit data format, no swizzle
__device__ inline __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
    // (readfirstlane returns a signed int: each half goes through uint32_t before widening, so
    // the low half cannot sign-extend over the high one)
    const uint64_t b = (uint64_t)base;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint64_t u = ((uint64_t)hi << 32) | (uint64_t)lo;
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), (short)0,
                                            (int)__builtin_amdgcn_readfirstlane(bytes), kBufWord3);
}
// Non-temporal: every weight byte is read once per launch.
__device__ inline uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
    return make_uint4(t.x, t.y, t.z, t.w);
}
// Read-through stores of new rows (streaming: nothing in this launch reads them again); an
// offset past the end drops the store.
__device__ inline void bstore(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint4 v) {
    const u32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(t, r, (int)off, 0, 2);
}

__device__ inline uint64_t ld_pair(const uint64_t* p) {
    return __hip_atomic_load(gmem(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_pair(uint64_t* p, uint32_t seq, float v) {
    __hip_atomic_store(gmem(p), ((uint64_t)__float_as_uint(v) << 32) | seq, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t pair_seq(uint64_t p) { return (uint32_t)p; }
__device__ inline float pair_val(uint64_t p) { return __uint_as_float((uint32_t)(p >> 32)); }

// Prefetch workgroup g of n_pf in a token launch: its share of every layer's delta, layer after
// layer (the same shares and chunk runs as scatter_flat). Each layer's parameters and share are
// read once, in parallel (one lane per layer), into LDS. When the (neuron, slot) lists of all its
// shares fit in LDS they are staged there too, and at each layer boundary the next layer's first
// loads are issued before the wait that completes the stores of the layers before it, so the
// workgroup keeps the host link busy while it publishes them: after that wait and a barrier, one
// agent-scope release (which writes this XCD's L2 back) raises each such layer's
// counts[kPfDoneSlot]. (The FFN workgroups that read those rows have read none of these lines
// since the launch began, so their caches hold no stale copy.) Otherwise each layer is copied,
// completed and published in turn.
struct PfLayer {
    const uint4* store;
    uint4* buf;
    const int32_t* d_in;
    const int32_t* slot_in;
    int32_t* counts;
    int64_t plane16;
    int32_t cb, row16, stride16, b0, M, K;
};
// Loads per lane in flight.
constexpr int kTokU = 8;
template <int NT>
__device__ __forceinline__ void prefetch_token(const NP_GLOBAL TokenArgs* __restrict__ ta, int g, int n_pf, int* s_n,
                                               int* s_s) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    __shared__ PfLayer s_ly[kTokenLayers];
    __shared__ int s_off[kTokenLayers + 1];
    const int nl = ta->n_layers;
    auto publish = [&](int l0, int l1) {  // layers [l0, l1): every wave has waited for its stores
        __syncthreads();
        if (threadIdx.x == 0)
            for (int l = l0; l < l1; ++l)
                __hip_atomic_fetch_add(gmem(s_ly[l].counts) + kPfDoneSlot, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    };
    if ((int)threadIdx.x < nl) {
        const auto* L = gmem(ta->src[threadIdx.x]);
        PfLayer y;
        y.store = reinterpret_cast<const uint4*>(L->store);
        y.buf = reinterpret_cast<uint4*>(L->buf);
        y.d_in = L->d_in;
        y.slot_in = L->slot_in;
        y.counts = L->counts;
        y.plane16 = L->plane16;
        y.cb = L->bundle16;
        y.row16 = L->row16;
        y.stride16 = L->stride16;
        y.M = L->M;
        y.K = L->K;
        const int n_in = max(0, min(gmem(L->counts)[0], y.K));  // the lists hold at most K entries
        y.b0 = (int)((int64_t)n_in * g / n_pf);
        s_off[threadIdx.x + 1] = (int)((int64_t)n_in * (g + 1) / n_pf) - y.b0;  // this share's length
        s_ly[threadIdx.x] = y;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        s_off[0] = 0;
        for (int l = 0; l < nl; ++l) s_off[l + 1] += s_off[l];
    }
    __syncthreads();
    const int total_entries = s_off[nl];
    if (total_entries > kWinMax) {  // lists too long for LDS (a cold start of large layers)
        for (int l = 0; l < nl; ++l) {
            scatter_flat<NT, kWinMax>(ta->src[l], g, n_pf, s_n, s_s);
            __builtin_amdgcn_s_waitcnt(0);
            publish(l, l + 1);
        }
        return;
    }
    uint64_t bad_layers = 0;  // layers with a list entry out of range (raised at the end)
    for (int e = threadIdx.x; e < total_entries; e += NT) {
        int l = 0;
        while (s_off[l + 1] <= e) ++l;
        const PfLayer& y = s_ly[l];
        const int i = y.b0 + e - s_off[l];
        const int n = gmem(y.d_in)[i], sl = gmem(y.slot_in)[i];
        const bool bad = (unsigned)n >= (unsigned)y.M || (unsigned)sl >= (unsigned)y.K;
        bad_layers |= bad ? 1ull << l : 0ull;
        s_n[e] = bad ? -1 : n;
        s_s[e] = sl;
    }
    __syncthreads();
    int pend = 0;  // layers [pend, l) are copied by this workgroup but not yet published
    for (int l = 0; l < nl; ++l) {
        const int cb = s_ly[l].cb, row16 = s_ly[l].row16, stride16 = s_ly[l].stride16;
        const int64_t plane16 = s_ly[l].plane16;
        const auto* store = gmem(reinterpret_cast<const u4*>(s_ly[l].store));
        auto* buf = gmem(reinterpret_cast<u4*>(s_ly[l].buf));
        const int off = s_off[l], total = (s_off[l + 1] - off) * cb;
        const int passes = (total + NT * kTokU - 1) / (NT * kTokU);
        for (int p = 0; p < passes; ++p) {
            const int k0 = p * NT * kTokU + (int)threadIdx.x;
            u4 v[kTokU];
#pragma unroll
            for (int u = 0; u < kTokU; ++u) {
                const int k = k0 + u * NT, b = k / cb, n = k < total ? s_n[off + b] : -1;
                if (n >= 0) v[u] = store[(size_t)n * cb + (k - b * cb)];
            }
            if (p == 0 && pend < l) {
                // this layer's first loads are in flight: complete and publish the layers before it
                __builtin_amdgcn_s_waitcnt(0);
                publish(pend, l);
                pend = l;
            }
#pragma unroll
            for (int u = 0; u < kTokU; ++u) {
                const int k = k0 + u * NT, b = k / cb, n = k < total ? s_n[off + b] : -1;
                if (n >= 0) buf[slot_chunk(s_s[off + b], k - b * cb, row16, stride16, plane16)] = v[u];
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    publish(pend, nl);
    for (; bad_layers; bad_layers &= bad_layers - 1) raise_err(s_ly[__builtin_ctzll(bad_layers)].counts, kErrBadList);
}

// NT threads; JX 16-byte x chunks per lane; SB slots per phase-1 batch per row lane;
// U2 down rows per lane per phase-2 batch; RT read-through of the slots filled this step (a
// separate instantiation, so that a profile tells the two kinds of launch apart); PF prefetch
// workgroups ahead of the FFN's (separate too: without them the kernel is unchanged); TOK the
// token launch (a.tok: every layer's scatter and FFN of a decode token in one grid); FCL, when
// not 0, the lanes per row (CL) fixed at compile time, together with 256-column tiles: the
// lane geometry then costs no runtime divisions or branches.
template <int NT, int JX, bool GATED, int SB, int U2, bool RT, bool PF, bool TOK, int FCL>
__global__ __launch_bounds__(NT) void k_sparse_ffn(FfnArgs a0) {
    constexpr int kWaves = NT / 64;
    constexpr int R = GATED ? 3 : 2;
    constexpr int NR1 = GATED ? 2 : 1;  // rows dotted with x per slot

    __shared__ float s_h[kWinMax];  // h of the window positions
    __shared__ float s_red1[kWaves * SB * NR1];  // wave sums of the gate/up dot products
    // partial-sum rows: one per wave of 256 columns with the compiled geometry, else up to 8 NT
    __shared__ float s_red2[FCL ? kWaves * 256 : NT * 8];
    // Token launch: this workgroup's layer's arguments. Read from LDS, they never wait behind
    // the row loads (a field read from global memory mid-stream would, returns being in order).
    __shared__ FfnArgs s_fa;

    if constexpr (PF) {
        if ((int)blockIdx.x < a0.pf_wgs) {
            __shared__ int s_pn[kWinMax], s_ps[kWinMax];
            scatter_flat<NT, kWinMax>(a0.pf, blockIdx.x, a0.pf_wgs, s_pn, s_ps);
            return;
        }
    }
    int w_tok = 0;
    const NP_GLOBAL TokenArgs* __restrict__ ta = gmem(a0.tok);
    if constexpr (TOK) {
        const int n_pf = ta->n_pf, nl = ta->n_layers;
        if ((int)blockIdx.x < n_pf) {
            __shared__ int s_pn[kWinMax], s_ps[kWinMax];
            prefetch_token<NT>(ta, blockIdx.x, n_pf, s_pn, s_ps);
            return;
        }
        // FFN workgroup b of the token: layer l, workgroup b - wg0[l] of its FFN. It starts once
        // all n_pf prefetch workgroups have finished layer l and, so that the layers run in
        // order as a model's do, all workgroups of layer l - 1's FFN have finished (both have
        // lower IDs and started first).
        const int b = blockIdx.x - n_pf;
        int l = 0;
        while (l + 1 < nl && b >= ta->wg0[l + 1]) ++l;
        static_assert(sizeof(FfnArgs) % 4 == 0 && sizeof(FfnArgs) / 4 <= NT, "FfnArgs copy");
        if (threadIdx.x < sizeof(FfnArgs) / 4)
            reinterpret_cast<int32_t*>(&s_fa)[threadIdx.x] =
                reinterpret_cast<const NP_GLOBAL int32_t*>(&ta->ffn[l])[threadIdx.x];
        if (threadIdx.x == 0) {
            const NP_GLOBAL int32_t* done = gmem(gmem(ta->src[l])->counts) + kPfDoneSlot;
            const NP_GLOBAL int32_t* prev = l > 0 ? gmem(gmem(ta->src[l - 1])->counts) + kFfnDoneSlot : nullptr;
            const int n_prev = l > 0 ? ta->wg0[l] - ta->wg0[l - 1] : 0;
            for (uint32_t it = 0;; ++it) {
                if (__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n_pf &&
                    (!prev || __hip_atomic_load(prev, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n_prev))
                    break;
                if (it >= kSpinLimit) {
                    raise_err(ta->ffn[l].counts, kErrSpin);
                    break;
                }
                __builtin_amdgcn_s_sleep(16);
            }
        }
        __syncthreads();
        w_tok = b - ta->wg0[l];
    }
    // This launch's arguments: the kernel argument, or the layer's entry of a token launch.
    const FfnArgs& a = TOK ? s_fa : a0;
    const int w = TOK ? w_tok : (PF ? blockIdx.x - a.pf_wgs : blockIdx.x), tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int d = a.d, cpr = d >> 3, K = a.K;
    // In a replayed decode step the per-token values come from the parameter block.
    const uint32_t seq = a.prm ? a.prm->seq[a.layer] : a.seq;
    const auto* xg = gmem(a.prm ? a.prm->x + (size_t)a.layer * a.d : a.x);
    const auto* act = gmem(a.act);
    const auto* act_src = gmem(a.act_src);

    // Phase-1 lane geometry: CL lanes share a row (power of two), RL row lanes.
    int CL_rt = NT;
    while (CL_rt > cpr && CL_rt > 1) CL_rt >>= 1;
    const int CL = FCL ? FCL : CL_rt;
    const int RL = NT / CL;
    const int rl = tid / CL, cl = tid % CL;

    // |S| comes from the host (it validated the capacity with it); the device count is only
    // checked against it, with a load that goes out beside the h polls below, whose wait covers
    // it (a wave's loads return in order: issued before the row loads it would hold them back,
    // and a check right after its load would wait for all of them). A replayed graph has no
    // host count and reads the device one.
    const bool host_n = a.n >= 0 && !a.prm;
    int n = host_n ? a.n : gmem(a.counts)[2];
    n = n < 0 ? 0 : (n > K ? K : n);
    // c * n <= 4096 * 65536 < 2^31: 32-bit arithmetic
    auto cbeg = [&](int c) { return (int)(((unsigned)c * (unsigned)n) / (unsigned)a.p1); };

    // Window of chunks handled in phase 2: [wlo, whi]; their slot positions [plo, phi).
    const int wlo = max(0, w - a.q + 1), whi = min(w, a.p1 - 1);
    const int plo = cbeg(wlo);
    int phi = cbeg(whi + 1);
    int err = 0;
    if (phi - plo > kWinMax) {
        err |= kErrWindow;
        phi = plo + kWinMax;
    }
    const int wn = phi - plo;
    const bool has1 = w < a.p1;
    const int c0 = has1 ? max(cbeg(w), plo) : 0, c1 = has1 ? min(cbeg(w + 1), phi) : 0;

    // Phase-2 lane geometry: down tile t, CT lanes per row segment, RL2 row lanes.
    const int t = w % a.q;
    const int col0 = t * a.tw;
    const int tcols = min(a.tw, d - col0);
    const int CT = FCL ? 32 : a.tw >> 3;
    const int RL2 = NT / CT;
    const int c2 = tid % CT, r2 = tid / CT;
    const bool cok = (c2 << 3) < tcols;

    // Row offsets. Slot buffer: row r of slot s at s * slot_stride + r * row_plane. Row store
    // (read-through): row r of neuron u at u * bundle + r * row bytes.
    const uint32_t rowb = (uint32_t)cpr * 16u, bundle = (uint32_t)R * rowb;
    const __amdgpu_buffer_rsrc_t rs_buf = buf_rsrc(a.buf, a.buf_bytes);
    const __amdgpu_buffer_rsrc_t rs_sto = buf_rsrc(RT ? a.store : a.buf, RT ? a.store_bytes : 0u);
    // A position's slot and (read-through) source neuron, from the lists; bad entries raise an
    // error bit and read nothing.
    auto slot_of = [&](int pos, bool valid, int& src) -> int {
        const int i = min(max(pos, 0), K - 1);
        const int s = act[i];
        const int u = RT ? act_src[i] : -1;
        err |= valid && ((unsigned)s >= (unsigned)K || u >= a.M) ? kErrBadList : 0;
        src = (u >= 0 && u < a.M) ? u : -1;
        return s;
    };

    // ---------------- list loads (issued before any row load) ----------------
    int sl1[SB], sr1[SB];
    const int rl_u = CL >= 64 ? __builtin_amdgcn_readfirstlane(rl) : rl;  // uniform when a row spans waves
#pragma unroll
    for (int i = 0; i < SB; ++i) sl1[i] = slot_of(c0 + rl_u + RL * i, c0 + rl_u + RL * i < c1, sr1[i]);
    int sl2[U2], sr2[U2];
#pragma unroll
    for (int u = 0; u < U2; ++u) sl2[u] = slot_of(plo + r2 + u * RL2, r2 + u * RL2 < wn, sr2[u]);
    fv4 xr[JX][2];
#pragma unroll
    for (int j = 0; j < JX; ++j) {
        const int c = min(cl + CL * j, cpr - 1);
        xr[j][0] = reinterpret_cast<const NP_GLOBAL fv4*>(xg)[2 * c];
        xr[j][1] = reinterpret_cast<const NP_GLOBAL fv4*>(xg)[2 * c + 1];
    }

    // ---------------- phase 1 loads: gate/up rows of chunk w (issued first) ----------------
    // Offsets of row r of the position with slot s / source u, at this lane's column chunk c.
    auto off_buf = [&](bool ok, int s, int r, uint32_t colb) -> uint32_t {
        return ok && (unsigned)s < (unsigned)K ? (uint32_t)s * a.slot_stride + (uint32_t)r * a.row_plane + colb : kOOB;
    };
    auto off_sto = [&](bool ok, int u, int r, uint32_t colb) -> uint32_t {
        return ok && u >= 0 ? (uint32_t)u * bundle + (uint32_t)r * rowb + colb : kOOB;
    };
    // Row r at position pos (slot s, source u): from the row store when read-through applies,
    // else from the slot buffer. One of the two loads is out of range and returns zeros.
    auto row_load = [&](bool ok, int s, int u, int r, uint32_t cb_buf, uint32_t cb_sto) -> uint4 {
        if constexpr (RT) {
            const uint4 p = bload(rs_buf, off_buf(ok && u < 0, s, r, cb_buf));
            const uint4 q = bload(rs_sto, off_sto(ok, u, r, cb_sto));
            return make_uint4(p.x | q.x, p.y | q.y, p.z | q.z, p.w | q.w);
        } else {
            return bload(rs_buf, off_buf(ok, s, r, cb_buf));
        }
    };
    // A gate/up position is the same for every lane of a wave when a row spans whole waves: its
    // read-through source then picks one buffer for the wave, and the row takes one load.
    auto row_load_u = [&](bool ok, int s, int u, int r, uint32_t cb) -> uint4 {
        const int uu = __builtin_amdgcn_readfirstlane(u);
        const bool from_store = uu >= 0;
        const __amdgpu_buffer_rsrc_t rsel = buf_rsrc(from_store ? (const void*)a.store : (const void*)a.buf,
                                                     from_store ? a.store_bytes : a.buf_bytes);
        return bload(rsel, from_store ? off_sto(ok, uu, r, cb) : off_buf(ok, s, r, cb));
    };
    uint4 wv[SB][NR1][JX];
    auto load_batch = [&](int b0, const int* sl, const int* sr) {
#pragma unroll
        for (int i = 0; i < SB; ++i) {
            const bool ok = b0 + rl + RL * i < c1;
#pragma unroll
            for (int r = 0; r < NR1; ++r)
#pragma unroll
                for (int j = 0; j < JX; ++j) {
                    const int c = cl + CL * j;
                    if (RT && CL >= 64)
                        wv[i][r][j] = row_load_u(ok && c < cpr, sl[i], sr[i], r, (uint32_t)c * 16u);
                    else
                        wv[i][r][j] = row_load(ok && c < cpr, sl[i], sr[i], r, (uint32_t)c * 16u, (uint32_t)c * 16u);
                }
        }
    };
    // h for the batch starting at b0: dot products, reduction over the row lane, store.
    XSplit xs[JX];
    auto compute_batch = [&](int b0, const int* sl, const int* sr) {
        constexpr int V = SB * NR1;  // partial dot products per lane (a power of two <= 64)
        if constexpr (RT) {
            // read-through: the gate/up pieces of slots filled this step go into their slots
#pragma unroll
            for (int i = 0; i < SB; ++i) {
                const bool ok = b0 + rl + RL * i < c1 && sr[i] >= 0;
#pragma unroll
                for (int r = 0; r < NR1; ++r)
#pragma unroll
                    for (int j = 0; j < JX; ++j) {
                        const int c = cl + CL * j;
                        bstore(rs_buf, off_buf(ok && c < cpr, sl[i], r, (uint32_t)c * 16u), wv[i][r][j]);
                    }
            }
        }
        float v[V];
#pragma unroll
        for (int i = 0; i < SB; ++i)
#pragma unroll
            for (int r = 0; r < NR1; ++r) {
                float acc = 0.f;
                // nothing to compute for an unused position (uniform over the wave when a row
                // spans whole waves); its loads returned zeros either way
                if (b0 + rl + RL * i < c1) {
#pragma unroll
                    for (int j = 0; j < JX; ++j) acc += dot8(wv[i][r][j], xs[j]);
                }
                v[i * NR1 + r] = acc;
            }
        if (CL >= 64) {
            // Transposing butterfly over the wave: each exchange halves the values a lane
            // holds (the lane with the offset bit set keeps the upper half), so V values need
            // V - 1 + log2(64 / V) exchanges instead of 6 V; the remaining offsets sum the one
            // value left. Afterwards lane L holds the wave sum of value vi(L), vi = the lane
            // bits 5, 4, ... read as a binary number.
            static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
            auto stage = [&](auto off_c) {
                constexpr int OFF = decltype(off_c)::value;
                constexpr int M = V * OFF / 32;  // values held before this exchange (when > 1)
                if constexpr (M > 1) {
#pragma unroll
                    for (int j = 0; j < M / 2; ++j) v[j] = lane_fold<OFF>(v[j], v[j + M / 2], lane);
                } else {
                    v[0] = lane_fold<OFF>(v[0], v[0], lane);
                }
            };
            stage(std::integral_constant<int, 32>{});
            stage(std::integral_constant<int, 16>{});
            stage(std::integral_constant<int, 8>{});
            stage(std::integral_constant<int, 4>{});
            stage(std::integral_constant<int, 2>{});
            stage(std::integral_constant<int, 1>{});
            if ((lane & (64 / V - 1)) == 0) s_red1[wave * V + (lane / (64 / V))] = v[0];
            __syncthreads();
            // across the waves of each row lane: thread i of the first wave finishes position i of
            // the batch (row lane i % RL, its slot i / RL). One wave does them all: split over the
            // row lanes' first waves, the h of a chunk came out later (measured).
            if (tid < SB * RL) {
                const int rlp = tid % RL, ip = tid / RL;
                const int pos = b0 + rlp + RL * ip;
                if (pos < c1) {
                    // the CL / 64 wave sums of each row: all reads issued, then added in order
                    float part[NR1][kWaves];
#pragma unroll
                    for (int r = 0; r < NR1; ++r)
#pragma unroll
                        for (int k = 0; k < kWaves; ++k)
                            part[r][k] = k < CL / 64 ? s_red1[(rlp * (CL / 64) + k) * V + ip * NR1 + r] : 0.f;
                    float g[NR1];
#pragma unroll
                    for (int r = 0; r < NR1; ++r) {
                        float sm = 0.f;
#pragma unroll
                        for (int k = 0; k < kWaves; ++k)
                            if (k < CL / 64) sm += part[r][k];
                        g[r] = sm;
                    }
                    const float h = neuron_h(g[0], g[NR1 - 1], GATED, a.activation);
                    st_pair(&a.hpair[pos], seq, h);
                    s_h[pos - plo] = h;
                }
            }
        } else {
            // a row lane lives inside one wave: butterfly over its CL lanes
#pragma unroll
            for (int k = 0; k < V; ++k)
                for (int off = CL >> 1; off > 0; off >>= 1) v[k] += __shfl_xor(v[k], off, 64);
            if (cl == 0) {
#pragma unroll
                for (int i = 0; i < SB; ++i) {
                    const int pos = b0 + rl + RL * i;
                    if (pos < c1) {
                        const float h = neuron_h(v[i * NR1], v[i * NR1 + NR1 - 1], GATED, a.activation);
                        st_pair(&a.hpair[pos], seq, h);
                        s_h[pos - plo] = h;
                    }
                }
            }
        }
    };
    // Unconditional: a workgroup without gate/up work issues out-of-range loads, so that the
    // wait counts below are the same on every path.
    load_batch(c0, sl1, sr1);
    // Every wave issues its gate/up loads before any wave issues down loads: each SIMD issues
    // its oldest wave's loads back to back, so without this barrier the down rows of the first
    // waves queue ahead of the gate/up rows of the last ones and h waits for the whole stream.
    __syncthreads();

    // ---------------- phase 2 loads: first batch of the down tile (overlaps phase 1) -------------
    const uint32_t dcol = ((uint32_t)(col0 >> 3) + c2) * 16u;  // this lane's columns within a down row
    uint4 dv[U2];
#pragma unroll
    for (int u = 0; u < U2; ++u) dv[u] = row_load(cok && r2 + u * RL2 < wn, sl2[u], sr2[u], R - 1, dcol, dcol);


    // x as bf16 halves (a lane past the row's end holds zeros)
#pragma unroll
    for (int j = 0; j < JX; ++j) xs[j] = split_x(xr[j][0], xr[j][1], cl + CL * j < cpr);

    // ---------------- phase 1 compute: h for chunk w ----------------
    if (has1) {
        compute_batch(c0, sl1, sr1);
        for (int b0 = c0 + SB * RL; b0 < c1; b0 += SB * RL) {
            if (CL >= 64) __syncthreads();  // s_red1 is reused by this batch
            int sl[SB], sr[SB];
#pragma unroll
            for (int i = 0; i < SB; ++i) sl[i] = slot_of(b0 + rl + RL * i, b0 + rl + RL * i < c1, sr[i]);
            load_batch(b0, sl, sr);
            compute_batch(b0, sl, sr);
        }
    }

    // ---------------- phase 2: down tile t over the window ----------------
    // The window's other chunks belong to lower workgroup IDs: their h words are polled, one
    // word per thread, until they carry this launch's sequence number, and go into LDS next
    // to this workgroup's own h (if any), so the down rows then take h from LDS.
    constexpr int kStage = (kWinMax + NT - 1) / NT;
    int n_dev = n;
    {
        const int n_other = (has1 ? c0 : phi) - plo;  // positions plo .. plo + n_other - 1
        // only the lanes that cover a position poll (the others would add memory-side reads
        // while the down rows stream)
        uint64_t hp[kStage];
#pragma unroll
        for (int k = 0; k < kStage; ++k) hp[k] = tid + k * NT < n_other ? ld_pair(&a.hpair[plo + tid + k * NT]) : 0;
        if (host_n && tid == 0)
            n_dev = __hip_atomic_load(gmem(a.counts) + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (uint32_t it = 0;; ++it) {
            bool ready = true;
#pragma unroll
            for (int k = 0; k < kStage; ++k) ready &= tid + k * NT >= n_other || pair_seq(hp[k]) == seq;
            if (ready) break;
            if (it >= kSpinLimit) {
                err |= kErrSpin;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int k = 0; k < kStage; ++k)
                if (tid + k * NT < n_other && pair_seq(hp[k]) != seq) hp[k] = ld_pair(&a.hpair[plo + tid + k * NT]);
        }
#pragma unroll
        for (int k = 0; k < kStage; ++k)
            if (tid + k * NT < n_other) s_h[tid + k * NT] = pair_val(hp[k]);
        __syncthreads();
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    const int r2_first = __builtin_amdgcn_readfirstlane(r2);  // the wave's first row lane
    for (int i0 = r2;;) {
#pragma unroll
        for (int u = 0; u < U2; ++u) {
            const int i = i0 + u * RL2;
            // a position past the window has zero rows (out-of-range loads) and zero h; a wave
            // whose positions are all past it skips the work (a branch uniform over the wave)
            const float h = i < wn ? s_h[min(i, kWinMax - 1)] : 0.f;
            if (i0 - r2 + r2_first + u * RL2 < wn) axpy8(acc, h, dv[u]);
            // read-through: this tile's piece of the down row goes into its slot
            if constexpr (RT) bstore(rs_buf, off_buf(cok && i < wn && sr2[u] >= 0, sl2[u], R - 1, dcol), dv[u]);
        }
        i0 += U2 * RL2;
        if (i0 >= wn) break;
#pragma unroll
        for (int u = 0; u < U2; ++u) sl2[u] = slot_of(plo + i0 + u * RL2, i0 + u * RL2 < wn, sr2[u]);
#pragma unroll
        for (int u = 0; u < U2; ++u) dv[u] = row_load(cok && i0 + u * RL2 < wn, sl2[u], sr2[u], R - 1, dcol, dcol);
    }

    // Reduce the RL2 row lanes: column c of wave k's partial sums sits at s_red2[k * TW + swz(c)],
    // where swz keeps c's group of 8 and rotates its position in the group by (c / 32) % 8. With
    // the plain [c2 * 8 + e] the 32 lanes storing one e hit 4 banks (an 8-way conflict on every
    // store); rotated, the lanes storing one e and the lanes reading 32 consecutive columns
    // each hit 32 different banks. Thread c then sums column c (consecutive columns per wave,
    // so the atomic adds below stay coalesced).
    auto swz = [](int c) { return (c & ~7) + (((c & 7) + (c >> 5)) & 7); };
    // When a row segment is narrower than a wave (CT <= 32), the 64 / CT row lanes of a wave
    // hold the same columns (lanes l and l + CT): they are added inside the wave first (lane
    // swaps over 32 and 16 lanes, a row rotation over 8) and one row per wave goes through LDS,
    // written by the wave's first CT lanes. Otherwise each row lane (one wave at CT = 64, two
    // at CT = 128) writes its own LDS row: NT / CT rows of 8 CT columns, 8 NT floats either way.
    if (CT <= 32) {  // uniform over the workgroup
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = lane_fold<32>(acc[e], acc[e], lane);
        if (CT <= 16) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = lane_fold<16>(acc[e], acc[e], lane);
        }
        if (CT <= 8) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = lane_fold<8>(acc[e], acc[e], lane);
        }
    }
    const int lds_rows = CT >= 64 ? RL2 : kWaves;
    if (CT >= 64 || lane < CT) {
        const int row = CT >= 64 ? r2 : wave;
#pragma unroll
        for (int e = 0; e < 8; ++e) s_red2[row * a.tw + swz((c2 << 3) + e)] = acc[e];
    }
    __syncthreads();
    const int mycol = tid;
    const bool colok = tid < tcols;

    const int ncontrib = (a.nwg - 1 - t) / a.q + 1;
    const bool reducer = !a.atomic_y && w == t + a.q * (ncontrib - 1);
    float own = 0.f;                          // this workgroup's partial of column tid (tid < tcols)
    if (colok) {
        const int sc = swz(tid);
        // the LDS rows, the reads issued together, added in row order
        float pr[kWaves];
#pragma unroll
        for (int k = 0; k < kWaves; ++k) pr[k] = k < lds_rows ? s_red2[k * a.tw + sc] : 0.f;
#pragma unroll
        for (int k = 0; k < kWaves; ++k)
            if (k < lds_rows) own += pr[k];
        if (a.atomic_y) {
            // Atomic reduction: every contributor adds its partial into y (cleared before the
            // launch or holding the value to add to). No exchange, no reducer; the order of
            // the additions, and so the last bits of y, may differ from run to run.
            float* yp = a.prm ? a.prm->y + (size_t)a.layer * a.d : a.y;
            unsafeAtomicAdd(yp + col0 + mycol, own);
        } else if (!reducer) {
            st_pair(&a.ppair[(size_t)w * a.tw + tid], seq, own);
        }
    }
    if (reducer) {
        // The tile's highest contributor sums the other contributors' partials: G groups of
        // threads per column each take contributors g, g + G, ... (ascending), then the group
        // sums and this workgroup's own partial are added in a fixed order.
        // Every thread polls the partial words it sums.
        __syncthreads();                      // s_red2 is reused for the group sums
        const int G = NT / a.tw;
        const int j = tid % a.tw, g = tid / a.tw;
        constexpr int kB = 8;
        float gs = 0.f;
        if (j < tcols) {
            for (int k0 = g; k0 < ncontrib - 1; k0 += kB * G) {
                uint64_t pp[kB];
#pragma unroll
                for (int k = 0; k < kB; ++k) {
                    const int kk = k0 + k * G;
                    pp[k] = kk < ncontrib - 1 ? ld_pair(&a.ppair[(size_t)(t + kk * a.q) * a.tw + j]) : (uint64_t)seq;
                }
                for (uint32_t it = 0;; ++it) {
                    bool ready = true;
#pragma unroll
                    for (int k = 0; k < kB; ++k) ready &= pair_seq(pp[k]) == seq;
                    if (ready) break;
                    if (it >= kSpinLimit) {
                        err |= kErrSpin;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
#pragma unroll
                    for (int k = 0; k < kB; ++k)
                        if (pair_seq(pp[k]) != seq)
                            pp[k] = ld_pair(&a.ppair[(size_t)(t + (k0 + k * G) * a.q) * a.tw + j]);
                }
#pragma unroll
                for (int k = 0; k < kB; ++k)
                    if (k0 + k * G < ncontrib - 1) gs += pair_val(pp[k]);
            }
        }
        s_red2[g * a.tw + j] = gs;
        __syncthreads();
        if (colok) {
            float yv = 0.f;
            for (int gg = 0; gg < G; ++gg) yv += s_red2[gg * a.tw + tid];
            auto* yg = gmem(a.prm ? gmem(a.prm)->y + (size_t)a.layer * a.d : a.y);
            const float y0 = a.accumulate ? yg[col0 + mycol] : 0.f;
            yg[col0 + mycol] = a.accumulate ? y0 + (yv + own) : yv + own;
        }
    }
    if (n_dev != n) err |= kErrCount;
    if (err) raise_err(a.counts, err);
    if constexpr (TOK) {
        // This workgroup of the layer's FFN is done (its stores have completed): the next
        // layer's FFN counts them. The next layer reads nothing this one wrote, so the count
        // orders the layers without a release (which would write the whole L2 back).
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) __hip_atomic_fetch_add(gmem(a.counts) + kFfnDoneSlot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int NT, int JX, bool G, int FCL>
hipError_t launch_k(const FfnArgs& a, const FfnShape& sh, hipStream_t s) {
    // Slots per row lane per phase-1 batch and down rows per lane per phase-2 batch,
    // sized so that about five slots per workgroup take one batch each.
    constexpr int SB = 4;
    constexpr int U2 = NT >= 1024 ? 4 : (NT >= 512 ? 6 : 12);
    const dim3 grid(sh.nwg + a.pf_wgs), block(NT);
    if (a.tok) {  // sh.nwg: the token's whole grid
        hipLaunchKernelGGL((k_sparse_ffn<NT, JX, G, SB, U2, false, false, true, FCL>), dim3(sh.nwg), block, 0, s, a);
    } else if (a.pf_wgs > 0) {
        if (a.read_through)
            hipLaunchKernelGGL((k_sparse_ffn<NT, JX, G, SB, U2, true, true, false, FCL>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((k_sparse_ffn<NT, JX, G, SB, U2, false, true, false, FCL>), grid, block, 0, s, a);
    } else if (a.read_through) {
        hipLaunchKernelGGL((k_sparse_ffn<NT, JX, G, SB, U2, true, false, false, FCL>), grid, block, 0, s, a);
    } else {
        hipLaunchKernelGGL((k_sparse_ffn<NT, JX, G, SB, U2, false, false, false, FCL>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

// The compiled lane geometry (rows of 512 lanes, 256-column tiles) for the shapes that have
// it: d_model 4096 with 1024 threads, and d_model above 4096 (up to 8192) with 512.
template <int NT, int JX, bool G>
hipError_t launch_t(const FfnArgs& a, const FfnShape& sh, hipStream_t s) {
    if constexpr ((NT == 1024 && JX == 1) || (NT == 512 && JX == 2)) {
        if (sh.fixed) return launch_k<NT, JX, G, 512>(a, sh, s);
    }
    return launch_k<NT, JX, G, 0>(a, sh, s);
}

template <int NT, bool G>
hipError_t launch_jx(const FfnArgs& a, const FfnShape& sh, hipStream_t s) {
    if (sh.jx == 1) return launch_t<NT, 1, G>(a, sh, s);
    if constexpr (NT < 1024) {  // 1024-thread workgroups hold one x chunk per lane
        switch (sh.jx) {
            case 2: return launch_t<NT, 2, G>(a, sh, s);
            case 3: return launch_t<NT, 3, G>(a, sh, s);
            case 4: return launch_t<NT, 4, G>(a, sh, s);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_sparse_ffn(const FfnArgs& a, const FfnShape& sh, bool gated, hipStream_t s) {
    if (sh.nt == 256) return gated ? launch_jx<256, true>(a, sh, s) : launch_jx<256, false>(a, sh, s);
    if (sh.nt == 512) return gated ? launch_jx<512, true>(a, sh, s) : launch_jx<512, false>(a, sh, s);
    if (sh.nt == 1024) return gated ? launch_jx<1024, true>(a, sh, s) : launch_jx<1024, false>(a, sh, s);
    return hipErrorInvalidValue;
}

hipError_t launch_token(const TokenArgs* ta, int grid, const FfnShape& sh, bool gated, hipStream_t s) {
    FfnArgs a{};
    a.tok = ta;
    FfnShape g = sh;
    g.nwg = grid;
    return launch_sparse_ffn(a, g, gated, s);
}

int ffn_win_max() { return kWinMax; }

}  // namespace np
