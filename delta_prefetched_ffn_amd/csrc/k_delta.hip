// Delta assignment for gfx950: active-set decode, set difference, slot release and
// deterministic slot assignment for every sparse layer of a decode step, one
// workgroup per layer (NeuroPrefetcher, section 3.4: the predicted active set
// comes from the gate and up centroid masks; the resident buffer is updated by
// set difference; outgoing rows release slots; incoming rows take freed slots;
// the slot map holds -1 for non-resident neurons; no compaction).
//
// All set state lives in LDS as 64-bit words (bit b of word w = neuron 64w+b).
// Ascending lists come from per-thread contiguous word ranges plus a
// workgroup-wide exclusive scan of popcounts, so the order is the ascending
// bit order regardless of how many lanes run.
#include "np_internal.hpp"

namespace np {
namespace {

constexpr int kNT = 256;
constexpr int kWaves = kNT / 64;

// Exclusive scan of one int per thread over the workgroup; *total gets the sum.
__device__ int block_excl_scan(int v, int* total, int* s_tmp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_tmp[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int w = 0; w < kWaves; ++w) {
            int t = s_tmp[w];
            s_tmp[w] = acc;
            acc += t;
        }
        s_tmp[kWaves] = acc;
    }
    __syncthreads();
    const int res = s_tmp[wave] + x - v;
    *total = s_tmp[kWaves];
    __syncthreads();
    return res;
}

__device__ inline uint64_t drop_low_bits(uint64_t w, int r) {
    for (int j = 0; j < r; ++j) w &= w - 1;
    return w;
}

constexpr int kOwnRegs = 32;  // owner entries per thread loaded with the masks (K <= 8192 in one pass)

__global__ __launch_bounds__(kNT) void k_delta_assign(DeltaLaunch a) {
    __shared__ uint64_t s_S[kMaxWords];
    __shared__ uint64_t s_R[kMaxWords];
    __shared__ uint64_t s_Fa[kMaxKWords];  // free slots before this step
    __shared__ uint64_t s_F0[kMaxKWords];  // free slots after the release
    __shared__ uint64_t s_F1[kMaxKWords];  // free slots after the assignment
    __shared__ int s_fpre[kMaxKWords];     // exclusive prefix of |F0| per word
    __shared__ int s_opre[kMaxKWords];     // exclusive prefix of occupied slots per word
    __shared__ int s_tmp[kWaves + 1];
    __shared__ int s_err;

    const LayerDev L = *a.layers[blockIdx.x];
    auto* const owner = gmem(L.owner);
    auto* const slot_map = gmem(L.slot_map);
    auto* const d_in = gmem(L.d_in);
    auto* const slot_in = gmem(L.slot_in);
    auto* const d_out = gmem(L.d_out);
    auto* const act = gmem(L.act);
    auto* const act_src = gmem(L.act_src);
    auto* const res = gmem(L.res);
    auto* const freeb = gmem(L.freeb);
    auto* const counts = gmem(L.counts);
    const int tid = threadIdx.x;
    if (tid == 0) s_err = 0;
    const int32_t cg = a.prm ? gmem(a.prm)->cid[a.layer0 + blockIdx.x][0] : a.cid[blockIdx.x][0];
    const int32_t cu = a.prm ? gmem(a.prm)->cid[a.layer0 + blockIdx.x][1] : a.cid[blockIdx.x][1];

    // Step 1: active set S from the selected gate/up masks; R from the resident bits. The
    // owner table (slot -> neuron) is read in the same round trip: it drives the release.
    const auto* ma = gmem(L.masks) + (size_t)cg * L.W;
    const auto* mb = gmem(L.masks) + ((size_t)(L.n_tables - 1) * L.C + cu) * L.W;
    int own[kOwnRegs];
#pragma unroll
    for (int k = 0; k < kOwnRegs; ++k) {
        const int sl = tid + k * kNT;
        own[k] = sl < L.K ? owner[sl] : -1;
    }
    for (int w = tid; w < L.W; w += kNT) {
        const uint64_t ga = ma[w], gb = mb[w];
        s_S[w] = L.mode == 0 ? (ga | gb) : L.mode == 1 ? (ga & gb) : ga;
        s_R[w] = res[w];
    }
    for (int v = tid; v < L.Kw; v += kNT) s_Fa[v] = s_F0[v] = freeb[v];
    __syncthreads();

    // Step 2: |D_in| and |D_out| per contiguous word range, scanned for list offsets;
    // D_out is written in ascending order.
    const int wpt = (L.W + kNT - 1) / kNT;
    const int w0 = min(tid * wpt, L.W), w1 = min(w0 + wpt, L.W);
    int c_in = 0, c_out = 0;
    for (int w = w0; w < w1; ++w) {
        c_in += __popcll(s_S[w] & ~s_R[w]);
        c_out += __popcll(s_R[w] & ~s_S[w]);
    }
    int n_in, n_out;
    const int base_in = block_excl_scan(c_in, &n_in, s_tmp);
    const int base_out = block_excl_scan(c_out, &n_out, s_tmp);
    {
        int k = base_out;
        for (int w = w0; w < w1; ++w) {
            uint64_t bits = s_R[w] & ~s_S[w];
            while (bits) {
                d_out[k++] = w * 64 + (__ffsll((unsigned long long)bits) - 1);
                bits &= bits - 1;
            }
        }
    }

    // Step 3: release the slots whose owner leaves the active set (slot map -1, free bit;
    // the owner entry is cleared below unless the slot is taken again). Every slot is
    // looked at once, so the owners of D_out are found without a slot-map lookup each.
    auto release = [&](int sl, int n) {
        if (n < 0) return 0;
        if (n >= L.M) {
            atomicOr(&s_err, kErrBadList);
            return 0;
        }
        const uint64_t bit = 1ull << (n & 63);
        if ((s_R[n >> 6] & bit) == 0) {  // an owned slot must belong to a resident neuron
            atomicOr(&s_err, kErrBadList);
            return 0;
        }
        if (s_S[n >> 6] & bit) return 0;  // stays resident
        slot_map[n] = -1;
        atomicOr((unsigned long long*)&s_F0[sl >> 6], 1ull << (sl & 63));
        return 1;
    };
    int c_rel = 0;
#pragma unroll
    for (int k = 0; k < kOwnRegs; ++k) c_rel += release(tid + k * kNT, own[k]);
    for (int sl = tid + kOwnRegs * kNT; sl < L.K; sl += kNT) c_rel += release(sl, owner[sl]);
    int n_rel;
    (void)block_excl_scan(c_rel, &n_rel, s_tmp);  // also orders the releases before what follows
    if (tid == 0 && n_rel != n_out) atomicOr(&s_err, kErrBadList);

    // Free slots after the release: per-word prefix counts (ascending slot order).
    const int kpt = (L.Kw + kNT - 1) / kNT;
    const int v0 = min(tid * kpt, L.Kw), v1 = min(v0 + kpt, L.Kw);
    int c_free = 0;
    for (int v = v0; v < v1; ++v) c_free += __popcll(s_F0[v]);
    int n_free;
    {
        int pre = block_excl_scan(c_free, &n_free, s_tmp);
        for (int v = v0; v < v1; ++v) {
            s_fpre[v] = pre;
            pre += __popcll(s_F0[v]);
        }
    }
    // Step 4 (set part): the n_in lowest free slots are taken; occupied slots per word.
    int c_occ = 0;
    for (int v = v0; v < v1; ++v) {
        const int take = min(max(n_in - s_fpre[v], 0), __popcll(s_F0[v]));
        const uint64_t fw = drop_low_bits(s_F0[v], take);
        s_F1[v] = fw;
        freeb[v] = fw;
        uint64_t gone = s_F0[v] & ~s_Fa[v] & fw;  // released and not taken again: no owner
        while (gone) {
            owner[v * 64 + __ffsll((unsigned long long)gone) - 1] = -1;
            gone &= gone - 1;
        }
        const uint64_t valid = (v == L.Kw - 1 && (L.K & 63)) ? ((1ull << (L.K & 63)) - 1) : ~0ull;
        c_occ += __popcll(~fw & valid);
    }
    int n_act;
    {
        int pre = block_excl_scan(c_occ, &n_act, s_tmp);  // the barrier inside publishes s_fpre, s_F1
        for (int v = v0; v < v1; ++v) {
            s_opre[v] = pre;
            const uint64_t valid = (v == L.Kw - 1 && (L.K & 63)) ? ((1ull << (L.K & 63)) - 1) : ~0ull;
            pre += __popcll(~s_F1[v] & valid);
        }
    }
    __syncthreads();

    // Step 4 (lists): the i-th incoming neuron (ascending) takes the i-th free slot
    // (ascending). Its position in the ascending occupied-slot list gets the neuron ID in
    // act_src, so that the FFN can read the new bundle where it still is (the row store).
    {
        int k = base_in;
        for (int w = w0; w < w1; ++w) {
            uint64_t bits = s_S[w] & ~s_R[w];
            while (bits) {
                const int n = w * 64 + (__ffsll((unsigned long long)bits) - 1);
                bits &= bits - 1;
                const int idx = k++;
                if (idx >= n_free) {
                    atomicOr(&s_err, kErrFreeExhausted);
                    continue;
                }
                int lo = 0, hi = L.Kw - 1;  // last word whose prefix is <= idx
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (s_fpre[mid] <= idx) lo = mid; else hi = mid - 1;
                }
                const uint64_t fw = drop_low_bits(s_F0[lo], idx - s_fpre[lo]);
                const int slot = lo * 64 + (__ffsll((unsigned long long)fw) - 1);
                const uint64_t below = (1ull << (slot & 63)) - 1;
                const int pos = s_opre[lo] + __popcll(~s_F1[lo] & below);
                d_in[idx] = n;
                slot_in[idx] = slot;
                slot_map[n] = slot;
                owner[slot] = n;
                act_src[pos] = n;
            }
        }
    }
    // Occupied slots in ascending order; slots kept from the last step have act_src -1.
    for (int v = v0; v < v1; ++v) {
        const uint64_t valid = (v == L.Kw - 1 && (L.K & 63)) ? ((1ull << (L.K & 63)) - 1) : ~0ull;
        const uint64_t taken = s_F0[v] & ~s_F1[v];
        uint64_t occ = ~s_F1[v] & valid;
        int o = s_opre[v];
        while (occ) {
            const int b = __ffsll((unsigned long long)occ) - 1;
            occ &= occ - 1;
            act[o] = v * 64 + b;
            if (!((taken >> b) & 1)) act_src[o] = -1;
            ++o;
        }
    }

    // Step 5: R = S.
    for (int w = tid; w < L.W; w += kNT) res[w] = s_S[w];
    __syncthreads();
    if (tid == 0) {
        counts[0] = n_in;
        counts[1] = n_out;
        counts[2] = n_act;
        if (s_err) atomicOr(&L.counts[3], s_err);
    }
}

__global__ void k_set_params(ParamsUpdate p, DecodeParams* dst) {
    for (int i = threadIdx.x; i < p.count; i += blockDim.x) {
        dst->cid[p.first + i][0] = p.cid[i][0];
        dst->cid[p.first + i][1] = p.cid[i][1];
        dst->seq[p.first + i] = p.seq[i];
    }
    if (threadIdx.x == 0 && p.first == 0) {
        dst->x = p.x;
        dst->y = p.y;
    }
}

}  // namespace

hipError_t launch_set_params(const ParamsUpdate& p, DecodeParams* dst, hipStream_t s) {
    hipLaunchKernelGGL(k_set_params, dim3(1), dim3(128), 0, s, p, dst);
    return hipGetLastError();
}

hipError_t launch_delta_assign(const DeltaLaunch& a, hipStream_t s) {
    hipLaunchKernelGGL(k_delta_assign, dim3(a.n_layers), dim3(kNT), 0, s, a);
    return hipGetLastError();
}

}  // namespace np
