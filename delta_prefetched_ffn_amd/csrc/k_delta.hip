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

__global__ __launch_bounds__(kNT) void k_delta_assign(DeltaLaunch a) {
    __shared__ uint64_t s_S[kMaxWords];
    __shared__ uint64_t s_R[kMaxWords];
    __shared__ uint64_t s_free[kMaxKWords];
    __shared__ int s_fpre[kMaxKWords];
    __shared__ int s_tmp[kWaves + 1];
    __shared__ int s_err;

    const LayerDev L = *a.layers[blockIdx.x];
    const int tid = threadIdx.x;
    if (tid == 0) s_err = 0;
    const int32_t cg = a.prm ? a.prm->cid[a.layer0 + blockIdx.x][0] : a.cid[blockIdx.x][0];
    const int32_t cu = a.prm ? a.prm->cid[a.layer0 + blockIdx.x][1] : a.cid[blockIdx.x][1];

    // Step 1: active set S from the selected gate/up masks; R from the resident bits.
    const uint64_t* ma = L.masks + (size_t)cg * L.W;
    const uint64_t* mb = L.masks + ((size_t)(L.n_tables - 1) * L.C + cu) * L.W;
    for (int w = tid; w < L.W; w += kNT) {
        const uint64_t ga = ma[w], gb = mb[w];
        s_S[w] = L.mode == 0 ? (ga | gb) : L.mode == 1 ? (ga & gb) : ga;
        s_R[w] = L.res[w];
    }
    for (int v = tid; v < L.Kw; v += kNT) s_free[v] = L.freeb[v];
    __syncthreads();

    // Step 2: |D_in| and |D_out| per contiguous word range, scanned for list offsets.
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

    // Step 3: D_out in ascending order; release its slots (owner -1, slot map -1, free bit).
    int k = base_out;
    for (int w = w0; w < w1; ++w) {
        uint64_t bits = s_R[w] & ~s_S[w];
        while (bits) {
            const int n = w * 64 + (__ffsll((unsigned long long)bits) - 1);
            bits &= bits - 1;
            L.d_out[k++] = n;
            const int s = L.slot_map[n];
            if ((unsigned)s < (unsigned)L.K) {
                L.owner[s] = -1;
                atomicOr((unsigned long long*)&s_free[s >> 6], 1ull << (s & 63));
            } else {
                atomicOr(&s_err, kErrBadList);
            }
            L.slot_map[n] = -1;
        }
    }
    __syncthreads();

    // Free slots after the release: per-word prefix counts (ascending slot order).
    const int kpt = (L.Kw + kNT - 1) / kNT;
    const int v0 = min(tid * kpt, L.Kw), v1 = min(v0 + kpt, L.Kw);
    int c_free = 0;
    for (int v = v0; v < v1; ++v) c_free += __popcll(s_free[v]);
    int n_free;
    int pre = block_excl_scan(c_free, &n_free, s_tmp);
    for (int v = v0; v < v1; ++v) {
        s_fpre[v] = pre;
        pre += __popcll(s_free[v]);
    }
    __syncthreads();

    // Step 4: the i-th incoming neuron (ascending) takes the i-th free slot (ascending).
    k = base_in;
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
            const uint64_t fw = drop_low_bits(s_free[lo], idx - s_fpre[lo]);
            const int slot = lo * 64 + (__ffsll((unsigned long long)fw) - 1);
            L.d_in[idx] = n;
            L.slot_in[idx] = slot;
            L.slot_map[n] = slot;
            L.owner[slot] = n;
        }
    }
    __syncthreads();

    // Taken slots leave the free set; occupied slots are listed in ascending order.
    int c_occ = 0;
    for (int v = v0; v < v1; ++v) {
        const int take = min(max(n_in - s_fpre[v], 0), __popcll(s_free[v]));
        const uint64_t fw = drop_low_bits(s_free[v], take);
        s_free[v] = fw;
        L.freeb[v] = fw;
        const uint64_t valid = (v == L.Kw - 1 && (L.K & 63)) ? ((1ull << (L.K & 63)) - 1) : ~0ull;
        c_occ += __popcll(~fw & valid);
    }
    int n_act;
    int o = block_excl_scan(c_occ, &n_act, s_tmp);
    for (int v = v0; v < v1; ++v) {
        const uint64_t valid = (v == L.Kw - 1 && (L.K & 63)) ? ((1ull << (L.K & 63)) - 1) : ~0ull;
        uint64_t occ = ~s_free[v] & valid;
        while (occ) {
            L.act[o++] = v * 64 + (__ffsll((unsigned long long)occ) - 1);
            occ &= occ - 1;
        }
    }

    // Step 5: R = S.
    for (int w = tid; w < L.W; w += kNT) L.res[w] = s_S[w];
    __syncthreads();
    if (tid == 0) {
        L.counts[0] = n_in;
        L.counts[1] = n_out;
        L.counts[2] = n_act;
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
