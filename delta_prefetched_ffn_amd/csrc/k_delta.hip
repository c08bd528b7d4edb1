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

constexpr int kNT = 512;
constexpr int kWaves = kNT / 64;

// Exclusive scans of two ints per thread over the workgroup in one pass; *ta and *tb get
// the sums.
__device__ inline void block_excl_scan2(int va, int vb, int* ea, int* eb, int* ta, int* tb, int* s_tmp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int xa = va, xb = vb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int ya = __shfl_up(xa, off, 64), yb = __shfl_up(xb, off, 64);
        if (lane >= off) {
            xa += ya;
            xb += yb;
        }
    }
    if (lane == 63) {
        s_tmp[2 * wave] = xa;
        s_tmp[2 * wave + 1] = xb;
    }
    __syncthreads();
    int pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int wa = s_tmp[2 * w], wb = s_tmp[2 * w + 1];
        if (w < wave) {
            pa += wa;
            pb += wb;
        }
        sa += wa;
        sb += wb;
    }
    *ea = pa + xa - va;
    *eb = pb + xb - vb;
    *ta = sa;
    *tb = sb;
    __syncthreads();  // s_tmp may be reused right away
}

// Sum of v over the 64 lanes of a wave, in every lane, without LDS: halves exchanged by the
// gfx950 lane-swap instructions, then row rotation, half-row mirror and quad permutations.
// The whole wave must be active. (Adding per-thread values into one LDS word with atomics
// instead serialises one read-modify-write per thread.)
__device__ inline int wave_sum_i(int v) {
    const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = (int)r32[0] + (int)r32[1];
    const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = (int)r16[0] + (int)r16[1];
    v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // lane ^ 8 within a row
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // lane i <-> 7 - i
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // lane ^ 2
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // lane ^ 1
    return v;
}

// w with its r lowest set bits removed (r >= popcount(w) gives 0): finds the r-th set bit
// (0-based) by halving the word six times, then clears everything below it.
__device__ inline uint64_t drop_low_bits(uint64_t w, int r) {
    if (r <= 0) return w;
    if (r >= (int)__popcll(w)) return 0;
    int pos = 0;
    uint64_t x = w;
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) {
        const int c = __popcll(x & ((1ull << sh) - 1));
        if (r >= c) {
            r -= c;
            x >>= sh;
            pos += sh;
        }
    }
    return w & ~((1ull << pos) - 1);
}

__device__ inline uint64_t valid_bits(int v, int Kw, int K) {
    return (v == Kw - 1 && (K & 63)) ? ((1ull << (K & 63)) - 1) : ~0ull;
}

constexpr int kOwnRegs = 16;  // owner entries per thread loaded with the masks (K <= 8192 in one pass)

// Bits of the positions below lim in word v.
__device__ inline uint64_t below(int v, int lim) {
    const int b = lim - v * 64;
    return b <= 0 ? 0ull : (b >= 64 ? ~0ull : ((1ull << b) - 1));
}

// Steps 3-4 of the compacted layout (LLM in a flash, section 3.3: the occupied rows form the
// prefix 0 .. n-1; a leaving row is replaced by a row from the end of the region; incoming
// rows are appended). On entry the leaving neurons' slot-map entries are -1 and their
// positions are set in s_F0 (s_Fa: the positions free before this step, i.e. n_occ and up).
// With n_keep = n_occ - |D_out|, the holes (leaving positions below n_keep, ascending) take
// the staying rows at n_keep and up in descending order (the move list, applied to the bytes
// by a copy kernel before the FFN), and the k-th incoming neuron goes to n_keep + k.
// Returns |S| (the rows 0 .. |S|-1 the FFN reads).
__device__ int compact_assign(const LayerDev& L, int n_in, int n_out, int base_in, int w0, int w1, int v0, int v1,
                              const uint64_t* s_S, const uint64_t* s_R, const uint64_t* s_Fa,
                              const uint64_t* s_F0, int* s_mpre, int* s_tmp, int* s_err) {
    const int tid = threadIdx.x, K = L.K, Kw = L.Kw;
    auto* const owner = gmem(L.owner);
    auto* const slot_map = gmem(L.slot_map);
    int c_fa = 0;
    for (int v = v0; v < v1; ++v) c_fa += __popcll(s_Fa[v]);
    int e_a, e_b, n_free0, unused;
    block_excl_scan2(c_fa, 0, &e_a, &e_b, &n_free0, &unused, s_tmp);
    const int n_occ = K - n_free0, n_keep = n_occ - n_out;
    auto holes = [&](int v) { return s_F0[v] & ~s_Fa[v] & below(v, n_keep); };
    auto movers = [&](int v) { return ~s_F0[v] & below(v, n_occ) & ~below(v, n_keep); };
    int c_h = 0, c_m = 0;
    for (int v = v0; v < v1; ++v) {
        c_h += __popcll(holes(v));
        c_m += __popcll(movers(v));
    }
    int pre_h, pre_m, n_h, n_m;
    block_excl_scan2(c_h, c_m, &pre_h, &pre_m, &n_h, &n_m, s_tmp);
    if (tid == 0 && (n_h != n_m || n_keep < 0)) atomicOr(s_err, kErrBadList);
    for (int v = v0; v < v1; ++v) {
        s_mpre[v] = pre_m;
        pre_m += __popcll(movers(v));
    }
    __syncthreads();
    // hole of ascending rank i <- mover of ascending rank n_m - 1 - i
    {
        int i = pre_h;
        for (int v = v0; v < v1; ++v) {
            uint64_t H = holes(v);
            while (H) {
                const int h = v * 64 + __ffsll((unsigned long long)H) - 1;
                H &= H - 1;
                const int j = n_m - 1 - i;
                if (j >= 0) {
                    int l0 = 0, h0 = Kw - 1;  // last word whose mover prefix is <= j
                    while (l0 < h0) {
                        const int mid = (l0 + h0 + 1) >> 1;
                        if (s_mpre[mid] <= j) l0 = mid; else h0 = mid - 1;
                    }
                    const uint64_t rest = drop_low_bits(movers(l0), j - s_mpre[l0]);
                    if (rest == 0) {  // only with an inconsistent state
                        atomicOr(s_err, kErrBadList);
                        ++i;
                        continue;
                    }
                    const int m = l0 * 64 + __ffsll((unsigned long long)rest) - 1;
                    const int nm = owner[m];
                    gmem(L.mv_src)[i] = m;
                    gmem(L.mv_dst)[i] = h;
                    owner[h] = nm;
                    if ((unsigned)nm < (unsigned)L.M) slot_map[nm] = h;
                    else atomicOr(s_err, kErrBadList);
                }
                ++i;
            }
        }
    }
    __syncthreads();  // every mover's owner entry has been read
    const int n_act = min(max(n_keep + n_in, 0), K);
    {
        int idx = base_in;
        for (int w = w0; w < w1; ++w) {
            uint64_t bits = s_S[w] & ~s_R[w];
            while (bits) {
                const int n = w * 64 + (__ffsll((unsigned long long)bits) - 1);
                bits &= bits - 1;
                const int pos = n_keep + idx;
                if (pos < 0 || pos >= K) {
                    atomicOr(s_err, kErrFreeExhausted);
                } else {
                    gmem(L.slot_in)[idx] = pos;
                    slot_map[n] = pos;
                    owner[pos] = n;
                    gmem(L.act_src)[pos] = n;
                }
                ++idx;
            }
        }
    }
    for (int p = max(n_act, 0) + tid; p < n_occ; p += kNT) owner[p] = -1;
    for (int p = tid; p < n_act; p += kNT) {
        gmem(L.act)[p] = p;
        if (p < n_keep) gmem(L.act_src)[p] = -1;
    }
    for (int v = tid; v < Kw; v += kNT) gmem(L.freeb)[v] = valid_bits(v, Kw, K) & ~below(v, n_act);
    if (tid == 0) gmem(L.counts)[5] = n_h;
    return n_act;
}

__global__ __launch_bounds__(kNT) void k_delta_assign(DeltaLaunch a) {
    __shared__ uint64_t s_S[kMaxWords];
    __shared__ uint64_t s_R[kMaxWords];
    __shared__ uint64_t s_Fa[kMaxKWords];  // free slots before this step
    __shared__ uint64_t s_F0[kMaxKWords];  // free slots after the release
    __shared__ uint64_t s_F1[kMaxKWords];  // free slots after the assignment
    __shared__ int s_fpre[kMaxKWords];     // exclusive prefix of |F0| per word
    __shared__ int s_opre[kMaxKWords];     // exclusive prefix of active slots per word
    __shared__ uint64_t s_Rn[kMaxWords];   // the new resident set R_t
    __shared__ uint64_t s_Ab[kMaxKWords];  // slots holding an active neuron (the FFN's list)
    __shared__ int s_cnt[kMaxClasses + 1]; // retained candidates per class (age or level)
    __shared__ int s_nS, s_jstar, s_allow;
    __shared__ int s_tmp[2 * kWaves];
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
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int M = L.M, K = L.K, W = L.W, Kw = L.Kw;
    if (tid == 0) {
        s_err = 0;
        s_nS = 0;
    }
    if (tid <= kMaxClasses) s_cnt[tid] = 0;
    const int win = L.window;
    const int tok = counts[4];  // tokens assigned before this one
    const int32_t cg = a.prm ? gmem(a.prm)->cid[a.layer0 + blockIdx.x][0] : a.cid[blockIdx.x][0];
    const int32_t cu = a.prm ? gmem(a.prm)->cid[a.layer0 + blockIdx.x][1] : a.cid[blockIdx.x][1];

    // Step 1: active set S from the selected gate/up masks; R from the resident bits. The
    // owner table (slot -> neuron) is read in the same round trip: it drives the release.
    const auto* ma = gmem(L.masks) + (size_t)cg * W;
    const auto* mb = gmem(L.masks) + ((size_t)(L.n_tables - 1) * L.C + cu) * W;
    int own[kOwnRegs];
#pragma unroll
    for (int k = 0; k < kOwnRegs; ++k) own[k] = owner[min(tid + k * kNT, K - 1)];
    for (int w = tid; w < W; w += kNT) {
        const uint64_t ga = ma[w], gb = mb[w];
        s_S[w] = L.mode == 0 ? (ga | gb) : L.mode == 1 ? (ga & gb) : ga;
        s_R[w] = res[w];
    }
    for (int v = tid; v < Kw; v += kNT) {
        s_Fa[v] = s_F0[v] = freeb[v];
        s_Ab[v] = 0;
    }
    __syncthreads();

    // Step 1b: the resident set R_t this token moves to. Exactly S (section 3.4), or S plus
    // resident neurons of retention classes j = 1, 2, ..., taken class by class and by
    // ascending ID within a class while |R_t| <= K:
    //   * window of k tokens (LLM in a flash, section 3.1): class j = last active j tokens ago
    //     (1 <= j < k). The active sets of the last k-1 tokens are kept as bit masks in a
    //     ring, so the class of a neuron is the first earlier mask that holds it;
    //   * frequency levels (DynamicInfer, key design 2: importance a + lambda f, every active
    //     neuron resident): class j = the j-th highest level, from static per-level masks.
    const int wpt = (W + kNT - 1) / kNT;
    const int w0 = min(tid * wpt, W), w1 = min(w0 + wpt, W);
    const bool by_level = L.n_levels > 0;
    if (win > 1 || by_level) {
        const auto* ring = gmem(L.ring);
        const auto* lvl = gmem(L.levels);
        const int nj = by_level ? L.n_levels : min(win - 1, tok);  // classes that exist
        auto ring_word = [&](int j, int w) -> uint64_t {
            return by_level ? lvl[(size_t)(j - 1) * W + w] : ring[(size_t)((tok - j) % (win - 1)) * W + w];
        };
        int cnt[kMaxClasses + 1];
#pragma unroll
        for (int j = 0; j <= kMaxClasses; ++j) cnt[j] = 0;
        int c_s = 0;
        for (int w = w0; w < w1; ++w) {
            const uint64_t base = s_R[w] & ~s_S[w];
            uint64_t covered = 0;
            c_s += __popcll(s_S[w]);
#pragma unroll
            for (int j = 1; j <= kMaxClasses; ++j) {  // guarded, not left with a break: it unrolls,
                if (j <= nj) {                        // so cnt[] stays in registers
                    const uint64_t A = ring_word(j, w);
                    cnt[j] += __popcll(A & base & ~covered);
                    covered |= A;
                }
            }
        }
        // per-wave sums, then one LDS add per wave
        const int ws = wave_sum_i(c_s);
        if (lane == 0) atomicAdd(&s_nS, ws);
#pragma unroll
        for (int j = 1; j <= kMaxClasses; ++j) {
            if (j <= nj) {  // nj is the same for the whole workgroup
                const int wc = wave_sum_i(cnt[j]);
                if (lane == 0 && wc) atomicAdd(&s_cnt[j], wc);
            }
        }
        __syncthreads();
        if (tid == 0) {
            int room = K - s_nS, js = kMaxClasses + 1, allow = 0;
            for (int j = 1; j <= nj; ++j) {
                if (s_cnt[j] <= room) {
                    room -= s_cnt[j];
                } else {
                    js = j;
                    allow = room;
                    break;
                }
            }
            s_jstar = js;
            s_allow = allow;
        }
        __syncthreads();
        const int js = s_jstar, allow = s_allow;
        // the cut age class keeps its lowest IDs: a workgroup scan of its per-thread counts
        int c_cut = 0;
        if (js <= nj)
            for (int w = w0; w < w1; ++w) {
                const uint64_t base = s_R[w] & ~s_S[w];
                uint64_t covered = 0;
                for (int j = 1; j <= js; ++j) {
                    const uint64_t A = ring_word(j, w);
                    if (j == js) c_cut += __popcll(A & base & ~covered);
                    covered |= A;
                }
            }
        int pre_cut, unused_e, unused_a, unused_b;
        block_excl_scan2(c_cut, 0, &pre_cut, &unused_e, &unused_a, &unused_b, s_tmp);
        for (int w = w0; w < w1; ++w) {
            const uint64_t base = s_R[w] & ~s_S[w];
            uint64_t covered = 0, kept = 0;
            for (int j = 1; j <= min(js, nj); ++j) {
                const uint64_t A = ring_word(j, w);
                const uint64_t E = A & base & ~covered;
                covered |= A;
                if (j < js) {
                    kept |= E;
                } else {
                    const int take = min(max(allow - pre_cut, 0), __popcll(E));
                    kept |= E ^ drop_low_bits(E, take);  // the take lowest bits of E
                    pre_cut += __popcll(E);
                }
            }
            s_Rn[w] = s_S[w] | kept;
        }
    } else {
        for (int w = w0; w < w1; ++w) s_Rn[w] = s_S[w];
    }
    __syncthreads();

    // Step 2: D_in = S \ R and D_out = R \ R_t in ascending order (R_t = S without a
    // window). Each thread takes a contiguous range of words (sparse in practice), a
    // workgroup scan gives list offsets.
    int c_in = 0, c_out = 0;
    for (int w = w0; w < w1; ++w) {
        c_in += __popcll(s_S[w] & ~s_R[w]);
        c_out += __popcll(s_R[w] & ~s_Rn[w]);
    }
    int base_in, base_out, n_in, n_out;
    block_excl_scan2(c_in, c_out, &base_in, &base_out, &n_in, &n_out, s_tmp);
    {
        int ki = base_in, ko = base_out;
        for (int w = w0; w < w1; ++w) {
            uint64_t bi = s_S[w] & ~s_R[w], bo = s_R[w] & ~s_Rn[w];
            while (bi) {
                d_in[ki++] = w * 64 + (__ffsll((unsigned long long)bi) - 1);
                bi &= bi - 1;
            }
            while (bo) {
                d_out[ko++] = w * 64 + (__ffsll((unsigned long long)bo) - 1);
                bo &= bo - 1;
            }
        }
    }

    // Step 3: release the slots whose owner leaves the resident set (slot map -1, free bit;
    // the owner entry is cleared below unless the slot is taken again). Every slot is
    // looked at once, so the owners of D_out are found without a slot-map lookup each.
    // (An owner that is not a resident neuron would be released too; the released count is
    // checked against |D_out| below.)
    // A slot whose owner stays and is active this token is marked in s_Ab (the FFN's list).
    // 0: slot free or owner stays inactive, 1: owner leaves, 2: owner stays and is active.
    auto fate = [&](int sl, int n) -> int {
        if (sl >= K || n < 0) return 0;
        if (n >= M) {
            atomicOr(&s_err, kErrBadList);
            return 0;
        }
        const uint64_t bit = 1ull << (n & 63);
        if ((s_Rn[n >> 6] & bit) == 0) return 1;
        return (s_S[n >> 6] & bit) ? 2 : 0;
    };
    int c_rel = 0;
    {
        // The 64 lanes of a wave look at the 64 slots of one word (slot = tid + k * kNT, and
        // kNT is a multiple of 64), so each word's bits come from one ballot and one lane
        // writes them: no LDS atomics on a word that 64 lanes share.
        auto mark = [&](int sl, int f) {
            const uint64_t b_act = __ballot(f == 2), b_rel = __ballot(f == 1);
            if (lane == 0 && sl < K) {
                s_Ab[sl >> 6] |= b_act;
                s_F0[sl >> 6] |= b_rel;
            }
        };
        int fv[kOwnRegs];
#pragma unroll
        for (int k = 0; k < kOwnRegs; ++k) fv[k] = fate(tid + k * kNT, own[k]);
#pragma unroll
        for (int k = 0; k < kOwnRegs; ++k) {
            mark(tid + k * kNT, fv[k]);
            if (fv[k] != 1) continue;
            slot_map[own[k]] = -1;
            ++c_rel;
        }
        for (int sl0 = kOwnRegs * kNT; sl0 < K; sl0 += kNT) {  // uniform trip count: ballots stay whole-wave
            const int sl = sl0 + tid;
            const int n = sl < K ? owner[sl] : -1;
            const int f = fate(sl, n);
            mark(sl, f);
            if (f != 1) continue;
            slot_map[n] = -1;
            ++c_rel;
        }
    }

    // Free slots after the release: per-word prefix counts (ascending slot order); the
    // released count is checked against |D_out|.
    const int kpt = (Kw + kNT - 1) / kNT;
    const int v0 = min(tid * kpt, Kw), v1 = min(v0 + kpt, Kw);
    __syncthreads();  // the releases' free bits are in s_F0, the kept active slots in s_Ab
    int c_free = 0;
    for (int v = v0; v < v1; ++v) c_free += __popcll(s_F0[v]);
    int pre_free, pre_rel, n_free, n_rel;
    block_excl_scan2(c_free, c_rel, &pre_free, &pre_rel, &n_free, &n_rel, s_tmp);
    if (tid == 0 && n_rel != n_out) atomicOr(&s_err, kErrBadList);

    int n_act = 0;
    if (L.compact) {
        n_act = compact_assign(L, n_in, n_out, base_in, w0, w1, v0, v1, s_S, s_R, s_Fa, s_F0, s_fpre, s_tmp, &s_err);
    } else {
    // Step 4 (set part): the n_in lowest free slots are taken (they join the active slots);
    // active slots per word.
    int c_occ = 0;
    for (int v = v0; v < v1; ++v) {
        s_fpre[v] = pre_free;
        const int take = min(max(n_in - pre_free, 0), __popcll(s_F0[v]));
        pre_free += __popcll(s_F0[v]);
        const uint64_t fw = drop_low_bits(s_F0[v], take);
        s_F1[v] = fw;
        freeb[v] = fw;
        s_Ab[v] |= s_F0[v] & ~fw;
        c_occ += __popcll(s_Ab[v]);
        uint64_t gone = s_F0[v] & ~s_Fa[v] & fw;  // released and not taken again: no owner
        while (gone) {
            owner[v * 64 + __ffsll((unsigned long long)gone) - 1] = -1;
            gone &= gone - 1;
        }
    }
    int pre_occ, unused_e, unused_t;
    block_excl_scan2(c_occ, 0, &pre_occ, &unused_e, &n_act, &unused_t, s_tmp);  // publishes s_fpre, s_F1, s_Ab
    for (int v = v0; v < v1; ++v) {
        s_opre[v] = pre_occ;
        pre_occ += __popcll(s_Ab[v]);
    }
    __syncthreads();

    // Step 4 (lists): the i-th incoming neuron (ascending) takes the i-th free slot
    // (ascending). A thread's incoming neurons have consecutive indexes, so after one
    // search for the first slot it walks the free bits. The slot's position in the
    // ascending active-slot list gets the neuron ID in act_src, so that the FFN can read
    // the new bundle where it still is (the row store).
    {
        int idx = base_in;
        int lo = -1;
        uint64_t fw = 0;
        for (int w = w0; w < w1; ++w) {
            uint64_t bits = s_S[w] & ~s_R[w];
            while (bits) {
                const int n = w * 64 + (__ffsll((unsigned long long)bits) - 1);
                bits &= bits - 1;
                if (idx >= n_free) {
                    atomicOr(&s_err, kErrFreeExhausted);
                    ++idx;
                    continue;
                }
                if (lo < 0) {
                    int l0 = 0, h0 = Kw - 1;  // last word whose prefix is <= idx
                    while (l0 < h0) {
                        const int mid = (l0 + h0 + 1) >> 1;
                        if (s_fpre[mid] <= idx) l0 = mid; else h0 = mid - 1;
                    }
                    lo = l0;
                    fw = drop_low_bits(s_F0[lo], idx - s_fpre[lo]);
                }
                while (fw == 0) fw = s_F0[++lo];  // idx < n_free: a free bit follows
                const int b = __ffsll((unsigned long long)fw) - 1;
                fw &= fw - 1;
                const int slot = lo * 64 + b;
                const int pos = s_opre[lo] + __popcll(s_Ab[lo] & ((1ull << b) - 1));
                slot_in[idx] = slot;
                slot_map[n] = slot;
                owner[slot] = n;
                act_src[pos] = n;
                ++idx;
            }
        }
    }
    // Active slots in ascending order (without a window: every occupied slot), one word per
    // wave and one slot per lane; slots kept from the last step have act_src -1.
    {
        constexpr int kU = 4;  // words per wave per round, their LDS reads issued together
        const uint64_t bit = 1ull << lane;
        for (int v0w = wave * kU; v0w < Kw; v0w += kWaves * kU) {
            uint64_t occ[kU], taken[kU];
            int o0[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int v = min(v0w + u, Kw - 1);
                occ[u] = v0w + u < Kw ? s_Ab[v] : 0;
                taken[u] = s_F0[v] & ~s_F1[v];
                o0[u] = s_opre[v];
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if (occ[u] & bit) {
                    const int o = o0[u] + __popcll(occ[u] & (bit - 1));
                    act[o] = (v0w + u) * 64 + lane;
                    if (!(taken[u] & bit)) act_src[o] = -1;
                }
            }
        }
    }
    }  // slot layout

    // y of this layer for FFN launches that add into it (stored last: a store ahead of the
    // loads above would make their waits wait for it too)
    if (a.zero_y) {
        float* yb = a.prm ? gmem(a.prm)->y : a.y;
        auto* yl = gmem(yb + (size_t)(a.layer0 + blockIdx.x) * a.d);
        for (int i = tid; i < a.d; i += kNT) yl[i] = 0.f;
    }

    // Step 5: R = R_t; with a window, S joins the ring of recent active sets.
    for (int w = tid; w < W; w += kNT) {
        res[w] = s_Rn[w];
        if (win > 1) gmem(L.ring)[(size_t)(tok % (win - 1)) * W + w] = s_S[w];
    }
    __syncthreads();
    if (tid == 0) {
        counts[0] = n_in;
        counts[1] = n_out;
        counts[2] = n_act;
        counts[4] = tok + 1;
        counts[kPfDoneSlot] = 0;  // a token launch counts its finished workgroups from here
        counts[kFfnDoneSlot] = 0;
        if (s_err) raise_err(L.counts, s_err);
        auto* acc = gmem(L.acc);
        acc[0] += (unsigned long long)n_act;
        acc[1] += (unsigned long long)n_in;
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
