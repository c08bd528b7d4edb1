// Fused gather-GEMV sparse FFN for gfx950 (batch 1, bf16 rows, fp32 math).
//
// Computes y = sum over the resident slots s of down_s * relu(gate_s . x) * (up_s . x)
// (gated bundle [gate|up|down^T]) or y = sum_s down_s * relu(up_s . x) (bundle
// [up|down^T]); NeuroPrefetcher, section 3.4: each active neuron i uses row i of
// gate, up and down^T; the slot map locates the rows, whose order in the buffer
// does not matter.
//
// Batch-1 decode is a memory-bound GEMV (about 1 flop per byte), so there is no
// MFMA here: the kernel is built so that every weight byte crosses HBM exactly
// once and the HBM queues fill immediately.
//
// Decomposition (n active slots, listed in ascending slot order):
//   * The slot list is cut into P1 balanced chunks. Workgroup w < P1 computes
//     h for its chunk (phase 1): full-row dot products of the gate and up rows
//     with x (x lives in registers: each lane always covers the same 16-byte
//     column chunks), reduced across the workgroup, then h goes to global
//     memory and a per-chunk flag is released.
//   * The down rows are cut into Q column tiles of TW columns. Workgroup w
//     (0 <= w < P1 + Q - 1) takes tile w mod Q over the window of chunks
//     [w - Q + 1, w] (phase 2): it issues its down-row loads first, then
//     waits for the flags of the window's chunks -- all produced by
//     workgroups with lower IDs or by itself, so the wait always ends once
//     the earlier workgroups, dispatched first, finish phase 1 -- and
//     accumulates h * down into TW fp32 partial sums.
//   * Over the contributors of a tile (w = t, t + Q, ...) the windows cover
//     every chunk exactly once. The last contributor to arrive sums the
//     tile's partials in ascending contributor order (fixed order, so results
//     are identical run to run) and writes y.
// Partial traffic is (P1 + Q - 1) * TW * 4 bytes, about 1% of the row bytes.
// The epoch word makes the flags reusable without clearing; the last
// workgroup of a launch advances it, and each tile's last contributor resets
// that tile's counter, so consecutive launches need no memset.
#include "np_internal.hpp"

namespace np {
namespace {

constexpr int kWinMax = 2048;         // staged window positions per workgroup
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline float dot8(const uint4 v, const float* xv) {
    float a = 0.f;
    a = fmaf(bf_lo(v.x), xv[0], a);
    a = fmaf(bf_hi(v.x), xv[1], a);
    a = fmaf(bf_lo(v.y), xv[2], a);
    a = fmaf(bf_hi(v.y), xv[3], a);
    a = fmaf(bf_lo(v.z), xv[4], a);
    a = fmaf(bf_hi(v.z), xv[5], a);
    a = fmaf(bf_lo(v.w), xv[6], a);
    a = fmaf(bf_hi(v.w), xv[7], a);
    return a;
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

__device__ inline uint32_t ld_acquire(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}

// NT threads; JX 16-byte x chunks per lane; SB slots per phase-1 batch per row lane;
// U2 rows per lane per phase-2 batch.
template <int NT, int JX, bool GATED, int SB, int U2>
__global__ __launch_bounds__(NT) void k_sparse_ffn(FfnArgs a) {
    constexpr int kWaves = NT / 64;
    constexpr int R = GATED ? 3 : 2;
    constexpr int NR1 = GATED ? 2 : 1;  // rows dotted with x per slot

    __shared__ int s_act[kWinMax];
    __shared__ float s_red1[kWaves * SB * NR1];
    __shared__ float s_red2[NT * 8];
    __shared__ int s_last;

    const int w = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int d = a.d;
    uint32_t* flags = a.flags;
    uint32_t* tcnt = a.tcnt;
    uint32_t* done = a.ctl;
    uint32_t* epoch = a.ctl + 1;
    const uint32_t tgt = __hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;

    int n = a.counts[2];
    n = n < 0 ? 0 : (n > a.K ? a.K : n);
    auto cbeg = [&](int c) { return (int)(((long long)c * n) / a.p1); };

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
    for (int i = tid; i < wn; i += NT) {
        int s = a.act[plo + i];
        if ((unsigned)s >= (unsigned)a.K) {
            err |= kErrBadList;
            s = 0;
        }
        s_act[i] = s;
    }
    __syncthreads();

    // ---------------- phase 1: h for chunk w ----------------
    if (w < a.p1) {
        const int c0 = max(cbeg(w), plo), c1 = min(cbeg(w + 1), phi);
        const int CPR = d >> 3;                              // 16-byte chunks per row
        int CL = NT;                                         // lanes per row lane (power of 2)
        while (CL > CPR && CL > 1) CL >>= 1;
        const int RL = NT / CL;                              // row lanes
        const int rl = tid / CL, cl = tid % CL;

        float xv[JX][8];
#pragma unroll
        for (int j = 0; j < JX; ++j) {
            const int c = cl + CL * j;
            if (c < CPR) {
                const float4 p = reinterpret_cast<const float4*>(a.x)[2 * c];
                const float4 q = reinterpret_cast<const float4*>(a.x)[2 * c + 1];
                xv[j][0] = p.x; xv[j][1] = p.y; xv[j][2] = p.z; xv[j][3] = p.w;
                xv[j][4] = q.x; xv[j][5] = q.y; xv[j][6] = q.z; xv[j][7] = q.w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) xv[j][e] = 0.f;
            }
        }

        for (int b0 = c0; b0 < c1; b0 += SB * RL) {
            float part[SB][NR1];
            uint4 wv[SB][NR1][JX];
#pragma unroll
            for (int i = 0; i < SB; ++i) {
                const int pos = b0 + rl * SB + i;
                const bool ok = pos < c1;
                const int slot = ok ? s_act[pos - plo] : 0;
                const uint4* row = reinterpret_cast<const uint4*>(a.buf + (size_t)slot * R * d);
#pragma unroll
                for (int r = 0; r < NR1; ++r)
#pragma unroll
                    for (int j = 0; j < JX; ++j) {
                        const int c = cl + CL * j;
                        if (ok && c < CPR) wv[i][r][j] = row[r * CPR + c];
                        else wv[i][r][j] = make_uint4(0, 0, 0, 0);
                    }
            }
#pragma unroll
            for (int i = 0; i < SB; ++i)
#pragma unroll
                for (int r = 0; r < NR1; ++r) {
                    float acc = 0.f;
#pragma unroll
                    for (int j = 0; j < JX; ++j) acc += dot8(wv[i][r][j], xv[j]);
                    part[i][r] = acc;
                }
            // reduce each partial over the CL lanes of the row lane
            const int xr_lim = CL < 64 ? CL : 64;
#pragma unroll
            for (int i = 0; i < SB; ++i)
#pragma unroll
                for (int r = 0; r < NR1; ++r)
                    for (int off = xr_lim >> 1; off > 0; off >>= 1)
                        part[i][r] += __shfl_xor(part[i][r], off, 64);
            if (CL >= 64) {
                if (lane == 0) {
#pragma unroll
                    for (int i = 0; i < SB; ++i)
#pragma unroll
                        for (int r = 0; r < NR1; ++r) s_red1[(wave * SB + i) * NR1 + r] = part[i][r];
                }
                __syncthreads();
            }
            if (cl == 0) {
#pragma unroll
                for (int i = 0; i < SB; ++i) {
                    const int pos = b0 + rl * SB + i;
                    if (pos < c1) {
                        float v[NR1];
#pragma unroll
                        for (int r = 0; r < NR1; ++r) {
                            if (CL >= 64) {
                                float s = 0.f;
                                for (int k = 0; k < CL / 64; ++k)
                                    s += s_red1[((rl * (CL / 64) + k) * SB + i) * NR1 + r];
                                v[r] = s;
                            } else {
                                v[r] = part[i][r];
                            }
                        }
                        float h;
                        if (GATED) h = fmaxf(v[0], 0.f) * v[1];
                        else h = fmaxf(v[0], 0.f);
                        a.hval[pos] = h;
                    }
                }
            }
            if (CL >= 64) __syncthreads();
        }
        __threadfence();
        __syncthreads();
        if (tid == 0) __hip_atomic_store(&flags[w], tgt, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---------------- phase 2: down tile t over the window ----------------
    const int t = w % a.q;
    const int col0 = t * a.tw;
    const int tcols = min(a.tw, d - col0);
    const int CT = a.tw >> 3;                 // lanes per row segment
    const int RL2 = NT / CT;                  // row lanes
    const int c2 = tid % CT, r2 = tid / CT;
    const bool cok = (c2 << 3) < tcols;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;

    const uint4* dbase = reinterpret_cast<const uint4*>(a.buf) + (size_t)(R - 1) * (d >> 3) + (col0 >> 3) + c2;
    const size_t slot_stride = (size_t)R * (d >> 3);

    uint4 dv[U2];
    int i0 = r2;                              // first window row of this lane
#pragma unroll
    for (int u = 0; u < U2; ++u) {
        const int i = i0 + u * RL2;
        if (cok && i < wn) dv[u] = dbase[(size_t)s_act[i] * slot_stride];
    }

    // Wait for the h values of the other chunks of the window (lower workgroup IDs).
    if (lane == 0) {
        for (int c = wlo; c <= whi; ++c) {
            if (c == w) continue;
            uint32_t it = 0;
            while (ld_acquire(&flags[c]) != tgt) {
                __builtin_amdgcn_s_sleep(2);
                if (++it > kSpinLimit) {
                    err |= kErrSpin;
                    break;
                }
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    while (true) {
#pragma unroll
        for (int u = 0; u < U2; ++u) {
            const int i = i0 + u * RL2;
            if (cok && i < wn) {
                const float h = __hip_atomic_load(&a.hval[plo + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                axpy8(acc, h, dv[u]);
            }
        }
        i0 += U2 * RL2;
        if (i0 >= wn) break;
#pragma unroll
        for (int u = 0; u < U2; ++u) {
            const int i = i0 + u * RL2;
            if (cok && i < wn) dv[u] = dbase[(size_t)s_act[i] * slot_stride];
        }
    }

    // Reduce the RL2 row lanes: s_red2[r2][c2*8 + e].
#pragma unroll
    for (int e = 0; e < 8; ++e) s_red2[r2 * a.tw + (c2 << 3) + e] = acc[e];
    __syncthreads();
    for (int j = tid; j < tcols; j += NT) {
        float s = 0.f;
        for (int r = 0; r < RL2; ++r) s += s_red2[r * a.tw + j];
        __hip_atomic_store(&a.partials[(size_t)w * a.tw + j], s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __threadfence();
    __syncthreads();
    const int ncontrib = (a.nwg - 1 - t) / a.q + 1;
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&tcnt[t], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == (uint32_t)(ncontrib - 1));
    }
    __syncthreads();
    if (s_last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        for (int j = tid; j < tcols; j += NT) {
            float s = 0.f;
            for (int k = 0; k < ncontrib; ++k)
                s += __hip_atomic_load(&a.partials[(size_t)(t + k * a.q) * a.tw + j], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            a.y[col0 + j] = s;
        }
        if (tid == 0) __hip_atomic_store(&tcnt[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (err) atomicOr(&a.counts[3], err);
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (old == (uint32_t)(a.nwg - 1)) {
            __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(epoch, tgt, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int NT, int JX, bool G>
hipError_t launch_t(const FfnArgs& a, const FfnShape& sh, hipStream_t s) {
    constexpr int SB = (JX <= 2) ? 8 : 4;
    hipLaunchKernelGGL((k_sparse_ffn<NT, JX, G, SB, 8>), dim3(sh.nwg), dim3(NT), 0, s, a);
    return hipGetLastError();
}

template <int NT, bool G>
hipError_t launch_jx(const FfnArgs& a, const FfnShape& sh, hipStream_t s) {
    switch (sh.jx) {
        case 1: return launch_t<NT, 1, G>(a, sh, s);
        case 2: return launch_t<NT, 2, G>(a, sh, s);
        case 3: return launch_t<NT, 3, G>(a, sh, s);
        case 4: return launch_t<NT, 4, G>(a, sh, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_sparse_ffn(const FfnArgs& a, const FfnShape& sh, bool gated, hipStream_t s) {
    if (sh.nt == 256) return gated ? launch_jx<256, true>(a, sh, s) : launch_jx<256, false>(a, sh, s);
    if (sh.nt == 512) return gated ? launch_jx<512, true>(a, sh, s) : launch_jx<512, false>(a, sh, s);
    return hipErrorInvalidValue;
}

int ffn_win_max() { return kWinMax; }

}  // namespace np
