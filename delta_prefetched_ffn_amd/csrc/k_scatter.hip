// Row scatter for gfx950: copies each incoming neuron's bundle from the backing
// row store into its assigned slot of the resident buffer (NeuroPrefetcher,
// section 3.5: one record per incoming neuron holds its gate, up and down^T
// rows; a GPU kernel places it at the slot the delta runtime assigned).
//
// The bundle is kept interleaved (one slot = one record), so the copy is a
// plain 128-bit gather-scatter: workgroup b copies bundles b, b + grid, ...,
// each lane moving U 16-byte chunks per pass with all U loads issued before
// the stores. The store may be device memory (an HBM-resident backing store)
// or pinned host memory (the loads then cross the host link).
#include "np_internal.hpp"

namespace np {
namespace {

constexpr int kNT = 256;
constexpr int kU = 8;

__global__ __launch_bounds__(kNT) void k_scatter_rows(int32_t* counts, const int32_t* __restrict__ d_in,
                                                      const int32_t* __restrict__ slot_in,
                                                      const uint4* __restrict__ store,
                                                      uint4* __restrict__ buf, int32_t M, int32_t K,
                                                      int32_t cb, int32_t row16, int32_t stride16, int64_t plane16) {
    const int n_in = min(counts[0], K);  // the lists hold at most K entries
    for (int i = blockIdx.x; i < n_in; i += gridDim.x) {
        const int n = d_in[i], s = slot_in[i];
        if ((unsigned)n >= (unsigned)M || (unsigned)s >= (unsigned)K) {
            if (threadIdx.x == 0) raise_err(counts, kErrBadList);
            continue;
        }
        const uint4* src = store + (size_t)n * cb;
        for (int c = threadIdx.x; c < cb; c += kNT * kU) {
            uint4 v[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (c + u * kNT < cb) v[u] = src[c + u * kNT];
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (c + u * kNT < cb) buf[slot_chunk(s, c + u * kNT, row16, stride16, plane16)] = v[u];
        }
    }
}

// All layers of a decode step at once: blockIdx.y picks the layer, blockIdx.x strides over
// that layer's incoming bundles.
__global__ __launch_bounds__(kNT) void k_scatter_all(ScatterLaunch a) {
    scatter_bundles<kNT, kU>(a.layers[blockIdx.y], blockIdx.x, gridDim.x);
}

// A row store in pinned host memory: a few workgroups of kFlatNT threads (scatter_flat).
constexpr int kFlatNT = 1024;
constexpr int kFlatCap = 2048;
__global__ __launch_bounds__(kFlatNT) void k_scatter_flat(const LayerDev* L) {
    __shared__ int s_n[kFlatCap], s_s[kFlatCap];
    scatter_flat<kFlatNT, kFlatCap>(L, blockIdx.x, gridDim.x, s_n, s_s);
}

// Compacted layout: the rows moved by the last assignment, buf[mv_dst[k]] = buf[mv_src[k]]
// for k < counts[5], all layers at once (blockIdx.y = layer). Sources (the end of the old
// region) and destinations (holes below it) are disjoint, so the copies are independent.
__global__ __launch_bounds__(kNT) void k_move_all(ScatterLaunch a) {
    const LayerDev* L = a.layers[blockIdx.y];
    const int K = L->K, cb = L->bundle16;
    const int n_mv = min(gmem(L->counts)[5], K);
    auto* buf = gmem(reinterpret_cast<uint4*>(L->buf));
    const auto* src_l = gmem(L->mv_src);
    const auto* dst_l = gmem(L->mv_dst);
    for (int i = blockIdx.x; i < n_mv; i += gridDim.x) {
        const int sp = src_l[i], dp = dst_l[i];
        if ((unsigned)sp >= (unsigned)K || (unsigned)dp >= (unsigned)K) {
            if (threadIdx.x == 0) raise_err(L->counts, kErrBadList);
            continue;
        }
        for (int c = threadIdx.x; c < cb; c += kNT * kU) {
            typedef uint32_t u4 __attribute__((ext_vector_type(4)));
            u4 v[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (c + u * kNT < cb)
                    v[u] = reinterpret_cast<const NP_GLOBAL u4*>(buf)[slot_chunk(sp, c + u * kNT, L->row16, L->stride16, L->plane16)];
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (c + u * kNT < cb)
                    reinterpret_cast<NP_GLOBAL u4*>(buf)[slot_chunk(dp, c + u * kNT, L->row16, L->stride16, L->plane16)] = v[u];
        }
    }
}

// Staged delta (the I/O shape of NeuroPrefetcher section 3.5): the host gathered cnt
// incoming bundles, in ascending neuron order, into a staging buffer that the DMA engine
// copied to device memory; bundle i goes to slot slot_in[i]. One record per bundle, kept
// interleaved in the slot, so the "deinterleave" is a plain bundle copy.
__global__ __launch_bounds__(kNT) void k_scatter_staged(int32_t* counts, const int32_t* __restrict__ slot_in,
                                                        const uint4* __restrict__ stage, uint4* __restrict__ buf,
                                                        int32_t cnt, int32_t K, int32_t cb, int32_t row16,
                                                        int32_t stride16, int64_t plane16) {
    for (int i = blockIdx.x; i < cnt; i += gridDim.x) {
        const int s = slot_in[i];
        if ((unsigned)s >= (unsigned)K) {
            if (threadIdx.x == 0) raise_err(counts, kErrBadList);
            continue;
        }
        const uint4* src = stage + (size_t)i * cb;
        for (int c = threadIdx.x; c < cb; c += kNT * kU) {
            uint4 v[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (c + u * kNT < cb) v[u] = src[c + u * kNT];
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (c + u * kNT < cb) buf[slot_chunk(s, c + u * kNT, row16, stride16, plane16)] = v[u];
        }
    }
}

// Streaming read: grid-stride, four non-temporal 16-byte loads in flight per lane, every lane
// folds the words it read into one value.
// (At 36 MiB per launch this shape, 512 workgroups of 1024 threads, was the fastest of
// 256-4096 workgroups of 256-1024 threads with 4 or 8 loads per lane.)
constexpr int kProbeNT = 1024;
constexpr int kProbeGrid = 512;
__device__ inline uint4 probe_ld(const uint4* p) {
    typedef uint32_t uv4 __attribute__((ext_vector_type(4)));
    const uv4 t = __builtin_nontemporal_load((const uv4*)p);
    return make_uint4(t.x, t.y, t.z, t.w);
}
__global__ __launch_bounds__(kProbeNT) void k_probe_read(const uint4* __restrict__ src, int64_t n16, float* sink) {
    const int64_t stride = (int64_t)gridDim.x * kProbeNT;
    uint32_t acc = 0;
    int64_t i = (int64_t)blockIdx.x * kProbeNT + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = probe_ld(src + i), b = probe_ld(src + i + stride), c = probe_ld(src + i + 2 * stride),
                    d = probe_ld(src + i + 3 * stride);
        acc += a.x ^ b.y ^ c.z ^ d.w;
    }
    for (; i < n16; i += stride) acc += src[i].x;
    // Every lane's value stays live through a store it makes only in an unlikely case, and
    // lane 0 of each workgroup writes its own. (Summing the workgroup's values with LDS
    // atomics on one word cost about 5 us per launch: 1024 serialised read-modify-writes.)
    if (acc == 0xffffffffu) sink[65535] = 1.f;
    if (threadIdx.x == 0) sink[blockIdx.x] = (float)(acc & 0xffffu);
}

__global__ __launch_bounds__(kNT) void k_probe_copy(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                    int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * kNT;
    for (int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// Raises error bits as a kernel that finds an inconsistency does (for tests of the reporting).
__global__ void k_raise_err(int32_t* counts, int bits) {
    if (threadIdx.x == 0) raise_err(counts, bits);
}

}  // namespace

hipError_t launch_raise_err(int32_t* counts, int bits, hipStream_t s) {
    hipLaunchKernelGGL(k_raise_err, dim3(1), dim3(64), 0, s, counts, bits);
    return hipGetLastError();
}

hipError_t launch_scatter(int32_t* counts, const int32_t* d_in, const int32_t* slot_in,
                          const uint16_t* store, uint16_t* buf, int32_t M, int32_t K,
                          int32_t bundle_elems, int32_t row16, int32_t stride16, int64_t plane16, int grid,
                          hipStream_t s) {
    hipLaunchKernelGGL(k_scatter_rows, dim3(grid), dim3(kNT), 0, s, counts, d_in, slot_in,
                       reinterpret_cast<const uint4*>(store), reinterpret_cast<uint4*>(buf), M, K,
                       bundle_elems / 8, row16, stride16, plane16);
    return hipGetLastError();
}

hipError_t launch_scatter_all(const ScatterLaunch& a, int wgs_per_layer, hipStream_t s) {
    hipLaunchKernelGGL(k_scatter_all, dim3(wgs_per_layer, a.n_layers), dim3(kNT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_scatter_flat(const LayerDev* L, int wgs, hipStream_t s) {
    hipLaunchKernelGGL(k_scatter_flat, dim3(wgs), dim3(kFlatNT), 0, s, L);
    return hipGetLastError();
}

hipError_t launch_move_all(const ScatterLaunch& a, int wgs_per_layer, hipStream_t s) {
    hipLaunchKernelGGL(k_move_all, dim3(wgs_per_layer, a.n_layers), dim3(kNT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_scatter_staged(int32_t* counts, const int32_t* slot_in, const void* stage, uint16_t* buf,
                                 int32_t cnt, int32_t K, int32_t bundle_elems, int32_t row16, int32_t stride16,
                                 int64_t plane16, hipStream_t s) {
    const int grid = std::max(1, std::min(cnt, 1024));
    hipLaunchKernelGGL(k_scatter_staged, dim3(grid), dim3(kNT), 0, s, counts, slot_in,
                       reinterpret_cast<const uint4*>(stage), reinterpret_cast<uint4*>(buf), cnt, K, bundle_elems / 8,
                       row16, stride16, plane16);
    return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, int64_t bytes, float* sink, hipStream_t s) {
    const int64_t n16 = bytes / 16;
    const int grid = (int)std::min<int64_t>(kProbeGrid, std::max<int64_t>(1, (n16 + kProbeNT * 4 - 1) / (kProbeNT * 4)));
    hipLaunchKernelGGL(k_probe_read, dim3(grid), dim3(kProbeNT), 0, s, reinterpret_cast<const uint4*>(src), n16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, int64_t bytes, hipStream_t s) {
    const int64_t n16 = bytes / 16;
    int grid = (int)std::min<int64_t>(256 * 16, std::max<int64_t>(1, (n16 + kNT - 1) / kNT));
    hipLaunchKernelGGL(k_probe_copy, dim3(grid), dim3(kNT), 0, s, reinterpret_cast<uint4*>(dst),
                       reinterpret_cast<const uint4*>(src), n16);
    return hipGetLastError();
}

}  // namespace np
