// gdn_snapshot.hip -- prefix-cache snapshots of the recurrent state: whole-slot
// copies between a state cache and a prefix pool (or within one cache).
//
// Automatic prefix caching on a recurrent hybrid (dflash-caddtree-integrations
// README, "What's in here": gdn_apc, prefix caching under speculative decoding
// with a warm start bitwise equal to a cold one) saves the committed state a
// sequence reached after a shared prefix and later restores it into another
// sequence's slot.  The copy is exact, so a restored state continues bit for
// bit like the recomputed one.  Pure data movement: 16-byte loads and stores,
// one grid row per copied slot.
#include <algorithm>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;  // 16-byte loads in flight per thread

__global__ __launch_bounds__(kCopyThreads) void slot_copy_kernel(const float4 *src, int src_total,
                                                                 const int32_t *src_slot, float4 *dst,
                                                                 int dst_total, const int32_t *dst_slot,
                                                                 size_t slot4) {
    const int e = blockIdx.y;
    const int s = src_slot[e], d = dst_slot[e];
    if (s < 0 || s >= src_total || d < 0 || d >= dst_total) return;
    const float4 *from = src + (size_t)s * slot4;
    float4 *to = dst + (size_t)d * slot4;
    const size_t per_block = (size_t)kCopyThreads * kCopyUnroll;
    for (size_t base = (size_t)blockIdx.x * per_block; base < slot4; base += (size_t)gridDim.x * per_block) {
        float4 r[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const size_t i = base + (size_t)u * kCopyThreads + threadIdx.x;
            if (i < slot4) r[u] = from[i];
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const size_t i = base + (size_t)u * kCopyThreads + threadIdx.x;
            if (i < slot4) to[i] = r[u];
        }
    }
}

}  // namespace

hipError_t launch_state_copy(const float *src, int src_total, const int32_t *src_slot, float *dst, int dst_total,
                             const int32_t *dst_slot, int count, size_t slot_floats, hipStream_t s) {
    const size_t slot4 = slot_floats / 4;
    const size_t per_block = (size_t)kCopyThreads * kCopyUnroll;
    const size_t blocks = (slot4 + per_block - 1) / per_block;
    const dim3 grid((unsigned)std::min<size_t>(blocks, 65535), (unsigned)count);
    hipLaunchKernelGGL(slot_copy_kernel, grid, dim3(kCopyThreads), 0, s, reinterpret_cast<const float4 *>(src),
                       src_total, src_slot, reinterpret_cast<float4 *>(dst), dst_total, dst_slot, slot4);
    return hipGetLastError();
}

}  // namespace gdn

// ---------------------------------------------------------------------------
// Streaming diagnostic: the plain read and copy rates of this part, the
// ceilings the state streams above are measured against.  64 KiB per
// 256-thread workgroup, 16-byte accesses, four in flight per thread; the read
// keeps one partial sum per workgroup so no load can be dropped.
// ---------------------------------------------------------------------------
namespace gdn {
namespace {

constexpr int kProbeThreads = 256;
constexpr size_t kProbeBlockBytes = 64 * 1024;

template <bool COPY>
__global__ __launch_bounds__(kProbeThreads) void probe_kernel(const float4 *src, float4 *dst, size_t n16) {
    const size_t base = (size_t)blockIdx.x * (kProbeBlockBytes / 16);
    float acc = 0.0f;
#pragma unroll 1
    for (size_t off = threadIdx.x; off < kProbeBlockBytes / 16; off += 4 * kProbeThreads) {
        float4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const size_t i = base + off + (size_t)u * kProbeThreads;
            x[u] = i < n16 ? src[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const size_t i = base + off + (size_t)u * kProbeThreads;
            if (COPY) {
                if (i < n16) dst[i] = x[u];
            } else {
                acc += (x[u].x + x[u].y) + (x[u].z + x[u].w);
            }
        }
    }
    if (!COPY) {
        for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
        if (threadIdx.x % 64 == 0) reinterpret_cast<float *>(dst)[blockIdx.x * (kProbeThreads / 64) + threadIdx.x / 64] = acc;
    }
}

}  // namespace

size_t probe_partials_bytes(size_t bytes) {
    return (bytes + kProbeBlockBytes - 1) / kProbeBlockBytes * (kProbeThreads / 64) * sizeof(float);
}

hipError_t launch_probe(int mode, const void *src, void *dst, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    const size_t blocks = (bytes + kProbeBlockBytes - 1) / kProbeBlockBytes;
    if (mode == 0)
        hipLaunchKernelGGL(probe_kernel<false>, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s,
                           static_cast<const float4 *>(src), static_cast<float4 *>(dst), n16);
    else
        hipLaunchKernelGGL(probe_kernel<true>, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s,
                           static_cast<const float4 *>(src), static_cast<float4 *>(dst), n16);
    return hipGetLastError();
}

}  // namespace gdn
