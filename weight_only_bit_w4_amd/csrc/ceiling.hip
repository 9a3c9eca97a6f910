// Measurement kernels: the achievable ceilings the benchmark reports beside
// the MI355X's published peaks.
//   w4_ceiling_stream_read - every byte of a buffer read once with 16-byte
//       non-temporal loads, each workgroup streaming one contiguous chunk
//       with four loads per lane in flight (the fastest plain read pattern
//       found for buffers of tens of MB to hundreds of MB: about 10 % faster
//       than a grid-stride loop on a 36.7 MB buffer), folded into one word
//       per lane so no load is dropped;
//   w4_ceiling_mfma - v_mfma_f32_32x32x16_f16 back to back on every SIMD
//       (four independent accumulators per wavefront, no memory traffic).
#include "w4mi_device.hpp"
#include "w4mi_host.hpp"

namespace w4mi {

constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 4;     // 16-byte loads in flight per lane
constexpr int kReadGroups = 1024;  // workgroups for large buffers (four per CU)

// Workgroup b reads pieces [b * per, min((b + 1) * per, pieces)) of 16 bytes;
// per is a multiple of 64 pieces, so every wavefront load covers one aligned
// kilobyte.
__global__ __launch_bounds__(kReadThreads) void ceiling_read_kernel(const u32x4* __restrict__ buf, int64_t pieces,
                                                                    int64_t per, uint32_t* __restrict__ sink) {
    const int64_t beg = (int64_t)blockIdx.x * per;
    const int64_t end = beg + per < pieces ? beg + per : pieces;
    int64_t i = beg + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kReadUnroll - 1) * kReadThreads < end; i += kReadUnroll * kReadThreads) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * kReadThreads);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < end; i += kReadThreads) {
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    // One word per lane of the first wavefront that holds any fold, written only when it is the
    // (practically impossible) value 0x9E3779B9, so the loads stay live without a store stream.
    if (acc == 0x9E3779B9u) sink[blockIdx.x & 1023] = acc;
}

constexpr int kMfmaThreads = 256;  // one wavefront per SIMD

__global__ __launch_bounds__(kMfmaThreads) void ceiling_mfma_kernel(uint32_t* __restrict__ sink, int iters) {
    const int lane = threadIdx.x & 63;
    f16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(0.001f * (float)(lane + i));
        b[i] = (_Float16)(0.002f * (float)i);
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
    }
    float r = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) r += c0[e] + c1[e] + c2[e] + c3[e];
    if (r == 12345.678f) sink[blockIdx.x & 1023] = __float_as_uint(r);
}

}  // namespace w4mi

using namespace w4mi;

extern "C" w4_status w4_ceiling_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink) return fail(W4_EINVAL, "w4_ceiling_stream_read: null pointer argument");
    if (bytes % 16 != 0 || ((uintptr_t)buf & 15u) != 0)
        return fail(W4_EINVAL, "w4_ceiling_stream_read: buffer must be 16-byte aligned and a multiple of 16 bytes");
    if (bytes == 0) return W4_OK;
    const int64_t pieces = (int64_t)(bytes / 16);
    // Four workgroups of eight wavefronts per CU, one contiguous chunk each
    // (fewer for a buffer under 32 KB per workgroup).
    const int64_t step = (int64_t)kReadThreads * kReadUnroll;
    const int64_t grid = std::min<int64_t>((pieces + step - 1) / step, kReadGroups);
    const int64_t per = ((pieces + grid - 1) / grid + 63) / 64 * 64;
    const unsigned launch = (unsigned)((pieces + per - 1) / per);
    hipLaunchKernelGGL(ceiling_read_kernel, dim3(launch), dim3(kReadThreads), 0, as_stream(stream),
                       reinterpret_cast<const u32x4*>(buf), pieces, per, sink);
    return launch_status("w4_ceiling_stream_read");
}

extern "C" w4_status w4_ceiling_mfma(uint32_t* sink, int32_t iters, void* stream) {
    if (!sink) return fail(W4_EINVAL, "w4_ceiling_mfma: sink is null");
    if (iters <= 0) return fail(W4_EINVAL, "w4_ceiling_mfma: iters must be positive, got %d", iters);
    // Two workgroups of 4 wavefronts per CU keep every SIMD's matrix core fed.
    hipLaunchKernelGGL(ceiling_mfma_kernel, dim3(kCUs * 2), dim3(kMfmaThreads), 0, as_stream(stream), sink, iters);
    return launch_status("w4_ceiling_mfma");
}
