// qmv_affine4: decode GEMV y[1, N] = x[1, K] . dequant(W)^T for affine INT4
// group-32 weights (INT4 MatMulNBits page: the M = 1 route).
//
// HBM-bound: every weight byte is read once. Each wavefront owns R output
// rows; its 64 lanes split K by quantisation group (lane l takes groups
// l, l + 64, ...), so one 128-bit load per lane and row fetches exactly one
// group's 32 nibbles and consecutive lanes read consecutive 16-byte pieces of
// the row. x stays in registers for all R rows. The per-group dot product
// uses bf16 pairs (128 + q) with v_dot2_f32_bf16, then
//   sum_k x_k (q_k s + b) = s * sum_k x_k (128 + q_k) + (b - 128 s) * sum_k x_k,
// so the scale and bias are applied once per group, not per weight.
#include "w4mi_device.hpp"
#include "w4mi_host.hpp"

namespace w4mi {

constexpr int kGemvThreads = 256;

// Lane view of one quantisation group of x: bf16 pairs matching the nibble
// pairs (i, i + 4) of each of the group's four words, and the group sum.
struct XGroup {
    uint32_t pair[4][4];
    float sum;
};

__device__ __forceinline__ void load_x_group(const uint16_t* __restrict__ x, int g, XGroup& xg) {
    const u32x4* xp = reinterpret_cast<const u32x4*>(x + (size_t)g * 32);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x4 v = xp[j];  // elements 8j .. 8j+7 as bf16 pairs (0,1) (2,3) (4,5) (6,7)
        xg.pair[j][0] = __builtin_amdgcn_perm(v[2], v[0], 0x05040100u);  // (8j+0, 8j+4)
        xg.pair[j][1] = __builtin_amdgcn_perm(v[2], v[0], 0x07060302u);  // (8j+1, 8j+5)
        xg.pair[j][2] = __builtin_amdgcn_perm(v[3], v[1], 0x05040100u);  // (8j+2, 8j+6)
        xg.pair[j][3] = __builtin_amdgcn_perm(v[3], v[1], 0x07060302u);  // (8j+3, 8j+7)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v[e]), as_bf16x2(0x3F803F80u), s, false);
    }
    xg.sum = s;
}

// sum over the group of x_k * (128 + q_k), f32 accumulation.
__device__ __forceinline__ float group_dot_biased(const u32x4& words, const XGroup& xg) {
    float d = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(affine_pair_biased_bf16(words[j], i)),
                                                as_bf16x2(xg.pair[j][i]), d, false);
    return d;
}

// R rows per wavefront; T = number of 64-group chunks of K when known at
// compile time (K <= 64 * 32 * T), or 0 for a runtime loop.
template <int R, int T>
__global__ __launch_bounds__(kGemvThreads) void qmv_affine4_kernel(
    const uint32_t* __restrict__ w, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int K, int N, int chunks) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int n0 = (blockIdx.x * (kGemvThreads / kWave) + wave) * R;
    if (n0 >= N) return;  // N % 32 == 0 and R | 32: a live wave owns R valid rows
    const int G = K / 32;
    const int nch = T > 0 ? T : chunks;

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;

    constexpr int TB = T > 0 ? T : 1;  // chunks loaded before any arithmetic
    for (int t0 = 0; t0 < nch; t0 += TB) {
        u32x4 wv[TB][R];
        uint32_t sv[TB][R], bv[TB][R];
        // Issue every load of this batch first: R rows x TB groups per lane.
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const int g = (t0 + t) * kWave + lane;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (g < G) {
                    const size_t row = (size_t)(n0 + r);
                    wv[t][r] = *reinterpret_cast<const u32x4*>(w + row * (K / 8) + (size_t)g * 4);
                    sv[t][r] = scales[row * G + g];
                    bv[t][r] = biases[row * G + g];
                } else {
                    wv[t][r] = u32x4{0u, 0u, 0u, 0u};
                    sv[t][r] = 0u;
                    bv[t][r] = 0u;
                }
            }
        }
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const int g = (t0 + t) * kWave + lane;
            if (g < G) {
                XGroup xg;
                load_x_group(x, g, xg);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float s = bf16_bits_to_f32(sv[t][r]);
                    const float b = bf16_bits_to_f32(bv[t][r]);
                    const float d = group_dot_biased(wv[t][r], xg);
                    acc[r] = __builtin_fmaf(s, d, acc[r]);
                    acc[r] = __builtin_fmaf(__builtin_fmaf(-128.f, s, b), xg.sum, acc[r]);
                }
            }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
    if (lane < R) {
        float v = acc[0];
#pragma unroll
        for (int r = 1; r < R; ++r)
            if (lane == r) v = acc[r];
        y[n0 + lane] = f32_to_bf16_bits(v);
    }
}

}  // namespace w4mi

using namespace w4mi;

extern "C" w4_status qmv_affine4(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                                 const uint16_t* x, uint16_t* y, int64_t M, int64_t K, int64_t N,
                                 int32_t group_size, int32_t bits, void* stream) {
    w4_status st = w4_check_affine(M, K, N, group_size, bits, 1);
    if (st != W4_OK) return st;
    if (M == 0) return W4_OK;
    if (!w || !scales || !biases || !x || !y) return fail(W4_EINVAL, "qmv_affine4: null pointer argument");
    if (((uintptr_t)w & 15u) || ((uintptr_t)x & 15u)) return fail(W4_EINVAL, "qmv_affine4: w and x must be 16-byte aligned");
    constexpr int R = 4;
    const int rows_per_block = (kGemvThreads / kWave) * R;
    const dim3 grid((unsigned)((N + rows_per_block - 1) / rows_per_block));
    const int G = (int)(K / 32);
    const int chunks = (G + kWave - 1) / kWave;
    hipStream_t s = as_stream(stream);
    switch (chunks) {
        case 1: hipLaunchKernelGGL((qmv_affine4_kernel<R, 1>), grid, dim3(kGemvThreads), 0, s, w, scales, biases, x, y, (int)K, (int)N, chunks); break;
        case 2: hipLaunchKernelGGL((qmv_affine4_kernel<R, 2>), grid, dim3(kGemvThreads), 0, s, w, scales, biases, x, y, (int)K, (int)N, chunks); break;
        case 3: hipLaunchKernelGGL((qmv_affine4_kernel<R, 3>), grid, dim3(kGemvThreads), 0, s, w, scales, biases, x, y, (int)K, (int)N, chunks); break;
        case 4: hipLaunchKernelGGL((qmv_affine4_kernel<R, 4>), grid, dim3(kGemvThreads), 0, s, w, scales, biases, x, y, (int)K, (int)N, chunks); break;
        default: hipLaunchKernelGGL((qmv_affine4_kernel<R, 0>), grid, dim3(kGemvThreads), 0, s, w, scales, biases, x, y, (int)K, (int)N, chunks); break;
    }
    return launch_status("qmv_affine4");
}
