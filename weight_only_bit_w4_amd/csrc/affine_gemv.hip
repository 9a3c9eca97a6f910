// qmv_affine4: decode GEMV y[1, N] = x[1, K] . dequant(W)^T for affine INT4
// group-32 weights (INT4 MatMulNBits page: the M = 1 route).
//
// HBM-bound: every weight byte is read once. Each wavefront (one per
// workgroup, so the rows spread evenly over the CUs) owns R output rows; its
// 64 lanes split K by quantisation group (lane l takes groups l, l + 64, ...),
// so one 128-bit load per lane and row fetches exactly one group's 32 nibbles
// and consecutive lanes read consecutive 16-byte pieces of the row. All loads
// of a wavefront are issued before its first arithmetic; x stays in registers
// for all R rows, and the R row sums are reduced across lanes together. The per-group dot product
// uses bf16 pairs (128 + q) with v_dot2_f32_bf16, then
//   sum_k x_k (q_k s + b) = s * sum_k x_k (128 + q_k) + (b - 128 s) * sum_k x_k,
// so the scale and bias are applied once per group, not per weight.
#include "w4mi_device.hpp"
#include "w4mi_host.hpp"

namespace w4mi {

constexpr int kGemvRows = 8;  // output rows per wavefront (one wavefront per workgroup)

// Lane view of one quantisation group of x: bf16 pairs matching the nibble
// pairs (i, i + 4) of each of the group's four words, and the group sum.
struct XGroup {
    uint32_t pair[4][4];
    float sum;
};

__device__ __forceinline__ void x_group_from_raw(const u32x4 (&v4)[4], XGroup& xg) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t v0 = v4[j][0], v1 = v4[j][1], v2 = v4[j][2], v3 = v4[j][3];
        // v0..v3: elements 8j .. 8j+7 as bf16 pairs (0,1) (2,3) (4,5) (6,7)
        xg.pair[j][0] = __builtin_amdgcn_perm(v2, v0, 0x05040100u);  // (8j+0, 8j+4)
        xg.pair[j][1] = __builtin_amdgcn_perm(v2, v0, 0x07060302u);  // (8j+1, 8j+5)
        xg.pair[j][2] = __builtin_amdgcn_perm(v3, v1, 0x05040100u);  // (8j+2, 8j+6)
        xg.pair[j][3] = __builtin_amdgcn_perm(v3, v1, 0x07060302u);  // (8j+3, 8j+7)
        s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v0), as_bf16x2(0x3F803F80u), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v1), as_bf16x2(0x3F803F80u), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v2), as_bf16x2(0x3F803F80u), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v3), as_bf16x2(0x3F803F80u), s, false);
    }
    xg.sum = s;
}

// sum over the group of x_k * (128 + q_k), f32 accumulation.
__device__ __forceinline__ float group_dot_biased(const u32x4& words, const XGroup& xg) {
    float d = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t word = words[j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(affine_pair_biased_bf16(word, i)), as_bf16x2(xg.pair[j][i]),
                                                d, false);
    }
    return d;
}

// Reduces R per-lane partial sums over the wavefront in log2(64) exchange
// steps: each of the first log2(R) steps halves the values a lane holds (the
// upper half of the lanes keeps the upper half of the rows), the rest add
// lane pairs. Afterwards lane l holds the full sum of row (l >> (6 - log2 R)).
template <int R>
__device__ __forceinline__ float wave_reduce_rows(float (&v)[R], int lane) {
    int off = 32;
#pragma unroll
    for (int cnt = R; cnt > 1; cnt >>= 1, off >>= 1) {
        const bool upper = (lane & off) != 0;
#pragma unroll
        for (int i = 0; i < cnt / 2; ++i) {
            const float keep = upper ? v[i + cnt / 2] : v[i];
            const float send = upper ? v[i] : v[i + cnt / 2];
            v[i] = keep + __shfl_xor(send, off, kWave);
        }
    }
    float t = v[0];
    for (; off >= 1; off >>= 1) t += __shfl_xor(t, off, kWave);
    return t;
}

// One wavefront computes R rows. K is covered in chunks of 64 groups (one
// group per lane); T chunks are loaded before any arithmetic so that every
// load of the wavefront is in flight at once. T = 0 selects a runtime loop
// over chunks (one chunk in flight at a time) for long K.
template <int R, int T>
__global__ __launch_bounds__(kWave) void qmv_affine4_kernel(
    const uint32_t* __restrict__ w, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int K, int N, int chunks) {
    const int lane = threadIdx.x;
    const int n0 = blockIdx.x * R;  // N % 32 == 0 and R | 32: rows n0 .. n0+R-1 exist
    const int G = K / 32;
    const size_t wrow = (size_t)(K / 8);

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;

    constexpr int TB = T > 0 ? T : 1;
    const int nch = T > 0 ? T : chunks;
    for (int t0 = 0; t0 < nch; t0 += TB) {
        u32x4 xr[TB][4];
        u32x4 wv[TB][R];
        uint32_t sv[TB][R], bv[TB][R];
        bool valid[TB];
        // x first (shared by all rows), then the weights, scales and biases.
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const int g = (t0 + t) * kWave + lane;
            valid[t] = g < G;
            const int gc = valid[t] ? g : G - 1;  // in-bounds address for idle lanes
            const u32x4* xp = reinterpret_cast<const u32x4*>(x + (size_t)gc * 32);
#pragma unroll
            for (int j = 0; j < 4; ++j) xr[t][j] = xp[j];
        }
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const int g = (t0 + t) * kWave + lane;
            const int gc = g < G ? g : G - 1;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const size_t row = (size_t)(n0 + r);
                wv[t][r] = *reinterpret_cast<const u32x4*>(w + row * wrow + (size_t)gc * 4);
                sv[t][r] = scales[row * G + gc];
                bv[t][r] = biases[row * G + gc];
            }
        }
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            XGroup xg;
            x_group_from_raw(xr[t], xg);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float s = bf16_bits_to_f32(sv[t][r]);
                const float b = bf16_bits_to_f32(bv[t][r]);
                const float d = group_dot_biased(wv[t][r], xg);
                const float part = __builtin_fmaf(s, d, __builtin_fmaf(-128.f, s, b) * xg.sum);
                acc[r] += valid[t] ? part : 0.f;
            }
        }
    }

    const float total = wave_reduce_rows<R>(acc, lane);
    constexpr int shift = 6 - (R == 1 ? 0 : R == 2 ? 1 : R == 4 ? 2 : R == 8 ? 3 : R == 16 ? 4 : 5);
    if ((lane & ((1 << shift) - 1)) == 0) y[n0 + (lane >> shift)] = f32_to_bf16_bits(total);
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
    constexpr int R = kGemvRows;
    const dim3 grid((unsigned)(N / R));
    const int G = (int)(K / 32);
    const int chunks = (G + kWave - 1) / kWave;
    hipStream_t s = as_stream(stream);
    switch (chunks) {
        case 1: hipLaunchKernelGGL((qmv_affine4_kernel<R, 1>), grid, dim3(kWave), 0, s, w, scales, biases, x, y, (int)K, (int)N, chunks); break;
        case 2: hipLaunchKernelGGL((qmv_affine4_kernel<R, 2>), grid, dim3(kWave), 0, s, w, scales, biases, x, y, (int)K, (int)N, chunks); break;
        case 3: hipLaunchKernelGGL((qmv_affine4_kernel<R, 3>), grid, dim3(kWave), 0, s, w, scales, biases, x, y, (int)K, (int)N, chunks); break;
        case 4: hipLaunchKernelGGL((qmv_affine4_kernel<R, 4>), grid, dim3(kWave), 0, s, w, scales, biases, x, y, (int)K, (int)N, chunks); break;
        default: hipLaunchKernelGGL((qmv_affine4_kernel<R, 0>), grid, dim3(kWave), 0, s, w, scales, biases, x, y, (int)K, (int)N, chunks); break;
    }
    return launch_status("qmv_affine4");
}
