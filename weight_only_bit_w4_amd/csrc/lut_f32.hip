// qmm_lut4_f32: the lookup-codebook matmul in single precision (lut4 page:
// the mlx_lookup4_matmul kernel that execute() takes when the compute type is
// f32 and the batch is small, and the CPU branch, both with the decoded
// weight left unrounded). For both weight layouts
//   y[m][n] = sum_k x[m][k] * W(n, k),   W = book[code(flat)] * scale[flat / block] (f32),
//   flat = n * K + k (transpose != 0, W stored [N, K]) or k * N + n (W stored [K, N]),
//   code(flat) = high nibble of packed[flat / 2] for even flat, low nibble for odd.
// Blocks run over the flat index, so they may straddle rows; any K, N and
// even block are taken. Each output's products are summed in 16-step K tiles
// whose partial sums are added with compensation (the page's kernel keeps a
// correction term the same way), then the partial results of the lanes (or
// wavefronts) that split K are added.
//
// Two lane maps, each reading the packed codes of its layout with consecutive
// lanes at consecutive flat indices:
//  - [N, K] (transpose): a wavefront owns 4 weight rows; lane l takes k = l,
//    l + 64, ...; x is read with the same lanes; the 64 lanes' sums are
//    reduced at the end.
//  - [K, N]: lane l owns column n0 + l; 16 wavefronts split K into contiguous
//    ranges; x[m][k] is the same for every lane (scalar loads); the 16
//    wavefronts' sums meet in LDS and are added in K order, compensated.
// Rows of x are taken 4 at a time (the grid's y dimension).
#include "w4mi_device.hpp"
#include "w4mi_host.hpp"

namespace w4mi {

constexpr int kF32M = 4;      // rows of x per workgroup
constexpr int kF32Tile = 16;  // products summed before each compensated add
constexpr int kF32RowWaves = 4, kF32Rows = 4;  // [N, K]: 4 wavefronts x 4 weight rows
constexpr int kF32ColWaves = 16;               // [K, N]: 16 wavefronts over K

struct LutBook {
    float v[16];
};

// acc += part with the running correction cor (the page's compensated step:
// a non-finite sum leaves no correction).
__device__ __forceinline__ void kahan_add(float& acc, float& cor, float part) {
    const float value = part - cor;
    const float added = acc + value;
    cor = __builtin_isfinite(added) ? (added - acc) - value : 0.f;
    acc = added;
}

// flat / block and flat % block, advanced by a fixed step without dividing.
struct BlockCursor {
    int64_t q;
    int32_t r;
    __device__ __forceinline__ void init(int64_t flat, int32_t block) {
        q = flat / block;
        r = (int32_t)(flat - q * block);
    }
    __device__ __forceinline__ void advance(int64_t step_q, int32_t step_r, int32_t block) {
        q += step_q;
        r += step_r;
        if (r >= block) {
            r -= block;
            ++q;
        }
    }
};

__device__ __forceinline__ float lut_weight(const uint8_t* __restrict__ packed, const float* __restrict__ scales,
                                            const float* book_s, int64_t flat, int64_t scale_index) {
    const uint32_t byte = packed[flat >> 1];
    const uint32_t code = (flat & 1) ? (byte & 15u) : (byte >> 4);
    return book_s[code] * scales[scale_index];
}

__global__ __launch_bounds__(kF32RowWaves * 64) void lut4_f32_rows_kernel(const float* __restrict__ x,
                                                                            const uint8_t* __restrict__ packed,
                                                                            const float* __restrict__ scales,
                                                                            LutBook book, float* __restrict__ y,
                                                                            int M, int K, int N, int block) {
    __shared__ float book_s[16];
    if (threadIdx.x < 16) book_s[threadIdx.x] = book.v[threadIdx.x];
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nb = (blockIdx.x * kF32RowWaves + wave) * kF32Rows;
    const int m0 = blockIdx.y * kF32M;
    float acc[kF32Rows][kF32M], cor[kF32Rows][kF32M], part[kF32Rows][kF32M];
    BlockCursor cur[kF32Rows];
#pragma unroll
    for (int r = 0; r < kF32Rows; ++r) {
        cur[r].init((int64_t)min(nb + r, N - 1) * K + lane, block);
#pragma unroll
        for (int m = 0; m < kF32M; ++m) acc[r][m] = cor[r][m] = part[r][m] = 0.f;
    }
    const int64_t sq = 64 / block;
    const int32_t sr = 64 % block;
    int it = 0;
    for (int k0 = 0; k0 < K; k0 += 64) {
        const int k = k0 + lane;
        const bool kv = k < K;
        float xv[kF32M];
#pragma unroll
        for (int m = 0; m < kF32M; ++m) xv[m] = (kv && m0 + m < M) ? x[(size_t)(m0 + m) * K + k] : 0.f;
#pragma unroll
        for (int r = 0; r < kF32Rows; ++r) {
            const int n = nb + r;
            const float w = (kv && n < N) ? lut_weight(packed, scales, book_s, (int64_t)n * K + k, cur[r].q) : 0.f;
#pragma unroll
            for (int m = 0; m < kF32M; ++m) part[r][m] = __builtin_fmaf(xv[m], w, part[r][m]);
            cur[r].advance(sq, sr, block);
        }
        if (++it == kF32Tile) {
            it = 0;
#pragma unroll
            for (int r = 0; r < kF32Rows; ++r)
#pragma unroll
                for (int m = 0; m < kF32M; ++m) {
                    kahan_add(acc[r][m], cor[r][m], part[r][m]);
                    part[r][m] = 0.f;
                }
        }
    }
#pragma unroll
    for (int r = 0; r < kF32Rows; ++r)
#pragma unroll
        for (int m = 0; m < kF32M; ++m) {
            kahan_add(acc[r][m], cor[r][m], part[r][m]);
            float v = acc[r][m];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            const int n = nb + r;
            if (lane == 0 && n < N && m0 + m < M) y[(size_t)(m0 + m) * N + n] = v;
        }
}

__global__ __launch_bounds__(kF32ColWaves * 64) void lut4_f32_cols_kernel(const float* __restrict__ x,
                                                                            const uint8_t* __restrict__ packed,
                                                                            const float* __restrict__ scales,
                                                                            LutBook book, float* __restrict__ y,
                                                                            int M, int K, int N, int block) {
    __shared__ float book_s[16];
    __shared__ float red[kF32ColWaves][kF32M][64];
    if (threadIdx.x < 16) book_s[threadIdx.x] = book.v[threadIdx.x];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = blockIdx.x * 64 + lane;
    const bool nv = n < N;
    const int m0 = blockIdx.y * kF32M;
    const int span = (K + kF32ColWaves - 1) / kF32ColWaves;
    const int kb = min(K, wave * span), ke = min(K, kb + span);
    float acc[kF32M], cor[kF32M], part[kF32M];
#pragma unroll
    for (int m = 0; m < kF32M; ++m) acc[m] = cor[m] = part[m] = 0.f;
    BlockCursor cur;
    cur.init((int64_t)kb * N + (nv ? n : 0), block);
    const int64_t sq = N / block;
    const int32_t sr = N % block;
    int it = 0;
    for (int k = kb; k < ke; ++k) {
        const float w = nv ? lut_weight(packed, scales, book_s, (int64_t)k * N + n, cur.q) : 0.f;
#pragma unroll
        for (int m = 0; m < kF32M; ++m) {
            const float xv = m0 + m < M ? x[(size_t)(m0 + m) * K + k] : 0.f;  // the same for every lane
            part[m] = __builtin_fmaf(xv, w, part[m]);
        }
        cur.advance(sq, sr, block);
        if (++it == kF32Tile) {
            it = 0;
#pragma unroll
            for (int m = 0; m < kF32M; ++m) {
                kahan_add(acc[m], cor[m], part[m]);
                part[m] = 0.f;
            }
        }
    }
#pragma unroll
    for (int m = 0; m < kF32M; ++m) {
        kahan_add(acc[m], cor[m], part[m]);
        red[wave][m][lane] = acc[m];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int m = 0; m < kF32M; ++m) {
            float a = 0.f, c = 0.f;
            for (int v = 0; v < kF32ColWaves; ++v) kahan_add(a, c, red[v][m][lane]);  // K order
            if (nv && m0 + m < M) y[(size_t)(m0 + m) * N + n] = a;
        }
    }
}

}  // namespace w4mi

using namespace w4mi;

extern "C" w4_status qmm_lut4_f32(const float* x, const uint8_t* packed, const float* scales, const float* book, float* y,
                                  int64_t M, int64_t K, int64_t N, int32_t block, int32_t transpose, void* stream) {
    w4_status st = w4_check_lut_f32(M, K, N, block, transpose);
    if (st != W4_OK) return st;
    if (M == 0) return W4_OK;
    if (!x || !packed || !scales || !book || !y) return fail(W4_EINVAL, "qmm_lut4_f32: null pointer argument");
    if (((uintptr_t)x & 3u) || ((uintptr_t)scales & 3u) || ((uintptr_t)y & 3u))
        return fail(W4_EINVAL, "qmm_lut4_f32: x, scales and y must be 4-byte aligned");
    LutBook b;
    for (int i = 0; i < 16; ++i) b.v[i] = book[i];
    hipStream_t s = as_stream(stream);
    const unsigned my = (unsigned)((M + kF32M - 1) / kF32M);
    if (transpose) {
        const dim3 grid((unsigned)((N + kF32RowWaves * kF32Rows - 1) / (kF32RowWaves * kF32Rows)), my);
        hipLaunchKernelGGL(lut4_f32_rows_kernel, grid, dim3(kF32RowWaves * 64), 0, s, x, packed, scales, b, y, (int)M,
                           (int)K, (int)N, (int)block);
    } else {
        const dim3 grid((unsigned)((N + 63) / 64), my);
        hipLaunchKernelGGL(lut4_f32_cols_kernel, grid, dim3(kF32ColWaves * 64), 0, s, x, packed, scales, b, y, (int)M,
                           (int)K, (int)N, (int)block);
    }
    return launch_status("qmm_lut4_f32");
}
