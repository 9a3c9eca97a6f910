// Unpack exports: write out, one byte per weight, the 4-bit codes the hot
// kernels decode, through the same device decode routines they use, so the
// decode can be checked bit for bit.
#include "w4mi_device.hpp"
#include "w4mi_host.hpp"

namespace w4mi {

constexpr int kUnpackThreads = 256;

// One thread per affine word. Both decoders in use are applied: the nibble
// extraction of the GEMM (affine_nibble) and the biased bf16 pairs of the
// GEMV; a disagreement is written as 0xFF so it cannot pass a bit-exact check.
__global__ void unpack_affine_kernel(const uint32_t* __restrict__ w, uint8_t* __restrict__ q, int64_t words) {
    const int64_t i = (int64_t)blockIdx.x * kUnpackThreads + threadIdx.x;
    if (i >= words) return;
    const uint32_t word = w[i];
    const uint32_t mask = vreg(kAffinePairMask), bias = vreg(kAffinePairBias);
    uint8_t out[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t pair = affine_pair_biased_bf16(word, p, mask, bias);  // nibbles p (low half) and p + 4 (high half)
        out[p] = (uint8_t)(pair & 0xFu);
        out[p + 4] = (uint8_t)((pair >> 16) & 0xFu);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) q[i * 8 + j] = (out[j] == affine_nibble(word, j)) ? out[j] : (uint8_t)0xFF;
}

__global__ void unpack_lut_kernel(const uint8_t* __restrict__ packed, uint8_t* __restrict__ codes, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * kUnpackThreads + threadIdx.x;
    if (i >= count) return;
    codes[i] = (uint8_t)lut_code(packed[i / 2], (uint32_t)(i & 1));
}

// One thread per block pair (64 weights), reading the nine dwords the
// grouped GEMM reads and splitting them the same way.
__global__ void unpack_q4_0_kernel(const uint8_t* __restrict__ w, uint8_t* __restrict__ q, uint16_t* __restrict__ d,
                                   int64_t pairs_total, int pairs_per_row) {
    const int64_t i = (int64_t)blockIdx.x * kUnpackThreads + threadIdx.x;
    if (i >= pairs_total) return;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(w + i * 36);
    uint32_t raw[9];
#pragma unroll
    for (int j = 0; j < 9; ++j) raw[j] = src[j];
    uint32_t dA, dB, qsA[4], qsB[4];
    q4_0_split_pair(raw, dA, dB, qsA, qsB);
    const int64_t row = i / pairs_per_row, pr = i % pairs_per_row;
    const int64_t K = (int64_t)pairs_per_row * 64;
    uint8_t* qo = q + row * K + pr * 64;
    d[i * 2] = (uint16_t)dA;
    d[i * 2 + 1] = (uint16_t)dB;
    const uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u, m_lo = 0x64006400u, m_hi = 0x54005400u;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) {
            // the grouped GEMM's and the mat-vec route's decode: 1024 + q for
            // low nibbles, 64 + q (nibble in mantissa bits 4..7) for high ones
            uint32_t pairs[4];
            q4_0_dot_pairs(b == 0 ? qsA[dw] : qsB[dw], lo, hi, m_lo, m_hi, pairs);
            uint8_t* o = qo + b * 32;
            o[4 * dw + 0] = pairs[0] & 0xFu;
            o[4 * dw + 2] = (pairs[0] >> 16) & 0xFu;
            o[16 + 4 * dw + 0] = (pairs[1] >> 4) & 0xFu;
            o[16 + 4 * dw + 2] = (pairs[1] >> 20) & 0xFu;
            o[4 * dw + 1] = pairs[2] & 0xFu;
            o[4 * dw + 3] = (pairs[2] >> 16) & 0xFu;
            o[16 + 4 * dw + 1] = (pairs[3] >> 4) & 0xFu;
            o[16 + 4 * dw + 3] = (pairs[3] >> 20) & 0xFu;
        }
}

static unsigned blocks_for(int64_t n) { return (unsigned)((n + kUnpackThreads - 1) / kUnpackThreads); }

}  // namespace w4mi

using namespace w4mi;

extern "C" w4_status w4_unpack_affine(const uint32_t* w, uint8_t* q, int64_t N, int64_t K, void* stream) {
    if (N < 0 || K < 0 || K % 8 != 0) return fail(W4_EINVAL, "w4_unpack_affine: need N, K >= 0 and K %% 8 == 0");
    if (N == 0 || K == 0) return W4_OK;
    if (!w || !q) return fail(W4_EINVAL, "w4_unpack_affine: null pointer argument");
    const int64_t words = N * (K / 8);
    hipLaunchKernelGGL(unpack_affine_kernel, dim3(blocks_for(words)), dim3(kUnpackThreads), 0, as_stream(stream), w, q,
                       words);
    return launch_status("w4_unpack_affine");
}

extern "C" w4_status w4_unpack_lut(const uint8_t* packed, uint8_t* codes, int64_t count, void* stream) {
    if (count < 0) return fail(W4_EINVAL, "w4_unpack_lut: count must be >= 0");
    if (count == 0) return W4_OK;
    if (!packed || !codes) return fail(W4_EINVAL, "w4_unpack_lut: null pointer argument");
    hipLaunchKernelGGL(unpack_lut_kernel, dim3(blocks_for(count)), dim3(kUnpackThreads), 0, as_stream(stream), packed,
                       codes, count);
    return launch_status("w4_unpack_lut");
}

extern "C" w4_status w4_unpack_q4_0(const uint8_t* w, uint8_t* q, uint16_t* d, int64_t rows, int64_t K, void* stream) {
    if (rows < 0 || K < 0 || K % 64 != 0) return fail(W4_EINVAL, "w4_unpack_q4_0: need rows, K >= 0 and K %% 64 == 0");
    if (rows == 0 || K == 0) return W4_OK;
    if (!w || !q || !d) return fail(W4_EINVAL, "w4_unpack_q4_0: null pointer argument");
    if ((uintptr_t)w & 3u) return fail(W4_EINVAL, "w4_unpack_q4_0: w must be 4-byte aligned");
    const int pairs_per_row = (int)(K / 64);
    const int64_t pairs = rows * pairs_per_row;
    hipLaunchKernelGGL(unpack_q4_0_kernel, dim3(blocks_for(pairs)), dim3(kUnpackThreads), 0, as_stream(stream), w, q, d,
                       pairs, pairs_per_row);
    return launch_status("w4_unpack_q4_0");
}
