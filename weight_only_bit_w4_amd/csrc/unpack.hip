// Unpack exports: write out, one byte per weight, the 4-bit codes the hot
// kernels decode, through the same device decode routines they use
// (w4mi_device.hpp), so the decode can be checked bit for bit.
#include "w4mi_device.hpp"
#include "w4mi_host.hpp"

namespace w4mi {

constexpr int kUnpackThreads = 256;

// One thread per affine word. Every affine decoder the kernels run is
// applied and must agree, else the code is written as 0xFF (which cannot
// pass a bit-exact check): the nibble extraction of the small-shape GEMM
// (affine_nibble), the biased bf16 pairs of the GEMV forms, one word at a
// time (affine_pair_biased_bf16) and two at a time with the word's real
// neighbours (affine_pairs2_biased_bf16, as the low word ahead of the next
// word and as the high word after the previous one), and the binary16 word
// decode of the prefill and weight-tile kernels (affine_word_f16 with scale
// 1 and bias 0, which gives q exactly, in both its forms: rounded in f32
// registers and straight into register halves).
__global__ void unpack_affine_kernel(const uint32_t* __restrict__ w, uint8_t* __restrict__ q, int64_t words) {
    const int64_t i = (int64_t)blockIdx.x * kUnpackThreads + threadIdx.x;
    if (i >= words) return;
    const uint32_t word = w[i];
    const uint32_t next = i + 1 < words ? w[i + 1] : ~word, prev = i > 0 ? w[i - 1] : ~word;
    const uint32_t mask = vreg(kAffinePairMask), bias = vreg(kAffinePairBias);
    uint32_t lo[2][4], hi[2][4];
    affine_pairs2_biased_bf16(word, next, mask, bias, lo);  // word as the low word
    affine_pairs2_biased_bf16(prev, word, mask, bias, hi);  // word as the high word
    uint8_t out[8];
    bool pairs_agree = true;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t pair = affine_pair_biased_bf16(word, p, mask, bias);  // nibbles p (low half) and p + 4 (high half)
        pairs_agree = pairs_agree && lo[0][p] == pair && hi[1][p] == pair;
        out[p] = (uint8_t)(pair & 0xFu);
        out[p + 4] = (uint8_t)((pair >> 16) & 0xFu);
    }
    const AffineGroupF16 unit = affine_group_f16(1.f, 0.f);
    const u32x4 h = affine_word_f16<false>(word, unit, vreg(0x000F000Fu), vreg(0x00F000F0u), vreg(0x64006400u));
    const u32x4 h32 = affine_word_f16<true>(word, unit, vreg(0x000F000Fu), vreg(0x00F000F0u), vreg(0x64006400u));
    const bool forms_agree = h[0] == h32[0] && h[1] == h32[1] && h[2] == h32[2] && h[3] == h32[3];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t bits = (j & 1) ? (h[j / 2] >> 16) : (h[j / 2] & 0xFFFFu);
        const float v = f16_bits_to_f32(bits);
        const bool same = pairs_agree && forms_agree && out[j] == affine_nibble(word, j) && v == (float)out[j];
        q[i * 8 + j] = same ? out[j] : (uint8_t)0xFF;
    }
}

// One thread per 8 codes (flat indices 8 t .. 8 t + 7, the bytes 4 t ..
// 4 t + 3). Every lookup decoder the kernels run is applied and must agree,
// else 0xFF: the per-element code (lut_code), the half-precision matrix-core
// decode (lut_decode8 on the byte-plane table of book[c] = c, scale 1, whose
// binary16 entries are the codes exactly) and the single-precision path's
// dword lookup in an LDS codebook (lut_offsets / lut_entry, book[c] = c).
__global__ void unpack_lut_kernel(const uint8_t* __restrict__ packed, uint8_t* __restrict__ codes, int64_t count) {
    __shared__ float book_s[16];
    if (threadIdx.x < 16) book_s[threadIdx.x] = (float)threadIdx.x;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * kUnpackThreads + threadIdx.x;
    const int64_t base = 8 * t;
    if (base >= count) return;
    const int64_t nbytes = (count + 1) / 2;
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        if (4 * t + b < nbytes) word |= (uint32_t)packed[4 * t + b] << (8 * b);
    Book16 ident;
#pragma unroll
    for (int c = 0; c < 16; ++c) ident.v[c] = (float)c;
    const u32x4 h = lut_decode8(word, lut_planes(ident, 1.f));
    uint32_t hi4, lo4;
    lut_offsets(word, hi4, lo4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (base + j >= count) break;
        const uint32_t c = lut_code((word >> (8 * (j / 2))) & 0xFFu, (uint32_t)j);
        const uint32_t bits = (j & 1) ? (h[j / 2] >> 16) : (h[j / 2] & 0xFFFFu);
        const bool same = f16_bits_to_f32(bits) == (float)c && lut_entry(book_s, hi4, lo4, j) == (float)c;
        codes[base + j] = same ? (uint8_t)c : (uint8_t)0xFF;
    }
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
    hipLaunchKernelGGL(unpack_lut_kernel, dim3(blocks_for((count + 7) / 8)), dim3(kUnpackThreads), 0, as_stream(stream),
                       packed, codes, count);
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
