// Device-side building blocks shared by the w4mi kernels (gfx950 only).
//
// Operand types for the CDNA4 matrix cores, the 4-bit decode routines every
// kernel and the unpack exports share, and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4mi {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef _Float16 f16x2 __attribute__((__vector_size__(2 * sizeof(_Float16))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

constexpr int kWave = 64;

// Reinterpret a 32-bit value as a packed pair. Always pass a plain scalar:
// hipcc (ROCm 7.2) mis-reads __builtin_bit_cast applied directly to a
// vector-element expression such as v[e] (it reads element 0).
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }
__device__ __forceinline__ f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// ---------------------------------------------------------------- 16-bit floats
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// Round-to-nearest-even narrowing (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2 r;
    r[0] = (_Float16)lo;
    r[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// ---------------------------------------------------------------- 4-bit decode
// Affine INT4 word (INT4 MatMulNBits page, kernel W load): eight weights
// k0..k0+7 of one row, nibble j at bits 4j..4j+3 (least significant first).
__device__ __forceinline__ uint32_t affine_nibble(uint32_t word, int j) { return (word >> (4 * j)) & 0xFu; }

// Eight nibbles of an affine word as f32 values 0..15, in k order.
__device__ __forceinline__ void affine_word_to_f32(uint32_t word, float (&q)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = (float)affine_nibble(word, j);
}

// ---------------------------------------------------------------- integer helpers
// A 32-bit constant held in a vector register (gfx9 VOP3 encodings take no
// literal and read at most one scalar register, so a three-operand integer
// op with two constants needs one of them in a VGPR).
__device__ __forceinline__ uint32_t vreg(uint32_t c) {
    uint32_t r = c;
    asm("" : "+v"(r));
    return r;
}

// (a & m) | c; with m and c in vector registers (vreg) the compiler selects
// one v_and_or_b32.
__device__ __forceinline__ uint32_t and_or_u32(uint32_t a, uint32_t m, uint32_t c) { return (a & m) | c; }

// ---------------------------------------------------------------- binary16 matrix-core operands
// The affine matrix-core kernels multiply in binary16, as the INT4
// MatMulNBits page's kernel does (module doc "Algorithm": bf16 activations
// cast to half, weights dequantized into half tiles, float accumulation).

// Smallest magnitude that rounds to infinity in binary16 (65504 + half an ulp).
constexpr float kF16Overflow = 65520.f;
// True for a finite value that binary16 cannot hold (it would become an
// infinity); infinities and NaN are not counted.
__device__ __forceinline__ bool out_of_f16_range(float v) {
    const float a = __builtin_fabsf(v);
    return a >= kF16Overflow && a <= 3.4028235e38f;
}

// A bf16 pair (one dword, element 0 in the low half) as a binary16 pair,
// round to nearest even. Exact for magnitudes in [2^-14, 65504] and zero;
// smaller ones keep binary16's subnormal step (2^-24); 65520 and above
// become infinity.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t d) {
    return pack_f16x2(__uint_as_float(d << 16), __uint_as_float(d & 0xFFFF0000u));
}
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(const u32x4& v) {
    return u32x4{bf16x2_to_f16x2(v[0]), bf16x2_to_f16x2(v[1]), bf16x2_to_f16x2(v[2]), bf16x2_to_f16x2(v[3])};
}

// Per-group constants of affine_word_f16: with s, b the group's scale and
// bias, c = b - 1024 s, s16 = s / 16, c16 = b - 64 s.
struct AffineGroupF16 {
    float s, c, s16, c16;
};
__device__ __forceinline__ AffineGroupF16 affine_group_f16(float s, float b) {
    return AffineGroupF16{s, __builtin_fmaf(-1024.f, s, b), 0.0625f * s, __builtin_fmaf(-64.f, s, b)};
}
// Eight affine weights of one word (k = 8j .. 8j + 7) as binary16 pairs in k
// order, w = q s + b rounded to binary16. One AND-OR per nibble pair places
// the nibble in a binary16 mantissa under the exponent of 1024 (magic
// 0x6400): the even nibbles of a byte read as 1024 + q, the odd ones (bits
// 4..7) as 1024 + 16 q; a fused multiply-add then forms (1024 + q) s +
// (b - 1024 s) or (1024 + 16 q) s/16 + (b - 64 s) in f32 and that is rounded
// to binary16. The f32 value is q s + b exactly when b = 0 or |b| lies within
// 2^-6 .. 2^15 of |s| (both terms then fit f32's 24 bits), so the weight is
// q s + b rounded once; outside that band the f32 step can round first (by at
// most 2^-14 |s| below it, 2^-22 |b| above it). F32: the eight sums round in f32 registers and
// v_cvt_pk_f16_f32 packs them (v_fma_mix_f32 issues in about 3.4 cycles per
// wave64 instruction, the half-writing v_fma_mix{lo,hi}_f16 in 5.9);
// otherwise they round straight into register halves (fewer registers). Both
// give the same bits. m_lo = 0x000F000F, m_hi = 0x00F000F0, magic =
// 0x64006400 in vector registers (vreg).
template <bool F32 = false>
__device__ __forceinline__ u32x4 affine_word_f16(uint32_t word, const AffineGroupF16& g, uint32_t m_lo, uint32_t m_hi,
                                                 uint32_t magic) {
    const uint32_t w8 = word >> 8;
    const f16x2 p0 = as_f16x2(and_or_u32(word, m_lo, magic));  // 1024 + n0, 1024 + n4
    const f16x2 p1 = as_f16x2(and_or_u32(word, m_hi, magic));  // 1024 + 16 n1, 1024 + 16 n5
    const f16x2 p2 = as_f16x2(and_or_u32(w8, m_lo, magic));    // 1024 + n2, 1024 + n6
    const f16x2 p3 = as_f16x2(and_or_u32(w8, m_hi, magic));    // 1024 + 16 n3, 1024 + 16 n7
    if constexpr (F32) {
        float f0 = __builtin_fmaf((float)p0[0], g.s, g.c), f1 = __builtin_fmaf((float)p1[0], g.s16, g.c16);
        float f2 = __builtin_fmaf((float)p2[0], g.s, g.c), f3 = __builtin_fmaf((float)p3[0], g.s16, g.c16);
        float f4 = __builtin_fmaf((float)p0[1], g.s, g.c), f5 = __builtin_fmaf((float)p1[1], g.s16, g.c16);
        float f6 = __builtin_fmaf((float)p2[1], g.s, g.c), f7 = __builtin_fmaf((float)p3[1], g.s16, g.c16);
        // opaque to the compiler, which would otherwise fold each rounding
        // back into a half-writing v_fma_mix
        asm("" : "+v"(f0), "+v"(f1), "+v"(f2), "+v"(f3), "+v"(f4), "+v"(f5), "+v"(f6), "+v"(f7));
        return u32x4{pack_f16x2(f0, f1), pack_f16x2(f2, f3), pack_f16x2(f4, f5), pack_f16x2(f6, f7)};
    } else {
        f16x2 r0, r1, r2, r3;
        r0[0] = (_Float16)__builtin_fmaf((float)p0[0], g.s, g.c);
        r0[1] = (_Float16)__builtin_fmaf((float)p1[0], g.s16, g.c16);
        r1[0] = (_Float16)__builtin_fmaf((float)p2[0], g.s, g.c);
        r1[1] = (_Float16)__builtin_fmaf((float)p3[0], g.s16, g.c16);
        r2[0] = (_Float16)__builtin_fmaf((float)p0[1], g.s, g.c);
        r2[1] = (_Float16)__builtin_fmaf((float)p1[1], g.s16, g.c16);
        r3[0] = (_Float16)__builtin_fmaf((float)p2[1], g.s, g.c);
        r3[1] = (_Float16)__builtin_fmaf((float)p3[1], g.s16, g.c16);
        return u32x4{as_u32(r0), as_u32(r1), as_u32(r2), as_u32(r3)};
    }
}

// ---------------------------------------------------------------- lookup-codebook table decode
// The half-precision lookup matmul's weight decode (lut4 page: value =
// fp16(book[code] * scale), code of flat index i = high nibble of byte i / 2
// for even i, low nibble for odd i). A lane builds its block's 16 table
// entries T[c] = fp16(book[c] * s) as byte planes and looks codes up four at
// a time with v_perm_b32.
struct Book16 {
    float v[16];
};
// The 16 table entries as byte planes: lo[j] holds the low bytes of entries
// 4j .. 4j + 3, hi[j] the high bytes.
struct LutPlanes {
    uint32_t lo[4], hi[4];
};
__device__ __forceinline__ LutPlanes lut_planes(const Book16& book, float s) {
    uint32_t t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = pack_f16x2(book.v[2 * i] * s, book.v[2 * i + 1] * s);
    LutPlanes P;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        P.lo[j] = __builtin_amdgcn_perm(t[2 * j + 1], t[2 * j], 0x06040200u);
        P.hi[j] = __builtin_amdgcn_perm(t[2 * j + 1], t[2 * j], 0x07050301u);
    }
    return P;
}
// Looks up four codes (one per byte, 0..15): returns the low and high bytes
// of their table entries. Selector byte 12 reads 0x00 and 13 reads 0xFF,
// which turns bit 3 of each code into a byte mask.
__device__ __forceinline__ void lut_lookup4(uint32_t codes, const LutPlanes& P, uint32_t& lo, uint32_t& hi) {
    const uint32_t sel = codes & 0x07070707u;
    const uint32_t mask = __builtin_amdgcn_perm(0u, 0u, ((codes >> 3) & 0x01010101u) | 0x0C0C0C0Cu);
    const uint32_t lo_a = __builtin_amdgcn_perm(P.lo[1], P.lo[0], sel), lo_b = __builtin_amdgcn_perm(P.lo[3], P.lo[2], sel);
    const uint32_t hi_a = __builtin_amdgcn_perm(P.hi[1], P.hi[0], sel), hi_b = __builtin_amdgcn_perm(P.hi[3], P.hi[2], sel);
    lo = (mask & lo_b) | (~mask & lo_a);
    hi = (mask & hi_b) | (~mask & hi_a);
}
// Eight weights k .. k + 7 from one packed dword (byte j: code of k + 2j in
// the high nibble, of k + 2j + 1 in the low one) as four fp16 pairs.
__device__ __forceinline__ u32x4 lut_decode8(uint32_t word, const LutPlanes& P) {
    uint32_t elo, ehi, olo, ohi;
    lut_lookup4((word >> 4) & 0x0F0F0F0Fu, P, elo, ehi);  // k, k + 2, k + 4, k + 6
    lut_lookup4(word & 0x0F0F0F0Fu, P, olo, ohi);         // k + 1, k + 3, k + 5, k + 7
    const uint32_t a0 = __builtin_amdgcn_perm(olo, elo, 0x05010400u), b0 = __builtin_amdgcn_perm(ohi, ehi, 0x05010400u);
    const uint32_t a1 = __builtin_amdgcn_perm(olo, elo, 0x07030602u), b1 = __builtin_amdgcn_perm(ohi, ehi, 0x07030602u);
    return u32x4{__builtin_amdgcn_perm(b0, a0, 0x05010400u), __builtin_amdgcn_perm(b0, a0, 0x07030602u),
                 __builtin_amdgcn_perm(b1, a1, 0x05010400u), __builtin_amdgcn_perm(b1, a1, 0x07030602u)};
}

// The single-precision lookup path's dword decode: a lane reads 8 codes (one
// dword) and looks them up in an LDS copy of the codebook. Byte t of the dword holds flat indices 2t (high
// nibble) and 2t + 1 (low nibble); the lookup offsets are taken as bytes of two
// masked copies of the dword, (word >> 2) and (word << 2) masked to 4 x code,
// hidden from the compiler, which would otherwise fold each pick back into a
// shift and a mask of the word.
__device__ __forceinline__ void lut_offsets(uint32_t word, uint32_t& hi4, uint32_t& lo4) {
    hi4 = (word >> 2) & 0x3C3C3C3Cu;
    lo4 = (word << 2) & 0x3C3C3C3Cu;
    asm("" : "+v"(hi4), "+v"(lo4));
}
// Codebook entry of column c (0..7) of a dword whose offsets are hi4 / lo4.
__device__ __forceinline__ float lut_entry(const float* book_s, uint32_t hi4, uint32_t lo4, int c) {
    const uint32_t off = (((c & 1) ? lo4 : hi4) >> (8 * (c / 2))) & 0xFFu;
    return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(book_s) + off);
}

// ---------------------------------------------------------------- buffer resources
// Raw buffer resource over [base, base + bytes): loads through it take a
// scalar offset per instruction and a 32-bit lane offset, and return zero
// past the end. The third descriptor word is the gfx9 raw-buffer setting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Pair form used by the decode GEMV: bf16 pairs holding 128 + q for nibbles
// (i, i + 4), i = 0..3, of an affine word. 128 + q (q <= 15) is exact in bf16
// (8 significant bits), so a bf16 dot product with these pairs yields
// sum (128 + q) x exactly up to f32 accumulation. mask = 0x000F000F and
// bias = 0x43004300 (bf16 128.0 twice), passed in vector registers.
__device__ __forceinline__ uint32_t affine_pair_biased_bf16(uint32_t word, int i, uint32_t mask, uint32_t bias) {
    return and_or_u32(i == 0 ? word : word >> (4 * i), mask, bias);
}
constexpr uint32_t kAffinePairMask = 0x000F000Fu;
constexpr uint32_t kAffinePairBias = 0x43004300u;

// The same four pairs for two words at once (p[h][i] = pair i of word h): a
// single 64-bit shift of (w1:w0) by 4i brings nibbles i and i + 4 of both
// words down. The bits of w1 that the shift moves into the low word land at
// bit 28 and above (i = 1), 24 (2) or 20 (3), outside the mask. One
// v_lshrrev_b64 in place of two 32-bit shifts; written as an instruction
// because the compiler splits a 64-bit shift whose result is masked.
__device__ __forceinline__ void affine_pairs2_biased_bf16(uint32_t w0, uint32_t w1, uint32_t mask, uint32_t bias,
                                                          uint32_t (&p)[2][4]) {
    const uint64_t v = ((uint64_t)w1 << 32) | w0;
    p[0][0] = and_or_u32(w0, mask, bias);
    p[1][0] = and_or_u32(w1, mask, bias);
#pragma unroll
    for (int i = 1; i < 4; ++i) {
        uint64_t s;
        asm("v_lshrrev_b64 %0, %1, %2" : "=v"(s) : "i"(4 * i), "v"(v));
        p[0][i] = and_or_u32((uint32_t)s, mask, bias);
        p[1][i] = and_or_u32((uint32_t)(s >> 32), mask, bias);
    }
}

// Lookup-codebook index order (lut4 page, decode kernel): flat index i uses
// the HIGH nibble of byte i/2 when i is even, the LOW nibble when i is odd.
__device__ __forceinline__ uint32_t lut_code(uint32_t byte, uint32_t i) {
    return (i & 1u) ? (byte & 0xFu) : (byte >> 4);
}

// GGML Q4_0 block: element i < 16 is the low nibble of qs[i], element i + 16
// its high nibble. One qs dword (bytes 4i..4i+3 of a block) as four fp16
// pairs for products against x pairs in the matching order, one shift and
// four AND-ORs: low nibbles sit at bits 0..3 of a binary16 whose exponent
// makes 1024 + q, high nibbles at bits 4..7 of one whose exponent makes
// 64 + q (ulp 1/16, so 16 q / 16 = q); all exact.
//   out[0] = (4i, 4i+2)        as 1024 + q
//   out[1] = (16+4i, 16+4i+2)  as 64 + q
//   out[2] = (4i+1, 4i+3)      as 1024 + q
//   out[3] = (16+4i+1, 16+4i+3) as 64 + q
// lo = 0x000F000F, hi = 0x00F000F0, m_lo = 0x64006400, m_hi = 0x54005400 in
// vector registers (vreg).
__device__ __forceinline__ void q4_0_dot_pairs(uint32_t qs, uint32_t lo, uint32_t hi, uint32_t m_lo, uint32_t m_hi,
                                               uint32_t (&out)[4]) {
    const uint32_t s8 = qs >> 8;
    out[0] = and_or_u32(qs, lo, m_lo);
    out[1] = and_or_u32(qs, hi, m_hi);
    out[2] = and_or_u32(s8, lo, m_lo);
    out[3] = and_or_u32(s8, hi, m_hi);
}
constexpr float kQ4DotBiasLo = 1032.f;  // 1024 + 8: removes the low-nibble magic and GGML's offset 8
constexpr float kQ4DotBiasHi = 72.f;    // 64 + 8

// Two consecutive Q4_0 blocks (36 bytes, read as nine 4-byte-aligned dwords):
// block A is bytes 0..17 (d at 0, qs at 2), block B bytes 18..35 (d at 18,
// qs at 20). Returns both scales' binary16 bits and both qs as aligned dwords.
__device__ __forceinline__ void q4_0_split_pair(const uint32_t (&raw)[9], uint32_t& dA, uint32_t& dB,
                                                uint32_t (&qsA)[4], uint32_t (&qsB)[4]) {
    dA = raw[0] & 0xFFFFu;
    dB = raw[4] >> 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        qsA[i] = __builtin_amdgcn_alignbyte(raw[i + 1], raw[i], 2);
        qsB[i] = raw[5 + i];
    }
}

// ---------------------------------------------------------------- reductions
// Sum over the 64 lanes of a wavefront; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

}  // namespace w4mi
