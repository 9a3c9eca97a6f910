// MFMA GEMMs with a fused 4-bit weight decode:
//   qmm_affine4 - y[M,N] bf16 = x[M,K] bf16 . (q*s + b)^T   (INT4 MatMulNBits
//                 page, prefill M > 1; bf16 operands, f32 accumulation)
//   qmm_lut4    - y[M,N] fp16 = x[M,K] fp16 . fp16(book[c]*scale)^T
//                 (lut4 page, decode + GEMM route; fp16 operands, f32 acc)
//
// One skeleton serves both: a workgroup of 4 wavefronts computes a BM x BN
// output tile; per K-step of 32 (one affine quantisation group) it stages the
// x tile (BM x 32) and the decoded weight tile (BN x 32, decoded once per
// workgroup in registers and written as 16-bit operands) in LDS, double
// buffered so the next step's global loads overlap this step's matrix-core
// work, with one barrier per step. Each wavefront owns a (16 FM) x (16 FN)
// sub-tile and issues v_mfma_f32_16x16x32_{bf16,f16}; LDS rows are padded
// to 80 bytes so the 16-byte operand reads of a 16-lane group hit distinct
// banks.
#include "w4mi_device.hpp"
#include "w4mi_host.hpp"

namespace w4mi {

constexpr int kGemmThreads = 256;
constexpr int kBK = 32;          // K per step
constexpr int kLds = kBK + 8;    // padded LDS row, in 16-bit elements

// ---------------------------------------------------------------- weight decoders
// Each decoder fills, for one weight row n and the 8 consecutive k of
// "piece" p (k = k0 + 8p .. +7), four u32 holding the 16-bit operand pairs
// (k, k+1) (k+2, k+3) (k+4, k+5) (k+6, k+7).

struct AffineB {
    const uint32_t* w;
    const uint16_t* scales;
    const uint16_t* biases;
    int K;
    struct Raw {
        uint32_t word, s, b;
    };
    __device__ __forceinline__ void load(int n, int k0, int p, bool valid, Raw& r) const {
        if (valid) {
            const int G = K / 32;
            r.word = w[(size_t)n * (K / 8) + (k0 / 8) + p];
            r.s = scales[(size_t)n * G + k0 / 32];
            r.b = biases[(size_t)n * G + k0 / 32];
        } else {
            r.word = 0u;
            r.s = 0u;
            r.b = 0u;
        }
    }
    // w = q * s + b in f32 (one rounding), then RNE to bf16.
    __device__ __forceinline__ void decode(const Raw& r, uint32_t (&out)[4]) const {
        const float s = bf16_bits_to_f32(r.s), b = bf16_bits_to_f32(r.b);
        float q[8];
        affine_word_to_f32(r.word, q);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[i] = pack_bf16x2(__builtin_fmaf(q[2 * i], s, b), __builtin_fmaf(q[2 * i + 1], s, b));
    }
};

struct LutB {
    const uint8_t* packed;
    const uint16_t* scales;
    int K;
    int block;
    const float* book;  // LDS copy of the 16 codebook values
    struct Raw {
        uint32_t bytes, s;
    };
    __device__ __forceinline__ void load(int n, int k0, int p, bool valid, Raw& r) const {
        if (valid) {
            const size_t flat = (size_t)n * K + k0 + 8 * p;  // multiple of 8
            r.bytes = *reinterpret_cast<const uint32_t*>(packed + flat / 2);
            r.s = scales[flat / block];
        } else {
            r.bytes = 0u;
            r.s = 0u;
        }
    }
    // value(i) = fp16(book[code(i)] * scale), code(i) = high nibble for even i.
    __device__ __forceinline__ void decode(const Raw& r, uint32_t (&out)[4]) const {
        const float s = f16_bits_to_f32(r.s);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t byte = (r.bytes >> (8 * i)) & 0xFFu;
            const float v0 = book[lut_code(byte, 0)] * s;  // flat index even
            const float v1 = book[lut_code(byte, 1)] * s;  // flat index odd
            out[i] = pack_f16x2(v0, v1);
        }
    }
};

template <bool kF16>
struct Mfma;
template <>
struct Mfma<false> {
    __device__ __forceinline__ static f32x4 run(const u32x4& a, const u32x4& b, const f32x4& c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                      0, 0, 0);
    }
};
template <>
struct Mfma<true> {
    __device__ __forceinline__ static f32x4 run(const u32x4& a, const u32x4& b, const f32x4& c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                     0, 0, 0);
    }
};

// ---------------------------------------------------------------- GEMM skeleton
// WM x WN wavefronts, each with FM x FN 16x16 fragments.
template <int WM, int WN, int FM, int FN, bool kF16, class BDec>
__device__ __forceinline__ void gemm_w4_body(const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int M, int K,
                                             int N, const BDec& bdec, uint16_t* As, uint16_t* Bs) {
    constexpr int BM = WM * FM * 16;
    constexpr int BN = WN * FN * 16;
    constexpr int XPT = BM * (kBK / 8) / kGemmThreads;  // 16-byte x pieces per thread
    constexpr int WPT = BN * (kBK / 8) / kGemmThreads;  // 8-weight pieces per thread
    static_assert(XPT >= 1 && WPT >= 1, "tile too small for the workgroup");
    static_assert(WM * WN * kWave == kGemmThreads, "4 wavefronts");

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave / WN, wn = wave % WN;
    const int tiles_n = (N + BN - 1) / BN;
    const int m0 = (blockIdx.x / tiles_n) * BM;
    const int n0 = (blockIdx.x % tiles_n) * BN;

    f32x4 acc[FM][FN];
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int g = 0; g < FN; ++g) acc[f][g] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 xr[XPT];
    typename BDec::Raw wr[WPT];

    auto load_step = [&](int k0) {
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int piece = tid + i * kGemmThreads;
            const int row = piece / 4, p = piece % 4;
            const int m = m0 + row;
            if (m < M)
                xr[i] = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + k0 + 8 * p);
            else
                xr[i] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int piece = tid + i * kGemmThreads;
            const int row = piece / 4, p = piece % 4;
            bdec.load(n0 + row, k0, p, n0 + row < N, wr[i]);
        }
    };
    auto store_step = [&](int buf) {
        uint16_t* as = As + buf * BM * kLds;
        uint16_t* bs = Bs + buf * BN * kLds;
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int piece = tid + i * kGemmThreads;
            *reinterpret_cast<u32x4*>(as + (piece / 4) * kLds + 8 * (piece % 4)) = xr[i];
        }
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int piece = tid + i * kGemmThreads;
            uint32_t v[4];
            bdec.decode(wr[i], v);
            *reinterpret_cast<u32x4*>(bs + (piece / 4) * kLds + 8 * (piece % 4)) = u32x4{v[0], v[1], v[2], v[3]};
        }
    };

    const int steps = K / kBK;
    load_step(0);
    store_step(0);
    __syncthreads();
    for (int kt = 0; kt < steps; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < steps) load_step((kt + 1) * kBK);
        const uint16_t* as = As + buf * BM * kLds;
        const uint16_t* bs = Bs + buf * BN * kLds;
        u32x4 a[FM], b[FN];
#pragma unroll
        for (int f = 0; f < FM; ++f)
            a[f] = *reinterpret_cast<const u32x4*>(as + (wm * FM * 16 + f * 16 + (lane & 15)) * kLds + 8 * (lane >> 4));
#pragma unroll
        for (int g = 0; g < FN; ++g)
            b[g] = *reinterpret_cast<const u32x4*>(bs + (wn * FN * 16 + g * 16 + (lane & 15)) * kLds + 8 * (lane >> 4));
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int g = 0; g < FN; ++g) acc[f][g] = Mfma<kF16>::run(a[f], b[g], acc[f][g]);
        if (kt + 1 < steps) store_step(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: lane holds rows 4*(lane/16)+r, column lane%16 of each fragment.
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int g = 0; g < FN; ++g) {
            const int n = n0 + wn * FN * 16 + g * 16 + (lane & 15);
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * FM * 16 + f * 16 + 4 * (lane >> 4) + r;
                if (m < M) y[(size_t)m * N + n] = kF16 ? f32_to_f16_bits(acc[f][g][r]) : f32_to_bf16_bits(acc[f][g][r]);
            }
        }
}

template <int WM, int WN, int FM, int FN>
__global__ __launch_bounds__(kGemmThreads) void qmm_affine4_kernel(const uint32_t* __restrict__ w,
                                                                    const uint16_t* __restrict__ scales,
                                                                    const uint16_t* __restrict__ biases,
                                                                    const uint16_t* __restrict__ x,
                                                                    uint16_t* __restrict__ y, int M, int K, int N) {
    constexpr int BM = WM * FM * 16, BN = WN * FN * 16;
    __shared__ __attribute__((aligned(16))) uint16_t As[2 * BM * kLds];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2 * BN * kLds];
    AffineB dec{w, scales, biases, K};
    gemm_w4_body<WM, WN, FM, FN, false>(x, y, M, K, N, dec, As, Bs);
}

struct Book16 {
    float v[16];
};

template <int WM, int WN, int FM, int FN>
__global__ __launch_bounds__(kGemmThreads) void qmm_lut4_kernel(const uint16_t* __restrict__ x,
                                                                 const uint8_t* __restrict__ packed,
                                                                 const uint16_t* __restrict__ scales, Book16 book,
                                                                 uint16_t* __restrict__ y, int M, int K, int N,
                                                                 int block) {
    constexpr int BM = WM * FM * 16, BN = WN * FN * 16;
    __shared__ __attribute__((aligned(16))) uint16_t As[2 * BM * kLds];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2 * BN * kLds];
    __shared__ float book_s[16];
    if (threadIdx.x < 16) book_s[threadIdx.x] = book.v[threadIdx.x];
    __syncthreads();
    LutB dec{packed, scales, K, block, book_s};
    gemm_w4_body<WM, WN, FM, FN, true>(x, y, M, K, N, dec, As, Bs);
}

}  // namespace w4mi

using namespace w4mi;

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

extern "C" w4_status qmm_affine4(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                                 const uint16_t* x, uint16_t* y, int64_t M, int64_t K, int64_t N,
                                 int32_t group_size, int32_t bits, void* stream) {
    w4_status st = w4_check_affine(M, K, N, group_size, bits, 0);
    if (st != W4_OK) return st;
    if (M == 0) return W4_OK;
    if (!w || !scales || !biases || !x || !y) return fail(W4_EINVAL, "qmm_affine4: null pointer argument");
    if (!aligned16(w) || !aligned16(x)) return fail(W4_EINVAL, "qmm_affine4: w and x must be 16-byte aligned");
    hipStream_t s = as_stream(stream);
    if (M <= 64) {
        constexpr int BM = 64, BN = 128;
        const unsigned tiles = (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
        hipLaunchKernelGGL((qmm_affine4_kernel<1, 4, 4, 2>), dim3(tiles), dim3(kGemmThreads), 0, s, w, scales, biases,
                           x, y, (int)M, (int)K, (int)N);
    } else {
        constexpr int BM = 256, BN = 128;
        const unsigned tiles = (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
        hipLaunchKernelGGL((qmm_affine4_kernel<2, 2, 8, 4>), dim3(tiles), dim3(kGemmThreads), 0, s, w, scales, biases,
                           x, y, (int)M, (int)K, (int)N);
    }
    return launch_status("qmm_affine4");
}

extern "C" w4_status qmm_lut4(const uint16_t* x, const uint8_t* packed, const uint16_t* scales, const float* book,
                              uint16_t* y, int64_t M, int64_t K, int64_t N, int32_t block, int32_t transpose,
                              void* stream) {
    w4_status st = w4_check_lut(M, K, N, block, transpose);
    if (st != W4_OK) return st;
    if (M == 0) return W4_OK;
    if (!x || !packed || !scales || !book || !y) return fail(W4_EINVAL, "qmm_lut4: null pointer argument");
    if (!aligned16(x) || ((uintptr_t)packed & 3u)) return fail(W4_EINVAL, "qmm_lut4: x must be 16-byte and packed 4-byte aligned");
    Book16 b;
    for (int i = 0; i < 16; ++i) b.v[i] = book[i];
    hipStream_t s = as_stream(stream);
    if (M <= 64) {
        constexpr int BM = 64, BN = 128;
        const unsigned tiles = (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
        hipLaunchKernelGGL((qmm_lut4_kernel<1, 4, 4, 2>), dim3(tiles), dim3(kGemmThreads), 0, s, x, packed, scales, b, y,
                           (int)M, (int)K, (int)N, (int)block);
    } else {
        constexpr int BM = 256, BN = 128;
        const unsigned tiles = (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
        hipLaunchKernelGGL((qmm_lut4_kernel<2, 2, 8, 4>), dim3(tiles), dim3(kGemmThreads), 0, s, x, packed, scales, b, y,
                           (int)M, (int)K, (int)N, (int)block);
    }
    return launch_status("qmm_lut4");
}
