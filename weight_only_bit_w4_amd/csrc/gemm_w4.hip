// MFMA GEMMs with a fused 4-bit weight decode:
//   qmm_affine4 - y[M,N] bf16 = x[M,K] bf16 . (q*s + b)^T   (INT4 MatMulNBits
//                 page, prefill M > 1). The matrix cores take binary16
//                 operands, as the page's kernel does: x is converted
//                 bf16 -> binary16 on its way into LDS and each weight is
//                 q*s + b rounded once to binary16; f32 accumulation, bf16
//                 output.
//   qmm_lut4    - y[M,N] fp16 = x[M,K] fp16 . fp16(book[c]*scale)^T
//                 (lut4 page, decode + GEMM route; fp16 operands, f32 acc)
//
// Operand range. A finite bf16 x of magnitude 65520 or more (or a weight
// q*s + b that large) becomes an infinity in binary16, which makes every
// output of its row of x (or of its weight row) an infinity or NaN, since
// an infinity times any weight, zero included, is not finite. So each
// affine kernel checks its finished outputs: only when one is not finite
// does it scan the inputs of that output tile, and if an x or weight value
// there is finite but out of binary16 range it adds one to a per-device
// event counter (w4_range_events). Inputs that are already infinite or NaN
// propagate as they would in the definition and are not counted.
//
// The small-shape kernels below share one skeleton: a workgroup of 4
// wavefronts computes a BM x BN output tile; per K-step of 32 (one affine
// quantisation group) it stages the x tile (BM x 32) and the decoded weight
// tile (BN x 32, decoded once per workgroup in registers and written as
// binary16 operands) in LDS, double buffered so the next step's global loads
// overlap this step's matrix-core work, with one barrier per step. Each
// wavefront owns a (16 FM) x (16 FN) sub-tile and issues
// v_mfma_f32_16x16x32_f16; LDS rows are padded to 80 bytes so the 16-byte
// operand reads of a 16-lane group hit distinct banks.
#include <atomic>
#include <type_traits>
#include <utility>

#include "w4mi_device.hpp"
#include "w4mi_host.hpp"

namespace w4mi {

constexpr int kGemmThreads = 256;
constexpr int kBK = 32;          // K per step
constexpr int kLds = kBK + 8;    // padded LDS row, in 16-bit elements
constexpr int kSmallDepth = 8;   // steps of global loads in flight in the small-M kernels

// ---------------------------------------------------------------- operand range events
// Per-device count of affine output tiles whose binary16 operands
// overflowed (see the top of this file). Read and reset by w4_range_events.
__device__ uint32_t g_range_events;

// True in every lane when any lane's accumulated value is not finite
// (v * 0 is NaN exactly for infinities and NaN).
template <int N>
__device__ __forceinline__ bool any_nonfinite(const float (&v)[N]) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) t = __builtin_fmaf(v[i], 0.f, t);
    return __builtin_amdgcn_ballot_w64(t != t) != 0;
}
// Run by one whole wavefront after its tile produced a non-finite output:
// looks for a finite x in rows [m_lo, m_hi) or a finite weight q*s + b in
// weight rows [n_lo, n_hi) that binary16 cannot hold, and counts the tile
// once if it finds one. Slow (element by element) and only reached when
// the output already shows the problem.
__device__ __noinline__ void affine_range_scan(const uint16_t* __restrict__ x, const uint32_t* __restrict__ w,
                                               const uint16_t* __restrict__ scales,
                                               const uint16_t* __restrict__ biases, int M, int K, int N, int m_lo,
                                               int m_hi, int n_lo, int n_hi, uint32_t* events) {
    const int lane = threadIdx.x & 63;
    m_hi = min(m_hi, M);
    n_hi = min(n_hi, N);
    bool found = false;
    for (int64_t i = (int64_t)m_lo * K + lane; i < (int64_t)m_hi * K && !found; i += 64)
        found = out_of_f16_range(bf16_bits_to_f32(x[i]));
    const int G = K / 32;
    for (int64_t i = (int64_t)n_lo * K + lane; i < (int64_t)n_hi * K && !found; i += 64) {
        const int64_t n = i / K, k = i % K;
        const float q = (float)affine_nibble(w[n * (K / 8) + k / 8], (int)(k % 8));
        found = out_of_f16_range(__builtin_fmaf(q, bf16_bits_to_f32(scales[n * G + k / 32]),
                                                bf16_bits_to_f32(biases[n * G + k / 32])));
    }
    if (__builtin_amdgcn_ballot_w64(found) != 0 && lane == 0) atomicAdd(events, 1u);
}

// ---------------------------------------------------------------- weight decoders
// Each decoder fills, for one weight row n and the 8 consecutive k of
// "piece" p (k = k0 + 8p .. +7), four u32 holding the 16-bit operand pairs
// (k, k+1) (k+2, k+3) (k+4, k+5) (k+6, k+7).

struct AffineB {
    static constexpr bool kAffine = true;  // x arrives as bf16 (converted to binary16), y is bf16
    const uint32_t* w;
    const uint16_t* scales;
    const uint16_t* biases;
    int K;
    uint32_t* events;
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
    // w = q * s + b in f32 (one rounding), then RNE to binary16.
    __device__ __forceinline__ void decode(const Raw& r, uint32_t (&out)[4]) const {
        const float s = bf16_bits_to_f32(r.s), b = bf16_bits_to_f32(r.b);
        float q[8];
        affine_word_to_f32(r.word, q);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[i] = pack_f16x2(__builtin_fmaf(q[2 * i], s, b), __builtin_fmaf(q[2 * i + 1], s, b));
    }
};

struct LutB {
    static constexpr bool kAffine = false;  // x and y are binary16
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

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- GEMM skeleton
// Calls f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>).
template <int... Is, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, Is...>, F&& f) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// WM x WN wavefronts, each with FM x FN 16x16 fragments. Global loads run D
// steps ahead in a register ring (a step has little matrix work next to
// the latency of its loads, so the loop is bound by how many are in flight);
// the LDS tiles are double buffered, one barrier per step.
template <int WM, int WN, int FM, int FN, class BDec, int D>
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

    u32x4 xr[D][XPT];
    typename BDec::Raw wr[D][WPT];

    auto load_step = [&](auto slot, int k0) {
        constexpr int S = decltype(slot)::value;
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int piece = tid + i * kGemmThreads;
            const int row = piece / 4, p = piece % 4;
            const int m = m0 + row;
            if (m < M)
                xr[S][i] = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + k0 + 8 * p);
            else
                xr[S][i] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int piece = tid + i * kGemmThreads;
            const int row = piece / 4, p = piece % 4;
            bdec.load(n0 + row, k0, p, n0 + row < N, wr[S][i]);
        }
    };
    auto store_step = [&](auto slot, int buf) {
        constexpr int S = decltype(slot)::value;
        uint16_t* as = As + buf * BM * kLds;
        uint16_t* bs = Bs + buf * BN * kLds;
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int piece = tid + i * kGemmThreads;
            *reinterpret_cast<u32x4*>(as + (piece / 4) * kLds + 8 * (piece % 4)) =
                BDec::kAffine ? bf16x8_to_f16x8(xr[S][i]) : xr[S][i];
        }
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int piece = tid + i * kGemmThreads;
            uint32_t v[4];
            bdec.decode(wr[S][i], v);
            *reinterpret_cast<u32x4*>(bs + (piece / 4) * kLds + 8 * (piece % 4)) = u32x4{v[0], v[1], v[2], v[3]};
        }
    };
    auto compute = [&](int buf) {
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
            for (int g = 0; g < FN; ++g) acc[f][g] = mfma16(a[f], b[g], acc[f][g]);
    };

    // Step kt's loads sit in slot kt % D. Writing LDS buffer kt & 1 at step kt
    // is safe: every wavefront passed step kt - 1's barrier, so it is done
    // with step kt - 2's reads of that buffer.
    const int steps = K / kBK;
    static_for<D>([&](auto S) {
        if (S < steps) load_step(S, S * kBK);
    });
    for (int kt0 = 0; kt0 < steps; kt0 += D) {
        static_for<D>([&](auto S) {
            const int kt = kt0 + S;
            if (kt < steps) {
                store_step(S, kt & 1);
                __syncthreads();
                if (kt + D < steps) load_step(S, (kt + D) * kBK);
                compute(kt & 1);
            }
        });
    }

    if constexpr (BDec::kAffine) {
        float v[FM * FN * 4];
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int g = 0; g < FN; ++g)
#pragma unroll
                for (int r = 0; r < 4; ++r) v[(f * FN + g) * 4 + r] = acc[f][g][r];
        if (any_nonfinite(v)) {
            const int ml = m0 + wm * FM * 16, nl = n0 + wn * FN * 16;
            affine_range_scan(x, bdec.w, bdec.scales, bdec.biases, M, K, N, ml, ml + FM * 16, nl, nl + FN * 16,
                              bdec.events);
        }
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
                if (m < M)
                    y[(size_t)m * N + n] =
                        BDec::kAffine ? f32_to_bf16_bits(acc[f][g][r]) : f32_to_f16_bits(acc[f][g][r]);
            }
        }
}

template <int WM, int WN, int FM, int FN>
__global__ __launch_bounds__(kGemmThreads) void qmm_affine4_kernel(const uint32_t* __restrict__ w,
                                                                    const uint16_t* __restrict__ scales,
                                                                    const uint16_t* __restrict__ biases,
                                                                    const uint16_t* __restrict__ x,
                                                                    uint16_t* __restrict__ y, int M, int K, int N,
                                                                    uint32_t* __restrict__ events) {
    constexpr int BM = WM * FM * 16, BN = WN * FN * 16;
    __shared__ __attribute__((aligned(16))) uint16_t As[2 * BM * kLds];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2 * BN * kLds];
    AffineB dec{w, scales, biases, K, events};
    gemm_w4_body<WM, WN, FM, FN, AffineB, kSmallDepth>(x, y, M, K, N, dec, As, Bs);
}

// ---------------------------------------------------------------- prefill GEMM (affine), register-staged
// qmm_affine4 for prefill shapes with K % 64 == 32 (the LDS-DMA form below
// takes K % 64 == 0): a 256 x 128 output tile per workgroup of 8 wavefronts
// in a 4 x 2 grid, two per SIMD so one's vector-ALU and LDS work fills the
// other's matrix-core time. Each wavefront owns a 64 x 64 sub-tile as 2 x 2
// accumulators of v_mfma_f32_32x32x16_f16. K advances 64 (two quantisation
// groups) per step; the last step holds one group and reads zeros for the
// other. Global loads run two steps ahead into registers and the LDS tiles
// are double buffered. Each thread converts its x pieces bf16 -> binary16 and
// decodes half a (weight row, group) per step (affine_word_f16). LDS rows
// are 144 bytes (64 operands + 16 bytes), which keeps the 16-byte operand
// reads of 16 consecutive rows conflict-free. Workgroups are assigned to
// tiles so that each XCD works on one block of tiles whose x rows and weight
// columns its L2 serves to all of them (prefill_tile).
constexpr int kPBM = 256, kPBN = 128, kPBK = 64;
constexpr int kPThreads = 512;
constexpr int kPLd = kPBK + 8;  // LDS row stride in 16-bit elements (144 bytes)
constexpr int kPTM = 2, kPTN = 2;  // 32 x 32 accumulator tiles per wavefront

// XCD-blocked tile order for a grid of tm x tn tiles (index m_tile * tn +
// n_tile). Workgroup b runs on XCD b % 8. Each XCD takes one block of
// (tm / pm) x (tn / pn) tiles, pm * pn = 8, with pm chosen so the blocks read
// the fewest bytes from outside the XCD: xb per row tile (its x rows), wb per
// column tile (its packed weights, scales and biases). Within a block, tiles
// go row by row, so the workgroups an XCD runs at once share their x rows.
// At M=2048, K=N=4096 (8 x 32 tiles) that is 2 x 16 tiles per XCD, 9.1 MB each
// against 12.2 MB for one row of 32 tiles. Grids that divide no such way keep
// a contiguous run of tiles per XCD (or the launch order).
__device__ __forceinline__ int prefill_tile(int b, int tm, int tn, uint64_t xb, uint64_t wb) {
    int pm = 0;
    uint64_t best = ~0ull;
    for (int p = 1; p <= 8; p *= 2)
        if (tm % p == 0 && tn % (8 / p) == 0) {
            const uint64_t bytes = (uint64_t)(tm / p) * xb + (uint64_t)(tn / (8 / p)) * wb;
            if (bytes < best) best = bytes, pm = p;
        }
    const int tiles = tm * tn;
    if (pm == 0) return tiles % 8 == 0 ? (b % 8) * (tiles / 8) + b / 8 : b;
    const int pn = 8 / pm, bm = tm / pm, bn = tn / pn, xcd = b % 8, i = b / 8;
    return ((xcd / pn) * bm + i / bn) * tn + (xcd % pn) * bn + i % bn;
}
__device__ __forceinline__ int prefill_tile(int b, int tm, int tn, int K) {
    return prefill_tile(b, tm, tn, (uint64_t)kPBM * (uint64_t)K * 2u,
                        (uint64_t)kPBN * ((uint64_t)K / 2u + (uint64_t)(K / 32) * 4u));
}

struct PrefillRegs {
    u32x4 x[4];       // x tile pieces i: row (tid / 8) + 64 i, 16-byte chunk tid % 8
    u32x2 w;          // two words (16 nibbles) of one quantisation group of one weight row
    uint32_t s, b;    // the group's scale and bias (bf16 bits)
};

// Offsets past a buffer's end read as zero (and stores there are dropped);
// kOob is far past any tile.
constexpr uint32_t kOob = 0x80000000u;

// Per-thread load offsets that stay fixed over the K loop; each step adds a
// wave-uniform (scalar register) offset. Thread t decodes weight row t / 4,
// group (t / 2) % 2 of the step, words 2 (t % 2), 2 (t % 2) + 1.
struct PrefillOffsets {
    uint32_t x, w, s;
};

template <bool kTail>
__device__ __forceinline__ void prefill_load(PrefillRegs& R, int kt, bool live, const PrefillOffsets& o, int tid, int K, int G,
                                             const __amdgpu_buffer_rsrc_t& xsrc, const __amdgpu_buffer_rsrc_t& wsrc,
                                             const __amdgpu_buffer_rsrc_t& ssrc, const __amdgpu_buffer_rsrc_t& bsrc) {
    // K % 64 == 32 (kTail): the last step holds one group; its other half is
    // read as zeros (x chunk past K, weight group past K / 32).
    // live == false (steps past the end): every offset is out of range, so
    // the loads fetch nothing and no branch splits the wait-counter state.
    const bool xv = live && (!kTail || kt * kPBK + 8 * (tid & 7) < K);
    const bool gv = live && (!kTail || 2 * kt + ((tid >> 1) & 1) < G);
    // Step offsets are wave-uniform; readfirstlane keeps them in scalar
    // registers (the buffer instructions' soffset operand).
    const int kx = __builtin_amdgcn_readfirstlane(kt * 2 * kPBK), kw = __builtin_amdgcn_readfirstlane(kt * 32);
    const int ks = __builtin_amdgcn_readfirstlane(kt * 4), xrow = __builtin_amdgcn_readfirstlane(128 * K);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        R.x[i] = __builtin_amdgcn_raw_buffer_load_b128(xsrc, xv ? o.x : kOob, i * xrow + kx, 0);
    R.w = __builtin_amdgcn_raw_buffer_load_b64(wsrc, gv ? o.w : kOob, kw, 0);
    R.s = __builtin_amdgcn_raw_buffer_load_b16(ssrc, gv ? o.s : kOob, ks, 0);
    R.b = __builtin_amdgcn_raw_buffer_load_b16(bsrc, gv ? o.s : kOob, ks, 0);
}

__device__ __forceinline__ void prefill_store(const PrefillRegs& R, int tid, uint16_t* As, uint16_t* Bs,
                                              uint32_t m_lo, uint32_t m_hi, uint32_t magic) {
    uint16_t* xa = As + (tid >> 3) * kPLd + 8 * (tid & 7);
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(xa + 64 * i * kPLd) = bf16x8_to_f16x8(R.x[i]);
    const AffineGroupF16 grp = affine_group_f16(bf16_bits_to_f32(R.s), bf16_bits_to_f32(R.b));
    uint16_t* dst = Bs + (tid >> 2) * kPLd + 16 * (tid & 3);
    *reinterpret_cast<u32x4*>(dst) = affine_word_f16<true>(R.w[0], grp, m_lo, m_hi, magic);
    *reinterpret_cast<u32x4*>(dst + 8) = affine_word_f16<true>(R.w[1], grp, m_lo, m_hi, magic);
}

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// One step (64 of K) of the wavefront's 64 x 64 sub-tile: per 16 of K, two
// A fragments (rows lane % 32 of each 32-row tile, k = 8 (lane / 32) .. +7)
// and two B fragments, four v_mfma_f32_32x32x16_f16.
__device__ __forceinline__ void prefill_mma(const uint16_t* As, const uint16_t* Bs, int wm, int wn, int lane,
                                            f32x16 (&acc)[kPTM][kPTN]) {
    const uint16_t* ab = As + (wm * 64 + (lane & 31)) * kPLd + 8 * (lane >> 5);
    const uint16_t* bb = Bs + (wn * 64 + (lane & 31)) * kPLd + 8 * (lane >> 5);
#pragma unroll
    for (int sub = 0; sub < kPBK / 16; ++sub) {
        u32x4 a[kPTM], b[kPTN];
#pragma unroll
        for (int f = 0; f < kPTM; ++f) a[f] = *reinterpret_cast<const u32x4*>(ab + f * 32 * kPLd + sub * 16);
#pragma unroll
        for (int g = 0; g < kPTN; ++g) b[g] = *reinterpret_cast<const u32x4*>(bb + g * 32 * kPLd + sub * 16);
#pragma unroll
        for (int f = 0; f < kPTM; ++f)
#pragma unroll
            for (int g = 0; g < kPTN; ++g)
                acc[f][g] = mfma32(a[f], b[g], acc[f][g]);
    }
}

// Affine epilogue range check for a wavefront's MT x NT grid of 32 x 32
// accumulators covering x rows [m_lo, m_lo + 32 MT) and weight rows
// [n_lo, n_lo + 32 NT).
template <int MT, int NT>
__device__ __forceinline__ void check_range32(const f32x16 (&acc)[MT][NT], const uint16_t* x, const uint32_t* w,
                                              const uint16_t* scales, const uint16_t* biases, int M, int K, int N,
                                              int m_lo, int n_lo, uint32_t* events) {
    float v[MT * NT * 16];
#pragma unroll
    for (int f = 0; f < MT; ++f)
#pragma unroll
        for (int g = 0; g < NT; ++g)
#pragma unroll
            for (int e = 0; e < 16; ++e) v[(f * NT + g) * 16 + e] = acc[f][g][e];
    if (any_nonfinite(v))
        affine_range_scan(x, w, scales, biases, M, K, N, m_lo, m_lo + 32 * MT, n_lo, n_lo + 32 * NT, events);
}

template <bool kTail>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void qmm_affine4_prefill_kernel(
    const uint32_t* __restrict__ w, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int M, int K, int N, uint32_t* __restrict__ events) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kPBM * kPLd];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kPBN * kPLd];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in a scalar register
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_m = (M + kPBM - 1) / kPBM, tiles_n = (N + kPBN - 1) / kPBN;
    const int t = prefill_tile(blockIdx.x, tiles_m, tiles_n, K);  // XCD-blocked order
    const int m0 = (t / tiles_n) * kPBM, n0 = (t % tiles_n) * kPBN;
    const int G = K / 32, steps = (K + kPBK - 1) / kPBK;

    const int mrows = min(kPBM, M - m0), nrows = min(kPBN, N - n0);
    const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(x + (size_t)m0 * K, (uint32_t)(mrows * K * 2));
    const __amdgpu_buffer_rsrc_t wsrc =
        make_rsrc(reinterpret_cast<const uint8_t*>(w) + (size_t)n0 * (K / 2), (uint32_t)(nrows * (K / 2)));
    const __amdgpu_buffer_rsrc_t ssrc = make_rsrc(scales + (size_t)n0 * G, (uint32_t)(nrows * G * 2));
    const __amdgpu_buffer_rsrc_t bsrc = make_rsrc(biases + (size_t)n0 * G, (uint32_t)(nrows * G * 2));
    const uint32_t m_lo = vreg(0x000F000Fu), m_hi = vreg(0x00F000F0u), magic = vreg(0x64006400u);
    PrefillOffsets o;
    o.x = (uint32_t)((tid >> 3) * K * 2 + 16 * (tid & 7));
    o.w = (uint32_t)((tid >> 2) * (K / 2) + 16 * ((tid >> 1) & 1) + 8 * (tid & 1));
    o.s = (uint32_t)(((tid >> 2) * G + ((tid >> 1) & 1)) * 2);

    f32x16 acc[kPTM][kPTN];
#pragma unroll
    for (int f = 0; f < kPTM; ++f)
#pragma unroll
        for (int g = 0; g < kPTN; ++g)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[f][g][e] = 0.f;

    PrefillRegs R0, R1;
    prefill_load<kTail>(R0, 0, true, o, tid, K, G, xsrc, wsrc, ssrc, bsrc);
    prefill_load<kTail>(R1, 1, steps > 1, o, tid, K, G, xsrc, wsrc, ssrc, bsrc);
    prefill_store(R0, tid, As[0], Bs[0], m_lo, m_hi, magic);
    __syncthreads();
    for (int kt = 0; kt < steps; kt += 2) {
        // even step: buffer 0 holds step kt; R1 holds step kt + 1
        prefill_load<kTail>(R0, kt + 2, kt + 2 < steps, o, tid, K, G, xsrc, wsrc, ssrc, bsrc);
        __builtin_amdgcn_sched_barrier(0);
        prefill_mma(As[0], Bs[0], wm, wn, lane, acc);
        if (kt + 1 < steps) prefill_store(R1, tid, As[1], Bs[1], m_lo, m_hi, magic);
        __syncthreads();
        if (kt + 1 >= steps) break;
        // odd step: buffer 1 holds step kt + 1; R0 holds step kt + 2
        prefill_load<kTail>(R1, kt + 3, kt + 3 < steps, o, tid, K, G, xsrc, wsrc, ssrc, bsrc);
        __builtin_amdgcn_sched_barrier(0);
        prefill_mma(As[1], Bs[1], wm, wn, lane, acc);
        if (kt + 2 < steps) prefill_store(R0, tid, As[0], Bs[0], m_lo, m_hi, magic);
        __syncthreads();
    }

    check_range32(acc, x, w, scales, biases, M, K, N, m0 + wm * 64, n0 + wn * 64, events);
    // Epilogue. Lane holds column lane % 32 of each 32 x 32 tile and, in
    // register e, row 8 (e / 4) + 4 (lane / 32) + e % 4. Stores go through a
    // buffer resource over the tile's rows, so rows past M are dropped by the
    // hardware; columns past N are sent out of range.
    const __amdgpu_buffer_rsrc_t ysrc = make_rsrc(y + (size_t)m0 * N, (uint32_t)(mrows * N * 2));
#pragma unroll
    for (int g = 0; g < kPTN; ++g) {
        const int n = n0 + wn * 64 + g * 32 + (lane & 31);
        const uint32_t voff = n < N ? (uint32_t)((4 * (lane >> 5)) * N + n) * 2u : kOob;
#pragma unroll
        for (int f = 0; f < kPTM; ++f)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = wm * 64 + f * 32 + 8 * (e >> 2) + (e & 3);
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(acc[f][g][e]), ysrc, voff, row * N * 2, 0);
            }
    }
}

// ---------------------------------------------------------------- prefill GEMM, specialised wavefronts
// The same 256 x 128 tile and K step of 64 for K % 64 == 0, with the work
// split by role so that the matrix pipe, the memory pipe and the vector ALU
// run at the same time: of the 12 wavefronts (three per SIMD), 4 consumers (a
// 2 x 2 grid of 128 x 64 sub-tiles, 8 accumulator tiles each) only read
// binary16 operands from LDS and issue v_mfma_f32_32x32x16_f16; 8 producers
// (two per SIMD, so that the vector ALU work of a step is issued by two
// wavefronts) load the next steps, convert x and decode the weights. One
// barrier per step hands the buffers over. Producer p, lane l, per step:
//   x       4 buffer loads of 16 bytes (rows 32 p + 8 i + l / 8, chunk l % 8
//           of the step's 128 bytes), converted bf16 -> binary16 and written
//           to a 2-slot LDS ring of [256 rows x 128 B], row r's chunk c at
//           position c ^ ((r / 2) % 8), which keeps the A-operand reads
//           (32 rows x 2 chunks per instruction) conflict-free;
//   W       8 bytes of nibbles (item 64 p + l: row item / 4, group
//           (item / 2) % 2, half item % 2: 16 of the group's 32 weights) and
//           the group's scale and bias, decoded (affine_word_f16) into one of
//           2 binary16 W tiles [128 rows x 144 B] (the 144-byte row keeps 16
//           consecutive rows' operand reads conflict-free).
// Loads run three steps ahead through a 3-deep register ring (the producer
// loop unrolled by 3), so a step's data has two steps of matrix work to
// arrive; the x of the 32 workgroups that one XCD runs (one row-block) stays
// in that XCD's L2. When K % 256 == 0 (a row's scales and biases fill whole
// 16-byte pieces), each lane loads the scales and the biases of its row for
// four steps (8 groups) at once, a 16-byte load each, four steps ahead, into
// a 3-deep ring of its own (loop unrolled by 12), and takes each step's pair
// from registers, instead of two 2-byte loads per step that each touch 16
// rows' cache lines for 128 bytes of data.
constexpr int kWsConsumers = 4, kWsProducers = 8;
constexpr int kWsThreads = (kWsConsumers + kWsProducers) * 64;
constexpr int kWsXp = kPBM * 8 / (kWsProducers * 64);   // 16-byte x pieces per producer lane per step (4)
constexpr int kDXBytes = kPBM * 128;    // x ring slot (also the LUT GEMM's)

// Byte address of an LDS object, for inline-asm LDS instructions.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Buffer-to-LDS DMA of 16 bytes per lane: lane l's bytes land at lds + 16 l;
// M0 carries the wave-uniform LDS base. Issued as inline asm so that the
// compiler, which cannot tell DMA targets apart, does not wait for all DMA in
// flight before every LDS access; completion is awaited explicitly
// (wait_vmcnt) before the data is read. Nothing else in these kernels uses M0.
__device__ __forceinline__ void lds_dma16(const __amdgpu_buffer_rsrc_t& rsrc, void* lds, uint32_t voff, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 ::"s"(lds_addr(lds)), "v"(voff), "s"(rsrc), "s"(soff));
}
// Loads into registers, also counted by hand (see above).
__device__ __forceinline__ void asm_load_b128(u32x4& d, const __amdgpu_buffer_rsrc_t& r, uint32_t voff, int soff) {
    asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen" : "=v"(d) : "v"(voff), "s"(r), "s"(soff));
}
__device__ __forceinline__ void asm_load_u16(uint32_t& d, const __amdgpu_buffer_rsrc_t& r, uint32_t voff, int soff) {
    asm volatile("buffer_load_ushort %0, %1, %2, %3 offen" : "=v"(d) : "v"(voff), "s"(r), "s"(soff));
}
// s_barrier with a compiler-only memory clobber (no hardware wait).
__device__ __forceinline__ void raw_barrier() { asm volatile("s_barrier" ::: "memory"); }
// s_waitcnt with only vmcnt (N < 64) or only lgkmcnt(0) constrained. gfx9
// encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14)); }

// A store to, and a load from, an LDS byte address.
template <typename T>
__device__ __forceinline__ void lds_st(uint32_t addr, const T& v) {
    *reinterpret_cast<__attribute__((address_space(3))) T*>((uintptr_t)addr) = v;
}
template <typename T>
__device__ __forceinline__ T lds_ld(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) T*>((uintptr_t)addr);
}

// One producer lane's share of a step: its x pieces, 2 words (16 nibbles,
// half a quantisation group of one row) and the group's scale and bias bits.
struct WsStep {
    u32x4 x[kWsXp];
    u32x2 words;
    uint32_t s, b;
};
// Makes a ring entry's registers opaque at this point, so that no work on
// them is scheduled before it (the conversions and decode of a step must not
// be hoisted above the barrier that frees the buffers they are written to).
__device__ __forceinline__ void ws_fence(WsStep& e) {
#pragma unroll
    for (int i = 0; i < kWsXp; ++i) asm volatile("" : "+v"(e.x[i]));
    asm volatile("" : "+v"(e.words), "+v"(e.s), "+v"(e.b));
}

// Step j's matrix work for a consumer: 4 sub-steps of k16, each 4 A reads
// (swizzled x slot), 2 B reads (W tile) and 8 MFMAs.
__device__ __forceinline__ void ws_mma(const uint8_t* xslot, const uint16_t* Bs, int wm, int wn, int lane,
                                       f32x16 (&acc)[4][2]) {
    const uint16_t* bb = Bs + (wn * 64 + (lane & 31)) * kPLd + 8 * (lane >> 5);
#pragma unroll
    for (int sub = 0; sub < kPBK / 16; ++sub) {
        u32x4 a[4], b[2];
        const int c = 2 * sub + (lane >> 5);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int row = wm * 128 + f * 32 + (lane & 31);
            a[f] = *reinterpret_cast<const u32x4*>(xslot + row * 128 + 16 * (c ^ ((row >> 1) & 7)));
        }
#pragma unroll
        for (int g = 0; g < 2; ++g) b[g] = *reinterpret_cast<const u32x4*>(bb + g * 32 * kPLd + sub * 16);
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int g = 0; g < 2; ++g) acc[f][g] = mfma32(a[f], b[g], acc[f][g]);
    }
}

template <bool SB4>
__global__ __launch_bounds__(kWsThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void qmm_affine4_prefill_ws_kernel(
    const uint32_t* __restrict__ w, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int M, int K, int N, uint32_t* __restrict__ events) {
    __shared__ __attribute__((aligned(1024))) uint8_t xring[2][kDXBytes];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kPBN * kPLd];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tiles_m = (M + kPBM - 1) / kPBM, tiles_n = (N + kPBN - 1) / kPBN;
    const int t = prefill_tile(blockIdx.x, tiles_m, tiles_n, K);  // XCD-blocked order
    const int m0 = (t / tiles_n) * kPBM, n0 = (t % tiles_n) * kPBN;
    const int G = K / 32, steps = K / kPBK;
    const int mrows = min(kPBM, M - m0), nrows = min(kPBN, N - n0);

    // The two roles run separate loops (so neither holds the other's
    // registers) with the same sequence of barriers, one per step: at barrier
    // j, x(j) and W(j) are in LDS, and the consumers are done with the buffers
    // of step j - 1.
    if (wave >= kWsConsumers) {
        const int pw = wave - kWsConsumers;
        const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(x + (size_t)m0 * K, (uint32_t)(mrows * K * 2));
        const __amdgpu_buffer_rsrc_t wsrc =
            make_rsrc(reinterpret_cast<const uint8_t*>(w) + (size_t)n0 * (K / 2), (uint32_t)(nrows * (K / 2)));
        const __amdgpu_buffer_rsrc_t ssrc = make_rsrc(scales + (size_t)n0 * G, (uint32_t)(nrows * G * 2));
        const __amdgpu_buffer_rsrc_t bsrc = make_rsrc(biases + (size_t)n0 * G, (uint32_t)(nrows * G * 2));
        const uint32_t m_lo = vreg(0x000F000Fu), m_hi = vreg(0x00F000F0u), magic = vreg(0x64006400u);
        uint32_t xo[kWsXp];   // source offsets of the lane's x pieces (step 0)
        uint32_t xd[kWsXp];   // LDS byte addresses of their places in slot 0 of the ring
#pragma unroll
        for (int i = 0; i < kWsXp; ++i) {
            const int row = 8 * (kWsXp * pw + i) + (lane >> 3), c = lane & 7;
            xo[i] = (uint32_t)(row * K * 2 + 16 * c);
            xd[i] = lds_addr(xring[0] + row * 128 + 16 * (c ^ ((row >> 1) & 7)));
        }
        const int item = 64 * pw + lane, r = item >> 2, g = (item >> 1) & 1, h = item & 1;
        const uint32_t wo = (uint32_t)(r * (K / 2) + 16 * g + 8 * h), so = (uint32_t)((r * G + g) * 2);
        const uint32_t bdst = lds_addr(Bs[0] + r * kPLd + 32 * g + 16 * h);
        WsStep ring[3];
        // SB4: the row's scales and biases of steps 4 blk .. 4 blk + 3 (groups 8 blk .. 8 blk + 7)
        struct WsSB {
            u32x4 s, b;
        };
        WsSB sb[3];
        const uint32_t sro = (uint32_t)(r * G * 2);
        auto issue_sb = [&](int blk, WsSB& e) {
            const int kb = __builtin_amdgcn_readfirstlane(4 * blk < steps ? blk * 16 : (int)kOob);
            e.s = __builtin_amdgcn_raw_buffer_load_b128(ssrc, sro, kb, 0);
            e.b = __builtin_amdgcn_raw_buffer_load_b128(bsrc, sro, kb, 0);
        };
        // Loads of step kt. Past the last step the wave-uniform offset is sent
        // past every buffer's end (the loads return zeros), which keeps the
        // per-lane offsets fixed.
        auto issue = [&](int kt, WsStep& e) {
            const bool live = kt < steps;
            const int kx = __builtin_amdgcn_readfirstlane(live ? kt * 2 * kPBK : (int)kOob);
            const int kw = __builtin_amdgcn_readfirstlane(live ? kt * 32 : (int)kOob);
            const int ks = __builtin_amdgcn_readfirstlane(live ? kt * 4 : (int)kOob);
#pragma unroll
            for (int i = 0; i < kWsXp; ++i) e.x[i] = __builtin_amdgcn_raw_buffer_load_b128(xsrc, xo[i], kx, 0);
            e.words = __builtin_amdgcn_raw_buffer_load_b64(wsrc, wo, kw, 0);
            if constexpr (!SB4) {
                e.s = __builtin_amdgcn_raw_buffer_load_b16(ssrc, so, ks, 0);
                e.b = __builtin_amdgcn_raw_buffer_load_b16(bsrc, so, ks, 0);
            } else {
                e.s = e.b = 0u;
            }
        };
        // Step data into LDS buffer `buf`: x converted, W decoded. SB4: the
        // step's scale and bias are dword D of sb set Q, half g.
        auto publish = [&](const WsStep& e, auto buf, auto q_c, auto d_c) {
            constexpr uint32_t xb = decltype(buf)::value * kDXBytes, wb = decltype(buf)::value * (kPBN * kPLd * 2);
#pragma unroll
            for (int i = 0; i < kWsXp; ++i) lds_st<u32x4>(xd[i] + xb, bf16x8_to_f16x8(e.x[i]));
            float sf, bf;
            if constexpr (SB4) {
                constexpr int Q = decltype(q_c)::value, D = decltype(d_c)::value;
                const uint32_t sv = sb[Q].s[D], bv = sb[Q].b[D];
                sf = __uint_as_float(g ? sv & 0xFFFF0000u : sv << 16);
                bf = __uint_as_float(g ? bv & 0xFFFF0000u : bv << 16);
            } else {
                sf = bf16_bits_to_f32(e.s);
                bf = bf16_bits_to_f32(e.b);
            }
            const AffineGroupF16 grp = affine_group_f16(sf, bf);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                lds_st<u32x4>(bdst + wb + 16 * i, affine_word_f16<true>(e.words[i], grp, m_lo, m_hi, magic));
        };
        // The prologue issues steps 0, 1, 2 in the loop's order (the
        // scheduling barriers keep the compiler from interleaving them, so its
        // wait counts at the loop head stay exact), after the first two
        // scale and bias blocks.
        using C0 = std::integral_constant<int, 0>;
        if constexpr (SB4) {
            issue_sb(0, sb[0]);
            issue_sb(1, sb[1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        issue(0, ring[0]);
        __builtin_amdgcn_sched_barrier(0);
        issue(1, ring[1]);
        __builtin_amdgcn_sched_barrier(0);
        issue(2, ring[2]);
        __builtin_amdgcn_sched_barrier(0);
        publish(ring[0], C0{}, C0{}, C0{});
        // Iteration j (j mod 3 == S0, j mod 2 == P): barrier j (this
        // wavefront's LDS writes of step j are complete), publish step j + 1
        // into the free buffers (past the last step: zeros into buffers no
        // consumer reads again), then load step j + 3 into the ring entry step
        // j used; SB4: at j = 3 mod 4, also the scale and bias block of steps
        // j + 5 .. j + 8, into the set that block j + 5 - 12 used. The loop is
        // unrolled by 6 (SB4: 12) so that every ring position is a constant
        // (I = j mod 6 or 12).
        auto body = [&](auto i_c, int j) {
            constexpr int I = decltype(i_c)::value, S0 = I % 3, S1 = (S0 + 1) % 3, P = I % 2;
            constexpr int Q = ((I + 1) / 4) % 3, D = (I + 1) % 4;  // step j + 1's scale set and dword
            wait_lgkmcnt0();
            raw_barrier();
            ws_fence(ring[S1]);
            publish(ring[S1], std::integral_constant<int, 1 - P>{}, std::integral_constant<int, Q>{},
                    std::integral_constant<int, D>{});
            issue(j + 3, ring[S0]);
            if constexpr (SB4 && I % 4 == 3) issue_sb((j + 5) / 4, sb[((I + 5) / 4) % 3]);
        };
        constexpr int U = SB4 ? 12 : 6;
        int j = 0;
        for (; j + U <= steps; j += U) static_for<U>([&](auto I) { body(I, j + I); });
        static_for<U - 1>([&](auto I) {
            if (j + I < steps) body(I, j + I);
        });
        return;
    }

    // Consumers issue at a higher wave priority than the producers that share
    // their SIMD, so the matrix pipe gets an instruction whenever it is free.
    __builtin_amdgcn_s_setprio(2);
    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc[4][2];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[f][g][e] = 0.f;
    for (int j = 0; j < steps; ++j) {
        raw_barrier();
        ws_mma(xring[j & 1], Bs[j & 1], wm, wn, lane, acc);
    }
    __builtin_amdgcn_s_setprio(0);

    check_range32(acc, x, w, scales, biases, M, K, N, m0 + wm * 128, n0 + wn * 64, events);
    const __amdgpu_buffer_rsrc_t ysrc = make_rsrc(y + (size_t)m0 * N, (uint32_t)(mrows * N * 2));
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int n = n0 + wn * 64 + g * 32 + (lane & 31);
        const uint32_t voff = n < N ? (uint32_t)((4 * (lane >> 5)) * N + n) * 2u : kOob;
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = wm * 128 + f * 32 + 8 * (e >> 2) + (e & 3);
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(acc[f][g][e]), ysrc, voff, row * N * 2, 0);
            }
    }
}

template <int WM, int WN, int FM, int FN, int D>
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
    gemm_w4_body<WM, WN, FM, FN, LutB, D>(x, y, M, K, N, dec, As, Bs);
}

// ---------------------------------------------------------------- LUT GEMM, specialised wavefronts
// y = x . W^T for the lookup-codebook weight (fp16 throughout, f32
// accumulation) on the same plan as the affine prefill: a 256 x 96 tile
// (M = 512, N = 11008 gives 230 tiles for 256 CUs), K step 64, x by LDS DMA
// into a swizzled 3-slot ring, and
//   4 consumer wavefronts, one per 64 x rows, each with all 96 weight rows
//     (2 x 3 accumulator tiles of v_mfma_f32_32x32x16_f16);
//   8 producer wavefronts issuing the x DMA (4 instructions each per step)
//     and, for the first 6 of them, decoding one (weight row, 16-wide K
//     quarter) per lane: 8 packed bytes and the block's scale arrive in a
//     3-deep register ring, the lane builds its row's 16-entry table
//     T[c] = fp16(book[c] * scale) as byte planes and looks codes up four at
//     a time with v_perm_b32.
// The block size must be a power of two of at least 16 (one scale per lane
// and step).
// With the weight stored [K, N] (transpose == 0, the lut4.rs page's
// decoded-weight route at M >= 128) a step's weights are 64 rows k of the
// tile's 96 columns, contiguous along n, and the first 6 producers decode
// one (2-row, 8-column) item per lane instead: a packed dword (8 codes along
// n) and the block's scale for each of the 2 rows, each code looked up in
// the 16 f32 codebook entries kept in LDS (64 lanes read at most 16
// addresses, one per bank: no bank conflicts), multiplied by its row's scale
// in f32 and rounded to binary16, and each column's 2 k values written to
// the [n][k] tile as one 4-byte store. That needs N % 8 == 0 and a power-of-two block of at least 8
// (a packed dword never straddles a block).
constexpr int kLBM = 256, kLBN = 96;
constexpr int kLConsumers = 4, kLProducers = 8;
constexpr int kLThreads = (kLConsumers + kLProducers) * 64;
constexpr int kLXb = 32 / kLProducers;              // x DMA instructions per producer per step
constexpr int kLDecodeWaves = kLBN * 4 / 64;        // producers that decode (one lane per row quarter)
constexpr int kLKnCols = kLBN / 8;                  // [K, N]: 8-column groups per tile
constexpr int kLKnRows = 2;                         // rows of a decode item
constexpr int kLKnDecodeWaves = kLKnCols * (kPBK / kLKnRows) / 64;  // 6: one lane per (2-row, 8-column) item

struct LutWeights {
    u32x2 words;  // 16 codes: the lane's K quarter of its row
    uint32_t s;   // the block's scale (binary16 bits)
};
__device__ __forceinline__ void lut_fence(LutWeights& e) { asm volatile("" : "+v"(e.words), "+v"(e.s)); }
struct LutKnWeights {
    uint32_t w[kLKnRows];  // rows kLKnRows kq + i: codes of the item's 8 columns
    uint32_t s[kLKnRows];  // and their blocks' scales (binary16 bits)
};
__device__ __forceinline__ void lut_fence(LutKnWeights& e) {
#pragma unroll
    for (int i = 0; i < kLKnRows; ++i) asm volatile("" : "+v"(e.w[i]), "+v"(e.s[i]));
}
__device__ __forceinline__ void asm_load_b32(uint32_t& d, const __amdgpu_buffer_rsrc_t& r, uint32_t voff, int soff) {
    asm volatile("buffer_load_dword %0, %1, %2, %3 offen" : "=v"(d) : "v"(voff), "s"(r), "s"(soff));
}
__device__ __forceinline__ void asm_load_b64(u32x2& d, const __amdgpu_buffer_rsrc_t& r, uint32_t voff, int soff) {
    asm volatile("buffer_load_dwordx2 %0, %1, %2, %3 offen" : "=v"(d) : "v"(voff), "s"(r), "s"(soff));
}

// XCD-aware tile order: workgroup b runs on XCD b % 8, and XCD x takes the
// contiguous range of tiles u = n_tile * tiles_m + m_tile that starts after
// the tiles of XCDs 0 .. x - 1 (XCDs below tiles % 8 get one more). The M
// tiles of a column tile, and neighbouring column tiles, then share one L2:
// a column tile's weights (and, for W stored [K, N], the 64-byte sectors its
// row segments share with the neighbouring tiles) come from HBM once.
__device__ __forceinline__ int xcd_tile(int b, int tiles) {
    const int xcd = b % 8, i = b / 8, base = tiles / 8, extra = tiles % 8;
    return xcd * base + min(xcd, extra) + i;
}

template <bool KN>
__global__ __launch_bounds__(kLThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void qmm_lut4_ws_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
    Book16 book, uint16_t* __restrict__ y, int M, int K, int N, int block_shift) {
    __shared__ __attribute__((aligned(1024))) uint8_t xring[3][kDXBytes];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kLBN * kPLd];
    __shared__ __attribute__((aligned(16))) float kn_book[16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tiles_m = (M + kLBM - 1) / kLBM, tiles_n = (N + kLBN - 1) / kLBN;
    const int u = xcd_tile(blockIdx.x, tiles_m * tiles_n);
    const int m0 = (u % tiles_m) * kLBM, n0 = (u / tiles_m) * kLBN;
    const int steps = K / kPBK;
    const int mrows = min(kLBM, M - m0), nrows = min(kLBN, N - n0);

    if (KN && wave >= kLConsumers) {
        const int pw = wave - kLConsumers;
        const bool decoder = pw < kLKnDecodeWaves;
        const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(x + (size_t)m0 * K, (uint32_t)(mrows * K * 2));
        // the whole weight (N * K / 2 < 2^31 bytes) and its scales
        const __amdgpu_buffer_rsrc_t psrc = make_rsrc(packed, (uint32_t)((uint64_t)N * (uint64_t)K / 2));
        const __amdgpu_buffer_rsrc_t ssrc =
            make_rsrc(scales, (uint32_t)((((uint64_t)N * (uint64_t)K + (1u << block_shift) - 1) >> block_shift) * 2));
        uint32_t xo[kLXb];
#pragma unroll
        for (int i = 0; i < kLXb; ++i) {
            const int row = 8 * (kLXb * pw + i) + (lane >> 3);
            xo[i] = (uint32_t)(row * K * 2 + 16 * ((lane & 7) ^ ((row >> 1) & 7)));
        }
        // item (kq, cg) = (rows kLKnRows kq .. of a step, tile columns 8 cg ..); lanes of one kq read one row's 48 bytes
        const int item = 64 * pw + lane, kq = item / kLKnCols, cg = item % kLKnCols;
        const uint32_t col = (uint32_t)(n0 + 8 * cg);
        const bool live = decoder && col < (uint32_t)N;
        // Every decoding wavefront writes the same 16 entries (and waits for
        // its own writes before its first lookup: no barrier is needed).
        const uint32_t kb = lds_addr(kn_book);
        if (decoder && lane < 16) {
            float v = 0.f;
#pragma unroll
            for (int c = 0; c < 16; ++c) v = lane == c ? book.v[c] : v;
            lds_st(kb + 4u * (uint32_t)lane, v);
        }
        LutKnWeights ring[3];
        auto issue = [&](int kt, int kw, uint8_t* xslot, LutKnWeights& e) {
            const bool xl = kt < steps, wl = live && kw < steps;
            const int kx = __builtin_amdgcn_readfirstlane(kt * 2 * kPBK);
#pragma unroll
            for (int i = 0; i < kLXb; ++i) lds_dma16(xsrc, xslot + (kLXb * pw + i) * 1024, xl ? xo[i] : kOob, kx);
            if (decoder) {
#pragma unroll
                for (int i = 0; i < kLKnRows; ++i) {
                    const uint32_t flat = (uint32_t)(kPBK * kw + kLKnRows * kq + i) * (uint32_t)N + col;  // < N K < 2^32
                    asm_load_b32(e.w[i], psrc, wl ? flat / 2 : kOob, 0);
                    asm_load_u16(e.s[i], ssrc, wl ? (flat >> block_shift) * 2u : kOob, 0);
                }
            }
        };
        // Columns 2 b and 2 b + 1 of the item are byte b's high and low codes.
        static_assert(kLKnRows == 2, "one 4-byte store per column");
        // The tile's row n keeps its 16-byte k chunk c at chunk c ^ ((n / 8) % 8): the 12 lanes of one
        // kq (columns 8 cg ..) would otherwise all store to one bank.
        const uint32_t kofs = 2u * (uint32_t)(8 * (((kLKnRows * kq) >> 3) ^ (cg & 7)) + ((kLKnRows * kq) & 7));
        auto decode = [&](const LutKnWeights& e, int buf) {
            const float s0 = f16_bits_to_f32(e.s[0]), s1 = f16_bits_to_f32(e.s[1]);
            const uint32_t dst = lds_addr(Bs[buf]) + 2u * (uint32_t)(8 * cg * kPLd) + kofs;
            // byte offsets 4 code of each row's codes: high nibbles (even
            // columns) and low nibbles (odd columns), one byte per code
            uint32_t hi4[kLKnRows], lo4[kLKnRows];
#pragma unroll
            for (int i = 0; i < kLKnRows; ++i) {
                hi4[i] = (e.w[i] >> 2) & 0x3C3C3C3Cu;
                lo4[i] = (e.w[i] << 2) & 0x3C3C3C3Cu;
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float h0 = lds_ld<float>(kb + ((hi4[0] >> (8 * b)) & 0xFFu));
                const float h1 = lds_ld<float>(kb + ((hi4[1] >> (8 * b)) & 0xFFu));
                const float l0 = lds_ld<float>(kb + ((lo4[0] >> (8 * b)) & 0xFFu));
                const float l1 = lds_ld<float>(kb + ((lo4[1] >> (8 * b)) & 0xFFu));
                lds_st(dst + 2u * (uint32_t)((2 * b) * kPLd), pack_f16x2(h0 * s0, h1 * s1));
                lds_st(dst + 2u * (uint32_t)((2 * b + 1) * kPLd), pack_f16x2(l0 * s0, l1 * s1));
            }
        };
        constexpr int kWl = 2 * kLKnRows;  // weight loads per decoding lane per step
        issue(steps, 0, xring[2], ring[0]);
        issue(0, 1, xring[0], ring[1]);
        issue(1, 2, xring[1], ring[2]);
        if (decoder) {
            wait_vmcnt<2 * (kLXb + kWl)>();
            wait_lgkmcnt0();  // the codebook written
            lut_fence(ring[0]);
            decode(ring[0], 0);
        }
        auto body = [&](auto slot, int j) {
            constexpr int S0 = decltype(slot)::value, S1 = (S0 + 1) % 3, S2 = (S0 + 2) % 3;
            if (decoder)
                wait_vmcnt<kLXb + kWl>();
            else
                wait_vmcnt<kLXb>();
            wait_lgkmcnt0();
            lut_fence(ring[S1]);
            raw_barrier();
            if (decoder) decode(ring[S1], (j + 1) & 1);
            issue(j + 2, j + 3, xring[S2], ring[S0]);
        };
        int j = 0;
        for (; j + 3 <= steps; j += 3) {
            body(std::integral_constant<int, 0>{}, j);
            body(std::integral_constant<int, 1>{}, j + 1);
            body(std::integral_constant<int, 2>{}, j + 2);
        }
        if (j < steps) body(std::integral_constant<int, 0>{}, j);
        if (j + 1 < steps) body(std::integral_constant<int, 1>{}, j + 1);
        // The trailing (all-zero) loads land before this wavefront ends; the
        // fences keep every ring entry's registers allocated until they have
        // (an asm load's output is otherwise free once unused, and a load
        // still in flight would overwrite whatever took its place).
        wait_vmcnt<0>();
#pragma unroll
        for (int i = 0; i < 3; ++i) lut_fence(ring[i]);
        return;
    }
    if (!KN && wave >= kLConsumers) {
        const int pw = wave - kLConsumers;
        const bool decoder = pw < kLDecodeWaves;
        const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(x + (size_t)m0 * K, (uint32_t)(mrows * K * 2));
        const __amdgpu_buffer_rsrc_t psrc = make_rsrc(packed + (size_t)n0 * (K / 2), (uint32_t)(nrows * (K / 2)));
        const int spr = K >> block_shift;  // scales per row
        const __amdgpu_buffer_rsrc_t ssrc = make_rsrc(scales + (size_t)n0 * spr, (uint32_t)(nrows * spr * 2));
        uint32_t xo[kLXb];
#pragma unroll
        for (int i = 0; i < kLXb; ++i) {
            const int row = 8 * (kLXb * pw + i) + (lane >> 3);
            xo[i] = (uint32_t)(row * K * 2 + 16 * ((lane & 7) ^ ((row >> 1) & 7)));
        }
        const int item = 64 * pw + lane;              // decode item: row item / 4, K quarter item % 4
        const int r = item >> 2, q = item & 3;
        const uint32_t po = (uint32_t)(r * (K / 2) + 8 * q);
        uint16_t* const bdst = Bs[0] + r * kPLd + 16 * q;
        LutWeights ring[3];
        auto issue = [&](int kt, int kw, uint8_t* xslot, LutWeights& e) {
            const bool xl = kt < steps, wl = kw < steps;
            const int kx = __builtin_amdgcn_readfirstlane(kt * 2 * kPBK);
#pragma unroll
            for (int i = 0; i < kLXb; ++i) lds_dma16(xsrc, xslot + (kLXb * pw + i) * 1024, xl ? xo[i] : kOob, kx);
            if (decoder) {
                // scale index r * spr + (64 kw + 16 q) >> block_shift
                const uint32_t so = (uint32_t)(r * spr + ((64 * kw + 16 * q) >> block_shift)) * 2u;
                asm_load_b64(e.words, psrc, wl ? po : kOob, __builtin_amdgcn_readfirstlane(kw * 32));
                asm_load_u16(e.s, ssrc, wl ? so : kOob, 0);
            }
        };
        // With blocks of 64 or more the four lanes of a quad (one row's four K
        // quarters of a step) share a scale: each builds a quarter of the
        // table (entries 4 q .. 4 q + 3, its planes lo[q] and hi[q]) and takes
        // the other quarters from its neighbours by quad permutes.
        const bool quad = block_shift >= 6;
        float bq[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = 0.f;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) v = q == qq ? book.v[4 * qq + i] : v;
            bq[i] = v;
        }
        auto decode = [&](const LutWeights& e, int buf) {
            const float sc = f16_bits_to_f32(e.s);
            LutPlanes P;
            if (quad) {
                const uint32_t t0 = pack_f16x2(bq[0] * sc, bq[1] * sc), t1 = pack_f16x2(bq[2] * sc, bq[3] * sc);
                const uint32_t lo = __builtin_amdgcn_perm(t1, t0, 0x06040200u), hi = __builtin_amdgcn_perm(t1, t0, 0x07050301u);
                P.lo[0] = __builtin_amdgcn_update_dpp(0u, lo, 0x00, 0xF, 0xF, false);
                P.lo[1] = __builtin_amdgcn_update_dpp(0u, lo, 0x55, 0xF, 0xF, false);
                P.lo[2] = __builtin_amdgcn_update_dpp(0u, lo, 0xAA, 0xF, 0xF, false);
                P.lo[3] = __builtin_amdgcn_update_dpp(0u, lo, 0xFF, 0xF, 0xF, false);
                P.hi[0] = __builtin_amdgcn_update_dpp(0u, hi, 0x00, 0xF, 0xF, false);
                P.hi[1] = __builtin_amdgcn_update_dpp(0u, hi, 0x55, 0xF, 0xF, false);
                P.hi[2] = __builtin_amdgcn_update_dpp(0u, hi, 0xAA, 0xF, 0xF, false);
                P.hi[3] = __builtin_amdgcn_update_dpp(0u, hi, 0xFF, 0xF, 0xF, false);
            } else {
                P = lut_planes(book, sc);
            }
            uint16_t* dst = bdst + buf * (kLBN * kPLd);
            *reinterpret_cast<u32x4*>(dst) = lut_decode8(e.words[0], P);
            *reinterpret_cast<u32x4*>(dst + 8) = lut_decode8(e.words[1], P);
        };
        issue(steps, 0, xring[2], ring[0]);
        issue(0, 1, xring[0], ring[1]);
        issue(1, 2, xring[1], ring[2]);
        if (decoder) {
            wait_vmcnt<2 * (kLXb + 2)>();
            lut_fence(ring[0]);
            decode(ring[0], 0);
        }
        auto body = [&](auto slot, int j) {
            constexpr int S0 = decltype(slot)::value, S1 = (S0 + 1) % 3, S2 = (S0 + 2) % 3;
            if (decoder)
                wait_vmcnt<kLXb + 2>();
            else
                wait_vmcnt<kLXb>();
            wait_lgkmcnt0();
            lut_fence(ring[S1]);
            raw_barrier();
            if (decoder) decode(ring[S1], (j + 1) & 1);
            issue(j + 2, j + 3, xring[S2], ring[S0]);
        };
        int j = 0;
        for (; j + 3 <= steps; j += 3) {
            body(std::integral_constant<int, 0>{}, j);
            body(std::integral_constant<int, 1>{}, j + 1);
            body(std::integral_constant<int, 2>{}, j + 2);
        }
        if (j < steps) body(std::integral_constant<int, 0>{}, j);
        if (j + 1 < steps) body(std::integral_constant<int, 1>{}, j + 1);
        // The trailing (all-zero) loads land before this wavefront ends; the
        // fences keep every ring entry's registers allocated until they have
        // (an asm load's output is otherwise free once unused, and a load
        // still in flight would overwrite whatever took its place).
        wait_vmcnt<0>();
#pragma unroll
        for (int i = 0; i < 3; ++i) lut_fence(ring[i]);
        return;
    }

    // Consumer c: x rows 64 c .. 64 c + 63 (A tiles f), weight rows 32 g (B tiles g).
    const int c = wave;
    f32x16 acc[2][3];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int g = 0; g < 3; ++g)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[f][g][e] = 0.f;
    for (int j = 0; j < steps; ++j) {
        raw_barrier();
        const uint8_t* xslot = xring[j % 3];
        const uint16_t* bb = Bs[j & 1] + (lane & 31) * kPLd + 8 * (lane >> 5);
#pragma unroll
        for (int sub = 0; sub < kPBK / 16; ++sub) {
            u32x4 a[2], b[3];
            const int ch = 2 * sub + (lane >> 5);
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const int row = 64 * c + 32 * f + (lane & 31);
                a[f] = *reinterpret_cast<const u32x4*>(xslot + row * 128 + 16 * (ch ^ ((row >> 1) & 7)));
            }
#pragma unroll
            for (int g = 0; g < 3; ++g) {
                if constexpr (KN) {
                    // [K, N] tiles: row n's 16-byte chunk c sits at chunk c ^ ((n / 8) % 8)
                    const int n = 32 * g + (lane & 31);
                    b[g] = *reinterpret_cast<const u32x4*>(Bs[j & 1] + n * kPLd + 8 * (ch ^ ((n >> 3) & 7)));
                } else {
                    b[g] = *reinterpret_cast<const u32x4*>(bb + g * 32 * kPLd + sub * 16);
                }
            }
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int g = 0; g < 3; ++g)
                    acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[f]),
                                                                      __builtin_bit_cast(f16x8, b[g]), acc[f][g], 0, 0, 0);
        }
    }
    const __amdgpu_buffer_rsrc_t ysrc = make_rsrc(y + (size_t)m0 * N, (uint32_t)(mrows * N * 2));
#pragma unroll
    for (int g = 0; g < 3; ++g) {
        const int n = n0 + g * 32 + (lane & 31);
        const uint32_t voff = n < N ? (uint32_t)((4 * (lane >> 5)) * N + n) * 2u : kOob;
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 64 * c + 32 * f + 8 * (e >> 2) + (e & 3);
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_f16_bits(acc[f][g][e]), ysrc, voff, row * N * 2, 0);
            }
    }
}

// ---------------------------------------------------------------- small batches, weight tiles
// qmm_affine4 for a few dozen rows of x (M <= 64, K % 256 == 0): the weights
// are read exactly once and every row of x is applied to them on the matrix
// cores. A workgroup of 16 wavefronts takes two 32-row weight tiles; wavefront
// (t, p) = (w / 8, w % 8) owns tile t and k-steps 2 p, 2 p + 1 (quantisation
// group p) of each 256-wide K window, against all M rows (MT 32-row tiles of
// x); at the end each of a tile's eight wavefronts sums 2 (MT = 2: 4) of the
// accumulator registers over the eight partial sums (through LDS) and stores
// them. Each lane decodes its own weight word straight into a binary16
// matrix-core operand (affine_word_f16: q s + b rounded once, in k order) and
// converts its x operands bf16 -> binary16 as it reads them. Weights (128
// packed bytes, 16 bytes of scales and 16 of biases per row per window) and x
// (M rows x 512 bytes per window, from L2) stream through one LDS ring (6
// slots for up to 32 rows of x, 3 for up to 64) by buffer-to-LDS DMA that all
// 16 wavefronts issue; each wavefront reads its operands of window j + 1 from
// LDS while it decodes and multiplies window j, one barrier per window.
constexpr int kTlWaves = 16, kTlThreads = kTlWaves * 64;
constexpr int kTlMinM = 6;                           // fewer rows may take the shared-x GEMV form
constexpr int kTlTiles = 2;                          // 32-row weight tiles per workgroup
constexpr int kTlParts = kTlWaves / kTlTiles;        // 8 wavefronts share a tile's K
constexpr int kTlSteps = 16 / kTlParts;              // k-steps (16 of K) per wavefront per window
constexpr int kTlWinK = 256;
constexpr int kTlRows = 32 * kTlTiles;               // 64 weight rows
constexpr int kTlWRow = kTlWinK / 2;                 // 128 packed bytes of a row per window
constexpr int kTlWBytes = kTlRows * kTlWRow;         // 8 KB
constexpr int kTlSBytes = kTlRows * 16;              // 1 KB: 8 groups' bf16 scales per row
constexpr int kTlWSlot = kTlWBytes + 2 * kTlSBytes;  // 10 KB: packed, scales, biases
constexpr int kTlXRow = kTlWinK * 2;                 // 512 bytes of an x row per window
constexpr int kTlWDma = kTlWBytes / 1024 + 2;        // 10 weight DMA instructions per window
template <int MT> struct TlShape {
    static constexpr int kXSlot = MT * 32 * kTlXRow;          // 16 or 32 KB
    static constexpr int kXDma = kXSlot / 1024;               // 16 or 32 x DMA instructions per window
    static constexpr int kDma = kTlWDma + kXDma;              // 26 or 42 per window
    static constexpr int kStages = MT == 1 ? 6 : 3;           // as deep as 160 KB of LDS allows
    static constexpr int kLds = kStages * (kTlWSlot + kXSlot);
};

// s_waitcnt vmcnt(n) for a run-time n (0 .. 23; larger waits for everything).
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
    switch (n) {
        case 16: wait_vmcnt<16>(); break;
        case 17: wait_vmcnt<17>(); break;
        case 18: wait_vmcnt<18>(); break;
        case 19: wait_vmcnt<19>(); break;
        case 20: wait_vmcnt<20>(); break;
        case 21: wait_vmcnt<21>(); break;
        case 22: wait_vmcnt<22>(); break;
        case 23: wait_vmcnt<23>(); break;
        case 1: wait_vmcnt<1>(); break;
        case 2: wait_vmcnt<2>(); break;
        case 3: wait_vmcnt<3>(); break;
        case 4: wait_vmcnt<4>(); break;
        case 5: wait_vmcnt<5>(); break;
        case 6: wait_vmcnt<6>(); break;
        case 7: wait_vmcnt<7>(); break;
        case 8: wait_vmcnt<8>(); break;
        case 9: wait_vmcnt<9>(); break;
        case 10: wait_vmcnt<10>(); break;
        case 11: wait_vmcnt<11>(); break;
        case 12: wait_vmcnt<12>(); break;
        case 13: wait_vmcnt<13>(); break;
        case 14: wait_vmcnt<14>(); break;
        case 15: wait_vmcnt<15>(); break;
        default: wait_vmcnt<0>(); break;
    }
}

// One lane's LDS reads of a window: two weight words, the group's scale and
// bias bits, and the x operands of its two k-steps (bf16, per x tile).
template <int MT> struct TlOps {
    uint32_t word[kTlSteps];
    u32x4 x[kTlSteps][MT];
    uint32_t s, b;
};

// DMA instruction i of a window (issued by wavefront i % 16), lane l:
//   i < 8: packed weights, 16-byte piece q = 64 i + l of the slot: row q / 8,
//          slot position q % 8 holding the row's piece (q % 8) ^ ((row / 2) % 8);
//   i = 8, 9: the 64 rows' 16 bytes of scales, of biases;
//   i >= 10: x, piece q = 64 (i - 10) + l: row q / 32, slot position q % 32
//          holding chunk (q % 32) ^ (row % 16).
// Window j + S - 1 (S slots) goes out after barrier j into the slot of window
// j - 1, which every wavefront finished reading before barrier j; each
// wavefront waits for its own DMA of window j + 1 before barrier j (its LDS
// reads run one window ahead). A lane whose row lies past N or M has an
// offset past its descriptor's range and reads zeros; an offset in range plus
// the window's scalar offset stays inside its own row.
template <int MT>
__global__ __launch_bounds__(kTlThreads) void qmm_affine4_tiles_kernel(
    const uint32_t* __restrict__ w, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int M, int K, int N, uint32_t* __restrict__ events) {
    using Sh = TlShape<MT>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[Sh::kLds];
    constexpr int kS = Sh::kStages;
    uint8_t* const wring = lds;
    uint8_t* const xring = lds + kS * kTlWSlot;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * kTlRows;
    const int rows = min(kTlRows, N - n0);
    const int G = K / 32, nwin = K / kTlWinK;
    const uint32_t wrow = (uint32_t)K / 2u, srow = (uint32_t)G * 2u;
    // This wavefront's DMA: instructions i = wave + 16 u, u < per_window. All
    // but the window is fixed for the launch and chosen here once: the
    // instruction's descriptor, its LDS position in slot 0 and the slot
    // stride, its lane offset, and the bytes a window advances (the
    // instruction's scalar offset; every lane offset that is in range stays in
    // its own row of W, scales, biases or x for every window).
    constexpr int kU = (Sh::kDma + kTlWaves - 1) / kTlWaves;
    const int per_window = (Sh::kDma - wave + kTlWaves - 1) / kTlWaves;
    static_assert(Sh::kDma > kTlWaves * (kU - 1), "every wavefront issues kU - 1 or kU instructions");
    __amdgpu_buffer_rsrc_t rs[kU];
    uint32_t off[kU], lbase[kU], lstride[kU], wstep[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int i = wave + kTlWaves * u;
        const bool isw = i < kTlWDma - 2, iss = i == kTlWDma - 2, isb = i == kTlWDma - 1, isx = i >= kTlWDma;
        const uint8_t* const base = isw   ? reinterpret_cast<const uint8_t*>(w) + (size_t)n0 * wrow
                                    : iss ? reinterpret_cast<const uint8_t*>(scales) + (size_t)n0 * srow
                                    : isb ? reinterpret_cast<const uint8_t*>(biases) + (size_t)n0 * srow
                                          : reinterpret_cast<const uint8_t*>(x);
        rs[u] = make_rsrc(base, isw ? (uint32_t)rows * wrow : isx ? (uint32_t)M * (uint32_t)K * 2u : (uint32_t)rows * srow);
        lbase[u] = isw ? lds_addr(wring) + 1024u * (uint32_t)i
                   : isx ? lds_addr(xring) + 1024u * (uint32_t)(i - kTlWDma)
                         : lds_addr(wring) + kTlWBytes + (isb ? kTlSBytes : 0);
        lstride[u] = isx ? Sh::kXSlot : kTlWSlot;
        wstep[u] = isw ? kTlWRow : isx ? kTlXRow : 16;
        if (isw) {
            const int q = 64 * i + lane, r = q >> 3, pc = (q & 7) ^ ((r >> 1) & 7);
            off[u] = r < rows ? (uint32_t)r * wrow + 16u * (uint32_t)pc : kOob;
        } else if (!isx) {
            off[u] = lane < rows ? (uint32_t)lane * srow : kOob;
        } else {
            const int q = 64 * (i - kTlWDma) + lane, m = q >> 5, c = (q & 31) ^ (m & 15);
            off[u] = m < M ? (uint32_t)m * (uint32_t)K * 2u + 16u * (uint32_t)c : kOob;
        }
    }
    // Window win into ring slot sl (win % S; a constant wherever the step
    // loop below calls it).
    auto issue = [&](int sl, int win) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (u >= per_window) break;
            const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane((int)(lbase[u] + (uint32_t)sl * lstride[u]));
            const int soff = __builtin_amdgcn_readfirstlane(win * (int)wstep[u]);
            asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m0v), "v"(off[u]), "s"(rs[u]),
                         "s"(soff));
        }
    };
    // Window 0 from every wavefront first: the barrier puts it ahead of the
    // later windows in the compute unit's memory queue.
    issue(0, 0);
    raw_barrier();
#pragma unroll
    for (int win = 1; win < kS - 1; ++win)
        if (win < nwin) issue(win, win);

    // Wavefront (t, p) = (w / 8, w % 8) takes weight tile t and k-steps
    // 2 p, 2 p + 1 (quantisation group p) of each window, against all MT x
    // tiles; every output has 8 partial sums.
    const int t = wave / kTlParts, part = wave % kTlParts;
    const int h = lane >> 5, n = lane & 31, row = 32 * t + n;
    const uint32_t m_lo = vreg(0x000F000Fu), m_hi = vreg(0x00F000F0u), magic = vreg(0x64006400u);
    // The lane's LDS read addresses in slot 0 (k-step u of the wavefront is
    // 2 p + u, its word of the row wd = 2 (2 p + u) + h, its group p),
    // kept whole in registers so that slot offsets fold into the instructions.
    uint32_t wa[kTlSteps], xa[kTlSteps][MT], xa2[kTlSteps][MT];
    const uint32_t sa = lds_addr(wring) + kTlWBytes + row * 16 + 2 * part;
#pragma unroll
    for (int u = 0; u < kTlSteps; ++u) {
        const int wd = 2 * (kTlSteps * part + u) + h;
        wa[u] = lds_addr(wring) + row * kTlWRow + 16 * ((wd >> 2) ^ ((row >> 1) & 7)) + 4 * (wd & 3);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            xa[u][mt] = lds_addr(xring) + (32 * mt + n) * kTlXRow + 16 * (wd ^ (n & 15));
            xa2[u][mt] = xa[u][mt] + 2 * Sh::kXSlot;  // slot 2: past the 16-bit offset field when MT = 2
        }
    }
#pragma unroll
    for (int u = 0; u < kTlSteps; ++u) {
        asm volatile("" : "+v"(wa[u]));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            asm volatile("" : "+v"(xa[u][mt]));
            if (MT > 1) asm volatile("" : "+v"(xa2[u][mt]));
        }
    }
    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
    using Ops = TlOps<MT>;
    // A window's LDS reads: the lane's weight words, its group's scale and
    // bias bits and its x operands (bf16).
    auto read = [&](auto ws_c) {
        constexpr int WS = decltype(ws_c)::value, XS = WS;
        Ops o;
        o.s = lds_ld<uint16_t>(sa + WS * kTlWSlot);
        o.b = lds_ld<uint16_t>(sa + WS * kTlWSlot + kTlSBytes);
#pragma unroll
        for (int u = 0; u < kTlSteps; ++u) {
            o.word[u] = lds_ld<uint32_t>(wa[u] + WS * kTlWSlot);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                o.x[u][mt] = (MT > 1 && XS == 2) ? lds_ld<u32x4>(xa2[u][mt]) : lds_ld<u32x4>(xa[u][mt] + XS * Sh::kXSlot);
        }
        return o;
    };
    auto compute = [&](const Ops& o) {
        const AffineGroupF16 grp = affine_group_f16(bf16_bits_to_f32(o.s), bf16_bits_to_f32(o.b));
        u32x4 bop[kTlSteps];
#pragma unroll
        for (int u = 0; u < kTlSteps; ++u) bop[u] = affine_word_f16<MT == 1>(o.word[u], grp, m_lo, m_hi, magic);
#pragma unroll
        for (int u = 0; u < kTlSteps; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma32(bf16x8_to_f16x8(o.x[u][mt]), bop[u], acc[mt]);
    };
    // The reads run one window ahead of the arithmetic, so that a window's
    // LDS traffic overlaps the previous window's decode and matrix work.
    // Window 0: its DMA landed for every wavefront at the barrier.
    wait_vmcnt_rt(min(kS - 2, nwin - 1) * per_window);
    raw_barrier();
    Ops ops[2];
    ops[0] = read(std::integral_constant<int, 0>{});
    // Step j: window j (slot j % S, a constant: the loop below is unrolled by
    // S) from registers, window j + 1's reads into the other register set.
    auto step = [&](auto ws_c, int j, Ops& cur, Ops& next) {
        constexpr int WS = decltype(ws_c)::value;
        // Window j + 1 has landed; windows j + 2 .. min(j + S - 2, nwin - 1)
        // may still be in flight. The barrier also marks every wavefront's
        // reads of window j - 1 done (they were used in step j - 1), so its
        // slot takes window j + S - 1.
        if constexpr (kS == 3) {
            wait_vmcnt<0>();
        } else if (j + kS - 2 < nwin) {  // the usual case: windows j + 2 .. j + S - 2 exist
            if (per_window == kU)
                wait_vmcnt<(kS - 3) * kU>();
            else
                wait_vmcnt<(kS - 3) * (kU - 1)>();
        } else {
            wait_vmcnt_rt(max(0, nwin - 2 - j) * per_window);
        }
        wait_lgkmcnt0();
        raw_barrier();
        if (j + kS - 1 < nwin) issue((WS + kS - 1) % kS, j + kS - 1);
        if (j + 1 < nwin) next = read(std::integral_constant<int, (WS + 1) % kS>{});
        __builtin_amdgcn_sched_barrier(0);  // the reads go out before the arithmetic below
        compute(cur);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;
    int j = 0;
    if constexpr (kS == 6) {
        for (; j + 5 < nwin; j += 6) {
            step(I0{}, j, ops[0], ops[1]);
            step(I1{}, j + 1, ops[1], ops[0]);
            step(I2{}, j + 2, ops[0], ops[1]);
            step(I3{}, j + 3, ops[1], ops[0]);
            step(I4{}, j + 4, ops[0], ops[1]);
            step(I5{}, j + 5, ops[1], ops[0]);
        }
        if (j < nwin) step(I0{}, j, ops[0], ops[1]);
        if (j + 1 < nwin) step(I1{}, j + 1, ops[1], ops[0]);
        if (j + 2 < nwin) step(I2{}, j + 2, ops[0], ops[1]);
        if (j + 3 < nwin) step(I3{}, j + 3, ops[1], ops[0]);
        if (j + 4 < nwin) step(I4{}, j + 4, ops[0], ops[1]);
    } else {
        static_assert(kS == 3, "slot sequences for 6 and 3 slots");
        // Three slots and two register sets: the loop runs six windows a turn.
        for (; j + 5 < nwin; j += 6) {
            step(I0{}, j, ops[0], ops[1]);
            step(I1{}, j + 1, ops[1], ops[0]);
            step(I2{}, j + 2, ops[0], ops[1]);
            step(I0{}, j + 3, ops[1], ops[0]);
            step(I1{}, j + 4, ops[0], ops[1]);
            step(I2{}, j + 5, ops[1], ops[0]);
        }
        if (j < nwin) step(I0{}, j, ops[0], ops[1]);
        if (j + 1 < nwin) step(I1{}, j + 1, ops[1], ops[0]);
        if (j + 2 < nwin) step(I2{}, j + 2, ops[0], ops[1]);
        if (j + 3 < nwin) step(I0{}, j + 3, ops[1], ops[0]);
        if (j + 4 < nwin) step(I1{}, j + 4, ops[0], ops[1]);
    }
    // The rings are free (every DMA landed before the last barrier, and the
    // barrier below waits for every wavefront's last reads). Of a tile's 8
    // wavefronts, wavefront p finishes the kOwn registers f = kOwn p + e
    // (flat index f = 16 mt + i over its accumulator tiles): it writes its
    // registers in groups of four, then adds the 7 other partial sums of its
    // own, in order of the writer. With kOwn = 4 its own group is not written.
    raw_barrier();
    constexpr int kRegs = 16 * MT, kOwn = kRegs / kTlParts;  // its registers, the ones it finishes
    constexpr bool kSkipOwn = kOwn == 4;
    constexpr int kGroups = kRegs / 4 - (kSkipOwn ? 1 : 0);  // groups a wavefront writes
    const int grp0 = t * kTlParts;                           // the tile's first writer
    // red[writer][group slot][lane]: writer q's group g (registers 4 g .. 4 g + 3)
    // at slot g, or with kSkipOwn g < q ? g : g - 1.
    u32x4* const red = reinterpret_cast<u32x4*>(lds);
    static_assert(kTlWaves * kGroups * 64 * 16 <= Sh::kLds, "exchange area fits the rings");
#pragma unroll
    for (int g = 0; g < kRegs / 4; ++g) {
        const u32x4 v = {__float_as_uint(acc[g >> 2][4 * (g & 3)]), __float_as_uint(acc[g >> 2][4 * (g & 3) + 1]),
                         __float_as_uint(acc[g >> 2][4 * (g & 3) + 2]), __float_as_uint(acc[g >> 2][4 * (g & 3) + 3])};
        if (!kSkipOwn)
            red[((grp0 + part) * kGroups + g) * 64 + lane] = v;
        else if (g != part)
            red[((grp0 + part) * kGroups + (g < part ? g : g - 1)) * 64 + lane] = v;
    }
    wait_lgkmcnt0();  // the partial sums written before another wavefront reads them
    raw_barrier();
    const int f0 = kOwn * part, gown = f0 >> 2;
    // the wavefront's own partial sums (a run-time register index)
    float fin[kOwn];
#pragma unroll
    for (int e = 0; e < kOwn; ++e) {
        float v = 0.f;
#pragma unroll
        for (int r = 0; r < kRegs; ++r) v = r == f0 + e ? acc[r >> 4][r & 15] : v;
        fin[e] = v;
    }
    // every writer's group read at once (the own one, q = part, at a valid
    // position and not added), then added in order of q
    float o[kTlParts][kOwn];
#pragma unroll
    for (int q = 0; q < kTlParts; ++q) {
        const int slot = !kSkipOwn ? gown : gown < q ? gown : q == part ? 0 : gown - 1;
        const float* const src = reinterpret_cast<const float*>(&red[((grp0 + q) * kGroups + slot) * 64 + lane]) + (f0 & 3);
        if constexpr (kOwn == 4) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[q][e] = __uint_as_float(v[e]);
        } else {
            static_assert(kOwn == 2, "two or four registers per wavefront");
            const u32x2 v = *reinterpret_cast<const u32x2*>(src);
            o[q][0] = __uint_as_float(v[0]);
            o[q][1] = __uint_as_float(v[1]);
        }
    }
#pragma unroll
    for (int q = 0; q < kTlParts; ++q)
#pragma unroll
        for (int e = 0; e < kOwn; ++e) fin[e] = q != part ? fin[e] + o[q][e] : fin[e];
    // Lane (n, h) holds, of accumulator register i, x row 8 (i / 4) + 4 h + i % 4
    // of the x tile and weight row n of the tile; the wavefront's registers
    // lie in x tile f0 / 16.
    static_assert(16 % kOwn == 0, "a wavefront's registers lie in one accumulator tile");
    const int mt_own = f0 >> 4, col = n0 + row;
    // Range check over the finished sums (every x row, the tile's weight rows).
    if (any_nonfinite(fin)) affine_range_scan(x, w, scales, biases, M, K, N, 0, M, n0 + 32 * t, n0 + 32 * t + 32, events);
#pragma unroll
    for (int e = 0; e < kOwn; ++e) {
        const int i = (f0 + e) & 15;
        const int m = 32 * mt_own + 8 * (i >> 2) + 4 * h + (i & 3);
        if (m < M && col < N) y[(size_t)m * N + col] = f32_to_bf16_bits(fin[e]);
    }
}

}  // namespace w4mi

using namespace w4mi;

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Device address of g_range_events on the current device, looked up once per
// device (each GPU holds its own copy of the variable).
namespace w4mi {
static constexpr int kMaxDevices = 64;
static std::atomic<uint32_t*> g_range_ptr[kMaxDevices];

w4_status range_counter(uint32_t** out, const char* fn) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(W4_ELAUNCH, "%s: no usable current device", fn);
    uint32_t* p = g_range_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        void* a = nullptr;
        const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(g_range_events));
        if (e != hipSuccess || !a)
            return fail(W4_ELAUNCH, "%s: cannot locate the range-event counter: %s", fn, hipGetErrorString(e));
        p = static_cast<uint32_t*>(a);
        g_range_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return W4_OK;
}
}  // namespace w4mi

extern "C" w4_status w4_range_events(uint32_t* count, int32_t reset) {
    if (!count) return fail(W4_EINVAL, "w4_range_events: count is null");
    uint32_t* p = nullptr;
    const w4_status st = range_counter(&p, "w4_range_events");
    if (st != W4_OK) return st;
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(count, p, sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (e == hipSuccess && reset) e = hipMemset(p, 0, sizeof(uint32_t));
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail(W4_ELAUNCH, "w4_range_events: %s", hipGetErrorString(e));
    clear_error();
    return W4_OK;
}

extern "C" w4_status qmm_affine4(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                                 const uint16_t* x, uint16_t* y, int64_t M, int64_t K, int64_t N,
                                 int32_t group_size, int32_t bits, void* stream) {
    w4_status st = w4_check_affine(M, K, N, group_size, bits, 0);
    if (st != W4_OK) return st;
    if (M == 0) return W4_OK;
    if (!w || !scales || !biases || !x || !y) return fail(W4_EINVAL, "qmm_affine4: null pointer argument");
    if (!aligned16(w) || !aligned16(x)) return fail(W4_EINVAL, "qmm_affine4: w and x must be 16-byte aligned");
    // Buffer descriptors cover one 256-row tile of x or y: 256 * K * 2 bytes must fit 32 bits.
    if (K > (1 << 21) || N > (1 << 21))
        return fail(W4_EUNSUPPORTED, "qmm_affine4: implemented for K and N up to 2097152 (K=%lld N=%lld)", (long long)K,
                    (long long)N);
    uint32_t* events = nullptr;
    st = range_counter(&events, "qmm_affine4");
    if (st != W4_OK) return st;
    hipStream_t s = as_stream(stream);
    const bool tiles_ok = K % kTlWinK == 0 && ((uintptr_t)scales & 3u) == 0 && ((uintptr_t)biases & 3u) == 0;
    if (M < kTlMinM && K <= kAffineBatchMaxK && (!tiles_ok || M <= xlds_batch_rows((int)M, (int)K))) {
        // A few rows: the GEMV form (each weight row read once for all of
        // them), where its rows fit one pass or the weight-tile form does not
        // apply; a second pass costs more than the tile form's whole launch.
        launch_xlds(w, scales, biases, x, y, (int)M, (int)K, (int)N, s);
    } else if (M <= 64 && tiles_ok) {
        // Up to 64 rows: weight tiles streamed once through the matrix cores.
        const dim3 grid((unsigned)((N + kTlRows - 1) / kTlRows));
        if (M <= 32)
            hipLaunchKernelGGL(qmm_affine4_tiles_kernel<1>, grid, dim3(kTlThreads), 0, s, w, scales, biases, x, y, (int)M,
                               (int)K, (int)N, events);
        else
            hipLaunchKernelGGL(qmm_affine4_tiles_kernel<2>, grid, dim3(kTlThreads), 0, s, w, scales, biases, x, y, (int)M,
                               (int)K, (int)N, events);
    } else if (M <= kAffineBatchRows && K <= kAffineBatchMaxK) {
        launch_xlds(w, scales, biases, x, y, (int)M, (int)K, (int)N, s);
    } else if (M <= 64) {
        constexpr int BM = 64, BN = 128;
        const unsigned tiles = (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
        hipLaunchKernelGGL((qmm_affine4_kernel<1, 4, 4, 2>), dim3(tiles), dim3(kGemmThreads), 0, s, w, scales, biases,
                           x, y, (int)M, (int)K, (int)N, events);
    } else {
        const unsigned tiles = (unsigned)(((M + kPBM - 1) / kPBM) * ((N + kPBN - 1) / kPBN));
        if (K % 256 == 0)
            hipLaunchKernelGGL(qmm_affine4_prefill_ws_kernel<true>, dim3(tiles), dim3(kWsThreads), 0, s, w, scales,
                               biases, x, y, (int)M, (int)K, (int)N, events);
        else if (K % kPBK == 0)
            hipLaunchKernelGGL(qmm_affine4_prefill_ws_kernel<false>, dim3(tiles), dim3(kWsThreads), 0, s, w, scales,
                               biases, x, y, (int)M, (int)K, (int)N, events);
        else
            hipLaunchKernelGGL(qmm_affine4_prefill_kernel<true>, dim3(tiles), dim3(kPThreads), 0, s, w, scales, biases,
                               x, y, (int)M, (int)K, (int)N, events);
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
    if (!transpose) {
        if (((uintptr_t)x & 1u) || ((uintptr_t)scales & 1u) || ((uintptr_t)y & 1u))
            return fail(W4_EINVAL, "qmm_lut4: x, scales and y must be 2-byte aligned");
        // Weight stored [K, N]. From 128 rows of x (the page's decoded-weight
        // threshold) the matrix cores, where the shape allows; otherwise column
        // kernels in the vector ALU (lut_f32.hip).
        if (M >= 128 && K % kPBK == 0 && N % 8 == 0 && block >= 8 && (block & (block - 1)) == 0 &&
            (uint64_t)N * (uint64_t)K / 2 < (1ull << 31) && aligned16(x) && ((uintptr_t)packed & 3u) == 0) {
            Book16 b;
            for (int i = 0; i < 16; ++i) b.v[i] = book[i];
            int shift = 0;
            while ((1 << shift) < block) ++shift;
            const unsigned tiles = (unsigned)(((M + kLBM - 1) / kLBM) * ((N + kLBN - 1) / kLBN));
            hipLaunchKernelGGL(qmm_lut4_ws_kernel<true>, dim3(tiles), dim3(kLThreads), 0, as_stream(stream), x, packed,
                               scales, b, y, (int)M, (int)K, (int)N, shift);
            return launch_status("qmm_lut4 ([K, N] matrix-core route)");
        }
        launch_lut4_kn_f16(x, packed, scales, book, y, M, K, N, block, as_stream(stream));
        return launch_status("qmm_lut4");
    }
    if (!aligned16(x) || ((uintptr_t)packed & 3u)) return fail(W4_EINVAL, "qmm_lut4: x must be 16-byte and packed 4-byte aligned");
    Book16 b;
    for (int i = 0; i < 16; ++i) b.v[i] = book[i];
    hipStream_t s = as_stream(stream);
    if (M <= 64) {
        constexpr int BM = 64, BN = 128;
        const unsigned tiles = (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
        hipLaunchKernelGGL((qmm_lut4_kernel<1, 4, 4, 2, kSmallDepth>), dim3(tiles), dim3(kGemmThreads), 0, s, x, packed, scales, b, y,
                           (int)M, (int)K, (int)N, (int)block);
    } else if (K % kPBK == 0 && block >= 16 && (block & (block - 1)) == 0 && K <= (1 << 21) && N <= (1 << 21)) {
        int shift = 0;
        while ((1 << shift) < block) ++shift;
        const unsigned tiles = (unsigned)(((M + kLBM - 1) / kLBM) * ((N + kLBN - 1) / kLBN));
        hipLaunchKernelGGL(qmm_lut4_ws_kernel<false>, dim3(tiles), dim3(kLThreads), 0, s, x, packed, scales, b, y, (int)M,
                           (int)K, (int)N, shift);
    } else {
        constexpr int BM = 256, BN = 128;
        const unsigned tiles = (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
        hipLaunchKernelGGL((qmm_lut4_kernel<2, 2, 8, 4, 2>), dim3(tiles), dim3(kGemmThreads), 0, s, x, packed, scales, b, y,
                           (int)M, (int)K, (int)N, (int)block);
    }
    return launch_status("qmm_lut4");
}
