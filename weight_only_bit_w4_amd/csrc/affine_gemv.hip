// qmv_affine4: decode GEMV y[1, N] = x[1, K] . dequant(W)^T for affine INT4
// group-32 weights (INT4 MatMulNBits page: the M = 1 route, which that page
// leaves to the library mat-vec).
//
// HBM-bound: every weight byte is read once. Each wavefront owns R output
// rows; its 64 lanes split K by quantisation group (lane l takes groups l,
// l + 64, ...), so one 128-bit load per lane and row fetches exactly one
// group's 32 nibbles and consecutive lanes read consecutive 16-byte pieces of
// the row. All weight loads of a wavefront are issued before its first
// arithmetic; rows are then consumed in load order, so arithmetic on early
// rows overlaps the arrival of later ones. The R row sums are reduced across
// lanes together, in the vector ALU (lane swaps and DPP moves).
//
// Arithmetic per group, for the bf16 pairs (128 + q) that one AND-OR makes
// from a shifted weight word (exact: 128 + q has 8 significant bits):
//   sum_k x_k (q_k s + b) = s * sum_k x_k (128 + q_k) + (b - 128 s) * sum_k x_k,
// so the scale and bias are applied once per group, not per weight, and the
// inner loop is 7 integer ops + 4 v_dot2_f32_bf16 per 8 weights.
//
// Up to 256 groups (K <= 8192) the x side is shared: a workgroup of 8
// wavefronts x 2 rows loads x once (one 16-byte piece per lane, ahead of its
// weight loads), turns each piece into its bf16 pairs and partial group sum,
// and publishes them in LDS, from which every wavefront reads its groups.
// That takes the x loads off the per-wavefront path (x was otherwise read
// 14 times per compute unit) and keeps each wavefront's post-load work, which
// sets the end of the kernel, short. Longer K uses one wavefront per
// workgroup with x in registers, one 64-group chunk at a time.
#include "w4mi_device.hpp"
#include "w4mi_host.hpp"

#include <cmath>

namespace w4mi {

constexpr int kGemvRows = 4;  // output rows per wavefront of the long-K form (one wavefront per workgroup)
constexpr int kGemvAux = 2;   // non-temporal weight loads: each byte is read once
constexpr int kGemvAcc = 2;   // independent partial sums per group dot product
constexpr int kXWaves = 8;    // wavefronts per workgroup of the shared-x form
constexpr int kXRows = 2;     // output rows per wavefront of the shared-x form
constexpr int kXChunks = 4;   // the shared-x form covers up to 4 x 64 groups
constexpr int kXStride = 20;  // LDS dwords per group: 16 pairs, the sum, pad (80 B: conflict-free 16-byte reads)

// Lane view of one quantisation group of x: bf16 pairs matching the nibble
// pairs (i, i + 4) of each of the group's four words, and the group sum.
struct XGroup {
    uint32_t pair[4][4];
    float sum;
};

// Builds the pairs from the group's 32 bf16 values (four 16-byte pieces);
// an idle lane (past the last group) gets zeros, so every row term it adds
// is zero.
__device__ __forceinline__ void x_group_from_raw(const u32x4 (&v4)[4], bool valid, XGroup& xg) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t v0 = valid ? v4[j][0] : 0u, v1 = valid ? v4[j][1] : 0u;
        const uint32_t v2 = valid ? v4[j][2] : 0u, v3 = valid ? v4[j][3] : 0u;
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

// sum over the group of x_k * (128 + q_k), f32 accumulation. `mask` and
// `bias` hold kAffinePairMask and kAffinePairBias in vector registers; the
// pairs of words (0, 1) and (2, 3) come from one 64-bit shift per pair index
// and one v_and_or_b32 each. NA independent partial sums (word j feeds sum
// j % NA) shorten the chain of dependent dot products.
template <int NA>
__device__ __forceinline__ float group_dot_biased(const u32x4& words, const XGroup& xg, uint32_t mask,
                                                  uint32_t bias) {
    float d[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) d[a] = 0.f;
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
        uint32_t p[2][4];
        affine_pairs2_biased_bf16(words[2 * jp], words[2 * jp + 1], mask, bias, p);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int j = 2 * jp + h;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                d[j % NA] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(p[h][i]), as_bf16x2(xg.pair[j][i]), d[j % NA], false);
        }
    }
#pragma unroll
    for (int a = 1; a < NA; ++a) d[0] += d[a];
    return d[0];
}

// Reduces R per-lane partial sums over the wavefront, all in the vector ALU
// (no LDS crossbar). The first log2(R) steps halve the values a lane holds,
// exchanging with the lane at distance 32, 16, 8 (the upper lane keeps the
// upper half of the rows); the rest add within the remaining lane group.
// Afterwards lane l holds the full sum of row (l >> (6 - log2 R)).
//  - distance 32 / 16: v_permlane32_swap / v_permlane16_swap with the pair
//    (v[i], v[i + h]) returns, in both lanes of each exchanged pair, exactly
//    the two values that lane must add;
//  - distance 8: DPP row_ror:8 within 16-lane rows, on a per-lane selected
//    value;
//  - the closing sums: DPP row_ror 8/4/2/1 over 16 lanes, or quad_perm
//    xor 1, xor 2 and row_half_mirror over 8 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_get(float v) {
    return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowRor = 0x120;     // + 1..15: rotate right within 16 lanes
constexpr int kDppHalfMirror = 0x141; // reverse within 8 lanes

template <int R>
__device__ __forceinline__ float wave_reduce_rows(float (&v)[R], int lane) {
    static_assert(R == 1 || R == 2 || R == 4 || R == 8, "rows per wavefront: 1, 2, 4 or 8");
    if constexpr (R >= 2) {
#pragma unroll
        for (int i = 0; i < R / 2; ++i) {
            const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + R / 2]), false, false);
            v[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
    }
    if constexpr (R >= 4) {
#pragma unroll
        for (int i = 0; i < R / 4; ++i) {
            const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + R / 4]), false, false);
            v[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
    }
    float t = v[0];
    if constexpr (R == 8) {
        const bool upper = (lane & 8) != 0;
        const float keep = upper ? v[1] : v[0];
        const float send = upper ? v[0] : v[1];
        t = keep + dpp_get<kDppRowRor + 8>(send);
    }
    if constexpr (R <= 4) {
        // 16 lanes share a row (R = 4), or more (R = 1, 2: finish across rows).
        t += dpp_get<kDppRowRor + 8>(t);
        t += dpp_get<kDppRowRor + 4>(t);
        t += dpp_get<kDppRowRor + 2>(t);
        t += dpp_get<kDppRowRor + 1>(t);
        if constexpr (R <= 2) {
            const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
            t = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
        if constexpr (R == 1) {
            const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
            t = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
    } else {
        t += dpp_get<kDppQuadXor1>(t);
        t += dpp_get<kDppQuadXor2>(t);
        t += dpp_get<kDppHalfMirror>(t);
    }
    return t;
}

template <int R>
constexpr int log2_rows() {
    return R == 1 ? 0 : R == 2 ? 1 : R == 4 ? 2 : R == 8 ? 3 : R == 16 ? 4 : 5;
}

// One wavefront computes R rows. K is covered in chunks of 64 groups (one
// group per lane); T chunks are loaded before any arithmetic so that every
// load of the wavefront is in flight at once. T = 0 selects a runtime loop
// over chunks (one chunk in flight at a time) for long K. Loads go through
// buffer resources over the wave's R rows: the row offset is a scalar
// register and the lane offset a 32-bit vector register, so addressing costs
// no vector ALU work. AUX is the load cache policy (0, or 2 = non-temporal);
// NA the number of independent partial sums per group dot product.
template <int R, int T, int AUX, int NA = 1>
__global__ __launch_bounds__(kWave) void qmv_affine4_kernel(
    const uint32_t* __restrict__ w, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int K, int N, int chunks) {
    const int lane = threadIdx.x;
    const int n0 = blockIdx.x * R;  // N % 32 == 0 and R | 32: rows n0 .. n0+R-1 exist
    const int G = K / 32;
    const uint32_t mask = vreg(kAffinePairMask), bias = vreg(kAffinePairBias);
    const int wrow = K / 2;  // bytes per packed weight row
    const int srow = G * 2;  // bytes per scale (bias) row
    const __amdgpu_buffer_rsrc_t wsrc =
        make_rsrc(reinterpret_cast<const uint8_t*>(w) + (size_t)n0 * wrow, (uint32_t)(R * wrow));
    const __amdgpu_buffer_rsrc_t ssrc =
        make_rsrc(reinterpret_cast<const uint8_t*>(scales) + (size_t)n0 * srow, (uint32_t)(R * srow));
    const __amdgpu_buffer_rsrc_t bsrc =
        make_rsrc(reinterpret_cast<const uint8_t*>(biases) + (size_t)n0 * srow, (uint32_t)(R * srow));
    const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(x, (uint32_t)(K * 2));

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;

    constexpr int TB = T > 0 ? T : 1;
    const int nch = T > 0 ? T : chunks;
    for (int t0 = 0; t0 < nch; t0 += TB) {
        u32x4 xr[TB][4];
        u32x4 wv[TB][R];
        uint32_t sv[TB][R], bv[TB][R];
        // Issue order = consumption order, because loads complete in issue
        // order for the wait counter: x and the (small) scales and biases
        // first, then the weights row by row, each pinned in place so the
        // arithmetic on row r waits only for loads up to row r. Idle lanes
        // (past the last group) read the last group again.
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const int g = (t0 + t) * kWave + lane;
            const uint32_t gc = (uint32_t)(g < G ? g : G - 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) xr[t][j] = __builtin_amdgcn_raw_buffer_load_b128(xsrc, gc * 64u + 16u * j, 0, 0);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                sv[t][r] = __builtin_amdgcn_raw_buffer_load_b16(ssrc, gc * 2u, r * srow, AUX);
                bv[t][r] = __builtin_amdgcn_raw_buffer_load_b16(bsrc, gc * 2u, r * srow, AUX);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const int g = (t0 + t) * kWave + lane;
            const uint32_t gc = (uint32_t)(g < G ? g : G - 1);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                wv[t][r] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, gc * 16u, r * wrow, AUX);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            XGroup xg;
            x_group_from_raw(xr[t], (t0 + t) * kWave + lane < G, xg);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float s = bf16_bits_to_f32(sv[t][r]);
                const float b = bf16_bits_to_f32(bv[t][r]);
                const float d = group_dot_biased<NA>(wv[t][r], xg, mask, bias);
                acc[r] = __builtin_fmaf(s, d, acc[r]);
                acc[r] = __builtin_fmaf(__builtin_fmaf(-128.f, s, b), xg.sum, acc[r]);
            }
        }
    }

    const float total = wave_reduce_rows<R>(acc, lane);
    constexpr int shift = 6 - log2_rows<R>();
    if ((lane & ((1 << shift) - 1)) == 0) y[n0 + (lane >> shift)] = f32_to_bf16_bits(total);
}


// Shared-x form: T chunks of 64 groups (T <= kXChunks), kXWaves wavefronts x
// kXRows weight rows per workgroup, and M rows of x taken MB at a time (a
// small batch: every weight row read once serves all of them). Piece p
// (16 bytes = 8 x values) of a batch's x is loaded by thread p mod 512 and
// becomes the four pairs (8j+i, 8j+i+4) of its group, piece j = p % 4, plus a
// partial sum that the group's four (adjacent) lanes add up. Pieces past the
// last group or row load as zeros (the buffer bound), so idle groups
// contribute nothing. Weights stay in registers across batches.
template <int T, int MB, int WPG = kXWaves>
__global__ __launch_bounds__(kWave * WPG) void qmv_affine4_xlds_kernel(
    const uint32_t* __restrict__ w, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int M, int K, int N) {
    constexpr int R = kXRows, kThreads = kWave * WPG;
    constexpr int kRowPieces = T * kWave * 4;  // pieces of one x row
    constexpr int kPieces = MB * kRowPieces;
    constexpr int kPerLane = (kPieces + kThreads - 1) / kThreads;
    constexpr int kVals = R * MB;              // row sums per lane, reduced together
    __shared__ __attribute__((aligned(16))) uint32_t xp[MB * T * kWave * kXStride];
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = (blockIdx.x * WPG + wave) * R;  // N is even: rows n0 and n0 + 1 exist when n0 < N
    const int G = K / 32;
    const uint32_t mask = vreg(kAffinePairMask), bias = vreg(kAffinePairBias);
    const int wrow = K / 2, srow = G * 2;
    // A wavefront past the last row (when N is not a multiple of the
    // workgroup's rows) reads nothing and stores nothing, but still takes
    // part in the barriers.
    const bool live = n0 < N;
    const size_t nl = live ? (size_t)n0 : 0;
    const __amdgpu_buffer_rsrc_t wsrc =
        make_rsrc(reinterpret_cast<const uint8_t*>(w) + nl * wrow, live ? (uint32_t)(R * wrow) : 0u);
    const __amdgpu_buffer_rsrc_t ssrc =
        make_rsrc(reinterpret_cast<const uint8_t*>(scales) + nl * srow, live ? (uint32_t)(R * srow) : 0u);
    const __amdgpu_buffer_rsrc_t bsrc =
        make_rsrc(reinterpret_cast<const uint8_t*>(biases) + nl * srow, live ? (uint32_t)(R * srow) : 0u);
    const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);

    // Issue order = consumption order (loads complete in issue order for the
    // wait counter): the first batch's x pieces, scales and biases, then the
    // weights row by row.
    auto load_x = [&](int m0, u32x4 (&xv)[kPerLane]) {
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int p = tid + i * kThreads, mm = p / kRowPieces, q = p % kRowPieces;
            const bool live = m0 + mm < M && q < 4 * G;
            xv[i] = __builtin_amdgcn_raw_buffer_load_b128(
                xsrc, live ? ((uint32_t)(m0 + mm) * (uint32_t)K * 2u + (uint32_t)q * 16u) : 0x80000000u, 0, 0);
        }
    };
    u32x4 xv[kPerLane];
    load_x(0, xv);
    uint32_t sv[T][R], bv[T][R];
    u32x4 wv[T][R];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int g = t * kWave + lane;
        const uint32_t gc = (uint32_t)(g < G ? g : G - 1);  // idle lanes re-read the last group
#pragma unroll
        for (int r = 0; r < R; ++r) {
            sv[t][r] = __builtin_amdgcn_raw_buffer_load_b16(ssrc, gc * 2u, r * srow, kGemvAux);
            bv[t][r] = __builtin_amdgcn_raw_buffer_load_b16(bsrc, gc * 2u, r * srow, kGemvAux);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int g = t * kWave + lane;
        const uint32_t gc = (uint32_t)(g < G ? g : G - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            wv[t][r] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, gc * 16u, r * wrow, kGemvAux);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    for (int m0 = 0; m0 < M; m0 += MB) {
        if (m0 > 0) {
            __syncthreads();  // every wavefront is done with the previous batch's x
            load_x(m0, xv);
        }
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int p = tid + i * kThreads, mm = p / kRowPieces, q = p % kRowPieces;
            const u32x4 v = xv[i];
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v[j]), as_bf16x2(0x3F803F80u), s, false);
            s += dpp_get<kDppQuadXor1>(s);
            s += dpp_get<kDppQuadXor2>(s);
            if (p < kPieces) {
                uint32_t* d = xp + (mm * T * kWave + (q >> 2)) * kXStride;
                *reinterpret_cast<u32x4*>(d + 4 * (q & 3)) =
                    u32x4{__builtin_amdgcn_perm(v[2], v[0], 0x05040100u), __builtin_amdgcn_perm(v[2], v[0], 0x07060302u),
                          __builtin_amdgcn_perm(v[3], v[1], 0x05040100u), __builtin_amdgcn_perm(v[3], v[1], 0x07060302u)};
                if ((q & 3) == 0) d[16] = __float_as_uint(s);
            }
        }
        __syncthreads();
        // Decode the weights afresh for each batch: hoisted out of the loop, the
        // pairs would hold 16 registers per group and row.
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int r = 0; r < R; ++r) asm volatile("" : "+v"(wv[t][r]));

        float acc[kVals];
#pragma unroll
        for (int v = 0; v < kVals; ++v) acc[v] = 0.f;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if constexpr (MB == 1) {
                XGroup xg;
                const uint32_t* d = xp + (t * kWave + lane) * kXStride;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(d + 4 * j);
#pragma unroll
                    for (int i = 0; i < 4; ++i) xg.pair[j][i] = v[i];
                }
                xg.sum = __uint_as_float(d[16]);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float s = bf16_bits_to_f32(sv[t][r]);
                    const float b = bf16_bits_to_f32(bv[t][r]);
                    const float dd = group_dot_biased<kGemvAcc>(wv[t][r], xg, mask, bias);
                    acc[r] = __builtin_fmaf(s, dd, acc[r]);
                    acc[r] = __builtin_fmaf(__builtin_fmaf(-128.f, s, b), xg.sum, acc[r]);
                }
            } else {
                // Each row's pairs once, against every x row of the batch.
                uint32_t pr[R][4][4];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i) pr[r][j][i] = affine_pair_biased_bf16(wv[t][r][j], i, mask, bias);
#pragma unroll
                for (int mm = 0; mm < MB; ++mm) {
                    const uint32_t* d = xp + (mm * T * kWave + t * kWave + lane) * kXStride;
                    u32x4 xq[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) xq[j] = *reinterpret_cast<const u32x4*>(d + 4 * j);
                    const float xs = __uint_as_float(d[16]);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        float d0 = 0.f, d1 = 0.f;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                float& dd = (j & 1) ? d1 : d0;
                                dd = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pr[r][j][i]), as_bf16x2(xq[j][i]), dd, false);
                            }
                        const float s = bf16_bits_to_f32(sv[t][r]);
                        const float b = bf16_bits_to_f32(bv[t][r]);
                        float& a = acc[r * MB + mm];
                        a = __builtin_fmaf(s, d0 + d1, a);
                        a = __builtin_fmaf(__builtin_fmaf(-128.f, s, b), xs, a);
                    }
                }
            }
        }
        const float total = wave_reduce_rows<kVals>(acc, lane);
        constexpr int shift = 6 - log2_rows<kVals>();
        const int v = lane >> shift;  // r * MB + mm
        if (live && (lane & ((1 << shift) - 1)) == 0 && m0 + v % MB < M)
            y[(size_t)(m0 + v % MB) * N + n0 + v / MB] = f32_to_bf16_bits(total);
    }
}

}  // namespace w4mi

using namespace w4mi;

namespace w4mi {

// The shared-x form for M rows of x (1 <= M <= kAffineBatchRows, K <=
// kAffineBatchMaxK = 64 * 32 * kXChunks): MB rows of x per batch (4, or 2 where 4 chunks would take 80 KB
// of LDS), one workgroup per 16 weight rows.
int xlds_batch_rows(int M, int K) {
    const int chunks = (K / 32 + kWave - 1) / kWave;
    return M == 1 ? 1 : (M == 2 || chunks > 2) ? 2 : 4;
}

void launch_xlds(const uint32_t* w, const uint16_t* scales, const uint16_t* biases, const uint16_t* x, uint16_t* y,
                 int M, int K, int N, hipStream_t s) {
    static_assert(kAffineBatchMaxK == 32 * kWave * kXChunks, "four chunks of 64 groups");
    const int chunks = (K / 32 + kWave - 1) / kWave;
    const int mb = xlds_batch_rows(M, K);
    const dim3 grid((unsigned)(N / (kXWaves * kXRows))), block(kWave * kXWaves);
    if (mb == 1) {
        // One row of x: pick 8, 7 or 6 wavefronts per workgroup so that the
        // workgroups fill whole rounds of the 256 compute units best (every
        // CU then streams the same share of the weights to the end).
        int best = kXWaves;
        double best_eff = 0.0;
        for (int wpg = kXWaves; wpg >= kXWaves - 2; --wpg) {
            const double rounds = (double)((N + 2 * wpg - 1) / (2 * wpg)) / kCUs;
            const double eff = rounds / std::ceil(rounds);
            if (eff > best_eff + 1e-9) {
                best_eff = eff;
                best = wpg;
            }
        }
        const dim3 g1((unsigned)((N + kXRows * best - 1) / (kXRows * best))), b1(kWave * best);
#define W4_XLDS1(T, W) hipLaunchKernelGGL((qmv_affine4_xlds_kernel<T, 1, W>), g1, b1, 0, s, w, scales, biases, x, y, M, K, N)
#define W4_XLDS1_T(T) \
    switch (best) {   \
        case 7: W4_XLDS1(T, 7); break; \
        case 6: W4_XLDS1(T, 6); break; \
        default: W4_XLDS1(T, kXWaves); break; \
    }
        switch (chunks) {
            case 1: W4_XLDS1_T(1); break;
            case 2: W4_XLDS1_T(2); break;
            case 3: W4_XLDS1_T(3); break;
            default: W4_XLDS1_T(4); break;
        }
#undef W4_XLDS1_T
#undef W4_XLDS1
        return;
    }
#define W4_XLDS(T, MB) hipLaunchKernelGGL((qmv_affine4_xlds_kernel<T, MB>), grid, block, 0, s, w, scales, biases, x, y, M, K, N)
    switch (chunks * 8 + mb) {
        case 1 * 8 + 2: W4_XLDS(1, 2); break;
        case 2 * 8 + 2: W4_XLDS(2, 2); break;
        case 3 * 8 + 2: W4_XLDS(3, 2); break;
        case 4 * 8 + 2: W4_XLDS(4, 2); break;
        case 1 * 8 + 4: W4_XLDS(1, 4); break;
        default: W4_XLDS(2, 4); break;
    }
#undef W4_XLDS
}

}  // namespace w4mi

extern "C" w4_status qmv_affine4(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                                 const uint16_t* x, uint16_t* y, int64_t M, int64_t K, int64_t N,
                                 int32_t group_size, int32_t bits, void* stream) {
    w4_status st = w4_check_affine(M, K, N, group_size, bits, 1);
    if (st != W4_OK) return st;
    if (M == 0) return W4_OK;
    if (!w || !scales || !biases || !x || !y) return fail(W4_EINVAL, "qmv_affine4: null pointer argument");
    if (((uintptr_t)w & 15u) || ((uintptr_t)x & 15u)) return fail(W4_EINVAL, "qmv_affine4: w and x must be 16-byte aligned");
    const int G = (int)(K / 32);
    const int chunks = (G + kWave - 1) / kWave;
    hipStream_t s = as_stream(stream);
    if (chunks <= kXChunks) {
        launch_xlds(w, scales, biases, x, y, 1, (int)K, (int)N, s);
    } else {
        hipLaunchKernelGGL((qmv_affine4_kernel<kGemvRows, 0, kGemvAux, kGemvAcc>), dim3((unsigned)(N / kGemvRows)), dim3(kWave),
                           0, s, w, scales, biases, x, y, (int)K, (int)N, chunks);
    }
    return launch_status("qmv_affine4");
}
