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
//    When every dword of codes lies in one block, a dword form reads one dword
//    (8 columns) per lane instead (lut4_kn8_kernel, below).
// Rows of x are taken 4 at a time (the grid's y dimension). Aligned shapes
// (8 codes along the contiguous axis within one block; [K, N] with N a
// multiple of the block) read a dword or a byte of codes and one scale at a
// time; the rest decode element by element from the flat index.
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

// Operand formats: single precision (the f32 path), or binary16 x, scales and
// y with the decoded weight rounded to binary16 before the products (the
// half-precision path's [K, N] layout; lut4 page, rounded_weight).
template <bool H>
struct LutIO;
template <>
struct LutIO<false> {
    using X = float;
    using S = float;
    using Y = float;
    __device__ __forceinline__ static float x(X v) { return v; }
    __device__ __forceinline__ static float s(S v) { return v; }
    __device__ __forceinline__ static float w(float v) { return v; }
    __device__ __forceinline__ static Y y(float v) { return v; }
};
template <>
struct LutIO<true> {
    using X = uint16_t;
    using S = uint16_t;
    using Y = uint16_t;
    __device__ __forceinline__ static float x(X v) { return f16_bits_to_f32(v); }
    __device__ __forceinline__ static float s(S v) { return f16_bits_to_f32(v); }
    __device__ __forceinline__ static float w(float v) { return (float)(_Float16)v; }
    __device__ __forceinline__ static Y y(float v) { return f32_to_f16_bits(v); }
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

template <bool H = false>
__device__ __forceinline__ float lut_weight(const uint8_t* __restrict__ packed,
                                            const typename LutIO<H>::S* __restrict__ scales, const float* book_s,
                                            int64_t flat, int64_t scale_index) {
    const uint32_t code = lut_code(packed[flat >> 1], (uint32_t)(flat & 1));
    return LutIO<H>::w(book_s[code] * LutIO<H>::s(scales[scale_index]));
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

template <bool H>
__global__ __launch_bounds__(kF32ColWaves * 64) void lut4_f32_cols_kernel(const typename LutIO<H>::X* __restrict__ x,
                                                                            const uint8_t* __restrict__ packed,
                                                                            const typename LutIO<H>::S* __restrict__ scales,
                                                                            LutBook book, typename LutIO<H>::Y* __restrict__ y,
                                                                            int M, int K, int N, int block) {
    using IO = LutIO<H>;
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
        const float w = nv ? lut_weight<H>(packed, scales, book_s, (int64_t)k * N + n, cur.q) : 0.f;
#pragma unroll
        for (int m = 0; m < kF32M; ++m) {
            const float xv = m0 + m < M ? IO::x(x[(size_t)(m0 + m) * K + k]) : 0.f;  // the same for every lane
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
            if (nv && m0 + m < M) y[(size_t)(m0 + m) * N + n] = IO::y(a);
        }
    }
}


// ---------------------------------------------------------------- aligned forms
// When each 8 consecutive codes along the contiguous axis share one block
// (block % 8 == 0 and the contiguous length a multiple of block), a lane reads
// 8 codes (one dword) and one scale at a time and looks the codes up in an LDS
// copy of the codebook (lut_offsets / lut_entry).
// [N, K], K % block == 0, block % 8 == 0: a wavefront owns 4 weight rows, lane
// l takes the 8-wide K groups l, l + 64, ... (one dword of codes per row).
// Steps of 64 whole groups run without checks, a last partial step reads the
// groups at or past K / 8 as zeros; rows at or past N (or M) are read as the
// last row and not written. The codes, scales and x come through buffer loads
// whose row offset is a scalar, and the next step's are loaded before this
// step's are used. P2: block / 8 is a power of two.
template <bool P2>
__global__ __launch_bounds__(kF32RowWaves * 64) void lut4_f32_rows8_kernel(const float* __restrict__ x,
                                                                             const uint8_t* __restrict__ packed,
                                                                             const float* __restrict__ scales,
                                                                             LutBook book, float* __restrict__ y,
                                                                             int M, int K, int N, int block) {
    __shared__ float book_s[16];
    if (threadIdx.x < 16) book_s[threadIdx.x] = book.v[threadIdx.x];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = (blockIdx.x * kF32RowWaves + wave) * kF32Rows;
    const int m0 = blockIdx.y * kF32M;
    const int G8 = K / 8, bpr = K / block, per8 = block / 8;  // 8-wide groups and blocks per row
    const __amdgpu_buffer_rsrc_t wsrc = make_rsrc(packed, (uint32_t)((int64_t)N * K / 2));
    const __amdgpu_buffer_rsrc_t ssrc = make_rsrc(scales, (uint32_t)((int64_t)N * bpr * 4));
    const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(x, (uint32_t)((int64_t)M * K * 4));
    int wro[kF32Rows], sro[kF32Rows], xro[kF32M];  // byte offsets of the rows (uniform)
#pragma unroll
    for (int r = 0; r < kF32Rows; ++r) {
        const int n = min(nb + r, N - 1);
        wro[r] = n * (K / 2);
        sro[r] = n * bpr * 4;
    }
#pragma unroll
    for (int m = 0; m < kF32M; ++m) xro[m] = min(m0 + m, M - 1) * K * 4;
    float acc[kF32Rows][kF32M], cor[kF32Rows][kF32M], part[kF32Rows][kF32M];
#pragma unroll
    for (int r = 0; r < kF32Rows; ++r)
#pragma unroll
        for (int m = 0; m < kF32M; ++m) acc[r][m] = cor[r][m] = part[r][m] = 0.f;
    // One step's operands: x (8 k of each row of x) and a dword of codes and a
    // scale for each weight row.
    struct Step {
        f32x4 xa[kF32M], xb[kF32M];
        uint32_t word[kF32Rows];
        float sc[kF32Rows];
    };
    // Block of group g within its row: g / per8, a shift when per8 is a power
    // of two.
    const int sh = __builtin_ctz((unsigned)per8);
    // full: every lane's group is below K / 8 (no checks).
    auto load = [&](auto full, int g0, Step& st) {
        const int g = g0 + lane;
        const bool gv = decltype(full)::value || g < G8;
        const int gc = gv ? g : G8 - 1;
        const uint32_t gx = (uint32_t)gc, sq = (uint32_t)(P2 ? gc >> sh : gc / per8);
#pragma unroll
        for (int m = 0; m < kF32M; ++m) {
            st.xa[m] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xsrc, 32u * gx, xro[m], 0));
            st.xb[m] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xsrc, 32u * gx + 16u, xro[m], 0));
        }
#pragma unroll
        for (int r = 0; r < kF32Rows; ++r) {
            st.word[r] = __builtin_amdgcn_raw_buffer_load_b32(wsrc, 4u * gx, wro[r], 0);
            st.sc[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ssrc, 4u * sq, sro[r], 0));
        }
        if (!decltype(full)::value && !gv) {
#pragma unroll
            for (int m = 0; m < kF32M; ++m) st.xa[m] = st.xb[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < kF32Rows; ++r) {
                st.word[r] = 0u;
                st.sc[r] = 0.f;
            }
        }
    };
    using Full = std::integral_constant<bool, true>;
    using Part = std::integral_constant<bool, false>;
    auto use = [&](const Step& st) {
#pragma unroll
        for (int r = 0; r < kF32Rows; ++r) {
            uint32_t hi4, lo4;
            lut_offsets(st.word[r], hi4, lo4);
#pragma unroll
            for (int m = 0; m < kF32M; ++m) {
                float p = part[r][m];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const float w = lut_entry(book_s, hi4, lo4, t) * st.sc[r];
                    p = __builtin_fmaf(t < 4 ? st.xa[m][t] : st.xb[m][t - 4], w, p);
                }
                part[r][m] = p;
            }
        }
    };
    auto close_tile = [&]() {
#pragma unroll
        for (int r = 0; r < kF32Rows; ++r)
#pragma unroll
            for (int m = 0; m < kF32M; ++m) {
                kahan_add(acc[r][m], cor[r][m], part[r][m]);
                part[r][m] = 0.f;
            }
    };
    // Full steps in pairs, two operand sets in turn (no copies, no branches
    // between loads and uses); each pair is one tile of 16 products per lane
    // and output, added with compensation. The prefetch past the last full
    // step rereads that step (in bounds, unused). Then an odd last full step
    // and a partial step, one tile each.
    const int nfull = G8 / 64;
    Step s0, s1;
    if (nfull > 0) load(Full{}, 0, s0);
    int st = 0;
    for (; st + 2 <= nfull; st += 2) {
        load(Full{}, 64 * (st + 1), s1);
        use(s0);
        load(Full{}, 64 * min(st + 2, nfull - 1), s0);
        use(s1);
        close_tile();
    }
    if (st < nfull) {
        use(s0);
        close_tile();
    }
    if (64 * nfull < G8) {
        load(Part{}, 64 * nfull, s1);
        use(s1);
        close_tile();
    }
#pragma unroll
    for (int r = 0; r < kF32Rows; ++r)
#pragma unroll
        for (int m = 0; m < kF32M; ++m) {
            float v = acc[r][m];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            const int n = nb + r;
            if (lane == 0 && n < N && m0 + m < M) y[(size_t)(m0 + m) * N + n] = v;
        }
}

// [K, N], N % block == 0, block % 2 == 0: lane l owns columns 2l, 2l + 1 of a
// 128-column group (one byte of codes per k; the two share a scale, since an
// even block never splits a byte); 16 wavefronts split K. A wavefront stages
// its slice of x in LDS (its own region, 256 k at a time, read back as
// broadcasts) and loads the codes and scales of 16 k before using them.
constexpr int kF32XChunk = 256;
template <bool H, int C>
__global__ __launch_bounds__(kF32ColWaves * 64) void lut4_f32_cols2_kernel(const typename LutIO<H>::X* __restrict__ x,
                                                                             const uint8_t* __restrict__ packed,
                                                                             const typename LutIO<H>::S* __restrict__ scales,
                                                                             LutBook book, typename LutIO<H>::Y* __restrict__ y,
                                                                             int M, int K, int N, int block) {
    using IO = LutIO<H>;
    __shared__ float book_s[16];
    __shared__ __attribute__((aligned(16))) float xs[kF32ColWaves][kF32M][kF32XChunk];
    __shared__ float red[kF32ColWaves][C * kF32M][64];
    if (threadIdx.x < 16) book_s[threadIdx.x] = book.v[threadIdx.x];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // C = 2: lane l owns columns 2l, 2l + 1 (its own byte); C = 1: column l
    // (two lanes read each byte).
    const int n = blockIdx.x * 64 * C + C * lane;
    const bool nv = n < N;  // with C = 2, N is even: both columns or neither
    const int m0 = blockIdx.y * kF32M;
    const int span = (K + kF32ColWaves - 1) / kF32ColWaves;
    const int kb = min(K, wave * span), ke = min(K, kb + span);
    const int bpr = N / block;
    float acc[C][kF32M], cor[C][kF32M], part[C][kF32M];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int m = 0; m < kF32M; ++m) acc[c][m] = cor[c][m] = part[c][m] = 0.f;
    const int nbyte = N / 2, sidx = nv ? n / block : 0;
    float* xw = &xs[wave][0][0];
    for (int c0 = kb; c0 < ke; c0 += kF32XChunk) {
        const int len = min(kF32XChunk, ke - c0);
        // This wavefront's x slice for k in [c0, c0 + len), zero past the end.
#pragma unroll
        for (int m = 0; m < kF32M; ++m)
            for (int t = lane; t < kF32XChunk; t += 64)
                xw[m * kF32XChunk + t] = (t < len && m0 + m < M) ? IO::x(x[(size_t)(m0 + m) * K + c0 + t]) : 0.f;
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wavefront's own LDS writes are done
        // Codes and scales go 8 steps at a time, the next 8 loaded before the
        // current 8 are used; every second batch closes a 16-product tile.
        constexpr int kB = kF32Tile / 2;
        uint32_t byte[kB], nbyte_[kB];
        float sc[kB], nsc[kB];
        auto load = [&](int t0, uint32_t (&bt)[kB], float (&st)[kB]) {
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const int k = c0 + t0 + u;
                const bool v = nv && t0 + u < len;
                bt[u] = v ? packed[(size_t)k * nbyte + (n >> 1)] : 0u;
                st[u] = v ? IO::s(scales[(size_t)k * bpr + sidx]) : 0.f;
            }
        };
        load(0, byte, sc);
        for (int t0 = 0; t0 < len; t0 += kB) {
            if (t0 + kB < len) load(t0 + kB, nbyte_, nsc);
#pragma unroll
            for (int u = 0; u < kB; u += 4) {
                f32x4 xv[kF32M];
#pragma unroll
                for (int m = 0; m < kF32M; ++m) xv[m] = *reinterpret_cast<const f32x4*>(xw + m * kF32XChunk + t0 + u);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (C == 2) {
                        const float w0 = IO::w(book_s[byte[u + e] >> 4] * sc[u + e]);
                        const float w1 = IO::w(book_s[byte[u + e] & 15u] * sc[u + e]);
#pragma unroll
                        for (int m = 0; m < kF32M; ++m) {
                            part[0][m] = __builtin_fmaf(xv[m][e], w0, part[0][m]);
                            part[C - 1][m] = __builtin_fmaf(xv[m][e], w1, part[C - 1][m]);
                        }
                    } else {
                        const uint32_t code = (n & 1) ? (byte[u + e] & 15u) : (byte[u + e] >> 4);
                        const float w0 = IO::w(book_s[code] * sc[u + e]);
#pragma unroll
                        for (int m = 0; m < kF32M; ++m) part[0][m] = __builtin_fmaf(xv[m][e], w0, part[0][m]);
                    }
                }
            }
            if ((t0 / kB) & 1) {
#pragma unroll
                for (int c = 0; c < C; ++c)
#pragma unroll
                    for (int m = 0; m < kF32M; ++m) {
                        kahan_add(acc[c][m], cor[c][m], part[c][m]);
                        part[c][m] = 0.f;
                    }
            }
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                byte[u] = nbyte_[u];
                sc[u] = nsc[u];
            }
        }
    }
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int m = 0; m < kF32M; ++m) {
            kahan_add(acc[c][m], cor[c][m], part[c][m]);
            part[c][m] = 0.f;
        }
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int m = 0; m < kF32M; ++m) red[wave][c * kF32M + m][lane] = acc[c][m];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int m = 0; m < kF32M; ++m) {
                float a = 0.f, e = 0.f;
                for (int v = 0; v < kF32ColWaves; ++v) kahan_add(a, e, red[v][c * kF32M + m][lane]);  // K order
                if (nv && m0 + m < M) y[(size_t)(m0 + m) * N + n + c] = IO::y(a);
            }
    }
}

// [K, N] with block % 8 == 0 and N % block == 0: each dword of codes holds 8
// consecutive columns of one k row under one scale. A workgroup owns 8D
// columns (D dwords of each row) for all of K; in each step lane l reads
// dword l % D of row l / D, so one load instruction covers 64 / D rows. The
// workgroups that share a 128-byte line of a row are numbered so that they run
// on one XCD at the same time and the line is fetched once into its L2.
// Wavefronts split K into contiguous ranges of whole 16-step chunks. For each
// chunk a wavefront stages x in its own LDS region as [k][m] (16 bytes per k),
// loads the chunk's 16 code dwords and scales, and sums the lane's 16 products
// of each of its 32 outputs (8 columns x 4 rows of x). The 64 / D lanes that
// hold the same outputs then reduce-scatter them, so that each lane ends with
// the chunk's sums of D / 2 outputs, which it adds to its running totals with
// compensation. At the end the lanes' and then the wavefronts' totals are
// merged as (sum, error) pairs, the wavefronts in K order.
// The group width is a trade: every workgroup makes one L2 request per k row
// for its codes and one for its scale, so narrow groups multiply the requests
// (16 columns: twice as slow as 64 at M = 4, K = 4096, N = 11008), while wide
// groups leave CUs idle (64 columns: 172 workgroups there).
constexpr int kKnWaves = 16;  // wavefronts per workgroup, splitting K
constexpr int kKnDwords = 8;  // code dwords per row per workgroup: 64 columns

// (hi, lo) += (bhi, blo), the rounding error of hi + bhi kept in lo (Knuth's
// two-sum); a non-finite sum carries no error term.
__device__ __forceinline__ void two_sum_merge(float& hi, float& lo, float bhi, float blo) {
    const float s = hi + bhi;
    const float bb = s - hi;
    const float err = (hi - (s - bb)) + (bhi - bb);
    lo = __builtin_isfinite(s) ? lo + blo + err : 0.f;
    hi = s;
}

template <bool H, int D>
__global__ __launch_bounds__(kKnWaves * 64, 4) void lut4_kn8_kernel(const typename LutIO<H>::X* __restrict__ x,
                                                                     const uint8_t* __restrict__ packed,
                                                                     const typename LutIO<H>::S* __restrict__ scales,
                                                                     LutBook book, typename LutIO<H>::Y* __restrict__ y,
                                                                     int M, int K, int N, int block, int groups) {
    using IO = LutIO<H>;
    constexpr int R = 64 / D;           // rows per step; lanes that share outputs
    constexpr int CH = 16 * R;          // rows per chunk
    constexpr int NO = 8 * kF32M;       // outputs per lane in a step
    constexpr int KEEP = NO / R;        // outputs each lane keeps after the reduce-scatter
    static_assert(D == 1 || D == 2 || D == 4 || D == 8, "1, 2, 4 or 8 dwords per row");
    // Workgroup b runs on XCD b % 8. Each XCD takes one contiguous range of
    // column groups, so the groups that share a 128-byte line of a code row
    // (32 / D of them) or of a scale row (up to 32) read it through one L2,
    // apart from the lines at the ends of a range.
    const int b = blockIdx.x, xcd = b % 8, base = groups / 8, extra = groups % 8;
    const int g = xcd * base + min(xcd, extra) + b / 8;  // the grid has exactly `groups` columns
    __shared__ float book_s[16];
    __shared__ __attribute__((aligned(16))) float xs[kKnWaves][CH][kF32M];
    __shared__ float red[kKnWaves][2][D * NO];
    if (threadIdx.x < 16) book_s[threadIdx.x] = book.v[threadIdx.x];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane % D, r = lane / D;
    const int n0 = g * 8 * D + 8 * j;
    const bool nv = n0 < N;  // N % 8 == 0: all 8 columns or none
    const int m0 = blockIdx.y * kF32M;
    const int chunks = (K + CH - 1) / CH, per_wave = (chunks + kKnWaves - 1) / kKnWaves;
    const int cb = min(chunks, wave * per_wave), ce = min(chunks, cb + per_wave);
    // Buffer loads return zero past the end of their buffer, which covers rows
    // at or past K of the codes and scales and rows of x at or past M; lanes
    // past N, and x columns at or past K, take an offset past every end.
    constexpr uint32_t kOut = 0x80000000u;
    constexpr uint32_t XB = sizeof(typename IO::X), SB = sizeof(typename IO::S);
    const __amdgpu_buffer_rsrc_t wsrc = make_rsrc(packed, (uint32_t)((int64_t)K * N / 2));
    const __amdgpu_buffer_rsrc_t ssrc = make_rsrc(scales, (uint32_t)((int64_t)K * (N / block) * SB));
    const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(x, (uint32_t)((int64_t)M * K * XB));
    const uint32_t wrow = (uint32_t)N / 2, srow = (uint32_t)(N / block) * SB;  // bytes per k row
    const uint32_t wcol = nv ? 4u * (uint32_t)(n0 >> 3) : kOut, scol = nv ? (uint32_t)(n0 / block) * SB : kOut;
    // After the reduce-scatter lane r keeps outputs o0 .. o0 + KEEP - 1 of its
    // 32 (output o = column 8j + o / 4, row of x m0 + o % 4): at the level
    // that pairs lanes r and r ^ 2^t it keeps the upper half of what remains
    // when bit t of r is set.
    int o0 = 0;
#pragma unroll
    for (int t = 0, h = NO / 2; h >= KEEP; ++t, h /= 2) o0 += ((r >> t) & 1) ? h : 0;
    float acc[KEEP], cor[KEEP];
#pragma unroll
    for (int e = 0; e < KEEP; ++e) acc[e] = cor[e] = 0.f;
    float* xw = &xs[wave][0][0];
    for (int ch = cb; ch < ce; ++ch) {
        const int kc = ch * CH;
        // x for rows [kc, kc + CH) of the chunk, zero past K or M.
        f32x4 xin[CH / 64];
#pragma unroll
        for (int u = 0; u < CH / 64; ++u) {
            const int k = kc + lane + 64 * u;
            const uint32_t xo = k < K ? ((uint32_t)m0 * K + k) * XB : kOut;
#pragma unroll
            for (int m = 0; m < kF32M; ++m) {
                const uint32_t off = xo + (uint32_t)(m * K) * XB;
                if constexpr (H)
                    xin[u][m] = IO::x(__builtin_amdgcn_raw_buffer_load_b16(xsrc, off, 0, 0));
                else
                    xin[u][m] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xsrc, off, 0, 0));
            }
        }
        uint32_t word[16];
        float sc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t k = (uint32_t)(kc + i * R + r);
            word[i] = __builtin_amdgcn_raw_buffer_load_b32(wsrc, k * wrow + wcol, 0, 0);
            if constexpr (H)
                sc[i] = IO::s(__builtin_amdgcn_raw_buffer_load_b16(ssrc, k * srow + scol, 0, 0));
            else
                sc[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ssrc, k * srow + scol, 0, 0));
        }
        // The previous chunk's LDS reads are done before its rows are written.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int u = 0; u < CH / 64; ++u) *reinterpret_cast<f32x4*>(xw + (lane + 64 * u) * kF32M) = xin[u];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        float part[NO];
#pragma unroll
        for (int o = 0; o < NO; ++o) part[o] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const f32x4 xv = *reinterpret_cast<const f32x4*>(xw + (i * R + r) * kF32M);
            // Byte t of the dword holds columns 2t (high nibble) and 2t + 1;
            // each byte of hi4 / lo4 is 4 x the code, the LDS byte offset of
            // its codebook entry.
            uint32_t hi4 = (word[i] >> 2) & 0x3C3C3C3Cu, lo4 = (word[i] << 2) & 0x3C3C3C3Cu;
            // Opaque to the compiler, which would otherwise fold each byte
            // pick back into a shift and a mask of the word (two operations
            // per code instead of one byte extract).
            asm("" : "+v"(hi4), "+v"(lo4));
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t off = (((c & 1) ? lo4 : hi4) >> (8 * (c / 2))) & 0xFFu;
                const float bk = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(book_s) + off);
                const float w = IO::w(bk * sc[i]);
#pragma unroll
                for (int m = 0; m < kF32M; ++m) part[c * kF32M + m] = __builtin_fmaf(xv[m], w, part[c * kF32M + m]);
            }
        }
        // Reduce-scatter over the R lanes r (lane distance D * 2^t at level t).
#pragma unroll
        for (int t = 0, h = NO / 2; h >= KEEP; ++t, h /= 2) {
            // All ones where this lane keeps the upper half; the halves are
            // picked by bits (a conditional pick of two array elements turns
            // into a run-time index into the whole array).
            const uint32_t up = ((r >> t) & 1) ? ~0u : 0u;
#pragma unroll
            for (int e = 0; e < h; ++e) {
                const uint32_t lo = __builtin_bit_cast(uint32_t, part[e]), hi = __builtin_bit_cast(uint32_t, part[e + h]);
                const float send = __builtin_bit_cast(float, (lo & up) | (hi & ~up));
                const float keep = __builtin_bit_cast(float, (hi & up) | (lo & ~up));
                part[e] = keep + __shfl_xor(send, D << t, 64);
            }
        }
#pragma unroll
        for (int e = 0; e < KEEP; ++e) kahan_add(acc[e], cor[e], part[e]);
    }
    // The wavefront's totals: lane (j, r) holds outputs o0 .. o0 + KEEP - 1 of
    // column group j.
#pragma unroll
    for (int e = 0; e < KEEP; ++e) {
        red[wave][0][j * NO + o0 + e] = acc[e];
        red[wave][1][j * NO + o0 + e] = -cor[e];  // kahan_add keeps the negated error
    }
    __syncthreads();
    for (int t = threadIdx.x; t < D * NO; t += kKnWaves * 64) {
        float hi = red[0][0][t], lo = red[0][1][t];
        for (int v = 1; v < kKnWaves; ++v) two_sum_merge(hi, lo, red[v][0][t], red[v][1][t]);  // K order
        const int o = t % NO, m = o % kF32M, col = g * 8 * D + (t / NO) * 8 + o / kF32M;
        if (col < N && m0 + m < M) y[(size_t)(m0 + m) * N + col] = IO::y(hi + lo);
    }
}

// The dword form's conditions: 8 columns of a dword share a block, packed
// dword-aligned, and every buffer offset it forms (up to one chunk past K, and
// the out-of-range marker added to any of them) fits in 32 bits.
inline bool kn8_ok(const void* packed, int64_t M, int64_t K, int64_t N, int32_t block, int64_t xb, int64_t sb) {
    const int64_t lim = int64_t(1) << 31, kk = K + 256;
    return N % block == 0 && block % 8 == 0 && ((uintptr_t)packed & 3u) == 0 && kk * (N / 2) < lim &&
           kk * (N / block) * sb < lim && M * K * xb < lim;
}

template <bool H, int D>
void launch_lut4_kn8(const typename LutIO<H>::X* x, const uint8_t* packed, const typename LutIO<H>::S* scales,
                     const LutBook& b, typename LutIO<H>::Y* y, int64_t M, int64_t K, int64_t N, int32_t block,
                     hipStream_t s) {
    const int groups = (int)((N + 8 * D - 1) / (8 * D));
    const dim3 grid((unsigned)groups, (unsigned)((M + kF32M - 1) / kF32M));
    hipLaunchKernelGGL((lut4_kn8_kernel<H, D>), grid, dim3(kKnWaves * 64), 0, s, x, packed, scales, b, y, (int)M,
                       (int)K, (int)N, (int)block, groups);
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
        const int64_t lim = int64_t(1) << 31;  // buffer offsets of the dword form fit in 31 bits
        if (block % 8 == 0 && K % block == 0 && ((uintptr_t)packed & 3u) == 0 && ((uintptr_t)x & 15u) == 0 &&
            N * (K / 2) < lim && N * (K / block) * 4 < lim && M * K * 4 < lim) {
            if (((block / 8) & (block / 8 - 1)) == 0)
                hipLaunchKernelGGL(lut4_f32_rows8_kernel<true>, grid, dim3(kF32RowWaves * 64), 0, s, x, packed, scales,
                                   b, y, (int)M, (int)K, (int)N, (int)block);
            else
                hipLaunchKernelGGL(lut4_f32_rows8_kernel<false>, grid, dim3(kF32RowWaves * 64), 0, s, x, packed, scales,
                                   b, y, (int)M, (int)K, (int)N, (int)block);
        } else {
            hipLaunchKernelGGL(lut4_f32_rows_kernel, grid, dim3(kF32RowWaves * 64), 0, s, x, packed, scales, b, y,
                               (int)M, (int)K, (int)N, (int)block);
        }
    } else if (kn8_ok(packed, M, K, N, block, 4, 4)) {
        launch_lut4_kn8<false, kKnDwords>(x, packed, scales, b, y, M, K, N, block, s);
    } else if (N % block == 0) {
        const dim3 grid((unsigned)((N + 63) / 64), my);
        hipLaunchKernelGGL((lut4_f32_cols2_kernel<false, 1>), grid, dim3(kF32ColWaves * 64), 0, s, x, packed, scales, b,
                           y, (int)M, (int)K, (int)N, (int)block);
    } else {
        const dim3 grid((unsigned)((N + 63) / 64), my);
        hipLaunchKernelGGL(lut4_f32_cols_kernel<false>, grid, dim3(kF32ColWaves * 64), 0, s, x, packed, scales, b, y,
                           (int)M, (int)K, (int)N, (int)block);
    }
    return launch_status("qmm_lut4_f32");
}

namespace w4mi {

// The half-precision lookup matmul with the weight stored [K, N] (qmm_lut4,
// transpose == 0): the column kernels above in binary16.
void launch_lut4_kn_f16(const uint16_t* x, const uint8_t* packed, const uint16_t* scales, const float* book, uint16_t* y,
                        int64_t M, int64_t K, int64_t N, int32_t block, hipStream_t s) {
    LutBook b;
    for (int i = 0; i < 16; ++i) b.v[i] = book[i];
    const unsigned my = (unsigned)((M + kF32M - 1) / kF32M);
    if (kn8_ok(packed, M, K, N, block, 2, 2)) {
        launch_lut4_kn8<true, kKnDwords>(x, packed, scales, b, y, M, K, N, block, s);
    } else if (N % block == 0) {
        const dim3 grid((unsigned)((N + 63) / 64), my);
        hipLaunchKernelGGL((lut4_f32_cols2_kernel<true, 1>), grid, dim3(kF32ColWaves * 64), 0, s, x, packed, scales, b,
                           y, (int)M, (int)K, (int)N, (int)block);
    } else {
        const dim3 grid((unsigned)((N + 63) / 64), my);
        hipLaunchKernelGGL(lut4_f32_cols_kernel<true>, grid, dim3(kF32ColWaves * 64), 0, s, x, packed, scales, b, y,
                           (int)M, (int)K, (int)N, (int)block);
    }
}

}  // namespace w4mi
