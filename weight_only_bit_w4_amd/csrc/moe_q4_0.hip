// qmm_id_q4_0: expert-routed matmul over GGML Q4_0 blocks (mlx-native MoE
// page): out[t*top_k + s][n] = sum_k (q - 8) d of expert ids[t*top_k + s],
// row n, times x[t][k].
//
// Two launches on the caller's stream, as the page's map0 + mm pair:
//  1. moe_group_kernel: workgroup 0 counts the routed rows per expert, scans
//     the counts and scatters row indices into per-expert lists (the page's
//     htpe / hids); the other workgroups store x as binary16 (the matrix-core
//     operand type). Stream order makes both visible to launch 2.
//  2. moe_gemm_kernel: one workgroup per (expert, 128 weight rows) reads that
//     slice of the expert's weights exactly once and applies it to every
//     routed row of the expert (up to 64 per pass) with
//     v_mfma_f32_16x16x32_f16, f32 accumulation. The routed rows' x is staged
//     in LDS per 256-wide K window; each lane decodes its Q4_0 nibbles to fp16
//     (q - 8) * d in registers.
#include "w4mi_device.hpp"
#include "w4mi_host.hpp"

namespace w4mi {

constexpr int kGroupThreads = 1024;

__global__ __launch_bounds__(kGroupThreads) void moe_group_kernel(const uint32_t* __restrict__ ids, const float* __restrict__ x,
                                                                  uint8_t* __restrict__ scratch, float* __restrict__ out,
                                                                  int n_rows, int n_experts, int N, int64_t x_count,
                                                                  IdScratchLayout lay) {
    if (blockIdx.x > 0) {
        // x -> binary16, 8 values per thread per step.
        uint16_t* xh = reinterpret_cast<uint16_t*>(scratch + lay.xh);
        const int64_t stride = (int64_t)(gridDim.x - 1) * kGroupThreads * 8;
        for (int64_t i = ((int64_t)(blockIdx.x - 1) * kGroupThreads + threadIdx.x) * 8; i < x_count; i += stride) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(x + i);
            const f32x4 b = *reinterpret_cast<const f32x4*>(x + i + 4);
            *reinterpret_cast<u32x4*>(xh + i) = u32x4{pack_f16x2(a[0], a[1]), pack_f16x2(a[2], a[3]),
                                                      pack_f16x2(b[0], b[1]), pack_f16x2(b[2], b[3])};
        }
        return;
    }
    extern __shared__ uint32_t cnt[];  // [n_experts], counts then cursors
    __shared__ uint32_t part[kGroupThreads];
    __shared__ uint32_t bad_s;
    const int tid = threadIdx.x;
    uint32_t* counts = reinterpret_cast<uint32_t*>(scratch + lay.counts);
    uint32_t* offsets = reinterpret_cast<uint32_t*>(scratch + lay.offsets);
    uint32_t* rows = reinterpret_cast<uint32_t*>(scratch + lay.rows);

    for (int e = tid; e < n_experts; e += kGroupThreads) cnt[e] = 0u;
    if (tid == 0) bad_s = 0u;
    __syncthreads();
    for (int r = tid; r < n_rows; r += kGroupThreads) {
        const uint32_t e = ids[r];
        if (e < (uint32_t)n_experts)
            atomicAdd(&cnt[e], 1u);
        else
            atomicAdd(&bad_s, 1u);
    }
    __syncthreads();
    // Exclusive scan: each thread sums a contiguous segment, then a scan of
    // the per-thread partial sums.
    const int seg = (n_experts + kGroupThreads - 1) / kGroupThreads;
    const int e0 = tid * seg, e1 = min(n_experts, e0 + seg);
    uint32_t local = 0u;
    for (int e = e0; e < e1; ++e) local += cnt[e];
    part[tid] = local;
    __syncthreads();
    for (int off = 1; off < kGroupThreads; off <<= 1) {
        const uint32_t v = tid >= off ? part[tid - off] : 0u;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    uint32_t run = part[tid] - local;  // exclusive prefix of this segment
    for (int e = e0; e < e1; ++e) {
        const uint32_t c = cnt[e];
        counts[e] = c;
        offsets[e] = run;
        cnt[e] = run;  // becomes the scatter cursor
        run += c;
    }
    if (tid == kGroupThreads - 1) offsets[n_experts] = part[kGroupThreads - 1];
    __syncthreads();
    for (int r = tid; r < n_rows; r += kGroupThreads) {
        const uint32_t e = ids[r];
        if (e < (uint32_t)n_experts) {
            rows[atomicAdd(&cnt[e], 1u)] = (uint32_t)r;
        } else {
            for (int n = 0; n < N; ++n) out[(size_t)r * N + n] = 0.f;  // no expert to read
        }
    }
    if (tid == 0) *reinterpret_cast<uint32_t*>(scratch + lay.bad_ids) = bad_s;
}

constexpr int kMoeThreads = 256;
constexpr int kMoeNS = 2;                       // 16-row weight sub-tiles per wavefront
constexpr int kMoeBN = 4 * 16 * kMoeNS;         // weight rows per workgroup
constexpr int kMoeMT = 4;                       // 16-row routed tiles per pass
constexpr int kMoeWin = 256;                    // K per window (8 Q4_0 blocks)
constexpr int kMoeXLd = kMoeWin + 8;            // padded LDS row, fp16 elements

// The eight weights a lane feeds one 16x16x32 fragment: from one aligned qs
// dword (bytes 4i..4i+3 of a block) the elements 4i..4i+3 (low nibbles) and
// 16+4i..16+4i+3 (high nibbles), as fp16 (q - 8) * d in that order.
__device__ __forceinline__ u32x4 q4_0_fragment(uint32_t qs, uint32_t d2) {
    uint32_t raw[4];
    q4_0_biased_pairs(qs, raw);
    const f16x2 bias = as_f16x2(0xE408E408u);  // -1032: (1024 + q) - 1032 = q - 8, exact
    const f16x2 d = as_f16x2(d2);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = as_u32((as_f16x2(raw[j]) + bias) * d);
    return o;
}

__global__ __launch_bounds__(kMoeThreads) void moe_gemm_kernel(const uint8_t* __restrict__ w, const uint8_t* __restrict__ scratch,
                                                               float* __restrict__ out, int N, int K, int top_k,
                                                               uint64_t expert_stride, IdScratchLayout lay) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[kMoeMT * 16 * kMoeXLd];
    const int tiles_n = (N + kMoeBN - 1) / kMoeBN;
    const int e = blockIdx.x / tiles_n;
    const int nt = blockIdx.x % tiles_n;
    const uint32_t cnt = reinterpret_cast<const uint32_t*>(scratch + lay.counts)[e];
    if (cnt == 0u) return;
    const uint32_t off = reinterpret_cast<const uint32_t*>(scratch + lay.offsets)[e];
    const uint32_t* rows = reinterpret_cast<const uint32_t*>(scratch + lay.rows) + off;
    const uint16_t* xh = reinterpret_cast<const uint16_t*>(scratch + lay.xh);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane >> 4;  // block pair of the window this lane loads
    const int nb = K / 32;    // blocks per row (even)
    const size_t row_bytes = (size_t)nb * 18;
    const uint8_t* wexp = w + (size_t)e * expert_stride;

    for (uint32_t m0 = 0; m0 < cnt; m0 += kMoeMT * 16) {
        const int mt = min(kMoeMT, (int)((cnt - m0 + 15) / 16));
        f32x4 acc[kMoeMT][kMoeNS];
#pragma unroll
        for (int i = 0; i < kMoeMT; ++i)
#pragma unroll
            for (int j = 0; j < kMoeNS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int k0 = 0; k0 < K; k0 += kMoeWin) {
            // Stage x rows m0 .. m0 + 16 mt - 1 of this expert, window k0.
            const int pieces = mt * 16 * (kMoeWin / 8);
            for (int p = tid; p < pieces; p += kMoeThreads) {
                const int rr = p / (kMoeWin / 8), kk = (p % (kMoeWin / 8)) * 8;
                u32x4 v = u32x4{0u, 0u, 0u, 0u};
                if (m0 + rr < cnt && k0 + kk < K) {
                    const uint32_t t = rows[m0 + rr] / (uint32_t)top_k;
                    v = *reinterpret_cast<const u32x4*>(xh + (size_t)t * K + k0 + kk);
                }
                *reinterpret_cast<u32x4*>(xs + rr * kMoeXLd + kk) = v;
            }
            // Raw weights: lane (n = lane%16, c) loads block pair c of the window
            // (36 bytes, 4-byte aligned) for each of its sub-tiles.
            uint32_t raw[kMoeNS][9];
            const int pair = k0 / 64 + c;
#pragma unroll
            for (int s = 0; s < kMoeNS; ++s) {
                const int n = nt * kMoeBN + wave * (16 * kMoeNS) + s * 16 + (lane & 15);
                if (n < N && pair < nb / 2) {
                    const uint32_t* src = reinterpret_cast<const uint32_t*>(wexp + (size_t)n * row_bytes + (size_t)pair * 36);
#pragma unroll
                    for (int j = 0; j < 9; ++j) raw[s][j] = src[j];
                } else {
#pragma unroll
                    for (int j = 0; j < 9; ++j) raw[s][j] = 0u;
                }
            }
            __syncthreads();
#pragma unroll
            for (int s = 0; s < kMoeNS; ++s) {
                uint32_t dA, dB, qsA[4], qsB[4];
                q4_0_split_pair(raw[s], dA, dB, qsA, qsB);
#pragma unroll
                for (int f = 0; f < 8; ++f) {
                    const int blk = 2 * c + (f >> 2);  // block within the window
                    const int i = f & 3;               // qs dword within the block
                    const uint32_t q = (f < 4) ? qsA[i] : qsB[i];
                    const uint32_t d = (f < 4) ? dA : dB;
                    const u32x4 b = q4_0_fragment(q, d | (d << 16));
                    const int kx = blk * 32 + 4 * i;
#pragma unroll
                    for (int m = 0; m < kMoeMT; ++m) {
                        if (m < mt) {
                            const uint16_t* xr = xs + (m * 16 + (lane & 15)) * kMoeXLd;
                            const u32x2 lo = *reinterpret_cast<const u32x2*>(xr + kx);
                            const u32x2 hi = *reinterpret_cast<const u32x2*>(xr + kx + 16);
                            const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
                            acc[m][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc[m][s], 0, 0, 0);
                        }
                    }
                }
            }
            __syncthreads();
        }
        // Scatter: fragment lane holds routed rows 4*(lane/16)+r, weight row lane%16.
#pragma unroll
        for (int m = 0; m < kMoeMT; ++m) {
            if (m >= mt) continue;
#pragma unroll
            for (int s = 0; s < kMoeNS; ++s) {
                const int n = nt * kMoeBN + wave * (16 * kMoeNS) + s * 16 + (lane & 15);
                if (n >= N) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t idx = m0 + m * 16 + 4 * (lane >> 4) + r;
                    if (idx < cnt) out[(size_t)rows[idx] * N + n] = acc[m][s][r];
                }
            }
        }
    }
}

}  // namespace w4mi

using namespace w4mi;

extern "C" w4_status qmm_id_q4_0(const float* x, const uint8_t* w, const uint32_t* ids, float* out,
                                 const w4_id_params* p, void* scratch, size_t scratch_bytes, void* stream) {
    w4_status st = w4_check_id(p, scratch_bytes);
    if (st != W4_OK) return st;
    if (!x || !w || !ids || !out || !scratch) return fail(W4_EINVAL, "qmm_id_q4_0: null pointer argument");
    if (p->k % 64 != 0)
        return fail(W4_EUNSUPPORTED, "qmm_id_q4_0: implemented for K %% 64 == 0 (whole 36-byte block pairs), got %u",
                    p->k);
    if (((uintptr_t)w & 3u) || (p->expert_stride & 3u) || ((uintptr_t)x & 15u) || ((uintptr_t)scratch & 255u))
        return fail(W4_EINVAL, "qmm_id_q4_0: w and expert_stride must be 4-byte, x 16-byte, scratch 256-byte aligned");
    const IdScratchLayout lay = id_scratch_layout(p->n_experts, p->n_tokens, p->top_k, p->k);
    const int n_rows = (int)(p->n_tokens * p->top_k);
    const int64_t x_count = (int64_t)p->n_tokens * p->k;
    hipStream_t s = as_stream(stream);
    const int conv_blocks = (int)std::min<int64_t>(1024, (x_count / 8 + kGroupThreads - 1) / kGroupThreads);
    hipLaunchKernelGGL(moe_group_kernel, dim3(1 + conv_blocks), dim3(kGroupThreads), p->n_experts * sizeof(uint32_t), s,
                       ids, x, (uint8_t*)scratch, out, n_rows, (int)p->n_experts, (int)p->n, x_count, lay);
    st = launch_status("qmm_id_q4_0 (group)");
    if (st != W4_OK) return st;
    const int tiles_n = (int)((p->n + kMoeBN - 1) / kMoeBN);
    hipLaunchKernelGGL(moe_gemm_kernel, dim3((unsigned)(p->n_experts * tiles_n)), dim3(kMoeThreads), 0, s, w,
                       (const uint8_t*)scratch, out, (int)p->n, (int)p->k, (int)p->top_k, p->expert_stride, lay);
    return launch_status("qmm_id_q4_0 (grouped GEMM)");
}
