// qmm_id_q4_0: expert-routed matmul over GGML Q4_0 blocks (mlx-native MoE
// page): out[t*top_k + s][n] = sum_k (q - 8) d of expert ids[t*top_k + s],
// row n, times x[t][k].
//
// Two launches on the caller's stream, as the page's map0 + mm pair:
//  1. moe_group_kernel: workgroup 0 counts the routed rows per expert, scans
//     the counts and scatters row indices into per-expert lists (the page's
//     htpe / hids); the other workgroups store x as binary16 (the matrix-core
//     operand type), each 32-wide K block in the order the weight decode
//     produces it. Stream order makes both visible to launch 2.
//  2. moe_gemm_kernel: one workgroup per (expert, 128 weight rows) reads that
//     slice of the expert's weights exactly once per 32 routed rows and
//     applies it with v_mfma_f32_32x32x16_f16, f32 accumulation. Weights and
//     the routed rows' x stream through LDS rings by buffer-to-LDS DMA, one
//     256-wide K window (8 Q4_0 blocks, 144 bytes of each weight row) per
//     step; each lane decodes two qs dwords per block into fp16 (q - 8) d.
#include <type_traits>

#include "w4mi_device.hpp"
#include "w4mi_host.hpp"

namespace w4mi {

constexpr int kGroupThreads = 1024;

__global__ __launch_bounds__(kGroupThreads) void moe_group_kernel(const uint32_t* __restrict__ ids, const float* __restrict__ x,
                                                                  uint8_t* __restrict__ scratch, float* __restrict__ out,
                                                                  int n_rows, int n_experts, int N, int64_t x_count,
                                                                  IdScratchLayout lay) {
    if (blockIdx.x > 0) {
        // x -> binary16, 8 values per thread per step: output positions
        // 8c .. 8c + 7 of a 32-wide block hold k = 4c .. 4c + 3 and
        // 16 + 4c .. 16 + 4c + 3 (the order q4_0_operand yields weights in).
        uint16_t* xh = reinterpret_cast<uint16_t*>(scratch + lay.xh);
        const int64_t stride = (int64_t)(gridDim.x - 1) * kGroupThreads * 8;
        for (int64_t i = ((int64_t)(blockIdx.x - 1) * kGroupThreads + threadIdx.x) * 8; i < x_count; i += stride) {
            const int64_t blk = i & ~(int64_t)31;
            const int c = (int)((i & 31) >> 3);
            const f32x4 a = *reinterpret_cast<const f32x4*>(x + blk + 4 * c);
            const f32x4 b = *reinterpret_cast<const f32x4*>(x + blk + 16 + 4 * c);
            *reinterpret_cast<u32x4*>(xh + i) = u32x4{pack_f16x2(a[0], a[1]), pack_f16x2(a[2], a[3]),
                                                      pack_f16x2(b[0], b[1]), pack_f16x2(b[2], b[3])};
        }
        return;
    }
    extern __shared__ uint32_t cnt[];  // [n_experts], counts then cursors
    __shared__ uint32_t part[kGroupThreads / 64];
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
    // Exclusive scan: each thread sums a contiguous segment of experts; the
    // segment sums are scanned within each wavefront (lane shifts, no
    // barrier), then across the 16 wavefront totals.
    const int seg = (n_experts + kGroupThreads - 1) / kGroupThreads;
    const int e0 = tid * seg, e1 = min(n_experts, e0 + seg);
    const int lane = tid & 63, wave = tid >> 6;
    uint32_t local = 0u;
    for (int e = e0; e < e1; ++e) local += cnt[e];
    uint32_t incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    if (lane == 63) part[wave] = incl;
    __syncthreads();
    uint32_t base = 0u;
    for (int w = 0; w < wave; ++w) base += part[w];
    uint32_t run = base + incl - local;  // exclusive prefix of this segment
    for (int e = e0; e < e1; ++e) {
        const uint32_t c = cnt[e];
        counts[e] = c;
        offsets[e] = run;
        cnt[e] = run;  // becomes the scatter cursor
        run += c;
    }
    if (tid == kGroupThreads - 1) offsets[n_experts] = base + incl;
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

constexpr int kMoeWaves = 16;          // 2 halves of 64 weight rows x 8 blocks of a window
constexpr int kMoeThreads = kMoeWaves * 64;
constexpr int kMoeKSplit = 8;          // wavefronts per 64 weight rows, one block of each window each
constexpr int kMoeBN = 128;            // weight rows per workgroup: 4 x 32
constexpr int kMoeMR = 32;             // routed rows per pass (one 32x32 MFMA tile)
constexpr int kMoeWinBlocks = 8;       // Q4_0 blocks per K window
constexpr int kMoeWRow = kMoeWinBlocks * 18;            // 144 bytes of a weight row per window
constexpr int kMoeWSlot = kMoeBN * kMoeWRow;            // 18 KB
constexpr int kMoeWDma = kMoeWSlot / 1024;              // 18 DMA instructions per W window
constexpr int kMoeXRow = kMoeWinBlocks * 32 * 2;        // 512 bytes of a routed row's x per window
constexpr int kMoeXSlot = kMoeMR * kMoeXRow;            // 16 KB
constexpr int kMoeXDma = kMoeXSlot / 1024;              // 16 DMA instructions per x window
constexpr int kMoeWStages = 4, kMoeXStages = 3;
constexpr uint32_t kMoeOob = 0x80000000u;

__device__ __forceinline__ uint32_t moe_lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Buffer-to-LDS DMA of 16 bytes per lane (lane l -> lds + 16 l). Inline asm
// so the compiler does not wait for every DMA before each LDS access; the
// issuing wavefront waits for its own DMA explicitly (moe_wait_vmcnt) before
// the barrier that publishes it.
__device__ __forceinline__ void moe_dma16(const __amdgpu_buffer_rsrc_t& rsrc, void* lds, uint32_t voff, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 ::"s"(moe_lds_addr(lds)), "v"(voff), "s"(rsrc), "s"(soff));
}
template <int N>
__device__ __forceinline__ void moe_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void moe_barrier() { asm volatile("s_barrier" ::: "memory"); }
// A scalar-cache load of one dword at a wave-uniform address. It is counted by
// lgkmcnt, so waiting for it does not wait for the DMA in flight.
// The address is passed through readfirstlane so that it is in scalar
// registers even where the compiler cannot prove it uniform.
__device__ __forceinline__ uint32_t moe_sload(const uint32_t* p) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    // readfirstlane returns int: widen through uint32_t, or the low word would sign-extend.
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint64_t sa = ((uint64_t)hi << 32) | (uint64_t)lo;
    uint32_t v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(sa) : "memory");
    return v;
}

// One lane's B operand for one Q4_0 block: qs dword c (elements 4c .. 4c + 3
// in the low nibbles, 16 + 4c .. 16 + 4c + 3 in the high ones) as fp16
// (q - 8) d, in the order (4c, 4c+1) (4c+2, 4c+3) (16+4c, 16+4c+1)
// (16+4c+2, 16+4c+3). Low nibbles become binary16 1024 + q and high ones
// 64 + q (the nibble in mantissa bits 4..7 under exponent 2^6); subtracting
// 1032 or 72 is exact and leaves q - 8, and the product with d rounds once.
struct Q4Consts {
    uint32_t m_lo, m_hi, magic_lo, magic_hi;  // held in VGPRs so each mask-and-insert is one v_and_or_b32
};
__device__ __forceinline__ u32x4 q4_0_operand(uint32_t qs, f16x2 dd, const Q4Consts& k) {
    const uint32_t t0 = __builtin_amdgcn_perm(0u, qs, 0x0C010C00u);  // [b0, 0, b1, 0]
    const uint32_t t1 = __builtin_amdgcn_perm(0u, qs, 0x0C030C02u);  // [b2, 0, b3, 0]
    const f16x2 lo_bias = as_f16x2(0xE408E408u), hi_bias = as_f16x2(0xD480D480u);  // -1032, -72
    u32x4 o;
    o[0] = as_u32((as_f16x2(and_or_u32(t0, k.m_lo, k.magic_lo)) + lo_bias) * dd);
    o[1] = as_u32((as_f16x2(and_or_u32(t1, k.m_lo, k.magic_lo)) + lo_bias) * dd);
    o[2] = as_u32((as_f16x2(and_or_u32(t0, k.m_hi, k.magic_hi)) + hi_bias) * dd);
    o[3] = as_u32((as_f16x2(and_or_u32(t1, k.m_hi, k.magic_hi)) + hi_bias) * dd);
    return o;
}

// Block b of one K window (ODD = b % 2) for a wavefront's 64 weight rows
// (two 32-row tiles) against the 32 routed rows. Lane (n, h) = (lane % 32,
// lane / 32) feeds MFMA k-step s with qs dword 2 s + h of row n of each tile;
// the x operand of lane (m, h) is the same eight elements of routed row m,
// which the xh order stores as 16 contiguous bytes (chunk 4 b + 2 s + h of
// the window row, kept at slot chunk ^ (m % 32)); one x read serves both
// tiles. A block past the row's end (a partial last window) gets d = 0, which
// zeroes its weights whatever the ring holds there.
template <int ODD>
__device__ __forceinline__ void moe_block(const uint8_t* wrows, const uint8_t* xs, int lane, int b, bool live,
                                          const Q4Consts& k, f32x16 (&acc)[2]) {
    const int h = lane >> 5, m = lane & 31;
    const uint8_t* xr = xs + m * kMoeXRow;
    uint32_t dd[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const uint32_t draw = *reinterpret_cast<const uint16_t*>(wrows + t * 32 * kMoeWRow + 18 * b);
        dd[t] = (live ? draw : 0u) * 0x10001u;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const u32x4 xop = *reinterpret_cast<const u32x4*>(xr + 16 * ((4 * b + 2 * s + h) ^ m));
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint8_t* blk = wrows + t * 32 * kMoeWRow + 18 * b;
            // qs dword 2 s + h: 4-byte aligned for odd b, else two bytes past
            // an aligned dword.
            uint32_t qs;
            if (ODD) {
                qs = *reinterpret_cast<const uint32_t*>(blk + 2 + 8 * s + 4 * h);
            } else {
                const uint32_t lo = *reinterpret_cast<const uint32_t*>(blk + 8 * s + 4 * h);
                const uint32_t hi = *reinterpret_cast<const uint32_t*>(blk + 8 * s + 4 * h + 4);
                qs = __builtin_amdgcn_alignbyte(hi, lo, 2);
            }
            const u32x4 wop = q4_0_operand(qs, as_f16x2(dd[t]), k);
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, xop), __builtin_bit_cast(f16x8, wop),
                                                            acc[t], 0, 0, 0);
        }
    }
}

// LDS (one array, so that the end-of-pass exchange can use all of it):
//   W  kMoeWStages x [128 rows x 144 B]: the window's 8 blocks of each row,
//      as stored (d then qs, 18 bytes a block);
//   x  kMoeXStages x [32 rows x 512 B]: routed row r's 16-byte chunk p
//      (xh order) at chunk slot p ^ (r % 32), which keeps the A-operand
//      reads of 32 rows conflict-free.
// Each of the 16 wavefronts issues its share of every window's DMA (W
// kMoeWStages - 1 windows ahead, x kMoeXStages - 1 ahead) and waits for its
// own DMA of window j before barrier j, after which every wavefront may read
// window j and the slots of window j - 1 are free. Wavefront w takes weight
// rows 64 (w % 2) .. + 63 and block w / 2 of each window (so each wavefront
// runs at least 4 to a SIMD, as the decode's vector-ALU work needs); the eight
// partial sums of a row half meet in LDS at the end of a pass.
constexpr int kMoeLds = kMoeWStages * kMoeWSlot + kMoeXStages * kMoeXSlot;

__global__ __launch_bounds__(kMoeThreads) void moe_gemm_kernel(const uint8_t* __restrict__ w, const uint8_t* __restrict__ scratch,
                                                               float* __restrict__ out, int N, int K, int top_k,
                                                               uint64_t expert_stride, IdScratchLayout lay, int n_tokens) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kMoeLds];
    uint8_t* const wring = lds;
    uint8_t* const xring = lds + kMoeWStages * kMoeWSlot;
    const int tiles_n = (N + kMoeBN - 1) / kMoeBN;
    const int e = blockIdx.x / tiles_n;
    const int n0 = (blockIdx.x % tiles_n) * kMoeBN;
    const uint32_t cnt = reinterpret_cast<const uint32_t*>(scratch + lay.counts)[e];
    if (cnt == 0u) return;
    const uint32_t* rows =
        reinterpret_cast<const uint32_t*>(scratch + lay.rows) + reinterpret_cast<const uint32_t*>(scratch + lay.offsets)[e];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = K / 32;
    const int nwin = (nb + kMoeWinBlocks - 1) / kMoeWinBlocks;
    const uint32_t row_bytes = (uint32_t)nb * 18u;
    const int nrows = min(kMoeBN, N - n0);
    const __amdgpu_buffer_rsrc_t wsrc =
        make_rsrc(w + (size_t)e * expert_stride + (size_t)n0 * row_bytes, (uint32_t)nrows * row_bytes);
    const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(scratch + lay.xh, (uint32_t)((size_t)n_tokens * (size_t)K * 2u));
    const Q4Consts k{vreg(0x000F000Fu), vreg(0x00F000F0u), vreg(0x64006400u), vreg(0x54005400u)};
    float* const red = reinterpret_cast<float*>(lds);  // pass-end exchange
    static_assert((kMoeKSplit - 1) * 2 * 2 * 16 * 64 * 4 <= kMoeLds, "exchange area fits the rings");

    // DMA plan: W instruction i (lane l covers 16-byte chunk q = 64 i + l of
    // the window: row q / 9, chunk q % 9) goes to wavefront i % 16, x
    // instruction i (routed rows 2 i, 2 i + 1) to wavefront i.
    static_assert(kMoeXDma == kMoeWaves, "one x DMA instruction per wavefront");
    constexpr int kWPer = (kMoeWDma + kMoeWaves - 1) / kMoeWaves;
    const int nw_dma = wave < kMoeWDma % kMoeWaves ? kWPer : kMoeWDma / kMoeWaves;
    uint32_t wo[kWPer];
#pragma unroll
    for (int t = 0; t < kWPer; ++t) {
        const int q = 64 * (wave + kMoeWaves * t) + lane, r = q / 9, j = q % 9;
        wo[t] = r < nrows ? (uint32_t)r * row_bytes + 16u * (uint32_t)j : kMoeOob;
    }
    const int rh = wave & 1, b = wave >> 1;
    const int nl = 64 * rh + (lane & 31);  // this lane's weight row in tile 0 (tile 1: + 32)

    for (uint32_t m0 = 0; m0 < cnt; m0 += kMoeMR) {
        // Routed rows past cnt are not loaded: their (stale) x only feeds
        // output rows that are never stored.
        const bool x_rows = m0 + 2u * (uint32_t)wave < cnt;
        // Iteration j issues W(j + 3) and x(j + 2); the prologue runs the
        // issues of iterations -3 .. -1 (x(-1) is all zeros, so every
        // iteration of a wavefront issues the same count).
        auto issue_w = [&](int j) {
            const int win = j + kMoeWStages - 1;
            const bool live = win < nwin;
            uint8_t* slot = wring + (win % kMoeWStages) * kMoeWSlot;
            const int soff = __builtin_amdgcn_readfirstlane(live ? win * kMoeWRow : 0);
#pragma unroll
            for (int t = 0; t < kWPer; ++t)
                if (t < nw_dma) moe_dma16(wsrc, slot + 1024 * (wave + kMoeWaves * t), live ? wo[t] : kMoeOob, soff);
        };
        // W(0), W(1) need no row ids, so they go out first.
        issue_w(-3);
        issue_w(-2);
        // This wavefront's x rows 2 wave, 2 wave + 1: their ids come by scalar
        // loads, which do not wait behind the DMA in flight.
        uint32_t xo;
        {
            const uint32_t r0 = __builtin_amdgcn_readfirstlane(min(m0 + 2u * (uint32_t)wave, cnt - 1u));
            const uint32_t r1 = __builtin_amdgcn_readfirstlane(min(r0 + 1u, cnt - 1u));
            const uint32_t id0 = moe_sload(rows + r0), id1 = moe_sload(rows + r1);
            const uint32_t rid = (lane >> 5) ? id1 : id0;
            const uint32_t r = m0 + 2 * wave + (lane >> 5);
            const int p = (lane & 31) ^ (2 * wave + (lane >> 5));
            xo = r < cnt ? (rid / (uint32_t)top_k) * (uint32_t)K * 2u + 16u * (uint32_t)p : kMoeOob;
        }
        auto issue_x = [&](int j) {
            if (x_rows) {
                const int win = j + kMoeXStages - 1;
                const bool live = win >= 0 && win < nwin;
                uint8_t* slot = xring + ((win + kMoeXStages) % kMoeXStages) * kMoeXSlot;
                const int soff = __builtin_amdgcn_readfirstlane(live ? win * kMoeXRow : 0);
                moe_dma16(xsrc, slot + 1024 * wave, live ? xo : kMoeOob, soff);
            }
        };
        auto issue = [&](int j) {
            issue_w(j);
            issue_x(j);
        };
        static_assert(kMoeWStages - 1 == 3 && kMoeXStages - 1 == 2, "prologue below assumes 3 and 2 windows ahead");
        // Order W(0) W(1) x(-1) x(0) W(2) x(1): at window 0 only the last
        // iteration's issue (W(2), x(1)) may still be in flight.
        issue_x(-3);
        issue_x(-2);
        issue(-1);
        f32x16 acc[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[0][i] = acc[1][i] = 0.f;
        // The window loop is specialised on the block parity once per pass
        // (a branch per window would make the compiler copy the accumulators).
        auto windows = [&](auto odd) {
            for (int win = 0; win < nwin; ++win) {
                // Everything but the last iteration's issue has landed: W(win), x(win).
                if (nw_dma == kWPer) {
                    if (x_rows)
                        moe_wait_vmcnt<kWPer + 1>();
                    else
                        moe_wait_vmcnt<kWPer>();
                } else {
                    if (x_rows)
                        moe_wait_vmcnt<kMoeWDma / kMoeWaves + 1>();
                    else
                        moe_wait_vmcnt<kMoeWDma / kMoeWaves>();
                }
                moe_barrier();
                moe_block<decltype(odd)::value>(wring + (win % kMoeWStages) * kMoeWSlot + nl * kMoeWRow,
                                                xring + (win % kMoeXStages) * kMoeXSlot, lane, b,
                                                b < nb - kMoeWinBlocks * win, k, acc);
                // After the window's matrix work, so that the 16 wavefronts' DMA
                // issues (which queue behind one another in the memory pipe) do
                // not all stall the compute at the start of the window.
                issue(win);
            }
        };
        if (b & 1)
            windows(std::integral_constant<int, 1>{});
        else
            windows(std::integral_constant<int, 0>{});
        moe_wait_vmcnt<0>();  // the trailing (all-zero) DMA has landed
        moe_barrier();        // every wavefront is done with the rings
        // Blocks 1 .. 7 hand their sums to block 0.
        if (b) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) red[((((b - 1) * 2 + rh) * 2 + t) * 16 + i) * 64 + lane] = acc[t][i];
        }
        moe_barrier();
        if (!b) {
            // Lane (n, h) of tile t holds routed rows 8 (i / 4) + 4 h + i % 4 of weight row n.
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ncol = n0 + nl + 32 * t;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const uint32_t idx = m0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                    float v = acc[t][i];
#pragma unroll
                    for (int q = 0; q < kMoeKSplit - 1; ++q) v += red[(((q * 2 + rh) * 2 + t) * 16 + i) * 64 + lane];
                    if (idx < cnt && ncol < N) out[(size_t)rows[idx] * N + ncol] = v;
                }
            }
        }
        moe_barrier();  // the exchange area is free again
    }
}


// ---------------------------------------------------------------- mat-vec route
// Below the page's routing threshold (n_tokens <= 32) a call is a set of
// mat-vecs, one per routed row (the page's mv_id dispatch): each weight row
// slice is applied to a handful of x rows, so the work is bound by reading
// the selected experts' weights once and the matrix cores would idle. One
// launch, no grouping pass and no scratch traffic:
//  - workgroup (tile, r) covers weight rows tile*32 .. +31 of expert ids[r].
//    If an earlier routed row has the same id it exits at once; otherwise it
//    serves every routed row with that id, so each selected expert's weights
//    are read once, and kept in registers across those rows.
//  - a wavefront owns 4 weight rows, 16 lanes each; lane j of a row takes
//    blocks 4j .. 4j+3 of each 64-block chunk, i.e. 72 contiguous bytes at a
//    4-byte-aligned offset (four 16-byte and one 8-byte load; consecutive
//    lanes read consecutive bytes of the row).
//  - x of the routed row's token is rounded to binary16 (as in the grouped
//    GEMM route) and laid out in LDS as the pairs q4_0_dot_pairs pairs
//    weights into, with each block's bias sum 1032 sum(lo) + 72 sum(hi);
//    sum_k x (q - 8) of a block is then 16 v_dot2_f32_f16 minus that sum.
constexpr int kMvWaves = 4;                    // wavefronts per workgroup
constexpr int kMvRows = 4;                     // weight rows per wavefront
constexpr int kMvTile = kMvWaves * kMvRows;    // weight rows per workgroup
constexpr int kMvChunk = 64;                   // Q4_0 blocks per chunk: 16 lanes x 4
constexpr int kMvMaxChunks = 4;                // K <= 8192 on this route
constexpr int kMvStride = 20;                  // LDS dwords per block: 16 pairs, bias sum, pad (80 B)
constexpr int kMvIdSlots = 4;                  // routed rows scanned per lane: n_tokens * top_k <= 256
constexpr uint32_t kMvMaxTokens = 32;          // the page's mv / mm routing threshold

// LDS slot of block b: within a chunk, lanes j = 0..15 reading block 4j + i
// hit 16 consecutive 80-byte records (conflict-free 16-byte reads).
__device__ __forceinline__ int mv_slot(int b) { return (b & ~(kMvChunk - 1)) + (b & 3) * 16 + ((b & (kMvChunk - 1)) >> 2); }

// SWIGLU: the fused form of the same page (quantized_matmul_id_swiglu_q4_0):
// the activation of routed row r is silu(gate[r]) * up[r] (x = gate, per
// routed row, not per token), formed in f32 when x is published.
template <int T, bool REALIGN, bool SWIGLU>
__global__ __launch_bounds__(kMvWaves * 64) void moe_mv_kernel(const float* __restrict__ x, const float* __restrict__ up,
                                                               const uint8_t* __restrict__ w,
                                                               const uint32_t* __restrict__ ids, float* __restrict__ out,
                                                               uint32_t* __restrict__ bad_ids, int N, int K, int top_k,
                                                               int n_rows, int n_experts, uint64_t expert_stride) {
    constexpr int kThreads = kMvWaves * 64;
    constexpr int kPieces = T * kMvChunk * 4;  // (block, quarter) pieces of x
    constexpr int kPer = (kPieces + kThreads - 1) / kThreads;
    __shared__ __attribute__((aligned(16))) uint32_t xp[T * kMvChunk * kMvStride];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = blockIdx.y;
    const int n0 = blockIdx.x * kMvTile;
    const int nb = K / 32;
    const uint32_t row_bytes = (uint32_t)nb * 18u;

    // The routed-row ids, all of them (n_rows <= 64 kMvIdSlots), one vector
    // load per slot, together with this workgroup's own id.
    const __amdgpu_buffer_rsrc_t isrc = make_rsrc(ids, (uint32_t)n_rows * 4u);
    uint32_t idv[kMvIdSlots];
#pragma unroll
    for (int q = 0; q < kMvIdSlots; ++q) idv[q] = __builtin_amdgcn_raw_buffer_load_b32(isrc, (uint32_t)(64 * q + lane) * 4u, 0, 0);
    const uint32_t e = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_raw_buffer_load_b32(isrc, (uint32_t)r * 4u, 0, 0));
    uint64_t match[kMvIdSlots];
    bool dup = false;
    uint32_t bad = 0;
#pragma unroll
    for (int q = 0; q < kMvIdSlots; ++q) {
        const int i = 64 * q + lane;
        dup |= __ballot(i < r && idv[q] == e) != 0;
        match[q] = __ballot(i >= r && i < n_rows && idv[q] == e);
        bad += __builtin_popcountll(__ballot(i < n_rows && idv[q] >= (uint32_t)n_experts));
    }
    if (bad_ids != nullptr && r == 0 && blockIdx.x == 0 && tid == 0) *bad_ids = bad;
    if (dup) return;  // an earlier routed row with this id serves it (uniform over the workgroup)

    const int lr = kMvRows * wave + (lane >> 4);  // this lane's weight row within the tile
    const int j = lane & 15;
    const int n = n0 + lr;
    if (e >= (uint32_t)n_experts) {
        // Out-of-range id: its rows are written as zeros.
#pragma unroll
        for (int q = 0; q < kMvIdSlots; ++q)
            for (uint64_t m = match[q]; m; m &= m - 1) {
                const int r2 = 64 * q + (int)__builtin_ctzll(m);
                if (j == 0 && n < N) out[(size_t)r2 * N + n] = 0.f;
            }
        return;
    }

    // x of the first routed row goes out first, then the weights.
    constexpr int kSrc = SWIGLU ? 2 : 1;  // gate and up, or x
    auto load_x = [&](int r2, f32x4 (&lo)[kSrc][kPer], f32x4 (&hi)[kSrc][kPer]) {
        const size_t row = SWIGLU ? (size_t)r2 : (size_t)(r2 / top_k);
#pragma unroll
        for (int v = 0; v < kSrc; ++v) {
            const __amdgpu_buffer_rsrc_t xsrc = make_rsrc((v ? up : x) + row * K, (uint32_t)K * 4u);
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int p = tid + i * kThreads, b = p >> 2, c = p & 3;
                // Pieces past the last block read past the row: zeros.
                const uint32_t off = b < nb ? (uint32_t)(32 * b + 4 * c) * 4u : 0x80000000u;
                lo[v][i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xsrc, off, 0, 0));
                hi[v][i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xsrc, off + 64u, 0, 0));
            }
        }
    };
    // silu(g) u = g u / (1 + e^-g); for g -> -inf the reciprocal of inf is 0.
    auto swiglu = [](f32x4 g, f32x4 u) {
        f32x4 a;
#pragma unroll
        for (int t = 0; t < 4; ++t) a[t] = g[t] * u[t] * __builtin_amdgcn_rcpf(1.f + __expf(-g[t]));
        return a;
    };
    auto publish_x = [&](const f32x4 (&src_lo)[kSrc][kPer], const f32x4 (&src_hi)[kSrc][kPer]) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int p = tid + i * kThreads, b = p >> 2, c = p & 3;
            f32x4 lo[1], hi[1];
            if constexpr (SWIGLU) {
                lo[0] = swiglu(src_lo[0][i], src_lo[1][i]);
                hi[0] = swiglu(src_hi[0][i], src_hi[1][i]);
            } else {
                lo[0] = src_lo[0][i];
                hi[0] = src_hi[0][i];
            }
            f16x2 l02, h02, l13, h13;
            l02[0] = (_Float16)lo[0][0]; l02[1] = (_Float16)lo[0][2];
            h02[0] = (_Float16)hi[0][0]; h02[1] = (_Float16)hi[0][2];
            l13[0] = (_Float16)lo[0][1]; l13[1] = (_Float16)lo[0][3];
            h13[0] = (_Float16)hi[0][1]; h13[1] = (_Float16)hi[0][3];
            float bs = 0.f;
            bs = __builtin_amdgcn_fdot2(l02, f16x2{(_Float16)kQ4DotBiasLo, (_Float16)kQ4DotBiasLo}, bs, false);
            bs = __builtin_amdgcn_fdot2(l13, f16x2{(_Float16)kQ4DotBiasLo, (_Float16)kQ4DotBiasLo}, bs, false);
            bs = __builtin_amdgcn_fdot2(h02, f16x2{(_Float16)kQ4DotBiasHi, (_Float16)kQ4DotBiasHi}, bs, false);
            bs = __builtin_amdgcn_fdot2(h13, f16x2{(_Float16)kQ4DotBiasHi, (_Float16)kQ4DotBiasHi}, bs, false);
            // The block's four quarters sit in four adjacent lanes.
            bs += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(bs), 0xB1, 0xF, 0xF, false));
            bs += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(bs), 0x4E, 0xF, 0xF, false));
            if (p < kPieces) {
                uint32_t* d = xp + mv_slot(b) * kMvStride;
                *reinterpret_cast<u32x4*>(d + 4 * c) = u32x4{as_u32(l02), as_u32(h02), as_u32(l13), as_u32(h13)};
                if (c == 0) d[16] = __float_as_uint(bs);
            }
        }
    };
    f32x4 xlo[kSrc][kPer], xhi[kSrc][kPer];
    load_x(r, xlo, xhi);
    __builtin_amdgcn_sched_barrier(0);  // keep the x loads ahead of the weights (the wait counter is in order)
    const int rows_here = min(kMvTile, N - n0);
    // The tile's bytes start at a 2-byte boundary; the descriptor starts at the
    // dword below it (dword accesses ignore the low two address bits) and
    // every lane offset carries the difference. Its length is rounded up to
    // whole dwords: the range check drops any dword not wholly inside it, and
    // a dword holding the tile's last bytes lies in the same page as they do.
    const uint8_t* tile = w + (uint64_t)e * expert_stride + (uint64_t)n0 * row_bytes;
    const uint32_t delta = (uint32_t)((uintptr_t)tile & 3u);
    const __amdgpu_buffer_rsrc_t wsrc = make_rsrc(tile - delta, ((uint32_t)rows_here * row_bytes + delta + 3u) & ~3u);
    uint32_t raw[T][18];
#pragma unroll
    for (int c = 0; c < T; ++c) {
        // Lanes whose blocks lie past the row read neighbouring bytes (or
        // zeros past the tile); their blocks are skipped below.
        const uint32_t off = delta + (uint32_t)lr * row_bytes + (uint32_t)(c * kMvChunk * 18 + 72 * j);
        if constexpr (!REALIGN) {
            // A 4-byte-aligned tile and an even block count keep every lane's span 4-byte aligned.
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wsrc, off + 16u * q, 0, 0);
#pragma unroll
                for (int t = 0; t < 4; ++t) raw[c][4 * q + t] = v[t];
            }
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wsrc, off + 64u, 0, 0);
            raw[c][16] = v[0];
            raw[c][17] = v[1];
        } else {
            // A span that starts 2 bytes past a dword boundary (odd block
            // count, or a tile so placed): load the 19 dwords around it and
            // shift them into place.
            const uint32_t base = off & ~3u, sh = off & 3u;
            uint32_t ld[19];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wsrc, base + 16u * q, 0, 0);
#pragma unroll
                for (int t = 0; t < 4; ++t) ld[4 * q + t] = v[t];
            }
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wsrc, base + 64u, 0, 0);
            ld[16] = v[0];
            ld[17] = v[1];
            ld[18] = __builtin_amdgcn_raw_buffer_load_b32(wsrc, base + 72u, 0, 0);
#pragma unroll
            for (int t = 0; t < 18; ++t) raw[c][t] = __builtin_amdgcn_alignbyte(ld[t + 1], ld[t], sh);
        }
    }
    const uint32_t m_lo = vreg(0x000F000Fu), m_hi = vreg(0x00F000F0u), mg_lo = vreg(0x64006400u), mg_hi = vreg(0x54005400u);

    // The routed rows this workgroup serves, in ascending order (the first is
    // r): wavefront 0 lists them in LDS, read after the first barrier.
    __shared__ int mlist[64 * kMvIdSlots];
    int count = 0;
#pragma unroll
    for (int q = 0; q < kMvIdSlots; ++q) {
        if (wave == 0 && ((match[q] >> lane) & 1u))
            mlist[count + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(match[q] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)match[q], 0u))] = 64 * q + lane;
        count += __builtin_popcountll(match[q]);
    }
    for (int k = 0; k < count; ++k) {
        int r2 = r;
        if (k > 0) {
            __syncthreads();  // every wavefront is done with the previous row's x
            r2 = __builtin_amdgcn_readfirstlane(mlist[k]);
            load_x(r2, xlo, xhi);
        }
        publish_x(xlo, xhi);
        __syncthreads();
        // Decode the weights afresh for each routed row: hoisted out of the
        // loop, the decoded pairs would take 16 registers per block.
#pragma unroll
        for (int c = 0; c < T; ++c)
#pragma unroll
            for (int t = 0; t < 18; ++t) asm volatile("" : "+v"(raw[c][t]));
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < T; ++c)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // Blocks 4j + 2h and 4j + 2h + 1: bytes 36 h .. 36 h + 35 of the lane's 72.
                uint32_t pr[9];
#pragma unroll
                for (int t = 0; t < 9; ++t) pr[t] = raw[c][9 * h + t];
                uint32_t dA, dB, qsA[4], qsB[4];
                q4_0_split_pair(pr, dA, dB, qsA, qsB);
#pragma unroll
                for (int ab = 0; ab < 2; ++ab) {
                    const int b = c * kMvChunk + 4 * j + 2 * h + ab;
                    const uint32_t* xs = xp + mv_slot(b) * kMvStride;
                    float dot = 0.f;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const u32x4 xv = *reinterpret_cast<const u32x4*>(xs + 4 * t);
                        uint32_t pw[4];
                        q4_0_dot_pairs(ab ? qsB[t] : qsA[t], m_lo, m_hi, mg_lo, mg_hi, pw);
#pragma unroll
                        for (int u = 0; u < 4; ++u) dot = __builtin_amdgcn_fdot2(as_f16x2(pw[u]), as_f16x2(xv[u]), dot, false);
                    }
                    const float v = f16_bits_to_f32(ab ? dB : dA) * (dot - __uint_as_float(xs[16]));
                    acc += b < nb ? v : 0.f;
                }
                // Bound the x pairs held in registers to two blocks' worth.
                asm volatile("" ::: "memory");
            }
        // Sum over the row's 16 lanes (one DPP row).
        acc += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(acc), 0x128, 0xF, 0xF, false));
        acc += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(acc), 0x124, 0xF, 0xF, false));
        acc += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(acc), 0x122, 0xF, 0xF, false));
        acc += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(acc), 0x121, 0xF, 0xF, false));
        if (j == 0 && n < N) out[(size_t)r2 * N + n] = acc;
    }
}

}  // namespace w4mi

using namespace w4mi;

namespace w4mi {

// One mat-vec launch over n_tokens * top_k routed rows (the caller checked
// n_routed <= 64 kMvIdSlots and K <= 32 kMvChunk kMvMaxChunks).
template <bool SWIGLU>
void mv_launch(const float* x, const float* up, const uint8_t* w, const uint32_t* ids, float* out, uint32_t* bad,
               const w4_id_params* p, hipStream_t s) {
    const uint32_t n_routed = p->n_tokens * p->top_k;
    const int chunks = (int)((p->k / 32 + kMvChunk - 1) / kMvChunk);
    const dim3 grid((unsigned)((p->n + kMvTile - 1) / kMvTile), n_routed), block(kMvWaves * 64);
    // Spans that may start off a dword boundary take the realigning form.
    const bool realign = ((p->k / 32) & 1u) || ((uintptr_t)w & 3u) || (p->expert_stride & 3u);
#define W4_MV_LAUNCH(T, RE)                                                                                      \
    hipLaunchKernelGGL((moe_mv_kernel<T, RE, SWIGLU>), grid, block, 0, s, x, up, w, ids, out, bad, (int)p->n,   \
                       (int)p->k, (int)p->top_k, (int)n_routed, (int)p->n_experts, p->expert_stride)
    switch (chunks * 2 + (realign ? 1 : 0)) {
        case 2: W4_MV_LAUNCH(1, false); break;
        case 3: W4_MV_LAUNCH(1, true); break;
        case 4: W4_MV_LAUNCH(2, false); break;
        case 5: W4_MV_LAUNCH(2, true); break;
        case 6: W4_MV_LAUNCH(3, false); break;
        case 7: W4_MV_LAUNCH(3, true); break;
        case 8: W4_MV_LAUNCH(4, false); break;
        default: W4_MV_LAUNCH(4, true); break;
    }
#undef W4_MV_LAUNCH
}

}  // namespace w4mi

extern "C" w4_status qmm_id_q4_0(const float* x, const uint8_t* w, const uint32_t* ids, float* out,
                                 const w4_id_params* p, void* scratch, size_t scratch_bytes, void* stream) {
    w4_status st = w4_check_id(p, scratch_bytes);
    if (st != W4_OK) return st;
    if (!x || !w || !ids || !out || !scratch) return fail(W4_EINVAL, "qmm_id_q4_0: null pointer argument");
    if (((uintptr_t)w & 1u) || (p->expert_stride & 1u) || ((uintptr_t)x & 15u) || ((uintptr_t)scratch & 255u))
        return fail(W4_EINVAL, "qmm_id_q4_0: w and expert_stride must be 2-byte, x 16-byte, scratch 256-byte aligned");
    const IdScratchLayout lay = id_scratch_layout(p->n_experts, p->n_tokens, p->top_k, p->k);
    hipStream_t s = as_stream(stream);
    const uint64_t n_routed = (uint64_t)p->n_tokens * p->top_k;
    const int chunks = (int)((p->k / 32 + kMvChunk - 1) / kMvChunk);
    if (p->n_tokens <= kMvMaxTokens && n_routed <= 64u * kMvIdSlots && chunks <= kMvMaxChunks) {
        // Mat-vec route (the page's mv_id below its routing threshold).
        uint32_t* bad = reinterpret_cast<uint32_t*>((uint8_t*)scratch + lay.bad_ids);
        mv_launch<false>(x, nullptr, w, ids, out, bad, p, s);
        return launch_status("qmm_id_q4_0 (mat-vec route)");
    }
    if (p->k % 64 != 0)
        return fail(W4_EUNSUPPORTED,
                    "qmm_id_q4_0: above 32 tokens, implemented for K %% 64 == 0 (whole 36-byte block pairs), got %u", p->k);
    if (((uintptr_t)w & 3u) || (p->expert_stride & 3u))
        return fail(W4_EUNSUPPORTED, "qmm_id_q4_0: above 32 tokens, implemented for 4-byte-aligned w and expert_stride");
    // Buffer descriptors cover the binary16 x copy and one 128-row weight slice in 32 bits.
    if ((uint64_t)p->n_tokens * p->k * 2u >= (1ull << 32) || 128ull * (p->k / 32) * 18u >= (1ull << 32))
        return fail(W4_EUNSUPPORTED, "qmm_id_q4_0: implemented for n_tokens * K * 2 < 2^32 bytes");
    const int n_rows = (int)(p->n_tokens * p->top_k);
    const int64_t x_count = (int64_t)p->n_tokens * p->k;
    const int conv_blocks = (int)std::min<int64_t>(1024, (x_count / 8 + kGroupThreads - 1) / kGroupThreads);
    hipLaunchKernelGGL(moe_group_kernel, dim3(1 + conv_blocks), dim3(kGroupThreads), p->n_experts * sizeof(uint32_t), s,
                       ids, x, (uint8_t*)scratch, out, n_rows, (int)p->n_experts, (int)p->n, x_count, lay);
    st = launch_status("qmm_id_q4_0 (group)");
    if (st != W4_OK) return st;
    const int tiles_n = (int)((p->n + kMoeBN - 1) / kMoeBN);
    hipLaunchKernelGGL(moe_gemm_kernel, dim3((unsigned)(p->n_experts * tiles_n)), dim3(kMoeThreads), 0, s, w,
                       (const uint8_t*)scratch, out, (int)p->n, (int)p->k, (int)p->top_k, p->expert_stride, lay,
                       (int)p->n_tokens);
    return launch_status("qmm_id_q4_0 (grouped GEMM)");
}

extern "C" w4_status qmm_id_swiglu_q4_0(const float* gate, const float* up, const uint8_t* w, const uint32_t* ids,
                                        float* out, const w4_id_params* p, uint32_t* bad_ids, void* stream) {
    w4_status st = w4_check_id_swiglu(p);
    if (st != W4_OK) return st;
    if (!gate || !up || !w || !ids || !out) return fail(W4_EINVAL, "qmm_id_swiglu_q4_0: null pointer argument");
    if (((uintptr_t)w & 1u) || (p->expert_stride & 1u) || ((uintptr_t)gate & 15u) || ((uintptr_t)up & 15u) ||
        ((uintptr_t)bad_ids & 3u))
        return fail(W4_EINVAL, "qmm_id_swiglu_q4_0: w and expert_stride must be 2-byte, gate and up 16-byte, bad_ids 4-byte aligned");
    const uint64_t n_routed = (uint64_t)p->n_tokens * p->top_k;
    const uint64_t chunks = (p->k / 32 + kMvChunk - 1) / kMvChunk;
    if (n_routed > 64u * kMvIdSlots || chunks > (uint64_t)kMvMaxChunks)
        return fail(W4_EUNSUPPORTED, "qmm_id_swiglu_q4_0: implemented for n_tokens * top_k <= %d and K <= %d",
                    64 * kMvIdSlots, 32 * kMvChunk * kMvMaxChunks);
    mv_launch<true>(gate, up, w, ids, out, bad_ids, p, as_stream(stream));
    return launch_status("qmm_id_swiglu_q4_0");
}
