// qmm_id_q4_0: expert-routed matmul over GGML Q4_0 blocks (mlx-native MoE
// page): out[t*top_k + s][n] = sum_k (q - 8) d of expert ids[t*top_k + s],
// row n, times x[t][k].
//
// Above the mat-vec threshold, up to 4096 routed rows take one launch
// (moe_fused_kernel, below the grouped GEMM); more take two launches on the
// caller's stream, as the page's map0 + mm pair:
//  1. moe_group_kernel: workgroup 0 counts the routed rows per expert, scans
//     the counts and scatters row indices into per-expert lists (the page's
//     htpe / hids); the other workgroups store x as binary16 (the matrix-core
//     operand type), each 32-wide K block in the order the weight decode
//     produces it. Stream order makes both visible to launch 2.
//  2. moe_gemm_kernel: workgroups split each expert's weight rows into
//     contiguous ranges of 32-row tiles (enough workgroups to fill the chip);
//     a range is read exactly once per 32 routed rows and applied with
//     v_mfma_f32_32x32x16_f16, f32 accumulation, one tile per wavefront.
//     Weights and the routed rows' x stream through a 3-slot LDS ring by
//     buffer-to-LDS DMA, one 128-wide K window (4 Q4_0 blocks, 72 bytes of
//     each weight row) per step; each lane decodes two blocks' qs dwords
//     into fp16 (q - 8) d. Rows that may start 2 bytes past a dword (an odd
//     block count, or w or the expert stride 2 mod 4) take a realigning
//     form of the same kernel.
#include <type_traits>

#include <atomic>

#include "w4mi_device.hpp"
#include "w4mi_host.hpp"

namespace w4mi {

constexpr int kGroupThreads = 1024;

__global__ __launch_bounds__(kGroupThreads) void moe_group_kernel(const uint32_t* __restrict__ ids, const float* __restrict__ x,
                                                                  uint8_t* __restrict__ scratch, float* __restrict__ out,
                                                                  int n_rows, int n_experts, int N, int64_t x_count,
                                                                  IdScratchLayout lay, uint32_t* __restrict__ events) {
    if (blockIdx.x > 0) {
        // A finite x beyond binary16's range becomes an infinity: each
        // wavefront that meets one counts one range event.
        bool oor = false;
        // x -> binary16, 8 values per thread per step: output positions
        // 8c .. 8c + 7 of a 32-wide block hold k = 4c, 4c + 2, 16 + 4c,
        // 16 + 4c + 2, 4c + 1, 4c + 3, 16 + 4c + 1, 16 + 4c + 3 (the order
        // q4_0_operand yields weights in).
        uint16_t* xh = reinterpret_cast<uint16_t*>(scratch + lay.xh);
        const int64_t stride = (int64_t)(gridDim.x - 1) * kGroupThreads * 8;
        for (int64_t i = ((int64_t)(blockIdx.x - 1) * kGroupThreads + threadIdx.x) * 8; i < x_count; i += stride) {
            const int64_t blk = i & ~(int64_t)31;
            const int c = (int)((i & 31) >> 3);
            const f32x4 a = *reinterpret_cast<const f32x4*>(x + blk + 4 * c);
            const f32x4 b = *reinterpret_cast<const f32x4*>(x + blk + 16 + 4 * c);
            *reinterpret_cast<u32x4*>(xh + i) = u32x4{pack_f16x2(a[0], a[2]), pack_f16x2(b[0], b[2]),
                                                      pack_f16x2(a[1], a[3]), pack_f16x2(b[1], b[3])};
#pragma unroll
            for (int t = 0; t < 4; ++t) oor |= out_of_f16_range(a[t]) || out_of_f16_range(b[t]);
        }
        if (__builtin_amdgcn_ballot_w64(oor) != 0 && (threadIdx.x & 63) == 0) atomicAdd(events, 1u);
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

// Grouped GEMM layout. A workgroup of 12 wavefronts takes one expert and a
// contiguous range of its 32-row weight tiles (the expert's tiles are split
// over enough workgroups to fill the chip) and streams them in chunks of up
// to 12 tiles, one tile per wavefront, over K in windows of 128 (four Q4_0
// blocks, 72 bytes of each weight row). A wavefront owns its tile for the
// whole of K, so its accumulators hold finished sums and no partial sums
// cross wavefronts.
constexpr int kMoeWaves = 12;                         // three to a SIMD: 168 registers each
constexpr int kMoeThreads = kMoeWaves * 64;
constexpr int kMoeTile = 32;                          // weight rows per wavefront (one 32x32 MFMA tile)
constexpr int kMoeMR = 32;                            // routed rows per pass
constexpr int kMoeChunkRows = kMoeTile * kMoeWaves;   // 384
constexpr int kMoeWinBlocks = 4;                      // Q4_0 blocks of a row per window (128 of K)
constexpr int kMoeWinBytes = 18 * kMoeWinBlocks;      // 72 bytes of a weight row per window
constexpr int kMoeSpan = 80;                          // ... moved as five 16-byte pieces (8 bytes read ahead)
constexpr int kMoeWDma = (kMoeChunkRows * kMoeSpan / 16 + 63) / 64;  // 30 DMA instructions per W window
constexpr int kMoeWSlot = kMoeWDma * 1024;            // 30 KB
constexpr int kMoeXRow = 32 * kMoeWinBlocks * 2;      // 256 bytes: 128 binary16 of a routed row per window
constexpr int kMoeXSlot = kMoeMR * kMoeXRow;          // 8 KB
constexpr int kMoeXDma = kMoeXSlot / 1024;            // 8 DMA instructions per x window
constexpr int kMoeStages = 3;                         // ring depth: window j + 1 in flight at window j
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
// Eight dwords at a wave-uniform address by one scalar-cache load (counted
// by lgkmcnt, so waiting for it does not wait for the DMA in flight). The
// address goes through readfirstlane so that it is in scalar registers even
// where the compiler cannot prove it uniform.
__device__ __forceinline__ void moe_sload8(const uint32_t* p, uint32_t (&v)[8]) {
    typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
    const uint64_t a = (uint64_t)(uintptr_t)p;
    // readfirstlane returns int: widen through uint32_t, or the low word would sign-extend.
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint64_t sa = ((uint64_t)hi << 32) | (uint64_t)lo;
    u32x8 r;
    asm volatile("s_load_dwordx8 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(sa) : "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = r[i];
}
// One lane's B operand for one Q4_0 block: qs dword c as fp16 (q - 8) d in
// the pair order of q4_0_dot_pairs, (4c, 4c+2) (16+4c, 16+4c+2) (4c+1, 4c+3)
// (16+4c+1, 16+4c+3): low nibbles arrive as binary16 1024 + q and high ones
// as 64 + q; subtracting 1032 or 72 is exact and leaves q - 8, and the
// product with d rounds once.
struct Q4Consts {
    uint32_t m_lo, m_hi, magic_lo, magic_hi;  // held in VGPRs so each mask-and-insert is one v_and_or_b32
};
__device__ __forceinline__ u32x4 q4_0_operand(uint32_t qs, f16x2 dd, const Q4Consts& k) {
    uint32_t p[4];
    q4_0_dot_pairs(qs, k.m_lo, k.m_hi, k.magic_lo, k.magic_hi, p);
    const f16x2 lo_bias = as_f16x2(0xE408E408u), hi_bias = as_f16x2(0xD480D480u);  // -1032, -72
    u32x4 o;
    o[0] = as_u32((as_f16x2(p[0]) + lo_bias) * dd);
    o[1] = as_u32((as_f16x2(p[1]) + hi_bias) * dd);
    o[2] = as_u32((as_f16x2(p[2]) + lo_bias) * dd);
    o[3] = as_u32((as_f16x2(p[3]) + hi_bias) * dd);
    return o;
}

// One 128-wide K window for a wavefront's 32 weight rows against the pass's
// 32 routed rows: eight MFMA k-steps t. Lane (n, h) = (lane % 32, lane / 32)
// takes blocks 2 h and 2 h + 1 of weight row n's window and in step t feeds
// qs dword t % 4 of block 2 h + t / 4. The x operand of lane (m, h) in step t
// is the same eight elements of routed row m: in the xh order the 16-byte
// chunk 4 (2 h + t / 4) + t % 4 = t + 8 h of the window row, kept at slot
// chunk ^ (m % 16) so that the 32-row reads are conflict-free. A lane reads
// its two blocks as 40 bytes of its row's 80-byte image (h = 0: bytes
// 0 .. 39, h = 1: bytes 32 .. 71) by two 16-byte reads, which eight lanes of
// consecutive rows spread over all 32 banks, and one 8-byte read. Every
// byte read is used: a dead part of a read's destination would let the
// compiler reuse it as a temporary and wait for the whole read first. The
// window's LDS reads (moe_read) are issued a window ahead of its arithmetic
// (moe_apply), so they overlap the previous window's decode and matrix work
// instead of following each barrier.
struct MoeOps {
    u32x4 x[8];  // x operands per step
    u32x4 w[2];  // the lane's first 32 bytes
    u32x2 w2;    // and the 8 after them
};
// The realigning form, for rows whose windows may start 2 bytes past a dword
// (an odd number of blocks per row, or w or the expert stride only 2-byte
// aligned): each row is moved from the dword at or below its window, so its
// window starts `phase` (0 or 2) bytes into its LDS image, and the lane's
// scales and qs dwords are read as 16-bit halves.
typedef uint16_t u16x2 __attribute__((__vector_size__(2 * sizeof(uint16_t))));
struct MoeOpsR {
    u32x4 x[8];
    uint32_t d[2];      // the lane's blocks' scales (binary16)
    uint32_t qs[2][4];  // and their qs dwords
};
// A lane's LDS read addresses (byte addresses) in slot 0 of the rings; slot
// s adds s slot sizes, folded into the instructions' 16-bit offsets. The
// register fence keeps each address whole in one register (otherwise the
// compiler folds the ring base into the offset, overflows the field and
// adds it back per read).
struct MoeLane {
    // aligned form: the lane's first piece, row image + 32 h; realigning
    // form: its first block, row image + phase + 36 h (the second block 18
    // bytes on; in each, d then the four qs dwords)
    uint32_t w;
    // step t's x chunk t + 8 h of routed row m, at its swizzled slot; in the
    // padded x layout (rows kMoeXRowP bytes apart, chunks in order) only x[0]
    // is set, and step t's chunk is 16 t bytes after it
    uint32_t x[8];
};
constexpr int kMoeXRowP = kMoeXRow + 16;       // padded x row: 32-row reads conflict-free without a swizzle
constexpr int kMoeXSlotP = kMoeMR * kMoeXRowP;  // 8.5 KB
template <bool RE, bool PAD = false>
__device__ __forceinline__ MoeLane moe_lane(const uint8_t* wring, const uint8_t* xring, int nl, int lane,
                                            uint32_t phase) {
    const int h = lane >> 5, m = lane & 31, sw = m & 15;
    MoeLane l;
    l.w = moe_lds_addr(wring) + nl * kMoeSpan + (RE ? phase + 36u * h : 32u * h);
    asm volatile("" : "+v"(l.w));
    if constexpr (PAD) {
        l.x[0] = moe_lds_addr(xring) + m * kMoeXRowP + 128 * h;
        asm volatile("" : "+v"(l.x[0]));
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            l.x[t] = moe_lds_addr(xring) + m * kMoeXRow + 16 * ((t + 8 * h) ^ sw);
            asm volatile("" : "+v"(l.x[t]));
        }
    }
    return l;
}
template <int SLOT, bool PAD>
__device__ __forceinline__ uint32_t moe_x_addr(const MoeLane& l, int t) {
    return PAD ? l.x[0] + 16 * t + SLOT * kMoeXSlotP : l.x[t] + SLOT * kMoeXSlot;
}
template <typename T>
__device__ __forceinline__ T moe_lds_load(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) T*>((uintptr_t)addr);
}
template <int SLOT, bool PAD = false>
__device__ __forceinline__ MoeOps moe_read(const MoeLane& l) {
    MoeOps o;
#pragma unroll
    for (int t = 0; t < 8; ++t) o.x[t] = moe_lds_load<u32x4>(moe_x_addr<SLOT, PAD>(l, t));
#pragma unroll
    for (int i = 0; i < 2; ++i) o.w[i] = moe_lds_load<u32x4>(l.w + SLOT * kMoeWSlot + 16 * i);
    o.w2 = moe_lds_load<u32x2>(l.w + SLOT * kMoeWSlot + 32);
    return o;
}
template <int SLOT, bool PAD = false>
__device__ __forceinline__ MoeOpsR moe_read_r(const MoeLane& l) {
    MoeOpsR o;
#pragma unroll
    for (int t = 0; t < 8; ++t) o.x[t] = moe_lds_load<u32x4>(moe_x_addr<SLOT, PAD>(l, t));
    const uint32_t w = l.w + SLOT * kMoeWSlot;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        o.d[b] = moe_lds_load<uint16_t>(w + 18 * b);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u16x2 v;
            v[0] = moe_lds_load<uint16_t>(w + 18 * b + 2 + 4 * i);
            v[1] = moe_lds_load<uint16_t>(w + 18 * b + 4 + 4 * i);
            o.qs[b][i] = __builtin_bit_cast(uint32_t, v);
        }
    }
    return o;
}
// The eight steps from the lane's two blocks' scales and qs dwords. Blocks at
// or past `live` (a part last window when K % 128 != 0) get d = 0, which
// zeroes their weights whatever the ring holds there; their x chunks were
// loaded as zeros.
__device__ __forceinline__ void moe_steps(const u32x4 (&x)[8], const uint32_t (&d)[2], const uint32_t (&qs)[2][4],
                                          int h, const Q4Consts& k, f32x16& acc, int live) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const f16x2 dd = as_f16x2((2 * h + b < live ? d[b] & 0xFFFFu : 0u) * 0x10001u);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x[4 * b + i]),
                                                         __builtin_bit_cast(f16x8, q4_0_operand(qs[b][i], dd, k)), acc, 0, 0, 0);
    }
}
__device__ __forceinline__ void moe_apply_r(const MoeOpsR& o, int h, const Q4Consts& k, f32x16& acc, int live) {
    moe_steps(o.x, o.d, o.qs, h, k, acc, live);
}
// Aligned form: h = 0 lanes' blocks start at byte 0 of what they read, h = 1
// lanes' at byte 4 (window byte 36); with the dwords shifted down one for
// h = 1, block 2 h sits at bytes 0 .. 17 and block 2 h + 1 at 18 .. 35.
__device__ __forceinline__ void moe_apply(const MoeOps& o, int h, const Q4Consts& k, f32x16& acc, int live) {
    uint32_t r[10], s[9];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) r[4 * i + j] = o.w[i][j];
    r[8] = o.w2[0];
    r[9] = o.w2[1];
#pragma unroll
    for (int i = 0; i < 9; ++i) s[i] = h ? r[i + 1] : r[i];
    const uint32_t d[2] = {s[0], s[4] >> 16};
    uint32_t qs[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        qs[0][i] = __builtin_amdgcn_alignbyte(s[i + 1], s[i], 2);
        qs[1][i] = s[5 + i];
    }
    moe_steps(o.x, d, qs, h, k, acc, live);
}
__device__ __forceinline__ void moe_wait_lgkm() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// LDS: kMoeStages slots of W [384 rows x 80 B] (row r's window bytes, as
// stored, at 80 r) and of x [32 rows x 256 B] (routed row m's chunk c at
// slot c ^ (m % 16)), then the pass's 32 output row indices.
// DMA roles: x instruction i (rows 4 i .. 4 i + 3) is issued by wavefront i,
// W instruction i (16-byte pieces 64 i .. 64 i + 63 of the slot: row q / 5,
// piece q % 5) by wavefront (i + 8) % 12, so no wavefront issues more than
// four per window. Window j + 2 is issued after barrier j into the slot of
// window j - 1, which every wavefront finished reading before barrier j; each
// wavefront waits for its own DMA of window j before barrier j, after which
// every wavefront may read it. All DMA offsets are per-lane (no scalar
// offset), so the descriptors' range checks cover every byte read: the 6 or
// 8 bytes read past a row's last window are the next row's (unused) or, past
// the chunk's last row, zeros.
constexpr int kMoeLds = kMoeStages * (kMoeWSlot + kMoeXSlot) + kMoeMR * 4;

template <bool RE>
__global__ __launch_bounds__(kMoeThreads) void moe_gemm_kernel(const uint8_t* __restrict__ w, const uint8_t* __restrict__ scratch,
                                                               float* __restrict__ out, int N, int K, int top_k,
                                                               uint64_t expert_stride, IdScratchLayout lay, int n_tokens,
                                                               int splits) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kMoeLds];
    uint8_t* const wring = lds;
    uint8_t* const xring = lds + kMoeStages * kMoeWSlot;
    uint32_t* const pass_rows = reinterpret_cast<uint32_t*>(xring + kMoeStages * kMoeXSlot);
    const int e = blockIdx.x / splits, part = blockIdx.x % splits;
    const int tiles = (N + kMoeTile - 1) / kMoeTile;
    const int t_begin = (int)((int64_t)part * tiles / splits), t_end = (int)((int64_t)(part + 1) * tiles / splits);
    const uint32_t cnt = reinterpret_cast<const uint32_t*>(scratch + lay.counts)[e];
    if (cnt == 0u || t_begin >= t_end) return;
    const uint32_t* rows =
        reinterpret_cast<const uint32_t*>(scratch + lay.rows) + reinterpret_cast<const uint32_t*>(scratch + lay.offsets)[e];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = K / 32;
    const int nwin = (nb + kMoeWinBlocks - 1) / kMoeWinBlocks;
    const int last_live = nb - kMoeWinBlocks * (nwin - 1);  // blocks in the last window (1 to 4)
    const uint32_t row_bytes = (uint32_t)nb * 18u;
    const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(scratch + lay.xh, (uint32_t)((size_t)n_tokens * (size_t)K * 2u));
    const Q4Consts k{vreg(0x000F000Fu), vreg(0x00F000F0u), vreg(0x64006400u), vreg(0x54005400u)};
    const bool x_dma = wave < kMoeXDma;
    const int wi0 = (wave + kMoeWaves - kMoeXDma) % kMoeWaves;  // this wavefront's W instructions: wi0 + 12 t
    // x DMA lane (wavefronts 0 .. 7): routed row m = 4 wave + lane / 16, LDS
    // position lane % 16 of that row holds chunk c = (lane % 16) ^ (m % 16),
    // from K block 4 w + c / 4 of window w.
    const int xm = 4 * wave + (lane >> 4);
    const int xc = (lane & 15) ^ (xm & 15);
    uint32_t xo = kMoeOob;  // the pass's routed row's lane offset (set per pass)
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    static_assert(kMoeStages == 3, "the slot sequences below are written for three slots");

    for (uint32_t m0 = 0; m0 < cnt; m0 += kMoeMR) {
        const uint32_t mcnt = min((uint32_t)kMoeMR, cnt - m0);
        moe_barrier();  // the previous pass's stores have read pass_rows
        for (int tc = t_begin; tc < t_end; tc += kMoeWaves) {
            const int n0 = tc * kMoeTile;
            const int crow = min(min(t_end - tc, kMoeWaves) * kMoeTile, N - n0);
            // The realigning form reads from the dword at or below the chunk
            // (delta bytes before it) through the dword holding its last byte.
            const uint8_t* const chunk = w + (size_t)e * expert_stride + (size_t)n0 * row_bytes;
            const uint32_t delta = RE ? (uint32_t)((uintptr_t)chunk & 3u) : 0u;
            const __amdgpu_buffer_rsrc_t wsrc =
                make_rsrc(chunk - delta, RE ? ((uint32_t)crow * row_bytes + delta + 3u) & ~3u : (uint32_t)crow * row_bytes);
            const int n_wi = (crow * (kMoeSpan / 16) + 63) / 64;  // W DMA instructions per window
            const int nw = (wi0 < n_wi ? 1 : 0) + (wi0 + kMoeWaves < n_wi ? 1 : 0) + (wi0 + 2 * kMoeWaves < n_wi ? 1 : 0);
            uint32_t wo[3];
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const int q = 64 * (wi0 + kMoeWaves * t) + lane, r = q / 5, j = q % 5;
                wo[t] = r < crow ? (((uint32_t)r * row_bytes + delta) & ~3u) + 16u * (uint32_t)j : kMoeOob;
            }
            // DMA of window win into ring slot SLOT (= win % kMoeStages).
            auto issue_w = [&](auto slot_c, int win) {
                constexpr int slot = decltype(slot_c)::value;
#pragma unroll
                for (int t = 0; t < 3; ++t)
                    if (t < nw)
                        moe_dma16(wsrc, wring + slot * kMoeWSlot + 1024 * (wi0 + kMoeWaves * t),
                                  wo[t] + (uint32_t)(kMoeWinBytes * win), 0);
            };
            auto issue_x = [&](auto slot_c, int win) {
                constexpr int slot = decltype(slot_c)::value;
                // Chunks of blocks past K (a part last window) land as zeros.
                if (x_dma)
                    moe_dma16(xsrc, xring + slot * kMoeXSlot + 1024 * wave,
                              kMoeWinBlocks * win + (xc >> 2) < nb ? xo + (uint32_t)(kMoeXRow * win) : kMoeOob, 0);
            };
            // Prologue, windows 0 and 1: the weights need no routing ids, so
            // W(0) goes out before the ids are read; then x(0), W(1), x(1).
            issue_w(S0{}, 0);
            if (tc == t_begin) {
                // This pass's routed rows: x DMA wavefront i (rows 4 i .. 4 i + 3)
                // reads its ids by one scalar load (not counted by vmcnt, so it
                // does not wait behind the DMA) and records them for the stores.
                // Ids past the pass's count are not used.
                if (x_dma) {
                    uint32_t id[8];
                    moe_sload8(rows + m0 + 4 * wave, id);
                    const int r = lane >> 4;
                    uint32_t rid = id[0], own = id[0];
#pragma unroll
                    for (int i = 1; i < 4; ++i) {
                        rid = r == i ? id[i] : rid;
                        own = lane == i ? id[i] : own;
                    }
                    xo = (uint32_t)xm < mcnt ? (rid / (uint32_t)top_k) * (uint32_t)K * 2u + 16u * (uint32_t)xc : kMoeOob;
                    if (lane < 4) pass_rows[4 * wave + lane] = own;
                }
            }
            issue_x(S0{}, 0);
            if (nwin > 1) {
                issue_w(S1{}, 1);
                issue_x(S1{}, 1);
            }
            const int per_window = nw + (x_dma ? 1 : 0);
            // At window j (>= 0) only this wavefront's DMA of window j + 1 may
            // still be in flight (each window's W then x, in window order).
            auto wait_window = [&](int j) {
                if (j + 1 >= nwin) {
                    moe_wait_vmcnt<0>();
                    return;
                }
                switch (per_window) {
                    case 0: moe_wait_vmcnt<0>(); break;
                    case 1: moe_wait_vmcnt<1>(); break;
                    case 2: moe_wait_vmcnt<2>(); break;
                    case 3: moe_wait_vmcnt<3>(); break;
                    default: moe_wait_vmcnt<4>(); break;
                }
            };
            f32x16 acc;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = 0.f;
            const bool busy = kMoeTile * wave < crow;
            const int nl = kMoeTile * wave + (lane & 31);  // this lane's weight row in the chunk
            const MoeLane ln = moe_lane<RE>(wring, xring, nl, lane, ((uint32_t)nl * row_bytes + delta) & 3u);
            // Two operand sets alternate (the loop is unrolled by six, a multiple
            // of the ring depth, so that neither set is copied and every slot
            // offset is a constant): after barrier j a wavefront reads window j
            // into one set, then decodes and multiplies window j - 1 from the
            // other.
            using Ops = std::conditional_t<RE, MoeOpsR, MoeOps>;
            auto read = [&](auto slot_c) {
                if constexpr (RE)
                    return moe_read_r<decltype(slot_c)::value>(ln);
                else
                    return moe_read<decltype(slot_c)::value>(ln);
            };
            const int h = lane >> 5;
            auto apply = [&](const Ops& o, int live) {
                if constexpr (RE)
                    moe_apply_r(o, h, k, acc, live);
                else
                    moe_apply(o, h, k, acc, live);
            };
            Ops ops[2];
            wait_window(0);
            moe_wait_lgkm();  // pass_rows written
            moe_barrier();
            if (busy) ops[0] = read(S0{});
            if (kMoeStages - 1 < nwin) {
                issue_w(S2{}, kMoeStages - 1);
                issue_x(S2{}, kMoeStages - 1);
            }
            auto step = [&](auto slot_c, int j, Ops& into, const Ops& from) {
                constexpr int slot = decltype(slot_c)::value;
                wait_window(j);
                moe_wait_lgkm();  // this wavefront's reads of window j - 1 are done: its slot is reused below
                moe_barrier();
                if (busy) {
                    into = read(slot_c);
                    __builtin_amdgcn_sched_barrier(0);  // the reads go out before the arithmetic below
                    apply(from, kMoeWinBlocks);
                }
                if (j + kMoeStages - 1 < nwin) {
                    using Next = std::integral_constant<int, (slot + kMoeStages - 1) % kMoeStages>;
                    issue_w(Next{}, j + kMoeStages - 1);
                    issue_x(Next{}, j + kMoeStages - 1);
                }
            };
            int j = 1;  // j % 6 == 1 at the top of each round
            for (; j + 5 < nwin; j += 6) {
                step(S1{}, j, ops[1], ops[0]);
                step(S2{}, j + 1, ops[0], ops[1]);
                step(S0{}, j + 2, ops[1], ops[0]);
                step(S1{}, j + 3, ops[0], ops[1]);
                step(S2{}, j + 4, ops[1], ops[0]);
                step(S0{}, j + 5, ops[0], ops[1]);
            }
            if (j < nwin) step(S1{}, j, ops[1], ops[0]);
            if (j + 1 < nwin) step(S2{}, j + 1, ops[0], ops[1]);
            if (j + 2 < nwin) step(S0{}, j + 2, ops[1], ops[0]);
            if (j + 3 < nwin) step(S1{}, j + 3, ops[0], ops[1]);
            if (j + 4 < nwin) step(S2{}, j + 4, ops[1], ops[0]);
            if (busy) {
                if ((nwin - 1) & 1)  // the last window's set
                    apply(ops[1], last_live);
                else
                    apply(ops[0], last_live);
                // Lane (n, h) holds routed rows 8 (i / 4) + 4 h + i % 4 of weight row n.
                const int ncol = n0 + nl;
                uint32_t pr = moe_lds_addr(pass_rows) + 16u * (uint32_t)(lane >> 5);  // row 4 h's id
                asm volatile("" : "+v"(pr));  // one base register, the rest in offsets
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const uint32_t mm = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                    const uint32_t row = moe_lds_load<uint32_t>(pr + 4u * (8 * (i >> 2) + (i & 3)));
                    if (mm < mcnt && ncol < N) out[(size_t)row * N + ncol] = acc[i];
                }
            }
            moe_wait_vmcnt<0>();  // stores done: the next chunk's DMA waits count only DMA
            moe_wait_lgkm();
            moe_barrier();        // every wavefront is done with the ring before the next chunk's DMA
        }
    }
}


// ---------------------------------------------------------------- one-launch grouped route
// Up to kFusedMaxRows routed rows the grouping pass and the binary16 copy of
// x move into the GEMM's workgroups, and the route is one launch:
//  - every workgroup scans the ids for its expert and lists the matching
//    routed rows in LDS (in any order: an output row's arithmetic does not
//    depend on its position in the tile); workgroup 0 also counts the ids
//    that name no expert and writes their rows as zeros.
//  - the routed rows' f32 x is moved by buffer-to-LDS DMA into a 2-slot
//    staging ring, a window ahead, and the wavefront that moved a row rounds
//    it to binary16 in the xh order into the x ring that the matrix steps
//    read; rows past the pass's count are neither moved nor rounded.
// The weight stream, the decode and the matrix steps are the grouped GEMM's.
constexpr int kFusedMaxRows = 4096;
constexpr int kFxRow = 32 * kMoeWinBlocks * 4;  // 512 bytes: a routed row's f32 x per window
constexpr int kFxSlot = kMoeMR * kFxRow;        // 16 KB
constexpr int kFusedLds = kMoeStages * (kMoeWSlot + kMoeXSlotP) + 2 * kFxSlot + kFusedMaxRows * 2 + kMoeMR * 4 + 16;
static_assert(kFusedLds <= 160 * 1024, "the one-launch route's LDS");

__device__ __forceinline__ void moe_wait_vm(int n) {
    switch (n) {
        case 0: moe_wait_vmcnt<0>(); break;
        case 1: moe_wait_vmcnt<1>(); break;
        case 2: moe_wait_vmcnt<2>(); break;
        case 3: moe_wait_vmcnt<3>(); break;
        case 4: moe_wait_vmcnt<4>(); break;
        case 5: moe_wait_vmcnt<5>(); break;
        case 6: moe_wait_vmcnt<6>(); break;
        case 7: moe_wait_vmcnt<7>(); break;
        default: moe_wait_vmcnt<8>(); break;
    }
}
// The lane index computed where it is used (volatile, so the compiler neither
// hoists it nor keeps it in a register across the loops).
__device__ __forceinline__ uint32_t moe_lane_id() {
    uint32_t v;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
    return v;
}
template <typename T>
__device__ __forceinline__ void moe_lds_store(uint32_t addr, const T& v) {
    *reinterpret_cast<__attribute__((address_space(3))) T*>((uintptr_t)addr) = v;
}

template <bool RE>
__global__ __launch_bounds__(kMoeThreads) void moe_fused_kernel(const float* __restrict__ x, const uint8_t* __restrict__ w,
                                                                const uint32_t* __restrict__ ids, float* __restrict__ out,
                                                                uint32_t* __restrict__ bad_out, int N, int K, int top_k,
                                                                int n_rows, int n_experts, uint64_t expert_stride,
                                                                int n_tokens, int splits, uint32_t* __restrict__ events) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kFusedLds];
    uint8_t* const wring = lds;
    uint8_t* const xring = wring + kMoeStages * kMoeWSlot;
    uint8_t* const xstage = xring + kMoeStages * kMoeXSlotP;
    uint16_t* const list = reinterpret_cast<uint16_t*>(xstage + 2 * kFxSlot);
    uint32_t* const pass_rows = reinterpret_cast<uint32_t*>(list + kFusedMaxRows);
    uint32_t* const counters = pass_rows + kMoeMR;  // the list's length, the ids naming no expert
    const int e = blockIdx.x / splits, part = blockIdx.x % splits;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tiles = (N + kMoeTile - 1) / kMoeTile;
    const int t_begin = (int)((int64_t)part * tiles / splits), t_end = (int)((int64_t)(part + 1) * tiles / splits);
    const int nb = K / 32;
    const int nwin = (nb + kMoeWinBlocks - 1) / kMoeWinBlocks;
    const uint32_t row_bytes = (uint32_t)nb * 18u;
    const int wi0 = (wave + kMoeWaves - kMoeXDma) % kMoeWaves;  // this wavefront's W instructions: wi0 + 12 t

    // The weight chunk of tiles tc .. : its descriptor, this wavefront's DMA
    // offsets and instruction count.
    int n0 = 0, crow = 0, nw = 0;
    uint32_t delta = 0u, wo[3];
    __amdgpu_buffer_rsrc_t wsrc;
    auto setup = [&](int tc) {
        n0 = tc * kMoeTile;
        crow = min(min(t_end - tc, kMoeWaves) * kMoeTile, N - n0);
        const uint8_t* const chunk = w + (size_t)e * expert_stride + (size_t)n0 * row_bytes;
        delta = RE ? (uint32_t)((uintptr_t)chunk & 3u) : 0u;
        wsrc = make_rsrc(chunk - delta, RE ? ((uint32_t)crow * row_bytes + delta + 3u) & ~3u : (uint32_t)crow * row_bytes);
        const int n_wi = (crow * (kMoeSpan / 16) + 63) / 64;
        nw = (wi0 < n_wi ? 1 : 0) + (wi0 + kMoeWaves < n_wi ? 1 : 0) + (wi0 + 2 * kMoeWaves < n_wi ? 1 : 0);
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const int q = 64 * (wi0 + kMoeWaves * t) + lane, r = q / 5, j = q % 5;
            wo[t] = r < crow ? (((uint32_t)r * row_bytes + delta) & ~3u) + 16u * (uint32_t)j : kMoeOob;
        }
    };
    // Window win's weights into ring slot SLOT.
    auto issue_w = [&](auto slot_c, int win) {
        constexpr int slot = decltype(slot_c)::value;
#pragma unroll
        for (int t = 0; t < 3; ++t)
            if (t < nw)
                moe_dma16(wsrc, wring + slot * kMoeWSlot + 1024 * (wi0 + kMoeWaves * t), wo[t] + (uint32_t)(kMoeWinBytes * win), 0);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    // The first chunk's weights of windows 0 and 1 need no routing: they go
    // out before the scan (whose loads wait for them too).
    const bool early = t_begin < t_end;
    if (early) {
        setup(t_begin);
        issue_w(S0{}, 0);
        if (nwin > 1) issue_w(S1{}, 1);
    }

    // This expert's routed rows.
    if (tid < 2) counters[tid] = 0u;
    __syncthreads();
    for (int r0 = 0; r0 < n_rows; r0 += kMoeThreads) {
        const int r = r0 + tid;
        const uint32_t id = r < n_rows ? ids[r] : 0u;
        const bool mine = r < n_rows && id == (uint32_t)e;
        const uint64_t bal = __builtin_amdgcn_ballot_w64(mine);
        if (bal != 0u) {
            uint32_t base = 0u;
            if (lane == 0) base = atomicAdd(&counters[0], (uint32_t)__popcll(bal));
            base = (uint32_t)__builtin_amdgcn_readfirstlane(base);
            const uint64_t below = lane == 0 ? 0u : bal & (~0ull >> (64 - lane));
            if (mine) list[base + (uint32_t)__popcll(below)] = (uint16_t)r;
        }
        if (blockIdx.x == 0 && r < n_rows && id >= (uint32_t)n_experts) {
            atomicAdd(&counters[1], 1u);
            for (int n = 0; n < N; ++n) out[(size_t)r * N + n] = 0.f;  // no expert to read
        }
    }
    moe_wait_vmcnt<0>();  // the early weights and the zero rows' stores: the DMA waits below count only DMA
    __syncthreads();
    const uint32_t cnt = counters[0];
    if (blockIdx.x == 0 && tid == 0) *bad_out = counters[1];
    if (cnt == 0u || t_begin >= t_end) return;

    const int last_live = nb - kMoeWinBlocks * (nwin - 1);  // blocks in the last window (1 to 4)
    const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(x, (uint32_t)((size_t)n_tokens * (size_t)K * 4u));
    // masks as constants (one scalar operand per v_and_or_b32), magic values in VGPRs
    const Q4Consts k{0x000F000Fu, 0x00F000F0u, vreg(0x64006400u), vreg(0x54005400u)};
    // x wavefronts 0 .. 7: wavefront v moves and rounds routed rows 4 v .. 4 v + 3
    // (DMA instruction 2 v + s: rows 4 v + 2 s + lane / 32, f32 piece lane % 32).
    const bool x_wave = wave < kMoeMR / 4;
    const bool count_events = part == 0;
    bool oor = false;
    static_assert(kMoeStages == 3, "the slot sequences below are written for three slots");

    for (uint32_t m0 = 0; m0 < cnt; m0 += kMoeMR) {
        const uint32_t mcnt = min((uint32_t)kMoeMR, cnt - m0);
        moe_barrier();  // the previous pass's stores have read pass_rows
        {
            // the thread index afresh (not held in a register across the loops)
            const uint32_t t = 64u * (uint32_t)wave + moe_lane_id();
            if (t < (uint32_t)kMoeMR) pass_rows[t] = t < mcnt ? (uint32_t)list[m0 + t] : 0u;
        }
        uint32_t xo[2];
        int nx = 0;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint32_t ln = moe_lane_id();  // afresh, as above
            const uint32_t xr = 4u * (uint32_t)wave + 2u * (uint32_t)s + (ln >> 5);
            xo[s] = x_wave && xr < mcnt ? ((uint32_t)list[m0 + xr] / (uint32_t)top_k) * (uint32_t)K * 4u + 16u * (ln & 31u)
                                        : kMoeOob;
            nx += x_wave && (uint32_t)(4 * wave + 2 * s) < mcnt ? 1 : 0;
        }
        for (int tc = t_begin; tc < t_end; tc += kMoeWaves) {
            // the first chunk of the first pass: set up, windows 0 and 1 of its weights landed
            const bool pre = m0 == 0 && tc == t_begin;
            if (!pre) setup(tc);
            const bool events_here = count_events && tc == t_begin;  // later chunks round the same x again
            // Window win's x into staging slot ST, then (unless already out) its
            // weights into ring slot SLOT.
            auto issue = [&](auto st_c, auto slot_c, int win, bool with_w) {
                constexpr int st = decltype(st_c)::value;
                // f32 pieces of blocks past K (a part last window) land as zeros
                const bool in_k = kMoeWinBlocks * win + ((lane & 31) >> 3) < nb;
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    if (x_wave && (uint32_t)(4 * wave + 2 * s) < mcnt)
                        moe_dma16(xsrc, xstage + st * kFxSlot + 1024 * (2 * wave + s),
                                  in_k ? xo[s] + (uint32_t)(kFxRow * win) : kMoeOob, 0);
                if (with_w) issue_w(slot_c, win);
            };
            // Round the routed rows' x of a window, staging slot ST -> x ring slot
            // SLOT: lane (r, c) writes chunk c of row r in the xh order, from the
            // two f32 pieces that hold it.
            auto convert = [&](auto st_c, auto slot_c) {
                constexpr int st = decltype(st_c)::value, slot = decltype(slot_c)::value;
                const int r = 4 * wave + (lane >> 4), c = lane & 15;
                if (x_wave && (uint32_t)r < mcnt) {
                    const uint32_t src = moe_lds_addr(xstage) + st * kFxSlot + r * kFxRow + 16 * (8 * (c >> 2) + (c & 3));
                    const f32x4 a = moe_lds_load<f32x4>(src), b = moe_lds_load<f32x4>(src + 64);
                    moe_lds_store(moe_lds_addr(xring) + slot * kMoeXSlotP + r * kMoeXRowP + 16 * c,
                                  u32x4{pack_f16x2(a[0], a[2]), pack_f16x2(b[0], b[2]), pack_f16x2(a[1], a[3]),
                                        pack_f16x2(b[1], b[3])});
                    if (events_here)
#pragma unroll
                        for (int t = 0; t < 4; ++t) oor |= out_of_f16_range(a[t]) || out_of_f16_range(b[t]);
                }
            };
            f32x16 acc;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = 0.f;
            const bool busy = kMoeTile * wave < crow;
            const int nl = kMoeTile * wave + (lane & 31);
            const MoeLane ln = moe_lane<RE, true>(wring, xring, nl, lane, ((uint32_t)nl * row_bytes + delta) & 3u);
            const int h = lane >> 5;
            using Ops = std::conditional_t<RE, MoeOpsR, MoeOps>;
            auto read = [&](auto slot_c) {
                if constexpr (RE)
                    return moe_read_r<decltype(slot_c)::value, true>(ln);
                else
                    return moe_read<decltype(slot_c)::value, true>(ln);
            };
            auto apply = [&](const Ops& o, int live) {
                if constexpr (RE)
                    moe_apply_r(o, h, k, acc, live);
                else
                    moe_apply(o, h, k, acc, live);
            };
            // Per window this wavefront issues nx x then nw weight DMA
            // instructions; waits count what may stay in flight behind the one
            // awaited, in issue order.
            const int per_window = nx + nw;
            // Issue order: x(0) W(0) x(1) W(1), or, for the first chunk, x(0) x(1)
            // after the weights' windows 0 and 1 have landed.
            Ops ops[2];
            issue(S0{}, S0{}, 0, !pre);
            if (nwin > 1) issue(S1{}, S1{}, 1, !pre);
            const int after_x0 = pre ? (nwin > 1 ? nx : 0) : nw + (nwin > 1 ? per_window : 0);
            moe_wait_vm(after_x0);                                   // x(0)
            convert(S0{}, S0{});
            moe_wait_vm(pre ? after_x0 : (nwin > 1 ? per_window : 0));  // W(0)
            moe_wait_lgkm();                                         // pass_rows, x(0) written
            moe_barrier();
            if (nwin > 2) issue(S0{}, S2{}, 2, true);
            if (busy) ops[0] = read(S0{});
            if (nwin > 1) {
                moe_wait_vm((pre ? 0 : nw) + (nwin > 2 ? per_window : 0));  // x(1)
                convert(S1{}, S1{});
            }
            // Step j: ring slot j % 3, staging parity j % 2.
            auto step = [&](auto slot_c, auto par_c, int j, Ops& into, const Ops& from) {
                constexpr int slot = decltype(slot_c)::value, par = decltype(par_c)::value;
                moe_wait_vm(j + 1 < nwin ? per_window : 0);  // W(j); x(j) was rounded in step j - 1
                moe_wait_lgkm();  // this wavefront's reads of window j - 1 and writes of x(j) are done
                moe_barrier();
                if (j + 2 < nwin) {
                    using Next = std::integral_constant<int, (slot + 2) % 3>;
                    issue(par_c, Next{}, j + 2, true);
                }
                if (busy) {
                    into = read(slot_c);
                    __builtin_amdgcn_sched_barrier(0);  // the reads go out before the arithmetic below
                    apply(from, kMoeWinBlocks);
                }
                if (j + 1 < nwin) {
                    using Other = std::integral_constant<int, 1 - par>;
                    using Next = std::integral_constant<int, (slot + 1) % 3>;
                    __builtin_amdgcn_sched_barrier(0);  // after the arithmetic: the set it read is free
                    moe_wait_vm(nw + (j + 2 < nwin ? per_window : 0));  // x(j + 1)
                    convert(Other{}, Next{});
                }
            };
            int j = 1;  // j % 6 == 1 at the top of each round
            for (; j + 5 < nwin; j += 6) {
                step(S1{}, S1{}, j, ops[1], ops[0]);
                step(S2{}, S0{}, j + 1, ops[0], ops[1]);
                step(S0{}, S1{}, j + 2, ops[1], ops[0]);
                step(S1{}, S0{}, j + 3, ops[0], ops[1]);
                step(S2{}, S1{}, j + 4, ops[1], ops[0]);
                step(S0{}, S0{}, j + 5, ops[0], ops[1]);
            }
            if (j < nwin) step(S1{}, S1{}, j, ops[1], ops[0]);
            if (j + 1 < nwin) step(S2{}, S0{}, j + 1, ops[0], ops[1]);
            if (j + 2 < nwin) step(S0{}, S1{}, j + 2, ops[1], ops[0]);
            if (j + 3 < nwin) step(S1{}, S0{}, j + 3, ops[0], ops[1]);
            if (j + 4 < nwin) step(S2{}, S1{}, j + 4, ops[1], ops[0]);
            if (busy) {
                if ((nwin - 1) & 1)  // the last window's set
                    apply(ops[1], last_live);
                else
                    apply(ops[0], last_live);
                const int ncol = n0 + nl;
                uint32_t pr = moe_lds_addr(pass_rows) + 16u * (uint32_t)(lane >> 5);
                asm volatile("" : "+v"(pr));
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const uint32_t mm = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                    const uint32_t row = moe_lds_load<uint32_t>(pr + 4u * (8 * (i >> 2) + (i & 3)));
                    if (mm < mcnt && ncol < N) out[(size_t)row * N + ncol] = acc[i];
                }
            }
            moe_wait_vmcnt<0>();  // stores done: the next chunk's DMA waits count only DMA
            moe_wait_lgkm();
            moe_barrier();        // every wavefront is done with the rings before the next chunk's DMA
        }
    }
    if (__builtin_amdgcn_ballot_w64(oor) != 0 && moe_lane_id() == 0) atomicAdd(events, 1u);
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
                                                               int n_rows, int n_experts, uint64_t expert_stride,
                                                               uint32_t* __restrict__ events) {
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
    // The first tile's workgroups check every activation they round to
    // binary16 (each routed row is served by exactly one of them) and count
    // a range event per wavefront that meets a finite value beyond its range.
    bool oor = false;
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
            if (blockIdx.x == 0 && p < kPieces)
#pragma unroll
                for (int t = 0; t < 4; ++t) oor |= out_of_f16_range(lo[0][t]) || out_of_f16_range(hi[0][t]);
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
    if (__builtin_amdgcn_ballot_w64(oor) != 0 && lane == 0) atomicAdd(events, 1u);
}

}  // namespace w4mi

using namespace w4mi;

namespace w4mi {

// One mat-vec launch over n_tokens * top_k routed rows (the caller checked
// n_routed <= 64 kMvIdSlots and K <= 32 kMvChunk kMvMaxChunks).
template <bool SWIGLU>
void mv_launch(const float* x, const float* up, const uint8_t* w, const uint32_t* ids, float* out, uint32_t* bad,
               const w4_id_params* p, hipStream_t s, uint32_t* events) {
    const uint32_t n_routed = p->n_tokens * p->top_k;
    const int chunks = (int)((p->k / 32 + kMvChunk - 1) / kMvChunk);
    const dim3 grid((unsigned)((p->n + kMvTile - 1) / kMvTile), n_routed), block(kMvWaves * 64);
    // Spans that may start off a dword boundary take the realigning form.
    const bool realign = ((p->k / 32) & 1u) || ((uintptr_t)w & 3u) || (p->expert_stride & 3u);
#define W4_MV_LAUNCH(T, RE)                                                                                      \
    hipLaunchKernelGGL((moe_mv_kernel<T, RE, SWIGLU>), grid, block, 0, s, x, up, w, ids, out, bad, (int)p->n,   \
                       (int)p->k, (int)p->top_k, (int)n_routed, (int)p->n_experts, p->expert_stride, events)
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
    uint32_t* events = nullptr;
    hipStream_t s = as_stream(stream);
    const uint64_t n_routed = (uint64_t)p->n_tokens * p->top_k;
    const int chunks = (int)((p->k / 32 + kMvChunk - 1) / kMvChunk);
    if (p->n_tokens <= kMvMaxTokens && n_routed <= 64u * kMvIdSlots && chunks <= kMvMaxChunks) {
        // Mat-vec route (the page's mv_id below its routing threshold).
        uint32_t* bad = reinterpret_cast<uint32_t*>((uint8_t*)scratch + lay.bad_ids);
        st = range_counter(&events, "qmm_id_q4_0");
        if (st != W4_OK) return st;
        mv_launch<false>(x, nullptr, w, ids, out, bad, p, s, events);
        return launch_status("qmm_id_q4_0 (mat-vec route)");
    }
    // Buffer descriptors cover the binary16 x copy and one 384-row weight chunk
    // in 32 bits, with in-range offsets below the out-of-range marker 2^31.
    if ((uint64_t)p->n_tokens * p->k * 2u >= (1ull << 32) || (uint64_t)kMoeChunkRows * (p->k / 32) * 18u >= (1ull << 31))
        return fail(W4_EUNSUPPORTED, "qmm_id_q4_0: implemented for n_tokens * K * 2 < 2^32 bytes and 384-row weight chunks below 2^31 bytes");
    st = range_counter(&events, "qmm_id_q4_0");
    if (st != W4_OK) return st;
    // Rows whose windows may start off a dword boundary take the realigning form.
    const bool realign = ((p->k / 32) & 1u) || ((uintptr_t)w & 3u) || (p->expert_stride & 3u);
    // Each expert's 32-row tiles are split over enough workgroups that the
    // experts together fill the CUs once (one workgroup per CU fits).
    const uint32_t tiles = (p->n + kMoeTile - 1) / kMoeTile;
    const uint32_t splits = std::max(1u, std::min(tiles, ((uint32_t)kCUs + p->n_experts - 1) / p->n_experts));
    if (n_routed <= (uint64_t)kFusedMaxRows && (uint64_t)p->n_tokens * p->k * 4u < (1ull << 31)) {
        // One launch: grouping and the binary16 copy of x inside the GEMM.
        uint32_t* bad = reinterpret_cast<uint32_t*>((uint8_t*)scratch + lay.bad_ids);
        hipLaunchKernelGGL(realign ? moe_fused_kernel<true> : moe_fused_kernel<false>, dim3(p->n_experts * splits),
                           dim3(kMoeThreads), 0, s, x, w, ids, out, bad, (int)p->n, (int)p->k, (int)p->top_k,
                           (int)n_routed, (int)p->n_experts, p->expert_stride, (int)p->n_tokens, (int)splits, events);
        return launch_status("qmm_id_q4_0 (one-launch grouped GEMM)");
    }
    const int n_rows = (int)(p->n_tokens * p->top_k);
    const int64_t x_count = (int64_t)p->n_tokens * p->k;
    const int conv_blocks = (int)std::min<int64_t>(1024, (x_count / 8 + kGroupThreads - 1) / kGroupThreads);
    hipLaunchKernelGGL(moe_group_kernel, dim3(1 + conv_blocks), dim3(kGroupThreads), p->n_experts * sizeof(uint32_t), s,
                       ids, x, (uint8_t*)scratch, out, n_rows, (int)p->n_experts, (int)p->n, x_count, lay, events);
    st = launch_status("qmm_id_q4_0 (group)");
    if (st != W4_OK) return st;
    hipLaunchKernelGGL(realign ? moe_gemm_kernel<true> : moe_gemm_kernel<false>, dim3(p->n_experts * splits),
                       dim3(kMoeThreads), 0, s, w, (const uint8_t*)scratch, out, (int)p->n, (int)p->k, (int)p->top_k,
                       p->expert_stride, lay, (int)p->n_tokens, (int)splits);
    return launch_status("qmm_id_q4_0 (grouped GEMM)");
}

// ---------------------------------------------------------------- no-allocation variant
// qmm_id_q4_0 for callers that cannot allocate: the grouping scratch is this
// file-scope device array instead of a caller buffer. Each GPU the library
// runs on holds its own copy until the process ends; calls that overlap on
// one GPU share it and race.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace w4mi {
namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<uint8_t*> g_scratch_ptr[kMaxScratchDevices];

// The array's device address on the current device (the name itself is a
// host-side stand-in), looked up once per device.
w4_status noalloc_scratch(uint8_t** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
        return fail(W4_ELAUNCH, "qmm_id_q4_0_noalloc: no usable current device");
    uint8_t* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        void* a = nullptr;
        const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !a)
            return fail(W4_ELAUNCH, "qmm_id_q4_0_noalloc: cannot locate the library scratch: %s", hipGetErrorString(e));
        ptr = static_cast<uint8_t*>(a);
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    *out = ptr;
    return W4_OK;
}
}  // namespace
}  // namespace w4mi

extern "C" w4_status qmm_id_q4_0_noalloc(const float* x, const uint8_t* w, const uint32_t* ids, float* out,
                                         const w4_id_params* p, uint32_t* bad_ids, void* stream) {
    // Validate everything but the scratch first (host only), then the size.
    w4_status st = w4_check_id(p, SIZE_MAX);
    if (st != W4_OK) return st;
    const size_t need = id_scratch_layout(p->n_experts, p->n_tokens, p->top_k, p->k).total;
    if (need > kNoAllocScratchBytes)
        return fail(W4_EUNSUPPORTED,
                    "qmm_id_q4_0_noalloc: the shapes need %zu bytes of scratch; the library's fixed scratch holds %zu "
                    "(use qmm_id_q4_0 with a caller buffer)",
                    need, kNoAllocScratchBytes);
    if (((uintptr_t)bad_ids & 3u)) return fail(W4_EINVAL, "qmm_id_q4_0_noalloc: bad_ids must be 4-byte aligned");
    uint8_t* ptr = nullptr;
    st = noalloc_scratch(&ptr);
    if (st != W4_OK) return st;
    st = qmm_id_q4_0(x, w, ids, out, p, ptr, kNoAllocScratchBytes, stream);
    if (st != W4_OK || !bad_ids) return st;
    const hipError_t e = hipMemcpyAsync(bad_ids, ptr + W4_ID_SCRATCH_BAD_IDS, sizeof(uint32_t),
                                        hipMemcpyDeviceToDevice, as_stream(stream));
    if (e != hipSuccess) return fail(W4_ELAUNCH, "qmm_id_q4_0_noalloc: copying the bad-id count: %s", hipGetErrorString(e));
    return W4_OK;
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
    uint32_t* events = nullptr;
    st = range_counter(&events, "qmm_id_swiglu_q4_0");
    if (st != W4_OK) return st;
    mv_launch<true>(gate, up, w, ids, out, bad_ids, p, as_stream(stream), events);
    return launch_status("qmm_id_swiglu_q4_0");
}
