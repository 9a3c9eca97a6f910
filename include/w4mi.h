/*
 * w4mi - weight-only 4-bit dequantize-and-multiply, y = x . dequant(W)^T,
 * for AMD Instinct MI355X (gfx950).
 *
 * C ABI. Every pointer argument named as "device" is a device pointer the
 * caller owns (a hipMalloc'd buffer, e.g. a torch-ROCm tensor's data_ptr);
 * "host" pointers are read during the call only. All tensors are dense and
 * row-major. Every entry point validates its arguments on the host before it
 * touches the GPU (shapes, alignment, and for the expert-routed calls the
 * byte length of every buffer; the affine and lookup calls take no buffer
 * lengths, so each buffer must hold what its stated shape needs - the Python
 * binding checks tensor shapes before calling), enqueues its kernels on
 * `stream` (a hipStream_t; NULL is
 * the default stream) and returns without synchronising; the library never
 * allocates device memory. Apart from w4_range_events (which synchronises),
 * a call enqueues only kernel launches (qmm_id_q4_0_noalloc also one
 * device-to-device copy), so it may be recorded into a HIP graph by stream
 * capture and replayed: each replay rewrites every output (the range-event
 * count of w4_range_events goes on adding up). The first call on
 * a device looks up the library's device variables (hipGetSymbolAddress):
 * make one call per device before capturing. On failure nothing is enqueued (W4_EINVAL,
 * W4_EUNSUPPORTED) or the launch error is reported (W4_ELAUNCH); the message
 * is available from w4_last_error() on the calling thread. There is no
 * fallback path: a status other than W4_OK means no result was produced.
 *
 * Sources of each operation:
 *   [P1] onnxruntime-ep-mlx 0.27.4, src/ops/quant_fastkernel.rs: INT4
 *        group-32 affine MatMulNBits (module doc "Algorithm", the kernel's
 *        W load, `eligible`, the tests' make_case);
 *   [P2] onnxruntime-ep-mlx 0.31.1, src/ops/lut4.rs: frozen 16-entry lookup
 *        decode (LookupMatMul, the decode kernel, rounded_weight, execute);
 *   [P3] mlx-native 0.9.0, src/ops/quantized_matmul_id_ggml.rs:
 *        expert-routed GGML block matmul (module doc,
 *        quantized_matmul_id_ggml validation, IdMmScratch, the map0 + mm
 *        two-stage dispatch).
 */
#ifndef W4MI_H
#define W4MI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4_OK = 0,
    W4_EINVAL = 1,       /* an argument violates the operation's contract */
    W4_EUNSUPPORTED = 2, /* a valid request this library does not implement */
    W4_ELAUNCH = 3       /* the HIP runtime rejected a launch */
} w4_status;

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* w4_last_error(void);

/* Library version string. */
const char* w4_version(void);

/* ------------------------------------------------------------------------
 * Affine INT4, group size 32 [P1].
 *
 * w       device uint32 [N, K/8]: the weight at (n, k) is nibble k % 8 of
 *         word (n, k / 8), least significant nibble first (bits 4j..4j+3).
 * scales  device bf16 bits [N, K/32]; biases device bf16 bits [N, K/32],
 *         bias = -zero_point * scale. Weight w[n][k] = q * scale + bias of
 *         group k / 32.
 * x       device bf16 bits [M, K]; y device bf16 bits [M, N] (written).
 * Contract: bits == 4, group_size == 32, K % 32 == 0, N % 32 == 0, K > 0,
 * N > 0 ([P1] `eligible`). M == 0 is a no-op. Accumulation is f32; y is the
 * round-to-nearest-even bf16 of the accumulator.
 *
 * qmm_affine4 is the prefill form and requires M > 1 ([P1] `eligible`:
 * the kernel is only used for M > 1). qmv_affine4 is the decode GEMV and
 * requires M == 1 ([P1]: single-row decode takes the library qmv path).
 * This library implements qmm_affine4 for K and N up to 2^21 (2,097,152);
 * larger valid shapes return W4_EUNSUPPORTED.
 *
 * Operand precision. qmv_affine4, and qmm_affine4 with K <= 8192 and either
 * at most 4 rows (K <= 4096) or 2 rows (K > 4096), or, when K % 256 != 0 or
 * the scales or biases are not 4-byte aligned, at most 16 rows, multiply the
 * bf16 x by the exact nibbles and apply scale and bias per group in f32: no
 * range limit beyond f32's. Every other qmm_affine4 shape runs on the matrix cores in binary16,
 * as [P1]'s kernel does (module doc "Algorithm"): x is converted bf16 ->
 * binary16 (round to nearest even; exact for magnitudes 2^-14 .. 65504,
 * binary16's subnormal step below) and each weight is q * scale + bias
 * rounded once to binary16 (exactly so when bias = 0 or |bias| lies within
 * 2^-6 .. 2^15 of |scale|, as it does for bias = -zero_point * scale;
 * outside that band an f32 step can round first, by at most 2^-14 |scale|
 * below it and 2^-22 |bias| above it).
 * A finite x (or weight) of magnitude 65520 or
 * more overflows binary16: the outputs of its row of x (or weight row) come
 * out as infinities or NaN, and the call adds one per affected output tile
 * to the device's range-event count (w4_range_events). Infinite or NaN
 * inputs propagate as in the definition and are not counted.
 * ---------------------------------------------------------------------- */
w4_status qmm_affine4(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                      const uint16_t* x, uint16_t* y, int64_t M, int64_t K, int64_t N,
                      int32_t group_size, int32_t bits, void* stream);

w4_status qmv_affine4(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                      const uint16_t* x, uint16_t* y, int64_t M, int64_t K, int64_t N,
                      int32_t group_size, int32_t bits, void* stream);

/* Operand range events on the CURRENT device (each GPU counts its own):
 * events since the last reset in which a finite value had to be rounded to
 * binary16 and could not be held (magnitude 65520 or more, which becomes an
 * infinity): qmm_affine4's matrix-core routes add one per output tile whose
 * x or weights held such a value (see "Operand precision" above);
 * qmm_id_q4_0 and qmm_id_swiglu_q4_0 add one per wavefront that rounded such
 * an activation (x, or silu(gate) * up). Zero means no call since the reset
 * met one. *count (host) receives the count; reset != 0 then clears it. The
 * call synchronises the device first, so it covers every call enqueued
 * before it. */
w4_status w4_range_events(uint32_t* count, int32_t reset);

/* ------------------------------------------------------------------------
 * Lookup-codebook 4-bit matmul [P2], half-precision path.
 *
 * The decoded weight is the [rows, cols] matrix with flat index i: its code
 * is the HIGH nibble of packed[i / 2] when i is even and the LOW nibble when
 * i is odd, and value(i) = fp16(book[code] * scale[i / block]) (the product
 * in f32, rounded to binary16 because the graph casts the decoded weight to
 * half before the MatMul). With transpose != 0 the weight is [N, K]
 * (rows = N, cols = K) and y = x . W^T.
 *
 * x       device fp16 bits [M, K]; y device fp16 bits [M, N] (written).
 * packed  device uint8 [ceil(N*K/block) * block / 2].
 * scales  device fp16 bits [ceil(N*K/block)].
 * book    HOST pointer to 16 f32 codebook values (copied at the call).
 * Contract: M >= 0, K > 0, N > 0, block > 0 and even ([P2] recognize).
 * This library implements transpose != 0 with K % 32 == 0, K % block == 0 and
 * block % 8 == 0 (matrix cores; x 16-byte and packed 4-byte aligned), and
 * transpose == 0 for any K and N with M up to 262,140: on the matrix cores
 * from M = 128 (the page's decoded-weight threshold) when K % 64 == 0,
 * N % 8 == 0, block is a power of two of at least 8, N * K < 2^32, x is
 * 16-byte and packed 4-byte aligned; otherwise on the vector ALU (K tiles
 * added with compensation). Other valid requests return W4_EUNSUPPORTED.
 * M == 0 is a no-op. Accumulation is f32; y is the round-to-nearest-even fp16
 * of it.
 * ---------------------------------------------------------------------- */
w4_status qmm_lut4(const uint16_t* x, const uint8_t* packed, const uint16_t* scales,
                   const float* book, uint16_t* y, int64_t M, int64_t K, int64_t N,
                   int32_t block, int32_t transpose, void* stream);

/* ------------------------------------------------------------------------
 * Lookup-codebook 4-bit matmul [P2], single-precision path (the page's
 * mlx_lookup4_matmul kernel and CPU branch, taken when the compute type is
 * f32: the decoded weight is not rounded).
 *
 *   y[m][n] = sum_k x[m][k] * W(n, k),  W = book[code(flat)] * scale[flat / block]
 *   (the product in f32), flat = n*K + k when transpose != 0 (W stored [N, K]),
 *   k*N + n when transpose == 0 (W stored [K, N]); code(flat) is the HIGH
 *   nibble of packed[flat / 2] for even flat, the LOW nibble for odd.
 *
 * x       device f32 [M, K]; y device f32 [M, N] (written).
 * packed  device uint8 [ceil(N*K/2)]; scales device f32 [ceil(N*K/block)].
 * book    HOST pointer to 16 f32 codebook values (copied at the call).
 * Blocks run over the flat index and may straddle rows. Products are summed
 * in K tiles whose partial sums are added with compensation ([P2] kernel's
 * correction term). Contract as qmm_lut4 (M >= 0, K > 0, N > 0, block > 0 and
 * even), both layouts, any K and N; M up to 262,140. M == 0 is a no-op.
 * ---------------------------------------------------------------------- */
w4_status qmm_lut4_f32(const float* x, const uint8_t* packed, const float* scales, const float* book, float* y,
                       int64_t M, int64_t K, int64_t N, int32_t block, int32_t transpose, void* stream);

/* ------------------------------------------------------------------------
 * Expert-routed matmul over GGML Q4_0 blocks [P3].
 *
 * For every routed row r = token * top_k + slot, e = ids[r] and
 *   out[r][n] = sum_k dequant(W[e][n][k]) * x[token][k].
 * A Q4_0 block holds 32 consecutive k of one weight row in 18 bytes: a
 * little-endian binary16 scale d, then 16 bytes qs; element i < 16 is the
 * low nibble of qs[i], element i + 16 its high nibble; value = (q - 8) * d.
 * Expert e's [N, K/32] blocks start at byte e * expert_stride of w.
 *
 * x       device f32 [n_tokens, K] (one row per token, shared by its slots).
 * w       device bytes, at least n_experts * N * (K/32) * 18 long.
 * ids     device uint32 [n_tokens * top_k].
 * out     device f32 [n_tokens * top_k, N] (written).
 * scratch device buffer of at least qmm_id_q4_0_scratch_bytes(...) bytes,
 *         256-byte aligned; its contents need no initialisation. Calls that
 *         share one scratch buffer must be ordered (same stream).
 * Routes ([P3] MM_ID_ROUTING_THRESHOLD = 32 and dispatch_id_mv / dispatch_id_mm):
 *   - n_tokens <= 32 (with n_tokens * top_k <= 256 and K <= 8192): one
 *     mat-vec launch; each selected expert's weights are read once and
 *     applied to every routed row that selects it. Scratch holds only the
 *     bad-id count.
 *   - otherwise a grouped matrix-core GEMM ([P3] map0 + mm): up to 4096
 *     routed rows in one launch, whose workgroups each list their expert's
 *     routed rows and round x to binary16 themselves (scratch holds only the
 *     bad-id count); above that, the routed rows are first grouped by
 *     expert into scratch, with x stored there as binary16 (caller-owned
 *     scratch as in IdMmScratch).
 * Both routes round x to binary16 (round to nearest even) before the
 * products: a finite |x| of 65520 or more becomes an infinity (its routed
 * rows' outputs are not finite) and is counted by w4_range_events;
 * accumulation is f32.
 * Contract ([P3] quantized_matmul_id_ggml): n_tokens, K, N, top_k and
 * n_experts > 0; K % 32 == 0; expert_stride >= N * (K/32) * 18; each byte
 * length in p at least what the shapes need. Ids must be < n_experts: a row
 * whose id is not is written as zeros, and the number of such rows is left
 * as a uint32 at byte offset W4_ID_SCRATCH_BAD_IDS of scratch.
 * x must be 16-byte aligned, w and expert_stride 2-byte aligned. This
 * library implements the grouped route for n_tokens * K * 2 < 2^32 and
 * 384 * (K/32) * 18 < 2^31; other valid requests that need it return
 * W4_EUNSUPPORTED.
 * ---------------------------------------------------------------------- */
typedef struct {
    uint32_t n_tokens;      /* input tokens */
    uint32_t top_k;         /* experts per token */
    uint32_t n;             /* output columns = weight rows per expert */
    uint32_t k;             /* reduction length, multiple of 32 */
    uint32_t n_experts;     /* experts in the stacked weight buffer */
    uint32_t reserved;      /* must be 0 */
    uint64_t expert_stride; /* bytes between consecutive experts' weights */
    uint64_t x_bytes;       /* byte length of x */
    uint64_t w_bytes;       /* byte length of w */
    uint64_t ids_bytes;     /* byte length of ids */
    uint64_t out_bytes;     /* byte length of out */
} w4_id_params;

#define W4_ID_SCRATCH_BAD_IDS 0

/* Scratch bytes qmm_id_q4_0 needs: the per-expert row grouping and a copy of
 * x in the matrix-core operand type (binary16). */
size_t qmm_id_q4_0_scratch_bytes(uint32_t n_experts, uint32_t n_tokens, uint32_t top_k, uint32_t k);

w4_status qmm_id_q4_0(const float* x, const uint8_t* w, const uint32_t* ids, float* out,
                      const w4_id_params* p, void* scratch, size_t scratch_bytes, void* stream);

/* qmm_id_q4_0 for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops, harnesses that forbid hipMalloc): the
 * same operation, routes, kernels, contract and results, with the scratch
 * taken from a fixed 4 MiB device array the library holds on each GPU it
 * runs on (until the process ends) instead of a caller buffer. The call
 * allocates nothing and makes no allocating library call. Requests whose
 * scratch (qmm_id_q4_0_scratch_bytes) exceeds 4 MiB return W4_EUNSUPPORTED
 * before any device work. bad_ids (device uint32, optional, NULL: not
 * reported) receives the out-of-range id count, copied on `stream`. Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams, or threads without ordering) race and must not be
 * issued; calls ordered on one stream are safe. */
w4_status qmm_id_q4_0_noalloc(const float* x, const uint8_t* w, const uint32_t* ids, float* out,
                              const w4_id_params* p, uint32_t* bad_ids, void* stream);

/* ------------------------------------------------------------------------
 * Fused SwiGLU + expert-routed Q4_0 mat-vec [P3] (quantized_matmul_id_swiglu_q4_0):
 * for every routed row r = t*top_k + s, e = ids[r] and
 *   out[r][n] = sum_k dequant(W[e][n][k]) * silu(gate[r][k]) * up[r][k],
 * silu(g) = g / (1 + exp(-g)). gate and up are per ROUTED ROW (the outputs of
 * that row's expert projections), not per token.
 *
 * gate, up  device f32 [n_tokens * top_k, K], 16-byte aligned; p->x_bytes is
 *           the byte length of each.
 * w, ids, out, p  as for qmm_id_q4_0 (same Q4_0 layout and params struct).
 * bad_ids   optional device uint32 (NULL: not reported) that receives the
 *           number of routed rows whose id is not < n_experts; those rows are
 *           written as zeros.
 * One launch, no scratch: each selected expert's weights are read once and
 * applied to every routed row that selects it. The activation is formed in
 * f32 and rounded to binary16 (round to nearest even) before the products;
 * a finite activation of magnitude 65520 or more becomes an infinity and is
 * counted by w4_range_events; accumulation is f32.
 * Contract ([P3]): n_tokens, K, N, top_k, n_experts > 0; K % 32 == 0;
 * expert_stride >= N * (K/32) * 18; byte lengths at least what the shapes
 * need. This library implements n_tokens * top_k <= 256 and K <= 8192 (the
 * page's decode use); larger valid requests return W4_EUNSUPPORTED.
 * ---------------------------------------------------------------------- */
w4_status qmm_id_swiglu_q4_0(const float* gate, const float* up, const uint8_t* w, const uint32_t* ids,
                             float* out, const w4_id_params* p, uint32_t* bad_ids, void* stream);

/* ------------------------------------------------------------------------
 * Host-only argument checks: the exact validation the entry points above
 * run before launching (no device access; callable without a GPU).
 * decode != 0 checks the qmv_affine4 contract, else qmm_affine4's.
 * ---------------------------------------------------------------------- */
w4_status w4_check_affine(int64_t M, int64_t K, int64_t N, int32_t group_size, int32_t bits,
                          int32_t decode);
w4_status w4_check_lut(int64_t M, int64_t K, int64_t N, int32_t block, int32_t transpose);
w4_status w4_check_lut_f32(int64_t M, int64_t K, int64_t N, int32_t block, int32_t transpose);
w4_status w4_check_id(const w4_id_params* p, size_t scratch_bytes);
w4_status w4_check_id_swiglu(const w4_id_params* p);

/* ------------------------------------------------------------------------
 * Unpack exports: the codes the hot kernels decode, written out one byte
 * per weight by the same device decode routines the kernels use, so that a
 * caller can check them bit for bit. Where the kernels decode one format
 * with several routines, every one of them is applied and a weight on which
 * they disagree is written as 0xFF. All pointers are device pointers.
 *   w4_unpack_affine: q [N, K] from w [N, K/8] ([P1] nibble order): the
 *                     nibble extraction, the GEMV's biased bf16 pairs and the
 *                     matrix-core kernels' binary16 word decode.
 *   w4_unpack_lut:    codes [count] from packed ([P2] high nibble first):
 *                     the per-element code, the matrix-core byte-plane table
 *                     decode and the single-precision path's dword lookup.
 *   w4_unpack_q4_0:   q [rows, K] codes and d [rows, K/32] binary16 bits
 *                     from `rows` consecutive Q4_0 weight rows.
 * ---------------------------------------------------------------------- */
w4_status w4_unpack_affine(const uint32_t* w, uint8_t* q, int64_t N, int64_t K, void* stream);
w4_status w4_unpack_lut(const uint8_t* packed, uint8_t* codes, int64_t count, void* stream);
w4_status w4_unpack_q4_0(const uint8_t* w, uint8_t* q, uint16_t* d, int64_t rows, int64_t K,
                         void* stream);

/* ------------------------------------------------------------------------
 * Measurement entry points: achievable ceilings of this GPU, for reporting
 * the kernels above against measured limits as well as published peaks.
 *   w4_ceiling_stream_read: reads `bytes` (a multiple of 16) of the 16-byte
 *       aligned device buffer `buf` once, with 16-byte non-temporal loads,
 *       each workgroup streaming one contiguous chunk (up to 1024 workgroups
 *       of 512 lanes, four loads per lane in flight); bytes / time is the
 *       streaming-read rate. `sink` is a device uint32 [1024] the kernel may
 *       write: a lane whose pieces fold (XOR of all their dwords) to
 *       0x9E3779B9 writes that value to one word, so the loads are live.
 *   w4_ceiling_mfma: every SIMD issues `iters` x 4 back-to-back
 *       v_mfma_f32_32x32x16_f16 (32,768 flop each) on 2 x 256 workgroups of 4
 *       wavefronts (no memory traffic): 2 * 256 * 4 * 4 * iters * 32768 flop.
 * Both are asynchronous on `stream` and return W4_EINVAL on bad arguments.
 * ---------------------------------------------------------------------- */
w4_status w4_ceiling_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, void* stream);
w4_status w4_ceiling_mfma(uint32_t* sink, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4MI_H */
