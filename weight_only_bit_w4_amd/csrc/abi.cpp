// Host-side part of the C ABI: error reporting and the argument contracts
// each entry point checks before it enqueues work.
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "w4mi_host.hpp"

namespace w4mi {

static thread_local std::string g_error;

w4_status fail(w4_status status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return status;
}

void clear_error() { g_error.clear(); }

w4_status launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(W4_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    clear_error();
    return W4_OK;
}

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

IdScratchLayout id_scratch_layout(uint32_t n_experts, uint32_t n_tokens, uint32_t top_k, uint32_t k) {
    IdScratchLayout l;
    size_t off = 0;
    l.bad_ids = off;
    off = align_up(off + 4, 256);
    l.counts = off;
    off = align_up(off + 4ull * n_experts, 256);
    l.offsets = off;
    off = align_up(off + 4ull * (n_experts + 1ull), 256);
    l.rows = off;
    off = align_up(off + 4ull * n_tokens * top_k, 256);
    l.xh = off;
    off = align_up(off + 2ull * n_tokens * k, 256);
    l.total = off;
    return l;
}

}  // namespace w4mi

using namespace w4mi;

extern "C" {

const char* w4_last_error(void) { return g_error.c_str(); }

const char* w4_version(void) { return "w4mi 0.1 (gfx950)"; }

// INT4 MatMulNBits page, `eligible`: bits 4, group size 32, M > 1 for the
// prefill kernel, K and N multiples of 32; single-row decode is the GEMV.
w4_status w4_check_affine(int64_t M, int64_t K, int64_t N, int32_t group_size, int32_t bits,
                          int32_t decode) {
    const char* fn = decode ? "qmv_affine4" : "qmm_affine4";
    if (bits != 4) return fail(W4_EINVAL, "%s: bits must be 4, got %d", fn, bits);
    if (group_size != 32) return fail(W4_EINVAL, "%s: group_size must be 32, got %d", fn, group_size);
    if (M < 0 || K <= 0 || N <= 0)
        return fail(W4_EINVAL, "%s: need M >= 0 and K, N > 0 (M=%lld K=%lld N=%lld)", fn, (long long)M,
                    (long long)K, (long long)N);
    if (K % 32 != 0) return fail(W4_EINVAL, "%s: K (%lld) must be a multiple of 32", fn, (long long)K);
    if (N % 32 != 0) return fail(W4_EINVAL, "%s: N (%lld) must be a multiple of 32", fn, (long long)N);
    if (M > INT32_MAX || K > INT32_MAX || N > INT32_MAX)
        return fail(W4_EINVAL, "%s: each dimension must fit in int32", fn);
    if (decode && M > 1) return fail(W4_EINVAL, "%s: the decode GEMV takes M == 1, got %lld", fn, (long long)M);
    if (!decode && M == 1)
        return fail(W4_EINVAL, "%s: the prefill GEMM takes M > 1; use qmv_affine4 for M == 1", fn);
    clear_error();
    return W4_OK;
}

// lut4 page, recognize/execute: block positive and even; K and N positive; M
// flattened. This library runs the transposed layout with whole blocks per
// row segment of 8.
w4_status w4_check_lut(int64_t M, int64_t K, int64_t N, int32_t block, int32_t transpose) {
    if (M < 0 || K <= 0 || N <= 0)
        return fail(W4_EINVAL, "qmm_lut4: need M >= 0 and K, N > 0 (M=%lld K=%lld N=%lld)", (long long)M,
                    (long long)K, (long long)N);
    if (block <= 0 || block % 2 != 0) return fail(W4_EINVAL, "qmm_lut4: block must be positive and even, got %d", block);
    if (M > INT32_MAX || K > INT32_MAX || N > INT32_MAX || N * K > (int64_t)1 << 40)
        return fail(W4_EINVAL, "qmm_lut4: dimensions too large");
    if (!transpose) {
        // [K, N]: any K, N and even block; rows of x go 4 per workgroup (grid y).
        if (M > 4ll * 65535)
            return fail(W4_EUNSUPPORTED, "qmm_lut4: the [K, N] layout is implemented for M up to 262140, got %lld",
                        (long long)M);
        clear_error();
        return W4_OK;
    }
    if (K % 32 != 0 || K % block != 0 || block % 8 != 0)
        return fail(W4_EUNSUPPORTED, "qmm_lut4: implemented for K %% 32 == 0, K %% block == 0, block %% 8 == 0 "
                                     "(K=%lld block=%d)", (long long)K, block);
    clear_error();
    return W4_OK;
}

// lut4 page, single-precision path: the same contract as qmm_lut4 (recognize:
// block positive and even; execute: M, K, N sizes), both weight layouts, any
// K and N, blocks over the flat index.
w4_status w4_check_lut_f32(int64_t M, int64_t K, int64_t N, int32_t block, int32_t transpose) {
    (void)transpose;
    if (M < 0 || K <= 0 || N <= 0)
        return fail(W4_EINVAL, "qmm_lut4_f32: need M >= 0 and K, N > 0 (M=%lld K=%lld N=%lld)", (long long)M,
                    (long long)K, (long long)N);
    if (block <= 0 || block % 2 != 0)
        return fail(W4_EINVAL, "qmm_lut4_f32: block must be positive and even, got %d", block);
    if (M > INT32_MAX || K > INT32_MAX || N > INT32_MAX || N * K > (int64_t)1 << 40)
        return fail(W4_EINVAL, "qmm_lut4_f32: dimensions too large");
    if (M > 4ll * 65535)
        return fail(W4_EUNSUPPORTED, "qmm_lut4_f32: implemented for M up to 262140, got %lld", (long long)M);
    clear_error();
    return W4_OK;
}

// Shared validation of the expert-routed calls (mlx-native MoE page,
// quantized_matmul_id_ggml: the contraction's sizes must be positive, K whole
// Q4_0 blocks, the expert stride at least one expert's blocks, and every
// buffer long enough for the shapes). `act_rows` is the number of activation
// rows the call reads: one per token for qmm_id_q4_0, one per routed row for
// the fused SwiGLU form (gate and up each).
static w4_status check_routed(const char* fn, const w4_id_params* p, uint64_t act_rows_per_token, const char* act_name) {
    if (!p) return fail(W4_EINVAL, "%s: no parameter block given", fn);
    if (!p->n_tokens || !p->top_k || !p->n || !p->k || !p->n_experts)
        return fail(W4_EINVAL, "%s: every size must be positive (n_tokens=%u top_k=%u n=%u k=%u n_experts=%u)", fn,
                    p->n_tokens, p->top_k, p->n, p->k, p->n_experts);
    if (p->reserved) return fail(W4_EINVAL, "%s: the reserved field is %u, not 0", fn, p->reserved);
    if (p->k % 32) return fail(W4_EINVAL, "%s: k=%u is not a whole number of 32-weight Q4_0 blocks", fn, p->k);
    const uint64_t routed = (uint64_t)p->n_tokens * p->top_k;
    if (routed > INT32_MAX) return fail(W4_EINVAL, "%s: %llu routed rows exceed int32", fn, (unsigned long long)routed);
    const uint64_t expert_bytes = (uint64_t)p->n * (p->k / 32) * 18u;
    if (p->expert_stride < expert_bytes)
        return fail(W4_EINVAL, "%s: experts are %llu bytes apart but each holds %llu bytes of blocks", fn,
                    (unsigned long long)p->expert_stride, (unsigned long long)expert_bytes);
    struct {
        const char* buffer;
        uint64_t have, need;
    } const lengths[] = {
        {act_name, p->x_bytes, (uint64_t)p->n_tokens * act_rows_per_token * p->k * 4u},
        {"w", p->w_bytes, (uint64_t)(p->n_experts - 1) * p->expert_stride + expert_bytes},
        {"ids", p->ids_bytes, routed * 4u},
        {"out", p->out_bytes, routed * p->n * 4u},
    };
    for (const auto& l : lengths)
        if (l.have < l.need)
            return fail(W4_EINVAL, "%s: %s holds %llu bytes; the shapes need %llu", fn, l.buffer,
                        (unsigned long long)l.have, (unsigned long long)l.need);
    return W4_OK;
}

w4_status w4_check_id(const w4_id_params* p, size_t scratch_bytes) {
    w4_status st = check_routed("qmm_id_q4_0", p, 1, "x");
    if (st != W4_OK) return st;
    if (p->n_experts > kMaxExperts)
        return fail(W4_EUNSUPPORTED, "qmm_id_q4_0: this library groups at most %u experts (asked for %u)", kMaxExperts,
                    p->n_experts);
    const size_t need_s = id_scratch_layout(p->n_experts, p->n_tokens, p->top_k, p->k).total;
    if (scratch_bytes < need_s)
        return fail(W4_EINVAL, "qmm_id_q4_0: scratch holds %zu bytes; the shapes need %zu", scratch_bytes, need_s);
    clear_error();
    return W4_OK;
}

w4_status w4_check_id_swiglu(const w4_id_params* p) {
    w4_status st = check_routed("qmm_id_swiglu_q4_0", p, p ? p->top_k : 0, "gate/up");
    if (st != W4_OK) return st;
    clear_error();
    return W4_OK;
}

size_t qmm_id_q4_0_scratch_bytes(uint32_t n_experts, uint32_t n_tokens, uint32_t top_k, uint32_t k) {
    return id_scratch_layout(n_experts, n_tokens, top_k, k).total;
}

}  // extern "C"
