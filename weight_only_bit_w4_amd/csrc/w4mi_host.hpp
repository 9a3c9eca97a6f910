// Host-side helpers shared by the w4mi entry points: the per-thread error
// message and the launch-status check.
#pragma once

#include <hip/hip_runtime.h>

#include "w4mi.h"

namespace w4mi {

constexpr int kCUs = 256;  // compute units of the MI355X (launch shapes that fill the chip once)

// Records a formatted message for w4_last_error() and returns `status`.
w4_status fail(w4_status status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the thread's message (called on success paths).
void clear_error();

// Checks the HIP runtime's launch status after enqueuing `what`.
w4_status launch_status(const char* what);

// Device address of the current device's operand-range event counter
// (w4_range_events), looked up once per device.
w4_status range_counter(uint32_t** out, const char* fn);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Internal layout of the expert-routed scratch buffer (see qmm_id_q4_0).
struct IdScratchLayout {
    size_t bad_ids;   // uint32 count of rows with an out-of-range id
    size_t counts;    // uint32 [n_experts] routed rows per expert
    size_t offsets;   // uint32 [n_experts + 1] exclusive prefix of counts
    size_t rows;      // uint32 [n_tokens * top_k] routed rows grouped by expert
    size_t xh;        // binary16 [n_tokens, k] activations in the MFMA operand type
    size_t total;
};
IdScratchLayout id_scratch_layout(uint32_t n_experts, uint32_t n_tokens, uint32_t top_k, uint32_t k);

// Affine INT4 GEMV form with x shared per workgroup (affine_gemv.hip), for
// 1 <= M <= kAffineBatchRows rows of x and K <= kAffineBatchMaxK (N % 16 == 0):
// every weight row is read once and applied to all M rows.
constexpr int kAffineBatchRows = 16;
constexpr int64_t kAffineBatchMaxK = 8192;
void launch_xlds(const uint32_t* w, const uint16_t* scales, const uint16_t* biases, const uint16_t* x, uint16_t* y,
                 int M, int K, int N, hipStream_t s);
// Rows of x the GEMV form applies per pass over its registers' weights (1, 2
// or 4); M rows take ceil(M / that) passes, each repeating the decode.
int xlds_batch_rows(int M, int K);

// Half-precision lookup matmul with the weight stored [K, N] (lut_f32.hip),
// any K, N and even block, M up to 4 * 65535.
void launch_lut4_kn_f16(const uint16_t* x, const uint8_t* packed, const uint16_t* scales, const float* book, uint16_t* y,
                        int64_t M, int64_t K, int64_t N, int32_t block, hipStream_t s);

// Largest expert count the grouping kernel keeps in its LDS histogram.
constexpr uint32_t kMaxExperts = 8192;

}  // namespace w4mi
