// C ABI of librudder: argument validation, error reporting and dispatch to
// the kernel launchers.  Nothing is launched unless every check passes.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "rudder_internal.h"

namespace {

thread_local std::string g_last_error;

rudder_status_t fail(rudder_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

rudder_status_t fail(rudder_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

bool misaligned(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u); }

rudder_status_t ok() {
    g_last_error.clear();
    return RUDDER_OK;
}

rudder_status_t from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(RUDDER_ERR_HIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

size_t rudder_packed_weight_bytes(int K, int N, int codes) {
    if (K <= 0 || N <= 0 || K % 32 || N % 32) return 0;
    if (codes == RUDDER_CODES_INT) return (size_t)N * (size_t)K / 2;
    if (codes == RUDDER_CODES_E2M3 && K % 64 == 0) return (size_t)N * (size_t)K * 3 / 4;
    return 0;
}

size_t rudder_packed_act_bytes(int M, int K, int abits, int codes) {
    if (M < 0 || K <= 0 || K % 32 || (abits != 4 && abits != 8)) return 0;
    const size_t rows = (size_t)((M + 31) / 32) * 32;
    if (codes == RUDDER_CODES_INT) return rows * (size_t)K * (size_t)abits / 8;
    if (codes == RUDDER_CODES_E2M3 && K % 64 == 0)
        return rows * (size_t)K * 3 / 4 * (abits == 8 ? 2 : 1);
    return 0;
}

size_t rudder_quant_act_workspace_bytes(int S) {
    (void)S;
    return rudder::quant_act_workspace_bytes();
}

rudder_status_t rudder_quantize_weights(const uint16_t* W, const float* smooth, int K, int N,
                                        int codes, uint8_t* Wq, float* w_scale,
                                        float* inv_smooth, void* stream) {
    const char* f = "rudder_quantize_weights";
    if (!W || !smooth || !Wq || !w_scale || !inv_smooth)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: null pointer argument", f);
    if (K <= 0 || N <= 0)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: K=%d and N=%d must be positive", f, K, N);
    if (K % 32 || N % 32)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: K=%d and N=%d must be multiples of 32", f, K, N);
    if (codes != RUDDER_CODES_INT && codes != RUDDER_CODES_E2M3)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: unknown code container %d", f, codes);
    if (codes == RUDDER_CODES_E2M3 && K % 64)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: K=%d must be a multiple of 64 for E2M3 codes",
                    f, K);
    if (misaligned(Wq) || misaligned(smooth) || misaligned(w_scale) || misaligned(inv_smooth))
        return fail(RUDDER_ERR_INVALID_ARG, "%s: Wq, smooth, w_scale and inv_smooth must be "
                    "16-byte aligned", f);
    if (K > RUDDER_MAX_K)
        return fail(RUDDER_ERR_UNSUPPORTED, "%s: K=%d exceeds %d", f, K, RUDDER_MAX_K);
    return from_hip(rudder::launch_quantize_weights(W, smooth, K, N, codes, Wq, w_scale,
                                                    inv_smooth, static_cast<hipStream_t>(stream)),
                    f);
}

rudder_status_t rudder_quant_act(const uint16_t* X, const uint8_t* stream_id,
                                 const float* inv_smooth, const float* act_scale,
                                 float* act_scale_out, void* workspace, int M, int K, int S,
                                 int abits, int codes, void* Xq, float* row_scale,
                                 void* stream) {
    const char* f = "rudder_quant_act";
    if (!X || !stream_id || !inv_smooth || !Xq || !row_scale)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: null pointer argument", f);
    if (act_scale == nullptr && workspace == nullptr)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: dynamic mode (act_scale NULL) needs a workspace",
                    f);
    if (M < 0 || K <= 0)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: M=%d must be >= 0 and K=%d > 0", f, M, K);
    if (K % 32) return fail(RUDDER_ERR_INVALID_ARG, "%s: K=%d must be a multiple of 32", f, K);
    if (S < 1 || S > RUDDER_MAX_STREAMS)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: S=%d must be in 1..%d", f, S, RUDDER_MAX_STREAMS);
    if (abits != 4 && abits != 8)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: abits=%d must be 4 or 8", f, abits);
    if (codes != RUDDER_CODES_INT && codes != RUDDER_CODES_E2M3)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: unknown code container %d", f, codes);
    if (codes == RUDDER_CODES_E2M3 && K % 64)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: K=%d must be a multiple of 64 for E2M3 codes",
                    f, K);
    if (misaligned(X) || misaligned(inv_smooth) || misaligned(Xq) || misaligned(workspace))
        return fail(RUDDER_ERR_INVALID_ARG, "%s: X, inv_smooth, Xq and workspace must be "
                    "16-byte aligned", f);
    if (K > RUDDER_MAX_K)
        return fail(RUDDER_ERR_UNSUPPORTED, "%s: K=%d exceeds %d", f, K, RUDDER_MAX_K);
    if (M == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (act_scale != nullptr)
        return from_hip(rudder::launch_quant_act_static(X, stream_id, inv_smooth, act_scale, M, K,
                                                        S, abits, codes, Xq, row_scale, st),
                        f);
    return from_hip(rudder::launch_quant_act_dynamic(X, stream_id, inv_smooth, act_scale_out,
                                                     workspace, M, K, S, abits, codes, Xq,
                                                     row_scale, st),
                    f);
}

rudder_status_t rudder_quant_act_noalloc(const uint16_t* X, const uint8_t* stream_id,
                                         const float* inv_smooth, float* act_scale_out, int M,
                                         int K, int S, int abits, int codes, void* Xq,
                                         float* row_scale, void* stream) {
    const char* f = "rudder_quant_act_noalloc";
    if (!X || !stream_id || !inv_smooth || !Xq || !row_scale)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: null pointer argument", f);
    if (M < 0 || K <= 0)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: M=%d must be >= 0 and K=%d > 0", f, M, K);
    if (K % 32) return fail(RUDDER_ERR_INVALID_ARG, "%s: K=%d must be a multiple of 32", f, K);
    if (S < 1 || S > RUDDER_MAX_STREAMS)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: S=%d must be in 1..%d", f, S, RUDDER_MAX_STREAMS);
    if (abits != 4 && abits != 8)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: abits=%d must be 4 or 8", f, abits);
    if (codes != RUDDER_CODES_INT && codes != RUDDER_CODES_E2M3)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: unknown code container %d", f, codes);
    if (codes == RUDDER_CODES_E2M3 && K % 64)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: K=%d must be a multiple of 64 for E2M3 codes",
                    f, K);
    if (misaligned(X) || misaligned(inv_smooth) || misaligned(Xq))
        return fail(RUDDER_ERR_INVALID_ARG, "%s: X, inv_smooth and Xq must be 16-byte aligned",
                    f);
    if (K > RUDDER_MAX_K)
        return fail(RUDDER_ERR_UNSUPPORTED, "%s: K=%d exceeds %d", f, K, RUDDER_MAX_K);
    // the scratch holds the fixed-size dynamic-mode workspace, whatever M and K
    if (rudder::quant_act_workspace_bytes() > rudder::quant_act_noalloc_scratch_bytes())
        return fail(RUDDER_ERR_UNSUPPORTED, "%s: the workspace (%zu bytes) exceeds the scratch "
                    "(%zu bytes)", f, rudder::quant_act_workspace_bytes(),
                    rudder::quant_act_noalloc_scratch_bytes());
    if (M == 0) return ok();
    return from_hip(rudder::launch_quant_act_dynamic_noalloc(X, stream_id, inv_smooth,
                                                             act_scale_out, M, K, S, abits, codes,
                                                             Xq, row_scale,
                                                             static_cast<hipStream_t>(stream)),
                    f);
}

namespace {

// Checks shared by rudder_linear and rudder_linear_gelu_quant (the output
// pointers are checked by the callers).
rudder_status_t check_linear(const char* f, const void* Xq, const float* row_scale,
                             const uint8_t* stream_id, const uint8_t* Wq, const float* w_scale,
                             const float* comp_a, const float* comp_b, int M, int N, int K,
                             int S, int abits, int codes) {
    if (!Xq || !row_scale || !stream_id || !Wq || !w_scale || !comp_a || !comp_b)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: null pointer argument", f);
    if (M < 0 || N <= 0 || K <= 0)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: M=%d must be >= 0, N=%d and K=%d > 0", f, M, N,
                    K);
    if (N % 32) return fail(RUDDER_ERR_INVALID_ARG, "%s: N=%d must be a multiple of 32", f, N);
    if (S < 1 || S > RUDDER_MAX_STREAMS)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: S=%d must be in 1..%d", f, S, RUDDER_MAX_STREAMS);
    if (abits != 4 && abits != 8)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: abits=%d must be 4 or 8", f, abits);
    if (codes != RUDDER_CODES_INT && codes != RUDDER_CODES_E2M3)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: unknown code container %d", f, codes);
    if (misaligned(Xq) || misaligned(Wq) || misaligned(w_scale) || misaligned(comp_a) ||
        misaligned(comp_b))
        return fail(RUDDER_ERR_INVALID_ARG, "%s: Xq, Wq, w_scale, comp_a and comp_b must be "
                    "16-byte aligned", f);
    if (K % 128)
        return fail(RUDDER_ERR_UNSUPPORTED, "%s: K=%d is not a multiple of 128", f, K);
    if (K > RUDDER_MAX_K)
        return fail(RUDDER_ERR_UNSUPPORTED, "%s: K=%d exceeds %d", f, K, RUDDER_MAX_K);
    if (codes == RUDDER_CODES_E2M3 && abits == 8 && K > RUDDER_MAX_K_E2M3_A8)
        return fail(RUDDER_ERR_UNSUPPORTED, "%s: K=%d exceeds %d for 8-bit E2M3 codes", f, K,
                    RUDDER_MAX_K_E2M3_A8);
    return RUDDER_OK;
}

}  // namespace

rudder_status_t rudder_linear(const void* Xq, const float* row_scale, const uint8_t* stream_id,
                              const uint8_t* Wq, const float* w_scale, const float* comp_a,
                              const float* comp_b, int M, int N, int K, int S, int abits,
                              int codes, uint16_t* Y, int32_t* acc_out, void* stream) {
    const char* f = "rudder_linear";
    if (!Y) return fail(RUDDER_ERR_INVALID_ARG, "%s: null pointer argument", f);
    if (misaligned(Y) || misaligned(acc_out))
        return fail(RUDDER_ERR_INVALID_ARG, "%s: Y and acc_out must be 16-byte aligned", f);
    const rudder_status_t st = check_linear(f, Xq, row_scale, stream_id, Wq, w_scale, comp_a,
                                            comp_b, M, N, K, S, abits, codes);
    if (st != RUDDER_OK) return st;
    if (M == 0) return ok();
    return from_hip(rudder::launch_linear(Xq, row_scale, stream_id, Wq, w_scale, comp_a, comp_b,
                                          M, N, K, S, abits, codes, Y, acc_out,
                                          static_cast<hipStream_t>(stream)),
                    f);
}

rudder_status_t rudder_linear_gelu_quant(const void* Xq, const float* row_scale,
                                         const uint8_t* stream_id, const uint8_t* Wq,
                                         const float* w_scale, const float* comp_a,
                                         const float* comp_b, int M, int N, int K, int S,
                                         int abits, int codes, const float* next_inv_smooth,
                                         const float* next_act_scale, int next_abits,
                                         int next_codes, void* next_Xq, float* next_row_scale,
                                         void* stream) {
    const char* f = "rudder_linear_gelu_quant";
    if (!next_inv_smooth || !next_act_scale || !next_Xq || !next_row_scale)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: null pointer argument", f);
    if (next_abits != 4 && next_abits != 8)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: next_abits=%d must be 4 or 8", f, next_abits);
    if (next_codes != RUDDER_CODES_INT && next_codes != RUDDER_CODES_E2M3)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: unknown code container %d", f, next_codes);
    if (next_codes == RUDDER_CODES_E2M3 && N % 64)
        return fail(RUDDER_ERR_INVALID_ARG,
                    "%s: E2M3 next codes need N a multiple of 64 (N=%d)", f, N);
    if (misaligned(next_inv_smooth) || misaligned(next_Xq))
        return fail(RUDDER_ERR_INVALID_ARG, "%s: next_inv_smooth and next_Xq must be 16-byte "
                    "aligned", f);
    const rudder_status_t st = check_linear(f, Xq, row_scale, stream_id, Wq, w_scale, comp_a,
                                            comp_b, M, N, K, S, abits, codes);
    if (st != RUDDER_OK) return st;
    if ((codes == RUDDER_CODES_E2M3 && abits == 8) ||
        (next_codes == RUDDER_CODES_E2M3 && next_abits == 8))
        return fail(RUDDER_ERR_UNSUPPORTED, "%s: 8-bit E2M3 codes are not built for this path",
                    f);
    if (M == 0) return ok();
    const rudder::NextLayerQuant next{next_inv_smooth, next_act_scale,
                                      static_cast<uint8_t*>(next_Xq), next_row_scale, next_abits,
                                      next_codes};
    return from_hip(rudder::launch_linear_gelu_quant(Xq, row_scale, stream_id, Wq, w_scale,
                                                     comp_a, comp_b, M, N, K, S, abits, codes,
                                                     next, static_cast<hipStream_t>(stream)),
                    f);
}

rudder_status_t rudder_gelu_bf16(const uint16_t* in, uint16_t* out, size_t n, void* stream) {
    const char* f = "rudder_gelu_bf16";
    if (n == 0) return ok();
    if (!in || !out) return fail(RUDDER_ERR_INVALID_ARG, "%s: null pointer argument", f);
    return from_hip(rudder::launch_gelu_bf16(in, out, n, static_cast<hipStream_t>(stream)), f);
}

rudder_status_t rudder_dequant_weights(const uint8_t* Wq, const float* w_scale, int K, int N,
                                       int codes, float* out, void* stream) {
    const char* f = "rudder_dequant_weights";
    if (!Wq || !w_scale || !out) return fail(RUDDER_ERR_INVALID_ARG, "%s: null pointer argument", f);
    if (K <= 0 || N <= 0 || K % 32 || N % 32)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: K=%d and N=%d must be positive multiples of 32",
                    f, K, N);
    if (codes != RUDDER_CODES_INT && codes != RUDDER_CODES_E2M3)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: unknown code container %d", f, codes);
    if (codes == RUDDER_CODES_E2M3 && K % 64)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: K=%d must be a multiple of 64 for E2M3 codes", f,
                    K);
    return from_hip(rudder::launch_dequant_weights(Wq, w_scale, K, N, codes, out,
                                                   static_cast<hipStream_t>(stream)),
                    f);
}

size_t rudder_stream_sq_error_workspace_bytes(void) {
    return rudder::stream_sq_error_workspace_bytes();
}

rudder_status_t rudder_stream_sq_error(const uint16_t* Y, const float* Yref,
                                       const uint8_t* stream_id, int M, int N, int S,
                                       void* workspace, double* sse, void* stream) {
    const char* f = "rudder_stream_sq_error";
    if (!Y || !Yref || !stream_id || !workspace || !sse)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: null pointer argument", f);
    if (M < 0 || N <= 0)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: M=%d must be >= 0 and N=%d > 0", f, M, N);
    if (S < 1 || S > RUDDER_MAX_STREAMS)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: S=%d must be in 1..%d", f, S, RUDDER_MAX_STREAMS);
    return from_hip(rudder::launch_stream_sq_error(Y, Yref, stream_id, M, N, S, workspace, sse,
                                                   static_cast<hipStream_t>(stream)),
                    f);
}

size_t rudder_mfma_ceiling_sink_bytes(void) { return rudder::mfma_ceiling_sink_bytes(); }

double rudder_mfma_ceiling_ops(int iters, int codes) {
    return iters > 0 ? rudder::mfma_ceiling_ops(iters, codes) : 0.0;
}

rudder_status_t rudder_mfma_ceiling(const uint8_t* Xq, const uint8_t* Wq, int M, int N, int K,
                                    int abits, int codes, int iters, int32_t* sink,
                                    void* stream) {
    return rudder_mfma_ceiling_shape(Xq, Wq, M, N, K, abits, codes, iters, RUDDER_CEILING_OWN,
                                     sink, stream);
}

rudder_status_t rudder_mfma_ceiling_shape(const uint8_t* Xq, const uint8_t* Wq, int M, int N,
                                          int K, int abits, int codes, int iters, int shape,
                                          int32_t* sink, void* stream) {
    const char* f = "rudder_mfma_ceiling";
    if (shape != RUDDER_CEILING_OWN && shape != RUDDER_CEILING_I8_16X16X64)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: unknown instruction shape %d", f, shape);
    if (shape == RUDDER_CEILING_I8_16X16X64 && codes != RUDDER_CODES_INT)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: the 16x16x64 int8 shape takes int codes", f);
    if (!Xq || !Wq || !sink) return fail(RUDDER_ERR_INVALID_ARG, "%s: null pointer argument", f);
    if (misaligned(Xq) || misaligned(Wq) || misaligned(sink))
        return fail(RUDDER_ERR_INVALID_ARG, "%s: Xq, Wq and sink must be 16-byte aligned", f);
    if (abits != 4 && abits != 8)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: abits=%d must be 4 or 8", f, abits);
    if (codes != RUDDER_CODES_INT && codes != RUDDER_CODES_E2M3)
        return fail(RUDDER_ERR_INVALID_ARG, "%s: unknown code container %d", f, codes);
    const int kmul = codes == RUDDER_CODES_E2M3 ? 64 : 32;
    if (M <= 0 || N <= 0 || K <= 0 || N % 32 || K % kmul)
        return fail(RUDDER_ERR_INVALID_ARG,
                    "%s: M=%d, N=%d, K=%d: need M > 0, N a multiple of 32, K a multiple of %d", f,
                    M, N, K, kmul);
    if (iters <= 0 || iters > (1 << 24))
        return fail(RUDDER_ERR_INVALID_ARG, "%s: iters=%d must be in 1..2^24", f, iters);
    return from_hip(rudder::launch_mfma_ceiling(Xq, Wq, M, N, K, abits, codes, iters, sink,
                                                static_cast<hipStream_t>(stream), shape),
                    f);
}

const char* rudder_status_string(rudder_status_t status) {
    switch (status) {
        case RUDDER_OK: return "RUDDER_OK";
        case RUDDER_ERR_INVALID_ARG: return "RUDDER_ERR_INVALID_ARG";
        case RUDDER_ERR_UNSUPPORTED: return "RUDDER_ERR_UNSUPPORTED";
        case RUDDER_ERR_HIP: return "RUDDER_ERR_HIP";
    }
    return "RUDDER_ERR_UNKNOWN";
}

const char* rudder_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
