// Internal declarations shared by the HIP translation units of librudder.
// Device helpers here implement the arithmetic stated in include/rudder.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rudder.h"
#include "rudder_diag.h"

namespace rudder {

// ---------------------------------------------------------------------------
// Launch-side entry points (one per kernel family).  Arguments are already
// validated by the C ABI layer; each returns the launch's hipError_t.
// ---------------------------------------------------------------------------
hipError_t launch_quantize_weights(const uint16_t* W, const float* smooth, int K, int N,
                                   int codes, uint8_t* Wq, float* w_scale, float* inv_smooth,
                                   hipStream_t stream);

hipError_t launch_quant_act_static(const uint16_t* X, const uint8_t* sid, const float* inv_smooth,
                                   const float* delta, int M, int K, int S, int abits, int codes,
                                   void* Xq, float* row_scale, hipStream_t stream);

hipError_t launch_quant_act_dynamic(const uint16_t* X, const uint8_t* sid,
                                    const float* inv_smooth, float* act_scale_out,
                                    void* workspace, int M, int K, int S, int abits, int codes,
                                    void* Xq, float* row_scale, hipStream_t stream);

size_t quant_act_workspace_bytes();

// Dynamic mode with the library's own per-device scratch instead of a caller
// workspace (no allocation on the call).
hipError_t launch_quant_act_dynamic_noalloc(const uint16_t* X, const uint8_t* sid,
                                            const float* inv_smooth, float* act_scale_out,
                                            int M, int K, int S, int abits, int codes, void* Xq,
                                            float* row_scale, hipStream_t stream);
size_t quant_act_noalloc_scratch_bytes();

hipError_t launch_linear(const void* Xq, const float* row_scale, const uint8_t* sid,
                         const uint8_t* Wq, const float* w_scale, const float* comp_a,
                         const float* comp_b, int M, int N, int K, int S, int abits, int codes,
                         uint16_t* Y, int32_t* acc_out, hipStream_t stream);

// The down layer's quantizer, fused into the up-projection epilogue.
struct NextLayerQuant {
    const float* inv_smooth;   // [N]
    const float* delta;        // [S]
    uint8_t* xq;               // packed codes of the down layer's input
    float* row_scale;          // [M]
    int abits;
    int codes;
};

hipError_t launch_linear_gelu_quant(const void* Xq, const float* row_scale, const uint8_t* sid,
                                    const uint8_t* Wq, const float* w_scale, const float* comp_a,
                                    const float* comp_b, int M, int N, int K, int S, int abits,
                                    int codes, const NextLayerQuant& next, hipStream_t stream);

hipError_t launch_gelu_bf16(const uint16_t* in, uint16_t* out, size_t n, hipStream_t stream);

hipError_t launch_dequant_weights(const uint8_t* Wq, const float* w_scale, int K, int N,
                                  int codes, float* out, hipStream_t stream);
size_t stream_sq_error_workspace_bytes();
hipError_t launch_stream_sq_error(const uint16_t* Y, const float* Yref, const uint8_t* sid, int M,
                                  int N, int S, void* workspace, double* sse, hipStream_t stream);

// Matrix-core ceiling measurement (include/rudder_diag.h).
size_t mfma_ceiling_sink_bytes();
double mfma_ceiling_ops(int iters, int codes);
hipError_t launch_mfma_ceiling(const uint8_t* Xq, const uint8_t* Wq, int M, int N, int K,
                               int abits, int codes, int iters, int32_t* sink,
                               hipStream_t stream, int shape = RUDDER_CEILING_OWN);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// bf16 bits -> fp32 (exact: bf16 is the upper half of an fp32 pattern).
__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
    return __uint_as_float(h << 16);
}

// fp32 -> bf16 bits with round-to-nearest-even (finite inputs).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Reciprocal of a step size: formed in fp64, rounded once to fp32; 0 -> 0.
__device__ __forceinline__ float step_reciprocal(float d) {
    return d > 0.0f ? (float)(1.0 / (double)d) : 0.0f;
}

// Symmetric quantizer: clamp to [-q, q], round half to even.
__device__ __forceinline__ int quantize_clamped(float v, float q) {
    v = fminf(fmaxf(v, -q), q);
    return (int)__builtin_rintf(v);
}

// Pack 8 codes (k0..k7) into one split-nibble word: byte i holds code i in
// bits 0..3 and code i+4 in bits 4..7.
__device__ __forceinline__ uint32_t split_nibble_word(const int* c) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t b = ((uint32_t)c[i] & 0xFu) | (((uint32_t)c[i + 4] & 0xFu) << 4);
        w |= b << (8 * i);
    }
    return w;
}

// Pack 4 int8 codes into a 32-bit word, byte i = code i.
__device__ __forceinline__ uint32_t byte_word(const int* c) {
    return ((uint32_t)c[0] & 0xFFu) | (((uint32_t)c[1] & 0xFFu) << 8) |
           (((uint32_t)c[2] & 0xFFu) << 16) | (((uint32_t)c[3] & 0xFFu) << 24);
}

// Byte offset of slot (row r, k) in an MFMA-tiled code matrix with K columns.
// Slot = 16 codes; bytes per slot = 16 (8-bit) or 8 (4-bit).
template <int BITS>
__device__ __forceinline__ size_t tiled_slot_offset(int r, int k, int K) {
    constexpr int SLOT_BYTES = 2 * BITS;           // 16 codes * BITS / 8
    constexpr int BLOCK_BYTES = 64 * SLOT_BYTES;
    size_t block = (size_t)(r >> 5) * (size_t)(K >> 5) + (size_t)(k >> 5);
    int slot = (r & 31) + 32 * ((k & 31) >> 4);
    return block * BLOCK_BYTES + (size_t)slot * SLOT_BYTES;
}

// Symmetric quantizer to an integer-valued float: clamp to [-q, q], round
// half to even, -0 folded to +0 (so a zero code always encodes as 0).
__device__ __forceinline__ float quantize_clamped_f(float v, float q) {
    v = fminf(fmaxf(v, -q), q);
    return __builtin_rintf(v) + 0.0f;
}

// Pack 32 integer-valued floats c_t in [-7, 7] (zero as +0) into the 192-bit
// little-endian string of 6-bit FP6 E2M3 fields, field t at bits 6t..6t+5,
// held in six dwords.  Each such value is exact in E2M3 (sign in bit 5,
// exponent bias 1 in bits 4..3, mantissa in bits 2..0), so the gfx950
// pack-convert with unit scale encodes it without rounding; that instruction
// fills alternating fields from its two 16-wide operands (even t from the
// first, odd t from the second).
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x6_t __attribute__((ext_vector_type(6)));
__device__ __forceinline__ void pack_e2m3x32(const float* c, uint32_t (&d)[6]) {
    f32x16_t even, odd;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        even[i] = c[2 * i];
        odd[i] = c[2 * i + 1];
    }
    const u32x6_t r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(even, odd, 1.0f);
#pragma unroll
    for (int i = 0; i < 6; ++i) d[i] = r[i];
}

// Byte offsets of slot (row r, k) in an E2M3 code matrix with K columns:
// plane 0 (16 bytes) and plane 1 (8 bytes) of the 1536-byte 32 x 64 block.
__device__ __forceinline__ size_t e2m3_block_offset(int r, int k, int K) {
    return ((size_t)(r >> 5) * (size_t)(K >> 6) + (size_t)(k >> 6)) * 1536;
}
__device__ __forceinline__ int e2m3_slot(int r, int k) { return (r & 31) + 32 * ((k & 63) >> 5); }

}  // namespace rudder
