/*
 * rudder.h -- C ABI of the stream-aware W4A8 / W4A4 linear layer on AMD
 * Instinct MI355X (gfx950).
 *
 * Method: "SteerQuant: Steering Quantization Error with Action-Guided Scaling
 * in World-Action Models" (paperlayer.ai digest).  A layer keeps ONE static
 * int4 weight matrix shared by every token stream (video, proprio, action)
 * and every denoising step (§1, §4.2); a shared positive diagonal rescales the
 * weights and inversely rescales the activations (§4.2); activations are
 * quantized with a step size per (stream, denoising step) taken from a
 * layer-step lookup table (§4.3); the fused kernels apply the scaling inside
 * activation quantization and follow the low-bit GEMM with dequantization,
 * inverse-gain compensation and bias, passing only integer activations and
 * row scales between the two kernels (§4.4, Rudder).  Bit widths: 4-bit
 * weights, 8- or 4-bit activations (App. D).
 *
 * Arithmetic (all fp32 steps round to nearest even):
 *   inv_smooth[k] = fl32(1 / s[k])                       (formed in fp64)
 *   w'[k][n]      = W[k][n] * s[k]
 *   w_scale[n]    = fl32(max_k |w'[k][n]| / 7)           (formed in fp64)
 *   qw[k][n]      = rne(clamp(w'[k][n] * fl32(1 / w_scale[n]), -7, 7))
 *   u             = X[m][k] * inv_smooth[k]
 *   qa[m][k]      = rne(clamp(u * fl32(1 / D[s]), -Qa, Qa)),  s = stream_id[m]
 *   row_scale[m]  = D[s]
 *   acc[m][n]     = sum_k qa[m][k] * qw[k][n]            (exact int32)
 *   y             = fmaf(a[s][n], (float)acc * (row_scale[m] * w_scale[n]), b[s][n])
 *   Y[m][n]       = bf16_rne(y)
 * with Qa = 127 (abits = 8) or 7 (abits = 4).  A zero scale has reciprocal 0
 * (its codes are 0 and its rows give Y = bf16(b)).
 *
 * ---------------------------------------------------------------------------
 * Conventions
 *   - Every buffer pointer is a DEVICE pointer (hipMalloc'd or torch CUDA
 *     memory) unless stated otherwise; `stream` is a hipStream_t passed as
 *     void* (NULL = the default stream).
 *   - The caller owns and allocates every buffer; the library never
 *     allocates, and its only device state is the fixed scratch array of
 *     rudder_quant_act_noalloc (one per GPU, from that call's first use).
 *   - Calls are asynchronous: they return once the work is enqueued on
 *     `stream`; results are valid after the stream is synchronized.  Calls
 *     are thread-safe.
 *   - Arguments are validated on the host before anything is launched; on a
 *     non-OK return nothing has been enqueued.  rudder_last_error() gives a
 *     thread-local description of the last failure.
 *   - Buffers read or written with vector accesses must be 16-byte aligned
 *     (each call lists them); a misaligned one gives RUDDER_ERR_INVALID_ARG.
 *   - Undefined behaviour (not checked): stream_id[m] >= S, non-finite X, W,
 *     s, scales or compensation values, overlapping output buffers.
 *
 * Packed-code layout ("MFMA-tiled"), shared by weight codes and activation
 * codes.  A code matrix C[R][K] (R = N for weights, M for activations) is cut
 * into 32 x 32 blocks.  Block (rb, kb) -- rows 32rb..32rb+31, k
 * 32kb..32kb+31 -- is stored contiguously at block index rb * (K/32) + kb.
 * Inside a block, slot l = (r % 32) + 32 * ((k % 32) / 16), l = 0..63, holds
 * the 16 codes of row r at k = 32kb + 16*(l/32) + j, j = 0..15:
 *   - 8-bit codes: 16 bytes, byte j = code j (two's complement);
 *     block = 1024 bytes;
 *   - 4-bit codes: 8 bytes = two little-endian 32-bit "split-nibble words",
 *     word w = j / 8 covering codes 8w..8w+7; byte i (0..3) of a word holds
 *     code 8w+i in bits 0..3 and code 8w+4+i in bits 4..7, as two's-
 *     complement nibbles; block = 512 bytes.
 * Rows from R up to the next multiple of 32 are padding and hold code 0.
 *
 * E2M3 container ("codes" = RUDDER_CODES_E2M3; 4-bit codes of W4A4 layers).
 * Each code c in [-7, 7] is held as the FP6 E2M3 encoding of the integer c
 * (bit 5 sign, bits 4..3 exponent with bias 1, bits 2..0 mantissa):
 * |c| = 0..7 -> 0x00, 0x08, 0x10, 0x14, 0x18, 0x1A, 0x1C, 0x1E, with bit 5 set
 * for negative c.  Every such value is exact, so the f8f6f4 matrix cores of
 * gfx950 multiply the codes exactly and their fp32 sums stay exact integers
 * (|sum| < 2^24 for K <= RUDDER_MAX_K).  A code matrix C[R][K] (K a multiple
 * of 64) is cut into 32 x 64 blocks of 1536 bytes; block (rb, kb) -- rows
 * 32rb..32rb+31, k 64kb..64kb+63 -- sits at block index rb * (K/64) + kb.
 * Slot l = (r % 32) + 32 * ((k % 64) / 32), l = 0..63, holds the 32 codes of
 * row r at k = 64kb + 32*(l/32) + t, t = 0..31, as a 192-bit little-endian
 * bit string (code t in bits 6t..6t+5).  Bits 0..127 of slot l are stored at
 * byte 16*l of the block (plane 0, 1024 bytes) and bits 128..191 at byte
 * 1024 + 8*l (plane 1, 512 bytes).  Padding rows hold code 0.
 *
 * E2M3 container for 8-bit activation codes (abits = 8, "codes" =
 * RUDDER_CODES_E2M3; the weights of such a layer use the E2M3 container
 * above).  Each code q in [-127, 127] is split into two digits,
 * q = 16 h + l with l = ((q + 8) mod 16) - 8 in [-8, 7] and
 * h = (q - l) / 16 in [-8, 8], and the digits are held as the E2M3 values
 * h / 2 and l / 2 (multiples of 1/2 with magnitude at most 4, all exact in
 * E2M3; the field of a value v is its standard E2M3 encoding:
 * |v| = m / 8 with exponent field 0, or (1 + m / 8) * 2^(e - 1) with
 * exponent field e = 1..3, mantissa field m, bit 5 the sign, +0 as 0x00).
 * The matrix is cut into 32 x 64 blocks of 3072 bytes at block index
 * rb * (K/64) + kb: bytes 0..1535 hold the h / 2 values of the block and
 * bytes 1536..3071 the l / 2 values, each half laid out as a 1536-byte block
 * above.  The matrix cores multiply each half with the weight codes under
 * E8M0 block scales 2^5 and 2^1, so the fp32 accumulator holds sum q * w
 * exactly while |sum| < 2^24, which 127 * 7 * K guarantees for
 * K <= RUDDER_MAX_K_E2M3_A8.  Padding rows hold code 0.
 * ---------------------------------------------------------------------------
 */
#ifndef RUDDER_H
#define RUDDER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RUDDER_OK = 0,
    RUDDER_ERR_INVALID_ARG = 1,   /* null required pointer, bad sizes or bit width */
    RUDDER_ERR_UNSUPPORTED = 2,   /* valid request outside the built shapes */
    RUDDER_ERR_HIP = 3            /* the HIP runtime reported a launch error */
} rudder_status_t;

/* Code containers of the packed weight and activation codes. */
typedef enum {
    RUDDER_CODES_INT = 0,   /* int4 split-nibble words / int8 bytes; int8 matrix cores */
    RUDDER_CODES_E2M3 = 1   /* codes held as FP6 E2M3 (8-bit activation codes as two
                               digit planes); f8f6f4 matrix cores */
} rudder_codes_t;

#define RUDDER_MAX_STREAMS 8      /* S, the number of token streams, is 1..8 */
#define RUDDER_MAX_K 65536        /* keeps every scaled int32 accumulator exact */
#define RUDDER_MAX_K_E2M3_A8 16384 /* keeps the fp32 sums of 8-bit E2M3 codes exact */

/* Bytes of packed weight codes for a K x N layer: N * K / 2 (RUDDER_CODES_INT;
 * K, N multiples of 32) or N * K * 3 / 4 (RUDDER_CODES_E2M3; K a multiple of
 * 64, N of 32).  Returns 0 for invalid sizes. */
size_t rudder_packed_weight_bytes(int K, int N, int codes);

/* Bytes of activation codes for M rows (rounded up to 32) of K channels:
 * ceil(M/32)*32 * K * abits / 8 (RUDDER_CODES_INT), or ceil(M/32)*32 * K * 3/4
 * (RUDDER_CODES_E2M3, abits = 4) or ceil(M/32)*32 * K * 3/2
 * (RUDDER_CODES_E2M3, abits = 8), K a multiple of 64 for E2M3.  0 for invalid
 * sizes. */
size_t rudder_packed_act_bytes(int M, int K, int abits, int codes);

/* Bytes of device workspace rudder_quant_act needs in dynamic mode. */
size_t rudder_quant_act_workspace_bytes(int S);

/*
 * Offline weight preparation (SteerQuant Fig. 2, offline weight preparation;
 * §4.2 shared-weight error routing).  Folds the smoothing diagonal into the
 * weights and quantizes each output channel to symmetric int4.
 *
 *   W          bf16 bits [K][N], row-major (input channel k, output channel n)
 *   smooth     fp32 [K], s[k] > 0
 *   K, N       > 0, multiples of 32 (K a multiple of 64 for RUDDER_CODES_E2M3)
 *   codes      container of Wq: RUDDER_CODES_INT or RUDDER_CODES_E2M3, the
 *              container the layer's activations use
 *   Wq         out: rudder_packed_weight_bytes(K, N, codes) bytes, MFMA-tiled
 *              layout with R = N (row = output channel)
 *   w_scale    out: fp32 [N]
 *   inv_smooth out: fp32 [K] = fl32(1 / s[k]), formed in fp64; this is what
 *              rudder_quant_act takes for the same layer
 * Errors: INVALID_ARG for a null pointer, K or N <= 0, K or N not a multiple
 * of 32 (K of 64 for E2M3), an unknown container, Wq/smooth/w_scale/
 * inv_smooth not 16-byte aligned; UNSUPPORTED for K > RUDDER_MAX_K.
 */
rudder_status_t rudder_quantize_weights(const uint16_t* W, const float* smooth, int K, int N,
                                        int codes, uint8_t* Wq, float* w_scale,
                                        float* inv_smooth, void* stream);

/*
 * Fused activation quantization (SteerQuant §4.4: scaling and stream gains
 * applied during activation quantization; §4.3: one step size per stream and
 * denoising step from the layer-step table).
 *
 *   X          bf16 bits [M][K], row-major
 *   stream_id  uint8 [M], each < S (row m belongs to stream stream_id[m])
 *   inv_smooth fp32 [K] from rudder_quantize_weights
 *   act_scale  fp32 [S]: the step sizes D[s] of this (layer, step), i.e. the
 *              table row of the current step.  NULL selects dynamic mode:
 *              D[s] = fl32(max |u| over the rows of stream s / Qa) (fp64
 *              divide); a stream with no rows gets D = 0.
 *   act_scale_out  fp32 [S], dynamic mode: receives D (may be NULL); ignored
 *              in static mode
 *   workspace  dynamic mode: rudder_quant_act_workspace_bytes(S) bytes of
 *              device scratch; ignored (may be NULL) in static mode
 *   M >= 0 (M = 0 is a no-op), K > 0 multiple of 32, 1 <= S <= 8,
 *   abits in {4, 8}
 *   codes      container of Xq: RUDDER_CODES_INT, or RUDDER_CODES_E2M3 (K a
 *              multiple of 64)
 *   Xq         out: rudder_packed_act_bytes(M, K, abits, codes) bytes,
 *              MFMA-tiled layout with R = M; padding rows are 0
 *   row_scale  out: fp32 [M], row_scale[m] = D[stream_id[m]]
 * Errors: INVALID_ARG for null X/stream_id/inv_smooth/Xq/row_scale, a null
 * workspace in dynamic mode, M < 0, K <= 0, K % 32 != 0, S outside 1..8,
 * abits not 4 or 8, an unknown container or E2M3 with K % 64 != 0,
 * X/inv_smooth/Xq/workspace not 16-byte aligned; UNSUPPORTED for
 * K > RUDDER_MAX_K.
 * Dynamic mode enqueues three kernels (partial absmax, finalize, quantize);
 * static mode one.
 */
rudder_status_t rudder_quant_act(const uint16_t* X, const uint8_t* stream_id,
                                 const float* inv_smooth, const float* act_scale,
                                 float* act_scale_out, void* workspace,
                                 int M, int K, int S, int abits, int codes,
                                 void* Xq, float* row_scale, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops, harnesses that forbid hipMalloc): the dynamic mode
 * of rudder_quant_act (act_scale = NULL) without a workspace argument.  The
 * partial maxima and step sizes live in a scratch array the library holds
 * per GPU, RUDDER_MAX_STREAMS * 1025 floats (32,800 bytes), from the first
 * call on that GPU until the process ends; the call itself allocates
 * nothing.  The scratch size does not depend on M or K, so every size
 * rudder_quant_act accepts fits.  Every call on one GPU shares that GPU's
 * scratch: calls that overlap on one GPU (several streams or threads) race
 * and must be serialized by the caller.  The device current on the calling
 * thread must be the device of `stream`.
 *
 *   arguments as for rudder_quant_act in dynamic mode; act_scale_out may be
 *   NULL
 * Results are identical to rudder_quant_act(X, stream_id, inv_smooth, NULL,
 * act_scale_out, workspace, ...).
 * Errors: those of rudder_quant_act (dynamic mode); RUDDER_ERR_HIP also when
 * the scratch's device address cannot be obtained.
 */
rudder_status_t rudder_quant_act_noalloc(const uint16_t* X, const uint8_t* stream_id,
                                         const float* inv_smooth, float* act_scale_out,
                                         int M, int K, int S, int abits, int codes,
                                         void* Xq, float* row_scale, void* stream);

/*
 * Low-bit GEMM with fused epilogue (SteerQuant §4.4: low-bit GEMM followed by
 * dequantization, inverse-gain compensation and bias; §1: Rudder fuses the
 * output compensation into the low-bit kernel).
 *
 *   Xq, row_scale, stream_id   from rudder_quant_act (same M, K, abits, codes)
 *   Wq, w_scale                from rudder_quantize_weights (same K, N, codes)
 *   codes      RUDDER_CODES_INT: int4 weights widened to int8 in registers
 *              feed int8 MFMA with int32 accumulation; RUDDER_CODES_E2M3:
 *              E2M3-held codes feed the f8f6f4 MFMA with fp32 accumulation,
 *              exact for these integer operands (abits = 8: two MFMAs per
 *              product, one per digit plane)
 *   comp_a, comp_b  fp32 [S][N]: the compensation of this (layer, step);
 *              y = a * t + b as one fp32 fma, the layer bias folded into b
 *   M >= 0 (M = 0 is a no-op), N > 0 multiple of 32, K > 0 multiple of 128,
 *   1 <= S <= 8, abits in {4, 8}
 *   Y          out: bf16 bits [M][N], row-major
 *   acc_out    optional out: int32 [M][N] row-major raw accumulators
 *              sum_k qa*qw (a verification aid; pass NULL on the hot path)
 * Launches: for M > 256 one tiled GEMM launch (its first blocks read the
 * packed weights once more, so that they are cache-resident for the tiles'
 * repeated reads; for some row counts its last blocks take the last rows in
 * narrower pieces); for M <= 256 one weight-streaming kernel.  On `stream`.
 * Errors: INVALID_ARG for a null required pointer, M < 0, N or K <= 0,
 * N % 32 != 0, S outside 1..8, abits not 4 or 8, an unknown container,
 * Xq/Wq/w_scale/comp_a/comp_b/Y/acc_out not 16-byte aligned; UNSUPPORTED for
 * K % 128 != 0, K > RUDDER_MAX_K, or K > RUDDER_MAX_K_E2M3_A8 with E2M3
 * codes and abits = 8.
 */
rudder_status_t rudder_linear(const void* Xq, const float* row_scale, const uint8_t* stream_id,
                              const uint8_t* Wq, const float* w_scale,
                              const float* comp_a, const float* comp_b,
                              int M, int N, int K, int S, int abits, int codes,
                              uint16_t* Y, int32_t* acc_out, void* stream);

/*
 * MLP up-projection with GELU and the down layer's activation quantizer fused
 * into the epilogue (SteerQuant §4.4: only integer activations and row scales
 * travel between kernels; App. D: GELU stays in BF16).  The bf16 output of
 * the up-projection never reaches HBM.
 *
 * Per element this computes exactly what the unfused chain computes:
 *   Y  = the bf16 output rudder_linear would write (same arguments);
 *   G  = gelu(Y): the exact (erf) form x * Phi(x) of the bf16 value Y,
 *        evaluated in fp64 and rounded to fp32, then to bf16 (RNE both
 *        times) -- rudder_gelu_bf16 applies the same function;
 *   then rudder_quant_act in static mode on G (as the down layer's input,
 *   K' = N channels) with next_inv_smooth and next_act_scale.
 *
 *   Xq ... codes    as for rudder_linear (the up-projection; M >= 0)
 *   next_inv_smooth fp32 [N]: the down layer's inverse smoothing factors
 *   next_act_scale  fp32 [S]: the down layer's step sizes D'[s] at this step
 *   next_abits      4 or 8;  next_codes  RUDDER_CODES_INT, or
 *                   RUDDER_CODES_E2M3 (next_abits = 4, N a multiple of 64)
 *   next_Xq         out: rudder_packed_act_bytes(M, N, next_abits,
 *                   next_codes) bytes, the down layer's packed activations
 *                   (padding rows 0)
 *   next_row_scale  out: fp32 [M] = D'[stream_id[m]]
 * Errors: those of rudder_linear, plus INVALID_ARG for a null
 * next_inv_smooth/next_act_scale/next_Xq/next_row_scale, next_abits not 4 or
 * 8, an unknown next container or E2M3 with N % 64 != 0,
 * next_inv_smooth/next_Xq not 16-byte aligned; UNSUPPORTED for E2M3 with
 * abits = 8 or next_abits = 8 (8-bit E2M3 codes are not built for this
 * path).
 */
rudder_status_t rudder_linear_gelu_quant(const void* Xq, const float* row_scale,
                                         const uint8_t* stream_id, const uint8_t* Wq,
                                         const float* w_scale, const float* comp_a,
                                         const float* comp_b, int M, int N, int K, int S,
                                         int abits, int codes, const float* next_inv_smooth,
                                         const float* next_act_scale, int next_abits,
                                         int next_codes, void* next_Xq, float* next_row_scale,
                                         void* stream);

/*
 * The GELU of rudder_linear_gelu_quant applied elementwise to n bf16 values
 * (device buffers; in and out may alias).  A table over the 65536 bf16
 * patterns: NaN -> quiet NaN of the same sign, +inf -> +inf, -inf -> -0.
 * Errors: INVALID_ARG for null in/out with n > 0.
 */
rudder_status_t rudder_gelu_bf16(const uint16_t* in, uint16_t* out, size_t n, void* stream);

/*
 * Calibration support (SteerQuant App. C.1: the activation-error target uses
 * unquantized activations and the fixed quantized weights).  Unpacks Wq
 * (either container) into out[k][n] = fl32(qw[k][n] * w_scale[n]), fp32
 * [K][N] row-major.  K, N as for rudder_quantize_weights.
 * Errors: INVALID_ARG for a null pointer, K or N <= 0 or not a multiple of 32
 * (K of 64 for E2M3), an unknown container.
 */
rudder_status_t rudder_dequant_weights(const uint8_t* Wq, const float* w_scale, int K, int N,
                                       int codes, float* out, void* stream);


/*
 * Calibration support (SteerQuant §4.2, §4.3, App. C: the shared diagonal and
 * the layer-step thresholds and stream gains are chosen offline by a
 * map-weighted reconstruction error whose weights differ per stream).
 * For each stream s < S:  sse[s] = sum over rows m with stream_id[m] = s and
 * all n of (float(Y[m][n]) - Yref[m][n])^2, accumulated in fp64 in a fixed
 * order (deterministic).
 *
 *   Y          bf16 bits [M][N] (e.g. rudder_linear's output)
 *   Yref       fp32 [M][N], the target
 *   stream_id  uint8 [M], each < S
 *   workspace  rudder_stream_sq_error_workspace_bytes() bytes of device scratch
 *   sse        out: fp64 [S] (device)
 *   M >= 0 (M = 0 writes sse = 0), N > 0, 1 <= S <= 8
 * Errors: INVALID_ARG for a null pointer, M < 0, N <= 0, S outside 1..8.
 */
size_t rudder_stream_sq_error_workspace_bytes(void);
rudder_status_t rudder_stream_sq_error(const uint16_t* Y, const float* Yref,
                                       const uint8_t* stream_id, int M, int N, int S,
                                       void* workspace, double* sse, void* stream);

/* Static string naming a status code. */
const char* rudder_status_string(rudder_status_t status);

/* Thread-local description of the last non-OK return on this thread
 * ("" if none).  The pointer stays valid until the next call on the thread. */
const char* rudder_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RUDDER_H */
