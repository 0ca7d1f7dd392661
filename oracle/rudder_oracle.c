/*
 * CPU oracle for the stream-aware W4A8 / W4A4 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or helper with the HIP library; it implements the method
 * from its description, one plain loop per step, in the order the steps are
 * stated below.
 *
 * Source of the method: "SteerQuant: Steering Quantization Error with
 * Action-Guided Scaling in World-Action Models" (paperlayer.ai digest):
 *   - §3.1 (WAM quantization): weights and activations use symmetric k-bit
 *     quantization; 4-bit weights, 8- or 4-bit activations (App. D).
 *   - §4.2 (Shared-weight error routing): one shared positive diagonal
 *     rescales the weights and inversely rescales the activations, with a
 *     single static quantized weight matrix per layer.
 *   - §4.3 (Stream-specific activation modulation): per (layer, step) a
 *     clipping threshold plus bounded per-stream gains, read from a LUT.
 *   - §4.4 (Rudder): scaling and gains are applied inside activation
 *     quantization; the low-bit GEMM is followed by dequantization,
 *     inverse-gain compensation and bias; only integer activations and row
 *     scales travel between the two kernels.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - "symmetric k-bit" means integer codes in [-(2^(k-1)-1), 2^(k-1)-1];
 *     rounding is round-to-nearest-even;
 *   - a step size is applied as a multiplication by its fp32 reciprocal,
 *     computed in fp64 and rounded once;
 *   - quantizer decisions are made in fp32 (the kernels' precision);
 *   - per-output-channel weight scales; one activation step size per
 *     (stream, step); the compensation is y = a[s,n] * t + b[s,n], one fp32
 *     fused multiply-add, with the layer bias folded into b.
 *
 * Every floating-point operation below is a single IEEE fp32 (or fp64 where
 * written) operation with round-to-nearest-even; the file is compiled with
 * -ffp-contract=off so no multiply-add is fused unless fmaf() is called.
 *
 * Packed 4-bit codes (a storage format, not part of the arithmetic): two
 * codes per byte along k, byte i of a row holding code 2i in bits 0..3 and
 * code 2i+1 in bits 4..7, as two's-complement nibbles.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_INPUT 1
#define ORACLE_OVERFLOW 2

/* ---- bf16 <-> fp32 ------------------------------------------------------ */

/* bf16 is the upper half of an fp32 bit pattern: widening is exact. */
static float bf16_to_float(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even (finite inputs). */
static uint16_t float_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* fp32 reciprocal formed in fp64 and rounded once; 0 maps to 0. */
static float recip_via_f64(float x) {
    if (x > 0.0f) return (float)(1.0 / (double)x);
    return 0.0f;
}

/* clamp to [-q, q], then round half to even. */
static int quantize_value(float v, int q) {
    float qf = (float)q;
    if (v > qf) v = qf;
    if (v < -qf) v = -qf;
    return (int)rintf(v);
}

/* ---- exported helpers for the tests ------------------------------------ */

void oracle_bf16_to_f32(const uint16_t* in, float* out, long n) {
    for (long i = 0; i < n; ++i) out[i] = bf16_to_float(in[i]);
}

void oracle_f32_to_bf16(const float* in, uint16_t* out, long n) {
    for (long i = 0; i < n; ++i) out[i] = float_to_bf16_rne(in[i]);
}

/* ---- weight preparation (offline; SteerQuant Fig. 2 and §4.2) ----------- */

/* inv_smooth[k] = 1 / s[k], formed in fp64, rounded once to fp32. */
int oracle_inv_smooth(const float* s, int K, float* inv_smooth) {
    for (int k = 0; k < K; ++k) {
        if (!(s[k] > 0.0f) || !isfinite(s[k])) return ORACLE_BAD_INPUT;
        inv_smooth[k] = (float)(1.0 / (double)s[k]);
    }
    return ORACLE_OK;
}

/*
 * Per output channel n:
 *   w'[k]      = W[k][n] * s[k]                     (fp32)
 *   amax       = max_k |w'[k]|
 *   w_scale[n] = amax / 7                           (fp64, rounded once)
 *   qw[n][k]   = rne(clamp(w'[k] * (1 / w_scale[n]), -7, 7))
 * W is bf16 [K][N] row-major; codes come out as int8 [N][K].
 */
int oracle_quantize_weights(const uint16_t* W, const float* s, int K, int N,
                            int8_t* qw, float* w_scale) {
    for (int n = 0; n < N; ++n) {
        float amax = 0.0f;
        for (int k = 0; k < K; ++k) {
            float w = bf16_to_float(W[(long)k * N + n]) * s[k];
            if (!isfinite(w)) return ORACLE_BAD_INPUT;
            float a = fabsf(w);
            if (a > amax) amax = a;
        }
        float ws = (float)((double)amax / 7.0);
        float iw = recip_via_f64(ws);
        w_scale[n] = ws;
        for (int k = 0; k < K; ++k) {
            float w = bf16_to_float(W[(long)k * N + n]) * s[k];
            qw[(long)n * K + k] = (int8_t)quantize_value(w * iw, 7);
        }
    }
    return ORACLE_OK;
}

/* ---- activation quantization (SteerQuant §4.3, §4.4) -------------------- */

/*
 * Dynamic step sizes: amax_s = max over rows of stream s and all k of
 * |X[m][k] * inv_smooth[k]|; delta[s] = amax_s / Qa (fp64, rounded once).
 * A stream with no rows gets delta 0.
 */
int oracle_dynamic_scales(const uint16_t* X, const uint8_t* stream_id, const float* inv_smooth,
                          int M, int K, int S, int qa, float* delta) {
    float amax[256];
    for (int s = 0; s < S; ++s) amax[s] = 0.0f;
    for (int m = 0; m < M; ++m) {
        int s = stream_id[m];
        if (s >= S) return ORACLE_BAD_INPUT;
        for (int k = 0; k < K; ++k) {
            float u = bf16_to_float(X[(long)m * K + k]) * inv_smooth[k];
            if (!isfinite(u)) return ORACLE_BAD_INPUT;
            float a = fabsf(u);
            if (a > amax[s]) amax[s] = a;
        }
    }
    for (int s = 0; s < S; ++s) delta[s] = (float)((double)amax[s] / (double)qa);
    return ORACLE_OK;
}

/*
 * Row m of stream s = stream_id[m], step size D = delta[s]:
 *   u  = X[m][k] * inv_smooth[k]       (fp32)
 *   v  = u * (1 / D)                   (fp32; 1/D formed in fp64; D = 0 -> 0)
 *   qa = rne(clamp(v, -Qa, Qa))
 *   row_scale[m] = D
 * Codes come out unpacked as int8 [M][K].
 */
int oracle_quant_act(const uint16_t* X, const uint8_t* stream_id, const float* inv_smooth,
                     const float* delta, int M, int K, int S, int qa,
                     int8_t* codes, float* row_scale) {
    for (int m = 0; m < M; ++m) {
        int s = stream_id[m];
        if (s >= S) return ORACLE_BAD_INPUT;
        float d = delta[s];
        float ia = recip_via_f64(d);
        row_scale[m] = d;
        for (int k = 0; k < K; ++k) {
            float x = bf16_to_float(X[(long)m * K + k]);
            if (!isfinite(x)) return ORACLE_BAD_INPUT;
            float u = x * inv_smooth[k];
            float v = u * ia;
            codes[(long)m * K + k] = (int8_t)quantize_value(v, qa);
        }
    }
    return ORACLE_OK;
}

/* ---- packing ------------------------------------------------------------ */

/* codes int8 [R][K] in [-8, 7] -> uint8 [R][K/2], two codes per byte:
 * byte i = (code 2i & 0xF) | (code 2i+1 & 0xF) << 4; K even. */
int oracle_pack_int4(const int8_t* codes, long R, int K, uint8_t* packed) {
    if (K % 2) return ORACLE_BAD_INPUT;
    for (long r = 0; r < R; ++r) {
        const int8_t* c = codes + r * K;
        uint8_t* p = packed + r * (K / 2);
        for (int i = 0; i < K / 2; ++i) {
            uint8_t lo = (uint8_t)(c[2 * i] & 0xF);
            uint8_t hi = (uint8_t)(c[2 * i + 1] & 0xF);
            p[i] = (uint8_t)(lo | (hi << 4));
        }
    }
    return ORACLE_OK;
}

/* uint8 [R][K/2] two codes per byte -> int8 codes [R][K] (sign-extended). */
int oracle_unpack_int4(const uint8_t* packed, long R, int K, int8_t* codes) {
    if (K % 2) return ORACLE_BAD_INPUT;
    for (long r = 0; r < R; ++r) {
        const uint8_t* p = packed + r * (K / 2);
        int8_t* c = codes + r * K;
        for (int i = 0; i < K / 2; ++i) {
            int lo = p[i] & 0xF;
            int hi = (p[i] >> 4) & 0xF;
            c[2 * i] = (int8_t)(lo >= 8 ? lo - 16 : lo);
            c[2 * i + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
        }
    }
    return ORACLE_OK;
}

/* ---- integer GEMM ------------------------------------------------------- */

/*
 * acc[m][n] = sum_k qa[m][k] * qw[n][k], explicit integer dot products.
 * Partial sums over chunks of 1024 k are int32 (|partial| <= 1024*127*127
 * < 2^24); chunks are added in int64 and the total must fit int32.
 */
int oracle_int_gemm(const int8_t* qa, const int8_t* qw, int M, int N, int K, int32_t* acc) {
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; ++m) {
        const int8_t* a = qa + (long)m * K;
        for (int n = 0; n < N; ++n) {
            const int8_t* b = qw + (long)n * K;
            int64_t total = 0;
            for (int k0 = 0; k0 < K; k0 += 1024) {
                int k1 = k0 + 1024 < K ? k0 + 1024 : K;
                int32_t part = 0;
                for (int k = k0; k < k1; ++k) part += (int32_t)a[k] * (int32_t)b[k];
                total += part;
            }
            if (total > INT32_MAX || total < INT32_MIN) {
#pragma omp atomic write
                status = ORACLE_OVERFLOW;
            }
            acc[(long)m * N + n] = (int32_t)total;
        }
    }
    return status;
}

/* ---- epilogue (SteerQuant §4.4: dequantize, compensate, bias) ----------- */

/*
 * f = (float)acc                       (exact while |acc| < 2^24)
 * d = row_scale[m] * w_scale[n]        (fp32)
 * t = f * d                            (fp32)
 * y = fmaf(a[s][n], t, b[s][n])        (one fused multiply-add)
 * Y = bf16_rne(y)
 */
int oracle_epilogue(const int32_t* acc, const float* row_scale, const uint8_t* stream_id,
                    const float* w_scale, const float* comp_a, const float* comp_b,
                    int M, int N, int S, uint16_t* Y) {
    for (int m = 0; m < M; ++m) {
        int s = stream_id[m];
        if (s >= S) return ORACLE_BAD_INPUT;
        for (int n = 0; n < N; ++n) {
            float f = (float)acc[(long)m * N + n];
            float d = row_scale[m] * w_scale[n];
            float t = f * d;
            float y = fmaf(comp_a[(long)s * N + n], t, comp_b[(long)s * N + n]);
            Y[(long)m * N + n] = float_to_bf16_rne(y);
        }
    }
    return ORACLE_OK;
}

/* ---- GELU between the MLP projections (SteerQuant App. D: GELU stays BF16) */

/*
 * The exact (erf) form on a bf16 input, gelu(x) = x * Phi(x), evaluated in
 * fp64 as 0.5 * x * erfc(-x / sqrt(2)) (erfc keeps the tail accurate for
 * negative x), then rounded to fp32 and from fp32 to bf16, both
 * round-to-nearest-even.  Non-finite inputs: NaN -> quiet NaN of the same
 * sign, +inf -> +inf, -inf -> -0.
 */
static uint16_t gelu_bf16_one(uint16_t h) {
    const uint32_t exp_bits = (h >> 7) & 0xFFu;
    const uint16_t sign = h & 0x8000u;
    if (exp_bits == 0xFFu) {
        if (h & 0x7Fu) return (uint16_t)(sign | 0x7FC0u);   /* NaN */
        return sign ? (uint16_t)0x8000u : (uint16_t)0x7F80u; /* -inf -> -0, +inf -> +inf */
    }
    const double x = (double)bf16_to_float(h);
    const double g = 0.5 * x * erfc(-x * 0.70710678118654752440);
    return float_to_bf16_rne((float)g);
}

void oracle_gelu_bf16(const uint16_t* in, uint16_t* out, long n) {
    for (long i = 0; i < n; ++i) out[i] = gelu_bf16_one(in[i]);
}

/* Thread count OpenMP will use (reported by the CPU baseline). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
