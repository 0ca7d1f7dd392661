// Calibration support: per-stream squared output error.
//
// SteerQuant ("SteerQuant: Steering Quantization Error with Action-Guided
// Scaling in World-Action Models", paperlayer.ai digest), §4.2 and §4.3,
// App. C / C.1: the shared diagonal and the per-(layer, step) threshold and
// bounded stream gains are calibrated offline by minimising a map-weighted
// reconstruction error, where the map weights differ per stream.  The
// quantity every candidate needs is, for each stream s, the sum over its rows
// and all output channels of (Y - Yref)^2, Y the bf16 output of the
// quantized layer and Yref an fp32 target.
//
// Two passes, deterministic: each block sums a fixed range of rows per stream
// in fp64 (per-thread partials, then a fixed-order tree in LDS), then one
// block adds the block partials in block order.
#include "rudder_internal.h"

namespace rudder {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 512;

__global__ __launch_bounds__(kThreads) void stream_sq_error_partial(
    const uint16_t* __restrict__ Y, const float* __restrict__ Yref,
    const uint8_t* __restrict__ sid, int M, int N, int S, int rows_per_block,
    double* __restrict__ partial) {
    __shared__ double red[RUDDER_MAX_STREAMS][kThreads];
    double acc[RUDDER_MAX_STREAMS];
#pragma unroll
    for (int s = 0; s < RUDDER_MAX_STREAMS; ++s) acc[s] = 0.0;
    const int r0 = blockIdx.x * rows_per_block;
    const int r1 = min(M, r0 + rows_per_block);
    for (int m = r0; m < r1; ++m) {
        const int s = sid[m] & (RUDDER_MAX_STREAMS - 1);
        double a = 0.0;
        for (int n = threadIdx.x; n < N; n += kThreads) {
            const double d = (double)bf16_bits_to_float(Y[(size_t)m * N + n]) -
                             (double)Yref[(size_t)m * N + n];
            a += d * d;
        }
#pragma unroll
        for (int t = 0; t < RUDDER_MAX_STREAMS; ++t)
            if (t == s) acc[t] += a;
    }
#pragma unroll
    for (int s = 0; s < RUDDER_MAX_STREAMS; ++s) red[s][threadIdx.x] = acc[s];
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
#pragma unroll
            for (int s = 0; s < RUDDER_MAX_STREAMS; ++s)
                red[s][threadIdx.x] += red[s][threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x < S) partial[(size_t)blockIdx.x * RUDDER_MAX_STREAMS + threadIdx.x] =
        red[threadIdx.x][0];
}

__global__ void stream_sq_error_final(const double* __restrict__ partial, int blocks, int S,
                                      double* __restrict__ out) {
    if (threadIdx.x < S) {
        double a = 0.0;
        for (int b = 0; b < blocks; ++b) a += partial[(size_t)b * RUDDER_MAX_STREAMS + threadIdx.x];
        out[threadIdx.x] = a;
    }
}

// Dequantized weights out[k][n] = fl32(code[n][k] * w_scale[n]) from the
// packed layout (one thread per (n, k); codes read back from either
// container: split-nibble int4, or the 6-bit E2M3 field of the integer code).
template <int CODES>
__global__ __launch_bounds__(kThreads) void dequant_weights_kernel(
    const uint8_t* __restrict__ Wq, const float* __restrict__ w_scale, int K, int N,
    float* __restrict__ out) {
    const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (size_t)K * N) return;
    const int k = (int)(i / N);
    const int n = (int)(i - (size_t)k * N);
    int code;
    if constexpr (CODES == RUDDER_CODES_E2M3) {
        const uint8_t* blk = Wq + e2m3_block_offset(n, k, K);
        const int slot = e2m3_slot(n, k);
        const int t = k & 31;                      // field t of the slot's 192-bit string
        const int bit = 6 * t;
        // fields 0..21 lie in plane 0 (bits 0..127), 22..31 in plane 1; field
        // 21 straddles them (bits 126..131)
        uint32_t v;
        if (bit + 6 <= 128) {
            const uint8_t* p0 = blk + slot * 16;
            const uint32_t lo = p0[bit >> 3] | ((bit >> 3) + 1 < 16 ? (uint32_t)p0[(bit >> 3) + 1] << 8 : 0u);
            v = (lo >> (bit & 7)) & 0x3Fu;
        } else if (bit >= 128) {
            const uint8_t* p1 = blk + 1024 + slot * 8;
            const int b = bit - 128;
            const uint32_t lo = p1[b >> 3] | ((b >> 3) + 1 < 8 ? (uint32_t)p1[(b >> 3) + 1] << 8 : 0u);
            v = (lo >> (b & 7)) & 0x3Fu;
        } else {
            const uint32_t lo = blk[slot * 16 + 15] >> (bit - 120);          // bits 126..127
            const uint32_t hi = blk[1024 + slot * 8] & 0xFu;                // bits 128..131
            v = (lo | (hi << 2)) & 0x3Fu;
        }
        // E2M3 value of an integer code: exponent field e, mantissa m
        const int e = (v >> 3) & 3, m = v & 7;
        const int mag = e == 0 ? 0 : ((8 + m) << (e - 1)) >> 3;   // (1 + m/8) * 2^(e-1)
        code = (v & 0x20u) ? -mag : mag;
    } else {
        // split-nibble int4 in 32 x 32 tiles: word w of the 16-code slot holds
        // codes 8w..8w+7, byte i = code 8w+i (low nibble), 8w+4+i (high)
        const uint8_t* slotp = Wq + tiled_slot_offset<4>(n, k, K);
        const int j = k & 15;                      // code within the slot
        const int w = j >> 3, c = j & 7;
        const uint8_t byte = slotp[4 * w + (c & 3)];
        const int nib = (c < 4) ? (byte & 0xF) : (byte >> 4);
        code = nib >= 8 ? nib - 16 : nib;
    }
    out[i] = (float)code * w_scale[n];
}

}  // namespace

hipError_t launch_dequant_weights(const uint8_t* Wq, const float* w_scale, int K, int N,
                                  int codes, float* out, hipStream_t stream) {
    const size_t total = (size_t)K * N;
    const unsigned blocks = (unsigned)((total + kThreads - 1) / kThreads);
    if (codes == RUDDER_CODES_E2M3)
        hipLaunchKernelGGL(dequant_weights_kernel<RUDDER_CODES_E2M3>, dim3(blocks),
                           dim3(kThreads), 0, stream, Wq, w_scale, K, N, out);
    else
        hipLaunchKernelGGL(dequant_weights_kernel<RUDDER_CODES_INT>, dim3(blocks),
                           dim3(kThreads), 0, stream, Wq, w_scale, K, N, out);
    return hipGetLastError();
}

size_t stream_sq_error_workspace_bytes() {
    return sizeof(double) * RUDDER_MAX_STREAMS * kMaxBlocks;
}

hipError_t launch_stream_sq_error(const uint16_t* Y, const float* Yref, const uint8_t* sid, int M,
                                  int N, int S, void* workspace, double* sse,
                                  hipStream_t stream) {
    double* partial = static_cast<double*>(workspace);
    int rows_per_block = (M + kMaxBlocks - 1) / kMaxBlocks;
    if (rows_per_block < 1) rows_per_block = 1;
    const int blocks = (M + rows_per_block - 1) / rows_per_block;   // 0 when M = 0
    if (blocks > 0) {
        hipLaunchKernelGGL(stream_sq_error_partial, dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, Y, Yref, sid, M, N, S, rows_per_block, partial);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(stream_sq_error_final, dim3(1), dim3(64), 0, stream, partial, blocks, S,
                       sse);
    return hipGetLastError();
}

}  // namespace rudder
