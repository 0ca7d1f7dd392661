// Quantization kernels: offline weight preparation and the fused activation
// quantizer.
//
// SteerQuant ("SteerQuant: Steering Quantization Error with Action-Guided
// Scaling in World-Action Models", paperlayer.ai digest):
//   Fig. 2 / §4.2  -- the shared smoothing diagonal is folded into one static
//                     int4 weight matrix per layer, prepared offline;
//   §4.3 / §4.4    -- activations are scaled (inverse diagonal, per-(stream,
//                     step) step size) inside the activation quantizer, which
//                     emits integer codes plus one scale per row.
//
// Both kernels are HBM-streaming codecs: no MFMA work, coalesced 16-byte
// loads of bf16 and contiguous stores of the MFMA-tiled code layout.
#include <mutex>

#include "rudder_internal.h"

namespace rudder {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxPartials = 1024;          // dynamic-mode partial-absmax blocks

// Code stores of the E2M3 codec (16- and 8-byte pieces of a code block).
__device__ __forceinline__ void store16(uint8_t* p, uint4 v) {
    *reinterpret_cast<uint4*>(p) = v;
}
__device__ __forceinline__ void store8(uint8_t* p, uint2 v) {
    *reinterpret_cast<uint2*>(p) = v;
}

// 16 consecutive floats at a wave-uniform, 16-byte-aligned address, held in
// scalar registers: marking each value wave-uniform keeps the loads scalar
// even when lanes later select between two such groups.
__device__ __forceinline__ void uniform_load16(const float* p, float (&o)[16]) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float4 v = q[j];
        o[4 * j] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v.x)));
        o[4 * j + 1] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v.y)));
        o[4 * j + 2] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v.z)));
        o[4 * j + 3] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v.w)));
    }
}

// ---------------------------------------------------------------------------
// Weight preparation: one block per 32 output channels.
// ---------------------------------------------------------------------------
template <int CODES>
__global__ __launch_bounds__(kThreads) void quantize_weights_kernel(
    const uint16_t* __restrict__ W, const float* __restrict__ smooth, int K, int N,
    uint8_t* __restrict__ Wq, float* __restrict__ w_scale, float* __restrict__ inv_smooth) {
    __shared__ float s_amax[8][32];
    __shared__ float s_inv_w[32];

    const int tid = threadIdx.x;
    const int j = tid & 31;            // channel within the block
    const int g = tid >> 5;            // k interleave group 0..7
    const int n = blockIdx.x * 32 + j;

    // inv_smooth: spread over the whole grid.
    for (int k = blockIdx.x * kThreads + tid; k < K; k += gridDim.x * kThreads)
        inv_smooth[k] = (float)(1.0 / (double)smooth[k]);

    // Column absmax of w' = W * s.
    float amax = 0.0f;
    for (int k = g; k < K; k += 8) {
        float w = bf16_bits_to_float(W[(size_t)k * N + n]) * smooth[k];
        amax = fmaxf(amax, fabsf(w));
    }
    s_amax[g][j] = amax;
    __syncthreads();
    if (g == 0) {
        float a = s_amax[0][j];
#pragma unroll
        for (int i = 1; i < 8; ++i) a = fmaxf(a, s_amax[i][j]);
        float ws = (float)((double)a / 7.0);
        w_scale[n] = ws;
        s_inv_w[j] = step_reciprocal(ws);
    }
    __syncthreads();

    // Codes: slot q -> (channel n0 + q % 32, kSlot k starting at kSlot * (q / 32)).
    constexpr int kSlot = CODES == RUDDER_CODES_E2M3 ? 32 : 16;
    const int slots = 32 * (K / kSlot);
    for (int q = tid; q < slots; q += kThreads) {
        const int jj = q & 31;
        const int nn = blockIdx.x * 32 + jj;
        const int k0 = kSlot * (q >> 5);
        const float iw = s_inv_w[jj];
        float c[kSlot];
#pragma unroll
        for (int i = 0; i < kSlot; ++i) {
            const int k = k0 + i;
            float w = bf16_bits_to_float(W[(size_t)k * N + nn]) * smooth[k];
            c[i] = quantize_clamped_f(w * iw, 7.0f);
        }
        if constexpr (CODES == RUDDER_CODES_E2M3) {
            uint32_t d[6];
            pack_e2m3x32(c, d);
            uint8_t* blk = Wq + e2m3_block_offset(nn, k0, K);
            const int slot = e2m3_slot(nn, k0);
            *reinterpret_cast<uint4*>(blk + slot * 16) = make_uint4(d[0], d[1], d[2], d[3]);
            *reinterpret_cast<uint2*>(blk + 1024 + slot * 8) = make_uint2(d[4], d[5]);
        } else {
            int ci[kSlot];
#pragma unroll
            for (int i = 0; i < kSlot; ++i) ci[i] = (int)c[i];
            uint2 out;
            out.x = split_nibble_word(ci);
            out.y = split_nibble_word(ci + 8);
            *reinterpret_cast<uint2*>(Wq + tiled_slot_offset<4>(nn, k0, K)) = out;
        }
    }
}

// ---------------------------------------------------------------------------
// Activation quantizer.  One wave per 32 x 32 (row, k) block of the tiled
// output: lane l handles row 32rb + l % 32 and the 16 k starting at
// 32kb + 16 (l / 32), so each wave writes one contiguous code block.
// ---------------------------------------------------------------------------
template <int ABITS>
__global__ __launch_bounds__(kThreads) void quant_act_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ sid,
    const float* __restrict__ inv_smooth, const float* __restrict__ delta, int M, int K, int S,
    uint8_t* __restrict__ Xq, float* __restrict__ row_scale) {
    __shared__ float s_delta[RUDDER_MAX_STREAMS];
    __shared__ float s_ia[RUDDER_MAX_STREAMS];
    const int tid = threadIdx.x;
    if (tid < RUDDER_MAX_STREAMS) {
        float d = tid < S ? delta[tid] : 0.0f;
        s_delta[tid] = d;
        s_ia[tid] = step_reciprocal(d);
    }
    __syncthreads();

    const int lane = tid & 63;
    const int kblocks = K >> 5;
    const int total = ((M + 31) >> 5) * kblocks;
    // the block coordinates are wave-uniform (scalar registers), so the 32
    // inverse smoothing factors of the block come through scalar loads and
    // each lane selects its half
    const int gw = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(tid >> 6);
    if (gw >= total) return;
    const int rb = gw / kblocks;
    const int kb = gw - rb * kblocks;
    const int r = rb * 32 + (lane & 31);
    const int k0 = kb * 32 + 16 * (lane >> 5);
    constexpr float Q = ABITS == 8 ? 127.0f : 7.0f;

    int c[16];
    if (r < M) {
        const int s = sid[r] & (RUDDER_MAX_STREAMS - 1);
        const float ia = s_ia[s];
        const uint4* xp = reinterpret_cast<const uint4*>(X + (size_t)r * K + k0);
        const uint4 x0 = xp[0], x1 = xp[1];
        const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        float lo[16], hi[16], is[16];
        uniform_load16(inv_smooth + kb * 32, lo);
        uniform_load16(inv_smooth + kb * 32 + 16, hi);
        const bool upper = lane >= 32;
#pragma unroll
        for (int i = 0; i < 16; ++i) is[i] = upper ? hi[i] : lo[i];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t h = (i & 1) ? (xw[i >> 1] >> 16) : (xw[i >> 1] & 0xFFFFu);
            const float u = bf16_bits_to_float(h) * is[i];
            c[i] = quantize_clamped(u * ia, Q);
        }
        if (kb == 0 && lane < 32) row_scale[r] = s_delta[s];
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) c[i] = 0;
    }

    if constexpr (ABITS == 8) {
        uint4 out;
        out.x = byte_word(c);
        out.y = byte_word(c + 4);
        out.z = byte_word(c + 8);
        out.w = byte_word(c + 12);
        *reinterpret_cast<uint4*>(Xq + tiled_slot_offset<8>(r, k0, K)) = out;
    } else {
        uint2 out;
        out.x = split_nibble_word(c);
        out.y = split_nibble_word(c + 8);
        *reinterpret_cast<uint2*>(Xq + tiled_slot_offset<4>(r, k0, K)) = out;
    }
}

// ---------------------------------------------------------------------------
// Activation quantizer, E2M3 container.  One wave per 32 x 64 (row, k)
// block: lane l handles row 32rb + l % 32 and the 32 k starting at
// 64kb + 32 (l / 32); plane 0 and plane 1 of each 1536-byte block are each
// written contiguously by the wave.  4-bit codes: one block of the codes.
// 8-bit codes q: two blocks, the digits of q = 16 h + l with
// l = ((q + 8) mod 16) - 8 in [-8, 7] and h = (q - l) / 16 in [-8, 8], held
// as the exact E2M3 values h / 2 and l / 2.
// ---------------------------------------------------------------------------
template <int ABITS>
__global__ __launch_bounds__(kThreads) void quant_act_e2m3_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ sid,
    const float* __restrict__ inv_smooth, const float* __restrict__ delta, int M, int K, int S,
    uint8_t* __restrict__ Xq, float* __restrict__ row_scale) {
    __shared__ float s_delta[RUDDER_MAX_STREAMS];
    __shared__ float s_ia[RUDDER_MAX_STREAMS];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int kblocks = K >> 6;
    const int total = ((M + 31) >> 5) * kblocks;
    const int gw = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool active = gw < total;
    const int rb = gw / kblocks;
    const int kb = gw - rb * kblocks;
    const int r = rb * 32 + (lane & 31);
    const int k0 = kb * 64 + 32 * (lane >> 5);

    // The block's bf16 loads go out before the step-size table is built, so
    // their latency overlaps it.
    const bool row = active && r < M;
    uint4 xv[4];
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = make_uint4(0, 0, 0, 0);
    if (row) {
        s = sid[r] & (RUDDER_MAX_STREAMS - 1);
        const uint4* xp = reinterpret_cast<const uint4*>(X + (size_t)r * K + k0);
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[i] = xp[i];
    }
    if (tid < RUDDER_MAX_STREAMS) {
        float d = tid < S ? delta[tid] : 0.0f;
        s_delta[tid] = d;
        s_ia[tid] = step_reciprocal(d);
    }
    __syncthreads();
    if (!active) return;

    float c[32];
    if (row) {
        const float ia = s_ia[s];
        // wave-uniform block: its 64 inverse smoothing factors through scalar
        // loads, each lane selecting its half
        const float* sb = inv_smooth + kb * 64;
        const bool upper = lane >= 32;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4 x0 = xv[2 * h], x1 = xv[2 * h + 1];
            const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            float lo[16], hi[16], is[16];
            uniform_load16(sb + 16 * h, lo);
            uniform_load16(sb + 32 + 16 * h, hi);
#pragma unroll
            for (int i = 0; i < 16; ++i) is[i] = upper ? hi[i] : lo[i];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t hbits = (i & 1) ? (xw[i >> 1] >> 16) : (xw[i >> 1] & 0xFFFFu);
                const float u = bf16_bits_to_float(hbits) * is[i];
                c[16 * h + i] = quantize_clamped_f(u * ia, ABITS == 8 ? 127.0f : 7.0f);
            }
        }
        if (kb == 0 && lane < 32) row_scale[r] = s_delta[s];
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) c[i] = 0.0f;
    }
    // Write-back stores: the codes then sit in the caches when the GEMM
    // that reads them starts (with streaming stores it found them in HBM,
    // and the 8192-deep down-projection ran 14% slower).
    const int slot = e2m3_slot(r, k0);
    if constexpr (ABITS == 8) {
        float ch[32], cl[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int q = (int)c[i];
            const int lo = ((q + 8) & 15) - 8;
            const int hi = (q - lo) / 16;
            ch[i] = (float)hi * 0.5f;
            cl[i] = (float)lo * 0.5f;
        }
        uint32_t dh[6], dl[6];
        pack_e2m3x32(ch, dh);
        pack_e2m3x32(cl, dl);
        uint8_t* blk = Xq + 2 * e2m3_block_offset(r, k0, K);
        store16(blk + slot * 16, make_uint4(dh[0], dh[1], dh[2], dh[3]));
        store8(blk + 1024 + slot * 8, make_uint2(dh[4], dh[5]));
        store16(blk + 1536 + slot * 16, make_uint4(dl[0], dl[1], dl[2], dl[3]));
        store8(blk + 1536 + 1024 + slot * 8, make_uint2(dl[4], dl[5]));
    } else {
        uint32_t d[6];
        pack_e2m3x32(c, d);
        uint8_t* blk = Xq + e2m3_block_offset(r, k0, K);
        store16(blk + slot * 16, make_uint4(d[0], d[1], d[2], d[3]));
        store8(blk + 1024 + slot * 8, make_uint2(d[4], d[5]));
    }
}

// ---------------------------------------------------------------------------
// Dynamic step sizes: per-stream absmax of u = X * inv_smooth.
// Pass 1: each block reduces its grid-stride share into partial[block][s]
// (wave-level butterfly reductions, then across the block's waves in LDS).
// Pass 2: one block folds the partials and forms D[s] = fl32(amax_s / Qa).
// max is order-independent, so the result is deterministic.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__global__ __launch_bounds__(kThreads) void act_absmax_partial_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ sid,
    const float* __restrict__ inv_smooth, int M, int K, float* __restrict__ partial) {
    __shared__ float s_red[kThreads / 64][RUDDER_MAX_STREAMS];
    float amax[RUDDER_MAX_STREAMS];
#pragma unroll
    for (int s = 0; s < RUDDER_MAX_STREAMS; ++s) amax[s] = 0.0f;

    const int chunks_per_row = K >> 4;
    const long total = (long)M * chunks_per_row;
    for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (long)gridDim.x * kThreads) {
        const int m = (int)(i / chunks_per_row);
        const int k0 = (int)(i - (long)m * chunks_per_row) * 16;
        const uint4* xp = reinterpret_cast<const uint4*>(X + (size_t)m * K + k0);
        const uint4 x0 = xp[0], x1 = xp[1];
        const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        float cmax = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t h = (e & 1) ? (xw[e >> 1] >> 16) : (xw[e >> 1] & 0xFFFFu);
            cmax = fmaxf(cmax, fabsf(bf16_bits_to_float(h) * inv_smooth[k0 + e]));
        }
        const int s = sid[m] & (RUDDER_MAX_STREAMS - 1);
#pragma unroll
        for (int t = 0; t < RUDDER_MAX_STREAMS; ++t)
            if (t == s) amax[t] = fmaxf(amax[t], cmax);
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int s = 0; s < RUDDER_MAX_STREAMS; ++s) {
        const float v = wave_max(amax[s]);
        if (lane == 0) s_red[wave][s] = v;
    }
    __syncthreads();
    if (threadIdx.x < RUDDER_MAX_STREAMS) {
        float v = s_red[0][threadIdx.x];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) v = fmaxf(v, s_red[w][threadIdx.x]);
        partial[blockIdx.x * RUDDER_MAX_STREAMS + threadIdx.x] = v;
    }
}

__global__ __launch_bounds__(kThreads) void act_scale_finalize_kernel(
    const float* __restrict__ partial, int nparts, int S, float qa, float* __restrict__ delta,
    float* __restrict__ act_scale_out) {
    __shared__ float s_red[kThreads / 64][RUDDER_MAX_STREAMS];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int s = 0; s < RUDDER_MAX_STREAMS; ++s) {
        float v = 0.0f;
        for (int p = threadIdx.x; p < nparts; p += kThreads)
            v = fmaxf(v, partial[p * RUDDER_MAX_STREAMS + s]);
        v = wave_max(v);
        if (lane == 0) s_red[wave][s] = v;
    }
    __syncthreads();
    if (threadIdx.x < RUDDER_MAX_STREAMS) {
        float v = s_red[0][threadIdx.x];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) v = fmaxf(v, s_red[w][threadIdx.x]);
        const float d = (float)((double)v / (double)qa);
        delta[threadIdx.x] = d;
        if (act_scale_out != nullptr && threadIdx.x < S) act_scale_out[threadIdx.x] = d;
    }
}

}  // namespace

size_t quant_act_workspace_bytes() {
    return sizeof(float) * RUDDER_MAX_STREAMS * (kMaxPartials + 1);
}

hipError_t launch_quantize_weights(const uint16_t* W, const float* smooth, int K, int N,
                                   int codes, uint8_t* Wq, float* w_scale, float* inv_smooth,
                                   hipStream_t stream) {
    if (codes == RUDDER_CODES_E2M3)
        hipLaunchKernelGGL(quantize_weights_kernel<RUDDER_CODES_E2M3>, dim3(N / 32),
                           dim3(kThreads), 0, stream, W, smooth, K, N, Wq, w_scale, inv_smooth);
    else
        hipLaunchKernelGGL(quantize_weights_kernel<RUDDER_CODES_INT>, dim3(N / 32),
                           dim3(kThreads), 0, stream, W, smooth, K, N, Wq, w_scale, inv_smooth);
    return hipGetLastError();
}

hipError_t launch_quant_act_static(const uint16_t* X, const uint8_t* sid, const float* inv_smooth,
                                   const float* delta, int M, int K, int S, int abits, int codes,
                                   void* Xq, float* row_scale, hipStream_t stream) {
    if (codes == RUDDER_CODES_E2M3) {
        const long waves = (long)((M + 31) / 32) * (K / 64);
        const dim3 grid((unsigned)((waves + 3) / 4));
        if (abits == 8)
            hipLaunchKernelGGL(quant_act_e2m3_kernel<8>, grid, dim3(kThreads), 0, stream, X, sid,
                               inv_smooth, delta, M, K, S, static_cast<uint8_t*>(Xq), row_scale);
        else
            hipLaunchKernelGGL(quant_act_e2m3_kernel<4>, grid, dim3(kThreads), 0, stream, X, sid,
                               inv_smooth, delta, M, K, S, static_cast<uint8_t*>(Xq), row_scale);
        return hipGetLastError();
    }
    const long waves = (long)((M + 31) / 32) * (K / 32);
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (abits == 8)
        hipLaunchKernelGGL(quant_act_kernel<8>, grid, dim3(kThreads), 0, stream, X, sid,
                           inv_smooth, delta, M, K, S, static_cast<uint8_t*>(Xq), row_scale);
    else
        hipLaunchKernelGGL(quant_act_kernel<4>, grid, dim3(kThreads), 0, stream, X, sid,
                           inv_smooth, delta, M, K, S, static_cast<uint8_t*>(Xq), row_scale);
    return hipGetLastError();
}

hipError_t launch_quant_act_dynamic(const uint16_t* X, const uint8_t* sid,
                                    const float* inv_smooth, float* act_scale_out,
                                    void* workspace, int M, int K, int S, int abits, int codes,
                                    void* Xq, float* row_scale, hipStream_t stream) {
    float* partial = static_cast<float*>(workspace);
    float* delta = partial + (size_t)kMaxPartials * RUDDER_MAX_STREAMS;
    const long chunks = (long)M * (K / 16);
    long nb = (chunks + kThreads - 1) / kThreads;
    if (nb > kMaxPartials) nb = kMaxPartials;
    if (nb < 1) nb = 1;
    hipLaunchKernelGGL(act_absmax_partial_kernel, dim3((unsigned)nb), dim3(kThreads), 0, stream,
                       X, sid, inv_smooth, M, K, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(act_scale_finalize_kernel, dim3(1), dim3(kThreads), 0, stream, partial,
                       (int)nb, S, abits == 8 ? 127.0f : 7.0f, delta, act_scale_out);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_quant_act_static(X, sid, inv_smooth, delta, M, K, S, abits, codes, Xq,
                                   row_scale, stream);
}

}  // namespace rudder

// ---------------------------------------------------------------------------
// Scratch of the no-allocation dynamic-mode entry point: the partial maxima
// and step sizes that rudder_quant_act keeps in its caller's workspace
// (RUDDER_MAX_STREAMS * (kMaxPartials + 1) floats, the same layout).  Each
// GPU holds its own copy until the process ends; every call on a GPU shares
// it, so calls that overlap on one GPU race.  Nothing in it has to start at
// zero: each call writes every partial it reads.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[RUDDER_MAX_STREAMS * (1024 + 1)];

namespace rudder {
namespace {

static_assert(sizeof(scratch) == sizeof(float) * RUDDER_MAX_STREAMS * (kMaxPartials + 1),
              "scratch holds the dynamic-mode workspace");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.  In host code the array's
// name is only a host-side stand-in, so kernels get this address instead.
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

size_t quant_act_noalloc_scratch_bytes() { return sizeof(scratch); }

hipError_t launch_quant_act_dynamic_noalloc(const uint16_t* X, const uint8_t* sid,
                                            const float* inv_smooth, float* act_scale_out,
                                            int M, int K, int S, int abits, int codes, void* Xq,
                                            float* row_scale, hipStream_t stream) {
    void* ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    return launch_quant_act_dynamic(X, sid, inv_smooth, act_scale_out, ws, M, K, S, abits, codes,
                                    Xq, row_scale, stream);
}

}  // namespace rudder
