// Low-bit GEMM with fused dequantization / compensation epilogue.
//
// SteerQuant ("SteerQuant: Steering Quantization Error with Action-Guided
// Scaling in World-Action Models", paperlayer.ai digest), §4.4 (Rudder): the
// low-bit GEMM consumes only integer activations and per-row scales, and its
// epilogue applies dequantization, inverse-gain compensation and bias, so the
// scaling costs no extra launch and no intermediate HBM round trip (§1).
//
// gfx950 mapping
//   * v_mfma_i32_32x32x32_i8: the MFMA "A" operand is a 32-channel slice of
//     the weights (output channel n = MFMA row i), the "B" operand a 32-row
//     slice of the activations (token m = MFMA column j), so each lane's
//     accumulators hold one token row and runs of 4 consecutive channels.
//   * There is no int4 MFMA.  4-bit codes are widened in registers: the
//     split-nibble word w turns into (w << 4) & 0xF0F0F0F0 and w & 0xF0F0F0F0,
//     i.e. bytes equal to 16 * code, in natural k order.  The int32 result is
//     then 16x (W4A8) or 256x (W4A4) the true accumulator, which is exact for
//     K <= RUDDER_MAX_K and is undone with an arithmetic shift.
//   * Codes arrive in the MFMA-tiled layout, so every global -> LDS copy is a
//     contiguous 16-byte-per-lane stream and every LDS read of a fragment is
//     a contiguous lane-ordered 8- or 16-byte access (no bank conflicts).
#include "rudder_internal.h"

namespace rudder {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 256;          // tokens per block tile
constexpr int BN = 256;          // output channels per block tile
constexpr int BK = 128;          // k per pipeline stage (4 MFMA k-steps)
constexpr int kWaves = 8;        // 2 (n) x 4 (m) waves, wave tile 128 n x 64 m
constexpr int kThreads = 64 * kWaves;

// LDS bytes of one stage
template <int ABITS>
struct Stage {
    static constexpr int kActBlock = 64 * 2 * ABITS;               // 1024 or 512
    static constexpr int kActBytes = (BM / 32) * (BK / 32) * kActBlock;
    static constexpr int kWBlock = 512;
    static constexpr int kWBytes = (BN / 32) * (BK / 32) * kWBlock;
    static constexpr int kActLoads = kActBytes / (16 * kThreads);  // 16-byte loads per thread
    static constexpr int kWLoads = kWBytes / (16 * kThreads);
};

__device__ __forceinline__ v4i widen_nibbles(uint32_t w0, uint32_t w1) {
    v4i r;
    r.x = (int)((w0 << 4) & 0xF0F0F0F0u);
    r.y = (int)(w0 & 0xF0F0F0F0u);
    r.z = (int)((w1 << 4) & 0xF0F0F0F0u);
    r.w = (int)(w1 & 0xF0F0F0F0u);
    return r;
}

template <int ABITS>
__global__ __launch_bounds__(kThreads, 1) void w4_gemm_kernel(
    const uint8_t* __restrict__ Xq, const float* __restrict__ row_scale,
    const uint8_t* __restrict__ sid, const uint8_t* __restrict__ Wq,
    const float* __restrict__ w_scale, const float* __restrict__ comp_a,
    const float* __restrict__ comp_b, int M, int N, int K, uint16_t* __restrict__ Y,
    int32_t* __restrict__ acc_out, int tiles_n) {
    using St = Stage<ABITS>;
    __shared__ __attribute__((aligned(16))) uint8_t lds_act[St::kActBytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds_w[St::kWBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave & 1;          // 128-channel half of the tile
    const int wm = wave >> 1;         // 64-token quarter of the tile

    const int tile_n = blockIdx.x % tiles_n;
    const int tile_m = blockIdx.x / tiles_n;
    const int kblocks = K >> 5;
    const int mblocks = (M + 31) >> 5;
    const int nblocks = N >> 5;

    // ---- global source pointers for this thread's 16-byte chunks --------
    // Activation stage: [mb 0..7][kb 0..3][block]; the 4 k-blocks of one
    // token block are contiguous in both global memory and LDS.
    constexpr int kActPerMb = (BK / 32) * St::kActBlock;     // bytes per token block per stage
    const uint8_t* act_src[St::kActLoads];
    bool act_ok[St::kActLoads];
#pragma unroll
    for (int i = 0; i < St::kActLoads; ++i) {
        const int c = (i * kThreads + tid) * 16;             // byte offset in stage
        const int mb = c / kActPerMb;
        const int rem = c - mb * kActPerMb;
        const int gmb = tile_m * (BM / 32) + mb;
        act_ok[i] = gmb < mblocks;
        act_src[i] = Xq + ((size_t)gmb * kblocks) * St::kActBlock + rem;
    }
    constexpr int kWPerNb = (BK / 32) * St::kWBlock;
    const uint8_t* w_src[St::kWLoads];
    bool w_ok[St::kWLoads];
#pragma unroll
    for (int i = 0; i < St::kWLoads; ++i) {
        const int c = (i * kThreads + tid) * 16;
        const int nb = c / kWPerNb;
        const int rem = c - nb * kWPerNb;
        const int gnb = tile_n * (BN / 32) + nb;
        w_ok[i] = gnb < nblocks;
        w_src[i] = Wq + ((size_t)gnb * kblocks) * St::kWBlock + rem;
    }

    uint4 act_reg[St::kActLoads];
    uint4 w_reg[St::kWLoads];
    auto load_stage = [&](int kt) {
        const size_t act_off = (size_t)kt * kActPerMb;
        const size_t w_off = (size_t)kt * kWPerNb;
#pragma unroll
        for (int i = 0; i < St::kActLoads; ++i)
            act_reg[i] = act_ok[i] ? *reinterpret_cast<const uint4*>(act_src[i] + act_off)
                                   : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < St::kWLoads; ++i)
            w_reg[i] = w_ok[i] ? *reinterpret_cast<const uint4*>(w_src[i] + w_off)
                               : make_uint4(0, 0, 0, 0);
    };
    auto store_stage = [&]() {
#pragma unroll
        for (int i = 0; i < St::kActLoads; ++i)
            *reinterpret_cast<uint4*>(lds_act + (i * kThreads + tid) * 16) = act_reg[i];
#pragma unroll
        for (int i = 0; i < St::kWLoads; ++i)
            *reinterpret_cast<uint4*>(lds_w + (i * kThreads + tid) * 16) = w_reg[i];
    };

    v16i acc[4][2];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][g][r] = 0;

    const int ksteps = K / BK;
    load_stage(0);
    for (int kt = 0; kt < ksteps; ++kt) {
        __syncthreads();                       // previous stage fully consumed
        store_stage();
        __syncthreads();
        if (kt + 1 < ksteps) load_stage(kt + 1);
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            v4i wf[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int nb = wn * 4 + f;
                const uint2 p = *reinterpret_cast<const uint2*>(
                    lds_w + nb * kWPerNb + kk * St::kWBlock + lane * 8);
                wf[f] = widen_nibbles(p.x, p.y);
            }
            v4i af[2];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int mb = wm * 2 + g;
                if constexpr (ABITS == 8) {
                    const uint4 p = *reinterpret_cast<const uint4*>(
                        lds_act + mb * kActPerMb + kk * St::kActBlock + lane * 16);
                    af[g] = v4i{(int)p.x, (int)p.y, (int)p.z, (int)p.w};
                } else {
                    const uint2 p = *reinterpret_cast<const uint2*>(
                        lds_act + mb * kActPerMb + kk * St::kActBlock + lane * 8);
                    af[g] = widen_nibbles(p.x, p.y);
                }
            }
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int g = 0; g < 2; ++g)
                    acc[f][g] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[f], af[g], acc[f][g],
                                                                      0, 0, 0);
        }
    }

    // ---- fused epilogue -------------------------------------------------
    constexpr int kShift = ABITS == 8 ? 4 : 8;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int m = tile_m * BM + wm * 64 + g * 32 + (lane & 31);
        if (m >= M) continue;
        const int s = sid[m] & (RUDDER_MAX_STREAMS - 1);
        const float rs = row_scale[m];
        const float* ca = comp_a + (size_t)s * N;
        const float* cb = comp_b + (size_t)s * N;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int n0 = tile_n * BN + wn * 128 + f * 32;
            if (n0 >= N) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + 8 * q + 4 * (lane >> 5);
                const float4 ws = *reinterpret_cast<const float4*>(w_scale + n);
                const float4 a = *reinterpret_cast<const float4*>(ca + n);
                const float4 b = *reinterpret_cast<const float4*>(cb + n);
                const int v0 = acc[f][g][4 * q + 0] >> kShift;
                const int v1 = acc[f][g][4 * q + 1] >> kShift;
                const int v2 = acc[f][g][4 * q + 2] >> kShift;
                const int v3 = acc[f][g][4 * q + 3] >> kShift;
                const float y0 = __builtin_fmaf(a.x, (float)v0 * (rs * ws.x), b.x);
                const float y1 = __builtin_fmaf(a.y, (float)v1 * (rs * ws.y), b.y);
                const float y2 = __builtin_fmaf(a.z, (float)v2 * (rs * ws.z), b.z);
                const float y3 = __builtin_fmaf(a.w, (float)v3 * (rs * ws.w), b.w);
                uint2 packed;
                packed.x = float_to_bf16_bits(y0) | (float_to_bf16_bits(y1) << 16);
                packed.y = float_to_bf16_bits(y2) | (float_to_bf16_bits(y3) << 16);
                *reinterpret_cast<uint2*>(Y + (size_t)m * N + n) = packed;
                if (acc_out != nullptr)
                    *reinterpret_cast<int4*>(acc_out + (size_t)m * N + n) =
                        make_int4(v0, v1, v2, v3);
            }
        }
    }
}

}  // namespace

hipError_t launch_linear(const void* Xq, const float* row_scale, const uint8_t* sid,
                         const uint8_t* Wq, const float* w_scale, const float* comp_a,
                         const float* comp_b, int M, int N, int K, int S, int abits, uint16_t* Y,
                         int32_t* acc_out, hipStream_t stream) {
    (void)S;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    const uint8_t* xq = static_cast<const uint8_t*>(Xq);
    if (abits == 8)
        hipLaunchKernelGGL(w4_gemm_kernel<8>, grid, dim3(kThreads), 0, stream, xq, row_scale,
                           sid, Wq, w_scale, comp_a, comp_b, M, N, K, Y, acc_out, tiles_n);
    else
        hipLaunchKernelGGL(w4_gemm_kernel<4>, grid, dim3(kThreads), 0, stream, xq, row_scale,
                           sid, Wq, w_scale, comp_a, comp_b, M, N, K, Y, acc_out, tiles_n);
    return hipGetLastError();
}

}  // namespace rudder
