// Matrix-core ceiling for a given set of packed codes (measurement only).
//
// The matrix cores of this part draw power in proportion to the bit activity
// of their operands, and the chip lowers its clock to stay within its power
// limit: the same MFMA stream runs markedly slower on random operands than on
// zeros.  A GEMM's attainable rate therefore depends on the codes it
// multiplies.  This kernel measures that rate for the codes of a real layer:
// every wave loads fragments of the layer's packed activation and weight
// codes once (the lane-ordered tiled layouts give one contiguous load per
// fragment), then issues the tiled GEMM's per-substep MFMA pattern (2 weight
// x 4 activation fragments, 8 independent accumulators) from registers only,
// once per fragment set (two sets) per iteration.  No LDS, no memory traffic in the
// loop: the result is the MFMA-only rate at the clock these operands allow.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rudder_diag.h"
#include "rudder_internal.h"

namespace rudder {
typedef int mfma_v6i __attribute__((ext_vector_type(6)));
typedef float mfma_v16f __attribute__((ext_vector_type(16)));

// The f8f6f4 scaled MFMA with the 6-dword operands it takes for FP6 formats
// (the same instruction form as the GEMM's).
__device__ mfma_v16f mfma_scale_f32_32x32x64_fp6(mfma_v6i a, mfma_v6i b, mfma_v16f c,
                                                 int cbsz, int blgp, int opsel_a, int scale_a,
                                                 int opsel_b, int scale_b)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v6i32.v6i32");
}  // namespace rudder

namespace rudder {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));


constexpr int kThreads = 256;
constexpr int kFW = 2, kFA = 4, kSets = 2;

// Block index of fragment j (0 .. kSets*(kFW+kFA)-1) of wave w: a fixed
// odd-multiplier hash spread over the available blocks.
__device__ __forceinline__ uint32_t pick_block(uint32_t w, uint32_t j, uint32_t nblocks) {
    uint32_t h = (w * 16u + j) * 2654435761u;
    h ^= h >> 15;
    h *= 2246822519u;
    h ^= h >> 13;
    return h % nblocks;
}

__device__ __forceinline__ v4i widen(uint2 w) {
    return v4i{(int)((w.x << 4) & 0xF0F0F0F0u), (int)(w.x & 0xF0F0F0F0u),
               (int)((w.y << 4) & 0xF0F0F0F0u), (int)(w.y & 0xF0F0F0F0u)};
}

// E8M0 scale bytes 2^0, 2^5 and 2^1 in one word (op_sel picks the byte), as
// the GEMM passes them for 8-bit codes in the E2M3 container.
constexpr int kDigitScaleWord = 127 | (127 + 5) << 8 | (127 + 1) << 16;

// ABITS 8: int8 activations x int4 weights (int8 MFMA); ABITS 4 with
// E2M3 = false: int4 x int4 widened to int8; E2M3: FP6 f8f6f4 MFMA (ABITS
// 8: two MFMAs per product, one per digit plane of the activation codes).
// SHAPE16 (int containers only): the same fragments fed to
// v_mfma_i32_16x16x64_i8 instead, two instructions (half the ops each) per
// 32x32x32 product of the pattern, into 16 independent accumulators, so an
// iteration carries the same op count.
template <int ABITS, bool E2M3, bool SHAPE16 = false>
__global__ __launch_bounds__(kThreads, 2) void mfma_ceiling_kernel(
    const uint8_t* __restrict__ Xq, uint32_t act_blocks, const uint8_t* __restrict__ Wq,
    uint32_t w_blocks, int iters, int32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const uint32_t w = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    int32_t out = 0;
    if constexpr (E2M3 && ABITS == 8) {
        // one set of fragments (both planes of each activation block), run
        // twice per iteration: 16 digit-plane pairs, the same products per
        // iteration as the other forms
        v6i wf[kFW], ah[kFA], al[kFA];
#pragma unroll
        for (int f = 0; f < kFW + kFA; ++f) {
            const bool is_w = f < kFW;
            const uint8_t* blk = is_w ? Wq + (size_t)pick_block(w, f, w_blocks) * 1536
                                      : Xq + (size_t)pick_block(w, f, act_blocks) * 3072;
#pragma unroll
            for (int p = 0; p < (is_w ? 1 : 2); ++p) {
                const uint8_t* b = blk + p * 1536;
                const v4i p0 = *reinterpret_cast<const v4i*>(b + lane * 16);
                const v2i p1 = *reinterpret_cast<const v2i*>(b + 1024 + lane * 8);
                const v6i v = __builtin_shufflevector(
                    p0, __builtin_shufflevector(p1, p1, 0, 1, -1, -1), 0, 1, 2, 3, 4, 5);
                if (is_w) wf[f] = v;
                else if (p == 0) ah[f - kFW] = v;
                else al[f - kFW] = v;
            }
        }
        v16f acc[kFW][kFA] = {};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int s = 0; s < kSets; ++s)
#pragma unroll
                for (int f = 0; f < kFW; ++f)
#pragma unroll
                    for (int g = 0; g < kFA; ++g) {
                        acc[f][g] = mfma_scale_f32_32x32x64_fp6(wf[f], ah[g], acc[f][g], 2, 2, 0,
                                                                kDigitScaleWord, 1,
                                                                kDigitScaleWord);
                        acc[f][g] = mfma_scale_f32_32x32x64_fp6(wf[f], al[g], acc[f][g], 2, 2, 0,
                                                                kDigitScaleWord, 2,
                                                                kDigitScaleWord);
                    }
        }
#pragma unroll
        for (int f = 0; f < kFW; ++f)
#pragma unroll
            for (int g = 0; g < kFA; ++g) out += __float_as_int(acc[f][g][lane & 15]);
    } else if constexpr (E2M3) {
        v6i wf[kSets][kFW], af[kSets][kFA];
#pragma unroll
        for (int s = 0; s < kSets; ++s) {
#pragma unroll
            for (int f = 0; f < kFW + kFA; ++f) {
                const bool is_w = f < kFW;
                const uint8_t* blk =
                    (is_w ? Wq : Xq) +
                    (size_t)pick_block(w, s * (kFW + kFA) + f, is_w ? w_blocks : act_blocks) * 1536;
                const v4i p0 = *reinterpret_cast<const v4i*>(blk + lane * 16);
                const v2i p1 = *reinterpret_cast<const v2i*>(blk + 1024 + lane * 8);
                const v6i v = __builtin_shufflevector(
                    p0, __builtin_shufflevector(p1, p1, 0, 1, -1, -1), 0, 1, 2, 3, 4, 5);
                if (is_w) wf[s][f] = v;
                else af[s][f - kFW] = v;
            }
        }
        v16f acc[kFW][kFA] = {};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int s = 0; s < kSets; ++s)
#pragma unroll
                for (int f = 0; f < kFW; ++f)
#pragma unroll
                    for (int g = 0; g < kFA; ++g)
                        acc[f][g] = mfma_scale_f32_32x32x64_fp6(wf[s][f], af[s][g], acc[f][g],
                                                                2, 2, 0, 127, 0, 127);
        }
#pragma unroll
        for (int f = 0; f < kFW; ++f)
#pragma unroll
            for (int g = 0; g < kFA; ++g) out += __float_as_int(acc[f][g][lane & 15]);
    } else {
        constexpr uint32_t kABlock = ABITS == 8 ? 1024 : 512;
        v4i wf[kSets][kFW], af[kSets][kFA];
#pragma unroll
        for (int s = 0; s < kSets; ++s) {
#pragma unroll
            for (int f = 0; f < kFW; ++f) {
                const uint8_t* blk = Wq + (size_t)pick_block(w, s * (kFW + kFA) + f, w_blocks) * 512;
                wf[s][f] = widen(*reinterpret_cast<const uint2*>(blk + lane * 8));
            }
#pragma unroll
            for (int g = 0; g < kFA; ++g) {
                const uint8_t* blk =
                    Xq + (size_t)pick_block(w, s * (kFW + kFA) + kFW + g, act_blocks) * kABlock;
                if constexpr (ABITS == 8) {
                    const uint4 v = *reinterpret_cast<const uint4*>(blk + lane * 16);
                    af[s][g] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
                } else {
                    af[s][g] = widen(*reinterpret_cast<const uint2*>(blk + lane * 8));
                }
            }
        }
        if constexpr (SHAPE16) {
            v4i acc[kFW][kFA][2] = {};
            for (int it = 0; it < iters; ++it) {
#pragma unroll
                for (int s = 0; s < kSets; ++s)
#pragma unroll
                    for (int f = 0; f < kFW; ++f)
#pragma unroll
                        for (int g = 0; g < kFA; ++g) {
                            acc[f][g][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                                wf[s][f], af[s][g], acc[f][g][0], 0, 0, 0);
                            acc[f][g][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                                af[s][g], wf[s][f], acc[f][g][1], 0, 0, 0);
                        }
            }
#pragma unroll
            for (int f = 0; f < kFW; ++f)
#pragma unroll
                for (int g = 0; g < kFA; ++g) out += acc[f][g][0][lane & 3] + acc[f][g][1][lane & 3];
        } else {
            v16i acc[kFW][kFA] = {};
            for (int it = 0; it < iters; ++it) {
#pragma unroll
                for (int s = 0; s < kSets; ++s)
#pragma unroll
                    for (int f = 0; f < kFW; ++f)
#pragma unroll
                        for (int g = 0; g < kFA; ++g)
                            acc[f][g] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                                wf[s][f], af[s][g], acc[f][g], 0, 0, 0);
            }
#pragma unroll
            for (int f = 0; f < kFW; ++f)
#pragma unroll
                for (int g = 0; g < kFA; ++g) out += acc[f][g][lane & 15];
        }
    }
    sink[blockIdx.x * kThreads + threadIdx.x] = out;
}

}  // namespace

size_t mfma_ceiling_sink_bytes() {
    return (size_t)RUDDER_CEILING_BLOCKS * kThreads * sizeof(int32_t);
}

double mfma_ceiling_ops(int iters, int codes) {
    const double per_mfma = codes == RUDDER_CODES_E2M3 ? 131072.0 : 65536.0;
    return (double)RUDDER_CEILING_BLOCKS * (kThreads / 64) * (double)iters * (kSets * kFW * kFA) *
           per_mfma;
}

hipError_t launch_mfma_ceiling(const uint8_t* Xq, const uint8_t* Wq, int M, int N, int K,
                               int abits, int codes, int iters, int32_t* sink,
                               hipStream_t stream, int shape) {
    const int ksub = codes == RUDDER_CODES_E2M3 ? 64 : 32;
    const uint32_t kb = (uint32_t)(K / ksub);
    const uint32_t act_blocks = (uint32_t)((M + 31) / 32) * kb;
    const uint32_t w_blocks = (uint32_t)(N / 32) * kb;
    const dim3 grid(RUDDER_CEILING_BLOCKS), block(kThreads);
    if (shape == RUDDER_CEILING_I8_16X16X64) {
        if (abits == 8)
            hipLaunchKernelGGL((mfma_ceiling_kernel<8, false, true>), grid, block, 0, stream, Xq,
                               act_blocks, Wq, w_blocks, iters, sink);
        else
            hipLaunchKernelGGL((mfma_ceiling_kernel<4, false, true>), grid, block, 0, stream, Xq,
                               act_blocks, Wq, w_blocks, iters, sink);
        return hipGetLastError();
    }
    if (codes == RUDDER_CODES_E2M3 && abits == 8)
        hipLaunchKernelGGL((mfma_ceiling_kernel<8, true>), grid, block, 0, stream, Xq, act_blocks,
                           Wq, w_blocks, iters, sink);
    else if (codes == RUDDER_CODES_E2M3)
        hipLaunchKernelGGL((mfma_ceiling_kernel<4, true>), grid, block, 0, stream, Xq, act_blocks,
                           Wq, w_blocks, iters, sink);
    else if (abits == 8)
        hipLaunchKernelGGL((mfma_ceiling_kernel<8, false>), grid, block, 0, stream, Xq,
                           act_blocks, Wq, w_blocks, iters, sink);
    else
        hipLaunchKernelGGL((mfma_ceiling_kernel<4, false>), grid, block, 0, stream, Xq,
                           act_blocks, Wq, w_blocks, iters, sink);
    return hipGetLastError();
}

}  // namespace rudder
