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
//     the weights (output channel n = MFMA row i), the "B" operand a 32-token
//     slice of the activations (token m = MFMA column j), so each lane's
//     accumulators hold one token row and runs of 4 consecutive channels.
//   * There is no int4 MFMA.  4-bit codes are widened in registers: the
//     split-nibble word w becomes (w << 4) & 0xF0F0F0F0 and w & 0xF0F0F0F0,
//     bytes equal to 16 * code in natural k order.  The int32 result is then
//     16x (W4A8) or 256x (W4A4) the true accumulator -- exact for
//     K <= RUDDER_MAX_K -- and an arithmetic shift undoes it.
//   * Codes arrive MFMA-tiled (32 x 32 blocks in lane order), so global ->
//     LDS traffic uses the gfx950 direct-to-LDS 16-byte loads (no VGPR
//     staging, one contiguous KiB per wave instruction) into an NS-stage LDS
//     ring, and every fragment read is a contiguous lane-ordered ds_read.
//   * One workgroup barrier per k-stage: loads for stage kt+NS-1 are issued
//     right after the barrier that retires stage kt-1's buffer.
//   * Epilogue: dequantize + compensate in registers, stage the bf16 tile in
//     LDS (XOR-swizzled 16-byte chunks), then store whole 512-byte row
//     segments with 16-byte stores so every HBM line is written once.
//   * E2M3 container (W4A4): 4-bit codes held as FP6 E2M3 feed
//     v_mfma_scale_f32_32x32x64_f8f6f4 directly (unit scales): no widening, and
//     twice the int8 rate.  Products of codes are small integers and every
//     fp32 partial sum is an integer below 2^24, so the fp32 accumulator holds
//     the exact integer dot product.
//   * Tile order: workgroups are dealt round-robin to the 8 XCDs; the grid is
//     remapped so each XCD walks a contiguous, m-grouped range of tiles and
//     the tiles in flight on one XCD share activation and weight panels in
//     that XCD's L2.
#include <type_traits>

#include "rudder_internal.h"

namespace rudder {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int BM = 128;          // tokens per block tile
constexpr int BN = 256;          // output channels per block tile
constexpr int BK = 128;          // k per pipeline stage (4 MFMA k-steps)
constexpr int kWavesN = 4;       // waves along the channel dimension
constexpr int kWavesM = 1;       // waves along the token dimension
constexpr int kBlocksPerCU = 2;  // two independent workgroups share each CU
constexpr int kWaves = kWavesN * kWavesM;
constexpr int kThreads = 64 * kWaves;
constexpr int FW = BN / kWavesN / 32;   // 32-channel fragments per wave (2)
constexpr int FA = BM / kWavesM / 32;   // 32-token fragments per wave (4)
constexpr int kXcds = 8;
constexpr int kGroupM = 8;       // m-tiles per tile group (L2 reuse of weight panels)

// Code formats of the GEMM.
constexpr int kFmtA8 = 0;        // int8 activations, int4 weights (int8 MFMA)
constexpr int kFmtA4 = 1;        // int4 activations and weights (int8 MFMA)
constexpr int kFmtF6 = 2;        // 4-bit codes held as E2M3 (f8f6f4 MFMA)

// Six dwords of one E2M3 fragment (plane 0: 16 bytes, plane 1: 8 bytes).
struct F6Frag {
    uint4 p0;
    uint2 p1;
};

template <int FMT>
struct Fmt;
template <>
struct Fmt<kFmtA8> {
    static constexpr int kKSub = 32;       // k per MFMA
    static constexpr int kABlock = 1024;   // bytes per 32-row x kKSub code block
    static constexpr int kWBlock = 512;
    static constexpr int kReadAhead = 2;   // substeps of fragment read-ahead
    typedef uint2 WFrag;
    typedef uint4 AFrag;
    typedef v16i Acc;
};
template <>
struct Fmt<kFmtA4> {
    static constexpr int kKSub = 32;
    static constexpr int kABlock = 512;
    static constexpr int kWBlock = 512;
    static constexpr int kReadAhead = 2;
    typedef uint2 WFrag;
    typedef uint2 AFrag;
    typedef v16i Acc;
};
template <>
struct Fmt<kFmtF6> {
    static constexpr int kKSub = 64;
    static constexpr int kABlock = 1536;
    static constexpr int kWBlock = 1536;
    static constexpr int kReadAhead = 1;
    typedef F6Frag WFrag;
    typedef F6Frag AFrag;
    typedef v16f Acc;
};

template <int FMT, int NS>
struct Cfg {
    using F = Fmt<FMT>;
    static constexpr int kActBlock = F::kABlock;
    static constexpr int kActPerMb = (BK / F::kKSub) * kActBlock;    // per 32-token block
    static constexpr int kActBytes = (BM / 32) * kActPerMb;
    static constexpr int kWBlock = F::kWBlock;
    static constexpr int kWPerNb = (BK / F::kKSub) * kWBlock;        // per 32-channel block
    static constexpr int kWBytes = (BN / 32) * kWPerNb;
    static constexpr int kStageBytes = kActBytes + kWBytes;
    static constexpr int kRingBytes = NS * kStageBytes;
    // 16-byte direct loads per thread per stage (each wave instruction = 1 KiB)
    static constexpr int kActLoads = kActBytes / (1024 * kWaves);
    static constexpr int kWLoads = kWBytes / (1024 * kWaves);
    static constexpr int kLoads = kActLoads + kWLoads;
    static constexpr int kEpiBytes = BM * BN * 2;                    // bf16 tile
    // Per-tile epilogue tables (w_scale, comp_a[S], comp_b[S] for the tile's
    // 256 channels, 1 KiB each) live after both the ring and the bf16 tile.
    static constexpr int kTableOffset = kRingBytes > kEpiBytes ? kRingBytes : kEpiBytes;
    static constexpr int lds_bytes(int S) { return kTableOffset + (1 + 2 * S) * 1024; }
};

// LDS per workgroup: the 160 KiB of a gfx950 CU shared by kBlocksPerCU.
constexpr int kLdsLimit = 160 * 1024 / kBlocksPerCU;

__device__ __forceinline__ v4i widen_nibbles(uint32_t w0, uint32_t w1) {
    v4i r;
    r.x = (int)((w0 << 4) & 0xF0F0F0F0u);
    r.y = (int)(w0 & 0xF0F0F0F0u);
    r.z = (int)((w1 << 4) & 0xF0F0F0F0u);
    r.w = (int)(w1 & 0xF0F0F0F0u);
    return r;
}

// Two fp32 -> packed bf16 with round-to-nearest-even (gfx950 hardware
// conversion; finite inputs): low half = a, high half = b.
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float a, float b) {
    uint32_t r;
    asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Direct-to-LDS 16-byte load: lane l reads 16 bytes at sbase + voff(l)
// (wave-uniform 64-bit base in SGPRs, 32-bit per-lane offset) and the wave
// writes them lane-linearly at LDS offset `lds` (M0).  Written as inline asm
// so the compiler does not add its own conservative vmcnt waits in front of
// LDS reads; the kernel orders these loads itself with wait_and_barrier().
// The instruction has no VGPR results.
__device__ __forceinline__ void load_lds16(const void* base, uint32_t voff, uint32_t lds) {
    // the base is wave-uniform by construction; make that explicit so it
    // is always held in SGPRs
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const void* sbase = reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
    const uint32_t slds = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(slds)
                 : "memory");
}

// Wait until this wave's LDS reads are complete and at most N of its
// vector-memory loads are in flight, then barrier the workgroup: afterwards
// every wave's loads up to that point have landed in LDS, and no wave still
// reads the buffer that the next loads overwrite.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

template <int L>
__device__ __forceinline__ void wait_stages_and_barrier(int stages_in_flight) {
    // stages_in_flight is 0..4
    if (stages_in_flight >= 4) wait_and_barrier<4 * L>();
    else if (stages_in_flight == 3) wait_and_barrier<3 * L>();
    else if (stages_in_flight == 2) wait_and_barrier<2 * L>();
    else if (stages_in_flight == 1) wait_and_barrier<L>();
    else wait_and_barrier<0>();
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}

// Map the linear workgroup id to (tile_m, tile_n): XCD-contiguous ranges,
// then groups of kGroupM m-tiles walked column by column.
__device__ __forceinline__ void tile_of_block(int bid, int nblk, int tiles_m, int tiles_n,
                                              int& tm, int& tn) {
    const int xcd = bid % kXcds;
    const int idx = bid / kXcds;
    const int per = nblk / kXcds;
    const int extra = nblk % kXcds;
    const int t = xcd * per + (xcd < extra ? xcd : extra) + idx;
    const int group = t / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gm = min(kGroupM, tiles_m - first_m);
    const int local = t - group * (kGroupM * tiles_n);
    tm = first_m + local % gm;
    tn = local / gm;
}

// Raw (still packed) fragment words of one k-substep.
template <int FMT>
struct RawFrags {
    typename Fmt<FMT>::WFrag w[FW];                 // channel blocks
    typename Fmt<FMT>::AFrag a[FA];                 // token blocks
};

template <typename T>
__device__ __forceinline__ void read_frag(const uint8_t* block, int lane, T& out);
template <>
__device__ __forceinline__ void read_frag<uint2>(const uint8_t* block, int lane, uint2& out) {
    out = *reinterpret_cast<const uint2*>(block + lane * 8);
}
template <>
__device__ __forceinline__ void read_frag<uint4>(const uint8_t* block, int lane, uint4& out) {
    out = *reinterpret_cast<const uint4*>(block + lane * 16);
}
template <>
__device__ __forceinline__ void read_frag<F6Frag>(const uint8_t* block, int lane, F6Frag& out) {
    out.p0 = *reinterpret_cast<const uint4*>(block + lane * 16);
    out.p1 = *reinterpret_cast<const uint2*>(block + 1024 + lane * 8);
}

template <int FMT, int NS>
__device__ __forceinline__ void read_frags(const uint8_t* stage, int kk, int wn, int wm,
                                           int lane, RawFrags<FMT>& fr) {
    using C = Cfg<FMT, NS>;
    const uint8_t* wst = stage + C::kActBytes;
#pragma unroll
    for (int f = 0; f < FW; ++f)
        read_frag(wst + (wn * FW + f) * C::kWPerNb + kk * C::kWBlock, lane, fr.w[f]);
#pragma unroll
    for (int g = 0; g < FA; ++g)
        read_frag(stage + (wm * FA + g) * C::kActPerMb + kk * C::kActBlock, lane, fr.a[g]);
}

__device__ __forceinline__ v8i f6_operand(const F6Frag& f) {
    return v8i{(int)f.p0.x, (int)f.p0.y, (int)f.p0.z, (int)f.p0.w, (int)f.p1.x, (int)f.p1.y,
               0, 0};
}

// One k-substep: widen 4-bit fragments where needed and issue the FW x FA
// MFMAs of the wave tile.
template <int FMT>
__device__ __forceinline__ void mma_substep(const RawFrags<FMT>& fr,
                                            typename Fmt<FMT>::Acc (&acc)[FW][FA]) {
    if constexpr (FMT == kFmtF6) {
        v8i wf[FW], af[FA];
#pragma unroll
        for (int f = 0; f < FW; ++f) wf[f] = f6_operand(fr.w[f]);
#pragma unroll
        for (int g = 0; g < FA; ++g) af[g] = f6_operand(fr.a[g]);
        // formats: 2 = FP6 E2M3 for both operands; scales 127 = 2^0 (E8M0)
#pragma unroll
        for (int f = 0; f < FW; ++f)
#pragma unroll
            for (int g = 0; g < FA; ++g)
                acc[f][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    wf[f], af[g], acc[f][g], 2, 2, 0, 127, 0, 127);
    } else {
        v4i wf[FW], af[FA];
#pragma unroll
        for (int f = 0; f < FW; ++f) wf[f] = widen_nibbles(fr.w[f].x, fr.w[f].y);
#pragma unroll
        for (int g = 0; g < FA; ++g) {
            if constexpr (FMT == kFmtA8)
                af[g] = v4i{(int)fr.a[g].x, (int)fr.a[g].y, (int)fr.a[g].z, (int)fr.a[g].w};
            else
                af[g] = widen_nibbles(fr.a[g].x, fr.a[g].y);
        }
#pragma unroll
        for (int f = 0; f < FW; ++f)
#pragma unroll
            for (int g = 0; g < FA; ++g)
                acc[f][g] =
                    __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[f], af[g], acc[f][g], 0, 0, 0);
    }
}

// Exact integer value of an accumulator element (the int8 path carries 16x
// (W4A8) or 256x (W4A4) the true sum, see widen_nibbles).
template <int FMT>
__device__ __forceinline__ int acc_value(const typename Fmt<FMT>::Acc& a, int r) {
    if constexpr (FMT == kFmtF6) return (int)a[r];
    else if constexpr (FMT == kFmtA8) return a[r] >> 4;
    else return a[r] >> 8;
}

template <int FMT, int NS, bool ACC_OUT>
__global__ __launch_bounds__(kThreads, kBlocksPerCU) void w4_gemm_kernel(
    const uint8_t* __restrict__ Xq, const float* __restrict__ row_scale,
    const uint8_t* __restrict__ sid, const uint8_t* __restrict__ Wq,
    const float* __restrict__ w_scale, const float* __restrict__ comp_a,
    const float* __restrict__ comp_b, int M, int N, int K, int S, uint16_t* __restrict__ Y,
    int32_t* __restrict__ acc_out, int tiles_m, int tiles_n) {
    using C = Cfg<FMT, NS>;
    using F = Fmt<FMT>;
    constexpr int L = C::kLoads;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave % kWavesN;    // channel slice of the tile (FW * 32 channels)
    const int wm = wave / kWavesN;    // token slice of the tile (FA * 32 tokens)
    const int uwave = __builtin_amdgcn_readfirstlane(wave);   // wave index as a scalar

    int tile_m, tile_n;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, tile_m, tile_n);
    const int kblocks = K / F::kKSub;                       // code blocks along k
    const int mblocks = (M + 31) >> 5;
    const int nblocks = N >> 5;
    const int ksteps = K / BK;
    const int n_tile0 = min(tile_n * BN, N - 32);            // first channel of the tile (clamped)

    // Row data of this lane's two token rows, fetched before the main loop
    // (plain loads; the compiler waits for them only in the epilogue).
    int row_stream[FA];
    float row_rs[FA];
#pragma unroll
    for (int g = 0; g < FA; ++g) {
        const int mc = min(tile_m * BM + wm * (FA * 32) + g * 32 + (lane & 31), M - 1);
        row_stream[g] = sid[mc] & (RUDDER_MAX_STREAMS - 1);
        row_rs[g] = row_scale[mc];
    }

    // ---- epilogue tables -> LDS (one KiB per table row, one wave each) ----
    // row 0: w_scale, rows 1..S: comp_a[s], rows S+1..2S: comp_b[s], each for
    // channels n_tile0 .. n_tile0 + 255 (a tile narrower than 256 channels
    // reads past its last channel only within the same row of the table
    // when N >= 256; narrower matrices clamp the window to the last 256).
    const uint32_t lds_base = lds_offset(lds);
    {
        const int nwin = N >= BN ? min(n_tile0, N - BN) : 0;
        const int cols = N >= BN ? BN : N;                   // columns present in the window
        const int per_lane = cols * 4 / 64;                  // bytes per lane (16 when cols = 256)
        for (int r = uwave; r < 1 + 2 * S; r += kWaves) {
            const float* src = r == 0 ? w_scale
                             : (r <= S ? comp_a + (size_t)(r - 1) * N
                                       : comp_b + (size_t)(r - 1 - S) * N);
            const uint32_t dst = lds_base + C::kTableOffset + r * 1024;
            if (per_lane == 16) {
                load_lds16(src + nwin, lane * 16, __builtin_amdgcn_readfirstlane(dst));
            } else {
                // N < 256: plain loads (rare, small layers)
                for (int c = lane; c < cols; c += 64)
                    reinterpret_cast<float*>(lds + C::kTableOffset + r * 1024)[c] = src[c];
            }
        }
    }

    // ---- per-wave direct-load sources ------------------------------------
    // Each wave instruction moves one contiguous KiB: for activations the
    // (32-token block, k-block) pairs of this stage, for weights the
    // (32-channel block, k-block) pairs.  Bases are wave-uniform (SGPRs);
    // every lane adds lane * 16.  Token / channel blocks past the matrix edge
    // are clamped to the last real block (their results are never stored).
    const uint32_t voff = lane * 16;
    const uint8_t* act_src[C::kActLoads];
    int act_dst[C::kActLoads];
#pragma unroll
    for (int i = 0; i < C::kActLoads; ++i) {
        const int byte = (uwave * C::kActLoads + i) * 1024;   // offset within the stage
        const int mb = byte / C::kActPerMb;
        const int rem = byte - mb * C::kActPerMb;
        const int gmb = min(tile_m * (BM / 32) + mb, mblocks - 1);
        act_src[i] = Xq + (size_t)gmb * kblocks * C::kActBlock + rem;
        act_dst[i] = byte;
    }
    const uint8_t* w_src[C::kWLoads];
    int w_dst[C::kWLoads];
#pragma unroll
    for (int i = 0; i < C::kWLoads; ++i) {
        const int byte = (uwave * C::kWLoads + i) * 1024;
        const int nb = byte / C::kWPerNb;
        const int rem = byte - nb * C::kWPerNb;
        const int gnb = min(tile_n * (BN / 32) + nb, nblocks - 1);
        w_src[i] = Wq + (size_t)gnb * kblocks * C::kWBlock + rem;
        w_dst[i] = C::kActBytes + byte;
    }

    auto issue_stage = [&](int kt) {
        const uint32_t base = lds_base + (uint32_t)((kt % NS) * C::kStageBytes);
        const size_t a_off = (size_t)kt * C::kActPerMb;
        const size_t w_off = (size_t)kt * C::kWPerNb;
#pragma unroll
        for (int i = 0; i < C::kActLoads; ++i)
            load_lds16(act_src[i] + a_off, voff, base + act_dst[i]);
#pragma unroll
        for (int i = 0; i < C::kWLoads; ++i)
            load_lds16(w_src[i] + w_off, voff, base + w_dst[i]);
    };

    typename F::Acc acc[FW][FA];
#pragma unroll
    for (int f = 0; f < FW; ++f)
#pragma unroll
        for (int g = 0; g < FA; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][g][r] = 0;

    // ---- main loop ----------------------------------------------------------
    // Prologue: fill all NS buffers, wait for stage 0.
    const int pre = min(NS, ksteps);
    for (int s = 0; s < pre; ++s) issue_stage(s);
    wait_stages_and_barrier<L>(pre - 1);

    // Fragments are read one k-substep ahead of the MFMAs that use them.  The
    // barrier that admits stage kt+1 sits after the reads of stage kt's last
    // substep and before its MFMAs, so the MFMA pipe has work queued while
    // the workgroup synchronizes and the next stage's first fragments load.
    // Fragments are read D k-substeps ahead of the MFMAs that use them
    // (global substep j = kt * P + kk uses register set fr[j % NSETS]).  The
    // barrier that admits stage kt+1 sits right before the first read of
    // that stage, after every read of stage kt, so the MFMA pipe still has
    // queued substeps while the workgroup synchronizes.
    constexpr int P = BK / F::kKSub;                 // substeps per stage
    constexpr int D = F::kReadAhead;                 // read-ahead distance
    constexpr int NSETS = 2 * D;                     // register sets in rotation
    constexpr int U = NSETS / P;                     // stages per unrolled iteration
    static_assert(U >= 1 && P * U == NSETS && D <= P, "substep bookkeeping");
    RawFrags<FMT> fr[NSETS];
#pragma unroll
    for (int j = 0; j < D; ++j)
        read_frags<FMT, NS>(lds + (j / P) * C::kStageBytes, j % P, wn, wm, lane, fr[j]);
    for (int kt0 = 0; kt0 < ksteps; kt0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kt = kt0 + u;
            if (kt < ksteps) {
#pragma unroll
                for (int kk = 0; kk < P; ++kk) {
                    const int j = u * P + kk;                // substep index mod NSETS
                    const int ahead = kk + D;                // substep to read, relative to stage kt
                    const int rk = ahead % P;
                    const int rst = kt + ahead / P;          // its stage
                    if (rst < ksteps) {
                        if (ahead / P == 1 && rk == 0) {
                            // first read of stage kt+1: admit it, refill the ring
                            wait_stages_and_barrier<L>(min(NS - 2, ksteps - 2 - kt));
                            if (kt + NS < ksteps) issue_stage(kt + NS);
                        }
                        read_frags<FMT, NS>(lds + (rst % NS) * C::kStageBytes, rk, wn, wm, lane,
                                            fr[(j + D) % NSETS]);
                    }
                    mma_substep<FMT>(fr[j], acc);
                }
            }
        }
    }

    // ---- fused epilogue -------------------------------------------------
    // 1. registers: t = float(acc) * (row_scale * w_scale); y = fma(a, t, b);
    //    bf16 (hardware round-to-nearest-even pack) into this wave's LDS
    //    staging area [FA*32 token rows][FW*32 channels]; 16-byte chunk c of
    //    row r sits at chunk c ^ ((r >> 1) & 7).  Per-channel values come
    //    from the LDS tables.
    // 2. each wave stores its own rows: 8 lanes per 128-byte row, so every
    //    store instruction writes whole cache lines.
    constexpr int kWaveRowBytes = FW * 32 * 2;                 // 128
    constexpr int kWaveRows = FA * 32;                         // 128
    __syncthreads();                                   // ring no longer read
    const float* tab = reinterpret_cast<const float*>(lds + C::kTableOffset);
    const int tab_shift = tile_n * BN - (N >= BN ? min(n_tile0, N - BN) : 0);
    uint8_t* wstage = lds + wave * (kWaveRows * kWaveRowBytes);
#pragma unroll
    for (int f = 0; f < FW; ++f) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int nl = wn * (FW * 32) + f * 32 + 8 * q + 4 * (lane >> 5);  // channel in tile
            const int ti = min(nl + tab_shift, 252);           // column in the table window
            const float4 ws = *reinterpret_cast<const float4*>(tab + ti);
            const int chunk = f * 4 + q;                       // 16-byte chunk in the wave row
#pragma unroll
            for (int g = 0; g < FA; ++g) {
                const int s = row_stream[g];
                const float rs = row_rs[g];
                const float4 a = *reinterpret_cast<const float4*>(tab + 256 * (1 + s) + ti);
                const float4 b = *reinterpret_cast<const float4*>(tab + 256 * (1 + S + s) + ti);
                const int v0 = acc_value<FMT>(acc[f][g], 4 * q + 0);
                const int v1 = acc_value<FMT>(acc[f][g], 4 * q + 1);
                const int v2 = acc_value<FMT>(acc[f][g], 4 * q + 2);
                const int v3 = acc_value<FMT>(acc[f][g], 4 * q + 3);
                const float y0 = __builtin_fmaf(a.x, (float)v0 * (rs * ws.x), b.x);
                const float y1 = __builtin_fmaf(a.y, (float)v1 * (rs * ws.y), b.y);
                const float y2 = __builtin_fmaf(a.z, (float)v2 * (rs * ws.z), b.z);
                const float y3 = __builtin_fmaf(a.w, (float)v3 * (rs * ws.w), b.w);
                uint2 packed;
                packed.x = pack_bf16x2_rne(y0, y1);
                packed.y = pack_bf16x2_rne(y2, y3);
                const int r = g * 32 + (lane & 31);
                *reinterpret_cast<uint2*>(wstage + r * kWaveRowBytes +
                                          ((chunk ^ ((r >> 1) & 7)) * 16) + (lane >> 5) * 8) =
                    packed;
                if constexpr (ACC_OUT) {
                    const int m = tile_m * BM + wm * kWaveRows + r;
                    const int n = tile_n * BN + nl;
                    if (m < M && n < N)
                        *reinterpret_cast<int4*>(acc_out + (size_t)m * N + n) =
                            make_int4(v0, v1, v2, v3);
                }
            }
        }
        // keep the accumulator reads of one fragment column together
        // (bounds the registers the epilogue needs)
        __builtin_amdgcn_sched_barrier(0);
    }
    // 2. whole-line stores of this wave's rows (its own LDS writes are
    //    ordered before these reads)
    const int c = lane & 7;
    const int m0 = tile_m * BM + wm * kWaveRows;
    const int n = tile_n * BN + wn * (FW * 32) + c * 8;
#pragma unroll 4
    for (int i = 0; i < kWaveRows / 8; ++i) {
        const int r = i * 8 + (lane >> 3);
        const uint4 v = *reinterpret_cast<const uint4*>(wstage + r * kWaveRowBytes +
                                                        ((c ^ ((r >> 1) & 7)) * 16));
        if (m0 + r < M && n < N)
            *reinterpret_cast<uint4*>(Y + (size_t)(m0 + r) * N + n) = v;
    }
}

template <int FMT, int NS, bool ACC_OUT>
hipError_t launch_variant(const uint8_t* xq, const float* row_scale, const uint8_t* sid,
                          const uint8_t* Wq, const float* w_scale, const float* comp_a,
                          const float* comp_b, int M, int N, int K, int S, uint16_t* Y,
                          int32_t* acc_out, hipStream_t stream) {
    using C = Cfg<FMT, NS>;
    static_assert(C::lds_bytes(1) <= kLdsLimit, "LDS budget");
    static_assert(C::lds_bytes(RUDDER_MAX_STREAMS) <= 160 * 1024, "LDS budget");
    // the attribute admits the full CU; a call whose tables do not fit the
    // per-workgroup share simply runs fewer workgroups per CU
    static const hipError_t attr = hipFuncSetAttribute(
        (const void*)w4_gemm_kernel<FMT, NS, ACC_OUT>,
        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    hipLaunchKernelGGL((w4_gemm_kernel<FMT, NS, ACC_OUT>), dim3((unsigned)(tiles_m * tiles_n)),
                       dim3(kThreads), C::lds_bytes(S), stream, xq, row_scale, sid, Wq, w_scale,
                       comp_a, comp_b, M, N, K, S, Y, acc_out, tiles_m, tiles_n);
    return hipGetLastError();
}

template <int FMT, bool ACC_OUT>
hipError_t launch_fmt(const uint8_t* xq, const float* row_scale, const uint8_t* sid,
                      const uint8_t* Wq, const float* w_scale, const float* comp_a,
                      const float* comp_b, int M, int N, int K, int S, uint16_t* Y,
                      int32_t* acc_out, hipStream_t stream) {
    // deepest ring that fits the per-workgroup LDS share with this call's tables
    constexpr int NS_MAX = FMT == kFmtA4 ? 3 : 2;
    if constexpr (NS_MAX > 2) {
        if (Cfg<FMT, NS_MAX>::lds_bytes(S) > kLdsLimit)
            return launch_variant<FMT, NS_MAX - 1, ACC_OUT>(xq, row_scale, sid, Wq, w_scale,
                                                            comp_a, comp_b, M, N, K, S, Y,
                                                            acc_out, stream);
    }
    return launch_variant<FMT, NS_MAX, ACC_OUT>(xq, row_scale, sid, Wq, w_scale, comp_a, comp_b,
                                                M, N, K, S, Y, acc_out, stream);
}

}  // namespace

hipError_t launch_linear(const void* Xq, const float* row_scale, const uint8_t* sid,
                         const uint8_t* Wq, const float* w_scale, const float* comp_a,
                         const float* comp_b, int M, int N, int K, int S, int abits, int codes,
                         uint16_t* Y, int32_t* acc_out, hipStream_t stream) {
    const uint8_t* xq = static_cast<const uint8_t*>(Xq);
#define RUDDER_LAUNCH(FMT)                                                                   \
    return acc_out ? launch_fmt<FMT, true>(xq, row_scale, sid, Wq, w_scale, comp_a, comp_b, M, \
                                           N, K, S, Y, acc_out, stream)                       \
                   : launch_fmt<FMT, false>(xq, row_scale, sid, Wq, w_scale, comp_a, comp_b,  \
                                            M, N, K, S, Y, acc_out, stream)
    if (codes == RUDDER_CODES_E2M3) RUDDER_LAUNCH(kFmtF6);
    if (abits == 8) RUDDER_LAUNCH(kFmtA8);
    RUDDER_LAUNCH(kFmtA4);
#undef RUDDER_LAUNCH
}

}  // namespace rudder
