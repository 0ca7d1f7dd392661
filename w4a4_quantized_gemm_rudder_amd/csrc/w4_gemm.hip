// Low-bit GEMM with fused dequantization / compensation epilogue.
//
// SteerQuant ("SteerQuant: Steering Quantization Error with Action-Guided
// Scaling in World-Action Models", paperlayer.ai digest), §4.4 (Rudder): the
// low-bit GEMM consumes only integer activations and per-row scales, and its
// epilogue applies dequantization, inverse-gain compensation and bias, so the
// scaling costs no extra launch and no intermediate HBM round trip (§1).
//
// gfx950 mapping
//   * The MFMA "A" operand is a slice of the weights (output channel n = MFMA
//     row i), the "B" operand a slice of the activations (token m = MFMA
//     column j), so each lane's accumulators hold token rows and runs of 4
//     consecutive channels.  The W4A8 tiled loop runs
//     v_mfma_i32_16x16x64_i8 (four per 32 x 32 fragment pair and 64 k; on
//     these codes it sustains a higher rate than v_mfma_i32_32x32x32_i8 at
//     the power-limited clock); W4A4 int codes and the weight-streaming
//     kernel use v_mfma_i32_32x32x32_i8.
//   * There is no int4 MFMA.  4-bit codes are widened in registers: the
//     split-nibble word w becomes (w << 4) & 0xF0F0F0F0 and w & 0xF0F0F0F0,
//     bytes equal to 16 * code in natural k order.  The int32 result is then
//     16x (W4A8) or 256x (W4A4) the true accumulator -- exact for
//     K <= RUDDER_MAX_K -- and an arithmetic shift undoes it.
//   * Codes arrive MFMA-tiled (blocks in lane order), so every fragment is
//     one contiguous lane-ordered load.  The activation fragments, shared by
//     the workgroup's four waves, go global -> LDS with the gfx950
//     direct-to-LDS 16-byte loads (no VGPR staging, one contiguous KiB per
//     wave instruction) into a two-stage ring, one workgroup barrier per
//     k-stage.  Each wave is the only reader of its weight fragments, so
//     those go straight from global memory into registers, two stages ahead,
//     and cost no LDS traffic.
//   * Epilogue: dequantize + compensate in registers, stage the bf16 tile in
//     LDS (XOR-swizzled 16-byte chunks), then store it with 16-byte stores
//     in whole 128-byte lines (64-byte halves for the narrow tiles below),
//     so every HBM line is written once.
//   * Ragged last round: when the rows spill a little past a whole number of
//     tile rounds, those rows run in the same launch, after the tiles: as
//     weight-streaming blocks (64 or 96 rows each) for narrow layers, as
//     half-width tiles for wider ones (int containers).  A partial round
//     with more tiles than compute units keeps one tile per CU and hands
//     the remaining rows to those forms.
//   * Weight touch: a few leading blocks of each launch read the packed
//     weights once, line by line, so that the tiles' many re-reads of them
//     hit the memory-side cache instead of HBM.
//   * E2M3 container (W4A4): 4-bit codes held as FP6 E2M3 feed
//     v_mfma_scale_f32_32x32x64_f8f6f4 directly (unit scales): no widening, and
//     twice the int8 rate.  Products of codes are small integers and every
//     fp32 partial sum is an integer below 2^24, so the fp32 accumulator holds
//     the exact integer dot product.  Its operands are the 6-dword form the
//     instruction takes for FP6, read straight into place.  8-bit codes in
//     this container are two digit planes, one MFMA each under E8M0 scales
//     2^5 and 2^1 (exact up to K = 16384).
//   * Tile order: workgroups are dealt round-robin to the 8 XCDs; the grid is
//     remapped so each XCD walks a contiguous, m-grouped range of tiles and
//     the tiles in flight on one XCD share activation and weight panels in
//     that XCD's L2.
#include <type_traits>

#include "rudder_internal.h"

namespace rudder {
typedef int mfma_v6i __attribute__((ext_vector_type(6)));
typedef float mfma_v16f __attribute__((ext_vector_type(16)));

// The f8f6f4 scaled MFMA with 6-dword operands, as the instruction takes them
// for FP6 formats (the clang builtin fixes 8-dword operands, which would make
// every fragment a padded 8-register tuple and cost register moves).  Called
// with cbsz = blgp = 2 (FP6 E2M3 A and B) and power-of-two E8M0 scales
// (unit, or the digit planes' 2^5 and 2^1).
__device__ mfma_v16f mfma_scale_f32_32x32x64_fp6(mfma_v6i a, mfma_v6i b, mfma_v16f c,
                                                 int cbsz, int blgp, int opsel_a, int scale_a,
                                                 int opsel_b, int scale_b)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v6i32.v6i32");
}  // namespace rudder

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
constexpr int kBlocksPerCU = 2;  // two independent workgroups share each CU
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;
constexpr int kGroupM = 8;       // m-tiles per tile group (L2 reuse of weight panels)

// GELU of every bf16 pattern (the exact erf form, rounded to fp32 then bf16),
// written at build time by gelu_table_gen.cpp.
__device__ const uint16_t kGeluBf16[65536] = {
#include "gelu_table.inc"
};

// Epilogue modes: the bf16 output, or GELU of it quantized as the next
// layer's input (int8 codes, split-nibble int4 codes, E2M3 codes).
constexpr int kEpiBf16 = 0;
constexpr int kEpiQ8 = 1;
constexpr int kEpiQ4 = 2;
constexpr int kEpiE2M3 = 3;

// Code formats of the GEMM.
constexpr int kFmtA8 = 0;        // int8 activations, int4 weights (int8 MFMA)
constexpr int kFmtA4 = 1;        // int4 activations and weights (int8 MFMA)
constexpr int kFmtF6 = 2;        // 4-bit codes held as E2M3 (f8f6f4 MFMA)
constexpr int kFmtD6 = 3;        // int8 activations as two E2M3 digit planes, E2M3 weights
                                 // (f8f6f4 MFMA, two per product)

// The formats whose operands are E2M3 fields (fp32 accumulators).
constexpr bool fp6_fmt(int fmt) { return fmt == kFmtF6 || fmt == kFmtD6; }

// The W4A8 tiled loop runs v_mfma_i32_16x16x64_i8: on the layers' own codes
// it sustains a higher rate than the 32x32x32 int8 shape at the
// power-limited clock.  (int4 activations keep 32x32x32: their widening per
// 16-token half costs more than the shape gains; the weight-streaming
// kernel keeps 32x32x32 too.)
constexpr bool i16_fmt(int fmt) { return fmt == kFmtA8; }

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v6i __attribute__((ext_vector_type(6)));


// Per-format traits.  The wave grid (kWavesN x kWavesM = 4 x 1) splits the
// 128 x 256 block tile; each wave owns FW = 2 32-channel and FA = 4 32-token
// fragments, so every k-substep it takes FW weight fragments (its own, from
// registers) and FA activation fragments (shared, from LDS) and issues
// FW * FA MFMAs per activation plane.  kPlanes activation planes share one
// weight fragment: the digit format holds each int8 code q as q = 16 h + l
// in two E2M3 planes (h / 2 and l / 2, both exact), and multiplies them with
// E8M0 block scales 2^5 and 2^1 into the same fp32 accumulator, which then
// holds sum q * w exactly.
template <int FMT>
struct Fmt;
template <>
struct Fmt<kFmtA8> {
    static constexpr int kKSub = 32;       // k per MFMA
    static constexpr int kABlock = 1024;   // bytes per 32-row x kKSub code block
    static constexpr int kWBlock = 512;
    static constexpr int kWavesN = 4;      // waves along the channel dimension
    typedef uint2 WFrag;
    typedef uint4 AFrag;
    typedef v16i Acc;
    static constexpr int kPlanes = 1;
};
template <>
struct Fmt<kFmtA4> {
    static constexpr int kKSub = 32;
    static constexpr int kABlock = 512;
    static constexpr int kWBlock = 512;
    static constexpr int kWavesN = 4;
    typedef uint2 WFrag;
    typedef uint2 AFrag;
    typedef v16i Acc;
    static constexpr int kPlanes = 1;
};
template <>
struct Fmt<kFmtF6> {
    static constexpr int kKSub = 64;
    static constexpr int kABlock = 1536;
    static constexpr int kWBlock = 1536;
    static constexpr int kWavesN = 4;
    typedef v6i WFrag;     // MFMA operand registers
    typedef v6i AFrag;
    typedef v16f Acc;
    static constexpr int kPlanes = 1;
    static constexpr int kPlaneBytes = 1536;
    // E8M0 scales (127 = 2^0): the word passed as both scale operands, the
    // byte the weights take and the byte activation plane p takes
    static constexpr int kScaleWord = 127;
    static constexpr int kWeightScaleSel = 0;
    static constexpr int plane_scale_sel(int) { return 0; }
};
template <>
struct Fmt<kFmtD6> {
    static constexpr int kKSub = 64;
    static constexpr int kABlock = 3072;   // high-digit plane, then low-digit plane
    static constexpr int kWBlock = 1536;
    static constexpr int kWavesN = 4;
    typedef v6i WFrag;
    typedef v6i AFrag;     // one plane
    typedef v16f Acc;
    static constexpr int kPlanes = 2;
    static constexpr int kPlaneBytes = 1536;
    // bytes 2^0, 2^5 (high digits), 2^1 (low digits) of one scale word, so
    // that every MFMA takes its scales from one register
    static constexpr int kScaleWord = 127 | (127 + 5) << 8 | (127 + 1) << 16;
    static constexpr int kWeightScaleSel = 0;
    static constexpr int plane_scale_sel(int p) { return p == 0 ? 1 : 2; }
};

template <int FMT, int TBN = BN>
struct Waves {
    static constexpr int kN = Fmt<FMT>::kWavesN;          // waves along channels
    static constexpr int kM = kWaves / kN;                // waves along tokens
    static constexpr int FW = TBN / kN / 32;              // 32-channel fragments per wave
    static constexpr int FA = BM / kM / 32;               // 32-token fragments per wave
    static_assert(kN * kM == kWaves && FW * kN * 32 == TBN && FA * kM * 32 == BM, "wave grid");
};

template <int FMT, int NS, int TBN = BN>
struct Cfg {
    using F = Fmt<FMT>;
    static constexpr int kActBlock = F::kABlock;
    static constexpr int kActPerMb = (BK / F::kKSub) * kActBlock;    // per 32-token block
    static constexpr int kActBytes = (BM / 32) * kActPerMb;
    // the ring holds activation codes only (weights go to registers)
    static constexpr int kStageBytes = kActBytes;
    static constexpr int kRingBytes = NS * kStageBytes;
    // 16-byte direct loads per thread per stage (each wave instruction = 1 KiB)
    static constexpr int kActLoads = kActBytes / (1024 * kWaves);
    static constexpr int kEpiBytes = BM * TBN * 2;                   // bf16 tile
    // Per-tile epilogue tables (w_scale, comp_a[S], comp_b[S] for the tile's
    // 256 channels, 1 KiB each) live after both the ring and the bf16 tile.
    static constexpr int kTableOffset = kRingBytes > kEpiBytes ? kRingBytes : kEpiBytes;
    static constexpr int lds_bytes(int S, int extra_rows = 0) {
        return kTableOffset + (1 + 2 * S + extra_rows) * 1024;
    }
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

// 16-byte store of the bf16 output with the streaming (non-temporal) hint:
// the output tiles are written once and are far larger than L2, so they
// should not evict the weight and activation panels other tiles still read.
__device__ __forceinline__ void store_y16(uint16_t* p, uint4 v) {
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(p));
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
// s_waitcnt immediate (gfx9 layout: vmcnt bits 3..0 and 15..14, expcnt 6..4,
// lgkmcnt 11..8) that waits for LDS / scalar-memory results only:
// vmcnt = 63 and expcnt = 7 (no wait), lgkmcnt = 0.
constexpr int kWaitLgkm0 = 0xC07F;

template <int N>
__device__ __forceinline__ void wait_and_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
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
// An E2M3 fragment, read straight into its 6-dword MFMA operand: plane 0
// (16 bytes) into dwords 0..3 and plane 1 (8 bytes) into dwords 4..5.
template <>
__device__ __forceinline__ void read_frag<v6i>(const uint8_t* block, int lane, v6i& out) {
    const v4i p0 = *reinterpret_cast<const v4i*>(block + lane * 16);
    // An opaque plane-1 address: otherwise the plane-1 reads of two fragments
    // merge into one two-address read whose halves must then be moved into
    // the two operand tuples.
    uint32_t a1 = lds_offset(block + 1024 + lane * 8);
    asm("" : "+v"(a1));
    typedef __attribute__((address_space(3))) const v2i* lds_v2i_ptr;
    const v2i p1 = *reinterpret_cast<lds_v2i_ptr>(static_cast<uintptr_t>(a1));
    const v4i p1x = __builtin_shufflevector(p1, p1, 0, 1, -1, -1);
    out = __builtin_shufflevector(p0, p1x, 0, 1, 2, 3, 4, 5);
}

// Accumulators of one 32-channel x 32-token fragment pair of the tiled
// W4A8 loop: four 16 x 16 blocks of v_mfma_i32_16x16x64_i8.  Block b = 2 sc + st
// covers channels 16 sc .. 16 sc + 15 and tokens 16 st .. 16 st + 15; lane l
// holds token 16 st + l % 16 and channels 16 sc + 4 (l / 16) .. + 3, so
// element 4 b + j of the fragment pair is channel j of that run of four.
struct I16Acc {
    v4i s[4];
    __device__ __forceinline__ int operator[](int r) const { return s[r >> 2][r & 3]; }
};
template <int FMT>
struct TileAcc {
    typedef typename Fmt<FMT>::Acc type;
};
template <>
struct TileAcc<kFmtA8> {
    typedef I16Acc type;
};

__device__ __forceinline__ void zero_acc(v16f& a) {
#pragma unroll
    for (int r = 0; r < 16; ++r) a[r] = 0.0f;
}
__device__ __forceinline__ void zero_acc(v16i& a) {
#pragma unroll
    for (int r = 0; r < 16; ++r) a[r] = 0;
}
__device__ __forceinline__ void zero_acc(I16Acc& a) {
#pragma unroll
    for (int b = 0; b < 4; ++b) a.s[b] = v4i{0, 0, 0, 0};
}
// Scheduling fence on an accumulator (keeps the MFMAs that write it ahead of
// what follows).
__device__ __forceinline__ void pin(v16f& a) { asm volatile("" : "+v"(a)); }
__device__ __forceinline__ void pin(v16i& a) { asm volatile("" : "+v"(a)); }
__device__ __forceinline__ void pin(I16Acc& a) {
    asm volatile("" : "+v"(a.s[0]), "+v"(a.s[1]), "+v"(a.s[2]), "+v"(a.s[3]));
}

// Byte offset, within the two consecutive 32-k code blocks (BLOCK bytes each,
// SLOT bytes per 16-code slot) of a 64-k substep, of the 16 codes lane l
// feeds to v_mfma_i32_16x16x64_i8 for rows 16 s .. 16 s + 15 of a 32-row
// fragment: row 16 s + l % 16, k 16 (l / 16) .. + 15 of the substep, i.e.
// block l / 32, slot (16 s + l % 16) + 32 ((l / 16) % 2).  Both operands use
// this map, so every k of the substep pairs one weight and one activation
// code whatever order the instruction sums them in.
template <int SLOT, int BLOCK>
__device__ __forceinline__ uint32_t i16_offset(int lane, int s) {
    return (uint32_t)((lane >> 5) * BLOCK + (16 * s + (lane & 15) + 32 * ((lane >> 4) & 1)) * SLOT);
}

// Exact integer value of an accumulator element (the int8 path carries 16x
// (W4A8) or 256x (W4A4) the true sum, see widen_nibbles).
template <int FMT, typename A>
__device__ __forceinline__ int acc_value(const A& a, int r) {
    if constexpr (fp6_fmt(FMT)) return (int)a[r];
    else if constexpr (FMT == kFmtA8) return a[r] >> 4;
    else return a[r] >> 8;
}

// The same value as an fp32 (exact: |acc| < 2^24).  The E2M3 accumulators
// already hold it; the int containers shift and convert.
template <int FMT, typename A>
__device__ __forceinline__ float acc_float(const A& a, int r) {
    if constexpr (fp6_fmt(FMT)) return a[r];
    else return (float)acc_value<FMT>(a, r);
}

// One block tile: rows tile_m * BM .. + BM - 1, channels tile_n * TBN ..
// + TBN - 1 (TBN = BN, or BN / 2 for the narrow tiles of a ragged last
// round).
template <int FMT, int NS, bool ACC_OUT, int EPI, int TBN>
__device__ __forceinline__ void gemm_tile(
    const uint8_t* __restrict__ Xq, const float* __restrict__ row_scale,
    const uint8_t* __restrict__ sid, const uint8_t* __restrict__ Wq,
    const float* __restrict__ w_scale, const float* __restrict__ comp_a,
    const float* __restrict__ comp_b, int M, int N, int K, int S, uint16_t* __restrict__ Y,
    int32_t* __restrict__ acc_out, int tile_m, int tile_n, const NextLayerQuant& nx) {
    using C = Cfg<FMT, NS, TBN>;
    using F = Fmt<FMT>;
    constexpr int FW = Waves<FMT, TBN>::FW, FA = Waves<FMT, TBN>::FA;
    constexpr int kWavesN = Waves<FMT, TBN>::kN;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave % kWavesN;    // channel slice of the tile (FW * 32 channels)
    const int wm = wave / kWavesN;    // token slice of the tile (FA * 32 tokens)
    const int uwave = __builtin_amdgcn_readfirstlane(wave);   // wave index as a scalar

    const int kblocks = K / F::kKSub;                       // code blocks along k
    const int mblocks = (M + 31) >> 5;
    const int nblocks = N >> 5;
    const int ksteps = K / BK;
    const int n_tile0 = min(tile_n * TBN, N - 32);           // first channel of the tile (clamped)

    // Stream id and row scale of this lane's token rows (plain loads, issued
    // after the main loop: holding them across it leaves the loop without
    // registers).  A lane's accumulators cover one token per fragment (32x32
    // shapes), or one token per 16-token half of it (W4A8, 16x16 blocks): TH
    // token rows per fragment, token_of(th) within the fragment.
    constexpr bool kI16 = i16_fmt(FMT);
    constexpr int TH = kI16 ? 2 : 1;
    auto token_of = [&](int th) { return kI16 ? 16 * th + (lane & 15) : (lane & 31); };
    int row_stream[FA][TH];
    float row_rs[FA][TH];
    auto fetch_row_data = [&]() {
#pragma unroll
        for (int g = 0; g < FA; ++g)
#pragma unroll
            for (int th = 0; th < TH; ++th) {
                const int mc = min(tile_m * BM + wm * (FA * 32) + g * 32 + token_of(th), M - 1);
                row_stream[g][th] = min(sid[mc] & (RUDDER_MAX_STREAMS - 1), S - 1);
                row_rs[g][th] = row_scale[mc];
            }
    };

    // ---- epilogue tables -> LDS (one KiB per table row, one wave each) ----
    // row 0: w_scale, rows 1..S: comp_a[s], rows S+1..2S: comp_b[s] (and, when
    // the epilogue quantizes for the next layer, row 2S+1: its inv_smooth), each for
    // channels n_tile0 .. n_tile0 + 255 (a tile narrower than 256 channels
    // reads past its last channel only within the same row of the table
    // when N >= 256; narrower matrices clamp the window to the last 256).
    const uint32_t lds_base = lds_offset(lds);
    {
        const int nwin = N >= BN ? min(n_tile0, N - BN) : 0;
        const int cols = N >= BN ? BN : N;                   // columns present in the window
        const int per_lane = cols * 4 / 64;                  // bytes per lane (16 when cols = 256)
        const int rows = 1 + 2 * S + (EPI != kEpiBf16 ? 1 : 0);
        for (int r = uwave; r < rows; r += kWaves) {
            const float* src = r == 0 ? w_scale
                             : (r <= S ? comp_a + (size_t)(r - 1) * N
                                       : (r <= 2 * S ? comp_b + (size_t)(r - 1 - S) * N
                                                     : nx.inv_smooth));
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
    // Each wave instruction moves one contiguous KiB of the stage's
    // activation codes (32-token block, k-block pairs).  Bases are
    // wave-uniform (SGPRs); every lane adds lane * 16.  Token blocks past the
    // matrix edge are clamped to the last real block (their results are never
    // stored).
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

    auto issue_stage = [&](int kt) {
        const uint32_t base = lds_base + (uint32_t)((kt % NS) * C::kStageBytes);
        const size_t a_off = (size_t)kt * C::kActPerMb;
#pragma unroll
        for (int i = 0; i < C::kActLoads; ++i)
            load_lds16(act_src[i] + a_off, voff, base + act_dst[i]);
    };

    typename TileAcc<FMT>::type acc[FW][FA];
#pragma unroll
    for (int f = 0; f < FW; ++f)
#pragma unroll
        for (int g = 0; g < FA; ++g) zero_acc(acc[f][g]);

    // ---- main loop ----------------------------------------------------------
    // Weights straight from global memory into registers, activations
    // through a two-stage LDS ring.  Each wave is the only reader of its
    // weight fragments (one wave per 64-channel slice), so those bypass LDS:
    // stage kt's weights sit in wreg[kt % 2], and each substep's slot is
    // refilled with stage kt+2's fragments as soon as that substep's MFMAs
    // are issued, which gives a weight load two stages to land.  Activation
    // fragments are read one substep ahead into fa[j % 2] (substep j).
    static_assert(NS == 2, "direct-weight loop bookkeeping");
    // A substep is one MFMA k-step: 32 k (int4 activations), 64 k (E2M3, and
    // the W4A8 16x16x64 shape, whose substep spans two 32-k code blocks).
    // W4A8 takes a substep's activations in two planes, one per 16-token
    // half of each fragment (the digit format's planes are its two digits).
    constexpr int KS = kI16 ? 64 : F::kKSub;         // k per substep
    constexpr int BPS = KS / F::kKSub;                // code blocks per substep
    constexpr int P = BK / KS;                        // substeps per stage
    static_assert(P % 2 == 0, "substep parity");
    constexpr bool kF6 = fp6_fmt(FMT);
    constexpr int PL = kI16 ? 2 : F::kPlanes;         // activation planes per substep
    constexpr int WL = (kF6 || kI16) ? 2 * FW : FW;   // weight loads per substep
    typedef typename std::conditional<kI16, uint4, typename F::WFrag>::type WOp;
    typedef typename F::AFrag AOp;
    // this wave's weight block rows (wave-uniform: scalar bases; every lane
    // adds its own offsets)
    const uint8_t* wblk[FW];
    const int uwn = uwave % kWavesN;
#pragma unroll
    for (int f = 0; f < FW; ++f) {
        const int gnb = min(tile_n * (TBN / 32) + uwn * FW + f, nblocks - 1);
        wblk[f] = Wq + (size_t)gnb * kblocks * F::kWBlock;
    }
    // per-lane offsets: E2M3 plane 0 and plane 1; W4A8 the two 16-channel
    // halves of a fragment (i16_offset)
    // (the second half's offset is the first's plus 16 slots, a constant the
    // load instructions take as an immediate)
    const uint32_t off0 = kI16 ? i16_offset<8, 512>(lane, 0) : lane * (kF6 ? 16 : 8);
    const uint32_t off1 = 1024 + lane * 8;
    constexpr int kASlot = F::kABlock / 64;           // bytes of one 16-code slot
    const uint32_t aoff0 = i16_offset<kASlot, F::kABlock>(lane, 0);
    auto load_w = [&](int kt, int kk, WOp (&dst)[FW], bool real = true) {
        const uint32_t o0 = real ? off0 : 0u, o1 = real ? off1 : 0u;
#pragma unroll
        for (int f = 0; f < FW; ++f) {
            const uint8_t* b = wblk[f] + (size_t)(kt * P + kk) * BPS * F::kWBlock;
            if constexpr (kI16) {
                const uint2 h0 = *reinterpret_cast<const uint2*>(b + o0);
                const uint2 h1 = *reinterpret_cast<const uint2*>(b + o0 + 16 * 8);
                dst[f] = make_uint4(h0.x, h0.y, h1.x, h1.y);
            } else if constexpr (kF6) {
                const v4i p0 = *reinterpret_cast<const v4i*>(b + o0);
                const v2i p1 = *reinterpret_cast<const v2i*>(b + o1);
                dst[f] = __builtin_shufflevector(
                    p0, __builtin_shufflevector(p1, p1, 0, 1, -1, -1), 0, 1, 2, 3, 4, 5);
            } else {
                dst[f] = *reinterpret_cast<const uint2*>(b + o0);
            }
        }
    };
    // js = kk * PL + plane: activation plane `plane` of substep kk
    auto read_acts = [&](int kt, int js, AOp (&dst)[FA]) {
        if constexpr (kI16) {
            // plane js % 2: the 16-token half of every fragment
            const uint8_t* st = lds + (kt % NS) * C::kStageBytes + (js / PL) * BPS * C::kActBlock;
            const uint8_t* sa = st + aoff0 + (js % PL) * 16 * kASlot;
#pragma unroll
            for (int g = 0; g < FA; ++g)
                dst[g] = *reinterpret_cast<const AOp*>(sa + (wm * FA + g) * C::kActPerMb);
        } else {
            int plane_off = 0;
            if constexpr (PL > 1) plane_off = (js % PL) * F::kPlaneBytes;
            const uint8_t* st =
                lds + (kt % NS) * C::kStageBytes + (js / PL) * C::kActBlock + plane_off;
#pragma unroll
            for (int g = 0; g < FA; ++g)
                read_frag(st + (wm * FA + g) * C::kActPerMb, lane, dst[g]);
        }
    };
    auto mma = [&](const WOp (&w)[FW], const AOp (&a)[FA], int first, int last, auto plane_) {
        constexpr int plane = decltype(plane_)::value;
#pragma unroll
        for (int f = 0; f < FW; ++f) {
            if constexpr (kF6) {
                // formats: 2 = FP6 E2M3 for both operands; E8M0 scales: 2^0
                // for the weights, the plane's own for the activations
                constexpr int sel = F::plane_scale_sel(plane);
#pragma unroll
                for (int g = 0; g < FA; ++g)
                    if (f * FA + g >= first && f * FA + g < last)
                        acc[f][g] = mfma_scale_f32_32x32x64_fp6(
                            w[f], a[g], acc[f][g], 2, 2, F::kWeightScaleSel, F::kScaleWord, sel,
                            F::kScaleWord);
            } else if constexpr (!kI16) {
                if (f * FA + FA <= first || f * FA >= last) continue;
                const v4i wf = widen_nibbles(w[f].x, w[f].y);
#pragma unroll
                for (int g = 0; g < FA; ++g) {
                    if (f * FA + g < first || f * FA + g >= last) continue;
                    const v4i af = widen_nibbles(a[g].x, a[g].y);
                    acc[f][g] =
                        __builtin_amdgcn_mfma_i32_32x32x32_i8(wf, af, acc[f][g], 0, 0, 0);
                }
            } else {
                // plane = 16-token half st: blocks (sc, st) for both
                // 16-channel halves sc of the weight fragment
                if (f * FA + FA <= first || f * FA >= last) continue;
                const v4i w0 = widen_nibbles(w[f].x, w[f].y);
                const v4i w1 = widen_nibbles(w[f].z, w[f].w);
#pragma unroll
                for (int g = 0; g < FA; ++g) {
                    if (f * FA + g < first || f * FA + g >= last) continue;
                    const v4i af = v4i{(int)a[g].x, (int)a[g].y, (int)a[g].z, (int)a[g].w};
                    acc[f][g].s[plane] =
                        __builtin_amdgcn_mfma_i32_16x16x64_i8(w0, af, acc[f][g].s[plane], 0, 0, 0);
                    acc[f][g].s[2 + plane] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        w1, af, acc[f][g].s[2 + plane], 0, 0, 0);
                }
            }
        }
    };

    // Prologue, in this order: ring stages 0 and 1, then the weights of
    // stages 0 and 1.  vmcnt counts in issue order; a wait for a ring stage
    // leaves outstanding only what was issued after it.  Weight loads are
    // issued unconditionally, which keeps the counts below fixed and the
    // compiler's own waits for the weight registers exact: past the last
    // stage a refill becomes a dummy load that every lane points at the
    // block's first 16 bytes (one cache line per instruction, nothing
    // left to prefetch), into a slot that is not read again.
    constexpr int LA = C::kActLoads;
    WOp wreg[2][P][FW];
    AOp fa[2][FA];
    const int klast = ksteps - 1;
    issue_stage(0);
    if (ksteps > 1) issue_stage(1);
#pragma unroll
    for (int kk = 0; kk < P; ++kk) load_w(0, kk, wreg[0][kk]);
#pragma unroll
    for (int kk = 0; kk < P; ++kk) load_w(min(1, klast), kk, wreg[1][kk]);
    if (ksteps > 1) wait_and_barrier<LA + 2 * P * WL>();
    else wait_and_barrier<2 * P * WL>();
    read_acts(0, 0, fa[0]);

    // One stage; u = kt % 2 selects the weight register set.
    auto stage = [&](int kt, auto u_) {
        constexpr int u = decltype(u_)::value;
        const bool prefetch = kt + 2 <= klast;     // stage kt+2 exists
#pragma unroll
        for (int kk = 0; kk < P; ++kk) {
            // One activation plane of substep kk (js = kk * PL + plane).
            auto plane_step = [&](auto pl_) {
                constexpr int pl = decltype(pl_)::value;
                const int js = kk * PL + pl;
                // The first MFMA goes ahead of the next reads.  It waits for
                // this plane's activation fragments, all read one plane
                // earlier; the explicit lgkmcnt(0) records that they have
                // landed, so the remaining MFMAs, issued after the next
                // reads, carry no wait on those reads.
                mma(wreg[u][kk], fa[js % 2], 0, 1, pl_);
                pin(acc[0][0]);
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                if (js + 1 < P * PL) {
                    read_acts(kt, js + 1, fa[(js + 1) % 2]);
                } else if (kt < klast) {
                    // Admit stage kt+1.  Its ring loads were issued at the
                    // previous boundary (in the prologue for kt = 0); after
                    // them came the weight refills of the substeps since then.
                    if (kt == 0) wait_and_barrier<(3 * P - 1) * WL>();
                    else wait_and_barrier<P * WL>();
                    if (kt + 2 < ksteps) issue_stage(kt + 2);
                    read_acts(kt + 1, 0, fa[0]);
                }
                mma(wreg[u][kk], fa[js % 2], 1, FW * FA, pl_);
                // keep these MFMAs ahead of what follows (no sinking past
                // the barrier or the slot refill)
#pragma unroll
                for (int f = 0; f < FW; ++f)
#pragma unroll
                    for (int g = 0; g < FA; ++g) pin(acc[f][g]);
            };
            plane_step(std::integral_constant<int, 0>{});
            if constexpr (PL > 1) plane_step(std::integral_constant<int, 1>{});
            load_w(min(kt + 2, klast), kk, wreg[u][kk], prefetch);
        }
    };
    int kt = 0;
    for (; kt + 1 < ksteps; kt += 2) {
        stage(kt, std::integral_constant<int, 0>{});
        stage(kt + 1, std::integral_constant<int, 1>{});
    }
    if (kt < ksteps) stage(kt, std::integral_constant<int, 0>{});

    // ---- fused epilogue -------------------------------------------------
    // 1. registers: t = float(acc) * (row_scale * w_scale); y = fma(a, t, b);
    //    bf16 (hardware round-to-nearest-even pack) into this wave's LDS
    //    staging area [FA*32 token rows][FW*32 channels]; 16-byte chunk c of
    //    row r sits at chunk c ^ swz(r), which spreads the 32 rows one
    //    instruction writes over the LDS banks.  Per-channel values come from
    //    the LDS tables.
    // 2. each wave stores its own rows: FW*4 lanes per row (128 or 256
    //    bytes), so every store instruction writes whole cache lines.
    constexpr int kWaveRowBytes = FW * 32 * 2;                 // 64, 128 or 256
    constexpr int kWaveRows = FA * 32;                         // 128 or 64
    constexpr int kRowChunks = kWaveRowBytes / 16;             // 4, 8 or 16
    fetch_row_data();
    auto swz = [](int r) {
        return kRowChunks == 4 ? ((r >> 1) & 3) : (kRowChunks == 8 ? ((r >> 1) & 7) : (r & 15));
    };
    __syncthreads();                                   // ring no longer read
    const float* tab = reinterpret_cast<const float*>(lds + C::kTableOffset);
    // next-layer quantizer (code epilogues): reciprocal step per row, Qa
    constexpr float kQNext = EPI == kEpiQ8 ? 127.0f : 7.0f;
    constexpr int kCodeRowBytes = FW * 32;                     // one byte per channel
    float next_ia[FA][TH];
    if constexpr (EPI != kEpiBf16) {
#pragma unroll
        for (int g = 0; g < FA; ++g)
#pragma unroll
            for (int th = 0; th < TH; ++th)
                next_ia[g][th] = step_reciprocal(nx.delta[row_stream[g][th]]);
    }
    const int tab_shift = tile_n * TBN - (N >= BN ? min(n_tile0, N - BN) : 0);
    uint8_t* wstage = lds + wave * (kWaveRows * kWaveRowBytes);
    // When every token row of the wave belongs to one stream (the usual case:
    // rows come stream by stream), the comp rows a[s], b[s] are read once per
    // channel quad instead of once per 32-token block.
    const int s_first = __builtin_amdgcn_readfirstlane(row_stream[0][0]);
    bool one_stream = true;
#pragma unroll
    for (int g = 0; g < FA; ++g)
#pragma unroll
        for (int th = 0; th < TH; ++th) one_stream = one_stream && row_stream[g][th] == s_first;
    const bool wave_one_stream = __builtin_amdgcn_ballot_w64(!one_stream) == 0;
    // Element 4 q + j of a fragment pair's accumulators is channel
    // quad_ch(q) + j of the fragment and token row token_of(q_th(q)) of it:
    // 32x32 shapes: channels 8 q + 4 (l / 32) .. + 3, token l % 32; int
    // formats' 16x16 blocks (q = 2 sc + st): channels 16 sc + 4 (l / 16)
    // .. + 3, token 16 st + l % 16.
    auto quad_ch = [&](int q) {
        return kI16 ? 16 * (q >> 1) + 4 * (lane >> 4) : 8 * q + 4 * (lane >> 5);
    };
    auto q_th = [&](int q) { return kI16 ? (q & 1) : 0; };
    // channel quad (f, q) of this lane, and its column in the table window
    auto table_col = [&](int f, int q) {
        return min(wn * (FW * 32) + f * 32 + quad_ch(q) + tab_shift, 252);
    };
    auto stage_tile = [&](auto uniform_) {
        constexpr bool kUniform = decltype(uniform_)::value;
        // one stream, bf16 output: every table value the wave needs, read up
        // front in one batch (the fragment registers of the k loop are free
        // by now; the code epilogues have no room for it)
        constexpr bool kPreload = kUniform && EPI == kEpiBf16;
        float4 pw[FW][4], pa[FW][4], pb[FW][4];
        if constexpr (kPreload) {
#pragma unroll
            for (int f = 0; f < FW; ++f)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int ti = table_col(f, q);
                    pw[f][q] = *reinterpret_cast<const float4*>(tab + ti);
                    pa[f][q] = *reinterpret_cast<const float4*>(tab + 256 * (1 + s_first) + ti);
                    pb[f][q] =
                        *reinterpret_cast<const float4*>(tab + 256 * (1 + S + s_first) + ti);
                }
        }
#pragma unroll
        for (int f = 0; f < FW; ++f) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wn * (FW * 32) + f * 32 + quad_ch(q);    // in the tile
                const int ti = table_col(f, q);
                const float4 ws =
                    kPreload ? pw[f][q] : *reinterpret_cast<const float4*>(tab + ti);
                const int ch = f * 32 + quad_ch(q);                // channel in the wave row
                const int chunk = ch >> 3;                         // its 16-byte chunk
                const int th = q_th(q);
                if constexpr (kUniform && !kPreload) {
                    pa[f][q] = *reinterpret_cast<const float4*>(tab + 256 * (1 + s_first) + ti);
                    pb[f][q] =
                        *reinterpret_cast<const float4*>(tab + 256 * (1 + S + s_first) + ti);
                }
#pragma unroll
                for (int g = 0; g < FA; ++g) {
                    const int s = row_stream[g][th];
                    const float rs = row_rs[g][th];
                    float4 a, b;
                    if constexpr (kUniform) {
                        a = pa[f][q];
                        b = pb[f][q];
                    } else {
                        a = *reinterpret_cast<const float4*>(tab + 256 * (1 + s) + ti);
                        b = *reinterpret_cast<const float4*>(tab + 256 * (1 + S + s) + ti);
                    }
                    const float t0 = acc_float<FMT>(acc[f][g], 4 * q + 0) * (rs * ws.x);
                    const float t1 = acc_float<FMT>(acc[f][g], 4 * q + 1) * (rs * ws.y);
                    const float t2 = acc_float<FMT>(acc[f][g], 4 * q + 2) * (rs * ws.z);
                    const float t3 = acc_float<FMT>(acc[f][g], 4 * q + 3) * (rs * ws.w);
                    const float y0 = __builtin_fmaf(a.x, t0, b.x);
                    const float y1 = __builtin_fmaf(a.y, t1, b.y);
                    const float y2 = __builtin_fmaf(a.z, t2, b.z);
                    const float y3 = __builtin_fmaf(a.w, t3, b.w);
                    uint2 packed;
                    packed.x = pack_bf16x2_rne(y0, y1);
                    packed.y = pack_bf16x2_rne(y2, y3);
                    const int r = g * 32 + token_of(th);
                    if constexpr (EPI == kEpiBf16) {
                        *reinterpret_cast<uint2*>(wstage + r * kWaveRowBytes +
                                                  ((chunk ^ swz(r)) * 16) + (ch & 4) * 2) =
                            packed;
                    } else {
                        // GELU of the bf16 values, then the next layer's quantizer:
                        // u = gelu * inv_smooth'[n]; q = rne(clamp(u * (1/D'[s])))
                        const float4 ni =
                            *reinterpret_cast<const float4*>(tab + 256 * (1 + 2 * S) + ti);
                        const float g0 = bf16_bits_to_float(kGeluBf16[packed.x & 0xFFFFu]);
                        const float g1 = bf16_bits_to_float(kGeluBf16[packed.x >> 16]);
                        const float g2 = bf16_bits_to_float(kGeluBf16[packed.y & 0xFFFFu]);
                        const float g3 = bf16_bits_to_float(kGeluBf16[packed.y >> 16]);
                        const float ia = next_ia[g][th];
                        const uint32_t word =
                            ((uint32_t)quantize_clamped((g0 * ni.x) * ia, kQNext) & 0xFFu) |
                            (((uint32_t)quantize_clamped((g1 * ni.y) * ia, kQNext) & 0xFFu) << 8) |
                            (((uint32_t)quantize_clamped((g2 * ni.z) * ia, kQNext) & 0xFFu) << 16) |
                            (((uint32_t)quantize_clamped((g3 * ni.w) * ia, kQNext) & 0xFFu) << 24);
                        // code staging: row r of the wave, 64 one-byte codes, 16-byte
                        // chunk k16 stored at chunk k16 ^ (r & 3)
                        *reinterpret_cast<uint32_t*>(
                            wstage + r * kCodeRowBytes + ((((ch >> 4)) ^ (r & 3)) * 16) +
                            (ch & 15)) = word;
                    }
                    if constexpr (ACC_OUT) {
                        const int m = tile_m * BM + wm * kWaveRows + r;
                        const int n = tile_n * TBN + nl;
                        if (m < M && n < N)
                            *reinterpret_cast<int4*>(acc_out + (size_t)m * N + n) =
                                make_int4(acc_value<FMT>(acc[f][g], 4 * q + 0),
                                          acc_value<FMT>(acc[f][g], 4 * q + 1),
                                          acc_value<FMT>(acc[f][g], 4 * q + 2),
                                          acc_value<FMT>(acc[f][g], 4 * q + 3));
                    }
                }
            }
            // keep the accumulator reads of one fragment column together
            // (bounds the registers the epilogue needs)
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (wave_one_stream) stage_tile(std::true_type{});
    else stage_tile(std::false_type{});
    if constexpr (EPI != kEpiBf16) {
        // 2'. the next layer's packed codes from the staged bytes (this wave's
        //     128 rows x 64 channels; rows M .. ceil32(M) - 1 get code 0) and
        //     its row scales
        const int m0 = tile_m * BM + wm * kWaveRows;
        const int n0w = tile_n * TBN + wn * (FW * 32);         // wave's first channel
        const int mpad = (M + 31) & ~31;
        if (tile_n == 0 && wn == 0 && lane < 32) {
#pragma unroll
            for (int g = 0; g < FA; ++g) {
                const int m = m0 + g * 32 + lane;
                if (m < M) nx.row_scale[m] = nx.delta[row_stream[g][kI16 ? (lane >> 4) & 1 : 0]];
            }
        }
        if (n0w >= N) return;
        if constexpr (EPI == kEpiE2M3) {
            // one 32 x 64 block per 32 rows: lane -> (row, 32-channel half)
            const int half = lane >> 5;
#pragma unroll
            for (int rb = 0; rb < FA; ++rb) {
                const int rr = rb * 32 + (lane & 31);
                const int m = m0 + rr;
                if (m >= mpad) continue;
                const uint4 lo = *reinterpret_cast<const uint4*>(
                    wstage + rr * kCodeRowBytes + (((2 * half) ^ (rr & 3)) * 16));
                const uint4 hi = *reinterpret_cast<const uint4*>(
                    wstage + rr * kCodeRowBytes + (((2 * half + 1) ^ (rr & 3)) * 16));
                const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                float c[32];
#pragma unroll
                for (int t = 0; t < 32; ++t)
                    c[t] = m < M ? (float)(int8_t)((w[t >> 2] >> (8 * (t & 3))) & 0xFFu) : 0.0f;
                uint32_t d[6];
                pack_e2m3x32(c, d);
                uint8_t* blk = nx.xq + e2m3_block_offset(m, n0w, N);
                const int slot = e2m3_slot(m, n0w + 32 * half);
                *reinterpret_cast<uint4*>(blk + slot * 16) = make_uint4(d[0], d[1], d[2], d[3]);
                *reinterpret_cast<uint2*>(blk + 1024 + slot * 8) = make_uint2(d[4], d[5]);
            }
        } else {
            // 16-code slots: lane -> (row, 16-channel group) in each 32 x 32 block
#pragma unroll
            for (int rb = 0; rb < FA; ++rb) {
#pragma unroll
                for (int kc = 0; kc < FW; ++kc) {
                    const int rr = rb * 32 + (lane & 31);
                    const int k16 = 2 * kc + (lane >> 5);          // 16-channel group
                    const int m = m0 + rr;
                    const int n = n0w + 16 * k16;
                    if (m >= mpad || n >= N) continue;
                    uint4 v = *reinterpret_cast<const uint4*>(wstage + rr * kCodeRowBytes +
                                                              ((k16 ^ (rr & 3)) * 16));
                    if (m >= M) v = make_uint4(0, 0, 0, 0);
                    if constexpr (EPI == kEpiQ8) {
                        *reinterpret_cast<uint4*>(nx.xq + tiled_slot_offset<8>(m, n, N)) = v;
                    } else {
                        // split-nibble words: byte i = code i (low), code i + 4 (high)
                        uint2 w;
                        w.x = (v.x & 0x0F0F0F0Fu) | ((v.y & 0x0F0F0F0Fu) << 4);
                        w.y = (v.z & 0x0F0F0F0Fu) | ((v.w & 0x0F0F0F0Fu) << 4);
                        *reinterpret_cast<uint2*>(nx.xq + tiled_slot_offset<4>(m, n, N)) = w;
                    }
                }
            }
        }
        return;
    }
    // 2. stores of this wave's rows (its own LDS writes are ordered before
    //    these reads): all of its staged rows are read back first (one LDS
    //    round trip), then stored, kRowChunks lanes per row.
    constexpr int kRowsPerStore = 64 / kRowChunks;
    constexpr int kStores = kWaveRows / kRowsPerStore;
    const int c = lane & (kRowChunks - 1);
    const int m0 = tile_m * BM + wm * kWaveRows;
    const int n = tile_n * TBN + wn * (FW * 32) + c * 8;
    uint4 out[kStores];
#pragma unroll
    for (int i = 0; i < kStores; ++i) {
        const int r = i * kRowsPerStore + lane / kRowChunks;
        out[i] = *reinterpret_cast<const uint4*>(wstage + r * kWaveRowBytes + ((c ^ swz(r)) * 16));
    }
#pragma unroll
    for (int i = 0; i < kStores; ++i) {
        const int r = i * kRowsPerStore + lane / kRowChunks;
        if (m0 + r < M && n < N) store_y16(Y + (size_t)(m0 + r) * N + n, out[i]);
    }
}

template <int FMT, int FA, int NW, bool ACC_OUT, int SW>
__device__ __forceinline__ void skinny_tile(
    const uint8_t* __restrict__ Xq, const float* __restrict__ row_scale,
    const uint8_t* __restrict__ sid, const uint8_t* __restrict__ Wq,
    const float* __restrict__ w_scale, const float* __restrict__ comp_a,
    const float* __restrict__ comp_b, int M, int N, int K, int S, uint16_t* __restrict__ Y,
    int32_t* __restrict__ acc_out, int cb, int rg, uint8_t* smem);

// The first touch_blocks blocks (a multiple of the XCD count, so the tile
// blocks keep their XCD assignment) load one dword per 128-byte line of the
// packed weights and exit.  The tiled kernel reads every weight panel from
// several XCDs, many times over, and its weight stream is latency-bound;
// with the weights cold in HBM (inside a model step each layer's weights
// were last read a whole step earlier) these loads bring them into the
// memory-side cache ahead of the tiles' own reads.
// The other blocks, numbered from 0: [0, narrow_first) are BM x BN tiles of
// rows 0 .. tiles_m * BM - 1 in the XCD-aware order.  The rows past the last
// whole round of tiles, when there are a few, take one of two forms after
// them in the same launch, which the compute units pick up as the full
// tiles drain:
//   - narrow layers (bf16 output): blocks from tail_first on cover rows
//     tail_m0 .. M - 1 as streaming blocks of tail_fa * 32 rows x 32 channels (the
//     weight-streaming kernel's work, its four waves splitting k);
//   - wider layers, int containers (bf16 output): blocks from narrow_first
//     on cover rows narrow_m0 .. M - 1 as tiles of BN / 2 channels, twice as
//     many and each about half as long on these MFMA-bound formats.  (An
//     E2M3 tile is bound by its operand stream, and a half-width one still
//     reads the whole activation panel: no gain there.)
template <int FMT, int NS, bool ACC_OUT, int EPI>
__global__ __launch_bounds__(kThreads, kBlocksPerCU) void w4_gemm_kernel(
    const uint8_t* __restrict__ Xq, const float* __restrict__ row_scale,
    const uint8_t* __restrict__ sid, const uint8_t* __restrict__ Wq,
    const float* __restrict__ w_scale, const float* __restrict__ comp_a,
    const float* __restrict__ comp_b, int M, int N, int K, int S, uint16_t* __restrict__ Y,
    int32_t* __restrict__ acc_out, int tiles_m, int tiles_n, int narrow_first, int narrow_m0,
    int touch_blocks, int tail_first, int tail_m0, int tail_fa, NextLayerQuant nx) {
    if ((int)blockIdx.x < touch_blocks) {
        const size_t bytes = fp6_fmt(FMT) ? (size_t)N * K * 3 / 4 : (size_t)N * K / 2;
        const size_t lines = bytes / 128;
        const uint32_t* p = reinterpret_cast<const uint32_t*>(Wq);
        uint32_t v = 0;
        for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < lines;
             i += (size_t)touch_blocks * kThreads)
            v ^= p[i * 32];
        asm volatile("" ::"v"(v));          // the loads are the point; the data is not used
        return;
    }
    const int bid = (int)blockIdx.x - touch_blocks;
    if constexpr (EPI == kEpiBf16) {
        if (bid >= tail_first) {
            extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
            using F = Fmt<FMT>;
            const int t = bid - tail_first;
            const int cbs = N / 32;
            const size_t a_off = (size_t)(tail_m0 / 32) * (K / F::kKSub) * F::kABlock;
            if constexpr (FMT != kFmtD6) {
                if (tail_fa == 3) {
                    skinny_tile<FMT, 3, 1, ACC_OUT, kWaves>(
                        Xq + a_off, row_scale + tail_m0, sid + tail_m0, Wq, w_scale, comp_a,
                        comp_b, M - tail_m0, N, K, S, Y + (size_t)tail_m0 * N,
                        ACC_OUT ? acc_out + (size_t)tail_m0 * N : acc_out, t % cbs, t / cbs, lds);
                    return;
                }
            }
            skinny_tile<FMT, 2, 1, ACC_OUT, kWaves>(
                Xq + a_off, row_scale + tail_m0, sid + tail_m0, Wq, w_scale, comp_a, comp_b,
                M - tail_m0, N, K, S, Y + (size_t)tail_m0 * N,
                ACC_OUT ? acc_out + (size_t)tail_m0 * N : acc_out, t % cbs, t / cbs, lds);
            return;
        }
    }
    if constexpr (EPI == kEpiBf16 && !fp6_fmt(FMT)) {
        if (bid >= narrow_first) {
            const int t = bid - narrow_first;
            const int rows = (M - narrow_m0 + BM - 1) / BM;       // narrow tile rows
            gemm_tile<FMT, NS, ACC_OUT, EPI, BN / 2>(Xq, row_scale, sid, Wq, w_scale, comp_a,
                                                     comp_b, M, N, K, S, Y, acc_out,
                                                     narrow_m0 / BM + t % rows, t / rows, nx);
            return;
        }
    }
    int tile_m, tile_n;
    tile_of_block(bid, narrow_first, tiles_m, tiles_n, tile_m, tile_n);
    gemm_tile<FMT, NS, ACC_OUT, EPI, BN>(Xq, row_scale, sid, Wq, w_scale, comp_a, comp_b, M, N,
                                         K, S, Y, acc_out, tile_m, tile_n, nx);
}

// ---------------------------------------------------------------------------
// Small-M path (few token rows: action / proprio-only calls).  The weights
// dominate the traffic, so the kernel is organised around streaming them
// at HBM rate: one workgroup per 32-channel block of the output and group of
// up to 32 * FA token rows (all rows in registers), the k range split
// across the workgroup's waves.  Fragments come straight from global memory (the tiled
// code layouts are lane-ordered, so every fragment is one contiguous load);
// there is no LDS ring and no barrier in the k loop.  Each wave's partial
// accumulators are summed into an LDS tile with LDS atomic adds: int32
// addition, and fp32 addition of integers below 2^24, give the same result in
// any order, so the sum is the exact dot product.  The epilogue applies the
// same arithmetic as the tiled kernel and stores 16-byte row segments.
// ---------------------------------------------------------------------------
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyMaxM = 256;                 // rows handled by the small-M kernel
constexpr int kTouchBlocks = 64;                 // weight touch blocks of a tiled launch
constexpr int kSplitMaxWidth = 8192;             // see launch_fmt
constexpr int kSkinnyThreads = 64 * kSkinnyWaves;

// Operand registers of one k-substep: NW weight fragments (NW consecutive
// 32-channel blocks) and up to FA activation fragments, already in MFMA
// operand form (E2M3 fragments are loaded straight into 6-dword operands;
// the digit format's activation fragment is its two planes).
struct F6Planes {
    v6i p[2];
};
template <int FMT, int FA, int NW>
struct SkinnyOps {
    typedef typename std::conditional<fp6_fmt(FMT), v6i, uint2>::type WOp;
    typedef typename std::conditional<
        FMT == kFmtD6, F6Planes,
        typename std::conditional<FMT == kFmtF6, v6i,
                                  typename std::conditional<FMT == kFmtA8, uint4,
                                                            uint2>::type>::type>::type AOp;
    WOp w[NW];
    AOp a[FA];
};

__device__ __forceinline__ v6i load_f6_operand(const uint8_t* block, int lane) {
    const v4i p0 = *reinterpret_cast<const v4i*>(block + lane * 16);
    const v2i p1 = *reinterpret_cast<const v2i*>(block + 1024 + lane * 8);
    return __builtin_shufflevector(p0, __builtin_shufflevector(p1, p1, 0, 1, -1, -1), 0, 1, 2,
                                   3, 4, 5);
}

template <int FMT, int FA, int NW>
__device__ __forceinline__ void skinny_load(const uint8_t* __restrict__ Xq,
                                            const uint8_t* __restrict__ Wq, int nb0, int j,
                                            int kblocks, int mb, int lane,
                                            SkinnyOps<FMT, FA, NW>& op) {
    using F = Fmt<FMT>;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint8_t* wblk = Wq + ((size_t)(nb0 + i) * kblocks + j) * F::kWBlock;
        if constexpr (fp6_fmt(FMT)) op.w[i] = load_f6_operand(wblk, lane);
        else op.w[i] = *reinterpret_cast<const uint2*>(wblk + lane * 8);
    }
#pragma unroll
    for (int g = 0; g < FA; ++g) {
        if (g < mb) {
            const uint8_t* ablk = Xq + ((size_t)g * kblocks + j) * F::kABlock;
            if constexpr (FMT == kFmtD6) {
                op.a[g].p[0] = load_f6_operand(ablk, lane);
                op.a[g].p[1] = load_f6_operand(ablk + Fmt<kFmtD6>::kPlaneBytes, lane);
            } else if constexpr (FMT == kFmtF6) op.a[g] = load_f6_operand(ablk, lane);
            else if constexpr (FMT == kFmtA8) op.a[g] = *reinterpret_cast<const uint4*>(ablk + lane * 16);
            else op.a[g] = *reinterpret_cast<const uint2*>(ablk + lane * 8);
        }
    }
}

template <int FMT, int FA, int NW>
__device__ __forceinline__ void skinny_mma(const SkinnyOps<FMT, FA, NW>& op, int mb,
                                           typename Fmt<FMT>::Acc (&acc)[NW][FA]) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        if constexpr (FMT == kFmtD6) {
            using F = Fmt<kFmtD6>;
#pragma unroll
            for (int g = 0; g < FA; ++g)
                if (g < mb) {
                    acc[i][g] = mfma_scale_f32_32x32x64_fp6(
                        op.w[i], op.a[g].p[0], acc[i][g], 2, 2, F::kWeightScaleSel,
                        F::kScaleWord, F::plane_scale_sel(0), F::kScaleWord);
                    acc[i][g] = mfma_scale_f32_32x32x64_fp6(
                        op.w[i], op.a[g].p[1], acc[i][g], 2, 2, F::kWeightScaleSel,
                        F::kScaleWord, F::plane_scale_sel(1), F::kScaleWord);
                }
        } else if constexpr (FMT == kFmtF6) {
#pragma unroll
            for (int g = 0; g < FA; ++g)
                if (g < mb)
                    acc[i][g] = mfma_scale_f32_32x32x64_fp6(op.w[i], op.a[g], acc[i][g], 2, 2, 0,
                                                            127, 0, 127);
        } else {
            const v4i wf = widen_nibbles(op.w[i].x, op.w[i].y);
#pragma unroll
            for (int g = 0; g < FA; ++g) {
                if (g < mb) {
                    v4i af;
                    if constexpr (FMT == kFmtA8)
                        af = v4i{(int)op.a[g].x, (int)op.a[g].y, (int)op.a[g].z, (int)op.a[g].w};
                    else
                        af = widen_nibbles(op.a[g].x, op.a[g].y);
                    acc[i][g] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf, af, acc[i][g], 0, 0, 0);
                }
            }
        }
    }
}

// Substeps per load chunk: every wave keeps two chunks in flight.  With two
// weight blocks the accumulators double, so the chunk shrinks to keep the
// operand buffers within ~200 registers with them.
template <int FMT, int FA, int NW>
struct SkinnyChunk {
    static constexpr int kRegs =
        NW * (fp6_fmt(FMT) ? 6 : 2) +
        FA * (FMT == kFmtD6 ? 12 : FMT == kFmtF6 ? 6 : (FMT == kFmtA8 ? 4 : 2));
    static constexpr int kFit = (200 - 16 * NW * FA) / (2 * kRegs);
    static constexpr int D = NW == 1 ? (kRegs <= 12 ? 8 : (kRegs < 24 ? 4 : 2))
                                     : (kFit >= 8 ? 8 : kFit >= 4 ? 4 : kFit >= 2 ? 2 : 1);
};

// LDS of one streaming block: the sum tile (exact integer dot products,
// summed as int32; fp32 partials of the E2M3 path are integers below 2^24
// and convert exactly), the epilogue operands w_scale[NC], comp_a[S][NC],
// comp_b[S][NC], and the rows' scales and streams.
template <int FA, int NW>
struct SkinnySmem {
    static constexpr int NC = NW * 32;               // channels of the block
    static constexpr int kPitch = NC + 1;            // row pitch (words) of the sum tile
    static constexpr int kTabMax = NC * (1 + 2 * RUDDER_MAX_STREAMS);
    static constexpr int kSumBytes = FA * 32 * kPitch * 4;
    static constexpr int kTabBytes = kTabMax * 4;
    static constexpr int kBytes = kSumBytes + kTabBytes + 2 * FA * 32 * 4;
};

// One streaming block (SW waves): channel block cb (NW * 32 channels) and
// row group rg (FA * 32 rows); smem holds SkinnySmem<FA, NW>::kBytes of LDS.
template <int FMT, int FA, int NW, bool ACC_OUT, int SW>
__device__ __forceinline__ void skinny_tile(
    const uint8_t* __restrict__ Xq, const float* __restrict__ row_scale,
    const uint8_t* __restrict__ sid, const uint8_t* __restrict__ Wq,
    const float* __restrict__ w_scale, const float* __restrict__ comp_a,
    const float* __restrict__ comp_b, int M, int N, int K, int S, uint16_t* __restrict__ Y,
    int32_t* __restrict__ acc_out, int cb, int rg, uint8_t* smem) {
    using F = Fmt<FMT>;
    using Acc = typename F::Acc;
    using L = SkinnySmem<FA, NW>;
    constexpr int kThr = 64 * SW;
    constexpr int NC = L::NC;
    constexpr int kPitch = L::kPitch;
    constexpr int kTabMax = L::kTabMax;
    constexpr int kTabPer = (kTabMax + kThr - 1) / kThr;
    static_assert(FA * 32 <= kThr, "one thread per row for the row data");
    int* sum = reinterpret_cast<int*>(smem);
    float* tab = reinterpret_cast<float*>(smem + L::kSumBytes);
    float* rows_rs = reinterpret_cast<float*>(smem + L::kSumBytes + L::kTabBytes);
    int* rows_s = reinterpret_cast<int*>(smem + L::kSumBytes + L::kTabBytes + FA * 32 * 4);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nb0 = cb * NW;                       // first 32-channel block
    const int kblocks = K / F::kKSub;
    // this block's rows: group rg of FA * 32 rows
    {
        const int row0 = rg * FA * 32;
        Xq += (size_t)(row0 >> 5) * kblocks * F::kABlock;
        row_scale += row0;
        sid += row0;
        Y += (size_t)row0 * N;
        if constexpr (ACC_OUT) acc_out += (size_t)row0 * N;
        M = min(M - row0, FA * 32);
    }
    const int mb = (M + 31) >> 5;                  // 32-row blocks present (<= FA)

    for (int i = tid; i < FA * 32 * kPitch; i += kThr) sum[i] = 0;

    // epilogue operands: fetched now (in flight with the k loop), written to
    // LDS after it
    const int ntab = NC * (1 + 2 * S);
    auto tab_src = [&](int i) -> const float* {
        if (i < NC) return w_scale + nb0 * 32 + i;
        i -= NC;
        const int half = i / (NC * S);             // 0: comp_a, 1: comp_b
        i -= half * NC * S;
        return (half ? comp_b : comp_a) + (size_t)(i / NC) * N + nb0 * 32 + (i % NC);
    };
    float e_tab[kTabPer];
#pragma unroll
    for (int t = 0; t < kTabPer; ++t) {
        const int i = tid + t * kThr;
        e_tab[t] = i < ntab ? *tab_src(i) : 0.0f;
    }
    const float e_rs = tid < M ? row_scale[tid] : 0.0f;
    const int e_s = tid < M ? min(sid[tid] & (RUDDER_MAX_STREAMS - 1), S - 1) : 0;

    Acc acc[NW][FA];
#pragma unroll
    for (int i = 0; i < NW; ++i)
#pragma unroll
        for (int g = 0; g < FA; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][g][r] = 0;

    // Each wave takes a contiguous range of k-substeps and walks it in chunks
    // of D substeps; the loads of chunk c+1 are issued before the MFMAs of
    // chunk c, so two chunks (the whole range for short K) are in flight.
    constexpr int D = SkinnyChunk<FMT, FA, NW>::D;
    const int per_wave = (kblocks + SW - 1) / SW;
    const int j0 = wave * per_wave;
    const int j1 = min(j0 + per_wave, kblocks);
    SkinnyOps<FMT, FA, NW> ops[2][D];
    auto load_chunk = [&](int jc, SkinnyOps<FMT, FA, NW>(&buf)[D]) {
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (jc + d < j1)
                skinny_load<FMT, FA, NW>(Xq, Wq, nb0, jc + d, kblocks, mb, lane, buf[d]);
    };
    auto mma_chunk = [&](int jc, const SkinnyOps<FMT, FA, NW>(&buf)[D]) {
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (jc + d < j1) skinny_mma<FMT, FA, NW>(buf[d], mb, acc);
    };
    if (j0 < j1) load_chunk(j0, ops[0]);
    for (int jc = j0; jc < j1; jc += 2 * D) {
        if (jc + D < j1) load_chunk(jc + D, ops[1]);
        mma_chunk(jc, ops[0]);
        if (jc + D < j1) {
            if (jc + 2 * D < j1) load_chunk(jc + 2 * D, ops[0]);
            mma_chunk(jc + D, ops[1]);
        }
    }
#pragma unroll
    for (int t = 0; t < kTabPer; ++t) {
        const int i = tid + t * kThr;
        if (i < ntab) tab[i] = e_tab[t];
    }
    if (tid < FA * 32) {
        rows_rs[tid] = e_rs;
        rows_s[tid] = e_s;
    }
    __syncthreads();                               // sum tile cleared, operands in LDS

    // partial sums -> LDS tile [row][channel] (row pitch NC + 1 words)
#pragma unroll
    for (int i = 0; i < NW; ++i) {
#pragma unroll
        for (int g = 0; g < FA; ++g) {
            if (g < mb) {
                const int m = g * 32 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    atomicAdd(&sum[m * kPitch + n], (int)acc[i][g][r]);
                }
            }
        }
    }
    __syncthreads();

    // epilogue: item = (row m, 8-channel group c); NC / 8 items per row
    constexpr int kGroups = NC / 8;
    for (int item = tid; item < mb * 32 * kGroups; item += kThr) {
        const int m = item / kGroups;
        const int c = item % kGroups;
        if (m >= M) continue;
        const int n0 = nb0 * 32 + c * 8;
        const int st = rows_s[m];
        const float rs = rows_rs[m];
        const float* ws = tab + c * 8;
        const float* a = tab + NC + st * NC + c * 8;
        const float* b = tab + NC + NC * S + st * NC + c * 8;
        int v[8];
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int w = sum[m * kPitch + c * 8 + i];
            if constexpr (fp6_fmt(FMT)) v[i] = w;
            else if constexpr (FMT == kFmtA8) v[i] = w >> 4;
            else v[i] = w >> 8;
            y[i] = __builtin_fmaf(a[i], (float)v[i] * (rs * ws[i]), b[i]);
        }
        uint4 out;
        out.x = pack_bf16x2_rne(y[0], y[1]);
        out.y = pack_bf16x2_rne(y[2], y[3]);
        out.z = pack_bf16x2_rne(y[4], y[5]);
        out.w = pack_bf16x2_rne(y[6], y[7]);
        store_y16(Y + (size_t)m * N + n0, out);
        if constexpr (ACC_OUT) {
            *reinterpret_cast<int4*>(acc_out + (size_t)m * N + n0) =
                make_int4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<int4*>(acc_out + (size_t)m * N + n0 + 4) =
                make_int4(v[4], v[5], v[6], v[7]);
        }
    }
}

template <int FMT, int FA, int NW, bool ACC_OUT>
__global__ __launch_bounds__(kSkinnyThreads, 1) void w4_skinny_kernel(
    const uint8_t* __restrict__ Xq, const float* __restrict__ row_scale,
    const uint8_t* __restrict__ sid, const uint8_t* __restrict__ Wq,
    const float* __restrict__ w_scale, const float* __restrict__ comp_a,
    const float* __restrict__ comp_b, int M, int N, int K, int S, uint16_t* __restrict__ Y,
    int32_t* __restrict__ acc_out) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[SkinnySmem<FA, NW>::kBytes];
    skinny_tile<FMT, FA, NW, ACC_OUT, kSkinnyWaves>(Xq, row_scale, sid, Wq, w_scale, comp_a,
                                                    comp_b, M, N, K, S, Y, acc_out, blockIdx.x,
                                                    blockIdx.y, smem);
}
int device_cus();

// One launch of the weight-streaming kernel with FA * 32-row groups and NW
// 32-channel blocks per workgroup.
template <int FMT, int FA, int NW, bool ACC_OUT>
hipError_t launch_skinny(const uint8_t* xq, const float* row_scale, const uint8_t* sid,
                         const uint8_t* Wq, const float* w_scale, const float* comp_a,
                         const float* comp_b, int M, int N, int K, int S, uint16_t* Y,
                         int32_t* acc_out, hipStream_t stream) {
    const unsigned row_groups = (unsigned)((M + FA * 32 - 1) / (FA * 32));
    hipLaunchKernelGGL((w4_skinny_kernel<FMT, FA, NW, ACC_OUT>),
                       dim3((unsigned)(N / (32 * NW)), row_groups), dim3(kSkinnyThreads), 0,
                       stream, xq, row_scale, sid, Wq, w_scale, comp_a, comp_b, M, N, K, S, Y,
                       acc_out);
    return hipGetLastError();
}

// Rows per streaming block (in 32-row groups: 2 or 3) for the rows past the
// tiles of a tiled launch.  Each block reads its 32 channels' weights and its
// rows' activation codes in full, and blocks sharing a compute unit share its
// bandwidth, so the time follows (blocks per CU, rounded up) x (bytes of one
// block); the smaller is taken, 64-row groups on a tie.  The digit format
// keeps 64-row groups (registers).
template <int FMT>
int tail_rows_per_block(int rows, int N, int K) {
    using F = Fmt<FMT>;
    if (FMT == kFmtD6) return 2;
    const double w = (double)F::kWBlock / (32.0 * F::kKSub);   // bytes per weight code
    const double a = (double)F::kABlock / (32.0 * F::kKSub);   // bytes per activation code
    const long cus = device_cus();
    int best_f = 2;
    double best = 1e300;
    for (int f = 2; f <= 3; ++f) {
        const long blocks = (long)((rows + 32 * f - 1) / (32 * f)) * (N / 32);
        const long per_cu = (blocks + cus - 1) / cus;
        const double bytes = per_cu * (32.0 * K * w + (double)min(rows, 32 * f) * K * a);
        if (bytes < best * (1.0 - 1e-9)) {
            best = bytes;
            best_f = f;
        }
    }
    return best_f;
}

// split_m > 0 (int containers, bf16 output): rows split_m .. M - 1 run as
// narrow tiles in the same launch; tail_m0 > 0 (bf16 output): rows
// tail_m0 .. M - 1 run as streaming blocks in the same launch (see
// w4_gemm_kernel).
template <int FMT, int NS, bool ACC_OUT, int EPI = kEpiBf16>
hipError_t launch_variant(const uint8_t* xq, const float* row_scale, const uint8_t* sid,
                          const uint8_t* Wq, const float* w_scale, const float* comp_a,
                          const float* comp_b, int M, int N, int K, int S, uint16_t* Y,
                          int32_t* acc_out, hipStream_t stream,
                          const NextLayerQuant& nx = NextLayerQuant{}, int split_m = 0,
                          int tail_m0 = 0) {
    using C = Cfg<FMT, NS>;
    static_assert(SkinnySmem<2, 1>::kBytes <= C::lds_bytes(1) &&
                      SkinnySmem<3, 1>::kBytes <= C::lds_bytes(1),
                  "streaming blocks' LDS");
    constexpr int kExtra = EPI != kEpiBf16 ? 1 : 0;
    static_assert(C::lds_bytes(1, kExtra) <= kLdsLimit, "LDS budget");
    static_assert(EPI == kEpiBf16 || Waves<FMT>::FW == 2, "code epilogue: 64 channels per wave");
    // the attribute admits the full CU; a call whose tables do not fit the
    // per-workgroup share simply runs fewer workgroups per CU
    static const hipError_t attr = hipFuncSetAttribute(
        (const void*)w4_gemm_kernel<FMT, NS, ACC_OUT, EPI>,
        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    const int tiles_n = (N + BN - 1) / BN;
    const bool split = EPI == kEpiBf16 && !fp6_fmt(FMT) && split_m > 0 && split_m < M &&
                       split_m % BM == 0;
    const bool tail = EPI == kEpiBf16 && !split && tail_m0 > 0 && tail_m0 < M &&
                      tail_m0 % BM == 0 && M - tail_m0 <= kSkinnyMaxM;
    const int tiles_m = split ? split_m / BM : (tail ? tail_m0 / BM : (M + BM - 1) / BM);
    const int main_tiles = tiles_m * tiles_n;
    const int narrow_tiles =
        split ? ((M - split_m + BM - 1) / BM) * ((N + BN / 2 - 1) / (BN / 2)) : 0;
    const int tail_fa = tail ? tail_rows_per_block<FMT>(M - tail_m0, N, K) : 2;
    const int tail_blocks =
        tail ? ((M - tail_m0 + 32 * tail_fa - 1) / (32 * tail_fa)) * (N / 32) : 0;
    // weight touch blocks (few-row launches read the weights only once or
    // twice and go without)
    const int touch_blocks = M > kSkinnyMaxM ? kTouchBlocks : 0;
    hipLaunchKernelGGL((w4_gemm_kernel<FMT, NS, ACC_OUT, EPI>),
                       dim3((unsigned)(touch_blocks + main_tiles + narrow_tiles + tail_blocks)),
                       dim3(kThreads),
                       C::lds_bytes(S, kExtra), stream, xq, row_scale, sid, Wq, w_scale, comp_a,
                       comp_b, M, N, K, S, Y, acc_out, tiles_m, tiles_n, main_tiles,
                       split ? split_m : M, touch_blocks,
                       tail ? main_tiles + narrow_tiles : 0x7FFFFFFF, tail ? tail_m0 : M,
                       tail_fa, nx);
    return hipGetLastError();
}

// Compute units of the current device (cached per device).
int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Workgroup shape of the weight-streaming kernel: FA * 32-row groups and NW
// 32-channel blocks per workgroup, one 8-wave workgroup per compute unit at
// a time.  Every workgroup reads its weight slice and its rows' activation
// codes in full, so the time follows the operand bytes on the busiest
// compute unit: rounds of workgroups x (weight bytes + activation bytes of
// one workgroup).  The shape minimizing that is taken, the fewest rows and
// then the fewest channels on a tie.  (Measured on six few-row layer shapes,
// 32..250 rows x 2048..16384 channels, this picks the fastest shape in each;
// the 96-channel, 128-row shape runs out of registers and is not offered.)
// The digit format keeps 64-row groups: its two activation planes per
// fragment leave no registers for more.
template <int FMT>
void skinny_shape(int M, int N, int& fa, int& nw) {
    using F = Fmt<FMT>;
    const double w = (double)F::kWBlock / (32.0 * F::kKSub);   // bytes per weight code
    const double a = (double)F::kABlock / (32.0 * F::kKSub);   // bytes per activation code
    const long cus = device_cus();
    double best = 1e300;
    fa = 2;
    nw = 1;
    for (int f = 2; f <= (FMT == kFmtD6 ? 2 : 4); ++f) {
        for (int n = 1; n <= (FMT == kFmtD6 ? 2 : 3); ++n) {
            if (f * n > 9 || N % (32 * n)) continue;
            const long groups = (M + 32 * f - 1) / (32 * f);
            const long wgs = (long)(N / (32 * n)) * groups;
            const long rounds = (wgs + cus - 1) / cus;
            const double bytes = rounds * (32.0 * n * w + (double)min(M, 32 * f) * a);
            if (bytes < best * (1.0 - 1e-9)) {
                best = bytes;
                fa = f;
                nw = n;
            }
        }
    }
}

template <int FMT, bool ACC_OUT>
hipError_t launch_small(const uint8_t* xq, const float* row_scale, const uint8_t* sid,
                        const uint8_t* Wq, const float* w_scale, const float* comp_a,
                        const float* comp_b, int M, int N, int K, int S, uint16_t* Y,
                        int32_t* acc_out, hipStream_t stream) {
    int fa, nw;
    skinny_shape<FMT>(M, N, fa, nw);
#define RUDDER_SKINNY(FA_, NW_)                                                                \
    if (fa == FA_ && nw == NW_)                                                                \
        return launch_skinny<FMT, FA_, NW_, ACC_OUT>(xq, row_scale, sid, Wq, w_scale, comp_a,  \
                                                     comp_b, M, N, K, S, Y, acc_out, stream);
    RUDDER_SKINNY(2, 1)
    RUDDER_SKINNY(2, 2)
    if constexpr (FMT != kFmtD6) {
        RUDDER_SKINNY(2, 3)
        RUDDER_SKINNY(3, 1)
        RUDDER_SKINNY(3, 2)
        RUDDER_SKINNY(3, 3)
        RUDDER_SKINNY(4, 1)
        RUDDER_SKINNY(4, 2)
    }
#undef RUDDER_SKINNY
    return hipErrorInvalidValue;          // not reached: skinny_shape offers only the above
}

// The tiled kernel's LDS ring holds two stages of activation codes.
constexpr int kRing = 2;

template <int FMT, bool ACC_OUT, int EPI = kEpiBf16>
hipError_t launch_tiled(const uint8_t* xq, const float* row_scale, const uint8_t* sid,
                        const uint8_t* Wq, const float* w_scale, const float* comp_a,
                        const float* comp_b, int M, int N, int K, int S, uint16_t* Y,
                        int32_t* acc_out, hipStream_t stream,
                        const NextLayerQuant& nx = NextLayerQuant{}, int split_m = 0,
                        int tail_m0 = 0) {
    // every stream count fits a CU (calls with many streams may run one
    // workgroup per CU instead of two)
    static_assert(Cfg<FMT, kRing>::lds_bytes(RUDDER_MAX_STREAMS, 1) <= 160 * 1024, "LDS budget");
    return launch_variant<FMT, kRing, ACC_OUT, EPI>(xq, row_scale, sid, Wq, w_scale, comp_a,
                                                    comp_b, M, N, K, S, Y, acc_out, stream, nx,
                                                    split_m, tail_m0);
}

template <int FMT, bool ACC_OUT>
hipError_t launch_fmt(const uint8_t* xq, const float* row_scale, const uint8_t* sid,
                      const uint8_t* Wq, const float* w_scale, const float* comp_a,
                      const float* comp_b, int M, int N, int K, int S, uint16_t* Y,
                      int32_t* acc_out, hipStream_t stream) {
    // few token rows: the weight-streaming kernel
    if (M <= kSkinnyMaxM)
        return launch_small<FMT, ACC_OUT>(xq, row_scale, sid, Wq, w_scale, comp_a, comp_b, M, N,
                                          K, S, Y, acc_out, stream);
    // Ragged last round: when the tiles fill whole rounds of resident
    // workgroups except for a few rows (at most kSkinnyMaxM), the tiles take
    // the rows of the full rounds and weight-streaming blocks appended to
    // the same launch take the rest, instead of a nearly empty extra round
    // of tiles; those blocks start as the tiles drain, with no launch gap.
    // Streaming reads the weights once per row group, so this pays only for
    // narrow layers: groups * N <= kSplitMaxWidth (measured on 2048-, 4096-
    // and 8192-wide layers, where a separate streaming launch saved 5-25%; on
    // 12288- and 16384-wide layers the partial round is cheaper, and the int
    // containers run it as half-width tiles).
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles = ((M + BM - 1) / BM) * tiles_n;
    const int per_cu = (int)((160 * 1024) / Cfg<FMT, kRing>::lds_bytes(S));
    const int slots = device_cus() * (per_cu < kBlocksPerCU ? per_cu : kBlocksPerCU);
    const int full = slots > 0 ? tiles / slots : 0;
    const int rem = tiles - full * slots;
    // The tiles that run as full tiles: whole rounds, and then at most one
    // more per compute unit.  A partial round with more tiles than compute
    // units puts two co-resident tiles on a few of them, and those set the
    // launch time (a lone tile takes well under the time of two together);
    // the rows past one tile per CU then go to the streaming blocks or
    // half-width tiles below, which fill the free second slots beside the
    // lone tiles.
    const int cus = device_cus();
    const bool pairs_in_last = rem > cus && per_cu >= kBlocksPerCU;
    const int lead = full * slots + (pairs_in_last ? cus : 0);
    if (rem != 0 && lead > 0) {
        const int m_main = (lead / tiles_n) * BM;
        const int tail = M - m_main;
        const int groups = (tail + 127) / 128;
        if (m_main > 0 && tail > 0 && tail <= kSkinnyMaxM && groups * N <= kSplitMaxWidth)
            return launch_tiled<FMT, ACC_OUT>(xq, row_scale, sid, Wq, w_scale, comp_a, comp_b, M,
                                              N, K, S, Y, acc_out, stream, NextLayerQuant{}, 0,
                                              m_main);
        // wider layers, int containers: the remainder as half-width tiles in
        // the same launch
        if (!fp6_fmt(FMT) && m_main > 0 && tail > 0 && tail <= kSkinnyMaxM && N >= BN)
            return launch_tiled<FMT, ACC_OUT>(xq, row_scale, sid, Wq, w_scale, comp_a, comp_b, M,
                                              N, K, S, Y, acc_out, stream, NextLayerQuant{},
                                              m_main);
    }
    return launch_tiled<FMT, ACC_OUT>(xq, row_scale, sid, Wq, w_scale, comp_a, comp_b, M, N, K,
                                      S, Y, acc_out, stream);
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
    if (codes == RUDDER_CODES_E2M3 && abits == 8) RUDDER_LAUNCH(kFmtD6);
    if (codes == RUDDER_CODES_E2M3) RUDDER_LAUNCH(kFmtF6);
    if (abits == 8) RUDDER_LAUNCH(kFmtA8);
    RUDDER_LAUNCH(kFmtA4);
#undef RUDDER_LAUNCH
}

namespace {

template <int FMT>
hipError_t launch_fused_fmt(const uint8_t* xq, const float* row_scale, const uint8_t* sid,
                            const uint8_t* Wq, const float* w_scale, const float* comp_a,
                            const float* comp_b, int M, int N, int K, int S,
                            const NextLayerQuant& nx, hipStream_t stream) {
    if (nx.codes == RUDDER_CODES_E2M3)
        return launch_tiled<FMT, false, kEpiE2M3>(xq, row_scale, sid, Wq, w_scale, comp_a,
                                                  comp_b, M, N, K, S, nullptr, nullptr, stream,
                                                  nx);
    if (nx.abits == 8)
        return launch_tiled<FMT, false, kEpiQ8>(xq, row_scale, sid, Wq, w_scale, comp_a,
                                                comp_b, M, N, K, S, nullptr, nullptr, stream, nx);
    return launch_tiled<FMT, false, kEpiQ4>(xq, row_scale, sid, Wq, w_scale, comp_a, comp_b,
                                            M, N, K, S, nullptr, nullptr, stream, nx);
}

// 8 values per thread with 16-byte loads and stores when both buffers are
// 16-byte aligned; element by element otherwise and for the tail.
__global__ __launch_bounds__(256) void gelu_bf16_kernel(const uint16_t* __restrict__ in,
                                                        uint16_t* __restrict__ out, size_t n) {
    const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * 256;
    size_t head = 0;
    if ((((uintptr_t)in | (uintptr_t)out) & 15u) == 0) {
        const size_t n8 = n / 8;
        for (size_t v = tid; v < n8; v += stride) {
            const uint4 x = reinterpret_cast<const uint4*>(in)[v];
            uint4 y;
            y.x = kGeluBf16[x.x & 0xFFFFu] | ((uint32_t)kGeluBf16[x.x >> 16] << 16);
            y.y = kGeluBf16[x.y & 0xFFFFu] | ((uint32_t)kGeluBf16[x.y >> 16] << 16);
            y.z = kGeluBf16[x.z & 0xFFFFu] | ((uint32_t)kGeluBf16[x.z >> 16] << 16);
            y.w = kGeluBf16[x.w & 0xFFFFu] | ((uint32_t)kGeluBf16[x.w >> 16] << 16);
            reinterpret_cast<uint4*>(out)[v] = y;
        }
        head = n8 * 8;
    }
    for (size_t i = head + tid; i < n; i += stride) out[i] = kGeluBf16[in[i]];
}

}  // namespace

hipError_t launch_linear_gelu_quant(const void* Xq, const float* row_scale, const uint8_t* sid,
                                    const uint8_t* Wq, const float* w_scale, const float* comp_a,
                                    const float* comp_b, int M, int N, int K, int S, int abits,
                                    int codes, const NextLayerQuant& next, hipStream_t stream) {
    const uint8_t* xq = static_cast<const uint8_t*>(Xq);
    // (8-bit codes in the E2M3 container are not built for this path)
    if (codes == RUDDER_CODES_E2M3 && abits == 8) return hipErrorInvalidValue;
    if (codes == RUDDER_CODES_E2M3)
        return launch_fused_fmt<kFmtF6>(xq, row_scale, sid, Wq, w_scale, comp_a, comp_b, M, N, K,
                                        S, next, stream);
    if (abits == 8)
        return launch_fused_fmt<kFmtA8>(xq, row_scale, sid, Wq, w_scale, comp_a, comp_b, M, N, K,
                                        S, next, stream);
    return launch_fused_fmt<kFmtA4>(xq, row_scale, sid, Wq, w_scale, comp_a, comp_b, M, N, K, S,
                                    next, stream);
}

hipError_t launch_gelu_bf16(const uint16_t* in, uint16_t* out, size_t n, hipStream_t stream) {
    const size_t blocks = (n / 8 + 255) / 256 + 1;
    hipLaunchKernelGGL(gelu_bf16_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                       dim3(256), 0, stream, in, out, n);
    return hipGetLastError();
}

}  // namespace rudder
