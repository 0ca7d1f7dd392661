/*
 * rudder_diag.h -- measurement entry point of librudder (not part of the
 * linear layer's data path).
 *
 * The matrix cores of the MI355X draw power in proportion to the bit
 * activity of their operands, and the chip lowers its clock to stay within
 * its power limit, so the attainable MFMA rate of a GEMM depends on the codes
 * it multiplies.  rudder_mfma_ceiling runs the tiled GEMM's per-substep MFMA
 * pattern (2 weight x 4 activation fragments of 32 channels / 32 tokens,
 * 8 independent accumulators) on fragments taken from a layer's own packed
 * codes, from registers only (no LDS, no memory traffic in the loop), so
 * that the GEMM's measured rate can be set against the MFMA-only rate those
 * operands allow.  Conventions (device pointers, stream, validation,
 * rudder_last_error) are those of rudder.h.
 */
#ifndef RUDDER_DIAG_H
#define RUDDER_DIAG_H

#include <stddef.h>
#include <stdint.h>

#include "rudder.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups of one rudder_mfma_ceiling launch (two per compute unit). */
#define RUDDER_CEILING_BLOCKS 512

/* Bytes of the int32 `sink` buffer a launch writes (one value per thread). */
size_t rudder_mfma_ceiling_sink_bytes(void);

/* Multiply-add ops (2 per multiply-accumulate) of one launch with `iters`
 * iterations for the container `codes`; 0 for iters <= 0. */
double rudder_mfma_ceiling_ops(int iters, int codes);

/* One launch of RUDDER_CEILING_BLOCKS x 256 threads.  Each wave reads 12
 * fragments (two sets of 2 weight and 4 activation fragments) of the packed
 * codes Xq (M x K, `abits`, `codes`; layout of rudder.h) and Wq (N x K),
 * from blocks picked by a fixed hash, then runs `iters` iterations of 16
 * MFMAs (8 per set) on them.  The same matrix-core instruction as
 * rudder_linear with the same (abits, codes): int8 MFMA for
 * RUDDER_CODES_INT (int4 codes widened), FP6 f8f6f4 MFMA for
 * RUDDER_CODES_E2M3 (abits = 8: one pair of MFMAs per product, one per
 * digit plane, from one set of 2 weight and 4 two-plane activation fragments
 * run twice per iteration; the op count per iteration is the same).
 * `sink` (rudder_mfma_ceiling_sink_bytes(), 16-byte
 * aligned) receives per-thread checksums so that no work is elided; its
 * values carry no meaning.  Time the launch on `stream` and divide
 * rudder_mfma_ceiling_ops(iters, codes) by its duration.
 * Returns RUDDER_ERR_INVALID_ARG for null or misaligned pointers, abits not
 * 4 / 8, an unknown container, M <= 0, N not a positive
 * multiple of 32, K not a positive multiple of 32 (64 for E2M3), or iters
 * outside 1..2^24; the code buffers must hold at least
 * rudder_packed_act_bytes(M, K, abits, codes) and
 * rudder_packed_weight_bytes(K, N, codes) bytes. */
rudder_status_t rudder_mfma_ceiling(const uint8_t* Xq, const uint8_t* Wq, int M, int N, int K,
                                    int abits, int codes, int iters, int32_t* sink, void* stream);

/* Instruction shapes for rudder_mfma_ceiling_shape. */
#define RUDDER_CEILING_OWN 0           /* the instruction rudder_linear uses */
#define RUDDER_CEILING_I8_16X16X64 1   /* v_mfma_i32_16x16x64_i8 (int containers) */

/* rudder_mfma_ceiling with a choice of matrix-core instruction: `shape`
 * RUDDER_CEILING_OWN is rudder_mfma_ceiling itself; RUDDER_CEILING_I8_16X16X64
 * feeds the same int8 fragments (int4 codes widened) to
 * v_mfma_i32_16x16x64_i8, two instructions per 32x32x32 product of the
 * pattern, so that rudder_mfma_ceiling_ops(iters, RUDDER_CODES_INT) still
 * counts the ops of a launch.  Errors as for rudder_mfma_ceiling, plus
 * RUDDER_ERR_INVALID_ARG for an unknown shape or RUDDER_CEILING_I8_16X16X64
 * with codes other than RUDDER_CODES_INT. */
rudder_status_t rudder_mfma_ceiling_shape(const uint8_t* Xq, const uint8_t* Wq, int M, int N,
                                          int K, int abits, int codes, int iters, int shape,
                                          int32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RUDDER_DIAG_H */
