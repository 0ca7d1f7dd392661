"""numpy wrappers around the C oracle (rudder_oracle.c).

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the
benchmark's CPU-baseline leg.  Parity status of each function is stated in
its docstring ("pinned by" lists the independent checks in
tests/test_oracle_pins.py).

Cited passages are from "SteerQuant: Steering Quantization Error with
Action-Guided Scaling in World-Action Models" (paperlayer.ai digest).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "build", "load", "bf16_to_f32", "f32_to_bf16", "inv_smooth", "quantize_weights",
    "dynamic_scales", "quant_act", "pack_int4", "unpack_int4", "int_gemm", "epilogue",
    "linear", "gelu_bf16", "linear_gelu_quant", "num_threads", "OracleError",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rudder_oracle.c")
_LIB = os.path.join(_HERE, "_build", "liboracle.so")
_CFLAGS = ["-O3", "-mavx2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra"]

_lib: Optional[ctypes.CDLL] = None


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile rudder_oracle.c with gcc into oracle/_build/liboracle.so."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=False)
        _lib = ctypes.CDLL(_LIB)
        _lib.oracle_num_threads.restype = ctypes.c_int
    return _lib


def _p(a: np.ndarray) -> ctypes.c_void_p:
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str) -> None:
    if rc == 1:
        raise OracleError(f"{what}: invalid input (non-finite value, bad stream id or bad size)")
    if rc == 2:
        raise OracleError(f"{what}: integer accumulator does not fit int32")
    if rc != 0:
        raise OracleError(f"{what}: status {rc}")


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(load().oracle_num_threads())


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float32)
    load().oracle_bf16_to_f32(_p(bits), _p(out), ctypes.c_long(bits.size))
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even.  Pinned by: torch's bf16 cast."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    load().oracle_f32_to_bf16(_p(x), _p(out), ctypes.c_long(x.size))
    return out


def inv_smooth(s: np.ndarray) -> np.ndarray:
    """fp32 1/s formed in fp64 (SteerQuant §4.2: activations are scaled by the
    inverse of the shared diagonal).  Pinned by: the fp64 identity test."""
    s = _c(s, np.float32)
    out = np.empty_like(s)
    _check(load().oracle_inv_smooth(_p(s), ctypes.c_int(s.size), _p(out)), "inv_smooth")
    return out


def quantize_weights(W: np.ndarray, s: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Fold the smoothing diagonal into W [K, N] (bf16 bits) and quantize each
    output channel to symmetric int4 (SteerQuant §4.2, Fig. 2 offline weight
    preparation; §3.1 symmetric quantizer).

    Returns (codes int8 [N, K], w_scale fp32 [N]).  Pinned by: brute-force
    nearest-code search, round-trip half-step bound, max-code invariant,
    fp64 identity.
    """
    W = _c(W, np.uint16)
    s = _c(s, np.float32)
    K, N = W.shape
    codes = np.empty((N, K), np.int8)
    ws = np.empty(N, np.float32)
    _check(load().oracle_quantize_weights(_p(W), _p(s), K, N, _p(codes), _p(ws)),
           "quantize_weights")
    return codes, ws


def dynamic_scales(X: np.ndarray, stream_id: np.ndarray, inv_s: np.ndarray, S: int,
                   abits: int) -> np.ndarray:
    """Per-stream step sizes from the absmax of the smoothed activations.
    Pinned by: max-code invariant per non-empty stream, brute force."""
    X = _c(X, np.uint16)
    sid = _c(stream_id, np.uint8)
    inv_s = _c(inv_s, np.float32)
    M, K = X.shape
    out = np.empty(S, np.float32)
    qa = 127 if abits == 8 else 7
    _check(load().oracle_dynamic_scales(_p(X), _p(sid), _p(inv_s), M, K, S, qa, _p(out)),
           "dynamic_scales")
    return out


def quant_act(X: np.ndarray, stream_id: np.ndarray, inv_s: np.ndarray, delta: np.ndarray,
              S: int, abits: int) -> Tuple[np.ndarray, np.ndarray]:
    """Fused activation quantization: smoothing, per-(stream, step) step size,
    RNE, clamp (SteerQuant §4.4 and §4.3).  Returns (codes int8 [M, K],
    row_scale fp32 [M]).  Pinned by: constructed RNE ties, brute-force
    nearest-code search, half-step round-trip bound, stream invariants."""
    X = _c(X, np.uint16)
    sid = _c(stream_id, np.uint8)
    inv_s = _c(inv_s, np.float32)
    delta = _c(delta, np.float32)
    M, K = X.shape
    codes = np.empty((M, K), np.int8)
    rs = np.empty(M, np.float32)
    qa = 127 if abits == 8 else 7
    _check(load().oracle_quant_act(_p(X), _p(sid), _p(inv_s), _p(delta), M, K, S, qa,
                                   _p(codes), _p(rs)), "quant_act")
    return codes, rs


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """int8 codes [R, K] -> uint8 [R, K/2], two codes per byte (code 2i in
    the low nibble of byte i, code 2i+1 in the high nibble).  A storage
    format only: parity compares unpacked codes.  Pinned by: a hand-derived
    byte fixture in tests/golden, one-code placement, round trip."""
    codes = _c(codes, np.int8)
    R, K = codes.shape
    out = np.empty((R, K // 2), np.uint8)
    _check(load().oracle_pack_int4(_p(codes), ctypes.c_long(R), K, _p(out)), "pack_int4")
    return out


def unpack_int4(packed: np.ndarray, K: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    R = packed.shape[0]
    out = np.empty((R, K), np.int8)
    _check(load().oracle_unpack_int4(_p(packed), ctypes.c_long(R), K, _p(out)), "unpack_int4")
    return out


def int_gemm(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k qa[m, k] * qw[n, k], explicit integer dot products
    (SteerQuant §4.4 low-bit GEMM).  Pinned by: Python-int brute force."""
    qa = _c(qa, np.int8)
    qw = _c(qw, np.int8)
    M, K = qa.shape
    N = qw.shape[0]
    assert qw.shape[1] == K
    acc = np.empty((M, N), np.int32)
    _check(load().oracle_int_gemm(_p(qa), _p(qw), M, N, K, _p(acc)), "int_gemm")
    return acc


def epilogue(acc: np.ndarray, row_scale: np.ndarray, stream_id: np.ndarray,
             w_scale: np.ndarray, comp_a: np.ndarray, comp_b: np.ndarray) -> np.ndarray:
    """Dequantize, per-(stream, output-channel) compensation and bias, bf16
    store (SteerQuant §4.4).  Returns bf16 bits [M, N].  Pinned by: a=1,b=0 and
    a=0 special cases, fp64 bound, textbook integer GEMM special case."""
    acc = _c(acc, np.int32)
    rs = _c(row_scale, np.float32)
    sid = _c(stream_id, np.uint8)
    ws = _c(w_scale, np.float32)
    ca = _c(comp_a, np.float32)
    cb = _c(comp_b, np.float32)
    M, N = acc.shape
    S = ca.shape[0]
    Y = np.empty((M, N), np.uint16)
    _check(load().oracle_epilogue(_p(acc), _p(rs), _p(sid), _p(ws), _p(ca), _p(cb),
                                  M, N, S, _p(Y)), "epilogue")
    return Y


def gelu_bf16(bits: np.ndarray) -> np.ndarray:
    """GELU between the MLP projections, kept in BF16 (SteerQuant App. D):
    the exact erf form of a bf16 input, fp64, rounded to fp32 then bf16.
    Pinned by: scipy's independent erfc over all 65536 inputs, closed-form
    values, the identity gelu(x) - gelu(-x) = x, the tails."""
    b = _c(bits, np.uint16)
    out = np.empty_like(b)
    load().oracle_gelu_bf16(_p(b), _p(out), ctypes.c_long(b.size))
    return out


def linear_gelu_quant(X, stream_id, codes_w, w_scale, inv_s, delta, comp_a, comp_b, S, abits,
                      next_inv_s, next_delta, next_abits):
    """Up-projection, GELU in BF16 and the next (down) layer's activation
    quantizer, as one fused call would compute them (SteerQuant §4.4: only
    integer activations and row scales travel between kernels; App. D: GELU
    stays BF16).  The composition of linear, gelu_bf16 and quant_act.
    Returns (next act codes, next row_scale)."""
    _, _, _, Y = linear(X, stream_id, codes_w, w_scale, inv_s, delta, comp_a, comp_b, S, abits)
    G = gelu_bf16(Y)
    return quant_act(G, stream_id, next_inv_s, next_delta, S, next_abits)


def linear(X, stream_id, codes_w, w_scale, inv_s, delta, comp_a, comp_b, S, abits):
    """The whole call at one step: quantize activations, integer GEMM,
    epilogue.  Returns (act codes, row_scale, acc, Y bits)."""
    qa, rs = quant_act(X, stream_id, inv_s, delta, S, abits)
    acc = int_gemm(qa, codes_w)
    Y = epilogue(acc, rs, stream_id, w_scale, comp_a, comp_b)
    return qa, rs, acc, Y
