"""Python binding of librudder (ctypes).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI declared in include/rudder.h.  torch supplies device memory
and the current HIP stream.  If the library is missing this module raises;
there is no CPU fallback.

The calls keep their C names and meanings:
  rudder_quantize_weights  -- offline weight preparation (SteerQuant Fig. 2, §4.2)
  rudder_quant_act         -- fused activation quantization (SteerQuant §4.3, §4.4)
  rudder_linear            -- low-bit GEMM + fused epilogue (SteerQuant §4.4)
  rudder_linear_gelu_quant -- MLP up-projection with GELU (kept in BF16, App. D)
                              and the down layer's quantizer in its epilogue
  rudder_gelu_bf16         -- that GELU alone, elementwise
(SteerQuant = "SteerQuant: Steering Quantization Error with Action-Guided
Scaling in World-Action Models", paperlayer.ai digest.)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_lib", "librudder.so")

CODES_INT = 0       # int4 split-nibble / int8 codes (int8 matrix cores)
CODES_E2M3 = 1      # codes held as FP6 E2M3 (8-bit codes as two digit planes); f8f6f4 MFMA

RUDDER_OK = 0
RUDDER_ERR_INVALID_ARG = 1
RUDDER_ERR_UNSUPPORTED = 2
RUDDER_ERR_HIP = 3
MAX_STREAMS = 8

EXPORTED = (
    "rudder_packed_weight_bytes", "rudder_packed_act_bytes", "rudder_quant_act_workspace_bytes",
    "rudder_quantize_weights", "rudder_quant_act", "rudder_quant_act_noalloc", "rudder_linear",
    "rudder_linear_gelu_quant", "rudder_gelu_bf16",
    "rudder_dequant_weights", "rudder_stream_sq_error_workspace_bytes", "rudder_stream_sq_error",
    "rudder_status_string", "rudder_last_error",
    "rudder_mfma_ceiling_sink_bytes", "rudder_mfma_ceiling_ops", "rudder_mfma_ceiling",
    "rudder_mfma_ceiling_shape",
)

_lib: Optional[ctypes.CDLL] = None


class RudderError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load the in-tree librudder.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RudderError(RUDDER_ERR_HIP,
                          f"{LIB_PATH} not found: build it with __graft_entry__.build() "
                          "or python w4a4_quantized_gemm_rudder_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.rudder_packed_weight_bytes.argtypes = [i, i, i]
    lib.rudder_packed_weight_bytes.restype = sz
    lib.rudder_packed_act_bytes.argtypes = [i, i, i, i]
    lib.rudder_packed_act_bytes.restype = sz
    lib.rudder_quant_act_workspace_bytes.argtypes = [i]
    lib.rudder_quant_act_workspace_bytes.restype = sz
    lib.rudder_quantize_weights.argtypes = [vp, vp, i, i, i, vp, vp, vp, vp]
    lib.rudder_quantize_weights.restype = i
    lib.rudder_quant_act.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp]
    lib.rudder_quant_act.restype = i
    lib.rudder_quant_act_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp]
    lib.rudder_quant_act_noalloc.restype = i
    lib.rudder_linear.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, vp, vp]
    lib.rudder_linear.restype = i
    lib.rudder_linear_gelu_quant.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i,
                                             vp, vp, i, i, vp, vp, vp]
    lib.rudder_linear_gelu_quant.restype = i
    lib.rudder_gelu_bf16.argtypes = [vp, vp, sz, vp]
    lib.rudder_gelu_bf16.restype = i
    lib.rudder_dequant_weights.argtypes = [vp, vp, i, i, i, vp, vp]
    lib.rudder_dequant_weights.restype = i
    lib.rudder_stream_sq_error_workspace_bytes.argtypes = []
    lib.rudder_stream_sq_error_workspace_bytes.restype = sz
    lib.rudder_stream_sq_error.argtypes = [vp, vp, vp, i, i, i, vp, vp, vp]
    lib.rudder_stream_sq_error.restype = i
    lib.rudder_mfma_ceiling_sink_bytes.argtypes = []
    lib.rudder_mfma_ceiling_sink_bytes.restype = sz
    lib.rudder_mfma_ceiling_ops.argtypes = [i, i]
    lib.rudder_mfma_ceiling_ops.restype = ctypes.c_double
    lib.rudder_mfma_ceiling.argtypes = [vp, vp, i, i, i, i, i, i, vp, vp]
    lib.rudder_mfma_ceiling.restype = i
    lib.rudder_mfma_ceiling_shape.argtypes = [vp, vp, i, i, i, i, i, i, i, vp, vp]
    lib.rudder_mfma_ceiling_shape.restype = i
    lib.rudder_status_string.argtypes = [i]
    lib.rudder_status_string.restype = ctypes.c_char_p
    lib.rudder_last_error.argtypes = []
    lib.rudder_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != RUDDER_OK:
        lib = load_library()
        name = lib.rudder_status_string(status).decode()
        raise RudderError(status, f"{name}: {lib.rudder_last_error().decode()}")


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (None -> NULL).  Plain ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to librudder must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# Size helpers
# ---------------------------------------------------------------------------

def packed_weight_bytes(K: int, N: int, codes: int = CODES_INT) -> int:
    return int(load_library().rudder_packed_weight_bytes(K, N, codes))


def packed_act_bytes(M: int, K: int, abits: int, codes: int = CODES_INT) -> int:
    return int(load_library().rudder_packed_act_bytes(M, K, abits, codes))


def quant_act_workspace_bytes(S: int) -> int:
    return int(load_library().rudder_quant_act_workspace_bytes(S))


# ---------------------------------------------------------------------------
# The three calls (same names and argument order as the C ABI, sizes passed
# explicitly; tensors are device tensors, bf16 data as torch.bfloat16 or
# int16/uint16 bit patterns)
# ---------------------------------------------------------------------------

def rudder_quantize_weights(W, smooth, K: int, N: int, codes: int, Wq, w_scale, inv_smooth,
                            stream=None) -> None:
    _check(load_library().rudder_quantize_weights(
        _ptr(W), _ptr(smooth), K, N, codes, _ptr(Wq), _ptr(w_scale), _ptr(inv_smooth),
        _stream(stream)))


def rudder_quant_act(X, stream_id, inv_smooth, act_scale, act_scale_out, workspace,
                     M: int, K: int, S: int, abits: int, codes: int, Xq, row_scale,
                     stream=None) -> None:
    _check(load_library().rudder_quant_act(
        _ptr(X), _ptr(stream_id), _ptr(inv_smooth), _ptr(act_scale), _ptr(act_scale_out),
        _ptr(workspace), M, K, S, abits, codes, _ptr(Xq), _ptr(row_scale), _stream(stream)))


def rudder_quant_act_noalloc(X, stream_id, inv_smooth, act_scale_out, M: int, K: int, S: int,
                             abits: int, codes: int, Xq, row_scale, stream=None) -> None:
    _check(load_library().rudder_quant_act_noalloc(
        _ptr(X), _ptr(stream_id), _ptr(inv_smooth), _ptr(act_scale_out), M, K, S, abits, codes,
        _ptr(Xq), _ptr(row_scale), _stream(stream)))


def rudder_linear(Xq, row_scale, stream_id, Wq, w_scale, comp_a, comp_b,
                  M: int, N: int, K: int, S: int, abits: int, codes: int, Y, acc_out=None,
                  stream=None) -> None:
    _check(load_library().rudder_linear(
        _ptr(Xq), _ptr(row_scale), _ptr(stream_id), _ptr(Wq), _ptr(w_scale), _ptr(comp_a),
        _ptr(comp_b), M, N, K, S, abits, codes, _ptr(Y), _ptr(acc_out), _stream(stream)))


def rudder_linear_gelu_quant(Xq, row_scale, stream_id, Wq, w_scale, comp_a, comp_b,
                             M: int, N: int, K: int, S: int, abits: int, codes: int,
                             next_inv_smooth, next_act_scale, next_abits: int, next_codes: int,
                             next_Xq, next_row_scale, stream=None) -> None:
    _check(load_library().rudder_linear_gelu_quant(
        _ptr(Xq), _ptr(row_scale), _ptr(stream_id), _ptr(Wq), _ptr(w_scale), _ptr(comp_a),
        _ptr(comp_b), M, N, K, S, abits, codes, _ptr(next_inv_smooth), _ptr(next_act_scale),
        next_abits, next_codes, _ptr(next_Xq), _ptr(next_row_scale), _stream(stream)))


def rudder_gelu_bf16(x, out, n: int, stream=None) -> None:
    _check(load_library().rudder_gelu_bf16(_ptr(x), _ptr(out), n, _stream(stream)))


def rudder_dequant_weights(Wq, w_scale, K: int, N: int, codes: int, out, stream=None) -> None:
    _check(load_library().rudder_dequant_weights(_ptr(Wq), _ptr(w_scale), K, N, codes, _ptr(out),
                                                 _stream(stream)))


def stream_sq_error_workspace_bytes() -> int:
    return int(load_library().rudder_stream_sq_error_workspace_bytes())


def rudder_stream_sq_error(Y, Yref, stream_id, M: int, N: int, S: int, workspace, sse,
                           stream=None) -> None:
    _check(load_library().rudder_stream_sq_error(_ptr(Y), _ptr(Yref), _ptr(stream_id), M, N, S,
                                                 _ptr(workspace), _ptr(sse), _stream(stream)))


# ---------------------------------------------------------------------------
# Allocating conveniences (torch allocates; the library computes)
# ---------------------------------------------------------------------------

def quantize_weights(W, smooth, codes: int = CODES_INT, stream=None):
    """W: bf16 [K, N] device tensor, smooth: fp32 [K].
    Returns (Wq uint8, w_scale fp32 [N], inv_smooth fp32 [K])."""
    import torch
    K, N = W.shape
    dev = W.device
    Wq = torch.empty(packed_weight_bytes(K, N, codes), dtype=torch.uint8, device=dev)
    w_scale = torch.empty(N, dtype=torch.float32, device=dev)
    inv_smooth = torch.empty(K, dtype=torch.float32, device=dev)
    rudder_quantize_weights(W, smooth, K, N, codes, Wq, w_scale, inv_smooth, stream)
    return Wq, w_scale, inv_smooth


def quant_act(X, stream_id, inv_smooth, act_scale, S: int, abits: int, codes: int = CODES_INT,
              stream=None, act_scale_out=None, workspace=None):
    """X: bf16 [M, K].  act_scale: fp32 [S] device tensor, or None for dynamic
    (absmax) step sizes.  Returns (Xq uint8, row_scale fp32 [M])."""
    import torch
    M, K = X.shape
    dev = X.device
    Xq = torch.empty(max(packed_act_bytes(M, K, abits, codes), 1), dtype=torch.uint8,
                     device=dev)
    row_scale = torch.empty(max(M, 1), dtype=torch.float32, device=dev)
    if act_scale is None and workspace is None:
        workspace = torch.empty(quant_act_workspace_bytes(S), dtype=torch.uint8, device=dev)
    rudder_quant_act(X, stream_id, inv_smooth, act_scale, act_scale_out, workspace, M, K, S,
                     abits, codes, Xq, row_scale, stream)
    return Xq, row_scale


def linear(Xq, row_scale, stream_id, Wq, w_scale, comp_a, comp_b, M: int, N: int, K: int,
           S: int, abits: int, codes: int = CODES_INT, stream=None, acc_out: bool = False):
    """Returns Y bf16 [M, N] (and int32 accumulators [M, N] if acc_out)."""
    import torch
    dev = Wq.device
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev) if acc_out else None
    rudder_linear(Xq, row_scale, stream_id, Wq, w_scale, comp_a, comp_b, M, N, K, S, abits,
                  codes, Y, acc, stream)
    return (Y, acc) if acc_out else Y


def linear_gelu_quant(Xq, row_scale, stream_id, Wq, w_scale, comp_a, comp_b, M: int, N: int,
                      K: int, S: int, abits: int, next_inv_smooth, next_act_scale,
                      next_abits: int, codes: int = CODES_INT, next_codes: int = CODES_INT,
                      stream=None):
    """Returns (next Xq uint8, next row_scale fp32 [M]): the down layer's
    packed input and row scales, from the up-projection's codes."""
    import torch
    dev = Wq.device
    nxq = torch.empty(max(packed_act_bytes(M, N, next_abits, next_codes), 1), dtype=torch.uint8,
                      device=dev)
    nrs = torch.empty(max(M, 1), dtype=torch.float32, device=dev)
    rudder_linear_gelu_quant(Xq, row_scale, stream_id, Wq, w_scale, comp_a, comp_b, M, N, K, S,
                             abits, codes, next_inv_smooth, next_act_scale, next_abits,
                             next_codes, nxq, nrs, stream)
    return nxq, nrs


def gelu_bf16(x, stream=None):
    """GELU of a bf16 tensor (same table as the fused epilogue)."""
    import torch
    out = torch.empty_like(x)
    rudder_gelu_bf16(x, out, x.numel(), stream)
    return out


# ---------------------------------------------------------------------------
# Measurement (include/rudder_diag.h)
# ---------------------------------------------------------------------------
def mfma_ceiling_sink_bytes() -> int:
    return int(load_library().rudder_mfma_ceiling_sink_bytes())


def mfma_ceiling_ops(iters: int, codes: int) -> float:
    return float(load_library().rudder_mfma_ceiling_ops(iters, codes))


def rudder_mfma_ceiling(Xq, Wq, M: int, N: int, K: int, abits: int, codes: int, iters: int,
                        sink, stream=None) -> None:
    _check(load_library().rudder_mfma_ceiling(_ptr(Xq), _ptr(Wq), M, N, K, abits, codes, iters,
                                              _ptr(sink), _stream(stream)))


CEILING_OWN = 0             # the instruction rudder_linear uses
CEILING_I8_16X16X64 = 1     # v_mfma_i32_16x16x64_i8 (int containers)


def rudder_mfma_ceiling_shape(Xq, Wq, M: int, N: int, K: int, abits: int, codes: int,
                              iters: int, shape: int, sink, stream=None) -> None:
    _check(load_library().rudder_mfma_ceiling_shape(_ptr(Xq), _ptr(Wq), M, N, K, abits, codes,
                                                    iters, shape, _ptr(sink), _stream(stream)))
