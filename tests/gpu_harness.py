"""Shared plumbing for the GPU parity tests: run the HIP path through the C
ABI and the CPU oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import sys
from typing import Dict, Optional

import numpy as np

import oracle
from tiled_layout import tile_codes, tile_codes_e2m3, tile_codes_e2m3_a8

CODES_INT, CODES_E2M3 = 0, 1


def tile_for(codes_kind: int, codes: np.ndarray, bits: int) -> np.ndarray:
    """Oracle codes -> the byte layout the library writes for that container."""
    if codes_kind == CODES_E2M3:
        return tile_codes_e2m3_a8(codes) if bits == 8 else tile_codes_e2m3(codes)
    return tile_codes(codes, bits)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_to_host_bits(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between two arrays of bf16 bit patterns."""
    def ordered(b):
        b = b.astype(np.int32)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def bf16_value(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def assert_bits_equal(name: str, got: np.ndarray, want: np.ndarray) -> None:
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    gv = got.view(np.uint8) if got.dtype != np.uint8 else got
    wv = want.view(np.uint8) if want.dtype != np.uint8 else want
    if not np.array_equal(gv, wv):
        bad = np.nonzero(got.reshape(-1).view(np.uint8 if got.dtype == np.uint8 else got.dtype)
                         != want.reshape(-1))[0] if got.dtype == want.dtype else None
        first = None if bad is None or len(bad) == 0 else int(bad[0])
        raise AssertionError(f"{name}: not bit-exact ({0 if bad is None else len(bad)} "
                             f"mismatches, first flat index {first})")


def assert_y_close(name: str, got: np.ndarray, want: np.ndarray, max_ulp: int = 2) -> Dict:
    d = ulp_distance(got, want)
    g = bf16_value(got).astype(np.float64)
    w = bf16_value(want).astype(np.float64)
    stats = dict(max_ulp=int(d.max()) if d.size else 0,
                 n_diff=int((d > 0).sum()),
                 max_abs=float(np.abs(g - w).max()) if d.size else 0.0)
    assert stats["max_ulp"] <= max_ulp, (name, stats)
    return stats


# The oracle's results of the last keyed run_step (one entry: full-size
# results take up to a few GB).
_ORACLE_CACHE: Dict = {}


class LayerRun:
    """One linear layer prepared on both sides (weights quantized once)."""

    def __init__(self, x_bits, stream_id, w_bits, smooth, comp_a, comp_b, S, abits,
                 codes=CODES_INT):
        from w4a4_quantized_gemm_rudder_amd import rudder
        import torch
        self.r = rudder
        self.torch = torch
        self.x_bits, self.sid, self.w_bits = x_bits, stream_id, w_bits
        self.smooth, self.comp_a, self.comp_b = smooth, comp_a, comp_b
        self.S, self.abits, self.codes = S, abits, codes
        self.M, self.K = x_bits.shape
        self.N = w_bits.shape[1]
        # device copies
        self.X = to_dev_bf16(x_bits)
        self.sid_d = to_dev(stream_id.astype(np.uint8))
        self.W = to_dev_bf16(w_bits)
        self.s_d = to_dev(smooth.astype(np.float32))
        self.Wq, self.w_scale, self.inv_smooth = rudder.quantize_weights(self.W, self.s_d,
                                                                         codes)
        # oracle weights
        self.o_inv = oracle.inv_smooth(smooth)
        self.o_qw, self.o_ws = oracle.quantize_weights(w_bits, smooth)

    def check_weights(self) -> None:
        assert_bits_equal("inv_smooth", self.inv_smooth.cpu().numpy(), self.o_inv)
        assert_bits_equal("w_scale", self.w_scale.cpu().numpy(), self.o_ws)
        assert_bits_equal("Wq", self.Wq.cpu().numpy(), tile_for(self.codes, self.o_qw, 4))

    def run_step(self, delta: Optional[np.ndarray], comp_a: np.ndarray, comp_b: np.ndarray,
                 rows: Optional[np.ndarray] = None, check_codes: bool = True,
                 label: str = "", oracle_key=None) -> Dict:
        """delta None -> dynamic mode.  rows: sampled rows for acc/Y (None = all).
        oracle_key: the oracle's results for this (inputs, step, rows) are kept
        under this key and reused by the next call with the same key (the
        same layer in another code container: the oracle does not depend on
        the container)."""
        torch, r = self.torch, self.r
        S, abits, M, K, N, codes = self.S, self.abits, self.M, self.K, self.N, self.codes
        ca, cb = to_dev(comp_a.astype(np.float32)), to_dev(comp_b.astype(np.float32))
        scale_out = None
        if delta is None:
            scale_out = torch.full((S,), -1.0, dtype=torch.float32, device="cuda")
            Xq, rs = r.quant_act(self.X, self.sid_d, self.inv_smooth, None, S, abits, codes,
                                 act_scale_out=scale_out)
        else:
            Xq, rs = r.quant_act(self.X, self.sid_d, self.inv_smooth, to_dev(delta), S, abits,
                                 codes)
        # Y exactly as the timed path produces it (no accumulator output) ...
        Y = r.linear(Xq, rs, self.sid_d, self.Wq, self.w_scale, ca, cb, M, N, K, S, abits,
                     codes)
        # ... and once more with the raw accumulators.
        Y2, acc = r.linear(Xq, rs, self.sid_d, self.Wq, self.w_scale, ca, cb, M, N, K, S,
                           abits, codes, acc_out=True)
        torch.cuda.synchronize()

        # oracle
        cached = _ORACLE_CACHE.get("key") == oracle_key and oracle_key is not None
        if delta is None:
            o_delta = oracle.dynamic_scales(self.x_bits, self.sid, self.o_inv, S, abits)
            assert_bits_equal(f"{label} act_scale_out", scale_out.cpu().numpy(), o_delta)
        else:
            o_delta = delta
        if cached:
            qa, o_rs, o_acc, o_Y = _ORACLE_CACHE["val"]
        else:
            _ORACLE_CACHE.clear()
            qa, o_rs = oracle.quant_act(self.x_bits, self.sid, self.o_inv, o_delta, S, abits)
        assert_bits_equal(f"{label} row_scale", rs.cpu().numpy()[:M], o_rs)
        if check_codes:
            assert_bits_equal(f"{label} Xq", Xq.cpu().numpy(), tile_for(codes, qa, abits))
        full = rows is None
        if rows is None:
            rows = np.arange(M)
        if not cached:
            o_acc = oracle.int_gemm(qa if full else np.ascontiguousarray(qa[rows]), self.o_qw)
            o_Y = oracle.epilogue(o_acc, o_rs[rows], self.sid[rows], self.o_ws, comp_a, comp_b)
            if oracle_key is not None:
                _ORACLE_CACHE.update(key=oracle_key, val=(qa, o_rs, o_acc, o_Y))
        g_acc = acc.cpu().numpy() if full else acc.cpu().numpy()[rows]
        assert_bits_equal(f"{label} acc", g_acc, o_acc)
        yb = bf16_to_host_bits(Y) if full else bf16_to_host_bits(Y)[rows]
        yb2 = bf16_to_host_bits(Y2) if full else bf16_to_host_bits(Y2)[rows]
        assert_bits_equal(f"{label} Y(acc_out) vs Y", yb2, yb)
        stats = assert_y_close(f"{label} Y", yb, o_Y)
        stats["rows"] = int(len(rows))
        return stats


def sample_rows(stream_id: np.ndarray, n_random: int = 48, seed: int = 0) -> np.ndarray:
    """First/last rows, the first and last row of every stream block, the
    last 40 rows (ragged tail tile), plus random rows."""
    M = len(stream_id)
    rng = np.random.default_rng(seed)
    picks = set(range(min(8, M))) | set(range(max(0, M - 40), M))
    change = np.nonzero(np.diff(stream_id.astype(np.int16)))[0]
    for c in change:
        picks |= {int(c), int(c) + 1}
    picks |= set(rng.integers(0, M, n_random).tolist())
    return np.array(sorted(picks), dtype=np.int64)
