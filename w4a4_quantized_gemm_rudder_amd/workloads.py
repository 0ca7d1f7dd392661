"""Seeded synthetic inputs for the stream-aware W4A8/W4A4 linear.

This module only *draws inputs*.  It holds none of the method's arithmetic
(no quantizer, no packing, no integer GEMM, no epilogue), so that both the
CPU oracle and the HIP path can be fed from it without sharing code.

Workloads are DiT-shaped token sets with three semantic streams
(0 = video, 1 = proprio, 2 = action), following the stream split of
world-action models in SteerQuant ("SteerQuant: Steering Quantization Error
with Action-Guided Scaling in World-Action Models", abstract and §1).

Drawing recipe (every draw is fp64, rounded to fp32 and then to bf16, or cast
to fp32 for scales; large tensors are drawn in blocks of 512 rows, each block
from its own generator, so that blocks can be drawn in parallel threads):
  * X rows ~ N(0, 1); a fixed number of outlier channels (chosen without
    replacement) are multiplied by a constant factor.
  * The MLP down-projection input is bf16(GELU_erf(Z)), Z ~ Student-t(nu=4).
  * W ~ N(0, sigma), stored [K in, N out].
  * Smoothing s_j = sqrt(max_m |X_mj| / max_n |W_jn|) (the SmoothQuant
    alpha = 0.5 rule, which SteerQuant §2 names as prior art; the calibrated
    diagonal of SteerQuant §4.2 needs a trained model).  A zero max gives 1.
  * Per-(step, stream) activation step sizes Delta = c / (gamma * Qa) with
    c = rho * max|X diag(s)^-1|, rho ~ U(0.7, 1.0) per step and bounded
    stream gains gamma log-uniform in [0.5, 2] (SteerQuant §4.3 and App. C.1:
    a shared per-(layer, step) clipping threshold, bounded stream gains, a
    larger gain narrowing the stream's range and rounding step).
  * Output compensation a ~ U(0.9, 1.1), b ~ N(0, 0.01) per (stream, output
    channel), either one set per layer or one per (step, stream).

bf16 tensors are returned as numpy uint16 bit patterns; the fp64 -> bf16
rounding is torch's own conversion (input synthesis only).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Callable, Dict, List, Optional, Tuple

import numpy as np

VIDEO, PROPRIO, ACTION = 0, 1, 2
STREAM_NAMES = ("video", "proprio", "action")

# Tensor tags used to derive independent RNG streams.
_TAGS = {
    "x": 1, "x2": 2, "w": 3, "rho": 4, "gamma": 5, "a": 6, "b": 7,
    "outlier_idx": 8, "z": 9, "calib": 10,
}


def rng_for(seed: int, workload_idx: int, tag: str, *extra: int) -> np.random.Generator:
    """PCG64 seeded from (seed, workload index, tensor tag, extra ints)."""
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, workload_idx, _TAGS[tag], *extra])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round an fp64/fp32 array to bf16 and return its uint16 bit pattern."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (used only to draw scales)."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    K: int
    N: int
    abits: int          # 8 -> W4A8, 4 -> W4A4
    x_kind: str         # which input tensor feeds it ("x", "x2", or "x_<name>")
    w_sigma: float


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    stream_rows: Tuple[Tuple[int, int], ...]   # (stream id, row count) blocks, in order
    layers: Tuple[Layer, ...]
    n_steps: int
    dynamic: bool                  # per-stream absmax scales (no LUT)
    per_step_comp: bool            # compensation per (step, stream) instead of per layer
    x_outliers: Tuple[int, float]  # (channel count, factor) for N(0,1) inputs
    description: str

    @property
    def M(self) -> int:
        return sum(r for _, r in self.stream_rows)

    @property
    def S(self) -> int:
        return 3

    def stream_ids(self) -> np.ndarray:
        return np.concatenate(
            [np.full(r, s, dtype=np.uint8) for s, r in self.stream_rows])

    def ops_per_step(self) -> int:
        return sum(2 * self.M * l.N * l.K for l in self.layers)


_ROLLOUT_2048 = ((VIDEO, 4096), (PROPRIO, 32), (ACTION, 64))

WORKLOADS: Dict[str, Workload] = {}


def _add(w: Workload) -> None:
    WORKLOADS[w.name] = w


_add(Workload(
    name="linear_m96_k256_n256_w4a8", index=0,
    stream_rows=((VIDEO, 64), (PROPRIO, 16), (ACTION, 16)),
    layers=(Layer("linear", 256, 256, 8, "x", 0.02),),
    n_steps=1, dynamic=True, per_step_comp=False, x_outliers=(4, 20.0),
    description="single 256->256 linear, 96 tokens (64 video, 16 proprio, 16 action), "
                "W4A8, per-stream absmax activation scales"))

_add(Workload(
    name="attn_proj_h2048_m4192_w4a8", index=1,
    stream_rows=_ROLLOUT_2048,
    layers=(Layer("qkv", 2048, 6144, 8, "x", 0.02),
            Layer("o", 2048, 2048, 8, "x", 0.02)),
    n_steps=10, dynamic=False, per_step_comp=False, x_outliers=(20, 30.0),
    description="attention QKV 2048->6144 and O 2048->2048 at W4A8, 4192 tokens "
                "(4096 video, 32 proprio, 64 action), 10 step-indexed scale sets"))

_add(Workload(
    name="mlp_h2048_m4192_w4a4", index=2,
    stream_rows=_ROLLOUT_2048,
    layers=(Layer("up", 2048, 8192, 4, "x", 0.02),
            Layer("down", 8192, 2048, 4, "x2", 0.02)),
    n_steps=10, dynamic=False, per_step_comp=False, x_outliers=(20, 30.0),
    description="MLP up 2048->8192 and down 8192->2048 at W4A4, 4192 tokens, "
                "down input GELU of Student-t(4), 10 step-indexed scale sets"))

_add(Workload(
    name="dit_block_h2048_m8384_16step", index=3,
    stream_rows=_ROLLOUT_2048 + _ROLLOUT_2048,
    layers=(Layer("qkv", 2048, 6144, 8, "x_qkv", 0.02),
            Layer("o", 2048, 2048, 8, "x_o", 0.02),
            Layer("up", 2048, 8192, 4, "x_up", 0.02),
            Layer("down", 8192, 2048, 4, "x2", 0.02)),
    n_steps=16, dynamic=False, per_step_comp=True, x_outliers=(20, 30.0),
    description="DiT block linear set (QKV, O at W4A8; MLP 2048->8192->2048 at W4A4), "
                "2 rollouts x 4192 tokens = 8384 rows, 16-step denoise loop, "
                "per-(step, stream) scales and compensation"))

_add(Workload(
    name="backbone_h4096_m16576_w4a4", index=4,
    stream_rows=((VIDEO, 16384), (PROPRIO, 64), (ACTION, 128)),
    layers=(Layer("qkv", 4096, 12288, 4, "x", 0.015),
            Layer("o", 4096, 4096, 4, "x", 0.015),
            Layer("up", 4096, 16384, 4, "x", 0.015),
            Layer("down", 16384, 4096, 4, "x2", 0.015)),
    n_steps=20, dynamic=False, per_step_comp=False, x_outliers=(20, 50.0),
    description="hidden-4096 backbone linears (QKV, O, MLP 4096->16384->4096), all W4A4, "
                "16576 tokens (16384 video, 64 proprio, 128 action), 20 scale sets"))

WORKLOAD_ORDER: List[str] = [w.name for w in sorted(WORKLOADS.values(), key=lambda w: w.index)]


# --------------------------------------------------------------------------
# Draws
# --------------------------------------------------------------------------

# Row-block drawing: each block of _BLOCK_ROWS rows has its own generator
# (the block index is the last seed word), so blocks are drawn in parallel
# threads and the result does not depend on the thread count.
_BLOCK_ROWS = 512


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw_blocked(M: int, K: int, fill) -> np.ndarray:
    """bf16 bits [M, K]; fill(block, rows) returns the fp64 values of row block
    `block` ([rows, K])."""
    out = np.empty((M, K), np.uint16)
    nblk = (M + _BLOCK_ROWS - 1) // _BLOCK_ROWS

    def work(b: int) -> None:
        r0 = b * _BLOCK_ROWS
        r1 = min(M, r0 + _BLOCK_ROWS)
        out[r0:r1] = to_bf16_bits(fill(b, r1 - r0))

    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(nblk)))
    return out


def draw_x_normal(M: int, K: int, n_outliers: int, factor: float,
                  rng_x: Callable[[int], np.random.Generator],
                  rng_idx: np.random.Generator) -> np.ndarray:
    """bf16 bits [M, K]: N(0,1) with n_outliers channels multiplied by factor.
    rng_x(block) gives the generator of a row block."""
    idx = rng_idx.choice(K, size=n_outliers, replace=False) if n_outliers else None

    def fill(b, rows):
        x = rng_x(b).standard_normal((rows, K))
        if idx is not None:
            x[:, idx] *= factor
        return x

    return _draw_blocked(M, K, fill)


def draw_x_gelu_t4(M: int, K: int, rng: Callable[[int], np.random.Generator]) -> np.ndarray:
    """bf16 bits [M, K] of GELU_erf(Z), Z ~ Student-t(4), evaluated in fp64.
    rng(block) gives the generator of a row block."""
    from scipy.special import erf

    def fill(b, rows):
        z = rng(b).standard_t(4.0, size=(rows, K))
        return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))

    return _draw_blocked(M, K, fill)


def draw_w(K: int, N: int, sigma: float, rng: Callable[[int], np.random.Generator]) -> np.ndarray:
    """bf16 bits [K, N] ~ N(0, sigma); rng(block) gives the generator of a
    block of input-channel rows."""
    return _draw_blocked(K, N, lambda b, rows: rng(b).standard_normal((rows, N)) * sigma)


def _abs_max_bits(bits: np.ndarray, axis: int) -> np.ndarray:
    """max |value| along an axis of finite bf16 bit patterns, as fp64.  The
    magnitude bits of finite bf16 values order the same way as the values'
    magnitudes, so the maximum is taken on the patterns (blocks in threads)."""
    if axis == 0:
        nblk = (bits.shape[0] + _BLOCK_ROWS - 1) // _BLOCK_ROWS

        def part(b):
            blk = bits[b * _BLOCK_ROWS:(b + 1) * _BLOCK_ROWS]
            return (blk & 0x7FFF).max(axis=0)

        with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
            m = np.max(np.stack(list(ex.map(part, range(nblk)))), axis=0)
    else:
        m = (bits & 0x7FFF).max(axis=1)
    return bf16_bits_to_f64(m.astype(np.uint16))


def smoothing_scale(x_bits: np.ndarray, w_bits: np.ndarray,
                    x_colmax: Optional[np.ndarray] = None) -> np.ndarray:
    """fp32 [K]: s_j = sqrt(max_m|X_mj| / max_n|W_jn|) in fp64 (1 where a max is 0)."""
    xm = _abs_max_bits(x_bits, 0) if x_colmax is None else x_colmax
    wm = _abs_max_bits(w_bits, 1)
    s = np.ones_like(xm)
    ok = (xm > 0) & (wm > 0)
    s[ok] = np.sqrt(xm[ok] / wm[ok])
    return s.astype(np.float32)


def draw_act_scales(x_bits: np.ndarray, s: np.ndarray, n_steps: int, S: int, qa: int,
                    rng_rho: np.random.Generator, rng_gamma: np.random.Generator,
                    x_colmax: Optional[np.ndarray] = None) -> np.ndarray:
    """fp32 [n_steps, S] step sizes Delta = c_t / (gamma_{s,t} * Qa), with
    c_t = rho_t * max_{m,j} |X_mj| / s_j.  Dividing by s_j > 0 is monotonic,
    so the maximum over m is taken first (the same fp64 value)."""
    xm = _abs_max_bits(x_bits, 0) if x_colmax is None else x_colmax
    c0 = float((xm / s.astype(np.float64)).max())
    rho = rng_rho.uniform(0.7, 1.0, size=n_steps)
    gamma = np.exp(rng_gamma.uniform(np.log(0.5), np.log(2.0), size=(n_steps, S)))
    delta = (rho[:, None] * c0) / (gamma * qa)
    return delta.astype(np.float32)


def draw_compensation(shape: Tuple[int, ...], rng_a: np.random.Generator,
                      rng_b: np.random.Generator) -> Tuple[np.ndarray, np.ndarray]:
    a = rng_a.uniform(0.9, 1.1, size=shape).astype(np.float32)
    b = (rng_b.standard_normal(size=shape) * 0.01).astype(np.float32)
    return a, b


@dataclasses.dataclass
class LayerInputs:
    layer: Layer
    x: np.ndarray            # bf16 bits [M, K]
    w: np.ndarray            # bf16 bits [K, N]
    smooth: np.ndarray       # fp32 [K]
    act_scale: Optional[np.ndarray]   # fp32 [T, S] (None in dynamic mode)
    comp_a: np.ndarray       # fp32 [S, N] or [T, S, N]
    comp_b: np.ndarray

    def step_comp(self, t: int) -> Tuple[np.ndarray, np.ndarray]:
        if self.comp_a.ndim == 3:
            return self.comp_a[t], self.comp_b[t]
        return self.comp_a, self.comp_b


@dataclasses.dataclass
class WorkloadInputs:
    workload: Workload
    stream_id: np.ndarray    # uint8 [M]
    layers: List[LayerInputs]


def make_inputs(name: str, seed: int = 0, rows: Optional[int] = None,
                layers: Optional[List[str]] = None) -> WorkloadInputs:
    """Draw every input of a workload.

    rows: optional cap on M (keeps the stream layout's order, truncating the
    video block first) for quick CPU runs; None means the full size.
    layers: optional subset of layer names.
    """
    wl = WORKLOADS[name]
    sid = wl.stream_ids()
    if rows is not None and rows < wl.M:
        # Keep every proprio/action row that fits, drop video rows first.
        small = np.nonzero(sid != VIDEO)[0]
        keep_small = small[: rows]
        n_video = rows - len(keep_small)
        video = np.nonzero(sid == VIDEO)[0][: n_video]
        keep = np.sort(np.concatenate([video, keep_small]))
        sid = sid[keep]
    M = len(sid)
    wi = wl.index
    tensors: Dict[str, np.ndarray] = {}

    colmax: Dict[str, np.ndarray] = {}

    def x_tensor(kind: str, K: int) -> np.ndarray:
        if kind in tensors:
            return tensors[kind]
        if kind == "x2":
            t = draw_x_gelu_t4(M, K, lambda b: rng_for(seed, wi, "z", K, b))
        else:
            sub = 0 if kind == "x" else sum(map(ord, kind))
            t = draw_x_normal(M, K, wl.x_outliers[0], wl.x_outliers[1],
                              lambda b: rng_for(seed, wi, "x", sub, K, b),
                              rng_for(seed, wi, "outlier_idx", sub, K))
        tensors[kind] = t
        colmax[kind] = _abs_max_bits(t, 0)
        return t

    out = []
    for li, layer in enumerate(wl.layers):
        if layers is not None and layer.name not in layers:
            continue
        x = x_tensor(layer.x_kind, layer.K)
        w = draw_w(layer.K, layer.N, layer.w_sigma, lambda b: rng_for(seed, wi, "w", li, b))
        s = smoothing_scale(x, w, colmax[layer.x_kind])
        qa = 127 if layer.abits == 8 else 7
        if wl.dynamic:
            delta = None
        else:
            delta = draw_act_scales(x, s, wl.n_steps, wl.S, qa,
                                    rng_for(seed, wi, "rho", li), rng_for(seed, wi, "gamma", li),
                                    colmax[layer.x_kind])
        shape = (wl.n_steps, wl.S, layer.N) if wl.per_step_comp else (wl.S, layer.N)
        a, b = draw_compensation(shape, rng_for(seed, wi, "a", li), rng_for(seed, wi, "b", li))
        out.append(LayerInputs(layer, x, w, s, delta, a, b))
    return WorkloadInputs(wl, sid, out)


# --------------------------------------------------------------------------
# Calibration batches (offline search of the diagonal and the layer-step
# table).  The action-impact map needs a trained model, so the map scores are
# a fixed synthetic schedule with the qualitative shape the pages report
# (proprioception leads at early steps, action at later ones [SteerQuant
# §B.3]); the streams' activation statistics drift with the step.
# --------------------------------------------------------------------------

CALIB_SCORES = np.array([
    # video, proprio, action
    [0.30, 1.00, 0.55],
    [0.35, 0.80, 0.75],
    [0.40, 0.55, 0.95],
    [0.40, 0.35, 1.00],
])


@dataclasses.dataclass
class CalibrationInputs:
    xs: List[np.ndarray]          # per step: bf16 bits [rows, K]
    sids: List[np.ndarray]        # per step: uint8 [rows]
    w: np.ndarray                 # bf16 bits [K, N]
    scores: np.ndarray            # [steps, 3]


def make_calibration(K: int, N: int, seed: int = 0, steps: int = 4,
                     rows: Tuple[int, int, int] = (192, 16, 48),
                     n_outliers: int = 0, outlier_factor: float = 20.0) -> CalibrationInputs:
    """Per-step calibration batches of one layer: `rows` rows per stream
    (video, proprio, action) at every step, video ~ N(0,1) with optional
    outlier channels, proprio ~ N(0, (1.3 - 0.2 t)^2), action ~
    N(0, (1.5 + 0.25 t)^2); W ~ N(0, 0.02)."""
    rng_idx = rng_for(seed, 100, "outlier_idx", K)
    out_idx = rng_idx.choice(K, size=n_outliers, replace=False) if n_outliers else None
    xs, sids = [], []
    for t in range(steps):
        rng = rng_for(seed, 100, "calib", K, N, t)
        parts, tags = [], []
        for st, (n, sig) in enumerate(zip(rows, (1.0, 1.3 - 0.2 * t, 1.5 + 0.25 * t))):
            x = rng.standard_normal((n, K)) * sig
            if out_idx is not None and st == 0:
                x[:, out_idx] *= outlier_factor
            parts.append(x)
            tags.append(np.full(n, st, np.uint8))
        xs.append(to_bf16_bits(np.concatenate(parts)))
        sids.append(np.concatenate(tags))
    w = draw_w(K, N, 0.02, lambda b: rng_for(seed, 100, "w", K, N, b))
    return CalibrationInputs(xs=xs, sids=sids, w=w, scores=CALIB_SCORES[:steps].copy())
