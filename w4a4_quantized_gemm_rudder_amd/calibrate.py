"""Offline calibration of the diagonal and of the layer-step table, with the
quantized layer run on the GPU through the C ABI for every candidate.

"SteerQuant: Steering Quantization Error with Action-Guided Scaling in
World-Action Models" (paperlayer.ai digest): §4.2 (one shared diagonal chosen
by a map-weighted reconstruction loss, one quantized weight matrix for all
streams and steps), §4.3 (per layer and step a shared clipping threshold and
bounded stream gains, kept in a layer-step lookup table), App. C (map scores
become positive weights: squared, offset by eta, tempered by rho < 1,
normalised), App. C.1 (a larger gain narrows the clipping range and the
rounding step; the activation-error target uses unquantized activations and
the fixed quantized weights).

The search, as implemented here:
  * weights w[t][s] = (score^2 + eta)^rho / mean;
  * stream error = mean over the stream's rows and all output channels of
    (Y - Yref)^2, Y the layer's bf16 output (compensation a = 1, b = 0),
    summed on the GPU in fp64 (rudder_stream_sq_error); loss = sum over
    (step, stream) with rows of w * error;
  * stage 1: s_j = max|X_j|^alpha / max|W_j|^(1-alpha) over an alpha grid,
    per-stream absmax step sizes, Yref = X @ W;
  * stage 2: per step, threshold c = rho_i * A (A the step's largest |x *
    inv_smooth|), gains g_j from a bounded grid, D = fl32(c / (g_j * Qa));
    each stream keeps its best gain per threshold and the threshold with the
    smallest weighted total wins; Yref = U @ Wdeq;
  * ties go to the first grid point.
Every quantize / GEMM / error step runs in librudder's kernels; torch only
provides buffers and the two reference products (X @ W, U @ Wdeq) in fp32,
which callers may replace with their own targets.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from . import rudder

DEFAULT_ALPHAS = tuple(round(0.1 * i, 1) for i in range(11))
DEFAULT_RHOS = (0.5, 0.6, 0.7, 0.8, 0.9, 1.0)
DEFAULT_GAINS = tuple(float(2.0 ** (e / 4.0)) for e in range(-4, 5))   # 0.5 .. 2, log grid


def map_weights(scores, eta: float = 1e-3, rho: float = 0.5) -> np.ndarray:
    w = (np.asarray(scores, np.float64) ** 2 + eta) ** rho
    return w / w.mean()


def _bf16_to_f32_host(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class CalibrationResult:
    alpha_index: int
    alpha: float
    smooth: np.ndarray                     # fp32 [K]
    stage1_loss: np.ndarray                # [len(alphas)]
    rho_index: List[int] = field(default_factory=list)        # per step
    gain_index: List[List[int]] = field(default_factory=list)  # per step, per stream
    threshold: List[float] = field(default_factory=list)
    delta: List[np.ndarray] = field(default_factory=list)      # fp32 [S] per step
    stage2_err: List[np.ndarray] = field(default_factory=list)  # [rho][gain][S] per step
    passes: int = 0


class _Layer:
    """Device buffers of one calibration problem (all steps)."""

    def __init__(self, Xs, sids, W, S, abits, codes):
        import torch
        self.torch = torch
        self.S, self.abits, self.codes = S, abits, codes
        self.K, self.N = W.shape
        self.W = torch.from_numpy(np.ascontiguousarray(W).view(np.int16)).cuda()
        self.Xs = [torch.from_numpy(np.ascontiguousarray(X).view(np.int16)).cuda() for X in Xs]
        self.sids = [torch.from_numpy(np.ascontiguousarray(sid, np.uint8)).cuda() for sid in sids]
        self.counts = [np.bincount(np.asarray(sid), minlength=S) for sid in sids]
        self.one = torch.ones((S, self.N), dtype=torch.float32, device="cuda")
        self.zero = torch.zeros((S, self.N), dtype=torch.float32, device="cuda")
        self.ws_err = torch.empty(rudder.stream_sq_error_workspace_bytes(), dtype=torch.uint8,
                                  device="cuda")
        self.ws_dyn = torch.empty(rudder.quant_act_workspace_bytes(S), dtype=torch.uint8,
                                  device="cuda")
        self.sse = torch.empty(S, dtype=torch.float64, device="cuda")

    def errors(self, t, Xq, rs, Wq, w_scale, yref) -> np.ndarray:
        """Mean squared error per stream of the quantized layer at step t."""
        torch = self.torch
        M = self.Xs[t].shape[0]
        Y = rudder.linear(Xq, rs, self.sids[t], Wq, w_scale, self.one, self.zero, M, self.N,
                          self.K, self.S, self.abits, self.codes)
        rudder.rudder_stream_sq_error(Y, yref, self.sids[t], M, self.N, self.S, self.ws_err,
                                      self.sse)
        sse = self.sse.cpu().numpy()
        c = self.counts[t]
        return np.where(c > 0, sse / np.maximum(c, 1) / self.N, 0.0)


def calibrate(Xs: Sequence[np.ndarray], sids: Sequence[np.ndarray], W: np.ndarray,
              weights: np.ndarray, S: int, abits: int, codes: int = rudder.CODES_INT,
              alphas: Sequence[float] = DEFAULT_ALPHAS, rhos: Sequence[float] = DEFAULT_RHOS,
              gains: Sequence[float] = DEFAULT_GAINS,
              stage1_targets: Optional[List[np.ndarray]] = None,
              stage2_targets: Optional[List[np.ndarray]] = None) -> CalibrationResult:
    """Calibrate one layer from per-step calibration batches.

    Xs[t]: bf16 bits [M_t, K]; sids[t]: uint8 [M_t]; W: bf16 bits [K, N];
    weights: [T][S] map weights (see map_weights).  Optional targets replace
    the fp32 reference products (fp32 [M_t, N] per step)."""
    L = _Layer(Xs, sids, W, S, abits, codes)
    torch = L.torch
    T = len(Xs)
    Qa = 127 if abits == 8 else 7
    Xf = [_bf16_to_f32_host(X) for X in Xs]
    ax = np.max([np.abs(x).max(axis=0) for x in Xf], axis=0).astype(np.float64)
    aw = np.abs(_bf16_to_f32_host(W)).max(axis=1).astype(np.float64)
    Wf = L.W.view(torch.bfloat16).float()
    if stage1_targets is None:
        y1 = [(X.view(torch.bfloat16).float() @ Wf).contiguous() for X in L.Xs]
    else:
        y1 = [torch.from_numpy(np.ascontiguousarray(y, np.float32)).cuda() for y in stage1_targets]
    passes = 0

    # ---- stage 1: the shared diagonal ------------------------------------
    def candidate(alpha):
        s = np.ones_like(ax)
        ok = (ax > 0) & (aw > 0)
        s[ok] = ax[ok] ** alpha / aw[ok] ** (1.0 - alpha)
        return s.astype(np.float32)

    losses = []
    for alpha in alphas:
        s_d = torch.from_numpy(candidate(alpha)).cuda()
        Wq, w_scale, inv = rudder.quantize_weights(L.W, s_d, codes)
        loss = 0.0
        for t in range(T):
            Xq, rs = rudder.quant_act(L.Xs[t], L.sids[t], inv, None, S, abits, codes,
                                      workspace=L.ws_dyn)
            err = L.errors(t, Xq, rs, Wq, w_scale, y1[t])
            loss += sum(weights[t][st] * err[st] for st in range(S) if L.counts[t][st] > 0)
            passes += 1
        losses.append(loss)
    a_best = int(np.argmin(losses))
    smooth = candidate(alphas[a_best])
    res = CalibrationResult(alpha_index=a_best, alpha=float(alphas[a_best]), smooth=smooth,
                            stage1_loss=np.array(losses))

    # ---- stage 2: thresholds and stream gains per step --------------------
    s_d = torch.from_numpy(smooth).cuda()
    Wq, w_scale, inv = rudder.quantize_weights(L.W, s_d, codes)
    Wdeq = torch.empty((L.K, L.N), dtype=torch.float32, device="cuda")
    rudder.rudder_dequant_weights(Wq, w_scale, L.K, L.N, codes, Wdeq)
    inv_h = inv.cpu().numpy()
    for t in range(T):
        U = (Xf[t] * inv_h[None, :]).astype(np.float32)
        A = float(np.abs(U).max())
        if stage2_targets is None:
            y2 = (torch.from_numpy(U).cuda() @ Wdeq).contiguous()
        else:
            y2 = torch.from_numpy(np.ascontiguousarray(stage2_targets[t], np.float32)).cuda()
        err = np.zeros((len(rhos), len(gains), S))
        for i, rho in enumerate(rhos):
            for j, g in enumerate(gains):
                d = torch.full((S,), float(np.float32(rho * A / (g * Qa))), dtype=torch.float32,
                               device="cuda")
                Xq, rs = rudder.quant_act(L.Xs[t], L.sids[t], inv, d, S, abits, codes)
                err[i, j] = L.errors(t, Xq, rs, Wq, w_scale, y2)
                passes += 1
        jbest = np.argmin(err, axis=1)
        tot = [sum(weights[t][st] * err[i, jbest[i, st], st] for st in range(S)
                   if L.counts[t][st] > 0) for i in range(len(rhos))]
        i_star = int(np.argmin(tot))
        gidx = [int(jbest[i_star, st]) for st in range(S)]
        res.rho_index.append(i_star)
        res.gain_index.append(gidx)
        res.threshold.append(rhos[i_star] * A)
        res.delta.append(np.array([np.float32(rhos[i_star] * A / (gains[gi] * Qa))
                                   for gi in gidx], np.float32))
        res.stage2_err.append(err)
    res.passes = passes
    return res
