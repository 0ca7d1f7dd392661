"""CPU reference of the offline calibration (test infrastructure only).

"SteerQuant: Steering Quantization Error with Action-Guided Scaling in
World-Action Models" (paperlayer.ai digest):
  §4.2  one shared positive diagonal rescales the weights and inversely the
        activations; it is chosen by a map-weighted reconstruction loss and
        leaves one quantized weight matrix for all streams and steps;
  §4.3  per layer and step, a shared clipping threshold and bounded stream
        gains, stored in a layer-step lookup table;
  App. C  map scores become positive weights: squared, offset by eta > 0,
        tempered by an exponent rho < 1, normalised;
  App. C.1  a larger gain narrows its stream's clipping range and rounding
        step; the activation-error target uses unquantized activations and
        the fixed quantized weights.

Readings (the pages give no formulas; each is restated in the design notes):
  * weights  w[t][s] = (score^2 + eta)^rho, divided by their mean;
  * error of stream s at step t: mean over its rows and all output channels
    of (Y - Yref)^2, Y the layer's bf16 output with compensation a = 1, b = 0;
    loss = sum over (t, s) with rows of w[t][s] * error;
  * diagonal (stage 1): s_j = max|X_j|^alpha / max|W_j|^(1-alpha) over an
    alpha grid (fp64, rounded to fp32; 1 where a maximum is 0), activations
    at per-stream absmax step sizes, Yref = X @ W (full precision);
  * table (stage 2): at step t, threshold c = rho_i * A_t with A_t the
    largest |x * inv_smooth| of the step, gain g_j from a bounded grid, step
    size D = fl32(c / (g_j * Qa)).  Streams' rows are independent, so each
    stream takes its best gain for each threshold, and the threshold with
    the smallest weighted total wins.  Yref = U @ Wdeq, U = fl32(x *
    inv_smooth), Wdeq = fl32(code * w_scale);
  * ties go to the first grid point.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from . import oracle as O

__all__ = ["map_weights", "smoothing_candidate", "stream_errors", "calibrate_smoothing",
           "calibrate_table"]


def map_weights(scores: np.ndarray, eta: float = 1e-3, rho: float = 0.5) -> np.ndarray:
    """Positive calibration weights from map scores (App. C)."""
    w = (np.asarray(scores, np.float64) ** 2 + eta) ** rho
    return w / w.mean()


def smoothing_candidate(ax: np.ndarray, aw: np.ndarray, alpha: float) -> np.ndarray:
    """s_j = ax_j^alpha / aw_j^(1-alpha) in fp64, rounded to fp32 (§4.2)."""
    ax = np.asarray(ax, np.float64)
    aw = np.asarray(aw, np.float64)
    s = np.ones_like(ax)
    ok = (ax > 0) & (aw > 0)
    s[ok] = ax[ok] ** alpha / aw[ok] ** (1.0 - alpha)
    return s.astype(np.float32)


def stream_errors(Ybits: np.ndarray, Yref: np.ndarray, sid: np.ndarray, S: int) -> np.ndarray:
    """Sum of squared errors per stream (fp64)."""
    d = O.bf16_to_f32(Ybits).astype(np.float64) - np.asarray(Yref, np.float64)
    rowsum = (d * d).sum(axis=1)
    return np.array([rowsum[sid == s].sum() for s in range(S)], np.float64)


def _weighted(sse: np.ndarray, counts: np.ndarray, N: int, w: np.ndarray) -> float:
    tot = 0.0
    for s in range(len(sse)):
        if counts[s] > 0:
            tot += w[s] * sse[s] / (counts[s] * N)
    return tot


def calibrate_smoothing(Xs: Sequence[np.ndarray], sids: Sequence[np.ndarray], W: np.ndarray,
                        weights: np.ndarray, S: int, abits: int, alphas: Sequence[float],
                        yrefs: Optional[List[np.ndarray]] = None):
    """Stage 1.  Returns (best index, losses [len(alphas)], s of the best)."""
    Xf = [O.bf16_to_f32(X) for X in Xs]
    ax = np.max([np.abs(x).max(axis=0) for x in Xf], axis=0)
    aw = np.abs(O.bf16_to_f32(W)).max(axis=1)
    Wf = O.bf16_to_f32(W).astype(np.float64)
    if yrefs is None:
        yrefs = [x.astype(np.float64) @ Wf for x in Xf]
    N = W.shape[1]
    one = np.ones((S, N), np.float32)
    zero = np.zeros((S, N), np.float32)
    losses = []
    for alpha in alphas:
        s = smoothing_candidate(ax, aw, alpha)
        inv = O.inv_smooth(s)
        qw, ws = O.quantize_weights(W, s)
        loss = 0.0
        for t, (X, sid) in enumerate(zip(Xs, sids)):
            d = O.dynamic_scales(X, sid, inv, S, abits)
            _, _, _, Y = O.linear(X, sid, qw, ws, inv, d, one, zero, S, abits)
            sse = stream_errors(Y, yrefs[t], sid, S)
            loss += _weighted(sse, np.bincount(sid, minlength=S), N, weights[t])
        losses.append(loss)
    best = int(np.argmin(losses))
    return best, np.array(losses), smoothing_candidate(ax, aw, alphas[best])


def calibrate_table(Xs: Sequence[np.ndarray], sids: Sequence[np.ndarray], W: np.ndarray,
                    s: np.ndarray, weights: np.ndarray, S: int, abits: int,
                    rhos: Sequence[float], gains: Sequence[float],
                    yrefs: Optional[List[np.ndarray]] = None):
    """Stage 2.  Returns dict with, per step: best threshold index, gain index
    per stream, threshold c, step sizes D[S] (fp32), and the error table
    err[t][i][j][s] (mean squared error per stream)."""
    Qa = 127 if abits == 8 else 7
    inv = O.inv_smooth(s)
    qw, ws = O.quantize_weights(W, s)
    Wdeq = (qw.T.astype(np.float32) * ws[None, :]).astype(np.float32)      # [K][N], fp32 products
    N = W.shape[1]
    one = np.ones((S, N), np.float32)
    zero = np.zeros((S, N), np.float32)
    out = {"rho_index": [], "gain_index": [], "threshold": [], "delta": [], "err": []}
    for t, (X, sid) in enumerate(zip(Xs, sids)):
        U = (O.bf16_to_f32(X) * inv[None, :]).astype(np.float32)
        A = float(np.abs(U).max())
        yref = yrefs[t] if yrefs is not None else U.astype(np.float64) @ Wdeq.astype(np.float64)
        counts = np.bincount(sid, minlength=S)
        err = np.zeros((len(rhos), len(gains), S))
        for i, rho in enumerate(rhos):
            for j, g in enumerate(gains):
                d = np.full(S, np.float32(rho * A / (g * Qa)), np.float32)
                _, _, _, Y = O.linear(X, sid, qw, ws, inv, d, one, zero, S, abits)
                sse = stream_errors(Y, yref, sid, S)
                err[i, j] = np.where(counts > 0, sse / np.maximum(counts, 1) / N, 0.0)
        # each stream's best gain per threshold, then the best threshold
        jbest = np.argmin(err, axis=1)                                     # [rho][S]
        tot = [sum(weights[t][st] * err[i, jbest[i, st], st] for st in range(S) if counts[st] > 0)
               for i in range(len(rhos))]
        i_star = int(np.argmin(tot))
        gidx = [int(jbest[i_star, st]) for st in range(S)]
        c = rhos[i_star] * A
        out["rho_index"].append(i_star)
        out["gain_index"].append(gidx)
        out["threshold"].append(c)
        out["delta"].append(np.array([np.float32(rhos[i_star] * A / (gains[gi] * Qa))
                                      for gi in gidx], np.float32))
        out["err"].append(err)
    return out
