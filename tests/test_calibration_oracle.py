"""Pins of the oracle's offline calibration (SteerQuant §4.2, §4.3, App. C):
constructed inputs whose optimum is known without running the search."""
import numpy as np
import pytest

import oracle
from oracle import calibration as CAL

ALPHAS = [round(0.1 * i, 1) for i in range(11)]
RHOS = [0.5, 0.6, 0.7, 0.8, 0.9, 1.0]
GAINS = [float(2.0 ** (e / 4.0)) for e in range(-4, 5)]


def _bits(x):
    return oracle.f32_to_bf16(np.asarray(x, np.float32))


def test_map_weights_definition():
    sc = np.array([[0.0, 0.5, 1.0], [2.0, 0.1, 0.0]])
    w = CAL.map_weights(sc, eta=1e-3, rho=0.5)
    assert np.all(w > 0)                                   # eta keeps zero scores positive
    assert abs(w.mean() - 1.0) < 1e-12                     # normalised
    flat, ws = sc.ravel(), w.ravel()
    order = np.argsort(flat)
    assert np.all(np.diff(ws[order]) >= 0)                 # monotone in the score
    # rho < 1 tempers: the weight ratio is smaller than the squared-score ratio
    assert ws[flat.argmax()] / ws[list(flat).index(0.5)] < (2.0 / 0.5) ** 2


def lossless_at_half(seed=0, M_per=32, K=64, N=64):
    """X = qa * D * s*, W = qw * c / s* with per-column code maxima m_j shared by
    X and W, D = c, s* powers of two: alpha = 0.5 recovers s* (and the codes)
    exactly; any other alpha gives a non-uniform diagonal."""
    rng = np.random.default_rng(seed)
    S, Qa = 2, 7
    m = rng.choice([1, 2, 3, 4, 6, 7], size=K)
    m[0] = 7
    s_star = 2.0 ** rng.integers(-2, 3, size=K)
    D = c = 2.0 ** -3
    M = S * M_per
    qa = np.stack([rng.integers(-m[j], m[j] + 1, size=M) for j in range(K)], axis=1)
    qa[1, :] = m                                          # every column reaches m_j
    for st in range(S):
        qa[st * M_per, 0] = 7                             # every stream reaches Qa
    qw = np.stack([rng.integers(-m[j], m[j] + 1, size=N) for j in range(K)], axis=0)
    qw[:, 1] = m                                          # every row reaches m_j
    qw[0, :] = 7                                          # every output column reaches 7
    X = _bits(qa * D * s_star[None, :])
    W = _bits(qw * c / s_star[:, None])
    sid = np.repeat(np.arange(S), M_per).astype(np.uint8)
    return X, sid, W, S, s_star


def test_stage1_picks_the_lossless_alpha():
    X, sid, W, S, s_star = lossless_at_half()
    w = CAL.map_weights(np.ones((1, S)))
    best, losses, s = CAL.calibrate_smoothing([X], [sid], W, w, S, 4, ALPHAS)
    assert ALPHAS[best] == 0.5, losses
    assert np.array_equal(s, s_star.astype(np.float32))
    others = np.delete(losses, best)
    assert losses[best] < 0.05 * others.min(), losses      # only bf16 output rounding remains


def lossless_table(seed=1, K=64, N=96):
    """s = 1 and three streams of exact multiples of power-of-two steps: stream
    0 of D_0 = A / Qa reaching Qa (so A = Qa * D_0), stream 1 of D_0 / 2 with
    odd codes up to Qa, stream 2 of 2 D_0 with odd codes up to Qa / 2."""
    rng = np.random.default_rng(seed)
    Qa = 7
    A = 2.0 ** 1 * Qa                                     # D_0 = 2
    D = [A / Qa, A / (2 * Qa), 2 * A / Qa]
    rows = 24
    parts = []
    c0 = rng.integers(-Qa, Qa + 1, size=(rows, K))
    c0[0, 0] = Qa
    parts.append(c0 * D[0])
    c1 = 2 * rng.integers(-3, 4, size=(rows, K)) + 1      # odd, |c| <= 7
    parts.append(c1 * D[1])
    c2 = 2 * rng.integers(-2, 2, size=(rows, K)) + 1      # odd, |c| <= 3 (Qa / 2)
    parts.append(c2 * D[2])
    X = _bits(np.concatenate(parts))
    sid = np.repeat(np.arange(3), rows).astype(np.uint8)
    W = _bits(rng.standard_normal((K, N)) * 0.05)
    return X, sid, W


def test_stage2_picks_an_exact_table_and_the_first_tie():
    """Every stream has an exact step size on the grid.  Thresholds 0.5 A and
    A are twins here (rho = 0.5 with every gain halved gives the same steps),
    so the first one is chosen: rho = 0.5, gains (0.5, 1, 0.5), steps (2, 1, 2)
    -- stream 2's 2 D_0 values are exact at D_0 too, the finer of its exact
    steps reached first on the gain grid."""
    X, sid, W = lossless_table()
    K = W.shape[0]
    s = np.ones(K, np.float32)
    w = CAL.map_weights(np.ones((1, 3)))
    out = CAL.calibrate_table([X], [sid], W, s, w, 3, 4, RHOS, GAINS)
    i, g = out["rho_index"][0], out["gain_index"][0]
    assert RHOS[i] == 0.5
    assert [GAINS[j] for j in g] == [0.5, 1.0, 0.5]
    assert np.array_equal(out["delta"][0], np.array([2.0, 1.0, 2.0], np.float32))
    err = out["err"][0]
    # the twin cells at rho = 1 (gains doubled) have the identical error
    for st, j in enumerate(g):
        assert err[RHOS.index(1.0), GAINS.index(2 * GAINS[j]), st] == err[i, j, st]
    # and each chosen cell is its stream's minimum over the whole grid
    for st, j in enumerate(g):
        assert err[i, j, st] == err[:, :, st].min()
    # stream 1 (odd multiples of D_0 / 2) is lossy one gain step coarser
    assert err[i, GAINS.index(0.5), 1] > 100 * err[i, g[1], 1]


def test_stage2_threshold_scales_with_the_input():
    """Scaling the activations by a power of two scales A, the thresholds and
    step sizes by it and leaves every index unchanged."""
    X, sid, W = lossless_table(seed=2)
    K = W.shape[0]
    s = np.ones(K, np.float32)
    w = CAL.map_weights(np.array([[0.3, 1.0, 0.6]]))
    a = CAL.calibrate_table([X], [sid], W, s, w, 3, 4, RHOS, GAINS)
    X4 = _bits(oracle.bf16_to_f32(X) * 4.0)
    b = CAL.calibrate_table([X4], [sid], W, s, w, 3, 4, RHOS, GAINS)
    assert a["rho_index"] == b["rho_index"] and a["gain_index"] == b["gain_index"]
    assert np.array_equal(b["delta"][0], a["delta"][0] * 4)
