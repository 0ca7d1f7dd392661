"""GPU parity of the calibration support calls and of the GPU-in-the-loop
calibration search against the oracle's (SteerQuant §4.2, §4.3, App. C)."""
import time

import numpy as np
import pytest

import oracle
from oracle import calibration as CAL
from gpu_harness import CODES_E2M3, CODES_INT, assert_bits_equal, log, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from w4a4_quantized_gemm_rudder_amd import rudder
    rudder.load_library()
    yield


@pytest.mark.parametrize("K,N,codes", [(128, 96, CODES_INT), (256, 64, CODES_E2M3),
                                       (2048, 512, CODES_INT)])
def test_dequant_weights_matches_oracle(K, N, codes):
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    log(f"case dequant K={K} N={N} codes={codes}")
    rng = np.random.default_rng(K + N)
    W = oracle.f32_to_bf16((rng.standard_normal((K, N)) * 0.03).astype(np.float32))
    s = rng.uniform(0.5, 2.0, K).astype(np.float32)
    Wq, ws, _ = rudder.quantize_weights(to_dev_bf16(W), to_dev(s), codes)
    out = torch.empty((K, N), dtype=torch.float32, device="cuda")
    rudder.rudder_dequant_weights(Wq, ws, K, N, codes, out)
    torch.cuda.synchronize()
    qw, wsc = oracle.quantize_weights(W, s)
    want = (qw.T.astype(np.float32) * wsc[None, :]).astype(np.float32)
    assert_bits_equal("Wdeq", out.cpu().numpy(), want)


@pytest.mark.parametrize("M,N,S", [(1, 32, 1), (300, 96, 3), (4100, 256, 8), (0, 64, 2)])
def test_stream_sq_error_matches_numpy(M, N, S):
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    log(f"case stream sq error M={M} N={N} S={S}")
    rng = np.random.default_rng(M + N + S)
    Y = oracle.f32_to_bf16(rng.standard_normal((max(M, 1), N)).astype(np.float32))[:M]
    Yref = rng.standard_normal((M, N)).astype(np.float32)
    sid = rng.integers(0, S, M).astype(np.uint8)
    ws = torch.empty(rudder.stream_sq_error_workspace_bytes(), dtype=torch.uint8, device="cuda")
    sse = torch.full((S,), -1.0, dtype=torch.float64, device="cuda")
    Yd = to_dev_bf16(Y) if M else torch.zeros(1, dtype=torch.bfloat16, device="cuda")
    Rd = to_dev(Yref) if M else torch.zeros(1, dtype=torch.float32, device="cuda")
    Sd = to_dev(sid) if M else torch.zeros(1, dtype=torch.uint8, device="cuda")
    rudder.rudder_stream_sq_error(Yd, Rd, Sd, M, N, S, ws, sse)
    torch.cuda.synchronize()
    want = CAL.stream_errors(Y, Yref, sid, S) if M else np.zeros(S)
    np.testing.assert_allclose(sse.cpu().numpy(), want, rtol=1e-12, atol=0)


def _oracle_targets(ci, S):
    """Full-precision targets of both stages (fp64 products, rounded to fp32)."""
    y1 = [(oracle.bf16_to_f32(X).astype(np.float64) @
           oracle.bf16_to_f32(ci.w).astype(np.float64)).astype(np.float32) for X in ci.xs]
    return y1


def _same_choice(got, want, losses, what):
    """Indices must agree; a differing choice is accepted only on a near-tie
    (the oracle's loss at the GPU's choice within 1e-9 of its minimum)."""
    if got == want:
        return
    lo = float(np.min(losses))
    assert abs(float(losses[got]) - lo) <= 1e-9 * max(abs(lo), 1e-30), (what, got, want)


@pytest.mark.parametrize("abits,codes", [(8, CODES_INT), (4, CODES_INT), (4, CODES_E2M3)])
def test_calibration_matches_oracle(abits, codes):
    from w4a4_quantized_gemm_rudder_amd import calibrate as GC
    from w4a4_quantized_gemm_rudder_amd import workloads as W
    log(f"case calibration abits={abits} codes={codes}")
    ci = W.make_calibration(256, 256, seed=3, steps=3, rows=(64, 16, 16), n_outliers=4)
    S = 3
    weights = CAL.map_weights(ci.scores)
    alphas, rhos, gains = GC.DEFAULT_ALPHAS, GC.DEFAULT_RHOS, GC.DEFAULT_GAINS
    y1 = _oracle_targets(ci, S)
    t0 = time.perf_counter()
    best, losses, s = CAL.calibrate_smoothing(ci.xs, ci.sids, ci.w, weights, S, abits, alphas,
                                              yrefs=y1)
    inv = oracle.inv_smooth(s)
    qw, ws = oracle.quantize_weights(ci.w, s)
    Wdeq = (qw.T.astype(np.float32) * ws[None, :]).astype(np.float64)
    y2 = [((oracle.bf16_to_f32(X) * inv[None, :]).astype(np.float32).astype(np.float64)
           @ Wdeq).astype(np.float32) for X in ci.xs]
    tab = CAL.calibrate_table(ci.xs, ci.sids, ci.w, s, weights, S, abits, rhos, gains,
                              yrefs=y2)
    t_cpu = time.perf_counter() - t0
    t0 = time.perf_counter()
    res = GC.calibrate(ci.xs, ci.sids, ci.w, weights, S, abits, codes, alphas, rhos, gains,
                       stage1_targets=y1, stage2_targets=y2)
    t_gpu = time.perf_counter() - t0
    log(f"  alpha {alphas[res.alpha_index]} (oracle {alphas[best]}), rho {res.rho_index} "
        f"(oracle {tab['rho_index']}), gains {res.gain_index} (oracle {tab['gain_index']}); "
        f"{res.passes} passes; gpu {t_gpu:.2f} s, oracle {t_cpu:.2f} s")
    _same_choice(res.alpha_index, best, losses, "alpha")
    if res.alpha_index == best:
        np.testing.assert_allclose(res.stage1_loss, losses, rtol=1e-9)
        st2 = res
    else:
        # a near-tie in stage 1: run the GPU search once more over the
        # oracle's diagonal alone, so that stage 2 is always compared
        log(f"  stage 1 near-tie: stage 2 rerun at the oracle's alpha {alphas[best]}")
        st2 = GC.calibrate(ci.xs, ci.sids, ci.w, weights, S, abits, codes, (alphas[best],),
                           rhos, gains, stage1_targets=y1, stage2_targets=y2)
    assert np.array_equal(st2.smooth, s)
    for t in range(len(ci.xs)):
        np.testing.assert_allclose(st2.stage2_err[t], tab["err"][t], rtol=1e-9, atol=0)
        assert st2.rho_index[t] == tab["rho_index"][t]
        assert st2.gain_index[t] == tab["gain_index"][t]
        assert_bits_equal(f"delta t{t}", st2.delta[t], tab["delta"][t])


def test_calibration_own_targets_agree():
    """With the GPU's own fp32 reference products the search picks the same
    points as with the oracle's fp64 ones (or a near-tie)."""
    from w4a4_quantized_gemm_rudder_amd import calibrate as GC
    from w4a4_quantized_gemm_rudder_amd import workloads as W
    log("case calibration with fp32 targets")
    ci = W.make_calibration(512, 384, seed=5, steps=2, rows=(64, 16, 16), n_outliers=6)
    weights = CAL.map_weights(ci.scores)
    a = GC.calibrate(ci.xs, ci.sids, ci.w, weights, 3, 8)
    y1 = _oracle_targets(ci, 3)
    b = GC.calibrate(ci.xs, ci.sids, ci.w, weights, 3, 8, stage1_targets=y1)
    np.testing.assert_allclose(a.stage1_loss, b.stage1_loss, rtol=1e-4)
    if a.alpha_index != b.alpha_index:                  # near-tie under fp32 targets only
        lo = b.stage1_loss.min()
        assert b.stage1_loss[a.alpha_index] - lo <= 1e-4 * lo
