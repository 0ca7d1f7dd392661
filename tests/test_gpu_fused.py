"""GPU parity of the fused MLP path -- up-projection, GELU kept in BF16, and
the down layer's activation quantizer in one epilogue
(rudder_linear_gelu_quant) -- and of its GELU, against the CPU oracle.

Bar: the GELU table bit-exact on all 65536 bf16 patterns; the down layer's
packed codes (padding rows included) and row scales bit-exact.
"""
import numpy as np
import pytest

import oracle
from gpu_harness import (CODES_E2M3, CODES_INT, assert_bits_equal, log, tile_for, to_dev,
                         to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from w4a4_quantized_gemm_rudder_amd import rudder
    rudder.load_library()
    yield


def _bf16(x):
    return oracle.f32_to_bf16(np.asarray(x, np.float32))


def test_gelu_every_bf16_pattern():
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    log("case gelu table")
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = torch.from_numpy(allb.view(np.int16).copy()).cuda()
    out = torch.empty_like(x)
    rudder.rudder_gelu_bf16(x, out, x.numel())
    torch.cuda.synchronize()
    assert_bits_equal("gelu", out.cpu().numpy().view(np.uint16), oracle.gelu_bf16(allb))


@pytest.mark.parametrize("offset,n", [(1, 1001), (0, 13), (3, 70000)])
def test_gelu_unaligned_and_tail(offset, n):
    """The element-by-element path (unaligned buffers) and the tail after
    the 8-wide groups."""
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    log(f"case gelu offset={offset} n={n}")
    rng = np.random.default_rng(n)
    vals = rng.integers(0, 65536, n + offset).astype(np.uint16)
    x = torch.from_numpy(vals.view(np.int16).copy()).cuda()
    out = torch.zeros(n + offset, dtype=torch.int16, device="cuda")
    rudder.rudder_gelu_bf16(x[offset:], out[offset:], n)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert_bits_equal("gelu", got[offset:], oracle.gelu_bf16(vals[offset:]))
    assert np.all(got[:offset] == 0)


def run_fused(X, sid, Wb, s, a, b, delta, ninv, ndelta, S, abits, codes, nabits, ncodes,
              label=""):
    """Run rudder_linear_gelu_quant on the GPU and the oracle's composition;
    compare the down layer's packed codes and row scales."""
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    M, K = X.shape
    N = Wb.shape[1]
    inv = oracle.inv_smooth(s)
    qw, ws = oracle.quantize_weights(Wb, s)
    want_q, want_rs = oracle.linear_gelu_quant(X, sid, qw, ws, inv, delta, a, b, S, abits,
                                               ninv, ndelta, nabits)
    Xd, sid_d = to_dev_bf16(X), to_dev(sid.astype(np.uint8))
    Wq, w_scale, inv_d = rudder.quantize_weights(to_dev_bf16(Wb), to_dev(s), codes)
    Xq, rs = rudder.quant_act(Xd, sid_d, inv_d, to_dev(delta), S, abits, codes)
    nxq, nrs = rudder.linear_gelu_quant(Xq, rs, sid_d, Wq, w_scale, to_dev(a), to_dev(b), M, N,
                                        K, S, abits, to_dev(ninv), to_dev(ndelta), nabits,
                                        codes, ncodes)
    torch.cuda.synchronize()
    assert_bits_equal(f"{label} next row_scale", nrs.cpu().numpy()[:M], want_rs)
    assert_bits_equal(f"{label} next codes", nxq.cpu().numpy(), tile_for(ncodes, want_q, nabits))
    nz = int((want_q != 0).sum())
    sat = int((np.abs(want_q) == (127 if nabits == 8 else 7)).sum())
    return dict(codes=int(want_q.size), nonzero=nz, saturated=sat)


def _step_sizes(u_abs_max_per_stream, q, rng):
    return (np.asarray(u_abs_max_per_stream) / q * rng.uniform(0.5, 1.0,
                                                               len(u_abs_max_per_stream))
            ).astype(np.float32)


def fused_random_case(M, K, N, S, abits, codes, nabits, ncodes, seed):
    rng = np.random.default_rng(2000 + seed)
    x = rng.standard_normal((M, K))
    x[:, rng.integers(0, K, 3)] *= 25.0
    X = _bf16(x)
    Wb = _bf16(rng.standard_normal((K, N)) * 0.05)
    sid = rng.integers(0, S, M).astype(np.uint8)
    s = rng.uniform(0.25, 4.0, K).astype(np.float32)
    a = rng.uniform(0.9, 1.1, (S, N)).astype(np.float32)
    b = (rng.standard_normal((S, N)) * 0.05).astype(np.float32)
    qa = 127 if abits == 8 else 7
    delta = _step_sizes([np.abs(x / s[None, :]).max()] * S, qa, rng)
    # the next layer's step sizes from the range of its actual input
    inv = oracle.inv_smooth(s)
    qw, ws = oracle.quantize_weights(Wb, s)
    _, _, _, Y = oracle.linear(X, sid, qw, ws, inv, delta, a, b, S, abits)
    ns = rng.uniform(0.25, 4.0, N).astype(np.float32)
    ninv = oracle.inv_smooth(ns)
    u = np.abs(oracle.bf16_to_f32(oracle.gelu_bf16(Y)) * ninv[None, :])
    nq = 127 if nabits == 8 else 7
    ndelta = _step_sizes([u.max()] * S, nq, rng)
    return run_fused(X, sid, Wb, s, a, b, delta, ninv, ndelta, S, abits, codes, nabits, ncodes,
                     label=f"fused{seed}")


FUSED = [
    # M, K, N, S, abits, codes, next_abits, next_codes, seed
    (200, 256, 512, 3, 4, CODES_INT, 4, CODES_INT, 1),
    (257, 128, 320, 3, 4, CODES_E2M3, 4, CODES_E2M3, 2),
    (33, 256, 256, 5, 8, CODES_INT, 8, CODES_INT, 3),
    (1, 128, 64, 1, 4, CODES_E2M3, 8, CODES_INT, 4),
    (600, 384, 768, 8, 4, CODES_INT, 4, CODES_E2M3, 5),
    (129, 256, 1024, 2, 8, CODES_INT, 4, CODES_E2M3, 6),
    (300, 256, 288, 3, 4, CODES_E2M3, 4, CODES_INT, 7),
    (97, 512, 2048, 3, 4, CODES_E2M3, 8, CODES_INT, 8),
]


@pytest.mark.parametrize("M,K,N,S,abits,codes,nabits,ncodes,seed", FUSED)
def test_fused_ragged(M, K, N, S, abits, codes, nabits, ncodes, seed):
    log(f"case fused M={M} K={K} N={N} S={S} abits={abits} codes={codes} next={nabits}/"
        f"{ncodes} seed={seed}")
    log(f"  {fused_random_case(M, K, N, S, abits, codes, nabits, ncodes, seed)}")


@pytest.mark.slow
@pytest.mark.parametrize("ncodes", [CODES_E2M3, CODES_INT])
def test_fused_full_size_mlp_h2048(ncodes):
    """The hidden-2048 MLP up-projection (4192 x 2048 -> 8192, W4A4) feeding
    the down layer: every code of its 4192 x 8192 input compared."""
    from w4a4_quantized_gemm_rudder_amd import workloads as W
    log(f"case fused full-size mlp_h2048_m4192 up -> down, next codes {ncodes}")
    wi = W.make_inputs("mlp_h2048_m4192_w4a4", seed=0, layers=["up", "down"])
    up, down = wi.layers
    t = 3
    a, b = up.step_comp(t)
    rng = np.random.default_rng(77)
    # the down layer's step sizes from the range of its actual (fused) input
    inv = oracle.inv_smooth(up.smooth)
    qw, ws = oracle.quantize_weights(up.w, up.smooth)
    _, _, _, Y = oracle.linear(up.x, wi.stream_id, qw, ws, inv, up.act_scale[t], a, b, 3, 4)
    ninv = oracle.inv_smooth(down.smooth)
    u = np.abs(oracle.bf16_to_f32(oracle.gelu_bf16(Y)) * ninv[None, :])
    ndelta = np.array([u[wi.stream_id == st].max() / 7 * rng.uniform(0.6, 1.0)
                       for st in range(3)], np.float32)
    st = run_fused(up.x, wi.stream_id, up.w, up.smooth, a, b, up.act_scale[t], ninv, ndelta, 3,
                   4, ncodes, 4, ncodes, label="full mlp")
    log(f"  {st}")
