"""The no-allocation entry point (rudder_quant_act_noalloc) against the
entry point it varies (rudder_quant_act in dynamic mode with a caller
workspace): codes, row scales and step sizes bit-exact, on two calls in a row
(the second with a smaller input, so stale scratch contents would show), in
every (bits, container) combination.  Both are called through the C ABI."""
import numpy as np
import pytest

from gpu_harness import CODES_E2M3, CODES_INT, assert_bits_equal, log, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _inputs(rng, M, K, S):
    import torch
    x = rng.standard_normal((M, K))
    x[:, rng.integers(0, K, 3)] *= 20.0
    X = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    sid = rng.integers(0, S, M).astype(np.uint8)
    if S >= 3:
        sid[sid == 1] = 0                         # an empty stream
    inv = rng.uniform(0.25, 4.0, K).astype(np.float32)
    return X.cuda(), to_dev(sid), to_dev(inv)


def _one(rudder, torch, X, sid, inv, M, K, S, abits, codes):
    nbytes = max(rudder.packed_act_bytes(M, K, abits, codes), 1)
    outs = []
    for noalloc in (False, True):
        Xq = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
        rs = torch.full((max(M, 1),), -1.0, dtype=torch.float32, device="cuda")
        d = torch.full((S,), -1.0, dtype=torch.float32, device="cuda")
        if noalloc:
            rudder.rudder_quant_act_noalloc(X, sid, inv, d, M, K, S, abits, codes, Xq, rs)
        else:
            ws = torch.empty(rudder.quant_act_workspace_bytes(S), dtype=torch.uint8,
                             device="cuda")
            rudder.rudder_quant_act(X, sid, inv, None, d, ws, M, K, S, abits, codes, Xq, rs)
        outs.append((Xq, rs, d))
    torch.cuda.synchronize()
    (q0, r0, d0), (q1, r1, d1) = outs
    assert_bits_equal("act_scale_out", d1.cpu().numpy(), d0.cpu().numpy())
    assert_bits_equal("row_scale", r1.cpu().numpy(), r0.cpu().numpy())
    assert_bits_equal("Xq", q1.cpu().numpy(), q0.cpu().numpy())
    return d0.cpu().numpy()


@pytest.mark.parametrize("abits,codes", [(8, CODES_INT), (4, CODES_INT), (4, CODES_E2M3),
                                         (8, CODES_E2M3)])
def test_noalloc_matches_workspace_entry_point(abits, codes):
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    rudder.load_library()
    rng = np.random.default_rng(900 + abits + 10 * codes)
    # a large call (many partial-max blocks), then a smaller one with a
    # different stream count: the scratch keeps the first call's contents
    for (M, K, S) in ((4192, 2048, 3), (70, 256, 2)):
        log(f"case noalloc M={M} K={K} S={S} abits={abits} codes={codes}")
        X, sid, inv = _inputs(rng, M, K, S)
        d = _one(rudder, torch, X, sid, inv, M, K, S, abits, codes)
        log(f"  step sizes {d.tolist()}")


def test_noalloc_validation():
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    rudder.load_library()
    f = torch.ones(64, dtype=torch.float32, device="cuda")
    b = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(rudder.RudderError) as e:
        rudder.rudder_quant_act_noalloc(b, b, f, None, 4, 48, 1, 8, CODES_INT, b, f)
    assert e.value.status == rudder.RUDDER_ERR_INVALID_ARG
    with pytest.raises(rudder.RudderError) as e:
        rudder.rudder_quant_act_noalloc(b, b, f, None, 4, 64, 9, 8, CODES_INT, b, f)
    assert e.value.status == rudder.RUDDER_ERR_INVALID_ARG
    rudder.rudder_quant_act_noalloc(b, b, f, None, 0, 64, 1, 8, CODES_INT, b, f)   # M = 0
