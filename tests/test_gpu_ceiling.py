"""The MFMA-ceiling measurement call runs on real packed codes, returns OK
and is deterministic (its sink holds exact integer or exactly-summed
checksums)."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("abits,codes", [(8, 0), (4, 0), (4, 1), (8, 1)])
def test_mfma_ceiling_runs_and_is_deterministic(abits, codes):
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    M, K, N = 96, 256, 128
    g = torch.Generator(device="cuda").manual_seed(3)
    Xq = torch.randint(0, 256, (rudder.packed_act_bytes(M, K, abits, codes),), dtype=torch.uint8,
                       device="cuda", generator=g)
    Wq = torch.randint(0, 256, (rudder.packed_weight_bytes(K, N, codes),), dtype=torch.uint8,
                       device="cuda", generator=g)
    sink = torch.empty(rudder.mfma_ceiling_sink_bytes() // 4, dtype=torch.int32, device="cuda")
    rudder.rudder_mfma_ceiling(Xq, Wq, M, N, K, abits, codes, 8, sink)
    first = sink.clone()
    rudder.rudder_mfma_ceiling(Xq, Wq, M, N, K, abits, codes, 8, sink)
    torch.cuda.synchronize()
    assert torch.equal(first, sink)
    zero = torch.zeros_like(Xq)
    rudder.rudder_mfma_ceiling(zero, Wq, M, N, K, abits, codes, 8, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().max()) == 0          # zero activations give zero sums


@pytest.mark.parametrize("abits", [8, 4])
def test_mfma_ceiling_16x16x64_shape(abits):
    """The int8 16x16x64 instruction shape of the ceiling probe runs, is
    deterministic and gives zero sums on zero activations; it takes int codes
    only."""
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    M, K, N = 96, 256, 128
    g = torch.Generator(device="cuda").manual_seed(4)
    Xq = torch.randint(0, 256, (rudder.packed_act_bytes(M, K, abits, 0),), dtype=torch.uint8,
                       device="cuda", generator=g)
    Wq = torch.randint(0, 256, (rudder.packed_weight_bytes(K, N, 0),), dtype=torch.uint8,
                       device="cuda", generator=g)
    sink = torch.empty(rudder.mfma_ceiling_sink_bytes() // 4, dtype=torch.int32, device="cuda")
    shape = rudder.CEILING_I8_16X16X64
    rudder.rudder_mfma_ceiling_shape(Xq, Wq, M, N, K, abits, 0, 8, shape, sink)
    first = sink.clone()
    rudder.rudder_mfma_ceiling_shape(Xq, Wq, M, N, K, abits, 0, 8, shape, sink)
    torch.cuda.synchronize()
    assert torch.equal(first, sink)
    rudder.rudder_mfma_ceiling_shape(torch.zeros_like(Xq), torch.zeros_like(Wq), M, N, K, abits,
                                     0, 8, shape, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().max()) == 0
    with pytest.raises(rudder.RudderError):
        rudder.rudder_mfma_ceiling_shape(Xq, Wq, M, N, K, 4, 1, 8, shape, sink)
