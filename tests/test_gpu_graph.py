"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Each case runs a sequence of library calls eagerly, captures the same
sequence into a graph, and replays it three times.  Before every replay the
outputs are overwritten with garbage, and eager work and synchronizations run
between the replays.  Every replay's codes, row scales, step sizes and bf16
outputs must equal the eager run's bit for bit.  The library allocates
nothing and records no memset node, which is what makes its calls safe to
capture; these cases check it on each launch form: the tiled GEMM with its
lone-tile and streamed-tail layout, the few-row kernel behind the dynamic
(absmax) quantizer, and the fused GELU-quantize epilogue.
"""
import pytest

from gpu_harness import CODES_E2M3, CODES_INT, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from w4a4_quantized_gemm_rudder_amd import rudder
    rudder.load_library()
    yield


def _inputs(M, K, N, S, seed):
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    X = torch.randn(M, K, generator=g, device="cuda").to(torch.bfloat16)
    W = (torch.randn(K, N, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    smooth = torch.rand(K, generator=g, device="cuda") + 0.5
    # rows in runs of one stream, as the workloads order them
    sid = torch.sort(torch.randint(0, S, (M,), generator=g, device="cuda")).values.to(torch.uint8)
    delta = torch.rand(S, generator=g, device="cuda") * 0.05 + 0.02
    a = torch.rand(S, N, generator=g, device="cuda") * 0.2 + 0.9
    b = torch.randn(S, N, generator=g, device="cuda") * 0.01
    return X, W, smooth, sid, delta, a, b


def _replay_and_compare(label, run, outputs):
    """run(): enqueue the calls on the current stream.  outputs: the tensors
    they write."""
    import torch
    run()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    scratch = torch.randn(512, 512, device="cuda")
    for rep in range(3):
        for o in outputs:
            o.view(torch.uint8).fill_(0xA5)
        (scratch @ scratch).sum().item()          # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outputs, want)):
            same = torch.equal(o.view(torch.uint8), w.view(torch.uint8))
            assert same, f"{label}: replay {rep}, output {i} differs from the eager run"
    del graph


@pytest.mark.parametrize("M,K,N,S,abits,codes,seed", [
    (4192, 512, 2048, 3, 8, CODES_INT, 200),     # one tile per CU + 96 streamed rows
    (2200, 256, 4096, 3, 4, CODES_E2M3, 201),    # one tile per CU + 152 rows, 96-row blocks
    (1000, 384, 768, 2, 4, CODES_INT, 202),      # ragged last tile
])
def test_static_step_graph(M, K, N, S, abits, codes, seed):
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    log(f"case graph static M={M} K={K} N={N} S={S} abits={abits} codes={codes}")
    X, W, smooth, sid, delta, a, b = _inputs(M, K, N, S, seed)
    Wq, ws, inv = rudder.quantize_weights(W, smooth, codes)
    Xq = torch.empty(rudder.packed_act_bytes(M, K, abits, codes), dtype=torch.uint8,
                     device="cuda")
    rs = torch.empty(M, dtype=torch.float32, device="cuda")
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")

    def run():
        rudder.rudder_quant_act(X, sid, inv, delta, None, None, M, K, S, abits, codes, Xq, rs)
        rudder.rudder_linear(Xq, rs, sid, Wq, ws, a, b, M, N, K, S, abits, codes, Y)

    _replay_and_compare("static", run, [Xq, rs, Y])


def test_dynamic_few_row_graph():
    """Dynamic step sizes (partial absmax, finalize, quantize) and the few-row
    GEMM: four launches per linear, all captured."""
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    M, K, N, S, abits, codes = 96, 256, 256, 3, 8, CODES_INT
    log(f"case graph dynamic M={M} K={K} N={N}")
    X, W, smooth, sid, _, a, b = _inputs(M, K, N, S, 203)
    Wq, ws, inv = rudder.quantize_weights(W, smooth, codes)
    Xq = torch.empty(rudder.packed_act_bytes(M, K, abits, codes), dtype=torch.uint8,
                     device="cuda")
    rs = torch.empty(M, dtype=torch.float32, device="cuda")
    dout = torch.empty(S, dtype=torch.float32, device="cuda")
    wsp = torch.empty(rudder.quant_act_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")

    def run():
        rudder.rudder_quant_act(X, sid, inv, None, dout, wsp, M, K, S, abits, codes, Xq, rs)
        rudder.rudder_linear(Xq, rs, sid, Wq, ws, a, b, M, N, K, S, abits, codes, Y)

    _replay_and_compare("dynamic", run, [Xq, rs, dout, Y])


def test_fused_gelu_quant_graph():
    """The up-projection with GELU and the down layer's quantizer in its
    epilogue, then the down-projection, as one captured chain."""
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    M, K, N, S = 1000, 256, 512, 2
    codes = CODES_E2M3
    log(f"case graph fused M={M} K={K} N={N}")
    X, W, smooth, sid, delta, a, b = _inputs(M, K, N, S, 204)
    _, W2, smooth2, _, delta2, a2, b2 = _inputs(N, N, K, S, 205)
    Wq, ws, inv = rudder.quantize_weights(W, smooth, codes)
    Wq2, ws2, inv2 = rudder.quantize_weights(W2, smooth2, codes)
    Xq = torch.empty(rudder.packed_act_bytes(M, K, 4, codes), dtype=torch.uint8, device="cuda")
    rs = torch.empty(M, dtype=torch.float32, device="cuda")
    Xq2 = torch.empty(rudder.packed_act_bytes(M, N, 4, codes), dtype=torch.uint8, device="cuda")
    rs2 = torch.empty(M, dtype=torch.float32, device="cuda")
    Y = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")

    def run():
        rudder.rudder_quant_act(X, sid, inv, delta, None, None, M, K, S, 4, codes, Xq, rs)
        rudder.rudder_linear_gelu_quant(Xq, rs, sid, Wq, ws, a, b, M, N, K, S, 4, codes, inv2,
                                        delta2, 4, codes, Xq2, rs2)
        rudder.rudder_linear(Xq2, rs2, sid, Wq2, ws2, a2, b2, M, K, N, S, 4, codes, Y)

    _replay_and_compare("fused", run, [Xq, rs, Xq2, rs2, Y])
