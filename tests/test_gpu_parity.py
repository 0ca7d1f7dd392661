"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: weight/activation codes, scales and int32 accumulators bit-exact; bf16
outputs within 2 bf16 ulp (the arithmetic is specified step by step, so the
expected difference is 0 and the observed count is logged).
"""
import numpy as np
import pytest

from gpu_harness import CODES_E2M3, CODES_INT, LayerRun, log, sample_rows, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from w4a4_quantized_gemm_rudder_amd import rudder
    rudder.load_library()
    yield


def _torch_bf16_bits(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------------------
# Single 256 -> 256 linear, 96 tokens, W4A8, absmax scales (the small case)
# ---------------------------------------------------------------------------

def test_linear_m96_k256_n256_w4a8_dynamic():
    from w4a4_quantized_gemm_rudder_amd import workloads as W
    wi = W.make_inputs("linear_m96_k256_n256_w4a8", seed=0)
    L = wi.layers[0]
    log("case linear_m96_k256_n256_w4a8 dynamic")
    run = LayerRun(L.x, wi.stream_id, L.w, L.smooth, L.comp_a, L.comp_b, 3, 8)
    run.check_weights()
    st = run.run_step(None, L.comp_a, L.comp_b, label="c1")
    log(f"  {st}")


# ---------------------------------------------------------------------------
# Random ragged shapes: M tails, shuffled stream tags, 1..8 streams, an empty
# stream, both bit widths, static and dynamic scales
# ---------------------------------------------------------------------------

RAGGED = [
    # M, K, N, S, abits, dynamic, seed
    (1, 128, 32, 1, 8, False, 0),
    (31, 128, 96, 3, 4, False, 1),
    (33, 256, 64, 3, 8, True, 2),
    (200, 384, 288, 5, 4, True, 3),
    (255, 256, 256, 8, 8, False, 4),
    (257, 512, 320, 3, 4, False, 5),
    (600, 256, 544, 2, 8, True, 6),
    (513, 1024, 256, 3, 4, True, 7),
    (97, 128, 1024, 7, 8, False, 8),
    # tiled kernel with 1, 3 and 5 k-stages (odd stage counts end the
    # two-stage weight/ring rotation on its first set), and 8 streams
    (300, 128, 256, 3, 8, False, 50),
    (301, 384, 512, 4, 4, True, 51),
    (520, 640, 288, 8, 8, False, 52),
]


# W4A4 with 4-bit codes held as FP6 E2M3 (K a multiple of 128)
RAGGED_E2M3 = [
    (1, 128, 32, 1, 4, False, 10),
    (31, 128, 96, 3, 4, True, 11),
    (200, 384, 288, 5, 4, True, 12),
    (257, 512, 320, 3, 4, False, 13),
    (513, 1024, 256, 8, 4, True, 14),
    (97, 256, 1024, 7, 4, False, 15),
    (300, 128, 256, 3, 4, False, 53),
    (301, 384, 512, 8, 4, True, 54),
    (520, 640, 288, 2, 4, False, 55),
]


# W4A8 with the 8-bit codes held as two E2M3 digit planes (K a multiple of
# 128): one, three and five k-stages, tails, 1..8 streams
RAGGED_E2M3_A8 = [
    (1, 128, 32, 1, 8, False, 70),
    (33, 256, 64, 3, 8, True, 71),
    (255, 256, 256, 8, 8, False, 72),
    (257, 512, 320, 3, 8, True, 73),
    (300, 128, 256, 3, 8, False, 74),
    (301, 384, 512, 4, 8, True, 75),
    (520, 640, 288, 2, 8, False, 76),
    (600, 256, 544, 2, 8, True, 77),
    (97, 1024, 1024, 7, 8, False, 78),
]


def _random_layer_case(M, K, N, S, abits, dynamic, seed, codes):
    rng = np.random.default_rng(1000 + seed)
    x = rng.standard_normal((M, K))
    x[:, rng.integers(0, K, 3)] *= 25.0
    X = _torch_bf16_bits(x)
    Wb = _torch_bf16_bits(rng.standard_normal((K, N)) * 0.02)
    sid = rng.integers(0, S, M).astype(np.uint8)
    if S >= 3:
        sid[sid == 1] = 0                        # stream 1 has no rows
    s = rng.uniform(0.25, 4.0, K).astype(np.float32)
    a = rng.uniform(0.9, 1.1, (S, N)).astype(np.float32)
    b = (rng.standard_normal((S, N)) * 0.01).astype(np.float32)
    run = LayerRun(X, sid, Wb, s, a, b, S, abits, codes)
    run.check_weights()
    if dynamic:
        delta = None
    else:
        qa = 127 if abits == 8 else 7
        u = np.abs(x / s[None, :]).max()
        delta = (rng.uniform(0.5, 1.0, S) * u / qa).astype(np.float32)
    return run.run_step(delta, a, b, label=f"case{seed}")


@pytest.mark.parametrize("M,K,N,S,abits,dynamic,seed,codes",
                         [r + (CODES_INT,) for r in RAGGED] +
                         [r + (CODES_E2M3,) for r in RAGGED_E2M3] +
                         [r + (CODES_E2M3,) for r in RAGGED_E2M3_A8])
def test_ragged_shapes(M, K, N, S, abits, dynamic, seed, codes):
    log(f"case ragged M={M} K={K} N={N} S={S} abits={abits} dynamic={dynamic} seed={seed} "
        f"codes={codes}")
    log(f"  {_random_layer_case(M, K, N, S, abits, dynamic, seed, codes)}")


# Few-row calls (the weight-streaming kernel): action/proprio-sized M against
# full-width weights, both sides of the row-count switch, every container.
SMALL_M = [
    # M, K, N, S, abits, dynamic, seed, codes
    (96, 2048, 6144, 3, 8, True, 20, CODES_INT),
    (64, 2048, 2048, 3, 8, False, 21, CODES_INT),
    (65, 2048, 2048, 2, 8, False, 22, CODES_INT),
    (128, 4096, 1024, 3, 4, False, 23, CODES_INT),
    (129, 1024, 512, 3, 4, True, 24, CODES_INT),
    (32, 8192, 2048, 3, 4, False, 25, CODES_E2M3),
    (100, 4096, 12288, 3, 4, True, 26, CODES_E2M3),
    (128, 128, 96, 5, 4, False, 27, CODES_E2M3),
    (2, 256, 64, 2, 8, True, 28, CODES_INT),
    # more than 128 rows on a narrow layer: 64-row groups fill more CUs
    (192, 2048, 2048, 3, 4, False, 29, CODES_E2M3),
    (250, 512, 1024, 3, 8, True, 30, CODES_INT),
    # wide layers: two 32-channel blocks per workgroup
    (192, 256, 16384, 3, 4, False, 31, CODES_E2M3),
    (250, 256, 16384, 3, 8, True, 32, CODES_INT),
    (60, 256, 16384, 2, 4, False, 33, CODES_INT),
    # every workgroup shape the few-row launch chooses (rows per group x
    # channels per workgroup), with channel counts that are odd multiples of
    # 32 where the choice needs them
    (193, 256, 2784, 3, 4, False, 80, CODES_INT),      # 64 x 96
    (193, 256, 2208, 3, 4, True, 81, CODES_INT),       # 96 x 32
    (193, 256, 4160, 3, 4, False, 82, CODES_INT),      # 96 x 64
    (193, 256, 6240, 3, 4, False, 83, CODES_INT),      # 96 x 96
    (97, 256, 4128, 3, 4, True, 84, CODES_INT),        # 128 x 32
    (193, 256, 5504, 3, 4, False, 85, CODES_INT),      # 128 x 64
    (193, 256, 2208, 3, 8, False, 86, CODES_INT),      # 64 x 96
    (65, 256, 4128, 3, 8, True, 87, CODES_INT),        # 96 x 32
    (193, 256, 4160, 3, 8, False, 88, CODES_INT),      # 96 x 64
    (193, 256, 6240, 3, 8, False, 89, CODES_INT),      # 96 x 96
    (193, 256, 2112, 3, 4, False, 90, CODES_E2M3),     # 64 x 64
    (193, 256, 2208, 3, 4, True, 91, CODES_E2M3),      # 96 x 32
    (193, 256, 6240, 3, 4, False, 92, CODES_E2M3),     # 96 x 96
    (97, 256, 4128, 3, 4, False, 93, CODES_E2M3),      # 128 x 32
    (193, 256, 5504, 3, 4, True, 94, CODES_E2M3),      # 128 x 64
    (192, 4096, 12288, 3, 4, False, 95, CODES_E2M3),   # the benchmark's 192-row call
    # 8-bit codes as E2M3 digit planes (64-row groups only)
    (96, 2048, 6144, 3, 8, True, 34, CODES_E2M3),
    (192, 2048, 2048, 3, 8, False, 35, CODES_E2M3),
    (250, 256, 16384, 3, 8, True, 36, CODES_E2M3),
    (2, 256, 64, 2, 8, False, 37, CODES_E2M3),
]


@pytest.mark.parametrize("M,K,N,S,abits,dynamic,seed,codes", SMALL_M)
def test_small_m(M, K, N, S, abits, dynamic, seed, codes):
    log(f"case small-M M={M} K={K} N={N} S={S} abits={abits} dynamic={dynamic} seed={seed} "
        f"codes={codes}")
    log(f"  {_random_layer_case(M, K, N, S, abits, dynamic, seed, codes)}")


# Row counts just past a whole number of tile rounds: the tiles take the rows
# of the full rounds and weight-streaming blocks in the same launch the
# remainder (8192 + 100 rows x 2048 channels = 520 tiles of 128 x 256 for 512
# resident workgroups).  Every row is compared.
@pytest.mark.parametrize("M,K,N,S,abits,dynamic,seed,codes", [
    (8292, 128, 2048, 3, 8, False, 40, CODES_INT),
    (8292, 256, 2048, 3, 4, True, 41, CODES_E2M3),
    (8292, 128, 2048, 2, 4, False, 42, CODES_INT),
    (8384, 256, 2048, 3, 4, False, 43, CODES_E2M3),     # 192-row remainder
    (8384, 512, 4096, 3, 8, True, 48, CODES_INT),       # two full rounds, 4096 wide
    (8292, 384, 4096, 4, 4, False, 49, CODES_E2M3),
    (8292, 128, 2048, 3, 8, False, 56, CODES_E2M3),     # 8-bit codes as digit planes
    (8384, 256, 2048, 3, 8, True, 57, CODES_E2M3),
    # a remainder of exactly 256 rows (the largest streamed: four 64-row
    # groups), and 257 rows (not streamed: a partial round of full tiles)
    (8448, 128, 2048, 3, 8, False, 58, CODES_INT),
    (8448, 256, 2048, 2, 4, True, 59, CODES_E2M3),
    (8449, 128, 2048, 3, 4, False, 60, CODES_INT),
    # less than one round but more tiles than compute units: 4192 rows x 2048
    # channels (264 tiles, 256 CUs) take 4096 rows as one tile per CU and
    # stream the other 96; 2200 x 4096 (288 tiles) streams 152 rows; a
    # 256-row remainder (the most streamed) and 257 (not streamed)
    (4192, 256, 2048, 3, 8, False, 61, CODES_INT),
    (4192, 512, 2048, 2, 4, True, 62, CODES_E2M3),
    (2200, 128, 4096, 3, 4, False, 63, CODES_INT),
    (2200, 256, 4096, 3, 8, False, 64, CODES_E2M3),
    (4352, 128, 2048, 3, 8, False, 65, CODES_INT),
    (4353, 256, 2048, 3, 4, False, 66, CODES_E2M3),
    # a full round, then more tiles than CUs (4192 x 6144: 792 tiles): the
    # first 4096 rows as tiles (one round plus one per CU), 96 rows streamed
    (4192, 256, 6144, 3, 8, False, 67, CODES_INT),
    (4192, 128, 6144, 2, 4, True, 68, CODES_E2M3),
    # eight streams: the epilogue tables leave one workgroup per CU, so a
    # round is 256 tiles and the 96 rows past it stream after the tiles
    (4192, 256, 2048, 8, 4, False, 70, CODES_E2M3),
    (4192, 128, 2048, 8, 8, True, 71, CODES_INT),
    # the same 2100 x 4128 in the E2M3 container: no half-width tiles, so all
    # 289 tiles run (a partial round), the last column 32 channels wide
    (2100, 256, 4128, 2, 4, True, 97, CODES_E2M3),
])
def test_round_remainder_split(M, K, N, S, abits, dynamic, seed, codes):
    log(f"case round split M={M} K={K} N={N} S={S} abits={abits} codes={codes}")
    log(f"  {_random_layer_case(M, K, N, S, abits, dynamic, seed, codes)}")


# Wider layers with the int containers: the rows past the last whole round
# run as half-width (128-channel) tiles in the same launch.  8192 + 192 rows
# x 6144 channels = 1584 tiles of 128 x 256 for 512 resident workgroups;
# 8192 + 100 rows x 12288 channels; 8128 channels, whose last half-width
# tile is half past N; one and two k-stages.  Every row is compared.
@pytest.mark.parametrize("M,K,N,S,abits,dynamic,seed,codes", [
    (8384, 128, 6144, 3, 8, False, 44, CODES_INT),
    (8384, 256, 6144, 3, 4, True, 45, CODES_INT),
    (8292, 128, 12288, 4, 8, False, 46, CODES_INT),
    (8384, 128, 8128, 3, 8, False, 47, CODES_INT),      # last narrow tile half outside N
    # 2100 x 12288 (816 tiles): one round plus one tile per CU, then 52 rows
    # as half-width tiles
    (2100, 128, 12288, 3, 8, False, 69, CODES_INT),
    # 2100 x 4128 (17 tile columns, the last 32 channels wide; 289 tiles):
    # one tile per CU over 1920 rows, then 180 rows as half-width tiles,
    # whose last column is mostly past N
    (2100, 128, 4128, 3, 8, False, 96, CODES_INT),
])
def test_round_remainder_narrow_tiles(M, K, N, S, abits, dynamic, seed, codes):
    log(f"case narrow tail M={M} K={K} N={N} S={S} abits={abits} codes={codes}")
    log(f"  {_random_layer_case(M, K, N, S, abits, dynamic, seed, codes)}")


# Rows in runs of one stream, as the workloads order them.  The tiled
# epilogue takes a batched path when all 128 token rows of a wave share one
# stream and a per-row gather otherwise; the runs below give both kinds of
# wave in one call: whole 128-row waves of one stream, run boundaries inside
# a wave and on a wave boundary, a single row of another stream inside a run,
# and a ragged last tile.
@pytest.mark.parametrize("abits,codes", [(8, CODES_INT), (4, CODES_INT), (4, CODES_E2M3),
                                         (8, CODES_E2M3)])
def test_stream_runs_uniform_and_mixed_waves(abits, codes):
    M, K, N, S = 700, 256, 512, 4
    rng = np.random.default_rng(60 + abits + codes)
    sid = np.zeros(M, np.uint8)
    sid[128:192] = 1          # boundary inside the second wave of tile 0
    sid[192:256] = 2
    sid[256:384] = 2          # a whole wave of stream 2
    sid[384:512] = 3
    sid[450] = 0              # one foreign row inside a stream-3 wave
    sid[512:640] = 1
    sid[640:] = 2             # ragged last tile
    x = rng.standard_normal((M, K))
    x[:, rng.integers(0, K, 3)] *= 25.0
    X = _torch_bf16_bits(x)
    Wb = _torch_bf16_bits(rng.standard_normal((K, N)) * 0.02)
    s = rng.uniform(0.25, 4.0, K).astype(np.float32)
    a = rng.uniform(0.9, 1.1, (S, N)).astype(np.float32)
    b = (rng.standard_normal((S, N)) * 0.01).astype(np.float32)
    qa = 127 if abits == 8 else 7
    delta = (rng.uniform(0.5, 1.0, S) * np.abs(x / s[None, :]).max() / qa).astype(np.float32)
    log(f"case stream runs M={M} K={K} N={N} S={S} abits={abits} codes={codes}")
    run = LayerRun(X, sid, Wb, s, a, b, S, abits, codes)
    run.check_weights()
    log(f"  {run.run_step(delta, a, b, label='runs')}")


@pytest.mark.parametrize("abits,codes,K,M", [(8, CODES_INT, 65536, 40), (4, CODES_INT, 65536, 40),
                                             (4, CODES_E2M3, 65536, 40),
                                             (8, CODES_E2M3, 16384, 40),
                                             (8, CODES_E2M3, 16384, 300)])
def test_saturated_codes_at_max_k(abits, codes, K, M):
    """The largest supported K (65536; 16384 for 8-bit E2M3 codes) with every
    weight and activation code at +-qmax: the accumulators reach K * 7 * qmax
    in magnitude and must still be exact (few-row and tiled kernels)."""
    log(f"case saturated K={K} M={M} abits={abits} codes={codes}")
    rng = np.random.default_rng(99)
    N, S = 64, 2
    sx = np.where(rng.random((M, K)) < 0.5, -1.0, 1.0)
    sw = np.where(rng.random((K, N)) < 0.5, -1.0, 1.0)
    sw[:, :4] = 1.0                               # some columns of all-equal signs
    sx[:2] = 1.0                                  # rows whose dot products hit the maximum
    X = _torch_bf16_bits(sx * 3.0)
    Wb = _torch_bf16_bits(sw * 0.5)
    sid = (np.arange(M) % S).astype(np.uint8)
    s = np.ones(K, np.float32)
    a = np.ones((S, N), np.float32)
    b = np.zeros((S, N), np.float32)
    run = LayerRun(X, sid, Wb, s, a, b, S, abits, codes)
    run.check_weights()
    qa = 127 if abits == 8 else 7
    delta = np.full(S, 3.0 / qa, np.float32) * np.float32(0.999)   # every code clamps to qmax
    st = run.run_step(delta, a, b, label="saturated")
    log(f"  {st}")


def test_zero_scale_stream_gives_bias():
    log("case zero step size")
    rng = np.random.default_rng(77)
    M, K, N, S = 70, 256, 128, 3
    X = _torch_bf16_bits(rng.standard_normal((M, K)))
    Wb = _torch_bf16_bits(rng.standard_normal((K, N)) * 0.02)
    sid = (np.arange(M) % 3).astype(np.uint8)
    s = np.ones(K, np.float32)
    a = np.ones((S, N), np.float32)
    b = (rng.standard_normal((S, N))).astype(np.float32)
    run = LayerRun(X, sid, Wb, s, a, b, S, 8)
    delta = np.array([0.02, 0.0, 0.03], np.float32)
    run.run_step(delta, a, b, label="zero-scale")


@pytest.mark.parametrize("codes", [CODES_INT, CODES_E2M3])
def test_repeat_calls_deterministic(codes):
    log(f"case determinism codes={codes}")
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    rng = np.random.default_rng(5)
    M, K, N, S = 300, 512, 256, 3
    X = to_dev_bf16(_torch_bf16_bits(rng.standard_normal((M, K))))
    Wd = to_dev_bf16(_torch_bf16_bits(rng.standard_normal((K, N)) * 0.02))
    sid = to_dev(rng.integers(0, S, M).astype(np.uint8))
    s = to_dev(np.ones(K, np.float32))
    Wq, ws, inv = rudder.quantize_weights(Wd, s, codes)
    ca = to_dev(np.ones((S, N), np.float32))
    cb = to_dev(np.zeros((S, N), np.float32))
    outs = []
    for _ in range(3):
        Xq, rs = rudder.quant_act(X, sid, inv, None, S, 4, codes)
        outs.append(rudder.linear(Xq, rs, sid, Wq, ws, ca, cb, M, N, K, S, 4, codes).clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))


def test_m0_is_noop_on_device():
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    Y = torch.full((4, 64), 7, dtype=torch.int16, device="cuda")
    dummy = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    f = torch.ones(64, dtype=torch.float32, device="cuda")
    rudder.rudder_linear(dummy, f, dummy, dummy, f, f, f, 0, 64, 128, 1, 8, CODES_INT, Y)
    torch.cuda.synchronize()
    assert int((Y != 7).sum()) == 0


@pytest.mark.parametrize("abits,codes", [(8, CODES_INT), (4, CODES_E2M3)])
def test_linear_row_scales_varying_within_a_stream(abits, codes):
    """rudder_linear takes any row scales: rows of one stream whose scales
    differ (some waves with one stream and one scale, some with one stream
    and several, a -0.0 scale beside +0.0) must match the oracle's
    epilogue on the same integer accumulators."""
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    log(f"case varying row scales abits={abits} codes={codes}")
    rng = np.random.default_rng(500 + abits)
    M, K, N, S = 640, 256, 512, 2
    x = rng.standard_normal((M, K))
    X = _torch_bf16_bits(x)
    Wb = _torch_bf16_bits(rng.standard_normal((K, N)) * 0.02)
    sid = np.zeros(M, np.uint8)
    sid[384:] = 1
    s = np.ones(K, np.float32)
    a = rng.uniform(0.9, 1.1, (S, N)).astype(np.float32)
    b = (rng.standard_normal((S, N)) * 0.01).astype(np.float32)
    b[:, :8] = -0.0
    run = LayerRun(X, sid, Wb, s, a, b, S, abits, codes)
    qa_max = 127 if abits == 8 else 7
    delta = (np.full(S, np.abs(x).max() / qa_max)).astype(np.float32)
    Xq, _ = run.r.quant_act(run.X, run.sid_d, run.inv_smooth, to_dev(delta), S, abits, codes)
    rs = delta[sid].copy()
    rs[130:140] *= np.float32(1.5)       # a wave of one stream, several scales
    rs[200] = np.float32(-0.0)           # -0.0 among +0.0 rows
    rs[201:256] = np.float32(0.0)
    rs[512:] = np.float32(0.75) * rs[512:]
    Y, acc = run.r.linear(Xq, to_dev(rs), run.sid_d, run.Wq, run.w_scale, to_dev(a), to_dev(b),
                          M, N, K, S, abits, codes, acc_out=True)
    torch.cuda.synchronize()
    import oracle
    from gpu_harness import assert_y_close, bf16_to_host_bits
    qa, _ = oracle.quant_act(X, sid, run.o_inv, delta, S, abits)
    o_acc = oracle.int_gemm(qa, run.o_qw)
    o_Y = oracle.epilogue(o_acc, rs, sid, run.o_ws, a, b)
    assert np.array_equal(acc.cpu().numpy(), o_acc)
    log(f"  {assert_y_close('Y', bf16_to_host_bits(Y), o_Y)}")


# ---------------------------------------------------------------------------
# Full-size workloads (the launch configuration the benchmark times), in
# every code container the benchmark can run them in.  Codes and row scales
# are compared in full at every step listed; accumulators and outputs on
# every row at the "full" steps, and on sampled rows (first/last rows, every
# stream boundary, the ragged tail, random rows) at the others.  The two
# containers of one layer are adjacent and share their full step, so the
# oracle runs once for both.
# ---------------------------------------------------------------------------

_C2, _C3 = "attn_proj_h2048_m4192_w4a8", "mlp_h2048_m4192_w4a4"
_C4, _C5 = "dit_block_h2048_m8384_16step", "backbone_h4096_m16576_w4a4"
FULL = [
    # workload, layer, codes, steps with every row, steps with sampled rows
    (_C2, "qkv", CODES_INT, [0], list(range(1, 10))),
    (_C2, "qkv", CODES_E2M3, [0], [9]),
    (_C2, "o", CODES_INT, [0], list(range(1, 10))),
    (_C2, "o", CODES_E2M3, [0], [4]),
    (_C3, "up", CODES_E2M3, [0], list(range(1, 10))),
    (_C3, "up", CODES_INT, [0], [6]),
    (_C3, "down", CODES_E2M3, [0], list(range(1, 10))),
    (_C3, "down", CODES_INT, [0], [3]),
    (_C4, "qkv", CODES_INT, [0], [15]),
    (_C4, "qkv", CODES_E2M3, [0], []),
    (_C4, "o", CODES_INT, [3], [12]),
    (_C4, "o", CODES_E2M3, [3], []),
    (_C4, "up", CODES_E2M3, [2], [7]),
    (_C4, "up", CODES_INT, [2], []),
    (_C4, "down", CODES_E2M3, [9], [15]),
    (_C4, "down", CODES_INT, [9], [0, 11]),
    (_C5, "qkv", CODES_E2M3, [5], [19]),
    (_C5, "qkv", CODES_INT, [5], []),
    (_C5, "o", CODES_E2M3, [19], [0]),
    (_C5, "o", CODES_INT, [19], []),
    (_C5, "up", CODES_E2M3, [4], [11]),
    (_C5, "up", CODES_INT, [4], []),
    (_C5, "down", CODES_E2M3, [13], [8]),
    (_C5, "down", CODES_INT, [13], []),
]

# the inputs of the last (workload, layer), shared by its containers
_INPUTS: dict = {}


def _layer_inputs(workload, layer):
    from w4a4_quantized_gemm_rudder_amd import workloads as W
    key = (workload, layer)
    if _INPUTS.get("key") != key:
        _INPUTS.clear()
        _INPUTS.update(key=key, val=W.make_inputs(workload, seed=0, layers=[layer]))
    return _INPUTS["val"]


@pytest.mark.slow
@pytest.mark.parametrize("workload,layer,codes,full_steps,sampled_steps", FULL)
def test_full_size_layer(workload, layer, codes, full_steps, sampled_steps):
    log(f"case full {workload}/{layer} codes={codes} every row at steps {full_steps}, "
        f"sampled rows at steps {sampled_steps}")
    wi = _layer_inputs(workload, layer)
    L = wi.layers[0]
    run = LayerRun(L.x, wi.stream_id, L.w, L.smooth, L.comp_a, L.comp_b, 3, L.layer.abits,
                   codes)
    run.check_weights()
    rows = sample_rows(wi.stream_id, seed=len(layer))
    for t in full_steps:
        a, b = L.step_comp(t)
        st = run.run_step(L.act_scale[t], a, b, rows=None, label=f"{workload}/{layer}/t{t}",
                          oracle_key=(workload, layer, t))
        log(f"  step {t} (every row): {st}")
    for t in sampled_steps:
        a, b = L.step_comp(t)
        st = run.run_step(L.act_scale[t], a, b, rows=rows, label=f"{workload}/{layer}/t{t}")
        log(f"  step {t}: {st}")
    del run


# ---------------------------------------------------------------------------
# Round-half-to-even ties on the GPU: activations and weights constructed so
# that the scaled value of many elements is exactly k + 1/2 (power-of-two
# step sizes and channel scales, unit smoothing), in every container.
# ---------------------------------------------------------------------------

def _tie_inputs(abits, M=96, K=256, N=64, seed=0):
    rng = np.random.default_rng(300 + seed)
    qa = 127 if abits == 8 else 7
    S = 2
    sid = (np.arange(M) % S).astype(np.uint8)
    delta = np.array([0.25, 1.0], np.float32)                  # exact reciprocals
    # activations: half-integers k + 1/2 (k up to Qa, so +-(Qa + 1/2) clamps),
    # mixed with integers and random values
    half = rng.integers(-qa - 1, qa + 1, (M, K)) + 0.5
    v = np.where(rng.random((M, K)) < 0.7, half, rng.uniform(-qa - 3, qa + 3, (M, K)))
    x = v * delta[sid][:, None].astype(np.float64)
    X = _torch_bf16_bits(x)
    xv = (np.asarray(X, np.uint32) << 16).view(np.float32)
    assert np.mean(np.abs(xv / delta[sid][:, None] % 1.0 - 0.5) == 0) > 0.5  # real ties
    # weights: column n has scale 2^e_n (one entry +-7 * 2^e_n sets the column
    # absmax), the others are half-integer multiples of 2^e_n
    e = rng.integers(-9, -5, N)
    wq = rng.integers(-7, 7, (K, N)) + 0.5
    wq[rng.integers(0, K, N), np.arange(N)] = 7.0 * np.where(rng.random(N) < 0.5, -1, 1)
    Wb = _torch_bf16_bits(wq * 2.0 ** e[None, :])
    s = np.ones(K, np.float32)
    a = rng.uniform(0.9, 1.1, (S, N)).astype(np.float32)
    b = (rng.standard_normal((S, N)) * 0.01).astype(np.float32)
    return X, sid, Wb, s, a, b, delta, S


@pytest.mark.parametrize("abits,codes", [(8, CODES_INT), (4, CODES_INT), (4, CODES_E2M3),
                                         (8, CODES_E2M3)])
def test_round_half_even_ties(abits, codes):
    log(f"case RNE ties abits={abits} codes={codes}")
    X, sid, Wb, s, a, b, delta, S = _tie_inputs(abits)
    run = LayerRun(X, sid, Wb, s, a, b, S, abits, codes)
    run.check_weights()
    # the oracle's codes hold the ties rounded to even (their values are
    # pinned on the CPU); here the GPU must produce the same bytes
    assert np.any(np.abs(run.o_qw) == 2) and np.any(np.abs(run.o_qw) == 6)
    log(f"  {run.run_step(delta, a, b, label='ties')}")
