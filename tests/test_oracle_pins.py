"""Pins for the CPU oracle: checks against closed forms, invariants, brute
force and library routines -- never against the oracle itself.

Passages: "SteerQuant: Steering Quantization Error with Action-Guided Scaling
in World-Action Models" (paperlayer.ai digest) §3.1 (symmetric quantizer),
§4.2 (shared diagonal rescales W and inversely rescales X), §4.3 (per
(stream, step) step sizes), §4.4 (quantize -> low-bit GEMM -> dequantize,
compensation, bias).  The pages print no worked numeric example, so every
pin here is a definition, an invariant, a bound or brute force.
"""
from fractions import Fraction
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def f32(x):
    return np.float32(x)


def bits_of(x_f32: np.ndarray) -> np.ndarray:
    """Exact bf16 bit pattern of fp32 values that are bf16-representable."""
    u = np.ascontiguousarray(x_f32, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def bf16_value(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def torch_bf16_bits(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------------------
# bf16 conversions
# ---------------------------------------------------------------------------

def test_bf16_rne_matches_torch(orc):
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    # force many exact ties and near-ties in the dropped half
    u[:50000] = (u[:50000] & 0xFFFF0000) | 0x8000
    u[50000:60000] = (u[50000:60000] & 0xFFFF0000) | 0x7FFF
    u[60000:70000] = (u[60000:70000] & 0xFFFF0000) | 0x8001
    x = u.view(np.float32)
    finite = np.isfinite(x)
    x = x[finite]
    got = orc.f32_to_bf16(x)
    want = torch_bf16_bits(x)
    # overflow to inf agrees too; compare bit patterns directly
    assert np.array_equal(got, want)


def test_bf16_widen_exact(orc):
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    v = orc.bf16_to_f32(bits)
    import torch
    want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    same = (v.view(np.uint32) == want.view(np.uint32)) | (np.isnan(v) & np.isnan(want))
    assert same.all()


# ---------------------------------------------------------------------------
# Symmetric quantizer: RNE ties, clamp, brute-force nearest code
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("abits,cases", [
    (8, [(2.5, 2), (3.5, 4), (-2.5, -2), (0.5, 0), (-0.5, 0), (1.5, 2), (126.5, 126),
         (127.5, 127), (-127.5, -127), (300.0, 127), (-1048576.0, -127), (0.0, 0)]),
    (4, [(2.5, 2), (3.5, 4), (-3.5, -4), (6.5, 6), (7.5, 7), (8.0, 7), (-8.0, -7),
         (-7.5, -7), (5.5, 6)]),
])
def test_act_quant_constructed_ties(orc, abits, cases):
    # step size 1, smoothing 1: the code is rne(clamp(x)) of the bf16 value x
    x = np.array([[v for v, _ in cases]], np.float32)
    X = bits_of(x)
    sid = np.zeros(1, np.uint8)
    inv = orc.inv_smooth(np.ones(x.shape[1], np.float32))
    codes, rs = orc.quant_act(X, sid, inv, np.array([1.0], np.float32), 1, abits)
    assert codes[0].tolist() == [c for _, c in cases]
    assert rs[0] == 1.0


def _nearest_even_code(v: Fraction, q: int) -> int:
    """Brute force: the integer in [-q, q] nearest to v, ties to the even one."""
    best = None
    for c in range(-q, q + 1):
        d = abs(v - c)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def _near_half(v: Fraction, rel: float) -> bool:
    frac = v - (v.numerator // v.denominator)
    return abs(frac - Fraction(1, 2)) <= Fraction(rel) * (abs(v) + 1)


@pytest.mark.parametrize("abits", [8, 4])
def test_act_quant_brute_force_exact_rationals(orc, abits):
    """Codes equal the nearest integer of the exact real x / s / Delta (ties
    even, clamped), except within a few fp32 ulps of a half-integer where the
    two fp32 products may legitimately round across it."""
    qa = 127 if abits == 8 else 7
    rng = np.random.default_rng(7)
    M, K, S = 6, 16, 3
    X = torch_bf16_bits(rng.standard_normal((M, K)) * 3)
    sid = rng.integers(0, S, M).astype(np.uint8)
    s = (rng.uniform(0.3, 3.0, K)).astype(np.float32)
    inv = orc.inv_smooth(s)
    delta = (rng.uniform(0.5, 2.0, S) * 6.0 / qa).astype(np.float32)
    codes, rs = orc.quant_act(X, sid, inv, delta, S, abits)
    checked = 0
    for m in range(M):
        d = Fraction(float(delta[sid[m]]))
        assert rs[m] == delta[sid[m]]
        for k in range(K):
            v = Fraction(float(bf16_value(X[m, k]))) / Fraction(float(s[k])) / d
            if _near_half(v, 2.0 ** -21):
                continue
            assert codes[m, k] == _nearest_even_code(v, qa), (m, k, float(v))
            checked += 1
    assert checked > M * K * 0.9


def test_weight_quant_brute_force_exact_rationals(orc):
    rng = np.random.default_rng(11)
    K, N = 16, 8
    W = torch_bf16_bits(rng.standard_normal((K, N)) * 0.02)
    s = rng.uniform(0.5, 4.0, K).astype(np.float32)
    codes, ws = orc.quantize_weights(W, s)
    assert codes.shape == (N, K)
    for n in range(N):
        wprime = [Fraction(float(bf16_value(W[k, n]))) * Fraction(float(s[k])) for k in range(K)]
        amax = max(abs(w) for w in wprime)
        # w_scale is amax/7 up to the two roundings (fp32 product, fp64 divide)
        assert abs(Fraction(float(ws[n])) - amax / 7) <= amax / 7 * Fraction(2.0 ** -22)
        for k in range(K):
            v = wprime[k] / Fraction(float(ws[n]))
            if _near_half(v, 2.0 ** -21):
                continue
            assert codes[n, k] == _nearest_even_code(v, 7), (n, k, float(v))
        # the largest-magnitude entry of each column reaches the code limit
        assert np.abs(codes[n]).max() == 7


@pytest.mark.parametrize("abits", [8, 4])
def test_act_quant_half_step_roundtrip(orc, abits):
    qa = 127 if abits == 8 else 7
    rng = np.random.default_rng(3)
    M, K, S = 64, 96, 3
    X = torch_bf16_bits(rng.standard_t(4, (M, K)))
    sid = rng.integers(0, S, M).astype(np.uint8)
    s = rng.uniform(0.2, 5, K).astype(np.float32)
    inv = orc.inv_smooth(s)
    delta = np.array([0.02, 0.05, 0.3], np.float32) * (127 / qa)
    codes, rs = orc.quant_act(X, sid, inv, delta, S, abits)
    u = bf16_value(X) / s.astype(np.float64)[None, :]
    D = delta.astype(np.float64)[sid][:, None]
    v = u / D
    q = codes.astype(np.float64)
    clipped = np.abs(q) == qa
    inner = ~clipped
    assert np.all(np.abs(u - q * D)[inner] <= D.repeat(K, 1)[inner] / 2 * (1 + 2.0 ** -20))
    # clipped codes carry the sign of v and |v| is at least Qa - 1/2
    assert np.all(np.sign(q[clipped]) == np.sign(v[clipped]))
    assert np.all(np.abs(v[clipped]) >= qa - 0.5 - 1e-5)
    assert np.abs(codes).max() <= qa


def test_weight_quant_half_step_roundtrip(orc):
    rng = np.random.default_rng(5)
    K, N = 128, 64
    W = torch_bf16_bits(rng.standard_normal((K, N)) * 0.02)
    s = rng.uniform(0.2, 5, K).astype(np.float32)
    codes, ws = orc.quantize_weights(W, s)
    wp = bf16_value(W) * s.astype(np.float64)[:, None]          # [K, N]
    err = np.abs(wp - codes.T.astype(np.float64) * ws.astype(np.float64)[None, :])
    assert np.all(err <= ws.astype(np.float64)[None, :] / 2 * (1 + 2.0 ** -20) + 1e-30)
    assert np.all(np.abs(codes).max(axis=1) == 7)
    assert codes.min() >= -7


def test_weight_quant_zero_column(orc):
    W = np.zeros((8, 2), np.uint16)
    W[:, 1] = bits_of(np.arange(1, 9, dtype=np.float32))
    codes, ws = orc.quantize_weights(W, np.ones(8, np.float32))
    assert ws[0] == 0 and np.all(codes[0] == 0)
    assert ws[1] == np.float32(8.0 / 7.0)


# ---------------------------------------------------------------------------
# Dynamic (absmax) step sizes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("abits", [8, 4])
def test_dynamic_scales_reach_code_limit(orc, abits):
    qa = 127 if abits == 8 else 7
    rng = np.random.default_rng(9)
    M, K, S = 40, 64, 4
    X = torch_bf16_bits(rng.standard_normal((M, K)))
    sid = np.array([0] * 20 + [1] * 12 + [3] * 8, np.uint8)     # stream 2 empty
    s = rng.uniform(0.5, 2, K).astype(np.float32)
    inv = orc.inv_smooth(s)
    delta = orc.dynamic_scales(X, sid, inv, S, abits)
    assert delta[2] == 0.0
    u = np.abs(bf16_value(X) * inv.astype(np.float64)[None, :])
    for st in (0, 1, 3):
        amax = u[sid == st].max()
        assert abs(float(delta[st]) * qa - amax) <= amax * 2.0 ** -22
    codes, _ = orc.quant_act(X, sid, inv, delta, S, abits)
    for st in (0, 1, 3):
        assert np.abs(codes[sid == st]).max() == qa


# ---------------------------------------------------------------------------
# Integer GEMM: brute force with Python ints
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(40))
def test_int_gemm_brute_force(orc, seed):
    rng = np.random.default_rng(100 + seed)
    M, N, K = 4, 8, 8
    qa_lim = 127 if seed % 2 == 0 else 7
    a = rng.integers(-qa_lim, qa_lim + 1, (M, K)).astype(np.int8)
    w = rng.integers(-7, 8, (N, K)).astype(np.int8)
    if seed % 5 == 0:   # extremes
        a[:] = qa_lim * (1 if seed % 10 == 0 else -1)
        w[:] = 7
    acc = orc.int_gemm(a, w)
    for m in range(M):
        for n in range(N):
            assert acc[m, n] == sum(int(a[m, k]) * int(w[n, k]) for k in range(K))


def test_int_gemm_long_k_brute_force(orc):
    rng = np.random.default_rng(2)
    M, N, K = 3, 5, 5000     # crosses the 1024-long partial-sum chunks, ragged
    a = rng.integers(-127, 128, (M, K)).astype(np.int8)
    w = rng.integers(-7, 8, (N, K)).astype(np.int8)
    acc = orc.int_gemm(a, w)
    A = a.astype(object)
    Wt = w.astype(object)
    for m in range(M):
        for n in range(N):
            assert acc[m, n] == int((A[m] * Wt[n]).sum())


def test_int_gemm_overflow_detected(orc):
    K = 140000
    a = np.full((1, K), 127, np.int8)
    w = np.full((1, K), 127, np.int8)
    with pytest.raises(orc.OracleError):
        orc.int_gemm(a, w)


# ---------------------------------------------------------------------------
# Epilogue
# ---------------------------------------------------------------------------

def test_epilogue_a0_gives_bias(orc):
    rng = np.random.default_rng(4)
    M, N, S = 5, 7, 3
    acc = rng.integers(-10**6, 10**6, (M, N)).astype(np.int32)
    sid = np.array([0, 1, 2, 1, 0], np.uint8)
    b = rng.standard_normal((S, N)).astype(np.float32)
    Y = orc.epilogue(acc, rng.uniform(0.01, 1, M).astype(np.float32), sid,
                     rng.uniform(0.01, 1, N).astype(np.float32), np.zeros((S, N), np.float32), b)
    assert np.array_equal(Y, torch_bf16_bits(b[sid]))


def test_epilogue_power_of_two_scales_exact(orc):
    rng = np.random.default_rng(6)
    M, N, S = 6, 9, 2
    acc = rng.integers(-2**20, 2**20, (M, N)).astype(np.int32)
    sid = rng.integers(0, S, M).astype(np.uint8)
    rs = (2.0 ** rng.integers(-8, 0, M)).astype(np.float32)
    ws = (2.0 ** rng.integers(-10, -2, N)).astype(np.float32)
    Y = orc.epilogue(acc, rs, sid, ws, np.ones((S, N), np.float32), np.zeros((S, N), np.float32))
    exact = acc.astype(np.float64) * rs[:, None].astype(np.float64) * ws[None, :].astype(np.float64)
    assert np.array_equal(Y, torch_bf16_bits(exact.astype(np.float32)))


def test_epilogue_fp64_bound(orc):
    rng = np.random.default_rng(8)
    M, N, S = 64, 48, 3
    acc = rng.integers(-2 * 10**6, 2 * 10**6, (M, N)).astype(np.int32)
    sid = rng.integers(0, S, M).astype(np.uint8)
    rs = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    a = rng.uniform(0.9, 1.1, (S, N)).astype(np.float32)
    b = (rng.standard_normal((S, N)) * 0.01).astype(np.float32)
    Y = bf16_value(orc.epilogue(acc, rs, sid, ws, a, b))
    at = a[sid].astype(np.float64) * acc * rs[:, None].astype(np.float64) * ws[None, :]
    ref = at + b[sid].astype(np.float64)
    # bf16 rounding (half ulp = 2^-9 relative) + three fp32 roundings
    bound = np.abs(ref) * 2.0 ** -8 + np.abs(at) * 2.0 ** -21
    assert np.all(np.abs(Y - ref) <= bound)


# Exact-rational reference of the epilogue ("SteerQuant" digest §4.4:
# dequantization, then inverse-gain compensation and bias; the compensation
# is one fp32 multiply-add).  Every value is held as an exact rational
# (integer numerator, power-of-two denominator) and rounded to fp32 only where
# the stated arithmetic rounds:
#   d = RNE32(rs * ws);  t = RNE32(f * d);  y = RNE32(a * t + b)  (one rounding)
# then Y = bf16 RNE (torch's cast).  Nothing here calls the oracle.

def _ratio(x):
    """fp32/fp64 value -> (numerator, denominator) exactly."""
    return float(x).as_integer_ratio()


def _rne_f32(num, den):
    """Round num/den (den a power of two) to the nearest fp32, ties to even
    (normal range; the epilogue's values never leave it)."""
    if num == 0:
        return 0.0
    neg = num < 0
    mag = -num if neg else num
    # scale so that the quotient has 24 bits before the point
    sh = 24 - (mag.bit_length() - (den.bit_length() - 1))
    # value * 2^sh has its leading bit at position 23 or 24
    q_num = mag << sh if sh >= 0 else mag
    q_den = den if sh >= 0 else den << (-sh)
    q, r = divmod(q_num, q_den)
    if q >= 1 << 24:                       # leading bit landed at 24: one less bit
        sh -= 1
        q_num = mag << sh if sh >= 0 else mag
        q_den = den if sh >= 0 else den << (-sh)
        q, r = divmod(q_num, q_den)
    assert (1 << 23) <= q < (1 << 24)
    if 2 * r > q_den or (2 * r == q_den and (q & 1)):
        q += 1
    val = float(q) * 2.0 ** (-sh)
    assert np.isfinite(val) and abs(val) >= 2.0 ** -126
    return -val if neg else val


def _mul_exact(x, y):
    (n1, d1), (n2, d2) = _ratio(x), _ratio(y)
    return n1 * n2, d1 * d2


def _fma_exact(a, t, b):
    n1, d1 = _mul_exact(a, t)
    n2, d2 = _ratio(b)
    d = max(d1, d2)
    return n1 * (d // d1) + n2 * (d // d2), d


def _epilogue_ref(f, rs, ws, a, b, form="fused"):
    """fp32 y of one output element.  form: "fused" (the stated arithmetic),
    "unfused" (a * t rounded before + b) or "reassoc" ((f * rs) * ws)."""
    if form == "reassoc":
        t = _rne_f32(*_mul_exact(_rne_f32(*_mul_exact(f, rs)), ws))
    else:
        t = _rne_f32(*_mul_exact(f, _rne_f32(*_mul_exact(rs, ws))))
    if form == "unfused":
        p = _rne_f32(*_mul_exact(a, t))
        n1, d1 = _ratio(p)
        n2, d2 = _ratio(b)
        d = max(d1, d2)
        return _rne_f32(n1 * (d // d1) + n2 * (d // d2), d)
    return _rne_f32(*_fma_exact(a, t, b))


def _bf16_of(y):
    return int(torch_bf16_bits(np.asarray([y], np.float32))[0])


def test_exact_rational_reference_selfcheck():
    """The rational rounding helper agrees with the correctly rounded fp64 ->
    fp32 conversion wherever fp64 holds the value exactly (products of two
    fp32 values), including constructed ties."""
    rng = np.random.default_rng(40)
    x = rng.uniform(-1e3, 1e3, 4000).astype(np.float32)
    y = rng.uniform(-1e-2, 1e-2, 4000).astype(np.float32)
    prod = x.astype(np.float64) * y.astype(np.float64)          # exact in fp64
    want = prod.astype(np.float32)
    got = np.array([_rne_f32(*_mul_exact(u, v)) for u, v in zip(x, y)], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # ties: 1 + 2^-24 -> 1 (even), 1 + 3 * 2^-24 -> 1 + 2^-22 (even), and negatives
    for num, den, v in (((1 << 24) + 1, 1 << 24, 1.0),
                        ((1 << 24) + 3, 1 << 24, 1.0 + 2.0 ** -22),
                        (-((1 << 24) + 1), 1 << 24, -1.0)):
        assert _rne_f32(num, den) == v


def _epilogue_random_inputs(rng, M, N, S):
    acc = rng.integers(-2 * 10**6, 2 * 10**6, (M, N)).astype(np.int32)
    acc[rng.random((M, N)) < 0.05] = 0
    sid = rng.integers(0, S, M).astype(np.uint8)
    rs = rng.uniform(1e-4, 1e-1, M).astype(np.float32)
    ws = rng.uniform(1e-5, 1e-2, N).astype(np.float32)
    a = rng.uniform(0.9, 1.1, (S, N)).astype(np.float32)
    b = (rng.standard_normal((S, N)) * rng.choice([1e-3, 1e-2, 1.0], (S, N))).astype(np.float32)
    return acc, sid, rs, ws, a, b


def test_epilogue_exact_rational_random(orc):
    """Over 10^5 random outputs the oracle equals the exact-rational
    reference bit for bit."""
    rng = np.random.default_rng(41)
    M, N, S = 400, 256, 3
    acc, sid, rs, ws, a, b = _epilogue_random_inputs(rng, M, N, S)
    Y = orc.epilogue(acc, rs, sid, ws, a, b)
    y = np.empty((M, N), np.float64)
    for m in range(M):
        s = sid[m]
        for n in range(N):
            y[m, n] = _epilogue_ref(int(acc[m, n]), rs[m], ws[n], a[s, n], b[s, n])
    assert np.array_equal(Y, torch_bf16_bits(y.astype(np.float32)))


def _constructed_fma_cases(rng, count):
    """Cancellation cases: b = -RNE32(a*t) + k*ulp32(a*t) for a small k, so
    that the exact a*t + b is k*ulp minus the low bits of the exact product.
    Rounding a*t before adding b drops exactly those bits (the unfused form
    gives k*ulp), the single-rounding form keeps them."""
    cases = []
    while len(cases) < count:
        f = int(rng.integers(1, 1 << 21))
        rs = np.float32(rng.uniform(1e-3, 1e-1))
        ws = np.float32(rng.uniform(1e-4, 1e-2))
        a = np.float32(rng.uniform(0.9, 1.1))
        t = _rne_f32(*_mul_exact(f, _rne_f32(*_mul_exact(rs, ws))))
        p32 = _rne_f32(*_mul_exact(a, t))
        ulp = 2.0 ** (np.floor(np.log2(abs(p32))) - 23)
        k = int(rng.integers(-3, 4))
        b = np.float32(-p32 + k * ulp)
        assert float(b) == -p32 + k * ulp               # exact by construction
        cases.append((f, rs, ws, a, b))
    return cases


def _constructed_assoc_cases(rng, count):
    """f * rs * ws placed on a bf16 rounding midpoint (9 significant bits),
    so that the one-ulp difference between RNE32(f * RNE32(rs * ws)) and
    RNE32(RNE32(f * rs) * ws) can decide the bf16 output (a = 1, b = 0)."""
    cases = []
    while len(cases) < count:
        f = int(rng.integers(1, 1 << 21))
        rs = np.float32(rng.uniform(1e-3, 1e-1))
        e = int(rng.integers(-12, -2))
        mid = (int(rng.integers(128, 256)) + 0.5) * 2.0 ** e
        ws = np.float32(mid / (f * float(rs)))
        cases.append((f, rs, ws, np.float32(1.0), np.float32(0.0)))
    return cases


def _discriminating(cases, other):
    keep = []
    for c in cases:
        ref = _bf16_of(_epilogue_ref(*c))
        alt = _bf16_of(_epilogue_ref(*c, form=other))
        if ref != alt:
            keep.append(c)
    return keep


@pytest.mark.parametrize("other,make", [("unfused", _constructed_fma_cases),
                                        ("reassoc", _constructed_assoc_cases)])
def test_epilogue_form_and_order_pinned(orc, other, make):
    """Constructed cases on which the single-rounding fma form (resp. the
    order f * (rs * ws)) and the plausible alternative -- a * t rounded
    before adding b, resp. (f * rs) * ws -- give different bf16 outputs.  The
    oracle must give the stated form's output on every one of them, so either
    mistake fails this test."""
    rng = np.random.default_rng(42 if other == "unfused" else 43)
    cases = _discriminating(make(rng, 6000), other)
    assert len(cases) >= 500, f"only {len(cases)} discriminating cases"
    cases = cases[:1000]
    # one call: case i is row i (its own step size and stream) and channel i
    # (its own channel scale and compensation); only the diagonal is used
    n = len(cases)
    acc = np.zeros((n, n), np.int32)
    acc[np.arange(n), np.arange(n)] = [c[0] for c in cases]
    rs = np.array([c[1] for c in cases], np.float32)
    ws = np.array([c[2] for c in cases], np.float32)
    a = np.array([[c[3] for c in cases]], np.float32)
    b = np.array([[c[4] for c in cases]], np.float32)
    Y = np.diagonal(orc.epilogue(acc, rs, np.zeros(n, np.uint8), ws, a, b)).copy()
    want = np.array([_bf16_of(_epilogue_ref(*c)) for c in cases], np.uint16)
    alt = np.array([_bf16_of(_epilogue_ref(*c, form=other)) for c in cases], np.uint16)
    assert np.array_equal(Y, want)
    assert not np.any(Y == alt)


# ---------------------------------------------------------------------------
# Whole chain
# ---------------------------------------------------------------------------

def _exact_chain_inputs(rng, M, K, N, qa, S):
    """Inputs on which every quantization step is lossless: s_k, Delta and the
    column scales are powers of two, X = code * s * Delta, W = code * c / s."""
    s = (2.0 ** rng.integers(-2, 3, K)).astype(np.float32)
    delta = (2.0 ** rng.integers(-4, -1, S)).astype(np.float32)
    sid = rng.integers(0, S, M).astype(np.uint8)
    qx = rng.integers(-qa, qa + 1, (M, K))
    qx[np.arange(M), rng.integers(0, K, M)] = qa          # not needed, keeps range full
    X = qx * s[None, :].astype(np.float64) * delta[sid][:, None].astype(np.float64)
    c = (2.0 ** rng.integers(-9, -5, N))
    qw = rng.integers(-7, 8, (K, N))
    qw[rng.integers(0, K, N), np.arange(N)] = 7           # each column reaches |code| = 7
    W = qw * c[None, :] / s[:, None].astype(np.float64)
    return (bits_of(X.astype(np.float32)), sid, s, delta, bits_of(W.astype(np.float32)),
            qx, qw, c)


@pytest.mark.parametrize("abits", [8, 4])
def test_chain_reduces_to_textbook_gemm(orc, abits):
    """With lossless quantization the layer is Y = bf16(X @ W) exactly
    (SteerQuant §4.2: the diagonal leaves the product unchanged)."""
    qa = 127 if abits == 8 else 7
    rng = np.random.default_rng(21 + abits)
    M, K, N, S = 12, 32, 16, 3
    X, sid, s, delta, W, qx, qw, c = _exact_chain_inputs(rng, M, K, N, qa, S)
    inv = orc.inv_smooth(s)
    codes_w, ws = orc.quantize_weights(W, s)
    assert np.array_equal(codes_w, qw.T)
    assert np.array_equal(ws, c.astype(np.float32))
    ones, zeros = np.ones((S, N), np.float32), np.zeros((S, N), np.float32)
    qa_codes, rs, acc, Y = orc.linear(X, sid, codes_w, ws, inv, delta, ones, zeros, S, abits)
    assert np.array_equal(qa_codes, qx)
    xw = bf16_value(X) @ bf16_value(W)                     # fp64, exact here
    assert np.array_equal(Y, torch_bf16_bits(xw.astype(np.float32)))


def test_smoothing_direction_fp64_identity(orc):
    """(X diag(s)^-1)(diag(s) W) = X W in fp64, and the oracle's layer output
    approximates X W within the quantization error bound; a flipped diagonal
    (X diag(s), W / s) breaks the bound for these strongly non-uniform s."""
    rng = np.random.default_rng(31)
    M, K, N, S = 4, 8, 8, 1
    x = rng.standard_normal((M, K))
    x[:, 3] *= 40.0                                      # an outlier channel
    X = torch_bf16_bits(x)
    W = torch_bf16_bits(rng.standard_normal((K, N)) * 0.02)
    Xd, Wd = bf16_value(X), bf16_value(W)
    s = np.sqrt(np.abs(Xd).max(0) / np.abs(Wd).max(1)).astype(np.float32)
    sd = s.astype(np.float64)
    ident = (Xd / sd[None, :]) @ (sd[:, None] * Wd)
    assert np.allclose(ident, Xd @ Wd, rtol=1e-12, atol=1e-14)

    inv = orc.inv_smooth(s)
    codes_w, ws = orc.quantize_weights(W, s)
    delta = orc.dynamic_scales(X, np.zeros(M, np.uint8), inv, S, 8)
    ones, zeros = np.ones((S, N), np.float32), np.zeros((S, N), np.float32)
    qa_codes, rs, acc, Y = orc.linear(X, np.zeros(M, np.uint8), codes_w, ws, inv, delta,
                                      ones, zeros, S, 8)
    ref = Xd @ Wd
    u = Xd / sd[None, :]
    wp = sd[:, None] * Wd
    # |Y - XW| <= sum_k (D/2 |w'_k| + |u_k| ws/2) + bf16 rounding of Y
    bound = (delta[0] / 2 * np.abs(wp).sum(0)[None, :]
             + np.abs(u) @ (np.ones((K, N)) * ws[None, :] / 2))
    bound = bound * (1 + 1e-5) + np.abs(ref) * 2.0 ** -8 + 1e-7
    assert np.all(np.abs(bf16_value(Y) - ref) <= bound)


def test_stream_invariants(orc):
    rng = np.random.default_rng(41)
    M, K, N, S = 24, 64, 16, 3
    X = torch_bf16_bits(rng.standard_normal((M, K)))
    W = torch_bf16_bits(rng.standard_normal((K, N)) * 0.02)
    s = rng.uniform(0.5, 2, K).astype(np.float32)
    sid = rng.integers(0, S, M).astype(np.uint8)
    inv = orc.inv_smooth(s)
    cw, ws = orc.quantize_weights(W, s)
    delta = np.array([0.02, 0.03, 0.05], np.float32)
    a = rng.uniform(0.9, 1.1, (S, N)).astype(np.float32)
    b = (rng.standard_normal((S, N)) * 0.01).astype(np.float32)
    _, _, _, Y = orc.linear(X, sid, cw, ws, inv, delta, a, b, S, 8)
    # 1. permuting rows together with their tags permutes Y
    p = rng.permutation(M)
    _, _, _, Yp = orc.linear(X[p], sid[p], cw, ws, inv, delta, a, b, S, 8)
    assert np.array_equal(Yp, Y[p])
    # 2. changing stream 2's step size leaves rows of streams 0 and 1 unchanged
    d2 = delta.copy()
    d2[2] *= 1.7
    _, _, _, Y2 = orc.linear(X, sid, cw, ws, inv, d2, a, b, S, 8)
    keep = sid != 2
    assert np.array_equal(Y2[keep], Y[keep])
    assert not np.array_equal(Y2[~keep], Y[~keep])
    # 3. scaling X and every step size by 2^e leaves the codes unchanged
    Xs = torch_bf16_bits(bf16_value(X) * 8.0)
    c0, _ = orc.quant_act(X, sid, inv, delta, S, 8)
    c1, _ = orc.quant_act(Xs, sid, inv, delta * 8, S, 8)
    assert np.array_equal(c0, c1)
    # 4. compensation of stream s only touches rows of stream s
    a2 = a.copy()
    a2[1] *= 1.05
    _, _, _, Y3 = orc.linear(X, sid, cw, ws, inv, delta, a2, b, S, 8)
    assert np.array_equal(Y3[sid != 1], Y[sid != 1])


def test_zero_step_size_gives_bias(orc):
    rng = np.random.default_rng(51)
    M, K, N, S = 6, 16, 8, 2
    X = torch_bf16_bits(rng.standard_normal((M, K)))
    sid = np.array([0, 1, 0, 1, 1, 0], np.uint8)
    inv = orc.inv_smooth(np.ones(K, np.float32))
    cw, ws = orc.quantize_weights(torch_bf16_bits(rng.standard_normal((K, N))), np.ones(K, np.float32))
    delta = np.array([0.0, 0.01], np.float32)
    a = np.ones((S, N), np.float32)
    b = rng.standard_normal((S, N)).astype(np.float32)
    codes, rs, acc, Y = orc.linear(X, sid, cw, ws, inv, delta, a, b, S, 8)
    assert np.all(codes[sid == 0] == 0) and np.all(rs[sid == 0] == 0)
    assert np.array_equal(Y[sid == 0], torch_bf16_bits(b[sid[sid == 0]]))


def test_non_finite_rejected(orc):
    X = bits_of(np.array([[1.0, np.inf]], np.float32))
    with pytest.raises(orc.OracleError):
        orc.quant_act(X, np.zeros(1, np.uint8), np.ones(2, np.float32),
                      np.array([1.0], np.float32), 1, 8)
    with pytest.raises(orc.OracleError):
        orc.quant_act(bits_of(np.ones((1, 2), np.float32)), np.array([3], np.uint8),
                      np.ones(2, np.float32), np.array([1.0], np.float32), 1, 8)


# ---------------------------------------------------------------------------
# Packing
# ---------------------------------------------------------------------------

def _golden_pack_rows():
    path = os.path.join(ROOT, "tests", "golden", "pack_int4_pairs.txt")
    rows = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        codes, packed = line.split("|")
        rows.append(([int(c) for c in codes.split(",")],
                     [int(h, 16) for h in packed.split()]))
    return rows


@pytest.mark.parametrize("codes,packed", _golden_pack_rows())
def test_pack_golden(orc, codes, packed):
    c = np.array([codes], np.int8)
    got = orc.pack_int4(c)
    assert got[0].tolist() == packed
    assert np.array_equal(orc.unpack_int4(got, len(codes)), c)


def test_pack_roundtrip_random(orc):
    rng = np.random.default_rng(12)
    c = rng.integers(-8, 8, (33, 256)).astype(np.int8)
    assert np.array_equal(orc.unpack_int4(orc.pack_int4(c), 256), c)


def test_pack_nibble_positions(orc):
    """Each code lands in the nibble its index names: code k of a row is
    nibble k % 2 of byte k // 2 (placed one at a time, all others zero)."""
    K = 16
    for k in range(K):
        for v in (-8, -1, 1, 7):
            c = np.zeros((1, K), np.int8)
            c[0, k] = v
            got = orc.pack_int4(c)[0]
            want = np.zeros(K // 2, np.uint8)
            want[k // 2] = (v & 0xF) << (4 * (k % 2))
            assert np.array_equal(got, want), (k, v)


# ---------------------------------------------------------------------------
# GELU between the MLP projections (kept in BF16: SteerQuant App. D), for the
# fused up-projection -> GELU -> down-layer quantizer path
# ---------------------------------------------------------------------------

def _all_bf16():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_gelu_matches_scipy_every_finite_input(orc):
    """An independent erfc (scipy's) in fp64 gives the same bf16 result for
    every finite bf16 input."""
    from scipy.special import erfc
    b = _all_bf16()
    x = orc.bf16_to_f32(b).astype(np.float64)
    fin = np.isfinite(x)
    g64 = 0.5 * x[fin] * erfc(-x[fin] / np.sqrt(2.0))
    ref = orc.f32_to_bf16(g64.astype(np.float32))
    got = orc.gelu_bf16(b)[fin]
    assert np.array_equal(got, ref), int((got != ref).sum())


def test_gelu_closed_form_values(orc):
    """gelu(x) = x * Phi(x) at points where Phi has textbook values."""
    phi = {1.0: 0.8413447460685429, 2.0: 0.9772498680518208, 0.5: 0.6914624612740131}
    for x, p in phi.items():
        for sx in (x, -x):
            want = sx * (p if sx > 0 else 1.0 - p)
            wb = orc.f32_to_bf16(np.array([want], np.float32))
            got = orc.gelu_bf16(orc.f32_to_bf16(np.array([sx], np.float32)))
            assert got[0] == wb[0], (sx, hex(int(got[0])), hex(int(wb[0])))


def test_gelu_odd_identity(orc):
    """gelu(x) - gelu(-x) = x exactly; after the two bf16 roundings the
    difference stays within half an ulp of each output."""
    b = _all_bf16()
    x = orc.bf16_to_f32(b).astype(np.float64)
    sel = np.isfinite(x) & (np.abs(x) > 1e-30) & (np.abs(x) < 1e30)
    bx = b[sel]
    gp = orc.bf16_to_f32(orc.gelu_bf16(bx)).astype(np.float64)
    gm = orc.bf16_to_f32(orc.gelu_bf16(bx ^ np.uint16(0x8000))).astype(np.float64)
    xx = x[sel]

    def half_ulp(v):
        e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
        return 2.0 ** (e - 8)
    assert np.all(np.abs(gp - gm - xx) <= half_ulp(gp) + half_ulp(gm) + 1e-300)


def test_gelu_tails_and_special_values(orc):
    b = _all_bf16()
    x = orc.bf16_to_f32(b).astype(np.float64)
    g = orc.gelu_bf16(b)
    gv = orc.bf16_to_f32(g).astype(np.float64)
    fin = np.isfinite(x)
    # large positive inputs pass through unchanged (x * Q(x) < half an ulp)
    big = fin & (x >= 4.0)
    assert np.array_equal(g[big], b[big])
    # negative inputs give non-positive outputs, bounded below by the minimum
    # of x * Phi(x) (about -0.17 near x = -0.75)
    neg = fin & (x < 0)
    assert np.all(gv[neg] <= 0) and np.all(gv[neg] >= -0.1702)
    # zeros keep their sign; far negative inputs underflow to -0
    assert orc.gelu_bf16(np.array([0x0000, 0x8000], np.uint16)).tolist() == [0x0000, 0x8000]
    far = fin & (x < -14.0)
    assert np.all(g[far] == 0x8000)
    # non-finite inputs
    sp = orc.gelu_bf16(np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1], np.uint16)).tolist()
    assert sp == [0x7F80, 0x8000, 0x7FC0, 0xFFC0]


def test_linear_gelu_quant_is_the_composition(orc):
    """The fused reference is the unfused chain: the layer's bf16 output,
    GELU, then the next layer's quantizer on it (each piece pinned above)."""
    rng = np.random.default_rng(31)
    M, K, N, S = 40, 64, 96, 3
    X = orc.f32_to_bf16(rng.standard_normal((M, K)).astype(np.float32))
    W = orc.f32_to_bf16((rng.standard_normal((K, N)) * 0.05).astype(np.float32))
    s = rng.uniform(0.5, 2.0, K).astype(np.float32)
    sid = (np.arange(M) % S).astype(np.uint8)
    inv = orc.inv_smooth(s)
    qw, ws = orc.quantize_weights(W, s)
    delta = np.array([0.02, 0.03, 0.025], np.float32)
    a = rng.uniform(0.9, 1.1, (S, N)).astype(np.float32)
    bb = (rng.standard_normal((S, N)) * 0.01).astype(np.float32)
    ninv = rng.uniform(0.5, 2.0, N).astype(np.float32)
    nd = np.array([0.01, 0.02, 0.015], np.float32)
    q2, rs2 = orc.linear_gelu_quant(X, sid, qw, ws, inv, delta, a, bb, S, 8, ninv, nd, 4)
    _, _, _, Y = orc.linear(X, sid, qw, ws, inv, delta, a, bb, S, 8)
    G = orc.gelu_bf16(Y)
    # the next quantizer, written out from its definition
    u = orc.bf16_to_f32(G) * ninv[None, :]
    ia = np.array([np.float32(1.0 / np.float64(d)) for d in nd], np.float32)
    v = (u * ia[sid][:, None]).astype(np.float32)
    want = np.rint(np.clip(v, -7, 7)).astype(np.int8)
    assert np.array_equal(q2, want)
    assert np.array_equal(rs2, nd[sid])
