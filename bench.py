"""Benchmark of the stream-aware W4A8/W4A4 linear on one MI355X.

A step is one denoising step's quantized linear set of a DiT block at
hidden 2048 over 2 rollouts x 4192 tokens (8384 rows: 8192 video, 64
proprio, 128 action): QKV 2048->6144 and O 2048->2048 at W4A8, MLP up
2048->8192 and down 8192->2048 at W4A4.  Each linear is one
rudder_quant_act (fused smoothing + per-(stream, step) quantization) and one
rudder_linear (int8-MFMA GEMM + fused dequant/compensation epilogue), i.e. 8
launches per step (the W4A4 linears hold their 4-bit codes as FP6 E2M3 by
default, see --w4a4-codes); the step index cycles through the 16-step denoise loop,
selecting that step's activation step sizes and compensation vectors
(SteerQuant §4.3 layer-step table, §4.4 Rudder).  Weights are prepared once
before timing (offline preparation, SteerQuant Fig. 2).  All inputs are
seeded synthetic tensors already resident in HBM.

Prints ONE JSON line.  `value` is whole-step throughput in TOPS (2*M*N*K
summed over the four linears, per second, both kernels of each linear
included); `us_per_step` is the mean latency of one step, timed over K steps
with nothing but the step's launches on the stream, after W untimed steps
(defaults: 20 timed steps after 5 warm-up steps, the latency protocol of the
SteerQuant digest's efficiency appendix).  The same K steps then run twice
more: once with an event at every step boundary (`step_us`: median, p10,
p90), and once with an event triple around every linear on the launch stream
(`us_per_step_with_kernel_events`: the records add gaps between launches).
Those events give `per_call` (every linear's GEMM and quantize+GEMM time,
median / p10 / p90), `gemm_kernels` and `roofline`, which describes the kernel
that takes the most time per step.  `large_gemms` runs the hidden-4096
backbone's linears (the largest W4A4 GEMMs) the same way.  `mfma_ceiling` is
the MFMA-only rate on this workload's own codes (the part's clock depends on
operand bit activity).  `cpu_baseline` times the CPU oracle on a bounded
sample of the same step (1 warm-up + 3 timed runs, median).  `mlp_chained`
times the same step with the MLP chained as in a DiT block (the down layer's
input is GELU, kept in BF16, of the up-projection's output): unfused (bf16
output, GELU kernel, quantizer) and fused (rudder_linear_gelu_quant).
`small_m` reports action/proprio-sized calls (96 and 192 rows against
full-width weights) as achieved HBM GB/s, timed as graph replays over
rotating buffer sets that exceed the memory-side cache (and, for context, on
one cache-resident set), beside a plain device copy that moves the same
bytes the same way.  `calibration` times the offline search of one
layer's diagonal and layer-step table with the GPU in the loop.

--workload picks another workload (each printed as one JSON line of the
same form, steps cycling through its step-indexed scale sets).
--w4a4-codes picks the code container of the W4A4 linears: "e2m3" (default:
the 4-bit codes held as FP6 E2M3 for the f8f6f4 matrix cores, fp32
accumulation, exact for integer codes) or "int" (int4 codes widened to int8
for the int8 matrix cores).  Outputs are identical either way.
--w4a8-codes does the same for the W4A8 linears: "int" (int8 codes, int8
matrix cores) or "e2m3" (each int8 code as two E2M3 digit planes, two f8f6f4
MFMAs per product).
Comparators (context only): torch.matmul in bf16 and torch._int_mm (hipBLASLt
int8 GEMM, no quantization or epilogue) on the same shapes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("fused W4A8/W4A4 linear TOPS and % int8-MFMA peak; "
          "µs per denoising-step layer set")
INT8_PEAK_TOPS = 5000.0          # MI355X dense int8 MFMA, published
FP6_PEAK_TFLOPS = 10100.0        # MI355X dense fp6/fp4 MFMA, published
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
DEFAULT_WORKLOAD = "dit_block_h2048_m8384_16step"
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["w4a4_quantized_gemm_rudder_amd/csrc/w4_gemm.hip",
                  "w4a4_quantized_gemm_rudder_amd/csrc/quantize.hip",
                  "w4a4_quantized_gemm_rudder_amd/csrc/rudder_internal.h"]


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: line comments and blank lines are
    dropped, so a comment edit does not void counters taken on the same
    kernels (the sources use no block comments)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    # 20 timed steps after 5 warm-up steps, as in the pages' latency
    # protocol.  The part's clocks settle under sustained load only after some
    # tens of milliseconds; --warmup 100 gives the steady state of a long
    # denoising loop.
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--w4a4-codes", choices=["int", "e2m3"], default="e2m3",
                   help="code container of the W4A4 linears (identical outputs)")
    p.add_argument("--w4a8-codes", choices=["int", "e2m3"], default="int",
                   help="code container of the W4A8 linears (identical outputs)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-small-m", action="store_true",
                   help="skip the few-row (weight-streaming) calls")
    p.add_argument("--no-chained", action="store_true",
                   help="skip the chained-MLP (unfused / fused GELU + quantize) timing")
    p.add_argument("--no-large", action="store_true",
                   help="skip the per-call timing of the hidden-4096 backbone's linears")
    p.add_argument("--no-calibration", action="store_true",
                   help="skip the offline-calibration timing")
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the MFMA-only ceiling on this workload's codes")
    p.add_argument("--no-bf16", action="store_true",
                   help="skip the library comparators (bf16 matmul, int8 GEMM)")
    p.add_argument("--cpu-rows", type=int, default=8384,
                   help="rows per linear in the CPU-oracle sample")
    p.add_argument("--cpu-step", type=int, default=0,
                   help="denoising step whose scale set the CPU-oracle sample uses")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="before warmup, run a plain device copy of this many bytes three "
                        "times (a known-size reference for HBM byte counters)")
    return p.parse_args()


def _to_dev_bf16(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _to_dev(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def prepare(wl_name: str, seed: int, torch, rudder, W, w4a4_codes: str = "int",
            w4a8_codes: str = "int"):
    wi = W.make_inputs(wl_name, seed=seed)
    wl = wi.workload
    S = wl.S
    M = wl.M
    sid_d = _to_dev(wi.stream_id, torch)
    xs = {}
    layers = []
    for L in wi.layers:
        key = id(L.x)
        if key not in xs:
            xs[key] = _to_dev_bf16(L.x, torch)
        X = xs[key]
        Wd = _to_dev_bf16(L.w, torch)
        s_d = _to_dev(L.smooth, torch)
        abits = L.layer.abits
        e2m3 = (w4a4_codes if abits == 4 else w4a8_codes) == "e2m3"
        codes = rudder.CODES_E2M3 if e2m3 else rudder.CODES_INT
        Wq, ws, inv = rudder.quantize_weights(Wd, s_d, codes)
        K, N = L.layer.K, L.layer.N
        if L.act_scale is not None:
            delta = _to_dev(L.act_scale, torch)                       # [T, S]
        else:
            delta = None
        comp_a = _to_dev(L.comp_a, torch)
        comp_b = _to_dev(L.comp_b, torch)
        Xq = torch.empty(rudder.packed_act_bytes(M, K, abits, codes), dtype=torch.uint8,
                         device="cuda")
        rs = torch.empty(M, dtype=torch.float32, device="cuda")
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        wsp = torch.empty(rudder.quant_act_workspace_bytes(S), dtype=torch.uint8, device="cuda")
        layers.append(dict(name=L.layer.name, K=K, N=N, abits=abits, codes=codes, X=X,
                           Wbf16=Wd, Wq=Wq,
                           w_scale=ws, inv=inv, delta=delta, comp_a=comp_a, comp_b=comp_b,
                           Xq=Xq, rs=rs, Y=Y, ws=wsp, src=L))
    return wi, sid_d, layers


def run_step(t: int, wl, sid_d, layers, rudder, ev=None):
    """Enqueue one step (all linears).  ev: optional list of (before quant_act,
    before GEMM, after GEMM) event triples per layer, recorded on the launch
    stream."""
    S, M = wl.S, wl.M
    T = wl.n_steps
    tt = t % T
    for i, Ly in enumerate(layers):
        K, N, abits, codes = Ly["K"], Ly["N"], Ly["abits"], Ly["codes"]
        if ev is not None:
            ev[i][0].record()
        if Ly["delta"] is None:
            rudder.rudder_quant_act(Ly["X"], sid_d, Ly["inv"], None, None, Ly["ws"], M, K, S,
                                    abits, codes, Ly["Xq"], Ly["rs"])
        else:
            rudder.rudder_quant_act(Ly["X"], sid_d, Ly["inv"], Ly["delta"][tt], None, None, M, K,
                                    S, abits, codes, Ly["Xq"], Ly["rs"])
        ca = Ly["comp_a"][tt] if Ly["comp_a"].dim() == 3 else Ly["comp_a"]
        cb = Ly["comp_b"][tt] if Ly["comp_b"].dim() == 3 else Ly["comp_b"]
        if ev is not None:
            ev[i][1].record()
        rudder.rudder_linear(Ly["Xq"], Ly["rs"], sid_d, Ly["Wq"], Ly["w_scale"], ca, cb, M, N, K,
                             S, abits, codes, Ly["Y"], None)
        if ev is not None:
            ev[i][2].record()


def run_chained_step(t: int, wl, sid_d, layers, rudder, fused: bool, gelu_buf):
    """One step with the MLP chained as in a DiT block: the down layer's input
    is GELU(up-projection output).  Unfused: up writes bf16, rudder_gelu_bf16,
    rudder_quant_act for the down layer.  Fused: rudder_linear_gelu_quant
    writes the down layer's codes and row scales from the up GEMM's epilogue.
    The attention projections run as in run_step."""
    S, M = wl.S, wl.M
    tt = t % wl.n_steps
    by_name = {Ly["name"]: Ly for Ly in layers}
    up, down = by_name["up"], by_name["down"]

    def comp(Ly):
        ca = Ly["comp_a"][tt] if Ly["comp_a"].dim() == 3 else Ly["comp_a"]
        cb = Ly["comp_b"][tt] if Ly["comp_b"].dim() == 3 else Ly["comp_b"]
        return ca, cb

    for Ly in layers:
        if Ly["name"] == "down":
            continue
        K, N, abits, codes = Ly["K"], Ly["N"], Ly["abits"], Ly["codes"]
        rudder.rudder_quant_act(Ly["X"], sid_d, Ly["inv"], Ly["delta"][tt], None, None, M, K, S,
                                abits, codes, Ly["Xq"], Ly["rs"])
        ca, cb = comp(Ly)
        if Ly is up and fused:
            rudder.rudder_linear_gelu_quant(up["Xq"], up["rs"], sid_d, up["Wq"], up["w_scale"], ca,
                                            cb, M, N, K, S, abits, codes, down["inv"],
                                            down["delta"][tt], down["abits"], down["codes"],
                                            down["Xq"], down["rs"])
        else:
            rudder.rudder_linear(Ly["Xq"], Ly["rs"], sid_d, Ly["Wq"], Ly["w_scale"], ca, cb, M, N,
                                 K, S, abits, codes, Ly["Y"], None)
    if not fused:
        rudder.rudder_gelu_bf16(up["Y"], gelu_buf, gelu_buf.numel())
        rudder.rudder_quant_act(gelu_buf, sid_d, down["inv"], down["delta"][tt], None, None, M,
                                down["K"], S, down["abits"], down["codes"], down["Xq"],
                                down["rs"])
    ca, cb = comp(down)
    rudder.rudder_linear(down["Xq"], down["rs"], sid_d, down["Wq"], down["w_scale"], ca, cb, M,
                         down["N"], down["K"], S, down["abits"], down["codes"], down["Y"], None)


def time_chained(wl, sid_d, layers, rudder, torch, steps: int, warmup: int):
    """µs per step of the chained-MLP step, unfused and fused."""
    names = {Ly["name"] for Ly in layers}
    if not {"up", "down"} <= names or any(Ly["delta"] is None for Ly in layers):
        return None
    up = next(Ly for Ly in layers if Ly["name"] == "up")
    gelu_buf = torch.empty_like(up["Y"])
    out = {}
    for label, fused in (("unfused_gelu_quant", False), ("fused_gelu_quant", True)):
        for t in range(warmup):
            run_chained_step(t, wl, sid_d, layers, rudder, fused, gelu_buf)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(steps):
            run_chained_step(t, wl, sid_d, layers, rudder, fused, gelu_buf)
        e1.record()
        torch.cuda.synchronize()
        out[label + "_us_per_step"] = round(e0.elapsed_time(e1) / steps * 1e3, 1)
    return out


def gemm_kernel_tag(Ly, rudder) -> str:
    """One tag per GEMM kernel instance (bit width and code container)."""
    if Ly["codes"] == rudder.CODES_E2M3:
        return f"w4a{Ly['abits']}_e2m3_gemm"
    return f"w4a{Ly['abits']}_gemm"


def mfma_ceiling(layers, rudder, torch, iters: int = 4000, reps: int = 5):
    """MFMA-only rate of each GEMM kernel's matrix-core instruction on
    fragments of that layer's own packed codes (as left by the timed steps),
    and on all-zero codes.  The chip's clock falls with operand bit activity,
    so the first figure is the attainable MFMA rate for this data.  For the
    int containers the 16x16x64 int8 shape is timed too; the rate of the
    instruction the tiled kernel issues is `kernel_instruction_tops`, and the
    GEMM's own rate is set against it in `frac_of_ceiling`."""
    sink = torch.empty(rudder.mfma_ceiling_sink_bytes() // 4, dtype=torch.int32, device="cuda")
    out = {}
    for Ly in layers:
        tag = gemm_kernel_tag(Ly, rudder)
        if tag in out:
            continue
        K, N, abits, codes = Ly["K"], Ly["N"], Ly["abits"], Ly["codes"]
        M = Ly["rs"].numel()
        ops = rudder.mfma_ceiling_ops(iters, codes)
        res = {}
        for name, Xq, Wq in (("workload_codes_tops", Ly["Xq"], Ly["Wq"]),
                             ("zero_codes_tops", torch.zeros_like(Ly["Xq"]),
                              torch.zeros_like(Ly["Wq"]))):
            run = lambda: rudder.rudder_mfma_ceiling(Xq, Wq, M, N, K, abits, codes, iters, sink)
            for _ in range(3):
                run()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                run()
            e1.record()
            torch.cuda.synchronize()
            res[name] = round(ops * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
        if codes != rudder.CODES_E2M3:
            # the other int8 instruction shape on the same codes
            shape = rudder.CEILING_I8_16X16X64
            run = lambda: rudder.rudder_mfma_ceiling_shape(Ly["Xq"], Ly["Wq"], M, N, K, abits,
                                                           codes, iters, shape, sink)
            for _ in range(3):
                run()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                run()
            e1.record()
            torch.cuda.synchronize()
            res["workload_codes_tops_i8_16x16x64"] = round(
                ops * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
        # the instruction the tiled kernel itself issues: 16x16x64 for
        # 8-bit int codes, 32x32x32 for 4-bit int codes, the FP6 shape for E2M3
        res["kernel_instruction_tops"] = (res["workload_codes_tops_i8_16x16x64"]
                                          if codes != rudder.CODES_E2M3 and abits == 8
                                          else res["workload_codes_tops"])
        res["layer"] = f"{Ly['name']} {K}->{N}"
        out[tag] = res
    return out


def load_traffic(kernel_tag: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources."""
    path = os.path.join(PROFILE_DIR, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel_tag)
    if not ent or ent.get("source_hash") != src_hash:
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(wi, rows_per_layer: int, step: int, seed: int):
    """Time the CPU oracle (quantize -> integer GEMM -> epilogue) on a bounded
    sample of the workload: rows_per_layer rows through every linear at one
    step's scale set, 1 untimed warm-up run then 3 timed runs, median.  The
    OpenMP thread count is the process's CPU affinity count (capped by an
    OMP_NUM_THREADS already set in the environment), set before the oracle
    library starts OpenMP."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    threads = min(affinity, int(env)) if env and env.isdigit() and int(env) > 0 else affinity
    os.environ["OMP_NUM_THREADS"] = str(threads)
    import oracle
    wl = wi.workload
    rng = np.random.default_rng(seed)
    M = wl.M
    rows = np.sort(rng.choice(M, size=min(rows_per_layer, M), replace=False))
    sid = np.ascontiguousarray(wi.stream_id[rows])
    prepared = []
    for L in wi.layers:
        inv = oracle.inv_smooth(L.smooth)
        qw, ws = oracle.quantize_weights(L.w, L.smooth)          # offline, untimed
        x = np.ascontiguousarray(L.x[rows])
        prepared.append((L, inv, qw, ws, x))
    t = step % wl.n_steps

    def one_run():
        ops = 0
        for (L, inv, qw, ws, x) in prepared:
            if L.act_scale is None:
                delta = oracle.dynamic_scales(x, sid, inv, wl.S, L.layer.abits)
            else:
                delta = L.act_scale[t]
            a, b = L.step_comp(t)
            oracle.linear(x, sid, qw, ws, inv, delta, a, b, wl.S, L.layer.abits)
            ops += 2 * len(rows) * L.layer.K * L.layer.N
        return ops

    one_run()                                                   # warm-up
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        ops = one_run()
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    return dict(value=ops / dt / 1e12, unit="TOPS", cores=oracle.num_threads(), kind="oracle",
                sample=f"{len(rows)} of {M} rows through all {len(wi.layers)} linears at step "
                       f"{t} (quantize + int32 GEMM + epilogue); 1 warm-up + 3 timed runs, "
                       f"median {dt:.2f} s per run",
                affinity_cpus=affinity, runs_s=[round(x, 3) for x in times])


def bf16_comparator(wl, layers, torch, reps: int = 10):
    """torch.matmul in bf16 (hipBLASLt) on the same [M,K] x [K,N] shapes."""
    M = wl.M
    tot = 0.0
    for Ly in layers:
        A = Ly["X"]
        B = Ly["Wbf16"]
        for _ in range(3):
            torch.matmul(A, B)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            torch.matmul(A, B)
        e1.record()
        torch.cuda.synchronize()
        tot += e0.elapsed_time(e1) / reps
    del M
    return tot * 1e3      # µs per step


def int8_library_comparator(wl, layers, torch, reps: int = 10):
    """hipBLASLt int8 x int8 -> int32 GEMM (torch._int_mm) on the same
    [M,K] x [K,N] shapes: a plain library integer GEMM with no quantization,
    no scales and no epilogue, for context.  Returns µs per step or None."""
    tot = 0.0
    for Ly in layers:
        a = torch.randint(-127, 128, (wl.M, Ly["K"]), dtype=torch.int8, device="cuda")
        b = torch.randint(-7, 8, (Ly["N"], Ly["K"]), dtype=torch.int8, device="cuda").t()
        try:
            for _ in range(3):
                torch._int_mm(a, b)
        except Exception:
            return None
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            torch._int_mm(a, b)
        e1.record()
        torch.cuda.synchronize()
        tot += e0.elapsed_time(e1) / reps
        del a, b
    return tot * 1e3


SMALL_M_CASES = (
    # name, M, K, N, abits, W4A4 codes: an action/proprio-sized call against
    # full-width weights (the weights dominate the bytes)
    ("m96_qkv_h2048_w4a8", 96, 2048, 6144, 8, "int"),
    ("m192_qkv_h4096_w4a4", 192, 4096, 12288, 4, "e2m3"),
)


MALL_BYTES = 256 * 2**20          # MI355X memory-side (Infinity) cache


def small_m_calls(torch, rudder, w4a4_codes: str, warm_reps: int = 20):
    """Few-row calls, each timed two ways as graph replays (a few-µs kernel
    is otherwise timed by the host's issue rate):
      - cold: one call per buffer set, cycling through at least 8 distinct
        sets (packed weights, codes, scales, outputs) that together hold more
        than 3x the memory-side cache, so every call reads its operands from
        HBM;
      - warm: `warm_reps` calls on the same set (operands cache-resident).
    Reports the GEMM kernel alone and quant_act + linear, with the GEMM's
    algorithmic bytes (packed weights + codes in + bf16 out + scales) per
    second."""
    out = {}
    S = 3
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    for name, M, K, N, abits, codes_name in SMALL_M_CASES:
        codes = rudder.CODES_E2M3 if (abits == 4 and (codes_name == "e2m3" and
                                                      w4a4_codes == "e2m3")) else rudder.CODES_INT
        wbytes = 0.75 if codes == rudder.CODES_E2M3 else 0.5
        abytes = 0.75 if codes == rudder.CODES_E2M3 else abits / 8
        gemm_bytes = N * K * wbytes + M * K * abytes + 2 * M * N + 4 * N + 8 * S * N + 5 * M
        set_bytes = gemm_bytes + 2 * M * K                       # + the bf16 input X
        n_sets = max(8, int(np.ceil(3 * MALL_BYTES / set_bytes)))
        sid = (torch.arange(M, device="cuda") % S).to(torch.uint8)
        smooth = torch.ones(K, device="cuda")
        delta = torch.tensor([0.02, 0.03, 0.025], device="cuda")
        sets = []
        for _ in range(n_sets):
            X = torch.randn(M, K, device="cuda", generator=gen).to(torch.bfloat16)
            Wt = (torch.randn(K, N, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
            Wq, ws, inv = rudder.quantize_weights(Wt, smooth, codes)
            del Wt
            ca = torch.rand(S, N, device="cuda", generator=gen) + 0.5
            cb = torch.randn(S, N, device="cuda", generator=gen) * 0.01
            Xq, rs = rudder.quant_act(X, sid, inv, delta, S, abits, codes)
            Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            sets.append((X, Wq, ws, inv, ca, cb, Xq, rs, Y))

        def gemm(i):
            X, Wq, ws, inv, ca, cb, Xq, rs, Y = sets[i]
            rudder.rudder_linear(Xq, rs, sid, Wq, ws, ca, cb, M, N, K, S, abits, codes, Y)

        def pair(i):
            X, Wq, ws, inv, ca, cb, Xq, rs, Y = sets[i]
            rudder.rudder_quant_act(X, sid, inv, delta, None, None, M, K, S, abits, codes, Xq, rs)
            gemm(i)

        def replay_us(seq, fn):
            for i in seq[:3]:
                fn(i)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                with torch.cuda.graph(g, stream=st):
                    for i in seq:
                        fn(i)
            torch.cuda.synchronize()
            g.replay()
            best = 1e9
            for _ in range(3):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                best = min(best, e0.elapsed_time(e1) / len(seq))
            del g
            return best * 1e3

        cold = list(range(n_sets))
        warm = [0] * warm_reps
        res = {"gemm_cold": replay_us(cold, gemm), "pair_cold": replay_us(cold, pair),
               "gemm_warm": replay_us(warm, gemm), "pair_warm": replay_us(warm, pair)}
        # reference: a plain device copy moving the same bytes (half read,
        # half written) from the same number of rotating buffers, replayed
        # the same way: what one launch of this size attains on this part
        half = int(gemm_bytes // 2) // 16 * 16
        copies = [(torch.empty(half, dtype=torch.uint8, device="cuda").fill_(1),
                   torch.empty(half, dtype=torch.uint8, device="cuda")) for _ in range(n_sets)]
        res["copy_cold"] = replay_us(cold, lambda i: copies[i][1].copy_(copies[i][0]))
        del copies
        gbs = gemm_bytes / (res["gemm_cold"] * 1e-6) / 1e9
        gbs_w = gemm_bytes / (res["gemm_warm"] * 1e-6) / 1e9
        out[name] = {"M": M, "K": K, "N": N,
                     "codes": "e2m3" if codes == rudder.CODES_E2M3 else "int",
                     "gemm_us": round(res["gemm_cold"], 2),
                     "quant_act_plus_gemm_us": round(res["pair_cold"], 2),
                     "gemm_bytes": int(gemm_bytes), "gemm_GBps": round(gbs, 1),
                     "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                     "copy_same_bytes_us": round(res["copy_cold"], 2),
                     "buffer_sets": n_sets,
                     "buffer_set_MB": round(set_bytes / 1e6, 1),
                     "mall_warm": {"gemm_us": round(res["gemm_warm"], 2),
                                   "quant_act_plus_gemm_us": round(res["pair_warm"], 2),
                                   "gemm_GBps": round(gbs_w, 1)}}
        del sets
        torch.cuda.empty_cache()
    return out


def calibration_run(torch, W):
    """Offline calibration of one hidden-2048 QKV layer (2048 -> 6144, W4A8)
    from 4 steps x 256 calibration rows, GPU in the loop: wall time of the
    whole search (both stages) and the number of quantize+GEMM passes."""
    from w4a4_quantized_gemm_rudder_amd import calibrate as GC
    ci = W.make_calibration(2048, 6144, seed=0, steps=4, rows=(192, 16, 48), n_outliers=20,
                            outlier_factor=30.0)
    weights = GC.map_weights(ci.scores)
    GC.calibrate(ci.xs[:1], ci.sids[:1], ci.w, weights, 3, 8, alphas=(0.5,), rhos=(1.0,),
                 gains=(1.0,))                                     # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res = GC.calibrate(ci.xs, ci.sids, ci.w, weights, 3, 8)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    return {"layer": "qkv 2048->6144 W4A8", "rows_per_step": 256, "steps": 4,
            "passes": res.passes, "ms": round(dt * 1e3, 1),
            "alpha": res.alpha, "rho_index": res.rho_index}


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _dist(xs_us):
    """median / p10 / p90 of a list of microsecond values."""
    a = np.asarray(xs_us, np.float64)
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2)}


def instrumented_steps(wl, sid_d, layers, rudder, torch, steps: int, t0: int = 0):
    """`steps` steps with an event triple around every linear (quant_act, GEMM)
    on the launch stream.  Returns per-layer lists of (quant+GEMM µs, GEMM µs)
    and the step time of this pass (the records add small gaps)."""
    ev = [[_events(3) for _ in layers] for _ in range(steps)]
    start, end = _events(2)
    torch.cuda.synchronize()
    start.record()
    for t in range(steps):
        run_step(t0 + t, wl, sid_d, layers, rudder, ev[t])
    end.record()
    torch.cuda.synchronize()
    per = [([], []) for _ in layers]
    for t in range(steps):
        for i in range(len(layers)):
            e = ev[t][i]
            per[i][0].append(e[0].elapsed_time(e[2]) * 1e3)
            per[i][1].append(e[1].elapsed_time(e[2]) * 1e3)
    return per, start.elapsed_time(end) / steps * 1e3


def per_call_table(wl, layers, per, rudder, tag_prefix=""):
    """Per-linear call statistics (median / p10 / p90 over the timed steps) of
    rudder_linear alone and of rudder_quant_act + rudder_linear, with the
    GEMM's rate against the int8 and FP6 matrix-core peaks."""
    out = {}
    for Ly, (pair, gemm) in zip(layers, per):
        ops = 2.0 * wl.M * Ly["N"] * Ly["K"]
        med = float(np.median(gemm))
        tops = ops / (med * 1e-6) / 1e12
        e2m3 = Ly["codes"] == rudder.CODES_E2M3
        key = (f"{tag_prefix}{Ly['name']} {wl.M}x{Ly['K']}->{Ly['N']} W4A{Ly['abits']}"
               f"{' e2m3' if e2m3 else ''}")
        ent = {"gemm_us": _dist(gemm), "quant_act_plus_gemm_us": _dist(pair),
               "gemm_tops": round(tops, 1),
               "fused_linear_tops": round(ops / (float(np.median(pair)) * 1e-6) / 1e12, 1),
               "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 1)}
        if e2m3:
            peak = FP6_PEAK_TFLOPS / (2 if Ly["abits"] == 8 else 1)
            ent["pct_fp6_peak"] = round(100 * tops / peak, 1)
        out[key] = ent
    return out


def large_gemm_calls(args, torch, rudder, W, steps: int = 20, warmup: int = 5):
    """The hidden-4096 backbone's four linears (16576 rows; QKV, O, MLP up and
    down, all W4A4), drawn with the workload generator and run as that
    workload's step loop (each layer's weights were last read a whole step
    earlier, as in a model): `warmup` untimed steps, then `steps` steps with
    per-call events."""
    name = "backbone_h4096_m16576_w4a4"
    wi, sid_d, layers = prepare(name, args.seed, torch, rudder, W, args.w4a4_codes,
                                args.w4a8_codes)
    wl = wi.workload
    for t in range(warmup):
        run_step(t, wl, sid_d, layers, rudder)
    per, step_us = instrumented_steps(wl, sid_d, layers, rudder, torch, steps, warmup)
    res = per_call_table(wl, layers, per, rudder)
    res["step_us_with_events"] = round(step_us, 1)
    res["protocol"] = f"{warmup} warm-up steps, {steps} timed steps, HIP events per call"
    del layers, sid_d, wi
    torch.cuda.empty_cache()
    return res


# The measured limiter of each GEMM kernel's main loop (from timing-only
# variants and counters; the roofline bound stays the matrix cores, whose
# arithmetic intensity is far above the HBM ridge).
LIMITER = {
    "w4a4_e2m3_gemm": "operand stream from L2 to the compute units (latency-bound loads)",
    "w4a8_e2m3_gemm": "operand stream from L2 to the compute units (latency-bound loads)",
    "w4a8_gemm": "matrix-core rate at the operands' power-limited clock",
    "w4a4_gemm": "matrix-core rate at the operands' power-limited clock",
}


def path_dtype(layers, rudder) -> str:
    """The arithmetic types the step's contractions run in: int8 MFMA with
    int32 sums (int containers), FP6 E2M3 MFMA with fp32 sums that hold exact
    integers (4-bit E2M3 codes), two FP6 MFMAs per product (8-bit codes as
    E2M3 digit planes)."""
    kinds = []
    for Ly in layers:
        if Ly["codes"] != rudder.CODES_E2M3:
            k = "int8"
        else:
            k = "fp6_e2m3" if Ly["abits"] == 4 else "fp6_e2m3_x2"
        if k not in kinds:
            kinds.append(k)
    return "+".join(kinds)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer shards by "
              "rows or output channels with no exchange, but no multi-GPU path is built.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from w4a4_quantized_gemm_rudder_amd import rudder
    from w4a4_quantized_gemm_rudder_amd import workloads as W
    rudder.load_library()
    torch.cuda.set_device(0)

    wi, sid_d, layers = prepare(args.workload, args.seed, torch, rudder, W, args.w4a4_codes,
                                args.w4a8_codes)
    wl = wi.workload
    torch.cuda.synchronize()

    if args.copy_bytes > 0:
        # a plain elementwise copy kernel (reads copy_bytes, writes copy_bytes)
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.add(src, 1, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for t in range(args.warmup):
        run_step(t, wl, sid_d, layers, rudder)
    torch.cuda.synchronize()

    # the timed steps: nothing but the step's own launches on the stream
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    start.record()
    for t in range(args.steps):
        run_step(t, wl, sid_d, layers, rudder)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    # Per-step distribution: the same K steps again with one event at every
    # step boundary (median / p10 / p90 of the step time).
    bounds = _events(args.steps + 1)
    torch.cuda.synchronize()
    bounds[0].record()
    for t in range(args.steps):
        run_step(t, wl, sid_d, layers, rudder)
        bounds[t + 1].record()
    torch.cuda.synchronize()
    step_dist = _dist([bounds[t].elapsed_time(bounds[t + 1]) * 1e3 for t in range(args.steps)])

    # The same K steps again with an event triple around every linear (on the
    # launch stream), for the per-kernel durations.  The event records add
    # gaps between launches, so this pass is kept out of the headline; its
    # step time is reported beside it.
    per, us_instrumented = instrumented_steps(wl, sid_d, layers, rudder, torch, args.steps)
    ms_per_step_instrumented = us_instrumented * 1e-3

    # per-kernel (GEMM) launch durations, grouped by kernel instance (abits)
    gemm_ms = {}
    gemm_ops = {}
    for i, Ly in enumerate(layers):
        key = gemm_kernel_tag(Ly, rudder)
        gemm_ms.setdefault(key, []).extend(d * 1e-3 for d in per[i][1])
        gemm_ops.setdefault(key, []).extend([2 * wl.M * Ly["N"] * Ly["K"]] * args.steps)
    dominant = max(gemm_ms, key=lambda k: sum(gemm_ms[k]))
    avg_ms = float(np.mean(gemm_ms[dominant]))
    ops_per_launch = float(np.mean(gemm_ops[dominant]))
    achieved = ops_per_launch / (avg_ms * 1e-3) / 1e12
    # a contraction is priced against the peak of the matrix-core type it runs
    # on; 8-bit codes in the E2M3 container take two FP6 MFMAs per product
    if "e2m3" not in dominant:
        dom_peak = INT8_PEAK_TOPS
    else:
        dom_peak = FP6_PEAK_TFLOPS / (2 if dominant.startswith("w4a8") else 1)
    per_kernel = {k: {"avg_launch_us": round(float(np.mean(v)) * 1e3, 2),
                      "launches_per_step": len(v) // args.steps,
                      "tops": round(float(np.mean(gemm_ops[k])) / (float(np.mean(v)) * 1e-3)
                                    / 1e12, 1)}
                  for k, v in gemm_ms.items()}
    src_hash = kernel_source_hash()
    traffic = load_traffic(f"{dominant}_{args.workload}", src_hash)

    ops_step = wl.ops_per_step()
    value = ops_step / (ms_per_step * 1e-3) / 1e12
    gemm_only_ms = sum(sum(v) for v in gemm_ms.values()) / args.steps

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "us_per_step": round(ms_per_step * 1e3, 1),
        "step_us": step_dist,
        "us_per_step_with_kernel_events": round(ms_per_step_instrumented * 1e3, 1),
        "pct_int8_peak": round(100 * value / INT8_PEAK_TOPS, 2),
        "gemm_only_tops": round(ops_step / (gemm_only_ms * 1e-3) / 1e12, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": path_dtype(layers, rudder),
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "tokens": wl.M,
            "streams": {W.STREAM_NAMES[s]: int((wi.stream_id == s).sum()) for s in range(wl.S)},
            "linears": [f"{Ly['name']} {Ly['K']}->{Ly['N']} W4A{Ly['abits']}"
                        + (" (E2M3 codes)" if Ly["codes"] == rudder.CODES_E2M3 else "")
                        for Ly in layers],
            "denoise_steps": wl.n_steps,
            "launches_per_step": 2 * len(layers) + (2 * len(layers) if wl.dynamic else 0),
        },
        "roofline": {
            "kernel": dominant,
            "bound": "mfma",
            "limiter": LIMITER.get(dominant),
            "achieved": round(achieved, 2),
            "peak": dom_peak,
            "unit": "TFLOP/s",
            "op_count": "2*M*N*K multiply-add ops of the integer codes",
            "frac": round(achieved / dom_peak, 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_ms * 1e3, 2),
            "ops_per_launch": ops_per_launch,
            "source_hash": src_hash,
        },
        "gemm_kernels": per_kernel,
        "per_call": per_call_table(wl, layers, per, rudder),
        "wall_s": round(wall, 3),
    }
    if not args.no_ceiling:
        ceil = mfma_ceiling(layers, rudder, torch)
        out["mfma_ceiling"] = ceil
        for k, v in out["gemm_kernels"].items():
            v["frac_of_ceiling"] = round(v["tops"] / ceil[k]["kernel_instruction_tops"], 4)
        out["roofline"]["mfma_ceiling_tops"] = ceil[dominant]["kernel_instruction_tops"]
        out["roofline"]["frac_of_ceiling"] = round(
            achieved / ceil[dominant]["kernel_instruction_tops"], 4)
    if not args.no_bf16:
        bf16_us = bf16_comparator(wl, layers, torch)
        out["bf16_matmul_us_per_step"] = round(bf16_us, 1)
        out["speedup_vs_bf16_matmul"] = round(bf16_us / (ms_per_step * 1e3), 3)
        i8_us = int8_library_comparator(wl, layers, torch)
        if i8_us is not None:
            out["int8_library_gemm_us_per_step"] = round(i8_us, 1)
    chained = (None if args.no_chained else
               time_chained(wl, sid_d, layers, rudder, torch, args.steps, args.warmup))
    if chained is not None:
        out["mlp_chained"] = chained
    if not args.no_small_m:
        out["small_m"] = small_m_calls(torch, rudder, args.w4a4_codes)
    if not args.no_large and args.workload != "backbone_h4096_m16576_w4a4":
        out["large_gemms"] = large_gemm_calls(args, torch, rudder, W)
    if not args.no_calibration:
        out["calibration"] = calibration_run(torch, W)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wi, args.cpu_rows, args.cpu_step, args.seed)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
