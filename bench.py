#!/usr/bin/env python3
"""Benchmark of the quantized linear on one MI355X.

Step = one pass of the hot path over the DiT-XL/2 MLP at W8A8 DualScale with
the CFG epilogue (16 images x 256 tokens, conditional + unconditional rows,
M = 4096): for fc1 (1152 -> 4608) and fc2 (4608 -> 1152), quantize the
activations (dual per-tensor max-reduce + quantize) and run the int8-MFMA GEMM
with the fused fp32 epilogue and guidance combine (w = 4).

Metric: MFMA int8 TOPS over the step (both DualScale contractions counted,
4*M*N*K per linear), plus the activation-quantization bandwidth. Inputs are
seeded synthetic tensors already resident in HBM when timing starts.

Prints ONE JSON line. Other workloads (--workload c1..c5) print their own
line for reference; the default is the MLP workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E, 8 TB/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="mlp", help="mlp (default) | block | c3 | c3s | c4 | c4g | c5 | c6 | c7 | c7f")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time budget of the oracle baseline")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run device-to-device copies of a known size (for scaling the "
                        "profiler's memory counters) and exit")
    return p.parse_args()


def layers_for(name):
    from workloads import configs
    if name == "mlp":
        wl = configs.WORKLOADS["c2"]
        return wl, [l for l in wl.layers if l.name in ("fc1", "fc2")]
    if name == "block":
        wl = configs.WORKLOADS["c2"]
        return wl, list(wl.layers)
    if name in ("c3", "c4"):
        wl = configs.WORKLOADS[name]
        return wl, list(wl.layers)
    if name in ("c7", "c7f"):
        wl = configs.WORKLOADS["c7"]
        return wl, list(wl.layers)
    if name == "c3s":
        return configs.WORKLOADS["c3"], list(configs.c3_single())
    if name == "c4g":
        # The MM-DiT stack with activation bits from the greedy allocation
        # (library host code) instead of the seeded mask.
        import dataclasses
        from bit_post_quantization_amd import qlinear_gamp_allocate
        wl, macs, gain, budget = configs.c4_gamp_inputs()
        bits, _ = qlinear_gamp_allocate(macs.tolist(), gain.tolist(), 4, budget)
        return wl, [dataclasses.replace(L, a_bits=b) for L, b in zip(wl.layers, bits)]
    raise SystemExit(f"unknown workload {name}")


class Layer:
    def __init__(self, torch, wl, L, use_branches=True):
        from bit_post_quantization_amd import QuantLinear
        from workloads import configs
        self.L, self.M = L, wl.M
        X = configs.make_x(wl, L)
        W = configs.make_w(wl, L)
        self.X_host, self.W_host = X, W
        self.X = torch.from_numpy(X.view(np.int16) if L.x_dtype == "bf16" else X).cuda()
        Wd = torch.from_numpy(W).cuda()
        seg = L.seg_offsets()
        self.ql = QuantLinear(Wd, w_bits=L.w_bits, a_bits=L.a_bits, hadamard_block=L.hadamard_block,
                              seg_offsets=None if seg is None else seg.tolist(),
                              w_scale=L.w_scale, a_scale=L.a_scale, x_dtype=L.x_dtype,
                              single_hadamard=L.single_hadamard,
                              k_seg_offsets=list(L.k_seg) if (L.k_seg and use_branches) else None)
        del Wd
        self.codes = self.ql.alloc_codes(self.M)
        nks = max(1, len(L.k_seg) - 1) if use_branches else 1
        self.scales = torch.empty(2 * nks, dtype=torch.float32, device="cuda")
        rows = self.M // 2 if L.cfg else self.M
        self.Y = torch.empty((rows, L.N), dtype=torch.float32, device="cuda")
        # Algorithmic work: two contractions per output with DualScale (both
        # polarity planes, 4*M*N*K int ops), one with symmetric codes. The
        # single Hadamard is one symmetric contraction of the method; the
        # kernel executes it as two int8 products (hi and lo weight planes),
        # reported apart as executed MFMA work.
        planes = 2 if L.a_scale == "dual" else 1
        self.mfma_ops = planes * 2.0 * self.M * L.N * L.K
        self.exec_ops = (2 if (L.a_scale == "dual" or L.single_hadamard) else 1) \
            * 2.0 * self.M * L.N * L.K
        self.eff_ops = 2.0 * self.M * L.N * L.K
        xbytes = 2 if L.x_dtype == "bf16" else 4
        self.quant_bytes = self.M * L.K * (xbytes + L.a_bits / 8.0)

    def quantize(self):
        from bit_post_quantization_amd import qlinear_quantize_act
        qlinear_quantize_act(self.ql.plan, self.X, self.M, 0, None, self.codes, self.scales)

    def quantize_static(self):
        """The single pass with given scales (the dynamic call's, kept apart)."""
        from bit_post_quantization_amd import qlinear_quantize_act
        qlinear_quantize_act(self.ql.plan, self.X, self.M, 0, self.static_scales, self.codes,
                             self.scales_out)

    def gemm(self):
        from bit_post_quantization_amd import qlinear_gemm
        qlinear_gemm(self.ql.plan, self.codes, self.scales, self.M, int(self.L.cfg),
                     self.L.guidance, self.Y)


DATA = {
    "gelu_outliers": "synthetic (seeded GELU(N(0,1)) activations with 0.1% x20 outlier channels, "
                     "N(0,0.02) weights)",
    "bf16_normal": "synthetic (seeded bf16(N(0,1)) activations, N(0,0.02) weights)",
    "silu": "synthetic (seeded SiLU(N(0,1)) activations, N(0,0.02) weights)",
    "branches": "synthetic (seeded concatenated branches: GELU(N(0,1)) with outliers, "
                "SiLU(N(0,1)), sin(3 N(0,1)); N(0,0.02) weights)",
}
SHAPE = {
    "c2": {"images": 16, "tokens_per_image": 256},
    "c3": {"images": 16, "tokens_per_image": 256},
    "c4": {"images": 4, "tokens_per_image": 4608},
    "c7": {"images": 16, "tokens_per_image": 256},
}


def per_layer_or_one(vals):
    return vals[0] if len(set(vals)) == 1 else vals


def bops_report(Ls, M):
    """Bit operations (MACs x w_bits x a_bits) of one guided step, both CFG
    halves, as the guidance-aware page asks, beside the single-pass count
    that standard metrics report and the uniform W4A8 / W4A4 stacks."""
    macs = [M * L.N * L.K for L in Ls]
    guided = sum(m * L.w_bits * L.a_bits for m, L in zip(macs, Ls))
    w4a8 = sum(m * 4 * 8 for m in macs)
    w4a4 = sum(m * 4 * 4 for m in macs)
    return {"a_bits": [L.a_bits for L in Ls], "guided_step": guided,
            "single_pass": guided // 2, "uniform_w4a8": w4a8, "uniform_w4a4": w4a4,
            "vs_w4a8": round(guided / w4a8, 4),
            "mean_a_bits_by_macs": round(guided / (4 * sum(macs)), 3)}


def host_info():
    """CPU model and core counts of the machine the oracle runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "cores_allowed": len(os.sched_getaffinity(0))}


def _oracle_rows(oracle, ly, codes, s, wp, rows):
    """GEMM + epilogue (+ CFG) of the oracle on a list of output rows
    (conditional rows with CFG: each is paired with its unconditional row)."""
    L = ly.L
    half = ly.M // 2
    for n in rows:
        r = np.array([n, n + half]) if L.cfg else np.array([n])
        y, _, _ = oracle.linear_rows(codes, s, wp, r, L.a_scale)
        if L.cfg:
            oracle.cfg_combine(y[:1], y[1:], L.guidance)


def cpu_baseline(layers, budget_s, threads=None):
    """The oracle, as it stands, on a bounded sample of the same workload:
    every activation code of every layer, and the GEMM + epilogue (+ CFG) on
    row pairs until the time budget is spent; scaled to the whole step.
    The timed thread is pinned to one host core. A secondary figure runs P
    threads, each the same single-threaded oracle on a disjoint shard of the
    rows (the library releases the interpreter lock while it computes)."""
    import concurrent.futures as cf
    import oracle
    allowed = sorted(os.sched_getaffinity(0))
    os.sched_setaffinity(0, {allowed[0]})
    try:
        t_quant = 0.0
        t_gemm_per_row = []
        rows_done = []
        prepared = []
        per_layer_budget = budget_s / max(1, len(layers))
        for ly in layers:
            L = ly.L
            t0 = time.perf_counter()
            x = oracle.bf16_to_f32(ly.X_host) if L.x_dtype == "bf16" else ly.X_host
            codes, s = oracle.quantize_activations(x, L.a_bits, B=L.hadamard_block, mode=L.a_scale)
            t_quant += time.perf_counter() - t0
            wp = oracle.WeightPlan(ly.W_host, L.w_bits, B=L.hadamard_block, mode=L.w_scale,
                                   seg_offsets=None if L.seg_offsets() is None else L.seg_offsets())
            prepared.append((codes, s, wp))
            top = ly.M // 2 if L.cfg else ly.M
            n = 0
            t0 = time.perf_counter()
            while True:
                _oracle_rows(oracle, ly, codes, s, wp, [n])
                n += 1
                el = time.perf_counter() - t0
                if (el > per_layer_budget and n >= 2) or n >= top:
                    break
            per = 2 if L.cfg else 1
            rows_done.append(n * per)
            t_gemm_per_row.append(el / (n * per))
    finally:
        os.sched_setaffinity(0, set(allowed))
    t_step = t_quant + sum(t * ly.M for t, ly in zip(t_gemm_per_row, layers))
    ops = sum(ly.mfma_ops for ly in layers)
    sample = ("full activation quantization of every layer; GEMM+epilogue+CFG on "
              + ", ".join(f"{r} of {ly.M} rows ({ly.L.name})" for r, ly in zip(rows_done, layers))
              + "; step time extrapolated linearly in rows")
    out = {"value": ops / t_step / 1e12, "unit": "TOPS", "cores": 1, "kind": "oracle",
           "sample": sample, "step_seconds_extrapolated": t_step,
           "host": {**host_info(), "pinned_to_core": allowed[0]}}
    # Secondary figure: P threads, each the single-threaded oracle on its own
    # shard of the output rows (GEMM + epilogue + CFG), for a fixed wall time.
    P = threads or min(16, len(allowed))
    wall = max(1.0, budget_s / 3.0)
    done_rows = []
    t_wall = []
    for ly, (codes, s, wp) in zip(layers, prepared):
        top = ly.M // 2 if ly.L.cfg else ly.M
        shards = np.array_split(np.arange(top), P)
        stop = time.perf_counter() + wall / max(1, len(layers))

        def work(rows, ly=ly, codes=codes, s=s, wp=wp, stop=stop):
            cnt = 0
            for n in rows:
                _oracle_rows(oracle, ly, codes, s, wp, [int(n)])
                cnt += 1
                if time.perf_counter() > stop:
                    break
            return cnt

        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=P) as ex:
            cnt = sum(ex.map(work, shards))
        t_wall.append(time.perf_counter() - t0)
        done_rows.append(cnt * (2 if ly.L.cfg else 1))
    t_step_p = t_quant + sum(t / r * ly.M for t, r, ly in zip(t_wall, done_rows, layers))
    out["parallel"] = {"threads": P, "value": ops / t_step_p / 1e12, "unit": "TOPS",
                       "sample": "GEMM+epilogue+CFG on " + ", ".join(
                           f"{r} rows ({ly.L.name})" for r, ly in zip(done_rows, layers))
                       + " over P disjoint row shards; quantization at the single-thread time; "
                         "scaled linearly in rows"}
    return out


COPY_BYTES = 512 << 20      # calibration copy: 512 MiB read + 512 MiB written per copy
COPY_REPS = 5
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k2_gemm_hbm_traffic_dit_xl2_mlp_w8a8_cfg.json")
GEMM_SOURCE = os.path.join(ROOT, "bit_post_quantization_amd", "csrc", "k_gemm.hip")


def copy_calibration(torch):
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(COPY_REPS):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "reps": COPY_REPS}), flush=True)


PROBE_ITERS = 4000   # per probe launch: ~0.5 ms of MFMA work on every SIMD


def measured_ceilings(torch):
    """What the chip sustains, measured live beside the spec peaks: the int8
    MFMA rate of the library's probe kernel (register operands, no memory,
    no barrier; random operands, which switch the multiplier inputs on every
    instruction as real codes do, and constant ones, which do not; the best
    of one and two waves per SIMD) and the rate of a device-to-device copy
    of 512 MiB (bytes read + written)."""
    from bit_post_quantization_amd import qlinear_probe_mfma
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    ops = {"random": torch.randint(-128, 128, (16, 64, 16), dtype=torch.int8, device="cuda",
                                   generator=g),
           "constant": torch.full((16, 64, 16), 3, dtype=torch.int8, device="cuda")}
    out = {}

    def timed(fn, reps=5):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    for name, o in ops.items():
        best = 0.0
        for wps in (1, 2):
            sink = torch.empty(cus * 256 * wps, dtype=torch.int32, device="cuda")
            t = timed(lambda: qlinear_probe_mfma(o, PROBE_ITERS, wps, sink))
            best = max(best, cus * 4 * wps * PROBE_ITERS * 16 * 32768 / t / 1e12)
        out[f"mfma_int8_{name}_operands_tops"] = round(best, 1)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src))
    out["hbm_copy_gbps"] = round(2 * COPY_BYTES / t / 1e9, 1)
    out["method"] = ("int8 MFMA: qlinear_probe_mfma, %d iterations of 16 independent "
                     "v_mfma_i32_16x16x64_i8 per wave, one workgroup per CU, best of 1 and 2 "
                     "waves per SIMD; copy: torch copy_ of 512 MiB, read + written bytes"
                     % PROBE_ITERS)
    del src, dst
    return out


def gemm_source_hash():
    """SHA-256 of the GEMM source's code: comments and blank lines removed,
    so that editing a comment does not invalidate a profile."""
    import hashlib
    import re
    with open(GEMM_SOURCE) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    code = "\n".join(line.rstrip() for line in src.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()


def measured_traffic():
    """HBM bytes per GEMM launch from the committed counter profile, or None if
    there is none or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("k_gemm_sha256") != gemm_source_hash():
        return None
    return t.get("bytes_per_launch")


def per_launch_rates(torch, calls):
    """Run `calls` [(kind, fn, amount)] once with an event pair around every
    launch (on the launching stream); per kind, the summed amount divided by
    the summed durations, and the mean duration."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in calls]
    torch.cuda.synchronize()
    for (kind, fn, amount), (a, b) in zip(calls, ev):
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    out = {}
    for (kind, fn, amount), (a, b) in zip(calls, ev):
        o = out.setdefault(kind, {"amount": 0.0, "s": 0.0, "n": 0})
        o["amount"] += amount
        o["s"] += a.elapsed_time(b) * 1e-3
        o["n"] += 1
    return {k: {"rate": v["amount"] / v["s"], "avg_us": v["s"] / v["n"] * 1e6}
            for k, v in out.items()}


def sweep_roofline(rates, ops_per_gemm, quant_bytes):
    g, q = rates["gemm"], rates["quant"]
    return ({"kernel": "k2_gemm (int8 MFMA, both polarity planes, fused epilogue)",
             "bound": "mfma", "achieved": round(g["rate"] / 1e12, 1), "peak": PEAK_INT8_TOPS,
             "unit": "TOPS", "frac": round(g["rate"] / 1e12 / PEAK_INT8_TOPS, 4),
             "ops_per_launch": ops_per_gemm, "avg_launch_us": round(g["avg_us"], 2),
             "traffic": None},
            {"kernels": "k1 (quantize)", "bound": "hbm", "achieved": round(q["rate"] / 1e9, 1),
             "peak": PEAK_HBM_GBPS, "unit": "GB/s",
             "frac": round(q["rate"] / 1e9 / PEAK_HBM_GBPS, 4), "bytes_per_step": quant_bytes})


class HostLayer:
    """Host copies of one layer's synthetic inputs, for the oracle baseline."""

    def __init__(self, wl, L):
        from workloads import configs
        self.L, self.M = L, wl.M
        self.X_host = configs.make_x(wl, L, step=0)
        self.W_host = configs.make_w(wl, L)
        self.mfma_ops = 2 * 2.0 * wl.M * L.N * L.K


def bench_tasq_sweep(torch, args):
    """The TASQ sweep: 28 DiT-XL/2 blocks x (qkv, proj, fc1, fc2) = 112 W8A8
    DualScale CFG linears per denoising step, each quantize call with the
    seeded LSB truncation depth k[t][l] in {0, 2, 4}, for `--steps` steps
    (50 by default for this workload). Weights and inputs are generated on
    the device with a seeded torch generator (same distributions as the
    parity workload: W ~ N(0, 0.02^2), X = SiLU(N(0,1))); a pool of four
    inputs per shape is cycled through."""
    from bit_post_quantization_amd import QuantLinear, qlinear_quantize_act, qlinear_gemm
    from workloads import configs
    wl = configs.WORKLOADS["c5"]
    sched = configs.c5_schedule()
    steps = min(args.steps, wl.steps)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    M = wl.M
    plans, pool, ys = [], {}, {}
    for L in wl.layers:
        W = torch.randn(L.N, L.K, device="cuda", generator=g) * 0.02
        plans.append(QuantLinear(W))
        del W
        if L.K not in pool:
            pool[L.K] = [torch.nn.functional.silu(torch.randn(M, L.K, device="cuda", generator=g))
                         for _ in range(4)]
        if L.N not in ys:
            ys[L.N] = torch.empty(M // 2, L.N, dtype=torch.float32, device="cuda")
    codes = {}
    for L, ql in zip(wl.layers, plans):
        if L.K not in codes:
            codes[L.K] = ql.alloc_codes(M)
    scales = torch.empty(2, dtype=torch.float32, device="cuda")
    ops_per_step = sum(4.0 * M * L.N * L.K for L in wl.layers)

    def step(t):
        for li, (L, ql) in enumerate(zip(wl.layers, plans)):
            X = pool[L.K][(t + li) % 4]
            qlinear_quantize_act(ql.plan, X, M, int(sched[t, li]), None, codes[L.K], scales)
            qlinear_gemm(ql.plan, codes[L.K], scales, M, 1, L.guidance, ys[L.N])

    for t in range(min(args.warmup, steps)):
        step(t)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for t in range(steps):
        step(t)
        evs[t + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[t].elapsed_time(evs[t + 1]) for t in range(steps)])
    total_ms = float(per.sum())
    calls = []
    for li, (L, ql) in enumerate(zip(wl.layers, plans)):
        X = pool[L.K][li % 4]
        k = int(sched[0, li])
        calls.append(("quant", lambda ql=ql, X=X, L=L, k=k: qlinear_quantize_act(
            ql.plan, X, M, k, None, codes[L.K], scales), M * L.K * 5.0))
        calls.append(("gemm", lambda ql=ql, L=L: qlinear_gemm(
            ql.plan, codes[L.K], scales, M, 1, L.guidance, ys[L.N]), 4.0 * M * L.N * L.K))
    roof, quant = sweep_roofline(per_launch_rates(torch, calls),
                                 ops_per_step / len(wl.layers),
                                 sum(M * L.K * 5.0 for L in wl.layers))
    out = {
        "metric": "quantized-linear int8 TOPS (% MFMA peak), TASQ 50-step sweep",
        "value": round(ops_per_step * steps / (total_ms * 1e-3) / 1e12, 2), "unit": "TOPS",
        "n_gpus": 1, "steps": steps, "warmup": min(args.warmup, steps),
        "ms_per_step": round(total_ms / steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8",
        "data": "synthetic (device-generated, seeded: X = SiLU(N(0,1)), W ~ N(0, 0.02^2))",
        "config": {"workload": "TASQ sweep: 28 DiT-XL/2 blocks x (qkv, proj, fc1, fc2), W8A8 "
                               "DualScale, CFG w=4, k[t][l] in {0,2,4}", "M": M,
                   "linears_per_step": len(wl.layers)},
        "per_step_tops": {"min": round(ops_per_step / (per.max() * 1e-3) / 1e12, 1),
                          "median": round(ops_per_step / (np.median(per) * 1e-3) / 1e12, 1),
                          "max": round(ops_per_step / (per.min() * 1e-3) / 1e12, 1)},
        "mfma_ops_per_step": ops_per_step,
        "roofline": roof, "act_quant": quant,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = sweep_cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def sweep_cpu_baseline(wl, budget_s):
    """The oracle on one block of the sweep (its four linears at step 0,
    host-generated inputs of the same recipe), as TOPS; a rate, so it holds
    for the whole sweep."""
    cb = cpu_baseline([HostLayer(wl, L) for L in wl.layers[:4]], budget_s)
    cb["sample"] = "one block (qkv, proj, fc1, fc2) at step 0: " + cb["sample"]
    return cb


def bench_tasq_weight_sweep(torch, args):
    """TASQ on the weight side: the same 112 DiT-XL/2 linears per step, each
    with ONE stored W8 plan and one operating view of it. The 50 steps fall in
    4 stages; at a stage change every view whose depth changes is rewritten
    from its stored plan (qlinear_plan_lsb_update, inside the timed region).
    Activations are quantized at per-step static scales from a table that an
    untimed calibration pass fills with the dynamic scales of a separate
    seeded batch (one quantize pass instead of two in the timed region)."""
    from bit_post_quantization_amd import (QuantLinear, qlinear_gemm, qlinear_plan_lsb_update,
                                           qlinear_quantize_act)
    from workloads import configs
    wl = configs.WORKLOADS["c6"]
    wsch = configs.c6_w_schedule()
    steps = min(args.steps, wl.steps)
    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    M = wl.M
    bases, views, pool, calib, ys = [], [], {}, {}, {}
    for li, L in enumerate(wl.layers):
        W = torch.randn(L.N, L.K, device="cuda", generator=g) * 0.02
        bases.append(QuantLinear(W))
        del W
        views.append(bases[-1].lsb_view(int(wsch[0, li])))
        if L.K not in pool:
            pool[L.K] = [torch.nn.functional.silu(torch.randn(M, L.K, device="cuda", generator=g))
                         for _ in range(4)]
            calib[L.K] = [torch.nn.functional.silu(torch.randn(M, L.K, device="cuda",
                                                               generator=g)) for _ in range(4)]
        if L.N not in ys:
            ys[L.N] = torch.empty(M // 2, L.N, dtype=torch.float32, device="cuda")
    codes = {}
    for L, ql in zip(wl.layers, bases):
        if L.K not in codes:
            codes[L.K] = ql.alloc_codes(M)
    scales = torch.empty(2, dtype=torch.float32, device="cuda")
    # Calibration: per-step, per-layer static scale table [steps, layers, 2].
    table = torch.empty(wl.steps, len(wl.layers), 2, dtype=torch.float32, device="cuda")
    for t in range(wl.steps):
        for li, (L, ql) in enumerate(zip(wl.layers, bases)):
            qlinear_quantize_act(ql.plan, calib[L.K][(t + 2 * li) % 4], M, 0, None, codes[L.K],
                                 table[t, li])
    torch.cuda.synchronize()
    ops_per_step = sum(4.0 * M * L.N * L.K for L in wl.layers)
    depth = [int(wsch[0, li]) for li in range(len(wl.layers))]
    n_updates = [0]

    def set_stage(grp):
        for li in range(len(wl.layers)):
            k = int(wsch[grp, li])
            if k != depth[li]:
                qlinear_plan_lsb_update(views[li].plan, bases[li].plan, k)
                depth[li] = k
                n_updates[0] += 1

    def step(t):
        set_stage(configs.stage_of(wl, t))
        for li, (L, v) in enumerate(zip(wl.layers, views)):
            X = pool[L.K][(t + li) % 4]
            qlinear_quantize_act(v.plan, X, M, 0, table[t, li], codes[L.K], scales)
            qlinear_gemm(v.plan, codes[L.K], scales, M, 1, L.guidance, ys[L.N])

    # Cost of one depth change of all 112 views (measured apart, untimed): the
    # views share their base's codes, so an update is host work only.
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for li in range(len(wl.layers)):
        qlinear_plan_lsb_update(views[li].plan, bases[li].plan, int(wsch[1, li]))
    torch.cuda.synchronize()
    update_all_ms = (time.perf_counter() - h0) * 1e3
    for li in range(len(wl.layers)):
        depth[li] = int(wsch[1, li])
    for t in range(min(args.warmup, steps)):
        step(t)
    set_stage(0)
    n_updates[0] = 0
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for t in range(steps):
        step(t)
        evs[t + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[t].elapsed_time(evs[t + 1]) for t in range(steps)])
    total_ms = float(per.sum())
    wbytes = sum(L.N * L.K for L in wl.layers)
    calls = []
    for li, (L, v) in enumerate(zip(wl.layers, views)):
        X = pool[L.K][li % 4]
        calls.append(("quant", lambda v=v, X=X, L=L, li=li: qlinear_quantize_act(
            v.plan, X, M, 0, table[0, li], codes[L.K], scales), M * L.K * 5.0))
        calls.append(("gemm", lambda v=v, L=L: qlinear_gemm(
            v.plan, codes[L.K], scales, M, 1, L.guidance, ys[L.N]), 4.0 * M * L.N * L.K))
    roof, quant = sweep_roofline(per_launch_rates(torch, calls),
                                 ops_per_step / len(wl.layers),
                                 sum(M * L.K * 5.0 for L in wl.layers))
    out = {
        "metric": "quantized-linear int8 TOPS (% MFMA peak), TASQ weight-side 50-step sweep",
        "value": round(ops_per_step * steps / (total_ms * 1e-3) / 1e12, 2), "unit": "TOPS",
        "n_gpus": 1, "steps": steps, "warmup": min(args.warmup, steps),
        "ms_per_step": round(total_ms / steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8",
        "data": "synthetic (device-generated, seeded: X = SiLU(N(0,1)), W ~ N(0, 0.02^2))",
        "config": {"workload": "TASQ weight-side sweep: 28 DiT-XL/2 blocks x (qkv, proj, fc1, "
                               "fc2), W8 storage, per-(stage, layer) weight depth in {0,2,4} over "
                               "4 stages, A8 DualScale at per-step static scales, CFG w=4",
                   "M": M, "linears_per_step": len(wl.layers), "stages": wl.stages},
        "per_step_tops": {"min": round(ops_per_step / (per.max() * 1e-3) / 1e12, 1),
                          "median": round(ops_per_step / (np.median(per) * 1e-3) / 1e12, 1),
                          "max": round(ops_per_step / (per.min() * 1e-3) / 1e12, 1)},
        "depth_updates_timed": n_updates[0],
        "depth_update_all_views_ms": round(update_all_ms, 4),
        "weight_bytes_stored": wbytes,
        "weight_bytes_operating_copies": 0,
        "mfma_ops_per_step": ops_per_step,
        "roofline": roof, "act_quant": quant,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = sweep_cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the quantized linear runs on one GPU; --gpus must be 1"}))
        raise SystemExit(2)
    import torch
    assert torch.cuda.is_available(), "bench needs a GPU"
    if args.copy_calibration:
        copy_calibration(torch)
        return
    import bit_post_quantization_amd  # noqa: F401  (raises if libqlinear.so is missing)

    if args.workload == "c5":
        bench_tasq_sweep(torch, args)
        return
    if args.workload == "c6":
        bench_tasq_weight_sweep(torch, args)
        return
    wl, Ls = layers_for(args.workload)
    layers = [Layer(torch, wl, L, use_branches=args.workload != "c7f") for L in Ls]
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step():
        for ly in layers:
            ly.quantize()
            ly.gemm()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region 1: K steps, events only at its two ends (the step time).
    start, end = ev(), ev()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps

    # Timed region 2: the same K steps with an event pair around every
    # launch on the launching stream (per-kernel durations; each pair also
    # brackets the dispatch of its launch, so these run a little above the
    # profiler's kernel-only figures).
    recs = [[[ev(), ev(), ev()] for _ in layers] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        for i, ly in enumerate(layers):
            e0, e1, e2 = recs[k][i]
            e0.record()
            ly.quantize()
            e1.record()
            ly.gemm()
            e2.record()
    torch.cuda.synchronize()

    q_ms = np.zeros(len(layers))
    g_ms = np.zeros(len(layers))
    for k in range(args.steps):
        for i in range(len(layers)):
            e0, e1, e2 = recs[k][i]
            q_ms[i] += e0.elapsed_time(e1)
            g_ms[i] += e1.elapsed_time(e2)
    q_ms /= args.steps
    g_ms /= args.steps

    # Timed region 3: per layer, `steps` launches of the same call back to
    # back between one event pair (launch-to-launch time: the kernel plus the
    # gap between dependent dispatches, without per-launch event overhead).
    # These durations feed the rooflines.
    def back_to_back(fn):
        a, b = ev(), ev()
        torch.cuda.synchronize()
        a.record()
        for _ in range(args.steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps
    qb_ms = np.array([back_to_back(ly.quantize) for ly in layers])
    gb_ms = np.array([back_to_back(ly.gemm) for ly in layers])
    # The quantizer with static scales (one pass over X at any size; TASQ's
    # per-step scale tables run it) on the layer with the most bytes.
    lys = max(layers, key=lambda ly: ly.quant_bytes)
    lys.static_scales = lys.scales.clone()
    lys.scales_out = torch.empty_like(lys.scales)
    lys.quantize_static()
    qs_ms = back_to_back(lys.quantize_static)

    step_ops = sum(ly.mfma_ops for ly in layers)
    value = step_ops / (ms_step * 1e-3) / 1e12
    # dominant kernel: the GEMM (k2), averaged over its launches in the step
    gemm_avg_s = float(np.mean(gb_ms)) * 1e-3
    ops_per_launch = float(np.mean([ly.mfma_ops for ly in layers]))
    gemm_tops = ops_per_launch / gemm_avg_s / 1e12
    qbytes = sum(ly.quant_bytes for ly in layers)
    q_gbps = qbytes / (float(np.sum(qb_ms)) * 1e-3) / 1e9

    per_layer = []
    for ly, q, g, qb, gb in zip(layers, q_ms, g_ms, qb_ms, gb_ms):
        per_layer.append({
            "layer": ly.L.name, "M": ly.M, "K": ly.L.K, "N": ly.L.N,
            "quant_us": round(qb * 1e3, 2), "quant_us_in_step_event_pair": round(q * 1e3, 2),
            "quant_gbps": round(ly.quant_bytes / (qb * 1e-3) / 1e9, 1),
            "gemm_us": round(gb * 1e3, 2), "gemm_us_in_step_event_pair": round(g * 1e3, 2),
            "gemm_tops": round(ly.mfma_ops / (gb * 1e-3) / 1e12, 1),
            "gemm_frac_int8_peak": round(ly.mfma_ops / (gb * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
            "gemm_executed_mfma_tops": round(ly.exec_ops / (gb * 1e-3) / 1e12, 1),
        })

    # K3, the standalone CFG combine, on the first layer's full output shape
    # (both halves of Y [M, N] in, [M/2, N] out): 12 bytes per output element.
    from bit_post_quantization_amd import qlinear_cfg_combine
    ly0 = layers[0]
    Yfull = torch.empty((ly0.M, ly0.L.N), dtype=torch.float32, device="cuda").normal_()
    Yc = torch.empty((ly0.M // 2, ly0.L.N), dtype=torch.float32, device="cuda")
    k3 = lambda: qlinear_cfg_combine(Yfull, ly0.M, ly0.L.N, 4.0, Yc)  # noqa: E731
    k3()
    k3_ms = back_to_back(k3)
    k3_bytes = 12.0 * (ly0.M // 2) * ly0.L.N
    del Yfull, Yc

    first = wl.layers[0] if args.workload != "mlp" else Ls[0]
    out = {
        "metric": "quantized-linear int8 TOPS (% MFMA peak) + act-quant GB/s, DiT-XL/2 MLP",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": DATA[first.x_kind],
        "config": {
            "workload": {"mlp": "DiT-XL/2 MLP fc1 1152->4608 + fc2 4608->1152",
                         "block": "DiT-XL/2 block QKV+proj+fc1+fc2",
                         "c3": "DiT-XL/2 block W4A4 + Hadamard-128",
                         "c3s": "DiT-XL/2 block W4A4, single Hadamard-128 on X only "
                                "(W as H W_int^T), symmetric activations",
                         "c4": "MM-DiT SegLinear layers W4 A4/A8",
                         "c4g": "MM-DiT SegLinear layers W4, A4/A8 by the greedy allocation",
                         "c7": "SegLinear input branches: [hidden|skip] 2304->1152 and "
                               "[temb 256|hidden 1152] 1408->1152, W8A8, CFG",
                         "c7f": "the c7 layers and inputs with one scale pair per tensor "
                                "(no input branches), for comparison"
                         }[args.workload],
            "M": wl.M, **SHAPE[wl.key], "cfg_guidance": first.guidance if first.cfg else None,
            "w_bits": first.w_bits, "a_bits": per_layer_or_one([L.a_bits for L in Ls]),
            "act_scales": first.a_scale,
            "weight_scales": per_layer_or_one([L.w_scale for L in Ls]),
            "hadamard_block": first.hadamard_block,
        },
        "roofline": {
            "kernel": "k2_gemm (int8 MFMA, both polarity planes, fused epilogue)",
            "bound": "mfma", "achieved": round(gemm_tops, 1), "peak": PEAK_INT8_TOPS,
            "unit": "TOPS", "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
            "ops_per_launch": ops_per_launch, "avg_launch_us": round(gemm_avg_s * 1e6, 2),
            "timing": "launch-to-launch time of back-to-back launches of each layer's GEMM "
                      "(HIP events on the launching stream), averaged over the layers",
            "traffic": measured_traffic() if args.workload == "mlp" else None,
        },
        "act_quant": {
            "kernels": "k1_fused (one pass) where X fits on chip, else k1_reduce + k1_quantize",
            "bound": "hbm",
            "achieved": round(q_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(q_gbps / PEAK_HBM_GBPS, 4),
            "bytes_per_step": qbytes,
            "timing": "launch-to-launch time of back-to-back quantize calls per layer",
        },
        "act_quant_static": {
            "kernel": "k1_quantize (static scales)", "bound": "hbm",
            "layer": lys.L.name, "shape": [lys.M, lys.L.K], "bytes_per_launch": lys.quant_bytes,
            "avg_launch_us": round(qs_ms * 1e3, 2),
            "achieved": round(lys.quant_bytes / (qs_ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": round(lys.quant_bytes / (qs_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        },
        "cfg_combine": {
            "kernel": "k3_cfg (standalone CFG combine)", "bound": "hbm",
            "shape": [ly0.M, ly0.L.N], "bytes_per_launch": k3_bytes,
            "avg_launch_us": round(k3_ms * 1e3, 2),
            "achieved": round(k3_bytes / (k3_ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": round(k3_bytes / (k3_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        },
        "effective_tops": round(sum(ly.eff_ops for ly in layers) / (ms_step * 1e-3) / 1e12, 2),
        "executed_mfma_tops": round(sum(ly.exec_ops for ly in layers) / (ms_step * 1e-3) / 1e12, 2),
        "layers": per_layer,
        "wall_s": round(wall, 3),
    }
    if args.workload in ("c4", "c4g"):
        out["bops"] = bops_report(Ls, wl.M)
    # the kernels against what the chip sustains (measured here), beside
    # their fractions of the spec peaks
    ceil = measured_ceilings(torch)
    out["ceilings"] = ceil
    out["roofline"]["frac_of_measured_ceiling"] = round(
        out["roofline"]["achieved"] / ceil["mfma_int8_random_operands_tops"], 4)
    out["act_quant"]["frac_of_measured_copy"] = round(
        out["act_quant"]["achieved"] / ceil["hbm_copy_gbps"], 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(layers, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
