"""Throughput of the FP8 W8A8 linear on one MI355X.

One step = the whole per-call hot path on one batch: dynamic per-token e4m3fn
quantisation of the bf16 activation, then the FP8 GEMM with the fused
activation-scale x weight-scale, bias and bf16 epilogue (two launches on one
stream). The headline workload is the FFN-up linear of the HunyuanVideo1.5 DiT
(M=4096 tokens, N=8192, K=2048). The weight is quantised per output channel and
the plan built before timing (construction-time work, as the method prescribes).

Inputs, weights and outputs rotate over enough independent sets (> 1 GiB in
total) that no step finds its operands in the 256 MB last-level cache; every
operand is resident in HBM when the timed region starts.

Prints one JSON line. `value` = 2 M N K / step time (TFLOP/s), from K steps timed
with events only at the two ends of the region, after 0.3 s of untimed back-to-back
steps (`preheat`: the clocks have dropped while the host built the inputs) and the W
warm-up steps. `roofline` is the GEMM kernel (the dominant launch): its average launch
duration comes from K launches of the GEMM alone, back to back with events on the
launch stream at the two ends; the quantiser's launches are too short to be fed from
Python one by one, so `quant.avg_launch_us` comes from K launches replayed from one HIP
graph. A second region of K steps with an event around every launch gives each kernel's
duration in its place in the step (`step_events_launch_us`: avg, p10, median, p90).
`roofline.traffic` is the HBM bytes per launch from the committed rocprofv3 counter
record, reported only while the GEMM's sources match the ones it was taken on.
`cpu_baseline` times the CPU oracle (numpy, float64) on a bounded sample of the same
workload.

Other legs (outside the headline step; `--legs` selects them):
  ffn_down      the FFN-down linear (M=4096, N=2048, K=8192, GELU(N(0,1)) input) as the
                same kind of step, with its own roofline and quantiser records
  quant_large   the per-token quantiser alone at [32760, 2048], [4096, 8192] and
                [32760, 8192] (graph-replayed launches over rotating inputs and outputs)
  w8a16         the FP8 weight-only linear (bf16 activation x per-channel e4m3fn weight
                on the bf16 matrix cores) on the FFN-up shape, against the bf16 peak
  producer      GELU (tanh form) -> per-token e4m3fn in one kernel against the unfused
                pair, at [4096, 8192] and [32760, 8192]
  tensor_quant  the per-tensor state-dict conversion (e4m3fn and e5m2) of [8192, 2048]
                and [32760, 8192]
  quant_gemm    the FFN-up step as one launch against the two-launch step
  blocks        the QKV config (one quantisation of [32760, 2048], three GEMMs, the
                26-row encoder input through the same weights) and the DiT block (4
                quantisations, 6 GEMMs at 32760 tokens) as whole steps, the GEMMs on
                one activation run as a group, beside the same step with separate calls
  cpu           the CPU oracle baseline

`clocks` reads the shader and memory clocks with amd-smi while the FFN-up step runs
back to back, and gives the GEMM's fraction of the dense-FP8 peak at that shader clock
(256 CUs x 8192 flop per clock) beside `roofline.frac`, which uses the published
2.4 GHz peak.
"""

import argparse
import ctypes
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 W8A8 linear TFLOP/s (quant+GEMM+epilogue), M4096 N8192 K2048; quant GB/s"
M, N, K = 4096, 8192, 2048
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP8_FLOP_PER_CU_CLK = 8192  # dense FP8 MFMA per CU per shader clock (5.0 PFLOP/s = 256 CUs x 8192 x 2.4 GHz)
N_CUS = 256
PERSISTENT_CONFIG = 6  # the persistent 256 x 256 GEMM form, the plan's choice at FFN-up
TRAFFIC_FILES = {name: os.path.join(ROOT, "profiles", f"gemm_fp8_{name}_traffic.json") for name in ("ffn_up", "ffn_down")}
# the FP8 GEMM kernel's sources (the committed counter record names the SHA-256 over both)
GEMM_SOURCES = [os.path.join(ROOT, "fp8_w8a8_quantized_token_amd", "csrc", f) for f in ("gemm_fp8.hip", "gemm_common.h")]


def gemm_bytes(m, n, k):
    # q8 A, q8 W, bf16 out, fp32 a-scale, fp32 w-scale, bf16 bias
    return m * k + n * k + 2 * m * n + 4 * m + 4 * n + 2 * n


def pct(sorted_xs, p):
    """p-th percentile (nearest rank) of an ascending list."""
    return sorted_xs[min(len(sorted_xs) - 1, max(0, round(p / 100 * (len(sorted_xs) - 1))))]


def quant_bytes(m, k):
    return 3 * m * k + 4 * m  # read bf16, write codes and fp32 scales


def traffic_from_profile(path):
    """HBM bytes per GEMM launch from a committed rocprofv3 counter record, if still current."""
    try:
        with open(path) as f:
            t = json.load(f)
        h = hashlib.sha256()
        for path in GEMM_SOURCES:
            with open(path, "rb") as f:
                h.update(f.read())
        src = h.hexdigest()
        if t.get("gemm_source_sha256") != src:
            return None
        return float(t["hbm_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def preheat(torch, fn, seconds=0.15, batch=20):
    """Call fn(i) back to back for about `seconds` (untimed), so a measurement that follows
    host-side set-up does not start while the clocks ramp up from idle. Returns the calls made."""
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


PRODUCER_SHAPES = ((4096, 8192, 8), (32760, 8192, 2))  # rows, cols, rotating input sets


def producer_bench(torch, fp8, lib, dev, stream, steps, only_rows=None):
    """Fused GELU -> per-token FP8 producer against the unfused pair, HBM-resident inputs."""
    from fp8_w8a8_quantized_token_amd import _lib
    from workloads.synth import activation
    table = fp8.act_table("gelu_tanh", dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def call(st, name):
        if st:
            raise _lib.Fp8W8A8Error(st, name)

    out = {"activation": "gelu_tanh", "bound": "hbm", "peak": PEAK_HBM_GBPS, "unit": "GB/s", "shapes": []}
    for rows, cols, nsets in PRODUCER_SHAPES:
        if only_rows is not None and rows != only_rows:
            continue
        xs = [activation(0, 3, 40 + i, rows, cols, "normal").to(dev) for i in range(nsets)]
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        sc = torch.empty((rows,), dtype=torch.float32, device=dev)
        y = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)

        def fused(i):
            call(lib.fp8_act_quant_rows(p(xs[i % nsets]), rows, cols, p(table), p(q), p(sc), sptr),
                 "fp8_act_quant_rows")

        def unfused(i):
            call(lib.fp8_act_rows(p(xs[i % nsets]), rows, cols, p(table), p(y), sptr), "fp8_act_rows")
            call(lib.fp8_quant_rows(p(y), rows, cols, p(q), p(sc), sptr), "fp8_quant_rows")

        res = {}
        for name, fn in (("fused", fused), ("unfused", unfused)):
            preheat(torch, fn)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(steps):
                fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) * 1e3 / steps
        algo = quant_bytes(rows, cols)
        gbps = algo / (res["fused"] * 1e-6) / 1e9
        out["shapes"].append({
            "rows": rows, "cols": cols, "fused_us": round(res["fused"], 2), "unfused_us": round(res["unfused"], 2),
            "speedup": round(res["unfused"] / res["fused"], 3), "algorithmic_bytes_per_launch": algo,
            "achieved": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4),
        })
        del xs, q, sc, y
        torch.cuda.empty_cache()
    return out


def _smi_clocks(text):
    """Mean shader and memory clock in MHz from `amd-smi metric --clock --json` (None if absent)."""
    d = json.loads(text)
    gpus = d["gpu_data"] if isinstance(d, dict) and "gpu_data" in d else d
    c = gpus[0]["clock"]
    gfx = [v["clk"]["value"] for key, v in c.items() if key.startswith("gfx_") and isinstance(v, dict)]
    mem = [v["clk"]["value"] for key, v in c.items() if key.startswith("mem") and isinstance(v, dict)]
    mean = lambda xs: round(sum(float(x) for x in xs) / len(xs), 1) if xs else None
    return mean(gfx), mean(mem)


def sample_clocks(torch, step, samples=2, warm_s=0.5):
    """Shader (SCLK) and memory (MCLK) clocks read with amd-smi while `step` runs back to back.

    The launches go on in this thread while each amd-smi child process runs, so every sample
    is taken under the timed workload. Returns None when amd-smi is not available."""
    try:
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < warm_s:
            for _ in range(20):
                step(i)
                i += 1
            torch.cuda.synchronize()
        gfx, mem = [], []
        for _ in range(samples):
            p = subprocess.Popen(["amd-smi", "metric", "--clock", "--json"], stdout=subprocess.PIPE,
                                 stderr=subprocess.DEVNULL, text=True)
            t1 = time.perf_counter()
            while p.poll() is None and time.perf_counter() - t1 < 30:
                for _ in range(20):
                    step(i)
                    i += 1
                torch.cuda.synchronize()
            out, _ = p.communicate(timeout=30)
            g, m = _smi_clocks(out)
            if g is not None:
                gfx.append(g)
            if m is not None:
                mem.append(m)
        if not gfx:
            return None
        return {"sclk_mhz": round(sum(gfx) / len(gfx), 1),
                "mclk_mhz": round(sum(mem) / len(mem), 1) if mem else None,
                "samples": len(gfx), "source": "amd-smi metric --clock (mean over XCDs) during back-to-back steps"}
    except (OSError, ValueError, KeyError, IndexError, TypeError, subprocess.SubprocessError):
        return None


def copy_calibration(torch, dev):
    """Three plain 1 GiB device-to-device copies: a kernel of known traffic for scaling counters."""
    src = torch.ones((1 << 28,), dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def w8a16_bench(torch, fp8, lib, dev, stream, steps, nsets=12):
    """FP8 weight-only linear on the FFN-up shape: per-launch events on the launch stream."""
    from workloads.synth import activation, bias as gen_bias, weight
    sptr = ctypes.c_void_p(stream.cuda_stream)
    sets = []
    for i in range(nsets):
        a = activation(0, 2, 60 + i, M, K, "normal").to(dev)
        lin = fp8.Fp8WeightOnlyLinear(weight(0, 2, 160 + i, N, K).to(dev), gen_bias(0, 2, 260 + i, N).to(dev))
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        sets.append((a, lin, out))
    torch.cuda.synchronize()

    def run(i):
        a, lin, out = sets[i % nsets]
        st = lib.fp8_w8a16_run(lin._plan, M, ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(out.data_ptr()), sptr)
        if st:
            from fp8_w8a8_quantized_token_amd import _lib
            raise _lib.Fp8W8A8Error(st, "fp8_w8a16_run")

    preheat(torch, run)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        evs[i][0].record(stream)
        run(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    # average launch duration: the same launches back to back, events only at the ends
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        run(i)
    e1.record(stream)
    torch.cuda.synchronize()
    avg = e0.elapsed_time(e1) / steps
    tflops = 2.0 * M * N * K / (avg * 1e-3) / 1e12
    cid, tm, tn, wg = sets[0][1].config(M)
    del sets
    torch.cuda.empty_cache()
    return {"kernel": "gemm_w8a16_kernel", "M": M, "N": N, "K": K, "avg_launch_us": round(avg * 1e3, 3),
            "median_launch_us_events": round(pct(ts, 50) * 1e3, 3), "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "bound": "mfma", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "config": {"id": cid, "tile_m": tm, "tile_n": tn, "workgroups": wg}}


def quant_gemm_bench(torch, fp8, lib, dev, stream, steps, nsets=12):
    """The FFN-up step as one launch (fp8_quant_gemm, the 256 x 256 tiles of configuration
    0) against the same step as two launches: fp8_quant_rows, then configuration 0 (the
    same tiles), and fp8_quant_rows, then the configuration the plan runs at this shape
    (the persistent 256 x 256 form, 6). Same inputs and loop shape, events only at the
    ends of `steps` back-to-back steps."""
    from workloads.synth import activation, bias as gen_bias, weight
    from fp8_w8a8_quantized_token_amd import _lib
    sptr = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    ws_bytes = lib.fp8_quant_gemm_workspace_bytes(M, K)
    codes_bytes = (M * K + 255) // 256 * 256
    sets = []
    for i in range(nsets):
        a = activation(0, 2, 70 + i, M, K, "normal").to(dev)
        qw, sw = fp8.quant_weights_per_channel(weight(0, 2, 170 + i, N, K).to(dev))
        b = gen_bias(0, 2, 270 + i, N).to(dev)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
        sets.append((a, qw, sw, b, out, ws))
    torch.cuda.synchronize()

    def one(i):
        a, qw, sw, b, out, ws = sets[i % nsets]
        st = lib.fp8_quant_gemm(M, N, K, P(a), P(qw), P(sw), P(b), P(out), P(ws), ws_bytes, sptr)
        if st:
            raise _lib.Fp8W8A8Error(st, "fp8_quant_gemm")

    def two_with(config):
        def two(i):
            a, qw, sw, b, out, ws = sets[i % nsets]
            scales = ctypes.c_void_p(ws.data_ptr() + codes_bytes)
            st = lib.fp8_quant_rows(P(a), M, K, P(ws), scales, sptr)
            st = st or lib.fp8_gemm_run_config(config, M, N, K, P(ws), scales, P(qw), P(sw), P(b), P(out), sptr)
            if st:
                raise _lib.Fp8W8A8Error(st, "fp8_quant_rows / fp8_gemm_run_config")
        return two

    two, two_p = two_with(0), two_with(PERSISTENT_CONFIG)
    res = {}
    for name, run in (("two_launch", two), ("single_launch", one), ("two_launch_persistent", two_p),
                      ("two_launch_again", two), ("single_launch_again", one),
                      ("two_launch_persistent_again", two_p)):
        preheat(torch, run)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            run(i)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps * 1e3
    del sets
    torch.cuda.empty_cache()
    two_us = min(res["two_launch"], res["two_launch_again"])
    one_us = min(res["single_launch"], res["single_launch_again"])
    two_p_us = min(res["two_launch_persistent"], res["two_launch_persistent_again"])
    flop = 2.0 * M * N * K
    return {"kernel": "gemm_fp8_kernel (single-launch form)", "M": M, "N": N, "K": K, "steps": steps,
            "single_launch_us_per_step": round(one_us, 3), "two_launch_us_per_step": round(two_us, 3),
            "two_launch_persistent_us_per_step": round(two_p_us, 3),
            "single_launch_tflops": round(flop / (one_us * 1e-6) / 1e12, 2),
            "two_launch_tflops": round(flop / (two_us * 1e-6) / 1e12, 2),
            "two_launch_persistent_tflops": round(flop / (two_p_us * 1e-6) / 1e12, 2),
            "speedup": round(two_us / one_us, 4),
            "speedup_vs_persistent_two_launch": round(two_p_us / one_us, 4)}


def block_bench(torch, fp8, lib, dev, stream, steps, config):
    """A whole synthetic config as one step: each activation quantised once per token, then
    every linear that reads it (QKV: one quantisation, three GEMMs, plus the 26-row encoder
    input through the same three weights; DiT block: 4 quantisations, 6 GEMMs)."""
    from fp8_w8a8_quantized_token_amd import _lib
    from workloads.synth import layer_specs, make_config
    sptr = ctypes.c_void_p(stream.cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    cfg = make_config(config)
    acts = {name: a.to(dev) for name, a in cfg["activations"].items()}
    codes = {name: (torch.empty(a.shape, dtype=torch.uint8, device=dev),
                    torch.empty((a.shape[0],), dtype=torch.float32, device=dev)) for name, a in acts.items()}
    lins, outs, flop = {}, {}, 0.0
    for layer, act, m, n, k in layer_specs(config):
        lins[layer] = fp8.Fp8Linear(cfg["weights"][layer].to(dev), cfg["biases"][layer].to(dev))
        outs[layer] = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        flop += 2.0 * m * n * k
    del cfg
    order = [(name, [(layer, act_m) for layer, act, act_m, _, _ in layer_specs(config) if act == name])
             for name in acts]

    # the layers reading one activation go out as one group (fp8_linear_run_group: one
    # persistent launch over all their tiles when each would take that form), and, for
    # comparison, as separate fp8_linear_run calls
    groups = {}
    for name, layers in order:
        g = len(layers)
        groups[name] = ((ctypes.c_void_p * g)(*[lins[layer]._plan.value for layer, _ in layers]),
                        (ctypes.c_void_p * g)(*[outs[layer].data_ptr() for layer, _ in layers]))

    def run(grouped):
        def step(_i):
            for name, layers in order:
                a = acts[name]
                q, sc = codes[name]
                st = lib.fp8_quant_rows(p(a), a.shape[0], a.shape[1], p(q), p(sc), sptr)
                if st:
                    raise _lib.Fp8W8A8Error(st, "fp8_quant_rows")
                if grouped:
                    plans, optrs = groups[name]
                    st = lib.fp8_linear_run_group(ctypes.cast(plans, ctypes.c_void_p), len(layers), layers[0][1], p(q),
                                                  _lib.A_E4M3, p(sc), ctypes.cast(optrs, ctypes.c_void_p), None, 0,
                                                  sptr)
                    if st:
                        raise _lib.Fp8W8A8Error(st, "fp8_linear_run_group")
                    continue
                for layer, m in layers:
                    st = lib.fp8_linear_run(lins[layer]._plan, m, p(q), _lib.A_E4M3, p(sc), p(outs[layer]), None, 0,
                                            sptr)
                    if st:
                        raise _lib.Fp8W8A8Error(st, "fp8_linear_run")

        return step

    steps_of = {False: run(False), True: run(True)}
    for fn in steps_of.values():
        preheat(torch, fn, batch=5)
    # the two forms alternate (5 rounds each, median): one run of each after the other
    # differed by +-2% from order and clock alone
    times = {False: [], True: []}
    for rnd in range(10):
        grouped = (rnd % 2 == 1) if (rnd // 2) % 2 == 0 else (rnd % 2 == 0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            steps_of[grouped](i)
        e1.record(stream)
        torch.cuda.synchronize()
        times[grouped].append(e0.elapsed_time(e1) / steps)
    ms_sep = sorted(times[False])[2]
    ms = sorted(times[True])[2]
    res = {"quantisations": len(order), "gemms": len(lins), "steps": steps, "rounds": 5, "flop_per_step": flop,
           "ms_per_step": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
           "grouped": True, "ms_per_step_separate_gemms": round(ms_sep, 4),
           "gemm_configs": {layer: lin.config(outs[layer].shape[0])[0] for layer, lin in lins.items()},
           # the configuration of each activation's single grouped launch (-1: its layers' own GEMMs)
           "group_configs": {name: fp8.group_config([lins[layer] for layer, _ in layers], layers[0][1])
                             for name, layers in order}}
    del acts, codes, lins, outs
    torch.cuda.empty_cache()
    return res


def tensor_quant_bench(torch, fp8, lib, dev, stream, steps):
    """Per-tensor quantisation (both formats), HBM-resident rotating inputs: the form
    fp8_quant_tensor picks (one pass up to 65536 elements per CU, else two passes), and
    at the shape that fits one pass the other form beside it."""
    from fp8_w8a8_quantized_token_amd import _lib
    from workloads.synth import activation
    sptr = ctypes.c_void_p(stream.cuda_stream)
    ws = torch.empty((lib.fp8_quant_tensor_workspace_bytes(),), dtype=torch.uint8, device=dev)
    scale = torch.empty((1,), dtype=torch.float32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = {"bound": "hbm", "peak": PEAK_HBM_GBPS, "unit": "GB/s", "shapes": []}
    for rows, cols, nsets in ((8192, 2048, 16), (32760, 8192, 2)):
        xs = [activation(0, 5, 80 + i, rows, cols, "normal").to(dev) for i in range(nsets)]
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        fits = rows * cols <= 65536 * cus
        for fmt_name, fmt in (("e4m3fn", _lib.FMT_E4M3FN), ("e5m2", _lib.FMT_E5M2)):
            one_pass = fits  # what fp8_quant_tensor picks
            def timed(form):
                def run(i):
                    st = lib.fp8_quant_tensor_form(form, ctypes.c_void_p(xs[i % nsets].data_ptr()), rows * cols, fmt,
                                                   ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(scale.data_ptr()),
                                                   ctypes.c_void_p(ws.data_ptr()), ws.numel(), sptr)
                    if st:
                        raise _lib.Fp8W8A8Error(st, "fp8_quant_tensor_form")
                preheat(torch, run)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(stream)
                for i in range(steps):
                    run(i)
                e1.record(stream)
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) * 1e3 / steps
            us = timed(_lib.TENSOR_FORMS["auto"])
            algo = 3 * rows * cols + 4
            rec = {"rows": rows, "cols": cols, "format": fmt_name, "form": "one_pass" if one_pass else "two_pass",
                   "us": round(us, 2), "algorithmic_bytes": algo, "achieved": round(algo / (us * 1e-6) / 1e9, 1),
                   "hbm_bytes_of_form": (3 if one_pass else 5) * rows * cols + 4,
                   "frac": round(algo / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
            if fits:  # the other form, for comparison
                other = "two_pass" if one_pass else "one_pass"
                rec[other + "_us"] = round(timed(_lib.TENSOR_FORMS[other]), 2)
            out["shapes"].append(rec)
        del xs, q
        torch.cuda.empty_cache()
    return out


def cpu_baseline(budget_s=20.0):
    """The CPU oracle (as it stands) on the FFN-up workload: quant + exact float64 linear."""
    import numpy as np
    from oracle import linear as ol, quant as oq
    from workloads import bf16_bits, make_config
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        blas_threads = None
    cfg = make_config("ffn_up")
    a = bf16_bits(cfg["activations"]["a"])
    w = bf16_bits(cfg["weights"]["ffn_up"])
    b = bf16_bits(cfg["biases"]["ffn_up"])
    qw, sw = oq.quant_weights_per_channel(w)  # construction-time, not timed
    # bounded sample: the first R rows of the activation, R chosen from a trial run
    rows = 256
    t0 = time.perf_counter()
    ol.linear_ref(a[:rows], qw, sw, b)
    t_trial = time.perf_counter() - t0
    rows = int(min(M, max(256, rows * budget_s / 3 / max(t_trial, 1e-3))))
    best = None
    for _ in range(3):
        t0 = time.perf_counter()
        ol.linear_ref(a[:rows], qw, sw, b)
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
    tflops = 2.0 * rows * N * K / best / 1e12
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {
        "value": tflops,
        "unit": "TFLOP/s",
        "cores": blas_threads or cores,
        "kind": "oracle",
        "sample": f"first {rows} of {M} token rows of the FFN-up workload (N={N}, K={K}): numpy per-token quant "
                  f"(1 core) + float64 exact dequantised matmul (BLAS threads={blas_threads}, affinity {cores} "
                  f"cores) + epilogue; best of 3, {best:.2f} s each; scaled to TFLOP/s by 2*rows*N*K",
    }


# The two FFN linears of the block as timed steps (quantise + GEMM), each over its own
# rotating sets: FFN-up is the headline workload, FFN-down (the GELU output as input, k =
# 8192) the second shape the GEMM bar is quoted on.
LINEAR_LEGS = {
    "ffn_up": {
        "M": 4096, "N": 8192, "K": 2048, "config_id": 2, "kind": "outlier", "sets": 16,
        "workload": "FFN-up linear M4096 N8192 K2048: bf16 activation N(0,1) with 1% channels x50 -> "
                    "per-token e4m3fn quant -> FP8 GEMM vs per-channel e4m3fn weight N(0,1/sqrt(2048)) "
                    "-> x a_scale x w_scale + bf16 bias -> bf16",
    },
    "ffn_down": {
        "M": 4096, "N": 2048, "K": 8192, "config_id": 3, "kind": "gelu", "sets": 12,
        "workload": "FFN-down linear M4096 N2048 K8192: bf16 activation GELU(N(0,1)) -> per-token e4m3fn "
                    "quant -> FP8 GEMM vs per-channel e4m3fn weight N(0,1/sqrt(8192)) -> x a_scale x w_scale "
                    "+ bf16 bias -> bf16",
    },
}

# Per-token quantiser at the large activation shapes of the configs: the QKV / DiT hidden
# input, the FFN-down input at 4096 tokens, the DiT FFN-down input (rows, cols, kind,
# config id, rotating sets; every set has its own input and its own code / scale buffers).
QUANT_SHAPES = ((32760, 2048, "outlier", 4, 4), (4096, 8192, "gelu", 3, 8), (32760, 8192, "outlier", 5, 2))


def _check_status(st, where):
    if st:
        from fp8_w8a8_quantized_token_amd import _lib
        raise _lib.Fp8W8A8Error(st, where)


def graph_avg(torch, dev, stream, fn, launches):
    """`launches` calls of fn(i, stream_ptr) captured in one HIP graph and replayed once with
    events at its two ends -> average duration per launch (ms). For launches too short to be
    fed from Python one by one without the GPU waiting on the host in between."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fn(0, ctypes.c_void_p(side.cuda_stream))
    side.synchronize()
    with torch.cuda.graph(g, stream=side):
        cap = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        for i in range(launches):
            fn(i, cap)
    torch.cuda.synchronize()
    g.replay()  # the first replay uploads the graph
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / launches


def back_to_back(torch, stream, fn, launches):
    """`launches` calls of fn(i) with events on the launch stream at the two ends -> ms per call."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(launches):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / launches


def linear_leg(torch, fp8, lib, dev, stream, name, steps, warmup, preheat_s, nsets=None, clocks=False):
    """One FFN linear as a timed step: per-token quantisation of the bf16 activation, then the
    plan's GEMM with the fused epilogue, over rotating input / weight / output sets."""
    from fp8_w8a8_quantized_token_amd import _lib
    from workloads.synth import activation, bias as gen_bias, outlier_channels, weight
    spec = LINEAR_LEGS[name]
    m, n, k, cid = spec["M"], spec["N"], spec["K"], spec["config_id"]
    nsets = nsets or spec["sets"]
    sptr = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    ch = outlier_channels(0, cid, 0, k, None) if spec["kind"] == "outlier" else None
    sets = []
    for i in range(nsets):
        a = activation(0, cid, 10 + i, m, k, spec["kind"], ch).to(dev)
        w = weight(0, cid, 100 + i, n, k).to(dev)
        b = gen_bias(0, cid, 200 + i, n).to(dev)
        lin = fp8.Fp8Linear(w, b)  # per-channel weight quant + plan: construction time
        del w
        q = torch.empty((m, k), dtype=torch.uint8, device=dev)
        s = torch.empty((m,), dtype=torch.float32, device=dev)
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        sets.append((a, q, s, lin, out))
    torch.cuda.synchronize()
    config = sets[0][3].config(m)

    def quant_only(i, on=sptr):
        a, q, s, lin, out = sets[i % nsets]
        _check_status(lib.fp8_quant_rows(P(a), m, k, P(q), P(s), on), "fp8_quant_rows")

    def gemm_only(i):
        a, q, s, lin, out = sets[i % nsets]
        _check_status(lib.fp8_linear_run(lin._plan, m, P(q), _lib.A_E4M3, P(s), P(out), None, 0, sptr),
                      "fp8_linear_run")

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        quant_only(i)
        if ev is not None:
            ev[1].record(stream)
        gemm_only(i)
        if ev is not None:
            ev[2].record(stream)

    # Pre-heat: after the host-side set-up the GPU has idled and its clocks have dropped;
    # without this the first few milliseconds of steps run while they ramp back up.
    t_pre = time.perf_counter()
    preheat_steps = preheat(torch, step, preheat_s, batch=50)
    preheat_wall = time.perf_counter() - t_pre
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region 1: exactly K steps, events only at its ends -> ms_per_step, value.
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / steps

    # Timed region 2: the same K steps with an event on the launch stream around every
    # launch -> each kernel's launch duration inside the step (avg, p10 / median / p90).
    # An event between two launches adds a wait of its own to the interval it closes.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    quant_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    gemm_ms = sorted(e[1].elapsed_time(e[2]) for e in evs)

    # Timed regions 3 and 4: K launches of each kernel alone over the same rotating sets,
    # events on the launch stream at the two ends only -> each kernel's average launch
    # duration (the roofline figures). The GEMM's launches go back to back from Python;
    # the quantiser's are replayed from one graph.
    g_avg = back_to_back(torch, stream, gemm_only, steps)
    q_avg_eager = back_to_back(torch, stream, quant_only, steps)
    q_avg = graph_avg(torch, dev, stream, quant_only, steps)

    clk = sample_clocks(torch, step) if clocks else None
    flop = 2.0 * m * n * k
    gemm_tflops = flop / (g_avg * 1e-3) / 1e12
    res = {
        "workload": spec["workload"], "M": m, "N": n, "K": k, "rotating_sets": nsets,
        "gemm_config": {"id": config[0], "tile_m": config[1], "tile_n": config[2], "workgroups": config[3]},
        "preheat": {"seconds": round(preheat_wall, 3), "steps": preheat_steps},
        "steps": steps, "ms_per_step": round(ms_per_step, 5),
        "tflops": round(flop / (ms_per_step * 1e-3) / 1e12, 2),
        "roofline": {
            "bound": "mfma",
            "kernel": "gemm_fp8_kernel",
            "achieved": round(gemm_tflops, 2),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
            "traffic": traffic_from_profile(TRAFFIC_FILES[name]),
            "avg_launch_us": round(g_avg * 1e3, 3),
            "avg_launch_us_source": "K GEMM launches back to back, events at the two ends",
            "algorithmic_flop_per_launch": flop,
            "algorithmic_bytes_per_launch": gemm_bytes(m, n, k),
            "step_events_launch_us": {"avg": round(sum(gemm_ms) / len(gemm_ms) * 1e3, 3),
                                      "p10": round(pct(gemm_ms, 10) * 1e3, 3),
                                      "median": round(pct(gemm_ms, 50) * 1e3, 3),
                                      "p90": round(pct(gemm_ms, 90) * 1e3, 3)},
        },
        "quant": {
            "kernel": "quant_rows_regs" if k <= 2048 else "quant_rows_split",
            "avg_launch_us": round(q_avg * 1e3, 3),
            "avg_launch_us_source": "K launches replayed from one HIP graph, events at the two ends",
            "avg_launch_us_eager_back_to_back": round(q_avg_eager * 1e3, 3),
            "step_events_launch_us": {"avg": round(sum(quant_ms) / len(quant_ms) * 1e3, 3),
                                      "p10": round(pct(quant_ms, 10) * 1e3, 3),
                                      "median": round(pct(quant_ms, 50) * 1e3, 3),
                                      "p90": round(pct(quant_ms, 90) * 1e3, 3)},
            "gbps": round(quant_bytes(m, k) / (q_avg * 1e-3) / 1e9, 1),
            "frac_hbm": round(quant_bytes(m, k) / (q_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "algorithmic_bytes_per_launch": quant_bytes(m, k),
        },
    }
    if clk is not None:
        # Peak at the clock the chip actually ran: 256 CUs x 8192 FP8 flop per CU per clock.
        sclk_peak = N_CUS * FP8_FLOP_PER_CU_CLK * clk["sclk_mhz"] * 1e6 / 1e12
        clk["gemm_peak_at_sclk_tflops"] = round(sclk_peak, 1)
        clk["gemm_frac_at_sclk"] = round(gemm_tflops / sclk_peak, 4)
    res["clocks"] = clk
    del sets
    torch.cuda.empty_cache()
    return res


def quant_large_bench(torch, lib, dev, stream, steps):
    """Per-token quantiser alone at the large activation shapes: K launches replayed from one
    HIP graph over rotating inputs and outputs, events at the two ends."""
    from workloads.synth import activation, outlier_channels
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    out = {"kernel": "quant_rows_regs / quant_rows_split", "bound": "hbm", "peak": PEAK_HBM_GBPS, "unit": "GB/s",
           "shapes": []}
    for rows, cols, kind, cid, nsets in QUANT_SHAPES:
        ch = outlier_channels(0, cid, 0, cols, None) if kind == "outlier" else None
        bufs = []
        for i in range(nsets):
            x = activation(0, cid, 30 + i, rows, cols, kind, ch).to(dev)
            q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
            s = torch.empty((rows,), dtype=torch.float32, device=dev)
            bufs.append((x, q, s))
        torch.cuda.synchronize()

        def run(i, on):
            x, q, s = bufs[i % nsets]
            _check_status(lib.fp8_quant_rows(P(x), rows, cols, P(q), P(s), on), "fp8_quant_rows")

        sptr = ctypes.c_void_p(stream.cuda_stream)
        preheat(torch, lambda i: run(i, sptr))
        ms = graph_avg(torch, dev, stream, run, steps)
        algo = quant_bytes(rows, cols)
        gbps = algo / (ms * 1e-3) / 1e9
        out["shapes"].append({"rows": rows, "cols": cols, "input": kind, "rotating_sets": nsets,
                              "avg_launch_us": round(ms * 1e3, 3), "algorithmic_bytes_per_launch": algo,
                              "achieved": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4)})
        del bufs
        torch.cuda.empty_cache()
    return out


LEGS = ("ffn_up", "ffn_down", "quant_large", "w8a16", "producer", "tensor_quant", "quant_gemm", "blocks", "cpu")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=None, help="rotating input/weight/output sets of the FFN legs")
    ap.add_argument("--preheat-s", type=float, default=0.3,
                    help="seconds of back-to-back steps before the warm-up steps, so the timed steps run at "
                         "the clocks the chip holds under this load rather than while it ramps up from idle")
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma-separated legs to run (default: all); without ffn_up the line carries only the "
                         f"legs' records (for kernel profiles). Legs: {', '.join(LEGS)}")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clocks", action="store_true", help="skip the amd-smi clock samples")
    ap.add_argument("--producer-only", type=int, metavar="ROWS", choices=[r for r, _, _ in PRODUCER_SHAPES],
                    help="time only the producer, at one row count (for kernel profiles)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run 3 plain 1 GiB device-to-device copies (a known-size kernel "
                         "for scaling HBM counter readings)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(tokens would shard across GPUs with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)
    legs = [x.strip() for x in args.legs.split(",") if x.strip()]
    unknown = [x for x in legs if x not in LEGS]
    if unknown:
        ap.error(f"unknown legs {unknown}; choose from {LEGS}")
    if args.no_cpu_baseline and "cpu" in legs:
        legs.remove("cpu")

    import torch
    import fp8_w8a8_quantized_token_amd as fp8
    from fp8_w8a8_quantized_token_amd import _lib

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda", 0)
    lib = _lib.lib()
    stream = torch.cuda.current_stream(dev)

    if args.producer_only:
        res = producer_bench(torch, fp8, lib, dev, stream, max(10, min(args.steps, 100)), args.producer_only)
        if args.copy_calibration:
            copy_calibration(torch, dev)
            res["copy_calibration_bytes"] = {"read": 1 << 30, "write": 1 << 30, "launches": 3}
        print(json.dumps({"producer": res}), flush=True)
        return

    result = {}
    if "ffn_up" in legs:
        up = linear_leg(torch, fp8, lib, dev, stream, "ffn_up", args.steps, args.warmup, args.preheat_s, args.sets,
                        clocks=not args.no_clocks)
        m, n, k = up["M"], up["N"], up["K"]
        result = {
            "metric": METRIC,
            "value": up["tflops"],
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "preheat": up["preheat"],
            "ms_per_step": up["ms_per_step"],
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "fp8e4m3 (fp32 accumulate, bf16 out)",
            "data": "synthetic",
            "config": {"workload": up["workload"], "M": m, "N": n, "K": k, "rotating_sets": up["rotating_sets"],
                       "gemm_config": up["gemm_config"]},
            "roofline": up["roofline"],
            "quant": up["quant"],
            "clocks": up["clocks"],
        }
    short = max(10, min(args.steps, 100))
    if "ffn_down" in legs:
        down = linear_leg(torch, fp8, lib, dev, stream, "ffn_down", args.steps, args.warmup, args.preheat_s,
                          args.sets, clocks=False)
        down.pop("clocks", None)
        result["ffn_down"] = down
    if "quant_large" in legs:
        result["quant_large"] = quant_large_bench(torch, lib, dev, stream, short)
    if "w8a16" in legs:
        result["w8a16"] = w8a16_bench(torch, fp8, lib, dev, stream, short)
    if "producer" in legs:
        result["producer"] = producer_bench(torch, fp8, lib, dev, stream, short)
    if "tensor_quant" in legs:
        result["tensor_quant"] = tensor_quant_bench(torch, fp8, lib, dev, stream, max(10, min(args.steps, 50)))
    if "quant_gemm" in legs:
        result["quant_gemm"] = quant_gemm_bench(torch, fp8, lib, dev, stream, short)
    if "blocks" in legs:
        result["configs"] = {name: block_bench(torch, fp8, lib, dev, stream, max(5, min(args.steps, 20)), name)
                             for name in ("qkv", "dit_block")}
    if args.copy_calibration:
        copy_calibration(torch, dev)
        result["copy_calibration_bytes"] = {"read": 1 << 30, "write": 1 << 30, "launches": 3}
    if "cpu" in legs:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
