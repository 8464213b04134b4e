#!/usr/bin/env python3
"""Benchmark of the union-path SwitchGLU-q4 MoE layer on one MI355X.

Metric: microseconds per MoE layer and effective expert-weight GB/s at
L = 1, 2, 4, 8 tokens on the GLM-5.2-style verify workload (E=256 experts,
top-8, hidden 6144, expert intermediate 2048, 4-bit affine group 64, bf16
activations), 75 layers chained with distinct weights and routes whose
adjacent-token overlap follows the measured depth-graded profile.

* Effective GB/s = unique experts x bytes per expert / time, where bytes per
  expert count the 4-bit codes plus the bf16 scales and biases of gate, up and
  down (the mlx issue "gather_qmm at M=1 streams 4-bit expert weights at ~half
  the bandwidth of M=4", section "Numbers", counts bytes per expert this way;
  here only distinct experts count, not token x top-k slots).
* A step is one pass over the chains (L = 1, 2, 3, 4, 8; 75 layers each);
  the headline value aggregates the chains at L = 1, 2, 4, 8 (total unique
  bytes / total time) and per_L reports every L.
  Inputs are resident in HBM before timing.  Two timing modes, as on the
  pages ("chained" and "isolated" in the issue above; in-graph and
  eval-per-call in the mlx discussion "Small-L fused expert gather for
  fine-grained MoE decode"):
  - chained: every layer of a chain is enqueued back to back on one stream
    with HIP events only at the chain ends; a GPU delay kernel ahead of each
    chain lets the host enqueue the whole chain first, so the events time the
    GPU, not Python.  This is the headline.
  - isolated: one layer between two events, median of 60, the layers rotated
    so no two consecutive reps share a bank (every chain holds > 1 GiB of
    banks, four times the 256 MiB Infinity Cache).  isolated_gpu puts a delay
    kernel before every rep (GPU time of a cold layer); isolated_eager
    synchronises before every rep (host submission included, the pages'
    eval-per-call mode).
  Per-kernel durations come from chains of one stage alone (gate+up, or
  down+combine) over the same layers, timed the same way.
* k_scaling: one token routed to k = 1, 8, 32, 128, 256 distinct experts of
  a full E=256 verify bank, gate+up stage (the one-position k sweep of the
  mlx discussion, section "Q1: it's occupancy").
* union_floor: each verify layer at L = 2, 3, 4, 8 against the same bank hit
  by ONE position routed to the layer's whole union set (the byte floor of
  the discussion's switch-bank table).
* A/B comparisons (per-pair baseline vs union; each codec vs the q4 bank on
  the same layers) run in A B B A order.
* codecs: the same verify routes and activations over banks in other codecs
  (mxfp4 gs32, the pages' GLM-5.2 format; nvfp4; 4-bit affine group 32;
  8-bit affine group 64; mxfp8), at L = 1, 2, 4, 8, each with its own bytes
  per expert.
* cpu_baseline: the CPU oracle (test infrastructure) timed on the host
  cores: 8 evenly spaced layers of every verify chain, median of 3 runs,
  plus a 1-core run; every layer of the tiny, GLM-5.3-Flash-shaped and
  small-expert configurations timed once and checked for parity.  Parity:
  fp32 output before the bf16 cast, per-row normwise error <= 1e-3, and the
  bf16 output equal to its round-to-nearest-even.

Prints one JSON line.  Progress goes to stderr.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/MoE layer + effective expert-weight GB/s at L=1/2/4/8, E=256 top-8 q4"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC_LS = (1, 2, 4, 8)
ISO_REPS = 60
TOL = 1e-3


def expert_bytes(H: int, I: int) -> int:
    """Bytes of one expert's gate, up and down matrices: 4-bit codes plus a bf16
    scale and a bf16 bias per group of 64 inputs (the size the mlx issue
    "gather_qmm at M=1 streams 4-bit expert weights..." counts per expert)."""
    per_matrix = H * I // 2 + (H * I // 64) * 2 * 2
    return 3 * per_matrix


def gateup_bytes(H: int, I: int) -> int:
    return 2 * (H * I // 2 + (H * I // 64) * 4)


def down_bytes(H: int, I: int) -> int:
    return H * I // 2 + (H * I // 64) * 4


def expert_bytes_codec(codec: str, H: int, I: int) -> int:
    """Bytes of one expert's gate, up and down in ``codec``: 4-bit codes plus
    the scales (and biases) of each group -- mxfp4: one byte per 32 inputs
    (about 20 MB at H=6144, I=2048, the size the mlx discussion "Small-L fused
    expert gather for fine-grained MoE decode" gives for the GLM-5.2 experts);
    nvfp4: one byte per 16; affine group 32: a bf16 scale and bias per 32;
    8-bit codecs: one byte per element plus a bf16 scale and bias per 64
    (affine) or one byte per 32 (mxfp8)."""
    bits, per = {"mxfp4": (4, 1 / 32), "nvfp4": (4, 1 / 16), "affine4_g32": (4, 4 / 32),
                 "affine8_g64": (8, 4 / 64), "mxfp8": (8, 1 / 32)}[codec]
    return 3 * (H * I * bits // 8 + round(H * I * per))


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comments and whitespace do not count,
    so the stored traffic figures stay valid across comment edits."""
    d = os.path.join(ROOT, "quantized_expert_gather_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h", ".cpp")):
            text = open(os.path.join(d, name), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
            text = re.sub(r"//[^\n]*", " ", text)                  # line comments
            h.update(name.encode())
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def read_traffic_profile():
    """HBM traffic of the gate+up kernel per unique-expert byte, from the
    committed rocprofv3 counter summary -- only while the kernel sources are
    the ones the counters were taken on."""
    path = os.path.join(ROOT, "profiles", "gateup_hbm_traffic_glm52verify.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_algorithmic_byte"])
    except (KeyError, ValueError):
        return None


def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cpus": affinity}


class Timer:
    """Chained and isolated GPU timing on one stream (see the module docstring)."""

    def __init__(self, torch, np, stream):
        self.torch, self.np, self.stream = torch, np, stream
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        self.cycles_per_ms = 1_000_000 / max(a.elapsed_time(b), 1e-3)

    def cycles(self, ms):
        return int(self.cycles_per_ms * ms)

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def chain(self, calls, delay_cycles):
        """Enqueue calls back to back behind a delay kernel; returns (start, end, host ms)."""
        self.torch.cuda._sleep(delay_cycles)
        e0, e1 = self.ev(), self.ev()
        e0.record()
        th = time.perf_counter()
        for c in calls:
            c()
        e1.record()
        return e0, e1, (time.perf_counter() - th) * 1e3

    def delay_for(self, calls):
        """Delay-kernel length covering the host enqueue of `calls` (measured once)."""
        self.torch.cuda.synchronize()
        _, _, host_ms = self.chain(calls, 0)
        self.torch.cuda.synchronize()
        return self.cycles(1.5 * host_ms + 1.0)

    def chained_ms(self, calls, reps, delay=None):
        """Median per-call ms of `reps` chains of `calls`."""
        delay = self.delay_for(calls) if delay is None else delay
        recs = [self.chain(calls, delay) for _ in range(reps)]
        self.torch.cuda.synchronize()
        return float(self.np.median([a.elapsed_time(b) for a, b, _ in recs])) / len(calls)

    def isolated_us(self, calls, reps=ISO_REPS):
        """Median of `reps` single calls, the calls rotated: (gpu, eager) in µs."""
        torch = self.torch
        one = self.cycles(0.15)  # covers the host enqueue of one call
        recs = []
        for i in range(reps):
            torch.cuda._sleep(one)
            e0, e1 = self.ev(), self.ev()
            e0.record()
            calls[(i * 7) % len(calls)]()
            e1.record()
            recs.append((e0, e1))
        torch.cuda.synchronize()
        gpu = float(self.np.median([a.elapsed_time(b) for a, b in recs])) * 1e3
        recs = []
        for i in range(reps):
            torch.cuda.synchronize()
            e0, e1 = self.ev(), self.ev()
            e0.record()
            calls[(i * 7 + 3) % len(calls)]()
            e1.record()
            recs.append((e0, e1))
        torch.cuda.synchronize()
        eager = float(self.np.median([a.elapsed_time(b) for a, b in recs])) * 1e3
        return gpu, eager

    def abba_ms(self, calls_a, calls_b, reps):
        """A B B A chains of two call lists of equal length; median per-call ms of each."""
        da, db = self.delay_for(calls_a), self.delay_for(calls_b)
        ra, rb = [], []
        for i in range(reps):
            order = (("a", "b"), ("b", "a"))[i % 2]
            for w in order:
                (ra if w == "a" else rb).append(self.chain(calls_a if w == "a" else calls_b, da if w == "a" else db))
        self.torch.cuda.synchronize()
        med = lambda r, n: float(self.np.median([a.elapsed_time(b) for a, b, _ in r])) / n  # noqa: E731
        return med(ra, len(calls_a)), med(rb, len(calls_b))


def rel_err_rows(np, got, ref):
    num = np.linalg.norm(got.astype(np.float64) - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def oracle_check(np, torch, q, oracle, x, ids_np, tw_np, bank, ids, tw, out_bf16, reps=1):
    """CPU oracle on one layer (median of `reps` timed runs) and the parity of
    the GPU's fp32 and bf16 outputs against it.  Returns (seconds, max row err, bf16 ok)."""
    bank_c = bank.to("cpu")
    xc = x.cpu()
    ts, ref = [], None
    for _ in range(reps):
        t = time.perf_counter()
        ref = oracle.forward_pairs(xc, ids_np, tw_np, bank_c)
        ts.append(time.perf_counter() - t)
    got = q.forward_bank(x, ids, tw, bank, out_dtype=torch.float32)
    err = float(rel_err_rows(np, got.cpu().numpy(), ref).max())
    ok16 = out_bf16 is None or bool(torch.equal(got.to(torch.bfloat16), out_bf16))
    return float(np.median(ts)), err, ok16


def bench_sorted(args, Ts, q, synth, torch, np, dev, stream, timer, codec="affine4_g64"):
    """Chains of distinct prefill layers (E=256 top-8 H=4096 I=2048, uniform routes)
    through the sorted path: full forward, then gate+up and down stages alone,
    and the isolated layer.  ``codec`` is affine4_g64 (the prefill configuration),
    mxfp4 or mxfp8."""
    w = synth.WORKLOADS["prefill"]
    H, I, E, k = w.H, w.I, w.E, w.k
    mx = codec in ("mxfp4", "mxfp8")
    eb = expert_bytes_codec(codec, H, I) if mx else expert_bytes(H, I)
    gu_eb, dn_eb = (2 * eb // 3, eb // 3) if mx else (gateup_bytes(H, I), down_bytes(H, I))
    out = {"workload": f"{w.name}{' in ' + codec if mx else ''}: uniform top-{k}, "
                       f"{args.sorted_layers} distinct layers per chain", "per_T": {}}
    stage_codes = (("all", q.MOE_Q4_STAGE_ALL), ("gateup", q.MOE_Q4_STAGE_GATEUP), ("down", q.MOE_Q4_STAGE_DOWN))
    for T in Ts:
        layers = []
        for layer in range(args.sorted_layers):
            if codec == "mxfp8":
                lay = synth.make_layer_q(codec, w, T, layer, seed=0, device=dev)
            else:
                lay = (synth.make_layer_mx if mx else synth.make_layer)(w, T, layer, seed=0, device=dev)
            ids = torch.from_numpy(lay.ids).to(dev)
            tw = torch.from_numpy(lay.weights).to(dev)
            o = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            bt = lay.bank.tensors()
            if mx:
                ws = torch.empty(q.moe_swiglu_codec_workspace_bytes(q.CODECS[codec][0], T, k, lay.bank.E, H, I),
                                 dtype=torch.uint8, device=dev)
                if codec == "mxfp4":  # the six-tensor mxfp4 bank
                    calls = {st: q.PreparedForwardMX(lay.x, ids, tw, bt, o, ws, code, stream) for st, code in stage_codes}
                else:
                    calls = {st: q.PreparedForwardCodec(codec, lay.x, ids, tw, bt, o, ws, code, stream)
                             for st, code in stage_codes}
            else:
                ws = q.new_workspace(T, k, E, H, I, dev)
                calls = {st: q.PreparedForward(lay.x, ids, tw, bt, o, ws, code, stream) for st, code in stage_codes}
            layers.append({"u": int(lay.bank.E), "keep": (lay, ids, tw, o, ws), "calls": calls,
                           "ws_bytes": ws.numel()})
        if not mx:
            assert q.moe_swiglu_q4_select_path(T, k, E, H, I) == q.MOE_Q4_PATH_SORTED
        torch.cuda.synchronize()
        layers[0]["calls"]["all"]()
        assert q.moe_q4_read_device_status(layers[0]["keep"][4], stream)[1] == q.MOE_Q4_PATH_SORTED
        reps = max(3, args.steps // 2)
        med = {wh: timer.chained_ms([l["calls"][wh] for l in layers], reps) for wh in ("all", "gateup", "down")}
        iso_gpu, iso_eager = timer.isolated_us([l["calls"]["all"] for l in layers], reps=args.iso_reps_sorted)
        u_sum = sum(l["u"] for l in layers)
        nl = len(layers)
        P = T * k
        flops = 6.0 * P * I * H                          # gate, up, down: 2 flops per weight per pair
        gu_bytes = (u_sum / nl) * gu_eb + 2 * T * H + 8 * T * k
        dn_bytes = (u_sum / nl) * dn_eb
        gb = (u_sum / nl) * eb / (med["all"] * 1e-3) / 1e9
        tf = flops / (med["all"] * 1e-3) / 1e12
        gu_ms, dn_ms = med["gateup"], med["down"]
        out["per_T"][str(T)] = {
            "us_per_layer": round(med["all"] * 1e3, 1), "u_mean": round(u_sum / nl, 1),
            "eff_GBps": round(gb, 1), "frac_hbm_peak": round(gb / PEAK_HBM_GBPS, 4),
            "TFLOPs": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "gateup_us": round(gu_ms * 1e3, 1), "down_combine_us": round(dn_ms * 1e3, 1),
            "gateup_GBps": round(gu_bytes / (gu_ms * 1e-3) / 1e9, 1),
            "gateup_TFLOPs": round(4.0 * P * I * H / (gu_ms * 1e-3) / 1e12, 1),
            "down_GBps": round(dn_bytes / (dn_ms * 1e-3) / 1e9, 1),
            "down_TFLOPs": round(2.0 * P * I * H / (dn_ms * 1e-3) / 1e12, 1),
            "isolated_gpu_us": round(iso_gpu, 1), "isolated_eager_us": round(iso_eager, 1),
            "scratch_bytes": int(layers[0]["ws_bytes"]),
        }
        log(f"sorted {codec} T={T}: {med['all'] * 1e3:.1f} us/layer chained ({iso_gpu:.1f} isolated), {gb:.0f} GB/s, "
            f"{tf:.0f} TFLOP/s; gate+up {gu_ms * 1e3:.1f} us, down+combine {dn_ms * 1e3:.1f} us")
        del layers
        torch.cuda.empty_cache()
    return out


def bench_workload(wname, args, q, synth, torch, np, dev, stream, timer, oracle=None):
    """Another q4 g64 decode / verify configuration: a chain of all its layers
    (distinct weights and routes) per L, full forward, chained and isolated;
    with the oracle, every layer is also timed on the CPU and checked."""
    w = synth.WORKLOADS[wname]
    H, I, k = w.H, w.I, w.k
    eb = expert_bytes(H, I)
    out = {"workload": f"{w.name}: {w.routing} routes, chain of {w.n_layers} layers", "per_L": {}}
    cpu = {"layers": 0, "seconds": 0.0, "bytes": 0.0, "max_row_rel_err_f32_out": 0.0, "bf16_out_is_rne": True}
    for L in w.Ls:
        layers = []
        for layer in range(w.n_layers):
            lay = synth.make_chain_layer(w, L, layer, seed=0, device=dev)
            ids = torch.from_numpy(lay.ids).to(dev)
            tw = torch.from_numpy(lay.weights).to(dev)
            o = torch.empty((L, H), dtype=torch.bfloat16, device=dev)
            ws = q.new_workspace(L, k, lay.bank.E, H, I, dev)
            call = q.PreparedForward(lay.x, ids, tw, lay.bank.tensors(), o, ws, q.MOE_Q4_STAGE_ALL, stream)
            layers.append({"u": int(lay.bank.E), "lay": lay, "ids": ids, "tw": tw, "out": o, "ws": ws, "call": call})
        torch.cuda.synchronize()
        calls = [l["call"] for l in layers]
        ms = timer.chained_ms(calls, max(3, args.steps))
        iso_gpu, iso_eager = timer.isolated_us(calls)
        nl = len(layers)
        u_mean = sum(l["u"] for l in layers) / nl
        gb = u_mean * eb / (ms * 1e-3) / 1e9
        out["per_L"][str(L)] = {"us_per_layer": round(ms * 1e3, 2), "u_mean": round(u_mean, 2),
                                "eff_GBps": round(gb, 1), "frac_peak": round(gb / PEAK_HBM_GBPS, 4),
                                "isolated_gpu_us": round(iso_gpu, 2), "isolated_eager_us": round(iso_eager, 2)}
        log(f"{w.name} L={L}: {ms * 1e3:.2f} us/layer chained, {iso_gpu:.2f} isolated, {gb:.0f} GB/s effective")
        if oracle is not None:
            for l in layers:
                s, err, ok16 = oracle_check(np, torch, q, oracle, l["lay"].x, l["lay"].ids, l["lay"].weights,
                                            l["lay"].bank, l["ids"], l["tw"], l["out"])
                cpu["layers"] += 1
                cpu["seconds"] += s
                cpu["bytes"] += l["u"] * eb
                cpu["max_row_rel_err_f32_out"] = max(cpu["max_row_rel_err_f32_out"], err)
                cpu["bf16_out_is_rne"] &= ok16
        del layers
        torch.cuda.empty_cache()
    if oracle is not None and cpu["layers"]:
        out["cpu"] = {"GBps": round(cpu["bytes"] / cpu["seconds"] / 1e9, 3), "layers": cpu["layers"],
                      "seconds": round(cpu["seconds"], 2), "threads": oracle.threads(), "timed_once": True}
        out["parity"] = {"layers": cpu["layers"], "max_row_rel_err_f32_out": float(f"{cpu['max_row_rel_err_f32_out']:.3e}"),
                         "tolerance": TOL, "bf16_out_is_rne_of_f32_out": cpu["bf16_out_is_rne"],
                         "pass": bool(cpu["max_row_rel_err_f32_out"] <= TOL and cpu["bf16_out_is_rne"])}
        log(f"{w.name}: oracle parity on all {cpu['layers']} layers, max row err {cpu['max_row_rel_err_f32_out']:.2e}")
    return out


def bench_codec(codec, args, Ls, chains, q, synth, torch, np, dev, stream, timer):
    """The verify workload over banks in another codec: chains of layers
    spread over the depth profile (so over the overlap range), full forward
    and gate+up alone, per L; the q4 bank of the same layers is timed beside
    it in A B B A order."""
    w = synth.WORKLOADS["verify"]
    H, I, E, k = w.H, w.I, w.E, w.k
    code = q.CODECS[codec][0]
    eb = expert_bytes_codec(codec, H, I)
    gub = 2 * eb // 3
    nlay = min(w.n_layers, args.layers)  # the q4 chains hold layers 0 .. nlay - 1
    layer_ids = sorted(set(np.linspace(0, nlay - 1, args.codec_layers).round().astype(int).tolist()))
    out = {"workload": f"{w.name} in {codec}, overlap chain of {len(layer_ids)} layers spread over the "
                       f"{nlay}-layer depth profile", "bytes_per_expert": eb, "per_L": {}}
    tot_b, tot_ms = 0.0, 0.0
    for L in Ls:
        layers = []
        for layer in layer_ids:
            lay = synth.make_chain_layer_q(codec, w, L, layer, seed=0, device=dev)
            ids = torch.from_numpy(lay.ids).to(dev)
            tw = torch.from_numpy(lay.weights).to(dev)
            o = torch.empty((L, H), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(max(256, q.moe_swiglu_codec_workspace_bytes(code, L, k, E, H, I)), dtype=torch.uint8,
                             device=dev)
            bt = lay.bank.tensors()
            layers.append({"u": int(lay.bank.E), "keep": (lay, ids, tw, o, ws),
                           "calls": {st: q.PreparedForwardCodec(codec, lay.x, ids, tw, bt, o, ws, sc, stream)
                                     for st, sc in (("all", q.MOE_Q4_STAGE_ALL),
                                                    ("gateup", q.MOE_Q4_STAGE_GATEUP))}})
        torch.cuda.synchronize()
        reps = max(3, args.steps)
        ms_all, ms_q4 = timer.abba_ms([l["calls"]["all"] for l in layers],
                                      [chains[L]["layers"][i]["calls"]["all"] for i in layer_ids], max(2, reps // 2))
        ms_gu = timer.chained_ms([l["calls"]["gateup"] for l in layers], reps)
        nl = len(layers)
        u_mean = sum(l["u"] for l in layers) / nl
        gb = u_mean * eb / (ms_all * 1e-3) / 1e9
        gu_gb = (u_mean * gub + 2 * L * H + 8 * L * k) / (ms_gu * 1e-3) / 1e9
        out["per_L"][str(L)] = {"us_per_layer": round(ms_all * 1e3, 2), "u_mean": round(u_mean, 2),
                                "eff_GBps": round(gb, 1), "frac_peak": round(gb / PEAK_HBM_GBPS, 4),
                                "gateup_us": round(ms_gu * 1e3, 2), "gateup_GBps": round(gu_gb, 1),
                                "q4_same_layers_us_abba": round(ms_q4 * 1e3, 2),
                                "time_over_q4": round(ms_all / ms_q4, 3)}
        if L in METRIC_LS:
            tot_b += u_mean * eb
            tot_ms += ms_all
        log(f"{codec} L={L}: {ms_all * 1e3:.2f} us/layer ({ms_all / ms_q4:.2f}x q4), {gb:.0f} GB/s effective; "
            f"gate+up {gu_gb:.0f} GB/s")
        del layers
        torch.cuda.empty_cache()
    if tot_ms > 0:
        out["eff_GBps_over_L"] = round(tot_b / (tot_ms * 1e-3) / 1e9, 1)
        out["frac_peak"] = round(out["eff_GBps_over_L"] / PEAK_HBM_GBPS, 4)
    pl = out["per_L"]
    if "1" in pl and "2" in pl:
        out["L2_over_L1_time"] = round(pl["2"]["us_per_layer"] / pl["1"]["us_per_layer"], 3)
    return out


def bench_k_scaling(args, q, synth, torch, np, dev, stream, timer):
    """One token routed to k distinct experts of a full E=256 verify bank
    (H=6144, I=2048): the gate+up stage, chained over calls that each draw
    their own k experts."""
    w = synth.WORKLOADS["verify"]
    H, I, E = w.H, w.I, w.E
    bank = synth.gen_bank(E, H, I, (0, w.name, "k-scaling"), device=dev)
    bt = bank.tensors()
    rng = synth.np_rng("k-scaling")
    out = {"workload": f"{w.name}: one token, k distinct experts of the full E={E} bank, gate+up stage, "
                       f"calls chained, each with its own experts", "per_k": {}}
    for kk in args.k_scaling:
        ncalls = max(4, min(32, 2048 // kk))
        calls = []
        for c in range(ncalls):
            ids = torch.from_numpy(rng.permutation(E)[:kk].astype(np.int32).reshape(1, kk)).to(dev)
            tw = torch.full((1, kk), 1.0 / kk, dtype=torch.float32, device=dev)
            x = synth.gen_x(1, H, (0, "k-scaling", kk, c), dev)
            o = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
            ws = q.new_workspace(1, kk, E, H, I, dev)
            calls.append(q.PreparedForward(x, ids, tw, bt, o, ws, q.MOE_Q4_STAGE_GATEUP, stream))
        torch.cuda.synchronize()
        ms = timer.chained_ms(calls, max(3, args.steps))
        gb = kk * gateup_bytes(H, I) / (ms * 1e-3) / 1e9
        out["per_k"][str(kk)] = {"us": round(ms * 1e3, 2), "GBps": round(gb, 1), "frac_peak": round(gb / PEAK_HBM_GBPS, 4)}
        log(f"k-scaling k={kk}: {ms * 1e3:.2f} us, {gb:.0f} GB/s")
    del bank, bt
    torch.cuda.empty_cache()
    return out


def bench_union_floor(args, Ls, chains, per_L, q, synth, torch, np, dev, stream, timer):
    """Each verify layer at L against the same bank hit by one position routed
    to the layer's whole union set (k = u: the same bytes, one token)."""
    w = synth.WORKLOADS["verify"]
    H, I = w.H, w.I
    out = {"workload": f"{w.name}: each layer of the chain vs one position routed to its union set "
                       f"(same bank, same bytes)", "per_L": {}}
    for L in Ls:
        if L == 1:
            continue
        layers = chains[L]["layers"][: args.floor_layers]
        fcalls = []
        for lay in layers:
            u = lay["u"]
            ids = torch.arange(u, dtype=torch.int32, device=dev).reshape(1, u)
            tw = torch.full((1, u), 1.0 / u, dtype=torch.float32, device=dev)
            o = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
            ws = q.new_workspace(1, u, u, H, I, dev)
            lay["floor_keep"] = (ids, tw, o, ws)
            fcalls.append(q.PreparedForward(lay["x"][:1], ids, tw, lay["bank"].tensors(), o, ws, q.MOE_Q4_STAGE_ALL,
                                            stream))
        torch.cuda.synchronize()
        ms_layer, ms_floor = timer.abba_ms([l["calls"]["all"] for l in layers], fcalls, max(2, args.steps // 2))
        rec = {"layers": len(layers), "layer_us": round(ms_layer * 1e3, 2), "floor_us": round(ms_floor * 1e3, 2),
               "layer_over_floor": round(ms_layer / ms_floor, 3)}
        if "1" in per_L:
            rec["floor_over_L1"] = round(ms_floor * 1e3 / per_L["1"]["us_per_layer"], 3)
            rec["layer_over_L1"] = round(ms_layer * 1e3 / per_L["1"]["us_per_layer"], 3)
        out["per_L"][str(L)] = rec
        log(f"union floor L={L}: layer {ms_layer * 1e3:.1f} us vs one position on its union set "
            f"{ms_floor * 1e3:.1f} us ({ms_layer / ms_floor:.3f}x)")
        for lay in layers:
            lay.pop("floor_keep", None)
    return out


def stream_references(q, torch, dev, stream, timer):
    """Plain streaming rates on this chip over 2 GiB (four times the MALL):
    a read-only kernel, torch's sum over bf16 (the pages' reference), a copy."""
    n = 2 * 2**30
    buf = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    q.moe_q4_stream_read(buf, sink, stream)
    torch.cuda.synchronize()
    res = {}
    e0, e1 = timer.ev(), timer.ev()
    e0.record()
    for _ in range(5):
        q.moe_q4_stream_read(buf, sink, stream)
    e1.record()
    torch.cuda.synchronize()
    res["stream_ref_read_GBps"] = round(5 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    bf = buf.view(torch.bfloat16)
    bf.sum()
    torch.cuda.synchronize()
    e0, e1 = timer.ev(), timer.ev()
    e0.record()
    for _ in range(5):
        bf.sum()
    e1.record()
    torch.cuda.synchronize()
    res["stream_ref_sum_bf16_GBps"] = round(5 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    dst = torch.empty_like(buf)
    dst.copy_(buf)
    e0, e1 = timer.ev(), timer.ev()
    e0.record()
    for _ in range(5):
        dst.copy_(buf)
    e1.record()
    torch.cuda.synchronize()
    res["stream_ref_copy_GBps"] = round(5 * 2 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del buf, dst, sink, bf
    torch.cuda.empty_cache()
    log(f"streaming references over 2 GiB: read {res['stream_ref_read_GBps']:.0f} GB/s, bf16 sum "
        f"{res['stream_ref_sum_bf16_GBps']:.0f} GB/s, copy {res['stream_ref_copy_GBps']:.0f} GB/s")
    return res


def profile_pass(args):
    """One forward call per layer, synchronised, in a fixed order: the first
    args.profile_pass layers of each verify chain (args.Ls), then of the
    pooled small-expert chains at L = 8, 16, 32.  Each call launches k_gateup
    then k_down (then k_combine when L > 1), so a counter trace lines up with
    the manifest printed here: per call the workload, L, layer, distinct
    experts and the algorithmic bytes of the gate+up and down kernels."""
    import numpy as np
    import torch

    import quantized_expert_gather_amd as q
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    calls = []
    plan = [("verify", int(v)) for v in args.Ls.split(",")] + [("small_pooled", L) for L in (8, 16, 32)]
    for wname, L in plan:
        w = synth.WORKLOADS[wname]
        for layer in range(args.profile_pass):
            lay = synth.make_chain_layer(w, L, layer, seed=0, device=dev)
            ids = torch.from_numpy(lay.ids).to(dev)
            tw = torch.from_numpy(lay.weights).to(dev)
            ws = q.new_workspace(L, w.k, lay.bank.E, w.H, w.I, dev)
            torch.cuda.synchronize()
            q.forward_bank(lay.x, ids, tw, lay.bank, workspace=ws)
            torch.cuda.synchronize()
            u = int(lay.bank.E)
            calls.append({"workload": wname, "L": L, "layer": layer, "u": u, "H": w.H, "I": w.I, "k": w.k,
                          "gateup_alg_bytes": u * gateup_bytes(w.H, w.I) + 2 * L * w.H + 8 * L * w.k,
                          "down_alg_bytes": u * down_bytes(w.H, w.I) + 2 * L * w.H + 8 * L * w.k})
        log(f"profile pass: {wname} L={L}, {args.profile_pass} layers")
    print(json.dumps({"profile_pass": calls}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=75)
    ap.add_argument("--Ls", default="1,2,3,4,8",
                    help="window sizes timed; value aggregates those of the metric (1, 2, 4, 8)")
    ap.add_argument("--sorted-Ts", default="512,2048,16384",
                    help="token counts of the prefill (sorted-path) measurement (512 and 2048 are the "
                         "prefill configuration; 16384 is the long-prefill regime); empty to skip")
    ap.add_argument("--sorted-layers", type=int, default=4, help="distinct layers per prefill chain")
    ap.add_argument("--iso-reps-sorted", type=int, default=20, help="isolated reps of each prefill layer timing")
    ap.add_argument("--sorted-mx-Ts", default="512,2048",
                    help="token counts of the same prefill workload over mxfp4 banks (sorted path); empty to skip")
    ap.add_argument("--sorted-mx8-Ts", default="512,2048",
                    help="token counts of the same prefill workload over mxfp8 banks (sorted path); empty to skip")
    ap.add_argument("--workloads", default="flash,small,small_pooled",
                    help="other q4 decode / verify configurations (flash: E=288 top-8 H=4096 I=2048 at L=1, 4; "
                         "small / small_pooled: E=256 top-8 H=2048 I=512 at L=8, 16, 32); empty to skip")
    ap.add_argument("--pair-layers", type=int, default=20,
                    help="layers of each chain timed again as a per-pair baseline (one call per token, so "
                         "an expert shared by tokens is streamed once per token); 0 to skip")
    ap.add_argument("--floor-layers", type=int, default=20,
                    help="layers of each chain timed against one position routed to their union set; 0 to skip")
    ap.add_argument("--k-scaling", default="1,8,32,128,256",
                    help="distinct experts of the one-token k sweep; empty to skip")
    ap.add_argument("--codecs", default="mxfp4,nvfp4,affine4_g32,affine8_g64,mxfp8",
                    help="other weight codecs timed on the verify workload (comma list; empty to skip)")
    ap.add_argument("--codec-layers", type=int, default=19,
                    help="layers per L of each codec's verify chains (spread over the depth profile)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline and the parity legs")
    ap.add_argument("--cpu-layers", type=int, default=8, help="evenly spaced verify layers per L timed on the CPU")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (reference for hardware "
                         "byte counters) and exit")
    ap.add_argument("--profile-pass", type=int, default=0, metavar="N",
                    help="only run N layers of each verify chain (--Ls) and of the pooled small-expert chains "
                         "(L = 8, 16, 32) once each, in a fixed order, for hardware-counter passes; prints a "
                         "JSON manifest of the calls (algorithmic bytes per kernel) and exits")
    args = ap.parse_args()
    args.k_scaling = [int(v) for v in args.k_scaling.split(",") if v.strip()]

    if args.copy_calibration:
        import torch
        n = args.copy_calibration * 2**20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return

    if args.profile_pass:
        profile_pass(args)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_expert_gather_amd as q
    import synth

    oracle = None
    if not args.no_cpu:
        import oracle
        oracle.build(force=False)

    Ls = [int(v) for v in args.Ls.split(",")]
    w = synth.WORKLOADS["verify"]
    H, I, E, k = w.H, w.I, w.E, w.k
    eb = expert_bytes(H, I)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    timer = Timer(torch, np, stream)

    # ---- inputs, resident in HBM ----
    t0 = time.time()
    chains = {}
    for L in Ls:
        layers = []
        for layer in range(args.layers):
            lay = synth.make_chain_layer(w, L, layer, seed=0, device=dev)
            layers.append({
                "x": lay.x, "bank": lay.bank, "u": int(lay.bank.E),
                "ids": torch.from_numpy(lay.ids).to(dev), "tw": torch.from_numpy(lay.weights).to(dev),
                "ids_np": lay.ids, "tw_np": lay.weights,
                "out": torch.empty((L, H), dtype=torch.bfloat16, device=dev),
            })
        for lay in layers:
            bt = lay["bank"].tensors()
            ws = q.new_workspace(L, k, E, H, I, dev)  # one per layer: stage-only chains read their own tables
            lay["calls"] = {st: q.PreparedForward(lay["x"], lay["ids"], lay["tw"], bt, lay["out"], ws, code, stream)
                            for st, code in (("all", q.MOE_Q4_STAGE_ALL), ("gateup", q.MOE_Q4_STAGE_GATEUP),
                                             ("down", q.MOE_Q4_STAGE_DOWN))}
        chains[L] = {"layers": layers}
        torch.cuda.synchronize()
        log(f"L={L}: {args.layers} layers generated, mean unique experts "
            f"{np.mean([l['u'] for l in layers]):.2f}, {time.time() - t0:.1f}s, "
            f"HBM used {torch.cuda.memory_allocated() / 2**30:.1f} GiB")

    def run_step(which="all"):
        return {L: timer.chain([l["calls"][which] for l in chains[L]["layers"]], delays[L]) for L in Ls}

    torch.cuda.synchronize()
    delays = {L: 0 for L in Ls}
    warm = run_step()  # first pass also measures the host enqueue time per chain
    torch.cuda.synchronize()
    delays = {L: timer.cycles(1.5 * warm[L][2] + 1.0) for L in Ls}
    for _ in range(max(0, args.warmup - 1)):
        run_step()
    torch.cuda.synchronize()
    log(f"warmup done; host enqueue {max(v[2] for v in warm.values()):.2f} ms per chain")

    # ---- timed steps: full forward chains, no events inside a chain ----
    torch.cuda.synchronize()
    recs = [run_step("all") for _ in range(args.steps)]
    torch.cuda.synchronize()
    # ---- per-kernel durations: chains of one stage only, same layers ----
    krecs = {w_: [run_step(w_) for _ in range(max(2, args.steps // 2))] for w_ in ("gateup", "down")}
    torch.cuda.synchronize()

    per_L = {}
    tot_bytes = 0.0
    tot_ms = 0.0
    gu_ms, gu_bytes, gu_n = 0.0, 0.0, 0
    dn_ms, dn_bytes, dn_n = 0.0, 0.0, 0
    for L in Ls:
        layers = chains[L]["layers"]
        nl = len(layers)
        u_sum = sum(l["u"] for l in layers)
        chain_ms = [rec[L][0].elapsed_time(rec[L][1]) for rec in recs]
        g_ms = [rec[L][0].elapsed_time(rec[L][1]) for rec in krecs["gateup"]]
        d_ms = [rec[L][0].elapsed_time(rec[L][1]) for rec in krecs["down"]]
        lay_bytes_gu = sum(l["u"] * gateup_bytes(H, I) + 2 * L * H + 8 * L * k for l in layers)
        lay_bytes_dn = sum(l["u"] * down_bytes(H, I) + 2 * L * H + 8 * L * k for l in layers)
        gu_ms += sum(g_ms); gu_bytes += lay_bytes_gu * len(g_ms); gu_n += nl * len(g_ms)
        dn_ms += sum(d_ms); dn_bytes += lay_bytes_dn * len(d_ms); dn_n += nl * len(d_ms)
        med = float(np.median(chain_ms))
        us_layer = med * 1e3 / nl
        gbps = u_sum * eb / (med * 1e-3) / 1e9
        iso_gpu, iso_eager = timer.isolated_us([l["calls"]["all"] for l in layers])
        per_L[str(L)] = {"us_per_layer": round(us_layer, 2), "eff_GBps": round(gbps, 1),
                         "frac_peak": round(gbps / PEAK_HBM_GBPS, 4), "u_mean": round(u_sum / nl, 2),
                         "gateup_us": round(float(np.median(g_ms)) * 1e3 / nl, 2),
                         "down_combine_us": round(float(np.median(d_ms)) * 1e3 / nl, 2),
                         "isolated_gpu_us": round(iso_gpu, 2), "isolated_eager_us": round(iso_eager, 2),
                         "isolated_gpu_eff_GBps": round(u_sum / nl * eb / (iso_gpu * 1e-6) / 1e9, 1),
                         "chain_ms_median": round(med, 4), "host_enqueue_ms": round(warm[L][2], 3)}
        if L in METRIC_LS or not any(v in METRIC_LS for v in Ls):
            tot_bytes += u_sum * eb * len(recs)
            tot_ms += sum(chain_ms)
        log(f"L={L}: {us_layer:.2f} us/layer, {gbps:.0f} GB/s effective ({gbps / PEAK_HBM_GBPS * 100:.1f}% of 8 TB/s);"
            f" gate+up {per_L[str(L)]['gateup_us']:.1f} us, down+combine {per_L[str(L)]['down_combine_us']:.1f} us;"
            f" isolated {iso_gpu:.1f} us (GPU), {iso_eager:.1f} us (eager)")

    # per-pair baseline: the same layers with one call per token (L = 1 each),
    # i.e. every (token, expert) route streams its expert's weights -- the
    # traffic of a per-pair gather without deduplication across tokens
    pair_result = None
    if args.pair_layers > 0:
        pair_result = {}
        for L in Ls:
            if L == 1:
                continue
            layers = chains[L]["layers"][: args.pair_layers]
            calls = []
            for lay in layers:
                ws1 = q.new_workspace(1, k, E, H, I, dev)
                lay["pair_ws"] = ws1
                for t in range(L):
                    calls.append(q.PreparedForward(lay["x"][t:t + 1], lay["ids"][t:t + 1], lay["tw"][t:t + 1],
                                                   lay["bank"].tensors(), lay["out"][t:t + 1], ws1,
                                                   q.MOE_Q4_STAGE_ALL, stream))
            ucalls = [lay["calls"]["all"] for lay in layers]
            # A B B A: union chain, per-pair chain, per-pair, union, ...
            ms_u, ms_p = timer.abba_ms(ucalls, calls, max(2, args.steps // 2))
            uu, us = ms_u * 1e3, ms_p * 1e3 * L  # per layer: a pair chain has L calls per layer
            pair_result[str(L)] = {"us_per_layer": round(us, 2), "layers": len(layers),
                                   "union_us_per_layer_same_layers": round(uu, 2),
                                   "per_pair_over_union": round(us / uu, 3),
                                   "slot_bytes_GBps": round(L * k * eb / (us * 1e-6) / 1e9, 1), "order": "ABBA"}
            log(f"per-pair L={L}: {us:.1f} us/layer vs union {uu:.1f} us/layer on the same {len(layers)} layers "
                f"({us / uu:.2f}x, A B B A)")

    union_floor = None
    if args.floor_layers > 0:
        union_floor = bench_union_floor(args, Ls, chains, per_L, q, synth, torch, np, dev, stream, timer)

    refs = stream_references(q, torch, dev, stream, timer)

    value = tot_bytes / (tot_ms * 1e-3) / 1e9
    ms_per_step = tot_ms / len(recs)
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "q4xbf16->f32", "data": "synthetic",
        "config": {"workload": f"{w.name} overlap chain, {args.layers} layers per L", "E": E, "k": k, "H": H,
                   "I": I, "group_size": 64, "bits": 4, "L": Ls,
                   "value_over_L": [v for v in Ls if v in METRIC_LS] or Ls, "layers": args.layers,
                   "bytes_per_expert": eb, "timing": "GPU events, chains enqueued back to back"},
        "per_L": per_L,
        "per_pair_baseline": pair_result,
        "union_floor": union_floor,
        **refs,
    }
    result["frac_of_stream_ref_read"] = round(value / refs["stream_ref_read_GBps"], 4)
    if "1" in per_L and "2" in per_L:
        r = per_L["2"]["us_per_layer"] / per_L["1"]["us_per_layer"]
        result["L2_over_L1_time"] = round(r, 3)
        result["L2_over_L1_targets"] = {"target": 1.3,
                                        "byte_floor": round(per_L["2"]["u_mean"] / per_L["1"]["u_mean"], 3)}

    if gu_n:
        achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
        ratio = read_traffic_profile()
        result["roofline"] = {
            "kernel": "k_gateup (fused gate+up dequant GEMV + silu*up)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": None if ratio is None else round(ratio * gu_bytes / gu_n, 0),
            "avg_launch_us": round(gu_ms * 1e3 / gu_n, 3),
            "algorithmic_bytes_per_launch": round(gu_bytes / gu_n, 0),
            "timing": "back-to-back chains of this kernel alone, HIP events at the chain ends",
        }
        result["down_kernel"] = {"kernel": "k_down + k_combine",
                                 "achieved_GBps": round(dn_bytes / (dn_ms * 1e-3) / 1e9, 1),
                                 "avg_launch_us": round(dn_ms * 1e3 / dn_n, 3)}

    if args.k_scaling:
        result["k_scaling"] = bench_k_scaling(args, q, synth, torch, np, dev, stream, timer)

    # ---- CPU oracle baseline: evenly spaced layers of every verify chain ----
    if oracle is not None:
        try:
            info = cpu_info()
            threads = oracle.threads()
            sel = sorted(set(np.linspace(0, args.layers - 1, args.cpu_layers).round().astype(int).tolist()))
            cpu_s, cpu_bytes, max_err, bf16_ok, per = 0.0, 0.0, 0.0, True, {}
            for L in Ls:
                n_l = 0
                for li in sel:
                    lay = chains[L]["layers"][li]
                    s, err, ok16 = oracle_check(np, torch, q, oracle, lay["x"], lay["ids_np"], lay["tw_np"],
                                                lay["bank"], lay["ids"], lay["tw"], lay["out"], reps=3)
                    cpu_s += s
                    cpu_bytes += lay["u"] * eb
                    max_err = max(max_err, err)
                    bf16_ok &= ok16
                    n_l += 1
                per[str(L)] = n_l
            # one core: the first selected layer of the L = 1 chain, median of 3
            lay = chains[Ls[0]]["layers"][sel[0]]
            oracle.set_threads(1)
            s1, _, _ = oracle_check(np, torch, q, oracle, lay["x"], lay["ids_np"], lay["tw_np"], lay["bank"],
                                    lay["ids"], lay["tw"], None, reps=3)
            oracle.set_threads(threads)
            cpu_gbps = cpu_bytes / cpu_s / 1e9
            result["cpu_baseline"] = {
                "value": round(cpu_gbps, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": f"per-pair fp64 C oracle (OpenMP, {threads} threads) on {args.cpu_layers} evenly spaced "
                          f"layers of each verify chain {per}, median of 3 runs each; {3 * cpu_s:.1f} s of CPU "
                          f"time; same unique-expert byte metric",
                "us_per_layer_mean": round(cpu_s * 1e6 / max(1, sum(per.values())), 1),
                "one_core_GBps": round(lay["u"] * eb / s1 / 1e9, 4),
                "one_core_sample": f"layer {sel[0]} of the L={Ls[0]} chain, median of 3",
                **info,
            }
            result["parity"] = {
                "layers": int(sum(per.values())), "max_row_rel_err_f32_out": float(f"{max_err:.3e}"),
                "tolerance": TOL, "pass": bool(max_err <= TOL and bf16_ok), "bf16_out_is_rne_of_f32_out": bf16_ok,
            }
            # the tiny configuration: its one layer, full bank, checked and timed
            tl = synth.tiny_layer(device=dev)
            tids, ttw = torch.from_numpy(tl.ids).to(dev), torch.from_numpy(tl.weights).to(dev)
            tout = q.forward_bank(tl.x, tids, ttw, tl.bank)
            s, err, ok16 = oracle_check(np, torch, q, oracle, tl.x, tl.ids, tl.weights, tl.bank, tids, ttw, tout,
                                        reps=3)
            result["parity_tiny"] = {"max_row_rel_err_f32_out": float(f"{err:.3e}"), "bf16_out_is_rne_of_f32_out": ok16,
                                     "pass": bool(err <= TOL and ok16), "cpu_us": round(s * 1e6, 1)}
            log(f"cpu baseline: {cpu_gbps:.2f} GB/s on {threads} threads, one core {lay['u'] * eb / s1 / 1e9:.3f} GB/s; "
                f"parity max row err {max_err:.2e} (verify), {err:.2e} (tiny)")
        except Exception as exc:  # the baseline must not hide the GPU result
            log(f"cpu baseline failed: {exc!r}")
            result["cpu_baseline"] = None

    # ---- prefill workload through the sorted path (grouped MFMA GEMMs) ----
    sorted_Ts = [int(v) for v in args.sorted_Ts.split(",") if v.strip()]
    if sorted_Ts:
        result["sorted_path"] = bench_sorted(args, sorted_Ts, q, synth, torch, np, dev, stream, timer)
    # the same prefill workload over the block-scaled banks
    for key, opt, codec in (("sorted_path_mxfp4", args.sorted_mx_Ts, "mxfp4"),
                            ("sorted_path_mxfp8", args.sorted_mx8_Ts, "mxfp8")):
        cTs = [int(v) for v in opt.split(",") if v.strip()]
        if cTs:
            result[key] = bench_sorted(args, cTs, q, synth, torch, np, dev, stream, timer, codec=codec)

    # ---- the other decode / verify configurations, with CPU parity on every layer ----
    wnames = [v for v in args.workloads.split(",") if v.strip()]
    if wnames:
        result["other_workloads"] = {n: bench_workload(n, args, q, synth, torch, np, dev, stream, timer, oracle)
                                     for n in wnames}

    # ---- the same verify workload over banks in other codecs ----
    codecs = [c for c in args.codecs.split(",") if c.strip()]
    if codecs and args.codec_layers > 0:
        cLs = [v for v in Ls if v in METRIC_LS] or Ls
        result["codecs"] = {c: bench_codec(c, args, cLs, chains, q, synth, torch, np, dev, stream, timer)
                            for c in codecs}

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
