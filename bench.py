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
  Inputs are resident in HBM before timing.  Every layer of a chain is
  enqueued back to back on one stream with HIP events only at the chain ends;
  a GPU delay kernel ahead of each chain lets the host enqueue the whole
  chain first, so the events time the GPU, not Python.  Per-kernel durations
  come from chains of one stage alone (gate+up, or down+combine) over the
  same layers, timed the same way.
* codecs: the same verify routes and activations over banks in other codecs
  (mxfp4 gs32, the pages' GLM-5.2 format; nvfp4; 4-bit affine group 32;
  8-bit affine group 64; mxfp8), at L = 1, 2, 4, 8, each with its own bytes
  per expert.
* cpu_baseline: the CPU oracle (test infrastructure) timed on a bounded
  sample of the same layers on the host cores, with the same metric; the
  same layers are checked for parity (fp32 output before the bf16 cast,
  per-row normwise error <= 1e-3).

Prints one JSON line.  Progress goes to stderr.
"""

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/MoE layer + effective expert-weight GB/s at L=1/2/4/8, E=256 top-8 q4"
PEAK_HBM_GBPS = 8000.0
METRIC_LS = (1, 2, 4, 8)


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


PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def bench_sorted(args, Ts, q, synth, torch, np, dev, stream, sleep_cycles_for, codec="affine4_g64"):
    """Chains of distinct prefill layers (E=256 top-8 H=4096 I=2048, uniform routes)
    through the sorted path: full forward, then gate+up and down stages alone.
    ``codec`` is affine4_g64 (the prefill configuration), mxfp4 or mxfp8."""
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
            layers.append({"u": int(lay.bank.E), "keep": (lay, ids, tw, o, ws), "calls": calls})
        if not mx:
            assert q.moe_swiglu_q4_select_path(T, k, E, H, I) == q.MOE_Q4_PATH_SORTED
        torch.cuda.synchronize()
        if mx:
            layers[0]["calls"]["all"]()
            assert q.moe_q4_read_device_status(layers[0]["keep"][4], stream)[1] == q.MOE_Q4_PATH_SORTED

        def chain(which, delay):
            torch.cuda._sleep(delay)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            th = time.perf_counter()
            for lay in layers:
                lay["calls"][which]()
            e1.record()
            return e0, e1, (time.perf_counter() - th) * 1e3

        warm = chain("all", 0)
        torch.cuda.synchronize()
        delay = sleep_cycles_for(1.5 * warm[2] + 1.0)
        chain("all", delay)
        torch.cuda.synchronize()
        recs = {wh: [chain(wh, delay) for _ in range(max(3, args.steps // 2))] for wh in ("all", "gateup", "down")}
        torch.cuda.synchronize()
        nl = len(layers)
        med = {wh: float(np.median([a.elapsed_time(b) for a, b, _ in v])) / nl for wh, v in recs.items()}
        u_sum = sum(l["u"] for l in layers)
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
        }
        log(f"sorted T={T}: {med['all'] * 1e3:.1f} us/layer, {gb:.0f} GB/s, {tf:.0f} TFLOP/s; "
            f"gate+up {gu_ms * 1e3:.1f} us, down+combine {dn_ms * 1e3:.1f} us")
        del layers
        torch.cuda.empty_cache()
    return out


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


def bench_workload(wname, q, synth, torch, np, dev, stream, sleep_cycles_for, steps):
    """Another q4 g64 decode / verify configuration, for context: a chain of
    all its layers (distinct weights and routes) per L of the workload, full
    forward; µs per layer and effective expert-weight GB/s."""
    w = synth.WORKLOADS[wname]
    H, I, k = w.H, w.I, w.k
    eb = expert_bytes(H, I)
    out = {"workload": f"{w.name}: {w.routing} routes, chain of {w.n_layers} layers", "per_L": {}}
    for L in w.Ls:
        layers = []
        for layer in range(w.n_layers):
            lay = synth.make_chain_layer(w, L, layer, seed=0, device=dev)
            ids = torch.from_numpy(lay.ids).to(dev)
            tw = torch.from_numpy(lay.weights).to(dev)
            o = torch.empty((L, H), dtype=torch.bfloat16, device=dev)
            ws = q.new_workspace(L, k, lay.bank.E, H, I, dev)
            call = q.PreparedForward(lay.x, ids, tw, lay.bank.tensors(), o, ws, q.MOE_Q4_STAGE_ALL, stream)
            layers.append({"u": int(lay.bank.E), "keep": (lay, ids, tw, o, ws), "call": call})
        torch.cuda.synchronize()

        def chain(delay):
            torch.cuda._sleep(delay)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            th = time.perf_counter()
            for lay in layers:
                lay["call"]()
            e1.record()
            return e0, e1, (time.perf_counter() - th) * 1e3

        warm = chain(0)
        torch.cuda.synchronize()
        delay = sleep_cycles_for(1.5 * warm[2] + 1.0)
        recs = [chain(delay) for _ in range(max(3, steps))]
        torch.cuda.synchronize()
        nl = len(layers)
        ms = float(np.median([a.elapsed_time(b) for a, b, _ in recs])) / nl
        u_mean = sum(l["u"] for l in layers) / nl
        gb = u_mean * eb / (ms * 1e-3) / 1e9
        out["per_L"][str(L)] = {"us_per_layer": round(ms * 1e3, 2), "u_mean": round(u_mean, 2),
                                "eff_GBps": round(gb, 1), "frac_peak": round(gb / PEAK_HBM_GBPS, 4)}
        log(f"{w.name} L={L}: {ms * 1e3:.2f} us/layer, {gb:.0f} GB/s effective")
        del layers
    return out


def bench_codec(codec, args, Ls, q, synth, torch, np, dev, stream, sleep_cycles_for):
    """The verify workload over banks in another codec: chains of layers
    spread over the depth profile (so over the overlap range), full forward
    and gate+up alone, per L."""
    w = synth.WORKLOADS["verify"]
    H, I, E, k = w.H, w.I, w.E, w.k
    code = q.CODECS[codec][0]
    eb = expert_bytes_codec(codec, H, I)
    gub = 2 * eb // 3
    layer_ids = sorted(set(np.linspace(0, w.n_layers - 1, args.codec_layers).round().astype(int).tolist()))
    out = {"workload": f"{w.name} in {codec}, overlap chain of {len(layer_ids)} layers spread over the "
                       f"{w.n_layers}-layer depth profile", "bytes_per_expert": eb, "per_L": {}}
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

        def chain(which, delay):
            torch.cuda._sleep(delay)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            th = time.perf_counter()
            for lay in layers:
                lay["calls"][which]()
            e1.record()
            return e0, e1, (time.perf_counter() - th) * 1e3

        warm = chain("all", 0)
        torch.cuda.synchronize()
        delay = sleep_cycles_for(1.5 * warm[2] + 1.0)
        chain("all", delay)
        torch.cuda.synchronize()
        recs = {wh: [chain(wh, delay) for _ in range(max(3, args.steps))] for wh in ("all", "gateup")}
        torch.cuda.synchronize()
        nl = len(layers)
        med = {wh: float(np.median([a.elapsed_time(b) for a, b, _ in v])) / nl for wh, v in recs.items()}
        u_mean = sum(l["u"] for l in layers) / nl
        gb = u_mean * eb / (med["all"] * 1e-3) / 1e9
        gu_gb = (u_mean * gub + 2 * L * H + 8 * L * k) / (med["gateup"] * 1e-3) / 1e9
        out["per_L"][str(L)] = {"us_per_layer": round(med["all"] * 1e3, 2), "u_mean": round(u_mean, 2),
                                "eff_GBps": round(gb, 1), "frac_peak": round(gb / PEAK_HBM_GBPS, 4),
                                "gateup_us": round(med["gateup"] * 1e3, 2), "gateup_GBps": round(gu_gb, 1)}
        if L in METRIC_LS:
            tot_b += u_mean * eb
            tot_ms += med["all"]
        log(f"{codec} L={L}: {med['all'] * 1e3:.2f} us/layer, {gb:.0f} GB/s effective; gate+up {gu_gb:.0f} GB/s")
        del layers
        torch.cuda.empty_cache()
    if tot_ms > 0:
        out["eff_GBps_over_L"] = round(tot_b / (tot_ms * 1e-3) / 1e9, 1)
        out["frac_peak"] = round(out["eff_GBps_over_L"] / PEAK_HBM_GBPS, 4)
    pl = out["per_L"]
    if "1" in pl and "2" in pl:
        out["L2_over_L1_time"] = round(pl["2"]["us_per_layer"] / pl["1"]["us_per_layer"], 3)
    return out


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
    ap.add_argument("--sorted-mx-Ts", default="512,2048",
                    help="token counts of the same prefill workload over mxfp4 banks (sorted path); empty to skip")
    ap.add_argument("--workloads", default="flash,small,small_pooled",
                    help="other q4 decode / verify configurations timed for context (flash: E=288 top-8 H=4096 "
                         "I=2048 at L=1, 4; small / small_pooled: E=256 top-8 H=2048 I=512 at L=8, 16, 32); "
                         "empty to skip")
    ap.add_argument("--sorted-mx8-Ts", default="512,2048",
                    help="token counts of the same prefill workload over mxfp8 banks (sorted path); empty to skip")
    ap.add_argument("--pair-layers", type=int, default=20,
                    help="layers of each chain timed again as a per-pair baseline (one call per token, so "
                         "an expert shared by tokens is streamed once per token); 0 to skip")
    ap.add_argument("--codecs", default="mxfp4,nvfp4,affine4_g32,affine8_g64,mxfp8",
                    help="other weight codecs timed on the verify workload (comma list; empty to skip)")
    ap.add_argument("--codec-layers", type=int, default=19,
                    help="layers per L of each codec's verify chains (spread over the depth profile)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU work of the baseline sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (reference for hardware "
                         "byte counters) and exit")
    args = ap.parse_args()

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

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_expert_gather_amd as q
    import synth

    Ls = [int(v) for v in args.Ls.split(",")]
    w = synth.WORKLOADS["verify"]
    H, I, E, k = w.H, w.I, w.E, w.k
    eb = expert_bytes(H, I)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

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
            lay["calls"] = {
                "all": q.PreparedForward(lay["x"], lay["ids"], lay["tw"], bt, lay["out"], ws, q.MOE_Q4_STAGE_ALL,
                                         stream),
                "gateup": q.PreparedForward(lay["x"], lay["ids"], lay["tw"], bt, lay["out"], ws,
                                            q.MOE_Q4_STAGE_GATEUP, stream),
                "down": q.PreparedForward(lay["x"], lay["ids"], lay["tw"], bt, lay["out"], ws,
                                          q.MOE_Q4_STAGE_DOWN, stream),
            }
        chains[L] = {"layers": layers}
        torch.cuda.synchronize()
        log(f"L={L}: {args.layers} layers generated, mean unique experts "
            f"{np.mean([l['u'] for l in layers]):.2f}, {time.time() - t0:.1f}s, "
            f"HBM used {torch.cuda.memory_allocated() / 2**30:.1f} GiB")

    # ---- delay kernel calibration: long enough for the host to enqueue a chain ----
    def sleep_cycles_for(ms):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        per_ms = 1_000_000 / max(a.elapsed_time(b), 1e-3)
        return int(per_ms * ms)

    def run_chain(L, which):
        """Enqueue one chain of `which` calls behind a delay kernel; returns (start, end, host ms)."""
        layers = chains[L]["layers"]
        torch.cuda._sleep(sleep_cycles)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        th = time.perf_counter()
        for lay in layers:
            lay["calls"][which]()
        ev1.record()
        return ev0, ev1, (time.perf_counter() - th) * 1e3

    def run_step(which="all"):
        return {L: run_chain(L, which) for L in Ls}

    sleep_cycles = 0
    torch.cuda.synchronize()
    warm = run_step()  # first pass also measures the host enqueue time per chain
    torch.cuda.synchronize()
    host_chain_ms = max(v[2] for v in warm.values())
    sleep_cycles = sleep_cycles_for(1.5 * host_chain_ms + 1.0)
    for _ in range(max(0, args.warmup - 1)):
        run_step()
    torch.cuda.synchronize()
    log(f"warmup done; host enqueue {host_chain_ms:.2f} ms per chain, delay kernel {sleep_cycles} cycles")

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
        per_L[str(L)] = {"us_per_layer": round(us_layer, 2), "eff_GBps": round(gbps, 1),
                         "frac_peak": round(gbps / PEAK_HBM_GBPS, 4), "u_mean": round(u_sum / nl, 2),
                         "gateup_us": round(float(np.median(g_ms)) * 1e3 / nl, 2),
                         "down_combine_us": round(float(np.median(d_ms)) * 1e3 / nl, 2),
                         "chain_ms_median": round(med, 4), "host_enqueue_ms": round(warm[L][2], 3)}
        if L in METRIC_LS or not any(v in METRIC_LS for v in Ls):
            tot_bytes += u_sum * eb * len(recs)
            tot_ms += sum(chain_ms)
        log(f"L={L}: {us_layer:.2f} us/layer, {gbps:.0f} GB/s effective ({gbps / PEAK_HBM_GBPS * 100:.1f}% of 8 TB/s);"
            f" gate+up {per_L[str(L)]['gateup_us']:.1f} us, down+combine {per_L[str(L)]['down_combine_us']:.1f} us")

    # per-pair baseline: the same layers with one call per token (L = 1 each),
    # i.e. every (token, expert) route streams its expert's weights -- the
    # traffic of a per-pair gather without deduplication across tokens
    if args.pair_layers > 0:
        pair = {}
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

            def chain_of(cs):
                torch.cuda._sleep(sleep_cycles)
                e0_, e1_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0_.record()
                for c in cs:
                    c()
                e1_.record()
                return e0_, e1_

            chain_of(calls)
            torch.cuda.synchronize()
            nrep = max(3, args.steps // 2)
            recs_p = [chain_of(calls) for _ in range(nrep)]
            recs_u = [chain_of(ucalls) for _ in range(nrep)]  # the union path on the same layers
            torch.cuda.synchronize()
            us = float(np.median([a_.elapsed_time(b_) for a_, b_ in recs_p])) * 1e3 / len(layers)
            uu = float(np.median([a_.elapsed_time(b_) for a_, b_ in recs_u])) * 1e3 / len(layers)
            pair[str(L)] = {"us_per_layer": round(us, 2), "layers": len(layers),
                            "union_us_per_layer_same_layers": round(uu, 2),
                            "per_pair_over_union": round(us / uu, 3),
                            "slot_bytes_GBps": round(L * k * eb / (us * 1e-6) / 1e9, 1)}
            log(f"per-pair L={L}: {us:.1f} us/layer vs union {uu:.1f} us/layer on the same {len(layers)} layers "
                f"({us / uu:.2f}x)")
        pair_result = pair
    else:
        pair_result = None

    # streaming reference: a plain device copy (read + write bytes / time)
    ref_src = torch.empty(2 * 2**30, dtype=torch.uint8, device=dev).fill_(1)
    ref_dst = torch.empty_like(ref_src)
    ref_dst.copy_(ref_src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        ref_dst.copy_(ref_src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * ref_src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del ref_src, ref_dst

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
        "stream_ref_copy_GBps": round(copy_gbps, 1),
    }
    if "1" in per_L and "2" in per_L:
        result["L2_over_L1_time"] = round(per_L["2"]["us_per_layer"] / per_L["1"]["us_per_layer"], 3)

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

    # ---- prefill workload through the sorted path (grouped MFMA GEMMs) ----
    sorted_Ts = [int(v) for v in args.sorted_Ts.split(",") if v.strip()]
    if sorted_Ts:
        result["sorted_path"] = bench_sorted(args, sorted_Ts, q, synth, torch, np, dev, stream,
                                             lambda ms: sleep_cycles_for(ms))
    # the same prefill workload over the block-scaled banks
    for key, opt, codec in (("sorted_path_mxfp4", args.sorted_mx_Ts, "mxfp4"),
                            ("sorted_path_mxfp8", args.sorted_mx8_Ts, "mxfp8")):
        cTs = [int(v) for v in opt.split(",") if v.strip()]
        if cTs:
            result[key] = bench_sorted(args, cTs, q, synth, torch, np, dev, stream, lambda ms: sleep_cycles_for(ms),
                                       codec=codec)

    # ---- the other decode / verify configurations (context, not the metric) ----
    wnames = [v for v in args.workloads.split(",") if v.strip()]
    if wnames:
        result["other_workloads"] = {n: bench_workload(n, q, synth, torch, np, dev, stream,
                                                        lambda ms: sleep_cycles_for(ms), args.steps) for n in wnames}

    # ---- the same verify workload over banks in other codecs ----
    codecs = [c for c in args.codecs.split(",") if c.strip()]
    if codecs and args.codec_layers > 0:
        cLs = [v for v in Ls if v in METRIC_LS] or Ls
        result["codecs"] = {c: bench_codec(c, args, cLs, q, synth, torch, np, dev, stream,
                                           lambda ms: sleep_cycles_for(ms)) for c in codecs}

    # ---- CPU oracle baseline on a bounded sample, and parity of the same layers ----
    if not args.no_cpu:
        try:
            import oracle

            oracle.build(force=False)
            threads = oracle.threads()
            budget = args.cpu_seconds / len(Ls)  # equal CPU time per L, layers taken in chain order
            cpu_s, cpu_bytes, max_err, bf16_ok, done = 0.0, 0.0, 0.0, True, []
            for L in Ls:
                spent = 0.0
                for lay in chains[L]["layers"]:
                    if spent > budget:
                        break
                    bank = lay["bank"].to("cpu")
                    x = lay["x"].cpu()
                    t = time.perf_counter()
                    ref = oracle.forward_pairs(x, lay["ids_np"], lay["tw_np"], bank)
                    dt = time.perf_counter() - t
                    spent += dt
                    cpu_s += dt
                    cpu_bytes += lay["u"] * eb
                    # contract: fp32 output before the bf16 cast, per-row normwise error
                    got = q.forward_bank(lay["x"], lay["ids"], lay["tw"], lay["bank"], out_dtype=torch.float32)
                    g64 = got.cpu().numpy().astype(np.float64)
                    err = np.linalg.norm(g64 - ref, axis=1) / np.linalg.norm(ref, axis=1)
                    max_err = max(max_err, float(err.max()))
                    # the timed bf16 output is the round-to-nearest-even of that fp32 output
                    bf16_ok &= bool(torch.equal(got.to(torch.bfloat16), lay["out"]))
                    done.append(L)
            cpu_gbps = cpu_bytes / cpu_s / 1e9
            counts = {str(L): done.count(L) for L in Ls if done.count(L)}
            result["cpu_baseline"] = {
                "value": round(cpu_gbps, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": f"per-pair fp64 C oracle (OpenMP, {threads} threads) on the first layers of each "
                          f"chain {counts}; {cpu_s:.1f} s of CPU time; same unique-expert byte metric",
                "us_per_layer_mean": round(cpu_s * 1e6 / max(1, len(done)), 1),
            }
            result["parity"] = {
                "layers": len(done), "max_row_rel_err_f32_out": float(f"{max_err:.3e}"), "tolerance": 1e-3,
                "pass": bool(max_err <= 1e-3 and bf16_ok), "bf16_out_is_rne_of_f32_out": bf16_ok,
            }
        except Exception as exc:  # the baseline must not hide the GPU result
            log(f"cpu baseline failed: {exc!r}")
            result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
