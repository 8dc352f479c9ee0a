"""Benchmark of the GDN-2 token-mixer hot path on one MI355X.

One step = one chunked forward of the B4 H16 T2048 d128 workload (bf16 q/k/v,
fp32 gates and state; returns o and the final state).  The decode step of the
B256 H16 d128 workload (fp32 state updated in place) is timed after the steps,
in a loop of its own: run between two forwards, the write-back of its 268 MB
of state would land in the next forward's time.  Inputs are seeded synthetic
tensors resident in HBM before timing; three input sets (and three decode
states) are rotated so that consecutive calls never find their data in the
256 MB Infinity Cache.

Prints ONE JSON line.  `value` is the chunked forward's throughput in tokens/s
(8192 tokens per call divided by the call's GPU time, from HIP events on the
launch stream); the decode step's HBM rate is reported beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --copy-calibration      # plain 1 GiB copies, for counter scaling
    python bench.py --pmc-summary DIR ...   # fold rocprofv3 counter CSVs into profiles/
    python bench.py --util-summary DIR,...  # fold MFMA / LDS counter runs into profiles/
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0            # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0         # MI355X dense bf16 matrix, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
UTIL_FILE = os.path.join(ROOT, "profiles", "pmc_util.json")
KERNEL_SOURCES = ["gated_delta_rule_19_amd/csrc/gdn2_chunk.hip", "gated_delta_rule_19_amd/csrc/gdn2_recurrent.hip",
                  "gated_delta_rule_19_amd/csrc/gdn2_device.hpp", "gated_delta_rule_19_amd/csrc/gdn2_layout.hpp"]
KERNEL_NAMES = {"prep": "k_chunk_prep", "state": "k_chunk_state", "decode": "k_decode"}


def kernel_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic work (what the method must move / compute; workspace excluded)
# ---------------------------------------------------------------------------
def chunk_bytes_per_ht(dk, dv, io=2, gate=4):
    """q, k, v read + alpha, b, w read + o written, per head-token."""
    return io * (2 * dk + dv) + gate * (2 * dk + dv) + io * dv


def chunk_flops_per_ht(dk, dv, C=64):
    """A, P, W (3 * 2C dk) + U, P.Delta (2 * 2C dv) + W S, Qh S, Ktil^T Delta (3 * 2 dk dv) + solve."""
    return 3 * 2 * C * dk + 2 * 2 * C * dv + 3 * 2 * dk * dv + 2 * C * C / 3


def decode_bytes(B, H, dk, dv, io=2, gate=4):
    """state read + written (fp32) + q, k, v, alpha, b, w read + o written."""
    return B * H * (2 * 4 * dk * dv + io * (2 * dk + dv) + gate * (2 * dk + dv) + io * dv)


def parse_args(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first: the GPU needs ~15 ms of work to reach its steady clocks")
    ap.add_argument("--sets", type=int, default=3, help="rotated input sets (>= 3 defeats the 256 MB MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-chains", type=int, default=0,
                    help="(batch, head) chains in the oracle sample; 0 = the whole workload")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--pmc-summary", metavar="DIR", default=None)
    ap.add_argument("--copy-pmc", metavar="DIR", default=None)
    ap.add_argument("--util-summary", metavar="DIRS", default=None)
    ap.add_argument("--no-long", action="store_true", help="skip the long-context and expanded-value workloads")
    ap.add_argument("--no-prologue", action="store_true", help="skip the side legs (in-kernel prologue, grouped heads, packed batch, backward, output step, short convolution)")
    return ap.parse_args(argv)


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": ms,
                      "GBps": 2 * n / ms / 1e6}))


def _read_counter_csvs(d):
    """Sum counter values per (dispatch, kernel, counter) from rocprofv3 CSV output under d."""
    import csv
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection*.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append(r)
    per = {}
    for r in rows:
        name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
        ctr = r.get("Counter_Name") or r.get("Counter-Name")
        val = float(r.get("Counter_Value") or r.get("Counter-Value") or 0.0)
        disp = r.get("Dispatch_Id") or r.get("Dispatch-Id") or r.get("Correlation_Id")
        per.setdefault((disp, name, ctr), 0.0)
        per[(disp, name, ctr)] += val
    return per


def pmc_summary(dirs, copy_dirs):
    """Fold FETCH_SIZE / WRITE_SIZE runs into profiles/pmc_traffic.json (KiB per dispatch, averaged)."""
    out = {"kernel_sha": kernel_sha(), "kernels": {}, "copy": {}}

    def avg_for(per, match, ctr):
        vals = [v for (disp, name, c), v in per.items() if c == ctr and match(name)]
        return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)

    for d in dirs:
        per = _read_counter_csvs(d)
        for key, kname in KERNEL_NAMES.items():
            for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
                v, n = avg_for(per, lambda s, kname=kname: kname in s, ctr)
                if v is not None:
                    out["kernels"].setdefault(key, {})[ctr + "_KiB"] = v
                    out["kernels"][key][ctr + "_dispatches"] = n
    for d in copy_dirs:
        per = _read_counter_csvs(d)
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            # torch's same-dtype device copy is the runtime's blit kernel; median over its dispatches
            vals = sorted(v for (disp, name, c), v in per.items() if c == ctr and "copyBuffer" in name)
            if vals:
                out["copy"][ctr + "_KiB"] = vals[len(vals) // 2]
    n_kib = (1 << 30) / 1024.0
    f = out["copy"].get("FETCH_SIZE_KiB")
    w = out["copy"].get("WRITE_SIZE_KiB")
    out["copy"]["fetch_factor"] = None if not f else f / n_kib
    out["copy"]["write_factor"] = None if not w else w / n_kib
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
    print(json.dumps(out))


def util_summary(dirs):
    """Fold counter runs (MfmaUtil, MfmaFlopsBF16, LDS counters, ...) into profiles/pmc_util.json:
    per kernel, each counter averaged over its dispatches."""
    out = {"kernel_sha": kernel_sha(), "kernels": {}}
    for d in dirs:
        per = _read_counter_csvs(d)
        for key, kname in KERNEL_NAMES.items():
            ctrs = sorted({c for (disp, name, c) in per if kname in name})
            for ctr in ctrs:
                vals = [v for (disp, name, c), v in per.items() if c == ctr and kname in name]
                out["kernels"].setdefault(key, {})[ctr] = sum(vals) / len(vals)
                out["kernels"][key][ctr + "_dispatches"] = len(vals)
    os.makedirs(os.path.dirname(UTIL_FILE), exist_ok=True)
    with open(UTIL_FILE, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
    print(json.dumps(out))


def load_util(key):
    """Counter averages for kernel `key` from the committed summary, or None when stale."""
    try:
        with open(UTIL_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_sha():
        return None
    return t.get("kernels", {}).get(key)


def load_traffic(key):
    """HBM bytes per launch of kernel `key` from the committed counter summary, or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_sha():
        return None
    k = t.get("kernels", {}).get(key, {})
    c = t.get("copy", {})
    if k.get("FETCH_SIZE_KiB") is None or k.get("WRITE_SIZE_KiB") is None:
        return None
    ff, wf = c.get("fetch_factor"), c.get("write_factor")
    if not ff or not wf:
        return None
    return 1024.0 * (k["FETCH_SIZE_KiB"] / ff + k["WRITE_SIZE_KiB"] / wf)


def main(argv=None):
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "every (batch, head) chain is independent, so more GPUs would each run their own share "
              "without communication -- see the sharding notes in the design document.", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration()
    if args.util_summary:
        return util_summary(args.util_summary.split(","))
    if args.pmc_summary:
        dirs = args.pmc_summary.split(",")
        copy_dirs = args.copy_pmc.split(",") if args.copy_pmc else []
        return pmc_summary(dirs, copy_dirs)

    import torch

    import gated_delta_rule_19_amd as g
    from gated_delta_rule_19_amd import inputs

    dev = torch.device("cuda:0")
    wl_c = inputs.WORKLOADS[1]
    wl_d = inputs.WORKLOADS[2]
    B, T, H, dk, dv = wl_c.B, wl_c.T, wl_c.H, wl_c.dk, wl_c.dv
    sets = [inputs.make(wl_c, seed=100 + i, device=dev) for i in range(args.sets)]
    dsets = [inputs.make(wl_d, seed=200 + i, device=dev) for i in range(args.sets)]
    ws = g.alloc_workspace(g.chunk_fwd_workspace_size(B, T, H, dk, dv, wl_c.io_dtype), dev)
    outs = [torch.empty_like(s["v"]) for s in sets]
    states = [torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev) for _ in sets]
    douts = [torch.empty_like(s["v"]) for s in dsets]
    A = lambda s: (s["q"], s["k"], s["v"], s["alpha"], s["b"], s["w"])
    torch.cuda.synchronize()

    def step(i, ev=None):
        s = i % len(sets)
        if ev is not None:
            ev[0].record()
        g.chunk_fwd(*A(sets[s]), sets[s]["S0"], o=outs[s], S_out=states[s], workspace=ws)
        if ev is not None:
            ev[1].record()

    def decode(i, ev=None):
        d = i % len(dsets)
        if ev is not None:
            ev[0].record()
        g.recurrent_step(*A(dsets[d]), dsets[d]["S0"], o=douts[d], inplace=True)
        if ev is not None:
            ev[1].record()

    # the timed steps: chunked forwards back to back over rotating input sets
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / max(args.steps, 1)
    # the decode step in a loop of its own (its in-place state writes would
    # otherwise be written back during the next chunked forward)
    for i in range(args.warmup):
        decode(i)
    dev_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        decode(args.warmup + i, dev_evs[i])
    torch.cuda.synchronize()
    # the decode step with the layer's output step fused (gated RMS norm on the token's
    # row), and the same as two launches (decode, then the separate output step)
    gts = [torch.randn(d["v"].shape, device=dev).to(d["v"].dtype) for d in dsets]
    nw = torch.ones(wl_d.dv, device=dev)
    ys = [torch.empty_like(d["v"]) for d in dsets]
    gated_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    sep_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for which, evl in ((0, gated_evs), (1, sep_evs)):
        for i in range(args.warmup + args.steps):
            d = i % len(dsets)
            ev = evl[i - args.warmup] if i >= args.warmup else None
            if ev:
                ev[0].record()
            if which == 0:
                g.recurrent_step_gated(*A(dsets[d]), gts[d], nw, dsets[d]["S0"], y=ys[d], inplace=True)
            else:
                g.recurrent_step(*A(dsets[d]), dsets[d]["S0"], o=douts[d], inplace=True)
                g.gated_rmsnorm(douts[d], gts[d], nw, out=ys[d])
            if ev:
                ev[1].record()
    torch.cuda.synchronize()
    per_step = {"chunk": sorted(e[0].elapsed_time(e[1]) for e in evs),
                "decode": sorted(e[0].elapsed_time(e[1]) for e in dev_evs),
                "decode_gated": sorted(e[0].elapsed_time(e[1]) for e in gated_evs),
                "decode_sep": sorted(e[0].elapsed_time(e[1]) for e in sep_evs)}
    dec_ms = sum(per_step["decode"]) / args.steps
    spread = {k_: {"median_us": round(v_[len(v_) // 2] * 1e3, 2), "min_us": round(v_[0] * 1e3, 2)}
              for k_, v_ in per_step.items()}
    copy_gbps = device_copy_gbps(dev)
    chunk_ms = sum(per_step["chunk"]) / args.steps
    # the two launches of the same call timed apart (prep, then the state pass)
    split = split_leg(g, wl_c, sets, dev, args)

    ht = B * T * H
    tokens = B * T
    bpht = chunk_bytes_per_ht(dk, dv)
    alg_chunk = bpht * ht + B * H * dk * dv * 4                   # + final state written
    alg_dec = decode_bytes(wl_d.B, wl_d.H, wl_d.dk, wl_d.dv)
    flops = chunk_flops_per_ht(dk, dv) * ht
    gbps = lambda byts, ms: byts / (ms * 1e-3) / 1e9

    def roof(key, alg, ms, sp):
        ach = gbps(alg, ms)
        tr = load_traffic(key)
        r = {"kernel": KERNEL_NAMES[key], "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS,
             "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBPS, 4),
             "traffic": None if tr is None else round(tr), "alg_bytes": int(alg),
             "us_per_launch": round(ms * 1e3, 2)}
        r.update(sp)
        u = load_util(key)
        if u is not None and "MfmaUtil" in u:
            r["mfma_busy_pct"] = round(u["MfmaUtil"], 2)
        return r

    chunk_gbps = gbps(alg_chunk, chunk_ms)
    # the whole forward call (its two launches): algorithmic bytes over the call's time;
    # traffic = both kernels' counter bytes
    tr_p, tr_s = load_traffic("prep"), load_traffic("state")
    whole_roof = {"kernel": "k_chunk_prep + k_chunk_state (the whole chunked forward call)", "bound": "hbm",
                  "achieved": round(chunk_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                  "frac": round(chunk_gbps / PEAK_HBM_GBPS, 4),
                  "traffic": None if tr_p is None or tr_s is None else round(tr_p + tr_s),
                  "alg_bytes": int(alg_chunk), "us_per_launch": round(chunk_ms * 1e3, 2), **spread["chunk"]}
    result = {
        "metric": "chunk-fwd tokens/s (B4 H16 T2048 d128) + decode-step HBM GB/s; % roofline",
        "value": round(tokens / (chunk_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "chunk fwd B4 H16 T2048 dk=dv=128 (bf16 q/k/v, fp32 gates+state); "
                               "decode step B256 H16 d128 (fp32 state in place) timed in a loop of its own",
                   "global_batch": B, "seq_len": T, "heads": H, "dk": dk, "dv": dv, "chunk": 64,
                   "parallelism": "single GPU", "rotated_input_sets": args.sets},
        "roofline": whole_roof,
        "chunk_fwd": {"kernels": "k_chunk_prep (per-chunk factors to a workspace), then k_chunk_state "
                                 "(the chunks in order, state in matrix-core accumulators)",
                      "us": round(chunk_ms * 1e3, 2), "alg_GBps": round(chunk_gbps, 1),
                      "frac_hbm_roofline": round(chunk_gbps / PEAK_HBM_GBPS, 4),
                      "useful_TFLOPs": round(flops / (chunk_ms * 1e-3) / 1e12, 2),
                      "frac_bf16_mfma_peak": round(flops / (chunk_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "frac_bf16_mfma_peak_at_roofline": round(
                          flops / (alg_chunk / (PEAK_HBM_GBPS * 1e9)) / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "median_us": spread["chunk"]["median_us"], "min_us": spread["chunk"]["min_us"],
                      "stages": {**split,
                                 "roofline_prep": roof("prep", (bpht - 2 * dv) * ht, split["prep_us"] * 1e-3,
                                                       {"median_us": split["prep_median_us"]}),
                                 "roofline_state": roof("state", 2 * dv * ht + B * H * dk * dv * 4,
                                                        split["state_us"] * 1e-3,
                                                        {"median_us": split["state_median_us"]})}},
        "decode": {"us": round(dec_ms * 1e3, 2), "GBps": round(gbps(alg_dec, dec_ms), 1),
                   "frac_hbm_peak": round(gbps(alg_dec, dec_ms) / PEAK_HBM_GBPS, 4),
                   "device_copy_GBps": round(copy_gbps, 1),
                   "frac_of_device_copy": round(gbps(alg_dec, dec_ms) / copy_gbps, 4),
                   "roofline": roof("decode", alg_dec, dec_ms, spread["decode"]),
                   "with_output_step": {
                       "workload": "the same step with the layer's output step (gated RMS norm, SiLU gate) "
                                   "fused into its output write: reads g, writes y instead of o",
                       "us": round(sum(per_step["decode_gated"]) / args.steps * 1e3, 2),
                       "median_us": spread["decode_gated"]["median_us"],
                       "GBps": round(gbps(alg_dec + wl_d.B * wl_d.H * wl_d.dv * 2, sum(per_step["decode_gated"]) / args.steps), 1),
                       "separate_launches_us": round(sum(per_step["decode_sep"]) / args.steps * 1e3, 2),
                       "separate_launches_median_us": spread["decode_sep"]["median_us"]}},
    }
    if not args.no_long:
        result["chunk_fwd_long"] = workload_leg(g, inputs, 3, dev, args)
        result["chunk_fwd_expand_v"] = workload_leg(g, inputs, 4, dev, args)
    if not args.no_prologue:
        result["chunk_fwd_prologue"] = prologue_leg(g, inputs, wl_c, dev, args)
        result["chunk_fwd_grouped"] = grouped_leg(g, inputs, wl_c, dev, args)
        result["chunk_fwd_varlen"] = varlen_leg(g, inputs, wl_c, dev, args)
        result["chunk_bwd"] = backward_leg(g, inputs, wl_c, dev, args)
        result["chunk_bwd_varlen"] = bwd_varlen_leg(g, inputs, wl_c, dev, args)
        result["epilogue"] = epilogue_leg(g, outs, dev, args)
        result["short_conv"] = short_conv_leg(g, dev, args)
        result["conv_fused"] = conv_fused_leg(g, inputs, wl_c, dev, args)

    ok = bool(torch.isfinite(outs[0].float()).all() and torch.isfinite(states[0]).all()
              and torch.isfinite(douts[0].float()).all())
    result["outputs_finite"] = ok

    if not args.no_cpu_baseline:
        cb, ref = cpu_baseline(sets[0], args.cpu_chains, B, T, H, dk, dv)
        result["cpu_baseline"] = cb
        # the timed outputs of input set 0 against the oracle's (all chains)
        result["parity_relL2"] = parity_figures(outs[0], states[0], ref, cb["chains"], H)
        if "chunk_bwd" in result:
            result["chunk_bwd"]["cpu_baseline"] = cpu_baseline_backward(sets[0], B, T, H, dk, dv)
        for key, wi in (("chunk_fwd_long", 3), ("chunk_fwd_expand_v", 4)):
            if key in result:
                leg = result[key]
                x = leg.pop("_set0")
                cbl, refl = cpu_baseline(x["inp"], 0, *x["shape"])
                leg["cpu_baseline"] = cbl
                leg["parity_relL2"] = parity_figures(x["o"], x["S"], refl, cbl["chains"], x["shape"][2])
    for key in ("chunk_fwd_long", "chunk_fwd_expand_v"):
        if key in result:
            result[key].pop("_set0", None)
    print(json.dumps(result), flush=True)
    return 0


def _time_fwd(g, sets, outs, sts, flags, steps, warmup):
    """Time gdn2_chunk_fwd calls back to back over rotating input sets; returns the sorted
    milliseconds per call."""
    import torch
    A = lambda x: (x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"])
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(warmup + steps):
        j = i % len(sets)
        ev = evs[i - warmup] if i >= warmup else None
        if ev:
            ev[0].record()
        g.chunk_fwd(*A(sets[j]), sets[j]["S0"], o=outs[j], S_out=sts[j], flags=flags)
        if ev:
            ev[1].record()
    torch.cuda.synchronize()
    return sorted(e[0].elapsed_time(e[1]) for e in evs)


def _time_split(g, sets, prob, ws, outs, st, flags, steps, warmup):
    """Time the two stages (prep, state pass) over rotating input sets;
    returns (prep, state, total) lists of milliseconds, sorted."""
    import torch
    A = lambda x: (x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"])
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(warmup + steps):
        x = sets[i % len(sets)]
        ev = evs[i - warmup] if i >= warmup else None
        if ev:
            ev[0].record()
        g.chunk_prep(*A(x), ws, flags=flags)
        if ev:
            ev[1].record()
        g.chunk_state(prob, ws, outs[i % len(sets)], x["S0"], st)
        if ev:
            ev[2].record()
    torch.cuda.synchronize()
    return (sorted(e[0].elapsed_time(e[1]) for e in evs), sorted(e[1].elapsed_time(e[2]) for e in evs),
            sorted(e[0].elapsed_time(e[2]) for e in evs))


def _fwd_times(t):
    n = len(t)
    return {"us": round(sum(t) / n * 1e3, 2), "median_us": round(t[n // 2] * 1e3, 2), "min_us": round(t[0] * 1e3, 2)}


def split_leg(g, wl, sets, dev, args):
    """The main workload's two launches timed apart: k_chunk_prep writes every chunk's
    factors to a workspace (1,160 B per head-token at d = 128), k_chunk_state reads them
    back."""
    import torch
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    prob = g.problem(B, T, H, dk, dv, wl.io_dtype)
    ws = g.alloc_workspace(g.chunk_prep_workspace_size(B, T, H, dk, dv, wl.io_dtype), dev)
    outs = [torch.empty_like(x["v"]) for x in sets]
    st = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    steps = max(args.steps // 2, 5)
    prep, state, tot = _time_split(g, sets, prob, ws, outs, st, 0, steps, args.warmup)
    t = _leg_times(prep, state, tot)
    t["prep_median_us"] = round(prep[len(prep) // 2] * 1e3, 2)
    t["state_median_us"] = round(state[len(state) // 2] * 1e3, 2)
    t["tokens_per_s"] = round(B * T / (t["us"] * 1e-6), 1)
    del ws
    return t


def _leg_times(prep, state, tot):
    n = len(tot)
    return {"us": round(sum(tot) / n * 1e3, 2), "median_us": round(tot[n // 2] * 1e3, 2),
            "min_us": round(tot[0] * 1e3, 2), "prep_us": round(sum(prep) / n * 1e3, 2),
            "state_us": round(sum(state) / n * 1e3, 2)}


def workload_leg(g, inputs, idx, dev, args, nsets=3):
    """One of the other chunked workloads (long context B1 H16 T65536 with slow decay;
    expanded values B8 H16 T4096 dk128 dv256 with b in (0, 2) and a nonzero initial state),
    timed like the main workload: gdn2_chunk_fwd calls back to back over `nsets` rotated
    input sets resident in HBM.  Algorithmic bytes: the inputs read,
    o written, the initial state read when there is one and the final state written."""
    import torch
    wl = inputs.WORKLOADS[idx]
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    sets = [inputs.make(wl, seed=1000 * idx + i, device=dev) for i in range(nsets)]
    outs = [torch.empty_like(x["v"]) for x in sets]
    sts = [torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev) for _ in sets]
    steps = max(args.steps // 3, 5)
    t = _fwd_times(_time_fwd(g, sets, outs, sts, 0, steps, args.warmup))
    ms = t["us"] * 1e-3
    ht = B * T * H
    alg = chunk_bytes_per_ht(dk, dv) * ht + B * H * dk * dv * 4 * (2 if wl.s0_std is not None else 1)
    flops = chunk_flops_per_ht(dk, dv) * ht
    ach = alg / (ms * 1e-3) / 1e9
    t_roof = max(alg / (PEAK_HBM_GBPS * 1e9), flops / (PEAK_BF16_TFLOPS * 1e12))
    finite = bool(all(torch.isfinite(o.float()).all() and torch.isfinite(S).all() for o, S in zip(outs, sts)))
    out = {"workload": wl.note + f": B{B} H{H} T{T} dk{dk} dv{dv}, bf16 q/k/v, fp32 gates and state"
                                 + (", S0 ~ N(0, 0.05)" if wl.s0_std is not None else ", zero initial state")
                                 + (f", b = {wl.b_scale:g} sigmoid(N(0,1))" if wl.b_scale != 1.0 else "")
                                 + f", alpha = sigmoid(N({wl.alpha_mu:g}, 1))",
           "tokens_per_s": round(B * T / (ms * 1e-3), 1), **t, "alg_bytes": int(alg),
           "useful_GFLOP": round(flops / 1e9, 2),
           "useful_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
           "frac_bf16_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           # the useful-MFMA fraction a call at the HBM roofline would reach (its ceiling)
           "frac_bf16_mfma_peak_at_roofline": round(flops / t_roof / 1e12 / PEAK_BF16_TFLOPS, 4),
           "roofline": {"kernel": "k_chunk_prep + k_chunk_state (the whole chunked forward call)", "bound": "hbm",
                        "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                        "frac": round(ach / PEAK_HBM_GBPS, 4), "t_roofline_us": round(t_roof * 1e6, 1)},
           "frac_of_roofline_time": round(t_roof / (ms * 1e-3), 4),
           "rotated_input_sets": nsets, "outputs_finite": finite,
           "_set0": {"inp": sets[0], "o": outs[0], "S": sts[0], "shape": (B, T, H, dk, dv)}}
    return out


def prologue_leg(g, inputs, wl, dev, args):
    """The same chunked forward with the layer's prologue moved into the kernels: bf16 gate
    logits (sigmoid in-kernel, b x 2) and unnormalised q/k (L2 norm in-kernel).  Algorithmic
    bytes: q, k, v and the gates in bf16 + o = 1,792 B per head-token at d = 128."""
    import torch
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    flags = g.FLAG_GATE_LOGITS | g.FLAG_NEG_EIGVAL | g.FLAG_QK_L2NORM
    sets = [inputs.make_raw(B, T, H, dk, dv, wl.io_dtype, 300 + i, dev, gate_logits=True, unit_qk=False,
                            gate_dtype=torch.bfloat16) for i in range(args.sets)]
    outs = [torch.empty_like(x["v"]) for x in sets]
    sts = [torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev) for _ in sets]
    st = sts[0]
    steps = max(args.steps // 2, 5)
    t = _fwd_times(_time_fwd(g, sets, outs, sts, flags, steps, args.warmup))
    ms = t["us"] * 1e-3
    ht = B * T * H
    per_ht = 2 * (2 * dk + dv) + 2 * (2 * dk + dv) + 2 * dv
    alg = per_ht * ht + B * H * dk * dv * 4
    gbps = alg / (ms * 1e-3) / 1e9
    return {"workload": "chunk fwd B4 H16 T2048 d128, bf16 q/k/v and bf16 gate logits, flags gate-logits | "
                        "b x 2 | q/k L2 norm (prologue in-kernel), zero initial state",
            "tokens_per_s": round(B * T / (ms * 1e-3), 1), **t,
            "alg_bytes_per_head_token": per_ht,
            "alg_GBps": round(gbps, 1), "frac_hbm_roofline": round(gbps / PEAK_HBM_GBPS, 4),
            "outputs_finite": bool(torch.isfinite(outs[0].float()).all() and torch.isfinite(st).all())}


def grouped_leg(g, inputs, wl, dev, args, H=4):
    """The chunked workload with grouped value heads: 16 value heads (own state, gates,
    values) over 4 query/key heads, bf16 q/k/v, fp32 gates.  Algorithmic bytes per value
    head-token: q and k of its key head shared by 4 (2 x 256 / 4), v and o 256 each, fp32
    gates 1,536 -> 2,176 B at d = 128."""
    import torch
    B, T, Hv, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    sets = [inputs.make_raw(B, T, H, dk, dv, wl.io_dtype, 500 + i, dev, Hv=Hv) for i in range(args.sets)]
    outs = [torch.empty_like(x["v"]) for x in sets]
    sts = [torch.empty(B, Hv, dk, dv, dtype=torch.float32, device=dev) for _ in sets]
    st = sts[0]
    steps = max(args.steps // 2, 5)
    t = _fwd_times(_time_fwd(g, sets, outs, sts, 0, steps, args.warmup))
    ms = t["us"] * 1e-3
    vht = B * T * Hv
    per_vht = 2 * 2 * dk * H // Hv + 2 * dv + 4 * (2 * dk + dv) + 2 * dv
    alg = per_vht * vht + B * Hv * dk * dv * 4
    gbps = alg / (ms * 1e-3) / 1e9
    return {"workload": f"chunk fwd B{B} T{T} H{H} query/key heads, Hv{Hv} value heads, d{dk}, bf16 q/k/v, "
                        "fp32 gates, zero initial state",
            "tokens_per_s": round(B * T / (ms * 1e-3), 1), **t,
            "alg_bytes_per_value_head_token": per_vht,
            "alg_GBps": round(gbps, 1), "frac_hbm_roofline": round(gbps / PEAK_HBM_GBPS, 4),
            "outputs_finite": bool(torch.isfinite(outs[0].float()).all() and torch.isfinite(st).all())}


def varlen_leg(g, inputs, wl, dev, args):
    """The chunked workload's 8,192 tokens per head as a packed batch of sequences of mixed
    length (seeded log-uniform in [16, 4096]), each from a zero state: the whole call (chunk
    plan, prep, state pass) timed.  Algorithmic bytes as for the equal-length workload:
    2,560 B per head-token + the final states."""
    import torch
    H, dk, dv = wl.H, wl.dk, wl.dv
    lens = inputs.length_mix(wl.B * wl.T, seed=1)
    N, T = len(lens), sum(lens)
    sets = [inputs.make_packed(lens, H, dk, dv, wl.io_dtype, 700 + i, dev) for i in range(args.sets)]
    ws = g.alloc_workspace(g.chunk_fwd_varlen_workspace_size(N, T, H, dk, dv, wl.io_dtype), dev)
    outs = [torch.empty_like(x["v"]) for x in sets]
    st = torch.empty(N, H, dk, dv, dtype=torch.float32, device=dev)
    A = lambda x: (x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], x["cu"])
    steps = max(args.steps // 2, 5)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(args.warmup + steps):
        j = i % len(sets)
        ev = evs[i - args.warmup] if i >= args.warmup else None
        if ev:
            ev[0].record()
        g.chunk_fwd_varlen(*A(sets[j]), None, o=outs[j], S_out=st, workspace=ws)
        if ev:
            ev[1].record()
    torch.cuda.synchronize()
    t = sorted(e[0].elapsed_time(e[1]) for e in evs)
    ms = sum(t) / steps
    alg = chunk_bytes_per_ht(dk, dv) * T * H + N * H * dk * dv * 4
    gbps = alg / (ms * 1e-3) / 1e9
    return {"workload": f"packed batch of {N} sequences, {T} tokens (lengths log-uniform in [16, 4096], seed 1), "
                        f"H{H} d{dk}, bf16 q/k/v, fp32 gates, zero initial states",
            "lengths": lens, "tokens_per_s": round(T / (ms * 1e-3), 1), "us": round(ms * 1e3, 2),
            "median_us": round(t[len(t) // 2] * 1e3, 2), "min_us": round(t[0] * 1e3, 2),
            "alg_GBps": round(gbps, 1), "frac_hbm_roofline": round(gbps / PEAK_HBM_GBPS, 4),
            "outputs_finite": bool(torch.isfinite(outs[0].float()).all() and torch.isfinite(st).all())}


def grad_flops_per_chunk(dk, dv, C=64):
    """Useful flops of one chunk's gradient step (k_chunk_grad): the decayed key products
    A, P and their four transposed uses (per 16-column block), U, W, Delta, dDelta, dQh, dP,
    dKtil, dW, du, dT, dEh and the two products of dA."""
    blocks = sum(C - 16 * j for j in range(C // 16)) * 16          # rows x columns over the blocks
    decayed = 6 * blocks * dk * 2
    dense = 2 * (C * dv * C + C * dk * C + C * dv * dk + C * dv * (C + dk) + C * dk * dv + C * C * dv
                 + C * dk * dv + C * dk * dv + C * dv * C + C * C * (dv + dk) + C * dk * C + 2 * C * C * C)
    return decayed + dense


def backward_leg(g, inputs, wl, dev, args):
    """Backward of the chunked workload (B4 H16 T2048 d128, bf16 q/k/v, fp32 gates, zero
    initial state, gradients of o and of the final state): the whole call, which recomputes
    the forward (prep + state pass with checkpoints) before the reverse state pass and the
    per-chunk gradients."""
    import torch
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    sets = [inputs.make_raw(B, T, H, dk, dv, wl.io_dtype, 900 + i, dev) for i in range(2)]
    grads = [inputs.make_out_grads(B, T, H, dk, dv, wl.io_dtype, 950 + i, dev) for i in range(2)]
    ws = g.alloc_workspace(g.chunk_bwd_workspace_size(B, T, H, dk, dv, wl.io_dtype), dev)
    steps = max(args.steps // 5, 3)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    out = None
    for i in range(args.warmup + steps):
        x, (dO, dS) = sets[i % 2], grads[i % 2]
        ev = evs[i - args.warmup] if i >= args.warmup else None
        if ev:
            ev[0].record()
        out = g.chunk_bwd(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], dO, None, dS, workspace=ws)
        if ev:
            ev[1].record()
    torch.cuda.synchronize()
    t = sorted(e[0].elapsed_time(e[1]) for e in evs)
    ms = sum(t) / steps
    finite = all(torch.isfinite(v.float()).all() for v in out.values() if v is not None)
    # the same workload with bf16 gate logits, b x 2 and the q/k L2 norm
    fl = g.FLAG_GATE_LOGITS | g.FLAG_NEG_EIGVAL | g.FLAG_QK_L2NORM
    x = inputs.make_raw(B, T, H, dk, dv, wl.io_dtype, 990, dev, gate_dtype=torch.bfloat16, gate_logits=True,
                        unit_qk=False)
    del ws
    ws = g.alloc_workspace(g.chunk_bwd_workspace_size(B, T, H, dk, dv, wl.io_dtype, torch.bfloat16, flags=fl), dev)
    for i in range(args.warmup + steps):
        dO, dS = grads[i % 2]
        ev = evs[i - args.warmup] if i >= args.warmup else None
        if ev:
            ev[0].record()
        out = g.chunk_bwd(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], dO, None, dS, workspace=ws, flags=fl)
        if ev:
            ev[1].record()
    torch.cuda.synchronize()
    tf = sorted(e[0].elapsed_time(e[1]) for e in evs)
    msf = sum(tf) / steps
    finite = finite and all(torch.isfinite(v.float()).all() for v in out.values() if v is not None)
    nchunks = B * H * ((T + 63) // 64)
    flops = grad_flops_per_chunk(dk, dv) * nchunks
    # algorithmic bytes: q, k, v, dO (bf16) and alpha, b, w (fp32) read, their
    # gradients written in the same dtypes, plus dS_T read and dS0 written
    per_ht = 2 * (2 * dk + 2 * dv) + 4 * (2 * dk + dv) + 2 * (2 * dk + dv) + 4 * (2 * dk + dv)
    alg = per_ht * B * T * H + 2 * B * H * dk * dv * 4
    ach = alg / (ms * 1e-3) / 1e9
    return {"workload": f"chunked backward B{B} H{H} T{T} d{dk}, bf16 q/k/v/dO, fp32 gates, dS_T given",
            "tokens_per_s": round(B * T / (ms * 1e-3), 1), "us": round(ms * 1e3, 2),
            "median_us": round(t[len(t) // 2] * 1e3, 2), "min_us": round(t[0] * 1e3, 2),
            "alg_bytes_per_head_token": per_ht,
            "roofline": {"kernel": "whole backward call (forward recompute + reverse pass + gradients)",
                         "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(ach / PEAK_HBM_GBPS, 4), "alg_bytes": int(alg)},
            "grad_kernel_useful_GFLOP": round(flops / 1e9, 2),
            "with_prologue_flags": {"workload": "the same with bf16 gate logits, b x 2 and the q/k L2 norm",
                                    "us": round(msf * 1e3, 2), "median_us": round(tf[len(tf) // 2] * 1e3, 2)},
            "outputs_finite": bool(finite)}


def bwd_varlen_leg(g, inputs, wl, dev, args):
    """Backward of the packed batch the forward's varlen leg runs (the chunked workload's
    8,192 tokens per head in sequences of mixed length, zero initial states), offsets in
    device memory: the whole call (chunk plan, forward recompute, reverse pass, gradients)
    timed.  Algorithmic bytes as for the equal-length backward."""
    import torch
    H, dk, dv = wl.H, wl.dk, wl.dv
    lens = inputs.length_mix(wl.B * wl.T, seed=1)
    N, T = len(lens), sum(lens)
    sets = [inputs.make_packed(lens, H, dk, dv, wl.io_dtype, 800 + i, dev) for i in range(2)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(850)
    grads = [(torch.randn(1, T, H, dv, generator=gen, device=dev).to(wl.io_dtype),
              torch.randn(N, H, dk, dv, generator=gen, device=dev)) for _ in range(2)]
    ws = g.alloc_workspace(g.chunk_bwd_varlen_workspace_size(N, T, H, dk, dv, wl.io_dtype), dev)
    steps = max(args.steps // 5, 3)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    out = None
    for i in range(args.warmup + steps):
        x, (dO, dS) = sets[i % 2], grads[i % 2]
        ev = evs[i - args.warmup] if i >= args.warmup else None
        if ev:
            ev[0].record()
        out = g.chunk_bwd_varlen(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], dO, x["cu"], None, dS,
                                 workspace=ws)
        if ev:
            ev[1].record()
    torch.cuda.synchronize()
    t = sorted(e[0].elapsed_time(e[1]) for e in evs)
    ms = sum(t) / steps
    per_ht = 2 * (2 * dk + 2 * dv) + 4 * (2 * dk + dv) + 2 * (2 * dk + dv) + 4 * (2 * dk + dv)
    alg = per_ht * T * H + 2 * N * H * dk * dv * 4
    ach = alg / (ms * 1e-3) / 1e9
    finite = all(torch.isfinite(v.float()).all() for v in out.values() if v is not None)
    return {"workload": f"backward of a packed batch of {N} sequences, {T} tokens (lengths log-uniform in "
                        f"[16, 4096], seed 1), H{H} d{dk}, bf16 q/k/v/dO, fp32 gates, dS_T given",
            "tokens_per_s": round(T / (ms * 1e-3), 1), "us": round(ms * 1e3, 2),
            "median_us": round(t[len(t) // 2] * 1e3, 2), "min_us": round(t[0] * 1e3, 2),
            "alg_GBps": round(ach, 1), "frac_hbm_roofline": round(ach / PEAK_HBM_GBPS, 4),
            "outputs_finite": bool(finite)}


def epilogue_leg(g, outs, dev, args):
    """The output step (gated RMS norm with a SiLU gate) on the chunked forward's o
    (B4 H16 T2048 dv128, bf16): reads o and g, writes y -- 6 B per element."""
    import torch
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    gates = [torch.randn(o.shape, generator=gen, device=dev).to(o.dtype) for o in outs]
    wt = torch.ones(outs[0].shape[-1], device=dev)
    ys = [torch.empty_like(o) for o in outs]
    steps = max(args.steps // 2, 5)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(args.warmup + steps):
        j = i % len(outs)
        ev = evs[i - args.warmup] if i >= args.warmup else None
        if ev:
            ev[0].record()
        g.gated_rmsnorm(outs[j], gates[j], wt, out=ys[j])
        if ev:
            ev[1].record()
    torch.cuda.synchronize()
    t = sorted(e[0].elapsed_time(e[1]) for e in evs)
    ms = sum(t) / steps
    nbytes = 3 * outs[0].numel() * outs[0].element_size() + wt.numel() * 4
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "gated RMS norm + SiLU gate on o of the chunked workload, B4 T2048 H16 dv128 bf16",
            "us": round(ms * 1e3, 2), "median_us": round(t[len(t) // 2] * 1e3, 2), "min_us": round(t[0] * 1e3, 2),
            "alg_bytes": int(nbytes),
            "roofline": {"kernel": "k_gated_rmsnorm", "bound": "hbm", "achieved": round(gbps, 1),
                         "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4)}}


def short_conv_leg(g, dev, args, B=4, T=2048, C=3 * 16 * 128, K=4):
    """The short convolution of the prologue on the concatenated q/k/v projections of the
    chunked workload (B4 T2048, 3 x 16 heads x 128 = 6144 channels, bf16, K = 4 taps,
    SiLU, carried state in and out), forward and gradient over rotated input sets.
    Algorithmic bytes: x and y (forward); x, dy and dx (gradient), plus the states and
    the [C, K] weights; the gradient's time covers both of its launches."""
    import torch
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    dt = torch.bfloat16
    n_sets = max(args.sets, 1)
    xs = [torch.randn(B, T, C, generator=gen, device=dev).to(dt) for _ in range(n_sets)]
    dys = [torch.randn(B, T, C, generator=gen, device=dev).to(dt) for _ in range(n_sets)]
    sts = [torch.randn(B, K - 1, C, generator=gen, device=dev).to(dt) for _ in range(n_sets)]
    wt = torch.randn(C, K, generator=gen, device=dev) * 0.5
    ys = [torch.empty_like(x) for x in xs]
    so = torch.empty(B, K - 1, C, dtype=dt, device=dev)
    ws = g.alloc_workspace(g.short_conv_bwd_workspace_size(B, T, C, K), dev)
    steps = max(args.steps // 2, 5)

    def run(fn):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for i in range(args.warmup + steps):
            ev = evs[i - args.warmup] if i >= args.warmup else None
            if ev:
                ev[0].record()
            fn(i % n_sets)
            if ev:
                ev[1].record()
        torch.cuda.synchronize()
        return sorted(e[0].elapsed_time(e[1]) for e in evs)

    t_f = run(lambda j: g.short_conv(xs[j], wt, sts[j], silu=True, out=ys[j], state_out=so))
    t_b = run(lambda j: g.short_conv_bwd(xs[j], wt, dys[j], sts[j], silu=True, workspace=ws))
    el, st_b, w_b = B * T * C * 2, B * (K - 1) * C * 2, C * K * 4
    out = {"workload": f"short convolution B{B} T{T} C{C} (q/k/v of 16 heads x 128) K{K} SiLU bf16, state in/out"}
    for name, t, nbytes, kern in (("forward", t_f, 2 * el + 2 * st_b + w_b, "k_short_conv"),
                                  ("gradient", t_b, 3 * el + 2 * st_b + 2 * w_b,
                                   "k_short_conv_bwd + k_conv_dw_sum (whole call)")):
        ms = sum(t) / len(t)
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"us": round(ms * 1e3, 2), "median_us": round(t[len(t) // 2] * 1e3, 2),
                     "alg_bytes": int(nbytes),
                     "roofline": {"kernel": kern, "bound": "hbm", "achieved": round(gbps, 1),
                                  "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4)}}
    return out


def conv_fused_leg(g, inputs, wl, dev, args, K=4):
    """The prologue's short convolution fused into the chunked forward and into the decode
    step, against the unfused chain (the standalone convolution on the concatenated
    [q | k | v] projection, its three parts made contiguous, then the core call).  Both
    with bf16 gate logits and unnormalised q/k (flags gate-logits | b x 2 | L2 norm),
    K = 4 taps with SiLU and the window carried in and out.  The fused chunked call reads
    each input once: algorithmic bytes = q, k, v and the gates in bf16 + o per head-token,
    plus the [C, K] taps and the windows."""
    import torch
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    flags = g.FLAG_GATE_LOGITS | g.FLAG_NEG_EIGVAL | g.FLAG_QK_L2NORM
    C = 2 * H * dk + H * dv
    gen = torch.Generator(device=dev)
    gen.manual_seed(21)
    n_sets = max(args.sets, 1)
    sets = [inputs.make_raw(B, T, H, dk, dv, wl.io_dtype, 400 + i, dev, gate_logits=True, unit_qk=False,
                            gate_dtype=torch.bfloat16) for i in range(n_sets)]
    wt = torch.randn(C, K, generator=gen, device=dev) * 0.5
    wins = [(torch.randn(B, K - 1, C, generator=gen, device=dev) * 0.5).to(wl.io_dtype) for _ in range(n_sets)]
    xcat = [torch.cat([x["q"].reshape(B, T, -1), x["k"].reshape(B, T, -1), x["v"].reshape(B, T, -1)], -1)
            .contiguous() for x in sets]
    outs = [torch.empty_like(x["v"]) for x in sets]
    S = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    wout = torch.empty(B, K - 1, C, dtype=wl.io_dtype, device=dev)
    ws = g.alloc_workspace(g.chunk_fwd_workspace_size(B, T, H, dk, dv, wl.io_dtype), dev)
    steps = max(args.steps // 2, 5)

    def run(fn, nsteps=steps):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nsteps)]
        for i in range(args.warmup + nsteps):
            ev = evs[i - args.warmup] if i >= args.warmup else None
            if ev:
                ev[0].record()
            fn(i % n_sets)
            if ev:
                ev[1].record()
        torch.cuda.synchronize()
        t = sorted(e[0].elapsed_time(e[1]) for e in evs)
        return {"us": round(sum(t) / len(t) * 1e3, 2), "median_us": round(t[len(t) // 2] * 1e3, 2)}

    A = lambda x: (x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"])

    def fused(j):
        g.chunk_fwd_conv(*A(sets[j]), wt, wins[j], None, conv_silu=True, conv_state_out=wout, o=outs[j],
                         S_out=S, workspace=ws, flags=flags)

    def unfused(j):
        y, _ = g.short_conv(xcat[j], wt, wins[j], silu=True, state_out=wout)
        q = y[..., :H * dk].reshape(B, T, H, dk).contiguous()
        k = y[..., H * dk:2 * H * dk].reshape(B, T, H, dk).contiguous()
        v = y[..., 2 * H * dk:].reshape(B, T, H, dv).contiguous()
        x = sets[j]
        g.chunk_fwd(q, k, v, x["alpha"], x["b"], x["w"], None, o=outs[j], S_out=S, workspace=ws, flags=flags)

    tf, tu = run(fused), run(unfused)
    per_ht = 2 * (2 * dk + dv) + 2 * (2 * dk + dv) + 2 * dv
    alg = per_ht * B * T * H + B * H * dk * dv * 4 + C * K * 4 + 2 * B * (K - 1) * C * 2
    gbps = alg / (tf["us"] * 1e-6) / 1e9
    out = {"workload": f"chunk fwd B{B} H{H} T{T} d{dk}, bf16, gate logits | b x 2 | q/k L2 norm, "
                       f"short convolution K{K} SiLU fused (window in/out)",
           "fused": {**tf, "tokens_per_s": round(B * T / (tf["us"] * 1e-6), 1),
                     "alg_bytes": int(alg), "alg_GBps": round(gbps, 1), "frac_hbm_roofline": round(gbps / PEAK_HBM_GBPS, 4)},
           "unfused_chain": {**tu, "tokens_per_s": round(B * T / (tu["us"] * 1e-6), 1),
                             "calls": "gdn2_short_conv + 3 contiguous copies + gdn2_chunk_fwd"},
           "speedup": round(tu["us"] / tf["us"], 3)}

    # the decode step with its window: B 256, H 16, one token
    Bd = 256
    dsets = [inputs.make_raw(Bd, 1, H, dk, dv, wl.io_dtype, 500 + i, dev, s0_std=0.05, gate_logits=True,
                             unit_qk=False, gate_dtype=torch.bfloat16) for i in range(n_sets)]
    dwin = [(torch.randn(Bd, K - 1, C, generator=gen, device=dev) * 0.5).to(wl.io_dtype) for _ in range(2)]
    dS = torch.empty(Bd, H, dk, dv, dtype=torch.float32, device=dev)
    dout = torch.empty_like(dsets[0]["v"])
    dxcat = [torch.cat([x["q"].reshape(Bd, 1, -1), x["k"].reshape(Bd, 1, -1), x["v"].reshape(Bd, 1, -1)], -1)
             .contiguous() for x in dsets]

    def dfused(j):
        g.recurrent_step_conv(*A(dsets[j]), wt, dwin[j % 2], dsets[j]["S0"], conv_silu=True,
                              conv_state_out=dwin[(j + 1) % 2], o=dout, S_out=dS, flags=flags)

    def dunfused(j):
        y, _ = g.short_conv(dxcat[j], wt, dwin[j % 2], silu=True, state_out=dwin[(j + 1) % 2])
        q = y[..., :H * dk].reshape(Bd, 1, H, dk).contiguous()
        k = y[..., H * dk:2 * H * dk].reshape(Bd, 1, H, dk).contiguous()
        v = y[..., 2 * H * dk:].reshape(Bd, 1, H, dv).contiguous()
        x = dsets[j]
        g.recurrent_step(q, k, v, x["alpha"], x["b"], x["w"], x["S0"], o=dout, S_out=dS, flags=flags)

    df, du = run(dfused), run(dunfused)
    out["decode"] = {"workload": f"decode step B{Bd} H{H} d{dk} bf16 with its window (K{K} SiLU)",
                     "fused": df, "unfused_chain": {**du, "calls": "gdn2_short_conv + 3 copies + gdn2_recurrent_step"},
                     "speedup": round(du["us"] / df["us"], 3)}
    return out


def device_copy_gbps(dev, nbytes=1 << 30, reps=5):
    """Read + write rate of a plain 1 GiB device-to-device copy (the runtime's blit kernel):
    the HBM rate a streaming kernel can reach on this machine."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    """Threads the oracle may use: the process's CPU affinity, capped by OMP_NUM_THREADS when
    set (the GPU host sets it to its per-GPU share of the cores).  Returns (threads, affinity)."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    n = min(aff, int(cap)) if cap.isdigit() and int(cap) > 0 else aff
    return n, aff


def cpu_baseline(inp, chains, B, T, H, dk, dv):
    """The fp64 C oracle on the first `chains` (batch, head) chains (0 = all), all T tokens,
    timed on the host cores; tokens/s scaled by the share of chains run.  Returns the
    record and the oracle's (o, S) for those chains."""
    import torch

    from oracle import c_oracle
    nch = B * H if chains <= 0 else max(1, min(chains, B * H))
    nb = (nch + H - 1) // H
    f = lambda x: None if x is None else x[0:nb].detach().to("cpu", torch.float32).contiguous().numpy()
    arrs = [f(inp[k_]) for k_ in ("q", "k", "v", "alpha", "b", "w")]
    cores, aff = host_threads()
    t0 = time.perf_counter()
    ref = c_oracle.recurrent(*arrs, f(inp["S0"]), nthreads=cores, col_block=16)
    dt = time.perf_counter() - t0
    frac = nb * H / float(B * H)
    tok_s = B * T / (dt / frac)
    return {"value": round(tok_s, 2), "unit": "tokens/s", "cores": cores, "affinity_cores": aff,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"fp64 C oracle (OpenMP over head x 16-column blocks) on {nb * H} of {B * H} "
                      f"(batch, head) chains x {T} tokens of the same inputs: {dt:.2f} s",
            "seconds": round(dt, 3), "chains": nb * H}, ref


def parity_figures(o, S, ref, nchains, H):
    """rel-L2 of the GPU's o and S against the oracle's on the first `nchains` chains:
    whole tensors and the worst (batch, head) chain."""
    import torch

    from oracle.reference import rel_l2, rel_l2_chains
    nb = nchains // H
    on = o[0:nb].detach().to("cpu", torch.float32).numpy()
    Sn = S[0:nb].detach().to("cpu", torch.float32).numpy()
    ro, rS = ref
    return {"o": round(rel_l2(on, ro), 7), "S": round(rel_l2(Sn, rS), 7),
            "o_worst_chain": round(float(rel_l2_chains(on, ro, (0, 2)).max()), 7),
            "S_worst_chain": round(float(rel_l2_chains(Sn, rS, (0, 1)).max()), 7),
            "chains": nb * H, "tol": 2e-2}


def cpu_baseline_backward(inp, B, T, H, dk, dv):
    """The fp64 C backward oracle (token-by-token reverse of the recurrence, OpenMP over
    chains) on the whole workload, output gradients dO ~ N(0,1) and dS_T ~ N(0,1)."""
    import numpy as np
    import torch

    from oracle import c_oracle
    f = lambda x: x.detach().to("cpu", torch.float32).contiguous().numpy()
    rng = np.random.default_rng(5)
    dO = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    dS = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    cores, aff = host_threads()
    t0 = time.perf_counter()
    c_oracle.recurrent_bwd(*(f(inp[k_]) for k_ in ("q", "k", "v", "alpha", "b", "w")), None, dO, dS,
                           nthreads=cores)
    dt = time.perf_counter() - t0
    return {"value": round(B * T / dt, 2), "unit": "tokens/s", "cores": cores, "affinity_cores": aff,
            "kind": "oracle",
            "sample": f"fp64 C backward oracle (OpenMP over chains, reverse token loop) on all {B * H} "
                      f"(batch, head) chains x {T} tokens of the forward's inputs: {dt:.2f} s",
            "seconds": round(dt, 3)}


if __name__ == "__main__":
    sys.exit(main())
