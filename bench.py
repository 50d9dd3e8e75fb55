#!/usr/bin/env python3
"""Throughput of the batched speculative-sampling verify step on one MI355X.

One step = spec_verify_attn + spec_accept_compact (the sampler with the
padding-free compaction in its own kernels) over one batch of the workload (default: B=8 sequences, K=5 drafts, 32 heads x D128, ragged KV
lengths U{512..2048}, V=49152, bf16 KV, fp32 logits, T=0.8, nucleus 0.95).

Inputs are synthetic and seeded; `--sets` input sets (default 16, ~4.5 GB on
the default workload) are resident in HBM before timing and the steps rotate
through them, so the 256 MB Infinity Cache cannot serve a step from the
previous use of its inputs.  The `--warmup` steps and the `--steps` timed
steps are each captured into one HIP graph (the per-step host work of the
ctypes binding would otherwise exceed the GPU time); the timed region is one
replay between two device synchronisations.  The distribution of one step's
time (median, p10, p90) comes from `--steps` further steps launched eagerly
with an event after each (a graph per step would add ~10 us of launch per
step; the eager launches stay ahead of the GPU).  Each entry point alone is
timed both ways: one graph of `--steps` calls (mean) and eager calls with
events (distribution).  The dominant kernel's duration is then measured with
HIP events stamped by its own dispatch, over the same rotation of sets.

Compaction appends each set's accepted KV rows, so a set's KV grows by its
emitted tokens on every use, as in real decoding; the byte counts follow the
realised lengths.  Printed: one JSON line (metric, value = verified tokens/s,
roofline of the dominant kernel timed live with HIP events, the CPU oracle
baseline).
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "verified tokens/sec per verify step (B=8,K=5 ragged); % of HBM peak GB/s"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="bass_b8k5")
    ap.add_argument("--sets", type=int, default=16, help="rotating input sets resident in HBM")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample (0: skip)")
    ap.add_argument("--traffic-json", default=None,
                    help="HBM counter summary of the dominant kernel (default: profiles/)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="only run a plain device copy of this size (counter calibration)")
    ap.add_argument("--k-sweep", default=None,
                    help="comma-separated draft lengths: time the step and each entry point "
                         "per K on the workload's shape (one JSON line per K)")
    ap.add_argument("--sampler-variants", action="store_true",
                    help="time spec_accept alone under its filter and logit-type variants "
                         "(one JSON line each)")
    ap.add_argument("--overlap", action="store_true",
                    help="two-stage pipeline over independent batches: the sampler and compaction "
                         "of batch i on a second stream while batch i+1's attention runs")
    ap.add_argument("--lm-head", action="store_true",
                    help="the target LM head with row statistics (spec_lm_head_stats) and the "
                         "sampler that takes them (spec_accept_prestats), against the sampler "
                         "alone (one JSON line per shape)")
    ap.add_argument("--ragged", action="store_true",
                    help="time the step with ragged draft lengths K_b ~ U{0..K} (one JSON line)")
    ap.add_argument("--traffic-from", default=None,
                    help="only summarise counter passes under this directory (fetch/, write/, "
                         "calib_fetch/, calib_write/) into profiles/traffic_<config>.json")
    return ap.parse_args()


class Hip:
    """hipEvent helpers over libamdhip64 (torch events do not expose their handle)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.h.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.h.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        return ms.value if rc == 0 else None


def kernel_source_hash():
    with open(os.path.join(ROOT, "speculative_decoding_verify_04_amd", "csrc", "attn.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_copy_gbs(mib=1024, reps=5):
    """Bytes moved per second (read + write) by a plain elementwise copy of
    `mib` MiB on this GPU: the streaming rate an HBM-bound kernel can expect,
    reported beside the 8 TB/s specification."""
    import torch
    n = mib * (1 << 20)
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.add(src, 0, out=dst)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        torch.add(src, 0, out=dst)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * n / (ms * 1e-3) / 1e9, 1)


def copy_calibration(mib):
    """A plain elementwise copy kernel of `mib` MiB (reads and writes n bytes once)."""
    import torch
    n = mib * (1 << 20)
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.add(src, 0, out=dst)  # a kernel, unlike copy_, which may become a DMA copy
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


def _counter_rows(d, counter):
    """(kernel name, dispatch id, value) summed over counter instances, from the
    rocprofv3 csv files under directory d."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return [(k[0], k[1], v) for k, v in per.items()]


def traffic_summary(d, config, mib):
    """HBM bytes per launch of the verify-attention kernel from two counter
    passes (FETCH_SIZE and WRITE_SIZE, KiB per dispatch) over this script, each
    scaled by what the same counter reads for the plain copy of `mib` MiB."""
    n = mib * (1 << 20)
    out = {"config": config, "attn_source_sha256_16": kernel_source_hash(), "copy_bytes": n}
    total = 0.0
    for counter, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        calib = [v for k, _, v in _counter_rows(os.path.join(d, "calib_" + sub), counter)
                 if "add" in k.lower() and "random" not in k.lower()]
        kern = [v for k, _, v in _counter_rows(os.path.join(d, sub), counter)
                if "decode_bf16_kernel" in k or "decode_stream_kernel" in k]
        if not calib or not kern:
            raise SystemExit(f"no {counter} rows for the copy or the attention kernel under {d}")
        c_kib = sum(calib) / len(calib)
        factor = n / (c_kib * 1024.0)
        k_kib = sum(kern) / len(kern)
        out[counter] = {"copy_kib_per_dispatch": round(c_kib, 1), "scale": round(factor, 5),
                        "attn_kib_per_dispatch": round(k_kib, 1), "attn_dispatches": len(kern),
                        "attn_bytes_per_launch": int(k_kib * 1024.0 * factor)}
        total += k_kib * 1024.0 * factor
    out["traffic_bytes_per_launch"] = int(total)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the verify step is "
              "built and measured on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    if args.traffic_from:
        tr = traffic_summary(args.traffic_from, args.config, args.copy_calib_mib or 1024)
        with open(os.path.join(ROOT, "profiles", f"traffic_{args.config}.json"), "w") as f:
            json.dump(tr, f, indent=1)
            f.write("\n")
        print(json.dumps(tr), flush=True)
        return
    if args.copy_calib_mib:
        copy_calibration(args.copy_calib_mib)
        return
    if args.k_sweep:
        k_sweep(args, [int(k) for k in args.k_sweep.split(",")])
        return
    if args.ragged:
        ragged_bench(args)
        return
    if args.overlap:
        overlap_bench(args)
        return
    if args.sampler_variants:
        sampler_variants(args)
        return
    if args.lm_head:
        lm_head_bench(args)
        return

    import numpy as np

    from speculative_decoding_verify_04_amd import workloads as W

    cfg = W.CONFIGS[args.config]
    B, K = cfg.B, cfg.K
    S = args.sets
    steps, warmup = args.steps, args.warmup
    # uses of a set by compacting calls: warm-up, timed and eager steps, and
    # 2 S calls alone of each compacting entry point in each of the two timings
    n_comp = 2 * S
    uses_max = math.ceil((warmup + 2 * steps) / S) + 4 * math.ceil(n_comp / S) + 1
    growth = (K + 1) * (uses_max + 1)

    # the sets are generated before anything touches the GPU, in worker processes
    t_gen = time.perf_counter()
    sets = generate_sets(cfg, S, growth)
    print(f"# generated {S} input sets in {time.perf_counter() - t_gen:.1f}s",
          file=sys.stderr, flush=True)

    import torch

    from speculative_decoding_verify_04_amd import api
    from speculative_decoding_verify_04_amd.devio import to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    dsets = [to_device(w, dev) for w in sets]
    bounds = [[int(x) + growth for x in w.kv_len] for w in sets]

    P = cfg.prefix_len
    ws_attn = max(api.spec_verify_attn_workspace_size(B, K, cfg.Hq, cfg.Hkv, cfg.D,
                                                      api.SV_BF16 if cfg.kv_dtype == W.BF16
                                                      else api.SV_F32, bnd, P)
                  for bnd in bounds)
    ws_acc = api.spec_accept_workspace_size(B, K, cfg.V)
    wa = torch.zeros(ws_attn, dtype=torch.uint8, device=dev)
    wacc = torch.zeros(ws_acc, dtype=torch.uint8, device=dev)

    def attn(s):
        t = dsets[s]
        api.spec_verify_attn(t.q, t.k_cache, t.v_cache, t.kv_start, t.kv_len, bounds[s], t.k_new,
                             t.v_new, t.out, K, k_prefix=t.k_prefix, v_prefix=t.v_prefix,
                             status=t.status, workspace=wa)

    def accept(s):
        t = dsets[s]
        api.spec_accept(t.target_logits, None if cfg.greedy else t.draft_logits, t.draft_tokens,
                        t.u_accept, t.u_sample, cfg.temperature, cfg.top_p, cfg.greedy,
                        t.n_accepted, t.out_tokens, status=t.status, workspace=wacc)

    def compact(s):
        t = dsets[s]
        api.spec_compact_kv(t.n_accepted, t.out_tokens, t.kv_len, t.kv_start, t.k_cache,
                            t.v_cache, t.k_new, t.v_new, t.tokens_packed, t.cu_tokens,
                            status=t.status)

    def accept_compact(s):
        t = dsets[s]
        api.spec_accept_compact(t.target_logits, None if cfg.greedy else t.draft_logits,
                                t.draft_tokens, t.u_accept, t.u_sample, cfg.temperature,
                                cfg.top_p, cfg.greedy, t.n_accepted, t.out_tokens, t.kv_len,
                                t.kv_start, t.k_cache, t.v_cache, t.k_new, t.v_new,
                                t.tokens_packed, t.cu_tokens, status=t.status, workspace=wacc)

    def step(s):
        attn(s)
        accept_compact(s)

    # Reference tokens of every set (the sampler does not depend on the KV state).
    ref_n, ref_tok = [], []
    for s in range(S):
        accept(s)
        torch.cuda.synchronize()
        ref_n.append(dsets[s].n_accepted.cpu().numpy().copy())
        ref_tok.append(dsets[s].out_tokens.cpu().numpy().copy())
    emitted = [int((n + 1).sum()) for n in ref_n]

    # The warm-up steps and the timed steps are each captured into one graph
    # (step i uses input set i % S); one replay runs them back to back.
    cap_stream = torch.cuda.Stream()

    def capture(fn, first, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap_stream):
            for i in range(first, first + n):
                fn(i % S)
        return g

    g_warm = capture(step, 0, warmup) if warmup else None
    g_timed = capture(step, warmup, steps)
    torch.cuda.synchronize()
    uses = [0] * S
    if g_warm is not None:
        g_warm.replay()
        for i in range(warmup):
            uses[i % S] += 1
    torch.cuda.synchronize()
    use_at_start = list(uses)

    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    g_timed.replay()
    t_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_stop)
    timed_sets = [(warmup + i) % S for i in range(steps)]
    for s in timed_sets:
        uses[s] += 1
    del g_warm, g_timed

    # Check every set's last outputs against its reference (graph replays vs eager).
    for s in range(S):
        t = dsets[s]
        st = int(t.status.item())
        assert st == 0, f"set {s}: device status {st} ({api.device_error_name(st)})"
        assert np.array_equal(t.n_accepted.cpu().numpy(), ref_n[s]), f"set {s}: n_accepted"
        assert np.array_equal(t.out_tokens.cpu().numpy(), ref_tok[s]), f"set {s}: out_tokens"

    # Dominant kernel: the split-K chunk kernel of spec_verify_attn, timed with
    # HIP events that its own dispatch stamps at kernel start and end (eager
    # launches, over the same rotation of sets and the KV lengths the timed
    # steps left behind).
    hip = Hip()
    evs = [(hip.event(), hip.event()) for _ in range(steps)]
    kern_bytes = []
    for i in range(steps):
        s = timed_sets[i]
        api.sv_set_kernel_events(*evs[i])
        attn(s)
    api.sv_set_kernel_events(None, None)
    torch.cuda.synchronize()

    # The shared workspace served every set: each set's last attention output must
    # equal a run on a fresh workspace (same inputs: bit-identical).
    for s in range(S):
        t = dsets[s]
        prev = t.out.clone()
        fresh = torch.zeros_like(wa)
        api.spec_verify_attn(t.q, t.k_cache, t.v_cache, t.kv_start, t.kv_len, bounds[s], t.k_new,
                             t.v_new, t.out, K, k_prefix=t.k_prefix, v_prefix=t.v_prefix,
                             status=t.status, workspace=fresh)
        torch.cuda.synchronize()
        assert torch.equal(prev, t.out), f"set {s}: attention output differs on a fresh workspace"
        del fresh

    # Each entry point alone over the same rotation, then the per-step
    # distribution.  Attention and the sampler do not change the KV state;
    # compaction appends, so the steps and compactions run last, and their
    # extra uses stay inside the sets' spare rows.
    rot = [(warmup + i) % S for i in range(steps)]
    uses_after_timed = list(uses)
    alone = {}
    for name, fn, sel in (("spec_verify_attn", attn, rot), ("spec_accept", accept, rot),
                          ("spec_compact_kv", compact, list(range(n_comp))),
                          ("spec_accept_compact", accept_compact, list(range(n_comp)))):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap_stream):
            for s in sel:
                fn(s % S)
        torch.cuda.synchronize()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        g.replay()
        b_.record()
        torch.cuda.synchronize()
        graph_us = a_.elapsed_time(b_) * 1e3 / len(sel)
        del g
        _, per = eager_timed(fn, [x % S for x in sel])
        alone[name] = dict(pct(per), graph_mean=round(graph_us, 2))
    _, per_step = eager_timed(step, rot)
    for s in rot:
        uses[s] += 1

    # Bytes and tokens of every timed step from the realised lengths.
    es = 2 if cfg.kv_dtype == W.BF16 else 4
    row_kv = cfg.Hkv * cfg.D * es * 2
    R = cfg.rows
    tokens = 0
    step_bytes = 0
    acc_bytes = 0
    uses = list(use_at_start)
    for i in range(steps):
        s = timed_sets[i]
        L = sets[s].kv_len.astype(np.int64) + uses[s] * (ref_n[s].astype(np.int64) + 1)
        uses[s] += 1
        b = W.algorithmic_bytes(cfg, L, P)
        step_bytes += b["attn"] + b["accept"]
        acc_bytes += b["accept"]
        tokens += emitted[s]
    attn_alone_bytes = 0
    for i in range(steps):  # the kernel timing and the attention alone ran on these lengths
        s = timed_sets[i]
        L = sets[s].kv_len.astype(np.int64) + uses_after_timed[s] * (ref_n[s].astype(np.int64) + 1)
        kern_bytes.append(int(L.sum()) * row_kv + R * row_kv + R * cfg.Hq * cfg.D * es)
        attn_alone_bytes += W.algorithmic_bytes(cfg, L, P)["attn"]
    kern_ms = [hip.elapsed_ms(*evs[i]) for i in range(steps)]
    kern_ok = all(m is not None and m > 0 for m in kern_ms)
    kern_avg_us = 1e3 * sum(kern_ms) / steps if kern_ok else None
    achieved = (sum(kern_bytes) / (1e-3 * sum(kern_ms))) / 1e9 if kern_ok else None
    kern_pct = ([round(1e3 * float(v), 2) for v in np.percentile(kern_ms, [10, 50, 90])]
                if kern_ok else None)
    copy_gbs = measured_copy_gbs()

    # HBM counter summary (if one was taken for the current kernel source)
    traffic = None
    tj = args.traffic_json or os.path.join(ROOT, "profiles", f"traffic_{args.config}.json")
    if os.path.exists(tj):
        with open(tj) as f:
            tr = json.load(f)
        if tr.get("attn_source_sha256_16") == kernel_source_hash():
            traffic = tr.get("traffic_bytes_per_launch")

    ms_step = ms_total / steps
    value = tokens / (ms_total * 1e-3)
    med_attn = alone["spec_verify_attn"]["graph_mean"] * 1e-6
    med_acc = alone["spec_accept"]["graph_mean"] * 1e-6
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "verified tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.kv_dtype == W.BF16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: B={B}, K={K}, {cfg.Hq}/{cfg.Hkv} heads x D{cfg.D}, "
                         f"ragged KV {cfg.len_kind} [{cfg.len_lo},{cfg.len_hi}]"
                         + (f" + shared prefix {P}" if P else "")
                         + f", V={cfg.V}, T={cfg.temperature}, top_p={cfg.top_p}"
                         + (", greedy" if cfg.greedy else "")),
            "B": B, "K": K, "rotating_input_sets": S,
        },
        "step_us_eager": pct(per_step),
        "alone_us": alone,
        "hbm_frac_step": round(step_bytes / (ms_total * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "hbm_frac_attn_plus_accept_alone": round(
            (attn_alone_bytes + acc_bytes) / steps / (med_attn + med_acc) / 1e9 / HBM_PEAK_GBS, 4),
        "step_algorithmic_bytes_avg": int(step_bytes / steps),
        "verified_tokens_per_step_avg": round(tokens / steps, 3),
        "wall_s_timed": round(wall, 4),
        "roofline": {
            "kernel": ("decode_stream_kernel (split-K verify attention, grouped heads)"
                       if cfg.D == 128 and (cfg.Hq // cfg.Hkv) * (cfg.K + 1) > 16 and cfg.B <= 128
                       else "decode_bf16_kernel (split-K verify attention)") if cfg.kv_dtype == 1
                      else "attn_f32_kernel (split-K verify attention, fp32)",
            "bound": "hbm",
            "achieved": round(achieved, 1) if achieved else None,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
            "traffic": traffic,
            "algorithmic_bytes_per_launch_avg": int(sum(kern_bytes) / steps),
            "avg_launch_us": round(kern_avg_us, 3) if kern_avg_us else None,
            "launch_us_p10_p50_p90": kern_pct,
            "measured_copy_GBs": copy_gbs,
            "frac_of_measured_copy": (round(achieved / copy_gbs, 4)
                                      if achieved and copy_gbs else None),
        },
    }

    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(sets, cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def _make_set(cfg_name, sub_seed, growth):
    from speculative_decoding_verify_04_amd import workloads as W
    return W.make_workload(W.CONFIGS[cfg_name], sub_seed=sub_seed, growth_rows=growth)


def generate_sets(cfg, n, growth):
    """The n seeded input sets of a workload, built in worker processes that
    never touch the GPU (at most 8 at a time)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    workers = max(1, min(8, n, os.cpu_count() or 1))
    if workers == 1:
        return [_make_set(cfg.name, s, growth) for s in range(n)]
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        return list(ex.map(_make_set, [cfg.name] * n, range(n), [growth] * n))


def eager_timed(fn, sel):
    """Call fn(s) for s in sel back to back on the current stream with an event
    after each; returns (first-to-last ms, per-call ms).  A short spin kernel
    first lets the host queue the calls ahead of the GPU, so the events time
    GPU work, not launch latency."""
    import torch
    n = len(sel)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    torch.cuda._sleep(2_000_000)
    evs[0].record()
    for i, s in enumerate(sel):
        fn(s)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]
    return evs[0].elapsed_time(evs[n]), per


def pct(ms_list):
    """p10 / median / p90 in microseconds of a list of milliseconds."""
    import numpy as np
    if not ms_list:
        return None
    v = np.percentile(np.asarray(ms_list) * 1e3, [10, 50, 90])
    return {"p10": round(float(v[0]), 2), "median": round(float(v[1]), 2),
            "p90": round(float(v[2]), 2), "n": len(ms_list)}


def k_sweep(args, ks):
    """Verify cost against the draft length K on one workload shape (K = 0 is
    plain decode: one query per sequence, the bonus draw only).  Per K: the
    whole step (graph of `steps` steps), each entry point alone (graph of
    `steps` calls), and the emitted tokens."""
    import numpy as np
    import torch

    from speculative_decoding_verify_04_amd import api
    from speculative_decoding_verify_04_amd import workloads as W
    from speculative_decoding_verify_04_amd.devio import to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    base = W.CONFIGS[args.config]
    steps, S = args.steps, min(args.sets, 4)
    cap_stream = torch.cuda.Stream()

    def timed(fns):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap_stream):
            for fn in fns:
                fn()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / len(fns)  # us per call

    for K in ks:
        cfg = W.small_variant(base, K=K)
        B = cfg.B
        # every set is used 4 * ceil(steps / S) times by the two graphs that compact
        growth = (K + 1) * (4 * math.ceil(steps / S) + 2)
        sets = [W.make_workload(cfg, sub_seed=s, growth_rows=growth) for s in range(S)]
        dsets = [to_device(w, dev) for w in sets]
        bounds = [[int(x) + growth for x in w.kv_len] for w in sets]
        dt = api.SV_BF16 if cfg.kv_dtype == W.BF16 else api.SV_F32
        wa = torch.zeros(max(api.spec_verify_attn_workspace_size(B, K, cfg.Hq, cfg.Hkv, cfg.D, dt,
                                                                 bnd, cfg.prefix_len)
                             for bnd in bounds), dtype=torch.uint8, device=dev)
        wacc = torch.zeros(api.spec_accept_workspace_size(B, K, cfg.V), dtype=torch.uint8,
                           device=dev)

        def attn(s):
            t = dsets[s]
            api.spec_verify_attn(t.q, t.k_cache, t.v_cache, t.kv_start, t.kv_len, bounds[s],
                                 t.k_new, t.v_new, t.out, K, k_prefix=t.k_prefix,
                                 v_prefix=t.v_prefix, status=t.status, workspace=wa)

        def accept(s):
            t = dsets[s]
            api.spec_accept(t.target_logits, None if cfg.greedy else t.draft_logits,
                            t.draft_tokens, t.u_accept, t.u_sample, cfg.temperature, cfg.top_p,
                            cfg.greedy, t.n_accepted, t.out_tokens, status=t.status,
                            workspace=wacc)

        def compact(s):
            t = dsets[s]
            api.spec_compact_kv(t.n_accepted, t.out_tokens, t.kv_len, t.kv_start, t.k_cache,
                                t.v_cache, t.k_new, t.v_new, t.tokens_packed, t.cu_tokens,
                                status=t.status)

        emitted = []
        for s in range(S):
            accept(s)
            torch.cuda.synchronize()
            emitted.append(int((dsets[s].n_accepted.cpu().numpy() + 1).sum()))
        step_us = timed([lambda s=i % S: (attn(s), accept(s), compact(s)) for i in range(steps)])
        attn_us = timed([lambda s=i % S: attn(s) for i in range(steps)])
        acc_us = timed([lambda s=i % S: accept(s) for i in range(steps)])
        comp_us = timed([lambda s=i % S: compact(s) for i in range(steps)])
        for s in range(S):
            st = int(dsets[s].status.item())
            assert st == 0, f"K={K} set {s}: device status {st} ({api.device_error_name(st)})"
        tok = sum(emitted[i % S] for i in range(steps)) / steps
        L = np.concatenate([w.kv_len for w in sets]).astype(np.int64)
        attn_bytes = W.algorithmic_bytes(cfg, L, cfg.prefix_len)["attn"] / S
        print(json.dumps({
            "k_sweep": K, "config": cfg.name, "B": B, "steps": steps,
            "us_per_step": round(step_us, 2), "attn_us": round(attn_us, 2),
            "accept_us": round(acc_us, 2), "compact_us": round(comp_us, 2),
            "emitted_per_step": round(tok, 3),
            "emitted_per_scored_position": round(tok / (B * (K + 1)), 4),
            "verified_tokens_per_s": round(tok / (step_us * 1e-6), 1),
            "attn_GBs_at_start_lengths": round(attn_bytes / (attn_us * 1e-6) / 1e9, 1),
        }), flush=True)
        del dsets, wa, wacc
        torch.cuda.empty_cache()


def ragged_bench(args):
    """The step with ragged draft lengths (each sequence its own K_b ~ U{0..K},
    rows packed without padding): whole step and each entry point, graph-timed
    over rotating input sets; bytes from the realised lengths and row counts."""
    import numpy as np
    import torch

    from speculative_decoding_verify_04_amd import api
    from speculative_decoding_verify_04_amd import workloads as W
    from speculative_decoding_verify_04_amd.devio import ragged_to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    cfg = W.CONFIGS[args.config]
    B, K = cfg.B, cfg.K
    steps, S = args.steps, args.sets
    growth = (K + 1) * (4 * math.ceil(steps / S) + 2)
    rws = [W.make_ragged(W.make_workload(cfg, sub_seed=s, growth_rows=growth),
                         W.ragged_draft_lengths(cfg, s)) for s in range(S)]
    ts = [ragged_to_device(rw, dev) for rw in rws]
    bounds = [[int(x) + growth for x in rw.base.kv_len] for rw in rws]
    dt = api.SV_BF16 if cfg.kv_dtype == W.BF16 else api.SV_F32
    wa = torch.zeros(max(api.spec_verify_attn_ragged_workspace_size(
        B, cfg.Hq, cfg.Hkv, cfg.D, dt, bnd, rw.cu_q, cfg.prefix_len)
        for bnd, rw in zip(bounds, rws)), dtype=torch.uint8, device=dev)
    wacc = torch.zeros(max(api.spec_accept_ragged_workspace_size(B, rw.cu_q, cfg.V) for rw in rws),
                       dtype=torch.uint8, device=dev)
    cap_stream = torch.cuda.Stream()

    def attn(s):
        t = ts[s]
        api.spec_verify_attn_ragged(t.q, t.k_cache, t.v_cache, t.kv_start, t.kv_len, bounds[s],
                                    t.k_new, t.v_new, t.out, t.cu_q, t.cu_q_host,
                                    k_prefix=t.k_prefix, v_prefix=t.v_prefix, status=t.status,
                                    workspace=wa)

    def accept(s):
        t = ts[s]
        api.spec_accept_ragged(t.target_logits, None if cfg.greedy else t.draft_logits,
                               t.draft_tokens, t.u_accept, t.u_sample, t.cu_q, t.cu_q_host,
                               cfg.temperature, cfg.top_p, cfg.greedy, t.n_accepted, t.out_tokens,
                               status=t.status, workspace=wacc)

    def compact(s):
        t = ts[s]
        api.spec_compact_kv_ragged(t.n_accepted, t.out_tokens, t.kv_len, t.kv_start, t.k_cache,
                                   t.v_cache, t.k_new, t.v_new, t.tokens_packed, t.cu_tokens,
                                   t.cu_q, status=t.status)

    def timed(fns):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap_stream):
            for fn in fns:
                fn()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / len(fns)

    emitted = []
    for s in range(S):
        accept(s)
        torch.cuda.synchronize()
        emitted.append(int((ts[s].n_accepted.cpu().numpy() + 1).sum()))
    step_us = timed([lambda s=i % S: (attn(s), accept(s), compact(s)) for i in range(steps)])
    attn_us = timed([lambda s=i % S: attn(s) for i in range(steps)])
    acc_us = timed([lambda s=i % S: accept(s) for i in range(steps)])
    comp_us = timed([lambda s=i % S: compact(s) for i in range(steps)])
    for s in range(S):
        st = int(ts[s].status.item())
        assert st == 0, f"set {s}: device status {st} ({api.device_error_name(st)})"
    es = 2 if cfg.kv_dtype == W.BF16 else 4
    row_kv = cfg.Hkv * cfg.D * es * 2
    tok = sum(emitted[i % S] for i in range(steps)) / steps
    nt = np.mean([int(rw.cu_q[-1]) for rw in rws])
    attn_b = np.mean([int(rw.base.kv_len.sum()) * row_kv + int(rw.cu_q[-1]) * row_kv
                      + 2 * int(rw.cu_q[-1]) * cfg.Hq * cfg.D * es for rw in rws])
    acc_b = np.mean([(2 * int(rw.cu_q[-1]) - B) * cfg.V * 4 for rw in rws])
    print(json.dumps({
        "ragged": True, "config": cfg.name, "B": B, "K_max": K, "steps": steps,
        "K_b": [int(x) for x in rws[0].kb], "query_rows_avg": round(float(nt), 2),
        "us_per_step": round(step_us, 2), "attn_us": round(attn_us, 2),
        "accept_us": round(acc_us, 2), "compact_us": round(comp_us, 2),
        "emitted_per_step": round(tok, 3),
        "verified_tokens_per_s": round(tok / (step_us * 1e-6), 1),
        "attn_GBs_at_start_lengths": round(attn_b / (attn_us * 1e-6) / 1e9, 1),
        "step_hbm_frac_at_start_lengths": round((attn_b + acc_b) / (step_us * 1e-6) / 1e9
                                                / HBM_PEAK_GBS, 4),
    }), flush=True)


def overlap_bench(args):
    """The verify step as a two-stage pipeline over independent batches (the
    rotating input sets stand for independent groups of sequences): batch i's
    sampler and compaction wait for batch i's attention, as in a model, and
    run on a second stream while batch i+1's attention runs on the first; a
    batch's next attention waits for its previous compaction (which appended
    its KV rows).  Timed against the same schedule on one stream; both are
    captured into HIP graphs and replayed between two synchronisations."""
    import numpy as np
    import torch

    from speculative_decoding_verify_04_amd import api
    from speculative_decoding_verify_04_amd import workloads as W
    from speculative_decoding_verify_04_amd.devio import to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    cfg = W.CONFIGS[args.config]
    B, K, S = cfg.B, cfg.K, args.sets
    steps, warmup = args.steps, args.warmup
    uses_max = 4 * math.ceil((steps + warmup) / S) + 1  # four timed schedules below
    growth = (K + 1) * (uses_max + 1)
    sets = [W.make_workload(cfg, sub_seed=s, growth_rows=growth) for s in range(S)]
    dsets = [to_device(w, dev) for w in sets]
    bounds = [[int(x) + growth for x in w.kv_len] for w in sets]
    P = cfg.prefix_len
    dt = api.SV_BF16 if cfg.kv_dtype == W.BF16 else api.SV_F32
    wa = torch.zeros(max(api.spec_verify_attn_workspace_size(B, K, cfg.Hq, cfg.Hkv, cfg.D, dt, bnd, P)
                         for bnd in bounds), dtype=torch.uint8, device=dev)
    wacc = torch.zeros(api.spec_accept_workspace_size(B, K, cfg.V), dtype=torch.uint8, device=dev)

    def attn(s):
        t = dsets[s]
        api.spec_verify_attn(t.q, t.k_cache, t.v_cache, t.kv_start, t.kv_len, bounds[s], t.k_new,
                             t.v_new, t.out, K, k_prefix=t.k_prefix, v_prefix=t.v_prefix,
                             status=t.status, workspace=wa)

    def accept_compact(s):
        t = dsets[s]
        api.spec_accept(t.target_logits, None if cfg.greedy else t.draft_logits, t.draft_tokens,
                        t.u_accept, t.u_sample, cfg.temperature, cfg.top_p, cfg.greedy,
                        t.n_accepted, t.out_tokens, status=t.status, workspace=wacc)
        api.spec_compact_kv(t.n_accepted, t.out_tokens, t.kv_len, t.kv_start, t.k_cache,
                            t.v_cache, t.k_new, t.v_new, t.tokens_packed, t.cu_tokens,
                            status=t.status)

    # reference tokens of every set (the sampler does not read the KV state)
    ref_n, ref_tok = [], []
    for s in range(S):
        t = dsets[s]
        api.spec_accept(t.target_logits, None if cfg.greedy else t.draft_logits, t.draft_tokens,
                        t.u_accept, t.u_sample, cfg.temperature, cfg.top_p, cfg.greedy,
                        t.n_accepted, t.out_tokens, status=t.status, workspace=wacc)
        torch.cuda.synchronize()
        ref_n.append(t.n_accepted.cpu().numpy().copy())
        ref_tok.append(t.out_tokens.cpu().numpy().copy())
    emitted = [int((n + 1).sum()) for n in ref_n]
    kv0 = [t.kv_len.cpu().numpy().copy() for t in dsets]

    sA = torch.cuda.Stream()
    sB = torch.cuda.Stream()

    def capture(first, n, two_streams):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=sA):
            if not two_streams:
                for i in range(first, first + n):
                    attn(i % S)
                    accept_compact(i % S)
                return g
            sB.wait_stream(sA)
            done = [None] * S
            for i in range(first, first + n):
                s = i % S
                if done[s] is not None:
                    sA.wait_event(done[s])  # the batch's previous compaction
                attn(s)
                ea = torch.cuda.Event()
                ea.record(sA)
                with torch.cuda.stream(sB):
                    sB.wait_event(ea)
                    accept_compact(s)
                    ed = torch.cuda.Event()
                    ed.record(sB)
                done[s] = ed
            sA.wait_stream(sB)
        return g

    res = {}
    for mode in ("one_stream", "two_streams", "one_stream", "two_streams"):
        gw = capture(0, warmup, mode == "two_streams") if warmup else None
        gt = capture(warmup, steps, mode == "two_streams")
        torch.cuda.synchronize()
        if gw is not None:
            gw.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()  # replay() launches on the current stream
        gt.replay()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        tokens = sum(emitted[(warmup + i) % S] for i in range(steps))
        res.setdefault(mode, []).append((ms, tokens))
        for s in range(S):
            t = dsets[s]
            st = int(t.status.item())
            assert st == 0, f"{mode} set {s}: device status {st}"
            assert np.array_equal(t.n_accepted.cpu().numpy(), ref_n[s]), f"{mode} set {s}: n_accepted"
            assert np.array_equal(t.out_tokens.cpu().numpy(), ref_tok[s]), f"{mode} set {s}: tokens"
        del gw, gt
    # every compaction ran once per use: the lengths advanced by (n + 1) per use
    for s in range(S):
        uses_s = 0
        for _ in range(4):
            uses_s += sum(1 for i in range(warmup + steps) if i % S == s)
        want = kv0[s] + uses_s * (ref_n[s].astype(np.int64) + 1)
        assert np.array_equal(dsets[s].kv_len.cpu().numpy(), want), f"set {s}: kv_len"
    out = {"overlap": True, "config": cfg.name, "B": B, "K": K, "steps": steps, "sets": S}
    for mode, v in res.items():
        ms = min(x[0] for x in v)
        tokens = v[0][1]
        out[mode] = {"us_per_step": round(1e3 * ms / steps, 2),
                     "verified_tokens_per_s": round(tokens / (ms * 1e-3), 1)}
    out["speedup"] = round(out["one_stream"]["us_per_step"] / out["two_streams"]["us_per_step"], 3)
    print(json.dumps(out), flush=True)


def sampler_variants(args):
    """spec_accept alone on the workload's logits under each filter / logit-type
    variant: graph of `steps` calls over rotating input sets; bytes = every
    logit row read once (target rows only when greedy)."""
    import torch

    from speculative_decoding_verify_04_amd import api
    from speculative_decoding_verify_04_amd import workloads as W
    from speculative_decoding_verify_04_amd.devio import to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    base = W.CONFIGS[args.config]
    steps, S = args.steps, min(args.sets, 4)
    cap_stream = torch.cuda.Stream()
    variants = [
        ("fp32 logits, T, nucleus (the workload)", {}, torch.float32, 0),
        ("bf16 logits, T, nucleus", {}, torch.bfloat16, 0),
        ("fp32 logits, T, top-k 50", {"top_p": 1.0}, torch.float32, 50),
        ("fp32 logits, T, top-k 50, nucleus", {}, torch.float32, 50),
        ("fp32 logits, T, no filter", {"top_p": 1.0}, torch.float32, 0),
        ("fp32 logits, greedy", {"greedy": True}, torch.float32, 0),
    ]
    for name, over, ldt, top_k in variants:
        cfg = W.small_variant(base, **over)
        sets = [W.make_workload(cfg, sub_seed=s, with_kv=False) for s in range(S)]
        ds = [to_device(w, dev, logits_dtype=ldt) for w in sets]
        wacc = torch.zeros(api.spec_accept_workspace_size(cfg.B, cfg.K, cfg.V), dtype=torch.uint8,
                           device=dev)

        def call(s):
            t = ds[s]
            api.spec_accept(t.target_logits, None if cfg.greedy else t.draft_logits,
                            t.draft_tokens, t.u_accept, t.u_sample, cfg.temperature, cfg.top_p,
                            cfg.greedy, t.n_accepted, t.out_tokens, status=t.status,
                            workspace=wacc, top_k=top_k)

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap_stream):
            for i in range(steps):
                call(i % S)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / steps
        for t in ds:
            st = int(t.status.item())
            assert st == 0, f"{name}: device status {st}"
        rows = cfg.B * (cfg.K + 1) + (0 if cfg.greedy else cfg.B * cfg.K)
        nbytes = rows * cfg.V * (2 if ldt == torch.bfloat16 else 4)
        print(json.dumps({"sampler_variant": name, "config": cfg.name, "top_k": top_k,
                          "top_p": cfg.top_p, "greedy": cfg.greedy, "steps": steps,
                          "accept_us": round(us, 2), "logit_bytes": nbytes,
                          "GBs": round(nbytes / (us * 1e-6) / 1e9, 1)}), flush=True)
        del ds, wacc
        torch.cuda.empty_cache()


def lm_head_bench(args):
    """Target LM head (hidden [rows, H] x weight [V, H]^T, bf16 in, fp32 logits)
    with per-part row statistics, then the sampler without a filter, either
    from the logits alone (spec_accept: a statistics pass over every row, then
    the merge and draws) or with the LM head's statistics (spec_accept_prestats:
    no statistics pass).  Synthetic weights of std sigma/sqrt(H) give target
    logits of std sigma; the draft rows use weight a*W + W_noise (the workload's
    draft = a*target + N(0, s^2)) on the same hidden states; draft tokens are
    drawn from the draft softmax.  Shapes: the B=8, K=5 workload (H = 32*128,
    V = 49152, here without its nucleus) and the B=64, K=8 GQA workload
    (V = 128256, no filter).  Each entry point: a graph of `steps` calls over
    two rotating weight/input sets; hipBLASLt's bf16 GEMM of the same shape
    (bf16 output) is timed beside the LM head for context."""
    import torch

    from speculative_decoding_verify_04_amd import api
    from speculative_decoding_verify_04_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    steps, S = args.steps, 2
    cap_stream = torch.cuda.Stream()
    for cname in ("bass_b8k5", "gqa_b64k8"):
        cfg = W.CONFIGS[cname]
        B, K, V, T = cfg.B, cfg.K, cfg.V, cfg.temperature
        H = cfg.Hq * cfg.D
        nt, nd = B * (K + 1), B * K
        P = api.spec_lm_head_parts(V)
        g = torch.Generator(device=dev)
        g.manual_seed(cfg.seed)
        sets = []
        for s in range(S):
            hid = torch.randn((nt, H), generator=g, device=dev).to(torch.bfloat16)
            wt = (torch.randn((V, H), generator=g, device=dev) * (cfg.target_sigma / math.sqrt(H)))
            wd = (cfg.draft_a * wt + torch.randn((V, H), generator=g, device=dev)
                  * (cfg.draft_sigma / math.sqrt(H))).to(torch.bfloat16)
            wt = wt.to(torch.bfloat16)
            hd = hid.view(B, K + 1, H)[:, :K].reshape(nd, H).contiguous()
            d = {"hid": hid, "wt": wt,
                 "zt": torch.empty((nt, V), dtype=torch.float32, device=dev),
                 "pmt": torch.empty((nt, P), dtype=torch.float32, device=dev),
                 "pst": torch.empty((nt, P), dtype=torch.float64, device=dev),
                 "zd": torch.empty((nd, V), dtype=torch.float32, device=dev),
                 "pmd": torch.empty((nd, P), dtype=torch.float32, device=dev),
                 "psd": torch.empty((nd, P), dtype=torch.float64, device=dev),
                 "zb": torch.empty((nt, V), dtype=torch.bfloat16, device=dev),
                 "ua": (torch.randint(0, 1 << 24, (B, K), generator=g, device=dev)
                        .to(torch.float32) * 2.0 ** -24),
                 "us": (torch.randint(0, 1 << 24, (B,), generator=g, device=dev)
                        .to(torch.float32) * 2.0 ** -24),
                 "n": torch.zeros(B, dtype=torch.int32, device=dev),
                 "toks": torch.zeros((B, K + 1), dtype=torch.int32, device=dev),
                 "status": torch.zeros(1, dtype=torch.int32, device=dev)}
            # draft rows: the draft model's logits and statistics (computed
            # before the verify step; not timed)
            api.spec_lm_head_stats(hd, wd, T, d["zd"], d["pmd"], d["psd"])
            gum = -torch.log(-torch.log(torch.rand((nd, V), generator=g, device=dev)
                                        .clamp_(1e-30, 1.0 - 1e-7)))
            d["drafts"] = torch.argmax(d["zd"] / T + gum, dim=-1).to(torch.int32).view(B, K)
            del wd, gum
            api.spec_lm_head_stats(hid, wt, T, d["zt"], d["pmt"], d["pst"])
            sets.append(d)
        torch.cuda.synchronize()
        wacc = torch.zeros(api.spec_accept_workspace_size(B, K, V), dtype=torch.uint8, device=dev)

        def lm(s):
            d = sets[s]
            api.spec_lm_head_stats(d["hid"], d["wt"], T, d["zt"], d["pmt"], d["pst"])

        def blas(s):
            d = sets[s]
            torch.mm(d["hid"], d["wt"].t(), out=d["zb"])

        def acc(s):
            d = sets[s]
            api.spec_accept(d["zt"].view(B, K + 1, V), d["zd"].view(B, K, V), d["drafts"], d["ua"],
                            d["us"], T, 1.0, False, d["n"], d["toks"], status=d["status"],
                            workspace=wacc)

        def accp(s):
            d = sets[s]
            api.spec_accept_prestats(d["zt"].view(B, K + 1, V), d["zd"].view(B, K, V),
                                     d["drafts"], d["ua"], d["us"], T, 1.0, False, d["n"],
                                     d["toks"], d["pmt"], d["pst"], d["pmd"], d["psd"],
                                     status=d["status"], workspace=wacc)

        def graph_us(fn):
            fn(0)  # library handles and workspaces are created outside the capture
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=cap_stream):
                for i in range(steps):
                    fn(i % S)
            torch.cuda.synchronize()
            gr.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            gr.replay()
            b.record()
            torch.cuda.synchronize()
            del gr
            return a.elapsed_time(b) * 1e3 / steps

        # parity of the two sampler forms on these inputs (the same tokens
        # except where a decision is within rounding: none expected here)
        acc(0)
        n0, t0 = sets[0]["n"].clone(), sets[0]["toks"].clone()
        accp(0)
        torch.cuda.synchronize()
        same = bool(torch.equal(n0, sets[0]["n"]) and torch.equal(t0, sets[0]["toks"]))
        lm_us = graph_us(lm)
        blas_us = graph_us(blas)
        acc_us = graph_us(acc)
        accp_us = graph_us(accp)
        step_us = graph_us(lambda s: (lm(s), acc(s)))
        stepp_us = graph_us(lambda s: (lm(s), accp(s)))
        for d in sets:
            st = int(d["status"].item())
            assert st == 0, f"{cname}: device status {st}"
        lm_bytes = V * H * 2 + nt * H * 2 + nt * V * 4 + nt * P * 12
        lm_flops = 2.0 * nt * H * V
        logit_bytes = (nt + nd) * V * 4
        print(json.dumps({
            "lm_head": cname, "rows": nt, "H": H, "V": V, "parts": P, "temperature": T,
            "top_p": 1.0, "steps": steps,
            "lm_head_us": round(lm_us, 2),
            "lm_head_roofline": {
                "algorithmic_bytes": lm_bytes, "flops": lm_flops,
                "GBs": round(lm_bytes / (lm_us * 1e-6) / 1e9, 1),
                "hbm_frac": round(lm_bytes / (lm_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 3),
                "TFLOPs": round(lm_flops / (lm_us * 1e-6) / 1e12, 1),
                "mfma_frac": round(lm_flops / (lm_us * 1e-6) / 1e12 / 2500.0, 3),
                "bound": "hbm" if lm_flops / lm_bytes < 2500.0 / 8.0 else "mfma"},
            "hipblaslt_bf16_gemm_us": round(blas_us, 2),
            "accept_us": round(acc_us, 2), "accept_prestats_us": round(accp_us, 2),
            "sampler_logit_bytes": logit_bytes,
            "step_lm_head_accept_us": round(step_us, 2),
            "step_lm_head_accept_prestats_us": round(stepp_us, 2),
            "same_tokens": same}), flush=True)
        del sets, wacc
        torch.cuda.empty_cache()


def cpu_baseline(sets, cfg, budget_s):
    """The CPU oracle as it stands (single-threaded fp64 C) on whole verify steps."""
    import numpy as np

    from oracle import specref as Ref

    # whole steps over the input sets in turn until the time budget is spent
    # (at most 64 steps); the oracle does not modify its inputs
    tokens, spent, n = 0, 0.0, 0
    while spent < budget_s and n < 64:
        w = sets[n % len(sets)]
        t0 = time.perf_counter()
        Ref.workload_attn(w)
        a = Ref.workload_accept(w)
        Ref.compact_kv(a["n_accepted"], a["out_tokens"], w.kv_len, w.kv_start, w.k_cache,
                       w.v_cache, w.k_new, w.v_new, cfg.K, cfg.Hkv, cfg.D)
        spent += time.perf_counter() - t0
        tokens += int((a["n_accepted"] + 1).sum())
        n += 1
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for l in f:
                if l.startswith("model name"):
                    cpu = l.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(tokens / spent, 3), "unit": "verified tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"{n} whole verify steps of {cfg.name} (input sets taken in turn): fp64 "
                       f"attention of all {cfg.rows}x{cfg.Hq} query rows, sampler on all rows, "
                       f"compaction; {spent:.1f}s on 1 thread of {cpu}")}


if __name__ == "__main__":
    main()
