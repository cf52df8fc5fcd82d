"""Benchmark: KDA chunked prefill (headline) and decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload: prefill B=1, H=32, T=8192, dk=dv=128, bf16 q/k/v, fp32 g,
beta and states, chunk 64, h0 ~ N(0, 0.02).  One step = one kda_chunk_prefill
call over the whole batch (all of its kernels), inputs resident in HBM.
value = tokens/s = B*T / (time per call).

Half a second of untimed calls precedes the W warmup calls (the GPU's
clocks ramp up over the first tens of milliseconds of sustained work).  The
K timed calls carry one event between consecutive calls and none inside a
call: ms_per_step is their mean, "timing" their median and p10/p90.  Per-kernel durations come from a second timed pass of K calls
with HIP events around every launch on its stream; "roofline" takes the
kernel with the longest time per call and charges each of its launches its
share of the whole call's algorithmic bytes (1,540 B per token-head plus the
states; the headline call runs as two chunk windows, so each of its kernels
launches twice and a launch covers half the tokens), "kernel_scoped" with
its own bytes, "path_roofline" gives the whole call's fraction.

Also measured and reported in the same JSON line: decode (256 sequences x 32
heads, d = 128, 128 consecutive in-place steps); packed variable-length
prefill (64 sequences of U[256, 4096] tokens, H = 16); under "next":
speculative verify/commit of 4 draft tokens on the decode batch (token by
token, from the update vectors a verify kept, and a whole round of commit and
verify in one pass over the states), the
headline prefill with a state checkpoint every 512 tokens, and the 1M-token
x 8-head prefill (segment-parallel chain, and the single chain for
comparison); roofline fractions against MI355X peaks (HBM 8 TB/s; bf16 MFMA
2.5 PFLOP/s), and the fp64 oracle timed on the host cores on the same inputs
(a reported baseline, with a parity check of the benchmarked output).

Progress goes to stderr; stdout carries exactly one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (H=32,d=128,T=8192 bf16) + decode steps/s; % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s

# Algorithmic accounting (per token-head, d = 128): q, k, v bf16 (768 B),
# g fp32 (512 B), beta fp32 (4 B), o bf16 (256 B); plus the fp32 state read
# (h0) and written (ht) once per (sequence, head).  Flops: 141,013 per
# token-head at chunk 64 (exact lower triangles, inversion, three state
# products).  Per kernel: the intra-chunk kernel must read q, k, v, g, beta;
# the state kernel must read h0 and write o and ht.
BYTES_PER_TOKEN_HEAD = 1540
INTRA_BYTES_PER_TOKEN_HEAD = 1284
INTER_BYTES_PER_TOKEN_HEAD = 256
FLOPS_PER_TOKEN_HEAD = 141013
DECODE_BYTES_PER_SEQ_HEAD = 132612  # 2 x 64 KiB fp32 state + 1540 B of vectors


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def source_digest():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "gated_delta_rule_97_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(kernel)
    if not rec or rec.get("workload") != workload or rec.get("source_digest") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


PREFILL_WORKLOAD = "prefill B=1 H=32 T=8192 d=128 bf16 chunk=64"
DECODE_WORKLOAD = "decode N=256 H=32 d=128 bf16"
VERIFY_WORKLOAD = "verify N=256 H=32 d=128 bf16, 4 draft tokens"
VERIFY_K = 4
CALIB_BYTES = 1 << 30  # the calibration copy moves 1 GiB each way


def ingest_pmc(fetch_dir, write_dir):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE; both with --headline-only --calibration-copy) into profiles/traffic.json:
    HBM bytes per launch of each KDA kernel, each counter scaled by what it
    reads for the 1 GiB calibration copy."""
    import csv
    import statistics

    def load(d, counter):
        vals = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                key = ("kda_intra" if "kda_intra_kernel" in name
                       else "kda_inter" if ("kda_inter_kernel" in name or "kda_inter_ws_kernel" in name)
                       else "kda_decode" if "kda_decode_kernel" in name
                       else "kda_decode_verify" if "kda_decode_wave_kernel" in name
                       else "copy" if "copy" in name.lower() and float(r["Counter_Value"]) > 0 else None)
                if key:
                    vals.setdefault(key, []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    calib_kib = CALIB_BYTES / 1024
    f_scale = calib_kib / max(fetch["copy"])   # the copy is the largest copy-named dispatch
    w_scale = calib_kib / max(write["copy"])
    out = {"calibration": {"copy_bytes": CALIB_BYTES, "fetch_size_kib": max(fetch["copy"]),
                           "write_size_kib": max(write["copy"]), "fetch_scale": round(f_scale, 4),
                           "write_scale": round(w_scale, 4)}}
    for k, wl in (("kda_intra", PREFILL_WORKLOAD), ("kda_inter", PREFILL_WORKLOAD), ("kda_decode", DECODE_WORKLOAD),
                  ("kda_decode_verify", VERIFY_WORKLOAD)):
        if k in fetch and k in write:
            for c, vals in (("FETCH_SIZE", fetch[k]), ("WRITE_SIZE", write[k])):
                # every dispatch must be the one workload: a run that also launched the
                # kernel on other shapes (the rows beyond the headline) would skew the mean
                if max(vals) > 1.25 * min(vals) + 64:
                    raise SystemExit(f"{k}: {c} ranges {min(vals):.0f}..{max(vals):.0f} KiB over {len(vals)} "
                                     "dispatches; take the counter runs with --headline-only")
            fk, wk = statistics.mean(fetch[k]), statistics.mean(write[k])
            out[k] = {"workload": wl, "source_digest": source_digest(), "dispatches": len(fetch[k]),
                      "fetch_size_kib": round(fk, 1), "write_size_kib": round(wk, 1),
                      "read_bytes_per_launch": int(fk * 1024 * f_scale),
                      "write_bytes_per_launch": int(wk * 1024 * w_scale),
                      "hbm_bytes_per_launch": int(fk * 1024 * f_scale + wk * 1024 * w_scale)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def trace_summary(trace_dir):
    """Markdown table of a rocprofv3 --kernel-trace run of this script, one row
    per KDA kernel, grid, workgroup size and workload: the same kernel launched
    on several workloads keeps a row for each instead of one merged average.
    Persistent kernels keep their grid across workloads, so launches of one
    shape are further split where the sorted durations jump by more than 2x."""
    import csv
    rows = {}
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            if "kda" not in name:
                continue
            key = (name, int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
            rows.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("| kernel | grid | workgroup | calls | avg us | min us | max us |")
    print("|---|---|---|---|---|---|---|")
    for (name, grid, wg), ts in sorted(rows.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        groups = []
        for t in sorted(ts):
            if groups and t <= 2.0 * groups[-1][0]:
                groups[-1].append(t)
            else:
                groups.append([t])
        for g in groups:
            print(f"| `{name}` | {grid} | {wg} | {len(g)} | {sum(g) / len(g):.1f} | {min(g):.1f} | {max(g):.1f} |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-passes", type=int, default=3)
    ap.add_argument("--prewarm-seconds", type=float, default=0.5,
                    help="untimed prefill calls for this long before the warmup steps (the GPU clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="finish with a 1 GiB device-to-device copy (counter calibration)")
    ap.add_argument("--headline-only", action="store_true",
                    help="run only the headline prefill and decode (counter runs: no other launches of "
                         "these kernels on other shapes)")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="print per-launch-shape kernel times of a rocprofv3 --kernel-trace run; no GPU needed")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs; no GPU needed")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.ingest_pmc:
        ingest_pmc(*args.ingest_pmc)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_97_amd as kda
    import workloads

    dev = torch.device("cuda:0")
    spec = workloads.PREFILL_H32_T8K
    B, T, H, dk, dv, C = spec.B, spec.T, spec.H, spec.dk, spec.dv, spec.chunk
    log(f"generating {spec.name}")
    x = workloads.make_prefill(spec)
    d = {k: (v.to(dev) if v is not None else None) for k, v in x.items()}
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_bytes(B, T, H, dk, dv, B, C, kda.KDA_DTYPE_BF16), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def step():
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], chunk_size=C, o=o, ht=ht,
                          workspace=ws)

    # The GPU's clocks ramp up over the first tens of milliseconds of sustained
    # work: right after a few warmup calls the headline call measured ~331 us,
    # ~296 us once warm, with every timing method (events between calls, one
    # pair around all calls, fence-free events).  Untimed calls for a fixed
    # wall time first, then the warmup steps, so the timed calls see steady state.
    log(f"prefill prewarm {args.prewarm_seconds:.2f} s, then warmup x{args.warmup}")
    t_pre = time.perf_counter()
    n_pre = 0
    while time.perf_counter() - t_pre < args.prewarm_seconds:
        for _ in range(16):
            step()
        n_pre += 16
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def timed_calls(fn, n):
        """n back-to-back calls with one event between consecutive calls (no
        event inside a call); returns the per-call times in ms."""
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i in range(n):
            fn()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        return [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]

    def spread(ts):
        s = sorted(ts)
        pick = lambda f: s[min(len(s) - 1, max(0, int(round(f * (len(s) - 1)))))]
        return {"median_us": round(1e3 * pick(0.5), 2), "p10_us": round(1e3 * pick(0.1), 2),
                "p90_us": round(1e3 * pick(0.9), 2), "calls": len(s)}

    log(f"prefill timed x{args.steps}")
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    call_ms = timed_calls(step, args.steps)
    wall = time.perf_counter() - w0
    ms_step = sum(call_ms) / args.steps
    tokens = B * T
    value = tokens / (ms_step * 1e-3)
    headline_spread = spread(call_ms)
    log(f"prefill {ms_step * 1e3:.1f} us/call (median {headline_spread['median_us']:.1f}, p10 "
        f"{headline_spread['p10_us']:.1f}, p90 {headline_spread['p90_us']:.1f}) -> {value / 1e6:.2f} M tokens/s "
        f"(host wall {wall * 1e3 / args.steps:.3f} ms/call)")

    # per-kernel durations: a second timed pass of the same calls, every
    # launch bracketed by events on its stream (kept out of the pass above)
    kda.kda_profile_start(8 * args.steps + 8)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = kda.kda_profile_stop()

    per_kernel_us = {name: 1e3 * tot / n for name, (n, tot) in kt.items()}
    # launches of each kernel per call (2 when the call runs as two chunk
    # windows): a launch covers that share of the call's tokens
    per_call = {name: n / args.steps for name, (n, tot) in kt.items()}
    th = B * T * H
    state_bytes = 2 * B * H * dk * dv * 4
    path_bytes = BYTES_PER_TOKEN_HEAD * th + state_bytes
    kernel_bytes = {"kda_intra": INTRA_BYTES_PER_TOKEN_HEAD * th,
                    "kda_inter": INTER_BYTES_PER_TOKEN_HEAD * th + state_bytes}
    dom = max(per_kernel_us, key=lambda k: per_kernel_us[k] * per_call[k])
    dom_us = per_kernel_us[dom]
    dom_launches = per_call[dom]
    achieved = path_bytes / dom_launches / (dom_us * 1e-6) / 1e9
    own = kernel_bytes.get(dom, 0) / dom_launches / (dom_us * 1e-6) / 1e9
    workload = PREFILL_WORKLOAD
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": load_traffic(dom, workload),
                "avg_launch_us": round(dom_us, 2), "launches_per_call": round(dom_launches, 2),
                "algorithmic_bytes_per_launch": int(path_bytes / dom_launches),
                "kernel_scoped": {"bytes_per_launch": int(kernel_bytes.get(dom, 0) / dom_launches),
                                  "achieved": round(own, 1), "frac": round(own / HBM_PEAK_GBS, 4)}}
    path_gbs = path_bytes / (ms_step * 1e-3) / 1e9
    path_tflops = FLOPS_PER_TOKEN_HEAD * th / (ms_step * 1e-3) / 1e12
    floor_us = path_bytes / (HBM_PEAK_GBS * 1e9) * 1e6
    path_roofline = {"bound": "hbm", "algorithmic_bytes": path_bytes,
                     "achieved_GBps": round(path_gbs, 1), "hbm_frac": round(path_gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_flops": FLOPS_PER_TOKEN_HEAD * th,
                     "achieved_TFLOPs": round(path_tflops, 2),
                     "mfma_frac": round(path_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "attainable_frac": round(floor_us / (ms_step * 1e3), 4),
                     "hbm_floor_us": round(floor_us, 2)}

    # ---------------------------------------------------------------- decode
    dspec = workloads.DECODE
    log(f"decode inputs: {dspec.name}")
    state0 = workloads.make_decode_state(dspec, device=dev)
    state = state0.clone()
    steps_in = [workloads.make_decode_step(dspec, s, device=dev) for s in range(dspec.steps)]
    od = torch.empty((dspec.N, dspec.H, dspec.dv), dtype=torch.bfloat16, device=dev)

    def decode_pass():
        for s in range(dspec.steps):
            xi = steps_in[s]
            kda.decode_step(xi["q"], xi["k"], xi["v"], xi["g"], xi["beta"], state, o=od)

    decode_pass()  # warmup
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    dec_kt = {}
    for p in range(args.decode_passes):
        state.copy_(state0)
        torch.cuda.synchronize()
        if p == args.decode_passes - 1:
            kda.kda_profile_start(dspec.steps + 4)
        ev0.record(stream)
        decode_pass()
        ev1.record(stream)
        torch.cuda.synchronize()
        if p == args.decode_passes - 1:
            dec_kt = kda.kda_profile_stop()
        times.append(ev0.elapsed_time(ev1))
    t_pass = min(times) * 1e-3
    dec_steps_s = dspec.steps / t_pass
    dec_launch_us = 1e3 * dec_kt["kda_decode"][1] / dec_kt["kda_decode"][0]
    dec_bytes = DECODE_BYTES_PER_SEQ_HEAD * dspec.N * dspec.H
    dec_gbs = dec_bytes / (dec_launch_us * 1e-6) / 1e9
    log(f"decode {t_pass * 1e3:.2f} ms / {dspec.steps} steps -> {dec_steps_s:.0f} steps/s, "
        f"{dec_launch_us:.1f} us/launch, {dec_gbs:.0f} GB/s")
    decode = {"workload": "decode N=256 H=32 d=128 bf16, 128 in-place steps",
              "steps_per_s": round(dec_steps_s, 1), "tokens_per_s": round(dec_steps_s * dspec.N, 1),
              "ms_per_step": round(1e3 * t_pass / dspec.steps, 4),
              "roofline": {"kernel": "kda_decode", "bound": "hbm", "achieved": round(dec_gbs, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                           "traffic": load_traffic("kda_decode", DECODE_WORKLOAD),
                           "avg_launch_us": round(dec_launch_us, 2),
                           "algorithmic_bytes_per_launch": dec_bytes}}

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps  # ms

    # ----------------------------- speculative verify / commit on the decode
    # batch (also in --headline-only runs, so its counters can be taken)
    def verify_row(with_commit):
        K = VERIFY_K
        drafts = workloads.make_decode_drafts(dspec, K, device=dev)
        ov = torch.empty((dspec.N, K, dspec.H, dspec.dv), dtype=torch.bfloat16, device=dev)
        nacc = torch.full((dspec.N,), K, dtype=torch.int32, device=dev)
        st_v = state0.clone()
        t_verify = timed(lambda: kda.decode_verify(drafts["q"], drafts["k"], drafts["v"], drafts["g"], drafts["beta"],
                                                   st_v, o=ov), 20)
        st_c = state0.clone()
        t_commit = (timed(lambda: kda.decode_commit(drafts["k"], drafts["v"], drafts["g"], drafts["beta"], nacc,
                                                    st_c), 20) if with_commit else float("nan"))
        if with_commit:  # verify that keeps the update vectors, and the commit from them
            uk = torch.empty((dspec.N, K, dspec.H, dspec.dv), dtype=torch.float32, device=dev)
            t_vkeep = timed(lambda: kda.decode_verify(drafts["q"], drafts["k"], drafts["v"], drafts["g"],
                                                      drafts["beta"], st_v, o=ov, u=uk), 20)
            st_k = state0.clone()
            t_ckept = timed(lambda: kda.decode_commit(drafts["k"], None, drafts["g"], None, nacc, st_k, u=uk), 20)
            # one round in one pass: the accepted drafts committed from their
            # kept u, then the next drafts verified from the committed state
            uk2, st_f = torch.empty_like(uk), state0.clone()
            t_round = timed(lambda: kda.decode_commit_verify((drafts["k"], drafts["g"], uk, nacc), drafts["q"],
                                                             drafts["k"], drafts["v"], drafts["g"], drafts["beta"],
                                                             st_f, o=ov, u=uk2), 20)
            del uk, uk2, st_k, st_f
        else:
            t_vkeep = t_ckept = t_round = float("nan")
        nh = dspec.N * dspec.H
        vbytes = nh * (dspec.dk * dspec.dv * 4 + K * 1540)            # state read once + K tokens' vectors
        cbytes = nh * (2 * dspec.dk * dspec.dv * 4 + K * 1284)        # state read + written, no q or o
        # state read + written; k (bf16), g (fp32) and the kept u (fp32) of K tokens
        kbytes = nh * (2 * dspec.dk * dspec.dv * 4 + K * (dspec.dk * 2 + dspec.dk * 4 + dspec.dv * 4))
        # a round in one pass: the state read + written, the accepted drafts' k, g, u, the new drafts'
        # vectors and outputs, and their kept u
        rbytes = kbytes + nh * K * (1540 + dspec.dv * 4)
        vgbs = vbytes / (t_verify * 1e-3) / 1e9
        cgbs = cbytes / (t_commit * 1e-3) / 1e9
        kgbs = kbytes / (t_ckept * 1e-3) / 1e9
        log(f"verify K={K}: {t_verify * 1e3:.1f} us ({vgbs:.0f} GB/s); commit {t_commit * 1e3:.1f} us ({cgbs:.0f} GB/s); "
            f"keeping u: verify {t_vkeep * 1e3:.1f} us, commit from u {t_ckept * 1e3:.1f} us ({kgbs:.0f} GB/s); "
            f"fused round {t_round * 1e3:.1f} us")
        r = lambda x, nd: None if x != x else round(x, nd)  # NaN (not measured) -> null
        verify = {"workload": f"decode batch N={dspec.N} H={dspec.H} d=128 bf16, {K} draft tokens",
                  "verify_us": round(t_verify * 1e3, 2), "commit_us": r(t_commit * 1e3, 2),
                  "draft_tokens_per_s": round(dspec.N * K / (t_verify * 1e-3), 1),
                  "vs_k_decode_steps": r(K * dec_launch_us / (t_verify * 1e3 + t_commit * 1e3), 3),
                  "roofline": {"kernel": "kda_decode_verify", "bound": "hbm", "achieved": round(vgbs, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(vgbs / HBM_PEAK_GBS, 4),
                               "traffic": load_traffic("kda_decode_verify", VERIFY_WORKLOAD),
                               "avg_launch_us": round(t_verify * 1e3, 2),
                               "algorithmic_bytes_per_launch": vbytes},
                  "commit_roofline": {"kernel": "kda_decode_commit", "bound": "hbm", "achieved": r(cgbs, 1),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": r(cgbs / HBM_PEAK_GBS, 4),
                                      "avg_launch_us": r(t_commit * 1e3, 2), "algorithmic_bytes_per_launch": cbytes},
                  # verify keeping each draft's update vector, then the commit from them
                  "verify_keep_us": r(t_vkeep * 1e3, 2), "commit_kept_us": r(t_ckept * 1e3, 2),
                  "vs_k_decode_steps_kept": r(K * dec_launch_us / (t_vkeep * 1e3 + t_ckept * 1e3), 3),
                  # a speculative round (commit of K accepted drafts + verify of K new ones) three ways
                  "round_us": {"commit_then_verify": r((t_commit + t_verify) * 1e3, 2),
                               "kept_commit_then_verify": r((t_ckept + t_vkeep) * 1e3, 2),
                               "commit_verify_one_pass": r(t_round * 1e3, 2)},
                  "commit_verify_roofline": {"kernel": "kda_decode_commit_verify", "bound": "hbm",
                                             "achieved": r(rbytes / (t_round * 1e-3) / 1e9, 1),
                                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                             "frac": r(rbytes / (t_round * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                             "avg_launch_us": r(t_round * 1e3, 2),
                                             "algorithmic_bytes_per_launch": rbytes},
                  "commit_kept_roofline": {"kernel": "kda_decode_commit_kept", "bound": "hbm", "achieved": r(kgbs, 1),
                                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                           "frac": r(kgbs / HBM_PEAK_GBS, 4), "avg_launch_us": r(t_ckept * 1e3, 2),
                                           "algorithmic_bytes_per_launch": kbytes}}
        del drafts, ov, st_v, st_c
        return verify

    # ------------------------------------- next rows: verify, checkpoints,
    # long context (each with its own algorithmic bytes and roofline)
    def next_rows():
        stride = 512
        nck = kda.checkpoint_count(T, stride, B)
        ck = torch.empty((nck, H, dk, dv), dtype=torch.float32, device=dev)
        t_plain = timed(step, 10)
        t_ck = timed(lambda: kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], chunk_size=C, o=o,
                                               ht=ht, workspace=ws, ckpt_stride=stride, ckpt=ck), 10)
        ckpt = {"workload": f"{workload}, a state checkpoint every {stride} tokens ({nck} per head)",
                "ms_per_call": round(t_ck, 4), "plain_ms_per_call": round(t_plain, 4),
                "overhead_frac": round(t_ck / t_plain - 1.0, 4), "checkpoint_bytes": nck * H * dk * dv * 4}
        log(f"checkpoints: {t_ck * 1e3:.1f} us/call vs {t_plain * 1e3:.1f} plain")
        del ck

        lspec = workloads.LONG_CONTEXT_1M
        log(f"long context: {lspec.name}")
        xl = workloads.make_prefill(lspec, device=dev)
        wl = torch.empty(kda.workspace_bytes(lspec.B, lspec.T, lspec.H, lspec.dk, lspec.dv, lspec.B, lspec.chunk,
                                             kda.KDA_DTYPE_BF16), dtype=torch.uint8, device=dev)
        ol = torch.empty((lspec.B, lspec.T, lspec.H, lspec.dv), dtype=torch.bfloat16, device=dev)
        hl = torch.empty((lspec.B, lspec.H, lspec.dk, lspec.dv), dtype=torch.float32, device=dev)

        def long_step(flags=0):
            kda.chunk_prefill(xl["q"], xl["k"], xl["v"], xl["g"], xl["beta"], None, chunk_size=lspec.chunk, o=ol, ht=hl,
                              workspace=wl, flags=flags)

        t_single = timed(lambda: long_step(kda.KDA_FLAG_NO_SEGMENTS), 2)
        long_step()
        torch.cuda.synchronize()
        kda.kda_profile_start(64)
        t_long = timed(long_step, 3)
        lkt = kda.kda_profile_stop()
        lth = lspec.B * lspec.T * lspec.H
        lbytes = BYTES_PER_TOKEN_HEAD * lth + lspec.B * lspec.H * lspec.dk * lspec.dv * 4
        lgbs = lbytes / (t_long * 1e-3) / 1e9
        log(f"long context: {t_long:.2f} ms/call segmented, {t_single:.2f} ms single chain")
        long_ctx = {"workload": lspec.name.replace("long-context prefill ", "prefill ") + " chunk=64",
                    "ms_per_call": round(t_long, 3), "tokens_per_s": round(lspec.B * lspec.T / (t_long * 1e-3), 1),
                    "single_chain_ms_per_call": round(t_single, 3),
                    "kernels_us": {k: round(1e3 * v[1] / v[0], 1) for k, v in lkt.items()},
                    "path_roofline": {"bound": "hbm", "algorithmic_bytes": lbytes, "achieved_GBps": round(lgbs, 1),
                                      "hbm_frac": round(lgbs / HBM_PEAK_GBS, 4),
                                      "hbm_floor_ms": round(lbytes / (HBM_PEAK_GBS * 1e9) * 1e3, 3)}}
        del xl, wl, ol, hl
        torch.cuda.empty_cache()
        return {"checkpoints": ckpt, "long_context": long_ctx}

    verify = verify_row(with_commit=not args.headline_only)

    # ------------------------- packed variable-length prefill (64 sequences)
    def varlen_row():
        vspec = workloads.VARLEN_64_SEQS
        log(f"varlen: {vspec.name}")
        xv = workloads.make_prefill(vspec, device=dev)
        Tv, Hv, Nv = vspec.total_tokens, vspec.H, vspec.num_seqs
        ov = torch.empty((1, Tv, Hv, vspec.dv), dtype=torch.bfloat16, device=dev)
        hv = torch.empty((Nv, Hv, vspec.dk, vspec.dv), dtype=torch.float32, device=dev)
        wv = torch.empty(kda.workspace_bytes(1, Tv, Hv, vspec.dk, vspec.dv, Nv, vspec.chunk, kda.KDA_DTYPE_BF16),
                         dtype=torch.uint8, device=dev)

        def vstep():
            kda.chunk_prefill(xv["q"], xv["k"], xv["v"], xv["g"], xv["beta"], xv["h0"], xv["cu_seqlens"],
                              chunk_size=vspec.chunk, o=ov, ht=hv, workspace=wv)

        for _ in range(3):
            vstep()
        ts = timed_calls(vstep, 20)
        sp = spread(ts)
        t_med = sp["median_us"] * 1e-6
        vbytes = BYTES_PER_TOKEN_HEAD * Tv * Hv + 2 * Nv * Hv * vspec.dk * vspec.dv * 4
        gbs = vbytes / t_med / 1e9
        kda.kda_profile_start(64)
        for _ in range(5):
            vstep()
        torch.cuda.synchronize()
        vkt = kda.kda_profile_stop()
        log(f"varlen: {sp['median_us']:.1f} us/call (median) -> {Tv / t_med / 1e6:.2f} M tokens/s, {gbs:.0f} GB/s")
        row = {"workload": f"{vspec.name} chunk=64, h0 N(0,0.02), T={Tv}",
               "tokens_per_s": round(Tv / t_med, 1), "timing": sp,
               "kernels_us": {k: round(1e3 * v[1] / v[0], 1) for k, v in vkt.items()},
               "path_roofline": {"bound": "hbm", "algorithmic_bytes": vbytes, "achieved_GBps": round(gbs, 1),
                                 "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                                 "hbm_floor_us": round(vbytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2)}}
        del xv, ov, hv, wv
        torch.cuda.empty_cache()
        return row

    varlen = None if args.headline_only else varlen_row()
    nxt = None if args.headline_only else next_rows()
    if nxt is not None:
        nxt["speculative_verify"] = verify

    # -------------------------------------------- oracle on the host cores
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        f = lambda t: workloads.to_numpy_f32(t)[0]
        q, k, v, g, b = (f(x[n]) for n in ("q", "k", "v", "g", "beta"))
        h0 = x["h0"].numpy().astype(np.float64)
        threads = oracle.max_threads()
        log(f"oracle on the host: full workload, {threads} threads")
        # the whole workload, repeated until about 10 s of wall time have passed
        reps, t0 = 0, time.perf_counter()
        while True:
            o_ref, ht_ref = oracle.prefill(q, k, v, g, b, h0)
            reps += 1
            t_cpu = time.perf_counter() - t0
            if t_cpu >= 10.0 or reps >= 64:
                break
        cpu = {"value": round(reps * tokens / t_cpu, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"the full headline workload ({T} tokens x {H} heads), fp64 token loop, "
                         f"{reps} runs in {t_cpu:.2f} s wall",
               "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}
        step()
        torch.cuda.synchronize()
        on = o[0].double().cpu().numpy()
        hn = ht.double().cpu().numpy()
        rel = lambda a, r: float(np.linalg.norm(a - r) / np.linalg.norm(r))
        parity = {"o_rel_l2": rel(on, o_ref), "ht_rel_l2": rel(hn, ht_ref), "tol": 2e-2}
        log(f"oracle {reps} x {t_cpu / reps:.2f} s; parity o {parity['o_rel_l2']:.2e} ht {parity['ht_rel_l2']:.2e}")

        # decode baseline: the first 4 steps of the decode workload
        ref_state = state0.double().cpu().numpy()
        nd, t0 = 0, time.perf_counter()
        while nd < dspec.steps:
            xi = steps_in[nd]
            oracle.decode_step(*(workloads.to_numpy_f32(xi[n]) for n in ("q", "k", "v", "g", "beta")),
                               ref_state)
            nd += 1
            if time.perf_counter() - t0 >= 5.0:
                break
        t_dec_cpu = (time.perf_counter() - t0) / nd
        decode["cpu_baseline"] = {"value": round(1.0 / t_dec_cpu, 3), "unit": "steps/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"the first {nd} of the {dspec.steps} decode steps, "
                                            f"{t_dec_cpu * nd:.2f} s wall"}

    if args.calibration_copy:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    out = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded generators: unit-norm q/k, N(0,1) v, sigmoid beta, g=-5*sigmoid(N(0,1)))",
           "config": {"workload": workload, "B": B, "T": T, "H": H, "dk": dk, "dv": dv, "chunk": C,
                      "h0": "N(0,0.02)"},
           "roofline": roofline, "path_roofline": path_roofline,
           "timing": dict(headline_spread, prewarm_calls=n_pre, prewarm_s=args.prewarm_seconds),
           "kernels_us": {k: round(v, 2) for k, v in per_kernel_us.items()},
           "kernel_launches_per_call": {k: round(v, 2) for k, v in per_call.items()},
           "cpu_baseline": cpu, "parity": parity, "decode": decode, "varlen": varlen,
           "next": nxt if nxt is not None else {"speculative_verify": verify},
           "source_digest": source_digest()}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
