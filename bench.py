"""ForkAttention round benchmark on one MI355X.

One timed step = one whole round of the hot path over a synthetic batch: for
every sub-round of the round (a round larger than the largest capacity is split
at request boundaries), host planning of the flat stream, choice of the
smallest captured capacity bucket, the metadata upload (pinned H2D copy) and the
bucket's graph replay, which expands the metadata, runs the GDN layer (trunk
call, then question call), rotates keys, runs the tree-masked attention
layer(s) and the selective readout.  Payloads are resident in HBM before the
timed region: every sub-round has a buffer set of its own, so the replays of a
round are enqueued back to back.

Default workload: the 64-question fan-out round (R=16 requests, P=8192, 64
questions of 16..64 tokens each, 2-8 options; GDN 16 heads x 128, attention 16 q
/ 4 kv heads x 256, hidden 2048, bf16 activations, fp32 GDN state): about 172k
stream rows, run as three replays of the 65536-row bucket (6 + 6 + 4 requests).

Prints one JSON line.  ``value`` is stream tokens per second of whole rounds
(each round holds one GDN layer, one attention layer and the readout).
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # fp32 matrix
COPY_BYTES = 256 << 20         # size of the reference copy of the counter pass


# Kernel sources behind each timed entry point (their hash pins the HBM counter figures).
KERNEL_SOURCES = {
    "fork_gdn_trunks": ["gdn_chunk_kernels.hip"], "fork_gdn_questions": ["gdn_chunk_kernels.hip"],
    "attn_prepare": ["attn_kernels.hip"], "attn_core": ["attn_kernels.hip"],
    "attn_prepare_swa": ["attn_kernels.hip"], "attn_core_swa": ["attn_kernels.hip"],
    "readout": ["readout_kernels.hip"],
}
COUNTERS_FILES = {1: "hbm_counters_short_rounds.md", 3: "hbm_counters_question_fanout.md"}


def source_digest(name: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name] + ["device_common.hpp", "flide_internal.hpp"]:
        with open(os.path.join(ROOT, "tree_forked_hybrid_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str, config: int):
    """HBM bytes per round of `name` (summed over the round's launches) from the committed rocprofv3
    counter summary of this workload (FETCH_SIZE + WRITE_SIZE, scaled by the reference copy), or None when
    there is none or the kernel source changed since."""
    fn = COUNTERS_FILES.get(config)
    path = os.path.join(ROOT, "profiles", fn) if fn else None
    if not path or not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) >= 5 and cells[0] == name:
                try:
                    return float(cells[4]) if cells[1] == source_digest(name) else None
                except ValueError:
                    return None
    return None


def _round_up(x: int, m: int) -> int:
    return ((x + m - 1) // m) * m


def algorithmic_work(rnd):
    """Algorithmic bytes / FLOPs per kernel of one (sub-)round (what the method must move or compute)."""
    s = rnd.shapes
    b = 2 if rnd.dtype == "bf16" else 4
    T = sum((r.P - r.m) + sum(r.q_len) for r in rnd.requests)
    R = len(rnd.requests)
    nq = sum(len(r.q_len) for r in rnd.requests)

    # attention: visible pairs per q head; a row at position t sees min(t + 1, W) keys (W = 0: t + 1)
    def pairs(W):
        tot = 0
        for r in rnd.requests:
            for t in list(range(r.m, r.P)) + [r.P + u for L in r.q_len for u in range(L)]:
                tot += min(t + 1, W) if W > 0 else t + 1
        return tot
    attn = {}
    for name, W in [("attn", 0)] + ([("swa", s.swa_window)] if s.swa_window > 0 else []):
        pr = pairs(W)
        flops = 4.0 * s.d * s.Hq * pr
        cached = sum(min(r.m, W) if W > 0 else r.m for r in rnd.requests)
        byts = T * (2 * s.Hq + 2 * s.Hkv) * s.d * b + cached * 2 * s.Hkv * s.d * b
        attn[name] = {"flops": flops, "bytes": byts, "pairs": pr,
                      # rotary K and transposed V: read k, v and write both once
                      "prep_bytes": 4 * T * s.Hkv * s.d * b}
    C = s.channels
    per_row = s.H * ((2 * s.dk + s.dv) * b + 8 + s.dv * b)
    state = 4 * s.H * s.dv * s.dk
    window = (s.conv_k - 1) * C * b
    trunk_rows = sum(r.P - r.m for r in rnd.requests)
    q_rows = T - trunk_rows
    resumed = sum(1 for r in rnd.requests if r.m > 0)
    gdn0 = trunk_rows * per_row + R * (state + window) + resumed * (state + window)
    gdn1 = q_rows * per_row + sum(1 for r in rnd.requests if r.q_len) * (state + window)
    n_opt = sum(sum(r.n_opt) for r in rnd.requests)
    ro = nq * s.hidden * b + n_opt * (s.hidden * b + 8) + 4 * (nq + 1)
    return {"T": T, "attn": attn, "gdn0": gdn0, "gdn1": gdn1, "readout": ro}


def _host_cpu() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for ln in out.splitlines():
            if ln.startswith("Model name:"):
                return ln.split(":", 1)[1].strip()
    except Exception:  # noqa: BLE001
        pass
    return platform.processor() or "unknown"


def cpu_baseline(rnd, n_trunk_sample: int = 48):
    """The oracle (as it stands) on a bounded sample of the round's first request: its GDN over the whole
    trunk and its first question (per-token recurrence: the full cost of those rows), its attention at
    ``n_trunk_sample`` trunk rows at evenly spaced positions plus every row of the question, and the
    question's readout.  The trunk's attention time is scaled to all trunk rows by the ratio of visible keys
    (the oracle's per-row attention cost is linear in them); value = sampled rows / (measured GDN, question
    attention and readout time + scaled trunk attention time).  Timed with one BLAS thread (the reported
    value) and again with a BLAS thread per logical CPU of the host."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # noqa: BLE001
        threadpool_limits = None
    from oracle.attention import prompt_attention
    from oracle.gdn import gdn_prompt
    from oracle.readout import option_probs
    sub = rnd.subset([0])
    r = sub.requests[0]
    pl = sub.payload(0, keep=True)
    conv_w = sub.conv_w()
    sh = sub.shapes
    tn = r.P - r.m
    L = r.q_len[0] if r.q_len else 0
    rows = np.arange(tn + L)
    pos = np.concatenate([np.arange(r.m, r.P), np.arange(r.P, r.P + L)])
    samp = sorted(set(np.linspace(0, tn - 1, min(n_trunk_sample, tn)).astype(int).tolist())) if tn else []
    vis_all = sum(t + 1 for t in range(r.m, r.P))
    vis_samp = sum(int(pos[a]) + 1 for a in samp) or 1

    def timed(threads):
        limiter = threadpool_limits(threads) if threadpool_limits else None
        try:
            t0 = time.perf_counter()
            gdn_prompt(pl["gdn_x"][rows], pl["alpha"][rows], pl["eta"][rows], conv_w, sh.H, sh.dk, sh.dv,
                       pl.get("ckpt_window"), pl.get("ckpt_state"), sh.gdn_act)
            t1 = time.perf_counter()
            ck = (pl.get("kv_k"), pl.get("kv_v")) if r.m > 0 else (None, None)
            prompt_attention(pl["attn_q"][rows], pl["attn_k"][rows], pl["attn_v"][rows], pos, sh.theta,
                             cache_k=ck[0], cache_v=ck[1], rows=samp)
            t2 = time.perf_counter()
            prompt_attention(pl["attn_q"][rows], pl["attn_k"][rows], pl["attn_v"][rows], pos, sh.theta,
                             cache_k=ck[0], cache_v=ck[1], rows=list(range(tn, tn + L)))
            if L:
                option_probs(pl["hidden"][tn + L - 1], pl["w_opt"][:r.n_opt[0]])
            t3 = time.perf_counter()
        finally:
            if limiter is not None:
                limiter.unregister()
        t_trunk_attn = (t2 - t1) * vis_all / vis_samp
        return (tn + L) / ((t1 - t0) + t_trunk_attn + (t3 - t2)), (t1 - t0, t2 - t1, t_trunk_attn, t3 - t2)

    v1, (g, a, ta, q) = timed(1)
    n_cpu = os.cpu_count() or 1
    vn, _ = timed(n_cpu)
    return {"value": round(v1, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": (f"request 0 of the round ({tn} trunk rows) with its first question ({L} rows), memo order, "
                       f"fp64, one BLAS thread: GDN over all {tn + L} rows {g:.1f} s; attention at "
                       f"{len(samp)} evenly spaced trunk rows {a:.1f} s, scaled by visible keys to all "
                       f"{tn} trunk rows = {ta:.1f} s (extrapolated); question attention + readout "
                       f"{q:.1f} s; host {n_cpu} logical CPUs, {_host_cpu()}"),
            "host_cpus": n_cpu,
            "all_cores": {"value": round(vn, 3), "cores": n_cpu, "blas_threads": n_cpu}}


def measured_peaks(torch):
    """Device-to-device copy bandwidth, a large bf16 GEMM (the vendor library) and a loop of independent bf16
    matrix products (libflide's flide_measure_mfma_peak) in this job: practical ceilings beside the published
    peaks."""
    n = 1 << 30
    a = torch.empty(n // 2, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(10):
        b.copy_(a)
    ev[1].record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 10 / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9
    del a, b
    m = 8192
    x = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    y = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    z = x @ y
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(10):
        z = x @ y
    ev[1].record()
    torch.cuda.synchronize()
    gemm = 2 * m ** 3 * 10 / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e12
    del x, y, z
    from tree_forked_hybrid_amd import flide as F
    mfma = F.flide_measure_mfma_peak(4096, torch.cuda.current_stream())
    return {"d2d_copy_GB/s": round(copy_gbs, 1), "bf16_gemm_8192_TFLOP/s": round(gemm, 1),
            "bf16_mfma_loop_TFLOP/s": round(mfma, 1)}


def stack_main(args):
    """A multi-layer hybrid stack over the short-round workload's structure (64 requests, P~U[256,768], one
    question of 16..48 rows each): model width 1024, SwiGLU MLP of 2816, eight layers (three GDN layers of
    16 heads x 128, then full attention of 16 q / 4 kv heads x 256; again, ending with a sliding-window layer
    of W=1024), bf16, seeded random weights.  Prints one JSON line: whole-stack stream tokens/s (graph
    replays back to back, each after its metadata upload) and tokens/s per layer (HIP events around each
    layer of an eager run on the launch stream)."""
    import numpy as np
    import torch

    from tree_forked_hybrid_amd import flide as F
    from tree_forked_hybrid_amd.runner import StackRunner
    from workloads import StackShapes, make_round, make_stack

    shapes = StackShapes(Dm=1024, F=2816, layers=("gdn", "gdn", "gdn", "attn", "gdn", "gdn", "gdn", "swa"), H=16,
                         dk=128, dv=128, conv_k=4, Hq=16, Hkv=4, d=256, theta=1e6, window=1024)
    reqs = make_round(1, args.seed).requests
    stack = make_stack(shapes, "bf16", reqs, base=9000 + args.seed)
    T = sum((r.P - r.m) + sum(r.q_len) for r in reqs)
    n_q = sum(len(r.q_len) for r in reqs)
    n_opt = sum(sum(r.n_opt) for r in reqs)
    ctx = F.Context(0)
    sr = StackRunner(stack, T_cap=_round_up(T, 4096), R_cap=_round_up(len(reqs), 64), Q_cap=_round_up(n_q, 64),
                     opt_cap=n_opt)
    img = F.flide_plan_round(reqs, sr.caps)
    sr.fill(F.decode_image(img, sr.caps))
    st = torch.cuda.current_stream()
    sr.upload(ctx, img, st)
    # per-layer times: events after every layer of an eager run (the last entry: final norm + readout)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(shapes.layers) + 2)]
    per_layer = np.zeros(len(shapes.layers) + 1)
    reps = 3
    for _ in range(reps):
        sr.fill(F.decode_image(img, sr.caps))
        torch.cuda.synchronize()
        ev[0].record(st)
        sr.run(ctx, st, layer_hook=lambda i: ev[i + 1].record(st))
        ev[-1].record(st)
        torch.cuda.synchronize()
        per_layer += [ev[i].elapsed_time(ev[i + 1]) for i in range(len(ev) - 1)]
    per_layer *= 1e3 / reps  # us
    F.flide_check_device(ctx, sr.caps, sr.dev_meta)
    sr.capture(ctx)
    for _ in range(args.warmup):
        sr.replay(ctx, img)
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        sr.replay(ctx, img)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    F.flide_check_device(ctx, sr.caps, sr.dev_meta)
    ms = (t1 - t0) * 1e3 / args.steps
    # the row-wise layers' kernels at this workload's shapes (layer 0 weights, all stream rows), HIP events on
    # the launch stream; the linear layers are MFMA-bound: 2 T N K FLOPs per call
    L0 = sr.layers[0]
    fd, ALL, Dm, Fm = F.FLIDE_BF16, F.FLIDE_ROWS_ALL, shapes.Dm, shapes.F
    C = shapes.gdn_channels
    calls = {
        "linear_gate_up": (lambda: F.flide_linear(ctx, sr.caps, sr.dev_meta, ALL, fd, 2 * Fm, Dm, sr.h, Dm,
                                                  L0["gate_up"], None, sr.gu, 2 * Fm, st), 2.0 * T * 2 * Fm * Dm),
        "linear_down": (lambda: F.flide_linear(ctx, sr.caps, sr.dev_meta, ALL, fd, Dm, Fm, sr.mid, Fm, L0["down"],
                                               None, sr.hf, Dm, st), 2.0 * T * Dm * Fm),
        "linear_gdn_in": (lambda: F.flide_linear(ctx, sr.caps, sr.dev_meta, ALL, fd, C, Dm, sr.h, Dm, L0["w_x"],
                                                 None, sr.xg, C, st), 2.0 * T * C * Dm),
        "rmsnorm": (lambda: F.flide_rmsnorm(ctx, sr.caps, sr.dev_meta, ALL, fd, Dm, sr.x, L0["norm1"], 1e-6, sr.h,
                                            st), None),
        "swiglu": (lambda: F.flide_swiglu(ctx, sr.caps, sr.dev_meta, ALL, fd, Fm, sr.gu, sr.mid, st), None),
    }
    kern = {}
    for name, (fn, flops) in calls.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(args.kernel_reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.kernel_reps
        kern[name] = {"us": round(us, 2)}
        if flops:
            kern[name]["TFLOP/s"] = round(flops / (us * 1e-6) / 1e12, 1)
            kern[name]["mfma_frac"] = round(flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)
    dom = max((k for k in kern if k.startswith("linear")), key=lambda k: kern[k]["us"])
    roof = {"bound": "mfma", "achieved": kern[dom]["TFLOP/s"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": kern[dom]["mfma_frac"], "traffic": None, "kernel": dom, "avg_launch_us": kern[dom]["us"],
            "algorithmic_per_launch": round(calls[dom][1])}
    layers = [{"layer": i, "kind": k, "us": round(per_layer[i], 1), "tokens_per_s": round(T / (per_layer[i] * 1e-6), 1)}
              for i, k in enumerate(shapes.layers)]
    rec = {
        "metric": "hybrid stack tokens/s per layer (row-wise layers + ForkAttention token mixers)",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic (seeded random weights)",
        "config": {"workload": "8-layer hybrid stack (GDN x3, full attention, GDN x3, sliding window W=1024), width "
                               "1024, MLP 2816, over the short-round structure (64 requests, one question each)",
                   "stream_rows": T, "questions": n_q},
        "per_layer": layers,
        "final_norm_and_readout_us": round(per_layer[-1], 1),
        "kernels": kern,
        "roofline": roof,
        "cpu_baseline": stack_cpu_baseline(shapes, 9000 + args.seed) if args.cpu_sample > 0 else None,
    }
    print(json.dumps(rec), flush=True)
    ctx.close()


def stack_cpu_baseline(shapes, base: int):
    """The stack oracle (as it stands: fp64 NumPy, rows one at a time through every layer, one BLAS thread)
    on a bounded sample of the workload: one request of the same weights with a 96-row trunk and one
    16-row question, memo order; tokens/s = its rows / wall time."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # noqa: BLE001
        threadpool_limits = None
    from oracle import stack as ostack
    from workloads import Request, make_stack
    small = make_stack(shapes, "bf16", [Request(P=96, m=0, q_len=(16,), n_opt=(3,), out_slot=0)], base=base)
    small.weights()
    small.payload(0)
    limiter = threadpool_limits(1) if threadpool_limits else None
    try:
        t0 = time.perf_counter()
        ostack.run_stack_request(small, 0, "memo")
        t1 = time.perf_counter()
    finally:
        if limiter is not None:
            limiter.unregister()
    return {"value": round(112 / (t1 - t0), 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"one request of the stack's weights, 96 trunk rows + one 16-row question (112 rows through "
                      f"all {len(shapes.layers)} layers), memo order, fp64, one BLAS thread: {t1 - t0:.1f} s; "
                      f"host {os.cpu_count()} logical CPUs, {_host_cpu()}",
            "host_cpus": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample", type=int, default=48,
                    help="trunk rows of the oracle's attention sample (0: skip the CPU baseline)")
    ap.add_argument("--kernel-reps", type=int, default=5)
    ap.add_argument("--counters", action="store_true",
                    help="counter pass: one launch of every kernel per sub-round plus a 256 MiB device copy (for "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE and the copy-kernel scale factor); prints no JSON")
    ap.add_argument("--nondeterministic", action="store_true",
                    help="GDN chunk boundaries on the stream's 64-row grid (bits then depend on the round's "
                         "composition); the default is the composition-independent mode")
    ap.add_argument("--serial-subrounds", action="store_true",
                    help="replay every sub-round on the launch stream, one after another (the default lets "
                         "runner.FrontScheduler run trunk GDN calls beside other work)")
    ap.add_argument("--stack", action="store_true",
                    help="time the multi-layer hybrid stack instead of the ForkAttention round (its own JSON line)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the ForkAttention round runs on a single MI355X "
              "(request-sharded multi-GPU rounds are not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.stack:
        stack_main(args)
        return

    import torch

    from tree_forked_hybrid_amd import flide as F
    from tree_forked_hybrid_amd.runner import BucketTable, FrontScheduler, bucket_capacities, spec_for_round
    from workloads import CONFIGS, make_round

    spec_cfg = CONFIGS[args.config]
    rnd = make_round(args.config, args.seed)
    T = sum((r.P - r.m) + sum(r.q_len) for r in rnd.requests)
    first, eager = F.flide_split_round(rnd.requests, rnd.t_max)
    if any(eager):
        print("a request of this workload exceeds the largest capacity (eager path): not a benchmark round",
              file=sys.stderr)
        sys.exit(2)
    subs = [rnd.subset(list(range(first[i], first[i + 1]))) for i in range(len(eager))]
    R_cap = _round_up(max(len(s.requests) for s in subs), 8)
    Q_cap = _round_up(max(max(sum(len(r.q_len) for r in s.requests) for s in subs), 1), 64)
    opt_cap = max(sum(sum(r.n_opt) for r in s.requests) for s in subs)
    caps_table = bucket_capacities(rnd.t_max, R_cap, Q_cap)
    spec = spec_for_round(rnd, T_cap=rnd.t_max, R_cap=R_cap, Q_cap=Q_cap, opt_cap=opt_cap)
    spec.deterministic = not args.nondeterministic
    print(f"[bench] {spec_cfg.name}: {T} rows, {len(subs)} sub-round(s), table of {len(caps_table)} buckets "
          f"(R_cap {R_cap}, Q_cap {Q_cap})", flush=True)
    tables = []
    for k, sub in enumerate(subs):  # one buffer set per sub-round: replays of a round go back to back
        tab = BucketTable(spec, caps_table)
        bid, img = tab.plan(sub.requests)
        tab.bufs.fill(sub, F.decode_image(img, tab.caps_of(bid)))
        tables.append(tab)
        print(f"[bench] sub-round {k}: {len(sub.requests)} requests, bucket T_cap {tab.caps_of(bid).T_cap}",
              flush=True)
    sub_reqs = [s.requests for s in subs]
    # runner.FrontScheduler picks the schedule: trunk GDN calls beside the attention when they are small,
    # else the sub-rounds' fronts side by side and the backs in order (a single sub-round: in order).
    # --serial-subrounds replays every sub-round on the launch stream, one after another.
    co_schedule = not args.serial_subrounds
    sched = FrontScheduler(len(tables)) if co_schedule else None

    def step():
        if sched is not None:
            sched.run(tables, sub_reqs)
            return
        for tab, reqs in zip(tables, sub_reqs):
            tab.run(reqs)

    step()
    torch.cuda.synchronize()
    for tab in tables:
        tab.check()
    # A serving loop keeps the collector out of the round's critical path: the setup heap is frozen and
    # collection is paused while rounds are timed (a full collection costs tens of ms here).
    gc.collect()
    gc.freeze()
    gc.disable()
    # Warm-up rounds right before the timed region: after an idle stretch (setup, the collection above)
    # the device runs its first few milliseconds of rounds at a lower clock (measured: the first rounds of
    # a short-round loop took about 2 ms each instead of 0.8).
    for _ in range(args.warmup):
        step()
    # Throughput (the timed region): rounds back to back, as a serving loop runs them.  Each round is
    # planned on the host while the device still runs the previous one; its metadata uploads and graph
    # replays are ordered after that round on the stream, and each bucket's double-buffered pinned staging
    # keeps an image intact until its copy has executed.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # Round latency, host: plan, upload and replay every sub-round of one round, copy its option
    # probabilities into pinned host memory and wait for them.  Device: HIP events on the launch stream
    # around the round's replays (the side streams join it before the round ends).
    n_opt = [sum(sum(r.n_opt) for r in reqs) for reqs in sub_reqs]
    host_probs = [torch.empty(max(1, n), dtype=torch.float32, pin_memory=True) for n in n_opt]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    lat = []
    for i in range(args.steps):
        s0 = time.perf_counter()
        ev[i][0].record()
        step()
        ev[i][1].record()
        for tab, hp, n in zip(tables, host_probs, n_opt):
            hp[:n].copy_(tab.bufs.probs[:n], non_blocking=True)
        torch.cuda.synchronize()
        lat.append(time.perf_counter() - s0)
    dev_ms = sorted(a.elapsed_time(b) for a, b in ev)
    gc.enable()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    for tab in tables:
        tab.check()

    # Per-kernel durations: each entry point launched on its own on every sub-round's buffers and bucket,
    # timed with HIP events on the launch stream (torch's current stream); summed over the round.
    st = torch.cuda.current_stream()
    launches = []  # (name, sub-round, fn)
    for k, tab in enumerate(tables):
        bid = tab.last[0]
        caps, dm, b = tab.caps_of(bid), tab.dev_meta_of(bid), tab.bufs
        F.flide_meta_upload(tab.ctx, caps, tab.last[1], dm, st)
        ctx = tab.ctx
        for phase, name in ((0, "fork_gdn_trunks"), (1, "fork_gdn_questions")):
            launches.append((name, k, lambda ph=phase, ctx=ctx, caps=caps, dm=dm, b=b: F.flide_fork_gdn(
                ctx, caps, dm, b.gdn_params, ph, b.x, b.conv_w, b.alpha, b.eta, b.state_pool, b.conv_pool,
                b.spec.n_slots, b.o_gdn, stream=st)))
        for l in range(b.n_attn):
            sfx = "" if l == 0 else "_swa"
            launches.append(("attn_prepare" + sfx, k, lambda l=l, ctx=ctx, caps=caps, dm=dm, b=b: F.flide_attn_prepare(
                ctx, caps, dm, b.attn_params[l], b.k[l], b.v[l], b.ws[l], stream=st)))
            launches.append(("attn_core" + sfx, k, lambda l=l, ctx=ctx, caps=caps, dm=dm, b=b: F.flide_attn_core(
                ctx, caps, dm, b.attn_params[l], b.q[l], b.v[l], b.k_cache[l], b.v_cache[l], b.o_attn[l], b.ws[l],
                stream=st)))
        launches.append(("readout", k, lambda ctx=ctx, caps=caps, dm=dm, b=b: F.flide_readout(
            ctx, caps, dm, b.ro_params, b.h, b.w_opt, b.opt_off, b.opt_id, max(1, b.spec.opt_cap), b.probs,
            stream=st)))
    if args.counters:
        for _, _, fn in launches:
            fn()
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)  # reference copy of known size: scales FETCH_SIZE / WRITE_SIZE
        torch.cuda.synchronize()
        print(f"counter pass done: {len(launches)} launches, copy {COPY_BYTES} bytes", flush=True)
        for tab in tables:
            tab.close()
        return
    kernels, launches_of = {}, {}
    for name, k, fn in launches:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(args.kernel_reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        kernels[name] = kernels.get(name, 0.0) + ev[0].elapsed_time(ev[1]) * 1e3 / args.kernel_reps  # us
        launches_of[name] = launches_of.get(name, 0) + 1
    for tab in tables:
        tab.check()

    works = [algorithmic_work(s) for s in subs]
    tot = lambda f: sum(f(w) for w in works)  # noqa: E731
    rows = {
        "fork_gdn_trunks": ("hbm", tot(lambda w: w["gdn0"]), None),
        "fork_gdn_questions": ("hbm", tot(lambda w: w["gdn1"]), None),
        "attn_prepare": ("hbm", tot(lambda w: w["attn"]["attn"]["prep_bytes"]), None),
        "attn_core": ("mfma", tot(lambda w: w["attn"]["attn"]["bytes"]), tot(lambda w: w["attn"]["attn"]["flops"])),
        "readout": ("hbm", tot(lambda w: w["readout"]), None),
    }
    if "swa" in works[0]["attn"]:
        rows["attn_prepare_swa"] = ("hbm", tot(lambda w: w["attn"]["swa"]["prep_bytes"]), None)
        rows["attn_core_swa"] = ("mfma", tot(lambda w: w["attn"]["swa"]["bytes"]),
                                 tot(lambda w: w["attn"]["swa"]["flops"]))
    per_kernel = {}
    for name, us in kernels.items():
        bound, byts, flops = rows[name]
        ent = {"us_per_round": round(us, 2), "launches_per_round": launches_of[name],
               "GB/s": round(byts / (us * 1e-6) / 1e9, 1)}
        ent["hbm_frac"] = round(ent["GB/s"] / PEAK_HBM_GBS, 4)
        if flops:
            tf = flops / (us * 1e-6) / 1e12
            ent["TFLOP/s"] = round(tf, 1)
            ent["mfma_frac"] = round(tf / PEAK_BF16_TFLOPS, 4)
        per_kernel[name] = ent
    dom = max(kernels, key=kernels.get)
    bound, byts, flops = rows[dom]
    us = kernels[dom]
    if flops and rnd.dtype == "bf16":
        # the binding roof of a contraction is whichever of MFMA time and HBM time is larger
        bound = "mfma" if flops / (PEAK_BF16_TFLOPS * 1e12) >= byts / (PEAK_HBM_GBS * 1e9) else "hbm"
    traffic = measured_traffic(dom, args.config)
    nl = launches_of[dom]
    if bound == "mfma":
        ach = flops / (us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    else:
        ach = byts / (us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    roof.update({"traffic": None if traffic is None else round(traffic / nl), "kernel": dom,
                 "launches_per_round": nl, "avg_launch_us": round(us / nl, 2),
                 "algorithmic_per_launch": round((flops if bound == "mfma" else byts) / nl)})

    peaks = measured_peaks(torch)
    cpu = cpu_baseline(rnd, args.cpu_sample) if args.cpu_sample > 0 else None

    lat_ms = sorted(x * 1e3 for x in lat)
    value = T / (ms_per_step * 1e-3)
    n_req = [len(s.requests) for s in subs]
    sub_note = (f"whole round as {len(subs)} replays ({' + '.join(map(str, n_req))} requests) of the "
                f"{'/'.join(str(t.caps_of(t.last[0]).T_cap) for t in tables)}-row buckets") if len(subs) > 1 else \
        f"one replay of the {tables[0].caps_of(tables[0].last[0]).T_cap}-row bucket"
    rec = {
        "metric": "ForkAttention tokens/s per layer + round latency (ms); % MFMA / HBM roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if rnd.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{spec_cfg.name}: {spec_cfg.description}; {sub_note}",
                   "stream_rows": T, "requests": len(rnd.requests),
                   "questions": sum(len(r.q_len) for r in rnd.requests),
                   "bucket_table_T_caps": [c.T_cap for c in caps_table], "seed": args.seed,
                   "deterministic": spec.deterministic,
                   "schedule": sched.last_mode if sched is not None else "in order"},
        "round_latency_ms": {"p10": round(lat_ms[len(lat_ms) // 10], 4), "median": round(lat_ms[len(lat_ms) // 2], 4),
                             "p90": round(lat_ms[(9 * len(lat_ms)) // 10], 4),
                             "what": "host: plan, metadata upload, replays, probabilities copied to host"},
        "device_round_ms": {"p10": round(dev_ms[len(dev_ms) // 10], 4), "median": round(dev_ms[len(dev_ms) // 2], 4),
                            "p90": round(dev_ms[(9 * len(dev_ms)) // 10], 4),
                            "what": "HIP events on the launch stream around one round's replays"},
        "per_layer_tokens_per_s": {
            "gdn": round(T / ((kernels["fork_gdn_trunks"] + kernels["fork_gdn_questions"]) * 1e-6), 1),
            "attn": round(T / ((kernels["attn_prepare"] + kernels["attn_core"]) * 1e-6), 1),
        },
        "kernels": per_kernel,
        "roofline": roof,
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
    }
    if "attn_core_swa" in kernels:
        rec["per_layer_tokens_per_s"]["swa"] = round(T / ((kernels["attn_prepare_swa"] + kernels["attn_core_swa"])
                                                          * 1e-6), 1)
    print(json.dumps(rec), flush=True)
    for tab in tables:
        tab.close()


if __name__ == "__main__":
    main()
