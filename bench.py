"""ForkAttention round benchmark on one MI355X.

One timed step = one whole round of the hot path over a synthetic batch:
host planning of the flat stream, the metadata upload (pinned H2D copy) and a
graph replay that expands the metadata, runs the GDN layer (trunk call, then
question call), rotates keys, runs the tree-masked attention layer(s) and the
selective readout.  Inputs are resident in HBM before the timed region.

Default workload: short single-question rounds (R=64 requests, P~U[256,768],
one question of 16..48 tokens each, 2-5 options; GDN 16 heads x 128, attention
16 q / 4 kv heads x 256, hidden 2048, bf16 activations, fp32 GDN state).

Prints one JSON line.  ``value`` is stream tokens per second of whole rounds
(each round holds one GDN layer, one attention layer and the readout).
"""
from __future__ import annotations

import argparse
import gc
import json
import os
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
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters_short_rounds.md")


def source_digest(name: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name] + ["device_common.hpp", "flide_internal.hpp"]:
        with open(os.path.join(ROOT, "tree_forked_hybrid_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch of `name` from the committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE,
    scaled by the reference copy), or None when there is none or the kernel source changed since."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    with open(COUNTERS_FILE) as fh:
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
    """Algorithmic bytes / FLOPs per kernel of one round (what the method must move or compute)."""
    s = rnd.shapes
    b = 2 if rnd.dtype == "bf16" else 4
    T = sum((r.P - r.m) + sum(r.q_len) for r in rnd.requests)
    R = len(rnd.requests)
    nq = sum(len(r.q_len) for r in rnd.requests)
    # attention: visible pairs per q head; every row x at position t sees min(t + 1, W) keys
    def pairs(W):
        tot = 0
        for r in rnd.requests:
            ts = list(range(r.m, r.P)) + [r.P + u for L in r.q_len for u in range(L)]
            for t in ts:
                tot += min(t + 1, W) if W > 0 else t + 1
        return tot
    cache_rows = sum(r.m for r in rnd.requests)
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
    return {"T": T, "attn": attn, "gdn0": gdn0, "gdn1": gdn1, "readout": ro, "cache_rows": cache_rows}


def cpu_baseline(rnd, n_req: int):
    """Time the oracle (as it stands) on the first n_req requests of the round, single-threaded."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # noqa: BLE001
        threadpool_limits = None
    from oracle import round as oround
    sub = rnd.subset(list(range(n_req)))
    conv_w = sub.conv_w()
    rows = sum((r.P - r.m) + sum(r.q_len) for r in sub.requests)
    for j in range(n_req):
        sub.payload(j, keep=True)
    ctx = threadpool_limits(1) if threadpool_limits else None
    t0 = time.perf_counter()
    for j in range(n_req):
        oround.run_request(sub, j, conv_w, "memo")
    dt = time.perf_counter() - t0
    if ctx is not None:
        ctx.unregister() if hasattr(ctx, "unregister") else None
    return {"value": rows / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n_req} of {len(rnd.requests)} requests ({rows} stream rows), memo mode "
                      f"(trunk once, every question from a copy of the trunk state), fp64, all layers + readout; "
                      f"{dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-requests", type=int, default=6, help="requests of the oracle CPU sample (0: skip)")
    ap.add_argument("--subround", type=int, default=None,
                    help="for a workload over one capacity (question fan-out): which of its replays to time")
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--counters", action="store_true",
                    help="counter pass: one launch of every kernel plus a 256 MiB device copy (for rocprofv3 --pmc "
                         "FETCH_SIZE / WRITE_SIZE and the copy-kernel scale factor); prints no JSON")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the ForkAttention round runs on a single MI355X "
              "(request-sharded multi-GPU rounds are not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from tree_forked_hybrid_amd import flide as F
    from tree_forked_hybrid_amd.runner import RoundBuffers, spec_for_round
    from workloads import CONFIGS, make_round

    spec_cfg = CONFIGS[args.config]
    rnd = make_round(args.config, args.seed)
    T = sum((r.P - r.m) + sum(r.q_len) for r in rnd.requests)
    sub_note = None
    if T > rnd.t_max:
        # a round over the capacity runs as several replays: time one of them (--subround)
        first, eager = F.flide_split_round(rnd.requests, rnd.t_max)
        k = args.subround
        if args.subround is None or not 0 <= k < len(eager) or eager[k]:
            print(f"this workload runs as {len(eager)} replays of <= {rnd.t_max} rows; pick one with --subround "
                  f"0..{len(eager) - 1}", file=sys.stderr)
            sys.exit(2)
        rnd = rnd.subset(list(range(first[k], first[k + 1])))
        T = sum((r.P - r.m) + sum(r.q_len) for r in rnd.requests)
        sub_note = f"replay {k} of {len(eager)} (requests {first[k]}..{first[k + 1] - 1})"
    R = len(rnd.requests)
    nq = sum(len(r.q_len) for r in rnd.requests)
    spec = spec_for_round(rnd, T_cap=_round_up(T, 4096), R_cap=_round_up(R, 64), Q_cap=_round_up(max(nq, 1), 64))
    ctx = F.Context(0)
    bufs = RoundBuffers(spec)
    image = F.flide_plan_round(rnd.requests, bufs.caps)
    placement = F.decode_image(image, bufs.caps)
    bufs.fill(rnd, placement)
    bid = F.flide_graph_capture(ctx, bufs.round_bufs())
    caps = bufs.caps

    def step():
        img = F.flide_plan_round(rnd.requests, caps, image)
        F.flide_graph_replay(ctx, bid, img)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    F.flide_check_device(ctx, caps, bufs.dev_meta)
    # A serving loop keeps the collector out of the round's critical path: the setup heap is frozen
    # and collection is paused while rounds are timed (a full collection costs tens of ms here).
    gc.collect()
    gc.freeze()
    gc.disable()
    # Round latency: plan, upload and replay one round, then wait for it.
    lat = []
    for _ in range(args.steps):
        s0 = time.perf_counter()
        step()
        torch.cuda.synchronize()
        lat.append(time.perf_counter() - s0)
    # Throughput (the timed region): rounds back to back, as a serving loop runs them.  Each round is
    # planned on the host while the device still runs the previous one; its metadata upload and graph
    # replay are ordered after that round on the stream, and the replay's double-buffered pinned staging
    # keeps a round's image intact until its copy has executed.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    F.flide_check_device(ctx, caps, bufs.dev_meta)

    # per-kernel durations, measured with HIP events on the launch stream (the null stream)
    bufs.upload(ctx, image)
    kernels = {}

    def timed(name, fn):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(args.kernel_reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        kernels[name] = ev[0].elapsed_time(ev[1]) * 1e3 / args.kernel_reps  # us

    st = torch.cuda.current_stream()  # events and kernels on one stream
    gp = bufs.gdn_params
    launches = {}
    for phase, name in ((0, "fork_gdn_trunks"), (1, "fork_gdn_questions")):
        launches[name] = lambda ph=phase: F.flide_fork_gdn(ctx, caps, bufs.dev_meta, gp, ph, bufs.x, bufs.conv_w,
                                                           bufs.alpha, bufs.eta, bufs.state_pool, bufs.conv_pool,
                                                           spec.n_slots, bufs.o_gdn, stream=st)
    for l in range(bufs.n_attn):
        sfx = "" if l == 0 else "_swa"
        launches["attn_prepare" + sfx] = lambda l=l: F.flide_attn_prepare(
            ctx, caps, bufs.dev_meta, bufs.attn_params[l], bufs.k[l], bufs.v[l], bufs.ws[l], stream=st)
        launches["attn_core" + sfx] = lambda l=l: F.flide_attn_core(
            ctx, caps, bufs.dev_meta, bufs.attn_params[l], bufs.q[l], bufs.v[l], bufs.k_cache[l], bufs.v_cache[l],
            bufs.o_attn[l], bufs.ws[l], stream=st)
    launches["readout"] = lambda: F.flide_readout(ctx, caps, bufs.dev_meta, bufs.ro_params, bufs.h, bufs.w_opt,
                                                  bufs.opt_off, bufs.opt_id, max(1, spec.opt_cap), bufs.probs,
                                                  stream=st)
    if args.counters:
        for fn in launches.values():
            fn()
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)  # reference copy of known size: scales FETCH_SIZE / WRITE_SIZE
        torch.cuda.synchronize()
        print(f"counter pass done: {len(launches)} kernels, copy {COPY_BYTES} bytes", flush=True)
        ctx.close()
        return
    for name, fn in launches.items():
        timed(name, fn)
    torch.cuda.synchronize()

    work = algorithmic_work(rnd)
    rows = {
        "fork_gdn_trunks": ("hbm", work["gdn0"], None),
        "fork_gdn_questions": ("hbm", work["gdn1"], None),
        "attn_prepare": ("hbm", work["attn"]["attn"]["prep_bytes"], None),
        "attn_core": ("mfma", work["attn"]["attn"]["bytes"], work["attn"]["attn"]["flops"]),
        "readout": ("hbm", work["readout"], None),
    }
    if "swa" in work["attn"]:
        rows["attn_prepare_swa"] = ("hbm", work["attn"]["swa"]["prep_bytes"], None)
        rows["attn_core_swa"] = ("mfma", work["attn"]["swa"]["bytes"], work["attn"]["swa"]["flops"])
    per_kernel = {}
    for name, us in kernels.items():
        bound, byts, flops = rows[name]
        ent = {"us": round(us, 2), "GB/s": round(byts / (us * 1e-6) / 1e9, 1), "hbm_frac": None, "mfma_frac": None}
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
        t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
        t_hbm = byts / (PEAK_HBM_GBS * 1e9)
        bound = "mfma" if t_mfma >= t_hbm else "hbm"
    if bound == "mfma":
        ach = flops / (us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(dom), "kernel": dom}
    else:
        ach = byts / (us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": measured_traffic(dom), "kernel": dom}

    cpu = None
    if args.cpu_requests > 0:
        cpu = cpu_baseline(rnd, min(args.cpu_requests, R))

    lat_ms = sorted(x * 1e3 for x in lat)
    value = T / (ms_per_step * 1e-3)
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
        "config": {"workload": spec_cfg.name + ": " + spec_cfg.description + (f"; {sub_note}" if sub_note else ""),
                   "stream_rows": T, "requests": R, "questions": nq, "bucket_T_cap": caps.T_cap, "seed": args.seed},
        "round_latency_ms": {"p10": round(lat_ms[len(lat_ms) // 10], 4), "median": round(lat_ms[len(lat_ms) // 2], 4),
                             "p90": round(lat_ms[(9 * len(lat_ms)) // 10], 4)},
        "per_layer_tokens_per_s": {
            "gdn": round(T / ((kernels["fork_gdn_trunks"] + kernels["fork_gdn_questions"]) * 1e-6), 1),
            "attn": round(T / ((kernels["attn_prepare"] + kernels["attn_core"]) * 1e-6), 1),
        },
        "kernels": per_kernel,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    ctx.close()


if __name__ == "__main__":
    main()
