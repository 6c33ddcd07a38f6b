"""Device buffers of one round and the calls that run it — marshalling only.

``RoundBuffers`` allocates every tensor of a round at a capacity with torch
(device memory only), places request payloads at the stream rows a placement
names (the caller's job in a serving loop: writing the round's rows into the
capacity buffers before a replay), and hands raw pointers to the C ABI.  All
computation happens in libflide.so's kernels.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from . import flide as F

__all__ = ["RoundSpec", "RoundBuffers", "spec_for_round", "bucket_capacities", "BucketTable", "SplitExecutor"]


def _torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _flide_dtype(dtype: str) -> int:
    return F.FLIDE_BF16 if dtype == "bf16" else F.FLIDE_F32


@dataclass
class RoundSpec:
    """Static shape of the buffers (independent of a particular round)."""
    shapes: object          # workloads.LayerShapes
    dtype: str              # "bf16" or "f32"
    T_cap: int
    R_cap: int
    Q_cap: int
    n_slots: int
    opt_cap: int            # rows of w_opt / entries of probs
    cache_rows: int = 0     # K/V cache rows per slot (0: no cache)
    max_pos: int = 1 << 16
    # composition-independent bits (the default); False puts GDN chunk boundaries on the stream's 64-row grid
    deterministic: bool = True


class RoundBuffers:
    def __init__(self, spec: RoundSpec, device: str = "cuda"):
        self.spec = spec
        s = spec.shapes
        dt = _torch_dtype(spec.dtype)
        self.device = device
        self.caps = F.caps_of(spec.T_cap, spec.R_cap, spec.Q_cap)
        self.layout = F.flide_meta_layout_for(self.caps)
        T = spec.T_cap
        z = lambda *shape, dtype=dt: torch.zeros(*shape, dtype=dtype, device=device)  # noqa: E731
        self.dev_meta = z(self.layout.dev_words, dtype=torch.int32)
        self.n_attn = 2 if s.swa_window > 0 else 1
        self.q = [z(T, s.Hq, s.d) for _ in range(self.n_attn)]
        self.k = [z(T, s.Hkv, s.d) for _ in range(self.n_attn)]
        self.v = [z(T, s.Hkv, s.d) for _ in range(self.n_attn)]
        self.o_attn = [z(T, s.Hq, s.d) for _ in range(self.n_attn)]
        self.attn_params = []
        self.k_cache, self.v_cache, self.ws = [], [], []
        for layer in range(self.n_attn):
            p = F.flide_attn_params(s.Hq, s.Hkv, s.d, 0 if layer == 0 else s.swa_window, float(s.theta),
                                    int(spec.max_pos), int(spec.cache_rows),
                                    int(spec.n_slots if spec.cache_rows > 0 else 0), _flide_dtype(spec.dtype),
                                    int(spec.deterministic))
            self.attn_params.append(p)
            if spec.cache_rows > 0:
                # keys [slot, row, kv head, d]; values transposed [slot, kv head, d, row]
                self.k_cache.append(z(spec.n_slots, spec.cache_rows, s.Hkv, s.d))
                self.v_cache.append(z(spec.n_slots, s.Hkv, s.d, spec.cache_rows))
            else:
                self.k_cache.append(None)
                self.v_cache.append(None)
            nbytes = F.flide_attn_workspace_bytes(self.caps, p)
            self.ws.append(torch.zeros(nbytes, dtype=torch.uint8, device=device))
        C = s.channels
        act = 1 if getattr(s, "gdn_act", "none") == "silu" else 0
        self.gdn_params = F.flide_gdn_params(s.H, s.dk, s.dv, s.conv_k, act, 64, _flide_dtype(spec.dtype),
                                             int(spec.deterministic))
        self.x = z(T, C)
        self.conv_w = z(C, s.conv_k, dtype=torch.float32)
        self.alpha = z(T, s.H, dtype=torch.float32)
        self.eta = z(T, s.H, dtype=torch.float32)
        self.state_pool = z(spec.n_slots, s.H, s.dv, s.dk, dtype=torch.float32)
        self.conv_pool = z(spec.n_slots, max(1, s.conv_k - 1), C)
        self.o_gdn = z(T, s.H, s.dv)
        self.ro_params = F.flide_readout_params(s.hidden, _flide_dtype(spec.dtype))
        self.h = z(T, s.hidden)
        self.w_opt = z(max(1, spec.opt_cap), s.hidden)
        self.opt_off = z(spec.Q_cap + 1, dtype=torch.int32)
        self.opt_id = z(max(1, spec.opt_cap), dtype=torch.int32)
        self.probs = z(max(1, spec.opt_cap), dtype=torch.float32)
        self.n_opt_rows = 0
        self._struct = None

    # ------------------------------------------------------------------ placement
    def fill(self, rnd, placement: Dict[str, np.ndarray], conv_w: Optional[np.ndarray] = None,
             clear: bool = True) -> None:
        """Copy ``rnd``'s payloads to the stream rows named by ``placement``.

        placement: ``req_trunk_row0`` [R], ``req_q_seg0`` [R] and ``seg_row0`` [n_seg]
        (from the library's plan or an independent builder).
        """
        s, spec = rnd.shapes, self.spec
        dt = _torch_dtype(spec.dtype)
        T = int(sum((r.P - r.m) + sum(r.q_len) for r in rnd.requests))
        if T > spec.T_cap:
            raise ValueError("round does not fit the buffers")
        names = ["attn_q", "attn_k", "attn_v"] + (["swa_q", "swa_k", "swa_v"] if self.n_attn == 2 else []) + \
                ["gdn_x", "alpha", "eta", "hidden"]
        host = {}
        # generated once per request; requests have generators of their own, so they are drawn in parallel
        with ThreadPoolExecutor(max_workers=max(1, min(8, len(rnd.requests)))) as ex:
            pls = list(ex.map(rnd.payload, range(len(rnd.requests))))
        rows_idx = np.empty(T, np.int64)
        at = 0
        for j in range(len(rnd.requests)):
            segs = rnd.segment_rows(j)
            s0, n0 = segs[0]
            r0 = int(placement["req_trunk_row0"][j])
            rows_idx[at:at + n0] = np.arange(r0, r0 + n0)
            at += n0
            q0 = int(placement["req_q_seg0"][j])
            for i, (_, L) in enumerate(segs[1:]):
                rr = int(placement["seg_row0"][q0 + i])
                rows_idx[at:at + L] = np.arange(rr, rr + L)
                at += L
        # concatenated request payloads, in request-local order
        for name in names:
            parts = [pl[name] for pl in pls]
            cat = np.concatenate(parts, axis=0) if parts else np.zeros((0,))
            buf = np.zeros((T,) + cat.shape[1:], np.float32)
            buf[rows_idx] = cat
            host[name] = buf
        tgt = {"attn_q": self.q[0], "attn_k": self.k[0], "attn_v": self.v[0], "gdn_x": self.x,
               "alpha": self.alpha, "eta": self.eta, "hidden": self.h}
        if self.n_attn == 2:
            tgt.update({"swa_q": self.q[1], "swa_k": self.k[1], "swa_v": self.v[1]})
        for name, t in tgt.items():
            if clear:
                t.zero_()
            t[:T].copy_(torch.from_numpy(host[name]).to(t.dtype))
        cw = rnd.conv_w() if conv_w is None else conv_w
        self.conv_w.copy_(torch.from_numpy(np.ascontiguousarray(cw, np.float32)))
        # options: question order of the stream = request order, then question order
        blocks, off = [], [0]
        for j, r in enumerate(rnd.requests):
            w = pls[j]["w_opt"]
            blocks.append(w)
            for n in r.n_opt:
                off.append(off[-1] + int(n))
        n_opt = off[-1]
        if n_opt > spec.opt_cap:
            raise ValueError("too many options for the buffers")
        if n_opt:
            w_cat = np.concatenate(blocks, axis=0)
            perm = rnd.option_permutation(n_opt)          # option k lives at row perm[k]
            w_glob = np.zeros_like(w_cat)
            w_glob[perm] = w_cat
            self.w_opt[:n_opt].copy_(torch.from_numpy(w_glob).to(dt))
            self.opt_id[:n_opt].copy_(torch.from_numpy(perm.astype(np.int32)))
        self.opt_off[:len(off)].copy_(torch.from_numpy(np.asarray(off, np.int32)))
        self.n_opt_rows = n_opt
        self.n_opt = n_opt
        # checkpoints
        for j, r in enumerate(rnd.requests):
            if r.m > 0:
                pl = pls[j]
                self.state_pool[r.ckpt_slot].copy_(torch.from_numpy(pl["ckpt_state"]))
                self.conv_pool[r.ckpt_slot].copy_(torch.from_numpy(pl["ckpt_window"]).to(dt))
                for layer, pre in enumerate(["kv", "swa_kv"][:self.n_attn]):
                    if r.m > spec.cache_rows:
                        raise ValueError("checkpoint longer than the K/V cache")
                    self.k_cache[layer][r.ckpt_slot, :r.m].copy_(torch.from_numpy(pl[pre + "_k"]).to(dt))
                    vv = torch.from_numpy(np.ascontiguousarray(np.transpose(pl[pre + "_v"], (1, 2, 0))))
                    self.v_cache[layer][r.ckpt_slot, :, :, :r.m].copy_(vv.to(dt))
        self.rows_idx = rows_idx
        self._struct = None

    # ------------------------------------------------------------------ C structure
    def round_bufs(self) -> F.flide_round_bufs:
        if self._struct is None:
            self._struct = self.round_bufs_for(self.caps, self.dev_meta)
        return self._struct

    def round_bufs_for(self, caps: F.flide_caps, dev_meta) -> F.flide_round_bufs:
        """The round structure over these buffers for a capacity at most theirs (a smaller bucket uses the
        first rows of every tensor) with its own metadata buffer ``dev_meta``."""
        if caps.T_cap > self.caps.T_cap or caps.R_cap > self.caps.R_cap or caps.Q_cap > self.caps.Q_cap:
            raise ValueError("bucket capacity above the buffers' capacity")
        for l in range(self.n_attn):
            if F.flide_attn_workspace_bytes(caps, self.attn_params[l]) > self.ws[l].numel():
                raise ValueError("attention workspace too small for the bucket")
        b = F.flide_round_bufs()
        b.caps = caps
        b.dev_meta = dev_meta.data_ptr() if hasattr(dev_meta, "data_ptr") else int(dev_meta)
        b.n_attn = self.n_attn
        for l in range(self.n_attn):
            b.attn[l] = self.attn_params[l]
            b.q[l] = self.q[l].data_ptr()
            b.k[l] = self.k[l].data_ptr()
            b.v[l] = self.v[l].data_ptr()
            b.k_cache[l] = self.k_cache[l].data_ptr() if self.k_cache[l] is not None else None
            b.v_cache[l] = self.v_cache[l].data_ptr() if self.v_cache[l] is not None else None
            b.o_attn[l] = self.o_attn[l].data_ptr()
            b.attn_ws[l] = self.ws[l].data_ptr()
        b.gdn = self.gdn_params
        b.x = self.x.data_ptr()
        b.conv_w = self.conv_w.data_ptr()
        b.alpha = self.alpha.data_ptr()
        b.eta = self.eta.data_ptr()
        b.state_pool = self.state_pool.data_ptr()
        b.conv_pool = self.conv_pool.data_ptr()
        b.n_slots = self.spec.n_slots
        b.o_gdn = self.o_gdn.data_ptr()
        b.ro = self.ro_params
        b.h = self.h.data_ptr()
        b.w_opt = self.w_opt.data_ptr()
        b.opt_off = self.opt_off.data_ptr()
        b.opt_id = self.opt_id.data_ptr()
        b.n_opt_rows = max(1, self.spec.opt_cap)
        b.probs = self.probs.data_ptr()
        return b

    # ------------------------------------------------------------------ direct kernel calls
    def upload(self, ctx: F.Context, image: np.ndarray, stream=None) -> None:
        F.flide_meta_upload(ctx, self.caps, image, self.dev_meta, stream)

    def run_layers(self, ctx: F.Context, stream=None) -> None:
        """GDN call 0, GDN call 1, the attention layer(s) and the readout, one call each."""
        s = self.spec.shapes
        for phase in (F.FLIDE_GDN_TRUNKS, F.FLIDE_GDN_QUESTIONS):
            F.flide_fork_gdn(ctx, self.caps, self.dev_meta, self.gdn_params, phase, self.x, self.conv_w,
                             self.alpha, self.eta, self.state_pool, self.conv_pool, self.spec.n_slots, self.o_gdn,
                             stream)
        for l in range(self.n_attn):
            F.flide_fork_attn(ctx, self.caps, self.dev_meta, self.attn_params[l], self.q[l], self.k[l], self.v[l],
                              self.k_cache[l], self.v_cache[l], self.o_attn[l], self.ws[l], stream)
        F.flide_readout(ctx, self.caps, self.dev_meta, self.ro_params, self.h, self.w_opt, self.opt_off,
                        self.opt_id, max(1, self.spec.opt_cap), self.probs, stream)
        del s

    def save_checkpoint_kv(self, ctx: F.Context, stream=None) -> None:
        """After a round: the attention K/V of every request's interior checkpoint (save_m > 0) into its
        cache slot, per attention layer, from the workspace the round's prepare step left (the GDN half
        was written by the trunk call)."""
        for l in range(self.n_attn):
            F.flide_attn_save_kv(ctx, self.caps, self.dev_meta, self.attn_params[l], self.v[l], self.ws[l],
                                 self.k_cache[l], self.v_cache[l], stream)


def spec_for_round(rnd, T_cap: Optional[int] = None, R_cap: Optional[int] = None, Q_cap: Optional[int] = None,
                   opt_cap: Optional[int] = None) -> RoundSpec:
    """Buffer shape that holds ``rnd`` (optionally larger capacities)."""
    T = int(sum((r.P - r.m) + sum(r.q_len) for r in rnd.requests))
    R = len(rnd.requests)
    Q = int(sum(len(r.q_len) for r in rnd.requests))
    n_opt = int(sum(sum(r.n_opt) for r in rnd.requests))
    slots = [r.out_slot for r in rnd.requests] + [r.ckpt_slot for r in rnd.requests if r.m > 0]
    slots += [r.save_slot for r in rnd.requests if getattr(r, "save_m", 0) > 0]
    max_m = max([r.m for r in rnd.requests] + [getattr(r, "save_m", 0) for r in rnd.requests] + [0])
    max_m = (max_m + 7) // 8 * 8
    max_pos = max([r.P + (max(r.q_len) if r.q_len else 0) for r in rnd.requests] + [1])
    return RoundSpec(rnd.shapes, rnd.dtype, T_cap or max(T, 1), R_cap or max(R, 1), Q_cap if Q_cap is not None else Q,
                     max(slots + [0]) + 1, opt_cap or max(n_opt, 1), max_m, max_pos)


def bucket_capacities(t_max: int, R_cap: int, Q_cap: int, t_min: int = 2048) -> List[F.flide_caps]:
    """Capacity table: T_cap = t_min, 1.5 t_min, 2 t_min, 3 t_min, ... up to t_max (powers of two and
    1.5 times powers of two), each holding R_cap requests and Q_cap questions."""
    out, t = [], t_min
    while t < t_max:
        out.append(t)
        if t + t // 2 < t_max:
            out.append(t + t // 2)
        t *= 2
    out.append(t_max)
    return [F.caps_of(t, R_cap, Q_cap) for t in sorted(set(out))]


class BucketTable:
    """One set of round buffers at the largest capacity and a captured graph per capacity of ``caps``
    (flat-graph execution with capacity buckets: the Korean summary §어떻게 쓰나).  Every bucket's graph
    reads and writes the same tensors (a bucket uses their first rows) and has a metadata buffer of its
    own.  The table owns a context of its own, so ``flide_select_bucket`` chooses among this table's
    buckets; several tables let the sub-rounds of a split round be replayed back to back, each on its
    own buffers."""

    def __init__(self, spec: RoundSpec, caps: Sequence[F.flide_caps], device: int = 0):
        self.ctx = F.Context(device)
        big = max(caps, key=lambda c: c.T_cap)
        self.bufs = RoundBuffers(RoundSpec(**{**spec.__dict__, "T_cap": big.T_cap,
                                              "R_cap": max(c.R_cap for c in caps),
                                              "Q_cap": max(c.Q_cap for c in caps)}))
        # one workspace per layer, sized for the largest bucket
        for l in range(self.bufs.n_attn):
            need = max(F.flide_attn_workspace_bytes(c, self.bufs.attn_params[l]) for c in caps)
            if need > self.bufs.ws[l].numel():
                self.bufs.ws[l] = torch.zeros(need, dtype=torch.uint8, device=self.bufs.device)
        self.buckets: Dict[int, tuple] = {}   # bucket id -> (caps, dev_meta, host image)
        for c in sorted(caps, key=lambda c: c.T_cap):
            L = F.flide_meta_layout_for(c)
            dev_meta = torch.zeros(L.dev_words, dtype=torch.int32, device=self.bufs.device)
            bid = F.flide_graph_capture(self.ctx, self.bufs.round_bufs_for(c, dev_meta))
            self.buckets[bid] = (c, dev_meta, np.zeros(L.host_words, np.int32))
        self.last = None  # (bucket id, image) of the last round run

    def select(self, requests) -> int:
        T, _, nq = F.flide_plan_sizes(requests)
        return F.flide_select_bucket(self.ctx, T, len(requests), nq)

    def plan(self, requests, bid: Optional[int] = None):
        """(bucket id, metadata image) of a round: the smallest bucket that holds it, unless given."""
        if bid is None:
            bid = self.select(requests)
        caps, _, img = self.buckets[bid]
        return bid, F.flide_plan_round(requests, caps, img)

    def run(self, requests, stream=None, bid: Optional[int] = None) -> int:
        """Plan the round for its bucket, upload the metadata and replay the bucket's graph (the request list
        is marshalled for the C ABI once, for both the bucket choice and the plan)."""
        bid, img = self.plan(F.Requests(requests), bid)
        F.flide_graph_replay(self.ctx, bid, img, stream)
        self.last = (bid, img)
        return bid

    def run_front(self, requests, stream=None, bid: Optional[int] = None) -> int:
        """Plan the round, upload its metadata and replay the front of its bucket (metadata expansion and the
        trunk GDN call); run_back replays the rest."""
        bid, img = self.plan(F.Requests(requests), bid)
        F.flide_graph_replay_front(self.ctx, bid, img, stream)
        self.last = (bid, img)
        return bid

    def run_back(self, stream=None) -> None:
        F.flide_graph_replay_back(self.ctx, self.last[0], stream)

    def run_parts(self, parts: int, requests=None, stream=None, bid: Optional[int] = None) -> None:
        """Replay the parts of the bucket's round whose bits are set (0 metadata upload and expansion, 1 GDN
        call 1, 2 attention, 3 GDN call 2 and readout); with part 0 the round is planned from `requests`,
        else the last planned round's bucket is used."""
        if parts & 1:
            bid, img = self.plan(F.Requests(requests), bid)
            F.flide_graph_replay_parts(self.ctx, bid, img, parts, stream)
            self.last = (bid, img)
        else:
            F.flide_graph_replay_parts(self.ctx, self.last[0], None, parts, stream)

    def caps_of(self, bid: int) -> F.flide_caps:
        return self.buckets[bid][0]

    def dev_meta_of(self, bid: int):
        return self.buckets[bid][1]

    def check(self, bid: Optional[int] = None) -> None:
        bid = self.last[0] if bid is None else bid
        F.flide_check_device(self.ctx, self.caps_of(bid), self.dev_meta_of(bid))

    def close(self) -> None:
        if self.ctx.handle:
            torch.cuda.synchronize()
            for bid in list(self.buckets):
                F.flide_graph_release(self.ctx, bid)
            self.buckets.clear()
            self.ctx.close()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


class SplitExecutor:
    """A round over the largest capacity split at request boundaries (``flide_split_round``, the Korean
    summary §어떻게 쓰나): sub-round i runs in bucket table i mod n of ``tables``, so consecutive replays
    use different buffers and are enqueued back to back; a request longer than every capacity runs
    eagerly (``flide_round_eager``) in buffers of its own size."""

    def __init__(self, tables: Sequence[BucketTable]):
        self.tables = list(tables)
        self.t_max = max(c.T_cap for t in self.tables for c, _, _ in t.buckets.values())

    def split(self, requests):
        first, eager = F.flide_split_round(requests, self.t_max)
        return [(first[i], first[i + 1], eager[i]) for i in range(len(eager))]

    def table_of(self, k: int) -> BucketTable:
        return self.tables[k % len(self.tables)]


class FrontScheduler:
    """The sub-rounds of one round (a split round, or a single one), each in a bucket table of its own,
    replayed part by part (BucketTable.run_parts) on the launch stream and one side stream per sub-round.
    The trunk GDN call runs one workgroup per (trunk, head), each holding a whole CU for its chunk chain:

    * rounds whose trunk calls have few such pairs (at most a quarter of the CUs over all sub-rounds: the
      long-document round's 64) run each trunk call on a side stream beside the attention of its own
      sub-round, which does not read it (long document 2.78 -> 2.16 ms per round on MI355X); the question
      call and the readout follow on the launch stream after both;
    * otherwise every sub-round's front (metadata expansion, trunk call) runs on its side stream, all side
      by side, and the backs (attention, question call, readout) in order on the launch stream, each after
      its own front (fan-out 17.0-18.0 -> 14.7 ms; overlapping attention too gains nothing there, and the
      agent-resume round's attention loses 1% beside its 128 trunk workgroups);
    * a single sub-round without the overlap replays on the launch stream alone.

    The attention launches, which fill the GPU, stay in order (side by side they slow each other down).  The
    next round's work on a table follows this round's on the launch stream, which waits for every side
    stream before its question calls."""

    def __init__(self, n: int, overlap_attention: Optional[bool] = None):
        self.side = [torch.cuda.Stream() for _ in range(n)]
        self.start = torch.cuda.Event()
        self.expanded = [torch.cuda.Event() for _ in range(n)]
        self.done = [torch.cuda.Event() for _ in range(n)]
        self.overlap_attention = overlap_attention
        self.n_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
        self.last_mode = None

    def mode(self, tables: Sequence[BucketTable], sub_requests) -> str:
        if self.overlap_attention is None:
            pairs = sum(len(reqs) * tab.bufs.spec.shapes.H for tab, reqs in zip(tables, sub_requests))
            overlap = 4 * pairs <= self.n_cus
        else:
            overlap = self.overlap_attention
        if overlap:
            return "trunk calls beside attention"
        return "side by side" if len(tables) > 1 else "in order"

    def run(self, tables: Sequence[BucketTable], sub_requests, stream=None) -> None:
        assert len(tables) == len(sub_requests) <= len(self.side)
        assert len({id(t) for t in tables}) == len(tables), "each sub-round needs a table of its own"
        main = stream if stream is not None else torch.cuda.current_stream()
        self.last_mode = mode = self.mode(tables, sub_requests)
        if mode == "in order":
            for tab, reqs in zip(tables, sub_requests):
                tab.run(reqs, stream=main)
            return
        if mode == "side by side":
            self.start.record(main)
            for k, (tab, reqs) in enumerate(zip(tables, sub_requests)):
                self.side[k].wait_event(self.start)
                tab.run_front(reqs, stream=self.side[k])
                self.done[k].record(self.side[k])
            for k, tab in enumerate(tables):
                main.wait_event(self.done[k])
                tab.run_back(stream=main)
            return
        for k, (tab, reqs) in enumerate(zip(tables, sub_requests)):
            tab.run_parts(1, reqs, stream=main)  # upload and expansion
            self.expanded[k].record(main)
        for k, tab in enumerate(tables):
            self.side[k].wait_event(self.expanded[k])
            tab.run_parts(2, stream=self.side[k])  # trunk call
            self.done[k].record(self.side[k])
        for k, tab in enumerate(tables):
            tab.run_parts(4, stream=main)  # attention
            main.wait_event(self.done[k])
            tab.run_parts(8, stream=main)  # question call, readout


class StackRunner:
    """Device buffers and launch sequence of a multi-layer hybrid stack at one capacity — marshalling only.

    Per layer (pre-norm residual block): rmsnorm -> the token mixer (GDN: input projection, gate projection
    and gates, the two GDN calls, output projection with the residual add; attention: q, k, v projections,
    the tree-masked attention, output projection with the residual add) -> rmsnorm -> SwiGLU MLP with the
    residual add.  After the last token mixer the row-wise layers run on question-final rows only
    (selective readout), then the final norm and the readout.  Every step is a call of the C ABI; the
    whole sequence can be captured into one HIP graph (``capture``) and replayed after each round's
    metadata upload."""

    def __init__(self, stack, T_cap: int, R_cap: int, Q_cap: int, opt_cap: int, device: str = "cuda"):
        s = stack.shapes
        self.stack, self.s = stack, s
        self.dtype = stack.dtype
        fd = _flide_dtype(stack.dtype)
        self.fd = fd
        dt = _torch_dtype(stack.dtype)
        self.device = device
        self.caps = F.caps_of(T_cap, R_cap, Q_cap)
        self.layout = F.flide_meta_layout_for(self.caps)
        T = T_cap
        z = lambda *shape, dtype=dt: torch.zeros(*shape, dtype=dtype, device=device)  # noqa: E731
        self.dev_meta = z(self.layout.dev_words, dtype=torch.int32)
        self.n_slots = max(r.out_slot for r in stack.requests) + 1
        kinds = set(s.layers)
        self.x, self.h, self.hf = z(T, s.Dm), z(T, s.Dm), z(T, s.Dm)
        self.gu, self.mid = z(T, 2 * s.F), z(T, s.F)
        if "gdn" in kinds:
            C = s.gdn_channels
            self.xg, self.zab = z(T, C), z(T, 2 * s.H)
            self.alpha, self.eta = z(T, s.H, dtype=torch.float32), z(T, s.H, dtype=torch.float32)
            self.o_gdn = z(T, s.H, s.dv)
            self.gdn_params = F.flide_gdn_params(s.H, s.dk, s.dv, s.conv_k, 0, 64, fd, 1)
        if kinds & {"attn", "swa"}:
            self.q, self.k, self.v = z(T, s.Hq, s.d), z(T, s.Hkv, s.d), z(T, s.Hkv, s.d)
            self.o_attn = z(T, s.Hq, s.d)
        max_pos = max([r.P + (max(r.q_len) if r.q_len else 0) for r in stack.requests] + [1])
        w = stack.weights()
        self.layers = []
        for L in w["layers"]:
            D = {"kind": L["kind"]}
            for name, val in L.items():
                if name == "kind":
                    continue
                t = torch.from_numpy(np.ascontiguousarray(val))
                keep_f32 = name in ("norm1", "norm2", "b_ab", "conv_w")
                D[name] = t.to(device=device, dtype=torch.float32 if keep_f32 else dt)
            if L["kind"] == "gdn":
                D["state_pool"] = z(self.n_slots, s.H, s.dv, s.dk, dtype=torch.float32)
                D["conv_pool"] = z(self.n_slots, max(1, s.conv_k - 1), s.gdn_channels)
            else:
                p = F.flide_attn_params(s.Hq, s.Hkv, s.d, s.window if L["kind"] == "swa" else 0, float(s.theta),
                                        int(max_pos), 0, 0, fd, 1)
                D["params"] = p
                D["ws"] = torch.zeros(F.flide_attn_workspace_bytes(self.caps, p), dtype=torch.uint8, device=device)
            self.layers.append(D)
        self.norm_f = torch.from_numpy(w["norm_f"]).to(device)
        self.ro_params = F.flide_readout_params(s.Dm, fd)
        self.w_opt = z(max(1, opt_cap), s.Dm)
        self.opt_off = z(Q_cap + 1, dtype=torch.int32)
        self.opt_id = z(max(1, opt_cap), dtype=torch.int32)
        self.probs = z(max(1, opt_cap), dtype=torch.float32)
        self.opt_cap = max(1, opt_cap)
        self.graph = None

    def fill(self, placement) -> None:
        """Input embeddings at the stream rows named by ``placement`` and the round's option rows (CSR over
        questions in stream order)."""
        st = self.stack
        self.x.zero_()
        host = np.zeros((self.caps.T_cap, self.s.Dm), np.float32)
        w_rows, off = [], [0]
        for j, r in enumerate(st.requests):
            pl = st.payload(j)
            segs = st.segment_rows(j)
            r0 = int(placement["req_trunk_row0"][j])
            host[r0:r0 + segs[0][1]] = pl["x0"][:segs[0][1]]
            q0 = int(placement["req_q_seg0"][j])
            for i, (a, L) in enumerate(segs[1:]):
                rr = int(placement["seg_row0"][q0 + i])
                host[rr:rr + L] = pl["x0"][a:a + L]
            w_rows.append(pl["w_opt"])
            for n in r.n_opt:
                off.append(off[-1] + int(n))
        self.x.copy_(torch.from_numpy(host).to(self.x.dtype))
        n_opt = off[-1]
        if n_opt > self.opt_cap:
            raise ValueError("too many options for the buffers")
        if n_opt:
            self.w_opt[:n_opt].copy_(torch.from_numpy(np.concatenate(w_rows, axis=0)).to(self.w_opt.dtype))
            self.opt_id[:n_opt].copy_(torch.arange(n_opt, dtype=torch.int32))
        self.opt_off[:len(off)].copy_(torch.from_numpy(np.asarray(off, np.int32)))

    def upload(self, ctx: F.Context, image: np.ndarray, stream=None) -> None:
        F.flide_meta_upload(ctx, self.caps, image, self.dev_meta, stream)

    def run(self, ctx: F.Context, stream=None, selective: bool = True, layer_hook=None) -> None:
        """The whole stack over the uploaded round.  selective=False runs the last layer's MLP on every row
        (for comparing every row of the final layer).  layer_hook(i) is called after layer i is enqueued."""
        s, c, m, fd = self.s, self.caps, self.dev_meta, self.fd
        ALL, QF = F.FLIDE_ROWS_ALL, F.FLIDE_ROWS_QFINAL
        nl = len(self.layers)
        for li, L in enumerate(self.layers):
            F.flide_rmsnorm(ctx, c, m, ALL, fd, s.Dm, self.x, L["norm1"], 1e-6, self.h, stream)
            if L["kind"] == "gdn":
                C = s.gdn_channels
                F.flide_linear(ctx, c, m, ALL, fd, C, s.Dm, self.h, s.Dm, L["w_x"], None, self.xg, C, stream)
                F.flide_linear(ctx, c, m, ALL, fd, 2 * s.H, s.Dm, self.h, s.Dm, L["w_ab"], None, self.zab, 2 * s.H,
                               stream)
                F.flide_gdn_gates(ctx, c, m, fd, s.H, self.zab, L["b_ab"], self.alpha, self.eta, stream)
                for phase in (F.FLIDE_GDN_TRUNKS, F.FLIDE_GDN_QUESTIONS):
                    F.flide_fork_gdn(ctx, c, m, self.gdn_params, phase, self.xg, L["conv_w"], self.alpha, self.eta,
                                     L["state_pool"], L["conv_pool"], self.n_slots, self.o_gdn, stream)
                F.flide_linear(ctx, c, m, ALL, fd, s.Dm, s.H * s.dv, self.o_gdn, s.H * s.dv, L["w_o"], self.x, self.x,
                               s.Dm, stream)
            else:
                F.flide_linear(ctx, c, m, ALL, fd, s.Hq * s.d, s.Dm, self.h, s.Dm, L["w_q"], None, self.q,
                               s.Hq * s.d, stream)
                F.flide_linear(ctx, c, m, ALL, fd, s.Hkv * s.d, s.Dm, self.h, s.Dm, L["w_k"], None, self.k,
                               s.Hkv * s.d, stream)
                F.flide_linear(ctx, c, m, ALL, fd, s.Hkv * s.d, s.Dm, self.h, s.Dm, L["w_v"], None, self.v,
                               s.Hkv * s.d, stream)
                F.flide_fork_attn(ctx, c, m, L["params"], self.q, self.k, self.v, None, None, self.o_attn, L["ws"],
                                  stream)
                F.flide_linear(ctx, c, m, ALL, fd, s.Dm, s.Hq * s.d, self.o_attn, s.Hq * s.d, L["w_o"], self.x,
                               self.x, s.Dm, stream)
            rows = QF if (selective and li == nl - 1) else ALL
            F.flide_rmsnorm(ctx, c, m, rows, fd, s.Dm, self.x, L["norm2"], 1e-6, self.h, stream)
            F.flide_linear(ctx, c, m, rows, fd, 2 * s.F, s.Dm, self.h, s.Dm, L["gate_up"], None, self.gu, 2 * s.F,
                           stream)
            F.flide_swiglu(ctx, c, m, rows, fd, s.F, self.gu, self.mid, stream)
            F.flide_linear(ctx, c, m, rows, fd, s.Dm, s.F, self.mid, s.F, L["down"], self.x, self.x, s.Dm, stream)
            if layer_hook is not None:
                layer_hook(li)
        F.flide_rmsnorm(ctx, c, m, QF, fd, s.Dm, self.x, self.norm_f, 1e-6, self.hf, stream)
        F.flide_readout(ctx, c, m, self.ro_params, self.hf, self.w_opt, self.opt_off, self.opt_id, self.opt_cap,
                        self.probs, stream)

    def capture(self, ctx: F.Context) -> None:
        """Capture ``run`` into one HIP graph (after an eager run, which builds the rotary tables)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run(ctx, side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run(ctx, torch.cuda.current_stream())
        self.graph = g

    def replay(self, ctx: F.Context, image: np.ndarray) -> None:
        """Upload the round's metadata on the current stream, then replay the captured stack."""
        self.upload(ctx, image, torch.cuda.current_stream())
        self.graph.replay()
