"""Seeded synthetic decision rounds (structure + per-token payloads).

A round is a list of requests ``(P, m, q_len[], n_opt[], ckpt_slot, out_slot)``.
Payloads are generated *per request*, in request-local row order: the trunk
rows for positions ``m .. P-1`` first, then the rows of question 1, question 2,
and so on.  Every request has its own generators, so a request's values do not
depend on which other requests share its round (needed for the
round-composition invariance checks), and no tensor's values depend on the
size of another tensor.

Value distributions follow the workload descriptions of the benchmark
configurations: q, k, v and the GDN inputs ~ N(0, 1); alpha = sigmoid(N(2, 0.5));
eta = sigmoid(N(0, 1)); conv weights ~ N(0, 1/K); option vectors
~ N(0, 1/hidden); hidden rows ~ N(0, 1).  Activations of a "bf16" workload are
drawn in float32 and rounded to bfloat16 (round to nearest even); they are
stored here as float32 arrays that hold bf16-representable values.

No method arithmetic lives in this module.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

# Stable ids for the per-tensor generators (appending is fine, reordering is not).
TENSOR_IDS = {
    "structure": 0,
    "attn_q": 1, "attn_k": 2, "attn_v": 3,
    "swa_q": 4, "swa_k": 5, "swa_v": 6,
    "gdn_x": 7, "conv_w": 8, "alpha": 9, "eta": 10,
    "hidden": 11, "w_opt": 12,
    "ckpt_state": 13, "ckpt_window": 14,
    "kv_k": 15, "kv_v": 16, "swa_kv_k": 17, "swa_kv_v": 18,
    "opt_perm": 19,
    "stack_x": 20, "stack_w": 21, "stack_opt": 22,
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    # finite inputs cannot overflow 32 bits here
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def _rng(base: int, name: str, *extra: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(base), TENSOR_IDS[name], *map(int, extra)]))


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-z.astype(np.float64)))).astype(np.float32)


@dataclass(frozen=True)
class LayerShapes:
    # Gated DeltaNet layer
    H: int
    dk: int
    dv: int
    conv_k: int
    # full-attention layer (and the optional sliding-window layer)
    Hq: int
    Hkv: int
    d: int
    theta: float
    # readout
    hidden: int
    swa_window: int = 0  # 0: no sliding-window layer in the round
    gdn_act: str = "none"  # activation after the GDN conv: "none" or "silu"

    @property
    def channels(self) -> int:
        """Channels of the packed GDN input row: q (H*dk) | k (H*dk) | v (H*dv)."""
        return self.H * (2 * self.dk + self.dv)


@dataclass(frozen=True)
class Request:
    P: int                      # trunk length, including any checkpointed prefix
    m: int                      # resume position (0 = fresh); stream holds trunk positions m..P-1
    q_len: tuple                # question lengths (each >= 1)
    n_opt: tuple                # options per question
    ckpt_slot: int = -1         # pool slot holding the checkpoint at m (m > 0)
    out_slot: int = -1          # pool slot receiving S_P and the conv window
    save_m: int = 0             # 0, or the trunk position of a checkpoint to create in the same pass
    save_slot: int = -1         # pool slot receiving that checkpoint (save_m > 0)


def rows_of(r: Request) -> int:
    return (r.P - r.m) + int(sum(r.q_len))


@dataclass(frozen=True)
class ConfigSpec:
    name: str
    dtype: str                  # "f32" or "bf16" (activation storage type)
    shapes: LayerShapes
    sample: Callable[[np.random.Generator], List[Request]]
    t_max: int = 65536          # largest stream capacity a round is split to
    deterministic: bool = False
    description: str = ""


def _c0(_rng_):
    return [Request(P=48, m=0, q_len=(5, 7, 9), n_opt=(4, 4, 4), ckpt_slot=-1, out_slot=0)]


def _c1(rng):
    R = 64
    P = rng.integers(256, 768, size=R, endpoint=True)
    L = rng.integers(16, 48, size=R, endpoint=True)
    O = rng.integers(2, 5, size=R, endpoint=True)
    return [Request(int(P[j]), 0, (int(L[j]),), (int(O[j]),), -1, j) for j in range(R)]


def _c2(rng):
    R, n = 4, 48
    P = rng.integers(3000, 8000, size=R, endpoint=True)
    L = rng.integers(12, 40, size=(R, n), endpoint=True)
    return [Request(int(P[j]), 0, tuple(int(x) for x in L[j]), (4,) * n, -1, j) for j in range(R)]


def _c3(rng):
    R, n = 16, 64
    L = rng.integers(16, 64, size=(R, n), endpoint=True)
    O = rng.integers(2, 8, size=(R, n), endpoint=True)
    return [Request(8192, 0, tuple(int(x) for x in L[j]), tuple(int(x) for x in O[j]), -1, j)
            for j in range(R)]


def _c4(rng):
    R, n = 8, 8
    L = rng.integers(16, 48, size=(R, n), endpoint=True)
    O = rng.integers(2, 5, size=(R, n), endpoint=True)
    return [Request(32768, 30720, tuple(int(x) for x in L[j]), tuple(int(x) for x in O[j]), j, R + j)
            for j in range(R)]


_BIG = LayerShapes(H=16, dk=128, dv=128, conv_k=4, Hq=16, Hkv=4, d=256, theta=1e6, hidden=2048)

CONFIGS: Dict[int, ConfigSpec] = {
    0: ConfigSpec("tiny fork round, fp32", "f32",
                  LayerShapes(H=2, dk=32, dv=32, conv_k=4, Hq=2, Hkv=1, d=32, theta=1e4, hidden=32),
                  _c0, t_max=65536,
                  description="1 request, P=48, questions of 5/7/9 tokens, 4 options each"),
    1: ConfigSpec("short single-question rounds", "bf16", _BIG, _c1, t_max=65536,
                  description="R=64, P~U[256,768], n=1, |q|~U[16,48], 2-5 options"),
    2: ConfigSpec("long-document multi-question rounds", "bf16",
                  LayerShapes(**{**_BIG.__dict__, "swa_window": 1024}), _c2, t_max=65536,
                  description="R=4, P~U[3000,8000], n=48, |q|~U[12,40], 4 options, plus a W=1024 SWA layer"),
    3: ConfigSpec("question fan-out", "bf16", _BIG, _c3, t_max=65536,
                  description="R=16, P=8192, n=64, |q|~U[16,64], 2-8 options, split at T<=65536"),
    4: ConfigSpec("incremental agent-state fork, deterministic", "bf16", _BIG, _c4, t_max=65536,
                  deterministic=True,
                  description="R=8, P=32768 resumed at m=30720, n=8, |q|~U[16,48], 2-5 options"),
}


@dataclass
class Round:
    """A synthetic round: structure plus lazily generated per-request payloads."""
    base: int                   # seed base (1000*config + seed for the benchmark configs)
    dtype: str
    shapes: LayerShapes
    requests: List[Request]
    req_ids: List[int]          # payload identity of each request (index into the generating structure)
    t_max: int = 65536
    deterministic: bool = False
    _cache: Dict[int, dict] = field(default_factory=dict, repr=False)

    # -- global (per-layer) weights ------------------------------------------------
    def conv_w(self) -> np.ndarray:
        s = self.shapes
        w = _rng(self.base, "conv_w").standard_normal((s.channels, s.conv_k))
        return (w * (1.0 / np.sqrt(s.conv_k))).astype(np.float32)

    # -- per-request payloads -------------------------------------------------------
    def _act(self, x: np.ndarray) -> np.ndarray:
        return bf16_round(x) if self.dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)

    def payload(self, j: int, keep: bool = False) -> dict:
        """Payload arrays of request ``j`` in request-local row order (see module doc)."""
        if j in self._cache:
            return self._cache[j]
        r, rid, s = self.requests[j], self.req_ids[j], self.shapes
        n = rows_of(r)
        b = self.base
        out = {}

        def normal(name, shape, scale=1.0):
            z = _rng(b, name, rid).standard_normal(shape)
            if scale != 1.0:
                z *= scale
            return z.astype(np.float32)

        out["attn_q"] = self._act(normal("attn_q", (n, s.Hq, s.d)))
        out["attn_k"] = self._act(normal("attn_k", (n, s.Hkv, s.d)))
        out["attn_v"] = self._act(normal("attn_v", (n, s.Hkv, s.d)))
        if s.swa_window > 0:
            out["swa_q"] = self._act(normal("swa_q", (n, s.Hq, s.d)))
            out["swa_k"] = self._act(normal("swa_k", (n, s.Hkv, s.d)))
            out["swa_v"] = self._act(normal("swa_v", (n, s.Hkv, s.d)))
        out["gdn_x"] = self._act(normal("gdn_x", (n, s.channels)))
        out["alpha"] = _sigmoid(2.0 + 0.5 * normal("alpha", (n, s.H)))
        out["eta"] = _sigmoid(normal("eta", (n, s.H)))
        out["hidden"] = self._act(normal("hidden", (n, s.hidden)))
        n_opt = int(sum(r.n_opt))
        out["w_opt"] = self._act(normal("w_opt", (n_opt, s.hidden), 1.0 / np.sqrt(s.hidden)))
        if r.m > 0:
            out["ckpt_state"] = normal("ckpt_state", (s.H, s.dv, s.dk), 1.0 / np.sqrt(s.dk))
            out["ckpt_window"] = self._act(normal("ckpt_window", (s.conv_k - 1, s.channels)))
            out["kv_k"] = self._act(normal("kv_k", (r.m, s.Hkv, s.d)))
            out["kv_v"] = self._act(normal("kv_v", (r.m, s.Hkv, s.d)))
            if s.swa_window > 0:
                out["swa_kv_k"] = self._act(normal("swa_kv_k", (r.m, s.Hkv, s.d)))
                out["swa_kv_v"] = self._act(normal("swa_kv_v", (r.m, s.Hkv, s.d)))
        if keep:
            self._cache[j] = out
        return out

    def option_permutation(self, n_total: int) -> np.ndarray:
        """Seeded permutation used to scatter the concatenated option rows of a round."""
        return _rng(self.base, "opt_perm", n_total).permutation(n_total).astype(np.int64)

    def segment_rows(self, j: int) -> List[tuple]:
        """Request-local (start, length) of the trunk and of each question, in payload order."""
        r = self.requests[j]
        segs = [(0, r.P - r.m)]
        at = r.P - r.m
        for L in r.q_len:
            segs.append((at, L))
            at += L
        return segs

    def subset(self, idx: Sequence[int], slots: Optional[Sequence[tuple]] = None) -> "Round":
        """Round made of some of this round's requests (same payloads), optionally re-slotted."""
        reqs = []
        for k, j in enumerate(idx):
            r = self.requests[j]
            if slots is not None:
                r = Request(r.P, r.m, r.q_len, r.n_opt, slots[k][0], slots[k][1])
            reqs.append(r)
        return Round(self.base, self.dtype, self.shapes, reqs, [self.req_ids[j] for j in idx],
                     self.t_max, self.deterministic)


def make_round(config: int, seed: int = 0, requests: Optional[Sequence[int]] = None) -> Round:
    """Round of benchmark configuration ``config`` (0-4) with structure seed ``seed``."""
    spec = CONFIGS[config]
    base = 1000 * config + seed
    reqs = spec.sample(_rng(base, "structure"))
    rnd = Round(base, spec.dtype, spec.shapes, reqs, list(range(len(reqs))), spec.t_max, spec.deterministic)
    if requests is not None:
        rnd = rnd.subset(list(requests))
    return rnd


def custom_round(shapes: LayerShapes, dtype: str, requests: Sequence[Request], base: int = 7,
                 t_max: int = 65536) -> Round:
    """Round with a hand-written structure (edge cases, probes)."""
    reqs = list(requests)
    return Round(base, dtype, shapes, reqs, list(range(len(reqs))), t_max)


# ----------------------------------------------------------------------------------------------------
# Multi-layer synthetic hybrid stacks: seeded random weights of a pre-norm residual stack whose token
# mixers are Gated DeltaNet, full-attention and sliding-window attention layers, each followed by a
# SwiGLU MLP.  Only random draws (and bf16 rounding) live here; what the stack computes is written in
# the oracle and in the HIP kernels.
# ----------------------------------------------------------------------------------------------------

LAYER_KINDS = ("gdn", "attn", "swa")


@dataclass(frozen=True)
class StackShapes:
    Dm: int                     # model width (multiple of 32)
    F: int                      # MLP width (multiple of 32)
    layers: tuple               # kinds of the token mixers, in order
    H: int                      # GDN heads
    dk: int
    dv: int
    conv_k: int
    Hq: int                     # attention heads
    Hkv: int
    d: int
    theta: float
    window: int                 # window of the "swa" layers

    @property
    def gdn_channels(self) -> int:
        return self.H * (2 * self.dk + self.dv)


@dataclass
class Stack:
    """A seeded stack and a round of requests whose rows are its input embeddings."""
    base: int
    dtype: str                  # "f32" or "bf16": storage type of weights and activations
    shapes: StackShapes
    requests: List[Request]
    _w: Optional[dict] = field(default=None, repr=False)
    _cache: Dict[int, dict] = field(default_factory=dict, repr=False)

    def _act(self, x: np.ndarray) -> np.ndarray:
        return bf16_round(x) if self.dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)

    def weights(self) -> dict:
        """Per layer: ``norm1``, ``norm2`` gains [Dm] (fp32); mixer projections stored [out, in]; ``gate_up``
        [2F, Dm] (gate rows, then up rows) and ``down`` [Dm, F].  GDN layers: ``w_x`` [C, Dm] (q | k | v
        channels), ``w_ab`` [2H, Dm] and ``b_ab`` [2H] (alpha, then eta pre-activations), ``conv_w`` [C, K]
        (fp32), ``w_o`` [Dm, H dv].  Attention layers: ``w_q`` [Hq d, Dm], ``w_k``, ``w_v`` [Hkv d, Dm],
        ``w_o`` [Dm, Hq d].  Also ``norm_f`` [Dm], the final norm before the readout."""
        if self._w is not None:
            return self._w
        s = self.shapes
        out = {"layers": []}

        def normal(shape, scale, *ids):
            z = _rng(self.base, "stack_w", *ids).standard_normal(shape) * scale
            return z.astype(np.float32)

        for li, kind in enumerate(s.layers):
            if kind not in LAYER_KINDS:
                raise ValueError(kind)
            L = {"kind": kind}
            L["norm1"] = (1.0 + normal((s.Dm,), 0.1, li, 0)).astype(np.float32)
            L["norm2"] = (1.0 + normal((s.Dm,), 0.1, li, 1)).astype(np.float32)
            L["gate_up"] = self._act(normal((2 * s.F, s.Dm), 1.0 / np.sqrt(s.Dm), li, 2))
            L["down"] = self._act(normal((s.Dm, s.F), 0.5 / np.sqrt(s.F), li, 3))
            if kind == "gdn":
                C = s.gdn_channels
                L["w_x"] = self._act(normal((C, s.Dm), 1.0 / np.sqrt(s.Dm), li, 4))
                # alpha = sigmoid(N(2, 0.5)) and eta = sigmoid(N(0, 1)) for unit-variance normalised inputs
                w_a = normal((s.H, s.Dm), 0.5 / np.sqrt(s.Dm), li, 5)
                w_e = normal((s.H, s.Dm), 1.0 / np.sqrt(s.Dm), li, 6)
                L["w_ab"] = self._act(np.concatenate([w_a, w_e], axis=0))
                L["b_ab"] = np.concatenate([np.full(s.H, 2.0), np.zeros(s.H)]).astype(np.float32)
                L["conv_w"] = normal((C, s.conv_k), 1.0 / np.sqrt(s.conv_k), li, 7)
                L["w_o"] = self._act(normal((s.Dm, s.H * s.dv), 0.5 / np.sqrt(s.H * s.dv), li, 8))
            else:
                L["w_q"] = self._act(normal((s.Hq * s.d, s.Dm), 1.0 / np.sqrt(s.Dm), li, 9))
                L["w_k"] = self._act(normal((s.Hkv * s.d, s.Dm), 1.0 / np.sqrt(s.Dm), li, 10))
                L["w_v"] = self._act(normal((s.Hkv * s.d, s.Dm), 1.0 / np.sqrt(s.Dm), li, 11))
                L["w_o"] = self._act(normal((s.Dm, s.Hq * s.d), 0.5 / np.sqrt(s.Hq * s.d), li, 12))
            out["layers"].append(L)
        out["norm_f"] = (1.0 + normal((s.Dm,), 0.1, 999, 0)).astype(np.float32)
        self._w = out
        return out

    def payload(self, j: int) -> dict:
        """Request j: input embeddings ``x0`` [rows, Dm] (request-local order: trunk, then each question)
        and option vectors ``w_opt`` [sum n_opt, Dm]."""
        if j in self._cache:
            return self._cache[j]
        r = self.requests[j]
        n = rows_of(r)
        x0 = _rng(self.base, "stack_x", j).standard_normal((n, self.shapes.Dm)).astype(np.float32)
        w = _rng(self.base, "stack_opt", j).standard_normal((int(sum(r.n_opt)), self.shapes.Dm))
        out = {"x0": self._act(x0), "w_opt": self._act((w / np.sqrt(self.shapes.Dm)).astype(np.float32))}
        self._cache[j] = out
        return out

    def segment_rows(self, j: int) -> List[tuple]:
        r = self.requests[j]
        segs = [(0, r.P - r.m)]
        at = r.P - r.m
        for L in r.q_len:
            segs.append((at, L))
            at += L
        return segs


def make_stack(shapes: StackShapes, dtype: str, requests: Sequence[Request], base: int = 5) -> Stack:
    """A stack of the given shapes over a round with a hand-written structure."""
    for r in requests:
        if r.m != 0:
            raise ValueError("stack rounds start every trunk at position 0")
    return Stack(base, dtype, shapes, list(requests))
