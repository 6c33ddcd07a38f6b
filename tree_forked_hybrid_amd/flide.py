"""ctypes binding of libflide.so — argument marshalling only.

Every function here has the name of the C entry point it calls and does no
computation of its own: it converts Python/NumPy arguments to C structures,
passes device buffers as raw pointers (anything with ``data_ptr()``, e.g. a
torch tensor on ROCm, or a plain integer address) and turns a non-OK status
into ``FlideError``.  torch is never imported here; callers use it for device
memory and streams.
"""
from __future__ import annotations

import ctypes as C
import itertools
import os
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflide.so")

FLIDE_OK, FLIDE_E_INVALID_ARG, FLIDE_E_CAPACITY, FLIDE_E_UNSUPPORTED, FLIDE_E_HIP, FLIDE_E_DEVICE, \
    FLIDE_E_INTERNAL = range(7)
FLIDE_F32, FLIDE_BF16 = 0, 1
FLIDE_GDN_TRUNKS, FLIDE_GDN_QUESTIONS = 0, 1
FLIDE_ROWS_ALL, FLIDE_ROWS_QFINAL = 0, 1


class FlideError(RuntimeError):
    def __init__(self, status: int, where: str, message: str = ""):
        self.status = status
        text = f"{where}: {_status_string(status)}"
        if message:
            text += f" ({message})"
        super().__init__(text)


class flide_request(C.Structure):
    _fields_ = [("P", C.c_int32), ("m", C.c_int32), ("n_q", C.c_int32), ("q_len", C.POINTER(C.c_int32)),
                ("ckpt_slot", C.c_int32), ("out_slot", C.c_int32), ("save_m", C.c_int32),
                ("save_slot", C.c_int32)]


class flide_caps(C.Structure):
    _fields_ = [("T_cap", C.c_int32), ("R_cap", C.c_int32), ("Q_cap", C.c_int32)]


class flide_meta_layout(C.Structure):
    _fields_ = [(n, C.c_int64) for n in (
        "host_words", "dev_words", "hdr", "seg_row0", "seg_len", "seg_req", "seg_branch", "seg_pos0",
        "seg_state", "seg_vcol0", "req_trunk_row0", "req_P", "req_m", "req_ckpt", "req_out", "req_q_seg0", "req_nq",
        "req_save_m", "req_save_slot",
        "qfin_row", "tile_seg", "tile_row0", "tile_swa", "gdn_order", "tok_j", "tok_c", "tok_t", "tile_desc", "dev_error")] + \
        [("seg_cap", C.c_int32), ("tile_cap", C.c_int32), ("tile_rows", C.c_int32), ("reserved", C.c_int32)]


class flide_attn_params(C.Structure):
    _fields_ = [("Hq", C.c_int32), ("Hkv", C.c_int32), ("d", C.c_int32), ("window", C.c_int32),
                ("theta", C.c_double), ("max_pos", C.c_int32), ("cache_rows", C.c_int32),
                ("cache_slots", C.c_int32), ("dtype", C.c_int32), ("deterministic", C.c_int32)]


class flide_gdn_params(C.Structure):
    _fields_ = [("H", C.c_int32), ("dk", C.c_int32), ("dv", C.c_int32), ("conv_k", C.c_int32),
                ("act", C.c_int32), ("chunk", C.c_int32), ("dtype", C.c_int32), ("deterministic", C.c_int32)]


class flide_readout_params(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("dtype", C.c_int32)]


class flide_round_bufs(C.Structure):
    _fields_ = [
        ("caps", flide_caps), ("dev_meta", C.c_void_p), ("n_attn", C.c_int32),
        ("attn", flide_attn_params * 2),
        ("q", C.c_void_p * 2), ("k", C.c_void_p * 2), ("v", C.c_void_p * 2),
        ("k_cache", C.c_void_p * 2), ("v_cache", C.c_void_p * 2), ("o_attn", C.c_void_p * 2),
        ("attn_ws", C.c_void_p * 2),
        ("gdn", flide_gdn_params), ("x", C.c_void_p), ("conv_w", C.c_void_p), ("alpha", C.c_void_p),
        ("eta", C.c_void_p), ("state_pool", C.c_void_p), ("conv_pool", C.c_void_p), ("n_slots", C.c_int32),
        ("o_gdn", C.c_void_p),
        ("ro", flide_readout_params), ("h", C.c_void_p), ("w_opt", C.c_void_p), ("opt_off", C.c_void_p),
        ("opt_id", C.c_void_p), ("n_opt_rows", C.c_int32), ("probs", C.c_void_p),
    ]


# name -> (restype, argtypes) of every exported entry point (kept in the order of flide.h)
_VP = C.c_void_p
_SIGNATURES = {
    "flide_status_string": (C.c_char_p, [C.c_int32]),
    "flide_version": (C.c_char_p, []),
    "flide_meta_layout_for": (C.c_int, [C.POINTER(flide_caps), C.POINTER(flide_meta_layout)]),
    "flide_plan_sizes": (C.c_int, [C.POINTER(flide_request), C.c_int32, C.POINTER(C.c_int32),
                                   C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    "flide_plan_round": (C.c_int, [C.POINTER(flide_request), C.c_int32, C.POINTER(flide_caps),
                                   C.POINTER(C.c_int32), C.c_int64]),
    "flide_split_round": (C.c_int, [C.POINTER(flide_request), C.c_int32, C.c_int32, C.POINTER(C.c_int32),
                                    C.POINTER(C.c_int32), C.POINTER(C.c_uint8)]),
    "flide_store_create": (C.c_int, [C.POINTER(_VP), C.c_int32, C.c_int32]),
    "flide_store_destroy": (None, [_VP]),
    "flide_store_lookup": (C.c_int, [_VP, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_uint64),
                                     C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    "flide_store_reserve": (C.c_int, [_VP, C.c_int32, C.c_uint64, C.POINTER(C.c_int32)]),
    "flide_store_commit": (C.c_int, [_VP, C.c_int32]),
    "flide_store_release": (C.c_int, [_VP, C.c_int32]),
    "flide_store_stats": (C.c_int, [_VP, C.POINTER(C.c_int64)]),
    "flide_create": (C.c_int, [C.POINTER(_VP), C.c_int32]),
    "flide_destroy": (None, [_VP]),
    "flide_last_error": (C.c_char_p, [_VP]),
    "flide_last_hip_error": (C.c_int32, [_VP]),
    "flide_meta_upload": (C.c_int, [_VP, C.POINTER(flide_caps), C.POINTER(C.c_int32), _VP, _VP]),
    "flide_attn_workspace_bytes": (C.c_int, [C.POINTER(flide_caps), C.POINTER(flide_attn_params),
                                             C.POINTER(C.c_int64)]),
    "flide_fork_attn": (C.c_int, [_VP, C.POINTER(flide_caps), _VP, C.POINTER(flide_attn_params), _VP, _VP, _VP,
                                  _VP, _VP, _VP, _VP, _VP]),
    "flide_fork_attn_noalloc": (C.c_int, [_VP, C.POINTER(flide_caps), _VP, C.POINTER(flide_attn_params), _VP, _VP,
                                          _VP, _VP, _VP, _VP, _VP]),
    "flide_attn_prepare": (C.c_int, [_VP, C.POINTER(flide_caps), _VP, C.POINTER(flide_attn_params), _VP, _VP, _VP,
                                     _VP]),
    "flide_attn_save_kv": (C.c_int, [_VP, C.POINTER(flide_caps), _VP, C.POINTER(flide_attn_params), _VP, _VP, _VP,
                                     _VP, _VP]),
    "flide_attn_core": (C.c_int, [_VP, C.POINTER(flide_caps), _VP, C.POINTER(flide_attn_params), _VP, _VP, _VP, _VP,
                                  _VP, _VP, _VP]),
    "flide_fork_gdn": (C.c_int, [_VP, C.POINTER(flide_caps), _VP, C.POINTER(flide_gdn_params), C.c_int32, _VP,
                                 _VP, _VP, _VP, _VP, _VP, C.c_int32, _VP, _VP]),
    "flide_readout": (C.c_int, [_VP, C.POINTER(flide_caps), _VP, C.POINTER(flide_readout_params), _VP, _VP, _VP,
                                _VP, C.c_int32, _VP, _VP]),
    "flide_rmsnorm": (C.c_int, [_VP, C.POINTER(flide_caps), _VP, C.c_int32, C.c_int32, C.c_int32, _VP, _VP,
                                C.c_float, _VP, _VP]),
    "flide_linear": (C.c_int, [_VP, C.POINTER(flide_caps), _VP, C.c_int32, C.c_int32, C.c_int32, C.c_int32, _VP,
                               C.c_int64, _VP, _VP, _VP, C.c_int64, _VP]),
    "flide_swiglu": (C.c_int, [_VP, C.POINTER(flide_caps), _VP, C.c_int32, C.c_int32, C.c_int32, _VP, _VP, _VP]),
    "flide_gdn_gates": (C.c_int, [_VP, C.POINTER(flide_caps), _VP, C.c_int32, C.c_int32, _VP, _VP, _VP, _VP, _VP]),
    "flide_graph_capture": (C.c_int, [_VP, C.POINTER(flide_round_bufs), _VP, C.POINTER(C.c_int32)]),
    "flide_select_bucket": (C.c_int, [_VP, C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_int32)]),
    "flide_graph_replay": (C.c_int, [_VP, C.c_int32, C.POINTER(C.c_int32), _VP]),
    "flide_graph_replay_front": (C.c_int, [_VP, C.c_int32, C.POINTER(C.c_int32), _VP]),
    "flide_graph_replay_back": (C.c_int, [_VP, C.c_int32, _VP]),
    "flide_graph_replay_parts": (C.c_int, [_VP, C.c_int32, C.POINTER(C.c_int32), C.c_int32, _VP]),
    "flide_graph_release": (C.c_int, [_VP, C.c_int32]),
    "flide_round_eager": (C.c_int, [_VP, C.POINTER(flide_round_bufs), C.POINTER(C.c_int32), _VP]),
    "flide_check_device": (C.c_int, [_VP, C.POINTER(flide_caps), _VP, _VP]),
    "flide_measure_mfma_peak": (C.c_int, [C.c_int32, _VP, C.POINTER(C.c_double)]),
}

_lib: Optional[C.CDLL] = None


def load_library(path: str = LIB_PATH) -> C.CDLL:
    """Load libflide.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    # torch bundles its own HIP runtime; when torch is installed, load it first so
    # that libflide.so binds to the same runtime instance (one runtime per process).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m tree_forked_hybrid_amd.build` "
                          "(the HIP library is required; there is no fallback path)")
    lib = C.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _status_string(status: int) -> str:
    try:
        return load_library().flide_status_string(int(status)).decode()
    except Exception:  # noqa: BLE001 - only used while formatting an error
        return f"status {status}"


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    if isinstance(x, np.ndarray):
        return int(x.ctypes.data)
    raise TypeError(f"cannot take a device pointer of {type(x)!r}")


def _stream(s) -> Optional[int]:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)  # torch.cuda.Stream


def _check(status: int, where: str, ctx: Optional[int] = None) -> None:
    if status != FLIDE_OK:
        msg = ""
        if ctx:
            msg = load_library().flide_last_error(ctx).decode()
        raise FlideError(status, where, msg)


# ----------------------------------------------------------------------------- host structures

# numpy image of struct flide_request (int32 P, m, n_q; pointer q_len; int32 ckpt_slot, out_slot, save_m,
# save_slot)
_REQ_FIELDS = ("P", "m", "n_q", "q_len", "ckpt_slot", "out_slot", "save_m", "save_slot")
_REQ_DTYPE = np.dtype({"names": list(_REQ_FIELDS),
                       "formats": ["<u8" if n == "q_len" else "<i4" for n in _REQ_FIELDS],
                       "offsets": [getattr(flide_request, n).offset for n in _REQ_FIELDS],
                       "itemsize": C.sizeof(flide_request)})


class Requests:
    """A round's requests as a C array of flide_request (keeps the q_len storage alive).  Built as one
    numpy record array from one pass over the requests: per-field ctypes assignment costs more host time
    than the planner itself.  The binding's planner functions accept an instance in place of the request
    sequence, so a caller that plans one round several ways marshals it once."""

    def __init__(self, requests: Sequence):
        n = len(requests)
        self.n = n
        qls = [r.q_len for r in requests]
        ints = np.array([(r.P, r.m, len(q), r.ckpt_slot, r.out_slot, getattr(r, "save_m", 0),
                          getattr(r, "save_slot", -1)) for r, q in zip(requests, qls)],
                        dtype=np.int64).reshape(n, 7)
        nq = ints[:, 2]
        total = int(nq.sum())
        self._q = np.fromiter(itertools.chain.from_iterable(qls), np.int32, total) if total else np.zeros(1, np.int32)
        rec = np.zeros(max(1, n), _REQ_DTYPE)
        if n:
            rec["P"][:n], rec["m"][:n], rec["n_q"][:n] = ints[:, 0], ints[:, 1], nq
            rec["ckpt_slot"][:n], rec["out_slot"][:n] = ints[:, 3], ints[:, 4]
            rec["save_m"][:n], rec["save_slot"][:n] = ints[:, 5], ints[:, 6]
            off = np.cumsum(nq) - nq
            rec["q_len"][:n] = np.where(nq > 0, self._q.ctypes.data + 4 * off, 0).astype(np.uint64)
        self._rec = rec
        self.arr = rec.ctypes.data_as(C.POINTER(flide_request))

    def __len__(self) -> int:
        return self.n


def _marshal(requests) -> Requests:
    return requests if isinstance(requests, Requests) else Requests(requests)


def caps_of(T_cap: int, R_cap: int, Q_cap: int) -> flide_caps:
    return flide_caps(int(T_cap), int(R_cap), int(Q_cap))


def flide_version() -> str:
    return load_library().flide_version().decode()


def flide_meta_layout_for(caps: flide_caps) -> flide_meta_layout:
    out = flide_meta_layout()
    _check(load_library().flide_meta_layout_for(C.byref(caps), C.byref(out)), "flide_meta_layout_for")
    return out


def flide_plan_sizes(requests: Sequence) -> Tuple[int, int, int]:
    rq = _marshal(requests)
    T, ns, nq = C.c_int32(), C.c_int32(), C.c_int32()
    _check(load_library().flide_plan_sizes(rq.arr, rq.n, C.byref(T), C.byref(ns), C.byref(nq)), "flide_plan_sizes")
    return T.value, ns.value, nq.value


def flide_plan_round(requests: Sequence, caps: flide_caps, image: Optional[np.ndarray] = None) -> np.ndarray:
    """Host planner; returns (or fills) the int32 metadata image for ``caps``."""
    L = flide_meta_layout_for(caps)
    if image is None:
        image = np.zeros(L.host_words, np.int32)
    rq = _marshal(requests)
    _check(load_library().flide_plan_round(rq.arr, rq.n, C.byref(caps),
                                           image.ctypes.data_as(C.POINTER(C.c_int32)), int(image.size)),
           "flide_plan_round")
    return image


def flide_split_round(requests: Sequence, T_max: int) -> Tuple[List[int], List[bool]]:
    rq = _marshal(requests)
    first = (C.c_int32 * (rq.n + 1))()
    eager = (C.c_uint8 * max(1, rq.n))()
    n_sub = C.c_int32()
    _check(load_library().flide_split_round(rq.arr, rq.n, int(T_max), first, C.byref(n_sub), eager),
           "flide_split_round")
    return [first[i] for i in range(n_sub.value + 1)], [bool(eager[i]) for i in range(n_sub.value)]


def decode_image(image: np.ndarray, caps: flide_caps) -> dict:
    """Named views of a host metadata image (for tests and tooling)."""
    L = flide_meta_layout_for(caps)
    hdr = image[L.hdr:L.hdr + 16]
    T, R, n_seg, n_qst, n_tiles = (int(v) for v in hdr[:5])
    out = {"T": T, "R": R, "n_seg": n_seg, "n_qst": n_qst, "n_tiles": n_tiles, "max_pos": int(hdr[5]),
           "tile_group": int(hdr[6])}
    for name in ("seg_row0", "seg_len", "seg_req", "seg_branch", "seg_pos0", "seg_state", "seg_vcol0"):
        off = getattr(L, name)
        out[name] = image[off:off + n_seg].copy()
    for name in ("req_trunk_row0", "req_P", "req_m", "req_ckpt", "req_out", "req_q_seg0", "req_nq", "req_save_m",
                 "req_save_slot"):
        off = getattr(L, name)
        out[name] = image[off:off + R].copy()
    out["qfin_row"] = image[L.qfin_row:L.qfin_row + n_qst].copy()
    # attention work list: [n_tiles, 4] units (segment -1: no unit)
    out["tile_seg"] = image[L.tile_seg:L.tile_seg + 4 * n_tiles].reshape(n_tiles, 4).copy()
    out["tile_row0"] = image[L.tile_row0:L.tile_row0 + 4 * n_tiles].reshape(n_tiles, 4).copy()
    out["tile_swa"] = image[L.tile_swa:L.tile_swa + L.tile_cap].copy()  # windowed layer's order, -1: none
    out["gdn_order"] = image[L.gdn_order:L.gdn_order + n_seg].copy()
    return out


# ----------------------------------------------------------------------------- checkpoint store

class CheckpointStore:
    """A flide_ckpt_store over pool slots [first_slot, first_slot + n_slots) (host only)."""

    def __init__(self, first_slot: int, n_slots: int):
        h = C.c_void_p()
        _check(load_library().flide_store_create(C.byref(h), int(first_slot), int(n_slots)), "flide_store_create")
        self.handle = h.value

    def close(self) -> None:
        if self.handle:
            load_library().flide_store_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001
            pass

    def lookup(self, positions: Sequence[int], digests: Sequence[int]) -> Tuple[int, int]:
        """(m, slot) of the longest committed prefix among the candidates, (0, -1) if none."""
        n = len(positions)
        pos = np.ascontiguousarray(positions, np.int32)
        dig = np.ascontiguousarray(np.asarray(digests, dtype=np.uint64))
        m, slot = C.c_int32(), C.c_int32()
        _check(load_library().flide_store_lookup(self.handle, n, pos.ctypes.data_as(C.POINTER(C.c_int32)),
                                                 dig.ctypes.data_as(C.POINTER(C.c_uint64)), C.byref(m),
                                                 C.byref(slot)), "flide_store_lookup")
        return m.value, slot.value

    def reserve(self, m: int, digest: int) -> int:
        slot = C.c_int32()
        _check(load_library().flide_store_reserve(self.handle, int(m), C.c_uint64(int(digest)), C.byref(slot)),
               "flide_store_reserve")
        return slot.value

    def commit(self, slot: int) -> None:
        _check(load_library().flide_store_commit(self.handle, int(slot)), "flide_store_commit")

    def release(self, slot: int) -> None:
        _check(load_library().flide_store_release(self.handle, int(slot)), "flide_store_release")

    def stats(self) -> dict:
        out = (C.c_int64 * 7)()
        _check(load_library().flide_store_stats(self.handle, out), "flide_store_stats")
        keys = ("slots", "used", "committed", "held", "hits", "misses", "evictions")
        return {k: int(out[i]) for i, k in enumerate(keys)}


# ----------------------------------------------------------------------------- context + kernels

class Context:
    """Owns a flide_ctx on one HIP device."""

    def __init__(self, device: int = 0):
        lib = load_library()
        h = C.c_void_p()
        _check(lib.flide_create(C.byref(h), int(device)), "flide_create")
        self.handle = h.value

    def close(self) -> None:
        if self.handle:
            load_library().flide_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001
            pass

    def last_error(self) -> str:
        return load_library().flide_last_error(self.handle).decode()


def flide_meta_upload(ctx: Context, caps: flide_caps, image: np.ndarray, dev_meta, stream=None) -> None:
    image = np.ascontiguousarray(image, dtype=np.int32)
    _check(load_library().flide_meta_upload(ctx.handle, C.byref(caps), image.ctypes.data_as(C.POINTER(C.c_int32)),
                                            _ptr(dev_meta), _stream(stream)), "flide_meta_upload", ctx.handle)


def flide_attn_workspace_bytes(caps: flide_caps, p: flide_attn_params) -> int:
    b = C.c_int64()
    _check(load_library().flide_attn_workspace_bytes(C.byref(caps), C.byref(p), C.byref(b)),
           "flide_attn_workspace_bytes")
    return b.value


def flide_fork_attn(ctx: Context, caps: flide_caps, dev_meta, p: flide_attn_params, q, k, v, k_cache, v_cache, o,
                    workspace, stream=None) -> None:
    _check(load_library().flide_fork_attn(ctx.handle, C.byref(caps), _ptr(dev_meta), C.byref(p), _ptr(q), _ptr(k),
                                          _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(workspace),
                                          _stream(stream)), "flide_fork_attn", ctx.handle)


def flide_fork_attn_noalloc(ctx: Context, caps: flide_caps, dev_meta, p: flide_attn_params, q, k, v, k_cache,
                            v_cache, o, stream=None) -> None:
    _check(load_library().flide_fork_attn_noalloc(ctx.handle, C.byref(caps), _ptr(dev_meta), C.byref(p), _ptr(q),
                                                  _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(o),
                                                  _stream(stream)), "flide_fork_attn_noalloc", ctx.handle)


def flide_attn_prepare(ctx: Context, caps: flide_caps, dev_meta, p: flide_attn_params, k, v, workspace,
                       stream=None) -> None:
    _check(load_library().flide_attn_prepare(ctx.handle, C.byref(caps), _ptr(dev_meta), C.byref(p), _ptr(k), _ptr(v),
                                             _ptr(workspace), _stream(stream)), "flide_attn_prepare", ctx.handle)


def flide_attn_save_kv(ctx: Context, caps: flide_caps, dev_meta, p: flide_attn_params, v, workspace, k_cache,
                       v_cache, stream=None) -> None:
    _check(load_library().flide_attn_save_kv(ctx.handle, C.byref(caps), _ptr(dev_meta), C.byref(p), _ptr(v),
                                             _ptr(workspace), _ptr(k_cache), _ptr(v_cache), _stream(stream)),
           "flide_attn_save_kv", ctx.handle)


def flide_attn_core(ctx: Context, caps: flide_caps, dev_meta, p: flide_attn_params, q, v, k_cache, v_cache, o,
                    workspace, stream=None) -> None:
    _check(load_library().flide_attn_core(ctx.handle, C.byref(caps), _ptr(dev_meta), C.byref(p), _ptr(q), _ptr(v),
                                          _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(workspace), _stream(stream)),
           "flide_attn_core", ctx.handle)


def flide_fork_gdn(ctx: Context, caps: flide_caps, dev_meta, p: flide_gdn_params, phase: int, x, conv_w, alpha,
                   eta, state_pool, conv_pool, n_slots: int, o, stream=None) -> None:
    _check(load_library().flide_fork_gdn(ctx.handle, C.byref(caps), _ptr(dev_meta), C.byref(p), int(phase), _ptr(x),
                                         _ptr(conv_w), _ptr(alpha), _ptr(eta), _ptr(state_pool), _ptr(conv_pool),
                                         int(n_slots), _ptr(o), _stream(stream)), "flide_fork_gdn", ctx.handle)


def flide_readout(ctx: Context, caps: flide_caps, dev_meta, p: flide_readout_params, h, w_opt, opt_off, opt_id,
                  n_opt_rows: int, probs, stream=None) -> None:
    _check(load_library().flide_readout(ctx.handle, C.byref(caps), _ptr(dev_meta), C.byref(p), _ptr(h), _ptr(w_opt),
                                        _ptr(opt_off), _ptr(opt_id), int(n_opt_rows), _ptr(probs), _stream(stream)),
           "flide_readout", ctx.handle)


def flide_rmsnorm(ctx: Context, caps: flide_caps, dev_meta, rows: int, dtype: int, D: int, x, g, eps: float, y,
                  stream=None) -> None:
    _check(load_library().flide_rmsnorm(ctx.handle, C.byref(caps), _ptr(dev_meta), int(rows), int(dtype), int(D),
                                        _ptr(x), _ptr(g), float(eps), _ptr(y), _stream(stream)), "flide_rmsnorm",
           ctx.handle)


def flide_linear(ctx: Context, caps: flide_caps, dev_meta, rows: int, dtype: int, N: int, K: int, a, lda: int, w,
                 resid, c, ldc: int, stream=None) -> None:
    _check(load_library().flide_linear(ctx.handle, C.byref(caps), _ptr(dev_meta), int(rows), int(dtype), int(N),
                                       int(K), _ptr(a), int(lda), _ptr(w), _ptr(resid), _ptr(c), int(ldc),
                                       _stream(stream)), "flide_linear", ctx.handle)


def flide_swiglu(ctx: Context, caps: flide_caps, dev_meta, rows: int, dtype: int, F: int, gu, out,
                 stream=None) -> None:
    _check(load_library().flide_swiglu(ctx.handle, C.byref(caps), _ptr(dev_meta), int(rows), int(dtype), int(F),
                                       _ptr(gu), _ptr(out), _stream(stream)), "flide_swiglu", ctx.handle)


def flide_gdn_gates(ctx: Context, caps: flide_caps, dev_meta, dtype: int, H: int, z, bias, alpha, eta,
                    stream=None) -> None:
    _check(load_library().flide_gdn_gates(ctx.handle, C.byref(caps), _ptr(dev_meta), int(dtype), int(H), _ptr(z),
                                          _ptr(bias), _ptr(alpha), _ptr(eta), _stream(stream)), "flide_gdn_gates",
           ctx.handle)


def flide_graph_capture(ctx: Context, bufs: flide_round_bufs, stream=None) -> int:
    bid = C.c_int32()
    _check(load_library().flide_graph_capture(ctx.handle, C.byref(bufs), _stream(stream), C.byref(bid)),
           "flide_graph_capture", ctx.handle)
    return bid.value


def flide_select_bucket(ctx: Context, T: int, R: int, n_q: int) -> int:
    bid = C.c_int32()
    _check(load_library().flide_select_bucket(ctx.handle, int(T), int(R), int(n_q), C.byref(bid)),
           "flide_select_bucket", ctx.handle)
    return bid.value


def flide_graph_replay(ctx: Context, bucket_id: int, image: np.ndarray, stream=None) -> None:
    image = np.ascontiguousarray(image, dtype=np.int32)
    _check(load_library().flide_graph_replay(ctx.handle, int(bucket_id), image.ctypes.data_as(C.POINTER(C.c_int32)),
                                             _stream(stream)), "flide_graph_replay", ctx.handle)


def flide_graph_replay_front(ctx: Context, bucket_id: int, image: np.ndarray, stream=None) -> None:
    image = np.ascontiguousarray(image, dtype=np.int32)
    _check(load_library().flide_graph_replay_front(ctx.handle, int(bucket_id),
                                                   image.ctypes.data_as(C.POINTER(C.c_int32)), _stream(stream)),
           "flide_graph_replay_front", ctx.handle)


def flide_graph_replay_back(ctx: Context, bucket_id: int, stream=None) -> None:
    _check(load_library().flide_graph_replay_back(ctx.handle, int(bucket_id), _stream(stream)),
           "flide_graph_replay_back", ctx.handle)


def flide_graph_replay_parts(ctx: Context, bucket_id: int, image: Optional[np.ndarray], parts: int,
                             stream=None) -> None:
    ptr = None
    if image is not None:
        image = np.ascontiguousarray(image, dtype=np.int32)
        ptr = image.ctypes.data_as(C.POINTER(C.c_int32))
    _check(load_library().flide_graph_replay_parts(ctx.handle, int(bucket_id), ptr, int(parts), _stream(stream)),
           "flide_graph_replay_parts", ctx.handle)


def flide_graph_release(ctx: Context, bucket_id: int) -> None:
    _check(load_library().flide_graph_release(ctx.handle, int(bucket_id)), "flide_graph_release", ctx.handle)


def flide_last_hip_error(ctx: Optional[Context]) -> int:
    return int(load_library().flide_last_hip_error(ctx.handle if ctx is not None else None))


def flide_round_eager(ctx: Context, bufs: flide_round_bufs, image: np.ndarray, stream=None) -> None:
    image = np.ascontiguousarray(image, dtype=np.int32)
    _check(load_library().flide_round_eager(ctx.handle, C.byref(bufs), image.ctypes.data_as(C.POINTER(C.c_int32)),
                                            _stream(stream)), "flide_round_eager", ctx.handle)


def flide_check_device(ctx: Context, caps: flide_caps, dev_meta, stream=None) -> None:
    _check(load_library().flide_check_device(ctx.handle, C.byref(caps), _ptr(dev_meta), _stream(stream)),
           "flide_check_device", ctx.handle)


def flide_measure_mfma_peak(iters: int = 4096, stream=None) -> float:
    """TFLOP/s of a loop of independent bf16 matrix products (a measured ceiling; synchronises `stream`)."""
    out = C.c_double(0.0)
    _check(load_library().flide_measure_mfma_peak(int(iters), _stream(stream), C.byref(out)), "flide_measure_mfma_peak")
    return out.value


def exported_names() -> Iterable[str]:
    return list(_SIGNATURES)
