"""ctypes binding of libkvsel.so (the C ABI declared in include/kvsel.h).

Argument marshalling only: every function here forwards device pointers,
sizes and the caller's current HIP stream to the C entry point of the same
name and raises KvselError when it returns a non-OK status.  PyTorch supplies
device memory and the stream; no step of the path runs in Python.
Loading fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvsel.so")

KVSEL_OK, KVSEL_EINVAL, KVSEL_EUNSUPPORTED, KVSEL_ENOSPC, KVSEL_EHIP = range(5)
KVSEL_FP32, KVSEL_BF16 = 0, 1
KVSEL_SEL_TOPB, KVSEL_SEL_CHUNK, KVSEL_SEL_POLICY = 0, 1, 2
KVSEL_HEAD_GLOBAL, KVSEL_HEAD_LOCAL, KVSEL_HEAD_SPECIAL = 0, 1, 2

_STATUS = {1: "EINVAL", 2: "EUNSUPPORTED", 3: "ENOSPC", 4: "EHIP"}


class KvselError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


class Rope(ctypes.Structure):
    _fields_ = [("cos_sin", ctypes.c_void_p), ("max_pos", ctypes.c_int64), ("half", ctypes.c_int32),
                ("pairs", ctypes.c_void_p), ("q_pos", ctypes.c_int64)]


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("rope", ctypes.POINTER(Rope))]


class SelectParams(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("budget", ctypes.c_void_p),
                ("n_chunks", ctypes.c_int64), ("chunk_end", ctypes.c_void_p),
                ("keep_tokens", ctypes.c_int64), ("head_kind", ctypes.c_void_p),
                ("local_window", ctypes.c_int64), ("special_pos", ctypes.c_void_p),
                ("n_special", ctypes.c_int64), ("local_chunks", ctypes.c_int64),
                ("top_chunks", ctypes.c_int64)]


_lib = None

_SIGS = {
    "kvsel_score_workspace": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int32]),
    "kvsel_score": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int64,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "kvsel_chunk_vote_workspace": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int32,
                                                     ctypes.c_int32]),
    "kvsel_chunk_vote": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "kvsel_select": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.POINTER(SelectParams),
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "kvsel_compact": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p]),
    "kvsel_decode_attn_noalloc": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                                 ctypes.c_void_p, ctypes.c_void_p]),
    "kvsel_decode_workspace": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int64]),
    "kvsel_decode_attn": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]),
    "kvsel_lmba_workspace": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int32]),
    "kvsel_lmba": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_void_p]),
    "kvsel_append": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_void_p]),
    "kvsel_zigzag_budgets": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.c_int32,
                                            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.POINTER(ctypes.c_int32)]),
    "kvsel_last_error": (ctypes.c_char_p, []),
    "kvsel_version": (ctypes.c_char_p, []),
}

EXPORTED = tuple(_SIGS)


def lib() -> ctypes.CDLL:
    """Load libkvsel.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_decode_attention_window_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(status: int, fn: str) -> None:
    if status != KVSEL_OK:
        raise KvselError(status, fn, lib().kvsel_last_error().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_rope(cos_sin, pairs, q_pos: int = 0) -> Rope:
    """kvsel_rope over a [max_pos][half][2] fp32 cos/sin table and a
    [hkv][head_dim/2] int32 kept-pair list (both device tensors, which the
    caller keeps alive)."""
    return Rope(_ptr(cos_sin), int(cos_sin.shape[0]), int(cos_sin.shape[1]), _ptr(pairs),
                int(q_pos))


def make_shape(batch, hq, hkv, head_dim, n, dtype, scale, rope: Rope | None = None) -> Shape:
    dt = {"fp32": KVSEL_FP32, "bf16": KVSEL_BF16}.get(dtype, dtype)
    sh = Shape(int(batch), int(hq), int(hkv), int(head_dim), int(n), int(dt), float(scale))
    if rope is not None:
        sh.rope = ctypes.pointer(rope)
        sh._rope = rope    # the descriptor lives as long as the shape
    return sh


def kvsel_score_workspace(shape: Shape, w: int) -> int:
    return lib().kvsel_score_workspace(ctypes.byref(shape), int(w))


def kvsel_score(shape: Shape, w: int, q_pos0: int, q_win, k, scores, ws, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().kvsel_score(ctypes.byref(shape), int(w), int(q_pos0), _ptr(q_win), _ptr(k),
                             _ptr(scores), _ptr(ws), nbytes, _stream(stream)), "kvsel_score")


def select_params(mode, budget=None, n_chunks=0, chunk_end=None, keep_tokens=0,
                  head_kind=None, local_window=0, special_pos=None, n_special=0,
                  local_chunks=0, top_chunks=0) -> SelectParams:
    return SelectParams(int(mode), _ptr(budget), int(n_chunks), _ptr(chunk_end), int(keep_tokens),
                        _ptr(head_kind), int(local_window), _ptr(special_pos), int(n_special),
                        int(local_chunks), int(top_chunks))


def kvsel_chunk_vote_workspace(shape: Shape, layers: int, top_k: int) -> int:
    return lib().kvsel_chunk_vote_workspace(ctypes.byref(shape), int(layers), int(top_k))


def kvsel_chunk_vote(shape: Shape, layers: int, top_k: int, local_chunks: int, scores, key, ws,
                     stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().kvsel_chunk_vote(ctypes.byref(shape), int(layers), int(top_k), int(local_chunks),
                                  _ptr(scores), _ptr(key), _ptr(ws), nbytes, _stream(stream)),
           "kvsel_chunk_vote")


def kvsel_select(shape: Shape, params: SelectParams, scores, seg_off, seg_len, idx, r_cap: int,
                 stream=None, _keep=None) -> None:
    _check(lib().kvsel_select(ctypes.byref(shape), ctypes.byref(params), _ptr(scores),
                              _ptr(seg_off), _ptr(seg_len), _ptr(idx), int(r_cap),
                              _stream(stream)), "kvsel_select")


def kvsel_compact(shape: Shape, k, v, seg_off, seg_len, idx, k_c, v_c, r_cap: int,
                  stream=None) -> None:
    _check(lib().kvsel_compact(ctypes.byref(shape), _ptr(k), _ptr(v), _ptr(seg_off),
                               _ptr(seg_len), _ptr(idx), _ptr(k_c), _ptr(v_c), int(r_cap),
                               _stream(stream)), "kvsel_compact")


def kvsel_decode_workspace(shape: Shape, r_cap: int) -> int:
    return lib().kvsel_decode_workspace(ctypes.byref(shape), int(r_cap))


def kvsel_decode_attn(shape: Shape, q, k_c, v_c, seg_off, seg_len, r_cap: int, out, ws,
                      stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().kvsel_decode_attn(ctypes.byref(shape), _ptr(q), _ptr(k_c), _ptr(v_c),
                                   _ptr(seg_off), _ptr(seg_len), int(r_cap), _ptr(out), _ptr(ws),
                                   nbytes, _stream(stream)), "kvsel_decode_attn")


def kvsel_decode_attn_noalloc(shape: Shape, q, k_c, v_c, seg_off, seg_len, r_cap: int, out,
                              stream=None) -> None:
    _check(lib().kvsel_decode_attn_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k_c), _ptr(v_c),
                                           _ptr(seg_off), _ptr(seg_len), int(r_cap), _ptr(out),
                                           _stream(stream)), "kvsel_decode_attn_noalloc")


def kvsel_lmba_workspace(shape: Shape, w: int) -> int:
    return int(lib().kvsel_lmba_workspace(ctypes.byref(shape), int(w)))


def kvsel_lmba(shape: Shape, w: int, q_pos0: int, q_win, k, lmba, ws, seg_off=None, seg_len=None,
               idx=None, r_cap: int = 0, kept_mass=None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().kvsel_lmba(ctypes.byref(shape), int(w), int(q_pos0), _ptr(q_win), _ptr(k),
                            _ptr(lmba), _ptr(seg_off), _ptr(seg_len), _ptr(idx), int(r_cap),
                            _ptr(kept_mass), _ptr(ws), nbytes, _stream(stream)), "kvsel_lmba")


def kvsel_append(shape: Shape, k_new, v_new, pos: int, seg_off, seg_cap, limit, seg_len, idx,
                 k_c, v_c, r_cap: int, stream=None) -> None:
    _check(lib().kvsel_append(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), int(pos),
                              _ptr(seg_off), _ptr(seg_cap), _ptr(limit), _ptr(seg_len), _ptr(idx),
                              _ptr(k_c), _ptr(v_c), int(r_cap), _stream(stream)), "kvsel_append")


def kvsel_zigzag_budgets(profile, n: int, avg_budget: int, floor_budget: int):
    """Host helper: returns a list of L integer budgets."""
    vals = [float(x) for x in profile]
    L = len(vals)
    arr = (ctypes.c_double * max(L, 1))(*vals)
    out = (ctypes.c_int32 * max(L, 1))()
    _check(lib().kvsel_zigzag_budgets(arr, L, int(n), int(avg_budget), int(floor_budget), out),
           "kvsel_zigzag_budgets")
    return [int(out[i]) for i in range(L)]


def kvsel_last_error() -> str:
    return lib().kvsel_last_error().decode()


def kvsel_version() -> str:
    return lib().kvsel_version().decode()
