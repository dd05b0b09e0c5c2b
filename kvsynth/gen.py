"""Seeded generators for the five workloads.

Every random draw comes from numpy's PCG64 seeded by
``SeedSequence([20261203, config id, layer, batch, kv head, tensor id])`` so
that any single (layer, batch, KV head) segment can be regenerated on its own,
which is what the full-size parity tests do for their sampled segments.

Value laws (per layer and KV head, u = g / |g| with g ~ N(0, I)):
  keys     N(0, I) + 3u at position 0 (sink) and at round(f n) heavy-hitter
           positions drawn without replacement from 1..n-1, + 0.5u on the last
           `recency` keys (C1, C2)
  queries  2u + N(0, I)  (window queries and the decode query)
  values   N(0, I)
C3 keys and queries are drawn in 128 dims, rotated by RoPE at their positions
(half-split pairing (x, x + 64), base 10000; the decode query sits at position
n) and stored with 44 of the 64 pairs kept as [firsts | seconds]; values keep
the same 88 dims.  C4 chunk keys are the last key of each chunk times a seeded
Gaussian 128 x 64 matrix, the chunk query is the decode query times the same
matrix.  fp32 draws are rounded to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Config

SEED_ROOT = 20261203

# tensor ids in the seed tuple
T_U, T_K, T_V, T_QWIN, T_QDEC, T_HH, T_PROFILE, T_HHFRAC, T_HEADKIND, T_SPECIAL, \
    T_PAIRS, T_CHUNKS, T_PROJ = range(13)
T_STEP = 13   # decode step t draws tensor ids T_STEP + 3t (key), + 1 (value), + 2 (queries)
T_CSTEP = 1 << 20   # C4 decode step t: tensor id T_CSTEP + t draws the chunk-boundary flag

HEAD_GLOBAL, HEAD_LOCAL, HEAD_SPECIAL = 0, 1, 2

ROPE_BASE = 10000.0


def _rng(cfg: Config, layer: int, b: int, kvh: int, tid: int) -> np.random.Generator:
    ss = np.random.SeedSequence([SEED_ROOT, cfg.cid, layer, b, kvh, tid])
    return np.random.Generator(np.random.PCG64(ss))


# --------------------------------------------------------------------------
# bf16 bit handling (input storage only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); return the uint16 words."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 words to float32."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(cfg: Config, x32: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(x32) if cfg.dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def stored_to_f32(cfg: Config, x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(x) if cfg.dtype == "bf16" else np.asarray(x, np.float32)


# --------------------------------------------------------------------------
# per-layer / per-model draws
# --------------------------------------------------------------------------

def head_direction(cfg: Config, layer: int, kvh: int) -> np.ndarray:
    g = _rng(cfg, layer, 0, kvh, T_U).standard_normal(cfg.d_gen)
    return (g / np.linalg.norm(g)).astype(np.float32)


def layer_hh_frac(cfg: Config, layer: int) -> float:
    if cfg.hh_frac_range:
        lo, hi = cfg.hh_frac_range
        return float(_rng(cfg, layer, 0, 0, T_HHFRAC).uniform(lo, hi))
    return cfg.hh_frac


def heavy_hitters(cfg: Config, layer: int, b: int, kvh: int) -> np.ndarray:
    cnt = cfg.hh_count(layer_hh_frac(cfg, layer))
    cnt = min(cnt, cfg.n - 1)
    pos = _rng(cfg, layer, b, kvh, T_HH).choice(np.arange(1, cfg.n), size=cnt, replace=False)
    return np.sort(pos)


def zigzag_profile(cfg: Config) -> np.ndarray:
    """Synthetic per-layer uncertainty profile x_l ~ lognormal(0, 0.5) (float64)."""
    return _rng(cfg, 0, 0, 0, T_PROFILE).lognormal(0.0, 0.5, size=cfg.layers)


def head_kinds(cfg: Config, layer: int = 0) -> np.ndarray:
    """C3: seeded permutation of local/special/global kinds over the KV heads (int8)."""
    nl, ns, ng = cfg.head_ratio
    kinds = np.array([HEAD_LOCAL] * nl + [HEAD_SPECIAL] * ns + [HEAD_GLOBAL] * ng, np.int8)
    assert kinds.size == cfg.hkv
    return kinds[_rng(cfg, layer, 0, 0, T_HEADKIND).permutation(cfg.hkv)].astype(np.int8)


def special_positions(cfg: Config, b: int, layer: int = 0) -> np.ndarray:
    """C3: sorted special-token positions of batch element b, sink (0) included (int32)."""
    pos = _rng(cfg, layer, b, 0, T_SPECIAL).choice(np.arange(1, cfg.n), size=cfg.n_special,
                                                   replace=False)
    return np.concatenate([[0], np.sort(pos)]).astype(np.int32)


def kept_pairs(cfg: Config, layer: int, kvh: int) -> np.ndarray:
    """C3: sorted indices of the RoPE pairs kept for (layer, KV head)."""
    npairs = cfg.d_rope // 2
    return np.sort(_rng(cfg, layer, 0, kvh, T_PAIRS).choice(npairs, size=cfg.kept_pairs,
                                                           replace=False))


def chunk_ends(cfg: Config, b: int = 0, layer: int = 0) -> np.ndarray:
    """C4: exclusive chunk end positions, strictly increasing, last == n (int64).

    Lengths are i.i.d. Geometric(1/mean) on {1, 2, ...}; the last chunk is cut at n.
    One draw per layer, shared by every batch element and KV head (`b` is ignored).
    """
    r = _rng(cfg, layer, 0, 0, T_CHUNKS)
    ends = []
    pos = 0
    while pos < cfg.n:
        draw = r.geometric(1.0 / cfg.chunk_mean, size=4096)
        for ln in draw:
            pos = min(cfg.n, pos + int(ln))
            ends.append(pos)
            if pos >= cfg.n:
                break
    return np.asarray(ends, np.int64)


def chunk_projection(cfg: Config, layer: int = 0) -> np.ndarray:
    """C4: seeded d x chunk_dim Gaussian projection, entries N(0, 1/chunk_dim) (float64)."""
    return _rng(cfg, layer, 0, 0, T_PROJ).standard_normal((cfg.d, cfg.chunk_dim)) / np.sqrt(
        cfg.chunk_dim)


# --------------------------------------------------------------------------
# RoPE layout for C3 (input preparation only)
# --------------------------------------------------------------------------

def rope_rotate(x: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Rotate rows of x (.., 128) at positions pos with half-split pairing, in float64."""
    dr = x.shape[-1]
    half = dr // 2
    theta = ROPE_BASE ** (-np.arange(half, dtype=np.float64) / half)
    ang = np.asarray(pos, np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half].astype(np.float64), x[..., half:].astype(np.float64)
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def rope_table(max_pos: int, half: int = 64) -> np.ndarray:
    """The model's RoPE table: [max_pos][half][2] float32 (cos, sin) of the
    angle t * base^(-p / half) of rotary pair p at position t (computed in
    float64, rounded once).  Model constants, like the weights."""
    theta = ROPE_BASE ** (-np.arange(half, dtype=np.float64) / half)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * theta[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def prune_pairs(x: np.ndarray, pairs: np.ndarray, half: int) -> np.ndarray:
    """Keep pair p as dims (p, p + half); store as [firsts | seconds]."""
    return np.concatenate([x[..., pairs], x[..., pairs + half]], axis=-1)


# --------------------------------------------------------------------------
# one segment = one (layer, batch element, KV head)
# --------------------------------------------------------------------------

def segment_kv(cfg: Config, layer: int, b: int, kvh: int):
    """Return (K, V) for one segment in storage format, shapes [n][d]."""
    n, dg = cfg.n, cfg.d_gen
    u = head_direction(cfg, layer, kvh)
    K = _rng(cfg, layer, b, kvh, T_K).standard_normal((n, dg), dtype=np.float32)
    plant = np.zeros(n, np.float32)
    plant[heavy_hitters(cfg, layer, b, kvh)] = 3.0
    plant[0] = 3.0
    if cfg.recency:
        plant[n - cfg.recency:] += np.float32(0.5)
    K += plant[:, None] * u[None, :]
    V = _rng(cfg, layer, b, kvh, T_V).standard_normal((n, dg), dtype=np.float32)
    if cfg.d_rope:
        pairs = kept_pairs(cfg, layer, kvh)
        half = dg // 2
        K = prune_pairs(rope_rotate(K, np.arange(n)), pairs, half).astype(np.float32)
        V = prune_pairs(V, pairs, half)
    return _store(cfg, K), _store(cfg, V)


def segment_queries(cfg: Config, layer: int, b: int, kvh: int):
    """Window queries [G][w][d] (None when w == 0) and decode queries [G][d]."""
    G, dg = cfg.G, cfg.d_gen
    u = head_direction(cfg, layer, kvh)
    qwin = None
    if cfg.w:
        qw = _rng(cfg, layer, b, kvh, T_QWIN).standard_normal((G, cfg.w, dg), dtype=np.float32)
        qw += np.float32(2.0) * u
        qwin = _store(cfg, qw)
    qd = _rng(cfg, layer, b, kvh, T_QDEC).standard_normal((G, dg), dtype=np.float32)
    qd += np.float32(2.0) * u
    if cfg.d_rope:
        pairs = kept_pairs(cfg, layer, kvh)
        qd = prune_pairs(rope_rotate(qd, np.full(G, cfg.n)), pairs, dg // 2).astype(np.float32)
    return qwin, _store(cfg, qd)


def step_token(cfg: Config, layer: int, b: int, kvh: int, t: int, rotated: bool = True):
    """Decode step t of one segment: the token at position n + t.

    Returns (k [d], v [d], q [G][d]) in storage format: the new key and value
    drawn like the cache's bulk keys and values (no planted structure), the G
    query heads drawn like the decode query.  C3 rotates key and queries at
    position n + t and keeps the segment's RoPE pairs; with rotated=False it
    keeps the pairs but leaves the rotation to the consumer.
    """
    G, dg = cfg.G, cfg.d_gen
    u = head_direction(cfg, layer, kvh)
    k = _rng(cfg, layer, b, kvh, T_STEP + 3 * t).standard_normal(dg, dtype=np.float32)
    v = _rng(cfg, layer, b, kvh, T_STEP + 3 * t + 1).standard_normal(dg, dtype=np.float32)
    q = _rng(cfg, layer, b, kvh, T_STEP + 3 * t + 2).standard_normal((G, dg), dtype=np.float32)
    q += np.float32(2.0) * u
    if cfg.d_rope:
        pairs = kept_pairs(cfg, layer, kvh)
        half = dg // 2
        pos = cfg.n + t
        if rotated:
            k = rope_rotate(k[None, :], np.array([pos]))[0]
            q = rope_rotate(q, np.full(G, pos))
        k = prune_pairs(k[None, :], pairs, half)[0]
        q = prune_pairs(q, pairs, half)
        v = prune_pairs(v, pairs, half)
    return (_store(cfg, k.astype(np.float32)), _store(cfg, v.astype(np.float32)),
            _store(cfg, q.astype(np.float32)))


def step_inputs(cfg: Config, layer: int, t: int, rotated: bool = True) -> dict:
    """Decode step t for a whole layer: k_new, v_new [b][hkv][d], q [b][hq][d]."""
    B, Hkv, G, d = cfg.batch, cfg.hkv, cfg.G, cfg.d
    sdt = np.uint16 if cfg.dtype == "bf16" else np.float32
    kn = np.empty((B, Hkv, d), sdt)
    vn = np.empty((B, Hkv, d), sdt)
    q = np.empty((B, cfg.hq, d), sdt)
    for b in range(B):
        for kvh in range(Hkv):
            kn[b, kvh], vn[b, kvh], q[b, kvh * G:(kvh + 1) * G] = step_token(cfg, layer, b, kvh, t,
                                                                              rotated)
    return {"k_new": kn, "v_new": vn, "q": q, "pos": cfg.n + t}


def chunk_step_inputs(cfg: Config, layer: int, t: int) -> dict:
    """C4 decode step t: step_inputs plus whether token n + t closes a chunk
    (Bernoulli(1 / chunk_mean): the Geometric chunk lengths continued past n,
    one draw per layer shared by the batch), the chunk key that token gives
    (its key times the projection) [b][hkv][chunk_dim] and each query head's
    chunk query (its decode query times the projection) [b][hq][1][chunk_dim]."""
    st = step_inputs(cfg, layer, t)
    P = chunk_projection(cfg, layer)
    boundary = bool(_rng(cfg, layer, 0, 0, T_CSTEP + t).random() < 1.0 / cfg.chunk_mean)
    ck = (stored_to_f32(cfg, st["k_new"]).astype(np.float64) @ P).astype(np.float32)
    cq = (stored_to_f32(cfg, st["q"]).astype(np.float64) @ P).astype(np.float32)
    st.update(boundary=boundary, chunk_key=_store(cfg, ck), chunk_q=_store(cfg, cq[:, :, None, :]))
    return st


def segment_chunk_inputs(cfg: Config, K_seg: np.ndarray, qdec_seg: np.ndarray,
                         ends: np.ndarray, P: np.ndarray):
    """C4: chunk keys [nc][chunk_dim] and chunk queries [G][1][chunk_dim] (storage format)."""
    k_last = stored_to_f32(cfg, K_seg[ends - 1]).astype(np.float64)
    ck = (k_last @ P).astype(np.float32)
    cq = (stored_to_f32(cfg, qdec_seg).astype(np.float64) @ P).astype(np.float32)
    return _store(cfg, ck), _store(cfg, cq[:, None, :])


def segment_inputs(cfg: Config, layer: int, b: int, kvh: int) -> dict:
    """All inputs that one (layer, b, kvh) segment needs, in storage format."""
    K, V = segment_kv(cfg, layer, b, kvh)
    qwin, qdec = segment_queries(cfg, layer, b, kvh)
    out = {"K": K, "V": V, "q_win": qwin, "q_dec": qdec}
    if cfg.mode == "chunk":
        ends = chunk_ends(cfg, b, layer)
        ck, cq = segment_chunk_inputs(cfg, K, qdec, ends, chunk_projection(cfg, layer))
        out.update(chunk_end=ends, chunk_keys=ck, chunk_q=cq)
    if cfg.mode == "policy":
        out.update(head_kind=int(head_kinds(cfg, layer)[kvh]),
                   special_pos=special_positions(cfg, b, layer))
    return out


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def layer_inputs(cfg: Config, layer: int = 0, threads: int | None = None) -> dict:
    """Full-layer tensors in storage format.

    K, V      [b][hkv][n][d]
    q_win     [b][hq][w][d]          (w > 0)
    q_dec     [b][hq][d]
    chunk     chunk_end [b][nc] int64, chunk_keys [b][hkv][nc][cd], chunk_q [b][hq][1][cd]
    policy    head_kind [hkv] int8, special_pos [b][n_special + 1] int32
    """
    B, Hkv, Hq, G, n, d = cfg.batch, cfg.hkv, cfg.hq, cfg.G, cfg.n, cfg.d
    sdt = np.uint16 if cfg.dtype == "bf16" else np.float32
    K = np.empty((B, Hkv, n, d), sdt)
    V = np.empty((B, Hkv, n, d), sdt)
    qwin = np.empty((B, Hq, cfg.w, d), sdt) if cfg.w else None
    qdec = np.empty((B, Hq, d), sdt)

    def one(seg):
        b, kvh = divmod(seg, Hkv)
        K[b, kvh], V[b, kvh] = segment_kv(cfg, layer, b, kvh)
        qw, qd = segment_queries(cfg, layer, b, kvh)
        if qwin is not None:
            qwin[b, kvh * G:(kvh + 1) * G] = qw
        qdec[b, kvh * G:(kvh + 1) * G] = qd

    nthreads = threads or _workers()
    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(one, range(B * Hkv)))

    out = {"K": K, "V": V, "q_win": qwin, "q_dec": qdec}
    if cfg.mode == "chunk":
        P = chunk_projection(cfg, layer)
        ends = [chunk_ends(cfg, b, layer) for b in range(B)]
        nc = ends[0].size
        cks = np.empty((B, Hkv, nc, cfg.chunk_dim), sdt)
        cqs = np.empty((B, Hq, 1, cfg.chunk_dim), sdt)
        for b in range(B):
            for kvh in range(Hkv):
                ck, cq = segment_chunk_inputs(cfg, K[b, kvh], qdec[b, kvh * G:(kvh + 1) * G],
                                              ends[b], P)
                cks[b, kvh] = ck
                cqs[b, kvh * G:(kvh + 1) * G] = cq
        out.update(chunk_end=np.stack(ends), chunk_keys=cks, chunk_q=cqs)
    if cfg.mode == "policy":
        out.update(head_kind=head_kinds(cfg, layer),
                   special_pos=np.stack([special_positions(cfg, b, layer) for b in range(B)]))
    return out
