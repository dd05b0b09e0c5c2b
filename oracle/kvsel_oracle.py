"""Float64 reference for every step of the selection-then-decode path.

TEST INFRASTRUCTURE ONLY (see the package docstring): the tests, the smoke
check and the benchmark's CPU-baseline leg use it; nothing on the product
path may.

Sources (pages are cited by title and the equation / section they give):
  [ZZ]  "ZigZagkv: Dynamic KV Cache Compression for Long-context Modeling based
        on Layer Uncertainty" (arXiv 2412.09036) -- Eq. 3 (LMBA), Eq. 4
        (normalised layer uncertainty), Eq. 6 (bounded per-layer budget),
        Eq. 7 (token score = attention summed over the last w queries).
  [FG]  "Model Tells You What to Discard: Adaptive KV Cache Compression for
        LLMs" (arXiv 2310.01801) -- core claim: local heads drop long-range
        tokens, special-token heads keep only special tokens, global heads keep
        everything.
  [CK]  "ChunkLLM: A Lightweight Pluggable Framework for Accelerating LLMs
        Inference" (arXiv 2510.02361) -- QK Adapter (§2.2, Eq. 3): chunk
        attention is a softmax over compressed query . chunk-key products;
        only the top-k chunks stay in the KV cache.
  [RAP] "RAP: KV-Cache Compression via RoPE-Aligned Pruning" (arXiv
        2602.02599) -- decode-step attention over the cached keys and values
        (Fig. 2 / Eq. 2); RoPE turns 2-D pairs, so a head that keeps whole
        pairs is rotated pair by pair with each kept pair's frequency and
        pruning commutes with the rotation (§3, Eq. 5-10).

Readings where the pages are silent (each is also listed with the design
notes): window query i sits at position q_pos0 + i and sees keys j <= q_pos0+i;
GQA query heads of one KV head add their mass; ties in a score order go to the
lower index and kept indices are emitted ascending; NaN scores order last;
budgets are integerised by largest remainder (ties to the lower layer) and
capped at n with the excess spread over the uncapped layers in proportion to
their uncertainty.

Every floating-point step is float64, except the RoPE rotation, whose
arithmetic is fixed as fp32 (each product and sum rounded on its own, then
rounded to the storage type) so that a rotated bf16 row has exactly one
correct value.  bf16 inputs arrive as uint16 words and are widened exactly.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "to_f64", "softmax", "window_scores", "lmba_row", "layer_lmba",
    "zigzag_budgets", "score_order", "select_topb", "select_chunks",
    "select_policy", "compact", "decode_attention", "decode_partial",
    "combine_partials", "append_token", "window_probabilities", "attention_loss",
    "round_bf16", "rope_pairs", "chunk_votes", "vote_chunks",
    "HEAD_GLOBAL", "HEAD_LOCAL", "HEAD_SPECIAL",
]

HEAD_GLOBAL, HEAD_LOCAL, HEAD_SPECIAL = 0, 1, 2


# ---------------------------------------------------------------------------
# input widening
# ---------------------------------------------------------------------------

def to_f64(x: np.ndarray) -> np.ndarray:
    """Widen stored inputs to float64: uint16 arrays are bf16 words, others are floats."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# ---------------------------------------------------------------------------
# A1  window score  [ZZ Eq. 7]
# ---------------------------------------------------------------------------

def softmax(logits: np.ndarray) -> np.ndarray:
    """Softmax of one row; entries at -inf (masked) get probability 0."""
    m = np.max(logits)
    e = np.exp(logits - m)
    return e / np.sum(e)


def window_scores(q_win: np.ndarray, k: np.ndarray, scale: float, q_pos0: int) -> np.ndarray:
    """Score of every cached key of one KV head.

    q_win  [G][w][d]  window queries of the G query heads that share this KV head
    k      [n][d]     cached keys
    Returns s [n] with s_j = sum over heads h and window rows i of A^h_ij, the
    softmax attention weight of window query i on key j ([ZZ Eq. 7]).  Window
    query i sits at position q_pos0 + i and attends causally to keys
    j <= q_pos0 + i.
    """
    q_win = np.asarray(q_win, np.float64)
    k = np.asarray(k, np.float64)
    G, w, _ = q_win.shape
    n = k.shape[0]
    pos = np.arange(n)
    s = np.zeros(n)
    for h in range(G):
        logits = scale * (q_win[h] @ k.T)          # [w][n]
        for i in range(w):
            row = np.where(pos <= q_pos0 + i, logits[i], -np.inf)
            s += softmax(row)
    return s


def window_probabilities(q_win: np.ndarray, k: np.ndarray, scale: float, q_pos0: int) -> np.ndarray:
    """The attention rows behind window_scores: P [G*w][n], row h*w + i is the
    softmax of window query i of head h over the keys it sees (j <= q_pos0 + i,
    zero elsewhere) [ZZ Eq. 1 / Eq. 7]."""
    q_win = np.asarray(q_win, np.float64)
    k = np.asarray(k, np.float64)
    G, w, _ = q_win.shape
    n = k.shape[0]
    pos = np.arange(n)
    P = np.zeros((G * w, n))
    for h in range(G):
        logits = scale * (q_win[h] @ k.T)
        for i in range(w):
            P[h * w + i] = softmax(np.where(pos <= q_pos0 + i, logits[i], -np.inf))
    return P


def attention_loss(P: np.ndarray, kept, mass: float = 0.9) -> np.ndarray:
    """Per-row attention loss of a kept token set [ZZ §5.5, Table 3: the
    deviation from keeping 0.9 of the attention]: max(0, mass - sum of the
    row's weights on the kept tokens).  The reported figure is the mean."""
    P = np.asarray(P, np.float64)
    kept = np.asarray(kept, np.int64)
    got = P[:, kept].sum(axis=1) if kept.size else np.zeros(P.shape[0])
    return np.maximum(0.0, mass - got)


# ---------------------------------------------------------------------------
# LMBA  [ZZ Eq. 3]
# ---------------------------------------------------------------------------

def _exact(v) -> Fraction:
    """Exact rational value of a Fraction, an integer or a float64."""
    if isinstance(v, Fraction):
        return v
    if isinstance(v, (int, np.integer)):
        return Fraction(int(v))
    return Fraction(float(v))


def lmba_row(p, mass=Fraction(9, 10)) -> int:
    """Smallest number of tokens whose attention weights reach `mass` of the row's total.

    Exact: every float64 weight is taken at its exact binary value, so a
    uniform row of n entries needs exactly ceil(0.9 n) tokens.
    """
    seq = p if isinstance(p, (list, tuple)) else list(np.asarray(p).ravel())
    vals = [_exact(v) for v in seq]
    if not vals:
        return 0
    mass = Fraction(mass)
    total = sum(vals, Fraction(0))
    target = mass * total
    acc = Fraction(0)
    for k, v in enumerate(sorted(vals, reverse=True), start=1):
        acc += v
        if acc >= target:
            return k
    return len(vals)


def layer_lmba(attn_rows, mass=Fraction(9, 10)) -> float:
    """Mean over attention rows (heads, and window rows within a head) of lmba_row."""
    rows = [r for r in attn_rows]
    return float(np.mean([lmba_row(r, mass) for r in rows])) if rows else 0.0


# ---------------------------------------------------------------------------
# A2  bounded per-layer budgets  [ZZ Eq. 4, Eq. 6]
# ---------------------------------------------------------------------------

def zigzag_budgets(profile, n: int, avg_budget: int, floor_budget: int) -> np.ndarray:
    """Integer per-layer budgets b_l, sum L*avg_budget, each in [floor_budget, n].

    Eq. 4: u_l = x_l / sum_l x_l (x = per-layer LMBA profile).
    Eq. 6: beta_l = B_bound + (B - B_bound) * L * u_l with B = avg_budget and
    B_bound = floor_budget.  Layers whose beta exceeds n are fixed at n and
    Eq. 6 is re-applied to the remaining layers with the remaining total (the
    excess goes to the uncapped layers in proportion to u_l).  The real
    budgets are rounded down and the leftover units go one each to the
    largest fractional parts, ties to the lower layer.
    Sums run sequentially in layer order in float64.
    """
    x = [float(v) for v in profile]
    L = len(x)
    F, B = int(floor_budget), int(avg_budget)
    if L == 0:
        return np.zeros(0, np.int64)
    if not (0 <= F <= B) or n < 0 or B > n:
        raise ValueError("need 0 <= floor <= avg <= n")
    if any(not (v > 0.0) or v != v or v == float("inf") for v in x):
        raise ValueError("profile entries must be finite and > 0")
    total = L * B
    sx = 0.0
    for v in x:
        sx += v
    u = [v / sx for v in x]                      # Eq. 4

    capped = [False] * L
    while True:
        free = [l for l in range(L) if not capped[l]]
        remaining = total - n * (L - len(free))
        su = 0.0
        for l in free:
            su += u[l]
        spread = remaining - F * len(free)       # integer: (B - B_bound) * L on the first pass
        beta = {}
        for l in free:
            share = u[l] if len(free) == L else u[l] / su
            beta[l] = F + spread * share         # Eq. 6
        over = [l for l in free if beta[l] > n]
        if not over:
            break
        for l in over:
            capped[l] = True

    out = np.zeros(L, np.int64)
    for l in range(L):
        if capped[l]:
            out[l] = n
    base = {l: int(np.floor(beta[l])) for l in beta}
    for l, v in base.items():
        out[l] = v
    leftover = total - int(out.sum())
    frac_order = sorted(beta.keys(), key=lambda l: (-(beta[l] - base[l]), l))
    i = 0
    while leftover > 0:
        l = frac_order[i % len(frac_order)]
        if out[l] < n:
            out[l] += 1
            leftover -= 1
        i += 1
    return out


# ---------------------------------------------------------------------------
# A3  selection  [ZZ Eq. 7 top tokens; CK chunk top-k; FG head policies]
# ---------------------------------------------------------------------------

def score_order(s: np.ndarray) -> np.ndarray:
    """Indices by score descending, lower index first on equal scores, NaN last."""
    s = np.asarray(s, np.float64)
    key = np.where(np.isnan(s), np.inf, -s)      # NaN after every real score
    key = np.where(key == 0.0, 0.0, key)         # -0 and +0 are one score
    nan_last = np.isnan(s).astype(np.int8)
    return np.lexsort((np.arange(s.size), key, nan_last))


def select_topb(s: np.ndarray, budget: int) -> np.ndarray:
    """Keep the min(budget, n) highest-score tokens; return their indices ascending."""
    b = max(0, min(int(budget), s.size))
    return np.sort(score_order(s)[:b]).astype(np.int64)


def select_chunks(chunk_scores: np.ndarray, chunk_end: np.ndarray, keep_tokens: int,
                  local_chunks: int = 0, top_chunks: int = 0) -> np.ndarray:
    """Chunk selection [CK §2.3; the operating points of §3.2]: the last
    `local_chunks` chunks are always kept; then

      top_chunks > 0   the `top_chunks` highest-scoring other chunks are kept
                       (a fixed chunk count, the top_k = 256 setting);
      top_chunks == 0  other chunks are taken in score order until the kept
                       token count (local chunks included) reaches keep_tokens.

    chunk_end is the exclusive end of each chunk (the first starts at 0).
    Returns the kept token positions ascending (chunks are kept whole).
    """
    ends = np.asarray(chunk_end, np.int64)
    starts = np.concatenate([[0], ends[:-1]])
    nc = ends.size
    n_local = max(0, min(int(local_chunks), nc))
    chosen = list(range(nc - n_local, nc))
    got = int(sum(int(ends[c] - starts[c]) for c in chosen))
    others = [int(c) for c in score_order(chunk_scores) if c < nc - n_local]
    if top_chunks > 0:
        chosen += others[:int(top_chunks)]
    elif got < keep_tokens:
        for c in others:
            chosen.append(c)
            got += int(ends[c] - starts[c])
            if got >= keep_tokens:
                break
    chosen.sort()
    if not chosen:
        return np.zeros(0, np.int64)
    return np.concatenate([np.arange(starts[c], ends[c]) for c in chosen]).astype(np.int64)


def chunk_votes(layer_scores, top_k: int):
    """Ballots of the layer-wise chunk vote [CK §2.3, where the rule is given
    only in words; the reading taken]: layer l votes for its own top_k chunks,
    select_topb on its chunk scores.  layer_scores [L][nc].  Returns
    (votes [nc] int64: how many layers voted for each chunk,
     total [nc] float64: each chunk's attention summed over the layers)."""
    S = np.asarray(layer_scores, np.float64)
    L, nc = S.shape
    votes = np.zeros(nc, np.int64)
    for layer in range(L):
        votes[select_topb(S[layer], top_k)] += 1
    total = np.array([math.fsum(S[:, c]) for c in range(nc)], np.float64)
    return votes, total


def vote_chunks(layer_scores, top_k: int, chunk_end, local_chunks: int = 0) -> np.ndarray:
    """The chunks one (batch element, KV head) keeps for all layers under the
    layer-wise vote [CK §2.3; reading taken]: the last local_chunks chunks,
    plus the top_k other chunks ordered by most votes, then larger attention
    summed over the layers, then lower index.  Chunk c covers
    [chunk_end[c-1], chunk_end[c]).  Returns the kept token positions in
    ascending order (int64), as select_chunks does."""
    votes, total = chunk_votes(layer_scores, top_k)
    ends = np.asarray(chunk_end, np.int64)
    starts = np.concatenate([[0], ends[:-1]])
    nc = ends.size
    n_local = max(0, min(int(local_chunks), nc))
    others = sorted(range(nc - n_local), key=lambda c: (-int(votes[c]), -float(total[c]), c))
    chosen = sorted(list(range(nc - n_local, nc)) + others[:int(top_k)])
    if not chosen:
        return np.zeros(0, np.int64)
    return np.concatenate([np.arange(starts[c], ends[c]) for c in chosen]).astype(np.int64)


def select_policy(kind: int, n: int, local_window: int, special_pos) -> np.ndarray:
    """[FG] head policies: GLOBAL keeps all n, LOCAL the last local_window, SPECIAL its set."""
    if kind == HEAD_GLOBAL:
        return np.arange(n, dtype=np.int64)
    if kind == HEAD_LOCAL:
        return np.arange(max(0, n - int(local_window)), n, dtype=np.int64)
    if kind == HEAD_SPECIAL:
        return np.unique(np.asarray(special_pos, np.int64))
    raise ValueError(f"unknown head kind {kind}")


# ---------------------------------------------------------------------------
# A4  gather-compact
# ---------------------------------------------------------------------------

def compact(K: np.ndarray, V: np.ndarray, idx: np.ndarray):
    """Rows idx of K and V, in idx order (an exact copy of the stored words)."""
    idx = np.asarray(idx, np.int64)
    return K[idx], V[idx]


# ---------------------------------------------------------------------------
# A5 / A6  decode attention over the compacted cache  [RAP Fig. 2 / Eq. 2]
# ---------------------------------------------------------------------------

def decode_attention(q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q . K_c^T) V_c for one query head; zeros for an empty cache."""
    q = np.asarray(q, np.float64)
    Kc = np.asarray(Kc, np.float64)
    Vc = np.asarray(Vc, np.float64)
    if Kc.shape[0] == 0:
        return np.zeros(Vc.shape[1] if Vc.ndim == 2 else q.shape[0])
    p = softmax(scale * (Kc @ q))
    return p @ Vc


def decode_partial(q, K, V, scale):
    """(m, l, o): max logit, sum of exp(logit - m), and the exp-weighted sum of V rows."""
    q, K, V = (np.asarray(a, np.float64) for a in (q, K, V))
    logits = scale * (K @ q)
    m = np.max(logits)
    e = np.exp(logits - m)
    return m, np.sum(e), e @ V


def combine_partials(parts) -> np.ndarray:
    """Merge (m, l, o) partials of disjoint row sets into the normalised output."""
    M = max(m for m, _, _ in parts)
    L = sum(np.exp(m - M) * l for m, l, _ in parts)
    O = sum(np.exp(m - M) * o for m, _, o in parts)
    return O / L


# ---------------------------------------------------------------------------
# decode-time cache maintenance  [FG: the per-head eviction rule holds for the
# rest of generation]
# ---------------------------------------------------------------------------

def append_token(idx, Kc, Vc, pos: int, k_new, v_new, cap: int, limit: int):
    """Add the token just produced (position `pos`, rows k_new / v_new) to one
    segment whose rows are (idx, Kc, Vc), under the segment's rule:

      limit < 0   the token is not added (a special-token head, ordinary token)
      limit == 0  the segment grows up to `cap` rows (a global head)
      limit > 0   at most min(limit, cap) rows (a local head's window)

    Below that bound the row is appended at the end; at (or above) it, the row
    holding the smallest position -- the oldest token -- is overwritten in
    place (the first such row).  Returns new (idx, Kc, Vc) arrays.
    """
    idx = np.array(idx, np.int64)
    Kc = np.array(Kc)
    Vc = np.array(Vc)
    if limit < 0:
        return idx, Kc, Vc
    bound = cap if limit == 0 else min(cap, limit)
    if bound <= 0:
        return idx, Kc, Vc
    if idx.size < bound:
        return (np.append(idx, pos), np.concatenate([Kc, np.asarray(k_new)[None]]),
                np.concatenate([Vc, np.asarray(v_new)[None]]))
    j = int(np.argmin(idx))          # first row with the smallest position
    idx[j] = pos
    Kc[j] = k_new
    Vc[j] = v_new
    return idx, Kc, Vc


# ---------------------------------------------------------------------------
# pair-pruned RoPE  [RAP §3, Eq. 5-10]
# ---------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """float32 values rounded to the nearest bf16 (ties to the even pattern),
    as uint16 words.  Written from the definition: the two bf16 values that
    bracket x are its pattern truncated to 16 bits and the next pattern away
    from zero; the nearer one wins, a tie goes to the one whose last bit is 0.
    NaN becomes a quiet NaN."""
    f = np.asarray(x, np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lo = u & 0xFFFF0000
    hi = lo + 0x10000
    with np.errstate(invalid="ignore"):     # inf and NaN bracket themselves with NaNs
        f64 = f.astype(np.float64)
        v_lo = (lo.astype(np.uint32)).view(np.float32).astype(np.float64)
        v_hi = (hi.astype(np.uint32)).view(np.float32).astype(np.float64)
        d_lo, d_hi = np.abs(f64 - v_lo), np.abs(v_hi - f64)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (((lo >> 16) & 1) == 1))
    out = np.where(take_hi, hi, lo) >> 16
    out = np.where(np.isnan(f), (u >> 16) | 0x40, out)
    return out.astype(np.uint16)


def rope_pairs(x, pos, cos_sin, pairs, dtype: str) -> np.ndarray:
    """Rotate rows of a pair-pruned head at their positions [RAP §3].

    x        [..., d] rows in storage form (bf16: uint16 words; fp32: float32);
             kept pair e is elements e and e + d/2
    pos      [...] position of each row
    cos_sin  [max_pos][half][2] fp32 table of (cos, sin) per position and
             rotary pair of the unpruned head
    pairs    [d/2] kept pair index of each stored pair
    Pair (x, y) becomes (x c - y s, x s + y c), (c, s) = cos_sin[pos][pairs[e]],
    every product and the two sums rounded to fp32 on their own, the result
    rounded to the storage type.  Returns rows in storage form.
    """
    x = np.asarray(x)
    d = x.shape[-1]
    h2 = d // 2
    if dtype == "bf16":
        xf = (x.astype(np.uint32) << 16).view(np.float32)
    else:
        xf = x.astype(np.float32)
    a, b = xf[..., :h2], xf[..., h2:]
    tab = np.asarray(cos_sin, np.float32)
    pos = np.asarray(pos, np.int64)
    pr = np.asarray(pairs, np.int64)
    c = tab[pos[..., None], pr, 0]
    s = tab[pos[..., None], pr, 1]
    xc, ys, xs, yc = a * c, b * s, a * s, b * c       # float32 products, each rounded
    out = np.concatenate([xc - ys, xs + yc], axis=-1).astype(np.float32)
    return round_bf16(out) if dtype == "bf16" else out
