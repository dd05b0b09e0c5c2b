"""Pins for the CPU oracle: closed forms, invariants, brute force and the
hand-worked fixtures under tests/golden/.  None of these re-types an oracle
formula; each checks the oracle against something the pages or the
mathematics fix independently.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sigmoid(x):
    return 1.0 / (1.0 + math.exp(-x))


# ---------------------------------------------------------------------------
# window score (ZigZagkv page, Eq. 7)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("G,w,n,d,q_pos0", [(2, 8, 512, 64, 504), (4, 3, 37, 16, 34),
                                             (1, 1, 9, 8, 100), (3, 5, 20, 8, 2)])
def test_score_mass_sums_to_rows(G, w, n, d, q_pos0):
    # every softmax row sums to one, so the scores of one KV head sum to G*w
    r = np.random.default_rng(1)
    s = oracle.window_scores(r.standard_normal((G, w, d)), r.standard_normal((n, d)),
                             1 / math.sqrt(d), q_pos0)
    assert s.shape == (n,)
    assert abs(s.sum() - G * w) < 1e-10
    assert (s >= 0).all()
    # keys no window row can see get nothing
    assert np.all(s[np.arange(n) > q_pos0 + w - 1] == 0)


def test_score_zero_query_is_uniform_over_visible_keys():
    # q = 0 makes every visible logit equal: row i puts 1/(q_pos0+i+1) on keys 0..q_pos0+i
    G, w, n, d = 3, 4, 11, 5
    q_pos0 = n - w
    s = oracle.window_scores(np.zeros((G, w, d)), np.random.default_rng(2).standard_normal((n, d)),
                             0.37, q_pos0)
    want = np.zeros(n)
    for i in range(w):
        want[:q_pos0 + i + 1] += G / (q_pos0 + i + 1)
    np.testing.assert_allclose(s, want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("a,c,scale", [(1.5, 2.0, 0.125), (-0.7, 3.0, 1 / math.sqrt(128)),
                                       (4.0, -1.0, 1.0)])
def test_score_two_key_logistic(a, c, scale):
    # two keys, one query: logits (scale*a*c, 0) give weights sigmoid(+-scale*a*c)
    d = 4
    k = np.zeros((2, d)); k[0, 1] = a
    q = np.zeros((1, 1, d)); q[0, 0, 1] = c
    s = oracle.window_scores(q, k, scale, q_pos0=1)
    x = scale * a * c
    assert abs(s[0] - _sigmoid(x)) < 1e-15
    assert abs(s[1] - _sigmoid(-x)) < 1e-15


def test_score_gqa_heads_add():
    # head 0 has q = 0 (uniform 1/n), head 1 points at key 2 with logit x
    n, d, x = 6, 3, 2.5
    k = np.zeros((n, d)); k[2, 0] = 1.0
    q = np.zeros((2, 1, d)); q[1, 0, 0] = x
    s = oracle.window_scores(q, k, 1.0, q_pos0=n - 1)
    den = math.exp(x) + n - 1
    want = np.full(n, 1.0 / n + 1.0 / den)
    want[2] = 1.0 / n + math.exp(x) / den
    np.testing.assert_allclose(s, want, rtol=0, atol=1e-15)


def test_score_causal_boundary():
    # the first window row must not see the key right after its own position
    n, d = 8, 2
    k = np.zeros((n, d)); k[5, 0] = 50.0     # a key that would dominate if visible
    q = np.zeros((1, 2, d)); q[0, :, 0] = 1.0
    s = oracle.window_scores(q, k, 1.0, q_pos0=4)   # rows at positions 4 and 5
    # row 0 (pos 4) is uniform over keys 0..4; row 1 (pos 5) is almost all on key 5
    den = math.exp(50.0) + 5
    want = np.zeros(n)
    want[:5] = 1 / 5 + 1 / den
    want[5] = math.exp(50.0) / den
    np.testing.assert_allclose(s, want, rtol=1e-15, atol=1e-15)


# ---------------------------------------------------------------------------
# LMBA (ZigZagkv page, Eq. 3)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", list(range(1, 41)) + [100, 1000])
def test_lmba_uniform_row_is_ceil_nine_tenths(n):
    assert oracle.lmba_row(np.full(n, 1.0 / n)) == math.ceil(Fraction(9, 10) * n)


@pytest.mark.parametrize("n,hot", [(1, 0), (7, 3), (512, 511)])
def test_lmba_one_hot(n, hot):
    row = np.zeros(n); row[hot] = 1.0
    assert oracle.lmba_row(row) == 1


def test_lmba_golden_rows():
    g = _load("lmba.json")
    mass = Fraction(g["mass"])
    for case in g["rows"]:
        row = [Fraction(v) for v in case["row"]]
        assert oracle.lmba_row(row, mass) == case["expect"], case


def test_layer_lmba_mean_of_rows():
    rows = [np.full(10, 0.1), np.array([1.0, 0, 0]), np.array([0.5, 0.3, 0.2])]
    assert oracle.layer_lmba(rows) == pytest.approx((9 + 1 + 3) / 3, abs=0)


# ---------------------------------------------------------------------------
# bounded budgets (ZigZagkv page, Eq. 4 + Eq. 6)
# ---------------------------------------------------------------------------

def test_budgets_golden():
    for case in _load("zigzag_budgets.json")["cases"]:
        got = oracle.zigzag_budgets(case["profile"], case["n"], case["avg_budget"],
                                    case["floor_budget"])
        assert got.tolist() == case["expect"], case["name"]


@pytest.mark.parametrize("seed", range(20))
def test_budgets_sum_floor_cap(seed):
    r = np.random.default_rng(seed)
    L = int(r.integers(1, 40))
    n = int(r.integers(50, 40000))
    B = int(r.integers(1, n + 1))
    F = int(r.integers(0, B + 1))
    prof = r.lognormal(0, float(r.uniform(0.1, 2.0)), size=L)
    b = oracle.zigzag_budgets(prof, n, B, F)
    assert b.sum() == L * B
    assert (b >= F).all() and (b <= n).all()
    # more uncertain layers never get fewer tokens (Eq. 6 is increasing in u_l),
    # up to the one unit the rounding can move
    order = np.argsort(prof, kind="stable")
    assert np.all(np.diff(b[order]) >= -1)


def test_budgets_c2_shape():
    # C2: 32 layers, n = 32768, mean 20 % (6553) and floor 5 % (1639)
    import kvsynth
    cfg = kvsynth.get_config(2)
    b = oracle.zigzag_budgets(kvsynth.zigzag_profile(cfg), cfg.n, cfg.avg_budget,
                              cfg.floor_budget)
    assert cfg.avg_budget == 6553 and cfg.floor_budget == 1639
    assert b.sum() == 32 * 6553 and b.min() >= 1639 and b.max() <= 32768
    assert len(set(b.tolist())) > 10          # genuinely non-uniform


def test_budgets_reject_bad_arguments():
    with pytest.raises(ValueError):
        oracle.zigzag_budgets([1, 2], 100, 10, 11)      # floor above average
    with pytest.raises(ValueError):
        oracle.zigzag_budgets([1, 2], 100, 101, 0)      # average above n
    with pytest.raises(ValueError):
        oracle.zigzag_budgets([1, 0], 100, 10, 1)       # non-positive profile


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def _brute_topb(scores, B):
    """Among all B-subsets take the max-sum one, ties broken by the
    lexicographically smallest sorted index tuple (integer scores: exact)."""
    n = len(scores)
    B = min(B, n)
    best = None
    for sub in itertools.combinations(range(n), B):
        key = (-sum(scores[j] for j in sub), sub)
        if best is None or key < best:
            best = key
    return list(best[1]) if best else []


@pytest.mark.parametrize("seed", range(60))
def test_topb_brute_force_with_ties(seed):
    r = np.random.default_rng(100 + seed)
    n = int(r.integers(1, 11))
    scores = [int(v) for v in r.integers(0, 4, size=n)]   # small ints force ties
    B = int(r.integers(0, n + 2))
    got = oracle.select_topb(np.array(scores, np.float64), B).tolist()
    assert got == _brute_topb(scores, B)


def test_topb_golden():
    for case in _load("select.json")["topb"]:
        s = np.array([float(v) for v in case["scores"]])
        assert oracle.select_topb(s, case["budget"]).tolist() == case["expect"], case["why"]


def test_topb_budget_n_keeps_all():
    s = np.random.default_rng(5).standard_normal(300)
    assert oracle.select_topb(s, 300).tolist() == list(range(300))


def _chunk_properties(cs, ends, target, kept):
    starts = np.concatenate([[0], ends[:-1]])
    lens = ends - starts
    chosen = sorted({int(np.searchsorted(ends, t, side="right")) for t in kept})
    # whole chunks
    want = np.concatenate([np.arange(starts[c], ends[c]) for c in chosen]) if chosen else []
    assert list(kept) == list(want)
    if target <= 0:
        assert not chosen
        return
    tot = int(lens[chosen].sum())
    assert tot >= min(target, int(lens.sum()))
    # every chosen chunk ranks above every unchosen one (score desc, index asc)
    rank = lambda c: (-cs[c], c)
    unchosen = [c for c in range(len(cs)) if c not in chosen]
    if unchosen:
        assert max(rank(c) for c in chosen) < min(rank(c) for c in unchosen)
    # minimal: dropping the lowest-ranked chosen chunk falls short
    worst = max(chosen, key=rank)
    assert tot - lens[worst] < target


@pytest.mark.parametrize("seed", range(40))
def test_chunk_selection_properties(seed):
    r = np.random.default_rng(200 + seed)
    nc = int(r.integers(1, 30))
    ends = np.cumsum(r.integers(1, 9, size=nc)).astype(np.int64)
    cs = r.integers(0, 5, size=nc).astype(np.float64)
    target = int(r.integers(0, ends[-1] + 3))
    kept = oracle.select_chunks(cs, ends, target)
    _chunk_properties(cs, ends, target, kept)


def test_chunk_golden():
    for case in _load("select.json")["chunk"]:
        got = oracle.select_chunks(np.array(case["chunk_scores"], float),
                                   np.array(case["chunk_end"]), case["keep_tokens"])
        assert got.tolist() == case["expect"], case["why"]


def test_policy_golden():
    kinds = {"global": oracle.HEAD_GLOBAL, "local": oracle.HEAD_LOCAL,
             "special": oracle.HEAD_SPECIAL}
    for case in _load("select.json")["policy"]:
        got = oracle.select_policy(kinds[case["kind"]], case["n"], case["local_window"],
                                   case["special_pos"])
        assert got.tolist() == case["expect"]


# ---------------------------------------------------------------------------
# compaction
# ---------------------------------------------------------------------------

def test_compact_identity_and_empty():
    r = np.random.default_rng(3)
    K = r.integers(0, 65535, size=(20, 8), dtype=np.uint16)
    V = r.integers(0, 65535, size=(20, 8), dtype=np.uint16)
    Kc, Vc = oracle.compact(K, V, np.arange(20))
    assert np.array_equal(Kc, K) and np.array_equal(Vc, V)
    Kc, Vc = oracle.compact(K, V, np.zeros(0, np.int64))
    assert Kc.shape == (0, 8) and Vc.shape == (0, 8)
    Kc, _ = oracle.compact(K, V, np.array([19, 0]))
    assert np.array_equal(Kc[0], K[19]) and np.array_equal(Kc[1], K[0])


# ---------------------------------------------------------------------------
# decode attention (RAP page, Fig. 2 / Eq. 2) and the split combine
# ---------------------------------------------------------------------------

def test_decode_one_row_returns_that_value():
    r = np.random.default_rng(4)
    v = r.standard_normal((1, 16))
    out = oracle.decode_attention(r.standard_normal(16), r.standard_normal((1, 16)), v, 0.3)
    np.testing.assert_array_equal(out, v[0])


def test_decode_identical_keys_average_values():
    r = np.random.default_rng(5)
    k = np.tile(r.standard_normal(8), (9, 1))
    V = r.standard_normal((9, 8))
    out = oracle.decode_attention(r.standard_normal(8), k, V, 0.5)
    np.testing.assert_allclose(out, V.mean(0), rtol=0, atol=1e-14)


def test_decode_two_key_logistic():
    d, a, c, scale = 4, 1.25, -2.0, 0.25
    K = np.zeros((2, d)); K[1, 3] = a
    q = np.zeros(d); q[3] = c
    V = np.array([[1.0, 0, 0, 0], [0, 0, 0, 1.0]])
    out = oracle.decode_attention(q, K, V, scale)
    p1 = _sigmoid(scale * a * c)
    np.testing.assert_allclose(out, [1 - p1, 0, 0, p1], rtol=0, atol=1e-15)


def test_decode_empty_cache_is_zero():
    out = oracle.decode_attention(np.ones(8), np.zeros((0, 8)), np.zeros((0, 8)), 1.0)
    assert out.shape == (8,) and not out.any()


@pytest.mark.parametrize("seed", range(8))
def test_split_combine_matches_unsplit(seed):
    r = np.random.default_rng(300 + seed)
    n, d = int(r.integers(2, 400)), 32
    q = 3 * r.standard_normal(d)
    K, V = r.standard_normal((n, d)), r.standard_normal((n, d))
    cuts = np.sort(r.choice(np.arange(1, n), size=min(n - 1, int(r.integers(1, 6))),
                            replace=False))
    parts = [oracle.decode_partial(q, K[a:b], V[a:b], 0.2)
             for a, b in zip(np.r_[0, cuts], np.r_[cuts, n])]
    np.testing.assert_allclose(oracle.combine_partials(parts),
                               oracle.decode_attention(q, K, V, 0.2), rtol=0, atol=1e-12)


def test_full_budget_reproduces_full_attention():
    # budget = n keeps every token, so decode over the compacted cache is full attention
    r = np.random.default_rng(6)
    n, d = 50, 16
    K, V, q = r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal(d)
    s = oracle.window_scores(r.standard_normal((2, 3, d)), K, 0.25, n - 3)
    idx = oracle.select_topb(s, n)
    Kc, Vc = oracle.compact(K, V, idx)
    full = oracle.decode_attention(q, K, V, 0.25)
    np.testing.assert_array_equal(oracle.decode_attention(q, Kc, Vc, 0.25), full)
    # and against softmax written with the log-sum-exp identity on the uncompacted cache
    logits = 0.25 * K @ q
    lse = np.log(np.sum(np.exp(logits - logits.max()))) + logits.max()
    np.testing.assert_allclose(full, np.exp(logits - lse) @ V, rtol=0, atol=1e-12)


def test_bf16_widening_exact():
    words = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F], np.uint16)
    got = oracle.to_f64(words)
    assert got.tolist()[:5] == [1.0, -1.0, 3.140625, 0.0, -0.0]
    assert got[5] == 255 * 2.0 ** 120          # largest finite bf16, (2 - 2^-7) * 2^127


# ---------------------------------------------------------------------------
# decode-time maintenance (FastGen page: eviction rules hold during generation)
# ---------------------------------------------------------------------------

def _rows(n, d=4, base=0):
    return (np.arange(n * d, dtype=np.float32).reshape(n, d) + base)


@pytest.mark.parametrize("W,steps", [(1, 3), (5, 12), (8, 8)])
def test_append_sliding_window_closed_form(W, steps):
    n = 100
    idx = np.arange(n - W, n)
    K, V = _rows(W), _rows(W, base=1000)
    for t in range(steps):
        idx, K, V = oracle.append_token(idx, K, V, n + t, np.full(4, -t, np.float32),
                                        np.full(4, t, np.float32), cap=W + 50, limit=W)
        # the window holds exactly the W most recent positions
        assert sorted(idx.tolist()) == list(range(n - W + t + 1, n + t + 1))
        # token n + t' sits in slot t' mod W (slots recycle oldest first)
        assert idx[t % W] == n + t
        assert K[t % W][0] == -t and V[t % W][0] == t


def test_append_grows_to_capacity_then_replaces_oldest():
    idx, K, V = np.array([5, 9]), _rows(2), _rows(2, base=100)
    idx, K, V = oracle.append_token(idx, K, V, 20, np.ones(4), np.ones(4), cap=3, limit=0)
    assert idx.tolist() == [5, 9, 20] and K.shape == (3, 4)
    idx, K, V = oracle.append_token(idx, K, V, 21, np.full(4, 2.0), np.full(4, 3.0), cap=3, limit=0)
    assert idx.tolist() == [21, 9, 20]            # position 5 was the oldest
    assert K[0].tolist() == [2.0] * 4 and V[0].tolist() == [3.0] * 4


def test_append_skip_and_bounds():
    idx, K, V = np.array([3, 1, 2]), _rows(3), _rows(3)
    a = oracle.append_token(idx, K, V, 7, np.zeros(4), np.zeros(4), cap=10, limit=-1)
    assert a[0].tolist() == [3, 1, 2] and np.array_equal(a[1], K)
    # the window bound is capped by the capacity
    b = oracle.append_token(idx, K, V, 7, np.zeros(4), np.zeros(4), cap=3, limit=9)
    assert b[0].tolist() == [3, 7, 2]
    # a segment already above its bound keeps its length; the oldest row goes
    c = oracle.append_token(idx, K, V, 7, np.zeros(4), np.zeros(4), cap=10, limit=2)
    assert c[0].tolist() == [3, 7, 2]
    # zero capacity: nothing changes
    d = oracle.append_token(np.array([], np.int64), np.zeros((0, 4)), np.zeros((0, 4)), 7,
                            np.zeros(4), np.zeros(4), cap=0, limit=0)
    assert d[0].size == 0


# ---------------------------------------------------------------------------
# chunk selection with forced local chunks and a fixed chunk count
# (ChunkLLM page, §2.3 and the §3.2 operating points)
# ---------------------------------------------------------------------------

def _chunks_of(kept, ends):
    starts = np.concatenate([[0], ends[:-1]])
    return sorted({int(np.searchsorted(ends, p, side="right")) for p in kept}), starts


@pytest.mark.parametrize("seed", range(30))
def test_chunk_local_and_count_modes(seed):
    """Properties that define the two modes (no restated algorithm): local
    chunks always kept; the kept non-local chunks outrank every dropped one
    (score, then lower index); count mode keeps exactly k of them; token mode
    keeps the fewest that reach the target."""
    r = np.random.default_rng(500 + seed)
    nc = int(r.integers(1, 60))
    lens = r.integers(1, 9, size=nc)
    ends = np.cumsum(lens)
    cs = r.random(nc)
    if seed % 3 == 0:
        cs = np.round(cs, 1)                      # ties
    L = int(r.integers(0, nc + 2))
    k = int(r.integers(1, nc + 3))
    local = set(range(nc - min(L, nc), nc))
    others = [c for c in range(nc) if c not in local]

    def outranks(a, b):
        return cs[a] > cs[b] or (cs[a] == cs[b] and a < b)

    def check_ranked(kept_set):
        kept_o = [c for c in others if c in kept_set]
        drop_o = [c for c in others if c not in kept_set]
        assert all(outranks(a, b) for a in kept_o for b in drop_o)
        return kept_o

    for kept, mode in ((oracle.select_chunks(cs, ends, 0, local_chunks=L, top_chunks=k), "count"),
                       (None, "token")):
        if mode == "token":
            target = int(r.integers(0, ends[-1] + 5))
            kept = oracle.select_chunks(cs, ends, target, local_chunks=L)
        chunks, _ = _chunks_of(kept, ends)
        assert np.all(np.diff(kept) > 0)
        assert len(kept) == sum(int(lens[c]) for c in chunks)      # whole chunks only
        assert local <= set(chunks)
        kept_o = check_ranked(set(chunks))
        if mode == "count":
            assert len(kept_o) == min(k, len(others))
        else:
            tok = len(kept)
            assert tok >= min(target, int(ends[-1]))
            if kept_o:   # minimal: without the lowest-ranked extra chunk the target is missed
                worst = min(kept_o, key=lambda c: (cs[c], -c))
                assert tok - int(lens[worst]) < target


def test_chunk_local_zero_matches_plain():
    r = np.random.default_rng(9)
    ends = np.cumsum(r.integers(1, 6, size=40))
    cs = r.random(40)
    for target in (0, 1, 17, int(ends[-1])):
        assert np.array_equal(oracle.select_chunks(cs, ends, target),
                              oracle.select_chunks(cs, ends, target, local_chunks=0, top_chunks=0))


# ---------------------------------------------------------------------------
# attention rows, LMBA on them, attention loss (ZigZagkv Eq. 3, §5.5 Table 3)
# ---------------------------------------------------------------------------

def test_window_probabilities_rows_and_mask():
    r = np.random.default_rng(31)
    G, w, n, d, q0 = 2, 3, 40, 8, 30
    q, k = r.standard_normal((G, w, d)), r.standard_normal((n, d))
    P = oracle.window_probabilities(q, k, 0.3, q0)
    assert P.shape == (G * w, n)
    assert np.allclose(P.sum(axis=1), 1.0, atol=1e-13)
    for h in range(G):
        for i in range(w):
            assert np.all(P[h * w + i, q0 + i + 1:] == 0.0)          # causal
            assert np.all(P[h * w + i, :q0 + i + 1] > 0.0)


def test_lmba_zero_query_is_ceil_nine_tenths_of_visible():
    n, w, q0 = 53, 4, 40
    P = oracle.window_probabilities(np.zeros((1, w, 8)), np.ones((n, 8)), 1.0, q0)
    for i in range(w):
        vis = q0 + i + 1
        assert oracle.lmba_row(P[i]) == math.ceil(0.9 * vis)


def test_attention_loss_closed_forms():
    # two keys, logits a and 0: p = logistic(a); keeping key 0 loses max(0, 0.9 - p)
    for a in (-1.0, 0.5, 2.0, 4.0):
        q = np.array([[[a]]])
        k = np.array([[1.0], [0.0]])
        P = oracle.window_probabilities(q, k, 1.0, 1)
        p0 = 1.0 / (1.0 + math.exp(-a))
        assert abs(oracle.attention_loss(P, [0])[0] - max(0.0, 0.9 - p0)) < 1e-15
        assert oracle.attention_loss(P, [0, 1])[0] == 0.0
        assert abs(oracle.attention_loss(P, [])[0] - 0.9) < 1e-15


# ---------------------------------------------------------------------------
# bf16 rounding and pair-pruned RoPE (RAP §3, Eq. 5-10)
# ---------------------------------------------------------------------------

def test_round_bf16_hand_values_and_library():
    one = 1.0
    cases = [(one, 0x3F80), (-2.0, 0xC000),
             (one + 2.0 ** -8, 0x3F80),                # halfway 0x3F80 / 0x3F81: even wins
             (one + 3 * 2.0 ** -8, 0x3F82),            # halfway 0x3F81 / 0x3F82: even wins
             (one + 2.0 ** -8 + 2.0 ** -20, 0x3F81),   # just above halfway
             (-(one + 2.0 ** -8), 0xBF80), (0.0, 0x0000), (-0.0, 0x8000),
             (3.0e38, 0x7F62), (float("inf"), 0x7F80)]
    got = oracle.round_bf16(np.array([v for v, _ in cases], np.float32))
    assert [int(g) for g in got] == [h for _, h in cases]
    assert (int(oracle.round_bf16(np.float32("nan"))) & 0x7FC0) == 0x7FC0
    # torch's float -> bfloat16 conversion rounds to nearest even as well
    import torch
    x = np.random.default_rng(7).standard_normal(20000).astype(np.float32) * np.float32(50.0)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_bf16(x), ref)


def _rope_rows(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(2.0)
    return oracle.round_bf16(x) if dtype == "bf16" else x


def _as_f32(x, dtype):
    return (np.asarray(x).astype(np.uint32) << 16).view(np.float32) if dtype == "bf16" else x


def test_rope_table_is_the_rope_formula():
    import kvsynth
    t = kvsynth.rope_table(300, 64)
    for pos, p in [(0, 0), (1, 0), (1, 63), (257, 5), (299, 31), (123, 40)]:
        ang = pos * math.exp(-p / 64 * math.log(10000.0))
        assert t[pos, p, 0] == np.float32(math.cos(ang))
        assert t[pos, p, 1] == np.float32(math.sin(ang))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_rope_position_zero_is_identity(dtype):
    import kvsynth
    r = np.random.default_rng(3)
    x = _rope_rows(r, (5, 88), dtype)
    pairs = np.sort(r.choice(64, 44, replace=False))
    out = oracle.rope_pairs(x, np.zeros(5, np.int64), kvsynth.rope_table(4, 64), pairs, dtype)
    assert np.array_equal(np.asarray(out).view(np.uint8), np.asarray(x).view(np.uint8))


def test_rope_matches_textbook_rotation():
    """Identity pair list on a full 128-dim head equals the half-split rotation
    by angle t * 10000^(-2p/128) computed in float64 from the formula."""
    import kvsynth
    r = np.random.default_rng(4)
    x = r.standard_normal((6, 128)).astype(np.float32)
    pos = np.array([0, 1, 17, 4095, 30000, 32767])
    out = oracle.rope_pairs(x, pos, kvsynth.rope_table(32768, 64), np.arange(64), "fp32")
    p = np.arange(64)
    ang = pos[:, None] * np.power(10000.0, -2.0 * p / 128.0)[None, :]
    a, b = x[:, :64].astype(np.float64), x[:, 64:].astype(np.float64)
    want = np.concatenate([a * np.cos(ang) - b * np.sin(ang), a * np.sin(ang) + b * np.cos(ang)], 1)
    assert np.max(np.abs(out - want)) <= 2e-6 * np.max(np.abs(x))
    # the sign convention: pair 0 at a quarter turn maps (1, 0) to (0, 1)
    quarter = np.zeros((2, 1, 2), np.float32)
    quarter[1, 0] = (0.0, 1.0)
    y = oracle.rope_pairs(np.array([[1.0, 0.0]], np.float32), np.array([1]), quarter, [0], "fp32")
    assert np.array_equal(y, np.array([[0.0, 1.0]], np.float32))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_rope_commutes_with_pair_pruning(dtype):
    """RAP's absorption identity: rotating the full head and then keeping pairs P
    equals keeping P and rotating each kept pair with its own frequency."""
    import kvsynth
    r = np.random.default_rng(5)
    x = _rope_rows(r, (7, 128), dtype)
    pos = r.integers(0, 5000, 7)
    tab = kvsynth.rope_table(5000, 64)
    P = np.sort(r.choice(64, 44, replace=False))
    full = oracle.rope_pairs(x, pos, tab, np.arange(64), dtype)
    keep = lambda z: np.concatenate([z[:, P], z[:, P + 64]], axis=1)
    assert np.array_equal(keep(full), oracle.rope_pairs(keep(x), pos, tab, P, dtype))


def test_rope_preserves_pair_norms_and_relative_position():
    import kvsynth
    r = np.random.default_rng(6)
    tab = kvsynth.rope_table(9000, 64)
    P = np.sort(r.choice(64, 44, replace=False))
    q, k = r.standard_normal((2, 88)).astype(np.float32)
    rq = oracle.rope_pairs(q[None], np.array([700]), tab, P, "fp32")[0].astype(np.float64)
    n0 = q[:44].astype(np.float64) ** 2 + q[44:].astype(np.float64) ** 2
    n1 = rq[:44] ** 2 + rq[44:] ** 2
    assert np.max(np.abs(n1 - n0) / n0) < 2e-6
    # the attention logit depends on the positions only through their difference
    def logit(m, j):
        a = oracle.rope_pairs(q[None], np.array([m]), tab, P, "fp32")[0].astype(np.float64)
        b = oracle.rope_pairs(k[None], np.array([j]), tab, P, "fp32")[0].astype(np.float64)
        return float(a @ b)
    for m, j, dlt in [(500, 20, 300), (4000, 3999, 4000), (100, 100, 8000)]:
        assert abs(logit(m, j) - logit(m + dlt, j + dlt)) < 1e-4 * (np.linalg.norm(q) * np.linalg.norm(k))


# ---------------------------------------------------------------------------
# ChunkLLM layer-wise voting (CK §2.3; the rule is only described in words)
# ---------------------------------------------------------------------------

def _voted_chunks(layer_scores, k, local, ends):
    toks = oracle.vote_chunks(layer_scores, k, ends, local)
    return sorted(set(np.searchsorted(ends, toks, side="right").tolist()))


def test_vote_hand_worked():
    # three layers, six one-token chunks, top-2 per layer:
    #   layer 0 votes {3, 1}, layer 1 {2, 3}, layer 2 {3, 0}: chunk 3 has 3 votes,
    #   chunks 0, 1, 2 one each; summed attention 1.0, 0.8, 1.1 -> chunk 2 joins
    s = [[0.1, 0.5, 0.2, 0.9, 0.0, 0.0],
         [0.3, 0.1, 0.8, 0.7, 0.0, 0.1],
         [0.6, 0.2, 0.1, 0.65, 0.05, 0.0]]
    ends = np.arange(1, 7)
    votes, total = oracle.chunk_votes(s, 2)
    assert votes.tolist() == [1, 1, 1, 3, 0, 0]
    assert np.allclose(total, [1.0, 0.8, 1.1, 2.25, 0.05, 0.1], rtol=0, atol=1e-15)
    assert _voted_chunks(s, 2, 0, ends) == [2, 3]
    assert _voted_chunks(s, 2, 1, ends) == [2, 3, 5]          # chunk 5 forced (local)
    assert _voted_chunks(s, 1, 0, ends) == [3]
    # chunk 3 forced as a local chunk: the two best others are then 2 and 0
    assert _voted_chunks(s, 2, 3, ends) == [0, 2, 3, 4, 5]


def test_vote_counts_beat_summed_attention():
    # top-1 per layer: layer 0 votes chunk 1 (0.95), layers 1 and 2 vote chunk 0
    # (0.30 against 0.29).  Chunk 1 has the larger summed attention (1.53 vs
    # 0.60) but one vote; chunk 0 has two and is kept.
    s = [[0.00, 0.95, 0.05, 0.00],
         [0.30, 0.29, 0.21, 0.20],
         [0.30, 0.29, 0.21, 0.20]]
    ends = np.array([1, 2, 3, 4])
    assert _voted_chunks(s, 1, 0, ends) == [0]
    assert _voted_chunks(s, 2, 0, ends) == [0, 1]


def _near_tie_layers(b_sum_rel):
    # Six layers, top-2 per layer, five chunks.  Chunk 0 is every layer's best
    # (six votes).  Layers 0-2 also vote chunk 1 and layers 3-5 chunk 2, so
    # both have three votes and compete for the one slot left; chunk 2's
    # summed attention is (1 + b_sum_rel) times chunk 1's (0.0045).  Chunks 3
    # and 4 get no votes.
    s = np.full((6, 5), 0.0002)
    s[:, 0] = 0.01
    s[:3, 1], s[3:, 1] = 0.001, 0.0005
    s[:3, 2], s[3:, 2] = 0.0005, 0.001 + 0.0045 * b_sum_rel / 3
    return s


def test_vote_near_tie_in_summed_attention_goes_to_the_larger():
    # Relative differences of 1e-4 and 2e-5 are outside the 1e-5 tie band, so
    # the larger sum (chunk 2, the higher index) must win; at 2e-6 the rule
    # still orders them exactly.  (One fp32 key votes + 0.5 * sum / (L * G),
    # G = 4, rounds chunks 1 and 2 to the same value at these magnitudes and
    # would keep chunk 1.)
    ends = np.arange(1, 6)
    for rel in (1e-4, 2e-5, 2e-6):
        s = _near_tie_layers(rel)
        votes, total = oracle.chunk_votes(s, 2)
        assert votes.tolist() == [6, 3, 3, 0, 0]
        assert total[2] > total[1]
        assert _voted_chunks(s, 2, 0, ends) == [0, 2]
        # the mirror image: the larger sum on the lower index
        m = s.copy()
        m[:, [1, 2]] = s[:, [2, 1]]
        assert _voted_chunks(m, 2, 0, ends) == [0, 1]
    # exact ties in votes and in summed attention go to the lower index
    s = _near_tie_layers(0.0)
    s[:3, 2], s[3:, 2] = 0.0005, 0.001
    assert _voted_chunks(s, 2, 0, ends) == [0, 1]


def test_vote_single_layer_is_its_own_top_k():
    r = np.random.default_rng(12)
    ends = np.cumsum(r.integers(1, 9, 200))
    for k, local in [(10, 0), (17, 3), (1, 5)]:
        sc = r.random(200).astype(np.float32)
        # one layer: the ballot is the layer's top k over all chunks, and the
        # kept set is the locals plus the k best other chunks by score
        want = oracle.select_chunks(sc.astype(np.float64), ends, 0, local, k)
        votes, _ = oracle.chunk_votes(sc[None], k)
        if local == 0:
            assert np.array_equal(np.flatnonzero(votes), np.sort(oracle.select_topb(sc, k)))
        got = oracle.vote_chunks(sc[None], k, ends, local)
        assert np.array_equal(got, want)
        # identical layers vote as one
        got3 = oracle.vote_chunks(np.stack([sc] * 3), k, ends, local)
        assert np.array_equal(got3, want)


def test_vote_against_rank_counting():
    """The vote written a second way, by counting ranks instead of sorting: a
    chunk is on layer l's ballot iff fewer than k chunks beat it there (higher
    score, or equal score and lower index), and a non-local chunk is kept iff
    fewer than k other non-local chunks beat it on (votes, summed attention,
    lower index).  Random layers with planted exact ties in scores and in
    summed attention."""
    r = np.random.default_rng(13)
    for trial in range(60):
        L = int(r.integers(1, 7))
        nc = int(r.integers(1, 40))
        k = int(r.integers(1, nc + 3))
        local = int(r.integers(0, 4))
        sc = r.integers(0, 6, (L, nc)).astype(np.float64) / 8.0   # many exact ties
        if trial % 3 == 0:
            sc = r.random((L, nc))
        ends = np.arange(1, nc + 1)
        votes = np.zeros(nc, np.int64)
        for l in range(L):
            for c in range(nc):
                beat = sum(1 for j in range(nc)
                           if sc[l, j] > sc[l, c] or (sc[l, j] == sc[l, c] and j < c))
                votes[c] += beat < k
        tot = [sum(sorted(sc[:, c])) for c in range(nc)]   # exact: multiples of 1/8
        nl = nc - min(local, nc)

        def beats(j, c):
            return (votes[j], tot[j], -j) > (votes[c], tot[c], -c)
        want = [c for c in range(nc)
                if c >= nl or sum(1 for j in range(nl) if j != c and beats(j, c)) < k]
        got_votes, _ = oracle.chunk_votes(sc, k)
        assert np.array_equal(got_votes, votes), trial
        assert _voted_chunks(sc, k, local, ends) == want, trial


def test_score_c0_against_plain_loops():
    """A guard against array-broadcasting slips: the C0 window score written as
    plain loops over heads, window rows, keys and dimensions (math.exp, fsum)
    equals the vectorised oracle on one C0 segment."""
    import kvsynth
    cfg = kvsynth.get_config(0)
    x = kvsynth.segment_inputs(cfg, 0, 0, 1)
    q = oracle.to_f64(x["q_win"])          # [G][w][d]
    k = oracle.to_f64(x["K"])              # [n][d]
    G, w, d = q.shape
    n = k.shape[0]
    q0 = n - w
    kl, ql = k.tolist(), q.tolist()
    s = [0.0] * n
    for h in range(G):
        for i in range(w):
            vis = q0 + i + 1
            logits = [cfg.scale * math.fsum(ql[h][i][c] * kl[j][c] for c in range(d))
                      for j in range(vis)]
            m = max(logits)
            e = [math.exp(v - m) for v in logits]
            z = math.fsum(e)
            for j in range(vis):
                s[j] += e[j] / z
    want = oracle.window_scores(q, k, cfg.scale, q0)
    assert np.max(np.abs(np.array(s) - want)) < 1e-12
