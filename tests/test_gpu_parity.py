"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Every case prints its name before touching the GPU.  Sizes: the small
configurations in full; reduced variants (ragged n, several tiles); and
full-size layers in the launch configuration the benchmark times, checked on
sampled segments the oracle recomputes one by one.
"""
import math
import sys

import numpy as np
import pytest

import kvsynth
import oracle
from tests import parity_util as pu

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def kv():
    import torch
    import sparse_decode_attention_window_amd as kvsel
    from sparse_decode_attention_window_amd import pipeline
    assert torch.cuda.is_available()
    kvsel.lib()  # raises if the library is missing: no silent fallback
    return kvsel, pipeline, torch


def _run(kv, cfg, layer=0, budget=None):
    kvsel, pipeline, torch = kv
    inputs = kvsynth.layer_inputs(cfg, layer)
    run = pipeline.build_layer(cfg, inputs, budget=budget)
    run.run()
    torch.cuda.synchronize()
    return inputs, run


def _host(run):
    h = {
        "seg_off": pu.to_host(run.seg_off), "seg_len": pu.to_host(run.seg_len),
        "idx": pu.to_host(run.idx), "k_c": pu.to_host(run.k_c), "v_c": pu.to_host(run.v_c),
        "out": pu.to_host(run.out),
    }
    h["scores"] = pu.to_host(run.scores) if run.scores is not None else None
    return h


def _check_segments(cfg, inputs, run, segs, budgets=None, layer=0, local=0, top=0):
    h = _host(run)
    G, w, d = cfg.G, cfg.w, cfg.d
    stats = {"score_rel": 0.0, "out_abs": 0.0}
    for s in segs:
        b, kvh = divmod(s, cfg.hkv)
        what = f"{cfg.name} layer {layer} seg {s}"
        K, V = inputs["K"][b, kvh], inputs["V"][b, kvh]
        off, ln = int(h["seg_off"][s]), int(h["seg_len"][s])
        idx = h["idx"][off:off + ln].astype(np.int64)
        if cfg.mode == "topb":
            n = cfg.n
            s_gpu = h["scores"][s * n:(s + 1) * n]
            s_ref = oracle.window_scores(oracle.to_f64(inputs["q_win"][b, kvh * G:(kvh + 1) * G]),
                                         oracle.to_f64(K), cfg.scale, n - w)
            stats["score_rel"] = max(stats["score_rel"],
                                     pu.check_scores(s_gpu, s_ref, G * w, what))
            B = int(budgets[s]) if budgets is not None else cfg.budget
            pu.check_topb_selection(idx, s_gpu, s_ref, B, what)
        elif cfg.mode == "chunk":
            ends = inputs["chunk_end"][b]
            nc = ends.size
            cs_gpu = h["scores"][s * nc:(s + 1) * nc]
            cs_ref = oracle.window_scores(oracle.to_f64(inputs["chunk_q"][b, kvh * G:(kvh + 1) * G]),
                                          oracle.to_f64(inputs["chunk_keys"][b, kvh]), cfg.scale,
                                          nc - 1)
            stats["score_rel"] = max(stats["score_rel"], pu.check_scores(cs_gpu, cs_ref, G, what))
            pu.check_chunk_selection(idx, cs_gpu, cs_ref, ends, cfg.keep_tokens, what, local, top)
        else:
            want = oracle.select_policy(int(inputs["head_kind"][kvh]), cfg.n, cfg.local_window,
                                        inputs["special_pos"][b])
            assert np.array_equal(idx, want), f"{what}: policy selection differs"
        pu.check_compact(h["k_c"][off:off + ln], h["v_c"][off:off + ln], K, V, idx, what)
        out = h["out"][b, kvh * G:(kvh + 1) * G]
        stats["out_abs"] = max(stats["out_abs"],
                               pu.check_decode(out, inputs["q_dec"][b, kvh * G:(kvh + 1) * G], K, V,
                                               idx, cfg.scale, cfg.dtype, what))
    print(f"  {cfg.name}: max score rel err {stats['score_rel']:.2e}, "
          f"max decode abs err {stats['out_abs']:.2e}", flush=True)
    return h


# ---------------------------------------------------------------------------
# whole configurations
# ---------------------------------------------------------------------------

def test_c0_tiny_fp32_full(kv):
    cfg = kvsynth.get_config(0)
    _say(cfg.name)
    inputs, run = _run(kv, cfg)
    _check_segments(cfg, inputs, run, range(cfg.batch * cfg.hkv))


def test_c1_llama_layer_full(kv):
    cfg = kvsynth.get_config(1)
    _say(cfg.name)
    inputs, run = _run(kv, cfg)
    _check_segments(cfg, inputs, run, range(cfg.batch * cfg.hkv))


def test_eight_head_groups_end_to_end(kv):
    """C1's layer with 64 query heads over 8 KV heads (G = 8: 256 window rows
    per KV head, the LDS-staged score passes; the decode's largest head
    group) and a ragged n: score, select, compact and decode of every segment
    against the oracle."""
    cfg = kvsynth.get_config(1, hq=64, n=3000 + 37, budget=333)
    assert cfg.G == 8 and cfg.G * cfg.w == 256
    _say(cfg.name, "G", cfg.G, "n", cfg.n)
    inputs, run = _run(kv, cfg)
    _check_segments(cfg, inputs, run, range(cfg.batch * cfg.hkv))


@pytest.mark.parametrize("layer", [0, 9])
def test_c2_reduced_ragged(kv, layer):
    cfg = kvsynth.get_config(2, batch=2, n=5000 + 77)
    _say(cfg.name, "reduced n", cfg.n, "layer", layer)
    bl = pu.zigzag_layer_budgets(cfg)[layer]
    inputs, run = _run(kv, cfg, layer, budget=bl)
    _check_segments(cfg, inputs, run, range(cfg.batch * cfg.hkv),
                    budgets=np.full(cfg.batch * cfg.hkv, bl), layer=layer)


def test_max_segments_per_call(kv):
    """The largest call the boundary accepts: batch * Hkv = 2048 segments (C0's
    shapes at batch 1024, n = 160 so every segment ends in a partial tile)
    through score, select, compact and decode; sampled segments against the
    oracle, every segment's length against its budget."""
    cfg = kvsynth.get_config(0, batch=1024, n=160, budget=40)
    S = cfg.batch * cfg.hkv
    assert S == 2048
    _say(cfg.name, "segments", S)
    inputs, run = _run(kv, cfg)
    h = _check_segments(cfg, inputs, run, [0, 1, 777, 1500, S - 2, S - 1])
    assert np.all(h["seg_len"] == cfg.budget)
    sc = h["scores"].reshape(S, cfg.n).astype(np.float64)
    assert np.all(np.abs(sc.sum(1) - cfg.G * cfg.w) < 1e-3)


def test_c2_full_layer_sampled(kv):
    cfg = kvsynth.get_config(2)
    layer = 3
    _say(cfg.name, "full layer", layer)
    bl = pu.zigzag_layer_budgets(cfg)[layer]
    inputs, run = _run(kv, cfg, layer, budget=bl)
    h = _check_segments(cfg, inputs, run, [0, 13, 31], budgets=np.full(32, bl), layer=layer)
    # every segment: exact budget, mass G*w
    assert np.all(h["seg_len"] == bl)
    sc = h["scores"].reshape(32, cfg.n).astype(np.float64)
    assert np.all(np.abs(sc.sum(1) - cfg.G * cfg.w) < 1e-3)


def test_c3_reduced(kv):
    cfg = kvsynth.get_config(3, batch=2, n=3000 + 5)
    _say(cfg.name, "reduced n", cfg.n)
    inputs, run = _run(kv, cfg)
    _check_segments(cfg, inputs, run, range(cfg.batch * cfg.hkv))


def test_c3_full_sampled(kv):
    cfg = kvsynth.get_config(3)
    _say(cfg.name, "full")
    inputs, run = _run(kv, cfg)
    kinds = inputs["head_kind"]
    segs = [7 * cfg.hkv + int(np.nonzero(kinds == k)[0][0]) for k in (0, 1, 2)]
    h = _check_segments(cfg, inputs, run, segs)
    assert int(h["seg_len"].sum()) == 8 * 73648


def test_c4_reduced(kv):
    cfg = kvsynth.get_config(4, n=20000 + 3)
    _say(cfg.name, "reduced n", cfg.n)
    inputs, run = _run(kv, cfg)
    _check_segments(cfg, inputs, run, range(cfg.batch * cfg.hkv))


@pytest.mark.parametrize("local,top,keep_frac", [(16, 256, 0.48), (15, 0, 0.45)])
def test_c4_chunk_operating_points(kv, local, top, keep_frac):
    """ChunkLLM's two operating points on a reduced C4 layer: 16 forced local
    chunks + the 256 best others; 15 local chunks + a 45 % token target."""
    kvsel, pipeline, torch = kv
    cfg = kvsynth.get_config(4, n=20000 + 3, keep_frac=keep_frac)
    _say(cfg.name, "reduced, local", local, "top", top, "keep", cfg.keep_tokens)
    inputs = kvsynth.layer_inputs(cfg, 0)
    run = pipeline.build_layer(cfg, inputs, local_chunks=local, top_chunks=top)
    run.run()
    torch.cuda.synchronize()
    _check_segments(cfg, inputs, run, range(cfg.batch * cfg.hkv), local=local, top=top)


def test_c4_full_sampled(kv):
    cfg = kvsynth.get_config(4)
    _say(cfg.name, "full")
    inputs, run = _run(kv, cfg)
    h = _check_segments(cfg, inputs, run, [0, 5])
    assert np.all(h["seg_len"] >= cfg.keep_tokens)


def test_determinism_c1(kv):
    cfg = kvsynth.get_config(1, n=3001)
    _say(cfg.name, "determinism")
    inputs, run = _run(kv, cfg)
    a = _host(run)
    run.run()
    kv[2].cuda.synchronize()
    b = _host(run)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


# ---------------------------------------------------------------------------
# single kernels on crafted inputs
# ---------------------------------------------------------------------------

def _select_topb(kv, scores: np.ndarray, budgets, hkv=1):
    kvsel, pipeline, torch = kv
    S, n = scores.shape
    shape = kvsel.make_shape(S // hkv, hkv, hkv, 64, n, "bf16", 1.0)
    bud = np.asarray(budgets, np.int32)
    cap = pipeline.capacities(kvsel.KVSEL_SEL_TOPB, S // hkv, hkv, n, budget=bud)
    off, r_cap = pipeline.offsets(cap)
    bt = pipeline.device_tensor(bud)
    st = pipeline.device_tensor(scores.astype(np.float32).ravel())
    ot = pipeline.device_tensor(off)
    lt = torch.empty(S, dtype=torch.int32, device="cuda")
    it = torch.full((max(r_cap, 1),), -7, dtype=torch.int32, device="cuda")
    kvsel.kvsel_select(shape, kvsel.select_params(kvsel.KVSEL_SEL_TOPB, budget=bt), st, ot, lt, it,
                       r_cap)
    torch.cuda.synchronize()
    lens, idx = pu.to_host(lt), pu.to_host(it)
    return [idx[off[s]:off[s] + lens[s]] for s in range(S)], lens


@pytest.mark.parametrize("n", [1, 37, 1000, 32768, 45000])
def test_select_topb_exact_with_ties(kv, n):
    _say("select topb n", n)
    r = np.random.default_rng(n)
    rows = [
        r.random(n).astype(np.float32),                         # distinct
        r.integers(0, 5, n).astype(np.float32),                 # heavy ties
        np.full(n, 0.25, np.float32),                           # all equal
        np.where(r.random(n) < 0.1, np.nan, r.random(n)).astype(np.float32),   # NaN
        np.where(r.random(n) < 0.5, -0.0, 0.0).astype(np.float32),             # +-0
        (r.standard_normal(n) * 1e-30).astype(np.float32),     # tiny, signed
    ]
    scores = np.stack(rows)
    budgets = [max(0, n // 5), n // 3, min(n, 7), n - 1 if n > 1 else 1, n + 5, 0]
    got, lens = _select_topb(kv, scores, budgets)
    for s in range(len(rows)):
        want = oracle.select_topb(scores[s].astype(np.float64), budgets[s])
        assert lens[s] == want.size, (s, lens[s], want.size)
        assert np.array_equal(got[s], want), f"row {s}"


@pytest.mark.parametrize("n,count", [(5000, 600), (120000, 7000), (240000, 14000)])
def test_select_chunk_exact(kv, n, count):
    """Crafted chunk selections (ties, all-equal scores, forced local chunks,
    fixed counts, targets of 0 and past n) at about 250, 6 000 and 12 000
    chunks: one, eight and sixteen chunks per thread (the gathered write of
    the kept positions up to 8192 chunks, the per-chunk loop above)."""
    kvsel, pipeline, torch = kv
    _say("select chunk crafted", n, count)
    r = np.random.default_rng(7 + n)
    lens_c = r.geometric(1 / 20, size=count)
    ends = np.minimum(np.cumsum(lens_c), n)
    ends = np.unique(ends)
    if ends[-1] != n:
        ends = np.append(ends, n)
    nc = ends.size
    hkv = 3
    cs = np.stack([r.random(nc), r.integers(0, 3, nc), np.full(nc, 1.0)]).astype(np.float32)
    cases = [(keep, 0, 0) for keep in [1, 777, 2400, n // 2, n, n + 10, 0]]
    cases += [(777, 5, 0), (0, 16, 0), (n, 3, 0), (0, 16, 50), (0, 0, 1), (0, 3, nc), (0, nc + 4, 2)]
    for keep, local, top in cases:
        shape = kvsel.make_shape(1, hkv, hkv, 64, n, "bf16", 1.0)
        maxc = int(np.diff(np.concatenate([[0], ends])).max())
        cap = pipeline.capacities(kvsel.KVSEL_SEL_CHUNK, 1, hkv, n, keep_tokens=keep, max_chunk=maxc,
                                  local_chunks=local, top_chunks=top)
        off, r_cap = pipeline.offsets(cap)
        et = pipeline.device_tensor(ends[None, :].astype(np.int64))
        st = pipeline.device_tensor(cs.ravel())
        ot = pipeline.device_tensor(off)
        lt = torch.empty(hkv, dtype=torch.int32, device="cuda")
        it = torch.full((max(r_cap, 1),), -7, dtype=torch.int32, device="cuda")
        p = kvsel.select_params(kvsel.KVSEL_SEL_CHUNK, n_chunks=nc, chunk_end=et, keep_tokens=keep,
                                local_chunks=local, top_chunks=top)
        kvsel.kvsel_select(shape, p, st, ot, lt, it, r_cap)
        torch.cuda.synchronize()
        ln, ix = pu.to_host(lt), pu.to_host(it)
        for s in range(hkv):
            want = oracle.select_chunks(cs[s].astype(np.float64), ends, keep, local, top)
            assert ln[s] == want.size, (keep, local, top, s)
            assert np.array_equal(ix[off[s]:off[s] + ln[s]], want), (keep, local, top, s)
            # nothing written past the kept positions (the segment's workgroups each
            # write one slice of them)
            end = int(off[s + 1]) if s + 1 < hkv else r_cap
            assert np.all(ix[off[s] + ln[s]:end] == -7), (keep, local, top, s)


def test_compact_gaps_empty_and_bad_indices(kv):
    kvsel, pipeline, torch = kv
    _say("compact crafted")
    r = np.random.default_rng(11)
    B, hkv, n, d = 2, 3, 700, 88
    K = r.integers(0, 65535, size=(B, hkv, n, d), dtype=np.uint16)
    V = r.integers(0, 65535, size=(B, hkv, n, d), dtype=np.uint16)
    lens = np.array([0, 5, 700, 1, 33, 0], np.int32)
    off = np.array([0, 3, 20, 730, 740, 800], np.int64)    # gaps between segments
    r_cap = 790                                            # clips segment 4 (740 + 33 > 790? no)
    idx = np.full(r_cap, -1, np.int32)
    for s in range(6):
        m = min(lens[s], r_cap - off[s]) if off[s] < r_cap else 0
        idx[off[s]:off[s] + m] = np.sort(r.choice(n, size=m, replace=False))
    idx[25] = n + 3          # out of range -> zero row
    idx[26] = -5
    shape = kvsel.make_shape(B, hkv, hkv, d, n, "bf16", 1.0)
    kc = torch.full((r_cap, d), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vc = torch.full((r_cap, d), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    kt, vt = pipeline.device_tensor(K), pipeline.device_tensor(V)
    kvsel.kvsel_compact(shape, kt, vt, pipeline.device_tensor(off), pipeline.device_tensor(lens),
                        pipeline.device_tensor(idx), kc, vc, r_cap)
    torch.cuda.synchronize()
    kch, vch = pu.to_host(kc), pu.to_host(vc)
    for s in range(6):
        b, h = divmod(s, hkv)
        m = max(0, min(lens[s], r_cap - off[s]))
        for rr in range(m):
            row = off[s] + rr
            j = idx[row]
            if 0 <= j < n:
                assert np.array_equal(kch[row], K[b, h, j]) and np.array_equal(vch[row], V[b, h, j])
            else:
                assert not kch[row].any() and not vch[row].any()
    # rows outside every segment are untouched
    assert np.all(kch[0:3] == 7) and np.all(kch[733:740] == 7)


@pytest.mark.parametrize("dtype,d,G", [("bf16", 128, 4), ("bf16", 88, 4), ("bf16", 64, 2),
                                       ("fp32", 64, 2), ("fp32", 128, 3), ("bf16", 128, 1),
                                       ("fp32", 88, 4), ("bf16", 128, 8), ("bf16", 88, 6),
                                       ("fp32", 64, 5), ("fp32", 128, 8), ("bf16", 64, 7)])
def test_decode_ragged_segments(kv, dtype, d, G):
    kvsel, pipeline, torch = kv
    _say("decode", dtype, d, G)
    r = np.random.default_rng(d * 10 + G)
    B, hkv = 2, 2
    S = B * hkv
    lens = np.array([0, 1, 257, 1000], np.int32)[:S]
    off, r_cap = pipeline.offsets(lens.astype(np.int64) + 3)   # 3 spare rows per segment
    Kc = r.standard_normal((r_cap, d)).astype(np.float32)
    Vc = r.standard_normal((r_cap, d)).astype(np.float32)
    q = (2 * r.standard_normal((B, hkv * G, d))).astype(np.float32)
    store = (lambda x: kvsynth.f32_to_bf16_bits(x)) if dtype == "bf16" else (lambda x: x)
    Kc, Vc, q = store(Kc), store(Vc), store(q)
    shape = kvsel.make_shape(B, hkv * G, hkv, d, 1000, dtype, 1 / math.sqrt(d))
    out = torch.empty((B, hkv * G, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(kvsel.kvsel_decode_workspace(shape, r_cap), dtype=torch.uint8, device="cuda")
    kvsel.kvsel_decode_attn(shape, pipeline.device_tensor(q), pipeline.device_tensor(Kc),
                            pipeline.device_tensor(Vc), pipeline.device_tensor(off),
                            pipeline.device_tensor(lens), r_cap, out, ws)
    torch.cuda.synchronize()
    o = pu.to_host(out)
    for s in range(S):
        b, h = divmod(s, hkv)
        rows = np.arange(off[s], off[s] + lens[s])
        for g in range(G):
            ref = oracle.decode_attention(oracle.to_f64(q[b, h * G + g]), oracle.to_f64(Kc[rows]),
                                          oracle.to_f64(Vc[rows]), 1 / math.sqrt(d))
            err = np.max(np.abs(o[b, h * G + g] - ref))
            assert err <= pu.OUT_ATOL[dtype], (s, g, err)
            if lens[s] == 0:
                assert not o[b, h * G + g].any()


@pytest.mark.parametrize("dtype,d,G,w,n,q_pos0", [
    ("bf16", 128, 4, 32, 1500, 1468), ("bf16", 128, 4, 32, 700, 10**9),
    ("fp32", 64, 2, 8, 513, 505), ("bf16", 64, 4, 1, 999, 998), ("bf16", 88, 4, 5, 2049, 100),
    ("fp32", 128, 1, 3, 90, 87), ("bf16", 128, 8, 32, 600, 568)])
def test_score_shapes(kv, dtype, d, G, w, n, q_pos0):
    kvsel, pipeline, torch = kv
    _say("score", dtype, d, G, w, n, q_pos0)
    r = np.random.default_rng(n + d)
    B, hkv = 1, 2
    q = (r.standard_normal((B, hkv * G, w, d)) * 1.5).astype(np.float32)
    Kf = r.standard_normal((B, hkv, n, d)).astype(np.float32)
    store = (lambda x: kvsynth.f32_to_bf16_bits(x)) if dtype == "bf16" else (lambda x: x)
    q, Kf = store(q), store(Kf)
    shape = kvsel.make_shape(B, hkv * G, hkv, d, n, dtype, 1 / math.sqrt(d))
    sc = torch.empty(B * hkv * n, dtype=torch.float32, device="cuda")
    ws = torch.empty(kvsel.kvsel_score_workspace(shape, w), dtype=torch.uint8, device="cuda")
    kvsel.kvsel_score(shape, w, q_pos0, pipeline.device_tensor(q), pipeline.device_tensor(Kf), sc, ws)
    torch.cuda.synchronize()
    s_gpu = pu.to_host(sc).reshape(B * hkv, n)
    for s in range(B * hkv):
        b, h = divmod(s, hkv)
        ref = oracle.window_scores(oracle.to_f64(q[b, h * G:(h + 1) * G]), oracle.to_f64(Kf[b, h]),
                                   1 / math.sqrt(d), q_pos0)
        pu.check_scores(s_gpu[s], ref, G * w, f"score seg {s}")


def _drifting_logits(r, n_keys, d, n_q, slope):
    """Keys and queries along one shared direction u, so that scale * q.k is
    about a_j = slope * 10 * (2 j / (n_keys - 1) - 1) plus noise: the logits
    drift by ~30 log2 units along the sequence (rising for slope > 0, falling
    for slope < 0), so a running max changes many times (or never after the
    first keys), and the per-tile and per-item rescaling of the online softmax
    spans factors down to ~2^-30."""
    u = r.standard_normal(d)
    u /= np.linalg.norm(u)
    a = slope * 10.0 * np.linspace(-1.0, 1.0, n_keys)
    keys = (a[:, None] * u[None, :] + 0.3 * r.standard_normal((n_keys, d))).astype(np.float32)
    qs = (math.sqrt(d) * u[None, :] + 0.3 * r.standard_normal((n_q, d))).astype(np.float32)
    return keys, qs


@pytest.mark.parametrize("dtype,d,G,w,n,slope", [("fp32", 64, 2, 8, 3000, 1.0),
                                                 ("fp32", 128, 4, 16, 5000, -1.0),
                                                 ("bf16", 128, 4, 32, 4100, 1.0),
                                                 ("bf16", 88, 4, 32, 2600, -1.0)])
def test_score_drifting_logits(kv, dtype, d, G, w, n, slope):
    """Online-softmax statistics under logits that rise or fall by ~30 log2
    units along the keys (window queries at the end, causal)."""
    kvsel, pipeline, torch = kv
    _say("score drift", dtype, d, G, w, n, slope)
    r = np.random.default_rng(n + d + int(slope > 0))
    B, hkv = 1, 2
    q = np.empty((B, hkv * G, w, d), np.float32)
    Kf = np.empty((B, hkv, n, d), np.float32)
    for h in range(hkv):
        keys, qs = _drifting_logits(r, n, d, G * w, slope)
        Kf[0, h] = keys
        q[0, h * G:(h + 1) * G] = qs.reshape(G, w, d)
    store = (lambda x: kvsynth.f32_to_bf16_bits(x)) if dtype == "bf16" else (lambda x: x)
    q, Kf = store(q), store(Kf)
    shape = kvsel.make_shape(B, hkv * G, hkv, d, n, dtype, 1 / math.sqrt(d))
    sc = torch.empty(B * hkv * n, dtype=torch.float32, device="cuda")
    ws = torch.empty(kvsel.kvsel_score_workspace(shape, w), dtype=torch.uint8, device="cuda")
    kvsel.kvsel_score(shape, w, n - w, pipeline.device_tensor(q), pipeline.device_tensor(Kf), sc,
                      ws)
    torch.cuda.synchronize()
    s_gpu = pu.to_host(sc).reshape(B * hkv, n)
    for s in range(B * hkv):
        ref = oracle.window_scores(oracle.to_f64(q[0, s * G:(s + 1) * G]), oracle.to_f64(Kf[0, s]),
                                   1 / math.sqrt(d), n - w)
        # the drift is real: most of the mass sits in one tenth of the keys
        end = ref[-n // 10:] if slope > 0 else ref[:n // 10]
        assert end.sum() > 0.8 * G * w
        pu.check_scores(s_gpu[s], ref, G * w, f"score drift seg {s}")


@pytest.mark.parametrize("dtype,d,G,w,n", [("bf16", 128, 4, 32, 6000), ("fp32", 64, 2, 8, 3000),
                                           ("bf16", 88, 4, 32, 2600)])
def test_score_late_spikes(kv, dtype, d, G, w, n):
    """Window statistics when a key far above the others appears after the
    first key block of a wavefront's run: 1 % of the keys carry a spike of
    8, 16, 23, 30 or 45 log2 units over a flat background, so some runs keep
    their first block's maximum as the reference (sums up to 2^23) and
    others exceed 2^24 and are summed again in the exact form."""
    kvsel, pipeline, torch = kv
    _say("score spikes", dtype, d, G, w, n)
    r = np.random.default_rng(7 * n + d)
    B, hkv = 1, 2
    q = np.empty((B, hkv * G, w, d), np.float32)
    Kf = np.empty((B, hkv, n, d), np.float32)
    for h in range(hkv):
        u = r.standard_normal(d)
        u /= np.linalg.norm(u)
        a = np.zeros(n)
        pos = r.choice(np.arange(1, n - w), size=max(4, n // 100), replace=False)
        a[pos] = r.choice([8.0, 16.0, 23.0, 30.0, 45.0], size=pos.size) / math.log2(math.e)
        Kf[0, h] = a[:, None] * u[None, :] + 0.3 * r.standard_normal((n, d))
        q[0, h * G:(h + 1) * G] = (math.sqrt(d) * u[None, :]
                                   + 0.3 * r.standard_normal((G * w, d))).reshape(G, w, d)
    store = (lambda x: kvsynth.f32_to_bf16_bits(x)) if dtype == "bf16" else (lambda x: x)
    q, Kf = store(q), store(Kf)
    shape = kvsel.make_shape(B, hkv * G, hkv, d, n, dtype, 1 / math.sqrt(d))
    sc = torch.empty(B * hkv * n, dtype=torch.float32, device="cuda")
    ws = torch.empty(kvsel.kvsel_score_workspace(shape, w), dtype=torch.uint8, device="cuda")
    kvsel.kvsel_score(shape, w, n - w, pipeline.device_tensor(q), pipeline.device_tensor(Kf), sc,
                      ws)
    torch.cuda.synchronize()
    s_gpu = pu.to_host(sc).reshape(B * hkv, n)
    for s in range(B * hkv):
        ref = oracle.window_scores(oracle.to_f64(q[0, s * G:(s + 1) * G]), oracle.to_f64(Kf[0, s]),
                                   1 / math.sqrt(d), n - w)
        pu.check_scores(s_gpu[s], ref, G * w, f"score spikes seg {s}")


@pytest.mark.parametrize("dtype,d,G,slope", [("fp32", 128, 4, 1.0), ("fp32", 64, 2, -1.0),
                                             ("bf16", 128, 4, -1.0), ("bf16", 88, 4, 1.0)])
def test_decode_drifting_logits(kv, dtype, d, G, slope):
    """Split-K decode where the logits rise or fall by ~30 log2 units along
    each segment, so its items' partial maxima differ by up to that much and
    the merge rescales them by factors down to ~2^-30."""
    kvsel, pipeline, torch = kv
    _say("decode drift", dtype, d, G, slope)
    r = np.random.default_rng(d * 10 + G + int(slope > 0))
    B, hkv = 1, 3
    S = B * hkv
    lens = np.array([20000, 7001, 333], np.int32)
    off, r_cap = pipeline.offsets(lens.astype(np.int64))
    Kc = np.empty((r_cap, d), np.float32)
    q = np.empty((B, hkv * G, d), np.float32)
    for s in range(S):
        keys, qs = _drifting_logits(r, int(lens[s]), d, G, slope)
        Kc[off[s]:off[s] + lens[s]] = keys
        q[0, s * G:(s + 1) * G] = qs
    Vc = r.standard_normal((r_cap, d)).astype(np.float32)
    store = (lambda x: kvsynth.f32_to_bf16_bits(x)) if dtype == "bf16" else (lambda x: x)
    Kc, Vc, q = store(Kc), store(Vc), store(q)
    shape = kvsel.make_shape(B, hkv * G, hkv, d, int(lens.max()), dtype, 1 / math.sqrt(d))
    out = torch.empty((B, hkv * G, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(kvsel.kvsel_decode_workspace(shape, r_cap), dtype=torch.uint8, device="cuda")
    kvsel.kvsel_decode_attn(shape, pipeline.device_tensor(q), pipeline.device_tensor(Kc),
                            pipeline.device_tensor(Vc), pipeline.device_tensor(off),
                            pipeline.device_tensor(lens), r_cap, out, ws)
    torch.cuda.synchronize()
    o = pu.to_host(out)
    for s in range(S):
        rows = np.arange(off[s], off[s] + lens[s])
        for g in range(G):
            ref = oracle.decode_attention(oracle.to_f64(q[0, s * G + g]), oracle.to_f64(Kc[rows]),
                                          oracle.to_f64(Vc[rows]), 1 / math.sqrt(d))
            err = np.max(np.abs(o[0, s * G + g] - ref))
            assert err <= pu.OUT_ATOL[dtype], (s, g, err)


@pytest.mark.parametrize("dtype,d,G", [("fp32", 128, 4), ("bf16", 128, 4), ("bf16", 88, 4),
                                       ("bf16", 128, 8)])
def test_decode_late_spikes(kv, dtype, d, G):
    """Split-K decode whose exponent reference is set by an ordinary bulk of
    keys (logits spread about 1.4 log2 units around zero) and then overtaken
    late in each segment: keys aligned with a query head lift its logit to
    7.5, 8.5, 14, 22 and 40 log2 units at positions past most of the
    segment's tiles, so a wavefront either keeps a reference that a logit
    passes by less than its margin or moves it (and rescales its sums) after
    many tiles."""
    kvsel, pipeline, torch = kv
    _say("decode spikes", dtype, d, G)
    r = np.random.default_rng(7000 + d + G)
    B, hkv = 1, 2
    S = B * hkv
    lens = np.array([9000, 2500], np.int32)
    off, r_cap = pipeline.offsets(lens.astype(np.int64))
    c = math.log2(math.e) / math.sqrt(d)             # log2 units per unit of q.k
    Kc = r.standard_normal((r_cap, d)).astype(np.float32)
    q = r.standard_normal((B, hkv * G, d)).astype(np.float32)
    for s in range(S):
        n = int(lens[s])
        for j, (frac, lift) in enumerate([(0.55, 7.5), (0.62, 8.5), (0.71, 14.0), (0.83, 22.0),
                                          (0.97, 40.0)]):
            h = (j % G)
            qh = q[0, s * G + h]
            Kc[off[s] + int(frac * n)] = qh * (lift / c / float(qh @ qh))
    Vc = r.standard_normal((r_cap, d)).astype(np.float32)
    store = (lambda x: kvsynth.f32_to_bf16_bits(x)) if dtype == "bf16" else (lambda x: x)
    Kc, Vc, q = store(Kc), store(Vc), store(q)
    shape = kvsel.make_shape(B, hkv * G, hkv, d, int(lens.max()), dtype, 1 / math.sqrt(d))
    out = torch.empty((B, hkv * G, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(kvsel.kvsel_decode_workspace(shape, r_cap), dtype=torch.uint8, device="cuda")
    kvsel.kvsel_decode_attn(shape, pipeline.device_tensor(q), pipeline.device_tensor(Kc),
                            pipeline.device_tensor(Vc), pipeline.device_tensor(off),
                            pipeline.device_tensor(lens), r_cap, out, ws)
    torch.cuda.synchronize()
    o = pu.to_host(out)
    worst = 0.0
    for s in range(S):
        rows = np.arange(off[s], off[s] + lens[s])
        for g in range(G):
            ref = oracle.decode_attention(oracle.to_f64(q[0, s * G + g]), oracle.to_f64(Kc[rows]),
                                          oracle.to_f64(Vc[rows]), 1 / math.sqrt(d))
            err = float(np.max(np.abs(o[0, s * G + g] - ref)))
            worst = max(worst, err)
            assert err <= pu.OUT_ATOL[dtype], (s, g, err)
    pu.record(f"decode_abs_{dtype}", worst)


# ---------------------------------------------------------------------------
# workspace state and graph replays
# ---------------------------------------------------------------------------

def test_decode_garbage_workspace(kv):
    """The decode scratch needs no initialisation: fill it with junk bytes."""
    kvsel, pipeline, torch = kv
    cfg = kvsynth.get_config(1, n=2500)
    _say(cfg.name, "decode with a junk-filled workspace")
    inputs, run = _run(kv, cfg)
    want = pu.to_host(run.out).copy()
    for fill in (0xFF, 0x01, 0x7F):
        run.ws_dec.fill_(fill)
        run.decode()
        torch.cuda.synchronize()
        assert np.array_equal(pu.to_host(run.out), want), hex(fill)


@pytest.mark.parametrize("cid", [1, 3, 4])
def test_graph_replays_match_eager(kv, cid):
    """Capture one layer (score, select, compact, decode) in a HIP graph; replay
    it several times with eager work in between; every replay must reproduce
    the eager results bit for bit."""
    kvsel, pipeline, torch = kv
    over = {1: dict(n=3000), 3: dict(batch=2, n=3000), 4: dict(n=9000)}[cid]
    cfg = kvsynth.get_config(cid, **over)
    _say(cfg.name, "graph replay")
    inputs, run = _run(kv, cfg)
    want = _host(run)
    other_inputs, other = _run(kv, kvsynth.get_config(1, n=1111))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.run()
    torch.cuda.synchronize()
    for rep in range(4):
        run.out.zero_()
        run.idx.fill_(-3)
        other.run()                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _host(run)
        for key in ("seg_off", "seg_len", "scores", "out"):
            if want[key] is not None:
                assert np.array_equal(got[key], want[key]), (rep, key)
        # packed rows: only each segment's written prefix is defined
        for s, (o, n_) in enumerate(zip(want["seg_off"], want["seg_len"])):
            for key in ("idx", "k_c", "v_c"):
                assert np.array_equal(got[key][o:o + n_], want[key][o:o + n_]), (rep, key, s)


# ---------------------------------------------------------------------------
# decode-time maintenance: append / sliding window (FastGen eviction rules)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d", [("fp32", 64), ("bf16", 88), ("bf16", 128)])
def test_append_steps_match_oracle(kv, dtype, d):
    """Six appends in a row on ragged segments with every kind of rule:
    skip, grow, grow into capacity, sliding windows (also already over the
    window); state compared bit for bit with the oracle after every step."""
    kvsel, pipeline, torch = kv
    rng = np.random.default_rng(7 + d)
    B, hkv, n = 3, 3, 500
    S = B * hkv
    _say("append", dtype, d)
    sdt = np.uint16 if dtype == "bf16" else np.float32

    def rows(k):
        x = rng.standard_normal((k, d)).astype(np.float32)
        return kvsynth.f32_to_bf16_bits(x) if dtype == "bf16" else x

    caps = np.array([0, 5, 9, 4, 12, 6, 3, 7, 10], np.int64)
    limits = np.array([0, 0, 3, -1, 4, 0, 1, 2, 5], np.int32)
    lens = np.array([0, 2, 3, 2, 6, 6, 0, 5, 1], np.int64)       # seg 4, 7: above the window
    gaps = np.array([1, 0, 2, 0, 3, 1, 0, 2, 1], np.int64)         # unused rows between segments
    off = np.zeros(S, np.int64)
    for s in range(1, S):
        off[s] = off[s - 1] + caps[s - 1] + gaps[s - 1]
    r_cap = int(off[-1] + caps[-1] + gaps[-1])
    idx_h = np.full(r_cap, -7, np.int32)
    kc_h = rows(r_cap)
    vc_h = rows(r_cap)
    segs = []
    for s in range(S):
        pos = rng.choice(n, size=lens[s], replace=False).astype(np.int64)
        idx_h[off[s]:off[s] + lens[s]] = pos
        segs.append([pos, kc_h[off[s]:off[s] + lens[s]].copy(), vc_h[off[s]:off[s] + lens[s]].copy()])
    shape = kvsel.make_shape(B, B * hkv, hkv, d, n, dtype, 0.125)
    dev = lambda a: pipeline.device_tensor(a)
    t_off, t_cap, t_lim = dev(off), dev(caps), dev(limits)
    t_len, t_idx = dev(lens.astype(np.int32)), dev(idx_h)
    t_kc, t_vc = dev(kc_h), dev(vc_h)
    for t in range(6):
        kn, vn = rows(S), rows(S)
        pos = n + t
        kvsel.kvsel_append(shape, dev(kn.reshape(B, hkv, d)), dev(vn.reshape(B, hkv, d)), pos,
                           t_off, t_cap, t_lim, t_len, t_idx, t_kc, t_vc, r_cap)
        torch.cuda.synchronize()
        g_len, g_idx = pu.to_host(t_len), pu.to_host(t_idx)
        g_kc, g_vc = pu.to_host(t_kc), pu.to_host(t_vc)
        for s in range(S):
            segs[s] = list(oracle.append_token(segs[s][0], segs[s][1], segs[s][2], pos, kn[s], vn[s],
                                               int(caps[s]), int(limits[s])))
            want_idx, want_k, want_v = segs[s]
            ln = int(g_len[s])
            what = f"append step {t} seg {s}"
            assert ln == want_idx.size, f"{what}: len {ln} != {want_idx.size}"
            o = int(off[s])
            assert np.array_equal(g_idx[o:o + ln], want_idx.astype(np.int32)), what
            assert np.array_equal(g_kc[o:o + ln], want_k), what
            assert np.array_equal(g_vc[o:o + ln], want_v), what
        # rows outside every segment's current rows are untouched
        used = np.zeros(r_cap, bool)
        for s in range(S):
            used[off[s]:off[s] + int(g_len[s])] = True
        assert np.all(g_idx[~used] == -7), f"append step {t}: rows outside segments written"


@pytest.mark.parametrize("fused", [False, True])
def test_c3_decode_loop_with_append(kv, fused):
    """FastGen serving loop on a reduced C3 layer: policy select, compact, then
    three decode steps; before each step the new token joins the cache under
    its head rule (local: sliding window, special: not added, global: grows),
    and the step's decode output is checked against the oracle.  fused: the
    new key and the queries arrive unrotated and the library rotates them with
    the segment's kept RoPE pairs (RAP §3); the oracle rotates them itself."""
    kvsel, pipeline, torch = kv
    steps = 3
    cfg = kvsynth.get_config(3, batch=2, n=3000 + 5)
    _say(cfg.name, "decode loop with append, n", cfg.n, "fused RoPE" if fused else "")
    if fused:
        pairs = np.stack([kvsynth.kept_pairs(cfg, 0, kvh)
                          for kvh in range(cfg.hkv)]).astype(np.int32)
        tab = kvsynth.rope_table(cfg.n + steps, cfg.d_rope // 2)
        tab_d, pairs_d = pipeline.device_tensor(tab), pipeline.device_tensor(pairs)
    inputs = kvsynth.layer_inputs(cfg, 0)
    run = pipeline.build_layer(cfg, inputs, slack=steps)
    run.select()
    run.compact()
    torch.cuda.synchronize()
    h = _host(run)
    kinds = np.asarray(inputs["head_kind"])
    rule = {kvsynth.HEAD_LOCAL: cfg.local_window, kvsynth.HEAD_SPECIAL: -1,
            kvsynth.HEAD_GLOBAL: 0}
    S = cfg.batch * cfg.hkv
    limits = np.array([rule[int(kinds[s % cfg.hkv])] for s in range(S)], np.int32)
    caps = pu.to_host(run.seg_cap)
    t_lim = pipeline.device_tensor(limits)
    segs = []
    for s in range(S):
        b, kvh = divmod(s, cfg.hkv)
        o, ln = int(h["seg_off"][s]), int(h["seg_len"][s])
        idx = h["idx"][o:o + ln].astype(np.int64)
        Kc, Vc = oracle.compact(inputs["K"][b, kvh], inputs["V"][b, kvh], idx)
        segs.append([idx, Kc, Vc])
    worst = 0.0
    for t in range(steps):
        st = kvsynth.step_inputs(cfg, 0, t, rotated=not fused)
        pos = st["pos"]
        shape = run.shape
        if fused:
            sh = run.shape
            shape = kvsel.make_shape(sh.batch, sh.hq, sh.hkv, sh.head_dim, sh.n, sh.dtype, sh.scale,
                                     rope=kvsel.make_rope(tab_d, pairs_d, q_pos=pos))
        kvsel.kvsel_append(shape, pipeline.device_tensor(st["k_new"]),
                           pipeline.device_tensor(st["v_new"]), pos, run.seg_off, run.seg_cap,
                           t_lim, run.seg_len, run.idx, run.k_c, run.v_c, run.r_cap)
        q = pipeline.device_tensor(st["q"])
        kvsel.kvsel_decode_attn(shape, q, run.k_c, run.v_c, run.seg_off, run.seg_len,
                                run.r_cap, run.out, run.ws_dec)
        torch.cuda.synchronize()
        out = pu.to_host(run.out)
        rot = (lambda x, kvh: oracle.rope_pairs(x[None], np.array([pos]), tab, pairs[kvh],
                                                cfg.dtype)[0]) if fused else (lambda x, kvh: x)
        for s in range(S):
            b, kvh = divmod(s, cfg.hkv)
            segs[s] = list(oracle.append_token(segs[s][0], segs[s][1], segs[s][2], pos,
                                               rot(st["k_new"][b, kvh], kvh), st["v_new"][b, kvh],
                                               int(caps[s]), int(limits[s])))
            Kc, Vc = oracle.to_f64(segs[s][1]), oracle.to_f64(segs[s][2])
            for g in range(cfg.G):
                h_ = kvh * cfg.G + g
                want = oracle.decode_attention(oracle.to_f64(rot(st["q"][b, h_], kvh)), Kc, Vc,
                                               cfg.scale)
                err = float(np.max(np.abs(out[b, h_] - want)))
                worst = max(worst, err)
                assert err <= pu.OUT_ATOL[cfg.dtype], f"step {t} seg {s} head {g}: err {err}"
    print(f"  decode loop: max abs err {worst:.2e}", flush=True)


# ---------------------------------------------------------------------------
# LMBA and kept attention (ZigZagkv Eq. 3, §5.5 Table 3)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d,G,w,n,q_pos0", [("fp32", 64, 2, 8, 512, 504),
                                                 ("bf16", 128, 4, 32, 3001, 2969),
                                                 ("bf16", 88, 4, 5, 700, 10)])
def test_lmba_uniform_rows_exact(kv, dtype, d, G, w, n, q_pos0):
    """Zero queries give uniform rows over the visible keys: LMBA is exactly
    ceil(0.9 * visible) for every row."""
    kvsel, pipeline, torch = kv
    _say("lmba uniform", dtype, d, G, w, n, q_pos0)
    B, hkv = 2, 2
    sdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    shape = kvsel.make_shape(B, G * hkv, hkv, d, n, dtype, 1 / math.sqrt(d))
    q = torch.zeros(B, G * hkv, w, d, dtype=sdt, device="cuda")
    k = torch.randn(B, hkv, n, d, device="cuda").to(sdt)
    lm = torch.empty(B * hkv * G * w, dtype=torch.int32, device="cuda")
    km = torch.empty(B * hkv * G * w, dtype=torch.float32, device="cuda")
    ws = torch.empty(kvsel.kvsel_lmba_workspace(shape, w), dtype=torch.uint8, device="cuda")
    # segment s lists positions 0 .. 37*(s+1)-1, then one of them again and two
    # outside [0, n): the kept mass counts each listed position once
    S = B * hkv
    lists = [list(range(37 * (s + 1))) + [5, -1, n] for s in range(S)]
    off = np.cumsum([0] + [len(x) for x in lists])
    idx = pipeline.device_tensor(np.concatenate(lists).astype(np.int32))
    seg_off = pipeline.device_tensor(off[:-1].astype(np.int64))
    seg_len = pipeline.device_tensor(np.diff(off).astype(np.int32))
    kvsel.kvsel_lmba(shape, w, q_pos0, q, k, lm, ws)
    torch.cuda.synchronize()
    got = pu.to_host(lm).reshape(S, G * w)
    lm.fill_(-7)
    kvsel.kvsel_lmba(shape, w, q_pos0, q, k, lm, ws, seg_off, seg_len, idx, int(off[-1]), km)
    torch.cuda.synchronize()
    assert np.array_equal(pu.to_host(lm).reshape(S, G * w), got)
    kept = pu.to_host(km).reshape(S, G * w)
    for s in range(S):
        for r in range(G * w):
            vis = min(q_pos0 + r % w, n - 1) + 1
            assert got[s, r] == math.ceil(0.9 * vis - 1e-12), (s, r, got[s, r], vis)
            want = min(37 * (s + 1), vis) / vis
            assert abs(kept[s, r] - want) <= 1e-6, (s, r, kept[s, r], want)


@pytest.mark.parametrize("cid", [0, 1])
def test_lmba_and_kept_mass_match_oracle(kv, cid):
    """Per-row LMBA within the float64 band, and the attention the pipeline's
    top-B selection keeps per row within 1e-5, on whole C0 / C1 layers."""
    kvsel, pipeline, torch = kv
    cfg = kvsynth.get_config(cid)
    _say(cfg.name, "lmba + kept mass")
    inputs, run = _run(kv, cfg)
    R, S = cfg.G * cfg.w, cfg.batch * cfg.hkv
    lm = torch.empty(S * R, dtype=torch.int32, device="cuda")
    km = torch.empty(S * R, dtype=torch.float32, device="cuda")
    ws = torch.empty(kvsel.kvsel_lmba_workspace(run.shape, cfg.w), dtype=torch.uint8, device="cuda")
    kvsel.kvsel_lmba(run.shape, cfg.w, cfg.n - cfg.w, run.q_win, run.k, lm, ws, run.seg_off,
                     run.seg_len, run.idx, run.r_cap, km)
    torch.cuda.synchronize()
    got_k = pu.to_host(lm).reshape(S, R)
    got_m = pu.to_host(km).reshape(S, R)
    h = _host(run)
    worst = 0.0
    for s in range(S):
        b, kvh = divmod(s, cfg.hkv)
        P = oracle.window_probabilities(oracle.to_f64(inputs["q_win"][b, kvh * cfg.G:(kvh + 1) * cfg.G]),
                                        oracle.to_f64(inputs["K"][b, kvh]), cfg.scale, cfg.n - cfg.w)
        pu.check_lmba(got_k[s], P, f"{cfg.name} seg {s}")
        if cid == 0:   # the exact oracle on every row: inside the band, equal when it is one value
            for r in range(R):
                exact = oracle.lmba_row(P[r])
                cum = np.cumsum(np.sort(P[r])[::-1])
                lo = int(np.searchsorted(cum, 0.9 * (1 - 1e-5) * cum[-1])) + 1
                hi = int(np.searchsorted(cum, 0.9 * (1 + 1e-5) * cum[-1])) + 1
                assert lo <= exact <= hi
                if lo == hi:
                    assert got_k[s, r] == exact, (s, r, got_k[s, r], exact)
        off, ln = int(h["seg_off"][s]), int(h["seg_len"][s])
        kept = h["idx"][off:off + ln].astype(np.int64)
        want = 0.9 - oracle.attention_loss(P, kept)      # kept mass where below 0.9
        ref_mass = P[:, kept].sum(axis=1)
        err = float(np.max(np.abs(got_m[s] - ref_mass)))
        worst = max(worst, err)
        assert err <= 1e-5, f"{cfg.name} seg {s}: kept mass err {err}"
        assert np.all(np.minimum(got_m[s], 0.9) <= want + 1e-5)
    print(f"  {cfg.name}: layer LMBA {got_k.mean():.1f} of n={cfg.n}, kept-mass err {worst:.1e}, "
          f"mean attention loss {np.maximum(0, 0.9 - got_m).mean():.4f}", flush=True)


@pytest.mark.parametrize("dtype,d,G,w,n,slope", [("fp32", 64, 2, 8, 3000, 1.0),
                                                 ("bf16", 128, 4, 32, 4100, -3.0),
                                                 ("bf16", 88, 4, 16, 2600, 3.0)])
def test_lmba_drifting_logits(kv, dtype, d, G, w, n, slope):
    """LMBA of rows whose weights span ~30 to ~90 log2 units (logits drifting
    along the keys): 90 % of each row sits in about 100 to 350 keys, and at
    slope 3 the smallest weights fall below the radix select's 2^-40 floor.
    Per row within the float64 band of the exact answer."""
    kvsel, pipeline, torch = kv
    _say("lmba drift", dtype, d, G, w, n, slope)
    r = np.random.default_rng(7 * n + d)
    B, hkv = 1, 2
    q = np.empty((B, hkv * G, w, d), np.float32)
    Kf = np.empty((B, hkv, n, d), np.float32)
    for h in range(hkv):
        keys, qs = _drifting_logits(r, n, d, G * w, slope)
        Kf[0, h] = keys
        q[0, h * G:(h + 1) * G] = qs.reshape(G, w, d)
    store = (lambda x: kvsynth.f32_to_bf16_bits(x)) if dtype == "bf16" else (lambda x: x)
    q, Kf = store(q), store(Kf)
    shape = kvsel.make_shape(B, hkv * G, hkv, d, n, dtype, 1 / math.sqrt(d))
    R = G * w
    lm = torch.empty(B * hkv * R, dtype=torch.int32, device="cuda")
    ws = torch.empty(kvsel.kvsel_lmba_workspace(shape, w), dtype=torch.uint8, device="cuda")
    kvsel.kvsel_lmba(shape, w, n - w, pipeline.device_tensor(q), pipeline.device_tensor(Kf), lm,
                     ws)
    torch.cuda.synchronize()
    got = pu.to_host(lm).reshape(B * hkv, R)
    for s in range(B * hkv):
        P = oracle.window_probabilities(oracle.to_f64(q[0, s * G:(s + 1) * G]),
                                        oracle.to_f64(Kf[0, s]), 1 / math.sqrt(d), n - w)
        assert np.median(got[s]) < n // 8   # concentrated rows, not near-uniform ones
        pu.check_lmba(got[s], P, f"lmba drift seg {s}")


# ---------------------------------------------------------------------------
# fused pair-pruned RoPE (RAP §3, Eq. 5-10): rows arrive unrotated and are
# rotated inside the kernels; the rotation is fixed fp32 arithmetic, so the
# fused path must equal the same kernels fed the oracle's rotated rows bit for
# bit, and the oracle within the usual bars.
# ---------------------------------------------------------------------------

def _rope_setup(kv, dtype, d, half, hkv, max_pos, seed):
    kvsel, pipeline, torch = kv
    r = np.random.default_rng(seed)
    if d // 2 == half:
        pairs = np.tile(np.arange(half, dtype=np.int32), (hkv, 1))
    else:
        pairs = np.stack([np.sort(r.choice(half, d // 2, replace=False))
                          for _ in range(hkv)]).astype(np.int32)
    tab = kvsynth.rope_table(max_pos, half)
    store = (lambda x: kvsynth.f32_to_bf16_bits(x)) if dtype == "bf16" else (lambda x: x)
    dev = (pipeline.device_tensor(tab), pipeline.device_tensor(pairs))
    return r, pairs, tab, store, dev


@pytest.mark.parametrize("dtype,d,half,G,w,n", [("bf16", 128, 64, 4, 32, 3000),
                                               ("bf16", 88, 64, 4, 8, 1500),
                                               ("fp32", 64, 64, 2, 8, 777),
                                               ("fp32", 88, 64, 1, 3, 300)])
def test_rope_score_and_lmba_fused(kv, dtype, d, half, G, w, n):
    kvsel, pipeline, torch = kv
    _say("rope score", dtype, d, half, G, w, n)
    B, hkv = 2, 2
    q_pos0 = n - w
    r, pairs, tab, store, (tab_d, pairs_d) = _rope_setup(kv, dtype, d, half, hkv, n + 5, n * 7 + d)
    q = store((r.standard_normal((B, hkv * G, w, d)) * 1.5).astype(np.float32))
    K = store(r.standard_normal((B, hkv, n, d)).astype(np.float32))
    q_rot = np.empty_like(q)
    for b in range(B):
        for h in range(hkv * G):
            q_rot[b, h] = oracle.rope_pairs(q[b, h], q_pos0 + np.arange(w), tab, pairs[h // G], dtype)
    plain = kvsel.make_shape(B, hkv * G, hkv, d, n, dtype, 1 / math.sqrt(d))
    fused = kvsel.make_shape(B, hkv * G, hkv, d, n, dtype, 1 / math.sqrt(d),
                             rope=kvsel.make_rope(tab_d, pairs_d))
    Kd = pipeline.device_tensor(K)
    # unrotated queries need room for their rotated copy: the fused shape's size serves both
    assert kvsel.kvsel_score_workspace(fused, w) > kvsel.kvsel_score_workspace(plain, w)
    ws = torch.empty(kvsel.kvsel_score_workspace(fused, w), dtype=torch.uint8, device="cuda")
    s1 = torch.empty(B * hkv * n, dtype=torch.float32, device="cuda")
    s2 = torch.empty_like(s1)
    kvsel.kvsel_score(fused, w, q_pos0, pipeline.device_tensor(q), Kd, s1, ws)
    kvsel.kvsel_score(plain, w, q_pos0, pipeline.device_tensor(q_rot), Kd, s2, ws)
    lws = torch.empty(kvsel.kvsel_lmba_workspace(fused, w), dtype=torch.uint8, device="cuda")
    l1 = torch.empty(B * hkv * G * w, dtype=torch.int32, device="cuda")
    l2 = torch.empty_like(l1)
    kvsel.kvsel_lmba(fused, w, q_pos0, pipeline.device_tensor(q), Kd, l1, lws)
    kvsel.kvsel_lmba(plain, w, q_pos0, pipeline.device_tensor(q_rot), Kd, l2, lws)
    torch.cuda.synchronize()
    a, b_ = pu.to_host(s1), pu.to_host(s2)
    assert np.array_equal(a.view(np.uint32), b_.view(np.uint32)), "fused RoPE score differs"
    assert np.array_equal(pu.to_host(l1), pu.to_host(l2)), "fused RoPE LMBA differs"
    a = a.reshape(B * hkv, n)
    for s in range(B * hkv):
        bb, kh = divmod(s, hkv)
        ref = oracle.window_scores(oracle.to_f64(q_rot[bb, kh * G:(kh + 1) * G]),
                                   oracle.to_f64(K[bb, kh]), 1 / math.sqrt(d), q_pos0)
        pu.check_scores(a[s], ref, G * w, f"rope score seg {s}")


@pytest.mark.parametrize("dtype,d,half,G", [("bf16", 88, 64, 4), ("bf16", 128, 64, 4),
                                           ("fp32", 88, 64, 2), ("bf16", 64, 64, 1),
                                           ("bf16", 128, 64, 8)])
def test_rope_decode_fused(kv, dtype, d, half, G):
    kvsel, pipeline, torch = kv
    _say("rope decode", dtype, d, half, G)
    B, hkv = 2, 2
    S = B * hkv
    q_pos = 40000
    r, pairs, tab, store, (tab_d, pairs_d) = _rope_setup(kv, dtype, d, half, hkv, q_pos + 1, d + G)
    lens = np.array([0, 3, 700, 2500], np.int32)
    off, r_cap = pipeline.offsets(lens.astype(np.int64))
    Kc = store(r.standard_normal((r_cap, d)).astype(np.float32))
    Vc = store(r.standard_normal((r_cap, d)).astype(np.float32))
    q = store((2 * r.standard_normal((B, hkv * G, d))).astype(np.float32))
    q_rot = np.empty_like(q)
    for b in range(B):
        for h in range(hkv * G):
            q_rot[b, h] = oracle.rope_pairs(q[b, h][None], np.array([q_pos]), tab, pairs[h // G],
                                            dtype)[0]
    plain = kvsel.make_shape(B, hkv * G, hkv, d, 2500, dtype, 1 / math.sqrt(128))
    fused = kvsel.make_shape(B, hkv * G, hkv, d, 2500, dtype, 1 / math.sqrt(128),
                             rope=kvsel.make_rope(tab_d, pairs_d, q_pos=q_pos))
    ws = torch.empty(kvsel.kvsel_decode_workspace(plain, r_cap), dtype=torch.uint8, device="cuda")
    o1 = torch.empty((B, hkv * G, d), dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(o1)
    args = (pipeline.device_tensor(Kc), pipeline.device_tensor(Vc), pipeline.device_tensor(off),
            pipeline.device_tensor(lens), r_cap)
    kvsel.kvsel_decode_attn(fused, pipeline.device_tensor(q), *args, o1, ws)
    kvsel.kvsel_decode_attn(plain, pipeline.device_tensor(q_rot), *args, o2, ws)
    torch.cuda.synchronize()
    a = pu.to_host(o1)
    assert np.array_equal(a.view(np.uint32), pu.to_host(o2).view(np.uint32)), "fused RoPE decode differs"
    for s in range(S):
        b, h = divmod(s, hkv)
        rows = np.arange(off[s], off[s] + lens[s])
        pu.check_decode(a[b, h * G:(h + 1) * G], q_rot[b, h * G:(h + 1) * G], Kc, Vc, rows,
                        1 / math.sqrt(128), dtype, f"rope decode seg {s}")


@pytest.mark.parametrize("dtype,d", [("bf16", 88), ("fp32", 128)])
def test_rope_append_rotates_new_key(kv, dtype, d):
    """The appended key is the oracle's rotation of the new key at pos, bit for
    bit; the value row is copied unchanged."""
    kvsel, pipeline, torch = kv
    _say("rope append", dtype, d)
    B, hkv, G = 2, 2, 2
    S = B * hkv
    pos = 9000
    r, pairs, tab, store, (tab_d, pairs_d) = _rope_setup(kv, dtype, d, 64, hkv, pos + 1, 11 + d)
    cap = np.array([4, 4, 4, 4], np.int64)
    lens = np.array([0, 2, 4, 4], np.int32)
    limit = np.array([0, 0, 3, -1], np.int32)
    off, r_cap = pipeline.offsets(cap)
    Kc = store(r.standard_normal((r_cap, d)).astype(np.float32))
    Vc = store(r.standard_normal((r_cap, d)).astype(np.float32))
    idx = np.arange(r_cap, dtype=np.int32) * 7
    k_new = store(r.standard_normal((B, hkv, d)).astype(np.float32))
    v_new = store(r.standard_normal((B, hkv, d)).astype(np.float32))
    fused = kvsel.make_shape(B, hkv * G, hkv, d, 5000, dtype, 0.1,
                             rope=kvsel.make_rope(tab_d, pairs_d))
    kc_d, vc_d, idx_d = (pipeline.device_tensor(Kc), pipeline.device_tensor(Vc),
                         pipeline.device_tensor(idx))
    len_d = pipeline.device_tensor(lens)
    kvsel.kvsel_append(fused, pipeline.device_tensor(k_new), pipeline.device_tensor(v_new), pos,
                       pipeline.device_tensor(off), pipeline.device_tensor(cap),
                       pipeline.device_tensor(limit), len_d, idx_d, kc_d, vc_d, r_cap)
    torch.cuda.synchronize()
    kg, vg, ig = pu.to_host(kc_d), pu.to_host(vc_d), pu.to_host(idx_d)
    Kw, Vw, Iw = Kc.copy(), Vc.copy(), idx.copy()
    for s in range(S):
        b, h = divmod(s, hkv)
        o = int(off[s])
        rows = slice(o, o + int(lens[s]))
        k_rot = oracle.rope_pairs(k_new[b, h][None], np.array([pos]), tab, pairs[h], dtype)[0]
        i2, k2, v2 = oracle.append_token(idx[rows], Kc[rows], Vc[rows], pos, k_rot, v_new[b, h],
                                         int(cap[s]), int(limit[s]))
        Iw[o:o + len(i2)], Kw[o:o + len(i2)], Vw[o:o + len(i2)] = i2, k2, v2
    assert np.array_equal(ig, Iw)
    assert np.array_equal(kg.view(np.uint8), Kw.view(np.uint8)), "rotated key rows differ"
    assert np.array_equal(vg.view(np.uint8), Vw.view(np.uint8))


# ---------------------------------------------------------------------------
# serving loop: periodic re-scoring and re-selection over the resident full cache
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cid,over,steps", [(0, {}, 20),
                                            (1, dict(n=3000, budget=400, w=16, batch=2), 33)])
def test_serving_loop_periodic_reselection(kv, cid, over, steps):
    """Each step the new token joins the full and the compacted cache and the
    decode reads the compacted cache (checked against the oracle over the
    GPU's kept rows); every w steps the score of the last w decode queries over
    the full cache is taken again (oracle within the score bar, keys not yet
    generated score 0) and the top-B selection (tie band) and compaction
    (bit-exact) are redone."""
    kvsel, pipeline, torch = kv
    cfg = kvsynth.get_config(cid, **over)
    _say(cfg.name, "serving loop, n", cfg.n, "w", cfg.w, "steps", steps)
    inputs = kvsynth.layer_inputs(cfg, 0)
    run = pipeline.build_layer(cfg, inputs, slack=cfg.w)
    run.score(); run.select(); run.compact()
    loop = pipeline.ServingLoop.start(run, run.k, run.v, cfg.n, steps)
    torch.cuda.synchronize()
    S, G, w, B = cfg.batch * cfg.hkv, cfg.G, cfg.w, cfg.budget
    Kf = [[inputs["K"][b, h] for h in range(cfg.hkv)] for b in range(cfg.batch)]
    Vf = [[inputs["V"][b, h] for h in range(cfg.hkv)] for b in range(cfg.batch)]
    h0 = _host(run)
    sel = {s: h0["idx"][int(h0["seg_off"][s]):int(h0["seg_off"][s]) + int(h0["seg_len"][s])]
           .astype(np.int64) for s in range(S)}
    since = cfg.n          # first position appended after the current selection
    qs = []
    worst = 0.0
    for t in range(steps):
        st = kvsynth.step_inputs(cfg, 0, t)
        pos = st["pos"]
        redone = loop.step(pipeline.device_tensor(st["k_new"]), pipeline.device_tensor(st["v_new"]),
                           pipeline.device_tensor(st["q"]))
        torch.cuda.synchronize()
        qs.append(st["q"])
        h = _host(run)
        for s in range(S):
            b, kvh = divmod(s, cfg.hkv)
            Kf[b][kvh] = np.concatenate([Kf[b][kvh], st["k_new"][b, kvh][None]])
            Vf[b][kvh] = np.concatenate([Vf[b][kvh], st["v_new"][b, kvh][None]])
            # this step's decode read the selection plus every token appended since
            idx = np.concatenate([sel[s], np.arange(since, pos + 1)])
            if not redone:
                o, ln = int(h["seg_off"][s]), int(h["seg_len"][s])
                assert np.array_equal(h["idx"][o:o + ln], idx), f"t={t} seg {s}: kept rows"
                pu.check_compact(h["k_c"][o:o + ln], h["v_c"][o:o + ln], Kf[b][kvh], Vf[b][kvh],
                                 idx, f"t={t} seg {s}")
            err = pu.check_decode(h["out"][b, kvh * G:(kvh + 1) * G],
                                  st["q"][b, kvh * G:(kvh + 1) * G], Kf[b][kvh], Vf[b][kvh], idx,
                                  cfg.scale, cfg.dtype, f"t={t} seg {s}")
            worst = max(worst, err)
        if redone:
            assert t % w == w - 1
            sc = h["scores"].reshape(S, -1)
            win = np.stack(qs[-w:], axis=2)           # [b][hq][w][d], positions pos-w+1 .. pos
            for s in range(S):
                b, kvh = divmod(s, cfg.hkv)
                o, ln = int(h["seg_off"][s]), int(h["seg_len"][s])
                idx = h["idx"][o:o + ln].astype(np.int64)
                ref = oracle.window_scores(oracle.to_f64(win[b, kvh * G:(kvh + 1) * G]),
                                           oracle.to_f64(Kf[b][kvh]), cfg.scale, pos - w + 1)
                assert not sc[s, pos + 1:].any(), "keys not yet generated must score 0"
                pu.check_scores(sc[s, :pos + 1], ref, G * w, f"t={t} seg {s}")
                pu.check_topb_selection(idx, sc[s, :pos + 1], ref, B, f"t={t} seg {s}")
                pu.check_compact(h["k_c"][o:o + ln], h["v_c"][o:o + ln], Kf[b][kvh], Vf[b][kvh],
                                 idx, f"t={t} seg {s}")
                sel[s] = idx
            since = pos + 1
    assert loop.reselections == steps // w
    print(f"  {cfg.name}: {loop.reselections} re-selections, decode max abs err {worst:.2e}",
          flush=True)


def test_model_serving_loop_matches_layer_loops(kv):
    """The serving loop for three layers at once (re-selection of every layer
    in one score, one select and one compact call) gives, step by step, the
    same bits as one ServingLoop per layer (checked against the oracle in
    test_serving_loop_periodic_reselection): decode outputs every step, and
    at each re-selection the scores, kept rows and compacted K/V of every
    segment."""
    kvsel, pipeline, torch = kv
    cfg = kvsynth.get_config(2, n=3000, layers=3, batch=2)
    L, S, w, n = cfg.layers, cfg.batch * cfg.hkv, cfg.w, cfg.n
    steps = 2 * w + 5
    _say(cfg.name, "model serving loop, layers", L, "n", n, "steps", steps)
    budgets = kvsel.kvsel_zigzag_budgets(kvsynth.zigzag_profile(cfg), n, 600, 150)
    ins = [kvsynth.layer_inputs(cfg, l) for l in range(L)]
    loops = []
    for l in range(L):
        run = pipeline.build_layer(cfg, ins[l], budget=budgets[l], slack=w)
        run.score(); run.select(); run.compact()
        loops.append(pipeline.ServingLoop.start(run, run.k, run.v, n, steps))
    dt = lambda a: pipeline.device_tensor(a)
    k = torch.cat([dt(x["K"]) for x in ins])
    v = torch.cat([dt(x["V"]) for x in ins])
    q_win = torch.cat([dt(x["q_win"]) for x in ins])
    ml = pipeline.ModelServingLoop.start(cfg, budgets, k, v, q_win, steps)
    torch.cuda.synchronize()

    def same(a, b, what):
        assert np.array_equal(pu.to_host(a).view(np.uint8), pu.to_host(b).view(np.uint8)), what

    def same_selection(t):
        for l in range(L):
            run = loops[l].run
            r = slice(l * S, (l + 1) * S)
            same(ml.seg_len[r], run.seg_len, f"t={t} layer {l} seg_len")
            off_m, off_l = pu.to_host(ml.seg_off[r]), pu.to_host(run.seg_off)
            lens = pu.to_host(run.seg_len)
            for s in range(S):
                a, b, ln = int(off_m[s]), int(off_l[s]), int(lens[s])
                what = f"t={t} layer {l} seg {s}"
                same(ml.idx[a:a + ln], run.idx[b:b + ln], what + " idx")
                same(ml.k_c[a:a + ln], run.k_c[b:b + ln], what + " k_c")
                same(ml.v_c[a:a + ln], run.v_c[b:b + ln], what + " v_c")
    same_selection(-1)
    for t in range(steps):
        for l in range(L):
            st = kvsynth.step_inputs(cfg, l, t)
            kn, vn, q = dt(st["k_new"]), dt(st["v_new"]), dt(st["q"])
            loops[l].step(kn, vn, q)
            ml.step_layer(l, kn, vn, q)
        redone = ml.end_step()
        torch.cuda.synchronize()
        for l in range(L):
            same(ml.out[l], loops[l].run.out, f"t={t} layer {l} decode")
        if redone:
            for l in range(L):
                nc = ml.full_shape.n
                same(ml.scores[l * S * nc:(l + 1) * S * nc], loops[l].run.scores,
                     f"t={t} layer {l} scores")
            same_selection(t)
    assert ml.reselections == steps // w and all(lp.reselections == steps // w for lp in loops)
    print(f"  {cfg.name}: {L} layers, {steps} steps, {ml.reselections} batched re-selections "
          f"identical to per-layer loops", flush=True)


def test_chunk_serving_loop_reselects_at_boundaries(kv):
    """ChunkLLM decode loop on a reduced C4 layer (§2.3, ICAC): 4 local chunks
    + the 16 best others; the selection is redone only at the steps whose token
    closes a chunk.  At those steps the chunk scores (oracle within the score
    bar), the chunk selection (tie band) and the compaction (bit-exact) are
    checked; every step's decode is checked against the oracle over the rows
    the GPU kept (the selection plus the tokens appended since)."""
    kvsel, pipeline, torch = kv
    local, top, steps = 4, 16, 100
    cfg = kvsynth.get_config(4, n=3000)
    _say(cfg.name, "chunk serving loop, n", cfg.n, "steps", steps)
    inputs = kvsynth.layer_inputs(cfg, 0)
    run = pipeline.build_layer(cfg, inputs, local_chunks=local, top_chunks=top,
                               slack=(local + top + 1) * steps)
    run.run()
    loop = pipeline.ChunkServingLoop.start(run, run.k, run.v, cfg.n, steps, run.score_keys,
                                           np.asarray(inputs["chunk_end"], np.int64), local, top)
    torch.cuda.synchronize()
    S, G, hkv = cfg.batch * cfg.hkv, cfg.G, cfg.hkv
    Kf = [[inputs["K"][b, h] for h in range(hkv)] for b in range(cfg.batch)]
    Vf = [[inputs["V"][b, h] for h in range(hkv)] for b in range(cfg.batch)]
    CK = [[inputs["chunk_keys"][b, h] for h in range(hkv)] for b in range(cfg.batch)]
    ends = [np.asarray(inputs["chunk_end"][b], np.int64) for b in range(cfg.batch)]
    h0 = _host(run)
    sel = {s: h0["idx"][int(h0["seg_off"][s]):int(h0["seg_off"][s]) + int(h0["seg_len"][s])]
           .astype(np.int64) for s in range(S)}
    since = cfg.n
    worst, nb = 0.0, 0
    for t in range(steps):
        st = kvsynth.chunk_step_inputs(cfg, 0, t)
        pos = st["pos"]
        redone = loop.step(pipeline.device_tensor(st["k_new"]), pipeline.device_tensor(st["v_new"]),
                           pipeline.device_tensor(st["q"]), st["boundary"],
                           pipeline.device_tensor(st["chunk_key"]),
                           pipeline.device_tensor(st["chunk_q"]))
        torch.cuda.synchronize()
        assert redone == st["boundary"]
        h = _host(run)
        for s in range(S):
            b, kvh = divmod(s, hkv)
            Kf[b][kvh] = np.concatenate([Kf[b][kvh], st["k_new"][b, kvh][None]])
            Vf[b][kvh] = np.concatenate([Vf[b][kvh], st["v_new"][b, kvh][None]])
            idx = np.concatenate([sel[s], np.arange(since, pos + 1)])
            if not redone:
                o, ln = int(h["seg_off"][s]), int(h["seg_len"][s])
                assert np.array_equal(h["idx"][o:o + ln], idx), f"t={t} seg {s}: kept rows"
            err = pu.check_decode(h["out"][b, kvh * G:(kvh + 1) * G],
                                  st["q"][b, kvh * G:(kvh + 1) * G], Kf[b][kvh], Vf[b][kvh], idx,
                                  cfg.scale, cfg.dtype, f"t={t} seg {s}")
            worst = max(worst, err)
        if not redone:
            continue
        nb += 1
        nc = loop.nc
        sc = pu.to_host(loop.sc).reshape(S, -1)
        for b in range(cfg.batch):
            ends[b] = np.append(ends[b], pos + 1)
            assert len(ends[b]) == nc
        for s in range(S):
            b, kvh = divmod(s, hkv)
            CK[b][kvh] = np.concatenate([CK[b][kvh], st["chunk_key"][b, kvh][None]])
            o, ln = int(h["seg_off"][s]), int(h["seg_len"][s])
            idx = h["idx"][o:o + ln].astype(np.int64)
            ref = oracle.window_scores(oracle.to_f64(st["chunk_q"][b, kvh * G:(kvh + 1) * G]),
                                       oracle.to_f64(CK[b][kvh]), cfg.scale, nc - 1)
            assert not sc[s, nc:].any()
            pu.check_scores(sc[s, :nc], ref, G, f"t={t} seg {s} chunk scores")
            pu.check_chunk_selection(idx, sc[s, :nc], ref, ends[b], 0, f"t={t} seg {s}",
                                     local=local, top=top)
            pu.check_compact(h["k_c"][o:o + ln], h["v_c"][o:o + ln], Kf[b][kvh], Vf[b][kvh], idx,
                             f"t={t} seg {s}")
            sel[s] = idx
        since = pos + 1
    assert nb >= 2 and loop.reselections == nb
    print(f"  {cfg.name}: {nb} boundary re-selections in {steps} steps, decode max abs err "
          f"{worst:.2e}", flush=True)


# ---------------------------------------------------------------------------
# ChunkLLM layer-wise chunk voting (§2.3; reading: votes, then summed attention)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,layers,top,local", [(3000, 4, 16, 4), (20000, 6, 64, 8)])
def test_chunk_vote_matches_oracle(kv, n, layers, top, local):
    """Chunk scores of several layers over shared chunk boundaries (the chunk
    adapter sits at the bottom layer), voted into one key per chunk: each
    layer's ballot differs from the float64 one only inside the tie band, and
    the CHUNK selection over the key keeps the chunks of the plain rule (most
    votes, then larger summed attention, then lower index) up to the tie band
    on the summed attention -- on the GPU's own fp32 scores, and end to end
    on the float64 scores whenever the layers' ballots agree."""
    from kvsynth import gen
    kvsel, pipeline, torch = kv
    cfg = kvsynth.get_config(4, n=n)
    _say(cfg.name, "chunk vote, n", n, "layers", layers, "top", top, "local", local)
    B, hkv, hq, G, cd = cfg.batch, cfg.hkv, cfg.hq, cfg.G, cfg.chunk_dim
    S = B * hkv
    ends = [gen.chunk_ends(cfg, b, 0) for b in range(B)]
    nc = len(ends[0])
    sshape = kvsel.make_shape(B, hq, hkv, cd, nc, cfg.dtype, cfg.scale)
    allsc = torch.empty(layers * S * nc, dtype=torch.float32, device="cuda")
    ws = torch.empty(kvsel.kvsel_score_workspace(sshape, 1), dtype=torch.uint8, device="cuda")
    ref = np.zeros((layers, S, nc))
    for l in range(layers):
        P = gen.chunk_projection(cfg, l)
        ck = np.empty((B, hkv, nc, cd), np.uint16)
        cq = np.empty((B, hq, 1, cd), np.uint16)
        for b in range(B):
            for h in range(hkv):
                K, _ = gen.segment_kv(cfg, l, b, h)
                _, qd = gen.segment_queries(cfg, l, b, h)
                ck[b, h], cq[b, h * G:(h + 1) * G] = gen.segment_chunk_inputs(cfg, K, qd, ends[b], P)
                ref[l, b * hkv + h] = oracle.window_scores(
                    oracle.to_f64(cq[b, h * G:(h + 1) * G]), oracle.to_f64(ck[b, h]), cfg.scale,
                    nc - 1)
        kvsel.kvsel_score(sshape, 1, nc - 1, pipeline.device_tensor(cq), pipeline.device_tensor(ck),
                          allsc[l * S * nc:(l + 1) * S * nc], ws)
    key = torch.empty(S * nc, dtype=torch.float32, device="cuda")
    vws = torch.empty(kvsel.kvsel_chunk_vote_workspace(sshape, layers, top), dtype=torch.uint8,
                      device="cuda")
    kvsel.kvsel_chunk_vote(sshape, layers, top, local, allsc, key, vws)
    # the shared selection: local chunks + the top best keys, over the voted key
    shape = kvsel.make_shape(B, hq, hkv, cfg.d, n, cfg.dtype, cfg.scale)
    et = pipeline.device_tensor(np.stack(ends).astype(np.int64))
    cap = pipeline.capacities(kvsel.KVSEL_SEL_CHUNK, B, hkv, n, max_chunk=int(max(
        np.diff(np.concatenate([[0], e])).max() for e in ends)), local_chunks=local, top_chunks=top)
    off, r_cap = pipeline.offsets(cap)
    ln = torch.empty(S, dtype=torch.int32, device="cuda")
    idx = torch.empty(max(r_cap, 1), dtype=torch.int32, device="cuda")
    prm = kvsel.select_params(kvsel.KVSEL_SEL_CHUNK, n_chunks=nc, chunk_end=et,
                              local_chunks=local, top_chunks=top)
    kvsel.kvsel_select(shape, prm, key, pipeline.device_tensor(off), ln, idx, r_cap)
    torch.cuda.synchronize()
    sc = pu.to_host(allsc).reshape(layers, S, nc)
    lens, ig = pu.to_host(ln), pu.to_host(idx)
    in_band = e2e = 0
    for s in range(S):
        b = s // hkv
        agree = True
        for l in range(layers):
            pu.check_scores(sc[l, s], ref[l, s], G, f"layer {l} seg {s}")
            ballot = oracle.select_topb(sc[l, s].astype(np.float64), top)
            pu.check_topb_selection(ballot, sc[l, s], ref[l, s], top, f"ballot layer {l} seg {s}")
            agree &= np.array_equal(ballot, oracle.select_topb(ref[l, s], top))
        got = ig[off[s]:off[s] + lens[s]]
        in_band += pu.check_voted_selection(got, sc[:, s], ends[b], local, top, f"seg {s}")
        if agree:
            e2e += 1
            pu.check_voted_selection(got, ref[:, s], ends[b], local, top, f"seg {s} (float64)")
    print(f"  {cfg.name}: voted selections checked on {S} segments ({e2e} also end to end), "
          f"{in_band} chunks differ inside the tie band", flush=True)


def test_chunk_vote_near_ties(kv):
    """Layer-wise vote on C4-shaped chunk scores (6 layers, 4096 chunks, 4
    query heads per KV head, top 64, 8 local chunks) drawn flat enough that
    many chunks share the boundary vote count with summed attentions close
    together (about 1e-3 per layer): the kept chunks follow the plain rule on
    the same fp32 scores, up to the tie band on summed attention.  Scores are
    uploaded directly, 96 independent segments in one call."""
    kvsel, pipeline, torch = kv
    L, nc, G, top, local, B, hkv = 6, 4096, 4, 64, 8, 12, 8
    S = B * hkv
    _say("chunk vote near ties, segments", S)
    r = np.random.default_rng(20261203)
    sc = np.empty((L, S, nc), np.float32)
    for s in range(S):
        a, b = [(0.3, 0.3), (0.1, 0.5), (1.0, 0.1), (0.5, 0.2)][s % 4]
        z = r.standard_normal(nc)
        for l in range(L):
            lg = a * z + b * r.standard_normal(nc)
            p = np.exp(lg - lg.max())
            sc[l, s] = (G * p / p.sum()).astype(np.float32)
    ends = np.arange(1, nc + 1, dtype=np.int64) * 32
    n = int(ends[-1])
    sshape = kvsel.make_shape(B, hkv * G, hkv, 64, nc, kvsel.KVSEL_BF16, 0.125)
    allsc = pipeline.device_tensor(sc.reshape(-1))
    key = torch.empty(S * nc, dtype=torch.float32, device="cuda")
    vws = torch.empty(kvsel.kvsel_chunk_vote_workspace(sshape, L, top), dtype=torch.uint8,
                      device="cuda")
    kvsel.kvsel_chunk_vote(sshape, L, top, local, allsc, key, vws)
    shape = kvsel.make_shape(B, hkv * G, hkv, 128, n, kvsel.KVSEL_BF16, 0.125)
    et = pipeline.device_tensor(np.tile(ends, (B, 1)))
    cap = pipeline.capacities(kvsel.KVSEL_SEL_CHUNK, B, hkv, n, max_chunk=32,
                              local_chunks=local, top_chunks=top)
    off, r_cap = pipeline.offsets(cap)
    ln = torch.empty(S, dtype=torch.int32, device="cuda")
    idx = torch.empty(max(r_cap, 1), dtype=torch.int32, device="cuda")
    prm = kvsel.select_params(kvsel.KVSEL_SEL_CHUNK, n_chunks=nc, chunk_end=et,
                              local_chunks=local, top_chunks=top)
    kvsel.kvsel_select(shape, prm, key, pipeline.device_tensor(off), ln, idx, r_cap)
    torch.cuda.synchronize()
    lens, ig = pu.to_host(ln), pu.to_host(idx)
    in_band = 0
    for s in range(S):
        got = ig[off[s]:off[s] + lens[s]]
        assert lens[s] == (top + local) * 32, f"seg {s}: kept {lens[s]} tokens"
        in_band += pu.check_voted_selection(got, sc[:, s], ends, local, top, f"seg {s}")
    print(f"  near ties: {S} segments, {in_band} chunks differ inside the tie band", flush=True)


# ---------------------------------------------------------------------------
# the whole model in one layout: one compression call per step, decode per layer
# ---------------------------------------------------------------------------

def test_model_run_matches_layer_runs(kv):
    """Score, select and compact for all layers in one call each (segments of
    every layer) give bit for bit what the per-layer calls give, and the
    per-layer decode over the shared packed cache equals a separate layer's."""
    kvsel, pipeline, torch = kv
    cfg = kvsynth.get_config(2, n=3000, layers=3, batch=2)
    _say(cfg.name, "model run, layers", cfg.layers, "n", cfg.n)
    budgets = kvsel.kvsel_zigzag_budgets(kvsynth.zigzag_profile(cfg), cfg.n, 600, 150)
    inputs = [kvsynth.layer_inputs(cfg, l) for l in range(cfg.layers)]
    mr = pipeline.ModelRun.build(cfg, budgets, lambda l: inputs[l])
    mr.score(); mr.select(); mr.compact()
    for l in range(cfg.layers):
        mr.decode(l)
    torch.cuda.synchronize()
    S, n = cfg.batch * cfg.hkv, cfg.n
    sc_all, len_all = pu.to_host(mr.scores).copy(), pu.to_host(mr.seg_len).copy()
    idx_all, kc_all, out_all = pu.to_host(mr.idx).copy(), pu.to_host(mr.k_c).copy(), \
        pu.to_host(mr.out).copy()
    # per-layer calls on the same buffers
    mr.scores.zero_(); mr.idx.fill_(-1); mr.k_c.zero_(); mr.out.zero_()
    for l in range(cfg.layers):
        mr.score_layer(l); mr.select_layer(l); mr.compact_layer(l); mr.decode(l)
    torch.cuda.synchronize()
    assert np.array_equal(pu.to_host(mr.scores).view(np.uint32), sc_all.view(np.uint32))
    assert np.array_equal(pu.to_host(mr.seg_len), len_all)
    assert np.array_equal(pu.to_host(mr.idx), idx_all)
    assert np.array_equal(pu.to_host(mr.k_c).view(np.uint16), kc_all.view(np.uint16))
    assert np.array_equal(pu.to_host(mr.out).view(np.uint32), out_all.view(np.uint32))
    off = pu.to_host(mr.seg_off)
    for l in range(cfg.layers):
        run = pipeline.build_layer(cfg, inputs[l], budget=budgets[l])
        run.run()
        torch.cuda.synchronize()
        h = _host(run)
        assert np.array_equal(h["scores"].view(np.uint32),
                              sc_all[l * S * n:(l + 1) * S * n].view(np.uint32))
        assert np.array_equal(h["out"].view(np.uint32), out_all[l].view(np.uint32))
        for s in range(S):
            g = l * S + s
            a = h["idx"][h["seg_off"][s]:h["seg_off"][s] + h["seg_len"][s]]
            b = idx_all[off[g]:off[g] + len_all[g]]
            assert np.array_equal(a, b), (l, s)


def test_c2_model_full_sampled(kv):
    """The bench's launch configuration: all 32 C2 layers at full size, score,
    select and compact as one call each (1024 segments), decode per layer.
    Every segment: kept count = its layer's budget, indices strictly ascending
    inside [0, n).  Sampled segments across the layers: scores, selection
    (tie band), compaction (bit-exact) and decode against the oracle; one
    layer's LMBA rows (float64 band) and kept mass on two of them.  Then the
    whole step runs again over poisoned outputs and must give the same bits."""
    kvsel, pipeline, torch = kv
    cfg = kvsynth.get_config(2)
    _say(cfg.name, "full model, one compression call per phase")
    L, S, n, G, w = cfg.layers, cfg.batch * cfg.hkv, cfg.n, cfg.G, cfg.w
    budgets = kvsel.kvsel_zigzag_budgets(kvsynth.zigzag_profile(cfg), n, cfg.avg_budget,
                                         cfg.floor_budget)
    mr = pipeline.ModelRun.build(cfg, budgets, lambda l: kvsynth.layer_inputs(cfg, l))
    mr.score(); mr.select(); mr.compact()
    for l in range(L):
        mr.decode(l)
    torch.cuda.synchronize()
    lens = pu.to_host(mr.seg_len).reshape(L, S)
    off = pu.to_host(mr.seg_off)
    idx = pu.to_host(mr.idx)
    for l in range(L):
        assert np.all(lens[l] == budgets[l]), l
    for g in range(L * S):
        seg = idx[off[g]:off[g] + lens.ravel()[g]]
        assert seg[0] >= 0 and seg[-1] < n and np.all(np.diff(seg) > 0), g
    sc = pu.to_host(mr.scores).reshape(L * S, n)
    kc, vc, out = pu.to_host(mr.k_c), pu.to_host(mr.v_c), pu.to_host(mr.out)
    for l, s in [(0, 0), (7, 13), (19, 5), (31, 31)]:
        b, kvh = divmod(s, cfg.hkv)
        g = l * S + s
        x = kvsynth.segment_inputs(cfg, l, b, kvh)
        ref = oracle.window_scores(oracle.to_f64(x["q_win"]), oracle.to_f64(x["K"]), cfg.scale,
                                   n - w)
        kept = idx[off[g]:off[g] + lens[l, s]].astype(np.int64)
        what = f"layer {l} seg {s}"
        pu.check_scores(sc[g], ref, G * w, what)
        pu.check_topb_selection(kept, sc[g], ref, int(budgets[l]), what)
        pu.check_compact(kc[off[g]:off[g] + len(kept)], vc[off[g]:off[g] + len(kept)], x["K"],
                         x["V"], kept, what)
        pu.check_decode(out[l, b, kvh * G:(kvh + 1) * G], x["q_dec"], x["K"], x["V"], kept,
                        cfg.scale, cfg.dtype, what)
    # LMBA and kept mass of layer 5 (the bench's calibration extra), two segments
    l, B = 5, cfg.batch
    ls, R = mr.layer_shape, G * w
    rows = slice(l * S, (l + 1) * S)
    lm = torch.empty(S * R, dtype=torch.int32, device="cuda")
    km = torch.empty(S * R, dtype=torch.float32, device="cuda")
    ws = torch.empty(kvsel.kvsel_lmba_workspace(ls, w), dtype=torch.uint8, device="cuda")
    kvsel.kvsel_lmba(ls, w, n - w, mr.q_win[l * B:(l + 1) * B], mr.k[l * B:(l + 1) * B], lm, ws,
                     mr.seg_off[rows], mr.seg_len[rows], mr.idx, mr.r_cap, km)
    torch.cuda.synchronize()
    lmh, kmh = pu.to_host(lm).reshape(S, R), pu.to_host(km).reshape(S, R)
    for s in (2, 29):
        b, kvh = divmod(s, cfg.hkv)
        x = kvsynth.segment_inputs(cfg, l, b, kvh)
        P = oracle.window_probabilities(oracle.to_f64(x["q_win"]), oracle.to_f64(x["K"]),
                                        cfg.scale, n - w)
        pu.check_lmba(lmh[s], P, f"layer {l} seg {s}")
        g = l * S + s
        kept = idx[off[g]:off[g] + lens[l, s]].astype(np.int64)
        assert np.max(np.abs(kmh[s] - P[:, kept].sum(axis=1))) <= 1e-5
    # determinism at full size: the whole model's score, select, compact and
    # per-layer decode run a second time give the same bits everywhere
    first = {k: getattr(mr, k).clone() for k in ("scores", "seg_len", "idx", "k_c", "v_c", "out")}
    for t in (mr.scores, mr.idx, mr.k_c, mr.v_c, mr.out):
        t.view(torch.uint8).fill_(0xA5)
    mr.score(); mr.select(); mr.compact()
    for l in range(L):
        mr.decode(l)
    torch.cuda.synchronize()
    for k, t in first.items():
        assert torch.equal(getattr(mr, k).view(torch.uint8), t.view(torch.uint8)), k
    print(f"  {cfg.name}: second full-model run bit-identical (scores, selection, compacted "
          f"K/V, decode outputs)", flush=True)


def test_graph_replays_lmba_vote_rope(kv):
    """The multi-launch entry points under HIP graph capture: kvsel_lmba (rows,
    mask, row select), kvsel_chunk_vote (setup, per-layer select, keys) and the
    fused-RoPE score and decode, captured once and replayed with eager work and
    workspace clobbering in between; every replay equals the eager results bit
    for bit."""
    kvsel, pipeline, torch = kv
    _say("graph replay: lmba, chunk vote, fused RoPE")
    cfg = kvsynth.get_config(1, n=3000)
    inputs, run = _run(kv, cfg)
    S, R = cfg.batch * cfg.hkv, cfg.G * cfg.w
    lm = torch.empty(S * R, dtype=torch.int32, device="cuda")
    km = torch.empty(S * R, dtype=torch.float32, device="cuda")
    lws = torch.empty(kvsel.kvsel_lmba_workspace(run.shape, cfg.w), dtype=torch.uint8, device="cuda")
    # chunk vote over three "layers" of scores (the window scores, scaled differently)
    vsh = kvsel.make_shape(cfg.batch, cfg.hq, cfg.hkv, 64, cfg.n, "bf16", 1.0)
    lay = torch.stack([run.scores, run.scores.flip(0), run.scores * 0.5]).contiguous()
    key = torch.empty(S * cfg.n, dtype=torch.float32, device="cuda")
    vws = torch.empty(kvsel.kvsel_chunk_vote_workspace(vsh, 3, 40), dtype=torch.uint8,
                      device="cuda")
    # fused RoPE score and decode on the same layer (identity pair list)
    tab = pipeline.device_tensor(kvsynth.rope_table(cfg.n + 8, 64))
    pairs = pipeline.device_tensor(np.tile(np.arange(64, dtype=np.int32), (cfg.hkv, 1)))
    sh = run.shape
    fused = kvsel.make_shape(sh.batch, sh.hq, sh.hkv, sh.head_dim, sh.n, sh.dtype, sh.scale,
                             rope=kvsel.make_rope(tab, pairs, q_pos=cfg.n))
    rsc = torch.empty_like(run.scores)
    rws = torch.empty(kvsel.kvsel_score_workspace(fused, cfg.w), dtype=torch.uint8, device="cuda")
    rout = torch.empty_like(run.out)

    def work():
        kvsel.kvsel_lmba(run.shape, cfg.w, cfg.n - cfg.w, run.q_win, run.k, lm, lws,
                         run.seg_off, run.seg_len, run.idx, run.r_cap, km)
        kvsel.kvsel_chunk_vote(vsh, 3, 40, 0, lay, key, vws)
        kvsel.kvsel_score(fused, cfg.w, cfg.n - cfg.w, run.q_win, run.k, rsc, rws)
        kvsel.kvsel_decode_attn(fused, run.q_dec, run.k_c, run.v_c, run.seg_off, run.seg_len,
                                run.r_cap, rout, run.ws_dec)
    outs = (lm, km, key, rsc, rout)
    work()
    torch.cuda.synchronize()
    want = [pu.to_host(t).copy() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    other_inputs, other = _run(kv, kvsynth.get_config(1, n=1111))
    for rep in range(3):
        for t in outs:
            t.zero_()
        for w_ in (lws, vws, rws):
            w_.fill_(0x5A + rep)
        other.run()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, t in enumerate(outs):
            got = pu.to_host(t)
            assert np.array_equal(got.view(np.uint8), want[i].view(np.uint8)), (rep, i)
