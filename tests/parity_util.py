"""Helpers for the GPU-vs-oracle parity tests (imported by tests only)."""
from __future__ import annotations

import os

import numpy as np

import kvsynth
import oracle

# Bars: scores relative (fp32 arithmetic against fp64), outputs max-abs per dtype.
SCORE_RTOL = 1e-5
TIE_BAND = 1e-5
OUT_ATOL = {"fp32": 1e-5, "bf16": 1e-2}


# Largest margin each test reached, per kind (written out by conftest at the
# end of a session that ran GPU tests): score relative error, decode max-abs
# error per dtype, selection entries that differ inside the tie band, LMBA
# counts off the float64 row's own count (inside the band).
MARGINS: dict = {}


def record(kind: str, value) -> None:
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    d = MARGINS.setdefault(test, {})
    d[kind] = max(d.get(kind, 0), value)


def to_host(t) -> np.ndarray:
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def zigzag_layer_budgets(cfg) -> np.ndarray:
    return oracle.zigzag_budgets(kvsynth.zigzag_profile(cfg), cfg.n, cfg.avg_budget,
                                 cfg.floor_budget)


def check_scores(s_gpu: np.ndarray, s_ref: np.ndarray, rows: int, what: str) -> float:
    """Elementwise relative check; returns the max relative error seen."""
    s_gpu = s_gpu.astype(np.float64)
    err = np.abs(s_gpu - s_ref)
    tol = SCORE_RTOL * np.abs(s_ref) + 1e-30
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, (f"{what}: {bad.size} scores off, first j={bad[0]} gpu={s_gpu[bad[0]]!r} "
                           f"ref={s_ref[bad[0]]!r}")
    assert abs(s_gpu.sum() - rows) < 1e-4 * rows, f"{what}: mass {s_gpu.sum()} != {rows}"
    nz = s_ref > 0
    rel = float(np.max(err[nz] / s_ref[nz])) if nz.any() else 0.0
    record("score_rel", rel)
    return rel


def check_topb_selection(idx_gpu: np.ndarray, s_gpu: np.ndarray, s_ref: np.ndarray, budget: int,
                         what: str) -> None:
    n = s_ref.size
    B = max(0, min(budget, n))
    assert idx_gpu.size == B, f"{what}: kept {idx_gpu.size}, want {B}"
    assert np.all(np.diff(idx_gpu) > 0), f"{what}: kept indices not strictly ascending"
    # exact: same fp32 scores give exactly one answer
    want = oracle.select_topb(s_gpu.astype(np.float64), B)
    assert np.array_equal(idx_gpu, want), f"{what}: select differs from the oracle on GPU scores"
    # end to end: differences to the fp64 selection only inside the tie band
    if B == 0 or B == n:
        return
    ref = oracle.select_topb(s_ref, B)
    diff = np.setxor1d(ref, idx_gpu)
    if diff.size:
        sB = np.sort(s_ref)[::-1][B - 1]
        out = diff[np.abs(s_ref[diff] - sB) > TIE_BAND * abs(sB)]
        assert out.size == 0, f"{what}: {out.size} selections differ outside the tie band"
        record("tie_band_diffs", int(diff.size))


def check_chunk_selection(idx_gpu, cs_gpu, cs_ref, ends, keep, what, local=0, top=0):
    want = oracle.select_chunks(cs_gpu.astype(np.float64), ends, keep, local, top)
    assert np.array_equal(idx_gpu, want), f"{what}: chunk select differs on GPU scores"
    ref = oracle.select_chunks(cs_ref, ends, keep, local, top)
    if np.array_equal(ref, idx_gpu):
        return
    chunk_of = lambda toks: set(np.searchsorted(ends, toks, side="right").tolist())
    nc = len(ends)
    forced = set(range(nc - min(local, nc), nc))
    cg, cr = chunk_of(idx_gpu) - forced, chunk_of(ref) - forced
    assert cr, f"{what}: selections differ with only forced chunks kept"
    last = max(cr, key=lambda c: (-cs_ref[c], c))
    band = TIE_BAND * abs(cs_ref[last])
    for c in cg ^ cr:
        assert abs(cs_ref[c] - cs_ref[last]) <= band, f"{what}: chunk {c} differs outside band"
    record("tie_band_diffs", len(cg ^ cr))


def check_voted_selection(idx_gpu, layer_scores, ends, local, top, what):
    """ChunkLLM layer-wise vote: the kept tokens against the plain rule
    (oracle.vote_chunks) on the same fp32 layer scores.  The ballots are then
    identical; the GPU sums the layers in fp32, so a chunk may differ from
    the oracle's choice only when it has the boundary's vote count and its
    float64 summed attention lies within the tie band of the boundary's."""
    sc = np.asarray(layer_scores, np.float64)
    want = oracle.vote_chunks(sc, top, ends, local)
    if np.array_equal(idx_gpu, want):
        return 0
    chunk_of = lambda toks: set(np.searchsorted(ends, toks, side="right").tolist())
    nc = len(ends)
    forced = set(range(nc - min(local, nc), nc))
    votes, total = oracle.chunk_votes(sc, top)
    cg, cr = chunk_of(idx_gpu) - forced, chunk_of(want) - forced
    assert len(cg) == len(cr), f"{what}: kept {len(cg)} voted chunks, want {len(cr)}"
    last = min(cr, key=lambda c: (votes[c], total[c], -c))
    band = TIE_BAND * abs(total[last])
    for c in cg ^ cr:
        assert votes[c] == votes[last] and abs(total[c] - total[last]) <= band, (
            f"{what}: chunk {c} (votes {votes[c]}, sum {total[c]!r}) differs from the rule "
            f"outside the tie band (boundary votes {votes[last]}, sum {total[last]!r})")
    record("tie_band_diffs", len(cg ^ cr))
    return len(cg ^ cr)


def check_compact(kc_gpu, vc_gpu, K, V, idx, what):
    kr, vr = oracle.compact(K, V, idx)
    assert np.array_equal(kc_gpu, kr) and np.array_equal(vc_gpu, vr), f"{what}: compaction not exact"


def check_decode(out_gpu, q_dec, K, V, idx, scale, dtype, what) -> float:
    """out_gpu [G][d] against the oracle over the rows idx; returns max abs error."""
    Kc, Vc = oracle.compact(oracle.to_f64(K), oracle.to_f64(V), idx)
    qd = oracle.to_f64(q_dec)
    err = 0.0
    for g in range(qd.shape[0]):
        ref = oracle.decode_attention(qd[g], Kc, Vc, scale)
        err = max(err, float(np.max(np.abs(out_gpu[g].astype(np.float64) - ref))) if ref.size else 0)
    assert err <= OUT_ATOL[dtype], f"{what}: decode max-abs error {err}"
    record(f"decode_abs_{dtype}", err)
    return err


def check_lmba(k_gpu, P_rows, what, eps=1e-5):
    """GPU per-row LMBA against float64 attention rows: the count must lie in
    the band of counts whose top-k mass reaches 0.9 of the row within a
    relative eps (fp32 rows and fixed-point masses on the GPU)."""
    off_center = 0
    for r, row in enumerate(np.asarray(P_rows)):
        cum = np.cumsum(np.sort(row)[::-1])
        tot = cum[-1]
        lo = int(np.searchsorted(cum, 0.9 * (1 - eps) * tot)) + 1
        hi = int(np.searchsorted(cum, 0.9 * (1 + eps) * tot)) + 1
        assert lo <= int(k_gpu[r]) <= hi, f"{what} row {r}: lmba {k_gpu[r]} outside [{lo}, {hi}]"
        exact = int(np.searchsorted(cum, 0.9 * tot)) + 1
        off_center += int(int(k_gpu[r]) != exact)
    record("lmba_rows", len(P_rows))
    record("lmba_off_center", off_center)
