"""Checks of the seeded input generator (shared by the oracle side and the HIP
side; it holds no selection or attention arithmetic)."""
import math

import numpy as np
import pytest

import kvsynth
import oracle
from kvsynth import gen


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -2.5, 3.0e38], np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1); 1 + 1.5 * 2^-8 rounds up
    want = np.array([0x3F80, 0x3F80, 0x3F81, 0x3F81, 0xC020, 0x7F62], np.uint16)
    assert np.array_equal(kvsynth.f32_to_bf16_bits(x), want)
    assert np.array_equal(kvsynth.bf16_bits_to_f32(want)[:5],
                          np.array([1.0, 1.0, 1.0078125, 1.0078125, -2.5], np.float32))


def test_segments_regenerate_bit_identically():
    cfg = kvsynth.get_config(1, n=1024)
    full = kvsynth.layer_inputs(cfg, threads=3)
    seg = kvsynth.segment_inputs(cfg, 0, 0, 5)
    assert np.array_equal(full["K"][0, 5], seg["K"])
    assert np.array_equal(full["V"][0, 5], seg["V"])
    assert np.array_equal(full["q_win"][0, 20:24], seg["q_win"])
    assert np.array_equal(full["q_dec"][0, 20:24], seg["q_dec"])


def test_c1_planted_structure_ranks_high():
    # sink and heavy hitters carry +3u against queries 2u + noise: they must
    # land in the top-1024 of the window score for a C1 segment
    cfg = kvsynth.get_config(1)
    seg = kvsynth.segment_inputs(cfg, 0, 0, 3)
    s = oracle.window_scores(oracle.to_f64(seg["q_win"]), oracle.to_f64(seg["K"]), cfg.scale,
                             cfg.n - cfg.w)
    top = set(oracle.select_topb(s, cfg.budget).tolist())
    hh = gen.heavy_hitters(cfg, 0, 0, 3)
    assert len(hh) == 82
    assert 0 in top
    assert np.mean([h in top for h in hh]) > 0.9


def test_c2_layer_fractions_in_range():
    cfg = kvsynth.get_config(2)
    fr = [gen.layer_hh_frac(cfg, l) for l in range(cfg.layers)]
    assert min(fr) >= 0.005 and max(fr) <= 0.04 and np.std(fr) > 0.003


def test_c3_policy_inputs():
    cfg = kvsynth.get_config(3)
    kinds = kvsynth.head_kinds(cfg)
    assert sorted(kinds.tolist()) == [0, 0, 1, 1, 1, 2, 2, 2]
    sp = kvsynth.special_positions(cfg, 5)
    assert sp.size == 656 and sp[0] == 0 and np.all(np.diff(sp) > 0) and sp[-1] < cfg.n
    rows = {0: cfg.n, 1: cfg.local_window, 2: sp.size}
    assert sum(rows[int(k)] for k in kinds) == 73648


def test_c4_chunk_boundaries():
    cfg = kvsynth.get_config(4)
    e = kvsynth.chunk_ends(cfg)
    assert e[-1] == cfg.n and np.all(np.diff(e) > 0) and e[0] >= 1
    assert abs(cfg.n / e.size - 32) < 2
    assert cfg.keep_tokens == 62915


def test_rap_pair_pruned_logits_equal_masked_full_logits():
    # RAP page (§3, Fig. 3): pruning whole RoPE pairs keeps each 2x2 rotation,
    # so the 88-dim dot product equals the 128-dim one with pruned pairs zeroed
    r = np.random.default_rng(0)
    pairs = np.sort(r.choice(64, 44, replace=False))
    k = gen.rope_rotate(r.standard_normal((10, 128)), np.arange(10))
    q = gen.rope_rotate(r.standard_normal((3, 128)), np.full(3, 10))
    mask = np.zeros(128); mask[pairs] = 1; mask[pairs + 64] = 1
    lhs = gen.prune_pairs(q, pairs, 64) @ gen.prune_pairs(k, pairs, 64).T
    rhs = q @ (k * mask).T
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)


def test_rap_rope_commutes_with_pair_expansion():
    # RoPE(X A) B = RoPE(X A B) for A keeping whole pairs and B its binary expansion
    r = np.random.default_rng(1)
    pairs = np.sort(r.choice(64, 44, replace=False))
    cols = np.concatenate([pairs, pairs + 64])
    W = r.standard_normal((32, 128))
    A = W[:, cols]                                  # 32 x 88 kept columns
    Bexp = np.zeros((88, 128)); Bexp[np.arange(88), cols] = 1
    X = r.standard_normal((7, 32))
    pos = np.arange(7) * 13

    def rope_pruned(Y):
        # rotate the 88-dim layout at the kept pairs' own frequencies
        theta = gen.ROPE_BASE ** (-pairs / 64.0)
        ang = pos[:, None] * theta
        a, b = Y[:, :44], Y[:, 44:]
        return np.concatenate([a * np.cos(ang) - b * np.sin(ang),
                               a * np.sin(ang) + b * np.cos(ang)], axis=1)

    lhs = rope_pruned(X @ A) @ Bexp
    rhs = gen.rope_rotate(X @ A @ Bexp, pos)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)
