"""kvsel_decode_attn_noalloc against kvsel_decode_attn through the C ABI (needs
an MI355X): the allocation-free entry point runs the same kernels with its
partials in the library's static scratch, so its output must equal the
workspace entry point's bit for bit; calls in a row, each smaller than the one
before, show that nothing left in the shared scratch leaks into the next call."""
import sys

import numpy as np
import pytest

import kvsynth
from tests import parity_util as pu

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _layer(cfg, layer=0, budget=None):
    import torch
    from sparse_decode_attention_window_amd import pipeline
    run = pipeline.build_layer(cfg, kvsynth.layer_inputs(cfg, layer), budget=budget)
    run.run()
    torch.cuda.synchronize()
    return run


def test_decode_noalloc_matches_workspace_entry():
    import torch
    import sparse_decode_attention_window_amd as kvsel
    assert torch.cuda.is_available()
    kvsel.lib()
    # each call smaller than the one before; the middle one has eight query heads
    # per KV head (the decode's largest head group)
    cases = [kvsynth.get_config(2, batch=2, n=5000 + 77),
             kvsynth.get_config(1, hq=64, n=3000 + 37, budget=333), kvsynth.get_config(0)]
    for cfg in cases:
        _say("decode noalloc", cfg.name, "n", cfg.n, "batch", cfg.batch)
        bl = pu.zigzag_layer_budgets(cfg)[3] if cfg.mode == "topb" and cfg.layers > 1 else None
        run = _layer(cfg, budget=bl)
        want = pu.to_host(run.out).copy()
        got = torch.full_like(run.out, float("nan"))
        kvsel.kvsel_decode_attn_noalloc(run.shape, run.q_dec, run.k_c, run.v_c, run.seg_off,
                                        run.seg_len, run.r_cap, got)
        torch.cuda.synchronize()
        g = pu.to_host(got)
        assert np.all(np.isfinite(g))
        assert np.array_equal(g.view(np.uint32), want.view(np.uint32)), cfg.name
        # twice in a row on the same inputs: the scratch holds the last call's
        # partials, which the next call overwrites before reading
        got2 = torch.zeros_like(run.out)
        kvsel.kvsel_decode_attn_noalloc(run.shape, run.q_dec, run.k_c, run.v_c, run.seg_off,
                                        run.seg_len, run.r_cap, got2)
        torch.cuda.synchronize()
        assert np.array_equal(pu.to_host(got2).view(np.uint32), want.view(np.uint32)), cfg.name
        print(f"  {cfg.name}: {run.r_cap} rows, noalloc output identical", flush=True)
