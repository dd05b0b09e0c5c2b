"""The C ABI on the host: the library loads, exports every entry point
include/kvsel.h declares, rejects bad arguments before launching anything,
and its host-only budget helper matches the oracle exactly."""
import ctypes
import os
import re

import numpy as np
import pytest

import kvsynth
import oracle
import sparse_decode_attention_window_amd as kvsel
from sparse_decode_attention_window_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "kvsel.h")

FAKE = 0x1000   # never dereferenced: every call below fails its host checks first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvsel_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert "kvsel_score" in names and "kvsel_decode_attn" in names
    lib = kvsel.lib()
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.EXPORTED)


def test_struct_layouts_match_header(tmp_path):
    """The ctypes mirrors of kvsel_shape, kvsel_rope and kvsel_select_params
    have the sizes and field offsets the C compiler gives the header's structs."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = {"kvsel_shape": [f for f, _ in _lib.Shape._fields_],
              "kvsel_rope": [f for f, _ in _lib.Rope._fields_],
              "kvsel_select_params": [f for f, _ in _lib.SelectParams._fields_]}
    lines = []
    for st, fs in fields.items():
        lines.append(f'printf("{st} %zu\\n", sizeof({st}));')
        lines += [f'printf("{st}.{f} %zu\\n", offsetof({st}, {f}));' for f in fs]
    src = tmp_path / "probe.c"
    src.write_text('#include "kvsel.h"\n#include <stdio.h>\n#include <stddef.h>\n'
                   "int main(void) {\n" + "\n".join(lines) + "\nreturn 0;\n}\n")
    exe = tmp_path / "probe"
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    subprocess.run([cc, "-D__HIP_PLATFORM_AMD__", "-I" + os.path.dirname(HEADER),
                    "-I" + os.path.join(rocm, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], check=True, capture_output=True,
                                                       text=True).stdout.splitlines())
    for st, cls in (("kvsel_shape", _lib.Shape), ("kvsel_rope", _lib.Rope),
                    ("kvsel_select_params", _lib.SelectParams)):
        assert int(got[st]) == ctypes.sizeof(cls), st
        for f in fields[st]:
            assert int(got[f"{st}.{f}"]) == getattr(cls, f).offset, (st, f)


def test_version():
    assert "gfx950" in kvsel.kvsel_version()


def shape(**kw):
    base = dict(batch=1, hq=4, hkv=2, head_dim=64, n=512, dtype="fp32", scale=0.125)
    base.update(kw)
    return kvsel.make_shape(**base)


def call_score(sh, w=8, q_pos0=0, q=FAKE, k=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return kvsel.lib().kvsel_score(ctypes.byref(sh), w, q_pos0, q, k, out, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), _lib.KVSEL_EINVAL), (dict(hq=3), _lib.KVSEL_EINVAL),
    (dict(n=0), _lib.KVSEL_EINVAL), (dict(head_dim=96), _lib.KVSEL_EUNSUPPORTED),
    (dict(dtype=7), _lib.KVSEL_EUNSUPPORTED), (dict(scale=float("inf")), _lib.KVSEL_EINVAL),
    (dict(scale=0.0), _lib.KVSEL_EINVAL), (dict(scale=-0.125), _lib.KVSEL_EINVAL),
    (dict(scale=float("nan")), _lib.KVSEL_EINVAL),
    (dict(batch=2049, hkv=1, hq=1), _lib.KVSEL_EUNSUPPORTED)])
def test_score_rejects_bad_shape(kw, code):
    assert call_score(shape(**kw)) == code
    assert kvsel.kvsel_last_error()


def test_score_rejects_bad_args():
    sh = shape()
    assert call_score(sh, w=0) == _lib.KVSEL_EINVAL
    assert call_score(sh, w=200) == _lib.KVSEL_EUNSUPPORTED      # G*w = 400 rows
    assert call_score(sh, q_pos0=-1) == _lib.KVSEL_EINVAL
    assert call_score(sh, q=None) == _lib.KVSEL_EINVAL
    need = kvsel.kvsel_score_workspace(sh, 8)
    assert need > 0
    assert call_score(sh, ws_bytes=need - 1) == _lib.KVSEL_ENOSPC
    assert "workspace" in kvsel.kvsel_last_error()


def test_select_rejects_bad_args():
    sh = shape()
    lib = kvsel.lib()

    def sel(p, scores=FAKE, off=FAKE, ln=FAKE, ix=FAKE, r_cap=10):
        return lib.kvsel_select(ctypes.byref(sh), ctypes.byref(p), scores, off, ln, ix, r_cap, None)

    topb = _lib.SelectParams(mode=0, budget=FAKE)
    assert sel(_lib.SelectParams(mode=0, budget=None)) == _lib.KVSEL_EINVAL
    assert sel(topb, scores=None) == _lib.KVSEL_EINVAL
    assert sel(topb, r_cap=-1) == _lib.KVSEL_EINVAL
    assert sel(topb, off=None) == _lib.KVSEL_EINVAL
    assert sel(_lib.SelectParams(mode=1, chunk_end=FAKE, n_chunks=0)) == _lib.KVSEL_EINVAL
    assert sel(_lib.SelectParams(mode=1, chunk_end=FAKE, n_chunks=513)) == _lib.KVSEL_EINVAL
    assert sel(_lib.SelectParams(mode=2, head_kind=FAKE, local_window=-1)) == _lib.KVSEL_EINVAL
    assert sel(_lib.SelectParams(mode=2, head_kind=FAKE, n_special=3)) == _lib.KVSEL_EINVAL
    assert sel(_lib.SelectParams(mode=9)) == _lib.KVSEL_EINVAL


def test_compact_and_decode_reject_bad_args():
    sh = shape()
    lib = kvsel.lib()
    assert lib.kvsel_compact(ctypes.byref(sh), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 4,
                             None) == _lib.KVSEL_EINVAL
    assert lib.kvsel_compact(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -4,
                             None) == _lib.KVSEL_EINVAL
    need = kvsel.kvsel_decode_workspace(sh, 100)
    assert need > 0
    assert lib.kvsel_decode_attn(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 100, FAKE, FAKE,
                                 need - 1, None) == _lib.KVSEL_ENOSPC
    big_group = shape(hq=32, hkv=2)   # G = 16: decode is built for groups of up to 8
    assert lib.kvsel_decode_attn(ctypes.byref(big_group), FAKE, FAKE, FAKE, FAKE, FAKE, 100, FAKE,
                                 FAKE, 1 << 30, None) == _lib.KVSEL_EUNSUPPORTED
    assert "exceeds 8" in kvsel.kvsel_last_error()


def test_lmba_rejects_bad_args():
    sh = shape()
    lib = kvsel.lib()
    need = kvsel.kvsel_lmba_workspace(sh, 8)
    assert need >= 2 * (2 * 8) * 512 * 4       # holds the fp32 attention rows

    def lm(w=8, q_pos0=0, out=FAKE, km=None, off=None, ws_bytes=1 << 40):
        return lib.kvsel_lmba(ctypes.byref(sh), w, q_pos0, FAKE, FAKE, out, off, None, None, 0,
                              km, FAKE, ws_bytes, None)
    assert lm(w=0) == _lib.KVSEL_EINVAL
    assert lm(w=200) == _lib.KVSEL_EUNSUPPORTED
    assert lm(q_pos0=-1) == _lib.KVSEL_EINVAL
    assert lm(out=None) == _lib.KVSEL_EINVAL
    assert lm(km=FAKE) == _lib.KVSEL_EINVAL        # kept mass without a selection
    assert lm(ws_bytes=need - 1) == _lib.KVSEL_ENOSPC


def test_lmba_kept_mass_lds_limit():
    """With kept_mass, the n-bit position mask and the row kernel's own LDS
    (its bins, candidate list and block-scan words: 45,488 bytes with slack for
    rows longer than 32768 keys) must fit one workgroup's LDS.  At the limit
    the call passes the check (and fails on the too-small workspace); one
    mask word more is refused as unsupported, before anything is enqueued."""
    import torch
    max_lds = 163840 if torch.cuda.is_available() else 65536   # gfx950, or no device
    words = (max_lds - 45488) // 4
    lib = kvsel.lib()

    def lm(n):
        sh = shape(n=n)
        return lib.kvsel_lmba(ctypes.byref(sh), 8, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1,
                              FAKE, FAKE, 16, None)
    assert lm(32 * words) == _lib.KVSEL_ENOSPC
    assert lm(32 * words + 32) == _lib.KVSEL_EUNSUPPORTED
    assert "position mask" in kvsel.kvsel_last_error()


def test_chunk_vote_rejects_bad_args():
    sh = shape(n=100)
    lib = kvsel.lib()
    need = kvsel.kvsel_chunk_vote_workspace(sh, 4, 16)
    assert need >= 4 * 2 * 16 * 4                  # the layers' ballots

    def vote(layers=4, k=16, sc=FAKE, key=FAKE, ws_bytes=1 << 30, local=0):
        return lib.kvsel_chunk_vote(ctypes.byref(sh), layers, k, local, sc, key, FAKE, ws_bytes,
                                    None)
    assert vote(layers=0) == _lib.KVSEL_EINVAL
    assert vote(layers=256) == _lib.KVSEL_EINVAL
    assert vote(k=0) == _lib.KVSEL_EINVAL
    assert vote(local=-1) == _lib.KVSEL_EINVAL
    assert vote(sc=None) == _lib.KVSEL_EINVAL
    assert vote(key=None) == _lib.KVSEL_EINVAL
    assert vote(ws_bytes=need - 1) == _lib.KVSEL_ENOSPC
    big = shape(n=1 << 20)
    assert lib.kvsel_chunk_vote(ctypes.byref(big), 4, 16, 0, FAKE, FAKE, FAKE, 1 << 40,
                                None) == _lib.KVSEL_EUNSUPPORTED


def test_append_rejects_bad_args():
    sh = shape()
    lib = kvsel.lib()

    def app(k_new=FAKE, seg_cap=FAKE, pos=600, r_cap=16, k_c=FAKE):
        return lib.kvsel_append(ctypes.byref(sh), k_new, FAKE, pos, FAKE, seg_cap, None, FAKE,
                                FAKE, k_c, FAKE, r_cap, None)
    assert app(k_new=None) == _lib.KVSEL_EINVAL
    assert app(seg_cap=None) == _lib.KVSEL_EINVAL
    assert app(k_c=None) == _lib.KVSEL_EINVAL
    assert app(pos=-1) == _lib.KVSEL_EINVAL
    assert app(pos=1 << 31) == _lib.KVSEL_EINVAL
    assert app(r_cap=-1) == _lib.KVSEL_EINVAL
    assert app(r_cap=0) == _lib.KVSEL_OK          # an empty cache: nothing to do, nothing launched
    assert lib.kvsel_append(ctypes.byref(shape(head_dim=96)), FAKE, FAKE, 1, FAKE, FAKE, None,
                            FAKE, FAKE, FAKE, FAKE, 16, None) == _lib.KVSEL_EUNSUPPORTED


def test_rope_rejects_bad_descriptors():
    """RoPE descriptor checks run before any launch: missing table or pair list,
    half below head_dim/2, and positions outside the table."""
    lib = kvsel.lib()

    def rope(**kw):
        base = dict(cos_sin=FAKE, max_pos=1024, half=32, pairs=FAKE, q_pos=10)
        base.update(kw)
        return _lib.Rope(**base)

    def score(r, w=8, q_pos0=0):
        sh = shape(rope=r)
        return lib.kvsel_score(ctypes.byref(sh), w, q_pos0, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert score(rope(cos_sin=None)) == _lib.KVSEL_EINVAL
    assert score(rope(pairs=None)) == _lib.KVSEL_EINVAL
    assert score(rope(half=31)) == _lib.KVSEL_EINVAL            # head_dim 64 keeps 32 pairs
    assert score(rope(max_pos=0)) == _lib.KVSEL_EINVAL
    assert score(rope(), q_pos0=1017) == _lib.KVSEL_EINVAL      # rows reach position 1024
    sh = shape(rope=rope(q_pos=1024))
    assert lib.kvsel_decode_attn(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, FAKE,
                                 1 << 30, None) == _lib.KVSEL_EINVAL
    sh = shape(rope=rope())
    assert lib.kvsel_append(ctypes.byref(sh), FAKE, FAKE, 1024, FAKE, FAKE, None, FAKE, FAKE,
                            FAKE, FAKE, 16, None) == _lib.KVSEL_EINVAL
    sh = shape(rope=rope(q_pos=-1))
    assert lib.kvsel_decode_attn(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, FAKE,
                                 1 << 30, None) == _lib.KVSEL_EINVAL


# ---------------------------------------------------------------------------
# host budget helper vs the oracle (ZigZagkv page, Eq. 4 + Eq. 6): exact
# ---------------------------------------------------------------------------

def test_budgets_c2_profile_exact():
    cfg = kvsynth.get_config(2)
    p = kvsynth.zigzag_profile(cfg)
    got = kvsel.kvsel_zigzag_budgets(p, cfg.n, cfg.avg_budget, cfg.floor_budget)
    want = oracle.zigzag_budgets(p, cfg.n, cfg.avg_budget, cfg.floor_budget)
    assert got == want.tolist()


@pytest.mark.parametrize("seed", range(200))
def test_budgets_random_exact(seed):
    r = np.random.default_rng(1000 + seed)
    L = int(r.integers(1, 64))
    n = int(r.integers(1, 200000))
    B = int(r.integers(0, n + 1))
    F = int(r.integers(0, B + 1))
    p = r.lognormal(0, float(r.uniform(0.05, 3.0)), size=L)
    if seed % 7 == 0:
        p = np.round(p, 1) + 0.1          # ties in the profile
    got = kvsel.kvsel_zigzag_budgets(p, n, B, F)
    want = oracle.zigzag_budgets(p, n, B, F)
    assert got == want.tolist()


def test_budgets_reject():
    with pytest.raises(kvsel.KvselError):
        kvsel.kvsel_zigzag_budgets([1.0, 2.0], 100, 10, 11)
    with pytest.raises(kvsel.KvselError):
        kvsel.kvsel_zigzag_budgets([1.0, -2.0], 100, 10, 1)
    with pytest.raises(kvsel.KvselError):
        kvsel.kvsel_zigzag_budgets([], 100, 10, 1)


def test_decode_noalloc_rejects_bad_args():
    """The allocation-free decode checks its arguments like kvsel_decode_attn
    and refuses, before anything is enqueued, a call whose partials exceed
    the static scratch."""
    sh = shape(dtype="bf16", head_dim=128, batch=4, hq=32, hkv=8, n=32768)
    lib = kvsel.lib()

    def call(s=sh, q=FAKE, kc=FAKE, out=FAKE, r_cap=1000):
        return lib.kvsel_decode_attn_noalloc(ctypes.byref(s), q, kc, FAKE, FAKE, FAKE, r_cap, out,
                                             None)
    assert call(q=None) == _lib.KVSEL_EINVAL
    assert call(out=None) == _lib.KVSEL_EINVAL
    assert call(kc=None) == _lib.KVSEL_EINVAL
    assert call(r_cap=-1) == _lib.KVSEL_EINVAL
    assert call(s=shape(hq=32, hkv=2)) == _lib.KVSEL_EUNSUPPORTED
    assert call(r_cap=(1 << 31) - 1) == _lib.KVSEL_ENOSPC
    assert "static scratch" in kvsel.kvsel_last_error()
