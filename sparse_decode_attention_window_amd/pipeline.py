"""One layer of the hot path through the C ABI: score -> select -> compact ->
decode.  PyTorch only allocates the device buffers; every step runs in the
HIP kernels behind libkvsel.so.

Capacity layout of the packed cache (caller-chosen, as the C ABI requires):
segment s = b * hkv + kvh gets rows [seg_off[s], seg_off[s] + cap[s]) with
  TOPB    cap = min(budget, n)
  CHUNK   cap = min(n, keep_tokens + longest chunk - 1)  (a chunk prefix that
          first reaches keep_tokens overshoots by less than one chunk)
  POLICY  cap = n (global), min(local_window, n) (local), n_special (special)
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import _lib as K


def device_tensor(arr: np.ndarray, device="cuda"):
    """Upload a numpy array; uint16 arrays are bf16 words and become bfloat16."""
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def capacities(mode: int, batch: int, hkv: int, n: int, *, budget=None, keep_tokens=0,
               max_chunk=0, head_kind=None, local_window=0, n_special=0, local_chunks=0,
               top_chunks=0) -> np.ndarray:
    """Rows reserved per segment (int64 [batch*hkv])."""
    S = batch * hkv
    if mode == K.KVSEL_SEL_TOPB:
        cap = np.minimum(np.maximum(np.asarray(budget, np.int64).reshape(S), 0), n)
    elif mode == K.KVSEL_SEL_CHUNK:
        local = local_chunks * max_chunk
        if top_chunks > 0:
            rows = min(n, (local_chunks + top_chunks) * max_chunk)
        else:
            rows = 0 if keep_tokens <= 0 and local == 0 else \
                min(n, max(keep_tokens + max(0, max_chunk - 1), local))
        cap = np.full(S, rows, np.int64)
    else:
        per_kind = {K.KVSEL_HEAD_GLOBAL: n, K.KVSEL_HEAD_LOCAL: min(local_window, n),
                    K.KVSEL_HEAD_SPECIAL: n_special}
        kinds = np.asarray(head_kind).reshape(hkv)
        cap = np.array([per_kind.get(int(kinds[s % hkv]), n) for s in range(S)], np.int64)
    return cap


def offsets(cap: np.ndarray) -> tuple[np.ndarray, int]:
    off = np.zeros(cap.size, np.int64)
    off[1:] = np.cumsum(cap)[:-1]
    return off, int(cap.sum())


@dataclass
class LayerRun:
    """Device buffers of one layer and the calls that fill them."""
    shape: K.Shape
    k: object
    v: object
    q_dec: object
    mode: int
    r_cap: int
    seg_off: object
    seg_cap: object = None                 # rows reserved per segment (int64)
    w: int = 0
    q_pos0: int = 0
    q_win: object = None
    score_shape: K.Shape | None = None     # chunk keys use their own shape
    score_keys: object = None               # keys that kvsel_score reads
    params: K.SelectParams | None = None
    keep: list = field(default_factory=list)   # tensors the params point at
    scores: object = None
    seg_len: object = None
    idx: object = None
    k_c: object = None
    v_c: object = None
    out: object = None
    ws_score: object = None
    ws_dec: object = None

    def allocate(self):
        import torch
        dev = self.k.device
        S = self.shape.batch * self.shape.hkv
        if self.q_win is not None:
            ss = self.score_shape or self.shape
            self.scores = torch.empty(ss.batch * ss.hkv * ss.n, dtype=torch.float32, device=dev)
            nb = K.kvsel_score_workspace(ss, self.w)
            self.ws_score = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        self.seg_len = torch.empty(S, dtype=torch.int32, device=dev)
        self.idx = torch.empty(max(self.r_cap, 1), dtype=torch.int32, device=dev)
        d = self.shape.head_dim
        self.k_c = torch.empty((max(self.r_cap, 1), d), dtype=self.k.dtype, device=dev)
        self.v_c = torch.empty((max(self.r_cap, 1), d), dtype=self.k.dtype, device=dev)
        self.out = torch.empty((self.shape.batch, self.shape.hq, d), dtype=torch.float32,
                               device=dev)
        nb = K.kvsel_decode_workspace(self.shape, self.r_cap)
        self.ws_dec = torch.zeros(max(nb, 1), dtype=torch.uint8, device=dev)
        return self

    def score(self, stream=None):
        if self.q_win is not None:
            K.kvsel_score(self.score_shape or self.shape, self.w, self.q_pos0, self.q_win,
                          self.score_keys if self.score_keys is not None else self.k,
                          self.scores, self.ws_score, stream)

    def select(self, stream=None):
        K.kvsel_select(self.shape, self.params, self.scores, self.seg_off, self.seg_len, self.idx,
                       self.r_cap, stream)

    def compact(self, stream=None):
        K.kvsel_compact(self.shape, self.k, self.v, self.seg_off, self.seg_len, self.idx,
                        self.k_c, self.v_c, self.r_cap, stream)

    def decode(self, stream=None):
        K.kvsel_decode_attn(self.shape, self.q_dec, self.k_c, self.v_c, self.seg_off,
                            self.seg_len, self.r_cap, self.out, self.ws_dec, stream)

    def append(self, k_new, v_new, pos: int, limit=None, stream=None):
        """Add one decoded token to every segment under its head rule (limit)."""
        K.kvsel_append(self.shape, k_new, v_new, pos, self.seg_off, self.seg_cap, limit,
                       self.seg_len, self.idx, self.k_c, self.v_c, self.r_cap, stream)

    def run(self, stream=None):
        self.score(stream)
        self.select(stream)
        self.compact(stream)
        self.decode(stream)
        return self


def build_layer(cfg, inputs: dict, *, budget=None, slack: int = 0, local_chunks: int = 0,
                top_chunks: int = 0, device="cuda") -> LayerRun:
    """LayerRun for one synthetic layer (cfg: a kvsynth Config, inputs: layer_inputs()).
    `slack` extra rows per segment leave room for tokens appended while decoding;
    `local_chunks` / `top_chunks` select the chunk-selection options (chunk mode)."""
    import torch
    B, hq, hkv, d, n = cfg.batch, cfg.hq, cfg.hkv, cfg.d, cfg.n
    shape = K.make_shape(B, hq, hkv, d, n, cfg.dtype, cfg.scale)
    k = device_tensor(inputs["K"], device)
    v = device_tensor(inputs["V"], device)
    qd = device_tensor(inputs["q_dec"], device)
    keep = []
    if cfg.mode == "topb":
        mode = K.KVSEL_SEL_TOPB
        bud = np.full(B * hkv, cfg.budget, np.int32) if budget is None else \
            np.broadcast_to(np.asarray(budget, np.int32), (B * hkv,)).copy()
        cap = capacities(mode, B, hkv, n, budget=bud)
        bt = device_tensor(bud, device)
        keep.append(bt)
        params = K.select_params(mode, budget=bt)
        run = LayerRun(shape, k, v, qd, mode, 0, None, w=cfg.w, q_pos0=n - cfg.w,
                       q_win=device_tensor(inputs["q_win"], device), params=params)
    elif cfg.mode == "chunk":
        mode = K.KVSEL_SEL_CHUNK
        ends = np.asarray(inputs["chunk_end"], np.int64)
        nc = ends.shape[1]
        cap = capacities(mode, B, hkv, n, keep_tokens=cfg.keep_tokens,
                         max_chunk=int(np.diff(np.concatenate([np.zeros((B, 1), np.int64), ends],
                                                              axis=1)).max()),
                         local_chunks=local_chunks, top_chunks=top_chunks)
        et = device_tensor(ends, device)
        keep.append(et)
        params = K.select_params(mode, n_chunks=nc, chunk_end=et, keep_tokens=cfg.keep_tokens,
                                 local_chunks=local_chunks, top_chunks=top_chunks)
        sshape = K.make_shape(B, hq, hkv, cfg.chunk_dim, nc, cfg.dtype, cfg.scale)
        run = LayerRun(shape, k, v, qd, mode, 0, None, w=1, q_pos0=nc - 1,
                       q_win=device_tensor(inputs["chunk_q"], device), score_shape=sshape,
                       score_keys=device_tensor(inputs["chunk_keys"], device), params=params)
    else:
        mode = K.KVSEL_SEL_POLICY
        kinds = np.asarray(inputs["head_kind"], np.int8)
        sp = np.asarray(inputs["special_pos"], np.int32)
        cap = capacities(mode, B, hkv, n, head_kind=kinds, local_window=cfg.local_window,
                         n_special=sp.shape[1])
        kt, st = device_tensor(kinds, device), device_tensor(sp, device)
        keep += [kt, st]
        params = K.select_params(mode, head_kind=kt, local_window=cfg.local_window,
                                 special_pos=st, n_special=sp.shape[1])
        run = LayerRun(shape, k, v, qd, mode, 0, None, params=params)
    cap = cap + int(slack)
    off, r_cap = offsets(cap)
    run.seg_off = device_tensor(off, device)
    run.seg_cap = device_tensor(cap.astype(np.int64), device)
    run.r_cap = r_cap
    run.keep = keep
    return run.allocate()


@dataclass
class ServingLoop:
    """Decode-time maintenance of one layer's selection (ZigZagkv: the token
    score is the attention of the last w queries, Eq. 7; FastGen: the per-head
    rule keeps holding while generating).  The full cache stays resident in
    HBM; every step the new token joins it and the compacted cache, and the
    decode reads the compacted cache; every `period` steps the score is taken
    again from the last w decode queries over the full cache and the
    selection and compaction are redone from it.  `period` == w, so the
    window buffer holds exactly the queries of the last period, in order.

    All arithmetic runs in the library's kernels (append, decode, score,
    select, compact); this class only owns buffers and orders the calls.
    """
    run: LayerRun            # the compacted cache (TOPB), slack >= period
    n0: int                  # tokens before the first decode step
    k_full: object = None    # [b][hkv][n_cap][d], rows >= current length zero
    v_full: object = None
    full_shape: K.Shape | None = None
    full_off: object = None
    full_cap: object = None
    full_len: object = None
    full_idx: object = None
    q_buf: object = None     # [b][hq][w][d]: the last w decode queries
    period: int = 0
    t: int = 0
    reselections: int = 0

    @staticmethod
    def start(run: LayerRun, k, v, n0: int, steps: int) -> "ServingLoop":
        """Full cache of n0 tokens (k, v: [b][hkv][n0][d] device tensors) with
        room for `steps` more; the compacted run must already hold a selection."""
        import torch
        sh = run.shape
        B, hkv, d, w = sh.batch, sh.hkv, sh.head_dim, run.w
        assert run.mode == K.KVSEL_SEL_TOPB and w >= 1 and run.q_win is not None
        assert not sh.rope, "the loop takes rotated queries and keys"
        n_cap = n0 + steps
        S = B * hkv
        kf = torch.zeros((B, hkv, n_cap, d), dtype=k.dtype, device=k.device)
        vf = torch.zeros_like(kf)
        kf[:, :, :n0] = k.view(B, hkv, n0, d)
        vf[:, :, :n0] = v.view(B, hkv, n0, d)
        full_shape = K.make_shape(B, sh.hq, hkv, d, n_cap, sh.dtype, sh.scale)
        off = device_tensor(np.arange(S, dtype=np.int64) * n_cap, k.device)
        cap = device_tensor(np.full(S, n_cap, np.int64), k.device)
        ln = device_tensor(np.full(S, n0, np.int32), k.device)
        idx = device_tensor(np.tile(np.arange(n_cap, dtype=np.int32), S), k.device)
        loop = ServingLoop(run, n0, kf, vf, full_shape, off, cap, ln, idx, period=w)
        loop.q_buf = torch.zeros((B, sh.hq, w, d), dtype=k.dtype, device=k.device)
        # scores and score workspace sized for the full cache
        run.scores = torch.empty(S * n_cap, dtype=torch.float32, device=k.device)
        run.ws_score = torch.empty(max(K.kvsel_score_workspace(full_shape, w), 1),
                                   dtype=torch.uint8, device=k.device)
        return loop

    def step(self, k_new, v_new, q, stream=None):
        """Decode step at position n0 + t: k_new, v_new [b][hkv][d], q [b][hq][d].
        Returns True when the selection was redone after this step's decode."""
        run = self.run
        sh = run.shape
        pos = self.n0 + self.t
        full = self.full_shape
        K.kvsel_append(full, k_new, v_new, pos, self.full_off, self.full_cap, None,
                       self.full_len, self.full_idx, self.k_full.view(-1, sh.head_dim),
                       self.v_full.view(-1, sh.head_dim), self.full_len.numel() * full.n, stream)
        K.kvsel_append(sh, k_new, v_new, pos, run.seg_off, run.seg_cap, None, run.seg_len,
                       run.idx, run.k_c, run.v_c, run.r_cap, stream)
        self.q_buf[:, :, self.t % self.period].copy_(q.view(sh.batch, sh.hq, sh.head_dim))
        K.kvsel_decode_attn(sh, q, run.k_c, run.v_c, run.seg_off, run.seg_len, run.r_cap,
                            run.out, run.ws_dec, stream)
        self.t += 1
        if self.t % self.period:
            return False
        # re-score from the last w queries (positions pos-w+1 .. pos) over the full cache;
        # keys past pos are masked by the causal window and score 0
        K.kvsel_score(self.full_shape, run.w, pos - run.w + 1, self.q_buf, self.k_full,
                      run.scores, run.ws_score, stream)
        K.kvsel_select(self.full_shape, run.params, run.scores, run.seg_off, run.seg_len,
                       run.idx, run.r_cap, stream)
        K.kvsel_compact(self.full_shape, self.k_full, self.v_full, run.seg_off, run.seg_len,
                        run.idx, run.k_c, run.v_c, run.r_cap, stream)
        self.reselections += 1
        return True


@dataclass
class ChunkServingLoop:
    """ChunkLLM decode loop (ChunkLLM page, §2.3: by intra-chunk attention
    consistency the chunk selection is redone only when the current token
    closes a chunk).  The full cache stays resident; every step the new token
    joins it and the compacted cache and the decode reads the compacted
    cache.  When the token closes a chunk, its chunk key joins the chunk keys,
    the chunks are scored with this step's chunk query, the `local` last
    chunks plus the `top` best others are selected, and the compacted cache is
    rebuilt from the full cache.  All arithmetic runs in the library's
    kernels; this class owns buffers and orders the calls (the torch copies
    below only move data into the layouts the calls take)."""
    run: LayerRun                 # chunk mode, count form (top_chunks > 0)
    n0: int
    local: int
    top: int
    k_full: object = None
    v_full: object = None
    full_shape: K.Shape | None = None
    full_off: object = None
    full_cap: object = None
    full_len: object = None
    full_idx: object = None
    ck: object = None             # chunk keys [b][hkv][nc_cap][chunk_dim]
    ends: object = None           # chunk ends [b][nc_cap] int64
    ck_shape: K.Shape | None = None
    sc: object = None             # chunk scores [b*hkv][nc_cap]
    sc_c: object = None           # the same, [b*hkv][nc] contiguous for select
    ends_c: object = None
    ws: object = None
    nc: int = 0
    t: int = 0
    reselections: int = 0

    @staticmethod
    def start(run: LayerRun, k, v, n0: int, steps: int, chunk_keys, ends: np.ndarray,
              local: int, top: int) -> "ChunkServingLoop":
        """k, v [b][hkv][n0][d] and chunk_keys [b][hkv][nc0][chunk_dim] device
        tensors, ends [b][nc0] host int64 (last == n0); the run must hold the
        selection over them; `steps` bounds the tokens and chunks to come."""
        import torch
        sh, ss = run.shape, run.score_shape
        B, hkv, d = sh.batch, sh.hkv, sh.head_dim
        assert run.mode == K.KVSEL_SEL_CHUNK and top > 0 and not sh.rope
        S = B * hkv
        n_cap, nc0 = n0 + steps, ends.shape[1]
        nc_cap = nc0 + steps
        kf = torch.zeros((B, hkv, n_cap, d), dtype=k.dtype, device=k.device)
        vf = torch.zeros_like(kf)
        kf[:, :, :n0] = k.view(B, hkv, n0, d)
        vf[:, :, :n0] = v.view(B, hkv, n0, d)
        lp = ChunkServingLoop(run, n0, local, top, kf, vf,
                              K.make_shape(B, sh.hq, hkv, d, n_cap, sh.dtype, sh.scale),
                              device_tensor(np.arange(S, dtype=np.int64) * n_cap, k.device),
                              device_tensor(np.full(S, n_cap, np.int64), k.device),
                              device_tensor(np.full(S, n0, np.int32), k.device),
                              device_tensor(np.tile(np.arange(n_cap, dtype=np.int32), S),
                                            k.device))
        cd = ss.head_dim
        lp.ck = torch.zeros((B, hkv, nc_cap, cd), dtype=k.dtype, device=k.device)
        lp.ck[:, :, :nc0] = chunk_keys.view(B, hkv, nc0, cd)
        e = np.zeros((B, nc_cap), np.int64)
        e[:, :nc0] = ends
        lp.ends = device_tensor(e, k.device)
        lp.ck_shape = K.make_shape(B, ss.hq, hkv, cd, nc_cap, ss.dtype, ss.scale)
        lp.sc = torch.empty(S * nc_cap, dtype=torch.float32, device=k.device)
        lp.sc_c = torch.empty_like(lp.sc)
        lp.ends_c = torch.empty_like(lp.ends).view(-1)
        lp.ws = torch.empty(max(K.kvsel_score_workspace(lp.ck_shape, 1), 1), dtype=torch.uint8,
                            device=k.device)
        lp.nc = nc0
        return lp

    def step(self, k_new, v_new, q, boundary: bool, chunk_key=None, chunk_q=None,
             stream=None) -> bool:
        """Decode step at position n0 + t.  When `boundary`, chunk_key
        [b][hkv][chunk_dim] and chunk_q [b][hq][1][chunk_dim] are the closing
        token's chunk key and chunk query.  Returns True when the selection was
        redone (after this step's decode)."""
        run, sh = self.run, self.run.shape
        pos = self.n0 + self.t
        B, hkv = sh.batch, sh.hkv
        S = B * hkv
        K.kvsel_append(self.full_shape, k_new, v_new, pos, self.full_off, self.full_cap, None,
                       self.full_len, self.full_idx, self.k_full.view(-1, sh.head_dim),
                       self.v_full.view(-1, sh.head_dim), S * self.full_shape.n, stream)
        K.kvsel_append(sh, k_new, v_new, pos, run.seg_off, run.seg_cap, None, run.seg_len,
                       run.idx, run.k_c, run.v_c, run.r_cap, stream)
        K.kvsel_decode_attn(sh, q, run.k_c, run.v_c, run.seg_off, run.seg_len, run.r_cap,
                            run.out, run.ws_dec, stream)
        self.t += 1
        if not boundary:
            return False
        nc_cap = self.ends.shape[1]
        assert self.nc < nc_cap
        self.ends[:, self.nc] = pos + 1
        self.ck[:, :, self.nc].copy_(chunk_key.view(B, hkv, -1))
        self.nc += 1
        nc = self.nc
        # chunk attention of this step's chunk query over the nc chunk keys (the
        # causal window masks the free key slots)
        K.kvsel_score(self.ck_shape, 1, nc - 1, chunk_q, self.ck, self.sc, self.ws, stream)
        self.sc_c[:S * nc].view(S, nc).copy_(self.sc.view(S, nc_cap)[:, :nc])
        self.ends_c[:B * nc].view(B, nc).copy_(self.ends[:, :nc])
        params = K.select_params(K.KVSEL_SEL_CHUNK, n_chunks=nc, chunk_end=self.ends_c,
                                 local_chunks=self.local, top_chunks=self.top)
        K.kvsel_select(self.full_shape, params, self.sc_c, run.seg_off, run.seg_len, run.idx,
                       run.r_cap, stream)
        K.kvsel_compact(self.full_shape, self.k_full, self.v_full, run.seg_off, run.seg_len,
                        run.idx, run.k_c, run.v_c, run.r_cap, stream)
        self.reselections += 1
        return True


@dataclass
class ModelRun:
    """Every layer of a top-B model in one layout, so that the compression
    step (score, select, compact) can run as one call each for the whole model
    (L*b*hkv segments fill the chip where one layer's b*hkv do not) while the
    decode stays one call per layer, as a model runs it.

    Segment g = l*S + s of layer l (s = b*hkv + kvh): keys and values
    [L*b][hkv][n][d] (layer-major), window queries [L*b][hq][w][d], scores
    [L*S][n], one packed cache in which layer l's segments occupy rows
    [base[l], base[l] + r_caps[l]).  seg_off holds absolute rows (select,
    compact, append); seg_off_rel[l] the rows relative to base[l] (decode,
    which sizes its launch from one layer's rows)."""
    L: int
    shape: K.Shape
    layer_shape: K.Shape
    k: object
    v: object
    q_win: object
    q_dec: object
    w: int
    q_pos0: int
    budget: object
    params: K.SelectParams
    seg_off: object
    seg_cap: object
    seg_off_rel: list
    base: list
    r_caps: list
    r_cap: int
    scores: object = None
    ws_score: object = None
    ws_score_layer: object = None
    seg_len: object = None
    idx: object = None
    k_c: object = None
    v_c: object = None
    out: object = None
    ws_dec: object = None
    keep: list = field(default_factory=list)

    @staticmethod
    def build(cfg, budgets, inputs_of, device="cuda", log=None) -> "ModelRun":
        """cfg: a top-B kvsynth Config; budgets [L] per-layer budgets;
        inputs_of(l) -> kvsynth.layer_inputs(cfg, l) (called once per layer)."""
        import torch
        assert cfg.mode == "topb"
        L, B, hq, hkv, d, n, w = cfg.layers, cfg.batch, cfg.hq, cfg.hkv, cfg.d, cfg.n, cfg.w
        S = B * hkv
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        k = torch.empty((L * B, hkv, n, d), dtype=tdt, device=device)
        v = torch.empty_like(k)
        q_win = torch.empty((L * B, hq, w, d), dtype=tdt, device=device)
        q_dec = torch.empty((L, B, hq, d), dtype=tdt, device=device)
        for l in range(L):
            inp = inputs_of(l)
            k[l * B:(l + 1) * B] = device_tensor(inp["K"], device)
            v[l * B:(l + 1) * B] = device_tensor(inp["V"], device)
            q_win[l * B:(l + 1) * B] = device_tensor(inp["q_win"], device)
            q_dec[l] = device_tensor(inp["q_dec"], device)
            del inp
            if log:
                log(l)
        bud = np.repeat(np.asarray(budgets, np.int32), S)
        cap = capacities(K.KVSEL_SEL_TOPB, L * B, hkv, n, budget=bud)
        off, r_cap = offsets(cap)
        base = [int(off[l * S]) for l in range(L)]
        r_caps = [int(cap[l * S:(l + 1) * S].sum()) for l in range(L)]
        shape = K.make_shape(L * B, hq, hkv, d, n, cfg.dtype, cfg.scale)
        layer_shape = K.make_shape(B, hq, hkv, d, n, cfg.dtype, cfg.scale)
        bt = device_tensor(bud, device)
        run = ModelRun(L, shape, layer_shape, k, v, q_win, q_dec, w, n - w, bt,
                       K.select_params(K.KVSEL_SEL_TOPB, budget=bt),
                       device_tensor(off, device), device_tensor(cap.astype(np.int64), device),
                       [device_tensor(off[l * S:(l + 1) * S] - base[l], device) for l in range(L)],
                       base, r_caps, r_cap)
        run.keep = [bt]
        run.scores = torch.empty(L * S * n, dtype=torch.float32, device=device)
        run.ws_score = torch.empty(K.kvsel_score_workspace(shape, w), dtype=torch.uint8,
                                   device=device)
        run.ws_score_layer = torch.empty(K.kvsel_score_workspace(layer_shape, w),
                                         dtype=torch.uint8, device=device)
        run.seg_len = torch.empty(L * S, dtype=torch.int32, device=device)
        run.idx = torch.empty(max(r_cap, 1), dtype=torch.int32, device=device)
        run.k_c = torch.empty((max(r_cap, 1), d), dtype=tdt, device=device)
        run.v_c = torch.empty_like(run.k_c)
        run.out = torch.empty((L, B, hq, d), dtype=torch.float32, device=device)
        nb = max(K.kvsel_decode_workspace(layer_shape, rc) for rc in r_caps)
        run.ws_dec = torch.zeros(max(nb, 1), dtype=torch.uint8, device=device)
        return run

    # ---- the whole model, one call each ----------------------------------
    def score(self, stream=None):
        K.kvsel_score(self.shape, self.w, self.q_pos0, self.q_win, self.k, self.scores,
                      self.ws_score, stream)

    def select(self, stream=None):
        K.kvsel_select(self.shape, self.params, self.scores, self.seg_off, self.seg_len,
                       self.idx, self.r_cap, stream)

    def compact(self, stream=None):
        K.kvsel_compact(self.shape, self.k, self.v, self.seg_off, self.seg_len, self.idx,
                        self.k_c, self.v_c, self.r_cap, stream)

    # ---- one layer -------------------------------------------------------
    def _rows(self, l):
        S = self.layer_shape.batch * self.layer_shape.hkv
        return slice(l * S, (l + 1) * S)

    def decode(self, l, stream=None):
        b0 = self.base[l]
        K.kvsel_decode_attn(self.layer_shape, self.q_dec[l], self.k_c[b0:], self.v_c[b0:],
                            self.seg_off_rel[l], self.seg_len[self._rows(l)], self.r_caps[l],
                            self.out[l], self.ws_dec, stream)

    def score_layer(self, l, stream=None):
        B, n = self.layer_shape.batch, self.layer_shape.n
        r = self._rows(l)
        K.kvsel_score(self.layer_shape, self.w, self.q_pos0, self.q_win[l * B:(l + 1) * B],
                      self.k[l * B:(l + 1) * B], self.scores[r.start * n:r.stop * n],
                      self.ws_score_layer, stream)

    def select_layer(self, l, stream=None):
        n = self.layer_shape.n
        r = self._rows(l)
        prm = K.select_params(K.KVSEL_SEL_TOPB, budget=self.budget[r])
        K.kvsel_select(self.layer_shape, prm, self.scores[r.start * n:r.stop * n],
                       self.seg_off[r], self.seg_len[r], self.idx, self.r_cap, stream)

    def compact_layer(self, l, stream=None):
        B = self.layer_shape.batch
        r = self._rows(l)
        K.kvsel_compact(self.layer_shape, self.k[l * B:(l + 1) * B], self.v[l * B:(l + 1) * B],
                        self.seg_off[r], self.seg_len[r], self.idx, self.k_c, self.v_c,
                        self.r_cap, stream)

    def append_layer(self, l, k_new, v_new, pos: int, limit=None, stream=None):
        r = self._rows(l)
        K.kvsel_append(self.layer_shape, k_new, v_new, pos, self.seg_off[r], self.seg_cap[r],
                       limit, self.seg_len[r], self.idx, self.k_c, self.v_c, self.r_cap, stream)


@dataclass
class ModelServingLoop:
    """ServingLoop for every layer of a top-B model at once (the same reading of
    ZigZagkv Eq. 7 and FastGen's rules as ServingLoop).  Each step runs layer
    by layer, as a model does: the new token joins layer l's full and
    compacted caches and layer l decodes.  Every `period` steps the
    re-selection of all layers is one score, one select and one compact call
    over the L*b*hkv segments (the layout of ModelRun), so it fills the chip
    where one layer's b*hkv segments do not.  Same kernels and data as one
    ServingLoop per layer, so the same bits."""
    L: int
    B: int
    S: int
    n0: int
    period: int
    layer_shape: K.Shape = None      # one layer, compacted cache
    full_layer_shape: K.Shape = None  # one layer, full cache (n = capacity)
    full_shape: K.Shape = None       # every layer's full cache (batch L*b)
    k_full: object = None            # [L*b][hkv][n_cap][d]
    v_full: object = None
    full_off: object = None
    full_cap: object = None
    full_len: object = None
    full_idx: object = None
    q_buf: object = None             # [L*b][hq][w][d]
    params: K.SelectParams = None
    budget: object = None
    seg_off: object = None           # [L*S] absolute rows of the packed cache
    seg_cap: object = None
    seg_len: object = None
    idx: object = None
    k_c: object = None
    v_c: object = None
    r_cap: int = 0
    base: list = field(default_factory=list)
    r_caps: list = field(default_factory=list)
    seg_off_rel: list = field(default_factory=list)
    scores: object = None
    ws_score: object = None
    ws_dec: object = None
    out: object = None               # [L][b][hq][d]
    t: int = 0
    reselections: int = 0

    @staticmethod
    def start(cfg, budgets, k, v, q_win, steps: int, device="cuda") -> "ModelServingLoop":
        """k, v [L*b][hkv][n0][d], q_win [L*b][hq][w][d] (the prompt's last w
        queries of every layer); room for `steps` decoded tokens.  The first
        selection of every layer is made here from q_win."""
        import torch
        L, B, hq, hkv, d, w = cfg.layers, cfg.batch, cfg.hq, cfg.hkv, cfg.d, cfg.w
        n0 = k.shape[2]
        S = B * hkv
        n_cap = n0 + steps
        kf = torch.zeros((L * B, hkv, n_cap, d), dtype=k.dtype, device=device)
        vf = torch.zeros_like(kf)
        kf[:, :, :n0] = k
        vf[:, :, :n0] = v
        lp = ModelServingLoop(L, B, S, n0, w)
        lp.layer_shape = K.make_shape(B, hq, hkv, d, n_cap, cfg.dtype, cfg.scale)
        lp.full_layer_shape = lp.layer_shape
        lp.full_shape = K.make_shape(L * B, hq, hkv, d, n_cap, cfg.dtype, cfg.scale)
        lp.k_full, lp.v_full = kf, vf
        lp.full_off = device_tensor(np.arange(L * S, dtype=np.int64) * n_cap, device)
        lp.full_cap = device_tensor(np.full(L * S, n_cap, np.int64), device)
        lp.full_len = device_tensor(np.full(L * S, n0, np.int32), device)
        lp.full_idx = device_tensor(np.tile(np.arange(n_cap, dtype=np.int32), L * S), device)
        lp.q_buf = q_win.clone()
        bud = np.repeat(np.asarray(budgets, np.int32), S)
        cap = capacities(K.KVSEL_SEL_TOPB, L * B, hkv, n_cap, budget=bud) + w
        off, r_cap = offsets(cap)
        lp.base = [int(off[l * S]) for l in range(L)]
        lp.r_caps = [int(cap[l * S:(l + 1) * S].sum()) for l in range(L)]
        lp.seg_off_rel = [device_tensor(off[l * S:(l + 1) * S] - lp.base[l], device)
                          for l in range(L)]
        lp.budget = device_tensor(bud, device)
        lp.params = K.select_params(K.KVSEL_SEL_TOPB, budget=lp.budget)
        lp.seg_off = device_tensor(off, device)
        lp.seg_cap = device_tensor(cap.astype(np.int64), device)
        lp.r_cap = r_cap
        lp.seg_len = torch.empty(L * S, dtype=torch.int32, device=device)
        lp.idx = torch.empty(max(r_cap, 1), dtype=torch.int32, device=device)
        lp.k_c = torch.empty((max(r_cap, 1), d), dtype=k.dtype, device=device)
        lp.v_c = torch.empty_like(lp.k_c)
        lp.scores = torch.empty(L * S * n_cap, dtype=torch.float32, device=device)
        lp.ws_score = torch.empty(max(K.kvsel_score_workspace(lp.full_shape, w), 1),
                                  dtype=torch.uint8, device=device)
        nb = max(K.kvsel_decode_workspace(lp.layer_shape, rc) for rc in lp.r_caps)
        lp.ws_dec = torch.zeros(max(nb, 1), dtype=torch.uint8, device=device)
        lp.out = torch.empty((L, B, hq, d), dtype=torch.float32, device=device)
        lp.reselect(n0 - w)
        lp.reselections = 0
        return lp

    def reselect(self, q_pos0: int, stream=None):
        """Score every layer's keys from its window buffer, select and compact:
        one call each for all L*b*hkv segments."""
        K.kvsel_score(self.full_shape, self.period, q_pos0, self.q_buf, self.k_full,
                      self.scores, self.ws_score, stream)
        K.kvsel_select(self.full_shape, self.params, self.scores, self.seg_off, self.seg_len,
                       self.idx, self.r_cap, stream)
        K.kvsel_compact(self.full_shape, self.k_full, self.v_full, self.seg_off, self.seg_len,
                        self.idx, self.k_c, self.v_c, self.r_cap, stream)
        self.reselections += 1

    def step_layer(self, l: int, k_new, v_new, q, stream=None):
        """Layer l of the decode step at position n0 + t: k_new, v_new
        [b][hkv][d], q [b][hq][d]."""
        sh = self.layer_shape
        S, B, d = self.S, self.B, sh.head_dim
        pos = self.n0 + self.t
        r = slice(l * S, (l + 1) * S)
        K.kvsel_append(sh, k_new, v_new, pos, self.full_off[r], self.full_cap[r], None,
                       self.full_len[r], self.full_idx, self.k_full.view(-1, d),
                       self.v_full.view(-1, d), self.full_len.numel() * sh.n, stream)
        K.kvsel_append(sh, k_new, v_new, pos, self.seg_off[r], self.seg_cap[r], None,
                       self.seg_len[r], self.idx, self.k_c, self.v_c, self.r_cap, stream)
        self.q_buf[l * B:(l + 1) * B, :, self.t % self.period].copy_(q.view(B, sh.hq, d))
        b0 = self.base[l]
        K.kvsel_decode_attn(sh, q, self.k_c[b0:], self.v_c[b0:], self.seg_off_rel[l],
                            self.seg_len[r], self.r_caps[l], self.out[l], self.ws_dec, stream)

    def end_step(self, stream=None) -> bool:
        """After every layer's step_layer: advance; every `period` steps redo
        every layer's selection.  Returns True when it did."""
        pos = self.n0 + self.t
        self.t += 1
        if self.t % self.period:
            return False
        self.reselect(pos - self.period + 1, stream)
        return True
