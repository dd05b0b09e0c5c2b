"""kvsel for MI355X (gfx950): attention-mass KV token selection and decode
attention over the compacted cache, as hand-written HIP kernels behind a C ABI
(include/kvsel.h).  This package is the thin Python binding over that library;
see `_lib` for the entry points."""
from ._lib import (  # noqa: F401
    EXPORTED,
    KVSEL_BF16,
    KVSEL_FP32,
    KVSEL_HEAD_GLOBAL,
    KVSEL_HEAD_LOCAL,
    KVSEL_HEAD_SPECIAL,
    KVSEL_SEL_CHUNK,
    KVSEL_SEL_POLICY,
    KVSEL_SEL_TOPB,
    KvselError,
    Shape,
    SelectParams,
    kvsel_append,
    kvsel_compact,
    kvsel_decode_attn,
    kvsel_decode_workspace,
    kvsel_last_error,
    kvsel_lmba,
    kvsel_lmba_workspace,
    kvsel_score,
    kvsel_score_workspace,
    kvsel_select,
    kvsel_version,
    kvsel_zigzag_budgets,
    lib,
    make_shape,
    select_params,
)
