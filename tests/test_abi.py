"""C-ABI contract on the host: the library loads, exports every declared
symbol, and rejects bad arguments with the documented status before any launch
(these calls make no HIP call, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

from long_context_attention_csa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa_hip.h")

OK, NULL, SHAPE, UNSUP, WS = 0, 1, 2, 3, 4
P = ctypes.c_void_p(0x1000)   # a non-NULL pointer that is never dereferenced (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), set(names) ^ set(_lib.SIGNATURES)


def test_status_strings():
    lib = _lib.lib()
    assert lib.csa_status_string(0) == b"CSA_OK"
    assert lib.csa_status_string(4) == b"CSA_ERR_WORKSPACE"
    assert b"gfx950" in lib.csa_version()


def _err(lib):
    return lib.csa_last_error().decode()


def test_compress_validation():
    lib = _lib.lib()
    assert lib.csa_compress(P, P, P, P, 1, 1, 64, 96, 4, P, 1, None, None) == UNSUP      # width
    assert "width" in _err(lib)
    assert lib.csa_compress(P, P, P, P, 2, 1, 64, 128, 4, P, 1, None, None) == UNSUP     # fp8 input
    assert lib.csa_compress(P, P, P, P, 1, 1, 64, 128, 0, P, 1, None, None) == SHAPE     # ratio 0
    assert lib.csa_compress(P, P, P, P, 1, -1, 64, 128, 4, P, 1, None, None) == SHAPE    # B < 0
    assert lib.csa_compress(None, P, P, P, 1, 1, 64, 128, 4, P, 1, None, None) == NULL
    assert lib.csa_compress(P, P, P, P, 1, 1, 64, 128, 4, P, 2, None, None) == NULL      # fp8 without scale
    assert lib.csa_compress(P, P, P, P, 1, 1, 64, 128, 4, P, 1, P, None) == SHAPE        # scale for bf16 out
    assert lib.csa_compress(None, None, None, None, 1, 1, 3, 128, 4, None, 1, None, None) == OK  # nothing to do
    assert lib.hca_compress(P, P, 1, 1, 256, 128, 0, P, 1, None) == SHAPE
    assert lib.hca_compress(P, P, 1, 1, 256, 128, 128, P, 2, None) == UNSUP
    assert lib.csa_quantize_rows(P, 1, 4, 48, P, 3, P, None) == SHAPE                   # fp4 width % 32
    assert lib.csa_quantize_rows(P, 1, 4, 64, P, 1, P, None) == UNSUP


def test_indexer_validation():
    lib = _lib.lib()
    args = lambda **kw: dict(dict(q=P, qs=P, w=P, k=P, ks=P, fmt=2, pos=P, B=1, Tq=1, N=64, H=64, d=128, ratio=4,
                                  kk=16, out=P, so=None, ws=P, wsb=1 << 40), **kw)
    call = lambda a: lib.indexer_topk(a["q"], a["qs"], a["w"], a["k"], a["ks"], a["fmt"], a["pos"], a["B"], a["Tq"],
                                      a["N"], a["H"], a["d"], a["ratio"], a["kk"], a["out"], a["so"], a["ws"],
                                      a["wsb"], None)
    assert call(args(kk=0)) == SHAPE
    assert call(args(kk=2049)) == SHAPE
    assert call(args(H=65)) == UNSUP
    assert call(args(d=96)) == UNSUP
    assert call(args(qs=None)) == NULL
    assert call(args(fmt=0)) == SHAPE              # scales given for float operands
    assert call(args(fmt=7)) == UNSUP
    assert call(args(ws=None)) == WS
    need = lib.indexer_topk_workspace_size(1, 1, 64, 64, 128, 16, 2)
    assert need > 0 and call(args(wsb=need - 1)) == WS
    assert call(args(B=0)) == OK


def test_indexer_bf16_scores_validation():
    """The bfloat16-score entry point validates like indexer_topk and stores two
    bytes per score instead of four."""
    lib = _lib.lib()
    args = lambda **kw: dict(dict(q=P, qs=P, w=P, k=P, ks=P, fmt=2, pos=P, B=1, Tq=1, N=64, H=64, d=128, ratio=4,
                                  kk=16, out=P, so=None, ws=P, wsb=1 << 40), **kw)
    call = lambda a: lib.indexer_topk_bf16_scores(a["q"], a["qs"], a["w"], a["k"], a["ks"], a["fmt"], a["pos"],
                                                  a["B"], a["Tq"], a["N"], a["H"], a["d"], a["ratio"], a["kk"],
                                                  a["out"], a["so"], a["ws"], a["wsb"], None)
    assert call(args(kk=0)) == SHAPE
    assert call(args(H=65)) == UNSUP
    assert call(args(qs=None)) == NULL
    assert call(args(fmt=7)) == UNSUP
    assert call(args(ws=None)) == WS
    need = lib.indexer_topk_bf16_scores_workspace_size(1, 1, 64, 64, 128, 16, 2)
    assert need > 0 and call(args(wsb=need - 1)) == WS
    assert call(args(B=0)) == OK
    assert lib.indexer_topk_bf16_scores_workspace_size(0, 1, 64, 64, 128, 16, 2) == 0
    # rows that fit one pass of either variant: half the score bytes
    small = (1, 64, 1 << 16, 64, 128, 512, 2)
    f32 = lib.indexer_topk_workspace_size(*small)
    b16 = lib.indexer_topk_bf16_scores_workspace_size(*small)
    assert 0 < b16 < f32 and f32 - b16 == 64 * (1 << 16) * 2
    # a pass's score buffer is capped (1 GiB): the bf16 variant fits twice the rows in about the same space
    big = (1, 8192, 1 << 18, 64, 128, 1024, 2)
    assert abs(lib.indexer_topk_bf16_scores_workspace_size(*big) - lib.indexer_topk_workspace_size(*big)) < 1 << 24
    assert call(args(d=96)) == UNSUP
    assert lib.csa_last_error().startswith(b"indexer_topk_bf16_scores:")


def test_attention_validation():
    lib = _lib.lib()
    f = lib.sparse_attn_fwd
    #       q  kv idx xw ws0 sink pos t  B  Tq N   T_win ring H   d    k   win  scale out lse ws  wsb      stream
    base = [P, P, P, P, P, None, P, 1, 1, 1, 64, 128, 0, 64, 128, 64, 128, 1.0, P, None, P, 1 << 40, None]
    def call(**kw):
        a = list(base)
        pos = {"t": 7, "ring": 12, "H": 13, "d": 14, "k": 15, "window": 16, "q": 0, "ws": 20, "wsb": 21, "idx": 2}
        for k_, v in kw.items():
            a[pos[k_]] = v
        return f(*a)
    assert call(d=64) == UNSUP
    assert call(H=24) == UNSUP
    assert call(t=2) == UNSUP
    assert call(k=0) == SHAPE
    assert call(window=-1) == SHAPE
    assert call(ring=2) == SHAPE
    assert call(q=None) == NULL
    assert call(idx=None) == NULL
    g = lib.dense_compressed_attn_fwd
    assert g(P, P, P, P, None, P, 1, 1, 1, 64, 128, 0, 64, 128, 0, 128, 1.0, P, None, P, 1 << 40, None) == SHAPE
    assert g(P, P, P, P, None, P, 1, 1, 1, 64, 128, -1, 64, 128, 4, 128, 1.0, P, None, P, 1 << 40, None) == SHAPE
    # decode shapes need a split workspace
    need = lib.dense_attn_workspace_size(1, 1, 8192, 128, 128, 128)
    assert need > 0
    assert g(P, P, P, P, None, P, 1, 1, 1, 8192, 128, 1, 128, 128, 128, 128, 1.0, P, None, None, 0, None) == WS


def test_window_append_validation():
    lib = _lib.lib()
    f = lib.csa_window_append
    assert f(P, 2, 2, 128, P, P, 128, None) == UNSUP         # fp8 rows
    assert f(P, 1, 2, 64, P, P, 128, None) == UNSUP          # d != 128
    assert f(P, 1, 2, 128, P, P, 0, None) == SHAPE           # empty ring
    assert f(None, 1, 2, 128, P, P, 128, None) == NULL
    assert f(ctypes.c_void_p(0x1008), 1, 2, 128, P, P, 128, None) == SHAPE   # misaligned
    assert f(P, 1, 0, 128, None, None, 128, None) == OK      # B = 0: nothing to do


def test_timer_validation():
    lib = _lib.lib()
    assert lib.csa_kernel_timer_start(0, 4) == SHAPE
    assert lib.csa_kernel_timer_start(4, 0) == SHAPE


def test_append_validation():
    lib = _lib.lib()
    # width 96 unsupported; ratio 0; fp8 cache without its scale; NULL state
    assert lib.csa_compress_append(P, P, P, P, 1, 2, 96, 4, P, P, 10, P, 1, None, None) == UNSUP
    assert lib.csa_compress_append(P, P, P, P, 1, 2, 128, 0, P, P, 10, P, 1, None, None) == SHAPE
    assert lib.csa_compress_append(P, P, P, P, 1, 2, 128, 4, P, P, 10, P, 2, None, None) == NULL
    assert lib.csa_compress_append(P, P, P, P, 1, 2, 128, 4, P, None, 10, P, 1, None, None) == NULL
    assert lib.csa_compress_append(P, P, P, P, 1, 0, 128, 4, None, None, 10, None, 1, None, None) == OK
    assert lib.hca_compress_append(P, P, 1, 2, 128, 128, P, P, 10, P, 2, None) == UNSUP   # fp8 output
    assert lib.hca_compress_append(P, P, 1, 2, 128, 0, P, P, 10, P, 1, None) == SHAPE
    assert lib.hca_compress_append(P, P, 1, 2, 128, 128, None, P, 10, P, 1, None) == NULL


def test_batch_invariant_switch():
    """Host logic of the batch-invariant mode: the switch, and the attention
    workspace of a decode batch that plans each sequence's splits alone."""
    from long_context_attention_csa_amd import ops
    assert not ops.batch_invariant()
    default8 = ops.dense_attn_workspace_size(8, 1, 8192, 128, 128, 128)
    one = ops.dense_attn_workspace_size(1, 1, 8192, 128, 128, 128)
    ops.set_batch_invariant(True)
    try:
        assert ops.batch_invariant()
        assert ops.dense_attn_workspace_size(8, 1, 8192, 128, 128, 128) == 8 * one
        assert ops.sparse_attn_workspace_size(8, 1, 128, 128, 1024, 128) == \
            8 * ops.sparse_attn_workspace_size(1, 1, 128, 128, 1024, 128)
    finally:
        ops.set_batch_invariant(False)
    assert not ops.batch_invariant()
    assert ops.dense_attn_workspace_size(8, 1, 8192, 128, 128, 128) == default8


def test_backward_workspace_passes():
    """The backward's workspace holds at most 4 GiB of per-(query, key)
    gradient rows: it grows with the query rows until that budget, then the
    rows run in passes and the workspace stays bounded."""
    lib = _lib.lib()
    ws = lambda Tq: lib.sparse_attn_bwd_workspace_size(1, Tq, 16384, Tq, 64, 128, 512, 128)
    small, mid, big = ws(64), ws(4096), ws(65536)
    assert 0 < small < mid < big
    assert mid >= 4096 * 640 * 512                     # every row's slots fit one pass
    assert big < 5 * (1 << 30)                          # 65,536 rows: passes, bounded buffer
    assert lib.sparse_attn_bwd_workspace_size(0, 1, 16, 16, 64, 128, 8, 128) == 0
    # dense layers: contribution rows for the window slots only (the entries'
    # gradients are summed per block of entries and segment of query rows)
    d = lambda Tq, N, T_win: lib.dense_attn_bwd_workspace_size(1, Tq, N, T_win, 64, 128, 128)
    assert 64 * 128 * 512 < d(64, 65536, 256) < 64 * 65536 * 512
    assert d(131072, 1024, 131072) < 6 * (1 << 30)      # 4 GiB of window rows per pass + segment partials
