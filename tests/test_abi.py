"""C-ABI contract on the host: the library loads, exports every declared
symbol, and rejects bad arguments with the documented status before any launch
(these calls make no HIP call, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

from long_context_attention_csa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("csa_hip.h", "csa_hip_timer.h")]

OK, NULL, SHAPE, UNSUP, WS = 0, 1, 2, 3, 4
P = ctypes.c_void_p(0x1000)   # a non-NULL pointer that is never dereferenced (validation fails first)


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
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
    #       q  kv idx xw ws0 sink pos t  B  Tq N   T_win H   d    k   win  scale out lse ws  wsb      flags stream
    base = [P, P, P, P, P, None, P, 1, 1, 1, 64, 128, 64, 128, 64, 128, 1.0, P, None, P, 1 << 40, 0, None]
    def call(**kw):
        a = list(base)
        pos = {"t": 7, "H": 12, "d": 13, "k": 14, "window": 15, "scale": 16, "q": 0, "ws": 19, "wsb": 20,
               "flags": 21, "idx": 2}
        for k_, v in kw.items():
            a[pos[k_]] = v
        return f(*a)
    assert call(d=64) == UNSUP
    assert call(H=24) == UNSUP
    assert call(t=2) == UNSUP
    assert call(k=0) == SHAPE
    assert call(window=-1) == SHAPE
    assert call(flags=4) == SHAPE      # unknown option bit
    assert "flags" in _err(lib)
    assert call(q=None) == NULL
    assert call(idx=None) == NULL
    # the softmax scale must be finite and positive (keys are masked with a -inf logit)
    for bad in (0.0, -0.5, float("nan"), float("inf")):
        assert call(scale=bad) == SHAPE, bad
        assert "scale" in _err(lib)
    h = lib.sparse_attn_bwd
    #       q  kv idx xw ws0 sink pos t  B  Tq N   T_win H   d    k   win  scale out lse dout dq dkv dxw dsink ws wsb stream
    assert h(P, P, P, P, P, None, P, 1, 1, 1, 64, 128, 64, 128, 64, 128, -1.0, P, P, P, P, P, P, None, P, 1 << 40,
             None) == SHAPE
    assert "scale" in _err(lib)
    g = lib.dense_compressed_attn_fwd
    #   q  kv xw ws0 sink pos t  B  Tq N   T_win H   d    ratio win scale out lse ws wsb     flags stream
    assert g(P, P, P, P, None, P, 1, 1, 1, 64, 128, 64, 128, 0, 128, 1.0, P, None, P, 1 << 40, 0, None) == SHAPE
    assert g(P, P, P, P, None, P, 1, 1, 1, 64, -1, 64, 128, 4, 128, 1.0, P, None, P, 1 << 40, 0, None) == SHAPE
    assert g(P, P, P, P, None, P, 1, 1, 1, 64, 128, 64, 128, 4, 128, 1.0, P, None, P, 1 << 40, 8, None) == SHAPE
    # decode shapes need a split workspace
    need = lib.dense_attn_workspace_size(1, 1, 8192, 128, 128, 128, 0)
    assert need > 0
    assert g(P, P, P, P, None, P, 1, 1, 1, 8192, 128, 128, 128, 128, 128, 1.0, P, None, None, 0, 0, None) == WS
    # a workspace sized without the batch-invariant flag is too small for a call with it
    b8 = lib.dense_attn_workspace_size(8, 1, 8192, 128, 128, 128, 0)
    b8i = lib.dense_attn_workspace_size(8, 1, 8192, 128, 128, 128, 2)
    assert b8i > b8
    assert g(P, P, P, P, None, P, 1, 8, 1, 8192, 128, 128, 128, 128, 128, 1.0, P, None, P, b8, 2, None) == WS


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


def test_batch_invariant_flag_workspace():
    """Host logic of batch-invariant planning, a per-call flag: the attention
    workspace of a decode batch planned per sequence is the sum of the
    single-sequence workspaces, the default plan's is not, and asking with
    the flag leaves later queries without it unchanged (no mode state)."""
    from long_context_attention_csa_amd import ops
    default8 = ops.dense_attn_workspace_size(8, 1, 8192, 128, 128, 128)
    one = ops.dense_attn_workspace_size(1, 1, 8192, 128, 128, 128)
    assert one == ops.dense_attn_workspace_size(1, 1, 8192, 128, 128, 128, batch_invariant=True)
    assert ops.dense_attn_workspace_size(8, 1, 8192, 128, 128, 128, batch_invariant=True) == 8 * one
    assert default8 != 8 * one
    assert ops.sparse_attn_workspace_size(8, 1, 128, 128, 1024, 128, batch_invariant=True) == \
        8 * ops.sparse_attn_workspace_size(1, 1, 128, 128, 1024, 128)
    assert ops.dense_attn_workspace_size(8, 1, 8192, 128, 128, 128) == default8



def test_attention_split_plan():
    """Host logic of the attention split plan, read back from the workspace
    query (rows x heads x splits x (128 + 2) float32 values): about 256 blocks,
    >= 128 keys per split, and at 128 heads, when that leaves at most 320
    keys per split, one 16-head block per wave (two blocks per row), which
    halves the splits; long splits, other head counts and unsplit grids keep
    their plans."""
    from long_context_attention_csa_amd import ops

    def splits(ws, rows, H):
        assert ws % (rows * H * 130 * 4) == 0
        return ws // (rows * H * 130 * 4)
    # dense decode, 8,192 entries + 128 window rows
    assert splits(ops.dense_attn_workspace_size(8, 1, 8192, 128, 128, 128), 8, 128) == 16   # short: 32 -> 16
    assert splits(ops.dense_attn_workspace_size(32, 1, 8192, 128, 128, 128), 32, 128) == 8  # 1,040 keys: kept
    assert splits(ops.dense_attn_workspace_size(2, 1, 60000, 128, 128, 128), 2, 128) == 128  # ~470 keys: kept
    assert splits(ops.dense_attn_workspace_size(8, 1, 8192, 64, 128, 128), 8, 64) == 32    # 64 heads: unchanged
    # sparse decode, 1,024 selected + 128 window rows
    assert splits(ops.sparse_attn_workspace_size(8, 1, 128, 128, 1024, 128), 8, 128) == 9   # short, key-bound
    assert splits(ops.sparse_attn_workspace_size(64, 1, 128, 128, 1024, 128), 64, 128) == 2  # short: 4 -> 2
    assert splits(ops.sparse_attn_workspace_size(128, 1, 128, 128, 1024, 128), 128, 128) == 2  # 576 keys: kept
    # enough rows for one split: no workspace
    assert ops.sparse_attn_workspace_size(1, 300, 128, 128, 1024, 128) == 0


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


def test_headers_compile_as_c(tmp_path):
    """Both headers are plain C: a C11 translation unit that includes them and
    takes the address of every declared function compiles with gcc."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = tmp_path / "abi.c"
    names = declared_functions()
    body = "\n".join(f"  (void)&{n};" for n in names)
    src.write_text('#include "csa_hip.h"\n#include "csa_hip_timer.h"\nint main(void) {\n' + body + "\n  return 0;\n}\n")
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-c", str(src),
                        "-o", str(tmp_path / "abi.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_state_cache_validation():
    lib = _lib.lib()
    Q = ctypes.c_void_p(0x1008)   # 8-byte aligned only
    assert lib.csa_state_checkpoint(P, 2, 100, P, 1024, P, 4, None) == SHAPE      # bytes not a multiple of 16
    assert lib.csa_state_checkpoint(P, 2, 128, P, 0, P, 4, None) == SHAPE        # period 0
    assert lib.csa_state_checkpoint(P, 2, 128, P, 1024, P, 0, None) == SHAPE     # no slot
    assert lib.csa_state_checkpoint(None, 2, 128, P, 1024, P, 4, None) == NULL
    assert lib.csa_state_checkpoint(Q, 2, 128, P, 1024, P, 4, None) == SHAPE     # misaligned
    assert lib.csa_state_checkpoint(None, 0, 128, None, 1024, None, 4, None) == OK
    assert lib.csa_state_restore(P, 70000, 128, 4, P, P, None) == SHAPE         # B > 65535
    assert lib.csa_state_restore(P, 2, 128, 4, None, P, None) == NULL
    assert lib.csa_ring_fill(P, 2, 10, 24, P, 8, P, None) == SHAPE               # row bytes
    assert lib.csa_ring_fill(P, 2, 10, 32, P, 0, P, None) == SHAPE               # R = 0
    assert lib.csa_ring_fill(P, 2, 10, 32, None, 8, P, None) == NULL
    assert lib.csa_ring_fill(None, 2, 0, 32, None, 8, None, None) == OK          # empty history


def test_projection_validation():
    lib = _lib.lib()
    BF16, F32, FP8 = 1, 0, 2
    Q = ctypes.c_void_p(0x1008)   # 8-byte aligned only
    lin = lib.csa_linear_bf16
    # A, lda, sA, W, ldw, sW, C, out_t, ldc, sC, M, N, K, G, stream
    assert lin(P, 64, 0, P, 64, 0, P, FP8, 64, 0, 10, 10, 64, 1, None) == UNSUP     # output type
    assert lin(P, 96, 0, P, 96, 0, P, BF16, 64, 0, 10, 10, 96, 1, None) == SHAPE    # K not a multiple of 64
    assert lin(P, 64, 0, P, 64, 0, P, BF16, 64, 0, 10, 10, 64, 70000, None) == SHAPE  # G > 65535
    assert lin(P, 60, 0, P, 64, 0, P, BF16, 64, 0, 10, 10, 64, 1, None) == SHAPE    # lda < K
    assert lin(P, 68, 0, P, 68, 0, P, BF16, 64, 0, 10, 10, 64, 1, None) == SHAPE    # lda = 68: rows not 16-byte aligned
    assert lin(Q, 64, 0, P, 64, 0, P, BF16, 64, 0, 10, 10, 64, 1, None) == SHAPE    # A base misaligned
    assert lin(None, 64, 0, P, 64, 0, P, BF16, 64, 0, 10, 10, 64, 1, None) == NULL
    assert lin(P, 64, 0, P, 64, 0, P, BF16, 1 << 30, 0, 1 << 30, 1 << 30, 64, 1, None) == SHAPE  # tile count
    assert lin(None, 64, 0, None, 64, 0, None, BF16, 64, 0, 0, 10, 64, 1, None) == OK  # empty
    gop = lib.csa_grouped_out_proj
    # o, w_group, w_out, T, H, d, G, r, D, out, ws, ws_bytes, stream
    need = lib.csa_grouped_out_proj_workspace_size(8, 4, 64)
    assert need >= 8 * 4 * 64 * 2
    assert gop(P, P, P, 8, 64, 128, 5, 64, 256, P, P, need, None) == SHAPE          # H not a multiple of G
    assert gop(P, P, P, 8, 64, 12, 8, 64, 256, P, P, need, None) == SHAPE           # (H/G) d = 96: not a multiple of 64
    assert gop(P, P, P, 8, 64, 128, 4, 8, 256, P, P, need, None) == SHAPE           # G r not a multiple of 64
    assert gop(None, P, P, 8, 64, 128, 4, 64, 256, P, P, need, None) == NULL
    assert gop(P, P, P, 8, 64, 128, 4, 64, 256, P, P, need - 1, None) == WS
    qps = lib.csa_query_proj_shared
    # x, w_dq, w_uq, w_iq, T, D, r_q, n_q, n_i, q, q_idx, ws, ws_bytes, stream
    need = lib.csa_query_proj_shared_workspace_size(8, 128)
    assert need >= 8 * 128 * 2
    assert qps(P, P, P, P, 8, 100, 128, 256, 256, P, P, P, need, None) == SHAPE     # D not a multiple of 64
    assert qps(P, P, P, P, 8, 128, 96, 256, 256, P, P, P, need, None) == SHAPE      # r_q not a multiple of 64
    assert qps(P, P, P, P, 8, 128, 128, 256, 256, P, None, P, need, None) == NULL
    assert qps(P, P, P, P, 8, 128, 128, 256, 256, P, P, P, need - 1, None) == WS
    kvp = lib.csa_kv_proj
    # x, w, T, D, n_streams, width, streams, out_t, stream
    assert kvp(P, P, 8, 100, 4, 128, P, BF16, None) == SHAPE      # D not a multiple of 64
    assert kvp(P, P, 8, 128, 0, 128, P, BF16, None) == SHAPE      # no stream
    assert kvp(P, P, 8, 128, 4, 128, P, FP8, None) == UNSUP       # output type
    assert kvp(P, None, 8, 128, 4, 128, P, BF16, None) == NULL
    assert kvp(None, None, 0, 128, 4, 128, None, BF16, None) == OK   # no rows
