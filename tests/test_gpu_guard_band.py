"""Guard bands: every output (and workspace) of every entry point is placed in
the middle of a larger buffer whose bytes around it hold a canary pattern;
after the call the canaries must be intact (no write past either end), and
outputs the contract leaves untouched (index scores past n(p)) keep their
pattern. Calls go straight through the C ABI with the guarded pointers."""
import ctypes

import numpy as np
import pytest
import torch

import csa_synth as syn
import long_context_attention_csa_amd as C
from long_context_attention_csa_amd import _lib
from tests.gpu_common import dev

pytestmark = pytest.mark.gpu
BF = torch.bfloat16
PAD = 4096
CANARY = 0xA5


class Guarded:
    """A view of `shape`/`dtype` inside a canary-filled byte buffer."""

    def __init__(self, shape, dtype, fill=CANARY):
        self.n = int(np.prod(shape)) * torch.empty(0, dtype=dtype).element_size()
        self.buf = torch.full((self.n + 2 * PAD,), fill, dtype=torch.uint8, device="cuda")
        self.t = self.buf[PAD:PAD + self.n].view(dtype).view(*shape) if self.n else self.buf[PAD:PAD].view(dtype)

    def ptr(self):
        return ctypes.c_void_p(self.t.data_ptr())

    def intact(self):
        torch.cuda.synchronize()
        return bool((self.buf[:PAD] == CANARY).all()) and bool((self.buf[PAD + self.n:] == CANARY).all())


def _s():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ok(st):
    assert st == 0, _lib.lib().csa_last_error().decode()


def test_guard_quantize_and_compressors():
    lib = _lib.lib()
    B, T, W = 2, 1030, 128
    x = [dev(syn.normal(900 + i, (B, T, W), bf16=True), BF) for i in range(4)]
    # quantiser: fp8 and fp4
    for fmt, cw, sshape, sdt in ((2, W, (B * T,), torch.float32), (3, W // 2, (B * T, W // 32), torch.uint8)):
        out, sc = Guarded((B * T, cw), torch.uint8), Guarded(sshape, sdt)
        _ok(lib.csa_quantize_rows(_p(x[0]), 1, B * T, W, out.ptr(), fmt, sc.ptr(), _s()))
        assert out.intact() and sc.intact()
    # CSA compressor to bf16 and to fp8 codes + scales
    N = T // 4
    out = Guarded((B, N, W), BF)
    _ok(lib.csa_compress(*[_p(t) for t in x], 1, B, T, W, 4, out.ptr(), 1, None, _s()))
    assert out.intact()
    out, sc = Guarded((B, N, W), torch.uint8), Guarded((B, N), torch.float32)
    _ok(lib.csa_compress(*[_p(t) for t in x], 1, B, T, W, 4, out.ptr(), 2, sc.ptr(), _s()))
    assert out.intact() and sc.intact()
    out = Guarded((B, T // 128, W), BF)
    _ok(lib.hca_compress(_p(x[0]), _p(x[1]), 1, B, T, W, 128, out.ptr(), 1, _s()))
    assert out.intact()
    # decode-time steps: state rings and caches
    rows = [dev(syn.normal(910 + i, (B, W), bf16=True), BF) for i in range(4)]
    pos = dev(np.array([7, 127], np.int32), torch.int32)
    state = Guarded((B, 8, 4, W), BF, fill=0)
    state.buf[:PAD] = CANARY
    state.buf[PAD + state.n:] = CANARY
    cache = Guarded((B, 64, W), BF)
    _ok(lib.csa_compress_append(*[_p(t) for t in rows], 1, B, W, 4, _p(pos), state.ptr(), 64, cache.ptr(), 1, None,
                                _s()))
    assert state.intact() and cache.intact()
    hstate = Guarded((B, 128, 2, W), BF, fill=0)
    hstate.buf[:PAD] = CANARY
    hstate.buf[PAD + hstate.n:] = CANARY
    hcache = Guarded((B, 4, W), BF)
    _ok(lib.hca_compress_append(_p(rows[0]), _p(rows[1]), 1, B, W, 128, _p(pos), hstate.ptr(), 4, hcache.ptr(), 1,
                                _s()))
    assert hstate.intact() and hcache.intact()
    ring = Guarded((B, 128, W), BF)
    _ok(lib.csa_window_append(_p(rows[0]), 1, B, W, _p(pos), ring.ptr(), 128, _s()))
    assert ring.intact()


@pytest.mark.parametrize("Tq,N,k,fmt", [(1, 40000, 128, 2), (1, 9000, 256, 3), (300, 3000, 64, 2)])
@pytest.mark.parametrize("bf16_scores", [False, True])
def test_guard_indexer(Tq, N, k, fmt, bf16_scores):
    """Decode list mode, short decode rows and prefill rows; float32 and bf16
    scores. Scores past n(p) keep their pattern."""
    lib = _lib.lib()
    B, H_I = 2, 64
    qi32 = dev(syn.normal(920, (B, Tq, H_I, 128)))
    ki32 = dev(syn.normal(921, (B, N, 128)))
    f = "fp8" if fmt == 2 else "fp4"
    qc, qs = C.csa_quantize_rows(qi32, f)
    kc, ks = C.csa_quantize_rows(ki32, f)
    w = dev(syn.uniform(922, (B, Tq, H_I)))
    q_pos = np.stack([np.linspace(4 * N // 3, 4 * N + 5, Tq).astype(np.int32) - 9 * b for b in range(B)])
    dq_pos = dev(q_pos, torch.int32)
    sdt = BF if bf16_scores else torch.float32
    idx = Guarded((B, Tq, k), torch.int32)
    sc = Guarded((B, Tq, N), sdt)
    name = "indexer_topk_bf16_scores" if bf16_scores else "indexer_topk"
    nws = getattr(lib, name + "_workspace_size")(B, Tq, N, H_I, 128, k, fmt)
    ws = Guarded((nws,), torch.uint8)
    _ok(getattr(lib, name)(_p(qc), _p(qs), _p(w), _p(kc), _p(ks), fmt, _p(dq_pos), B, Tq, N, H_I, 128, 4, k,
                           idx.ptr(), sc.ptr(), ws.ptr(), nws, _s()))
    assert idx.intact() and sc.intact() and ws.intact()
    raw = sc.buf[PAD:PAD + sc.n].view(torch.int16 if bf16_scores else torch.int32).view(B, Tq, N).cpu().numpy()
    pat = np.int16(-23131) if bf16_scores else np.int32(-1515870811)      # 0xA5A5 / 0xA5A5A5A5
    n_vis = np.minimum(N, (q_pos.astype(np.int64) + 1) // 4)
    for b in range(B):
        for t in range(Tq):
            assert np.all(raw[b, t, n_vis[b, t]:] == pat), (b, t)


@pytest.mark.parametrize("B,Tq,H", [(8, 1, 128), (1, 700, 64)])
def test_guard_attention(B, Tq, H):
    lib = _lib.lib()
    N, k, W = 5000, 512, 128
    q = dev(syn.normal(930, (B, Tq, H, 128), scale=1 / np.sqrt(128), bf16=True), BF)
    kv = dev(syn.normal(931, (B, N, 128), bf16=True), BF)
    L = 4 * N
    q_pos_np = np.stack([np.arange(L - Tq, L) for _ in range(B)]).astype(np.int32)
    xw = dev(syn.normal(932, (B, Tq + W - 1, 128), bf16=True), BF)
    w0 = dev(np.full(B, L - Tq - W + 1, np.int32), torch.int32)
    sink = dev(syn.normal(933, (H,)))
    g = np.random.default_rng(934)
    idx = dev(np.stack([[np.sort(g.choice(N, k, replace=False)) for _ in range(Tq)] for _ in range(B)]).astype(
        np.int32), torch.int32)
    q_pos = dev(q_pos_np, torch.int32)
    T_win = Tq + W - 1
    for sparse in (True, False):
        out, lse = Guarded((B, Tq, H, 128), BF), Guarded((B, Tq, H), torch.float32)
        if sparse:
            nws = lib.sparse_attn_workspace_size(B, Tq, H, 128, k, W, 0)
            ws = Guarded((max(nws, 1),), torch.uint8)
            _ok(lib.sparse_attn_fwd(_p(q), _p(kv), _p(idx), _p(xw), _p(w0), _p(sink), _p(q_pos), 1, B, Tq, N, T_win,
                                    H, 128, k, W, 1.0, out.ptr(), lse.ptr(), ws.ptr(), nws, 0, _s()))
        else:
            nws = lib.dense_attn_workspace_size(B, Tq, N, H, 128, W, 0)
            ws = Guarded((max(nws, 1),), torch.uint8)
            _ok(lib.dense_compressed_attn_fwd(_p(q), _p(kv), _p(xw), _p(w0), _p(sink), _p(q_pos), 1, B, Tq, N,
                                              T_win, H, 128, 4, W, 1.0, out.ptr(), lse.ptr(), ws.ptr(), nws, 0,
                                              _s()))
        assert out.intact() and lse.intact() and ws.intact(), f"sparse={sparse}"
        # backward: dq, dkv, dx_win, dsink
        dout = dev(syn.normal(935, (B, Tq, H, 128), bf16=True), BF)
        dq = Guarded((B, Tq, H, 128), BF)
        dkv, dxw, dsk = Guarded((B, N, 128), torch.float32), Guarded((B, T_win, 128), torch.float32), \
            Guarded((H,), torch.float32)
        if sparse:
            nb = lib.sparse_attn_bwd_workspace_size(B, Tq, N, T_win, H, 128, k, W)
            wb = Guarded((nb,), torch.uint8)
            _ok(lib.sparse_attn_bwd(_p(q), _p(kv), _p(idx), _p(xw), _p(w0), _p(sink), _p(q_pos), 1, B, Tq, N, T_win,
                                    H, 128, k, W, 1.0, out.ptr(), lse.ptr(), _p(dout), dq.ptr(), dkv.ptr(),
                                    dxw.ptr(), dsk.ptr(), wb.ptr(), nb, _s()))
        else:
            nb = lib.dense_attn_bwd_workspace_size(B, Tq, N, T_win, H, 128, W)
            wb = Guarded((nb,), torch.uint8)
            _ok(lib.dense_compressed_attn_bwd(_p(q), _p(kv), _p(xw), _p(w0), _p(sink), _p(q_pos), 1, B, Tq, N,
                                              T_win, H, 128, 4, W, 1.0, out.ptr(), lse.ptr(), _p(dout), dq.ptr(),
                                              dkv.ptr(), dxw.ptr(), dsk.ptr(), wb.ptr(), nb, _s()))
        assert dq.intact() and dkv.intact() and dxw.intact() and dsk.intact() and wb.intact(), f"bwd sparse={sparse}"
    # the allocation-free variant
    out2, lse2 = Guarded((B, Tq, H, 128), BF), Guarded((B, Tq, H), torch.float32)
    _ok(lib.sparse_attn_fwd_noalloc(_p(q), _p(kv), _p(idx), _p(xw), _p(w0), _p(sink), _p(q_pos), 1, B, Tq, N, T_win,
                                    H, 128, k, W, 1.0, out2.ptr(), lse2.ptr(), 0, _s()))
    assert out2.intact() and lse2.intact()
