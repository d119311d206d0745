"""Attention at decode shapes (few rows, bf16: key splits over blocks and
their merge). Checked against the oracle on shapes with one and several head
groups, H not a multiple of 32, splits with no key (rows near position 0),
selections with holes and indices past N, windows clipped by the supplied
rows and rings, no sink; repeated calls give the same bits, and one
workspace serves calls of different shapes in a row."""
import numpy as np
import pytest
import torch

import csa_synth as syn
import long_context_attention_csa_amd as C
from oracle import csa_oracle as O
from tests.gpu_common import assert_close, dev, host

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _print(*a):
    print(*a, flush=True)


def _case(seed, B, Tq, N, H, T_win):
    q = syn.normal(seed * 10 + 1, (B, Tq, H, 128), scale=1 / np.sqrt(128), bf16=True)
    kv = syn.normal(seed * 10 + 2, (B, N, 128), bf16=True)
    xw = syn.normal(seed * 10 + 3, (B, T_win, 128), bf16=True)
    sink = syn.normal(seed * 10 + 4, (H,))
    return q, kv, xw, sink


@pytest.mark.parametrize("B,Tq,H,N,use_sink,window", [
    (8, 1, 128, 8192, True, 128), (2, 1, 64, 3001, True, 128), (3, 2, 48, 900, False, 5),
    (1, 1, 16, 5000, True, 0), (5, 1, 128, 40, True, 128),
    # 128 heads split across the keys: 8,320 keys in splits of at most five
    # tiles (one head block per wave) above; 60,128 in 128 splits of ~470
    # keys here (two head blocks per wave)
    (2, 1, 128, 60000, True, 128)])
def test_dense_decode(B, Tq, H, N, use_sink, window):
    ratio = 128
    L = ratio * N + 77
    T_win = 128 + Tq - 1
    q, kv, xw, sink = _case(31, B, Tq, N, H, T_win)
    # row 0 at the end of the cache; others earlier, the last near position 0
    starts = [L - Tq + 1 - 911 * b for b in range(B)]
    starts[-1] = min(starts[-1], 3)
    q_pos = np.stack([np.arange(st, st + Tq) for st in starts]).astype(np.int32)
    win_start = np.maximum(q_pos[:, 0] - 127, 0).astype(np.int32)
    args = (dev(q, BF), dev(kv, BF), dev(xw, BF), dev(win_start, torch.int32), dev(sink) if use_sink else None,
            dev(q_pos, torch.int32), ratio, window, 1.0)
    _print("dense decode", B, Tq, H, N, use_sink, window)
    out, lse = C.dense_compressed_attn_fwd(*args, want_lse=True)
    out2, lse2 = C.dense_compressed_attn_fwd(*args, want_lse=True)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    s_or = sink if use_sink else np.full(H, -np.inf)
    for b in range(B):
        o, l = O.dense_attn(q[b], kv[b], xw[b], int(win_start[b]), s_or, q_pos[b], ratio, window)
        assert_close(host(out)[b], o, "bf16", f"dense decode b={b}")
        got_l = host(lse)[b]
        fin = np.isfinite(l)
        assert np.array_equal(fin, np.isfinite(got_l))
        np.testing.assert_allclose(got_l[fin], l[fin], rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("B,Tq,H,k,N", [(8, 1, 128, 1024, 262144), (3, 5, 64, 512, 16384), (2, 1, 32, 4096, 9000)])
def test_sparse_decode(B, Tq, H, k, N):
    T_win = 128 + Tq - 1
    q, kv, xw, sink = _case(32, B, Tq, N, H, T_win)
    g = np.random.default_rng(33)
    idx = np.full((B, Tq, k), -1, np.int32)
    for b in range(B):
        for t in range(Tq):
            m = k if (b + t) % 3 else k // 3          # some rows padded with -1
            idx[b, t, :m] = np.sort(g.choice(N, size=m, replace=False))
    idx[0, 0, 1] = N + 5                              # an index past N is skipped
    L = 4 * N + 3
    q_pos = np.stack([np.arange(L - Tq - 17 * b, L - 17 * b) for b in range(B)]).astype(np.int32)
    win_start = (q_pos[:, 0] - 127 + 40).astype(np.int32)   # the window clipped by the supplied rows
    args = (dev(q, BF), dev(kv, BF), dev(idx, torch.int32), dev(xw, BF), dev(win_start, torch.int32), dev(sink),
            dev(q_pos, torch.int32), 128, 1.0)
    _print("sparse decode", B, Tq, H, k, N)
    out, lse = C.sparse_attn_fwd(*args, want_lse=True)
    assert torch.equal(out, C.sparse_attn_fwd(*args))
    for b in range(B):
        o, l = O.sparse_attn(q[b], kv[b], idx[b], xw[b], int(win_start[b]), sink, q_pos[b], 128)
        assert_close(host(out)[b], o, "bf16", f"sparse decode b={b}")
        np.testing.assert_allclose(host(lse)[b], l, rtol=1e-4, atol=1e-4)


def test_decode_ring_window():
    """The window read from a ring (position t at row t mod T_win)."""
    B, H, N, T_win = 4, 128, 5000, 128
    q, kv, xw, sink = _case(34, B, 1, N, H, T_win)
    L = 128 * N + 300
    q_pos = np.array([[L - 3 * b] for b in range(B)], np.int32)
    w0 = (q_pos[:, 0] - 127).astype(np.int32)
    ring = np.stack([np.roll(xw[b], shift=int(w0[b]) % T_win, axis=0) for b in range(B)])
    out = C.dense_compressed_attn_fwd(dev(q, BF), dev(kv, BF), dev(ring, BF), dev(w0, torch.int32), dev(sink),
                                      dev(q_pos, torch.int32), 128, 128, 1.0, win_ring=True)
    for b in range(B):
        o, _ = O.dense_attn(q[b], kv[b], xw[b], int(w0[b]), sink, q_pos[b], 128, 128)
        assert_close(host(out)[b], o, "bf16", f"ring b={b}")


def test_decode_workspace_reuse():
    """One caller workspace serves a sparse call, a dense call and a smaller
    sparse call in a row (twice), each equal to a call with its own fresh
    workspace."""
    B, H, N, k = 8, 128, 20000, 1024
    q, kv, xw, sink = _case(35, B, 1, N, H, 128)
    g = np.random.default_rng(36)
    idx = np.stack([np.sort(g.choice(N, size=k, replace=False)) for _ in range(B)])[:, None].astype(np.int32)
    q_pos = np.full((B, 1), 128 * N + 5, np.int32)
    w0 = (q_pos[:, 0] - 127).astype(np.int32)
    dq, dkv, dxw, dsink = dev(q, BF), dev(kv, BF), dev(xw, BF), dev(sink)
    dqp, dw0, didx = dev(q_pos, torch.int32), dev(w0, torch.int32), dev(idx, torch.int32)
    n_sp = C.sparse_attn_workspace_size(B, 1, H, 128, k, 128)
    n_dn = C.dense_attn_workspace_size(B, 1, N, H, 128, 128)
    ws = torch.empty(max(n_sp, n_dn), dtype=torch.uint8, device="cuda")
    for rep in range(2):
        a = C.sparse_attn_fwd(dq, dkv, didx, dxw, dw0, dsink, dqp, 128, 1.0, ws=ws)
        b_ = C.dense_compressed_attn_fwd(dq, dkv, dxw, dw0, dsink, dqp, 128, 128, 1.0, ws=ws)
        c = C.sparse_attn_fwd(dq[:3], dkv[:3], didx[:3], dxw[:3], dw0[:3], dsink, dqp[:3], 128, 1.0, ws=ws)
        assert torch.equal(a, C.sparse_attn_fwd(dq, dkv, didx, dxw, dw0, dsink, dqp, 128, 1.0))
        assert torch.equal(b_, C.dense_compressed_attn_fwd(dq, dkv, dxw, dw0, dsink, dqp, 128, 128, 1.0))
        assert torch.equal(c, C.sparse_attn_fwd(dq[:3], dkv[:3], didx[:3], dxw[:3], dw0[:3], dsink, dqp[:3], 128,
                                                1.0))
