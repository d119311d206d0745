"""Window state cache: the attention calls reading their window rows from a ring
(position t at row t mod T_win) give exactly the results of the same rows laid
out in order, and csa_window_append keeps the ring up to date token by token."""
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


def _to_ring(lin, w0, R):
    """ring[b, (w0[b] + i) mod R] = lin[b, i] for the R rows of each sequence."""
    ring = np.zeros_like(lin)
    for b in range(lin.shape[0]):
        for i in range(R):
            ring[b, (int(w0[b]) + i) % R] = lin[b, i]
    return ring


@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("sparse", [True, False])
@pytest.mark.parametrize("Tq", [1, 70])
def test_ring_equals_linear(kind, sparse, Tq):
    B, N, H, T_win, k, ratio = 3, 900, 64 if kind == "bf16" else 16, 160, 96, 4
    dt = BF if kind == "bf16" else torch.float32
    bf = kind == "bf16"
    w0 = np.array([5, 127, 200], np.int32)            # wraps at rows 155, 33 and 120 of the ring
    q_pos = np.stack([np.arange(Tq) + int(w0[b]) + T_win - Tq for b in range(B)]).astype(np.int32)
    q = syn.normal(31, (B, Tq, H, 128), scale=1 / np.sqrt(128), bf16=bf)
    kv = syn.normal(32, (B, N, 128), bf16=bf)
    lin = syn.normal(33, (B, T_win, 128), bf16=bf)
    sink = syn.normal(34, (H,))
    ring = _to_ring(lin, w0, T_win)
    g = np.random.default_rng(35)
    idx = np.stack([[np.sort(g.choice(N, size=k, replace=False)) for _ in range(Tq)] for _ in range(B)])
    idx = idx.astype(np.int32)
    args = lambda xw: [dev(q, dt), dev(kv, dt)] + ([dev(idx, torch.int32)] if sparse else []) + \
        [dev(xw, dt), dev(w0, torch.int32), dev(sink), dev(q_pos, torch.int32)]
    _print("ring vs linear", kind, sparse, Tq)
    if sparse:
        a = C.sparse_attn_fwd(*args(lin), 128, 1.0, want_lse=True)
        b = C.sparse_attn_fwd(*args(ring), 128, 1.0, want_lse=True, win_ring=True)
    else:
        a = C.dense_compressed_attn_fwd(*args(lin), ratio, 128, 1.0, want_lse=True)
        b = C.dense_compressed_attn_fwd(*args(ring), ratio, 128, 1.0, want_lse=True, win_ring=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # and against the oracle on the linear rows
    for bb in range(B):
        o = (O.sparse_attn(q[bb], kv[bb], idx[bb], lin[bb], int(w0[bb]), sink, q_pos[bb], 128) if sparse else
             O.dense_attn(q[bb], kv[bb], lin[bb], int(w0[bb]), sink, q_pos[bb], ratio, 128))[0]
        assert_close(host(b[0])[bb], o, kind, f"ring b={bb}")


def test_window_append_decode_loop():
    """Token by token: append the new token's row, then attend with the ring;
    every step equals the attention over the whole history laid out in order."""
    B, H, R, N, k = 2, 64, 128, 600, 64
    steps = 300
    hist = syn.normal(41, (B, steps, 128), bf16=True)
    kv = syn.normal(42, (B, N, 128), bf16=True)
    sink = syn.normal(43, (H,))
    g = np.random.default_rng(44)
    ring = torch.zeros(B, R, 128, dtype=BF, device="cuda")
    hist_d = dev(hist, BF)
    kv_d = dev(kv, BF)
    for p in range(steps):
        pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
        C.window_append(hist_d[:, p].contiguous(), pos, ring)
        if p % 37 != 36 and p != steps - 1:
            continue
        q = dev(syn.normal(1000 + p, (B, 1, H, 128), scale=1 / np.sqrt(128), bf16=True), BF)
        idx = dev(np.stack([[np.sort(g.choice(N, size=k, replace=False))] for _ in range(B)]), torch.int32)
        qp = torch.full((B, 1), p, dtype=torch.int32, device="cuda")
        w_ring = torch.full((B,), max(0, p - R + 1), dtype=torch.int32, device="cuda")
        w_lin = torch.zeros(B, dtype=torch.int32, device="cuda")
        _print("decode step", p)
        a = C.sparse_attn_fwd(q, kv_d, idx, ring, w_ring, dev(sink), qp, 128, 1.0, win_ring=True)
        b = C.sparse_attn_fwd(q, kv_d, idx, hist_d[:, : p + 1].contiguous(), w_lin, dev(sink), qp, 128, 1.0)
        assert torch.equal(a, b), p
    want = np.zeros((B, R, 128), np.float32)
    for t in range(steps - R, steps):
        want[:, t % R] = hist[:, t]
    assert np.array_equal(host(ring), want)
