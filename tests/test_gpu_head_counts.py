"""Attention at head counts whose 16-head blocks do not split evenly into the
kernels' usual block shapes — 48 (3 blocks), 80 (5), 144 (9) — at 128 (8:
at decode, whose key splits here are short, one head block per wave) and at
the largest supported count, 256 (16), for sparse and dense attention, bf16 and
float32, with many query rows (one split per row) and at decode (one query
row per sequence, the keys split across blocks and merged). Outputs and
log-sum-exps against the oracle."""
import numpy as np
import pytest
import torch

import csa_synth as syn
import long_context_attention_csa_amd as C
from oracle import csa_oracle as O
from tests.gpu_common import assert_close, dev, host

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _inputs(seed, B, Tq, N, H, T_win, kind):
    bf = kind == "bf16"
    q = syn.normal(seed * 10 + 1, (B, Tq, H, 128), scale=1 / np.sqrt(128), bf16=bf)
    kv = syn.normal(seed * 10 + 2, (B, N, 128), bf16=bf)
    xw = syn.normal(seed * 10 + 3, (B, T_win, 128), bf16=bf)
    sink = syn.normal(seed * 10 + 4, (H,))
    return q, kv, xw, sink


def _shape(mode):
    # (B, Tq): many rows of one sequence, or one decode row per sequence
    return (1, 300) if mode == "prefill" else (2, 1)


def _check(kind, got, got_l, want, want_l, what):
    assert_close(got, want, kind, what)
    np.testing.assert_allclose(got_l, want_l, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("H", [48, 80, 128, 144, 256])
@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_sparse_head_counts(kind, H, mode):
    B, Tq = _shape(mode)
    N, k = 3000, 256
    T_win = 128 + Tq - 1
    q_pos = np.stack([np.arange(4 * N - Tq, 4 * N) - 5 * b for b in range(B)]).astype(np.int32)
    win_start = (q_pos[:, 0] - 127).astype(np.int32)
    q, kv, xw, sink = _inputs(101 + H, B, Tq, N, H, T_win, kind)
    g = np.random.default_rng(102 + H)
    idx = np.stack([[np.sort(g.choice(N, size=k, replace=False)) for _ in range(Tq)] for _ in range(B)])
    idx = idx.astype(np.int32)
    idx[:, ::7, -9:] = -1   # padded rows
    dt = torch.float32 if kind == "f32" else BF
    print("sparse heads", kind, H, mode, flush=True)
    out, lse = C.sparse_attn_fwd(dev(q, dt), dev(kv, dt), dev(idx, torch.int32), dev(xw, dt),
                                 dev(win_start, torch.int32), dev(sink), dev(q_pos, torch.int32), 128, 1.0,
                                 want_lse=True)
    got, got_l = host(out), host(lse)
    for b in range(B):
        o, l = O.sparse_attn(q[b], kv[b], idx[b], xw[b], int(win_start[b]), sink, q_pos[b], 128)
        _check(kind, got[b], got_l[b], o, l, f"sparse H={H} {mode} b={b}")


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("H", [48, 80, 128, 144, 256])
@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_dense_head_counts(kind, H, mode):
    B, Tq = _shape(mode)
    ratio, N = 16, 400
    L = ratio * N + 9
    T_win = 128 + Tq - 1
    q_pos = np.stack([np.arange(L - Tq, L) - 700 * b for b in range(B)]).astype(np.int32)
    win_start = (q_pos[:, 0] - 127).astype(np.int32)
    q, kv, xw, sink = _inputs(111 + H, B, Tq, N, H, T_win, kind)
    dt = torch.float32 if kind == "f32" else BF
    print("dense heads", kind, H, mode, flush=True)
    out, lse = C.dense_compressed_attn_fwd(dev(q, dt), dev(kv, dt), dev(xw, dt), dev(win_start, torch.int32),
                                           dev(sink), dev(q_pos, torch.int32), ratio, 128, 1.0, want_lse=True)
    got, got_l = host(out), host(lse)
    for b in range(B):
        o, l = O.dense_attn(q[b], kv[b], xw[b], int(win_start[b]), sink, q_pos[b], ratio, 128)
        _check(kind, got[b], got_l[b], o, l, f"dense H={H} {mode} b={b}")
