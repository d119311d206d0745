"""Batch-invariant planning (the CSA_ATTN_BATCH_INVARIANT flag of one call): a
sequence's attention output and LSE are the same bits whether it runs alone or
inside a batch (decode rows, where the default plan splits keys by batch
size, and multi-query rows); results still match the oracle. Calls without
the flag in the same process are unaffected (no mode state)."""
import numpy as np
import pytest
import torch

import csa_synth as syn
import long_context_attention_csa_amd as C
from oracle import csa_oracle as O
from tests.gpu_common import assert_close, dev, host

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _case(seed, B, Tq, N, H, T_win):
    q = syn.normal(seed * 10 + 1, (B, Tq, H, 128), scale=1 / np.sqrt(128), bf16=True)
    kv = syn.normal(seed * 10 + 2, (B, N, 128), bf16=True)
    xw = syn.normal(seed * 10 + 3, (B, T_win, 128), bf16=True)
    sink = syn.normal(seed * 10 + 4, (H,))
    return q, kv, xw, sink


@pytest.mark.parametrize("B,Tq,H", [(5, 1, 128), (3, 6, 64)])
def test_dense_attn_batch_invariant(B, Tq, H):
    N = 3000
    L = 128 * N + 50
    T_win = 128 + Tq - 1
    q_pos = np.stack([np.arange(L - Tq, L) - 7 * b for b in range(B)]).astype(np.int32)
    win_start = (q_pos[:, 0] - 127).astype(np.int32)
    q, kv, xw, sink = _case(11, B, Tq, N, H, T_win)
    args = lambda sl: (dev(q[sl], BF), dev(kv[sl], BF), dev(xw[sl], BF), dev(win_start[sl], torch.int32),
                       dev(sink), dev(q_pos[sl], torch.int32), 128, 128)
    print("dense batch-invariant", B, Tq, H, flush=True)
    out, lse = C.dense_compressed_attn_fwd(*args(slice(None)), want_lse=True, batch_invariant=True)
    plain = C.dense_compressed_attn_fwd(*args(slice(None)))          # interleaved call without the flag
    for b in (0, B - 1):
        o1, l1 = C.dense_compressed_attn_fwd(*args(slice(b, b + 1)), want_lse=True, batch_invariant=True)
        assert torch.equal(out[b:b + 1], o1) and torch.equal(lse[b:b + 1], l1), f"sequence {b}"
    assert torch.equal(C.dense_compressed_attn_fwd(*args(slice(None))), plain)
    o, _ = O.dense_attn(q[0], kv[0], xw[0], int(win_start[0]), sink, q_pos[0], 128, 128)
    assert_close(host(out)[0], o, "bf16", "dense batch-invariant vs oracle")


@pytest.mark.parametrize("B,Tq,H,k", [(4, 1, 128, 1024), (3, 5, 64, 512)])
def test_sparse_attn_batch_invariant(B, Tq, H, k):
    N = 5000
    T_win = 128 + Tq - 1
    q_pos = np.stack([np.arange(4 * N - Tq, 4 * N) + b for b in range(B)]).astype(np.int32)
    win_start = (q_pos[:, 0] - 127).astype(np.int32)
    q, kv, xw, sink = _case(12, B, Tq, N, H, T_win)
    g = np.random.default_rng(13)
    idx = np.stack([[np.sort(g.choice(N, size=k, replace=False)) for _ in range(Tq)] for _ in range(B)]).astype(np.int32)
    args = lambda sl: (dev(q[sl], BF), dev(kv[sl], BF), dev(idx[sl], torch.int32), dev(xw[sl], BF),
                       dev(win_start[sl], torch.int32), dev(sink), dev(q_pos[sl], torch.int32), 128, 1.0)
    print("sparse batch-invariant", B, Tq, H, k, flush=True)
    out, lse = C.sparse_attn_fwd(*args(slice(None)), want_lse=True, batch_invariant=True)
    plain = C.sparse_attn_fwd(*args(slice(None)))
    for b in (0, B - 1):
        o1, l1 = C.sparse_attn_fwd(*args(slice(b, b + 1)), want_lse=True, batch_invariant=True)
        assert torch.equal(out[b:b + 1], o1) and torch.equal(lse[b:b + 1], l1), f"sequence {b}"
    assert torch.equal(C.sparse_attn_fwd(*args(slice(None))), plain)
    o, _ = O.sparse_attn(q[0], kv[0], idx[0], xw[0], int(win_start[0]), sink, q_pos[0], 128)
    assert_close(host(out)[0], o, "bf16", "sparse batch-invariant vs oracle")
