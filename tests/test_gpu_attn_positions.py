"""Dense attention at prefill sizes (bf16, 32 or 64 heads, more than a
thousand query rows, one split per row) against the oracle: consecutive
prefill positions with an odd row count, a window shorter than 128 or none,
and arbitrary positions (repeated, decreasing, far apart, before the window
start); batch-invariant calls stay bit-identical per sequence at these
sizes."""
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


def _run_check(q, kv, xw, win_start, sink, q_pos, ratio, window, what):
    print(what, flush=True)
    out, lse = C.dense_compressed_attn_fwd(dev(q, BF), dev(kv, BF), dev(xw, BF), dev(win_start, torch.int32),
                                           dev(sink), dev(q_pos, torch.int32), ratio, window, want_lse=True)
    got, got_l = host(out), host(lse)
    for b in range(q.shape[0]):
        o, l = O.dense_attn(q[b], kv[b], xw[b], int(win_start[b]), sink, q_pos[b], ratio, window)
        assert_close(got[b], o, "bf16", f"{what} b={b}")
        np.testing.assert_allclose(got_l[b], l, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("H,T,ratio,window", [(64, 1025, 4, 128), (32, 1200, 128, 128), (64, 1100, 16, 50),
                                              (32, 1031, 4, 0)])
def test_prefill_positions(H, T, ratio, window):
    """Consecutive positions 0 .. T-1 of one sequence."""
    N = T // ratio
    q_pos = np.arange(T, dtype=np.int32)[None]
    q, kv, xw, sink = _case(81, 1, T, N, H, T)
    _run_check(q, kv, xw, np.zeros(1, np.int32), sink, q_pos, ratio, window, f"dense prefill H={H} T={T}")


def test_arbitrary_positions():
    """Two sequences of 1030 query rows at arbitrary positions: sorted runs,
    repeats, a decreasing pair, neighbouring rows thousands of positions
    apart, and positions before the window start."""
    B, Tq, H, ratio, L = 2, 1030, 64, 4, 6000
    N = L // ratio
    g = np.random.default_rng(82)
    q_pos = np.empty((B, Tq), np.int32)
    q_pos[0] = np.sort(g.integers(0, L, Tq))
    q_pos[1] = g.integers(0, L, Tq)                        # unsorted: neighbouring rows far apart
    q_pos[0, 100:110] = 2000                               # repeats
    q_pos[0, 200:202] = [3000, 2990]                       # a decreasing pair
    w0 = np.array([0, 1500], np.int32)                     # sequence 1: the window rows start at 1500
    T_win = L - 1500
    q, kv, xw, sink = _case(83, B, Tq, N, H, L)
    xw = xw[:, :T_win].copy()
    q_pos[1] = np.maximum(q_pos[1], 0)
    _run_check(q, kv, xw, w0, sink, q_pos, ratio, 128, "dense arbitrary positions")


def test_prefill_batch_invariant():
    """Batch-invariant planning at prefill sizes: a sequence alone and inside
    a batch gives the same bits."""
    B, Tq, H, ratio = 3, 1100, 64, 16
    N = 2000
    q_pos = np.stack([np.arange(Tq) + 700 * b for b in range(B)]).astype(np.int32)
    T_win = Tq + 1400
    q, kv, xw, sink = _case(84, B, Tq, N, H, T_win)
    args = lambda sl: (dev(q[sl], BF), dev(kv[sl], BF), dev(xw[sl], BF), dev(np.zeros(B, np.int32)[sl], torch.int32),
                       dev(sink), dev(q_pos[sl], torch.int32), ratio, 128)
    print("dense prefill batch-invariant", flush=True)
    out, lse = C.dense_compressed_attn_fwd(*args(slice(None)), want_lse=True, batch_invariant=True)
    for b in (0, B - 1):
        o1, l1 = C.dense_compressed_attn_fwd(*args(slice(b, b + 1)), want_lse=True, batch_invariant=True)
        assert torch.equal(out[b:b + 1], o1) and torch.equal(lse[b:b + 1], l1), f"sequence {b}"
    o, _ = O.dense_attn(q[2], kv[2], xw[2], 0, sink, q_pos[2], ratio, 128)
    assert_close(host(out)[2], o, "bf16", "dense prefill batch-invariant vs oracle")
