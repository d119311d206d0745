"""GPU results against closed forms of the method, with no oracle in between
(pins P-b, P-c and P-d of the hot path applied to the kernels directly):

* one-hot gates (logit 0 at one token, -1e4 elsewhere: the other weights
  underflow to exactly 0) reduce both compressors to selecting that token's
  row, bit for bit (cf-1.com write-up §3.1 gated weights; §3.2);
* the HCA compressor at ratio 1 is the identity, bit for bit;
* with every key and value row equal to ones, a query's logits are all
  scale * sum(q), so attention over n keys with sink s gives
  lse = log(e^s + n e^l) and o = 1 - e^(s - lse) in every channel (cf-1.com
  write-up §3.3: the sink enters the denominator only), for sparse and dense
  attention, bf16 and float32, with and without the sink."""
import numpy as np
import pytest
import torch

import csa_synth as syn
import long_context_attention_csa_amd as C
from tests.gpu_common import dev, host

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


@pytest.mark.parametrize("dt", [torch.float32, BF])
def test_csa_compress_one_hot_gates_select(dt):
    B, T, W = 2, 400, 128
    g = np.random.default_rng(131)
    c_a = syn.normal(132, (B, T, W), bf16=dt == BF)
    c_b = syn.normal(133, (B, T, W), bf16=dt == BF)
    N = T // 4
    # per (entry, channel): which of the 8 gated tokens wins (A tokens 4j..4j+3,
    # B tokens 4j-4..4j-1; entry 0 has no B tokens)
    pick = g.integers(0, 8, size=(B, N, W))
    pick[:, 0] = pick[:, 0] % 4
    z_a = np.full((B, T, W), -1e4, np.float32)
    z_b = np.full((B, T, W), -1e4, np.float32)
    want = np.empty((B, N, W), np.float32)
    for b in range(B):
        for j in range(N):
            for s in range(8):
                ch = pick[b, j] == s
                if s < 4:
                    z_a[b, 4 * j + s, ch] = 0.0
                    want[b, j, ch] = c_a[b, 4 * j + s, ch]
                else:
                    z_b[b, 4 * j - 4 + (s - 4), ch] = 0.0
                    want[b, j, ch] = c_b[b, 4 * j - 4 + (s - 4), ch]
    # a token of stream A is gated by entry j only; one of stream B by entry j + 1
    # only: the zero logits above never collide
    out = C.csa_compress(dev(c_a, dt), dev(c_b, dt), dev(z_a, dt), dev(z_b, dt), 4)
    assert np.array_equal(host(out), want)


@pytest.mark.parametrize("dt", [torch.float32, BF])
def test_hca_compress_one_hot_and_ratio_one(dt):
    B, T, W, R = 2, 1024, 128, 128
    g = np.random.default_rng(141)
    c = syn.normal(142, (B, T, W), bf16=dt == BF)
    N = T // R
    pick = g.integers(0, R, size=(B, N, W))
    z = np.full((B, T, W), -1e4, np.float32)
    want = np.empty((B, N, W), np.float32)
    for b in range(B):
        for j in range(N):
            for cc in range(W):
                z[b, R * j + pick[b, j, cc], cc] = 0.0
                want[b, j, cc] = c[b, R * j + pick[b, j, cc], cc]
    assert np.array_equal(host(C.hca_compress(dev(c, dt), dev(z, dt), R)), want)
    zz = syn.normal(143, (B, T, W), bf16=dt == BF)
    assert np.array_equal(host(C.hca_compress(dev(c, dt), dev(zz, dt), 1)), c)


def _window_count(p, window, w0, T_win):
    lo = max(0, p - window + 1, w0)
    hi = min(p, w0 + T_win - 1)
    return max(0, hi - lo + 1) if window > 0 else 0


def _check_ones(q, n_keys, sink, got_o, got_l, kind):
    """q [rows, H, d] (the values the kernel read), n_keys [rows]."""
    l = q.astype(np.float64).sum(axis=-1)                       # [rows, H]
    s = np.full(q.shape[1], -np.inf) if sink is None else sink.astype(np.float64)
    with np.errstate(divide="ignore"):
        lse = np.logaddexp(s[None, :], np.log(n_keys)[:, None] + l)
    o = 1.0 - np.exp(s[None, :] - lse)
    np.testing.assert_allclose(got_l, lse, rtol=1e-5, atol=1e-5)
    tol = 4e-3 if kind == "bf16" else 1e-4   # float32: the sums of ~2,000 equal terms round
    assert np.abs(got_o - o[..., None]).max() <= tol


@pytest.mark.parametrize("use_sink", [True, False])
@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("B,Tq", [(1, 300), (3, 1)])
def test_attention_ones_closed_form(B, Tq, kind, use_sink):
    H, N, k, window, ratio = 64, 2000, 256, 128, 16
    dt = torch.float32 if kind == "f32" else BF
    bf = kind == "bf16"
    T_win = 128 + Tq - 1
    q = syn.normal(151, (B, Tq, H, 128), scale=1 / np.sqrt(128), bf16=bf)
    sink = syn.normal(152, (H,)) if use_sink else None
    ones_kv = np.ones((B, N, 128), np.float32)
    ones_w = np.ones((B, T_win, 128), np.float32)
    g = np.random.default_rng(153)
    idx = np.stack([[np.sort(g.choice(N, size=k, replace=False)) for _ in range(Tq)] for _ in range(B)])
    idx = idx.astype(np.int32)
    idx[:, ::5, -17:] = -1
    # sparse: positions near the end of a 4:1 context; dense: a 16:1 context
    for mode in ("sparse", "dense"):
        L = 4 * N if mode == "sparse" else ratio * N
        q_pos = np.stack([np.arange(L - Tq, L) - 37 * b for b in range(B)]).astype(np.int32)
        w0 = np.maximum(q_pos[:, 0] - 127, 0).astype(np.int32)
        print("ones closed form", mode, kind, B, Tq, use_sink, flush=True)
        sk = dev(sink) if use_sink else None
        if mode == "sparse":
            out, lse = C.sparse_attn_fwd(dev(q, dt), dev(ones_kv, dt), dev(idx, torch.int32), dev(ones_w, dt),
                                         dev(w0, torch.int32), sk, dev(q_pos, torch.int32), window, 1.0,
                                         want_lse=True)
        else:
            out, lse = C.dense_compressed_attn_fwd(dev(q, dt), dev(ones_kv, dt), dev(ones_w, dt),
                                                   dev(w0, torch.int32), sk, dev(q_pos, torch.int32), ratio,
                                                   window, 1.0, want_lse=True)
        got_o, got_l = host(out), host(lse)
        for b in range(B):
            n = []
            for t in range(Tq):
                p = int(q_pos[b, t])
                sel = int(((idx[b, t] >= 0) & (idx[b, t] < N)).sum()) if mode == "sparse" \
                    else min(N, (p + 1) // ratio)
                n.append(sel + _window_count(p, window, int(w0[b]), T_win))
            _check_ones(q[b], np.array(n, np.float64), sink, got_o[b], got_l[b], kind)
