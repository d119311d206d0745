"""The attention kernels' online-softmax branches, driven on purpose and
checked against the oracle (cf-1.com write-up §3.3: the softmax over the
selected entries, the window and the sink).

The bf16 kernels take a block's first tile with its largest logit found
first; later tiles take the exponentials against the running max first and
are redone only when a lane's probabilities outgrow the lazy headroom or no
running max exists yet. Inputs here make that happen:

* logit ramps along the key order (the queries point along one direction u,
  key i carries a multiple of u that grows with i; the queries are long and
  the keys short, so the logits reach the hundreds while the values stay of
  order one, inside the outputs' tolerance): gentle ramps stay inside
  the headroom, medium ones overflow the probability sum without a new max,
  steep ones raise the max on every tile;
* rows whose leading selected entries are all padding, so that a block's
  first tiles hold no key and the running max stays unset;
* a row with no key at all (every index padding, window 0).

Sparse and dense attention, bf16 and float32, many query rows (one split per
row) and decode (keys split across blocks and merged)."""
import numpy as np
import pytest
import torch

import csa_synth as syn
import long_context_attention_csa_amd as C
from oracle import csa_oracle as O
from tests.gpu_common import assert_close, dev, host

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _ramp_inputs(seed, B, Tq, N, H, T_win, slope, kind):
    """Queries 64 u + noise; entry i = slope * i * u / 64 + noise, so that the
    logit of entry i grows by about `slope` (natural units) per entry while
    the values stay of order one; window rows sit at the ramp's top."""
    g = np.random.default_rng(seed)
    u = g.standard_normal(128)
    u /= np.linalg.norm(u)
    q = 64.0 * u[None, None, None, :] + 0.05 * g.standard_normal((B, Tq, H, 128))
    step = slope / 64.0
    kv = (step * np.arange(N))[None, :, None] * u[None, None, :] + 0.01 * g.standard_normal((B, N, 128))
    xw = (step * N * (0.9 + 0.1 * g.random((B, T_win, 1)))) * u[None, None, :] + \
        0.01 * g.standard_normal((B, T_win, 128))
    sink = g.standard_normal(H)
    cast = (lambda x: syn.round_bf16(x.astype(np.float32))) if kind == "bf16" else (lambda x: x.astype(np.float32))
    return cast(q), cast(kv), cast(xw), sink.astype(np.float32)


def _shape(mode):
    return (1, 200) if mode == "prefill" else (2, 1)


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("slope", [0.02, 0.07, 0.2])
@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_sparse_logit_ramp(kind, slope, mode):
    B, Tq = _shape(mode)
    H, N, k = 64, 1500, 512
    T_win = 128 + Tq - 1
    q, kv, xw, sink = _ramp_inputs(700 + int(slope * 100), B, Tq, N, H, T_win, slope, kind)
    g = np.random.default_rng(701)
    idx = np.stack([[np.sort(g.choice(N, size=k, replace=False)) for _ in range(Tq)] for _ in range(B)])
    idx = idx.astype(np.int32)
    q_pos = np.stack([np.arange(4 * N - Tq, 4 * N) - 3 * b for b in range(B)]).astype(np.int32)
    w0 = (q_pos[:, 0] - 127).astype(np.int32)
    dt = torch.float32 if kind == "f32" else BF
    print("sparse ramp", kind, slope, mode, flush=True)
    out, lse = C.sparse_attn_fwd(dev(q, dt), dev(kv, dt), dev(idx, torch.int32), dev(xw, dt), dev(w0, torch.int32),
                                 dev(sink), dev(q_pos, torch.int32), 128, 1.0, want_lse=True)
    got, got_l = host(out), host(lse)
    for b in range(B):
        o, l = O.sparse_attn(q[b], kv[b], idx[b], xw[b], int(w0[b]), sink, q_pos[b], 128)
        assert_close(got[b], o, kind, f"sparse ramp {slope} {mode} b={b}")
        np.testing.assert_allclose(got_l[b], l, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("slope", [0.02, 0.07, 0.2])
@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_dense_logit_ramp(kind, slope, mode):
    B, Tq = _shape(mode)
    H, ratio, N = 64, 16, 700
    L = ratio * N + 5
    T_win = 128 + Tq - 1
    q, kv, xw, sink = _ramp_inputs(720 + int(slope * 100), B, Tq, N, H, T_win, slope, kind)
    q_pos = np.stack([np.arange(L - Tq, L) - 900 * b for b in range(B)]).astype(np.int32)
    w0 = (q_pos[:, 0] - 127).astype(np.int32)
    dt = torch.float32 if kind == "f32" else BF
    print("dense ramp", kind, slope, mode, flush=True)
    out, lse = C.dense_compressed_attn_fwd(dev(q, dt), dev(kv, dt), dev(xw, dt), dev(w0, torch.int32), dev(sink),
                                           dev(q_pos, torch.int32), ratio, 128, 1.0, want_lse=True)
    got, got_l = host(out), host(lse)
    for b in range(B):
        o, l = O.dense_attn(q[b], kv[b], xw[b], int(w0[b]), sink, q_pos[b], ratio, 128)
        assert_close(got[b], o, kind, f"dense ramp {slope} {mode} b={b}")
        np.testing.assert_allclose(got_l[b], l, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_leading_padding_and_empty_rows(kind, mode):
    B, Tq = _shape(mode)
    H, N, k = 64, 3000, 512
    T_win = 128 + Tq - 1
    bf = kind == "bf16"
    q = syn.normal(741, (B, Tq, H, 128), scale=1 / np.sqrt(128), bf16=bf)
    kv = syn.normal(742, (B, N, 128), bf16=bf)
    xw = syn.normal(743, (B, T_win, 128), bf16=bf)
    sink = syn.normal(744, (H,))
    g = np.random.default_rng(745)
    idx = np.stack([[np.sort(g.choice(N, size=k, replace=False)) for _ in range(Tq)] for _ in range(B)])
    idx = idx.astype(np.int32)
    lead = g.integers(60, 400, size=(B, Tq))          # whole tiles of padding, then a ragged one
    for b in range(B):
        for t in range(Tq):
            idx[b, t, :lead[b, t]] = -1
    idx[:, ::3, :] = -1                               # every third row: no selected entry at all
    q_pos = np.stack([np.arange(4 * N - Tq, 4 * N) - 11 * b for b in range(B)]).astype(np.int32)
    w0 = (q_pos[:, 0] - 127).astype(np.int32)
    dt = torch.float32 if kind == "f32" else BF
    for window, use_sink in ((128, True), (0, False)):
        print("leading padding", kind, mode, window, use_sink, flush=True)
        sk = dev(sink) if use_sink else None
        out, lse = C.sparse_attn_fwd(dev(q, dt), dev(kv, dt), dev(idx, torch.int32), dev(xw, dt),
                                     dev(w0, torch.int32), sk, dev(q_pos, torch.int32), window, 1.0, want_lse=True)
        got, got_l = host(out), host(lse)
        for b in range(B):
            o, l = O.sparse_attn(q[b], kv[b], idx[b], xw[b], int(w0[b]), sink if use_sink else np.full(H, -np.inf),
                                 q_pos[b], window)
            assert_close(got[b], o, kind, f"leading padding {mode} window={window} b={b}")
            np.testing.assert_allclose(got_l[b], l, rtol=1e-4, atol=1e-4)
            if window == 0 and not use_sink:
                # rows with no key at all: o = 0 and lse = -inf exactly
                empty = (idx[b] < 0).all(axis=-1)
                assert empty.any()
                assert np.all(got[b][empty] == 0) and np.all(np.isneginf(got_l[b][empty]))
