"""GPU parity of the bfloat16 index-score variant (indexer_topk_bf16_scores)
against the oracle's bfloat16 selection.

On exact grids every float32 score is exact, so rounding it to bfloat16 is a
single decision that both sides take on the same value: the returned scores and
the indices must match the oracle bit for bit. The grid scores run to about
1e5, far beyond bfloat16's 8 significant bits, so many distinct scores merge
into ties that the lower index wins. On N(0,1) operands the float32 sums differ
from float64 by rounding, which can move a score across a bfloat16 rounding
boundary: there the selection on the kernel's own bfloat16 scores must be
exact, the scores may differ by one bfloat16 step on at most 0.1% of
entries, and recall against the oracle stays at or above 0.99.
"""
import numpy as np
import pytest
import torch

import csa_synth as syn
import long_context_attention_csa_amd as C
from oracle import csa_oracle as O
from tests.gpu_common import dev, host, recall, visible_scores
from tests.test_gpu_parity import _grid_operands

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def _oracle_bf16(q_i, w, k_i, q_pos, ratio, k):
    """float64 scores, their bfloat16 rounding and the bfloat16 selection, per batch."""
    B = q_i.shape[0]
    N = k_i.shape[1]
    scores = np.stack([O.indexer_scores(q_i[b], w[b], k_i[b], q_pos[b], ratio) for b in range(B)])
    idx = np.stack([O.topk_select_bf16(scores[b], O.visible_entries(q_pos[b], ratio, N), k) for b in range(B)])
    return scores, O.bf16_round(scores), idx


def _check_exact(idx, sc, q_i, w, k_i, q_pos, k):
    scores, rounded, want = _oracle_bf16(q_i, w, k_i, q_pos, 4, k)
    got_s = host(sc)
    vis = np.isfinite(scores)
    assert np.array_equal(got_s[vis], rounded[vis])
    # the rounding must actually merge distinct scores for this test to bite
    assert np.count_nonzero(rounded[vis] != scores[vis]) > 0
    assert np.array_equal(host(idx), want)


@pytest.mark.parametrize("fmt", ["fp8", "fp4", "f32", "bf16"])
@pytest.mark.parametrize("N,k", [(5003, 256), (20011, 128)])
def test_bf16_scores_exact_grid_decode(fmt, N, k):
    """One query per sequence: the full-row path (N = 5003) and the
    group-maximum path (N = 20011, n/16 >= 4k)."""
    B, d_I = 2, 128
    d = syn.csa_decode(61, B=B, N=N, H=16, H_I=64, d_I=d_I, key_grid=("fp4" if fmt == "fp4" else "int"))
    q_i = d["q_i"][:, None]
    q_pos = np.array([[4 * N + 2], [4 * (N // 2) + 1]], np.int32)
    _print("bf16 scores grid decode", fmt, N, k)
    qc, qs, kc, ks = _grid_operands(fmt, q_i, d["k_i"])
    idx, sc = C.indexer_topk(qc, qs, dev(d["w"][:, None]), kc, ks, fmt, dev(q_pos, torch.int32), 4, k, d_I,
                             want_scores=True, bf16_scores=True)
    assert sc.dtype == torch.bfloat16
    _check_exact(idx, sc, q_i, d["w"][:, None], d["k_i"], q_pos, k)


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
@pytest.mark.parametrize("H_I", [19, 64])
def test_bf16_scores_exact_grid_prefill_batched(fmt, H_I):
    """Prefill rows (matrix-core score kernel, short-row selector): two
    sequences with shifted positions, a partial last query group, padded head
    blocks when H_I < 64."""
    B, T, d_I, k = 2, 1001, 128, 96
    N = 260
    if fmt == "fp4":
        q_i, k_i = syn.fp4_grid(71, (B, T, H_I, d_I)), syn.fp4_grid(72, (B, N, d_I))
    else:
        q_i, k_i = syn.integers(71, (B, T, H_I, d_I), -4, 4), syn.integers(72, (B, N, d_I), -4, 4)
    w = syn.grid_weights(73, (B, T, H_I))
    q_pos = np.stack([np.arange(T), np.arange(T) + 37]).astype(np.int32)
    _print("bf16 scores grid prefill batched", fmt, H_I)
    qc, qs, kc, ks = _grid_operands(fmt, q_i, k_i)
    idx, sc = C.indexer_topk(qc, qs, dev(w), kc, ks, fmt, dev(q_pos, torch.int32), 4, k, d_I, want_scores=True,
                             bf16_scores=True)
    _check_exact(idx, sc, q_i, w, k_i, q_pos, k)


@pytest.mark.parametrize("fmt", ["fp8", "f32"])
def test_bf16_scores_exact_grid_prefill_d64(fmt):
    """d_I = 64 and few heads: the vector score kernel on prefill rows."""
    T, H_I, d_I, k = 1203, 4, 64, 64
    N = T // 4
    q_i, k_i = syn.integers(81, (1, T, H_I, d_I), -4, 4), syn.integers(82, (1, N, d_I), -4, 4)
    w = syn.grid_weights(83, (1, T, H_I))
    q_pos = np.arange(T, dtype=np.int32)[None]
    _print("bf16 scores grid prefill d64", fmt)
    qc, qs, kc, ks = _grid_operands(fmt, q_i, k_i)
    idx, sc = C.indexer_topk(qc, qs, dev(w), kc, ks, fmt, dev(q_pos, torch.int32), 4, k, d_I, want_scores=True,
                             bf16_scores=True)
    _check_exact(idx, sc, q_i, w, k_i, q_pos, k)


def _normal_checks(idx, sc, q_i, w, k_i, q_pos, k):
    got_idx, got_s = host(idx), host(sc)
    scores, rounded, want = _oracle_bf16(q_i, w, k_i, q_pos, 4, k)
    N = k_i.shape[1]
    B, Tq = q_pos.shape
    ndiff = ntot = 0
    for b in range(B):
        n_vis = O.visible_entries(q_pos[b], 4, N)
        # selection on the kernel's own bfloat16 scores is bit-exact
        assert np.array_equal(got_idx[b], O.topk_select(visible_scores(got_s[b], n_vis), n_vis, k))
        for t in range(Tq):
            n = int(n_vis[t])
            g, r = got_s[b, t, :n].astype(np.float64), rounded[b, t, :n]
            diff = g != r
            # the float32 sum and the float64 value can round to neighbouring
            # bfloat16 values: one step apart at most
            step = np.exp2(np.floor(np.log2(np.maximum(np.abs(r[diff]), 2.0 ** -126))) - 7)
            assert np.all(np.abs(g[diff] - r[diff]) <= step)
            ndiff += int(diff.sum())
            ntot += n
    # float32 summation error (about 2^-20 relative here) crosses a bfloat16
    # rounding boundary (2^-8 relative apart) for roughly 1 score in 4000
    _print("bf16 scores differing from the oracle's rounding", ndiff, "of", ntot)
    assert ndiff <= 1e-3 * ntot
    rec = recall(got_idx, want)
    _print("bf16 scores recall vs oracle bf16 selection", rec.min(), rec.mean())
    assert rec.min() >= 0.99


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_bf16_scores_normal_decode_group_path(fmt):
    """N(0,1) operands quantised by the oracle's quantiser, n = 70,000, k = 1024."""
    B, N, H_I, d_I, k = 2, 70001, 64, 128, 1024
    d = syn.csa_decode(62, B=B, N=N, H=16, H_I=H_I, d_I=d_I)
    q_i = d["q_i"][:, None]
    q_pos = np.array([[4 * N], [4 * 66000 + 1]], np.int32)
    quant, dequant = ((O.quant_fp8_rows, O.dequant_fp8_rows) if fmt == "fp8"
                      else (O.quant_mxfp4_rows, O.dequant_mxfp4_rows))
    qc, qs = quant(q_i)
    kc, ks = quant(d["k_i"])
    sdt = torch.uint8 if fmt == "fp4" else torch.float32
    _print("bf16 scores normal decode", fmt)
    idx, sc = C.indexer_topk(dev(qc, torch.uint8), dev(qs, sdt), dev(d["w"][:, None]), dev(kc, torch.uint8),
                             dev(ks, sdt), fmt, dev(q_pos, torch.int32), 4, k, d_I, want_scores=True,
                             bf16_scores=True)
    _normal_checks(idx, sc, dequant(qc, qs), d["w"][:, None], dequant(kc, ks), q_pos, k)


def test_bf16_scores_normal_prefill_short_rows():
    """N(0,1) fp8 operands on prefill rows with n up to 4096 (short-row selector)."""
    B, T, H_I, d_I, k = 1, 1024, 64, 128, 512
    N = 4096
    q_i = syn.normal(91, (B, T, H_I, d_I))
    k_i = syn.normal(92, (B, N, d_I))
    w = syn.uniform(93, (B, T, H_I))
    q_pos = (np.arange(T) * 16 + 15).astype(np.int32)[None]
    qc, qs = O.quant_fp8_rows(q_i)
    kc, ks = O.quant_fp8_rows(k_i)
    _print("bf16 scores normal prefill")
    idx, sc = C.indexer_topk(dev(qc, torch.uint8), dev(qs), dev(w), dev(kc, torch.uint8), dev(ks), "fp8",
                             dev(q_pos, torch.int32), 4, k, d_I, want_scores=True, bf16_scores=True)
    _normal_checks(idx, sc, O.dequant_fp8_rows(qc, qs), w, O.dequant_fp8_rows(kc, ks), q_pos, k)


def test_bf16_scores_ties_and_padding():
    """All-equal scores (threshold bucket holds every entry), three values, a
    row short of k, and rows with no visible entry: lowest indices win."""
    N, k = 12000, 400
    q_i = np.zeros((1, 5, 4, 64), np.float32)
    q_i[0, 1, :, 0] = 1.0
    k_i = np.ones((1, N, 64), np.float32)
    k_i[0, :, 0] = (np.arange(N) % 3).astype(np.float32)
    w = np.ones((1, 5, 4), np.float32)
    q_pos = np.array([[4 * N, 4 * N, 4 * 200, 2, 4 * N]], np.int32)
    idx = C.indexer_topk(dev(q_i), None, dev(w), dev(k_i), None, "f32", dev(q_pos, torch.int32), 4, k, 64,
                         bf16_scores=True)
    got = host(idx)[0]
    assert np.array_equal(got[0], np.arange(k))
    assert np.array_equal(got[1], np.arange(2, 3 * k, 3))
    assert np.array_equal(got[2, :200], np.arange(200)) and np.all(got[2, 200:] == -1)
    assert np.all(got[3] == -1)
    assert np.array_equal(got[4], np.arange(k))


def test_bf16_scores_match_f32_variant_where_exact():
    """Small integer scores (below 256) are exact in bfloat16: both variants
    return the same indices and the same score values."""
    B, N, H_I, d_I, k = 2, 9000, 4, 64, 300
    q_i = np.zeros((B, 1, H_I, d_I), np.float32)
    q_i[:, 0, 0, :4] = 1.0
    k_i = syn.integers(95, (B, N, d_I), 0, 15)
    w = np.zeros((B, 1, H_I), np.float32)
    w[:, 0, 0] = 1.0
    q_pos = np.array([[4 * N], [4 * 5000]], np.int32)
    a, sa = C.indexer_topk(dev(q_i), None, dev(w), dev(k_i), None, "f32", dev(q_pos, torch.int32), 4, k, d_I,
                           want_scores=True)
    b, sb = C.indexer_topk(dev(q_i), None, dev(w), dev(k_i), None, "f32", dev(q_pos, torch.int32), 4, k, d_I,
                           want_scores=True, bf16_scores=True)
    assert np.array_equal(host(a), host(b))
    for r in range(B):
        n = int(O.visible_entries(q_pos[r, 0], 4, N))
        assert np.array_equal(host(sa)[r, 0, :n], host(sb)[r, 0, :n])
