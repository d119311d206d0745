"""Top-k selection of long decode rows in list mode: the decode score kernel
keeps, per wave of 256 entries, its largest selection composites, and the
selection kernel works from those lists (reading back the entries of waves
whose lists are full). The indices must equal the oracle's selection bit for
bit whenever the scores are exact (integer / e2m1-grid operands), through
every branch: the usual case, rows with fewer listed composites than k, full
waves read back from the scores, and the full-row fallback for many full
waves. Long decode rows are rows of one or a few queries, fp8 or fp4 keys of
width 128 and more than 16,384 entries."""
import numpy as np
import pytest
import torch

import csa_synth as syn
import long_context_attention_csa_amd as C
from oracle import csa_oracle as O
from tests.gpu_common import certified_index_mismatches, dev, host, visible_scores

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def _codes(fmt, x):
    """Unit-scale codes of grid values x [..., 128] (exact in both formats)."""
    if fmt == "fp8":
        return dev(O.e4m3_encode(x), torch.uint8), dev(np.ones(x.shape[:-1], np.float32))
    c = O.e2m1_encode(x)
    packed = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    return dev(packed, torch.uint8), dev(np.full(x.shape[:-1] + (x.shape[-1] // 32,), 127, np.uint8), torch.uint8)


def _grid(fmt, seed, shape):
    return syn.fp4_grid(seed, shape) if fmt == "fp4" else syn.integers(seed, shape, -4, 4)


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
@pytest.mark.parametrize("N,k", [(40000, 128), (20000, 256), (70001, 512)])
def test_lists_exact_grid(fmt, N, k):
    """Exact-grid operands (many tied scores): full rows, a row with fewer
    listed composites than k (n = k + 5), and rows in between."""
    B, H_I = 4, 64
    q_i = _grid(fmt, 51, (B, 1, H_I, 128))
    k_i = _grid(fmt, 52, (B, N, 128))
    w = syn.grid_weights(53, (B, 1, H_I))
    q_pos = np.array([[4 * N + 3], [4 * (k + 5) + 1], [4 * 3000], [4 * (N - 700) + 2]], np.int32)
    _print("lists exact grid", fmt, N, k)
    qc, qs = _codes(fmt, q_i)
    kc, ks = _codes(fmt, k_i)
    idx, sc = C.indexer_topk(qc, qs, dev(w), kc, ks, fmt, dev(q_pos, torch.int32), 4, k, 128, want_scores=True)
    got, got_s = host(idx), host(sc)
    for b in range(B):
        n_vis = O.visible_entries(q_pos[b], 4, N)
        scores = O.indexer_scores(q_i[b], w[b], k_i[b], q_pos[b], 4)
        n = int(n_vis[0])
        assert np.array_equal(got_s[b, 0, :n], scores[0, :n]), f"scores b={b}"
        assert np.array_equal(got[b], O.topk_select(scores, n_vis, k)), f"indices b={b}"


def _single_dim_case(fmt, N, value_of):
    """Keys whose only nonzero channel is channel 0 with grid value value_of(s),
    one query head of ones: the score of entry s is value_of(s) exactly
    (ReLU of a non-negative value, weight 1)."""
    v = value_of(np.arange(N)).astype(np.float32)
    k_i = np.zeros((1, N, 128), np.float32)
    k_i[0, :, 0] = v
    q_i = np.zeros((1, 1, 1, 128), np.float32)
    q_i[..., 0] = 1.0
    w = np.ones((1, 1, 1), np.float32)
    return q_i, k_i, w, v.astype(np.float64)


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_lists_full_waves_read_back(fmt):
    """Scores that rise in steps of 1000 entries: the top-k sit in a few waves
    that each hold more of them than their lists keep, so those waves are read
    back from the stored scores; ties go to the lowest index."""
    N, k = 40000, 128
    q_i, k_i, w, s = _single_dim_case(fmt, N, lambda e: (e // 1000) % 5)
    qc, qs = _codes(fmt, q_i)
    kc, ks = _codes(fmt, k_i)
    q_pos = np.array([[4 * N]], np.int32)
    idx = C.indexer_topk(qc, qs, dev(w), kc, ks, fmt, dev(q_pos, torch.int32), 4, k, 128)
    want = O.topk_select(s[None], [N], k)
    assert np.array_equal(host(idx)[0], want)
    assert np.array_equal(want[0], np.arange(4000, 4000 + k))


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_lists_many_full_waves_fallback(fmt):
    """The first 25 entries of every 256 score 1, the rest 0, and k = 2048: the
    top-k spread over more than 64 full waves, so the row takes the full-row
    path."""
    N, k = 450000, 2048
    q_i, k_i, w, s = _single_dim_case(fmt, N, lambda e: ((e % 256) < 25).astype(np.float32))
    qc, qs = _codes(fmt, q_i)
    kc, ks = _codes(fmt, k_i)
    q_pos = np.array([[4 * N]], np.int32)
    _print("lists many full waves", fmt)
    idx = C.indexer_topk(qc, qs, dev(w), kc, ks, fmt, dev(q_pos, torch.int32), 4, k, 128)
    assert np.array_equal(host(idx)[0], O.topk_select(s[None], [N], k))


def test_lists_all_equal_scores():
    """Every score 0 (zero queries): the k lowest indices win."""
    N, k = 60000, 300
    q_i = np.zeros((2, 1, 64, 128), np.float32)
    k_i = syn.integers(61, (2, N, 128), -4, 4)
    qc, qs = _codes("fp8", q_i)
    kc, ks = _codes("fp8", k_i)
    q_pos = np.array([[4 * N], [4 * 20000 + 1]], np.int32)
    idx = C.indexer_topk(qc, qs, dev(np.ones((2, 1, 64), np.float32)), kc, ks, "fp8", dev(q_pos, torch.int32),
                         4, k, 128)
    got = host(idx)
    assert np.array_equal(got[0, 0], np.arange(k)) and np.array_equal(got[1, 0], np.arange(k))


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_lists_normal_operands(fmt):
    """N(0,1) operands quantised by the library, 131,072 entries, k = 512: the
    selection over the kernel's own scores is exact, and differences from the
    float64 oracle on the same operands are certified near-ties."""
    B, N, H_I, k = 2, 131072, 64, 512
    d = syn.csa_decode(62, B=B, N=N, H=16, H_I=H_I, d_I=128)
    q_pos = np.array([[4 * N], [4 * 100000 + 3]], np.int32)
    qc, qs = C.csa_quantize_rows(dev(d["q_i"][:, None]), fmt)
    kc, ks = C.csa_quantize_rows(dev(d["k_i"]), fmt)
    _print("lists normal", fmt)
    idx, sc = C.indexer_topk(qc, qs, dev(d["w"][:, None]), kc, ks, fmt, dev(q_pos, torch.int32), 4, k, 128,
                             want_scores=True)
    got, got_s = host(idx), host(sc)
    deq = O.dequant_fp8_rows if fmt == "fp8" else O.dequant_mxfp4_rows
    for b in range(B):
        n_vis = O.visible_entries(q_pos[b], 4, N)
        assert np.array_equal(got[b], O.topk_select(visible_scores(got_s[b], n_vis), n_vis, k))
        qd = deq(host(qc)[b], host(qs)[b])
        kd = deq(host(kc)[b], host(ks)[b])
        scores = O.indexer_scores(qd, d["w"][b][None], kd, q_pos[b], 4)
        want = O.topk_select(scores, n_vis, k)
        assert certified_index_mismatches(got[b], want, scores, n_vis, k) <= 1


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_lists_stale_slots_masked(fmt):
    """One workspace for two calls: the first fills every list slot (whole
    rows visible), the second sees shorter rows, so the slots of score blocks
    past a row's visible entries still hold the first call's composites; the
    selection must ignore them. The second call also has a row with n <= k
    (the short-row exit, whose list loads are already in flight)."""
    B, N, H_I, k = 3, 40000, 64, 128
    q_i = _grid(fmt, 71, (B, 1, H_I, 128))
    k_i = _grid(fmt, 72, (B, N, 128))
    w = syn.grid_weights(73, (B, 1, H_I))
    qc, qs = _codes(fmt, q_i)
    kc, ks = _codes(fmt, k_i)
    ws = torch.empty(C.indexer_topk_workspace_size(B, 1, N, H_I, 128, k, fmt), dtype=torch.uint8, device="cuda")
    _print("lists stale slots", fmt)
    for q_pos in (np.full((B, 1), 4 * N, np.int32), np.array([[4 * 3001 + 2], [4 * 100], [4 * 20000]], np.int32)):
        idx = C.indexer_topk(qc, qs, dev(w), kc, ks, fmt, dev(q_pos, torch.int32), 4, k, 128, ws=ws)
        got = host(idx)
        for b in range(B):
            n_vis = O.visible_entries(q_pos[b], 4, N)
            scores = O.indexer_scores(q_i[b], w[b], k_i[b], q_pos[b], 4)
            assert np.array_equal(got[b], O.topk_select(scores, n_vis, k)), f"q_pos={q_pos[b]} b={b}"
