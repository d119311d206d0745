"""GPU parity at the full workload sizes, run exactly as bench.py runs them
(same entry points, shapes, formats and launch configurations), checked on
sampled outputs that the oracle computes one by one:

* decode pair at a 1,048,576-token context (B=8, fp4 indexer keys, top-1024,
  128 heads; HCA over 8192 entries) and CSA decode at 262,144 (B=32, fp8);
* CSA prefill T=65,536 (compressors, fp8 indexer, top-512, 64 heads);
* HCA prefill T=131,072 (128:1 compressor, dense attention);
* an 8192-query prefill chunk at the end of the 1M context (fp4 indexer over
  262,144 entries, sparse and HCA attention, 128 heads).

Index selection is checked bit-exactly against the oracle's selection over
the GPU's own float32 scores (the same definition applied to the same
numbers); the scores themselves against float64 oracle scores on the same
quantised operands; recall against the oracle's selection on those operands
(>= 0.99). Attention outputs are checked against the oracle run with the
GPU's indices (bf16: max-abs 2e-2, rel-L2 1e-2). Prefill score rows are
recomputed for the sampled queries alone: each score is one MFMA column over
its own query and key, so it does not depend on which queries share a block.
"""
import numpy as np
import pytest
import torch

import csa_synth as syn
import long_context_attention_csa_amd as C
from oracle import csa_oracle as O
from tests.gpu_common import DEV, assert_close, host, recall, visible_scores

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _print(*a):
    print(*a, flush=True)


def _deq(fmt, codes, scales):
    codes, scales = host(codes), host(scales)
    return O.dequant_mxfp4_rows(codes, scales) if fmt == "fp4" else O.dequant_fp8_rows(codes, scales)


def _check_selection_and_scores(fmt, qi, qs, w, kc, ks, q_pos_row, ratio, k, got_idx_row, got_scores_row, what):
    """One query row: exact selection over the GPU's scores, scores vs float64
    oracle scores on the same quantised operands, recall vs the oracle."""
    N = kc.shape[0]
    n_vis = O.visible_entries([q_pos_row], ratio, N)
    sel = O.topk_select(visible_scores(got_scores_row[None], n_vis), n_vis, k)[0]
    assert np.array_equal(sel, got_idx_row), f"{what}: selection differs from the oracle's over the GPU scores"
    qd = _deq(fmt, qi, qs)[None]                                # [1, H_I, d_I]
    kd = _deq(fmt, kc, ks)                                      # [N, d_I]
    want = O.indexer_scores(qd, host(w)[None], kd, [q_pos_row], ratio)[0]
    n = int(n_vis[0])
    np.testing.assert_allclose(got_scores_row[:n], want[:n], rtol=2e-5, atol=1e-3, err_msg=what)
    want_idx = O.topk_select(want[None], n_vis, k)
    rec = recall(got_idx_row[None], want_idx)[0]
    _print(what, "recall vs oracle on the same operands", rec)
    assert rec >= 0.99, f"{what}: recall {rec}"


# ---------------------------------------------------------------- decode

@pytest.mark.parametrize("case", ["pair_1m_fp4", "csa_262k_fp8"])
def test_full_decode(case):
    if case == "pair_1m_fp4":
        B, L, fmt, hca, s = 8, 1 << 20, "fp4", True, 7000
    else:
        B, L, fmt, hca, s = 32, 1 << 18, "fp8", False, 7100
    H, H_I, d_I, k = 128, 64, 128, 1024
    N, NH = L // 4, L // 128
    _print("full decode", case)
    ki32 = syn.normal_device(s + 2, (B, N, d_I), DEV)
    kc, ks = C.csa_quantize_rows(ki32, fmt)
    del ki32
    kv = syn.normal_device(s + 1, (B, N, 128), DEV, BF)
    xw = syn.normal_device(s + 3, (B, 128, 128), DEV, BF)
    q = syn.normal_device(s + 4, (B, 1, H, 128), DEV, BF, scale=1 / np.sqrt(128))
    qi32 = syn.normal_device(s + 5, (B, 1, H_I, d_I), DEV)
    qi, qs = C.csa_quantize_rows(qi32, fmt)
    w = syn.uniform_device(s + 6, (B, 1, H_I), DEV)
    sink = syn.normal_device(s + 7, (H,), DEV)
    q_pos = torch.full((B, 1), L, dtype=torch.int32, device=DEV)
    win_start = torch.full((B,), L - 127, dtype=torch.int32, device=DEV)
    idx, sc = C.indexer_topk(qi, qs, w, kc, ks, fmt, q_pos, 4, k, d_I, want_scores=True)
    out = C.sparse_attn_fwd(q, kv, idx, xw, win_start, sink, q_pos, 128, 1.0)
    if hca:
        kvh = syn.normal_device(s + 11, (B, NH, 128), DEV, BF)
        xh = syn.normal_device(s + 12, (B, 128, 128), DEV, BF)
        qh = syn.normal_device(s + 13, (B, 1, H, 128), DEV, BF, scale=1 / np.sqrt(128))
        sinkh = syn.normal_device(s + 14, (H,), DEV)
        outh = C.dense_compressed_attn_fwd(qh, kvh, xh, win_start, sinkh, q_pos, 128, 128, 1.0)
        assert torch.equal(outh, C.dense_compressed_attn_fwd(qh, kvh, xh, win_start, sinkh, q_pos, 128, 128, 1.0))
    # repeated calls give the same bits
    idx2, sc2 = C.indexer_topk(qi, qs, w, kc, ks, fmt, q_pos, 4, k, d_I, want_scores=True)
    assert torch.equal(idx, idx2) and torch.equal(sc, sc2)
    assert torch.equal(out, C.sparse_attn_fwd(q, kv, idx, xw, win_start, sink, q_pos, 128, 1.0))
    torch.cuda.synchronize()
    got_idx, got_s = host(idx)[:, 0], host(sc)[:, 0]
    # every row: the selection is the oracle's selection over the GPU's scores
    for b in range(B):
        sel = O.topk_select(got_s[b][None].astype(np.float64), O.visible_entries([L], 4, N), k)[0]
        assert np.array_equal(sel, got_idx[b]), f"row {b}: selection"
    for b in (0, B - 1):
        _check_selection_and_scores(fmt, qi[b, 0], qs[b, 0], w[b, 0], kc[b], ks[b], L, 4, k, got_idx[b], got_s[b],
                                    f"{case} row {b}")
        sel = got_idx[b]
        o, _ = O.sparse_attn(host(q[b]), host(kv[b][torch.from_numpy(sel.astype(np.int64)).to(DEV)]),
                             np.arange(k)[None], host(xw[b]), L - 127, host(sink), [L], 128)
        assert_close(host(out[b]), o, "bf16", f"{case} sparse attention row {b}")
        if hca:
            oh, _ = O.dense_attn(host(qh[b]), host(kvh[b]), host(xh[b]), L - 127, host(sinkh), [L], 128, 128)
            assert_close(host(outh[b]), oh, "bf16", f"{case} HCA attention row {b}")


# ---------------------------------------------------------------- CSA prefill

def test_full_csa_prefill_T65536():
    T, H, H_I, d_I, k, W = 65536, 64, 64, 128, 512, 128
    N = T // 4
    s = 7200
    _print("full CSA prefill T=65536")
    c = [syn.normal_device(s + i, (1, T, 128), DEV, BF) for i in range(4)]
    ci = [syn.normal_device(s + 10 + i, (1, T, d_I), DEV, BF) for i in range(4)]
    q = syn.normal_device(s + 20, (1, T, H, 128), DEV, BF, scale=1 / np.sqrt(128))
    qi32 = syn.normal_device(s + 21, (1, T, H_I, d_I), DEV)
    qi, qs = C.csa_quantize_rows(qi32, "fp8")
    del qi32
    w = syn.uniform_device(s + 22, (1, T, H_I), DEV)
    sink = syn.normal_device(s + 23, (H,), DEV)
    q_pos = torch.arange(T, dtype=torch.int32, device=DEV)[None]
    win_start = torch.zeros(1, dtype=torch.int32, device=DEV)
    E = C.csa_compress(c[0], c[1], c[2], c[3], 4)
    kc, ks = C.csa_compress(ci[0], ci[1], ci[2], ci[3], 4, out_fmt="fp8")
    idx = C.indexer_topk(qi, qs, w, kc, ks, "fp8", q_pos, 4, k, d_I)
    out = C.sparse_attn_fwd(q, E, idx, c[0], win_start, sink, q_pos, W, 1.0)
    # repeated calls give the same bits
    assert torch.equal(idx, C.indexer_topk(qi, qs, w, kc, ks, "fp8", q_pos, 4, k, d_I))
    assert torch.equal(out, C.sparse_attn_fwd(q, E, idx, c[0], win_start, sink, q_pos, W, 1.0))
    torch.cuda.synchronize()
    # compressor: every entry against the oracle
    ch = [host(x[0]) for x in c]
    assert_close(host(E[0]), O.csa_compress(ch[0], ch[1], ch[2], ch[3], 4), "bf16", "compressed KV")
    # stratified rows: the first queries, the boundary n(p) = k, the last query
    g = np.random.default_rng(11)
    fixed = [0, 1, 2, 3, 4 * k - 5, 4 * k - 1, 4 * k, 4 * k + 3, T - 2, T - 1]
    rows = np.array(sorted(set(fixed) | set(g.choice(T, 64 - len(fixed), replace=False).tolist())))[:64]
    rt = torch.from_numpy(rows).to(DEV)
    idx_s, sc_s = C.indexer_topk(qi[:, rt].contiguous(), qs[:, rt].contiguous(), w[:, rt].contiguous(), kc, ks,
                                 "fp8", q_pos[:, rt].contiguous(), 4, k, d_I, want_scores=True)
    got_full = host(idx)[0][rows]
    assert np.array_equal(host(idx_s)[0], got_full), "row subset selects what the full run selected"
    got_s = host(sc_s)[0]
    kd = _deq("fp8", kc[0], ks[0])
    qd = _deq("fp8", qi[0, rt], qs[0, rt])
    want = O.indexer_scores(qd, host(w[0, rt]), kd, rows, 4)
    n_vis = O.visible_entries(rows, 4, N)
    for i, p in enumerate(rows):
        n = int(n_vis[i])
        sel = O.topk_select(got_s[i][None].astype(np.float64), [n], k)[0]
        assert np.array_equal(sel, got_full[i]), f"p={p}: selection over the GPU scores"
        np.testing.assert_allclose(got_s[i, :n], want[i, :n], rtol=2e-5, atol=1e-3, err_msg=f"p={p}")
    rec = recall(got_full, O.topk_select(want, n_vis, k))
    _print("prefill recall min", rec.min())
    assert rec.min() >= 0.99
    o, _ = O.sparse_attn(host(q[0, rt]), host(E[0]), got_full, ch[0], 0, host(sink), rows, W)
    assert_close(host(out[0, rt]), o, "bf16", "CSA prefill attention (sampled rows)")


# ---------------------------------------------------------------- HCA prefill

def test_full_hca_prefill_T131072():
    T, H, W = 131072, 64, 128
    s = 7300
    _print("full HCA prefill T=131072")
    cc = syn.normal_device(s, (1, T, 128), DEV, BF)
    zz = syn.normal_device(s + 1, (1, T, 128), DEV, BF)
    q = syn.normal_device(s + 2, (1, T, H, 128), DEV, BF, scale=1 / np.sqrt(128))
    sink = syn.normal_device(s + 3, (H,), DEV)
    q_pos = torch.arange(T, dtype=torch.int32, device=DEV)[None]
    win_start = torch.zeros(1, dtype=torch.int32, device=DEV)
    E = C.hca_compress(cc, zz, 128)
    out = C.dense_compressed_attn_fwd(q, E, cc, win_start, sink, q_pos, 128, W, 1.0)
    assert torch.equal(out, C.dense_compressed_attn_fwd(q, E, cc, win_start, sink, q_pos, 128, W, 1.0))
    torch.cuda.synchronize()
    ch = host(cc[0])
    assert_close(host(E[0]), O.hca_compress(ch, host(zz[0]), 128), "bf16", "HCA compressed entries")
    g = np.random.default_rng(12)
    fixed = [0, 1, 126, 127, 128, 255, 256, T - 129, T - 128, T - 1]
    rows = np.array(sorted(set(fixed) | set(g.choice(T, 256 - len(fixed), replace=False).tolist())))[:256]
    rt = torch.from_numpy(rows).to(DEV)
    o, _ = O.dense_attn(host(q[0, rt]), host(E[0]), ch, 0, host(sink), rows, 128, W)
    assert_close(host(out[0, rt]), o, "bf16", "HCA prefill attention (sampled rows)")


# ---------------------------------------------------------------- 8192-query chunk at 1M

def test_full_prefill_chunk_1m():
    L, Tq, H, H_I, d_I, k, W = 1 << 20, 8192, 128, 64, 128, 1024, 128
    N, NH = L // 4, L // 128
    s = 7400
    _print("full prefill chunk 8192 queries at 1M")
    ki32 = syn.normal_device(s, (1, N, d_I), DEV)
    kc, ks = C.csa_quantize_rows(ki32, "fp4")
    del ki32
    E = syn.normal_device(s + 1, (1, N, 128), DEV, BF)
    xw = syn.normal_device(s + 2, (1, Tq + W - 1, 128), DEV, BF)
    q = syn.normal_device(s + 3, (1, Tq, H, 128), DEV, BF, scale=1 / np.sqrt(128))
    qi32 = syn.normal_device(s + 4, (1, Tq, H_I, d_I), DEV)
    qi, qs = C.csa_quantize_rows(qi32, "fp4")
    del qi32
    w = syn.uniform_device(s + 5, (1, Tq, H_I), DEV)
    sink = syn.normal_device(s + 6, (H,), DEV)
    Eh = syn.normal_device(s + 7, (1, NH, 128), DEV, BF)
    xh = syn.normal_device(s + 8, (1, Tq + W - 1, 128), DEV, BF)
    qh = syn.normal_device(s + 9, (1, Tq, H, 128), DEV, BF, scale=1 / np.sqrt(128))
    sinkh = syn.normal_device(s + 10, (H,), DEV)
    q_pos = torch.arange(L - Tq, L, dtype=torch.int32, device=DEV)[None]
    ws0 = L - Tq - W + 1
    win_start = torch.full((1,), ws0, dtype=torch.int32, device=DEV)
    idx = C.indexer_topk(qi, qs, w, kc, ks, "fp4", q_pos, 4, k, d_I)
    out = C.sparse_attn_fwd(q, E, idx, xw, win_start, sink, q_pos, W, 1.0)
    outh = C.dense_compressed_attn_fwd(qh, Eh, xh, win_start, sinkh, q_pos, 128, W, 1.0)
    # repeated calls give the same bits
    assert torch.equal(idx, C.indexer_topk(qi, qs, w, kc, ks, "fp4", q_pos, 4, k, d_I))
    assert torch.equal(out, C.sparse_attn_fwd(q, E, idx, xw, win_start, sink, q_pos, W, 1.0))
    assert torch.equal(outh, C.dense_compressed_attn_fwd(qh, Eh, xh, win_start, sinkh, q_pos, 128, W, 1.0))
    torch.cuda.synchronize()
    g = np.random.default_rng(13)
    fixed = [0, 1, Tq - 1]
    rows = np.array(sorted(set(fixed) | set(g.choice(Tq, 16 - len(fixed), replace=False).tolist())))[:16]
    rt = torch.from_numpy(rows).to(DEV)
    pos = rows + (L - Tq)
    idx_s, sc_s = C.indexer_topk(qi[:, rt].contiguous(), qs[:, rt].contiguous(), w[:, rt].contiguous(), kc, ks,
                                 "fp4", q_pos[:, rt].contiguous(), 4, k, d_I, want_scores=True)
    got_full = host(idx)[0][rows]
    assert np.array_equal(host(idx_s)[0], got_full), "row subset selects what the full run selected"
    got_s = host(sc_s)[0]
    kd = _deq("fp4", kc[0], ks[0])
    qd = _deq("fp4", qi[0, rt], qs[0, rt])
    n_vis = O.visible_entries(pos, 4, N)
    for i in range(len(rows)):
        n = int(n_vis[i])
        sel = O.topk_select(got_s[i][None].astype(np.float64), [n], k)[0]
        assert np.array_equal(sel, got_full[i]), f"row {rows[i]}: selection over the GPU scores"
        want = O.indexer_scores(qd[i:i + 1], host(w[0, rt[i:i + 1]]), kd, pos[i:i + 1], 4)[0]
        np.testing.assert_allclose(got_s[i, :n], want[:n], rtol=2e-5, atol=1e-3, err_msg=f"row {rows[i]}")
        rec = recall(got_full[i][None], O.topk_select(want[None], [n], k))[0]
        assert rec >= 0.99, f"row {rows[i]}: recall {rec}"
    Eh_h, xw_h, xh_h = host(Eh[0]), host(xw[0]), host(xh[0])
    for i, r in enumerate(rows):
        sel = got_full[i]
        o, _ = O.sparse_attn(host(q[0, r:r + 1]), host(E[0][torch.from_numpy(sel.astype(np.int64)).to(DEV)]),
                             np.arange(k)[None], xw_h, ws0, host(sink), pos[i:i + 1], W)
        assert_close(host(out[0, r:r + 1]), o, "bf16", f"chunk sparse attention row {r}")
    oh, _ = O.dense_attn(host(qh[0, rt]), Eh_h, xh_h, ws0, host(sinkh), pos, 128, W)
    assert_close(host(outh[0, rt]), oh, "bf16", "chunk HCA attention (sampled rows)")
