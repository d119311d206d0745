"""GPU parity of the attention backward (sparse_attn_bwd, dense_compressed_attn_bwd)
against the oracle's gradients on the same bf16-rounded inputs.

Tolerance: the kernels multiply bf16 operands (q, keys, dO, and the bf16-rounded
probabilities and logit gradients) with float32 accumulation, and read the
forward's bf16 output for D = dO . O. Each product term carries a relative
error of at most about 2^-8; over sums of many terms of mixed sign the error
behaves like a random walk, so a relative L2 error of 1e-2 and a largest error
of 2e-2 of the largest gradient magnitude leave a wide margin while any wrong
term (a missing scale, a transposed operand, a wrong key) fails by far more.
"""
import numpy as np
import pytest
import torch

import csa_synth as syn
import long_context_attention_csa_amd as C
from oracle import csa_oracle as O
from tests.gpu_common import dev, host

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _print(*a):
    print(*a, flush=True)


def check_grad(got, want, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    scale = max(1e-6, float(np.abs(want).max()) if want.size else 0.0)
    err = float(np.abs(got - want).max()) if got.size else 0.0
    den = np.linalg.norm(want)
    rel = np.linalg.norm(got - want) / den if den > 0 else np.linalg.norm(got)
    _print(f"  {what}: max-abs {err:.3e} (of {scale:.3e}), rel-L2 {rel:.3e}")
    assert err <= 2e-2 * scale and rel <= 1e-2, f"{what}: max-abs {err:.3e} / {scale:.3e}, rel-L2 {rel:.3e}"


def _inputs(seed, B, Tq, N, H, T_win):
    q = syn.normal(seed * 10 + 1, (B, Tq, H, 128), scale=1 / np.sqrt(128), bf16=True)
    kv = syn.normal(seed * 10 + 2, (B, N, 128), bf16=True)
    xw = syn.normal(seed * 10 + 3, (B, T_win, 128), bf16=True)
    sink = syn.normal(seed * 10 + 4, (H,))
    dout = syn.normal(seed * 10 + 5, (B, Tq, H, 128), bf16=True)
    return q, kv, xw, sink, dout


def _run_sparse(q, kv, idx, xw, w0, sink, q_pos, dout, window, scale):
    t = [dev(q, BF), dev(kv, BF), dev(idx, torch.int32), dev(xw, BF), dev(w0, torch.int32),
         None if sink is None else dev(sink), dev(q_pos, torch.int32)]
    out, lse = C.sparse_attn_fwd(*t, window, scale, want_lse=True)
    return C.sparse_attn_bwd(*t, out, lse, dev(dout, BF), window, scale)


def _compare(res, B, oracle_fn, sink):
    dq, dkv, dxw, dsink = (None if x is None else host(x) for x in res)
    ds_sum = 0.0
    for b in range(B):
        wq, wkv, wxw, wds = oracle_fn(b)
        check_grad(dq[b], wq, f"dq b={b}")
        check_grad(dkv[b], wkv, f"dkv b={b}")
        check_grad(dxw[b], wxw, f"dx_win b={b}")
        ds_sum = ds_sum + wds
    if sink is not None:
        check_grad(dsink, ds_sum, "dsink")
    else:
        assert dsink is None


@pytest.mark.parametrize("H,B,Tq,N,k,window,scale", [(64, 2, 37, 300, 48, 128, 1.0), (128, 1, 70, 500, 96, 64, 0.8),
                                                     (64, 3, 5, 4000, 512, 128, 1.0)])
def test_sparse_attn_bwd(H, B, Tq, N, k, window, scale):
    """Random selections with -1 holes and an out-of-range index, windows
    clipped by the supplied rows, several sequences."""
    T_win = 150
    g = np.random.default_rng(7)
    q_pos = np.stack([np.sort(g.integers(0, 4 * N, Tq)) for _ in range(B)]).astype(np.int32)
    w0 = np.array([max(0, int(q_pos[b, -1]) - T_win + 1) for b in range(B)], np.int32)
    idx = np.stack([[np.sort(g.choice(N, size=k, replace=False)) for _ in range(Tq)] for _ in range(B)])
    idx = idx.astype(np.int32)
    idx[:, ::4, -k // 3:] = -1
    idx[0, 1, 0] = N + 5                      # skipped like -1
    q, kv, xw, sink, dout = _inputs(11, B, Tq, N, H, T_win)
    _print("sparse_attn_bwd", H, B, Tq, N, k, window, scale)
    res = _run_sparse(q, kv, idx, xw, w0, sink, q_pos, dout, window, scale)
    _compare(res, B, lambda b: O.sparse_attn_bwd(q[b], kv[b], idx[b], xw[b], int(w0[b]), sink, q_pos[b], dout[b],
                                                 window, scale), sink)


def test_sparse_attn_bwd_no_sink_and_empty_rows():
    """No sink; rows whose key set is empty (no selected entry, window 0 rows
    visible) get zero gradients."""
    B, Tq, N, H, k, T_win = 1, 12, 100, 64, 16, 20
    q_pos = np.arange(Tq, dtype=np.int32)[None] * 3
    w0 = np.array([1000], np.int32)           # window rows lie after every query: no window keys
    g = np.random.default_rng(2)
    idx = np.full((B, Tq, k), -1, np.int32)
    for t in range(0, Tq, 2):
        idx[0, t, :5] = np.sort(g.choice(N, 5, replace=False))
    q, kv, xw, _, dout = _inputs(12, B, Tq, N, H, T_win)
    _print("sparse_attn_bwd no sink, empty rows")
    res = _run_sparse(q, kv, idx, xw, w0, None, q_pos, dout, 128, 1.0)
    # the oracle's softmax is 0/0 on an empty key set without a sink: it runs on
    # the rows that have keys, and the others must give exact zeros
    dq, dkv, dxw, dsink = (None if x is None else host(x) for x in res)
    assert dsink is None and np.all(dq[0, 1::2] == 0)
    wq, wkv, wxw, _ = O.sparse_attn_bwd(q[0, ::2], kv[0], idx[0, ::2], xw[0], int(w0[0]), np.full(H, -np.inf),
                                        q_pos[0, ::2], dout[0, ::2], 128, 1.0)
    check_grad(dq[0, ::2], wq, "dq")
    check_grad(dkv[0], wkv, "dkv")
    assert np.all(dxw == 0)


def _run_dense(q, kv, xw, w0, sink, q_pos, dout, ratio, window):
    t = [dev(q, BF), dev(kv, BF), dev(xw, BF), dev(w0, torch.int32), dev(sink), dev(q_pos, torch.int32)]
    out, lse = C.dense_compressed_attn_fwd(*t, ratio, window, 1.0, want_lse=True)
    return C.dense_compressed_attn_bwd(*t, out, lse, dev(dout, BF), ratio, window, 1.0)


@pytest.mark.parametrize("H,T,ratio", [(64, 600, 4), (128, 300, 16)])
def test_dense_attn_bwd_prefill(H, T, ratio):
    N = T // ratio
    q_pos = np.arange(T, dtype=np.int32)[None]
    w0 = np.zeros(1, np.int32)
    q, kv, xw, sink, dout = _inputs(13, 1, T, N, H, T)
    _print("dense_attn_bwd prefill", H, T, ratio)
    res = _run_dense(q, kv, xw, w0, sink, q_pos, dout, ratio, 128)
    _compare(res, 1, lambda b: O.dense_attn_bwd(q[b], kv[b], xw[b], 0, sink, q_pos[b], ratio, dout[b], 128), sink)


def test_dense_attn_bwd_multi_pass():
    """N = 65,536 entries makes each query row's slot budget large, so the 200
    query rows run in 4 passes whose key sums accumulate in pass order; rows
    of the 65,536 entries that no query sees get exact zeros."""
    B, Tq, N, H, ratio, T_win = 1, 200, 65536, 64, 4, 256
    q_pos = (np.arange(Tq) * 37 + 100).astype(np.int32)[None]
    w0 = np.array([int(q_pos[0, -1]) - T_win + 1], np.int32)
    q, kv, xw, sink, dout = _inputs(14, B, Tq, N, H, T_win)
    assert C.dense_attn_bwd_workspace_size(B, Tq, N, T_win, H, 128, 128) > 0
    _print("dense_attn_bwd multi-pass")
    res = _run_dense(q, kv, xw, w0, sink, q_pos, dout, ratio, 128)
    n_max = int(O.visible_entries(q_pos[0, -1], ratio, N))
    dkv = host(res[1])[0]
    assert np.all(dkv[n_max:] == 0)
    wq, wkv, wxw, wds = O.dense_attn_bwd(q[0], kv[0, :n_max], xw[0], int(w0[0]), sink, q_pos[0], ratio, dout[0], 128)
    check_grad(host(res[0])[0], wq, "dq")
    check_grad(dkv[:n_max], wkv, "dkv")
    check_grad(host(res[2])[0], wxw, "dx_win")
    check_grad(host(res[3]), wds, "dsink")


def test_attn_bwd_deterministic():
    """Two calls on the same inputs give identical bits (no float atomics)."""
    B, Tq, N, H, k, T_win = 1, 300, 2000, 64, 256, 427
    q_pos = (np.arange(Tq) + 7900).astype(np.int32)[None]
    w0 = np.array([7900 - 127], np.int32)
    g = np.random.default_rng(5)
    # neighbouring queries share most entries: many contributions per key
    base = np.sort(g.choice(N, size=k, replace=False))
    idx = np.full((1, Tq, k), -1, np.int32)
    for t in range(Tq):
        row = np.unique(np.concatenate([base[: k - 20], g.choice(N, 20)]))[:k]
        idx[0, t, :len(row)] = row
    q, kv, xw, sink, dout = _inputs(15, B, Tq, N, H, T_win)
    a = _run_sparse(q, kv, idx, xw, w0, sink, q_pos, dout, 128, 1.0)
    b = _run_sparse(q, kv, idx, xw, w0, sink, q_pos, dout, 128, 1.0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_sparse_attn_bwd_fullsize_sampled():
    """The CSA prefill shape the benchmark times (T = 65,536, 64 heads, top-512
    from the fp8 indexer, window 128, sink), run exactly as there: repeated
    calls are bit-identical; dq of sampled rows, dkv of sampled entries (the
    oracle's per-row gradients summed over every row that selected them) and
    dx_win of sampled window rows match the oracle."""
    dev_, bf = "cuda", BF
    T, H, H_I, d_I, k, W = 65536, 64, 64, 128, 512, 128
    N = T // 4
    s = 6000
    c = {n: syn.normal_device(s + i, (1, T, 128), dev_, bf) for i, n in enumerate(["c_a", "c_b", "z_a", "z_b"])}
    ci = {n: syn.normal_device(s + 10 + i, (1, T, d_I), dev_, bf) for i, n in enumerate(["a", "b", "za", "zb"])}
    q = syn.normal_device(s + 20, (1, T, H, 128), dev_, bf, scale=1 / np.sqrt(128))
    qi32 = syn.normal_device(s + 21, (1, T, H_I, d_I), dev_)
    qi, qs = C.csa_quantize_rows(qi32, "fp8")
    del qi32
    w = syn.uniform_device(s + 22, (1, T, H_I), dev_)
    sink = syn.normal_device(s + 23, (H,), dev_)
    dout = syn.normal_device(s + 24, (1, T, H, 128), dev_, bf)
    q_pos = torch.arange(T, dtype=torch.int32, device=dev_)[None]
    win_start = torch.zeros(1, dtype=torch.int32, device=dev_)
    E = C.csa_compress(c["c_a"], c["c_b"], c["z_a"], c["z_b"], 4)
    KI = C.csa_compress(ci["a"], ci["b"], ci["za"], ci["zb"], 4, out_fmt="fp8")
    idx = C.indexer_topk(qi, qs, w, KI[0], KI[1], "fp8", q_pos, 4, k, d_I)
    out, lse = C.sparse_attn_fwd(q, E, idx, c["c_a"], win_start, sink, q_pos, W, 1.0, want_lse=True)
    _print("bwd full size: first call")
    a = C.sparse_attn_bwd(q, E, idx, c["c_a"], win_start, sink, q_pos, out, lse, dout, W, 1.0)
    _print("bwd full size: second call")
    b = C.sparse_attn_bwd(q, E, idx, c["c_a"], win_start, sink, q_pos, out, lse, dout, W, 1.0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert torch.isfinite(a[3]).all()
    dq, dkv, dxw = host(a[0])[0], host(a[1])[0], host(a[2])[0]
    qh, Eh, xh = host(q)[0], host(E)[0], host(c["c_a"])[0]
    doh, idxh, sk = host(dout)[0], host(idx)[0], host(sink)

    def row_bwd(p):
        sel = idxh[p][(idxh[p] >= 0) & (idxh[p] < N)]
        rows = O.window_rows(p, W, 0, T)
        keys = np.concatenate([Eh[sel], xh[rows]], 0)
        dqr, dk, _ = O.attend_bwd(qh[p], keys, sk, doh[p], 1.0)
        return sel, rows, dqr, dk

    for p in (0, 1, 3, 4, 5, 130, 2047, 2048, 2049, 4099, 9000, 20000, 33333, 50000, 65534, 65535):
        check_grad(dq[p], row_bwd(p)[2], f"dq row {p}")
    counts = np.bincount(idxh[idxh >= 0], minlength=N)
    for e in (int(np.argmin(np.abs(counts - 300))), int(np.argmin(np.abs(counts - 40)))):
        want = np.zeros(128)
        for p in np.nonzero((idxh == e).any(axis=1))[0]:
            sel, _, _, dk = row_bwd(int(p))
            want += dk[int(np.nonzero(sel == e)[0][0])]
        _print(f"  entry {e}: selected by {counts[e]} rows")
        check_grad(dkv[e], want, f"dkv entry {e}")
    for t in (0, 40000, 65535):
        want = np.zeros(128)
        for p in range(t, min(T, t + W)):
            sel, rows, _, dk = row_bwd(p)
            want += dk[len(sel) + int(np.nonzero(rows == t)[0][0])]
        check_grad(dxw[t], want, f"dx_win row {t}")


def test_dense_attn_bwd_fullsize_sampled():
    """The HCA prefill shape the benchmark times (T = 131,072, 64 heads, ratio
    128: 1,024 entries, window 128, sink), run exactly as there: repeated calls
    are bit-identical; dq of sampled rows, dkv of the last entries (each seen
    by the few hundred rows after its block: the oracle's per-row gradients
    summed over all of them) and dx_win of sampled window rows match the
    oracle."""
    dev_, bf = "cuda", BF
    T, H, ratio, W = 131072, 64, 128, 128
    N = T // ratio
    s = 7000
    q = syn.normal_device(s, (1, T, H, 128), dev_, bf, scale=1 / np.sqrt(128))
    E = syn.normal_device(s + 1, (1, N, 128), dev_, bf)
    xw = syn.normal_device(s + 2, (1, T, 128), dev_, bf)
    sink = syn.normal_device(s + 3, (H,), dev_)
    dout = syn.normal_device(s + 4, (1, T, H, 128), dev_, bf)
    q_pos = torch.arange(T, dtype=torch.int32, device=dev_)[None]
    win_start = torch.zeros(1, dtype=torch.int32, device=dev_)
    out, lse = C.dense_compressed_attn_fwd(q, E, xw, win_start, sink, q_pos, ratio, W, 1.0, want_lse=True)
    _print("dense bwd full size: first call")
    a = C.dense_compressed_attn_bwd(q, E, xw, win_start, sink, q_pos, out, lse, dout, ratio, W, 1.0)
    _print("dense bwd full size: second call")
    b = C.dense_compressed_attn_bwd(q, E, xw, win_start, sink, q_pos, out, lse, dout, ratio, W, 1.0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert torch.isfinite(a[3]).all()
    entries = (N - 1, N - 2, N - 9)   # seen by rows from ratio * (e + 1) - 1 on
    dq_rows = (0, 1, 126, 127, 128, 255, 4099, 65535, 65536, 100001, T - 2, T - 1)
    win_rows = (0, 70000, T - 1)
    need = set(dq_rows)
    need.update(range(ratio * (min(entries) + 1) - 1, T))
    for t in win_rows:
        need.update(range(t, min(T, t + W)))
    rows = np.array(sorted(need), dtype=np.int64)
    at = {int(p): i for i, p in enumerate(rows)}
    ri = torch.as_tensor(rows, device=dev_)
    qh, doh = host(q[0, ri]), host(dout[0, ri])
    dq = host(a[0][0, ri])
    dkv, dxw = host(a[1])[0], host(a[2])[0]
    Eh, xh, sk = host(E)[0], host(xw)[0], host(sink)
    cache = {}

    def row_bwd(p):
        if p not in cache:
            n = int(O.visible_entries(p, ratio, N))
            wr = O.window_rows(p, W, 0, T)
            keys = np.concatenate([Eh[:n], xh[wr]], 0)
            dqr, dk, _ = O.attend_bwd(qh[at[p]], keys, sk, doh[at[p]], 1.0)
            cache[p] = (n, wr, dqr, dk)
        return cache[p]

    for p in dq_rows:
        check_grad(dq[at[p]], row_bwd(p)[2], f"dq row {p}")
    for e in entries:
        want = np.zeros(128)
        seen = range(ratio * (e + 1) - 1, T)
        for p in seen:
            want += row_bwd(p)[3][e]
        _print(f"  entry {e}: seen by {len(seen)} rows")
        check_grad(dkv[e], want, f"dkv entry {e}")
    for t in win_rows:
        want = np.zeros(128)
        for p in range(t, min(T, t + W)):
            n, wr, _, dk = row_bwd(p)
            want += dk[n + int(np.nonzero(wr == t)[0][0])]
        check_grad(dxw[t], want, f"dx_win row {t}")
