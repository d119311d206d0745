"""Properties of the path that hold at any size (GPU):

* P-h: a decode query at position p (one query row, decode kernels) selects
  the same entries as row p of a prefill over the same caches (prefill
  kernels), and its attention output agrees within the bf16 tolerance;
* P-i: the rows of a chunked prefill (the last C positions) equal the last C
  rows of the full prefill bit for bit (indices and attention);
* P-a: sparse attention with every visible entry selected equals dense
  attention over the compressed entries (cf-1.com write-up §3.2: dense means
  no selection), and both equal the oracle;
* the benchmarked decode step (bench.py's closure over the 1M-context layer
  pair: indexer with scores kept in the workspace, sparse attention, HCA
  attention), captured in a HIP graph and replayed, gives the eager call's
  bits on every replay, and the eager call's selection is the one the
  indexer returns with its scores written out.

Indexer operands are exact-grid codes (integers, unit scales), so scores are
exact in float32 whatever the summation order and the selections must agree
exactly across kernels."""
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


def _fp8_grid(seed, shape):
    x = syn.integers(seed, shape, -4, 4)
    return dev(O.e4m3_encode(x), torch.uint8), dev(np.ones(x.shape[:-1], np.float32)), x


def _caches(seed, T, H, H_I, ratio=4):
    N = T // ratio
    kc, ks, _ = _fp8_grid(seed + 1, (1, N, 128))
    kv = dev(syn.normal(seed + 2, (1, N, 128), bf16=True), BF)
    x = dev(syn.normal(seed + 3, (1, T, 128), bf16=True), BF)
    q = dev(syn.normal(seed + 4, (1, T, H, 128), scale=1 / np.sqrt(128), bf16=True), BF)
    qc, qs, _ = _fp8_grid(seed + 5, (1, T, H_I, 128))
    w = dev(syn.grid_weights(seed + 6, (1, T, H_I)))
    sink = dev(syn.normal(seed + 7, (H,)))
    return kc, ks, kv, x, q, qc, qs, w, sink


@pytest.mark.parametrize("T,k", [(2048, 64), (80000, 128)])
def test_decode_equals_prefill_row(T, k):
    """P-h. T = 80,000 takes the long-row selection paths (list mode at
    decode, group maxima at prefill)."""
    H, H_I = 64, 64
    kc, ks, kv, x, q, qc, qs, w, sink = _caches(800, T, H, H_I)
    q_pos = torch.arange(T, dtype=torch.int32, device="cuda")[None]
    w0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    _print("P-h prefill", T)
    idx = C.indexer_topk(qc, qs, w, kc, ks, "fp8", q_pos, 4, k, 128)
    out = C.sparse_attn_fwd(q, kv, idx, x, w0, sink, q_pos, 128, 1.0)
    for p in (0, 5, k * 4 + 3, T // 2 + 1, T - 1):
        pp = torch.tensor([[p]], dtype=torch.int32, device="cuda")
        idx1 = C.indexer_topk(qc[:, p:p + 1].contiguous(), qs[:, p:p + 1].contiguous(), w[:, p:p + 1].contiguous(),
                              kc, ks, "fp8", pp, 4, k, 128)
        assert torch.equal(idx1[0, 0], idx[0, p]), f"selection at p={p}"
        ws0 = torch.tensor([max(0, p - 127)], dtype=torch.int32, device="cuda")
        xw = x[:, max(0, p - 127):p + 1].contiguous()
        o1 = C.sparse_attn_fwd(q[:, p:p + 1].contiguous(), kv, idx1, xw, ws0, sink, pp, 128, 1.0)
        assert_close(host(o1)[0, 0], host(out)[0, p].astype(np.float64), "bf16", f"attention at p={p}")


def test_chunk_equals_full_prefill_rows():
    """P-i: the last 2048 rows of an 8192-token prefill, run as a chunk."""
    T, Cq, H, H_I, k = 8192, 2048, 64, 64, 256
    kc, ks, kv, x, q, qc, qs, w, sink = _caches(810, T, H, H_I)
    q_pos = torch.arange(T, dtype=torch.int32, device="cuda")[None]
    w0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    idx = C.indexer_topk(qc, qs, w, kc, ks, "fp8", q_pos, 4, k, 128)
    out, lse = C.sparse_attn_fwd(q, kv, idx, x, w0, sink, q_pos, 128, 1.0, want_lse=True)
    hq = C.dense_compressed_attn_fwd(q, kv, x, w0, sink, q_pos, 4, 128, 1.0)
    sl = slice(T - Cq, T)
    cq_pos = q_pos[:, sl].contiguous()
    xw = x[:, T - Cq - 127:].contiguous()
    cw0 = torch.tensor([T - Cq - 127], dtype=torch.int32, device="cuda")
    idx_c = C.indexer_topk(qc[:, sl].contiguous(), qs[:, sl].contiguous(), w[:, sl].contiguous(), kc, ks, "fp8",
                           cq_pos, 4, k, 128)
    assert torch.equal(idx_c, idx[:, sl])
    out_c, lse_c = C.sparse_attn_fwd(q[:, sl].contiguous(), kv, idx_c, xw, cw0, sink, cq_pos, 128, 1.0,
                                     want_lse=True)
    assert torch.equal(out_c, out[:, sl]) and torch.equal(lse_c, lse[:, sl])
    hq_c = C.dense_compressed_attn_fwd(q[:, sl].contiguous(), kv, xw, cw0, sink, cq_pos, 4, 128, 1.0)
    assert torch.equal(hq_c, hq[:, sl])


@pytest.mark.parametrize("kind,B,Tq,H", [("bf16", 2, 300, 64), ("bf16", 4, 1, 128), ("f32", 1, 200, 16)])
def test_full_selection_equals_dense(kind, B, Tq, H):
    """P-a on the GPU: every visible entry selected (then -1) = dense attention."""
    ratio, N = 8, 400
    bf = kind == "bf16"
    dt = BF if bf else torch.float32
    L = ratio * N
    q = syn.normal(820, (B, Tq, H, 128), scale=1 / np.sqrt(128), bf16=bf)
    kv = syn.normal(821, (B, N, 128), bf16=bf)
    xw = syn.normal(822, (B, L, 128), bf16=bf)
    sink = syn.normal(823, (H,))
    g = np.random.default_rng(824)
    q_pos = np.stack([np.sort(g.choice(L, size=Tq, replace=False)) for _ in range(B)]).astype(np.int32)
    n_vis = O.visible_entries(q_pos, ratio, N)
    k = int(n_vis.max()) + 3
    idx = np.full((B, Tq, k), -1, np.int32)
    for b in range(B):
        for t in range(Tq):
            idx[b, t, :n_vis[b, t]] = np.arange(n_vis[b, t])
    w0 = np.zeros(B, np.int32)
    a = C.sparse_attn_fwd(dev(q, dt), dev(kv, dt), dev(idx, torch.int32), dev(xw, dt), dev(w0, torch.int32),
                          dev(sink), dev(q_pos, torch.int32), 128, 1.0)
    d = C.dense_compressed_attn_fwd(dev(q, dt), dev(kv, dt), dev(xw, dt), dev(w0, torch.int32), dev(sink),
                                    dev(q_pos, torch.int32), ratio, 128, 1.0)
    assert_close(host(a), host(d).astype(np.float64), kind, "sparse(all) vs dense")
    for b in range(B):
        o, _ = O.dense_attn(q[b], kv[b], xw[b], 0, sink, q_pos[b], ratio, 128)
        assert_close(host(d)[b], o, kind, f"dense vs oracle b={b}")


def test_benchmarked_decode_step_graph_replay():
    """The 1M-context decode pair exactly as bench.py times it (one cache copy),
    eager and then captured in a HIP graph and replayed three times with eager
    work and synchronisations between the replays: every replay writes the
    eager call's indices and outputs bit for bit."""
    import bench
    import csa_synth
    st = bench.decode_workload(torch, C, csa_synth, "graph_check", B=8, L=1 << 20, H=128, H_I=64, d_I=128, k=1024,
                               fmt="fp4", hca=True, copies=1, wid=5, host_sample=False)
    st["step"](0)
    torch.cuda.synchronize()
    ref = {n: st[n].clone() for n in ("idx", "out", "outh")}
    # the selection with scores written out (the path the full-size tests
    # check against the oracle) equals the one kept in the workspace
    idx_s, _ = C.indexer_topk(st["qi"], st["qs"], st["w"], st["codes"][0], st["scales"][0], "fp4", st["q_pos"], 4,
                              1024, 128, want_scores=True)
    assert torch.equal(idx_s, ref["idx"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st["step"](0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st["step"](0)
    for rep in range(3):
        for n in ref:
            st[n].fill_(0 if n == "idx" else 1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in ref:
            assert torch.equal(st[n], ref[n]), f"replay {rep}: {n}"
        st["step"](0)          # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("fmt,Tq,N,d_I,H_I", [("fp4", 1, 262144, 128, 64), ("fp8", 2, 40000, 128, 64),
                                              ("fp8", 300, 5000, 128, 64), ("f32", 40, 3000, 64, 4)])
def test_score_stage_alone_equals_topk_scores(fmt, Tq, N, d_I, H_I):
    """indexer_scores writes the bits indexer_topk writes as its scores, and
    leaves the entries past n(p) untouched."""
    B = 2
    qi32 = dev(syn.normal(840, (B, Tq, H_I, d_I)))
    ki32 = dev(syn.normal(841, (B, N, d_I)))
    if fmt == "f32":
        qc, qs, kc, ks = qi32, None, ki32, None
    else:
        qc, qs = C.csa_quantize_rows(qi32, fmt)
        kc, ks = C.csa_quantize_rows(ki32, fmt)
    w = dev(syn.uniform(842, (B, Tq, H_I)))
    q_pos = dev(np.stack([np.linspace(N, 4 * N + 9, Tq).astype(np.int32) - 5 * b for b in range(B)]), torch.int32)
    _, sc = C.indexer_topk(qc, qs, w, kc, ks, fmt, q_pos, 4, 64, d_I, want_scores=True)
    out = torch.full((B, Tq, N), -7.0, dtype=torch.float32, device="cuda")
    C.indexer_scores(qc, qs, w, kc, ks, fmt, q_pos, 4, d_I, out=out)
    n_vis = np.minimum(N, (host(q_pos).astype(np.int64) + 1) // 4)
    got, ref = host(out), host(sc)
    for b in range(B):
        for t in range(Tq):
            n = n_vis[b, t]
            assert np.array_equal(got[b, t, :n].view(np.uint32), ref[b, t, :n].view(np.uint32)), (b, t)
            assert np.all(got[b, t, n:] == -7.0)
