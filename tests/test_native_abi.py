"""The C ABI used from a plain C program (tests/native/layer_demo.c, built by
build() with gcc against include/csa_hip.h and libcsa_hip.so): no Python,
PyTorch or ctypes between the caller and the library.

Host side: the program's `validate` mode checks status strings, the version
string and calls that must fail validation (no device work). GPU: its `run`
mode drives one CSA layer (both compressors, the float32 indexer with top-k,
sparse attention) and one HCA layer (compressor, dense attention) on seeded
inputs the test writes to files; every result is checked against the oracle:
compressed entries and scores within float32 rounding, the selection equal
to the oracle's selection over the program's own scores, attention outputs
and log-sum-exps within the float32 tolerance."""
import os
import subprocess

import numpy as np
import pytest

import csa_synth as syn
from oracle import csa_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "tests", "native", "layer_demo")


def _demo():
    assert os.path.exists(DEMO), "tests/native/layer_demo is not built (run __graft_entry__.build())"
    return DEMO


def test_native_validate():
    r = subprocess.run([_demo(), "validate"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "validate ok" in r.stdout and "gfx950" in r.stdout


@pytest.mark.gpu
def test_native_layers(tmp_path):
    T, H, H_I, d_I, k, window = 1024, 16, 4, 64, 64, 128
    inp = syn.csa_prefill(91, T=T, H=H, H_I=H_I, d_I=d_I, bf16=False)
    hca = syn.hca_prefill(92, T=T, H=H, bf16=False)
    files = {n + ".f32": inp[n] for n in ("c_a", "c_b", "z_a", "z_b", "ci_a", "ci_b", "zi_a", "zi_b", "q_i", "w",
                                         "q", "sink")}
    files.update({"c.f32": hca["c"], "z.f32": hca["z"], "q2.f32": hca["q"], "sink2.f32": hca["sink"]})
    for name, a in files.items():
        np.ascontiguousarray(a, dtype=np.float32).tofile(tmp_path / name)
    print("native layers", T, H, H_I, d_I, k, window, flush=True)
    r = subprocess.run([_demo(), "run", str(tmp_path), str(T), str(H), str(H_I), str(d_I), str(k), str(window)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    N, NH = T // 4, T // 128
    rd = lambda name, shape, dt=np.float32: np.fromfile(tmp_path / name, dtype=dt).reshape(shape)
    kv, k_i = rd("kv.out", (N, 128)), rd("k_i.out", (N, d_I))
    idx, scores = rd("idx.out", (T, k), np.int32), rd("scores.out", (T, N))
    o, lse = rd("o.out", (T, H, 128)), rd("lse.out", (T, H))
    kvh, o2, lse2 = rd("kvh.out", (NH, 128)), rd("o2.out", (T, H, 128)), rd("lse2.out", (T, H))
    q_pos = np.arange(T)
    n_vis = O.visible_entries(q_pos, 4, N)

    # compressors
    assert np.abs(kv - O.csa_compress(inp["c_a"], inp["c_b"], inp["z_a"], inp["z_b"], 4)).max() < 1e-4
    assert np.abs(k_i - O.csa_compress(inp["ci_a"], inp["ci_b"], inp["zi_a"], inp["zi_b"], 4)).max() < 1e-4
    assert np.abs(kvh - O.hca_compress(hca["c"], hca["z"], 128)).max() < 1e-4
    # indexer: scores of the visible entries against the oracle's on the same
    # keys, then the selection over the program's own scores
    ref_s = O.indexer_scores(inp["q_i"], inp["w"], k_i, q_pos, 4)
    vis = np.arange(N)[None, :] < n_vis[:, None]
    err = np.abs(scores - ref_s)[vis].max()
    assert err <= 1e-4 * max(1.0, np.abs(ref_s[vis]).max()), err
    got_s = np.where(vis, scores.astype(np.float64), 0.0)
    assert np.array_equal(idx, O.topk_select(got_s, n_vis, k))
    # attention on the program's own entries and selection
    want_o, want_l = O.sparse_attn(inp["q"], kv, idx, inp["c_a"], 0, inp["sink"], q_pos, window)
    _close(o, want_o, "csa attention")
    np.testing.assert_allclose(lse, want_l, rtol=1e-4, atol=1e-4)
    want_o2, want_l2 = O.dense_attn(hca["q"], kvh, hca["c"], 0, hca["sink"], q_pos, 128, window)
    _close(o2, want_o2, "hca attention")
    np.testing.assert_allclose(lse2, want_l2, rtol=1e-4, atol=1e-4)


def _close(got, want, what):
    err = np.abs(got - want).max()
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert err <= 2e-4 and rel <= 2e-5, f"{what}: max-abs {err:.3e}, rel-L2 {rel:.3e}"
