"""Projections around the attention core on the GPU (bf16 MFMA GEMM) against
the oracle: the general grouped GEMM (ragged M and N, several groups with
strides, bf16 and float32 outputs, shapes for both tile sizes), the grouped
output projection and the shared-latent query projections. Tolerance: inputs
are bf16 values (exact in both), products accumulate in float32, and each
bf16 output (and the bf16 intermediate of the two-stage projections) is
rounded once (2^-9 relative): max-abs 2e-2 of the largest output magnitude
and relative L2 1e-2."""
import numpy as np
import pytest
import torch

import csa_synth as syn
import long_context_attention_csa_amd as C
from long_context_attention_csa_amd import _lib
from oracle import csa_oracle as O
from tests.gpu_common import dev, host

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _close(got, want, what):
    got = np.asarray(got, np.float64)
    err = np.abs(got - want).max()
    scale = np.abs(want).max()
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert err <= 2e-2 * scale and rel <= 1e-2, f"{what}: max-abs {err:.3e} (scale {scale:.3e}), rel-L2 {rel:.3e}"


def _w(seed, shape, fan_in):
    return syn.normal(seed, shape, scale=1.0 / np.sqrt(fan_in), bf16=True)


@pytest.mark.parametrize("M,N,K", [(128, 128, 64), (300, 517, 192), (1, 64, 128), (1000, 100, 1024), (4100, 4000, 128)])
@pytest.mark.parametrize("out_dtype", [BF, torch.float32])
def test_linear(M, N, K, out_dtype):
    a = syn.normal(1100, (M, K), bf16=True)
    w = _w(1101, (N, K), K)
    got = C.linear_bf16(dev(a, BF), dev(w, BF), out_dtype)
    want = a.astype(np.float64) @ w.astype(np.float64).T
    _close(host(got), want, f"linear {M}x{N}x{K}")


def test_linear_groups_with_strides():
    """Three groups reading column blocks of one A and writing column blocks of
    one C (the first stage of the grouped projection), through the C ABI."""
    lib = _lib.lib()
    T, G, Kg, r = 257, 3, 128, 40
    a = syn.normal(1102, (T, G * Kg), bf16=True)
    w = _w(1103, (G, r, Kg), Kg)
    c = torch.full((T, G * r), 7.0, dtype=torch.float32, device="cuda")
    da, dw = dev(a, BF), dev(w, BF)
    import ctypes
    st = lib.csa_linear_bf16(ctypes.c_void_p(da.data_ptr()), G * Kg, Kg, ctypes.c_void_p(dw.data_ptr()), Kg, r * Kg,
                             ctypes.c_void_p(c.data_ptr()), 0, G * r, r, T, r, Kg, G,
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.csa_last_error()
    for g in range(G):
        want = a[:, g * Kg:(g + 1) * Kg].astype(np.float64) @ w[g].astype(np.float64).T
        _close(host(c)[:, g * r:(g + 1) * r], want, f"group {g}")


@pytest.mark.parametrize("T,H,G,r,D", [(300, 128, 8, 512, 1024), (77, 64, 4, 64, 256), (5, 16, 1, 128, 64),
                                       (33, 32, 32, 2, 100), (2100, 128, 8, 1024, 1000)])
def test_grouped_out_proj(T, H, G, r, D):
    d = 128
    o = syn.normal(1104, (T, H, d), bf16=True)
    wg = _w(1105, (G, r, (H // G) * d), (H // G) * d)
    wo = _w(1106, (D, G * r), G * r)
    got = C.grouped_out_proj(dev(o, BF), dev(wg, BF), dev(wo, BF))
    _close(host(got), O.grouped_output_projection(o, wg, wo), f"grouped T={T} H={H} G={G} r={r} D={D}")


def test_query_proj_shared():
    T, D, r_q, H, H_I = 333, 1024, 256, 64, 64
    x = syn.normal(1107, (T, D), bf16=True)
    wdq = _w(1108, (r_q, D), D)
    wuq = _w(1109, (H * 128, r_q), r_q)
    wiq = _w(1110, (H_I * 128, r_q), r_q)
    q, qi = C.query_proj_shared(dev(x, BF), dev(wdq, BF), dev(wuq, BF), dev(wiq, BF))
    wq, wqi = O.shared_query_projection(x, wdq, wuq, wiq)
    _close(host(q), wq, "attention queries")
    _close(host(qi), wqi, "indexer queries")


@pytest.mark.parametrize("B,T,D,S,width,out_dtype", [(1, 300, 512, 4, 128, BF), (2, 77, 256, 8, 64, torch.float32),
                                                     (1, 2048, 1024, 8, 128, BF)])
def test_kv_proj(B, T, D, S, width, out_dtype):
    """The compressor's input streams from the hidden state, then the CSA
    compressor on the projected streams, against the oracle."""
    x = syn.normal(1111, (B, T, D), bf16=True)
    w = _w(1112, (S, width, D), D)
    got = C.kv_proj(dev(x, BF), dev(w, BF), out_dtype)
    assert tuple(got.shape) == (S, B, T, width)
    want = O.kv_projection(x.reshape(B * T, D), w).reshape(S, B, T, width)
    _close(host(got), want, f"kv_proj B={B} T={T} D={D} S={S}")
    if S >= 4 and out_dtype == torch.float32:
        e = C.csa_compress(got[0], got[1], got[2], got[3], 4)
        for b in range(B):
            _close(host(e)[b], O.csa_compress(*(want[s, b] for s in range(4)), ratio=4), f"compress b={b}")
