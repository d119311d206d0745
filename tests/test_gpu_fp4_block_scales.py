"""The fp4 indexer with non-unit E8M0 block scales, bit for bit (pin P-g on
the GPU: FP4 -> FP8 dequantisation is lossless). Keys and queries are e2m1
grid values times a power of two per 32-element block (exponents -1, 0, 1),
so every product and every partial sum is exact in float32 and the scores do
not depend on summation order. The same values encoded as fp8 (e4m3 codes,
unit row scales) through the fp8 path must then give the same scores and
indices as the fp4 path, and both must equal the oracle's exactly — which pins
the fp4 kernels' handling of the block scales (each 32-element block of query
and key scaled by its own exponent) in the decode (list-mode) and prefill
score kernels."""
import numpy as np
import pytest
import torch

import csa_synth as syn
import long_context_attention_csa_amd as C
from oracle import csa_oracle as O
from tests.gpu_common import dev, host

pytestmark = pytest.mark.gpu


def _scaled_grid(seed, shape):
    """e2m1 grid values times 2^E, E in {-1, 0, 1} per 32-element block of the last axis."""
    v = syn.fp4_grid(seed, shape)
    e = syn.integers(seed + 1, shape[:-1] + (shape[-1] // 32,), -1, 1).astype(np.int64)
    return v * np.repeat(np.exp2(e), 32, axis=-1).astype(np.float32), v, e


def _fp4(v, e):
    c = O.e2m1_encode(v)
    packed = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    return dev(packed, torch.uint8), dev((e + 127).astype(np.uint8), torch.uint8)


def _fp8(x):
    return dev(O.e4m3_encode(x), torch.uint8), dev(np.ones(x.shape[:-1], np.float32))


@pytest.mark.parametrize("B,Tq,N,k", [(2, 1, 20000, 256), (1, 64, 4096, 128)])
def test_fp4_block_scales_match_fp8_and_oracle(B, Tq, N, k):
    H_I = 64
    x_q, v_q, e_q = _scaled_grid(121, (B, Tq, H_I, 128))
    x_k, v_k, e_k = _scaled_grid(123, (B, N, 128))
    assert np.array_equal(O.e4m3_decode(O.e4m3_encode(x_k)), x_k)   # exact in e4m3 too
    w = syn.grid_weights(125, (B, Tq, H_I))
    q_pos = np.stack([np.arange(4 * N - Tq, 4 * N) - 4000 * b for b in range(B)]).astype(np.int32)
    dq_pos, dw = dev(q_pos, torch.int32), dev(w)
    print("fp4 block scales", B, Tq, N, k, flush=True)
    q4, q4s = _fp4(v_q, e_q)
    k4, k4s = _fp4(v_k, e_k)
    idx4, s4 = C.indexer_topk(q4, q4s, dw, k4, k4s, "fp4", dq_pos, 4, k, 128, want_scores=True)
    q8, q8s = _fp8(x_q)
    k8, k8s = _fp8(x_k)
    idx8, s8 = C.indexer_topk(q8, q8s, dw, k8, k8s, "fp8", dq_pos, 4, k, 128, want_scores=True)
    g4, g8, i4, i8 = host(s4), host(s8), host(idx4), host(idx8)
    for b in range(B):
        n_vis = O.visible_entries(q_pos[b], 4, N)
        scores = O.indexer_scores(x_q[b], w[b], x_k[b], q_pos[b], 4)
        vis = np.arange(N)[None, :] < n_vis[:, None]
        assert np.array_equal(g4[b][vis], scores[vis]), f"fp4 scores b={b}"
        assert np.array_equal(g8[b][vis], scores[vis]), f"fp8 scores b={b}"
        want = O.topk_select(scores, n_vis, k)
        assert np.array_equal(i4[b], want) and np.array_equal(i8[b], want), f"indices b={b}"
