"""GPU parity of the decode-time compressor steps (csa_compress_append,
hca_compress_append): appending a sequence token by token builds the same
cache as the batch compressor over the whole prefix (bit for bit: both run the
same per-entry device code) and matches the oracle's compression (R1, R3)."""
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


def _step_rows(t, pos):
    """Rows [B, W] of t [B, T, W] at positions pos (clamped for skipped sequences)."""
    idx = torch.tensor([max(p, 0) for p in pos], device=t.device)
    return t[torch.arange(t.shape[0], device=t.device), idx].contiguous()


@pytest.mark.parametrize("kind,width,out_fmt", [("bf16", 128, None), ("f32", 64, None), ("bf16", 128, "fp8"),
                                                ("bf16", 128, "fp4")])
def test_csa_compress_append(kind, width, out_fmt):
    """Three sequences starting at different steps (the others skipped with a
    negative position meanwhile), a ragged tail of 3 tokens, spare cache rows
    left untouched."""
    B, T, ratio = 3, 4 * 23 + 3, 4
    delays = [0, 5, 13]
    dt = torch.float32 if kind == "f32" else BF
    inp = [syn.csa_prefill(60 + b, T=T, H=16, H_I=4, d_I=width, bf16=(kind == "bf16"), d=width) for b in range(B)]
    st = {n: dev(np.stack([x[n] for x in inp]), dt) for n in ("c_a", "c_b", "z_a", "z_b")}
    N, N_cap = T // ratio, T // ratio + 2
    if out_fmt is None:
        out, scale = torch.zeros(B, N_cap, width, dtype=dt, device="cuda"), None
    elif out_fmt == "fp8":
        out = torch.zeros(B, N_cap, width, dtype=torch.uint8, device="cuda")
        scale = torch.zeros(B, N_cap, dtype=torch.float32, device="cuda")
    else:
        out = torch.zeros(B, N_cap, width // 2, dtype=torch.uint8, device="cuda")
        scale = torch.zeros(B, N_cap, width // 32, dtype=torch.uint8, device="cuda")
    state = C.csa_append_state(B, width, ratio, dt)
    _print("csa_compress_append", kind, width, out_fmt)
    for s in range(T + max(delays)):
        pos = [s - d if 0 <= s - d < T else -1 for d in delays]
        rows = [_step_rows(st[n], pos) for n in ("c_a", "c_b", "z_a", "z_b")]
        C.csa_compress_append(*rows, torch.tensor(pos, dtype=torch.int32, device="cuda"), state, out, scale, ratio)
    batch = C.csa_compress(st["c_a"], st["c_b"], st["z_a"], st["z_b"], ratio, out_fmt=out_fmt)
    got = host(out)
    if out_fmt is None:
        assert np.array_equal(got[:, :N], host(batch))
        assert np.all(got[:, N:] == 0)
        for b in range(B):
            want = O.csa_compress(inp[b]["c_a"], inp[b]["c_b"], inp[b]["z_a"], inp[b]["z_b"], ratio)
            assert_close(got[b, :N], want, kind, f"csa_compress_append b={b}")
    else:
        codes, bscale = batch
        assert np.array_equal(got[:, :N], host(codes))
        assert np.array_equal(host(scale)[:, :N], host(bscale))
        assert np.all(got[:, N:] == 0)


@pytest.mark.parametrize("kind,ratio,T", [("bf16", 128, 128 * 3 + 7), ("f32", 16, 16 * 5 + 3)])
def test_hca_compress_append(kind, ratio, T):
    B, width = 2, 128
    delays = [0, 3]
    dt = torch.float32 if kind == "f32" else BF
    inp = [syn.hca_prefill(70 + b, T=T, H=16, bf16=(kind == "bf16")) for b in range(B)]
    c = dev(np.stack([x["c"] for x in inp]), dt)
    z = dev(np.stack([x["z"] for x in inp]), dt)
    N, N_cap = T // ratio, T // ratio + 1
    out = torch.zeros(B, N_cap, width, dtype=dt, device="cuda")
    state = C.hca_append_state(B, width, ratio, dt)
    _print("hca_compress_append", kind, ratio)
    for s in range(T + max(delays)):
        pos = [s - d if 0 <= s - d < T else -1 for d in delays]
        C.hca_compress_append(_step_rows(c, pos), _step_rows(z, pos), torch.tensor(pos, dtype=torch.int32,
                                                                                    device="cuda"), state, out, ratio)
    got = host(out)
    assert np.array_equal(got[:, :N], host(C.hca_compress(c, z, ratio)))
    assert np.all(got[:, N:] == 0)
    for b in range(B):
        assert_close(got[b, :N], O.hca_compress(inp[b]["c"], inp[b]["z"], ratio), kind, f"hca_compress_append b={b}")


def test_append_rejects_bad_arguments():
    B, width = 2, 128
    st = C.csa_append_state(B, width, 4, BF)
    rows = [torch.zeros(B, width, dtype=BF, device="cuda") for _ in range(4)]
    out = torch.zeros(B, 4, width, dtype=torch.uint8, device="cuda")
    with pytest.raises(C._lib.CsaError):   # fp8 cache without its scale tensor
        C.csa_compress_append(*rows, torch.zeros(B, dtype=torch.int32, device="cuda"), st, out, None, 4)
