"""The allocation-free sparse attention entry point (sparse_attn_fwd_noalloc):
through the C ABI, its outputs equal sparse_attn_fwd's with a workspace, bit
for bit, on two calls in a row (the second smaller), at decode shapes whose
split results use the library's scratch; shapes beyond the scratch are
rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import csa_synth as syn
import long_context_attention_csa_amd as C
from long_context_attention_csa_amd import _lib
from tests.gpu_common import dev

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _case(seed, B, N, H, k):
    q = dev(syn.normal(seed + 1, (B, 1, H, 128), scale=1 / np.sqrt(128), bf16=True), BF)
    kv = dev(syn.normal(seed + 2, (B, N, 128), bf16=True), BF)
    xw = dev(syn.normal(seed + 3, (B, 128, 128), bf16=True), BF)
    sink = dev(syn.normal(seed + 4, (H,)))
    g = np.random.default_rng(seed)
    idx = np.stack([np.sort(g.choice(N, size=k, replace=False)) for _ in range(B)])[:, None].astype(np.int32)
    q_pos = np.full((B, 1), 4 * N + 1, np.int32)
    w0 = (q_pos[:, 0] - 127).astype(np.int32)
    return q, kv, dev(idx, torch.int32), xw, dev(w0, torch.int32), sink, dev(q_pos, torch.int32)


def test_noalloc_matches_workspace_call():
    for (B, N, H, k), seed in (((8, 100000, 128, 1024), 900), ((3, 5000, 64, 512), 910)):
        args = _case(seed, B, N, H, k)
        assert C.sparse_attn_workspace_size(B, 1, H, 128, k, 128) > 0          # the path uses scratch
        out = torch.empty(B, 1, H, 128, dtype=BF, device="cuda")
        lse = torch.empty(B, 1, H, dtype=torch.float32, device="cuda")
        C.sparse_attn_fwd_noalloc(*args, 128, 1.0, out=out, lse=lse)
        ref, ref_lse = C.sparse_attn_fwd(*args, 128, 1.0, want_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), (B, N, H, k)


def test_noalloc_rejects_shapes_beyond_scratch():
    lib = _lib.lib()
    B, H, k = 255, 128, 4096          # 255 rows: two key splits each, 33.9 MB of split results
    need = C.sparse_attn_workspace_size(B, 1, H, 128, k, 128)
    assert need > C.sparse_attn_noalloc_scratch_bytes()
    P = ctypes.c_void_p(0x1000)
    st = lib.sparse_attn_fwd_noalloc(P, P, P, P, P, None, P, 1, B, 1, 1 << 20, 128, H, 128, k, 128, 1.0, P, None, 0,
                                     None)
    assert st == 4 and b"scratch" in lib.csa_last_error()
