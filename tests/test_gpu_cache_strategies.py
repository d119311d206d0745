"""The three state-cache strategies (cf-1.com write-up §4.4) on the GPU: a
decode run of three sequences (each at its own position; appends of the CSA
and HCA compressors and of the window ring, with a checkpoint of every ring
after every 1024th token) is interrupted at a prefix P and resumed

* from the last checkpoint (restore, then append the tokens since it again),
* from a full-length history of every ring's rows (full SWA caching), or
* from nothing (zero SWA caching: append the last 128 tokens again, their
  recomputed entries going to a scratch cache),

and then continued to the end. Every ring and every compressed entry must
equal the uninterrupted run's bit for bit, and so must a decode attention
call over them."""
import numpy as np
import pytest
import torch

import csa_synth as syn
import long_context_attention_csa_amd as C
from tests.gpu_common import dev

pytestmark = pytest.mark.gpu
BF = torch.bfloat16
T, B, W, R, PERIOD = 2600, 3, 128, 128, 1024
START = [0, 300, 600]                  # sequence b's position at step t is t - START[b]
RESUME = [2100, 1800, 1500]            # the prefix each sequence resumes at


def _streams():
    s = {n: dev(syn.normal(950 + i, (B, T, W), bf16=True), BF) for i, n in
         enumerate(["c_a", "c_b", "z_a", "z_b", "c", "z"])}
    return s


def _fresh(garbage_seed=None):
    """Rings and caches; rings filled with garbage (a resumed sequence has no
    valid state), caches zero."""
    def ring(shape):
        if garbage_seed is None:
            return torch.zeros(*shape, dtype=BF, device="cuda")
        return dev(syn.normal(garbage_seed + len(shape), shape, bf16=True), BF)
    return {"csa": ring((B, 8, 4, W)), "hca": ring((B, 128, 2, W)), "win": ring((B, R, W)),
            "E": torch.zeros(B, T // 4, W, dtype=BF, device="cuda"),
            "EH": torch.zeros(B, T // 128, W, dtype=BF, device="cuda")}


def _append(st, s, pos_np, cache_E=None, cache_EH=None):
    pos = dev(pos_np, torch.int32)
    idx = torch.from_numpy(np.maximum(pos_np, 0)).long().cuda()
    ar = torch.arange(B, device="cuda")
    rows = {n: s[n][ar, idx].contiguous() for n in s}
    C.csa_compress_append(rows["c_a"], rows["c_b"], rows["z_a"], rows["z_b"], pos, st["csa"],
                          st["E"] if cache_E is None else cache_E, None, 4)
    C.hca_compress_append(rows["c"], rows["z"], pos, st["hca"], st["EH"] if cache_EH is None else cache_EH, 128)
    C.window_append(rows["c_a"], pos, st["win"])
    return pos


def _positions(t):
    return np.array([t - START[b] for b in range(B)], np.int32)


def _run(st, s, t0, t1, ckpt=None, scratch=None):
    for t in range(t0, t1):
        pos_np = _positions(t)
        if scratch is not None:    # warm-up appends: entries go to the scratch caches
            pos = _append(st, s, pos_np, scratch["E"], scratch["EH"])
        else:
            pos = _append(st, s, pos_np)
        if ckpt is not None:
            for n in ("csa", "hca", "win"):
                C.state_checkpoint(st[n], pos, PERIOD, ckpt[n])


@pytest.fixture(scope="module")
def reference():
    s = _streams()
    st = _fresh()
    ckpt = {n: torch.zeros(B, 2, *st[n].shape[1:], dtype=BF, device="cuda") for n in ("csa", "hca", "win")}
    _run(st, s, 0, T, ckpt)
    torch.cuda.synchronize()
    return s, st, ckpt


def _cut_caches(ref_st, st):
    """Classical caches as they stand at each sequence's prefix (entries of
    completed blocks before P), the rest zero."""
    for b in range(B):
        P = RESUME[b]
        st["E"][b, :P // 4] = ref_st["E"][b, :P // 4]
        st["EH"][b, :P // 128] = ref_st["EH"][b, :P // 128]


def _check(ref_st, st, what):
    torch.cuda.synchronize()
    for n in ("csa", "hca", "win", "E", "EH"):
        assert torch.equal(st[n], ref_st[n]), f"{what}: {n}"
    # a decode attention call over the final rings and caches
    last = np.array([T - 1 - START[b] for b in range(B)], np.int32)
    q = dev(syn.normal(960, (B, 1, 64, W), scale=1 / np.sqrt(W), bf16=True), BF)
    sink = dev(syn.normal(961, (64,)))
    qp = dev(last[:, None], torch.int32)
    w0 = dev(np.maximum(last - R + 1, 0), torch.int32)
    a = C.dense_compressed_attn_fwd(q, st["EH"], st["win"], w0, sink, qp, 128, 128, 1.0, win_ring=True)
    r = C.dense_compressed_attn_fwd(q, ref_st["EH"], ref_st["win"], w0, sink, qp, 128, 128, 1.0, win_ring=True)
    assert torch.equal(a, r), f"{what}: attention"


def _t_of(P, b):
    return P + START[b]


def test_resume_from_checkpoint(reference):
    s, ref_st, ckpt = reference
    st = _fresh(garbage_seed=970)
    _cut_caches(ref_st, st)
    slot = dev(np.array([RESUME[b] // PERIOD - 1 for b in range(B)], np.int32), torch.int32)
    for n in ("csa", "hca", "win"):
        C.state_restore(ckpt[n], slot, st[n])
    # append again the tokens since each sequence's checkpoint, then continue
    for t in range(min(_t_of(PERIOD * (RESUME[b] // PERIOD), b) for b in range(B)), T):
        pos_np = _positions(t)
        for b in range(B):   # before its checkpoint a sequence skips (its state is restored)
            if pos_np[b] < PERIOD * (RESUME[b] // PERIOD):
                pos_np[b] = -1
        _append(st, s, pos_np)
    _check(ref_st, st, "checkpoint")


def test_resume_from_full_history(reference):
    s, ref_st, _ = reference
    st = _fresh(garbage_seed=980)
    _cut_caches(ref_st, st)
    # full SWA caching: every position's rows, laid out as the rings hold them
    hist = {"csa": torch.stack([s["c_a"], s["c_b"], s["z_a"], s["z_b"]], dim=2).contiguous(),
            "hca": torch.stack([s["c"], s["z"]], dim=2).contiguous(), "win": s["c_a"]}
    # the history of sequence b is indexed by its own positions
    P = dev(np.array(RESUME, np.int32), torch.int32)
    for n in ("csa", "hca", "win"):
        h = torch.stack([hist[n][b] for b in range(B)])
        C.ring_fill(h, P, st[n])
    for t in range(min(_t_of(RESUME[b], b) for b in range(B)), T):
        pos_np = _positions(t)
        for b in range(B):
            if pos_np[b] < RESUME[b]:
                pos_np[b] = -1
        _append(st, s, pos_np)
    _check(ref_st, st, "full history")


def test_resume_from_nothing(reference):
    s, ref_st, _ = reference
    st = _fresh(garbage_seed=990)
    _cut_caches(ref_st, st)
    scratch = _fresh()
    # zero SWA caching: the last 128 tokens before P appended again (their
    # recomputed entries may lack earlier tokens: they go to a scratch cache)
    for t in range(min(_t_of(RESUME[b] - 128, b) for b in range(B)), T):
        pos_np = _positions(t)
        warm = np.array([RESUME[b] - 128 <= pos_np[b] < RESUME[b] for b in range(B)])
        live = np.array([pos_np[b] >= RESUME[b] for b in range(B)])
        if warm.any():
            _append(st, s, np.where(warm, pos_np, -1).astype(np.int32), scratch["E"], scratch["EH"])
        if live.any():
            _append(st, s, np.where(live, pos_np, -1).astype(np.int32))
    _check(ref_st, st, "no state")
