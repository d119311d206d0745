"""Python binding of the C ABI: same names, argument marshalling only.

Each function takes torch tensors that already live on the GPU, allocates the
outputs (and workspace, unless one is passed in) with torch, and calls the
library on torch's current stream. Every step of the computation runs in the
HIP kernels of libcsa_hip.so; nothing here computes.
"""
from __future__ import annotations

import ctypes
import math

import torch

from ._lib import (ATTN_BATCH_INVARIANT, ATTN_WIN_RING, CSA_BF16, CSA_F32, CSA_FP4_E2M1, CSA_FP8_E4M3, KID,
                   check, lib)

FMT = {"f32": CSA_F32, "bf16": CSA_BF16, "fp8": CSA_FP8_E4M3, "fp4": CSA_FP4_E2M1}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _float_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")


def _torch_dtype(fmt: int):
    return {CSA_F32: torch.float32, CSA_BF16: torch.bfloat16}[fmt]


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _workspace(nbytes: int, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel()} < {nbytes}")
    return ws, ws.numel()


def _quant_out(shape_rows, width, fmt, device):
    if fmt == CSA_FP8_E4M3:
        return (torch.empty(*shape_rows, width, dtype=torch.uint8, device=device),
                torch.empty(*shape_rows, dtype=torch.float32, device=device))
    return (torch.empty(*shape_rows, width // 2, dtype=torch.uint8, device=device),
            torch.empty(*shape_rows, width // 32, dtype=torch.uint8, device=device))


def csa_quantize_rows(x: torch.Tensor, out_fmt: str):
    """Quantise the last axis of x to "fp8" (per-row float32 scale) or "fp4" (E8M0 per 32)."""
    _contig(x)
    fmt = FMT[out_fmt]
    width = x.shape[-1]
    rows = x.numel() // width if width else 0
    out, scale = _quant_out(tuple(x.shape[:-1]), width, fmt, x.device)
    check("csa_quantize_rows", lib().csa_quantize_rows(_ptr(x), _float_dtype(x), rows, width, _ptr(out), fmt,
                                                       _ptr(scale), _stream()))
    return out, scale


def csa_compress(c_a, c_b, z_a, z_b, ratio: int = 4, out_fmt: str | None = None):
    """CSA compressor. Inputs [B, T, width]; returns E [B, T//ratio, width] (and the
    scale tensor when out_fmt is "fp8"/"fp4")."""
    _contig(c_a, c_b, z_a, z_b)
    in_t = _float_dtype(c_a)
    B, T, width = c_a.shape
    N = T // ratio
    fmt = FMT[out_fmt] if out_fmt else in_t
    if fmt in (CSA_F32, CSA_BF16):
        out, scale = torch.empty(B, N, width, dtype=_torch_dtype(fmt), device=c_a.device), None
    else:
        out, scale = _quant_out((B, N), width, fmt, c_a.device)
    check("csa_compress", lib().csa_compress(_ptr(c_a), _ptr(c_b), _ptr(z_a), _ptr(z_b), in_t, B, T, width, ratio,
                                             _ptr(out), fmt, _ptr(scale), _stream()))
    return out if scale is None else (out, scale)


def hca_compress(c, z, ratio: int = 128, out_fmt: str | None = None):
    """HCA compressor. Inputs [B, T, width]; returns [B, T//ratio, width]."""
    _contig(c, z)
    in_t = _float_dtype(c)
    B, T, width = c.shape
    fmt = FMT[out_fmt] if out_fmt else in_t
    out = torch.empty(B, T // ratio, width, dtype=_torch_dtype(fmt), device=c.device)
    check("hca_compress", lib().hca_compress(_ptr(c), _ptr(z), in_t, B, T, width, ratio, _ptr(out), fmt, _stream()))
    return out


def csa_append_state(B: int, width: int, ratio: int = 4, dtype=torch.bfloat16, device="cuda"):
    """A zeroed state ring for csa_compress_append: [B, 2*ratio, 4, width]."""
    return torch.zeros(B, 2 * ratio, 4, width, dtype=dtype, device=device)


def hca_append_state(B: int, width: int, ratio: int = 128, dtype=torch.bfloat16, device="cuda"):
    """A zeroed state ring for hca_compress_append: [B, ratio, 2, width]."""
    return torch.zeros(B, ratio, 2, width, dtype=dtype, device=device)


def csa_compress_append(c_a, c_b, z_a, z_b, pos, state, out, out_scale=None, ratio: int = 4):
    """Decode-time CSA compressor step: new token rows [B, width] at positions pos
    (int32 [B]); updates state [B, 2*ratio, 4, width] and, for sequences whose
    token completes a block, writes that entry into out [B, N_cap, width] (and
    out_scale for fp8/fp4 caches)."""
    _contig(c_a, c_b, z_a, z_b, pos, state, out, out_scale)
    in_t = _float_dtype(c_a)
    B, width = c_a.shape
    N_cap = out.shape[1]
    if out.dtype == torch.uint8:
        fmt = CSA_FP8_E4M3 if out.shape[2] == width else CSA_FP4_E2M1
    else:
        fmt = _float_dtype(out)
    check("csa_compress_append", lib().csa_compress_append(_ptr(c_a), _ptr(c_b), _ptr(z_a), _ptr(z_b), in_t, B, width,
                                                           ratio, _ptr(pos), _ptr(state), N_cap, _ptr(out), fmt,
                                                           _ptr(out_scale), _stream()))


def hca_compress_append(c, z, pos, state, out, ratio: int = 128):
    """Decode-time HCA compressor step: new token rows [B, width] at positions pos;
    updates state [B, ratio, 2, width] and writes completed entries into out
    [B, N_cap, width]."""
    _contig(c, z, pos, state, out)
    in_t = _float_dtype(c)
    B, width = c.shape
    check("hca_compress_append", lib().hca_compress_append(_ptr(c), _ptr(z), in_t, B, width, ratio, _ptr(pos),
                                                           _ptr(state), out.shape[1], _ptr(out), _float_dtype(out),
                                                           _stream()))


def indexer_topk_workspace_size(B, Tq, N, H_I, d_I, k, fmt: str, bf16_scores: bool = False) -> int:
    fn = lib().indexer_topk_bf16_scores_workspace_size if bf16_scores else lib().indexer_topk_workspace_size
    return int(fn(B, Tq, N, H_I, d_I, k, FMT[fmt]))


def indexer_topk(q_idx, q_scale, w, k_idx, k_scale, fmt: str, q_pos, ratio: int, k: int, d_I: int,
                 want_scores: bool = False, ws=None, idx_out=None, bf16_scores: bool = False):
    """Indexer scores and top-k. q_idx [B, Tq, H_I, d_I(/2 for fp4)], w [B, Tq, H_I] float32,
    k_idx [B, N, d_I(/2)], q_pos int32 [B, Tq]. Returns idx int32 [B, Tq, k]
    (and the scores [B, Tq, N] when want_scores: float32, or bfloat16 when
    bf16_scores, in which case selection also runs on the bfloat16-rounded scores)."""
    _contig(q_idx, q_scale, w, k_idx, k_scale, q_pos)
    f = FMT[fmt]
    B, Tq, H_I = q_idx.shape[:3]
    N = k_idx.shape[1]
    dev = q_idx.device
    if idx_out is None:
        idx_out = torch.empty(B, Tq, k, dtype=torch.int32, device=dev)
    sdt = torch.bfloat16 if bf16_scores else torch.float32
    scores = torch.empty(B, Tq, N, dtype=sdt, device=dev) if want_scores else None
    ws, nbytes = _workspace(indexer_topk_workspace_size(B, Tq, N, H_I, d_I, k, fmt, bf16_scores), dev, ws)
    name = "indexer_topk_bf16_scores" if bf16_scores else "indexer_topk"
    check(name, getattr(lib(), name)(_ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(k_idx), _ptr(k_scale), f,
                                     _ptr(q_pos), B, Tq, N, H_I, d_I, ratio, k, _ptr(idx_out), _ptr(scores),
                                     _ptr(ws), nbytes, _stream()))
    return (idx_out, scores) if want_scores else idx_out


def _attn_flags(win_ring: bool, batch_invariant: bool) -> int:
    return (ATTN_WIN_RING if win_ring else 0) | (ATTN_BATCH_INVARIANT if batch_invariant else 0)


def indexer_scores(q_idx, q_scale, w, k_idx, k_scale, fmt: str, q_pos, ratio: int, d_I: int, out=None):
    """The indexer's score stage alone: float32 scores [B, Tq, N] for the visible
    entries (the rest of `out` is left as it was)."""
    _contig(q_idx, q_scale, w, k_idx, k_scale, q_pos, out)
    B, Tq, H_I = q_idx.shape[:3]
    N = k_idx.shape[1]
    if out is None:
        out = torch.zeros(B, Tq, N, dtype=torch.float32, device=q_idx.device)
    check("indexer_scores", lib().indexer_scores(_ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(k_idx), _ptr(k_scale),
                                                 FMT[fmt], _ptr(q_pos), B, Tq, N, H_I, d_I, ratio, _ptr(out),
                                                 _stream()))
    return out


def sparse_attn_workspace_size(B, Tq, H, d, k, window, batch_invariant: bool = False) -> int:
    return int(lib().sparse_attn_workspace_size(B, Tq, H, d, k, window, _attn_flags(False, batch_invariant)))


def sparse_attn_fwd(q, kv, idx, x_win, win_start, sink, q_pos, window: int = 128, scale: float = 1.0,
                    want_lse: bool = False, ws=None, out=None, win_ring: bool = False,
                    batch_invariant: bool = False):
    """CSA core attention. q [B, Tq, H, d], kv [B, N, d], idx int32 [B, Tq, k],
    x_win [B, T_win, d], win_start int32 [B], sink float32 [H] or None, q_pos int32 [B, Tq].
    win_ring: x_win is a ring holding position t at row t mod T_win.
    batch_invariant: plan the kernel from one sequence's rows (each sequence's
    result is then the same bits whatever else is in the batch)."""
    _contig(q, kv, idx, x_win, win_start, sink, q_pos)
    t = _float_dtype(q)
    B, Tq, H, d = q.shape
    N, T_win, k = kv.shape[1], x_win.shape[1], idx.shape[2]
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty(B, Tq, H, dtype=torch.float32, device=q.device) if want_lse else None
    ws, nbytes = _workspace(sparse_attn_workspace_size(B, Tq, H, d, k, window, batch_invariant), q.device, ws)
    check("sparse_attn_fwd", lib().sparse_attn_fwd(_ptr(q), _ptr(kv), _ptr(idx), _ptr(x_win), _ptr(win_start),
                                                   _ptr(sink), _ptr(q_pos), t, B, Tq, N, T_win, H, d, k, window,
                                                   scale, _ptr(out), _ptr(lse), _ptr(ws), nbytes,
                                                   _attn_flags(win_ring, batch_invariant), _stream()))
    return (out, lse) if want_lse else out


def sparse_attn_noalloc_scratch_bytes() -> int:
    return int(lib().sparse_attn_noalloc_scratch_bytes())


def sparse_attn_fwd_noalloc(q, kv, idx, x_win, win_start, sink, q_pos, window: int = 128, scale: float = 1.0,
                            out=None, lse=None, win_ring: bool = False, batch_invariant: bool = False):
    """sparse_attn_fwd without a workspace: the library's per-device scratch holds
    the split results. The caller passes the outputs (out [B, Tq, H, d], lse
    float32 [B, Tq, H] or None) to allocate nothing in the call."""
    _contig(q, kv, idx, x_win, win_start, sink, q_pos, out, lse)
    t = _float_dtype(q)
    B, Tq, H, d = q.shape
    N, T_win, k = kv.shape[1], x_win.shape[1], idx.shape[2]
    if out is None:
        out = torch.empty_like(q)
    check("sparse_attn_fwd_noalloc", lib().sparse_attn_fwd_noalloc(
        _ptr(q), _ptr(kv), _ptr(idx), _ptr(x_win), _ptr(win_start), _ptr(sink), _ptr(q_pos), t, B, Tq, N, T_win, H,
        d, k, window, scale, _ptr(out), _ptr(lse), _attn_flags(win_ring, batch_invariant), _stream()))
    return out


def dense_attn_workspace_size(B, Tq, N, H, d, window, batch_invariant: bool = False) -> int:
    return int(lib().dense_attn_workspace_size(B, Tq, N, H, d, window, _attn_flags(False, batch_invariant)))


def dense_compressed_attn_fwd(q, kv, x_win, win_start, sink, q_pos, ratio: int = 128, window: int = 128,
                              scale: float = 1.0, want_lse: bool = False, ws=None, out=None, win_ring: bool = False,
                              batch_invariant: bool = False):
    """HCA core attention over all visible entries plus window and sink."""
    _contig(q, kv, x_win, win_start, sink, q_pos)
    t = _float_dtype(q)
    B, Tq, H, d = q.shape
    N, T_win = kv.shape[1], x_win.shape[1]
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty(B, Tq, H, dtype=torch.float32, device=q.device) if want_lse else None
    ws, nbytes = _workspace(dense_attn_workspace_size(B, Tq, N, H, d, window, batch_invariant), q.device, ws)
    check("dense_compressed_attn_fwd", lib().dense_compressed_attn_fwd(
        _ptr(q), _ptr(kv), _ptr(x_win), _ptr(win_start), _ptr(sink), _ptr(q_pos), t, B, Tq, N, T_win, H, d, ratio,
        window, scale, _ptr(out), _ptr(lse), _ptr(ws), nbytes, _attn_flags(win_ring, batch_invariant), _stream()))
    return (out, lse) if want_lse else out


def sparse_attn_bwd_workspace_size(B, Tq, N, T_win, H, d, k, window) -> int:
    return int(lib().sparse_attn_bwd_workspace_size(B, Tq, N, T_win, H, d, k, window))


def _bwd_outputs(q, kv, x_win, sink):
    B, N, T_win = q.shape[0], kv.shape[1], x_win.shape[1]
    dev = q.device
    dq = torch.empty_like(q)
    dkv = torch.empty(B, N, q.shape[3], dtype=torch.float32, device=dev)
    dxw = torch.empty(B, T_win, q.shape[3], dtype=torch.float32, device=dev)
    dsink = torch.empty(q.shape[2], dtype=torch.float32, device=dev) if sink is not None else None
    return dq, dkv, dxw, dsink


def sparse_attn_bwd(q, kv, idx, x_win, win_start, sink, q_pos, out, lse, dout, window: int = 128,
                    scale: float = 1.0, ws=None):
    """Gradients of sparse_attn_fwd (bf16 q/kv/x_win/out/dout, H 64 or 128). Returns
    (dq [B, Tq, H, d] bf16, dkv [B, N, d] float32, dx_win [B, T_win, d] float32,
    dsink [H] float32 or None)."""
    _contig(q, kv, idx, x_win, win_start, sink, q_pos, out, lse, dout)
    t = _float_dtype(q)
    B, Tq, H, d = q.shape
    N, T_win, k = kv.shape[1], x_win.shape[1], idx.shape[2]
    dq, dkv, dxw, dsink = _bwd_outputs(q, kv, x_win, sink)
    ws, nbytes = _workspace(sparse_attn_bwd_workspace_size(B, Tq, N, T_win, H, d, k, window), q.device, ws)
    check("sparse_attn_bwd", lib().sparse_attn_bwd(
        _ptr(q), _ptr(kv), _ptr(idx), _ptr(x_win), _ptr(win_start), _ptr(sink), _ptr(q_pos), t, B, Tq, N, T_win, H,
        d, k, window, scale, _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dkv), _ptr(dxw), _ptr(dsink),
        _ptr(ws), nbytes, _stream()))
    return dq, dkv, dxw, dsink


def dense_attn_bwd_workspace_size(B, Tq, N, T_win, H, d, window) -> int:
    return int(lib().dense_attn_bwd_workspace_size(B, Tq, N, T_win, H, d, window))


def dense_compressed_attn_bwd(q, kv, x_win, win_start, sink, q_pos, out, lse, dout, ratio: int = 128,
                              window: int = 128, scale: float = 1.0, ws=None):
    """Gradients of dense_compressed_attn_fwd; same outputs as sparse_attn_bwd."""
    _contig(q, kv, x_win, win_start, sink, q_pos, out, lse, dout)
    t = _float_dtype(q)
    B, Tq, H, d = q.shape
    N, T_win = kv.shape[1], x_win.shape[1]
    dq, dkv, dxw, dsink = _bwd_outputs(q, kv, x_win, sink)
    ws, nbytes = _workspace(dense_attn_bwd_workspace_size(B, Tq, N, T_win, H, d, window), q.device, ws)
    check("dense_compressed_attn_bwd", lib().dense_compressed_attn_bwd(
        _ptr(q), _ptr(kv), _ptr(x_win), _ptr(win_start), _ptr(sink), _ptr(q_pos), t, B, Tq, N, T_win, H, d, ratio,
        window, scale, _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dkv), _ptr(dxw), _ptr(dsink), _ptr(ws),
        nbytes, _stream()))
    return dq, dkv, dxw, dsink


def window_append(x_new, pos, ring):
    """Write each sequence's new window row x_new [B, d] into ring [B, R, d] at row pos mod R."""
    _contig(x_new, pos, ring)
    t = _float_dtype(x_new)
    B, d = x_new.shape
    check("csa_window_append", lib().csa_window_append(_ptr(x_new), t, B, d, _ptr(pos), _ptr(ring), ring.shape[1],
                                                       _stream()))
    return ring


def kernel_timer_start(kernel: str, max_launches: int) -> None:
    check("csa_kernel_timer_start", lib().csa_kernel_timer_start(KID[kernel], max_launches))


def kernel_timer_read(capacity: int = 4096) -> list[float]:
    buf = (ctypes.c_float * capacity)()
    n = lib().csa_kernel_timer_read(buf, capacity)
    if n < 0:
        raise RuntimeError("csa_kernel_timer_read failed")
    return [buf[i] for i in range(min(n, capacity))]


def state_checkpoint(state, pos, period: int, ckpt):
    """Periodic checkpoint of one ring tensor state [B, ...]: sequences whose
    appended position pos[b] ends a period copy state[b] into ckpt[b, slot]
    (ckpt [B, n_slots, ...] of the same dtype)."""
    _contig(state, pos, ckpt)
    B = state.shape[0]
    seq = state[0].numel() * state.element_size() if B else 0
    n_slots = ckpt.shape[1]
    check("csa_state_checkpoint", lib().csa_state_checkpoint(_ptr(state), B, seq, _ptr(pos), period, _ptr(ckpt),
                                                             n_slots, _stream()))


def state_restore(ckpt, slot, state):
    """state[b] = ckpt[b, slot[b]] for slot[b] >= 0."""
    _contig(ckpt, slot, state)
    B = state.shape[0]
    seq = state[0].numel() * state.element_size() if B else 0
    check("csa_state_restore", lib().csa_state_restore(_ptr(ckpt), B, seq, ckpt.shape[1], _ptr(slot), _ptr(state),
                                                       _stream()))


def ring_fill(hist, pos, ring):
    """ring[b, t % R] = hist[b, t] for the R positions before pos[b]
    (hist [B, T_hist, ...] and ring [B, R, ...] with the same row shape)."""
    _contig(hist, pos, ring)
    B, T_hist = hist.shape[:2]
    R = ring.shape[1]
    row = hist[0, 0].numel() * hist.element_size() if B and T_hist else 16
    check("csa_ring_fill", lib().csa_ring_fill(_ptr(hist), B, T_hist, row, _ptr(pos), R, _ptr(ring), _stream()))


def linear_bf16(a, w, out_dtype=torch.bfloat16, out=None):
    """a [M, K] bf16 times w [N, K]^T (a linear layer's weight) -> [M, N]."""
    _contig(a, w, out)
    M, K = a.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=a.device)
    check("csa_linear_bf16", lib().csa_linear_bf16(_ptr(a), K, 0, _ptr(w), K, 0, _ptr(out), _float_dtype(out), N, 0,
                                                   M, N, K, 1, _stream()))
    return out


def grouped_out_proj_workspace_size(T, G, r) -> int:
    return int(lib().csa_grouped_out_proj_workspace_size(T, G, r))


def query_proj_shared_workspace_size(T, r_q) -> int:
    return int(lib().csa_query_proj_shared_workspace_size(T, r_q))


def grouped_out_proj(o, w_group, w_out, out=None, ws=None):
    """Grouped output projection: o [T, H, d] bf16, w_group [G, r, (H/G)*d], w_out [D, G*r] -> [T, D] bf16."""
    _contig(o, w_group, w_out, out)
    T, H, d = o.shape
    G, r = w_group.shape[:2]
    D = w_out.shape[0]
    if out is None:
        out = torch.empty(T, D, dtype=torch.bfloat16, device=o.device)
    ws, nbytes = _workspace(grouped_out_proj_workspace_size(T, G, r), o.device, ws)
    check("csa_grouped_out_proj", lib().csa_grouped_out_proj(_ptr(o), _ptr(w_group), _ptr(w_out), T, H, d, G, r, D,
                                                             _ptr(out), _ptr(ws), nbytes, _stream()))
    return out


def query_proj_shared(x, w_dq, w_uq, w_iq, ws=None):
    """Shared-latent query projections: x [T, D] -> (q [T, n_q], q_idx [T, n_i]), all bf16."""
    _contig(x, w_dq, w_uq, w_iq)
    T, D = x.shape
    r_q, n_q, n_i = w_dq.shape[0], w_uq.shape[0], w_iq.shape[0]
    q = torch.empty(T, n_q, dtype=torch.bfloat16, device=x.device)
    qi = torch.empty(T, n_i, dtype=torch.bfloat16, device=x.device)
    ws, nbytes = _workspace(query_proj_shared_workspace_size(T, r_q), x.device, ws)
    check("csa_query_proj_shared", lib().csa_query_proj_shared(_ptr(x), _ptr(w_dq), _ptr(w_uq), _ptr(w_iq), T, D,
                                                               r_q, n_q, n_i, _ptr(q), _ptr(qi), _ptr(ws), nbytes,
                                                               _stream()))
    return q, qi


def kv_proj(x, w, out_dtype=torch.bfloat16, out=None):
    """Compressor input streams from the hidden state: x [..., D] bf16 (rows of
    any leading shape), w [S, width, D] bf16 -> [S, ..., width] (stream s =
    x w[s]^T; for csa_compress the streams C_a, C_b, Z_a, Z_b)."""
    _contig(x, w, out)
    lead = x.shape[:-1]
    D = x.shape[-1]
    T = math.prod(lead)
    S, width = w.shape[:2]
    if out is None:
        out = torch.empty(S, *lead, width, dtype=out_dtype, device=x.device)
    check("csa_kv_proj", lib().csa_kv_proj(_ptr(x), _ptr(w), T, D, S, width, _ptr(out), _float_dtype(out),
                                           _stream()))
    return out
