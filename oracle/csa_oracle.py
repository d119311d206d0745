"""CPU oracle for the CSA/HCA hybrid attention forward (DeepSeek-V4, as the
public write-ups describe it).

TEST INFRASTRUCTURE ONLY. This module is imported by the tests, by the smoke
check and by the benchmark's CPU-baseline leg, and by nothing else. It shares
no code with the HIP library and never calls it.

Everything is plain NumPy in float64 (inputs are upcast), written to be read
against the pages, with no blocking, fusion or reordering beyond what each
definition states. Where a step decides an integer from floating point in the
kernel's precision (quantisation codes), this module takes that decision in
float32 as well, and says so.

Sources, cited by page address and section:
  [cf-1 §x]   DeepSeek-V4 write-up at www.cf-1.com/news/5231315
              (§3.1 how CSA works, §3.2 how HCA works, §3.3 layer layout,
              window branch and sink, §3.4 low-rank/low-precision indexer,
              §4.3 deterministic kernels, §4.4 FP4 QAT and KV-cache tiers)
  [yfxerp §x] "DeepSeek-V4 原理拆解" at www.yfxerp.com/news/211352
              (§1 module overview, §3 config skeleton with kv_compress_ratio 4,
              top_k_blocks 1024, indexer_rank 64, sliding_window 128,
              compress_ratio 128, attention_sink)

The pages print no equations. Each function states the reading it takes where
the pages leave a step open; all readings are listed in the design notes.

Parity status: every function here is pinned by the CPU tests (closed forms,
reductions to library routines, exhaustive code tables, brute force on tiny
inputs). What no pin can reach is agreement with the real model's layer (no
weights or worked example exist on the pages): the ReLU in the indexer score,
the choice of window rows and the quantisation formats are readings, and for
those the agreement with DeepSeek-V4 itself is parity unpinned.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

# ---------------------------------------------------------------------------
# Compression
# ---------------------------------------------------------------------------


def _softmax_weighted_sum(logits: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Per-channel softmax over axis 0 of ``logits``, then the weighted sum of ``values``.

    logits, values: [m, width]. Max-subtracted, in float64.
    """
    z = logits.astype(np.float64)
    v = values.astype(np.float64)
    zmax = z.max(axis=0, keepdims=True)
    e = np.exp(z - zmax)
    w = e / e.sum(axis=0, keepdims=True)
    return (w * v).sum(axis=0)


def csa_compress(c_a, c_b, z_a, z_b, ratio: int = 4) -> np.ndarray:
    """CSA compressor: overlapped, gated, two-stream, ``ratio``:1.

    [cf-1 §3.1]: every 4 tokens become one entry; two independent KV
    sequences are merged with softmax-normalised gate weights, and adjacent
    blocks share part of their tokens (overlap). [yfxerp §3]: ratio 4.

    Reading: entry j merges stream A over tokens [m*j, m*j+m) and stream B
    over the previous block [m*j-m, m*j), with ONE softmax per channel over the
    joint list of 2m gate logits. For j = 0 the B tokens do not exist and are
    left out (softmax over the m A logits only). Entry count N = floor(T/m); a
    trailing partial block is not compressed.

    c_a, c_b, z_a, z_b: [T, width]. Returns float64 [N, width].
    """
    c_a, c_b, z_a, z_b = (np.asarray(x, dtype=np.float64) for x in (c_a, c_b, z_a, z_b))
    T, width = c_a.shape
    m = int(ratio)
    N = T // m
    out = np.zeros((N, width), dtype=np.float64)
    for j in range(N):
        a = slice(m * j, m * j + m)
        if j == 0:
            logits, values = z_a[a], c_a[a]
        else:
            b = slice(m * j - m, m * j)
            logits = np.concatenate([z_a[a], z_b[b]], axis=0)
            values = np.concatenate([c_a[a], c_b[b]], axis=0)
        out[j] = _softmax_weighted_sum(logits, values)
    return out


def hca_compress(c, z, ratio: int = 128) -> np.ndarray:
    """HCA compressor: non-overlapped, single stream, ``ratio``:1.

    [cf-1 §3.2]: every 128 tokens become one entry. Reading: the same gated
    merge as CSA, per channel softmax over the block's ``ratio`` gate logits,
    one stream, no overlap. Ratio 1 is the identity (softmax of one logit).

    c, z: [T, width]. Returns float64 [T // ratio, width].
    """
    c = np.asarray(c, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    m = int(ratio)
    N = c.shape[0] // m
    out = np.zeros((N, c.shape[1]), dtype=np.float64)
    for j in range(N):
        blk = slice(m * j, m * j + m)
        out[j] = _softmax_weighted_sum(z[blk], c[blk])
    return out


# ---------------------------------------------------------------------------
# Low-precision number formats for the indexer ([cf-1 §3.4, §4.4]: the
# indexer's QK runs in FP4; FP4 -> FP8 dequantisation is lossless).
# Reading: OCP e4m3 with one float32 scale per row (amax/448), and OCP MX
# e2m1 with one E8M0 scale per 32 consecutive elements. These decide integer
# codes, so they are computed in float32, the kernel's precision.
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127  # largest finite bfloat16


def e4m3_decode(codes) -> np.ndarray:
    """OCP e4m3 code -> value (float64). 0x7F/0xFF are NaN."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def _round_half_even(x: np.ndarray) -> np.ndarray:
    return np.rint(x)  # numpy rounds half to even


def e4m3_encode(v) -> np.ndarray:
    """float32 value -> OCP e4m3 code, round to nearest even, saturating at 448.

    The sign bit is the sign of the input (so small negatives give 0x80).
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN input to e4m3_encode")
    sign = np.signbit(v).astype(np.int64) << 7
    a = np.abs(v)
    a = np.minimum(a, E4M3_MAX)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2^-9 (code 8 is the smallest normal, 2^-6)
    code = np.where(sub, _round_half_even(a / 2.0 ** -9).astype(np.int64), code)
    safe = np.where(sub, 1.0, a)
    e = np.floor(np.log2(safe)).astype(np.int64)
    # guard log2 rounding at exact powers of two
    e = np.where(np.exp2(e.astype(np.float64)) > safe, e - 1, e)
    e = np.where(np.exp2((e + 1).astype(np.float64)) <= safe, e + 1, e)
    mant = _round_half_even((safe / np.exp2(e.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    carry = mant == 8
    e = np.where(carry, e + 1, e)
    mant = np.where(carry, 0, mant)
    ncode = ((e + 7) << 3) | mant
    ncode = np.minimum(ncode, 0x7E)  # saturate (0x7F is NaN)
    code = np.where(sub, code, ncode)
    return (code | sign).astype(np.uint8)


def quant_fp8_rows(x):
    """Quantise rows (last axis) to e4m3 with one float32 scale per row.

    scale = fp32(amax / 448) (1.0 for an all-zero row); code = e4m3(fp32(x / scale)).
    Both divisions are IEEE float32, matching the kernel.
    Returns (codes uint8 [..., width], scale float32 [...]).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = (amax / F32(E4M3_MAX)).astype(np.float32)
    scale = np.where(scale == 0, F32(1.0), scale).astype(np.float32)
    v = (x / scale[..., None]).astype(np.float32)
    return e4m3_encode(v), scale


def dequant_fp8_rows(codes, scale) -> np.ndarray:
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c & 0x8, -1.0, 1.0) * E2M1_VALUES[c & 0x7]


def e2m1_encode(v) -> np.ndarray:
    """float32 value -> e2m1 code (4 bits), round to nearest even, saturating at 6.

    Written as exact comparisons against the midpoints of the grid
    {0, .5, 1, 1.5, 2, 3, 4, 6}; a tie goes to the code with an even last bit.
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    sign = np.signbit(v).astype(np.int64) << 3
    a = np.abs(v)
    mag = np.select(
        [a <= 0.25, a < 0.75, a <= 1.25, a < 1.75, a <= 2.5, a < 3.5, a <= 5.0],
        [0, 1, 2, 3, 4, 5, 6], default=7)
    return (mag | sign).astype(np.uint8)


def _pow2_f32(e: np.ndarray) -> np.ndarray:
    """2**e as float32, exact for e in [-149, 127]."""
    return np.ldexp(np.float32(1.0), np.asarray(e, dtype=np.int32)).astype(np.float32)


def quant_mxfp4_rows(x):
    """Quantise the last axis to e2m1 with one E8M0 scale per 32 elements (OCP MX).

    For each block: amax in float32; shared exponent E = floor(log2(amax)) - 2
    (2 is the largest exponent of e2m1), clamped to [-127, 127]; E = 0 for an
    all-zero block. Elements are fp32(x * 2**-E) encoded as e2m1.
    Returns (packed uint8 [..., width/2] with element 2i in the low nibble of
    byte i, scales uint8 [..., width/32] holding E + 127).
    """
    x = np.asarray(x, dtype=np.float32)
    width = x.shape[-1]
    assert width % 32 == 0
    blocks = x.reshape(x.shape[:-1] + (width // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(amax.astype(np.float64))  # amax = f * 2**ex, f in [0.5, 1)
    E = np.where(amax > 0, ex - 1 - 2, 0).astype(np.int64)
    E = np.clip(E, -127, 127)
    v = (blocks * _pow2_f32(-E)[..., None]).astype(np.float32)
    codes = e2m1_encode(v).reshape(x.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (E + 127).astype(np.uint8)


def dequant_mxfp4_rows(packed, scales) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    lo = e2m1_decode(packed & 0xF)
    hi = e2m1_decode(packed >> 4)
    vals = np.stack([lo, hi], axis=-1).reshape(packed.shape[:-1] + (packed.shape[-1] * 2,))
    sc = np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)
    width = vals.shape[-1]
    vals = vals.reshape(vals.shape[:-1] + (width // 32, 32)) * sc[..., None]
    return vals.reshape(vals.shape[:-2] + (width,))


# ---------------------------------------------------------------------------
# Lightning indexer and top-k ([cf-1 §3.1, §3.4]; [yfxerp §1, §3])
# ---------------------------------------------------------------------------


def visible_entries(p, ratio: int, N: int):
    """n(p) = min(N, floor((p+1)/ratio)): an entry is visible once its block is complete.

    Reading of causality (the pages are silent): entry j covers tokens up to
    ratio*j + ratio - 1, so the query at position p sees j iff that token <= p.
    """
    return np.minimum(N, (np.asarray(p, dtype=np.int64) + 1) // int(ratio))


def indexer_scores(q_i, w, k_i, q_pos, ratio: int) -> np.ndarray:
    """Index scores I(p, s) = sum_h w(p,h) * ReLU(q_i(p,h) . k_i(s)) for s < n(p).

    [cf-1 §3.1]: each query picks its top-k compressed entries through the
    lightning indexer; [cf-1 §3.4]: the indexer is low-rank and low-precision.
    Reading: the multi-head weighted ReLU form (without a per-head
    nonlinearity the weighted head sum would collapse to a single head), no
    scale and no positional term. Invisible entries get -inf.

    q_i: [Tq, H_I, d_I], w: [Tq, H_I], k_i: [N, d_I], q_pos: [Tq].
    Returns float64 [Tq, N].
    """
    q_i = np.asarray(q_i, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k_i = np.asarray(k_i, dtype=np.float64)
    Tq = q_i.shape[0]
    N = k_i.shape[0]
    n_vis = visible_entries(q_pos, ratio, N)
    out = np.full((Tq, N), -np.inf)
    for t in range(Tq):
        n = int(n_vis[t])
        if n == 0:
            continue
        logits = q_i[t] @ k_i[:n].T            # [H_I, n]
        out[t, :n] = w[t] @ np.maximum(logits, 0.0)
    return out


def topk_select(scores, n_vis, k: int) -> np.ndarray:
    """The min(k, n) entries with the largest scores, per row.

    [cf-1 §2.4, §3.1]: per-query top-k (512 or 1024) over compressed entries.
    Total order: score descending, then index ascending (ties go to the lower
    index); -0.0 equals +0.0. Output ascending by index, padded with -1.
    scores: [Tq, N] (entries >= n_vis[t] are ignored). Returns int32 [Tq, k].
    """
    scores = np.asarray(scores, dtype=np.float64)
    Tq = scores.shape[0]
    out = np.full((Tq, k), -1, dtype=np.int32)
    for t in range(Tq):
        n = int(n_vis[t])
        s = scores[t, :n]
        if np.isnan(s).any():
            raise ValueError("NaN score")
        if n <= k:
            out[t, :n] = np.arange(n)
            continue
        order = np.lexsort((np.arange(n), -s))   # primary: -score, secondary: index
        out[t] = np.sort(order[:k])
    return out


def bf16_round(x) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even; returns float64.

    bfloat16 keeps float32's 8-bit exponent and 8 significant bits (7 stored),
    so a normal value with exponent e sits on a grid of step 2**(e-7); below
    2**-126 the grid step is fixed at 2**-133 (subnormals). NaN and infinities
    pass through unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    fin = np.isfinite(x)
    a = np.where(fin, np.abs(x), 0.0)
    safe = np.where(a > 0, a, 1.0)
    e = np.floor(np.log2(safe)).astype(np.int64)
    # guard log2 rounding at exact powers of two
    e = np.where(np.exp2(e.astype(np.float64)) > safe, e - 1, e)
    e = np.where(np.exp2((e + 1).astype(np.float64)) <= safe, e + 1, e)
    e = np.maximum(e, -126)
    step = np.exp2((e - 7).astype(np.float64))
    r = _round_half_even(a / step) * step
    if (r > BF16_MAX).any():
        raise ValueError("bf16_round overflow")
    return np.where(fin & (a > 0), np.copysign(r, x), x)


def topk_select_bf16(scores, n_vis, k: int) -> np.ndarray:
    """Top-k selection on bfloat16 index scores.

    [cf-1 §4.4]: the index scores are quantised from FP32 to BF16 before the
    selector, which halves its score traffic at a small recall cost. Reading:
    each score is rounded once (nearest, ties to even) and the selection of
    ``topk_select`` runs on the rounded values, so scores that round to the
    same value tie and the lower index wins.
    """
    return topk_select(bf16_round(scores), n_vis, k)


# ---------------------------------------------------------------------------
# Core attention ([cf-1 §3.1, §3.2, §3.3]; [yfxerp §3])
# ---------------------------------------------------------------------------


def window_rows(p: int, window: int, win_start: int, T_win: int):
    """Absolute token positions of the window keys of the query at p.

    [cf-1 §3.3]: the KV of the latest 128 uncompressed tokens enters the core
    computation. Reading: tokens max(0, p-W+1) .. p (the current token
    included), restricted to the rows the caller supplied
    [win_start, win_start + T_win).
    """
    lo = max(0, p - window + 1, win_start)
    hi = min(p, win_start + T_win - 1)
    return np.arange(lo, hi + 1) if hi >= lo else np.zeros(0, dtype=np.int64)


def attend(q, keys, sink, scale: float = 1.0):
    """Softmax attention of one query over ``keys`` (keys are also the values) plus a sink.

    [cf-1 §3.3]: the attention sink is a learnable term added to the softmax
    denominator. o_h = sum_i e^{l_i} v_i / (e^{sink_h} + sum_i e^{l_i}), with
    l_i = scale * q_h . key_i; the sink adds no value and is not scaled.
    Shared KV with one KV head for all query heads (MQA).

    A head whose key set is empty and whose sink is -inf (no sink) has no
    term at all: o = 0 and lse = -inf. This is the limit of the formula as the
    sink logit goes to -inf with no keys (o is 0 for every finite sink), and
    the value the library's contract states for that case.

    q: [H, d], keys: [n, d], sink: [H]. Returns (o [H, d], lse [H]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    sink = np.asarray(sink, dtype=np.float64)
    logits = scale * (q @ keys.T)                                  # [H, n]
    M = np.maximum(sink, logits.max(axis=1) if keys.shape[0] else -np.inf)
    empty = M == -np.inf                                           # no key and no sink
    Ms = np.where(empty, 0.0, M)
    e = np.exp(logits - Ms[:, None])
    den = np.exp(sink - Ms) + e.sum(axis=1)
    o = np.where(empty[:, None], 0.0, (e @ keys) / np.where(empty, 1.0, den)[:, None])
    lse = np.where(empty, -np.inf, Ms + np.log(np.where(empty, 1.0, den)))
    return o, lse


def sparse_attn(q, kv, idx, x_win, win_start: int, sink, q_pos, window: int = 128,
                scale: float = 1.0):
    """CSA core attention: selected compressed entries + window tokens + sink.

    [cf-1 §3.1]: attention runs over the top-k compressed entries chosen by the
    indexer; [cf-1 §3.3]: plus the 128-token window branch and the sink.
    Reading: the key set is {kv[s] : s in idx, 0 <= s < N} joined with the
    window rows; entries whose tokens also lie in the window are kept (no
    de-duplication).

    q: [Tq, H, d], kv: [N, d], idx: [Tq, k] int, x_win: [T_win, d].
    Returns (o [Tq, H, d], lse [Tq, H]).
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    x_win = np.asarray(x_win, dtype=np.float64)
    Tq, H, d = q.shape
    N = kv.shape[0]
    o = np.zeros((Tq, H, d))
    lse = np.zeros((Tq, H))
    for t in range(Tq):
        p = int(q_pos[t])
        sel = np.asarray(idx[t], dtype=np.int64)
        sel = sel[(sel >= 0) & (sel < N)]
        rows = window_rows(p, window, win_start, x_win.shape[0]) - win_start
        keys = np.concatenate([kv[sel], x_win[rows]], axis=0)
        o[t], lse[t] = attend(q[t], keys, sink, scale)
    return o, lse


def dense_attn(q, kv, x_win, win_start: int, sink, q_pos, ratio: int, window: int = 128,
               scale: float = 1.0):
    """HCA core attention: every visible compressed entry + window tokens + sink.

    [cf-1 §3.2]: no sparse selection, dense attention over all entries;
    [cf-1 §3.3]: the same window branch and sink as CSA. This is
    ``sparse_attn`` with the selection set to all n(p) visible entries.
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)
    N = np.asarray(kv).shape[0]
    n_vis = visible_entries(q_pos, ratio, N)
    kmax = int(n_vis.max()) if len(n_vis) else 0
    idx = np.full((len(q_pos), max(kmax, 1)), -1, dtype=np.int64)
    for t, n in enumerate(n_vis):
        idx[t, :n] = np.arange(n)
    return sparse_attn(q, kv, idx, x_win, win_start, sink, q_pos, window, scale)


# ---------------------------------------------------------------------------
# Backward of the core attention ([cf-1 §4.3]: training runs a deterministic
# attention backward; the pages give no formulas, so these are the gradients
# of the forward definitions above)
# ---------------------------------------------------------------------------


def attend_bwd(q, keys, sink, dout, scale: float = 1.0):
    """Gradients of ``attend`` for one query: o_h = sum_i P_hi key_i with
    P_hi = e^{l_hi} / (e^{sink_h} + sum_j e^{l_hj}), l_hi = scale q_h . key_i.

    Keys are also the values, so each key row collects both roles:
      dP_hi  = dout_h . key_i              (value role)
      D_h    = dout_h . o_h = sum_i P_hi dP_hi
      dl_hi  = P_hi (dP_hi - D_h)          (softmax Jacobian; the sink is one
                                            more softmax term with no value)
      dq_h   = scale sum_i dl_hi key_i
      dkey_i = sum_h (scale dl_hi q_h + P_hi dout_h)
      dsink_h = -P_sink,h D_h,  P_sink,h = e^{sink_h} / (e^{sink_h} + sum_j e^{l_hj})

    q, dout: [H, d]; keys: [n, d]; sink: [H]. Returns (dq [H, d], dkeys [n, d],
    dsink [H]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    sink = np.asarray(sink, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    o, lse = attend(q, keys, sink, scale)
    P = np.exp(scale * (q @ keys.T) - lse[:, None])                 # [H, n]
    p_sink = np.exp(sink - lse)                                    # [H]
    dP = dout @ keys.T                                             # [H, n]
    D = np.sum(dout * o, axis=1)                                   # [H]
    dl = P * (dP - D[:, None])
    dq = scale * (dl @ keys)
    dkeys = scale * (dl.T @ q) + P.T @ dout
    dsink = -p_sink * D
    return dq, dkeys, dsink


def sparse_attn_bwd(q, kv, idx, x_win, win_start: int, sink, q_pos, dout, window: int = 128,
                    scale: float = 1.0):
    """Gradients of ``sparse_attn`` (same key sets, same readings).

    Each selected entry and each window row collects the gradient of every
    query that attends to it; the sink's gradient is summed over queries.
    Returns (dq [Tq, H, d], dkv [N, d], dx_win [T_win, d], dsink [H]).
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    x_win = np.asarray(x_win, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    Tq, H, d = q.shape
    N = kv.shape[0]
    dq = np.zeros_like(q)
    dkv = np.zeros_like(kv)
    dx_win = np.zeros_like(x_win)
    dsink = np.zeros(H)
    for t in range(Tq):
        p = int(q_pos[t])
        sel = np.asarray(idx[t], dtype=np.int64)
        sel = sel[(sel >= 0) & (sel < N)]
        rows = window_rows(p, window, win_start, x_win.shape[0]) - win_start
        keys = np.concatenate([kv[sel], x_win[rows]], axis=0)
        dq[t], dk, ds = attend_bwd(q[t], keys, sink, dout[t], scale)
        np.add.at(dkv, sel, dk[:len(sel)])
        np.add.at(dx_win, rows, dk[len(sel):])
        dsink += ds
    return dq, dkv, dx_win, dsink


def dense_attn_bwd(q, kv, x_win, win_start: int, sink, q_pos, ratio: int, dout, window: int = 128,
                   scale: float = 1.0):
    """Gradients of ``dense_attn``: ``sparse_attn_bwd`` with every visible entry selected."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    N = np.asarray(kv).shape[0]
    n_vis = visible_entries(q_pos, ratio, N)
    kmax = int(n_vis.max()) if len(n_vis) else 0
    idx = np.full((len(q_pos), max(kmax, 1)), -1, dtype=np.int64)
    for t, n in enumerate(n_vis):
        idx[t, :n] = np.arange(n)
    return sparse_attn_bwd(q, kv, idx, x_win, win_start, sink, q_pos, dout, window, scale)


# ---------------------------------------------------------------------------
# Whole layers (one sequence)
# ---------------------------------------------------------------------------


def csa_layer(inp: dict, k: int, ratio: int = 4, window: int = 128):
    """One CSA layer forward on one sequence of prefill tokens 0..T-1.

    compress KV streams -> compress indexer streams -> indexer scores ->
    top-k -> sparse attention with window and sink, all in float64 (the
    indexer operands are not quantised here; the quantised formats have their
    own functions above). [cf-1 §3.1, §3.3, §3.4]. The window rows are stream
    A's raw vectors (reading: the pages do not say which raw vector the window
    uses).
    Returns dict with kv, k_i, scores, idx, o, lse.
    """
    T = inp["c_a"].shape[0]
    kv = csa_compress(inp["c_a"], inp["c_b"], inp["z_a"], inp["z_b"], ratio)
    k_i = csa_compress(inp["ci_a"], inp["ci_b"], inp["zi_a"], inp["zi_b"], ratio)
    q_pos = np.arange(T)
    scores = indexer_scores(inp["q_i"], inp["w"], k_i, q_pos, ratio)
    idx = topk_select(scores, visible_entries(q_pos, ratio, kv.shape[0]), k)
    o, lse = sparse_attn(inp["q"], kv, idx, inp["c_a"], 0, inp["sink"], q_pos, window)
    return {"kv": kv, "k_i": k_i, "scores": scores, "idx": idx, "o": o, "lse": lse}


def hca_layer(inp: dict, ratio: int = 128, window: int = 128):
    """One HCA layer forward on one sequence of prefill tokens 0..T-1 [cf-1 §3.2, §3.3].

    compress (ratio:1, one stream) -> dense attention over every visible
    entry, the window rows (the raw stream C, the same reading as CSA's
    window) and the sink. Returns dict with kv, o, lse.
    """
    T = inp["c"].shape[0]
    kv = hca_compress(inp["c"], inp["z"], ratio)
    q_pos = np.arange(T)
    o, lse = dense_attn(inp["q"], kv, inp["c"], 0, inp["sink"], q_pos, ratio, window)
    return {"kv": kv, "o": o, "lse": lse}


# ---------------------------------------------------------------------------
# Projections around the attention core ([cf-1 §3.4]: the lightning indexer
# shares projection parameters with the main attention; the grouped output
# projection reduces each group of heads before the final projection). The
# pages give no group count, rank or width: all are arguments here.
# ---------------------------------------------------------------------------


def grouped_output_projection(o, w_group, w_out):
    """Grouped output projection (cf-1.com write-up §3.4: heads are grouped
    and each group's output reduced before the output projection).

    The H heads of o [T, H, d] form G groups of H/G consecutive heads; group
    g's heads, concatenated in head order, are reduced to rank r by w_group[g]
    ([r, (H/G)*d], a linear layer's [out, in] weight); the G group results are
    concatenated in group order and projected by w_out [D, G*r].
    Returns float64 [T, D].
    """
    o = np.asarray(o, dtype=np.float64)
    w_group = np.asarray(w_group, dtype=np.float64)
    w_out = np.asarray(w_out, dtype=np.float64)
    T, H, d = o.shape
    G, r, _ = w_group.shape
    og = o.reshape(T, G, (H // G) * d)
    y = np.einsum("tgk,grk->tgr", og, w_group)
    return y.reshape(T, G * r) @ w_out.T


def shared_query_projection(x, w_dq, w_uq, w_iq):
    """Query projections sharing one low-rank latent (cf-1.com write-up §3.4:
    the indexer's query projection is shared with the main attention's):
    latent = x w_dq^T, then the attention queries latent w_uq^T and the
    indexer queries latent w_iq^T. Returns float64 (q, q_idx)."""
    x = np.asarray(x, dtype=np.float64)
    latent = x @ np.asarray(w_dq, dtype=np.float64).T
    return latent @ np.asarray(w_uq, dtype=np.float64).T, latent @ np.asarray(w_iq, dtype=np.float64).T


def kv_projection(x, w):
    """The compressor's input streams from the hidden state (cf-1.com write-up
    §3.1: the compressed entries are built from per-token KV vectors and gate
    logits; §3.4: the indexer's keys are built the same way): stream s is
    x w[s]^T for x [T, D] and w [S, width, D] (one linear layer's weight per
    stream). Returns float64 [S, T, width]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return np.stack([x @ w[s].T for s in range(w.shape[0])])
