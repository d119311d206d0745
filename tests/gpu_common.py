"""Shared helpers for the GPU parity tests (host-side comparison utilities)."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda"

# Tolerances. bf16 outputs: max-abs 2e-2 and relative L2 1e-2 against the
# oracle. float32 outputs: the kernels accumulate in float32 with the hardware
# exp2 (about 2 ulp) on values of order one, so 2e-4 max-abs and 2e-5 relative
# L2 leave a wide margin above float32 rounding while still catching any wrong
# term.
TOL = {"bf16": (2e-2, 1e-2), "f32": (2e-4, 2e-5)}


def dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype)


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype.is_floating_point else t.detach().cpu().numpy()


def assert_close(got, want, kind: str, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, rl2 = TOL[kind]
    err = np.abs(got - want).max() if got.size else 0.0
    den = np.linalg.norm(want)
    rel = np.linalg.norm(got - want) / den if den > 0 else np.linalg.norm(got)
    assert err <= mx and rel <= rl2, f"{what}: max-abs {err:.3e} (tol {mx}), rel-L2 {rel:.3e} (tol {rl2})"


def visible_scores(s, n_vis) -> np.ndarray:
    """Score rows [Tq, N] as float64 with the entries past each row's visible
    count (which the kernels never write) replaced by -inf."""
    s = np.asarray(s)
    vis = np.arange(s.shape[-1])[None, :] < np.asarray(n_vis)[:, None]
    return np.where(vis, s, -np.inf).astype(np.float64)


def recall(got_idx: np.ndarray, want_idx: np.ndarray) -> np.ndarray:
    """Per-row |got & want| / |want| over the non-padding entries."""
    out = []
    for g, w in zip(got_idx.reshape(-1, got_idx.shape[-1]), want_idx.reshape(-1, want_idx.shape[-1])):
        ws = set(int(x) for x in w if x >= 0)
        gs = set(int(x) for x in g if x >= 0)
        out.append(len(ws & gs) / len(ws) if ws else 1.0)
    return np.array(out)


def certified_index_mismatches(got_idx, want_idx, scores64, n_vis, k):
    """Rows where the GPU's selection differs from the oracle's must be certified
    near-ties: the oracle's float64 gap between the k-th and (k+1)-th largest
    score is within float32 summation error (2^-20 relative + 2^-40). Returns
    the number of differing rows; raises if any difference is not certified."""
    bad = 0
    for r in range(got_idx.shape[0]):
        if np.array_equal(got_idx[r], want_idx[r]):
            continue
        n = int(n_vis[r])
        s = np.sort(scores64[r, :n])[::-1]
        assert n > k, f"row {r}: mismatch although every entry is selected"
        gap = s[k - 1] - s[k]
        tol = 2.0 ** -20 * abs(s[k - 1]) + 2.0 ** -40
        # the GPU must still have picked k valid, ascending, distinct entries
        g = got_idx[r]
        assert np.all(np.diff(g) > 0) and g.min() >= 0 and g.max() < n
        # every GPU pick must score within tol of the k-th oracle score
        assert scores64[r, g].min() >= s[k - 1] - tol, f"row {r}: uncertified mismatch (gap {gap:.3e})"
        bad += 1
    return bad
