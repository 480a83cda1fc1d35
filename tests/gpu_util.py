"""Helpers shared by the GPU parity tests."""

import numpy as np
import torch

# Attention tolerance from bf16 inputs with fp32 accumulation.
ATOL_MAX = 2e-2
ATOL_MEAN = 2e-3
# TopK rows whose R-th and (R+1)-th float64 scores differ by less than this are exempt.
GAP_EXEMPT = 1e-4


def to64(t):
    """Exact float64 host copy of a device tensor (bf16 / fp32).  Output
    buffers may hold slots the kernel never writes (the tests mask them); their
    bit patterns can be signalling NaNs, whose cast is not worth a warning."""
    with np.errstate(invalid="ignore"):
        return t.detach().float().cpu().numpy().astype(np.float64)


def attn_error(got, ref, mask=None):
    """(max abs, mean abs) over the valid elements of two float arrays."""
    g = to64(got) if isinstance(got, torch.Tensor) else got
    err = np.abs(g - ref)
    if mask is not None:
        err = err[mask]
    return float(err.max()), float(err.mean())


def assert_attn_close(got, ref, what, mask=None):
    mx, mean = attn_error(got, ref, mask)
    print("%s: max abs err %.3g, mean abs err %.3g" % (what, mx, mean), flush=True)
    assert mx <= ATOL_MAX and mean <= ATOL_MEAN, "%s: max %.3g mean %.3g" % (what, mx, mean)


def check_topk(got_idx, E, R, ref_idx, gap, cols=None, what="topk"):
    """Complete check of a TopK selection against float64 scores.

    got_idx: kept ids of every row (first R entries used; ascending), E: the
    float64 scores [..., J] of the same rows, ref_idx: the oracle's kept ids
    (ties to the lower index), gap: E_(R) - E_(R+1) per row.  ``cols``
    (b0, b1) restricts the selection to that column range (one H3 region).

    * every row: R distinct ascending ids inside the column range;
    * rows with gap >= GAP_EXEMPT: exactly the oracle's ids;
    * exempt rows (several answers are correct): a valid top-R within the
      gap -- every kept score >= E_(R) - GAP_EXEMPT and every dropped score
      <= E_(R+1) + GAP_EXEMPT.
    Asserts all three and returns the number of exempt rows."""
    got = got_idx.cpu().numpy() if isinstance(got_idx, torch.Tensor) else np.asarray(got_idx)
    J = E.shape[-1]
    b0, b1 = (0, J) if cols is None else cols
    g = got[..., :R].reshape(-1, R).astype(np.int64)
    r = np.asarray(ref_idx)[..., :R].reshape(-1, R)
    e = np.asarray(E, dtype=np.float64).reshape(-1, J)
    gp = np.asarray(gap, dtype=np.float64).reshape(-1)
    assert ((g >= b0) & (g < b1)).all(), what + ": id outside the column range"
    assert (np.diff(g, axis=-1) > 0).all() if R > 1 else True, what + ": ids not strictly increasing"
    exempt = gp < GAP_EXEMPT
    bad = int(((g != r).any(-1) & ~exempt).sum())
    sub = e[:, b0:b1]
    srt = -np.sort(-sub, axis=-1)
    e_r = srt[:, R - 1]
    e_r1 = srt[:, R] if R < b1 - b0 else np.full(len(sub), -np.inf)
    kept = np.take_along_axis(e, g, axis=-1)
    dropped = sub.copy()
    np.put_along_axis(dropped, g - b0, -np.inf, axis=-1)
    ok = (kept >= e_r[:, None] - GAP_EXEMPT).all(-1) & (dropped.max(-1) <= e_r1 + GAP_EXEMPT)
    invalid = int((~ok & exempt).sum())
    print("%s: %d rows, %d exempt near-ties (%d not a valid top-%d), %d mismatches"
          % (what, len(g), int(exempt.sum()), invalid, R, bad), flush=True)
    assert bad == 0, "%s: %d rows differ from the oracle" % (what, bad)
    assert invalid == 0, "%s: %d exempt rows are not a valid top-%d" % (what, invalid, R)
    assert ok[~exempt].all(), what + ": a non-exempt row fails the validity check"
    return int(exempt.sum())


def _spread3_10(v):
    """Bits 0..9 of v moved to bits 0, 3, 6, ..., 27 (a Morton interleave)."""
    out = np.zeros_like(v, dtype=np.uint64)
    for t in range(10):
        out |= ((v >> t) & 1).astype(np.uint64) << np.uint64(3 * t)
    return out


def expected_item_order(idx, num, num_first=0):
    """The processing order the routing calls document, from an index table
    (host arrays [B, H, J, kmax] and [B, H, J]): per (b, h), blocks sorted by
    the Morton code of the entries at positions (n-1)//4, (n-1)//2 and
    3(n-1)//4 of their kept list (each clamped to [0, J) and scaled to 10 bits
    as v * 1024 // J; code bit 3t + c is bit t of entry c), ties by block
    index, with blocks below num_first first in index order."""
    B, H, J, kmax = idx.shape
    n = np.minimum(num, kmax).astype(np.int64)
    code = np.zeros((B, H, J), dtype=np.uint64)
    pos = [np.maximum(n - 1, 0) // 4, np.maximum(n - 1, 0) // 2, 3 * np.maximum(n - 1, 0) // 4]
    for c in range(3):
        v = np.take_along_axis(idx, pos[c][..., None], axis=-1)[..., 0].astype(np.int64)
        v = np.clip(v, 0, J - 1) * 1024 // J
        code |= _spread3_10(v.astype(np.uint64)) << np.uint64(c)
    code[n == 0] = 0
    code[:, :, :num_first] = 0
    keys = (code << np.uint64(32)) | np.arange(J, dtype=np.uint64)
    return np.argsort(keys, axis=-1, kind="stable").astype(np.int32)
