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


def topk_mismatch(got_idx, ref_idx, gap):
    """(non-exempt mismatching rows, exempt rows)."""
    got = got_idx.cpu().numpy() if isinstance(got_idx, torch.Tensor) else got_idx
    diff = (got != ref_idx).any(-1)
    exempt = gap < GAP_EXEMPT
    return int((diff & ~exempt).sum()), int(exempt.sum())
