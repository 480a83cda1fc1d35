"""The no-allocation entry point bsa_forward_qouter_static, called through
the C ABI, against bsa_forward_qouter with a caller workspace: the same
kernels, so the outputs must be identical bit for bit (stronger than the
attention tolerance).  Two calls in a row, the second on a smaller problem
(the static scratch keeps the first call's counters and must be cleared).
Both problems run several rounds of the persistent grid, so the scratch is
in use; the call must not allocate device memory through torch either."""

import ctypes

import pytest
import torch

from workloads import scaled, vsa_inputs

pytestmark = pytest.mark.gpu

bsa = pytest.importorskip("block_sparse_attention_02_amd")
from block_sparse_attention_02_amd import _lib as L  # noqa: E402

DEV = torch.device("cuda:0")


def _problem(grid, h, R):
    cfg = scaled("video", grid=grid, h=h, R=R)
    x = vsa_inputs(cfg, device=DEV)
    geom = bsa.VsaGeometry(cfg["grid"], cfg["block"], device=DEV)
    idx, num = bsa.pool_route_topk(x["q"], x["k"], geom.perm, geom.block_len, geom.J, geom.M, R)
    return x, geom, idx, num


def _args(x, geom, idx, num, out, lse):
    a = bsa.api._qouter_args(x["q"], x["k"], x["v"], out, 1.0 / x["q"].shape[-1] ** 0.5, L.BSA_SEL_BLOCK, lse)
    P = bsa.api._ptr
    a.perm, a.block_len, a.J, a.M = P(geom.perm), P(geom.block_len), geom.J, geom.M
    a.q2k_idx, a.q2k_num, a.kmax = P(idx), P(num), idx.shape[-1]
    return a


@pytest.mark.parametrize("order", ["large_then_small"])
def test_static_entry_matches_workspace_entry(order):
    lib = L.load()
    stream = bsa.api._stream(DEV)
    ws = bsa.qouter_workspace(DEV)
    cases = [((30, 48, 80), 2, 192), ((16, 32, 40), 2, 32)]   # 3840 and 640 query blocks (> 512 resident)
    for grid, h, R in cases:
        x, geom, idx, num = _problem(grid, h, R)
        B, N, H, D = x["q"].shape
        ref = torch.empty_like(x["q"])
        ref_lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
        got = torch.full_like(x["q"], float("nan"))
        got_lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV)
        a_ref = _args(x, geom, idx, num, ref, ref_lse)
        L.check(lib.bsa_forward_qouter(ctypes.byref(a_ref), bsa.api._ptr(ws), ws.numel(), stream))
        torch.cuda.synchronize()
        a_got = _args(x, geom, idx, num, got, got_lse)
        before = torch.cuda.memory_allocated(DEV)
        for rep in range(2):
            L.check(lib.bsa_forward_qouter_static(ctypes.byref(a_got), stream))
            torch.cuda.synchronize()
            assert torch.cuda.memory_allocated(DEV) == before
            print("static call: grid %s, %d heads, rep %d" % (grid, h, rep), flush=True)
            assert torch.equal(got, ref) and torch.equal(got_lse, ref_lse)
        assert lib.bsa_check(stream) == L.BSA_OK


def test_static_entry_validates_like_the_workspace_entry():
    lib = L.load()
    x, geom, idx, num = _problem((8, 16, 16), 1, 4)
    out = torch.empty_like(x["q"])
    a = _args(x, geom, idx, num, out, None)
    a.M = 48
    assert lib.bsa_forward_qouter_static(ctypes.byref(a), None) == L.BSA_ERR_UNSUPPORTED
    a = _args(x, geom, idx, num, out, None)
    a.v = None
    assert lib.bsa_forward_qouter_static(ctypes.byref(a), None) == L.BSA_ERR_ARG
