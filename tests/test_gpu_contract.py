"""GPU checks of the boundary's contract (include/bsa.h, "Conventions"):

* two block-mode calls with their own workspaces run concurrently on two
  streams and give the same bits as the same calls run one after the other
  (the persistent grid's work counters live in the caller's workspace);
* a kept id that names no block (>= J in block mode, past the sequence in
  token mode and in the KV-outer schedule) is skipped exactly like a -1
  entry, and bsa_check reports it once as BSA_ERR_INDEX.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import to64
from workloads import msa_inputs, nsa_inputs, scaled, vsa_inputs

pytestmark = pytest.mark.gpu

bsa = pytest.importorskip("block_sparse_attention_02_amd")
from block_sparse_attention_02_amd import _lib as L  # noqa: E402

DEV = torch.device("cuda:0")


def _check_status():
    return L.load().bsa_check(bsa.api._stream(DEV))


def _video_case(grid, h, R, block=(4, 4, 4), D=128):
    cfg = scaled("video", grid=grid, h=h, R=R, block=block, D=D)
    x = vsa_inputs(cfg, device=DEV)
    geom = bsa.VsaGeometry(cfg["grid"], cfg["block"], device=DEV)
    idx, num = bsa.pool_route_topk(x["q"], x["k"], geom.perm, geom.block_len, geom.J, geom.M, R)
    return cfg, x, geom, idx, num


def test_concurrent_streams_match_serial_runs():
    """Full video grid, two heads: 3840 query blocks, several rounds of the
    persistent grid (its scheduler is in use).  Two calls on two streams at
    once, each with its own workspace, equal two serial calls bit for bit."""
    cfg, x, geom, idx, num = _video_case((30, 48, 80), 2, 192)
    x2 = {k_: (v_ * 0.5).contiguous() for k_, v_ in x.items()}   # a second, different problem
    idx2, num2 = bsa.pool_route_topk(x2["q"], x2["k"], geom.perm, geom.block_len, geom.J, geom.M, 192)
    ws_a, ws_b = bsa.qouter_workspace(DEV), bsa.qouter_workspace(DEV)
    args = lambda xx, ii, nn: (xx["q"], xx["k"], xx["v"], geom.perm, geom.block_len, geom.J, geom.M, ii, nn)
    ref_a = bsa.attention_vsa(*args(x, idx, num), workspace=ws_a)
    ref_b = bsa.attention_vsa(*args(x2, idx2, num2), workspace=ws_a)
    torch.cuda.synchronize()
    out_a, out_b = torch.empty_like(ref_a), torch.empty_like(ref_b)
    s1, s2 = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    for rep in range(3):
        out_a.zero_()
        out_b.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            bsa.attention_vsa(*args(x, idx, num), out=out_a, workspace=ws_a)
        with torch.cuda.stream(s2):
            bsa.attention_vsa(*args(x2, idx2, num2), out=out_b, workspace=ws_b)
        torch.cuda.synchronize()
        print("concurrent rep %d" % rep, flush=True)
        assert torch.equal(out_a, ref_a) and torch.equal(out_b, ref_b)
    assert _check_status() == L.BSA_OK


@pytest.mark.parametrize("case", ["m64", "m32", "f32", "m128"])
def test_block_id_past_J_is_skipped_and_reported(case):
    if case == "m64":
        cfg, x, geom, idx, num = _video_case((8, 16, 20), 2, 6)
    elif case == "m128":  # capacity 128 runs as halves: an id past J stays past the halves' count
        cfg, x, geom, idx, num = _video_case((10, 20, 18), 2, 5, block=(4, 8, 4))
    elif case == "m32":
        cfg, x, geom, idx, num = _video_case((8, 12, 16), 2, 10, block=(2, 4, 4))
    else:
        cfg = scaled("video", grid=(8, 8, 8), h=1, R=3, D=64, dtype="f32")
        x = vsa_inputs(cfg, device=DEV)
        geom = bsa.VsaGeometry(cfg["grid"], cfg["block"], device=DEV)
        idx, num = bsa.pool_route_topk(x["q"], x["k"], geom.perm, geom.block_len, geom.J, geom.M, cfg["R"])
    assert _check_status() == L.BSA_OK
    J = geom.J
    bad, skip = idx.clone(), idx.clone()
    rows = torch.arange(0, J, 3, device=DEV)
    bad[:, :, rows, 1] = J          # names no block
    bad[:, 1:, rows, 0] = J + 1000
    skip[:, :, rows, 1] = -1        # the same entries as explicit holes
    skip[:, 1:, rows, 0] = -1
    call = lambda ii: bsa.attention_vsa(x["q"], x["k"], x["v"], geom.perm, geom.block_len, J, geom.M, ii, num,
                                        need_lse=True)
    o_skip, l_skip = call(skip)
    assert _check_status() == L.BSA_OK
    o_bad, l_bad = call(bad)
    assert _check_status() == L.BSA_ERR_INDEX
    assert _check_status() == L.BSA_OK   # reported once, then cleared
    assert torch.equal(o_bad, o_skip) and torch.equal(l_bad, l_skip)
    # and the skipped entries really are skipped: the oracle with -1 holes
    tab = oracle.tile_index(*cfg["grid"], *cfg["block"])
    items = [(0, 0, int(i)) for i in rows[:4].tolist()]
    ref, _ = oracle.vsa_attention(to64(x["q"]), to64(x["k"]), to64(x["v"]), tab["perm"], tab["block_len"],
                                  tab["M"], skip.cpu().numpy(), num.cpu().numpy(), items=items)
    mask = ~np.isnan(ref)
    assert np.abs(to64(o_bad)[mask] - ref[mask]).max() <= 2e-2


def test_nsa_block_past_the_sequence_is_skipped_and_reported():
    cfg = scaled("nsa", T=640, HQ=16, H=2)
    q, k, v, idx, cnt = nsa_inputs(cfg, device=DEV)
    nb = (cfg["T"] + cfg["BS"] - 1) // cfg["BS"]
    bad, skip = idx.clone(), idx.clone()
    # the last slot within the count of every 5th token names a block past the end
    t = torch.arange(0, cfg["T"], 5, device=DEV)
    last = (cnt[0, t, 0] - 1).long()
    bad[0, t, 0, last] = nb + 3
    skip[0, t, 0, last] = -1
    assert _check_status() == L.BSA_OK
    o_skip = bsa.attention_nsa(q, k, v, skip, cnt, cfg["BS"])
    assert _check_status() == L.BSA_OK
    o_bad = bsa.attention_nsa(q, k, v, bad, cnt, cfg["BS"])
    assert _check_status() == L.BSA_ERR_INDEX
    assert _check_status() == L.BSA_OK
    assert torch.equal(o_bad, o_skip)


def test_kvouter_block_past_the_sequence_is_skipped_and_reported():
    cfg = scaled("msa", N=1024, Hq=16, Hkv=2, k=6)
    q, k, v, q2k = msa_inputs(cfg, device=DEV)
    nb = (cfg["N"] + cfg["BK"] - 1) // cfg["BK"]
    bad, skip = q2k.clone(), q2k.clone()
    pos = torch.arange(3, cfg["N"], 7, device=DEV)
    bad[0, pos, 1, -1] = nb       # the last slot of these rows names no block
    skip[0, pos, 1, -1] = -1
    assert _check_status() == L.BSA_OK
    o1, l1, n1 = bsa.kvouter(q, k, v, skip, cfg["BK"])
    r1 = bsa.combine(o1, l1, n1, cfg["Hkv"])
    assert _check_status() == L.BSA_OK
    o2, l2, n2 = bsa.kvouter(q, k, v, bad, cfg["BK"])
    r2 = bsa.combine(o2, l2, n2, cfg["Hkv"])
    assert _check_status() == L.BSA_ERR_INDEX
    assert _check_status() == L.BSA_OK
    assert torch.equal(n1, n2) and torch.equal(r1, r2)
