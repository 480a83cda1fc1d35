"""GPU parity of the NSA selected-branch mode (token selections, GQA) against
the float64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_attn_close, to64
from workloads import nsa_inputs, scaled, workload

pytestmark = pytest.mark.gpu

bsa = pytest.importorskip("block_sparse_attention_02_amd")
DEV = torch.device("cuda:0")

CASES = {
    "g16_bs64": scaled("nsa", T=1024, HQ=32, H=2),
    "g8_bs64": scaled("nsa", T=640, HQ=16, H=2),
    "g32_bs64": scaled("nsa", T=512, HQ=64, H=2),
    "g16_bs32": scaled("nsa", T=700, HQ=16, H=1, BS=32, S=8),
    "g16_bs128": scaled("nsa", T=1100, HQ=16, H=1, BS=128, S=6),
    "g4_d64_ragged": scaled("nsa", T=999, HQ=8, H=2, D=64, S=12),
    "g16_bs64_b2": scaled("nsa", B=2, T=600, HQ=32, H=2),
    "g16_bs16": scaled("nsa", T=400, HQ=16, H=2, BS=16, S=10),
    "g1_mha": scaled("nsa", T=500, HQ=3, H=3, S=6),          # one query head per KV head
}


def _run_and_check(cfg, name, causal=True, counts=True, tokens=None):
    q, k, v, idx, cnt = nsa_inputs(cfg, device=DEV)
    out, lse = bsa.attention_nsa(q, k, v, idx, cnt if counts else None, cfg["BS"], causal=causal, need_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.nsa_attention(to64(q), to64(k), to64(v), idx.cpu().numpy(),
                                        cnt.cpu().numpy() if counts else None, cfg["BS"], causal=causal,
                                        tokens=tokens)
    mask = None
    if tokens is not None:
        mask = np.zeros(ref.shape, dtype=bool)
        for (b, t) in tokens:
            mask[b, t] = True
        ref = np.nan_to_num(ref)
    assert_attn_close(out, ref, name, mask=mask)
    got_lse = to64(lse).transpose(0, 2, 1)          # [B, HQ, T] -> [B, T, HQ]
    sel = np.isfinite(ref_lse) if tokens is None else (mask[..., 0] & np.isfinite(ref_lse))
    assert np.abs(got_lse[sel] - ref_lse[sel]).max() <= 1e-3
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_nsa_causal(name):
    print("case", name, flush=True)
    _run_and_check(CASES[name], name)


def test_nsa_non_causal_and_no_counts():
    cfg = scaled("nsa", T=512, HQ=16, H=1)
    _run_and_check(cfg, "non-causal", causal=False)
    _run_and_check(cfg, "no counts", counts=False)


def test_nsa_padding_inside_count_and_future_blocks():
    """-1 entries below the count are skipped; blocks after the token are masked."""
    cfg = scaled("nsa", T=512, HQ=16, H=1)
    q, k, v, idx, cnt = nsa_inputs(cfg, device=DEV)
    idx = idx.clone()
    cnt = cnt.clone()
    NB = 512 // 64
    rng = np.random.default_rng(1)
    idx_h = idx.cpu().numpy()
    cnt_h = cnt.cpu().numpy()
    for t in rng.integers(0, 512, 40):
        row = idx_h[0, t, 0]
        c = cnt_h[0, t, 0]
        if c < 16:
            row[c] = rng.integers(0, NB)            # maybe a future block
            cnt_h[0, t, 0] = c + 1
        if c >= 2:
            row[0] = -1
    idx_d = torch.from_numpy(idx_h).to(DEV)
    cnt_d = torch.from_numpy(cnt_h).to(DEV)
    out = bsa.attention_nsa(q, k, v, idx_d, cnt_d, 64, causal=True)
    torch.cuda.synchronize()
    ref, _ = oracle.nsa_attention(to64(q), to64(k), to64(v), idx_h, cnt_h, 64, causal=True)
    assert_attn_close(out, ref, "padding / future blocks")


def test_nsa_determinism():
    cfg = CASES["g16_bs64"]
    q, k, v, idx, cnt = nsa_inputs(cfg, device=DEV)
    o1 = bsa.attention_nsa(q, k, v, idx, cnt, 64)
    o2 = bsa.attention_nsa(q, k, v, idx, cnt, 64)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_nsa_full_size_sampled():
    """The full NSA workload (32768 tokens, 64/4 heads) on sampled tokens."""
    cfg = workload("nsa")
    rng = np.random.default_rng(4)
    tokens = [(0, int(t)) for t in rng.integers(0, cfg["T"], 48)] + [(0, 0), (0, 63), (0, 64), (0, cfg["T"] - 1)]
    print("case nsa full size", flush=True)
    _run_and_check(cfg, "nsa full (sampled)", tokens=tokens)
