"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host with the documented status codes."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

bsa = pytest.importorskip("block_sparse_attention_02_amd")
from block_sparse_attention_02_amd import _lib as L  # noqa: E402


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "bsa.h"), encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), "libbsa.so does not export %s" % n
    assert set(names) == set(L.PROTOTYPES), "binding prototypes differ from include/bsa.h"


def test_version_and_dims():
    lib = L.load()
    assert b"gfx950" in lib.bsa_version()
    assert bsa.tile_dims(4, 4, 4, 4, 2, 2) == (4, 16)
    assert bsa.tile_dims(30, 48, 80, 4, 4, 4) == (1920, 64)
    assert bsa.tile_dims(5, 3, 4, 4, 2, 2) == (8, 16)
    with pytest.raises(L.BsaError) as e:
        bsa.tile_dims(0, 4, 4, 4, 2, 2)
    assert e.value.status == L.BSA_ERR_SHAPE


def test_budget():
    assert bsa.keep_budget(0.75, 256) == 64
    assert bsa.keep_budget(0.7, 10) == 3
    assert bsa.keep_budget(0.9, 1920) == 192
    assert bsa.keep_budget(1.0, 5) == 1 and bsa.keep_budget(0.0, 5) == 5
    assert L.load().vsa_budget(1.5, 4) == -1 and L.load().vsa_budget(0.5, 0) == -1


def _route_args(**kw):
    d = L.TDesc(1, 64, 1, 64, 64 * 64, 64, 64)
    a = L.RouteArgs(ctypes.c_void_p(256), ctypes.c_void_p(256), d, L.BSA_F32, ctypes.c_void_p(256),
                    ctypes.c_void_p(256), 4, 16, 2, 4, 0.125, ctypes.c_void_p(256), ctypes.c_void_p(256),
                    None, None, None)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("q", None, L.BSA_ERR_ARG),
    ("q2k_idx", None, L.BSA_ERR_ARG),
    ("R", 5, L.BSA_ERR_SHAPE),
    ("R", 0, L.BSA_ERR_SHAPE),
    ("kmax", 1, L.BSA_ERR_SHAPE),
    ("J", 5000, L.BSA_ERR_UNSUPPORTED),
    ("kbar", 260, L.BSA_ERR_ARG),   # not 16-byte aligned
    ("dt", 7, L.BSA_ERR_ARG),
])
def test_route_validation(field, value, status):
    lib = L.load()
    a = _route_args(**{field: value})
    n = ctypes.c_size_t()
    assert lib.vsa_pool_route_topk_ws(ctypes.byref(a), ctypes.byref(n)) == status
    assert lib.bsa_last_error()
    assert lib.vsa_pool_route_topk(ctypes.byref(a), None, 0, None) == status


def test_route_workspace_size_and_short_workspace():
    lib = L.load()
    a = _route_args()
    n = ctypes.c_size_t()
    assert lib.vsa_pool_route_topk_ws(ctypes.byref(a), ctypes.byref(n)) == L.BSA_OK
    # two [1,1,4,64] fp32 pooled-mean buffers, then the key planes: one
    # 16-column tile x 2 channel steps x 64 lanes x 16 bytes, hi and lo
    assert n.value == 2 * 1024 + 1 * 2 * 64 * 16 * 2
    assert lib.vsa_pool_route_topk(ctypes.byref(a), None, 0, None) == L.BSA_ERR_WORKSPACE


def _qouter_args(**kw):
    d = L.TDesc(1, 64, 2, 128, 64 * 2 * 128, 2 * 128, 128)
    a = L.QOuterArgs(q=ctypes.c_void_p(256), k=ctypes.c_void_p(256), v=ctypes.c_void_p(256),
                     out=ctypes.c_void_p(256), dq=d, dkv=d, dout=d, dt=L.BSA_BF16, scale=0.088,
                     mode=L.BSA_SEL_BLOCK, perm=ctypes.c_void_p(256), block_len=ctypes.c_void_p(256),
                     J=1, M=64, q2k_idx=ctypes.c_void_p(256), q2k_num=ctypes.c_void_p(256), kmax=1)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("v", None, L.BSA_ERR_ARG),
    ("perm", None, L.BSA_ERR_ARG),
    ("M", 256, L.BSA_ERR_UNSUPPORTED),
    ("M", 48, L.BSA_ERR_UNSUPPORTED),
    ("mode", 9, L.BSA_ERR_ARG),
    ("q", ctypes.c_void_p(258), L.BSA_ERR_SHAPE),
    ("dt", 3, L.BSA_ERR_ARG),
    ("scale", float("inf"), L.BSA_ERR_ARG),
    ("order_long", -1, L.BSA_ERR_ARG),
    ("order_long", 2, L.BSA_ERR_ARG),   # > J = 1
])
def test_qouter_validation(field, value, status):
    a = _qouter_args(**{field: value})
    assert L.load().bsa_forward_qouter(ctypes.byref(a), None, 0, None) == status
    n = ctypes.c_size_t(7)
    assert L.load().bsa_qouter_ws(ctypes.byref(a), ctypes.byref(n)) == status


def test_qouter_workspace():
    """Block mode in bf16 needs the scheduler workspace (the same size for any
    shape); token mode and fp32 need none.  A missing, short or misaligned
    workspace is rejected before anything is enqueued."""
    lib = L.load()
    n = ctypes.c_size_t()
    a = _qouter_args()
    assert lib.bsa_qouter_ws(ctypes.byref(a), ctypes.byref(n)) == L.BSA_OK
    need = n.value
    assert 0 < need <= 1 << 20 and need % 256 == 0
    d2 = L.TDesc(2, 4096, 8, 64, 4096 * 8 * 64, 8 * 64, 64)
    assert lib.bsa_qouter_ws(ctypes.byref(_qouter_args(dq=d2, dkv=d2, dout=d2, J=64)), ctypes.byref(n)) == L.BSA_OK
    assert n.value == need
    assert lib.bsa_forward_qouter(ctypes.byref(a), None, 0, None) == L.BSA_ERR_WORKSPACE
    assert lib.bsa_forward_qouter(ctypes.byref(a), ctypes.c_void_p(256), need - 1, None) == L.BSA_ERR_WORKSPACE
    assert lib.bsa_forward_qouter(ctypes.byref(a), ctypes.c_void_p(256 + 16), need, None) == L.BSA_ERR_WORKSPACE
    assert b"workspace" in lib.bsa_last_error()
    f32 = _qouter_args(dt=L.BSA_F32)
    assert lib.bsa_qouter_ws(ctypes.byref(f32), ctypes.byref(n)) == L.BSA_OK and n.value == 0
    tok = _qouter_args(mode=L.BSA_SEL_TOKEN, blk_idx=ctypes.c_void_p(256), S=16, BS=64)
    assert lib.bsa_qouter_ws(ctypes.byref(tok), ctypes.byref(n)) == L.BSA_OK and n.value == 0


def _r256(x):
    return (x + 255) // 256 * 256


def test_qouter_capacity_128_workspace_and_limits():
    """Capacity 128 runs as 64-token halves: the workspace adds the halves'
    kept lists (B*H*2J rows of 2*kmax), counts (B*H*2J), lengths (2J) and,
    with an item order, the halves' order (B*H*2J), each rounded up to 256
    bytes; it takes no coarse branch."""
    lib = L.load()
    n = ctypes.c_size_t()
    sched = ctypes.c_size_t()
    assert lib.bsa_qouter_ws(ctypes.byref(_qouter_args()), ctypes.byref(sched)) == L.BSA_OK
    d = L.TDesc(2, 4096, 3, 64, 4096 * 3 * 64, 3 * 64, 64)
    a = _qouter_args(dq=d, dkv=d, dout=d, J=32, M=128, kmax=5)
    rows = 2 * 3 * 2 * 32
    tables = _r256(rows * 10 * 4) + _r256(rows * 4) + _r256(64 * 4)
    assert lib.bsa_qouter_ws(ctypes.byref(a), ctypes.byref(n)) == L.BSA_OK
    assert n.value == sched.value + tables
    a.item_order = ctypes.c_void_p(256)
    assert lib.bsa_qouter_ws(ctypes.byref(a), ctypes.byref(n)) == L.BSA_OK
    assert n.value == sched.value + tables + _r256(rows * 4)
    f32 = _qouter_args(dq=d, dkv=d, dout=d, J=32, M=128, kmax=5, dt=L.BSA_F32)
    assert lib.bsa_qouter_ws(ctypes.byref(f32), ctypes.byref(n)) == L.BSA_OK and n.value == tables
    co = _qouter_args(M=128, coarse=ctypes.c_void_p(256), gate=ctypes.c_void_p(256))
    assert lib.bsa_qouter_ws(ctypes.byref(co), ctypes.byref(n)) == L.BSA_ERR_UNSUPPORTED
    assert b"coarse" in lib.bsa_last_error()
    big = _qouter_args(M=128, kmax=1 << 29)
    assert lib.bsa_qouter_ws(ctypes.byref(big), ctypes.byref(n)) == L.BSA_ERR_UNSUPPORTED


def test_check_without_a_device_is_an_error_not_a_crash():
    """bsa_check reports a missing device through BSA_ERR_HIP (the index-error
    flag lives on the device and is read only after a successful sync)."""
    if bsa_gpu_present():
        pytest.skip("a GPU is present")
    assert L.load().bsa_check(None) == L.BSA_ERR_HIP


def bsa_gpu_present():
    import torch
    return torch.cuda.device_count() > 0


def test_qouter_shape_checks():
    lib = L.load()
    d64 = L.TDesc(1, 64, 2, 96, 64 * 2 * 96, 2 * 96, 96)
    a = _qouter_args(dq=d64, dkv=d64, dout=d64)
    assert lib.bsa_forward_qouter(ctypes.byref(a), None, 0, None) == L.BSA_ERR_UNSUPPORTED   # D = 96
    dkv = L.TDesc(1, 64, 1, 128, 64 * 128, 128, 128)
    a = _qouter_args(dkv=dkv)
    assert lib.bsa_forward_qouter(ctypes.byref(a), None, 0, None) == L.BSA_ERR_UNSUPPORTED   # VSA needs Hq == Hkv
    bad = L.TDesc(1, 64, 2, 128, 64 * 2 * 128, 2 * 128 + 4, 128)
    a = _qouter_args(dq=bad)
    assert lib.bsa_forward_qouter(ctypes.byref(a), None, 0, None) == L.BSA_ERR_SHAPE         # stride % 8


def test_qouter_32bit_slice_limits():
    """Block mode addresses one (batch, head) K/V slice with 32-bit offsets: a
    slice of 4 GiB or more, N >= 2^24 or a token stride of 2^24 bytes is
    rejected on the host (no launch)."""
    lib = L.load()
    H, D = 24, 128
    big = 1 << 20  # 2^20 tokens x 24 heads x 128 x 2 bytes = 6 GiB slice span
    d = L.TDesc(1, big, H, D, big * H * D, H * D, D)
    assert lib.bsa_forward_qouter(ctypes.byref(_qouter_args(dq=d, dkv=d, dout=d)), None, 0, None) == L.BSA_ERR_UNSUPPORTED
    d = L.TDesc(1, 1 << 24, 1, 64, (1 << 24) * 64, 64, 64)  # 2 GiB slice, but N = 2^24
    assert lib.bsa_forward_qouter(ctypes.byref(_qouter_args(dq=d, dkv=d, dout=d)), None, 0, None) == L.BSA_ERR_UNSUPPORTED
    d = L.TDesc(1, 64, 1, 128, 64 * (1 << 23), 1 << 23, 128)  # token stride 2^24 bytes
    assert lib.bsa_forward_qouter(ctypes.byref(_qouter_args(dq=d, dkv=d, dout=d)), None, 0, None) == L.BSA_ERR_UNSUPPORTED
    # a 384 MiB slice span passes, and the call stops at the summaries check that follows
    ok = L.TDesc(1, 1 << 16, H, D, (1 << 16) * H * D, H * D, D)
    a = _qouter_args(dq=ok, dkv=ok, dout=ok, k_sum=ctypes.c_void_p(256))
    assert lib.bsa_forward_qouter(ctypes.byref(a), None, 0, None) == L.BSA_ERR_ARG


H3_CASES = [
    ([130, (2, 16, 16), 60, 200, (4, 16, 16)], (2, 8, 8)),   # the page's metadata example
    ([5, (3, 5, 6), 9, (2, 3, 3), 1, (5, 4, 2)], (2, 2, 2)),
    ([0, (7, 9, 13)], (4, 4, 4)),                            # an empty dense segment
    ([300, 77], (4, 4, 4)),                                  # dense only
]


@pytest.mark.parametrize("case", range(len(H3_CASES)))
def test_h3_dims_match_oracle(case):
    import oracle
    segments, block = H3_CASES[case]
    seg = bsa.api._segments(segments)
    J, M, N, P, nr = (ctypes.c_int() for _ in range(5))
    spans = (ctypes.c_int * 32)()
    assert L.load().h3_tile_dims(seg, len(seg), *block, ctypes.byref(J), ctypes.byref(M), ctypes.byref(N),
                                 ctypes.byref(P), ctypes.byref(nr), spans) == L.BSA_OK
    lay = oracle.h3_layout(segments, block)
    assert (J.value, M.value, N.value, P.value) == (lay["J"], lay["M"], lay["N"], lay["num_prefix"])
    assert [(spans[2 * r], spans[2 * r + 1]) for r in range(nr.value)] == lay["spans"]


@pytest.mark.parametrize("segments,status", [
    ([], L.BSA_ERR_ARG),                 # no segment list
    ([8] * 17, L.BSA_ERR_UNSUPPORTED),
    ([(0, 4, 4)], L.BSA_ERR_SHAPE),
    ([-3, (1, 4, 4)], L.BSA_ERR_SHAPE),
    ([0, 0], L.BSA_ERR_SHAPE),
])
def test_h3_layout_validation(segments, status):
    lib = L.load()
    seg = bsa.api._segments(segments) if segments else None
    J, M, N, P, nr = (ctypes.c_int() for _ in range(5))
    got = lib.h3_tile_dims(seg, len(segments), 4, 4, 4, ctypes.byref(J), ctypes.byref(M), ctypes.byref(N),
                           ctypes.byref(P), ctypes.byref(nr), None)
    assert got == status and lib.bsa_last_error()
    bad = (L.Segment * 1)(L.Segment(2, 4, 4, 4))
    assert lib.h3_tile_dims(bad, 1, 4, 4, 4, ctypes.byref(J), ctypes.byref(M), ctypes.byref(N), ctypes.byref(P),
                            ctypes.byref(nr), None) == L.BSA_ERR_ARG


def _h3_args(spans, budgets, num_prefix=2, J=10, kmax=10):
    d = L.TDesc(1, 640, 1, 64, 640 * 64, 64, 64)
    sp = (ctypes.c_int32 * max(1, len(spans)))(*spans)
    bu = (ctypes.c_int32 * max(1, len(budgets)))(*budgets)
    a = L.H3RouteArgs(q=ctypes.c_void_p(256), k=ctypes.c_void_p(256), d=d, dt=L.BSA_BF16, perm=ctypes.c_void_p(256),
                      block_len=ctypes.c_void_p(256), J=J, M=64, num_prefix=num_prefix, nregions=len(budgets),
                      spans=ctypes.cast(sp, ctypes.c_void_p), budgets=ctypes.cast(bu, ctypes.c_void_p), kmax=kmax,
                      scale=0.125, q2k_idx=ctypes.c_void_p(256), q2k_num=ctypes.c_void_p(256))
    return a, (sp, bu)


@pytest.mark.parametrize("spans,budgets,kw,status", [
    ([2, 5, 5, 10], [1, 2], {}, L.BSA_OK),
    ([2, 5, 6, 10], [1, 2], {}, L.BSA_ERR_SHAPE),           # a gap between regions
    ([3, 5, 5, 10], [1, 2], {}, L.BSA_ERR_SHAPE),           # does not start at num_prefix
    ([2, 5, 5, 9], [1, 2], {}, L.BSA_ERR_SHAPE),            # does not end at J
    ([2, 5, 5, 10], [0, 2], {}, L.BSA_ERR_SHAPE),           # empty budget
    ([2, 5, 5, 10], [4, 2], {}, L.BSA_ERR_SHAPE),           # budget above the region size
    ([2, 5, 5, 10], [1, 2], {"kmax": 9}, L.BSA_ERR_SHAPE),  # context rows need kmax >= J
    ([2, 5, 5, 10], [1, 2], {"num_prefix": 0, "kmax": 2}, L.BSA_ERR_SHAPE),  # below the 1 + 2 kept
    ([2, 5, 5, 10], [1, 2], {"num_prefix": 0, "kmax": 3}, L.BSA_OK),
    ([], [], {}, L.BSA_ERR_SHAPE),                          # video rows without regions
    ([], [], {"num_prefix": 10}, L.BSA_OK),                 # all context
])
def test_h3_route_validation(spans, budgets, kw, status):
    if kw.get("num_prefix") == 0:
        spans = [0, 5, 5, 10]
    a, keep = _h3_args(spans, budgets, **kw)
    n = ctypes.c_size_t()
    assert L.load().h3_pool_route_topk_ws(ctypes.byref(a), ctypes.byref(n)) == status
    if status == L.BSA_OK:
        # pooled means, plus the key planes of the widest region (at most 16
        # columns: one tile x 2 channel steps x 64 lanes x 16 bytes, hi and lo)
        planes = 1 * 2 * 64 * 16 * 2 if budgets else 0
        assert n.value == 2 * 10 * 64 * 4 + planes


def test_route_alignment_checks():
    """Pooled means given by the caller, and the workspace, must be 16-byte
    aligned (the key planes and means are read and written 16 bytes at a
    time); both calls refuse otherwise before anything is enqueued."""
    lib = L.load()
    n = ctypes.c_size_t()
    a, keep = _h3_args([2, 5, 5, 10], [1, 2])
    a.kbar = ctypes.c_void_p(264)
    assert lib.h3_pool_route_topk_ws(ctypes.byref(a), ctypes.byref(n)) == L.BSA_ERR_ARG
    assert b"aligned" in lib.bsa_last_error()
    a.kbar = None
    assert lib.h3_pool_route_topk_ws(ctypes.byref(a), ctypes.byref(n)) == L.BSA_OK
    assert lib.h3_pool_route_topk(ctypes.byref(a), ctypes.c_void_p(256 + 8), n.value, None) == L.BSA_ERR_WORKSPACE
    r = _route_args(qbar=ctypes.c_void_p(260))
    assert lib.vsa_pool_route_topk_ws(ctypes.byref(r), ctypes.byref(n)) == L.BSA_ERR_ARG
    r = _route_args()
    assert lib.vsa_pool_route_topk_ws(ctypes.byref(r), ctypes.byref(n)) == L.BSA_OK
    assert lib.vsa_pool_route_topk(ctypes.byref(r), ctypes.c_void_p(256 + 4), n.value, None) == L.BSA_ERR_WORKSPACE


def _kv_args(**kw):
    dq = L.TDesc(1, 256, 8, 128, 256 * 8 * 128, 8 * 128, 128)
    dkv = L.TDesc(1, 256, 2, 128, 256 * 2 * 128, 2 * 128, 128)
    ph = ctypes.c_void_p(256)
    a = L.KvOuterArgs(q=ph, k=ph, v=ph, dq=dq, dkv=dkv, dt=L.BSA_BF16, scale=0.088, causal=1, q2k=ph,
                      q2k_cnt=None, k_sel=4, BK=128, o_buf=ph, lse_buf=ph, nslot=ph, chunk_cap=0)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("q2k", None, L.BSA_ERR_ARG),
    ("nslot", None, L.BSA_ERR_ARG),
    ("dt", L.BSA_F32, L.BSA_ERR_UNSUPPORTED),
    ("BK", 96, L.BSA_ERR_UNSUPPORTED),
    ("k_sel", 0, L.BSA_ERR_UNSUPPORTED),
    ("k_sel", 65, L.BSA_ERR_UNSUPPORTED),
    ("chunk_cap", -1, L.BSA_ERR_ARG),
    ("scale", float("nan"), L.BSA_ERR_ARG),
    ("o_buf", ctypes.c_void_p(264), L.BSA_ERR_SHAPE),
    ("dkv", L.TDesc(1, 256, 3, 128, 256 * 3 * 128, 3 * 128, 128), L.BSA_ERR_SHAPE),   # 8 % 3
    ("dkv", L.TDesc(1, 255, 2, 128, 255 * 2 * 128, 2 * 128, 128), L.BSA_ERR_SHAPE),   # N differs
    ("dkv", L.TDesc(1, 256, 2, 96, 256 * 2 * 96, 2 * 96, 96), L.BSA_ERR_UNSUPPORTED),  # D differs / 96
])
def test_kvouter_validation(field, value, status):
    lib = L.load()
    a = _kv_args(**{field: value})
    n = ctypes.c_size_t()
    assert lib.bsa_kvouter_ws(ctypes.byref(a), ctypes.byref(n)) == status
    assert lib.bsa_forward_kvouter(ctypes.byref(a), None, 0, None) == status
    assert lib.bsa_last_error()


def test_kvouter_workspace_and_chunk_cap_bound():
    """The workspace holds counts, cursors, row pointers, the chunk list and
    the edges; a chunk cap above the number of possible edges (up to INT_MAX)
    acts as that bound, so the chunk list of the scan never overflows."""
    lib = L.load()
    n0, n1, n2 = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.bsa_kvouter_ws(ctypes.byref(_kv_args()), ctypes.byref(n0)) == L.BSA_OK
    emax = 256 * 2 * 4
    assert lib.bsa_kvouter_ws(ctypes.byref(_kv_args(chunk_cap=emax)), ctypes.byref(n1)) == L.BSA_OK
    assert lib.bsa_kvouter_ws(ctypes.byref(_kv_args(chunk_cap=2 ** 31 - 1)), ctypes.byref(n2)) == L.BSA_OK
    assert n1.value == n2.value > 0
    assert n0.value >= emax * 8   # the (position, slot) edge list alone
    a = _kv_args()
    assert lib.bsa_forward_kvouter(ctypes.byref(a), ctypes.c_void_p(256), n0.value - 1, None) == L.BSA_ERR_WORKSPACE
    assert lib.bsa_forward_kvouter(ctypes.byref(a), ctypes.c_void_p(256 + 128), n0.value,
                                   None) == L.BSA_ERR_WORKSPACE


@pytest.mark.parametrize("cap,eff", [(0, 2 * 4 * 128), (3, 3), (5000, 256 * 2 * 4), (2 ** 31 - 1, 256 * 2 * 4)])
def test_kvouter_index_layout(cap, eff):
    """The reverse index and schedule regions lie inside the workspace, do not
    overlap, are 256-byte aligned and have the sizes the header states."""
    lib = L.load()
    a = _kv_args(chunk_cap=cap)
    lay, n = L.KvOuterLayout(), ctypes.c_size_t()
    assert lib.bsa_kvouter_index_layout(ctypes.byref(a), ctypes.byref(lay)) == L.BSA_OK
    assert lib.bsa_kvouter_ws(ctypes.byref(a), ctypes.byref(n)) == L.BSA_OK
    rows, emax = 1 * 2 * 2, 256 * 2 * 4     # B * Hkv * ceil(256 / 128), B * N * Hkv * k_sel
    assert (lay.rows, lay.max_edges, lay.chunk_cap, lay.bytes) == (rows, emax, eff, n.value)
    assert lay.max_chunks == rows + -(-emax // eff)
    spans = sorted([(lay.off_count, 4 * rows), (lay.off_rowptr, 4 * (rows + 1)), (lay.off_nchunk, 4),
                    (lay.off_chunks, 16 * lay.max_chunks), (lay.off_edges, 8 * emax)])
    for (o0, n0), (o1, _) in zip(spans, spans[1:]):
        assert o0 + n0 <= o1
    assert all(o % 256 == 0 for o, _ in spans) and spans[-1][0] + spans[-1][1] <= lay.bytes
    assert lib.bsa_kvouter_index_layout(ctypes.byref(a), None) == L.BSA_ERR_ARG
    assert lib.bsa_kvouter_index_layout(ctypes.byref(_kv_args(k_sel=0)), ctypes.byref(lay)) == L.BSA_ERR_UNSUPPORTED


def _combine_args(**kw):
    ph = ctypes.c_void_p(256)
    d = L.TDesc(1, 256, 8, 128, 256 * 8 * 128, 8 * 128, 128)
    a = L.CombineArgs(o_buf=ph, lse_buf=ph, nslot=ph, k_sel=4, Hkv=2, dout=d, out=ph, lse=None)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("o_buf", None, L.BSA_ERR_ARG),
    ("out", None, L.BSA_ERR_ARG),
    ("Hkv", 3, L.BSA_ERR_SHAPE),
    ("Hkv", 0, L.BSA_ERR_SHAPE),
    ("k_sel", 0, L.BSA_ERR_UNSUPPORTED),
    ("out", ctypes.c_void_p(260), L.BSA_ERR_SHAPE),
    ("dout", L.TDesc(1, 256, 8, 512, 256 * 8 * 512, 8 * 512, 512), L.BSA_ERR_UNSUPPORTED),
    ("dout", L.TDesc(1, 256, 8, 128, 256 * 8 * 128, 8 * 128 + 4, 128), L.BSA_ERR_SHAPE),
])
def test_combine_validation(field, value, status):
    assert L.load().bsa_combine(ctypes.byref(_combine_args(**{field: value})), None) == status


def _coarse_args(**kw):
    ph = ctypes.c_void_p(256)
    d = L.TDesc(1, 2048, 2, 128, 2048 * 2 * 128, 2 * 128, 128)
    a = L.CoarseArgs(v=ph, d=d, dt=L.BSA_BF16, perm=ph, block_len=ph, J=32, M=64, E=ph, vbar=None, C=ph)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("E", None, L.BSA_ERR_ARG),
    ("C", None, L.BSA_ERR_ARG),
    ("dt", 5, L.BSA_ERR_ARG),
    ("J", 0, L.BSA_ERR_SHAPE),
    ("C", ctypes.c_void_p(264), L.BSA_ERR_SHAPE),
    ("d", L.TDesc(1, 2048, 2, 96, 2048 * 2 * 96, 2 * 96, 96), L.BSA_ERR_UNSUPPORTED),
])
def test_coarse_validation(field, value, status):
    lib = L.load()
    a = _coarse_args(**{field: value})
    n = ctypes.c_size_t()
    assert lib.vsa_coarse_ws(ctypes.byref(a), ctypes.byref(n)) == status
    assert lib.vsa_coarse(ctypes.byref(a), None, 0, None) == status


def test_coarse_workspace():
    lib = L.load()
    n = ctypes.c_size_t()
    assert lib.vsa_coarse_ws(ctypes.byref(_coarse_args()), ctypes.byref(n)) == L.BSA_OK
    # vbar (2 x 32 x 128 fp32) + the transposed bf16 hi/lo copy (2 x 2 x 128 x 64)
    assert n.value == 2 * 32 * 128 * 4 + 2 * 2 * 128 * 64 * 2
    assert lib.vsa_coarse(ctypes.byref(_coarse_args()), None, 0, None) == L.BSA_ERR_WORKSPACE


def _summary_args(**kw):
    ph = ctypes.c_void_p(256)
    d = L.TDesc(1, 2048, 2, 128, 2048 * 2 * 128, 2 * 128, 128)
    a = L.SummaryArgs(q=ph, k=ph, v=ph, d=d, dt=L.BSA_BF16, perm=ph, block_len=ph, J=32, M=64, scale=0.088,
                      anchor=None, anchor_out=None, k_sum=ph, v_sum=ph, b_sum=ph)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("k_sum", None, L.BSA_ERR_ARG),
    ("q", None, L.BSA_ERR_ARG),          # no anchor and no queries to take it from
    ("dt", L.BSA_F32, L.BSA_ERR_UNSUPPORTED),
    ("M", 65, L.BSA_ERR_SHAPE),
    ("scale", float("inf"), L.BSA_ERR_ARG),
    ("v", ctypes.c_void_p(264), L.BSA_ERR_SHAPE),
])
def test_summaries_validation(field, value, status):
    lib = L.load()
    a = _summary_args(**{field: value})
    n = ctypes.c_size_t()
    assert lib.spark_summaries_ws(ctypes.byref(a), ctypes.byref(n)) == status
    assert lib.spark_summaries(ctypes.byref(a), None, 0, None) == status


def test_summaries_workspace_only_without_anchor():
    lib = L.load()
    n = ctypes.c_size_t()
    assert lib.spark_summaries_ws(ctypes.byref(_summary_args()), ctypes.byref(n)) == L.BSA_OK and n.value > 0
    a = _summary_args(anchor=ctypes.c_void_p(256), q=None)
    assert lib.spark_summaries_ws(ctypes.byref(a), ctypes.byref(n)) == L.BSA_OK and n.value == 0


def _reblock_args(**kw):
    ph = ctypes.c_void_p(256)
    d = L.TDesc(1, 2048, 2, 128, 2048 * 2 * 128, 2 * 128, 128)
    a = L.ReblockArgs(q=ph, k=ph, d=d, dt=L.BSA_BF16, M=64, ridge=1e-4, perm=ph, block_len=ph)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("perm", None, L.BSA_ERR_ARG),
    ("dt", L.BSA_F32, L.BSA_ERR_UNSUPPORTED),
    ("M", 48, L.BSA_ERR_UNSUPPORTED),
    ("ridge", 0.0, L.BSA_ERR_ARG),
    ("ridge", float("nan"), L.BSA_ERR_ARG),
    ("q", ctypes.c_void_p(264), L.BSA_ERR_SHAPE),
    ("d", L.TDesc(1, 2048, 2, 32, 2048 * 2 * 32, 2 * 32, 32), L.BSA_ERR_UNSUPPORTED),
])
def test_reblock_validation(field, value, status):
    lib = L.load()
    a = _reblock_args(**{field: value})
    n = ctypes.c_size_t()
    assert lib.spark_reblock_ws(ctypes.byref(a), ctypes.byref(n)) == status
    assert lib.spark_reblock(ctypes.byref(a), None, 0, None) == status


def test_reblock_dims_and_workspace():
    lib = L.load()
    J, nl = ctypes.c_int(), ctypes.c_int()
    assert lib.spark_reblock_dims(115200, 64, ctypes.byref(J), ctypes.byref(nl)) == L.BSA_OK
    assert (J.value, nl.value) == (1800, 12)
    assert lib.spark_reblock_dims(0, 64, ctypes.byref(J), ctypes.byref(nl)) == L.BSA_ERR_SHAPE
    n = ctypes.c_size_t()
    assert lib.spark_reblock_ws(ctypes.byref(_reblock_args()), ctypes.byref(n)) == L.BSA_OK and n.value > 0
    assert lib.spark_reblock(ctypes.byref(_reblock_args()), ctypes.c_void_p(256), n.value - 1,
                             None) == L.BSA_ERR_WORKSPACE
