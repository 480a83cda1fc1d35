"""PyTorch-facing binding of libbsa (argument marshalling only).

Every function takes device tensors, fills the C structs of include/bsa.h and
enqueues the library call on the current HIP stream.  All arithmetic happens
in the library's kernels; torch only provides memory and streams.  Outputs are
allocated with torch when the caller does not pass them.
"""

import ctypes
import math

import torch

from . import _lib as L

__all__ = [
    "tile_dims", "tile_index", "keep_budget", "pool_route_topk", "route_workspace_bytes",
    "attention_vsa", "attention_nsa", "coarse_attention", "spark_summaries", "H3Geometry",
    "h3_pool_route_topk", "h3_forward", "spark_reblock", "reblock_forward", "kvouter", "combine", "VsaGeometry", "vsa_forward",
    "qouter_workspace", "check",
]


def check(device=None):
    """bsa_check on the current stream of ``device``: synchronises, then raises
    BsaError (BSA_ERR_INDEX) if a kernel met a block id that names no block."""
    dev = torch.device("cuda") if device is None else torch.device(device)
    L.check(_lib().bsa_check(_stream(dev)))


def _lib():
    return L.load()


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _desc(t):
    if t.dim() != 4:
        raise ValueError("expected a 4-D [B, N, H, D] tensor")
    if t.stride(3) != 1:
        raise ValueError("the last dimension must be contiguous")
    B, N, H, D = t.shape
    return L.TDesc(B, N, H, D, t.stride(0), t.stride(1), t.stride(2))


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return L.BSA_BF16
    if t.dtype == torch.float32:
        return L.BSA_F32
    raise TypeError("unsupported dtype %s (bf16 or float32)" % t.dtype)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libbsa works on device tensors only")


def tile_dims(T, H, W, bT, bH, bW):
    """(J, M) of a (T, H, W) token grid cut into (bT, bH, bW) blocks."""
    J, M = ctypes.c_int(), ctypes.c_int()
    L.check(_lib().bsa_tile_dims(T, H, W, bT, bH, bW, ctypes.byref(J), ctypes.byref(M)))
    return J.value, M.value


def tile_index(T, H, W, bT, bH, bW, device="cuda"):
    """perm [J*M], block_len [J], inv [T*H*W] int32 tensors on ``device``."""
    J, M = tile_dims(T, H, W, bT, bH, bW)
    perm = torch.empty(J * M, dtype=torch.int32, device=device)
    block_len = torch.empty(J, dtype=torch.int32, device=device)
    inv = torch.empty(T * H * W, dtype=torch.int32, device=device)
    L.check(_lib().vsa_tile_index(T, H, W, bT, bH, bW, _ptr(perm), _ptr(block_len), _ptr(inv),
                                  _stream(perm.device)))
    return perm, block_len, inv


def keep_budget(drop_ratio, J):
    r = _lib().vsa_budget(float(drop_ratio), int(J))
    if r < 0:
        raise ValueError("drop ratio must lie in [0, 1] and J >= 1")
    return r


def _route_args(q, k, perm, block_len, J, M, R, kmax, scale, q2k_idx, q2k_num, qbar, kbar, E, item_order=None):
    return L.RouteArgs(_ptr(q), _ptr(k), _desc(q), _dtype(q), _ptr(perm), _ptr(block_len), J, M, R, kmax,
                       scale, _ptr(q2k_idx), _ptr(q2k_num), _ptr(qbar), _ptr(kbar), _ptr(E), _ptr(item_order))


def route_workspace_bytes(q, J, M, R, kmax=None, debug=False):
    """Workspace size of pool_route_topk for these shapes."""
    kmax = R if kmax is None else kmax
    placeholder = ctypes.c_void_p(256)
    a = L.RouteArgs(placeholder, placeholder, _desc(q), _dtype(q), placeholder, placeholder, J, M, R, kmax,
                    1.0, placeholder, placeholder, placeholder if debug else None,
                    placeholder if debug else None, None)
    n = ctypes.c_size_t()
    L.check(_lib().vsa_pool_route_topk_ws(ctypes.byref(a), ctypes.byref(n)))
    return n.value


def pool_route_topk(q, k, perm, block_len, J, M, R, kmax=None, scale=None, debug=False,
                    out=None, workspace=None, item_order=None, scores=None, perm_bh_stride=0):
    """Per-block means, routing scores and TopK index table.

    q, k: [B, N, H, D] (bf16 or float32).  Returns (q2k_idx [B,H,J,kmax],
    q2k_num [B,H,J]) and, with ``debug``, also (qbar, kbar, E) in float32.
    ``item_order`` (optional int32 [B,H,J] tensor) is filled with a processing
    order of the query blocks for attention_vsa.  ``scores`` (optional
    contiguous float32 [B,H,J,J] tensor) receives E without the debug outputs.
    ``perm_bh_stride``: 0 (one shared table) or the distance between the
    per-(b, h) tables of ``perm`` (e.g. J*M for spark_reblock's layouts).
    """
    _need_cuda(q, k, perm, block_len)
    B, N, H, D = q.shape
    kmax = R if kmax is None else int(kmax)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dev = q.device
    if out is None:
        q2k_idx = torch.empty((B, H, J, kmax), dtype=torch.int32, device=dev)
        q2k_num = torch.empty((B, H, J), dtype=torch.int32, device=dev)
    else:
        q2k_idx, q2k_num = out
    qbar = kbar = E = None
    if debug:
        qbar = torch.empty((B, H, J, D), dtype=torch.float32, device=dev)
        kbar = torch.empty_like(qbar)
        E = torch.empty((B, H, J, J), dtype=torch.float32, device=dev)
    if scores is not None:
        _need_cuda(scores)
        if scores.dtype != torch.float32 or scores.numel() != B * H * J * J or not scores.is_contiguous():
            raise ValueError("scores must be a contiguous float32 tensor of B*H*J*J elements")
        if E is not None:
            raise ValueError("scores and debug are exclusive")
        E = scores
    if item_order is not None:
        _need_cuda(item_order)
        if item_order.dtype != torch.int32 or item_order.numel() != B * H * J or not item_order.is_contiguous():
            raise ValueError("item_order must be a contiguous int32 tensor of B*H*J elements")
    a = _route_args(q, k, perm, block_len, J, M, R, kmax, scale, q2k_idx, q2k_num, qbar, kbar, E, item_order)
    a.perm_bh_stride = int(perm_bh_stride)
    n = ctypes.c_size_t()
    L.check(_lib().vsa_pool_route_topk_ws(ctypes.byref(a), ctypes.byref(n)))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    L.check(_lib().vsa_pool_route_topk(ctypes.byref(a), _ptr(workspace), n.value, _stream(dev)))
    if debug:
        return q2k_idx, q2k_num, qbar, kbar, E
    return q2k_idx, q2k_num


def _qouter_args(q, k, v, out, scale, mode, lse):
    return L.QOuterArgs(q=_ptr(q), k=_ptr(k), v=_ptr(v), out=_ptr(out), dq=_desc(q), dkv=_desc(k),
                        dout=_desc(out), dt=_dtype(q), scale=scale, mode=mode, lse=_ptr(lse))


def _forward_qouter(a, device, workspace):
    """bsa_forward_qouter with the caller's workspace (allocated when None or
    too small; the library itself never allocates).  ``workspace="static"``
    calls bsa_forward_qouter_static instead, which needs no workspace (calls
    that overlap on one device then race; see include/bsa.h)."""
    lib = _lib()
    if isinstance(workspace, str):
        if workspace != "static":
            raise ValueError("workspace must be a tensor, None or 'static'")
        L.check(lib.bsa_forward_qouter_static(ctypes.byref(a), _stream(device)))
        return
    n = ctypes.c_size_t()
    L.check(lib.bsa_qouter_ws(ctypes.byref(a), ctypes.byref(n)))
    if n.value and (workspace is None or workspace.numel() < n.value):
        workspace = torch.empty(n.value, dtype=torch.uint8, device=device)
    L.check(lib.bsa_forward_qouter(ctypes.byref(a), _ptr(workspace if n.value else None), n.value,
                                   _stream(device)))


def qouter_workspace(device="cuda"):
    """A workspace for attention_vsa / attention_nsa that can be reused by
    every call ordered on one stream (its size does not depend on shapes)."""
    a = L.QOuterArgs()
    n = ctypes.c_size_t()
    # the size only depends on the mode and dtype: query a bf16 block-mode call
    ph = ctypes.c_void_p(256)
    a.q = a.k = a.v = a.out = a.perm = a.block_len = a.q2k_idx = a.q2k_num = ph
    a.dq = a.dkv = a.dout = L.TDesc(1, 64, 1, 64, 64 * 64, 64, 64)
    a.dt, a.scale, a.mode, a.J, a.M, a.kmax = L.BSA_BF16, 1.0, L.BSA_SEL_BLOCK, 1, 64, 1
    L.check(_lib().bsa_qouter_ws(ctypes.byref(a), ctypes.byref(n)))
    return torch.empty(max(1, n.value), dtype=torch.uint8, device=device)


def coarse_attention(v, perm, block_len, J, M, E, need_vbar=False, out=None):
    """Coarse pooled-V branch: C [B, H, J, D] fp32 = softmax(E) V_bar, with
    V_bar the per-block means of v [B, N, H, D] (bf16 or float32) and E the
    fp32 [B, H, J, J] routing scores.  With ``need_vbar`` also returns V_bar."""
    _need_cuda(v, perm, block_len, E)
    B, N, H, D = v.shape
    if E.dtype != torch.float32 or E.numel() != B * H * J * J or not E.is_contiguous():
        raise ValueError("E must be a contiguous float32 tensor of B*H*J*J elements")
    dev = v.device
    C = torch.empty((B, H, J, D), dtype=torch.float32, device=dev) if out is None else out
    if C.dtype != torch.float32 or C.numel() != B * H * J * D or not C.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor of B*H*J*D elements")
    vbar = torch.empty((B, H, J, D), dtype=torch.float32, device=dev) if need_vbar else None
    a = L.CoarseArgs(v=_ptr(v), d=_desc(v), dt=_dtype(v), perm=_ptr(perm), block_len=_ptr(block_len), J=J, M=M,
                     E=_ptr(E), vbar=_ptr(vbar), C=_ptr(C))
    lib = _lib()
    n = ctypes.c_size_t(0)
    L.check(lib.vsa_coarse_ws(ctypes.byref(a), ctypes.byref(n)))
    ws = torch.empty(n.value, dtype=torch.uint8, device=dev) if n.value else None
    L.check(lib.vsa_coarse(ctypes.byref(a), _ptr(ws), n.value, _stream(dev)))
    return (C, vbar) if need_vbar else C


def spark_summaries(q, k, v, perm, block_len, J, M, scale=None, anchor=None, need_anchor=False):
    """Spark-Reweight block summaries: bf16 k_sum, v_sum [B, H, J, D] and fp32
    b_sum [B, H, J] (plus the fp32 anchor [B, H, D] with ``need_anchor``).
    ``anchor``: optional fp32 [B, H, D] representative queries (default: the
    mean of q over all tokens of each head)."""
    _need_cuda(k, v, perm, block_len)
    if k.stride() != v.stride() or k.shape != v.shape or (q is not None and (q.stride() != k.stride()
                                                                               or q.shape != k.shape)):
        raise ValueError("q, k and v must share shape and strides")
    B, N, H, D = k.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dev = k.device
    k_sum = torch.empty((B, H, J, D), dtype=torch.bfloat16, device=dev)
    v_sum = torch.empty((B, H, J, D), dtype=torch.bfloat16, device=dev)
    b_sum = torch.empty((B, H, J), dtype=torch.float32, device=dev)
    anchor_out = torch.empty((B, H, D), dtype=torch.float32, device=dev) if need_anchor else None
    if anchor is not None:
        _need_cuda(anchor)
        if anchor.dtype != torch.float32 or anchor.numel() != B * H * D or not anchor.is_contiguous():
            raise ValueError("anchor must be a contiguous float32 tensor of B*H*D elements")
    a = L.SummaryArgs(q=_ptr(q), k=_ptr(k), v=_ptr(v), d=_desc(k), dt=_dtype(k), perm=_ptr(perm),
                      block_len=_ptr(block_len), J=J, M=M, scale=scale, anchor=_ptr(anchor),
                      anchor_out=_ptr(anchor_out), k_sum=_ptr(k_sum), v_sum=_ptr(v_sum), b_sum=_ptr(b_sum))
    lib = _lib()
    nbytes = ctypes.c_size_t(0)
    L.check(lib.spark_summaries_ws(ctypes.byref(a), ctypes.byref(nbytes)))
    ws = torch.empty(max(1, nbytes.value), dtype=torch.uint8, device=dev) if nbytes.value else None
    L.check(lib.spark_summaries(ctypes.byref(a), _ptr(ws), nbytes.value, _stream(dev)))
    return (k_sum, v_sum, b_sum, anchor_out) if need_anchor else (k_sum, v_sum, b_sum)


def attention_vsa(q, k, v, perm, block_len, J, M, q2k_idx, q2k_num, scale=None, need_lse=False, out=None,
                  item_order=None, summaries=None, coarse=None, perm_bh_stride=0, workspace=None, order_long=0):
    """Block-selected exact attention (VSA mode).  q, k, v: [B, N, H, D].
    ``item_order``: optional processing order (from pool_route_topk).
    ``summaries``: optional (k_sum, v_sum, b_sum) from spark_summaries; every
    block a query block does not keep then enters through its virtual token.
    ``coarse``: optional (C, gate) -- C fp32 [B,H,J,D] from coarse_attention,
    gate fp32 [H, D]; each token of block i then gets gate * C[:, :, i] added.
    ``perm_bh_stride``: per-(b, h) tables in ``perm`` (as in pool_route_topk).
    ``order_long``: the first order_long positions of every (b, h)'s order
    run first, across all (b, h) (long kept lists first; results unchanged).
    ``workspace``: optional uint8 device tensor from qouter_workspace (calls
    that share one must be ordered on one stream), or "static" for the
    library's no-allocation entry point."""
    _need_cuda(q, k, v, perm, block_len, q2k_idx, q2k_num)
    if k.stride() != v.stride() or k.shape != v.shape:
        raise ValueError("k and v must share shape and strides")
    B, N, H, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if need_lse else None
    a = _qouter_args(q, k, v, out, scale, L.BSA_SEL_BLOCK, lse)
    a.perm, a.block_len, a.J, a.M = _ptr(perm), _ptr(block_len), J, M
    a.q2k_idx, a.q2k_num, a.kmax = _ptr(q2k_idx), _ptr(q2k_num), q2k_idx.shape[-1]
    a.perm_bh_stride = int(perm_bh_stride)
    a.order_long = int(order_long)
    if item_order is not None:
        _need_cuda(item_order)
        if item_order.dtype != torch.int32 or item_order.numel() != B * H * J or not item_order.is_contiguous():
            raise ValueError("item_order must be a contiguous int32 tensor of B*H*J elements")
        a.item_order = _ptr(item_order)
    if summaries is not None:
        k_sum, v_sum, b_sum = summaries
        _need_cuda(k_sum, v_sum, b_sum)
        if (k_sum.dtype != torch.bfloat16 or v_sum.dtype != torch.bfloat16 or b_sum.dtype != torch.float32
                or k_sum.numel() != B * H * J * D or v_sum.numel() != B * H * J * D or b_sum.numel() != B * H * J
                or not (k_sum.is_contiguous() and v_sum.is_contiguous() and b_sum.is_contiguous())):
            raise ValueError("summaries must be contiguous bf16 [B,H,J,D] k_sum/v_sum and float32 [B,H,J] b_sum")
        a.k_sum, a.v_sum, a.b_sum = _ptr(k_sum), _ptr(v_sum), _ptr(b_sum)
    if coarse is not None:
        C, gate = coarse
        _need_cuda(C, gate)
        if (C.dtype != torch.float32 or gate.dtype != torch.float32 or C.numel() != B * H * J * D
                or gate.numel() != H * D or not (C.is_contiguous() and gate.is_contiguous())):
            raise ValueError("coarse must be a contiguous float32 C [B,H,J,D] and gate [H,D]")
        a.coarse, a.gate = _ptr(C), _ptr(gate)
    _forward_qouter(a, q.device, workspace)
    return (out, lse) if need_lse else out


def attention_nsa(q, k, v, block_indices, block_counts, block_size, causal=True, scale=None,
                  need_lse=False, out=None):
    """NSA selected-branch attention with GQA.  q [B,T,HQ,D], k/v [B,T,H,D]."""
    _need_cuda(q, k, v, block_indices, block_counts)
    if k.stride() != v.stride() or k.shape != v.shape:
        raise ValueError("k and v must share shape and strides")
    B, T, HQ, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, HQ, T), dtype=torch.float32, device=q.device) if need_lse else None
    a = _qouter_args(q, k, v, out, scale, L.BSA_SEL_TOKEN, lse)
    a.blk_idx, a.blk_cnt = _ptr(block_indices), _ptr(block_counts)
    a.S, a.BS, a.causal = block_indices.shape[-1], int(block_size), int(bool(causal))
    _forward_qouter(a, q.device, None)
    return (out, lse) if need_lse else out


def _kv_args(q, k, v, q2k, block_size, causal, q2k_cnt, scale, chunk_cap, o_buf, lse_buf, nslot):
    return L.KvOuterArgs(q=_ptr(q), k=_ptr(k), v=_ptr(v), dq=_desc(q), dkv=_desc(k), dt=_dtype(q),
                         scale=scale, causal=int(bool(causal)), q2k=_ptr(q2k), q2k_cnt=_ptr(q2k_cnt),
                         k_sel=q2k.shape[-1], BK=int(block_size), o_buf=_ptr(o_buf),
                         lse_buf=_ptr(lse_buf), nslot=_ptr(nslot), chunk_cap=int(chunk_cap))


def kvouter(q, k, v, q2k, block_size, causal=True, q2k_cnt=None, scale=None, chunk_cap=0,
            workspace=None, bufs=None, index=False):
    """KV-outer K1: returns (o_buf [B,ks,N,Hq,D] bf16, lse_buf [B,ks,N,Hq], nslot [B,N,Hkv]).

    With ``index=True`` a fourth item holds the reverse index and schedule the
    call left in its workspace (int32 views into it, valid until the
    workspace is reused): count [rows], rowptr [rows + 1], nchunk [1],
    chunks [max_chunks, 4] (the first nchunk are set), edges [max_edges, 2]
    (the first rowptr[rows] are set), plus rows and chunk_cap.
    """
    _need_cuda(q, k, v, q2k, q2k_cnt)
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    ks = q2k.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dev = q.device
    if bufs is None:
        o_buf = torch.empty((B, ks, N, Hq, D), dtype=torch.bfloat16, device=dev)
        lse_buf = torch.empty((B, ks, N, Hq), dtype=torch.float32, device=dev)
        nslot = torch.empty((B, N, Hkv), dtype=torch.int32, device=dev)
    else:
        o_buf, lse_buf, nslot = bufs
    a = _kv_args(q, k, v, q2k, block_size, causal, q2k_cnt, scale, chunk_cap, o_buf, lse_buf, nslot)
    n = ctypes.c_size_t()
    L.check(_lib().bsa_kvouter_ws(ctypes.byref(a), ctypes.byref(n)))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    L.check(_lib().bsa_forward_kvouter(ctypes.byref(a), _ptr(workspace), n.value, _stream(dev)))
    if not index:
        return o_buf, lse_buf, nslot
    lay = L.KvOuterLayout()
    L.check(_lib().bsa_kvouter_index_layout(ctypes.byref(a), ctypes.byref(lay)))

    def region(off, n_int32):
        return workspace[off:off + 4 * n_int32].view(torch.int32)

    views = {
        "rows": lay.rows,
        "chunk_cap": lay.chunk_cap,
        "count": region(lay.off_count, lay.rows),
        "rowptr": region(lay.off_rowptr, lay.rows + 1),
        "nchunk": region(lay.off_nchunk, 1),
        "chunks": region(lay.off_chunks, 4 * lay.max_chunks).view(lay.max_chunks, 4),
        "edges": region(lay.off_edges, 2 * lay.max_edges).view(lay.max_edges, 2),
    }
    return o_buf, lse_buf, nslot, views


def combine(o_buf, lse_buf, nslot, Hkv, need_lse=False, out=None):
    """KV-outer K2: exact LSE merge of the partials into out [B, N, Hq, D] (bf16)."""
    _need_cuda(o_buf, lse_buf, nslot)
    B, ks, N, Hq, D = o_buf.shape
    out = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device=o_buf.device) if out is None else out
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=o_buf.device) if need_lse else None
    a = L.CombineArgs(o_buf=_ptr(o_buf), lse_buf=_ptr(lse_buf), nslot=_ptr(nslot), k_sel=ks, Hkv=Hkv,
                      dout=_desc(out), out=_ptr(out), lse=_ptr(lse))
    L.check(_lib().bsa_combine(ctypes.byref(a), _stream(o_buf.device)))
    return (out, lse) if need_lse else out


class VsaGeometry:
    """Tiling tables of one (grid, block) geometry, built once on a device."""

    def __init__(self, grid, block, device="cuda"):
        T, H, W = grid
        bT, bH, bW = block
        self.grid, self.block = tuple(grid), tuple(block)
        self.J, self.M = tile_dims(T, H, W, bT, bH, bW)
        self.N = T * H * W
        self.perm, self.block_len, self.inv = tile_index(T, H, W, bT, bH, bW, device=device)


def vsa_forward(q, k, v, geom, R, kmax=None, scale=None, need_lse=False, workspace=None, index_out=None,
                gate=None):
    """Routed block-sparse attention: pool -> route -> TopK -> exact attention.
    ``gate`` (optional fp32 [H, D]) adds the coarse pooled-V branch.

    Returns (out, q2k_idx, q2k_num) (plus lse with ``need_lse``)."""
    B, _, H, _ = q.shape
    order = torch.empty((B, H, geom.J), dtype=torch.int32, device=q.device)
    E = None if gate is None else torch.empty((B, H, geom.J, geom.J), dtype=torch.float32, device=q.device)
    q2k_idx, q2k_num = pool_route_topk(q, k, geom.perm, geom.block_len, geom.J, geom.M, R, kmax=kmax,
                                       scale=scale, workspace=workspace, out=index_out, item_order=order,
                                       scores=E)
    coarse = None
    if gate is not None:
        coarse = (coarse_attention(v, geom.perm, geom.block_len, geom.J, geom.M, E), gate)
    res = attention_vsa(q, k, v, geom.perm, geom.block_len, geom.J, geom.M, q2k_idx, q2k_num, scale=scale,
                        need_lse=need_lse, item_order=order, coarse=coarse)
    if need_lse:
        return res[0], q2k_idx, q2k_num, res[1]
    return res, q2k_idx, q2k_num


def _segments(segments):
    """ctypes array of bsa_segment from ints (dense token counts) and (T, H, W) tuples."""
    arr = (L.Segment * len(segments))()
    for k, sg in enumerate(segments):
        if isinstance(sg, int):
            arr[k] = L.Segment(0, sg, 0, 0)
        else:
            T, H, W = sg
            arr[k] = L.Segment(1, int(T), int(H), int(W))
    return arr


class H3Geometry:
    """Tables of a multi-region layout (dense prefix chunks, then the video
    regions), built once on a device.  ``segments``: ints (dense segments of
    that many tokens) and (T, H, W) tuples (video regions) in original order."""

    def __init__(self, segments, block, device="cuda"):
        bT, bH, bW = block
        self.segments, self.block = list(segments), tuple(block)
        seg = _segments(self.segments)
        J, M, N, P, nr = (ctypes.c_int() for _ in range(5))
        spans = (ctypes.c_int * (2 * L.H3_MAX_SEGMENTS))()
        L.check(_lib().h3_tile_dims(seg, len(seg), bT, bH, bW, ctypes.byref(J), ctypes.byref(M), ctypes.byref(N),
                                    ctypes.byref(P), ctypes.byref(nr), spans))
        self.J, self.M, self.N, self.num_prefix = J.value, M.value, N.value, P.value
        self.spans = [(spans[2 * r], spans[2 * r + 1]) for r in range(nr.value)]
        self.perm = torch.empty(self.J * self.M, dtype=torch.int32, device=device)
        self.block_len = torch.empty(self.J, dtype=torch.int32, device=device)
        self.inv = torch.empty(self.N, dtype=torch.int32, device=device)
        L.check(_lib().h3_tile_index(seg, len(seg), bT, bH, bW, _ptr(self.perm), _ptr(self.block_len),
                                     _ptr(self.inv), _stream(self.perm.device)))

    def budgets(self, drop_ratio):
        """Keep budget of every video region for one drop ratio (or a list)."""
        ratios = drop_ratio if isinstance(drop_ratio, (list, tuple)) else [drop_ratio] * len(self.spans)
        return [keep_budget(r, b1 - b0) for r, (b0, b1) in zip(ratios, self.spans)]


def h3_pool_route_topk(q, k, geom, budgets, kmax=None, scale=None, item_order=None, debug=False, out=None,
                       workspace=None, fill=True):
    """Grouped routing over an H3 layout: context query blocks keep every
    block, video query blocks keep the prefix plus each region's TopK.
    Returns (q2k_idx [B,H,J,kmax], q2k_num [B,H,J]) (plus qbar, kbar with debug).
    ``fill=False`` leaves the entries past each row's count unwritten."""
    _need_cuda(q, k)
    B, N, H, D = q.shape
    J = geom.J
    kmax = J if kmax is None else int(kmax)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dev = q.device
    if out is None:
        q2k_idx = torch.empty((B, H, J, kmax), dtype=torch.int32, device=dev)
        q2k_num = torch.empty((B, H, J), dtype=torch.int32, device=dev)
    else:
        q2k_idx, q2k_num = out
    qbar = kbar = None
    if debug:
        qbar = torch.empty((B, H, J, D), dtype=torch.float32, device=dev)
        kbar = torch.empty_like(qbar)
    if item_order is not None:
        _need_cuda(item_order)
        if item_order.dtype != torch.int32 or item_order.numel() != B * H * J or not item_order.is_contiguous():
            raise ValueError("item_order must be a contiguous int32 tensor of B*H*J elements")
    nr = len(geom.spans)
    spans = (ctypes.c_int32 * max(1, 2 * nr))(*[v for sp in geom.spans for v in sp])
    buds = (ctypes.c_int32 * max(1, nr))(*[int(b) for b in budgets])
    a = L.H3RouteArgs(q=_ptr(q), k=_ptr(k), d=_desc(q), dt=_dtype(q), perm=_ptr(geom.perm),
                      block_len=_ptr(geom.block_len), J=J, M=geom.M, num_prefix=geom.num_prefix, nregions=nr,
                      spans=ctypes.cast(spans, ctypes.c_void_p), budgets=ctypes.cast(buds, ctypes.c_void_p),
                      kmax=kmax, scale=scale, q2k_idx=_ptr(q2k_idx), q2k_num=_ptr(q2k_num), qbar=_ptr(qbar),
                      kbar=_ptr(kbar), item_order=_ptr(item_order), no_fill=0 if fill else 1)
    lib = _lib()
    n = ctypes.c_size_t()
    L.check(lib.h3_pool_route_topk_ws(ctypes.byref(a), ctypes.byref(n)))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    L.check(lib.h3_pool_route_topk(ctypes.byref(a), _ptr(workspace), n.value, _stream(dev)))
    if debug:
        return q2k_idx, q2k_num, qbar, kbar
    return q2k_idx, q2k_num


def h3_forward(q, k, v, geom, budgets, scale=None, need_lse=False, workspace=None):
    """Multi-region routed attention: pool -> grouped route -> exact attention
    over the union of kept blocks (one softmax).  Returns (out, q2k_idx, q2k_num);
    the table's entries past each row's count are not written (no -1 fill)."""
    B, _, H, _ = q.shape
    order = torch.empty((B, H, geom.J), dtype=torch.int32, device=q.device)
    q2k_idx, q2k_num = h3_pool_route_topk(q, k, geom, budgets, scale=scale, item_order=order, workspace=workspace,
                                          fill=False)
    res = attention_vsa(q, k, v, geom.perm, geom.block_len, geom.J, geom.M, q2k_idx, q2k_num, scale=scale,
                        need_lse=need_lse, item_order=order, order_long=geom.num_prefix)
    if need_lse:
        return res[0], q2k_idx, q2k_num, res[1]
    return res, q2k_idx, q2k_num


def spark_reblock(q, k, M=64, ridge=1e-4, debug=False, workspace=None):
    """Spark-Reblock key layout per (batch, head), reused by the queries.

    q, k: bf16 [B, N, H, D] with the same strides.  Returns (perm int32
    [B*H, J*M], block_len int32 [J]); with ``debug`` also the fp32 moment and
    factor [B*H, D, D], the unit features [B*H, N, D], the per-level token
    orders int32 [nlevels, B*H, N] and split directions fp32
    [nlevels-1, B*H, 2^(nlevels-2), D].  Use with perm_bh_stride = J*M."""
    _need_cuda(q, k)
    if q.stride() != k.stride() or q.shape != k.shape:
        raise ValueError("q and k must share shape and strides")
    B, N, H, D = q.shape
    dev = q.device
    J, nl = ctypes.c_int(), ctypes.c_int()
    lib = _lib()
    L.check(lib.spark_reblock_dims(N, int(M), ctypes.byref(J), ctypes.byref(nl)))
    J, nl = J.value, nl.value
    perm = torch.empty((B * H, J * M), dtype=torch.int32, device=dev)
    block_len = torch.empty(J, dtype=torch.int32, device=dev)
    moment = factor = features = levels = dirs = None
    if debug:
        moment = torch.empty((B * H, D, D), dtype=torch.float32, device=dev)
        factor = torch.empty_like(moment)
        features = torch.empty((B * H, N, D), dtype=torch.float32, device=dev)
        levels = torch.empty((nl, B * H, N), dtype=torch.int32, device=dev)
        dirs = torch.zeros((max(nl - 1, 1), B * H, 1 << max(nl - 2, 0), D), dtype=torch.float32, device=dev)
    a = L.ReblockArgs(q=_ptr(q), k=_ptr(k), d=_desc(q), dt=_dtype(q), M=int(M), ridge=float(ridge), perm=_ptr(perm),
                      block_len=_ptr(block_len), moment=_ptr(moment), factor=_ptr(factor),
                      features=_ptr(features), levels=_ptr(levels), dirs=_ptr(dirs))
    n = ctypes.c_size_t()
    L.check(lib.spark_reblock_ws(ctypes.byref(a), ctypes.byref(n)))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    L.check(lib.spark_reblock(ctypes.byref(a), _ptr(workspace), n.value, _stream(dev)))
    if debug:
        return perm, block_len, moment, factor, features, levels, dirs
    return perm, block_len


def reblock_forward(q, k, v, R, M=64, ridge=1e-4, scale=None, need_lse=False):
    """Reblocked routed attention: Spark-Reblock key layout (reused by the
    queries) -> pool -> route -> TopK -> exact attention, outputs at the
    tokens' positions.  Returns (out, perm, q2k_idx, q2k_num)."""
    B, N, H, _ = q.shape
    perm, block_len = spark_reblock(q, k, M=M, ridge=ridge)
    J = block_len.numel()
    order = torch.empty((B, H, J), dtype=torch.int32, device=q.device)
    q2k_idx, q2k_num = pool_route_topk(q, k, perm, block_len, J, M, R, scale=scale, item_order=order,
                                       perm_bh_stride=J * M)
    res = attention_vsa(q, k, v, perm, block_len, J, M, q2k_idx, q2k_num, scale=scale, need_lse=need_lse,
                        item_order=order, perm_bh_stride=J * M)
    if need_lse:
        return res[0], perm, q2k_idx, q2k_num, res[1]
    return res, perm, q2k_idx, q2k_num
