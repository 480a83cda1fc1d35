"""KV-outer reverse index and scheduler: NumPy wrapper of the host C++ reference
in kv_schedule.cpp.

TEST INFRASTRUCTURE ONLY, like the rest of this package.  The C++ source
shares no code with the HIP library; it is compiled here with the host g++
into oracle/_build/ (``build()``; ``reference()`` builds it on first use when
it is missing or older than its source).

Source: "MSA 为什么采用 KV-outer Sparse Attention Forward" -- section 5 (q2k
turned into the k2q CSR: count, prefix sum, scatter) and section 7 (the
scheduler's chunks of at most ``cap`` edges of one hot KV tile; every
(query, block) partial has its own slot).  The readings the page leaves open
are listed at the top of kv_schedule.cpp.
"""

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "kv_schedule.cpp")
CHECKER = os.path.join(_HERE, "kv_schedule_check.cpp")
LIBRARY = os.path.join(_HERE, "_build", "libkv_schedule.so")

_lib = None


def build(out=LIBRARY):
    """Compile the reference into a shared library with the host g++."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["g++", "-std=c++17", "-O2", "-shared", "-fPIC", SOURCE, "-o", tmp], check=True)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        lib = ctypes.CDLL(LIBRARY)
        i32, i64, p = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        lib.kv_reference_sizes.restype = i32
        lib.kv_reference_sizes.argtypes = [i32] * 5 + [i64] + [ctypes.POINTER(i64)] * 3
        lib.kv_reference.restype = i32
        lib.kv_reference.argtypes = [p, p] + [i32] * 6 + [i64] + [p] * 6
        _lib = lib
    return _lib


def reference(q2k, BK, causal=True, q2k_cnt=None, cap=None):
    """Reverse index and schedule of the selections q2k [B, N, Hkv, ks] (-1
    padded), optional counts q2k_cnt [B, N, Hkv].  ``cap`` defaults to
    2 * ks * BK.  Returns a dict:

    count [rows], rowptr [rows + 1] (rows = B * Hkv * ceil(N / BK), in
    (b, r, block) order), chunks [nchunk, 4] {row, begin, end, 0},
    edges [rowptr[-1], 2] {position, slot} (each row by position, then slot),
    nslot [B, N, Hkv] and ``flagged`` (an id at or beyond the block count was
    skipped).
    """
    q2k = np.ascontiguousarray(q2k, dtype=np.int32)
    B, N, Hkv, ks = q2k.shape
    cnt = None if q2k_cnt is None else np.ascontiguousarray(q2k_cnt, dtype=np.int32)
    if cnt is not None and cnt.shape != (B, N, Hkv):
        raise ValueError("q2k_cnt must be [B, N, Hkv]")
    cap = 2 * ks * BK if cap is None else int(cap)
    lib = _load()
    rows, emax, max_chunks = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    if lib.kv_reference_sizes(B, N, Hkv, ks, BK, cap, ctypes.byref(rows), ctypes.byref(emax),
                              ctypes.byref(max_chunks)) != 0:
        raise ValueError("bad sizes")
    count = np.zeros(rows.value, np.int32)
    rowptr = np.zeros(rows.value + 1, np.int32)
    chunks = np.zeros((max_chunks.value, 4), np.int32)
    nchunk = np.zeros(1, np.int32)
    edges = np.zeros((max(emax.value, 1), 2), np.int32)
    nslot = np.zeros((B, N, Hkv), np.int32)

    def ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    rc = lib.kv_reference(ptr(q2k), ptr(cnt), B, N, Hkv, ks, BK, int(bool(causal)), cap, ptr(count), ptr(rowptr),
                          ptr(chunks), ptr(nchunk), ptr(edges), ptr(nslot))
    if rc < 0:
        raise ValueError("kv_reference rejected its arguments")
    return {"count": count, "rowptr": rowptr, "chunks": chunks[:nchunk[0]], "edges": edges[:rowptr[-1]],
            "nslot": nslot, "flagged": bool(rc)}
