"""CPU fp64 oracle for the native sparse attention forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library (``block_index_sparse_amd``) and does not import it.

``fwd`` wraps ``nsa_oracle.c`` (plain C, fp64, OpenMP over (token, kv head)):
it materialises each row's token mask from ``block_indices`` /
``block_counts`` and runs dense masked softmax attention.  ``fwd_qblock``
takes rows per query block and hands every token its query block's row.  ``brute`` holds a
pure-Python version for tiny inputs.  The definition and the readings it
takes are in the header of ``nsa_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_BUILD = os.path.join(_HERE, "_build")
_SO = os.path.join(_BUILD, "libnsa_oracle.so")
_SRC = os.path.join(_HERE, "nsa_oracle.c")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no fast-math)."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_SO)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.nsa_oracle_fwd.restype = ctypes.c_int
        lib.nsa_oracle_fwd.argtypes = [i64, i64, i64, i64, i64, i64, i64, p, p, p, p, p, p, i64,
                                       ctypes.c_double, p, i64, p, p, ctypes.c_int]
        lib.nsa_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().nsa_oracle_max_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fwd(q, k, v, block_indices, block_counts, block_size, scale, cu_seqlens=None,
        tokens=None, threads: int = 0):
    """Oracle forward.

    q: [B, T, Hq, D], k/v: [B, T, Hkv, D] (float32 arrays holding the exact
    input values); block_indices [B, T, Hkv, S] int32; block_counts
    [B, T, Hkv] int32; cu_seqlens [N+1] int32 or None (then B sequences of
    length T).  tokens: packed token ids (b*T + t) to evaluate, or None for
    all.  Returns (out [n, Hq, D] float64, lse [n, Hq] float64).
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    bi = np.ascontiguousarray(block_indices, dtype=np.int32)
    bc = np.ascontiguousarray(block_counts, dtype=np.int32)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    S = bi.shape[-1]
    assert k.shape == (B, T, Hkv, D) and v.shape == k.shape
    assert bi.shape == (B, T, Hkv, S) and bc.shape == (B, T, Hkv)
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    nseq = 0 if cu is None else len(cu) - 1
    tk = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    n = B * T if tk is None else len(tk)
    out = np.zeros((n, Hq, D), dtype=np.float64)
    lse = np.zeros((n, Hq), dtype=np.float64)
    rc = lib.nsa_oracle_fwd(B, T, Hq, Hkv, D, S, int(block_size), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(bi), _ptr(bc), _ptr(cu), nseq, float(scale), _ptr(tk), n,
                            _ptr(out), _ptr(lse), int(threads))
    if rc != 0:
        raise ValueError("oracle: bad arguments")
    return out, lse


def expand_query_block_rows(block_indices, block_counts, T, block_size):
    """Per-token rows from rows given per query block.

    The ``block_indices`` parameter of the NSA page ("Parameters" of ``run``)
    lists key blocks for each query block, ``[batch, num_kv_heads,
    num_query_blocks, ...]``, and ``block_counts`` counts them per query
    block.  Query block i holds tokens [i * block_size, (i + 1) *
    block_size), so token t takes row t // block_size.
    [B, Hkv, NQB, S] -> [B, T, Hkv, S] and [B, Hkv, NQB] -> [B, T, Hkv].
    """
    bi = np.asarray(block_indices)
    bc = np.asarray(block_counts)
    assert bi.ndim == 4 and bc.shape == bi.shape[:3]
    qb = np.arange(T) // int(block_size)
    assert bi.shape[2] > qb[-1], "fewer query-block rows than query blocks"
    bi_t = bi[:, :, qb, :].transpose(0, 2, 1, 3)
    bc_t = bc[:, :, qb].transpose(0, 2, 1)
    return np.ascontiguousarray(bi_t, dtype=np.int32), np.ascontiguousarray(bc_t, dtype=np.int32)


def fwd_qblock(q, k, v, block_indices, block_counts, block_size, scale, tokens=None, threads: int = 0):
    """Oracle forward with rows per query block (fixed-length sequences):
    every token uses its query block's row, then the per-token definition."""
    T = np.asarray(q).shape[1]
    bi, bc = expand_query_block_rows(block_indices, block_counts, T, block_size)
    return fwd(q, k, v, bi, bc, block_size, scale, tokens=tokens, threads=threads)


def fwd_workload(w, tokens=None, threads: int = 0):
    """Oracle forward on an object carrying q, k, v, block_indices,
    block_counts, block_size, scale and cu_seqlens attributes (and
    index_layout, "token" unless it says "query_block")."""
    if getattr(w, "index_layout", "token") == "query_block":
        assert w.cu_seqlens is None
        return fwd_qblock(w.q, w.k, w.v, w.block_indices, w.block_counts, w.block_size, w.scale,
                          tokens=tokens, threads=threads)
    return fwd(w.q, w.k, w.v, w.block_indices, w.block_counts, w.block_size, w.scale,
               cu_seqlens=w.cu_seqlens, tokens=tokens, threads=threads)
