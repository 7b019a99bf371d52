"""Pure-Python brute force of the native sparse attention forward.

TEST INFRASTRUCTURE ONLY (tiny inputs, T <= ~64).  A second, independent
writing of the definition in the header of ``nsa_oracle.c``: Python sets for
the visible keys, ``math.exp`` / ``math.log`` for the softmax, no numpy
arithmetic.  Used to pin the C oracle.
"""
from __future__ import annotations

import math


def visible_keys(block_indices_row, count, S, block_size, t, seqlen):
    """Set of key positions (relative to the sequence start) that query
    position t sees: keys of the listed blocks among the first
    clamp(count, 0, S) entries, restricted to 0 <= s <= t and s < seqlen."""
    n = max(0, min(int(count), S))
    blocks = {int(b) for b in block_indices_row[:n] if int(b) >= 0}
    keys = set()
    for b in blocks:
        for s in range(b * block_size, (b + 1) * block_size):
            if s <= t and s < seqlen:
                keys.add(s)
    return keys


def fwd(q, k, v, block_indices, block_counts, block_size, scale, cu_seqlens=None, query_block_rows=False):
    """Arguments as for ``oracle.fwd`` (nested lists or numpy arrays).
    Returns (out[B*T][Hq][D], lse[B*T][Hq]) as nested Python lists of floats.

    query_block_rows: block_indices [B][Hkv][NQB][S] and block_counts
    [B][Hkv][NQB] hold one row per query block (the page's description of
    ``block_indices``): the token at position t of sequence b reads row
    [b][h][t // block_size].  Fixed-length sequences only."""
    B, T, Hq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0][0])
    S = len(block_indices[0][0][0])
    G = Hq // Hkv
    assert not (query_block_rows and cu_seqlens is not None)
    # flatten tokens
    def tok(a, x):
        return a[x // T][x % T]
    if cu_seqlens is None:
        seqs = [(b * T, T) for b in range(B)]
    else:
        seqs = [(int(cu_seqlens[i]), int(cu_seqlens[i + 1]) - int(cu_seqlens[i]))
                for i in range(len(cu_seqlens) - 1)]
    out, lse = [], []
    for (bos, L) in seqs:
        for t in range(L):
            x = bos + t
            orow_all, lrow_all = [], []
            for hq in range(Hq):
                h = hq // G
                if query_block_rows:
                    b = x // T
                    row, cnt = list(block_indices[b][h][t // block_size]), block_counts[b][h][t // block_size]
                else:
                    row, cnt = list(tok(block_indices, x)[h]), tok(block_counts, x)[h]
                keys = visible_keys(row, cnt, S, block_size, t, L)
                qv = [float(a) for a in tok(q, x)[hq]]
                if not keys:
                    orow_all.append([0.0] * D)
                    lrow_all.append(-math.inf)
                    continue
                zs = {}
                for s in sorted(keys):
                    kv = tok(k, bos + s)[h]
                    zs[s] = scale * math.fsum(qv[d] * float(kv[d]) for d in range(D))
                m = max(zs.values())
                lse_v = m + math.log(math.fsum(math.exp(z - m) for z in zs.values()))
                o = []
                for d in range(D):
                    o.append(math.fsum(math.exp(zs[s] - lse_v) * float(tok(v, bos + s)[h][d]) for s in zs))
                orow_all.append(o)
                lrow_all.append(lse_v)
            out.append(orow_all)
            lse.append(lrow_all)
    return out, lse
