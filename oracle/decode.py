"""CPU fp64 oracle of the decode step (one query token per sequence).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the benchmark's
CPU-baseline leg, never by the product path.  It shares no code with the HIP
library.

What it computes: the native sparse attention of the NSA page (ejKernel
``native_sparse_attention`` API page, module description and "Parameters")
for the newest token of each sequence, whose keys are the first ``len_b``
rows of a per-sequence cache (the ragged key range of the ragged-decode
page's ``ragged_decode_mqa_xla``: query ``[B, Hq, D]``, cache
``[B, S, Hkv, D]``).  The query sits at position t = len_b - 1.  Following
the token-mask form of ``create_attention_mask`` on the ragged-decode page,
the row's listed blocks are turned into a boolean mask over the keys
0 .. len_b - 1 (key s visible iff s <= t and s // block_size is one of the
first clamp(count, 0, S) entries with 0 <= entry), then dense masked softmax
attention runs in float64.  An empty mask gives out = 0, lse = -inf.
"""
from __future__ import annotations

import numpy as np


def key_mask(row, count, S, block_size, length):
    """Boolean mask over keys 0 .. length - 1 for a query at t = length - 1."""
    n = max(0, min(int(count), S))
    listed = np.zeros(max(1, (length + block_size - 1) // block_size), dtype=bool)
    for e in np.asarray(row)[:n]:
        e = int(e)
        if 0 <= e < len(listed):
            listed[e] = True
    s = np.arange(length)
    return listed[s // block_size] & (s <= length - 1)


def decode(q, k, v, seq_lens, block_indices, block_counts, block_size, scale, sequences=None):
    """q [B, Hq, D]; k, v [B, Smax, Hkv, D] (exact input values); seq_lens [B];
    block_indices [B, Hkv, S]; block_counts [B, Hkv].  sequences: the b to
    evaluate (None = all).  Returns (out [n, Hq, D], lse [n, Hq]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Smax, Hkv = k.shape[1], k.shape[2]
    S = block_indices.shape[-1]
    G = Hq // Hkv
    bs_list = range(B) if sequences is None else [int(b) for b in sequences]
    out = np.zeros((len(bs_list), Hq, D), dtype=np.float64)
    lse = np.full((len(bs_list), Hq), -np.inf, dtype=np.float64)
    for r, b in enumerate(bs_list):
        length = max(0, min(int(seq_lens[b]), Smax))
        if length == 0:
            continue
        for h in range(Hkv):
            m = key_mask(block_indices[b, h], block_counts[b, h], S, block_size, length)
            if not m.any():
                continue
            kk = np.asarray(k[b, :length, h], dtype=np.float64)[m]      # [n_keys, D]
            vv = np.asarray(v[b, :length, h], dtype=np.float64)[m]
            qq = q[b, h * G:(h + 1) * G]                                 # [G, D]
            z = scale * (qq @ kk.T)                                      # [G, n_keys]
            zmax = z.max(axis=1, keepdims=True)
            e = np.exp(z - zmax)
            den = e.sum(axis=1, keepdims=True)
            lse[r, h * G:(h + 1) * G] = (zmax + np.log(den))[:, 0]
            out[r, h * G:(h + 1) * G] = (e / den) @ vv
    return out, lse


def decode_workload(w, sequences=None):
    return decode(w.q, w.k, w.v, w.seq_lens, w.block_indices, w.block_counts, w.block_size, w.scale,
                  sequences=sequences)
