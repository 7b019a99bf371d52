"""CPU fp64 oracle of the gradients of the native sparse attention forward.

TEST INFRASTRUCTURE ONLY (not imported by the product path; the GPU
counterpart is ``nsa_bwd``, which it checks).  The pages define the
forward only (ejKernel ``native_sparse_attention`` API page, module
description and "Parameters"); its gradients are those of that function.  With the token
mask of row (t, h) materialised from the indices exactly as the forward
oracle does, and for each query head hq of the group:

    P_s   = exp(scale * q.k_s - lse)              over the visible keys s
    O     = sum_s P_s v_s
    dV_s += P_s dO                                 (every (t, hq) that sees s)
    dP_s  = dO . v_s
    Delta = sum_s P_s dP_s  (= dO . O)
    dS_s  = P_s (dP_s - Delta)
    dQ    = scale * sum_s dS_s k_s
    dK_s += scale * dS_s q

(the chain rule through softmax; rows with no visible key contribute
nothing).  Plain numpy, one row at a time: for small inputs.

With ``terms=True`` the functions also return, for every gradient entry,
the sum of the magnitudes of the terms that make it up, the scale its
rounding error follows when P and dS are rounded (to bf16, relative error
2^-9 each) before being multiplied and summed:

    mdS_s = P_s (|dP_s| + |Delta| + sum_d |dO_d| |O_d|)   (|dS_s| <= mdS_s;
            the last term covers Delta formed from a rounded O)
    mQ    = |scale| sum_s mdS_s |k_s|
    mK_s += |scale| mdS_s |q|
    mV_s += P_s |dO|
"""
from __future__ import annotations

import numpy as np


def _visible(row, count, S, block_size, t):
    n = max(0, min(int(count), S))
    listed = {int(e) for e in np.asarray(row)[:n] if 0 <= int(e) <= t // block_size}
    return np.array([s for s in range(t + 1) if s // block_size in listed], dtype=np.int64)


def bwd(q, k, v, dout, block_indices, block_counts, block_size, scale, terms=False):
    """Fixed-length sequences.  q, dout [B, T, Hq, D]; k, v [B, T, Hkv, D];
    block_indices [B, T, Hkv, S]; block_counts [B, T, Hkv].  Returns
    (dq, dk, dv) in float64 with the shapes of q, k, v, followed by their
    term magnitudes (mq, mk, mv) when ``terms``."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    S = block_indices.shape[-1]
    G = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    mq, mk, mv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for t in range(T):
            for h in range(Hkv):
                keys = _visible(block_indices[b, t, h], block_counts[b, t, h], S, block_size, t)
                if len(keys) == 0:
                    continue
                K = k[b, keys, h]            # [n, D]
                V = v[b, keys, h]
                for hq in range(h * G, (h + 1) * G):
                    z = scale * (K @ q[b, t, hq])
                    p = np.exp(z - z.max())
                    p /= p.sum()
                    do = dout[b, t, hq]
                    dv[b, keys, h] += p[:, None] * do[None, :]
                    dp = V @ do
                    ds = p * (dp - p @ dp)
                    dq[b, t, hq] += scale * (ds @ K)
                    dk[b, keys, h] += scale * ds[:, None] * q[b, t, hq][None, :]
                    if terms:
                        mds = p * (np.abs(dp) + abs(p @ dp) + np.abs(do) @ np.abs(p @ V))
                        mq[b, t, hq] += abs(scale) * (mds @ np.abs(K))
                        mk[b, keys, h] += abs(scale) * mds[:, None] * np.abs(q[b, t, hq])[None, :]
                        mv[b, keys, h] += p[:, None] * np.abs(do)[None, :]
    if terms:
        return dq, dk, dv, mq, mk, mv
    return dq, dk, dv


def dq_rows(q, k, v, dout, block_indices, block_counts, block_size, scale, tokens, terms=False):
    """dq of the listed packed tokens (b * T + t) only, float64 [n, Hq, D]:
    a token's dq depends on its own row alone.  With ``terms`` also the term
    magnitudes mq of those rows."""
    q = np.asarray(q, np.float64)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    S = block_indices.shape[-1]
    G = Hq // Hkv
    out = np.zeros((len(tokens), Hq, D))
    mag = np.zeros((len(tokens), Hq, D))
    for r, x in enumerate(tokens):
        b, t = int(x) // T, int(x) % T
        for h in range(Hkv):
            keys = _visible(block_indices[b, t, h], block_counts[b, t, h], S, block_size, t)
            if len(keys) == 0:
                continue
            K = np.asarray(k[b, keys, h], np.float64)
            V = np.asarray(v[b, keys, h], np.float64)
            for hq in range(h * G, (h + 1) * G):
                z = scale * (K @ q[b, t, hq])
                p = np.exp(z - z.max())
                p /= p.sum()
                do = np.asarray(dout[b, t, hq], np.float64)
                dp = V @ do
                ds = p * (dp - p @ dp)
                out[r, hq] = scale * (ds @ K)
                if terms:
                    mds = p * (np.abs(dp) + abs(p @ dp) + np.abs(do) @ np.abs(p @ V))
                    mag[r, hq] = abs(scale) * (mds @ np.abs(K))
    if terms:
        return out, mag
    return out


def dkdv_blocks(q, k, v, dout, block_indices, block_counts, block_size, scale, blocks, terms=False):
    """dK and dV of the keys of the listed key blocks only, float64
    [n, block_size, D] each, for ``blocks`` = [(b, kv head, block), ...]
    (rows of keys past the sequence end stay zero).  A key's gradients
    gather the (token, query head) rows that see it: the rows whose kept
    entries (the first clamp(count, 0, S), 0 <= entry <= own block) hold its
    block; each such row contributes exactly its terms in ``bwd``.  With
    ``terms`` also their term magnitudes (mk, mv)."""
    B, T, Hq, D = np.shape(q)
    Hkv = np.shape(k)[2]
    S = block_indices.shape[-1]
    G = Hq // Hkv
    bs = block_size
    dk = np.zeros((len(blocks), bs, D))
    dv = np.zeros((len(blocks), bs, D))
    mk = np.zeros((len(blocks), bs, D))
    mv = np.zeros((len(blocks), bs, D))
    for r, (b, h, j) in enumerate(blocks):
        lo = j * bs
        for t in range(lo, T):
            n = max(0, min(int(block_counts[b, t, h]), S))
            listed = sorted({int(e) for e in block_indices[b, t, h, :n] if 0 <= int(e) <= t // bs})
            if j not in listed:
                continue
            keys = np.concatenate([np.arange(e * bs, min((e + 1) * bs, t + 1)) for e in listed])
            K = np.asarray(k[b, keys, h], np.float64)
            V = np.asarray(v[b, keys, h], np.float64)
            Qg = np.asarray(q[b, t, h * G:(h + 1) * G], np.float64)        # [G, D]
            dO = np.asarray(dout[b, t, h * G:(h + 1) * G], np.float64)
            z = scale * (Qg @ K.T)                                         # [G, n]
            p = np.exp(z - z.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dp = dO @ V.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            sel = (keys // bs) == j
            at = keys[sel] - lo
            dv[r, at] += p[:, sel].T @ dO
            dk[r, at] += scale * (ds[:, sel].T @ Qg)
            if terms:
                mds = p * (np.abs(dp) + np.abs((p * dp).sum(axis=1, keepdims=True))
                           + (np.abs(dO) * np.abs(p @ V)).sum(axis=1, keepdims=True))
                mv[r, at] += p[:, sel].T @ np.abs(dO)
                mk[r, at] += abs(scale) * (mds[:, sel].T @ np.abs(Qg))
    if terms:
        return dk, dv, mk, mv
    return dk, dv


def dkdv_head(q, k, v, dout, block_indices, block_counts, block_size, scale, b, h):
    """dK, dV of every key of kv head h of sequence b, and their term
    magnitudes, float64 [T, D] each: every token's row is formed once (the
    group's heads together) and its terms added to the keys it sees, as in
    ``bwd``.  For checking whole heads of large inputs."""
    B, T, Hq, D = np.shape(q)
    Hkv = np.shape(k)[2]
    S = block_indices.shape[-1]
    G = Hq // Hkv
    bs = block_size
    dk, dv, mk, mv = (np.zeros((T, D)) for _ in range(4))
    kh = np.asarray(k[b, :, h], np.float64)
    vh = np.asarray(v[b, :, h], np.float64)
    for t in range(T):
        keys = _visible(block_indices[b, t, h], block_counts[b, t, h], S, bs, t)
        if len(keys) == 0:
            continue
        K, V = kh[keys], vh[keys]
        Qg = np.asarray(q[b, t, h * G:(h + 1) * G], np.float64)
        dO = np.asarray(dout[b, t, h * G:(h + 1) * G], np.float64)
        z = scale * (Qg @ K.T)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dp = dO @ V.T
        delta = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - delta)
        dv[keys] += p.T @ dO
        dk[keys] += scale * (ds.T @ Qg)
        mds = p * (np.abs(dp) + np.abs(delta) + (np.abs(dO) * np.abs(p @ V)).sum(axis=1, keepdims=True))
        mv[keys] += p.T @ np.abs(dO)
        mk[keys] += abs(scale) * (mds.T @ np.abs(Qg))
    return dk, dv, mk, mv
