"""Pins of the CPU fp64 oracle against things other than itself.

Each test fixes a part of the definition a plausible mistake would break:
 - dense causal indices == torch scaled_dot_product_attention (scale, sign,
   operand order, inclusive diagonal, GQA head mapping, softmax);
 - pure-Python brute force on tiny sparse inputs (index -> token set,
   counts truncation, -1 padding, varlen offsets);
 - closed forms at t = 0 and q = 0 (lse in natural-log units, |M_t|);
 - the lse gradient identity d lse / d q = scale * softmax-weighted keys;
 - v -> a v + b equivariance (rows of P sum to one);
 - invariance to entry order, to entries past the count and to repeats;
 - the block-level causal example of the block-sparse mask page.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import nsa_inputs as ni
import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small(pattern, counts_mode="full", seqlens=(40,), Hq=4, Hkv=2, D=8, bs=8, S=4, seed=7,
          varlen=False, dtype="f32"):
    return ni.make_workload("t", dtype, list(seqlens), Hq, Hkv, D, bs, S, pattern, counts_mode, seed,
                            varlen=varlen)


def run(w, **kw):
    return oracle.fwd(w.q, w.k, w.v, w.block_indices, w.block_counts, w.block_size, w.scale,
                      cu_seqlens=w.cu_seqlens, **kw)


# --------------------------------------------------------------------------
# dense special case == library attention
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,Hq,Hkv,D,bs", [(96, 4, 2, 16, 16), (90, 4, 4, 8, 16), (70, 8, 1, 32, 32),
                                           (33, 2, 2, 8, 8)])
def test_dense_indices_equal_causal_sdpa(T, Hq, Hkv, D, bs):
    nb = (T + bs - 1) // bs
    w = ni.make_workload("dense", "f32", [T, T], Hq, Hkv, D, bs, nb, "dense", "full", seed=3)
    out, lse = run(w)
    q = torch.from_numpy(w.q).double().permute(0, 2, 1, 3)   # B H T D
    k = torch.from_numpy(w.k).double().permute(0, 2, 1, 3)
    v = torch.from_numpy(w.v).double().permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.scale,
                                                           enable_gqa=True)
    ref = ref.permute(0, 2, 1, 3).reshape(2 * T, Hq, D).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # lse against torch.logsumexp of the library's own score matrix
    G = Hq // Hkv
    kk = k.repeat_interleave(G, dim=1)
    sc = torch.matmul(q, kk.transpose(-1, -2)) * w.scale
    causal = torch.ones(T, T, dtype=torch.bool).tril()
    sc = sc.masked_fill(~causal, -math.inf)
    ref_lse = torch.logsumexp(sc, dim=-1).permute(0, 2, 1).reshape(2 * T, Hq).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# brute force on tiny inputs
# --------------------------------------------------------------------------
CASES = [
    dict(pattern="shuffled", counts_mode="uniform", seqlens=(40,), Hq=4, Hkv=1, D=8, bs=8, S=4),
    dict(pattern="local_random", counts_mode="full", seqlens=(48, 48), Hq=4, Hkv=2, D=8, bs=4, S=6),
    dict(pattern="local_random", counts_mode="uniform", seqlens=(37,), Hq=2, Hkv=2, D=4, bs=4, S=6),
    dict(pattern="sink_local_random", counts_mode="full", seqlens=(64,), Hq=8, Hkv=2, D=8, bs=4, S=8),
    dict(pattern="local_random", counts_mode="uniform", seqlens=(13, 30, 5), Hq=4, Hkv=2, D=8, bs=4, S=6,
         varlen=True),
]


@pytest.mark.parametrize("case", CASES)
def test_oracle_matches_brute_force(case):
    w = small(**case)
    out, lse = run(w)
    bout, blse = brute.fwd(w.q, w.k, w.v, w.block_indices, w.block_counts, w.block_size, w.scale,
                           cu_seqlens=w.cu_seqlens)
    bout, blse = np.array(bout), np.array(blse)
    assert np.array_equal(np.isinf(lse), np.isinf(blse))
    np.testing.assert_allclose(out, bout, rtol=0, atol=1e-12)
    fin = np.isfinite(blse)
    np.testing.assert_allclose(lse[fin], blse[fin], rtol=0, atol=1e-12)


def test_brute_force_with_hostile_entries():
    """-1 padding inside the count, blocks beyond own, blocks past the end,
    counts above S and below zero, repeated entries."""
    w = small("local_random", "full", seqlens=(32,), Hq=2, Hkv=1, D=4, bs=4, S=5, seed=11)
    rng = np.random.default_rng(0)
    bi = rng.integers(-3, 12, size=w.block_indices.shape).astype(np.int32)
    bc = rng.integers(-2, 8, size=w.block_counts.shape).astype(np.int32)
    w.block_indices, w.block_counts = bi, bc
    out, lse = run(w)
    bout, blse = brute.fwd(w.q, w.k, w.v, bi, bc, w.block_size, w.scale)
    bout, blse = np.array(bout), np.array(blse)
    assert np.array_equal(np.isinf(lse), np.isinf(blse))
    np.testing.assert_allclose(out, bout, rtol=0, atol=1e-12)
    fin = np.isfinite(blse)
    np.testing.assert_allclose(lse[fin], blse[fin], rtol=0, atol=1e-12)
    assert (~fin).any() and fin.any()


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def test_first_token_closed_form():
    w = small("local_random", "full", seqlens=(24, 24), Hq=4, Hkv=2, D=8, bs=8, S=3)
    out, lse = run(w)
    G = w.G
    for b in range(2):
        x = b * w.T
        for hq in range(w.Hq):
            h = hq // G
            assert np.array_equal(out[x, hq], w.v[b, 0, h].astype(np.float64))
            exp_lse = w.scale * float(np.dot(w.q[b, 0, hq].astype(np.float64), w.k[b, 0, h].astype(np.float64)))
            assert abs(lse[x, hq] - exp_lse) < 1e-12


@pytest.mark.parametrize("pattern,counts_mode", [("shuffled", "uniform"), ("sink_local_random", "full"),
                                                 ("local_random", "uniform")])
def test_zero_query_counts_and_mean(pattern, counts_mode):
    w = small(pattern, counts_mode, seqlens=(64,), Hq=4, Hkv=2, D=8, bs=8, S=4)
    w.q[:] = 0.0
    out, lse = run(w)
    G = w.G
    for t in range(w.T):
        for hq in range(w.Hq):
            h = hq // G
            keys = brute.visible_keys(list(w.block_indices[0, t, h]), w.block_counts[0, t, h], w.S,
                                      w.block_size, t, w.T)
            assert abs(lse[t, hq] - math.log(len(keys))) < 1e-12
            mean = np.mean([w.v[0, s, h].astype(np.float64) for s in sorted(keys)], axis=0)
            np.testing.assert_allclose(out[t, hq], mean, rtol=0, atol=1e-12)


def test_lse_gradient_identity():
    """d lse / d q[d] = scale * sum_s p_s k_s[d]: the oracle's output with v := k."""
    w = small("sink_local_random", "full", seqlens=(48,), Hq=2, Hkv=1, D=6, bs=4, S=6)
    wk = small("sink_local_random", "full", seqlens=(48,), Hq=2, Hkv=1, D=6, bs=4, S=6)
    wk.v = wk.k.copy()
    outk, _ = run(wk)
    eps = 1e-4
    for t in (5, 17, 47):
        for d in range(w.D):
            wp = small("sink_local_random", "full", seqlens=(48,), Hq=2, Hkv=1, D=6, bs=4, S=6)
            wm = small("sink_local_random", "full", seqlens=(48,), Hq=2, Hkv=1, D=6, bs=4, S=6)
            # q +/- eps e_d, with the step measured on the float32 values actually used
            wp.q[0, t, 0, d] += np.float32(eps)
            wm.q[0, t, 0, d] -= np.float32(eps)
            dq = float(wp.q[0, t, 0, d]) - float(wm.q[0, t, 0, d])
            _, lp = run(wp)
            _, lm = run(wm)
            fd = (lp[t, 0] - lm[t, 0]) / dq
            assert abs(fd - w.scale * outk[t, 0, d]) < 1e-6


def test_affine_equivariance_in_v():
    w = small("sink_local_random", "full", seqlens=(64,), Hq=4, Hkv=2, D=8, bs=8, S=4)
    w.v = (np.round(w.v * 4) / 4).astype(np.float32)   # dyadic values: 2 v + 0.5 is exact in float32
    out, _ = run(w)
    w.v = (np.float32(2.0) * w.v + np.float32(0.5)).astype(np.float32)
    out2, _ = run(w)
    np.testing.assert_allclose(out2, 2.0 * out + 0.5, rtol=0, atol=1e-12)
    w.v[:] = 1.0
    ones, _ = run(w)
    np.testing.assert_allclose(ones, 1.0, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# invariances of the index contract
# --------------------------------------------------------------------------
def test_entry_order_garbage_and_repeats_invariance():
    w = small("local_random", "uniform", seqlens=(64,), Hq=4, Hkv=2, D=8, bs=8, S=6)
    out, lse = run(w)
    rng = np.random.default_rng(5)
    bi = w.block_indices.copy()
    n = np.clip(w.block_counts, 0, w.S)
    for t in range(w.T):
        for h in range(w.Hkv):
            k = int(n[0, t, h])
            bi[0, t, h, :k] = rng.permutation(bi[0, t, h, :k])
            bi[0, t, h, k:] = rng.integers(-5, 50, size=w.S - k)
    w2 = small("local_random", "uniform", seqlens=(64,), Hq=4, Hkv=2, D=8, bs=8, S=6)
    w2.block_indices = bi
    out2, lse2 = run(w2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    # repeating a listed block inside the count changes nothing (set semantics)
    bi3 = w.block_indices.copy()
    bc3 = w.block_counts.copy()
    for t in range(w.T):
        for h in range(w.Hkv):
            k = int(n[0, t, h])
            if k < w.S:
                bi3[0, t, h, k] = bi3[0, t, h, 0]
                bc3[0, t, h] = k + 1
    w3 = small("local_random", "uniform", seqlens=(64,), Hq=4, Hkv=2, D=8, bs=8, S=6)
    w3.block_indices, w3.block_counts = bi3, bc3
    out3, lse3 = run(w3)
    assert np.array_equal(out, out3) and np.array_equal(lse, lse3)


def test_empty_rows():
    w = small("local_random", "full", seqlens=(32,), Hq=2, Hkv=1, D=4, bs=8, S=4)
    w.block_counts[0, 3, 0] = 0
    w.block_indices[0, 9, 0, :] = -1
    w.block_indices[0, 10, 0, :] = 3          # only a future block (own = 1)
    out, lse = run(w)
    for t in (3, 9, 10):
        assert np.all(out[t] == 0.0) and np.all(np.isneginf(lse[t]))
    assert np.all(np.isfinite(np.delete(lse, [3, 9, 10], axis=0)))


def test_varlen_equals_per_sequence():
    lens = [13, 30, 5, 17]
    w = small("local_random", "uniform", seqlens=lens, Hq=4, Hkv=2, D=8, bs=4, S=6, varlen=True)
    out, lse = run(w)
    cu = w.cu_seqlens
    for i, L in enumerate(lens):
        a, b = cu[i], cu[i + 1]
        o1, l1 = oracle.fwd(w.q[:, a:b], w.k[:, a:b], w.v[:, a:b], w.block_indices[:, a:b],
                            w.block_counts[:, a:b], w.block_size, w.scale)
        assert np.array_equal(o1, out[a:b]) and np.array_equal(l1, lse[a:b])


def test_token_subset_matches_full_run():
    w = small("sink_local_random", "full", seqlens=(64, 64), Hq=4, Hkv=2, D=8, bs=8, S=4)
    out, lse = run(w)
    toks = np.array([0, 5, 63, 64, 100, 127])
    o2, l2 = run(w, tokens=toks)
    assert np.array_equal(o2, out[toks]) and np.array_equal(l2, lse[toks])


def test_block_level_causal_example():
    """Page example: causal mask over 4 blocks, query block i attends [0, i+1)."""
    g = json.load(open(os.path.join(GOLDEN, "causal_4_blocks.json")))
    nb, bs = g["num_blocks"], 4
    T = nb * bs
    w = ni.make_workload("ex", "f32", [T], 1, 1, nb, bs, nb, "dense", "full", seed=1)
    w.q[:] = 0.0
    # v[s, d] = 1 iff key s is in block d: out[t, d] > 0 iff block d is visible to t
    w.v[:] = 0.0
    for s in range(T):
        w.v[0, s, 0, s // bs] = 1.0
    out, _ = run(w)
    for i, (lo, hi) in enumerate(g["attend_bounds"]):
        seen = set()
        for t in range(i * bs, (i + 1) * bs):
            seen |= {d for d in range(nb) if out[t, 0, d] > 0}
        assert seen == set(range(lo, hi))


# --------------------------------------------------------------------------
# rows per query block (the page's description of block_indices)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("B,T,Hq,Hkv,D,bs,S,pattern,counts_mode", [
    (2, 37, 4, 2, 8, 8, 4, "sink_local_random", "uniform"),
    (1, 40, 4, 1, 8, 4, 6, "local_random", "full"),
    (2, 24, 2, 2, 4, 8, 3, "shuffled", "uniform"),
])
def test_query_block_rows_match_brute_force(B, T, Hq, Hkv, D, bs, S, pattern, counts_mode):
    """The brute force reads the row [b][h][t // bs] itself; the oracle expands
    the rows to tokens and runs the per-token definition."""
    w = ni.make_qblock_workload("qb", "f32", B, T, Hq, Hkv, D, bs, S, pattern, counts_mode, seed=5)
    assert w.block_indices.shape == (B, Hkv, (T + bs - 1) // bs, S)
    out, lse = oracle.fwd_workload(w)
    bout, blse = brute.fwd(w.q, w.k, w.v, w.block_indices, w.block_counts, bs, w.scale,
                           query_block_rows=True)
    bout, blse = np.array(bout), np.array(blse)
    assert np.array_equal(np.isinf(lse), np.isinf(blse))
    np.testing.assert_allclose(out, bout, rtol=0, atol=1e-12)
    fin = np.isfinite(blse)
    np.testing.assert_allclose(lse[fin], blse[fin], rtol=0, atol=1e-12)


def test_query_block_rows_hostile_entries():
    """Negative entries, blocks past the query block or the sequence, repeats
    and counts outside [0, S], all in query-block rows."""
    w = ni.make_qblock_workload("qb", "f32", 2, 29, 2, 1, 4, 4, 5, "local_random", "full", seed=9)
    rng = np.random.default_rng(1)
    w.block_indices = rng.integers(-3, 10, size=w.block_indices.shape).astype(np.int32)
    w.block_counts = rng.integers(-2, 8, size=w.block_counts.shape).astype(np.int32)
    out, lse = oracle.fwd_workload(w)
    bout, blse = brute.fwd(w.q, w.k, w.v, w.block_indices, w.block_counts, 4, w.scale,
                           query_block_rows=True)
    bout, blse = np.array(bout), np.array(blse)
    assert np.array_equal(np.isinf(lse), np.isinf(blse))
    np.testing.assert_allclose(out, bout, rtol=0, atol=1e-12)
    fin = np.isfinite(blse)
    np.testing.assert_allclose(lse[fin], blse[fin], rtol=0, atol=1e-12)
    assert (~fin).any() and fin.any()


def test_query_block_dense_rows_equal_causal_sdpa():
    """Every query block listing all blocks up to itself is dense causal
    attention (the library routine, not the oracle's formula)."""
    B, T, Hq, Hkv, D, bs = 2, 50, 4, 2, 16, 8
    nqb = (T + bs - 1) // bs
    w = ni.make_qblock_workload("qbd", "f32", B, T, Hq, Hkv, D, bs, nqb, "dense", "full", seed=4)
    assert (w.block_counts == np.arange(1, nqb + 1)[None, None, :]).all()
    out, _ = oracle.fwd_workload(w)
    q = torch.from_numpy(w.q).double().permute(0, 2, 1, 3)
    k = torch.from_numpy(w.k).double().permute(0, 2, 1, 3)
    v = torch.from_numpy(w.v).double().permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.scale,
                                                           enable_gqa=True)
    np.testing.assert_allclose(out, ref.permute(0, 2, 1, 3).reshape(B * T, Hq, D).numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# decode step (one query token per sequence against its cache)
# --------------------------------------------------------------------------
from oracle import decode as odec   # noqa: E402


def _tiny_decode(seed=2, B=4, Smax=40, Hq=4, Hkv=2, D=8, bs=8, S=4, pattern="sink_local_random",
                 counts="uniform", lens=(1, 40)):
    w = ni.make_decode_workload("td", B, Smax, lens[0], lens[1], Hq, Hkv, D, bs, S, pattern, counts, seed)
    for a in ("q", "k", "v"):   # fp32 values for the fp64 comparisons
        setattr(w, a, getattr(w, a).astype(np.float32))
    return w


def test_decode_matches_per_token_oracle_at_the_last_token():
    """The decode oracle equals the C per-token oracle evaluated at position
    len - 1 of each sequence (cache rows as the keys, the decode row as that
    token's row)."""
    w = _tiny_decode(B=5, lens=(1, 40))
    w.seq_lens[0] = 1
    out, lse = odec.decode_workload(w)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        q = np.zeros((1, L, w.Hq, w.D), np.float32)
        q[0, L - 1] = w.q[b]
        bi = np.full((1, L, w.Hkv, w.S), -1, np.int32)
        bc = np.zeros((1, L, w.Hkv), np.int32)
        bi[0, L - 1] = w.block_indices[b]
        bc[0, L - 1] = w.block_counts[b]
        ro, rl = oracle.fwd(q, w.k[b:b + 1, :L], w.v[b:b + 1, :L], bi, bc, w.block_size, w.scale,
                            tokens=np.array([L - 1]))
        np.testing.assert_allclose(out[b], ro[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], rl[0], rtol=0, atol=1e-12)


def test_decode_brute_force_with_hostile_entries():
    """Python sets and math.fsum; negative, repeated and out-of-range entries,
    counts outside [0, S], a zero-length sequence."""
    w = _tiny_decode(seed=4, B=4, Smax=30, Hq=2, Hkv=1, D=4, bs=4, S=6)
    rng = np.random.default_rng(3)
    w.block_indices = rng.integers(-2, 9, size=w.block_indices.shape).astype(np.int32)
    w.block_counts = rng.integers(-1, 8, size=w.block_counts.shape).astype(np.int32)
    w.seq_lens[1] = 0
    out, lse = odec.decode_workload(w)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        keys = brute.visible_keys(list(w.block_indices[b, 0]), w.block_counts[b, 0], w.S, w.block_size,
                                  L - 1, L) if L > 0 else set()
        for hq in range(w.Hq):
            if not keys:
                assert lse[b, hq] == -math.inf and np.all(out[b, hq] == 0)
                continue
            z = {s: w.scale * math.fsum(float(w.q[b, hq, d]) * float(w.k[b, s, 0, d]) for d in range(w.D))
                 for s in keys}
            m = max(z.values())
            l = m + math.log(math.fsum(math.exp(x - m) for x in z.values()))
            assert abs(lse[b, hq] - l) < 1e-12
            for d in range(w.D):
                o = math.fsum(math.exp(z[s] - l) * float(w.v[b, s, 0, d]) for s in keys)
                assert abs(out[b, hq, d] - o) < 1e-12
    assert np.isneginf(lse).any() and np.isfinite(lse).any()


def test_decode_dense_selection_equals_sdpa():
    """All blocks up to the query's own: plain attention of the query over
    keys 0 .. len - 1 (library routine)."""
    w = _tiny_decode(seed=6, B=3, Smax=45, Hq=4, Hkv=2, D=16, bs=8, S=6, pattern="dense", counts="full",
                     lens=(20, 45))
    out, _ = odec.decode_workload(w)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        q = torch.from_numpy(w.q[b]).double()[:, None, None, :]                    # [Hq, 1, 1, D]
        k = torch.from_numpy(w.k[b, :L]).double().permute(1, 0, 2).repeat_interleave(w.G, 0)[:, None]
        v = torch.from_numpy(w.v[b, :L]).double().permute(1, 0, 2).repeat_interleave(w.G, 0)[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=w.scale)[:, 0, 0]
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=0, atol=1e-12)


def test_decode_zero_query_counts_and_mean():
    w = _tiny_decode(seed=8, B=4, Smax=50, lens=(5, 50))
    w.q[:] = 0
    out, lse = odec.decode_workload(w)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        for h in range(w.Hkv):
            m = odec.key_mask(w.block_indices[b, h], w.block_counts[b, h], w.S, w.block_size, L)
            n = int(m.sum())
            for hq in range(h * w.G, (h + 1) * w.G):
                assert abs(lse[b, hq] - math.log(n)) < 1e-12
                np.testing.assert_allclose(out[b, hq], w.v[b, :L, h][m].astype(np.float64).mean(0), atol=1e-12)


# --------------------------------------------------------------------------
# gradients (groundwork of the backward pass; CPU only)
# --------------------------------------------------------------------------
from oracle import backward as obwd   # noqa: E402


def _loss(w, q, k, v, dout):
    out, _ = oracle.fwd(q, k, v, w.block_indices, w.block_counts, w.block_size, w.scale)
    return float(np.sum(out.reshape(dout.shape) * dout))


def test_gradients_match_central_differences_of_the_forward():
    """Directional derivatives of L = <dO, out> through the (pinned) forward
    oracle, along random directions in q, k and v, against the gradients."""
    w = ni.make_workload("g", "f32", [24, 24], 4, 2, 8, 4, 4, "sink_local_random", "uniform", seed=12)
    rng = np.random.default_rng(0)
    dout = rng.standard_normal(w.q.shape)
    dq, dk, dv = obwd.bwd(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size, w.scale)
    eps = 1e-3
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        for trial in range(2):
            u = rng.standard_normal(grad.shape)
            x = getattr(w, name).astype(np.float64)
            args = {"q": w.q.astype(np.float64), "k": w.k.astype(np.float64), "v": w.v.astype(np.float64)}
            args[name] = x + eps * u
            lp = _loss(w, args["q"].astype(np.float32), args["k"].astype(np.float32), args["v"].astype(np.float32), dout)
            args[name] = x - eps * u
            lm = _loss(w, args["q"].astype(np.float32), args["k"].astype(np.float32), args["v"].astype(np.float32), dout)
            fd = (lp - lm) / (2 * eps)
            an = float(np.sum(grad * u))
            # the forward takes float32 inputs: the step's rounding sets the tolerance
            assert abs(fd - an) <= 2e-3 * max(1.0, abs(an)), (name, fd, an)


def test_gradients_dense_rows_equal_autograd_sdpa():
    """Dense causal rows: the library's autograd through SDPA in fp64."""
    T, Hq, Hkv, D, bs = 20, 4, 2, 8, 4
    nb = (T + bs - 1) // bs
    w = ni.make_workload("gd", "f32", [T], Hq, Hkv, D, bs, nb, "dense", "full", seed=13)
    rng = np.random.default_rng(1)
    dout = rng.standard_normal(w.q.shape)
    dq, dk, dv = obwd.bwd(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size, w.scale)
    q = torch.from_numpy(w.q).double().permute(0, 2, 1, 3).requires_grad_()
    k = torch.from_numpy(w.k).double().permute(0, 2, 1, 3).requires_grad_()
    v = torch.from_numpy(w.v).double().permute(0, 2, 1, 3).requires_grad_()
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.scale, enable_gqa=True)
    o.backward(torch.from_numpy(dout).permute(0, 2, 1, 3))
    np.testing.assert_allclose(dq, q.grad.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, k.grad.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, v.grad.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-11)


def test_gradients_of_empty_rows_and_unlisted_keys_vanish():
    w = ni.make_workload("ge", "f32", [16], 2, 1, 4, 4, 3, "local_random", "full", seed=14)
    w.block_counts[0, :8] = 0                      # tokens 0..7 see nothing
    w.block_indices[0, 8:, 0, :] = [1, 3, -1]      # tokens 8.. see blocks 1 and 3 only
    w.block_counts[0, 8:] = 3
    dout = np.ones(w.q.shape)
    dq, dk, dv = obwd.bwd(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size, w.scale)
    assert np.all(dq[0, :8] == 0)
    assert np.all(dk[0, 0:4] == 0) and np.all(dv[0, 0:4] == 0)     # block 0 never listed
    assert np.all(dk[0, 8:12] == 0) and np.all(dv[0, 8:12] == 0)   # block 2 never listed
    assert np.any(dv[0, 4:8] != 0) and np.any(dv[0, 12:16] != 0)


def test_gradient_rows_match_full_gradients():
    w = ni.make_workload("gr", "f32", [30, 30], 4, 2, 8, 4, 4, "sink_local_random", "uniform", seed=15)
    dout = np.random.default_rng(2).standard_normal(w.q.shape)
    dq, _, _ = obwd.bwd(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size, w.scale)
    rows = np.array([0, 7, 29, 30, 45, 59])
    got = obwd.dq_rows(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size, w.scale, rows)
    np.testing.assert_allclose(got, dq.reshape(-1, w.Hq, w.D)[rows], rtol=0, atol=1e-13)


def test_block_gradients_match_full_gradients():
    """The per-block dK/dV against the full gradients, with repeated,
    negative and out-of-range entries, counts outside [0, S] and a ragged
    last block (T = 30, block size 4)."""
    w = ni.make_workload("gb", "f32", [30, 30], 4, 2, 8, 4, 5, "sink_local_random", "uniform", seed=16)
    rng = np.random.default_rng(4)
    w.block_indices = rng.integers(-2, 9, size=w.block_indices.shape).astype(np.int32)
    w.block_counts = rng.integers(-1, 7, size=w.block_counts.shape).astype(np.int32)
    dout = rng.standard_normal(w.q.shape)
    _, dk, dv = obwd.bwd(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size, w.scale)
    blocks = [(0, 0, 0), (0, 1, 3), (1, 0, 5), (1, 1, 7), (0, 1, 7)]
    gk, gv = obwd.dkdv_blocks(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size, w.scale, blocks)
    for r, (b, h, j) in enumerate(blocks):
        n = min(4, 30 - 4 * j)
        np.testing.assert_allclose(gk[r, :n], dk[b, 4 * j:4 * j + n, h], rtol=0, atol=1e-12)
        np.testing.assert_allclose(gv[r, :n], dv[b, 4 * j:4 * j + n, h], rtol=0, atol=1e-12)
        assert np.all(gk[r, n:] == 0) and np.all(gv[r, n:] == 0)
    assert sum(bool(np.any(gv[r] != 0)) for r in range(len(blocks))) >= 3


# ---------------------------------------------------------------------------
# term magnitudes of the gradients (the per-entry tolerance scale of the GPU
# backward test)


def _grad_case(seed=3, G=4, D=64, bs=32, T=130):
    w = ni.make_workload("tm", "bf16", [T], 2 * G, 2, D, bs, 5, "sink_local_random", "uniform", seed=seed)
    x = ni.normal(seed + 50, 9, w.q.size).reshape(w.q.shape)
    dout = ni.bf16_bits_to_f32(ni.to_bf16_bits(x)).reshape(x.shape)
    return w, dout


def test_term_magnitudes_bound_the_gradients():
    """sum |terms| >= |sum terms| entry by entry (zero magnitude only with a
    zero gradient); asking for the magnitudes leaves the gradients unchanged."""
    w, dout = _grad_case()
    g = obwd.bwd(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size, w.scale)
    r = obwd.bwd(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size, w.scale, terms=True)
    for a, b in zip(g, r[:3]):
        assert np.array_equal(a, b)
    for grad, mag in zip(r[:3], r[3:]):
        assert np.all(mag >= np.abs(grad) * (1 - 1e-12))
        assert np.all(grad[mag == 0] == 0)
        assert np.any(mag > 0)


def test_per_head_dkdv_matches_full_backward():
    w, dout = _grad_case(seed=8, G=3, D=64, bs=32, T=97)
    _, dk, dv, _, mk, mv = obwd.bwd(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size, w.scale,
                                    terms=True)
    for h in range(w.Hkv):
        hk, hv, hmk, hmv = obwd.dkdv_head(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size,
                                          w.scale, 0, h)
        np.testing.assert_allclose(hk, dk[0, :, h], rtol=0, atol=1e-12)
        np.testing.assert_allclose(hv, dv[0, :, h], rtol=0, atol=1e-12)
        np.testing.assert_allclose(hmk, mk[0, :, h], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(hmv, mv[0, :, h], rtol=1e-12, atol=1e-12)


def _bf16(x):
    return ni.bf16_bits_to_f32(ni.to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64).reshape(np.shape(x))


def test_bf16_rounding_of_p_ds_and_o_stays_inside_the_term_bound():
    """The backward kernels round P (for dV), dS (for dQ, dK) and read O as
    bf16; recomputing the gradients that way here, each entry's error stays
    within 2^-8 of its term magnitude (the GPU test allows 2^-7)."""
    w, dout = _grad_case(seed=12, G=4, D=64, bs=32, T=160)
    q, k, v = (np.asarray(a, np.float64) for a in (w.q, w.k, w.v))
    B, T, Hq, D = q.shape
    G = Hq // w.Hkv
    rq, rk, rv, mq, mk, mv = obwd.bwd(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size,
                                      w.scale, terms=True)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for t in range(T):
        for h in range(w.Hkv):
            n = max(0, min(int(w.block_counts[0, t, h]), w.S))
            listed = {int(e) for e in w.block_indices[0, t, h, :n] if 0 <= int(e) <= t // w.block_size}
            keys = np.array([s for s in range(t + 1) if s // w.block_size in listed], dtype=np.int64)
            if len(keys) == 0:
                continue
            K, V = k[0, keys, h], v[0, keys, h]
            for hq in range(h * G, (h + 1) * G):
                z = w.scale * (K @ q[0, t, hq])
                p = np.exp(z - z.max())
                p /= p.sum()
                do = np.asarray(dout[0, t, hq], np.float64)
                o_b = _bf16(p @ V)                       # the forward's rounded output
                dp = V @ do
                ds = _bf16(p * (dp - do @ o_b))          # Delta from rounded O, dS rounded
                dv[0, keys, h] += _bf16(p)[:, None] * do[None, :]
                dq[0, t, hq] += w.scale * (ds @ K)
                dk[0, keys, h] += w.scale * ds[:, None] * q[0, t, hq][None, :]
    for got, ref, mag in ((dq, rq, mq), (dk, rk, mk), (dv, rv, mv)):
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * mag + 1e-12)
