"""Seeded generator: counter-based RNG pins, determinism and the structure
of every named workload."""
import json
import os

import numpy as np
import pytest

import nsa_inputs as ni

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_reference_outputs():
    g = json.load(open(os.path.join(GOLDEN, "splitmix64_seed0.json")))
    got = ["%016x" % int(x) for x in ni.hash_u64(0, 0, np.arange(3))]
    assert got == g["outputs_hex"]


def test_normals_are_standard():
    z = ni.normal(1, 0, 1 << 20).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.var() - 1) < 5e-3
    assert abs(np.mean(z ** 3)) < 1e-2 and abs(np.mean(z ** 4) - 3) < 3e-2
    # chunking and threading do not change the bytes
    a = ni.normal(9, 2, 100003, chunk=4096)
    b = ni.normal(9, 2, 100003, chunk=1 << 22)
    assert np.array_equal(a, b)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3, 1.0 + 2 ** -8 + 2 ** -9], dtype=np.float32)
    bits = ni.to_bf16_bits(x)
    back = ni.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.015625)
    assert back[3] == -2.5
    assert back[5] == np.float32(1.0078125)
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    rb = ni.bf16_bits_to_f32(ni.to_bf16_bits(r))
    assert np.all(np.abs(rb - r) <= np.abs(r) * 2.0 ** -8)


def test_determinism_and_seed_dependence():
    a, b = ni.make_config(0), ni.make_config(0)
    assert a.digest() == b.digest()
    c = ni.make_config(0, seed=123)
    assert c.digest() != a.digest()


def _valid_rows(w):
    n = np.clip(w.block_counts, 0, w.S)
    return n


def _own(w):
    if w.cu_seqlens is None:
        pos = np.tile(np.arange(w.T), (w.B, 1))
    else:
        pos = np.concatenate([np.arange(L) for L in w.seqlens])[None, :]
    return pos // w.block_size


def _check_rows(w, must_contain_own_first=False):
    own = _own(w)
    n = _valid_rows(w)
    for b in range(w.B):
        for t in range(w.T):
            for h in range(w.Hkv):
                row = w.block_indices[b, t, h]
                k = int(n[b, t, h])
                assert 1 <= k <= w.S
                vals = row[:k]
                assert len(set(vals.tolist())) == k, "entries must be distinct"
                assert np.all((vals >= 0) & (vals <= own[b, t]))
                if must_contain_own_first:
                    assert vals[0] == own[b, t]


def test_config0_structure():
    w = ni.make_config(0)
    assert (w.B, w.T, w.Hq, w.Hkv, w.D, w.block_size, w.S, w.dtype) == (1, 256, 4, 1, 64, 32, 4, "f32")
    assert w.scale == 0.125
    _check_rows(w)
    own = _own(w)
    # the full row (valid = min(4, own+1) entries) always includes the own block
    for t in range(w.T):
        valid = min(4, own[0, t] + 1)
        full = w.block_indices[0, t, 0, :valid]
        assert own[0, t] in full.tolist() and np.all(w.block_indices[0, t, 0, valid:] == -1)
        assert 1 <= w.block_counts[0, t, 0] <= valid
    # truncation drops the diagonal block for some rows (exercises both paths)
    dropped = [t for t in range(w.T)
               if own[0, t] not in w.block_indices[0, t, 0, :w.block_counts[0, t, 0]].tolist()]
    assert len(dropped) > 10


def test_config1_structure():
    w = ni.make_config(1)
    assert (w.B, w.T, w.Hq, w.Hkv, w.D, w.block_size, w.S) == (2, 4096, 32, 2, 128, 64, 16)
    own = _own(w)
    assert np.array_equal(w.block_counts, np.minimum(16, own + 1)[:, :, None].repeat(2, axis=2))
    sub = ni.make_workload("c1", "bf16", [4096] * 2, 32, 2, 128, 64, 16, "local_random", "full", 1)
    assert sub.digest() == w.digest()
    # local blocks first: own, own-1, own-2, own-3
    for t in (0, 64, 300, 4095):
        o = t // 64
        exp = [o - i for i in range(4) if o - i >= 0]
        assert w.block_indices[0, t, 0, :len(exp)].tolist() == exp
    # sampled rows: distinct, causal
    small = ni.make_workload("c1s", "bf16", [700] * 2, 4, 2, 8, 64, 16, "local_random", "full", 1)
    _check_rows(small, must_contain_own_first=True)


def test_config2_is_dense_causal():
    w = ni.make_config(2)
    assert (w.B, w.T, w.Hq, w.Hkv, w.S) == (4, 2048, 16, 16, 32)
    own = _own(w)
    for t in (0, 63, 64, 2047):
        o = t // 64
        assert w.block_indices[1, t, 3, :o + 1].tolist() == list(range(o + 1))
        assert np.all(w.block_indices[1, t, 3, o + 1:] == -1)
    assert np.array_equal(w.block_counts[..., 0], own + 1)


@pytest.mark.slow
def test_config3_structure():
    w = ni.make_config(3)
    assert (w.B, w.T, w.Hq, w.Hkv, w.D, w.block_size, w.S) == (1, 32768, 64, 4, 128, 64, 16)
    own = _own(w)[0]
    assert np.array_equal(w.block_counts[0, :, 0], np.minimum(16, own + 1))
    bi = w.block_indices[0]
    # sink first, then the own block and its two predecessors
    big = own >= 15
    assert np.all(bi[big, :, 0] == 0)
    assert np.all(bi[big, :, 1] == own[big, None])
    assert np.all(bi[big, :, 2] == own[big, None] - 1)
    assert np.all(bi[big, :, 3] == own[big, None] - 2)
    assert np.all((bi[big, :, 4:] >= 1) & (bi[big, :, 4:] <= own[big, None, None] - 3))
    srt = np.sort(bi[big], axis=-1)
    assert np.all(np.diff(srt, axis=-1) > 0)
    # short prefixes: all blocks 0..own
    for t in (0, 100, 64 * 14 + 3):
        o = t // 64
        assert sorted(bi[t, 0, :o + 1].tolist()) == list(range(o + 1))
    # values scaled by 0.5
    assert abs(float(np.std(w.q[0, :2048])) - 0.5) < 0.01


def test_config4_structure():
    w = ni.make_config(4)
    lens = w.seqlens
    assert len(lens) == 8 and sum(lens) <= 32768 and all(512 <= L <= 8192 for L in lens)
    assert w.B == 1 and w.T == sum(lens) and w.cu_seqlens[0] == 0 and w.cu_seqlens[-1] == w.T
    assert (w.Hq, w.Hkv, w.D, w.block_size, w.S) == (32, 2, 128, 64, 16)
    _check_rows(w, must_contain_own_first=True)
    own = _own(w)[0]
    assert np.all(w.block_counts[0, :, 0] <= np.minimum(16, own + 1))
    assert w.block_counts.min() == 1


def test_varlen_lengths_rejection():
    for s in range(5):
        lens = ni.varlen_lengths(s)
        assert sum(lens) <= 32768 and len(lens) == 8
