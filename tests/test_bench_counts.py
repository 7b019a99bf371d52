"""The benchmark's useful-FLOP count: |M_t| per row equals the oracle's
exp(lse) with q = 0 (every visible key then weighs exactly 1)."""
import numpy as np
import pytest

import nsa_inputs as ni
import oracle
import bench
from bench import visible_keys_per_row, useful_flops


@pytest.mark.parametrize("pattern,counts,varlen,lens", [
    ("shuffled", "uniform", False, [100, 100]),
    ("sink_local_random", "full", False, [300]),
    ("local_random", "uniform", True, [40, 1, 77, 130]),
])
def test_visible_key_count_matches_oracle(pattern, counts, varlen, lens):
    w = ni.make_workload("cnt", "f32", lens, 4, 2, 8, 16, 6, pattern, counts, seed=9, varlen=varlen)
    w.block_indices[..., -1] = w.block_indices[..., 0]    # a repeat past or inside the count
    w.q[:] = 0
    _, lse = oracle.fwd_workload(w)
    m = visible_keys_per_row(w)                            # [tokens, Hkv]
    exp = np.round(np.exp(lse)).astype(np.int64)          # [tokens, Hq]
    G = w.G
    assert np.array_equal(np.repeat(m, G, axis=1), exp)
    assert useful_flops(w) == 4 * w.D * int(exp.sum())


def test_visible_key_count_query_block_rows():
    w = ni.make_qblock_workload("cntq", "f32", 2, 90, 4, 2, 8, 16, 5, "sink_local_random", "uniform", seed=3)
    w.q[:] = 0
    _, lse = oracle.fwd_workload(w)
    m = visible_keys_per_row(w)
    exp = np.round(np.exp(lse)).astype(np.int64)
    assert np.array_equal(np.repeat(m, w.G, axis=1), exp)


def test_decode_visible_key_count_matches_oracle():
    from bench import decode_visible_keys
    from oracle import decode as odec
    w = ni.make_decode_workload("dc", 6, 90, 0, 90, 4, 2, 8, 16, 6, "sink_local_random", "uniform", seed=2)
    w.block_indices[..., -1] = w.block_indices[..., 0]
    w.q[:] = 0
    _, lse = odec.decode_workload(w)
    m = decode_visible_keys(w)
    got = np.repeat(m, w.G, axis=1)
    exp = np.where(np.isneginf(lse), 0, np.round(np.exp(np.where(np.isneginf(lse), 0, lse)))).astype(np.int64)
    assert np.array_equal(got, exp)


def test_backward_cpu_baseline_counts_dq_flop():
    """The backward line's CPU baseline times the oracle's dq on a token
    sample and counts 6 D FLOP per visible triple of the sampled rows."""
    w = ni.make_workload("bcb", "bf16", [96], 8, 2, 64, 32, 4, "sink_local_random", "uniform", seed=3)
    dout = np.random.default_rng(0).standard_normal(w.q.shape).astype(np.float32)
    r = bench.bwd_cpu_baseline(w, dout, seconds_target=0.0)    # stops after the first 16-token sample
    m = bench.visible_keys_per_row(w)
    rows = np.sort(np.random.default_rng(0).choice(96, size=16, replace=False))
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["tokens"] == 16
    want = 6 * w.D * w.G * int(m[rows].sum())
    assert abs(r["value"] * r["seconds"] * 1e12 - want) <= 1e-6 * want
