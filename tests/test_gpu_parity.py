"""GPU parity: the HIP library (through the C ABI) against the CPU fp64
oracle on the same seeded inputs.  Small cases and the five named workloads
at full size are compared element by element over every output row (the
full-size workloads in chunks of tokens, each chunk on all host threads)."""
import sys

import numpy as np
import pytest

import nsa_inputs as ni
import oracle
from tests._util import compare, compare_every_row, run_gpu, sample_rows

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SMALL = [
    # name, dtype, seqlens, Hq, Hkv, D, bs, S, pattern, counts, varlen
    ("bf16_g16_d128_bs64", "bf16", [200, 200], 32, 2, 128, 64, 4, "sink_local_random", "full", False),
    ("bf16_g16_d128_bs64_rand", "bf16", [333], 16, 1, 128, 64, 6, "local_random", "uniform", False),
    ("bf16_g4_d64_bs32", "bf16", [170], 8, 2, 64, 32, 5, "shuffled", "uniform", False),
    ("bf16_g1_d128_bs64_dense", "bf16", [300, 300], 4, 4, 128, 64, 5, "dense", "full", False),
    ("bf16_g8_d128_bs128", "bf16", [400], 16, 2, 128, 128, 4, "local_random", "uniform", False),
    ("bf16_g32_d128_bs64", "bf16", [150], 64, 2, 128, 64, 3, "local_random", "full", False),
    ("bf16_g48_d64_bs64", "bf16", [140], 48, 1, 64, 64, 3, "sink_local_random", "uniform", False),
    ("bf16_g64_d128_bs32", "bf16", [100, 37], 128, 2, 128, 32, 4, "shuffled", "uniform", True),
    ("bf16_g2_d64_bs64", "bf16", [130], 4, 2, 64, 64, 3, "shuffled", "uniform", False),
    ("bf16_g3_d64_bs32", "bf16", [97], 6, 2, 64, 32, 4, "local_random", "uniform", False),
    ("bf16_varlen_g16", "bf16", [65, 1, 200, 64, 129], 32, 2, 128, 64, 5, "local_random", "uniform", True),
    ("bf16_varlen_g1_d64_bs32", "bf16", [250, 5, 193, 384], 2, 2, 64, 32, 6, "local_random", "uniform", True),
    ("bf16_g1_d128_bs64_wide_items", "bf16", [700, 700], 2, 2, 128, 64, 8, "sink_local_random", "uniform", False),
    ("f32_g4_d64_bs32", "f32", [256], 4, 1, 64, 32, 4, "shuffled", "uniform", False),
    ("f32_g2_d128_bs64", "f32", [190, 190], 4, 2, 128, 64, 3, "sink_local_random", "full", False),
    ("f32_g16_d64_bs128", "f32", [300], 16, 1, 64, 128, 3, "local_random", "uniform", False),
    ("f32_varlen_g4", "f32", [40, 100, 7], 8, 2, 64, 32, 4, "local_random", "uniform", True),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases_all_outputs(case):
    name, dtype, lens, Hq, Hkv, D, bs, S, pattern, counts, varlen = case
    _say(f"[parity] {name}")
    w = ni.make_workload(name, dtype, lens, Hq, Hkv, D, bs, S, pattern, counts, seed=17, varlen=varlen)
    out, lse = run_gpu(w)
    ref_o, ref_l = oracle.fwd_workload(w)
    compare(w, out, lse, ref_o, ref_l, what=name)


@pytest.mark.parametrize("G,S", [(16, 6), (1, 8), (1, 7)])
def test_hostile_entries_and_duplicates(G, S):
    """Negative entries, blocks past own and past the end, counts outside
    [0, S], repeated blocks: all handled as the oracle's set semantics.  With
    one query head per kv head the items are 192 tokens wide and planned one
    lane per token (rows read 16 bytes at a time when S is a multiple of 4)."""
    _say(f"[parity] hostile entries G={G} S={S}")
    w = ni.make_workload("hostile", "bf16", [250, 250], 2 * G, 2, 128, 64, S, "local_random", "full", seed=5)
    rng = np.random.default_rng(1)
    w.block_indices = rng.integers(-3, 8, size=w.block_indices.shape).astype(np.int32)
    w.block_counts = rng.integers(-2, S + 3, size=w.block_counts.shape).astype(np.int32)
    out, lse = run_gpu(w)
    ref_o, ref_l = oracle.fwd_workload(w)
    compare(w, out, lse, ref_o, ref_l, what="hostile")
    assert np.isneginf(ref_l).any()


@pytest.mark.parametrize("dtype,scale", [("bf16", -0.3), ("bf16", 0.0), ("bf16", 2.5), ("f32", -0.125),
                                         ("f32", 0.0)])
def test_any_finite_scale(dtype, scale):
    """Negative, zero and large softmax scales (the bf16 kernel takes a
    separate path when the scale is not positive).  fp32 stays at the
    magnitude of 1/sqrt(D): its 1e-5 bar is absolute, and fp32 rounding of
    the scores grows with the scale."""
    _say(f"[parity] scale {scale} {dtype}")
    w = ni.make_workload(f"scale_{scale}", dtype, [230], 16, 1, 128 if dtype == "bf16" else 64, 64, 5,
                         "sink_local_random", "uniform", seed=23, scale=float(np.float32(scale)))
    out, lse = run_gpu(w)
    ref_o, ref_l = oracle.fwd_workload(w)
    compare(w, out, lse, ref_o, ref_l, what=f"scale {scale} {dtype}")


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_named_workload_full_size(cfg):
    _say(f"[parity] config {cfg}: generating")
    w = ni.make_config(cfg)
    _say(f"[parity] config {cfg} {w.name}: gpu run")
    out, lse = run_gpu(w)
    _say(f"[parity] config {cfg} {w.name}: oracle on every row")
    stats = compare_every_row(w, out, lse, what=w.name)
    _say(f"[parity] config {cfg}: {stats}")
    # properties that hold on every row: finite, and |out| bounded by max |v|
    o = out.float()
    assert bool(o.isfinite().all())
    vmax = float(np.abs(w.v).max())
    assert float(o.abs().max()) <= vmax * (1 + 1e-2) + 1e-2


def test_maximum_row_length_dense_rows():
    """The longest rows the header allows: S = 1024 entries per row, every
    causal block listed (bs = 32, T = 32763, not a multiple of the block),
    so items plan 12 x 1024 index entries on a workgroup each and merge
    1024-entry lists.  Sampled rows against the oracle; the q = 0 count
    probe gives exp(lse) = t + 1 exactly on every row."""
    import torch
    _say("[parity] maximum row length: generating")
    w = ni.make_workload("max_rows", "bf16", [32763], 16, 1, 64, 32, 1024, "dense", "full", seed=41)
    assert int(w.block_counts.max()) == 1024
    out, lse = run_gpu(w)
    rows = sample_rows(w, 48, seed=41)
    ref_o, ref_l = oracle.fwd_workload(w, tokens=rows)
    stats = compare(w, out, lse, ref_o, ref_l, rows=rows, what="max_rows")
    _say(f"[parity] maximum row length: {stats}")
    w.q[:] = 0
    w.q_bits[:] = 0
    _, lse0 = run_gpu(w)
    cnt = torch.exp(lse0.double().reshape(-1, w.Hq)).cpu().numpy()
    want = np.arange(1, w.T + 1, dtype=np.float64)[:, None]
    assert np.array_equal(np.round(cnt), np.broadcast_to(want, cnt.shape))
