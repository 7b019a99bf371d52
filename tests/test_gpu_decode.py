"""GPU parity of the decode step (nsa_decode: the newest token of each
sequence against its KV cache, with the block selection applied) against
the CPU fp64 decode oracle, plus bit-exact checks of its index plumbing."""
import math
import sys

import numpy as np
import pytest

import nsa_inputs as ni
from oracle import decode as odec
from tests._util import BF16_ATOL, BF16_RTOL

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_decode(w):
    import block_index_sparse_amd as nsa
    q, k, v, sl, bi, bc = ni.decode_to_torch(w)
    out, lse = nsa.decode(q, k, v, sl, bi, bc, w.block_size, w.scale)
    return out, lse


def check(w, out, lse, sequences=None, what=""):
    ref_o, ref_l = odec.decode_workload(w, sequences=sequences)
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    if sequences is not None:
        o, l = o[sequences], l[sequences]
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_l)), f"{what}: -inf lse pattern differs"
    fin = np.isfinite(ref_l)
    err_o = np.abs(o - ref_o)
    assert np.all(err_o <= BF16_ATOL + BF16_RTOL * np.abs(ref_o)), f"{what}: out max abs {err_o.max()}"
    assert np.all(np.abs(l[fin] - ref_l[fin]) <= BF16_ATOL + BF16_RTOL * np.abs(ref_l[fin])), f"{what}: lse"
    assert np.all(o[~fin] == 0.0), f"{what}: empty rows must be 0"
    return float(err_o.max(initial=0))


SMALL = [
    # name, B, Smax, lens, Hq, Hkv, D, bs, S, pattern, counts
    ("dec_g16_d128_bs64", 6, 700, (1, 700), 32, 2, 128, 64, 8, "sink_local_random", "uniform"),
    ("dec_g4_d64_bs32", 5, 300, (30, 300), 8, 2, 64, 32, 6, "shuffled", "uniform"),
    ("dec_g1_d128_bs128", 4, 900, (100, 900), 4, 4, 128, 128, 5, "local_random", "full"),
    ("dec_g64_d128_bs64", 3, 500, (200, 500), 64, 1, 128, 64, 4, "local_random", "uniform"),
    ("dec_g8_d64_bs64_dense_s64", 2, 4096, (3000, 4096), 16, 2, 64, 64, 64, "dense", "full"),
    ("dec_g16_d128_bs32_many_units", 2, 2048, (1500, 2048), 16, 1, 128, 32, 40, "local_random", "full"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_decode_small_cases_all_outputs(case):
    name, B, Smax, lens, Hq, Hkv, D, bs, S, pattern, counts = case
    _say(f"[decode] {name}")
    w = ni.make_decode_workload(name, B, Smax, lens[0], lens[1], Hq, Hkv, D, bs, S, pattern, counts, seed=13)
    w.seq_lens[0] = min(w.seq_lens[0], 1)
    out, lse = run_decode(w)
    check(w, out, lse, what=name)


def test_decode_hostile_entries_and_empty_sequences():
    _say("[decode] hostile entries")
    w = ni.make_decode_workload("dec_hostile", 8, 400, 0, 400, 32, 2, 128, 64, 8, "local_random", "full", seed=3)
    rng = np.random.default_rng(2)
    w.block_indices = rng.integers(-3, 9, size=w.block_indices.shape).astype(np.int32)
    w.block_counts = rng.integers(-2, 10, size=w.block_counts.shape).astype(np.int32)
    w.seq_lens[:3] = [0, 1, 400]
    out, lse = run_decode(w)
    check(w, out, lse, what="hostile")
    ref_o, ref_l = odec.decode_workload(w)
    assert np.isneginf(ref_l).any()


def test_decode_entries_past_count_are_invisible():
    """Rewriting entries past the count leaves out and lse bit-identical."""
    import torch
    w = ni.make_decode_workload("dec_past", 8, 1000, 300, 1000, 32, 2, 128, 64, 16, "sink_local_random",
                                "uniform", seed=5)
    out0, lse0 = run_decode(w)
    rng = np.random.default_rng(7)
    n = np.clip(w.block_counts, 0, w.S)
    junk = rng.integers(-5, 20, size=w.block_indices.shape).astype(np.int32)
    past = np.arange(w.S)[None, None, :] >= n[..., None]
    w.block_indices = np.where(past, junk, w.block_indices).astype(np.int32)
    out1, lse1 = run_decode(w)
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse0, lse1)


def test_decode_long_context_sampled_and_count_probe():
    """The benchmark's decode workload (128 sequences, cache of 8192 rows,
    Hq=64, Hkv=4, D=128, bs=64, S=16): sampled sequences against the oracle;
    with q = 0 every visible key weighs exactly 1, so exp(lse) is the visible
    key count on every (sequence, head)."""
    _say("[decode] long context: generating")
    w = ni.make_decode_config()
    out, lse = run_decode(w)
    seqs = np.unique(np.concatenate([[0, w.B - 1], np.random.default_rng(1).integers(0, w.B, 24)]))
    err = check(w, out, lse, sequences=seqs, what=w.name)
    _say(f"[decode] long context: max abs out err {err:.3e}")
    w.q[:] = 0
    w.q_bits[:] = 0
    _, lse0 = run_decode(w)
    cnt = np.exp(lse0.cpu().numpy().astype(np.float64))
    want = np.zeros((w.B, w.Hq), np.int64)
    for b in range(w.B):
        for h in range(w.Hkv):
            m = odec.key_mask(w.block_indices[b, h], w.block_counts[b, h], w.S, w.block_size, int(w.seq_lens[b]))
            want[b, h * w.G:(h + 1) * w.G] = int(m.sum())
    assert np.array_equal(np.round(cnt).astype(np.int64), want)
