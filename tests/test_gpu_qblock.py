"""GPU parity of the query-block index layout (one row of block_indices per
query block, shared by its tokens: nsa_fwd_qblock) against the CPU fp64
oracle, and its bit-exact agreement with the per-token entry point fed the
same rows copied to every token."""
import sys

import numpy as np
import pytest

import nsa_inputs as ni
import oracle
from tests._util import compare, run_gpu, sample_rows, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SMALL_QB = [
    # name, dtype, B, T, Hq, Hkv, D, bs, S, pattern, counts
    ("qb_bf16_g16_d128_bs64", "bf16", 2, 300, 32, 2, 128, 64, 6, "sink_local_random", "uniform"),
    ("qb_bf16_g1_d128_bs128", "bf16", 1, 520, 4, 4, 128, 128, 4, "local_random", "full"),
    ("qb_bf16_g4_d64_bs32", "bf16", 2, 170, 8, 2, 64, 32, 5, "shuffled", "uniform"),
    ("qb_bf16_g64_d128_bs64", "bf16", 1, 257, 64, 1, 128, 64, 4, "local_random", "uniform"),
    ("qb_bf16_g1_d128_bs64_dense", "bf16", 2, 400, 2, 2, 128, 64, 7, "dense", "full"),
    ("qb_f32_g4_d64_bs32", "f32", 1, 256, 4, 1, 64, 32, 4, "shuffled", "uniform"),
    ("qb_f32_g2_d128_bs64", "f32", 2, 190, 4, 2, 128, 64, 3, "sink_local_random", "full"),
]


def _qb(case, seed=29):
    name, dtype, B, T, Hq, Hkv, D, bs, S, pattern, counts = case
    return ni.make_qblock_workload(name, dtype, B, T, Hq, Hkv, D, bs, S, pattern, counts, seed)


@pytest.mark.parametrize("case", SMALL_QB, ids=[c[0] for c in SMALL_QB])
def test_qblock_small_cases_all_outputs(case):
    _say(f"[qblock] {case[0]}")
    w = _qb(case)
    out, lse = run_gpu(w)
    ref_o, ref_l = oracle.fwd_workload(w)
    compare(w, out, lse, ref_o, ref_l, what=case[0])


def _rows_per_token(w):
    """The query-block rows copied to every token of the block (test-side
    layout change, [B, Hkv, NQB, S] -> [B, T, Hkv, S])."""
    qb = np.arange(w.T) // w.block_size
    bi = np.ascontiguousarray(w.block_indices[:, :, qb, :].transpose(0, 2, 1, 3))
    bc = np.ascontiguousarray(w.block_counts[:, :, qb].transpose(0, 2, 1))
    return bi, bc


@pytest.mark.parametrize("case", [SMALL_QB[0], SMALL_QB[1], SMALL_QB[5]], ids=lambda c: c[0])
def test_qblock_equals_token_layout_bitwise(case):
    """Both entry points must build the same schedule from the same rows, so
    out and lse agree bit for bit."""
    import torch
    import block_index_sparse_amd as nsa
    _say(f"[qblock] bitwise vs token layout {case[0]}")
    w = _qb(case, seed=31)
    out_q, lse_q = run_gpu(w)
    q, k, v, _, _, _ = to_device(w)
    bi, bc = _rows_per_token(w)
    f = nsa.Forward(q, k, v, torch.from_numpy(bi).cuda(), torch.from_numpy(bc).cuda(), w.block_size, w.scale)
    out_t, lse_t = f.run()
    assert f.device_status() == 0
    assert torch.equal(out_q.view(torch.int16) if out_q.dtype == torch.bfloat16 else out_q,
                       out_t.view(torch.int16) if out_t.dtype == torch.bfloat16 else out_t)
    assert torch.equal(lse_q, lse_t)


def test_qblock_long_context_sampled_rows():
    """T = 32768, Hq = 64, Hkv = 4, D = 128, bs = 64, S = 16 (sink, local and
    random blocks per query block): sampled rows against the oracle, and the
    q = 0 count probe on every row."""
    _say("[qblock] long context: generating")
    w = ni.make_config(5)
    out, lse = run_gpu(w)
    rows = sample_rows(w, 160, seed=5)
    ref_o, ref_l = oracle.fwd_workload(w, tokens=rows)
    stats = compare(w, out, lse, ref_o, ref_l, rows=rows, what=w.name)
    _say(f"[qblock] long context: {stats}")
    assert bool(out.float().isfinite().all())
    # count probe: q = 0 makes exp(lse) the visible key count, exactly
    w.q[:] = 0
    w.q_bits[:] = 0
    _, lse0 = run_gpu(w)
    cnt = np.exp(lse0.reshape(-1, w.Hq).cpu().numpy().astype(np.float64))
    assert np.all(np.abs(cnt - np.round(cnt)) < 1e-3 * np.maximum(cnt, 1))
    _, ref_l0 = oracle.fwd_workload(w, tokens=rows)
    assert np.array_equal(np.round(cnt[rows]).astype(np.int64), np.round(np.exp(ref_l0)).astype(np.int64))


def test_qblock_hostile_entries():
    """Negative entries, blocks past the query block or the sequence, repeats
    and counts outside [0, S], in query-block rows."""
    _say("[qblock] hostile entries")
    w = ni.make_qblock_workload("qb_hostile", "bf16", 2, 330, 32, 2, 128, 64, 7, "local_random", "full", seed=3)
    rng = np.random.default_rng(4)
    w.block_indices = rng.integers(-3, 9, size=w.block_indices.shape).astype(np.int32)
    w.block_counts = rng.integers(-2, 10, size=w.block_counts.shape).astype(np.int32)
    out, lse = run_gpu(w)
    ref_o, ref_l = oracle.fwd_workload(w)
    compare(w, out, lse, ref_o, ref_l, what="qb_hostile")
    assert np.isneginf(ref_l).any()
