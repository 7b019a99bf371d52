"""Bit-exact checks of the block-index plumbing on the GPU."""
import math
import sys

import numpy as np
import pytest

import nsa_inputs as ni
import oracle
from tests._util import run_gpu, sample_rows, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_count_probe(cfg):
    """q = 0: every visible key scores 0, p = 2^0 = 1 exactly and the fp32
    normaliser counts the visible keys, so round(exp(lse)) == |M_t| exactly,
    on every (token, query head).  |M_t| comes from the host count of the
    listed blocks (pinned against the oracle's q = 0 rows on the CPU), and a
    sample of rows is checked against the oracle itself as well."""
    from bench import visible_keys_per_row
    _say(f"[plumbing] count probe config {cfg}")
    w = ni.make_config(cfg)
    w.q[:] = 0
    if w.q_bits is not None:
        w.q_bits[:] = 0
    out, lse = run_gpu(w)
    l = lse.reshape(-1, w.Hq).cpu().numpy().astype(np.float64)
    cnt = np.exp(l)
    # integral everywhere, and exactly the visible-key count of every row
    assert np.all(np.abs(cnt - np.round(cnt)) < 1e-3 * np.maximum(cnt, 1))
    want = np.repeat(visible_keys_per_row(w).astype(np.int64), w.G, axis=1)
    got = np.round(cnt).astype(np.int64)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"count probe differs on {len(bad)} (token, head) pairs, first {bad[:4].tolist()}"
    rows = sample_rows(w, 256, seed=100 + cfg)
    _, ref_l = oracle.fwd_workload(w, tokens=rows)
    assert np.array_equal(got[rows], np.round(np.exp(ref_l)).astype(np.int64))


def test_bit_plane_probe():
    """fp32, q = 0, v[s, h, d] = bit d of s: round(out * |M_t|) is the exact
    number of visible keys whose position has bit d set."""
    w = ni.make_config(0)
    w.q[:] = 0
    s = np.arange(w.T)
    for d in range(w.D):
        w.v[0, :, 0, d] = ((s >> (d % 9)) & 1).astype(np.float32)
    out, lse = run_gpu(w)
    ref_o, ref_l = oracle.fwd_workload(w)
    n = np.round(np.exp(lse.reshape(-1, w.Hq).cpu().numpy().astype(np.float64)))
    o = out.reshape(-1, w.Hq, w.D).cpu().numpy().astype(np.float64)
    got = np.round(o * n[..., None]).astype(np.int64)
    exp = np.round(ref_o * np.exp(ref_l)[..., None]).astype(np.int64)
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_entries_past_count_and_order_are_invisible(cfg):
    """Rewriting every entry past the count with garbage and reversing the
    order of the counted entries leaves out and lse bitwise identical (the
    planner merges each item's entries into one ascending list)."""
    _say(f"[plumbing] past-count and order invariance config {cfg}")
    w = ni.make_config(cfg)
    out0, lse0 = run_gpu(w)
    rng = np.random.default_rng(cfg)
    bi = w.block_indices.copy()
    n = np.clip(w.block_counts, 0, w.S)
    j = np.arange(w.S)
    past = j[None, None, None, :] >= n[..., None]
    bi = np.where(past, rng.integers(-100, 1000, size=bi.shape).astype(np.int32), bi)
    # reverse the valid prefix of every row
    idx = np.where(j[None, None, None, :] < n[..., None], n[..., None] - 1 - j, j)
    bi = np.take_along_axis(bi, idx, axis=-1).astype(np.int32)
    w.block_indices = bi
    out1, lse1 = run_gpu(w)
    import torch
    assert torch.equal(out0.view(torch.int16) if out0.dtype == torch.bfloat16 else out0,
                       out1.view(torch.int16) if out1.dtype == torch.bfloat16 else out1)
    assert torch.equal(lse0, lse1)


def test_varlen_equals_per_sequence():
    import torch
    w = ni.make_config(4)
    out, lse = run_gpu(w)
    cu = w.cu_seqlens
    for i in (0, 3, 7):
        a, b = int(cu[i]), int(cu[i + 1])
        ws = ni.Workload(name="seq", dtype=w.dtype, B=1, T=b - a, Hq=w.Hq, Hkv=w.Hkv, D=w.D,
                         block_size=w.block_size, S=w.S, scale=w.scale, q=w.q[:, a:b], k=w.k[:, a:b],
                         v=w.v[:, a:b], block_indices=w.block_indices[:, a:b],
                         block_counts=w.block_counts[:, a:b], q_bits=w.q_bits[:, a:b],
                         k_bits=w.k_bits[:, a:b], v_bits=w.v_bits[:, a:b])
        o1, l1 = run_gpu(ws)
        assert torch.equal(o1.view(torch.int16), out[:, a:b].view(torch.int16))
        assert torch.equal(l1, lse[:, a:b])


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_schedule_is_a_permutation(cfg):
    import torch
    import block_index_sparse_amd as nsa
    w = ni.make_config(cfg)
    q, k, v, bi, bc, cu = to_device(w)
    wl = nsa.schedule(bi, bc, w.Hq, w.D, w.block_size, w.dtype, cu_seqlens=cu).cpu().numpy()
    assert np.array_equal(np.sort(wl), np.arange(len(wl)))


def test_empty_rows_give_zero_and_neg_inf():
    w = ni.make_workload("empty", "bf16", [256], 16, 1, 128, 64, 4, "local_random", "full", seed=2)
    w.block_counts[0, 10:20, 0] = 0
    w.block_indices[0, 30:40, 0, :] = -1
    out, lse = run_gpu(w)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    for t in list(range(10, 20)) + list(range(30, 40)):
        assert np.all(o[0, t] == 0) and np.all(np.isneginf(l[0, t]))
    assert np.all(np.isfinite(l[0, :10]))


def test_misaligned_index_rows_read_one_entry_at_a_time():
    """block_indices that start 4 bytes past a 16-byte boundary (the C ABI
    asks no alignment of them) are read entry by entry instead of 16 bytes
    at a time by the planner of wide items (192-token items of the dense
    causal workload); the results are bitwise those of an aligned copy."""
    import torch
    import block_index_sparse_amd as nsa
    _say("[plumbing] misaligned index rows")
    w = ni.make_config(2)
    q, k, v, bi, bc, _ = to_device(w)
    out0, lse0 = nsa.fwd(q, k, v, bi, bc, w.block_size, w.scale)
    buf = torch.empty(bi.numel() + 4, dtype=torch.int32, device=bi.device)
    bi_off = buf[1:1 + bi.numel()].view(bi.shape)
    bi_off.copy_(bi)
    assert bi_off.data_ptr() % 16 == 4
    out1, lse1 = nsa.fwd(q, k, v, bi_off, bc, w.block_size, w.scale)
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse0, lse1)
