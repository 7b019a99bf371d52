"""GPU parity of the backward pass (nsa_bwd: dq, dk, dv) against the CPU
fp64 gradient oracle (oracle/backward.py, pinned by central differences of
the forward oracle and by autograd through SDPA).

Tolerance, derived from the arithmetic: the kernels round P and dS to bf16
(relative error <= 2^-9 each) and form Delta from the forward's bf16 out
before the MFMAs that accumulate dq, dk and dv in fp32, so each gradient
entry's error is at most 2^-9 times the sum of its terms' magnitudes to
first order (oracle/backward.py returns that sum per entry; a CPU test
recomputes the gradients with those roundings and finds every error within
2^-8 of it).  The bar, per element: |gpu - ref| <= 2^-7 sum|terms| +
1e-6 max(sum|terms|) (the last for fp32 accumulation order)."""
import sys

import numpy as np
import pytest

import nsa_inputs as ni
from oracle import backward as obwd
from tests._util import to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dout(w, seed):
    x = ni.normal(seed, 9, w.B * w.T * w.Hq * w.D).reshape(w.B, w.T, w.Hq, w.D)
    bits = ni.to_bf16_bits(x)
    return ni.bf16_bits_to_f32(bits).reshape(x.shape), bits.reshape(x.shape)


def run_bwd(w, dout_bits):
    import torch
    import block_index_sparse_amd as nsa
    q, k, v, bi, bc, _ = to_device(w)
    f = nsa.Forward(q, k, v, bi, bc, w.block_size, w.scale)
    out, lse = f.run()
    assert f.device_status() == 0
    dout = torch.from_numpy(np.ascontiguousarray(dout_bits).view(np.int16)).view(torch.bfloat16).cuda()
    return nsa.bwd(q, k, v, out, lse, dout, bi, bc, w.block_size, w.scale)


def check(name, got, ref, mag):
    """Per-element bar: |gpu - ref| <= 2^-7 mag + 1e-6 max(mag), mag = the
    entry's sum of |terms|."""
    g = (got.cpu().numpy() if hasattr(got, "cpu") else got).astype(np.float64)
    err = np.abs(g - ref)
    bar = 2.0 ** -7 * mag + 1e-6 * float(mag.max(initial=0))
    ratio = float((err / np.maximum(mag, 1e-30)).max(initial=0))
    _say(f"[bwd] {name}: max|err| {err.max(initial=0):.3e}, max|ref| {np.abs(ref).max(initial=0):.3e}, "
         f"max err/sum|terms| {ratio:.2e} (bar {2.0 ** -7:.2e})")
    bad = np.argwhere(err > bar)
    assert bad.size == 0, f"{name}: {len(bad)} entries past the bar, first {bad[:3].tolist()}"


CASES = [
    # name, B, T, Hq, Hkv, D, bs, S, pattern, counts
    ("bwd_g16_d128_bs64", 2, 300, 32, 2, 128, 64, 6, "sink_local_random", "uniform"),
    ("bwd_g4_d64_bs32", 1, 200, 8, 2, 64, 32, 5, "shuffled", "uniform"),
    ("bwd_g1_d128_bs128", 1, 300, 2, 2, 128, 128, 3, "local_random", "full"),
    ("bwd_g32_d64_bs64", 1, 150, 32, 1, 64, 64, 3, "sink_local_random", "full"),
    # two token segments, two key blocks per 64-key chunk, two head groups,
    # a ragged last chunk
    ("bwd_g32_d128_bs32_T1100", 1, 1100, 64, 2, 128, 32, 8, "sink_local_random", "uniform"),
    # three heads per group, T not a multiple of 32
    ("bwd_g3_d64_bs32_T33", 2, 33, 6, 2, 64, 32, 4, "local_random", "uniform"),
    # three head groups of 16, block size 128
    ("bwd_g48_d128_bs128_T260", 1, 260, 48, 1, 128, 128, 3, "sink_local_random", "uniform"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_small_cases_all_gradients(case):
    name, B, T, Hq, Hkv, D, bs, S, pattern, counts = case
    _say(f"[bwd] {name}")
    w = ni.make_workload(name, "bf16", [T] * B, Hq, Hkv, D, bs, S, pattern, counts, seed=19)
    dout, dbits = _dout(w, 19)
    dq, dk, dv = run_bwd(w, dbits)
    rq, rk, rv, mq, mk, mv = obwd.bwd(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, bs, w.scale,
                                      terms=True)
    check(f"{name} dq", dq, rq, mq)
    check(f"{name} dk", dk, rk, mk)
    check(f"{name} dv", dv, rv, mv)


def test_bwd_single_token_sequences():
    """T = 1: each row sees one key, so P = 1 and dS = P (dP - Delta) = 0:
    dq = dk = 0 exactly in the mathematics, dv = the group's sum of dO.  The
    kernels reach zero up to fp32 rounding of dP against Delta (a few ulp of
    |dO . v|), far below 1e-3 here."""
    _say("[bwd] single-token sequences")
    w = ni.make_workload("bwd_t1", "bf16", [1, 1, 1], 4, 2, 128, 64, 2, "sink_local_random", "full", seed=19)
    dout, dbits = _dout(w, 19)
    dq, dk, dv = run_bwd(w, dbits)
    rq, rk, rv, mq, mk, mv = obwd.bwd(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, 64, w.scale,
                                      terms=True)
    assert np.all(rq == 0) and np.all(rk == 0)
    assert float(dq.abs().max()) <= 1e-3 and float(dk.abs().max()) <= 1e-3
    check("T=1 dv", dv, rv, mv)
    want = dout.astype(np.float64).reshape(3, 1, 2, 2, 128).sum(axis=3)        # [B, T, Hkv, D]
    np.testing.assert_allclose(rv, want, rtol=0, atol=1e-12)


def test_bwd_hostile_entries():
    """Negative, repeated and out-of-range entries, counts outside [0, S],
    rows with no visible key (zero dq) and blocks no token reads (zero dk, dv)."""
    _say("[bwd] hostile entries")
    w = ni.make_workload("bwd_hostile", "bf16", [260, 260], 16, 1, 128, 64, 6, "local_random", "full", seed=7)
    rng = np.random.default_rng(3)
    w.block_indices = rng.integers(-3, 6, size=w.block_indices.shape).astype(np.int32)
    w.block_counts = rng.integers(-2, 8, size=w.block_counts.shape).astype(np.int32)
    dout, dbits = _dout(w, 7)
    dq, dk, dv = run_bwd(w, dbits)
    rq, rk, rv, mq, mk, mv = obwd.bwd(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, 64, w.scale,
                                      terms=True)
    check("hostile dq", dq, rq, mq)
    check("hostile dk", dk, rk, mk)
    check("hostile dv", dv, rv, mv)
    assert np.any(np.all(rq == 0, axis=(-1, -2)))   # some token sees nothing


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_bwd_named_workload_full_size(cfg):
    """Full-size workloads (config 2: one query head per kv head, so 16
    tokens share each MFMA tile in both kernels): dq of about 330 tokens
    (sampled, edges and a run of 64) against the oracle; at every
    (sequence, kv head, d) the invariants sum_s dV_s = sum over the group's
    (token, head) of dO (rows of P sum to one) and sum_s dK_s = 0 (each row's
    dS sums to zero)."""
    from tests._util import sample_rows
    _say(f"[bwd] config {cfg}: generating")
    w = ni.make_config(cfg)
    dout, dbits = _dout(w, 100 + cfg)
    dq, dk, dv = run_bwd(w, dbits)
    # a seeded sample, sequence starts and ends, block edges, and a run of
    # 64 consecutive tokens (whole work items of the dq gather and their
    # boundaries, for items of 12 and of 192 tokens)
    run0 = int(np.random.default_rng(50 + cfg).integers(0, w.B * w.T - 64))
    rows = np.union1d(sample_rows(w, 256, seed=cfg), np.arange(run0, run0 + 64))
    rq, mq = obwd.dq_rows(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size, w.scale, rows,
                          terms=True)
    check(f"config {cfg} dq rows", dq.reshape(-1, w.Hq, w.D)[rows], rq, mq)
    dvs = dv.double().sum(dim=1).cpu().numpy()                      # [B, Hkv, D]
    dks = dk.double().sum(dim=1).cpu().numpy()
    dos = dout.astype(np.float64).sum(axis=1).reshape(w.B, w.Hkv, w.G, w.D).sum(axis=2)
    dv_abs = dv.double().abs().sum(dim=1).cpu().numpy()
    dk_abs = dk.double().abs().sum(dim=1).cpu().numpy()
    err_v = np.abs(dvs - dos)
    _say(f"[bwd] config {cfg}: max|sum dV - sum dO| {err_v.max():.3e} (sum|dV| up to {dv_abs.max():.3e}), "
         f"max|sum dK| {np.abs(dks).max():.3e} (sum|dK| up to {dk_abs.max():.3e})")
    assert np.all(err_v <= 1e-2 * dv_abs + 1e-3)
    assert np.all(np.abs(dks) <= 1e-2 * dk_abs + 1e-3)
    assert bool(dq.isfinite().all() and dk.isfinite().all() and dv.isfinite().all())
    # dK, dV of sampled key blocks against the oracle: block 0 (read by
    # every token: every token segment contributes), the last block and a
    # few in between
    nb = (w.T + w.block_size - 1) // w.block_size
    rng = np.random.default_rng(cfg)
    blocks = [(0, 0, 0), (w.B - 1, w.Hkv - 1, nb - 1)]
    blocks += [(int(rng.integers(w.B)), int(rng.integers(w.Hkv)), int(rng.integers(1, nb))) for _ in range(3)]
    _check_blocks(w, dout, dk, dv, blocks, f"config {cfg}")
    if cfg in (1, 2):
        # every key of one kv head of one sequence (T = 4096, and the dense
        # causal workload, whose dk / dv kernel writes them directly)
        _say(f"[bwd] config {cfg}: oracle dK, dV of every key of sequence 0, kv head 0")
        hk, hv, hmk, hmv = obwd.dkdv_head(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size,
                                          w.scale, 0, 0)
        check(f"config {cfg} dk head", dk[0, :, 0], hk, hmk)
        check(f"config {cfg} dv head", dv[0, :, 0], hv, hmv)


def _check_blocks(w, dout, dk, dv, blocks, what):
    _say(f"[bwd] {what}: oracle dK, dV of key blocks {blocks}")
    rk, rv, mk, mv = obwd.dkdv_blocks(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size, w.scale,
                                      blocks, terms=True)
    bs = w.block_size
    gk = np.zeros_like(rk)
    gv = np.zeros_like(rv)
    dk_ = dk.cpu().numpy()
    dv_ = dv.cpu().numpy()
    for r, (b, h, j) in enumerate(blocks):
        n = min(bs, w.T - j * bs)
        gk[r, :n] = dk_[b, j * bs:j * bs + n, h]
        gv[r, :n] = dv_[b, j * bs:j * bs + n, h]
    check(f"{what} dk blocks", gk, rk, mk)
    check(f"{what} dv blocks", gv, rv, mv)


def test_bwd_segments_deterministic():
    """T = 2500 with an attention-sink block: block 0 is read by tokens in
    three token segments, whose partial sums the reduction adds in order.
    Two calls give bitwise-equal gradients; sampled blocks match the oracle."""
    import torch
    _say("[bwd] segments and determinism")
    w = ni.make_workload("bwd_seg", "bf16", [2500], 16, 1, 128, 64, 8, "sink_local_random", "uniform", seed=29)
    dout, dbits = _dout(w, 29)
    dq, dk, dv = run_bwd(w, dbits)
    dq2, dk2, dv2 = run_bwd(w, dbits)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    _check_blocks(w, dout, dk, dv, [(0, 0, 0), (0, 0, 1), (0, 0, 15), (0, 0, 20), (0, 0, 39)], "bwd_seg")


def test_bwd_dirty_workspace():
    """The workspace needs no initialisation: a workspace filled with 0xFF
    bytes (and one reused after a call on other dims) gives bit-identical
    gradients to a fresh one (the reader bitmaps are cleared and the dq
    gather's schedule is written by every call)."""
    import ctypes
    import torch
    import block_index_sparse_amd as nsa
    _say("[bwd] dirty workspace")
    w = ni.make_workload("bwd_dirty", "bf16", [700, 700], 32, 2, 128, 64, 6, "sink_local_random", "uniform", seed=23)
    dout, dbits = _dout(w, 23)
    q, k, v, bi, bc, _ = to_device(w)
    f = nsa.Forward(q, k, v, bi, bc, w.block_size, w.scale)
    out, lse = f.run()
    dO = torch.from_numpy(np.ascontiguousarray(dbits).view(np.int16)).view(torch.bfloat16).cuda()
    lib = nsa.load_library()
    need = lib.nsa_bwd_workspace_size(ctypes.byref(nsa._dims(w.B, w.T, w.Hq, w.Hkv, w.D, w.S, nsa.DTYPE_BF16)),
                                      w.block_size)
    ref = [g.clone() for g in nsa.bwd(q, k, v, out, lse, dO, bi, bc, w.block_size, w.scale)]
    ws = torch.full((need + 4096,), 255, dtype=torch.uint8, device="cuda")
    got = nsa.bwd(q, k, v, out, lse, dO, bi, bc, w.block_size, w.scale, workspace=ws)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{name}: dirty workspace changed the result"
    # the same workspace after a call on other dims (one sequence, T = 300)
    w2 = ni.make_workload("bwd_dirty2", "bf16", [300], 32, 2, 128, 64, 6, "local_random", "uniform", seed=24)
    _, d2 = _dout(w2, 24)
    q2, k2, v2, bi2, bc2, _ = to_device(w2)
    o2, l2 = nsa.Forward(q2, k2, v2, bi2, bc2, w2.block_size, w2.scale).run()
    dO2 = torch.from_numpy(np.ascontiguousarray(d2).view(np.int16)).view(torch.bfloat16).cuda()
    nsa.bwd(q2, k2, v2, o2, l2, dO2, bi2, bc2, w2.block_size, w2.scale, workspace=ws)
    got = nsa.bwd(q, k, v, out, lse, dO, bi, bc, w.block_size, w.scale, workspace=ws)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{name}: reused workspace changed the result"
