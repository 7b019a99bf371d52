"""Shared helpers of the GPU tests: device copies of seeded workloads and the
parity bars.  (bf16: |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise; fp32:
max-abs 1e-5; an lse of -inf must match exactly.)"""
import numpy as np

BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
F32_ATOL = 1e-5


def to_device(w, device="cuda"):
    import nsa_inputs as ni
    return ni.to_torch(w, device)


def run_gpu(w, device="cuda", **kw):
    """Forward through the C ABI; also asserts that no bounded wait inside
    the kernels expired."""
    import block_index_sparse_amd as nsa
    q, k, v, bi, bc, cu = to_device(w, device)
    kw.setdefault("index_layout", getattr(w, "index_layout", "token"))
    f = nsa.Forward(q, k, v, bi, bc, w.block_size, w.scale, cu_seqlens=cu, **kw)
    out, lse = f.run()
    assert f.device_status() == 0, "a bounded wait inside the kernel expired"
    return out, lse


def compare(w, out, lse, ref_out, ref_lse, rows=None, what=""):
    """out/lse: GPU tensors [B,T,Hq,D]/[B,T,Hq]; ref: oracle [n, Hq, D]/[n, Hq]
    for packed rows `rows` (None = all).  Raises AssertionError with stats."""
    o = out.float().reshape(-1, w.Hq, w.D).cpu().numpy().astype(np.float64)
    l = lse.reshape(-1, w.Hq).cpu().numpy().astype(np.float64)
    if rows is not None:
        o, l = o[rows], l[rows]
    return _compare_arrays(w, o, l, ref_out, ref_lse, what)


def _compare_arrays(w, o, l, ref_out, ref_lse, what=""):
    """o/l: GPU results as float64 arrays [n, Hq, D]/[n, Hq] matching the
    oracle's rows ref_out/ref_lse."""
    ninf_ref = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(l), ninf_ref), f"{what}: -inf lse pattern differs"
    fin = ~ninf_ref
    err_o = np.abs(o - ref_out)
    err_l = np.abs(l[fin] - ref_lse[fin])
    stats = dict(max_abs_out=float(err_o.max(initial=0)), max_abs_lse=float(err_l.max(initial=0)),
                 max_rel_out=float((err_o / np.maximum(np.abs(ref_out), 1e-6)).max(initial=0)))
    if w.dtype == "bf16":
        ok_o = np.all(err_o <= BF16_ATOL + BF16_RTOL * np.abs(ref_out))
        ok_l = np.all(err_l <= BF16_ATOL + BF16_RTOL * np.abs(ref_lse[fin]))
    else:
        ok_o = stats["max_abs_out"] <= F32_ATOL
        ok_l = stats["max_abs_lse"] <= F32_ATOL
    assert ok_o and ok_l, f"{what}: parity failed {stats}"
    assert np.all(o[np.repeat(ninf_ref[..., None], w.D, axis=-1)] == 0.0), f"{what}: empty rows must be 0"
    return stats


def compare_every_row(w, out, lse, chunk=4096, threads=0, what=""):
    """Every output row against the oracle, element by element, in chunks of
    `chunk` packed tokens (the oracle runs each chunk on all host threads),
    so host memory stays bounded at any workload size.  Returns the worst
    max-abs errors over all chunks."""
    import oracle
    total = w.B * w.T
    o_all = out.float().reshape(total, w.Hq, w.D).cpu().numpy()
    l_all = lse.reshape(total, w.Hq).cpu().numpy()
    worst = dict(max_abs_out=0.0, max_abs_lse=0.0, max_rel_out=0.0, rows=0)
    for a in range(0, total, chunk):
        rows = np.arange(a, min(total, a + chunk), dtype=np.int64)
        ref_o, ref_l = oracle.fwd_workload(w, tokens=rows, threads=threads)
        st = _compare_arrays(w, o_all[rows].astype(np.float64), l_all[rows].astype(np.float64), ref_o, ref_l,
                             what=f"{what} rows {a}..{rows[-1]}")
        for k in ("max_abs_out", "max_abs_lse", "max_rel_out"):
            worst[k] = max(worst[k], st[k])
        worst["rows"] += len(rows)
    assert worst["rows"] == total
    return worst


def sample_rows(w, n, seed=0):
    """Packed token ids: sequence starts/ends, block edges and a seeded sample."""
    rng = np.random.default_rng(seed)
    total = w.B * w.T
    picks = set()
    if w.cu_seqlens is None:
        starts = [b * w.T for b in range(w.B)]
        lens = [w.T] * w.B
    else:
        starts = [int(x) for x in w.cu_seqlens[:-1]]
        lens = w.seqlens
    for s, L in zip(starts, lens):
        for p in (0, 1, w.block_size - 1, w.block_size, L - 2, L - 1):
            if 0 <= p < L:
                picks.add(s + p)
    picks |= set(int(x) for x in rng.integers(0, total, size=n))
    return np.array(sorted(picks), dtype=np.int64)
