"""nsa_fwd_noalloc (workspace in the library's static device array) against
nsa_fwd (caller-provided workspace) through the C ABI: the same schedule and
kernels run, so out and lse must be bitwise identical.  Three calls in a row
on one GPU share the array, each smaller than the one before, so a call that
left stale state in the array for the next would show here."""
import sys

import numpy as np
import pytest

import nsa_inputs as ni
from tests._util import to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(w):
    import torch
    import block_index_sparse_amd as nsa
    q, k, v, bi, bc, _ = to_device(w)
    ref_o, ref_l = nsa.fwd(q, k, v, bi, bc, w.block_size, w.scale)
    status = torch.full((1,), -1, dtype=torch.int32, device=q.device)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.T, w.Hq), float("nan"), dtype=torch.float32, device=q.device)
    o, l = nsa.fwd_noalloc(q, k, v, bi, bc, w.block_size, w.scale, out=out, lse=lse, device_status=status,
                           check=False)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "a bounded wait expired in the no-alloc run"
    iv = (lambda t: t.view(torch.int16)) if w.dtype == "bf16" else (lambda t: t.view(torch.int32))
    assert torch.equal(iv(o), iv(ref_o)), f"{w.name}: out differs from nsa_fwd"
    assert torch.equal(l.view(torch.int32), ref_l.view(torch.int32)), f"{w.name}: lse differs from nsa_fwd"


def test_noalloc_matches_nsa_fwd_on_calls_in_a_row():
    cases = [ni.make_config(3),   # the largest named fixed-length workload (24.4 MiB of schedule)
             ni.make_config(1),
             ni.make_workload("noalloc_small", "bf16", [300], 32, 2, 128, 64, 6, "sink_local_random", "uniform",
                              seed=29)]
    for w in cases:
        _say(f"[noalloc] {w.name}: B={w.B} T={w.T}")
        _both(w)


def test_noalloc_fp32_and_checked_binding():
    import block_index_sparse_amd as nsa
    w = ni.make_config(0)
    _say(f"[noalloc] {w.name}")
    _both(w)
    q, k, v, bi, bc, _ = to_device(w)
    out, lse = nsa.fwd_noalloc(q, k, v, bi, bc, w.block_size, w.scale)   # check=True reads the status
    assert bool(np.isfinite(lse.cpu().numpy()).all())
