"""The forward's debug mode (NSA_DEBUG=1, read at every launch): the LDS
ring of the bf16 kernel then holds one unit at a time, every unit entering
only after all readers of every earlier unit have released it, so no load
overlaps a read.  Every attention wave still walks its units in the same
order, so the results must equal the overlapped ring's bit for bit; a
difference would mean a read of a slot raced a load into it (or a load
raced a read) in the release mode."""
import os
import sys

import numpy as np
import pytest

import nsa_inputs as ni
from tests._util import to_device

pytestmark = pytest.mark.gpu


def _run(w, debug):
    import block_index_sparse_amd as nsa
    q, k, v, bi, bc, cu = to_device(w)
    old = os.environ.get("NSA_DEBUG")
    try:
        if debug:
            os.environ["NSA_DEBUG"] = "1"
        else:
            os.environ.pop("NSA_DEBUG", None)
        f = nsa.Forward(q, k, v, bi, bc, w.block_size, w.scale, cu_seqlens=cu,
                        index_layout=getattr(w, "index_layout", "token"))
        out, lse = f.run()
        assert f.device_status() == 0
        return out.clone(), lse.clone()
    finally:
        if old is None:
            os.environ.pop("NSA_DEBUG", None)
        else:
            os.environ["NSA_DEBUG"] = old


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_serial_ring_equals_overlapped_ring(cfg):
    import torch
    w = ni.make_config(cfg)
    print(f"[debug-ring] {w.name}", flush=True)
    sys.stdout.flush()
    o0, l0 = _run(w, False)
    o1, l1 = _run(w, True)
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)), "out differs between the serial and overlapped ring"
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32)), "lse differs between the serial and overlapped ring"


def test_serial_ring_hostile_entries():
    import torch
    w = ni.make_workload("dbg_hostile", "bf16", [300, 300], 32, 2, 128, 64, 8, "sink_local_random", "uniform", seed=4)
    rng = np.random.default_rng(4)
    w.block_indices = rng.integers(-2, 7, size=w.block_indices.shape).astype(np.int32)
    w.block_counts = rng.integers(-1, 10, size=w.block_counts.shape).astype(np.int32)
    o0, l0 = _run(w, False)
    o1, l1 = _run(w, True)
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32))


def _hostile_bwd_workload():
    w = ni.make_workload("dbg_bwd_hostile", "bf16", [300, 300], 64, 2, 128, 64, 8, "sink_local_random", "uniform",
                         seed=5)
    rng = np.random.default_rng(5)
    w.block_indices = rng.integers(-2, 7, size=w.block_indices.shape).astype(np.int32)
    w.block_counts = rng.integers(-1, 10, size=w.block_counts.shape).astype(np.int32)
    return w


@pytest.mark.parametrize("cfg", [1, 2, 3, "hostile"])
def test_serial_ring_equals_overlapped_ring_backward(cfg):
    """The backward's dq runs the same ring in its gradient mode: dq (and the
    dk / dv that follow from its reader bitmaps) must not change bit for bit
    when the ring holds one unit at a time (named workloads, and hostile
    entries: negative, repeated and out-of-range indices, counts outside
    [0, S], two head groups per kv head)."""
    import torch
    import block_index_sparse_amd as nsa
    w = _hostile_bwd_workload() if cfg == "hostile" else ni.make_config(cfg)
    seed = 300 + (cfg if isinstance(cfg, int) else 9)
    print(f"[debug-ring] backward {w.name}", flush=True)
    sys.stdout.flush()
    q, k, v, bi, bc, _ = to_device(w)
    out, lse = _run(w, False)
    x = ni.normal(seed, 9, w.B * w.T * w.Hq * w.D).reshape(w.B, w.T, w.Hq, w.D)
    dout = torch.from_numpy(ni.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()
    grads = []
    old = os.environ.get("NSA_DEBUG")
    try:
        for debug in (False, True):
            if debug:
                os.environ["NSA_DEBUG"] = "1"
            else:
                os.environ.pop("NSA_DEBUG", None)
            grads.append([g.clone() for g in nsa.bwd(q, k, v, out, lse, dout, bi, bc, w.block_size, w.scale)])
    finally:
        if old is None:
            os.environ.pop("NSA_DEBUG", None)
        else:
            os.environ["NSA_DEBUG"] = old
    for name, a, b in zip(("dq", "dk", "dv"), grads[0], grads[1]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{name} differs between the serial and overlapped ring"
