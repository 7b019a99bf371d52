"""The C-ABI library loads, exports every symbol include/nsa.h declares and
rejects bad arguments before launching anything (runs without a GPU)."""
import ctypes
import os
import re

import pytest

import block_index_sparse_amd as nsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "nsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nsa_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = nsa.load_library()
    names = declared_functions()
    assert {"nsa_fwd", "nsa_fwd_varlen", "nsa_fwd_workspace_size", "nsa_status_string",
            "nsa_abi_version", "nsa_fwd_schedule", "nsa_fwd_qblock", "nsa_fwd_schedule_qblock"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.nsa_abi_version() == 3


def test_status_strings():
    lib = nsa.load_library()
    for code, name in enumerate(["NSA_SUCCESS", "NSA_ERROR_INVALID_VALUE", "NSA_ERROR_NOT_SUPPORTED",
                                 "NSA_ERROR_WORKSPACE_TOO_SMALL", "NSA_ERROR_LAUNCH_FAILED"]):
        assert lib.nsa_status_string(code).decode() == name


def _call(dims, bs=64, scale=1.0, ptr=256, ws_bytes=1 << 40, varlen=False, nseq=0, nulls=()):
    lib = nsa.load_library()
    p = [ctypes.c_void_p(None if i in nulls else ptr) for i in range(8)]
    if varlen:
        return lib.nsa_fwd_varlen(ctypes.byref(dims), p[0], p[1], p[2], p[3], p[4], p[5], nseq, bs,
                                  scale, p[6], None, p[7], ws_bytes, None)
    return lib.nsa_fwd(ctypes.byref(dims), p[0], p[1], p[2], p[3], p[4], bs, scale, p[6], None, p[7],
                       ws_bytes, None)


def D(B=1, T=128, Hq=16, Hkv=1, Dh=128, S=4, dt=1):
    return nsa.NsaDims(B, T, Hq, Hkv, Dh, S, dt)


@pytest.mark.parametrize("dims,kw,code", [
    (D(Hkv=3), {}, 1),                    # Hq % Hkv != 0
    (D(T=0), {}, 1),
    (D(S=0), {}, 1),
    (D(Dh=96), {}, 2),
    (D(), {"bs": 48}, 2),
    (D(dt=7), {}, 2),
    (D(Hq=24, Hkv=1), {}, 2),             # G = 24: neither <= 16 nor a multiple of 16
    (D(), {"scale": float("nan")}, 1),
    (D(), {"scale": float("inf")}, 1),
    (D(), {"nulls": (0,)}, 1),
    (D(), {"nulls": (6,)}, 1),
    (D(), {"nulls": (7,)}, 1),
    (D(), {"ptr": 264}, 1),               # misaligned
    (D(), {"ws_bytes": 16}, 3),
    (D(B=2), {"varlen": True, "nseq": 2}, 1),   # varlen needs B == 1
    (D(), {"varlen": True, "nseq": 0}, 1),
    (D(), {"varlen": True, "nseq": 1, "nulls": (5,)}, 1),  # cu_seqlens NULL
])
def test_bad_arguments_are_rejected(dims, kw, code):
    assert _call(dims, **kw) == code


def test_workspace_sizes():
    assert nsa.workspace_size(1, 32768, 64, 4, 128, 16, 64) > 0
    assert nsa.workspace_size(1, 256, 4, 1, 64, 4, 32, "f32") > 0
    assert nsa.workspace_size(1, 256, 4, 1, 96, 4, 32, "f32") == 0
    a = nsa.workspace_size(1, 30000, 32, 2, 128, 16, 64, num_seqs=8)
    b = nsa.workspace_size(1, 30000, 32, 2, 128, 16, 64, num_seqs=100)
    assert 0 < a < b


def test_wide_items_fall_back_where_the_scheduler_cannot_hold_them():
    """bf16 with one query head per kv head plans 192-token items; where such
    an item's merged list could exceed the scheduler's 2048 entries (more than
    2048 blocks per sequence) the plan falls back to 128-token items, so every
    shape the narrower items support stays supported."""
    T = 2049 * 64
    assert nsa.workspace_size(1, T, 2, 2, 64, 16, 64) > 0      # 128 x 16 = 2048 entries fit
    assert nsa.workspace_size(1, T, 2, 2, 64, 17, 64) == 0     # 128 x 17 > 2048 and 2049 blocks
    assert nsa.workspace_size(1, 4096, 2, 2, 64, 32, 64) > 0   # 192-token items


def test_device_status_rejects_bad_arguments():
    """Checked on the host before any copy is enqueued."""
    lib = nsa.load_library()
    st = ctypes.c_int32(-1)
    dims = D()
    ws = ctypes.c_void_p(256)
    assert lib.nsa_fwd_device_status(ctypes.byref(dims), 64, 0, ws, 1 << 40, None, None) == 1
    assert lib.nsa_fwd_device_status(ctypes.byref(dims), 64, 0, None, 1 << 40, None, ctypes.byref(st)) == 1
    assert lib.nsa_fwd_device_status(ctypes.byref(dims), 64, 0, ws, 16, None, ctypes.byref(st)) == 3
    assert lib.nsa_fwd_device_status(ctypes.byref(D(Dh=96)), 64, 0, ws, 1 << 40, None, ctypes.byref(st)) == 2
    assert st.value == -1


def _call_qblock(dims, bs=64, scale=1.0, ptr=256, ws_bytes=1 << 40, nulls=()):
    lib = nsa.load_library()
    p = [ctypes.c_void_p(None if i in nulls else ptr) for i in range(8)]
    return lib.nsa_fwd_qblock(ctypes.byref(dims), p[0], p[1], p[2], p[3], p[4], bs, scale, p[6], None, p[7],
                              ws_bytes, None)


@pytest.mark.parametrize("dims,kw,code", [
    (D(Hkv=3), {}, 1),
    (D(T=0), {}, 1),
    (D(Dh=96), {}, 2),
    (D(), {"bs": 48}, 2),
    (D(), {"scale": float("nan")}, 1),
    (D(), {"nulls": (0,)}, 1),
    (D(), {"nulls": (3,)}, 1),            # block_indices NULL
    (D(), {"nulls": (4,)}, 1),            # block_counts NULL
    (D(), {"ptr": 264}, 1),
    (D(), {"ws_bytes": 16}, 3),
])
def test_qblock_bad_arguments_are_rejected(dims, kw, code):
    assert _call_qblock(dims, **kw) == code


def test_qblock_schedule_rejects_bad_arguments():
    lib = nsa.load_library()
    off, n = ctypes.c_size_t(0), ctypes.c_int32(-1)
    p = ctypes.c_void_p(256)
    args = lambda dims, bi=p, ws=p, wsb=1 << 40: lib.nsa_fwd_schedule_qblock(
        ctypes.byref(dims), bi, p, 64, ws, wsb, None, ctypes.byref(off), ctypes.byref(n))
    assert args(D(), bi=None) == 1
    assert args(D(), ws=None) == 1
    assert args(D(), ws=ctypes.c_void_p(264)) == 1
    assert args(D(), wsb=16) == 3
    assert args(D(Dh=96)) == 2
    assert n.value == -1


def test_bwd_rejects_bad_arguments():
    """nsa_bwd checks its arguments on the host before anything is enqueued."""
    lib = nsa.load_library()
    p = ctypes.c_void_p(256)

    def call(dims, bs=64, scale=1.0, ptr=p, ws_bytes=1 << 40, null_at=None):
        args = [ptr] * 12
        if null_at is not None:
            args[null_at] = None
        return lib.nsa_bwd(ctypes.byref(dims), args[0], args[1], args[2], args[3], args[4], args[5], args[6],
                           args[7], bs, scale, args[8], args[9], args[10], args[11], ws_bytes, None)
    assert call(D(Hkv=3)) == 1
    assert call(D(dt=0)) == 2            # fp32: the backward is bf16 only
    assert call(D(Dh=96)) == 2
    assert call(D(S=65)) == 2
    assert call(D(), bs=48) == 2
    assert call(D(), scale=float("nan")) == 1
    assert call(D(), null_at=5) == 1     # dout
    assert call(D(), null_at=11) == 1    # workspace
    assert call(D(), ptr=ctypes.c_void_p(264)) == 1
    assert call(D(), ws_bytes=16) == 3
    assert lib.nsa_bwd_workspace_size(ctypes.byref(D()), 64) > 0
    assert lib.nsa_bwd_workspace_size(ctypes.byref(D(dt=0)), 64) == 0
    # the forward's limits hold too (dq is the forward's gather in gradient
    # mode): one head per kv head keeping 64 of 2049 blocks merges more
    # entries per work item than the forward's planner takes
    assert call(D(T=2049 * 32, Hq=1, S=64), bs=32) == 2
    assert call(D(T=2048 * 32, Hq=1, S=64), bs=32, ws_bytes=16) == 3
    st = ctypes.c_int32(7)
    assert lib.nsa_bwd_device_status(ctypes.byref(D(Dh=96)), 64, p, 1 << 40, None, ctypes.byref(st)) == 2
    assert lib.nsa_bwd_device_status(ctypes.byref(D()), 64, None, 1 << 40, None, ctypes.byref(st)) == 1
    assert lib.nsa_bwd_device_status(ctypes.byref(D()), 64, p, 16, None, ctypes.byref(st)) == 3
    assert st.value == 7


class _StatusLib:
    """Stands in for libnsa.so with the same call signatures: every launch
    returns NSA_SUCCESS and nsa_fwd_device_status reports `word`."""

    def __init__(self, word):
        self.word = word
        self.status_reads = 0

    def nsa_fwd(self, *args):
        return 0

    nsa_fwd_varlen = nsa_fwd_qblock = nsa_fwd_execute = nsa_fwd

    def nsa_fwd_device_status(self, dims, bs, nseq, ws, wsb, stream, status_ref):
        self.status_reads += 1
        status_ref._obj.value = self.word
        return 0


def _forward_with(lib):
    f = nsa.Forward.__new__(nsa.Forward)
    f.lib, f.qblock, f.cu, f.nseq, f.block_size, f.scale = lib, False, None, 0, 64, 0.125
    f.dims, f.ws_bytes, f.stream = D(), 1 << 20, None
    f.out, f.lse = "out", "lse"
    f._p = {n: None for n in ("q", "k", "v", "bi", "bc", "cu", "out", "lse", "workspace")}
    return f


@pytest.mark.parametrize("word", [1, 3])
def test_expired_wait_raises_through_the_binding(word):
    """A launch the C call accepted but whose device status word is non-zero
    (a bounded wait expired) raises NsaDeviceError from run() and execute()
    by default; check=False returns without reading the word."""
    lib = _StatusLib(word)
    f = _forward_with(lib)
    for call in (f.run, f.execute):
        with pytest.raises(nsa.NsaDeviceError) as e:
            call()
        assert e.value.status == word
    assert lib.status_reads == 2
    assert f.run(check=False) == ("out", "lse") and f.execute(check=False) == ("out", "lse")
    assert lib.status_reads == 2
    assert f.device_status() == word


def test_clean_status_returns_results():
    lib = _StatusLib(0)
    f = _forward_with(lib)
    assert f.run() == ("out", "lse") and f.execute() == ("out", "lse")
    assert lib.status_reads == 2


def test_noalloc_rejects_before_touching_a_device():
    """nsa_fwd_noalloc checks its arguments and the scratch limit on the host
    (no device needed): workspaces above NSA_NOALLOC_SCRATCH_BYTES are refused
    with NSA_ERROR_WORKSPACE_TOO_SMALL."""
    lib = nsa.load_library()
    p = ctypes.c_void_p(256)

    def call(dims, bs=64, scale=1.0, ptr=p, null_at=None):
        args = [ptr] * 6
        if null_at is not None:
            args[null_at] = None
        return lib.nsa_fwd_noalloc(ctypes.byref(dims), args[0], args[1], args[2], args[3], args[4], bs, scale,
                                   args[5], None, None, None)
    big = D(T=65536, Hq=64, Hkv=4, S=16)
    assert nsa.workspace_size(1, 65536, 64, 4, 128, 16, 64) > nsa.NOALLOC_SCRATCH_BYTES
    assert call(big) == 3
    assert call(D(Hkv=3)) == 1
    assert call(D(Dh=96)) == 2
    assert call(D(), null_at=0) == 1
    assert call(D(), null_at=3) == 1
    assert call(D(), ptr=ctypes.c_void_p(264)) == 1
    assert call(D(), scale=float("nan")) == 1
    src = open(os.path.join(ROOT, "include", "nsa.h")).read()
    assert re.search(r"#define NSA_NOALLOC_SCRATCH_BYTES \(32u << 20\)", src)
    assert nsa.NOALLOC_SCRATCH_BYTES == 32 << 20
