"""Python binding of the MI355X native sparse attention forward (``libnsa.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/nsa.h``.  PyTorch supplies device
memory and the current HIP stream.  If the library has not been built the
calls raise; there is no fallback path.

Call contract (ejKernel ``native_sparse_attention`` API page, "Parameters"):
``fwd(q, k, v, block_indices, block_counts, block_size, scale=None,
cu_seqlens=None) -> (out, lse)`` with q ``[B, T, Hq, D]``, k/v
``[B, T, Hkv, D]`` (bf16 or fp32, on the GPU), ``block_indices
[B, T, Hkv, S]`` int32, ``block_counts [B, T, Hkv]`` int32 or a Python int
(broadcast), ``scale`` defaulting to 1/sqrt(D), and an optional
``cu_seqlens [N+1]`` int32 for packed sequences (then B == 1).

``index_layout="query_block"`` takes the layout of the page's
``block_indices`` description instead: ``block_indices [B, Hkv, NQB, S]`` and
``block_counts [B, Hkv, NQB]`` (or an int), NQB = ceil(T / block_size), one
row per query block shared by its tokens (``nsa_fwd_qblock``; fixed-length
sequences only).
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["fwd", "fwd_noalloc", "Forward", "decode", "Decode", "bwd", "workspace_size", "schedule", "load_library", "library_path", "NsaError",
           "NsaDeviceError", "DTYPE_F32", "DTYPE_BF16"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_build", "libnsa.so")
_lib = None

DTYPE_F32, DTYPE_BF16 = 0, 1
DEVICE_WAIT_EXPIRED = 1


class NsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class NsaDeviceError(NsaError):
    """The launch was accepted (the C call returned NSA_SUCCESS) but the
    device status word of the run is not zero: a bounded wait inside the
    forward kernel (or the backward's dq gather) expired and its results are
    incomplete.  ``status`` holds the word (bit 0 = NSA_DEVICE_WAIT_EXPIRED)."""


class NsaDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("num_selected", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load ``libnsa.so`` (built by ``block_index_sparse_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"native library missing: {_LIB_PATH}; build it with "
                           "`python -m block_index_sparse_amd.build` (no fallback path exists)")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    dp = ctypes.POINTER(NsaDims)
    lib.nsa_fwd_workspace_size.restype = sz
    lib.nsa_fwd_workspace_size.argtypes = [dp, i32, i32]
    lib.nsa_fwd.restype = ctypes.c_int
    lib.nsa_fwd.argtypes = [dp, p, p, p, p, p, i32, f32, p, p, p, sz, p]
    lib.nsa_fwd_noalloc.restype = ctypes.c_int
    lib.nsa_fwd_noalloc.argtypes = [dp, p, p, p, p, p, i32, f32, p, p, p, p]
    lib.nsa_fwd_varlen.restype = ctypes.c_int
    lib.nsa_fwd_varlen.argtypes = [dp, p, p, p, p, p, p, i32, i32, f32, p, p, p, sz, p]
    lib.nsa_fwd_qblock.restype = ctypes.c_int
    lib.nsa_fwd_qblock.argtypes = [dp, p, p, p, p, p, i32, f32, p, p, p, sz, p]
    lib.nsa_fwd_schedule_qblock.restype = ctypes.c_int
    lib.nsa_fwd_schedule_qblock.argtypes = [dp, p, p, i32, p, sz, p, ctypes.POINTER(sz), ctypes.POINTER(i32)]
    lib.nsa_bwd_workspace_size.restype = sz
    lib.nsa_bwd_workspace_size.argtypes = [dp, i32]
    lib.nsa_bwd.restype = ctypes.c_int
    lib.nsa_bwd.argtypes = [dp, p, p, p, p, p, p, p, p, i32, f32, p, p, p, p, sz, p]
    lib.nsa_decode.restype = ctypes.c_int
    lib.nsa_decode.argtypes = [dp, p, p, p, p, p, p, i32, f32, p, p, p]
    lib.nsa_fwd_schedule.restype = ctypes.c_int
    lib.nsa_fwd_schedule.argtypes = [dp, p, p, p, i32, i32, p, sz, p, ctypes.POINTER(sz),
                                     ctypes.POINTER(i32)]
    lib.nsa_fwd_execute.restype = ctypes.c_int
    lib.nsa_fwd_execute.argtypes = [dp, p, p, p, i32, i32, f32, p, p, p, sz, p]
    lib.nsa_fwd_device_status.restype = ctypes.c_int
    lib.nsa_fwd_device_status.argtypes = [dp, i32, i32, p, sz, p, ctypes.POINTER(i32)]
    lib.nsa_bwd_device_status.restype = ctypes.c_int
    lib.nsa_bwd_device_status.argtypes = [dp, i32, p, sz, p, ctypes.POINTER(i32)]
    lib.nsa_status_string.restype = ctypes.c_char_p
    lib.nsa_status_string.argtypes = [ctypes.c_int]
    lib.nsa_abi_version.restype = i32
    lib.nsa_abi_version.argtypes = []
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise NsaError(status, lib.nsa_status_string(status).decode())


def _dims(B, T, Hq, Hkv, D, S, dtype_code) -> NsaDims:
    return NsaDims(B, T, Hq, Hkv, D, S, dtype_code)


def workspace_size(B, T, Hq, Hkv, D, S, block_size, dtype="bf16", num_seqs=0) -> int:
    code = DTYPE_BF16 if dtype in ("bf16", "bfloat16") else DTYPE_F32
    d = _dims(B, T, Hq, Hkv, D, S, code)
    return int(load_library().nsa_fwd_workspace_size(ctypes.byref(d), int(block_size), int(num_seqs)))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(torch, device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


INDEX_LAYOUTS = ("token", "query_block")


def _prepare(q, k, v, block_indices, block_counts, cu_seqlens, block_size=64, index_layout="token"):
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, T, H, D]")
    B, T, Hq, D = q.shape
    if k.shape[:2] != (B, T) or v.shape != k.shape or k.shape[3] != D:
        raise ValueError("k and v must be [B, T, Hkv, D] matching q")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share a dtype")
    if q.dtype == torch.bfloat16:
        code = DTYPE_BF16
    elif q.dtype == torch.float32:
        code = DTYPE_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    Hkv = k.shape[2]
    if index_layout == "token":
        rows, name = (B, T, Hkv), "[B, T, Hkv"
    elif index_layout == "query_block":
        if block_size <= 0:
            raise ValueError("block_size must be positive")
        if cu_seqlens is not None:
            raise ValueError("the query_block index layout takes fixed-length sequences only")
        rows, name = (B, Hkv, (T + block_size - 1) // block_size), "[B, Hkv, ceil(T / block_size)"
    else:
        raise ValueError(f"index_layout must be one of {INDEX_LAYOUTS}")
    if block_indices.dim() != 4 or tuple(block_indices.shape[:3]) != rows:
        raise ValueError(f"block_indices must be {name}, S]")
    S = block_indices.shape[3]
    bi = block_indices.to(device=q.device, dtype=torch.int32).contiguous()
    if isinstance(block_counts, int):
        bc = torch.full(rows, block_counts, dtype=torch.int32, device=q.device)
    else:
        if tuple(block_counts.shape) != rows:
            raise ValueError(f"block_counts must be {name}] or an int")
        bc = block_counts.to(device=q.device, dtype=torch.int32).contiguous()
    cu = None
    if cu_seqlens is not None:
        cu = cu_seqlens.to(device=q.device, dtype=torch.int32).contiguous()
        if B != 1:
            raise ValueError("cu_seqlens needs B == 1")
    return (q.contiguous(), k.contiguous(), v.contiguous(), bi, bc, cu, B, T, Hq, Hkv, D, S, code)


class Forward:
    """A prepared forward call: device buffers and ctypes arguments are built
    once, so repeated calls cost one C call each.

    ``run()`` is ``nsa_fwd`` / ``nsa_fwd_varlen`` / ``nsa_fwd_qblock``;
    ``schedule()`` and ``execute()`` are its two halves (``nsa_fwd_schedule``
    or ``nsa_fwd_schedule_qblock``, then ``nsa_fwd_execute``).  All launch on
    torch's current stream of q's device.

    ``run()`` and ``execute()`` check the device status word after the
    launch by default (``check=True``): that waits for the stream, and an
    expired bounded wait inside the kernel raises ``NsaDeviceError`` instead
    of returning incomplete rows.  ``check=False`` returns right after the
    launch (asynchronous); the caller then reads ``device_status()`` itself
    before trusting the results, as the benchmark does once after its timed
    launches.
    """

    def __init__(self, q, k, v, block_indices, block_counts, block_size: int = 64,
                 scale: float | None = None, cu_seqlens=None, out=None, lse=None, workspace=None,
                 return_lse: bool = True, index_layout: str = "token"):
        import torch
        self.lib = load_library()
        (self.q, self.k, self.v, self.bi, self.bc, self.cu, B, T, Hq, Hkv, D, S,
         code) = _prepare(q, k, v, block_indices, block_counts, cu_seqlens, int(block_size), index_layout)
        self.qblock = index_layout == "query_block"
        self.scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        self.block_size = int(block_size)
        self.nseq = 0 if self.cu is None else self.cu.numel() - 1
        self.dims = _dims(B, T, Hq, Hkv, D, S, code)
        need = int(self.lib.nsa_fwd_workspace_size(ctypes.byref(self.dims), self.block_size, self.nseq))
        need = max(need, 256)  # an unsupported shape is reported by the call itself
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=self.q.device)
        self.workspace = workspace
        self.out = torch.empty_like(self.q) if out is None else out
        self.lse = lse if lse is not None else (
            torch.empty((B, T, Hq), dtype=torch.float32, device=self.q.device) if return_lse else None)
        self.ws_bytes = workspace.numel() * workspace.element_size()
        self.stream = _stream(torch, self.q.device)
        self._p = {n: _ptr(getattr(self, n)) for n in ("q", "k", "v", "bi", "bc", "cu", "out", "lse",
                                                        "workspace")}

    def _check_device(self):
        word = self.device_status()
        if word != 0:
            raise NsaDeviceError(word, f"forward device status {word:#x}: a bounded wait inside the kernel "
                                       "expired (NSA_DEVICE_WAIT_EXPIRED); out and lse are incomplete")

    def run(self, check: bool = True):
        P, L = self._p, self.lib
        if self.qblock:
            st = L.nsa_fwd_qblock(ctypes.byref(self.dims), P["q"], P["k"], P["v"], P["bi"], P["bc"],
                                  self.block_size, self.scale, P["out"], P["lse"], P["workspace"],
                                  self.ws_bytes, self.stream)
        elif self.cu is None:
            st = L.nsa_fwd(ctypes.byref(self.dims), P["q"], P["k"], P["v"], P["bi"], P["bc"],
                           self.block_size, self.scale, P["out"], P["lse"], P["workspace"],
                           self.ws_bytes, self.stream)
        else:
            st = L.nsa_fwd_varlen(ctypes.byref(self.dims), P["q"], P["k"], P["v"], P["bi"], P["bc"],
                                  P["cu"], self.nseq, self.block_size, self.scale, P["out"], P["lse"],
                                  P["workspace"], self.ws_bytes, self.stream)
        _check(st)
        if check:
            self._check_device()
        return self.out, self.lse

    def schedule(self):
        """Scheduler only; returns (byte offset, length) of the work list."""
        P = self._p
        off = ctypes.c_size_t(0)
        n = ctypes.c_int32(0)
        if self.qblock:
            _check(self.lib.nsa_fwd_schedule_qblock(ctypes.byref(self.dims), P["bi"], P["bc"], self.block_size,
                                                    P["workspace"], self.ws_bytes, self.stream,
                                                    ctypes.byref(off), ctypes.byref(n)))
            return off.value, n.value
        _check(self.lib.nsa_fwd_schedule(ctypes.byref(self.dims), P["bi"], P["bc"], P["cu"], self.nseq,
                                         self.block_size, P["workspace"], self.ws_bytes, self.stream,
                                         ctypes.byref(off), ctypes.byref(n)))
        return off.value, n.value

    def execute(self, check: bool = True):
        P = self._p
        _check(self.lib.nsa_fwd_execute(ctypes.byref(self.dims), P["q"], P["k"], P["v"], self.nseq,
                                        self.block_size, self.scale, P["out"], P["lse"], P["workspace"],
                                        self.ws_bytes, self.stream))
        if check:
            self._check_device()
        return self.out, self.lse

    def device_status(self) -> int:
        """Device status word of the runs since the last schedule (0 = all
        completed; NSA_DEVICE_WAIT_EXPIRED = a bounded wait expired).
        Synchronises the stream."""
        st = ctypes.c_int32(0)
        _check(self.lib.nsa_fwd_device_status(ctypes.byref(self.dims), self.block_size, self.nseq,
                                              self._p["workspace"], self.ws_bytes, self.stream,
                                              ctypes.byref(st)))
        return st.value

    def work_list(self):
        """Run the scheduler and return a copy of the work list (int32)."""
        import torch
        off, n = self.schedule()
        return self.workspace[off: off + 4 * n].view(torch.int32).clone()


def fwd(q, k, v, block_indices, block_counts, block_size: int = 64, scale: float | None = None,
        cu_seqlens=None, out=None, lse=None, workspace=None, return_lse: bool = True,
        index_layout: str = "token", check: bool = True):
    """Native sparse attention forward on the GPU.  Returns (out, lse).
    With ``check`` (the default) the device status is read after the launch
    and an expired wait raises ``NsaDeviceError`` (see ``Forward``)."""
    return Forward(q, k, v, block_indices, block_counts, block_size, scale, cu_seqlens, out, lse,
                   workspace, return_lse, index_layout).run(check=check)


NOALLOC_SCRATCH_BYTES = 32 << 20


def fwd_noalloc(q, k, v, block_indices, block_counts, block_size: int = 64, scale: float | None = None,
                out=None, lse=None, return_lse: bool = True, device_status=None, check: bool = True):
    """``nsa_fwd_noalloc``: the fixed-length forward with its workspace in
    the library's static device array (NOALLOC_SCRATCH_BYTES per GPU), so
    the C call allocates nothing.  Calls on one GPU must be ordered on one
    stream (they share the array).  ``device_status``: an int32 GPU tensor of
    one element that receives the run's status word, or None; with ``check``
    one is made here, read after the call and an expired wait raises
    ``NsaDeviceError``.  Returns (out, lse)."""
    import torch
    lib = load_library()
    (q, k, v, bi, bc, _, B, T, Hq, Hkv, D, S, code) = _prepare(q, k, v, block_indices, block_counts, None,
                                                                int(block_size), "token")
    dims = _dims(B, T, Hq, Hkv, D, S, code)
    out = torch.empty_like(q) if out is None else out
    if lse is None and return_lse:
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    if device_status is None and check:
        device_status = torch.zeros(1, dtype=torch.int32, device=q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.nsa_fwd_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(bi), _ptr(bc), int(block_size),
                               scale, _ptr(out), _ptr(lse), _ptr(device_status), _stream(torch, q.device)))
    if check:
        word = int(device_status.item())
        if word != 0:
            raise NsaDeviceError(word, f"forward device status {word:#x}: a bounded wait inside the kernel "
                                       "expired (NSA_DEVICE_WAIT_EXPIRED); out and lse are incomplete")
    return out, lse


def schedule(block_indices, block_counts, Hq, D, block_size, dtype="bf16", cu_seqlens=None):
    """Run only the work scheduler; returns the work list (int32 tensor)."""
    import torch
    lib = load_library()
    B, T, Hkv, S = block_indices.shape
    code = DTYPE_BF16 if dtype in ("bf16", "bfloat16") else DTYPE_F32
    dims = _dims(B, T, Hq, Hkv, D, S, code)
    bi = block_indices.to(dtype=torch.int32).contiguous()
    bc = block_counts.to(dtype=torch.int32).contiguous()
    cu = None if cu_seqlens is None else cu_seqlens.to(dtype=torch.int32).contiguous()
    nseq = 0 if cu is None else cu.numel() - 1
    need = int(lib.nsa_fwd_workspace_size(ctypes.byref(dims), int(block_size), int(nseq)))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=bi.device)
    off = ctypes.c_size_t(0)
    n = ctypes.c_int32(0)
    status = lib.nsa_fwd_schedule(ctypes.byref(dims), _ptr(bi), _ptr(bc), _ptr(cu), int(nseq),
                                  int(block_size), _ptr(ws), ws.numel(), _stream(torch, bi.device),
                                  ctypes.byref(off), ctypes.byref(n))
    _check(status)
    return ws[off.value: off.value + 4 * n.value].view(torch.int32).clone()


class Decode:
    """A prepared decode step (``nsa_decode``): the newest token of each
    sequence, q ``[B, Hq, D]`` bf16, against its cache ``k_cache, v_cache
    [B, Smax, Hkv, D]`` bf16 holding ``seq_lens [B]`` (int32) keys, with the
    selected blocks ``block_indices [B, Hkv, S]`` and ``block_counts
    [B, Hkv]`` (or an int).  Arguments are checked and marshalled once;
    ``run()`` is one C call on torch's current stream and returns
    (out [B, Hq, D], lse [B, Hq])."""

    def __init__(self, q, k_cache, v_cache, seq_lens, block_indices, block_counts, block_size: int = 64,
                 scale: float | None = None, out=None, lse=None, return_lse: bool = True):
        import torch
        self.lib = load_library()
        if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
            raise ValueError("q must be [B, Hq, D] and k_cache, v_cache [B, Smax, Hkv, D]")
        B, Hq, D = q.shape
        _, Smax, Hkv, Dk = k_cache.shape
        if k_cache.shape[0] != B or Dk != D:
            raise ValueError("cache shape does not match q")
        if not (q.dtype == k_cache.dtype == v_cache.dtype == torch.bfloat16):
            raise ValueError("decode takes bf16 q, k_cache, v_cache")
        if not (q.is_cuda and k_cache.is_cuda and v_cache.is_cuda):
            raise ValueError("q and the cache must be GPU tensors")
        if block_indices.dim() != 3 or tuple(block_indices.shape[:2]) != (B, Hkv):
            raise ValueError("block_indices must be [B, Hkv, S]")
        S = block_indices.shape[2]
        dev = q.device
        self.bi = block_indices.to(device=dev, dtype=torch.int32).contiguous()
        if isinstance(block_counts, int):
            self.bc = torch.full((B, Hkv), block_counts, dtype=torch.int32, device=dev)
        else:
            if tuple(block_counts.shape) != (B, Hkv):
                raise ValueError("block_counts must be [B, Hkv] or an int")
            self.bc = block_counts.to(device=dev, dtype=torch.int32).contiguous()
        self.sl = seq_lens.to(device=dev, dtype=torch.int32).contiguous()
        if tuple(self.sl.shape) != (B,):
            raise ValueError("seq_lens must be [B]")
        self.q, self.k, self.v = q.contiguous(), k_cache.contiguous(), v_cache.contiguous()
        self.out = torch.empty_like(self.q) if out is None else out
        self.lse = lse if lse is not None else (
            torch.empty((B, Hq), dtype=torch.float32, device=dev) if return_lse else None)
        self.dims = _dims(B, Smax, Hq, Hkv, D, S, DTYPE_BF16)
        self.scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        self.block_size = int(block_size)
        self.stream = _stream(torch, dev)
        self._p = [_ptr(getattr(self, n)) for n in ("q", "k", "v", "sl", "bi", "bc", "out", "lse")]

    def run(self):
        q, k, v, sl, bi, bc, out, lse = self._p
        _check(self.lib.nsa_decode(ctypes.byref(self.dims), q, k, v, sl, bi, bc, self.block_size, self.scale,
                                   out, lse, self.stream))
        return self.out, self.lse


def decode(q, k_cache, v_cache, seq_lens, block_indices, block_counts, block_size: int = 64,
           scale: float | None = None, out=None, lse=None, return_lse: bool = True):
    """Decode step on the GPU (see ``Decode``).  Returns (out, lse)."""
    return Decode(q, k_cache, v_cache, seq_lens, block_indices, block_counts, block_size, scale, out, lse,
                  return_lse).run()


def bwd(q, k, v, out, lse, dout, block_indices, block_counts, block_size: int = 64,
        scale: float | None = None, workspace=None, check: bool = True):
    """Gradients of ``fwd`` (``nsa_bwd``; fixed-length, bf16): returns
    (dq, dk, dv) as float32 tensors shaped like q, k, v.  ``out`` and ``lse``
    are the forward's results for the same inputs and indices.  With
    ``check`` (the default) the device status word is read after the launch
    (``nsa_bwd_device_status``: waits for the stream) and a non-zero word
    raises NsaDeviceError."""
    import torch
    lib = load_library()
    (q, k, v, bi, bc, _, B, T, Hq, Hkv, D, S, code) = _prepare(q, k, v, block_indices, block_counts, None,
                                                                int(block_size), "token")
    if code != DTYPE_BF16:
        raise ValueError("the backward takes bf16 inputs")
    out, dout = out.contiguous(), dout.contiguous()
    if out.shape != q.shape or dout.shape != q.shape or out.dtype != q.dtype or dout.dtype != q.dtype:
        raise ValueError("out and dout must match q")
    lse = lse.to(torch.float32).contiguous()
    if tuple(lse.shape) != (B, T, Hq):
        raise ValueError("lse must be [B, T, Hq]")
    dims = _dims(B, T, Hq, Hkv, D, S, code)
    need = max(int(lib.nsa_bwd_workspace_size(ctypes.byref(dims), int(block_size))), 256)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    ws_bytes = workspace.numel() * workspace.element_size()
    stream = _stream(torch, q.device)
    _check(lib.nsa_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(bi),
                       _ptr(bc), int(block_size), scale, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                       ws_bytes, stream))
    if check:
        word = ctypes.c_int32(0)
        _check(lib.nsa_bwd_device_status(ctypes.byref(dims), int(block_size), _ptr(workspace), ws_bytes, stream,
                                         ctypes.byref(word)))
        if word.value != 0:
            raise NsaDeviceError(word.value, f"backward device status {word.value:#x}: a bounded wait inside "
                                             "the dq gather expired (NSA_DEVICE_WAIT_EXPIRED); dq, dk and dv "
                                             "are incomplete")
    return dq, dk, dv
