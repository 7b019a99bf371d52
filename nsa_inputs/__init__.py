"""Seeded synthetic inputs for native sparse attention (NSA) forward.

This module only draws numbers and lays them out.  It holds none of the
attention arithmetic: both the CPU oracle (``oracle/``) and the HIP library
(``block_index_sparse_amd``) consume what it produces, and neither imports
the other.

Random numbers
--------------
Every array is drawn from a counter-based generator, so its bytes depend only
on (seed, stream, element counter) and never on numpy's Generator version:

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): the n-th output of a stream whose state starts at
  ``base`` is ``mix(base + (n + 1) * 0x9E3779B97F4A7C15)``.
* ``base(seed, stream) = mix(seed * 0x9E3779B97F4A7C15 + stream * 0xD1B54A32D192ED03)``.
* A uniform in [0, 1) is the top 53 bits of a 64-bit output times 2**-53.
* Normals use the Box-Muller transform (Box and Muller, Ann. Math. Statist.
  29, 1958): outputs 2m and 2m+1 give u1 = 1 - U(2m) in (0, 1] and
  u2 = U(2m+1); element 2m is r*cos(2*pi*u2), element 2m+1 is r*sin(2*pi*u2),
  r = sqrt(-2 ln u1).  Computed in float64, rounded to float32, then to
  bfloat16 with round-to-nearest-even where the workload is bf16.
* A random subset without replacement (and a random order) comes from giving
  every candidate a 64-bit hash key and taking the smallest keys.

Workloads
---------
The five named workloads follow the synthetic configurations of the native
sparse attention forward (ejKernel ``native_sparse_attention`` API page,
"Parameters"): q/k/v ``[B, T, H, D]``, per-token ``block_indices
[B, T, Hkv, S]`` and ``block_counts [B, T, Hkv]`` (the type annotations of
``run`` / ``native_sparse_attention``), optional ``cu_seqlens``.  The index
patterns are the readings written down in the design notes (sink / local /
random blocks, dense causal, varlen relative blocks).

Query-block workloads (``index_layout == "query_block"``) carry the layout of
the page's ``block_indices`` parameter description instead: one row per
query block, ``block_indices [B, Hkv, NQB, S]`` and ``block_counts
[B, Hkv, NQB]``, drawn with the same patterns, the query block playing the
part of the token's own block.
"""
from __future__ import annotations

import hashlib
import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload", "make_config", "make_workload", "CONFIG_NAMES",
    "uniform", "normal", "hash_u64", "to_bf16_bits", "bf16_bits_to_f32",
    "sha256_arrays", "varlen_lengths", "to_torch", "make_qblock_workload",
    "DecodeWorkload", "make_decode_workload", "make_decode_config", "DECODE_NAME",
]

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_STREAM_MUL = np.uint64(0xD1B54A32D192ED03)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# stream ids, one per array kind
STREAM_Q, STREAM_K, STREAM_V, STREAM_IDX, STREAM_CNT, STREAM_LEN, STREAM_ORDER = range(7)


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _base(seed: int, stream: int) -> np.uint64:
    with np.errstate(over="ignore"):
        s = np.array([seed], dtype=np.uint64) * _GOLDEN + np.array([stream], dtype=np.uint64) * _STREAM_MUL
        return _mix(s)[0]


def hash_u64(seed: int, stream: int, counters: np.ndarray) -> np.ndarray:
    """64-bit SplitMix64 outputs for the given element counters."""
    c = np.asarray(counters, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(_base(seed, stream) + (c + np.uint64(1)) * _GOLDEN)


def uniform(seed: int, stream: int, counters: np.ndarray) -> np.ndarray:
    """Uniform float64 in [0, 1) for the given counters."""
    h = hash_u64(seed, stream, counters)
    return (h >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def _normal_chunk(seed: int, stream: int, start: int, stop: int) -> np.ndarray:
    # elements [start, stop) with start even
    n_pairs = (stop - start + 1) // 2
    m = np.arange(start // 2, start // 2 + n_pairs, dtype=np.uint64)
    u1 = 1.0 - uniform(seed, stream, m * np.uint64(2))
    u2 = uniform(seed, stream, m * np.uint64(2) + np.uint64(1))
    r = np.sqrt(-2.0 * np.log(u1))
    th = (2.0 * math.pi) * u2
    out = np.empty(2 * n_pairs, dtype=np.float64)
    out[0::2] = r * np.cos(th)
    out[1::2] = r * np.sin(th)
    return out[: stop - start].astype(np.float32)


def normal(seed: int, stream: int, n: int, chunk: int = 1 << 22, threads: int = 8) -> np.ndarray:
    """n standard normals (float32, rounded from float64), element i at counter i."""
    out = np.empty(n, dtype=np.float32)
    starts = list(range(0, n, chunk))

    def work(s):
        e = min(n, s + chunk)
        out[s:e] = _normal_chunk(seed, stream, s, e)

    if len(starts) <= 1:
        for s in starts:
            work(s)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, starts))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def sha256_arrays(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        if a is None:
            h.update(b"none")
            continue
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode())
        h.update(str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()


@dataclass
class Workload:
    """One seeded NSA forward problem.

    ``q``, ``k``, ``v`` hold float32 values; for a bf16 workload they are the
    exact widened bf16 values and ``q_bits``/``k_bits``/``v_bits`` hold the
    bf16 bit patterns.  Tokens are laid out ``[B, T, ...]``; a varlen
    workload has ``B == 1``, ``T`` = total packed tokens and ``cu_seqlens``.
    """
    name: str
    dtype: str                     # "f32" or "bf16"
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    S: int
    scale: float                   # a float32 value
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    block_indices: np.ndarray      # int32 [B, T, Hkv, S]  (query_block: [B, Hkv, NQB, S])
    block_counts: np.ndarray       # int32 [B, T, Hkv]     (query_block: [B, Hkv, NQB])
    cu_seqlens: np.ndarray | None = None   # int32 [N + 1]
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None
    meta: dict = field(default_factory=dict)
    index_layout: str = "token"    # "token" or "query_block"

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def seqlens(self) -> list[int]:
        if self.cu_seqlens is None:
            return [self.T] * self.B
        c = self.cu_seqlens
        return [int(c[i + 1] - c[i]) for i in range(len(c) - 1)]

    def digest(self) -> str:
        return sha256_arrays(self.q_bits if self.dtype == "bf16" else self.q,
                             self.k_bits if self.dtype == "bf16" else self.k,
                             self.v_bits if self.dtype == "bf16" else self.v,
                             self.block_indices, self.block_counts, self.cu_seqlens)


# ----------------------------------------------------------------------------
# index patterns
# ----------------------------------------------------------------------------

def _smallest_keys(keys: np.ndarray, k: int) -> np.ndarray:
    """Column ids of the k smallest keys per row, in increasing key order."""
    k = min(k, keys.shape[1])
    if k <= 0:
        return np.zeros((keys.shape[0], 0), dtype=np.int64)
    if k < keys.shape[1]:
        part = np.argpartition(keys, k - 1, axis=1)[:, :k]
    else:
        part = np.tile(np.arange(keys.shape[1]), (keys.shape[0], 1))
    sub = np.take_along_axis(keys, part, axis=1)
    order = np.argsort(sub, axis=1, kind="stable")
    return np.take_along_axis(part, order, axis=1)


_INVALID_KEY = np.uint64(0xFFFFFFFFFFFFFFFF)


def _random_subset(seed, row_ids, lo, hi, count, nb_max):
    """Per row r: `count[r]` distinct values drawn uniformly from [lo[r], hi[r]]
    (empty if hi < lo), in random order.  Returns (vals[R, maxcount], n[R])."""
    R = len(row_ids)
    n_avail = np.maximum(hi - lo + 1, 0)
    n_take = np.minimum(count, n_avail)
    kmax = int(n_take.max()) if R else 0
    vals = np.full((R, max(kmax, 1)), -1, dtype=np.int64)
    if kmax == 0:
        return vals[:, :0], n_take
    x = np.arange(nb_max, dtype=np.int64)
    ctr = (row_ids.astype(np.uint64)[:, None] * np.uint64(nb_max) + x.astype(np.uint64)[None, :])
    keys = hash_u64(seed, STREAM_IDX, ctr)
    ok = (x[None, :] >= lo[:, None]) & (x[None, :] <= hi[:, None])
    keys = np.where(ok, keys, _INVALID_KEY)
    cols = _smallest_keys(keys, kmax)
    j = np.arange(kmax)[None, :]
    vals = np.where(j < n_take[:, None], cols, -1)
    return vals, n_take


def _rows_for(seqlens, Hkv, block_size):
    """Row = (packed token, kv head).  Returns token-relative position, seq id."""
    pos = np.concatenate([np.arange(L, dtype=np.int64) for L in seqlens]) if seqlens else np.zeros(0, np.int64)
    seq = np.concatenate([np.full(L, i, dtype=np.int64) for i, L in enumerate(seqlens)]) if seqlens else np.zeros(0, np.int64)
    Ttot = len(pos)
    pos_r = np.repeat(pos, Hkv)
    seq_r = np.repeat(seq, Hkv)
    row_ids = np.arange(Ttot * Hkv, dtype=np.int64)
    own = pos_r // block_size
    return row_ids, pos_r, seq_r, own


def _build_rows(pattern, seqlens, Hkv, block_size, S, seed, counts_mode, chunk_rows=16384):
    """Index rows for every (packed token, kv head).  Returns (idx[R,S], counts[R])."""
    row_ids, pos, seq, own = _rows_for(seqlens, Hkv, block_size)
    nb_max = max(1, max((L + block_size - 1) // block_size for L in seqlens)) if seqlens else 1
    return _rows_from_own(pattern, row_ids, own, nb_max, S, seed, counts_mode, chunk_rows)


def _rows_from_own(pattern, row_ids, own, nb_max, S, seed, counts_mode, chunk_rows=16384):
    """Index rows given each row's id (its random stream) and own block."""
    R = len(row_ids)
    idx = np.full((R, S), -1, dtype=np.int32)
    valid = np.zeros(R, dtype=np.int64)
    for s in range(0, R, chunk_rows):
        e = min(R, s + chunk_rows)
        rid, o = row_ids[s:e], own[s:e]
        n = e - s
        if pattern == "dense":
            j = np.arange(S)[None, :]
            blk = np.where(j <= o[:, None], j, -1)
            idx[s:e] = blk
            valid[s:e] = np.minimum(o + 1, S)
        elif pattern == "local_random":
            # own, own-1, own-2, own-3 (those >= 0, at most S), then random
            # distinct blocks from [0, own-4]
            nl = min(4, S)
            loc = o[:, None] - np.arange(nl)[None, :]
            loc = np.where(loc >= 0, loc, -1)
            nloc = np.minimum(o + 1, nl)
            rnd, nr = _random_subset(seed, rid, np.zeros(n, np.int64), o - nl, np.full(n, S - nl), nb_max)
            row = np.full((n, S), -1, dtype=np.int64)
            row[:, :nl] = loc
            # loc is already left-aligned: entries >= nloc are -1
            for jj in range(rnd.shape[1]):
                col = nloc + jj
                m = jj < nr
                row[np.nonzero(m)[0], col[m]] = rnd[m, jj]
            idx[s:e] = row[:, :S]
            valid[s:e] = nloc + nr
        elif pattern == "sink_local_random":
            # block 0, then own, own-1, own-2, then random distinct from [1, own-3];
            # duplicates removed keeping the first occurrence
            row = np.full((n, S), -1, dtype=np.int64)
            cand = np.stack([np.zeros(n, np.int64), o, o - 1, o - 2], axis=1)
            rnd, nr = _random_subset(seed, rid, np.ones(n, np.int64), o - 3, np.full(n, S - 4), nb_max)
            cnt = np.zeros(n, dtype=np.int64)
            rows_i = np.arange(n)
            for jj in range(4):
                c = cand[:, jj]
                dup = np.zeros(n, dtype=bool)
                for prev in range(jj):
                    dup |= cand[:, prev] == c
                ok = (c >= 0) & ~dup
                row[rows_i[ok], cnt[ok]] = c[ok]
                cnt += ok
            for jj in range(rnd.shape[1]):
                m = jj < nr
                row[rows_i[m], cnt[m]] = rnd[m, jj]
                cnt += m
            idx[s:e] = row
            valid[s:e] = cnt
        elif pattern == "shuffled":
            # own plus (valid-1) random distinct from [0, own-1], in random order
            nval = np.minimum(S, o + 1)
            rnd, nr = _random_subset(seed, rid, np.zeros(n, np.int64), o - 1, nval - 1, nb_max)
            row = np.full((n, S), -1, dtype=np.int64)
            row[:, 0] = o
            for jj in range(rnd.shape[1]):
                m = jj < nr
                row[np.nonzero(m)[0], 1 + jj] = rnd[m, jj]
            # random order of the valid entries: sort by hash keys of (row, slot)
            ctr = rid.astype(np.uint64)[:, None] * np.uint64(S) + np.arange(S, dtype=np.uint64)[None, :]
            keys = hash_u64(seed, STREAM_ORDER, ctr)
            keys = np.where(np.arange(S)[None, :] < nval[:, None], keys, _INVALID_KEY)
            order = np.argsort(keys, axis=1, kind="stable")
            idx[s:e] = np.take_along_axis(row, order, axis=1)
            valid[s:e] = nval
        else:
            raise ValueError(f"unknown index pattern {pattern!r}")
    if counts_mode == "full":
        counts = valid.astype(np.int32)
    elif counts_mode == "uniform":
        u = uniform(seed, STREAM_CNT, row_ids.astype(np.uint64))
        counts = (1 + np.floor(u * valid)).astype(np.int32)
        counts = np.minimum(counts, valid).astype(np.int32)
    else:
        raise ValueError(counts_mode)
    return idx, counts


def varlen_lengths(seed: int, n_seqs: int = 8, lo: int = 512, hi: int = 8192, max_total: int = 32768):
    """Sequence lengths ~ U[lo, hi] (inclusive), redrawn as a whole until the sum is <= max_total."""
    attempt = 0
    while True:
        ctr = np.arange(attempt * n_seqs, (attempt + 1) * n_seqs, dtype=np.uint64)
        u = uniform(seed, STREAM_LEN, ctr)
        lens = lo + np.floor(u * (hi - lo + 1)).astype(np.int64)
        if lens.sum() <= max_total:
            return [int(x) for x in lens]
        attempt += 1
        if attempt > 100000:
            raise RuntimeError("rejection sampling did not converge")


def to_torch(w: Workload, device="cuda"):
    """Device copies (q, k, v, block_indices, block_counts, cu_seqlens) of a
    workload as torch tensors; bf16 values are moved as their bit patterns."""
    import torch
    if w.dtype == "bf16":
        def t(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)
        q, k, v = t(w.q_bits), t(w.k_bits), t(w.v_bits)
    else:
        q, k, v = (torch.from_numpy(np.ascontiguousarray(a)).to(device) for a in (w.q, w.k, w.v))
    bi = torch.from_numpy(np.ascontiguousarray(w.block_indices)).to(device)
    bc = torch.from_numpy(np.ascontiguousarray(w.block_counts)).to(device)
    cu = None if w.cu_seqlens is None else torch.from_numpy(w.cu_seqlens).to(device)
    return q, k, v, bi, bc, cu


def make_workload(name, dtype, seqlens, Hq, Hkv, D, block_size, S, pattern, counts_mode,
                  seed, varlen=False, value_scale=1.0, scale=None) -> Workload:
    """Generic seeded workload.  ``seqlens``: for fixed length, ``[T] * B``."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if varlen:
        B, T = 1, int(sum(seqlens))
        cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(seqlens)
    else:
        if len(set(seqlens)) != 1:
            raise ValueError("fixed-length workload needs equal lengths")
        B, T = len(seqlens), int(seqlens[0])
        cu = None
    ntok = B * T

    def gen(stream, H):
        x = normal(seed, stream, ntok * H * D).reshape(B, T, H, D)
        if value_scale != 1.0:
            x *= np.float32(value_scale)
        if dtype == "bf16":
            bits = to_bf16_bits(x)
            return bf16_bits_to_f32(bits).reshape(x.shape), bits.reshape(x.shape)
        return x, None

    q, qb = gen(STREAM_Q, Hq)
    k, kb = gen(STREAM_K, Hkv)
    v, vb = gen(STREAM_V, Hkv)
    idx, cnt = _build_rows(pattern, list(seqlens), Hkv, block_size, S, seed, counts_mode)
    idx = idx.reshape(B, T, Hkv, S)
    cnt = cnt.reshape(B, T, Hkv)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    return Workload(name=name, dtype=dtype, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size, S=S,
                    scale=float(np.float32(scale)), q=q, k=k, v=v, block_indices=idx, block_counts=cnt,
                    cu_seqlens=cu, q_bits=qb, k_bits=kb, v_bits=vb,
                    meta={"pattern": pattern, "counts_mode": counts_mode, "seed": seed,
                          "value_scale": value_scale})


CONFIG_NAMES = [
    "c0_tiny_fp32",
    "c1_bf16_gqa16_T4096",
    "c2_bf16_dense_causal_T2048",
    "c3_bf16_long_T32768",
    "c4_bf16_varlen_8seq",
]


def make_config(i: int, seed: int | None = None) -> Workload:
    """The five named workloads (seed defaults to the config number)."""
    s = i if seed is None else seed
    if i == 0:
        return make_workload(CONFIG_NAMES[0], "f32", [256], 4, 1, 64, 32, 4, "shuffled", "uniform", s)
    if i == 1:
        return make_workload(CONFIG_NAMES[1], "bf16", [4096] * 2, 32, 2, 128, 64, 16, "local_random", "full", s)
    if i == 2:
        return make_workload(CONFIG_NAMES[2], "bf16", [2048] * 4, 16, 16, 128, 64, 32, "dense", "full", s)
    if i == 3:
        return make_workload(CONFIG_NAMES[3], "bf16", [32768], 64, 4, 128, 64, 16, "sink_local_random", "full", s,
                             value_scale=0.5)
    if i == 4:
        lens = varlen_lengths(s)
        return make_workload(CONFIG_NAMES[4], "bf16", lens, 32, 2, 128, 64, 16, "local_random", "uniform", s,
                             varlen=True)
    if i == 5:
        return make_qblock_workload(EXTRA_NAMES[5], "bf16", 1, 32768, 64, 4, 128, 64, 16, "sink_local_random",
                                    "full", s, value_scale=0.5)
    if i == 6:
        return make_qblock_workload(EXTRA_NAMES[6], "bf16", 1, 32768, 64, 4, 64, 128, 8, "sink_local_random",
                                    "full", s, value_scale=0.5)
    if i == 7:
        return make_qblock_workload(EXTRA_NAMES[7], "bf16", 1, 32768, 64, 4, 128, 32, 32, "sink_local_random",
                                    "full", s, value_scale=0.5)
    raise ValueError(f"no config {i}")


# Workloads beyond the five named ones, by number: the long-context shapes
# with one index row per query block, at block size 64 (D = 128, S = 16),
# 128 (D = 64, S = 8) and 32 (D = 128, S = 32): the same 1024 selected keys
# per row at each block size.
EXTRA_NAMES = {5: "c3q_bf16_qblock_T32768", 6: "c3q_bf16_qblock_bs128_d64_T32768",
               7: "c3q_bf16_qblock_bs32_T32768"}


def workload_name(i: int) -> str:
    return CONFIG_NAMES[i] if i < len(CONFIG_NAMES) else EXTRA_NAMES[i]


def make_qblock_workload(name, dtype, B, T, Hq, Hkv, D, block_size, S, pattern, counts_mode, seed,
                         value_scale=1.0, scale=None) -> Workload:
    """Seeded fixed-length workload whose indices hold one row per query
    block: ``block_indices [B, Hkv, NQB, S]``, ``block_counts [B, Hkv, NQB]``,
    NQB = ceil(T / block_size).  The rows are drawn with the token patterns,
    query block qb taking the part of the own block."""
    w = make_workload(name, dtype, [T] * B, Hq, Hkv, D, block_size, 1, "dense", "full", seed,
                      value_scale=value_scale, scale=scale)
    nqb = (T + block_size - 1) // block_size
    # one pseudo-token per query block with block size 1: its own block is qb
    idx, cnt = _build_rows(pattern, [nqb] * B, Hkv, 1, S, seed, counts_mode)
    w.block_indices = np.ascontiguousarray(idx.reshape(B, nqb, Hkv, S).transpose(0, 2, 1, 3))
    w.block_counts = np.ascontiguousarray(cnt.reshape(B, nqb, Hkv).transpose(0, 2, 1))
    w.S = S
    w.index_layout = "query_block"
    w.meta.update({"pattern": pattern, "counts_mode": counts_mode, "index_layout": "query_block"})
    return w


# ----------------------------------------------------------------------------
# decode: one query token per sequence against its KV cache
# ----------------------------------------------------------------------------

STREAM_DEC_LEN = 8


@dataclass
class DecodeWorkload:
    """The newest token of each of B sequences against a bf16 KV cache of
    Smax rows per sequence: q ``[B, Hq, D]``, k/v ``[B, Smax, Hkv, D]``,
    ``seq_lens [B]`` (the query sits at position len - 1), and the query's
    selected blocks ``block_indices [B, Hkv, S]``, ``block_counts
    [B, Hkv]``.  float32 arrays hold the exact bf16 values; ``*_bits`` the
    bf16 bit patterns."""
    name: str
    B: int
    Smax: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    S: int
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    seq_lens: np.ndarray
    block_indices: np.ndarray
    block_counts: np.ndarray
    q_bits: np.ndarray
    k_bits: np.ndarray
    v_bits: np.ndarray
    meta: dict = field(default_factory=dict)
    dtype: str = "bf16"

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def digest(self) -> str:
        return sha256_arrays(self.q_bits, self.k_bits, self.v_bits, self.seq_lens, self.block_indices,
                             self.block_counts)


def make_decode_workload(name, B, Smax, len_lo, len_hi, Hq, Hkv, D, block_size, S, pattern, counts_mode,
                         seed, value_scale=1.0, scale=None) -> DecodeWorkload:
    """Seeded decode problem: lengths ~ U[len_lo, len_hi] (inclusive, capped at
    Smax), normal q/k/v rounded to bf16, and index rows drawn with the token
    patterns for the query position len - 1."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    u = uniform(seed, STREAM_DEC_LEN, np.arange(B, dtype=np.uint64))
    lens = np.minimum(len_lo + np.floor(u * (len_hi - len_lo + 1)).astype(np.int64), Smax).astype(np.int32)

    def gen(stream, shape):
        x = normal(seed, stream, int(np.prod(shape))).reshape(shape)
        if value_scale != 1.0:
            x *= np.float32(value_scale)
        bits = to_bf16_bits(x)
        return bf16_bits_to_f32(bits).reshape(shape), bits.reshape(shape)

    q, qb = gen(STREAM_Q, (B, Hq, D))
    k, kb = gen(STREAM_K, (B, Smax, Hkv, D))
    v, vb = gen(STREAM_V, (B, Smax, Hkv, D))
    own = np.repeat(np.maximum(lens.astype(np.int64) - 1, 0) // block_size, Hkv)
    nb_max = max(1, (Smax + block_size - 1) // block_size)
    idx, cnt = _rows_from_own(pattern, np.arange(B * Hkv, dtype=np.int64), own, nb_max, S, seed, counts_mode)
    idx = idx.reshape(B, Hkv, S)
    cnt = cnt.reshape(B, Hkv)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    return DecodeWorkload(name=name, B=B, Smax=Smax, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size, S=S,
                          scale=float(np.float32(scale)), q=q, k=k, v=v, seq_lens=lens, block_indices=idx,
                          block_counts=cnt, q_bits=qb, k_bits=kb, v_bits=vb,
                          meta={"pattern": pattern, "counts_mode": counts_mode, "seed": seed,
                                "lens": [len_lo, len_hi], "value_scale": value_scale})


DECODE_NAME = "d0_bf16_decode_B128_S8192"


def make_decode_config(seed: int = 6) -> DecodeWorkload:
    """Decode workload of the long-context shapes: 128 sequences with
    lengths ~ U[1024, 8192] in a cache of 8192 rows, Hq=64, Hkv=4, D=128,
    block_size=64, S=16 (sink, local and random blocks), 0.5 N(0, 1) values."""
    return make_decode_workload(DECODE_NAME, 128, 8192, 1024, 8192, 64, 4, 128, 64, 16, "sink_local_random",
                                "full", seed, value_scale=0.5)


def decode_to_torch(w: DecodeWorkload, device="cuda"):
    """Device copies (q, k, v, seq_lens, block_indices, block_counts)."""
    import torch

    def t(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)
    return (t(w.q_bits), t(w.k_bits), t(w.v_bits), torch.from_numpy(w.seq_lens).to(device),
            torch.from_numpy(np.ascontiguousarray(w.block_indices)).to(device),
            torch.from_numpy(np.ascontiguousarray(w.block_counts)).to(device))
