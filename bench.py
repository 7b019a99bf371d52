"""Benchmark of the native sparse attention forward on one MI355X.

A step is one whole forward call (scheduler + attention kernel) over the
seeded long-context workload: B=1, T=32768, Hq=64, Hkv=4 (GQA group 16),
D=128, block_size=64, S=16 (one sink block, three local blocks, twelve random
earlier blocks per token and kv head), bf16 inputs, inputs resident in HBM.

value = useful TFLOP/s = 4 * D * sum over (token, query head) of the visible
keys |M_t|, divided by the time per step.  The roofline entry describes the
attention kernel alone (its duration is measured with HIP events recorded on
the launch stream around that kernel inside every timed step).  The CPU
baseline times the fp64 oracle on a bounded token sample of the same
workload on the host's cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--no-cpu-baseline] [--cold]

--config 0..4 selects the other named workloads (parity cases, not the
headline); --config 5 is the same long-context shape with one index row per
query block (nsa_fwd_qblock); --config 6 and 7 repeat it at block sizes
128 (D = 64) and 32.  --decode measures the decode step
(nsa_decode: 128 sequences' newest tokens against a bf16 cache of 8192 rows,
Hq=64, Hkv=4, D=128, bs=64, S=16) against the HBM roofline.  --backward
measures nsa_bwd (dq, dk, dv) on --config's workload: useful FLOP = 10 D per
visible (token, query head, key) triple (S, dP, dQ, dK, dV).

HBM traffic of the attention kernel comes from two rocprofv3 counter runs
(FETCH_SIZE, then WRITE_SIZE) of this script, each scaled by what the same
counter reads for a plain copy kernel of known size (``--calibrate-copy``);
``--traffic-summary`` turns the four runs into ``profiles/`` JSON, which is
reported while the kernel sources still hash to what was profiled.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-attn fwd useful TFLOP/s + % of bf16 MFMA peak, T=32k 1 GPU"
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 dense bf16 FLOP/clk/CU x 2.4 GHz
PEAK_F32_TFLOPS = 157.3     # dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 1 << 30         # bytes read (and written) by the calibration copy
CSRC = os.path.join(ROOT, "block_index_sparse_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


FWD_KERNEL = "fwd_bf16_ring_kernel"   # the attention kernel of the bf16 forward

KERNEL_SOURCES = {
    # the forward kernel, the helpers it includes, the host code that sizes its
    # tiles and the scheduler that orders its work (the order moves its traffic)
    "fwd": ("nsa_fwd.hip", "nsa_device.h", "nsa_internal.h", "nsa_plan.h", "nsa_api.hip", "nsa_sched.hip"),
    "decode": ("nsa_decode.hip", "nsa_device.h", "nsa_internal.h", "nsa_plan.h"),
}


def kernel_source_digest(kind: str = "fwd") -> str:
    """sha256 over the sources that decide what a kernel does (comments and
    layout stripped: they do not change the kernel)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        h.update(f.encode())
        with open(os.path.join(CSRC, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def _kind(workload: str) -> str:
    return "decode" if workload.startswith("d") else "fwd"


def traffic_path(workload: str) -> str:
    prefix = "nsa_decode_traffic" if _kind(workload) == "decode" else "nsa_fwd_traffic"
    return os.path.join(PROFILES, f"{prefix}_{workload}.json")


def read_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel sources changed since it was taken."""
    p = traffic_path(workload)
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        t = json.load(fh)
    if t.get("kernel_source_sha256") != kernel_source_digest(_kind(workload)):
        return None
    return t["traffic_bytes_per_launch"]


def _pmc_rows(run_dir: str, counter: str):
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    out = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def _mean_for(rows, needle: str, skip: str = "\0") -> tuple:
    vals = [v for n, v in rows if needle in n and skip not in n]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel named like {needle!r}")
    return float(np.mean(vals)), len(vals)


def traffic_summary(workload: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str,
                    copy_write_dir: str, kernel: str):
    """Write the traffic summary of a workload (profiles/nsa_fwd_traffic_<workload>.json,
    or nsa_decode_traffic_<workload>.json for the decode step) from four --pmc runs."""
    copy_kib = COPY_BYTES / 1024.0
    cf, _ = _mean_for(_pmc_rows(copy_fetch_dir, "FETCH_SIZE"), "elementwise", skip="Fill")
    cw, _ = _mean_for(_pmc_rows(copy_write_dir, "WRITE_SIZE"), "elementwise", skip="Fill")
    kf, nf = _mean_for(_pmc_rows(fetch_dir, "FETCH_SIZE"), kernel)
    kw, nw = _mean_for(_pmc_rows(write_dir, "WRITE_SIZE"), kernel)
    ff, fw = copy_kib / cf, copy_kib / cw
    res = {
        "workload": workload, "kernel": kernel,
        "kernel_source_sha256": kernel_source_digest(_kind(workload)),
        "fetch_kib_per_launch_raw": kf, "write_kib_per_launch_raw": kw, "launches": [nf, nw],
        "copy_bytes": COPY_BYTES, "copy_fetch_kib_raw": cf, "copy_write_kib_raw": cw,
        "fetch_scale": ff, "write_scale": fw,
        "fetch_bytes_per_launch": kf * 1024 * ff, "write_bytes_per_launch": kw * 1024 * fw,
        "traffic_bytes_per_launch": kf * 1024 * ff + kw * 1024 * fw,
    }
    with open(traffic_path(workload), "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    print(json.dumps(res))


def counters_path(workload: str) -> str:
    prefix = "nsa_decode_counters" if _kind(workload) == "decode" else "nsa_fwd_counters"
    return os.path.join(PROFILES, f"{prefix}_{workload}.json")


def counters_summary(workload: str, sq_dir: str, ta_dir: str, kernel: str, n_cus: int = 256,
                     n_xcds: int = 8, simds_per_cu: int = 4):
    """Unit utilisations of a kernel from two rocprofv3 --pmc runs (SQ block:
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_LDS_IDX_ACTIVE, GRBM_GUI_ACTIVE, ...; TA
    block: TA_TA_BUSY, GRBM_GUI_ACTIVE), written next to the traffic record.
    GRBM_GUI_ACTIVE sums the cycles of the 8 XCDs; busy counters sum over
    CUs (SIMDs for the MFMA pipe)."""
    def means(d):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit(f"no counter_collection.csv under {d}")
        acc = {}
        for r in csv.DictReader(open(f[0])):
            if kernel in r["Kernel_Name"]:
                acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        return {k: float(np.mean(v)) for k, v in acc.items()}
    sq, ta = means(sq_dir), means(ta_dir)
    cyc_sq = sq["GRBM_GUI_ACTIVE"] / n_xcds
    cyc_ta = ta["GRBM_GUI_ACTIVE"] / n_xcds
    res = {
        "workload": workload, "kernel": kernel, "kernel_source_sha256": kernel_source_digest(_kind(workload)),
        "gpu_cycles": cyc_sq,
        "mfma_busy_frac": sq["SQ_VALU_MFMA_BUSY_CYCLES"] / (n_cus * simds_per_cu) / cyc_sq,
        "lds_active_frac": sq["SQ_LDS_IDX_ACTIVE"] / n_cus / cyc_sq,
        "lds_bank_conflicts": sq.get("SQ_LDS_BANK_CONFLICT"),
        "vmem_path_busy_frac": ta["TA_TA_BUSY"] / n_cus / cyc_ta,
        "raw": {"sq": sq, "ta": ta},
    }
    with open(counters_path(workload), "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    print(json.dumps(res))


def read_counters(workload: str):
    """Unit utilisations from the committed counter record, or None when
    there is none or the kernel sources changed since it was taken."""
    p = counters_path(workload)
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        t = json.load(fh)
    if t.get("kernel_source_sha256") != kernel_source_digest(_kind(workload)):
        return None
    return {k: round(t[k], 4) for k in ("mfma_busy_frac", "lds_active_frac", "vmem_path_busy_frac")}


def calibrate_copy():
    """A plain elementwise copy of COPY_BYTES (x * 1 into a second buffer)."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)   # contents irrelevant
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}), flush=True)


def visible_keys_per_row(w) -> np.ndarray:
    """|M_t| for every (packed token, kv head): keys of the distinct listed
    blocks 0 <= j <= own, the own block cut at the token's position."""
    bi, bc = w.block_indices, w.block_counts
    if getattr(w, "index_layout", "token") == "query_block":
        # one row per query block: token t reads row t // block_size
        qb = np.arange(w.T) // w.block_size
        bi, bc = bi[:, :, qb, :].transpose(0, 2, 1, 3), bc[:, :, qb].transpose(0, 2, 1)
    B, T, Hkv, S = bi.shape
    bi = bi.reshape(-1, Hkv, S).astype(np.int64)
    n = np.clip(bc.reshape(-1, Hkv), 0, S)
    if w.cu_seqlens is None:
        pos = np.tile(np.arange(T), B)
    else:
        pos = np.concatenate([np.arange(L) for L in w.seqlens])
    own = pos // w.block_size
    keep = (np.arange(S)[None, None, :] < n[..., None]) & (bi >= 0) & (bi <= own[:, None, None])
    vals = np.where(keep, bi, -1)
    vals = np.sort(vals, axis=-1)
    first = np.ones_like(vals, dtype=bool)
    first[..., 1:] = vals[..., 1:] != vals[..., :-1]
    distinct = first & (vals >= 0)
    full = distinct & (vals < own[:, None, None])
    diag = distinct & (vals == own[:, None, None])
    part = (pos - own * w.block_size + 1)[:, None]
    return full.sum(-1) * w.block_size + diag.sum(-1) * part


def useful_flops(w, rows=None) -> int:
    m = visible_keys_per_row(w)
    if rows is not None:
        m = m[rows]
    return int(4 * w.D * w.G * int(m.sum()))


def algorithmic_bytes(w) -> int:
    """q, k, v, out, lse, indices and counts, each moved once."""
    el = 2 if w.dtype == "bf16" else 4
    ntok = w.B * w.T
    return int(ntok * w.Hq * w.D * el * 2 + 2 * ntok * w.Hkv * w.D * el + ntok * w.Hq * 4
               + w.block_indices.nbytes + w.block_counts.nbytes)


_THREADS = []


def _oracle_threads() -> int:
    """The host threads the oracle runs on, read once before any call that
    sets a different count (OpenMP keeps the last count it was given)."""
    import oracle
    if not _THREADS:
        _THREADS.append(oracle.max_threads())
    return _THREADS[0]


def cpu_model() -> str:
    """The host CPU's model name (first `model name` of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, seconds_target=12.0, seed=0):
    """Time the fp64 oracle on a seeded token sample sized to ~seconds_target."""
    import oracle
    rng = np.random.default_rng(seed)
    total = w.B * w.T
    threads = _oracle_threads()
    n = 32
    used = 0.0
    rows = None
    while True:
        rows = np.sort(rng.choice(total, size=min(n, total), replace=False))
        t0 = time.perf_counter()
        oracle.fwd_workload(w, tokens=rows, threads=threads)
        used = time.perf_counter() - t0
        if used >= seconds_target * 0.6 or n >= total:
            break
        n = min(total, int(n * min(8.0, max(1.2, seconds_target / max(used, 1e-3)))))
    fl = useful_flops(w, rows)
    return {"value": fl / used / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} of {total} tokens (seeded uniform sample, all {w.Hq} query heads), "
                      f"{used:.2f} s fp64 on {threads} OpenMP threads",
            "seconds": used, "tokens": int(len(rows)), "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


def bwd_cpu_baseline(w, dout, seconds_target=12.0, seed=0):
    """Time the gradient oracle's per-token dq (oracle.backward.dq_rows, fp64
    numpy, BLAS held to one thread) on a seeded token sample sized to
    ~seconds_target.  Only the dq share of the backward is timed: 6 D FLOP
    per visible (token, query head, key) triple of the 10 D the metric
    counts."""
    from threadpoolctl import threadpool_limits
    from oracle import backward as obwd
    rng = np.random.default_rng(seed)
    total = w.B * w.T
    m = visible_keys_per_row(w)                                     # [B * T, Hkv]
    n = 16
    with threadpool_limits(limits=1):
        while True:
            rows = np.sort(rng.choice(total, size=min(n, total), replace=False))
            t0 = time.perf_counter()
            obwd.dq_rows(w.q, w.k, w.v, dout, w.block_indices, w.block_counts, w.block_size, w.scale, rows)
            used = time.perf_counter() - t0
            if used >= seconds_target * 0.6 or n >= total:
                break
            n = min(total, int(n * min(8.0, max(1.2, seconds_target / max(used, 1e-3)))))
    fl = 6 * w.D * w.G * int(m[rows].sum())
    return {"value": fl / used / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"dq of {len(rows)} of {total} tokens (seeded uniform sample, all {w.Hq} query heads; "
                      f"6 D FLOP per visible triple, dq's share of the 10 D), {used:.2f} s fp64 numpy on one thread",
            "seconds": used, "tokens": int(len(rows))}


METRIC_DECODE = "sparse-attn decode step: useful HBM GB/s + % of HBM peak, 1 GPU"


def decode_visible_keys(w) -> np.ndarray:
    """|M| for every (sequence, kv head) of a decode workload: keys of the
    distinct listed blocks 0 <= j <= own, the own block cut at t = len - 1."""
    S = w.block_indices.shape[-1]
    t = np.clip(w.seq_lens.astype(np.int64), 0, w.Smax) - 1                  # [B]
    own = np.where(t >= 0, t // w.block_size, -1)[:, None, None]
    n = np.clip(w.block_counts, 0, S)[..., None]
    bi = w.block_indices.astype(np.int64)
    keep = (np.arange(S)[None, None, :] < n) & (bi >= 0) & (bi <= own)
    vals = np.sort(np.where(keep, bi, -1), axis=-1)
    first = np.ones_like(vals, dtype=bool)
    first[..., 1:] = vals[..., 1:] != vals[..., :-1]
    distinct = first & (vals >= 0)
    part = (t - np.maximum(own[:, 0, 0], 0) * w.block_size + 1)[:, None]
    return ((distinct & (vals < own)).sum(-1) * w.block_size + (distinct & (vals == own)).sum(-1) * part)


def decode_algorithmic_bytes(w, m) -> int:
    """K and V rows of the visible keys once per kv head, q, out, lse, the
    index rows and the lengths."""
    return int(int(m.sum()) * w.D * 2 * 2 + 2 * w.B * w.Hq * w.D * 2 + w.B * w.Hq * 4
               + w.block_indices.nbytes + w.block_counts.nbytes + w.seq_lens.nbytes)


def decode_bench(args):
    import torch
    import block_index_sparse_amd as nsa
    import nsa_inputs as ni
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    w = ni.make_decode_config()
    print(f"[bench] {w.name}: generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    q, k, v, sl, bi, bc = ni.decode_to_torch(w, dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    m = decode_visible_keys(w)
    flop = int(4 * w.D * w.G * int(m.sum()))
    nbytes = decode_algorithmic_bytes(w, m)

    call = nsa.Decode(q, k, v, sl, bi, bc, w.block_size, w.scale, out=out, lse=lse).run

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record()
        call()
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    avg = float(np.mean(ms))
    gbs = nbytes / (avg * 1e-3) / 1e9
    line = {
        "metric": METRIC_DECODE, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(avg, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Smax": w.Smax, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "block_size": w.block_size, "S": w.S, "useful_flop_per_step": flop,
                   "useful_tflops": round(flop / (avg * 1e-3) / 1e12, 3), "input_sha256": w.digest()[:16]},
        "roofline": {"bound": "hbm", "kernel": "decode_bf16_kernel", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": read_traffic(w.name), "counters": read_counters(w.name),
                     "kernel_ms_avg": round(avg, 4),
                     "kernel_ms_min": round(float(np.min(ms)), 4), "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        import oracle.decode as odec
        t1 = time.perf_counter()
        odec.decode_workload(w)
        sec = time.perf_counter() - t1
        line["cpu_baseline"] = {"value": round(nbytes / sec / 1e9, 3), "unit": "GB/s", "cores": 1,
                                "kind": "oracle", "sample": f"all {w.B} sequences, numpy fp64, {sec:.2f} s",
                                "seconds": sec}
    print(json.dumps(line), flush=True)


METRIC_BWD = "sparse-attn bwd useful TFLOP/s + % of bf16 MFMA peak, 1 GPU"


def backward_bench(args):
    import torch
    import block_index_sparse_amd as nsa
    import nsa_inputs as ni
    dev = torch.device("cuda:0")
    w = ni.make_config(args.config)
    if w.dtype != "bf16" or w.cu_seqlens is not None or w.index_layout != "token":
        sys.exit("bench --backward: the backward takes fixed-length bf16 workloads with per-token rows")
    q, k, v, bi, bc, _ = ni.to_torch(w, dev)
    f = nsa.Forward(q, k, v, bi, bc, w.block_size, w.scale)
    out, lse = f.run()
    x = ni.normal(200 + args.config, 9, w.B * w.T * w.Hq * w.D).reshape(w.B, w.T, w.Hq, w.D)
    dout = torch.from_numpy(ni.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
    need = nsa.load_library().nsa_bwd_workspace_size(__import__("ctypes").byref(nsa._dims(
        w.B, w.T, w.Hq, w.Hkv, w.D, w.S, nsa.DTYPE_BF16)), w.block_size)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    flop = int(10 * w.D * w.G * int(visible_keys_per_row(w).sum()))

    def call(check=False):
        # the device status is read once after the timed steps (reading it
        # waits for the stream)
        return nsa.bwd(q, k, v, out, lse, dout, bi, bc, w.block_size, w.scale, workspace=ws, check=check)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        ev[i][0].record()
        call()
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    call(check=True)   # raises if a bounded wait of the dq gather expired
    avg = float(np.mean(ms))
    tf = flop / (avg * 1e-3) / 1e12
    line = {
        "metric": METRIC_BWD, "value": round(tf, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(avg, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "block_size": w.block_size, "S": w.S, "useful_flop_per_step": flop,
                   "input_sha256": w.digest()[:16]},
        "roofline": {"bound": "mfma", "kernel": "fwd_bf16_ring_kernel (gradient mode: dq) + bwd_dkdv_kernel", "achieved": round(tf, 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel_ms_avg": round(avg, 4), "kernel_ms_min": round(float(np.min(ms)), 4),
                     "algorithmic_flop_per_launch": flop},
    }
    if not args.no_cpu_baseline:
        dout_f = ni.bf16_bits_to_f32(ni.to_bf16_bits(x)).reshape(x.shape)
        line["cpu_baseline"] = bwd_cpu_baseline(w, dout_f, seconds_target=args.cpu_seconds)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", action="store_true",
                    help="also time the headline steps with 1 GiB of scratch written before each (cold L2 and MALL)")
    ap.add_argument("--decode", action="store_true", help="measure the decode step instead")
    ap.add_argument("--backward", action="store_true", help="measure the backward pass on --config")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--headline-only", dest="all_configs", action="store_false",
                    help="skip the per-workload lines of the other named workloads")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the copy kernel used to scale the traffic counters")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                           "COPY_WRITE_DIR"),
                    help="write the traffic summary of --config from four rocprofv3 --pmc runs")
    ap.add_argument("--counters-summary", nargs=2, metavar=("SQ_DIR", "TA_DIR"),
                    help="write the unit-utilisation summary of --config (or --decode) from two --pmc runs")
    args = ap.parse_args()
    if args.counters_summary:
        import nsa_inputs as ni
        if args.decode:
            name, kern = ni.DECODE_NAME, "decode_bf16_kernel"
        else:
            name = ni.workload_name(args.config)
            kern = "fwd_f32_kernel" if args.config == 0 else FWD_KERNEL
        counters_summary(name, *args.counters_summary, kernel=kern)
        return
    if args.traffic_summary:
        import nsa_inputs as ni
        if args.decode:
            name, kern = ni.DECODE_NAME, "decode_bf16_kernel"
        else:
            name = ni.workload_name(args.config)
            kern = "fwd_f32_kernel" if args.config == 0 else FWD_KERNEL
        traffic_summary(name, *args.traffic_summary, kernel=kern)
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for {args.gpus}); "
              "the path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.decode:
        decode_bench(args)
        return
    if args.backward:
        backward_bench(args)
        return

    import torch
    import nsa_inputs as ni

    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    w = ni.make_config(args.config)
    gen_s = time.perf_counter() - t0
    print(f"[bench] {w.name}: generated in {gen_s:.1f} s", file=sys.stderr, flush=True)
    flop = useful_flops(w)
    tm = time_forward(w, dev, args.warmup, args.steps)
    # the cold variant (--cold; reported beside the headline, never as its
    # value): the same steps with L2 and MALL flushed before each one
    tmc = time_forward(w, dev, 2, args.steps, cold=True) if args.cold else None
    step_ms = tm["window_ms"] / args.steps
    kern_avg = tm["kernel_ms"]["mean"]

    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    value = flop / (step_ms * 1e-3) / 1e12
    achieved = flop / (kern_avg * 1e-3) / 1e12
    props = torch.cuda.get_device_properties(dev)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
            "block_size": w.block_size, "S": w.S, "varlen_seqs": None if w.cu_seqlens is None else len(w.seqlens),
            "index_layout": w.index_layout,
            "useful_flop_per_step": flop, "pct_of_bf16_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
            "input_sha256": w.digest()[:16], "device": (getattr(props, "gcnArchName", "") or props.name or "gfx950").split(":")[0], "cus": props.multi_processor_count,
            "wall_s_timed": round(tm["wall_s"], 4),
        },
        "timing": {"step_ms": tm["step_ms"], "kernel_ms": tm["kernel_ms"]},
        "roofline": {
            "bound": "mfma",
            "kernel": FWD_KERNEL if w.dtype == "bf16" else "fwd_f32_kernel",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": read_traffic(w.name),
            "counters": read_counters(w.name),
            "kernel_ms_avg": round(kern_avg, 4),
            "kernel_ms_min": tm["kernel_ms"]["min"],
            "kernel_ms_median": tm["kernel_ms"]["median"],
            "kernel_ms_p90": tm["kernel_ms"]["p90"],
            "algorithmic_flop_per_launch": flop,
            "algorithmic_bytes_per_launch": algorithmic_bytes(w),
        },
    }
    if tmc is not None:
        line["timing_cold"] = {"step_ms": tmc["step_ms"], "kernel_ms": tmc["kernel_ms"],
                               "scratch_bytes_written_before_each_step": COLD_SCRATCH_BYTES}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, seconds_target=args.cpu_seconds)
    if args.all_configs:
        # every named workload, in the same run: one JSON line each on stderr,
        # a compact copy in the headline line
        summary = {}
        for cfg in range(5):
            if cfg == args.config:
                cl = {"workload": w.name, "step_ms": tm["step_ms"], "kernel_ms": tm["kernel_ms"],
                      "useful_flop": flop, "steps": args.steps, "warmup": args.warmup}
                cl.update(_rates(flop, tm, w))
                if "cpu_baseline" in line:
                    cl["oracle"] = line["cpu_baseline"]
            else:
                cl = config_line(cfg, dev, warmup=10, steps=50, cpu_seconds=0 if args.no_cpu_baseline else 2.5)
            print(json.dumps({"config_line": cl}), file=sys.stderr, flush=True)
            summary[cl["workload"]] = {k: cl[k] for k in ("kernel_tflops_median", "kernel_pct_peak_median",
                                                            "step_ms_median", "kernel_ms_median")}
            if "oracle" in cl:
                summary[cl["workload"]]["oracle_tflops"] = round(cl["oracle"]["value"], 5)
        line["all_configs"] = summary
    print(json.dumps(line), flush=True)


def _stats(xs) -> dict:
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "min": round(float(a.min()), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "mean": round(float(a.mean()), 4)}


COLD_SCRATCH_BYTES = 1 << 30   # written between steps of the cold variant (beyond L2 and MALL)


def time_forward(w, dev, warmup, steps, cold=False):
    """`warmup` untimed steps, then `steps` timed ones; a step is the whole
    call (scheduler, then the attention kernel).  HIP events on the launch
    stream bracket every step, every kernel and the whole timed window.
    With `cold`, 1 GiB of scratch is written before each timed step (outside
    its events), so every step starts with no input in L2 or MALL."""
    import torch
    import block_index_sparse_amd as nsa
    import nsa_inputs as ni
    q, k, v, bi, bc, cu = ni.to_torch(w, dev)
    f = nsa.Forward(q, k, v, bi, bc, w.block_size, w.scale, cu_seqlens=cu, index_layout=w.index_layout)
    torch.cuda.synchronize()
    for _ in range(warmup):
        f.schedule()
        f.execute(check=False)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    e_start, e_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    scratch = torch.empty(COLD_SCRATCH_BYTES // 4, dtype=torch.int32, device=dev) if cold else None
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e_start.record()
    for i in range(steps):
        if cold:
            scratch.fill_(i)
        ev[i][0].record()
        f.schedule()
        ev[i][1].record()
        f.execute(check=False)
        ev[i][2].record()
    e_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    # outside the timed region: every timed launch must have completed its
    # bounded waits, or the numbers describe a broken run
    if f.device_status() != 0:
        sys.exit(f"bench: a bounded wait in the forward kernel expired on {w.name}; no result reported")
    out = {"window_ms": e_start.elapsed_time(e_stop), "wall_s": wall,
           "step_ms": _stats([a.elapsed_time(c) for a, _, c in ev]),
           "kernel_ms": _stats([b.elapsed_time(c) for _, b, c in ev])}
    del f, q, k, v, bi, bc, cu, scratch
    torch.cuda.empty_cache()
    return out


def _rates(flop, tm, w):
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    kt = flop / (tm["kernel_ms"]["median"] * 1e-3) / 1e12
    return {"kernel_tflops_median": round(kt, 3), "kernel_pct_peak_median": round(100 * kt / peak, 2),
            "peak_tflops": peak, "step_ms_median": tm["step_ms"]["median"],
            "kernel_ms_median": tm["kernel_ms"]["median"],
            "step_tflops_median": round(flop / (tm["step_ms"]["median"] * 1e-3) / 1e12, 3)}


def config_line(cfg, dev, warmup=10, steps=50, cpu_seconds=2.5):
    """Median / min / p90 of `steps` timed steps of named workload `cfg`, and
    the oracle's time on a bounded sample (the whole workload, median of
    three, plus one single-thread run, when it is the tiny fp32 one)."""
    import nsa_inputs as ni
    import oracle
    w = ni.make_config(cfg)
    flop = useful_flops(w)
    tm = time_forward(w, dev, warmup, steps)
    cl = {"workload": w.name, "step_ms": tm["step_ms"], "kernel_ms": tm["kernel_ms"], "useful_flop": flop,
          "steps": steps, "warmup": warmup}
    cl.update(_rates(flop, tm, w))
    if cpu_seconds > 0:
        if w.B * w.T <= 4096:
            threads = _oracle_threads()
            runs = []
            for _ in range(3):
                t0 = time.perf_counter()
                oracle.fwd_workload(w, threads=threads)
                runs.append(time.perf_counter() - t0)
            t0 = time.perf_counter()
            oracle.fwd_workload(w, threads=1)
            one = time.perf_counter() - t0
            used = float(np.median(runs))
            cl["oracle"] = {"value": flop / used / 1e12, "unit": "TFLOP/s", "cores": threads,
                            "kind": "oracle", "seconds": used,
                            "sample": f"whole workload, median of 3 runs on {threads} OpenMP threads",
                            "single_thread_seconds": one}
        else:
            cl["oracle"] = cpu_baseline(w, seconds_target=cpu_seconds, seed=cfg)
    return cl


if __name__ == "__main__":
    main()
