"""Benchmark of paged MLA decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]
                    [--only] [--no-flush] [--no-cpu]

One step is one ``mla_decode`` call — split planner, decode kernel, LSE
combine — over one synthetic batch already resident in HBM. The headline
workload is the kernel-test shape of the CUTLASS_MLA fp8 review thread in bf16
(B=128, s_q=1, H=16, 4096-token contexts, page size 64). One JSON line carries:
  * value / ms_per_step: whole-call algorithmic GB/s of that workload;
  * roofline: the decode kernel alone against its bound (HBM or bf16 MFMA),
    with the whole call's and the reused-plan call's fractions beside it;
  * workloads: the same figures for the four bench workloads (16 heads bf16 and
    fp8, 128 heads bf16, 128 heads x 4 query tokens fp8), warm and with the
    256 MB Infinity Cache evicted before each call;
  * cpu_baseline: the float64 oracle on the host cores over a bounded sample
    of the headline workload, plus a one-thread figure for the 16-head ones.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mla_inputs as mi  # noqa: E402

DEFAULT_WORKLOAD = "b128_h16_L4096_bf16"
METRIC = "paged MLA decode: HBM GB/s + TFLOP/s (fraction of roofline), seqs/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2516.6    # dense bf16 MFMA
CSRC = os.path.join(ROOT, "mla_paged_decode_04_amd", "csrc")
# Sources whose digest a counter summary must match to be used: the kernel
# itself and the host file with the split planner, whose items decide how
# many partials the kernel writes.
KERNEL_SOURCES = {
    "mla_decode_narrow": ("mla_internal.h", "mla_narrow.hip", "mla_decode.hip"),
    "mla_decode_wide": ("mla_internal.h", "mla_wide.hip", "mla_decode.hip"),
    "mla_decode_wide128": ("mla_internal.h", "mla_wide128.hip", "mla_decode.hip"),
}


def algorithmic_bytes(inp) -> int:
    """q, every cached row a sequence reads (once), its block-table entries,
    seq_lens, out and lse."""
    wl = inp.wl
    B, s_q, H, bs = wl.batch, wl.s_q, wl.heads, wl.block_size
    row = 576 * (2 if wl.kv_dtype == "bf16" else 1)
    lens = inp.seq_lens.astype(np.int64)
    return int(lens.sum() * row + ((lens + bs - 1) // bs).sum() * 4 + B * 4
               + B * s_q * H * (576 * 2 + 512 * 2 + 4))


def algorithmic_flops(inp) -> int:
    """2 * (576 + 512) per (query row, visible key): q.k and p*v."""
    wl = inp.wl
    lens = inp.seq_lens.astype(np.int64)
    vis = 0
    for i in range(wl.s_q):
        v = lens - wl.s_q + 1 + i if wl.causal else lens
        vis += int(np.clip(v, 0, None).sum())
    return 2 * wl.heads * (576 + 512) * vis


def to_device(inp, torch):
    dev = torch.device("cuda:0")
    q = torch.from_numpy(inp.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    if inp.wl.kv_dtype == "bf16":
        kv = torch.from_numpy(inp.kv.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        kv = torch.from_numpy(inp.kv).to(dev).view(torch.float8_e4m3fn)
    return q, kv, torch.from_numpy(inp.block_table).to(dev), torch.from_numpy(inp.seq_lens).to(dev)


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_kernel_name(rows: int) -> str:
    """The decode kernel the library launches for this many query rows."""
    if rows <= 16:
        return "mla_decode_narrow"
    return "mla_decode_wide" if rows <= 64 else "mla_decode_wide128"


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per decode-kernel launch from the committed rocprofv3 counter
    summary, or None when there is none or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_b or m_src.group(1) != source_digest(kernel):
        return None
    return float(m_b.group(1))


def cpu_baseline(inp, budget_s: float = 12.0):
    """Float64 oracle on the host cores over the same workload: whole batches
    until about `budget_s` seconds of CPU work; throughput in GB/s of
    algorithmic bytes so that it reads in the unit of `value`."""
    from oracle import mla_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:   # pragma: no cover
        cores = os.cpu_count() or 1
    wl = inp.wl
    # a bounded sample: the first n sequences of the batch, as many passes as fit
    n = wl.batch
    t0 = time.perf_counter()
    passes = 0
    while True:
        orc.mla_decode(inp.q_bits[:n], inp.kv, inp.block_table[:n], inp.seq_lens[:n], wl.s_q,
                       wl.softmax_scale, inp.kv_scale, wl.kv_dtype, wl.causal)
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s or passes >= 20:
            break
    frac = n / wl.batch
    gbs = algorithmic_bytes(inp) * frac * passes / el / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{passes} pass(es) over all {n} sequences of the workload, "
                      f"float64 numpy oracle, {el:.1f} s wall",
            "seqs_per_s": round(n * passes / el, 3)}


def cpu_baseline_one_thread(names=("tiny", "b128_h16_L4096_bf16", "b128_h16_L4096_fp8"),
                            n_seqs: int = 4):
    """The oracle with one BLAS thread on the first `n_seqs` sequences of each
    workload (the tiny one whole): seqs/s and GB/s of algorithmic bytes."""
    from oracle import mla_oracle as orc
    try:
        from threadpoolctl import threadpool_limits
    except Exception:   # pragma: no cover
        return None
    res = {}
    with threadpool_limits(limits=1):
        for name in names:
            wl = mi.WORKLOADS[name]
            inp = mi.make_inputs(wl)
            n = min(n_seqs, wl.batch)
            t0 = time.perf_counter()
            orc.mla_decode(inp.q_bits[:n], inp.kv, inp.block_table[:n], inp.seq_lens[:n], wl.s_q,
                           wl.softmax_scale, inp.kv_scale, wl.kv_dtype, wl.causal)
            el = time.perf_counter() - t0
            gbs = algorithmic_bytes(inp) * (n / wl.batch) / el / 1e9
            res[name] = {"seqs_per_s": round(n / el, 3), "GB/s": round(gbs, 4), "seconds": round(el, 3),
                         "sequences": n}
    return {"cores": 1, "kind": "oracle", "workloads": res}


BENCH_WORKLOADS = ("b128_h16_L4096_bf16", "b128_h16_L4096_fp8", "b64_h128_L1k2k_bs128_bf16",
                   "b32_sq4_h128_L512_16k_fp8")


def roofline_of(nbytes: int, nflops: int, ms: float) -> dict:
    """Fraction of the bound (HBM or bf16 MFMA) the algorithmic work sets."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    tfs = nflops / (ms * 1e-3) / 1e12
    if nbytes / (HBM_PEAK_GBS * 1e9) >= nflops / (MFMA_BF16_PEAK_TFS * 1e12):
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
            "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)}


def measure(name: str, steps: int, warmup: int, flush: bool):
    """Time one workload: the whole mla_decode call (planner, decode kernel,
    combine), the call on a reused plan (decode kernel + combine), and the
    decode kernel alone, warm; with `flush`, also each of them with the 256 MB
    Infinity Cache evicted (a 512 MB read sweep) before every call."""
    import ctypes
    import torch
    import mla_paged_decode_04_amd as mla

    wl = mi.WORKLOADS[name]
    inp = mi.make_inputs(wl)
    q, kv, bt, sl = to_device(inp, torch)
    B, s_q, H = wl.batch, wl.s_q, wl.heads
    out = torch.empty((B, s_q, H, 512), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, s_q, H), dtype=torch.float32, device=q.device)
    desc = mla.make_desc(B, H, wl.block_size, kv.shape[0], bt.shape[1],
                         mla.MLA_DTYPE_BF16 if wl.kv_dtype == "bf16" else mla.MLA_DTYPE_FP8_E4M3FN,
                         wl.causal)
    ws_bytes = mla.workspace_size(s_q, desc)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    lib = mla.library()
    stream = torch.cuda.current_stream()
    args = (q.data_ptr(), kv.data_ptr(), bt.data_ptr(), sl.data_ptr(), s_q,
            float(wl.softmax_scale), float(inp.kv_scale), out.data_ptr(), lse.data_ptr(),
            ctypes.byref(desc), ws.data_ptr(), ws_bytes, stream.cuda_stream)

    def call(fn):
        st = fn(*args)
        if st != 0:
            raise RuntimeError(f"{fn.__name__} status {st}")

    full = lambda: call(lib.mla_decode)                 # noqa: E731
    reuse = lambda: call(lib.mla_decode_with_plan)      # noqa: E731
    kernel = lambda: call(lib.mla_decode_fwd_only)      # noqa: E731

    for _ in range(warmup):
        full()
    torch.cuda.synchronize()
    # the first calls of a process run slower while the clocks ramp up: a
    # fixed half second of untimed calls before anything is timed
    t_end = time.perf_counter() + 0.5
    while time.perf_counter() < t_end:
        full()
        torch.cuda.synchronize()

    def back_to_back(fn):
        """K calls between one event pair (the kernel-trace durations agree
        with this average within about 1 %)."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, (time.perf_counter() - t0) * 1e3

    def per_call(fn, scratch=None):
        """An event pair around every call (reads a few us above the trace),
        after a 512 MB read sweep when `scratch` is given; median. The sweep
        reads (the sum is discarded) rather than writes, so that it leaves
        clean lines: a write sweep leaves the Infinity Cache full of dirty
        lines whose write-back is then charged to the timed call."""
        ts = []
        for _ in range(steps):
            if scratch is not None:
                scratch.sum()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    plan = lambda: call_plan()   # noqa: E731

    def call_plan():
        st = lib.mla_decode_plan(sl.data_ptr(), s_q, ctypes.byref(desc), ws.data_ptr(), ws_bytes,
                                 stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"mla_decode_plan status {st}")

    r = {"workload": name}
    r["call_ms"], r["wall_ms_timed"] = back_to_back(full)
    r["reuse_ms"], _ = back_to_back(reuse)
    r["kernel_ms"], _ = back_to_back(kernel)
    r["plan_ms"], _ = back_to_back(plan)
    r["kernel_ms_event_pairs"] = per_call(kernel)
    r["call_ms_event_pairs"] = per_call(full)
    if flush:
        scratch = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=q.device)
        scratch.sum()
        torch.cuda.synchronize()
        r["kernel_ms_flushed"] = per_call(kernel, scratch)
        r["call_ms_flushed"] = per_call(full, scratch)
        r["reuse_ms_flushed"] = per_call(reuse, scratch)
        del scratch
    # leave a correct result behind (the kernel-only launches rewrite partials)
    full()
    torch.cuda.synchronize()
    r["nbytes"] = algorithmic_bytes(inp)
    r["nflops"] = algorithmic_flops(inp)
    r["kernel"] = decode_kernel_name(s_q * H)
    r["inp"] = inp
    return r


def workload_summary(r: dict) -> dict:
    """The per-workload figures of the JSON line: times in microseconds and the
    fraction of the roofline for the kernel, the call and the reused-plan call."""
    nb, nf = r["nbytes"], r["nflops"]
    us = lambda ms: round(ms * 1e3, 2)   # noqa: E731
    out = {"kernel": r["kernel"], "algorithmic_bytes": nb, "algorithmic_flops": nf,
           "bound": roofline_of(nb, nf, 1.0)["bound"],
           "kernel_us": us(r["kernel_ms"]), "call_us": us(r["call_ms"]),
           "reuse_plan_call_us": us(r["reuse_ms"]), "plan_us": us(r["plan_ms"]),
           "frac_kernel": roofline_of(nb, nf, r["kernel_ms"])["frac"],
           "frac_call": roofline_of(nb, nf, r["call_ms"])["frac"],
           "frac_reuse_plan_call": roofline_of(nb, nf, r["reuse_ms"])["frac"],
           "kernel_us_event_pairs": us(r["kernel_ms_event_pairs"]),
           "call_us_event_pairs": us(r["call_ms_event_pairs"])}
    if "kernel_ms_flushed" in r:
        out.update({"mall_flushed": {
            "kernel_us": us(r["kernel_ms_flushed"]), "call_us": us(r["call_ms_flushed"]),
            "reuse_plan_call_us": us(r["reuse_ms_flushed"]),
            "frac_kernel": roofline_of(nb, nf, r["kernel_ms_flushed"])["frac"],
            "frac_call": roofline_of(nb, nf, r["call_ms_flushed"])["frac"],
            "timing": "event pair around each call, after a 512 MB read sweep; median"}})
    out["hbm_frac_kernel"] = round(nb / (r["kernel_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    out["mfma_frac_kernel"] = round(nf / (r["kernel_ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4)
    return out


def bench_line(r: dict, steps: int, warmup: int, flush: bool, others=None, cpu=None):
    """The JSON line for one measured workload."""
    wl = r["inp"].wl
    nbytes, nflops, ms_step = r["nbytes"], r["nflops"], r["call_ms"]
    roof = roofline_of(nbytes, nflops, r["kernel_ms"])
    roof["traffic"] = traffic_from_profile(r["kernel"], wl.name)
    roof["kernel"] = r["kernel"]
    roof["kernel_ms"] = round(r["kernel_ms"], 5)
    roof["kernel_ms_event_pairs"] = round(r["kernel_ms_event_pairs"], 5)
    roof["hbm_frac"] = round(nbytes / (r["kernel_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    roof["mfma_frac"] = round(nflops / (r["kernel_ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4)
    roof["call_frac"] = roofline_of(nbytes, nflops, ms_step)["frac"]
    roof["reuse_plan_call_frac"] = roofline_of(nbytes, nflops, r["reuse_ms"])["frac"]
    if "kernel_ms_flushed" in r:
        roof["frac_mall_flushed"] = roofline_of(nbytes, nflops, r["kernel_ms_flushed"])["frac"]
        roof["kernel_ms_mall_flushed"] = round(r["kernel_ms_flushed"], 5)
    res = {
        "metric": METRIC,
        "value": round(nbytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.kv_dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "s_q": wl.s_q, "heads": wl.heads,
                   "seq_lens": wl.lens if wl.lens != "fixed" else list(set(wl.lens_arg)),
                   "seq_len_range": list(wl.lens_arg), "block_size": wl.block_size,
                   "kv_dtype": wl.kv_dtype, "d_qk": 576, "d_v": 512, "causal": wl.causal,
                   "parallelism": "single_gpu"},
        "tflops": round(nflops / (ms_step * 1e-3) / 1e12, 3),
        "seqs_per_s": round(wl.batch / (ms_step * 1e-3), 1),
        "algorithmic_bytes": nbytes,
        "algorithmic_flops": nflops,
        "wall_ms_timed": round(r["wall_ms_timed"], 3),
        "mall_flush": flush,
        "timing": ("value / ms_per_step: K back-to-back mla_decode calls (planner, decode kernel, "
                   "combine) between one event pair on the launch stream, warm; roofline: the decode "
                   "kernel alone, timed the same way; *_mall_flushed: an event pair around each call "
                   "after a 512 MB read sweep"),
        "roofline": roof,
    }
    if others is not None:
        res["workloads"] = others
    if cpu is not None:
        res["cpu_baseline"] = cpu
    return res


def bench_append(n_tokens: int, kv_dtype: str, steps: int, warmup: int):
    """mla_kv_append: n_tokens new rows scattered into a shuffled paged cache."""
    import torch
    import mla_paged_decode_04_amd as mla
    dev = torch.device("cuda:0")
    bs = 64
    nb = (n_tokens + bs - 1) // bs + 8
    rng = np.random.default_rng(21)
    rows = torch.randn((n_tokens, 576), dtype=torch.float32, device=dev).to(torch.bfloat16)
    slots = torch.from_numpy(rng.permutation(nb * bs)[:n_tokens].astype(np.int32)).to(dev)
    tdt = torch.bfloat16 if kv_dtype == "bf16" else torch.float8_e4m3fn
    kv = torch.zeros((nb, bs, 576), dtype=torch.uint8 if kv_dtype == "fp8" else torch.bfloat16,
                     device=dev).view(tdt)
    scale = 1.0 if kv_dtype == "bf16" else 0.0213
    for _ in range(warmup):
        mla.mla_kv_append(rows, slots, kv, scale)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        mla.mla_kv_append(rows, slots, kv, scale)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = n_tokens * (576 * 2 + 576 * (2 if kv_dtype == "bf16" else 1) + 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"metric": "paged cache append (mla_kv_append) GB/s", "value": round(gbs, 2),
            "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": kv_dtype, "data": "synthetic",
            "config": {"workload": f"append_{n_tokens}_{kv_dtype}", "tokens": n_tokens,
                       "block_size": bs, "kv_dtype": kv_dtype},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}}


def bench_absorb(T: int, H: int, d: int, steps: int, warmup: int):
    """mla_absorb_q (d -> 512 per head, q_pe copied) and mla_absorb_out (512 -> d)."""
    import torch
    import mla_paged_decode_04_amd as mla
    dev = torch.device("cuda:0")
    qn = torch.randn((T, H, d), device=dev).to(torch.bfloat16)
    pe = torch.randn((T, H, 64), device=dev).to(torch.bfloat16)
    w_uk = (torch.randn((H, d, 512), device=dev) * d ** -0.5).to(torch.bfloat16)
    o = torch.randn((T, H, 512), device=dev).to(torch.bfloat16)
    w_uv = (torch.randn((H, 512, d), device=dev) * 512 ** -0.5).to(torch.bfloat16)
    q = torch.empty((T, H, 576), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)

    def step():
        mla.mla_absorb_q(qn, pe, w_uk, out=q)
        mla.mla_absorb_out(o, w_uv, out=y)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2 * 2 * T * H * d * 512
    tfs = flops / (ms * 1e-3) / 1e12
    # algorithmic bytes: every operand read once, every result written once
    nbytes = 2 * (T * H * d + T * H * 64 + H * d * 512 + T * H * 576      # absorb_q
                  + T * H * 512 + H * 512 * d + T * H * d)                # absorb_out
    gbs = nbytes / (ms * 1e-3) / 1e9
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFS * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)}
    roof["traffic"] = None
    return {"metric": "absorbed projections (mla_absorb_q + mla_absorb_out) TFLOP/s",
            "value": round(tfs, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"absorb_T{T}_H{H}_d{d}", "tokens": T, "heads": H, "d": d},
            "gbs": round(gbs, 1), "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "roofline": roof}


def copy_calibration(mib: int = 1024, reps: int = 3):
    """A plain device-to-device copy of known size (torch's copy kernel), to
    scale the FETCH_SIZE / WRITE_SIZE counters of a profile run."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_copy": n * 4,
                                           "bytes_written_per_copy": n * 4, "copies": reps}}))


def peaks(reps: int = 5):
    """Achievable rates on this chip, as context for the roofline fractions
    (which stay against the published peaks): the MFMA probe for the shapes
    the kernels use, and torch's device fill and copy over 1 GiB. Times are HIP events around each launch on the launch stream;
    the median of `reps` after one untimed launch."""
    import torch
    import mla_paged_decode_04_amd as mla
    dev = torch.device("cuda:0")
    lib = mla.probe_library()
    published = {mla.PROBE_MFMA_16X16X32_BF16: 2.5e15, mla.PROBE_MFMA_32X32X16_BF16: 2.5e15,
                 mla.PROBE_MFMA_16X16X128_FP8: 5.0e15}
    names = {mla.PROBE_MFMA_16X16X32_BF16: "mfma_f32_16x16x32_bf16",
             mla.PROBE_MFMA_32X32X16_BF16: "mfma_f32_32x32x16_bf16",
             mla.PROBE_MFMA_16X16X128_FP8: "mfma_scale_f32_16x16x128_f8f6f4"}
    wgs, iters, x = 1024, 2048, 0.0625
    out = torch.empty(wgs * mla.PROBE_THREADS, dtype=torch.float32, device=dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    res = {"workgroups": wgs, "waves_per_workgroup": 8, "iters": iters}
    for shape, name in names.items():
        t = timed(lambda: mla.mla_probe_mfma(shape, wgs, iters, x, out))
        want = lib.mla_probe_mfma_expected(shape, iters, x)
        ok = bool(torch.all(out == want).item())
        flops = lib.mla_probe_mfma_flops(shape, wgs, iters)
        res[name] = {"tflops": round(flops / t / 1e12, 1), "frac_of_published": round(flops / t / published[shape], 3),
                     "us": round(t * 1e6, 1), "result_exact": ok}
    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    gib = float(n * 4)
    res["hbm"] = {
        "fill_gbs": round(gib / timed(lambda: b.fill_(1.0)) / 1e9, 1),
        "copy_gbs_read_plus_written": round(2 * gib / timed(lambda: b.copy_(a)) / 1e9, 1),
        "bytes": int(gib), "published_gbs": 8000.0,
    }
    return {"peaks": res, "n_gpus": 1, "data": "synthetic"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=list(mi.WORKLOADS))
    ap.add_argument("--all", action="store_true", help="one line per workload")
    ap.add_argument("--only", action="store_true",
                    help="time only --workload (no per-workload summary of the others); with "
                         "--absorb / --append, only the largest size")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the timings with the 256 MB Infinity Cache evicted before each call")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure achievable MFMA and device-memory rates (context)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for counter calibration)")
    ap.add_argument("--absorb", action="store_true",
                    help="only time the absorbed projections (d = 128 per head)")
    ap.add_argument("--append", action="store_true",
                    help="only time the cache append (128 and 65536 new rows, bf16 and fp8)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration()
        return
    if a.peaks:
        print(json.dumps(peaks()), flush=True)
        return
    if a.absorb:
        for T, H in ((4096, 128),) if a.only else ((128, 16), (64, 128), (4096, 128)):
            print(json.dumps(bench_absorb(T, H, 128, a.steps, a.warmup)), flush=True)
        return
    if a.append:
        for n in (65536,) if a.only else (128, 65536):
            for dt in ("bf16", "fp8"):
                print(json.dumps(bench_append(n, dt, a.steps, a.warmup)), flush=True)
        return
    flush = not a.no_flush
    if a.all:
        for n in BENCH_WORKLOADS:
            r = measure(n, a.steps, a.warmup, flush)
            print(json.dumps(bench_line(r, a.steps, a.warmup, flush, others={n: workload_summary(r)})),
                  flush=True)
        return
    head = measure(a.workload, a.steps, a.warmup, flush)
    others = {a.workload: workload_summary(head)}
    if not a.only:
        for n in BENCH_WORKLOADS:
            if n != a.workload:
                r = measure(n, a.steps, a.warmup, flush)
                others[n] = workload_summary(r)
                del r
                print(f"# timed {n}", file=sys.stderr, flush=True)
    cpu = None
    if not a.no_cpu:
        cpu = cpu_baseline(head["inp"])
        one = cpu_baseline_one_thread()
        if one is not None:
            cpu["one_thread"] = one
    print(json.dumps(bench_line(head, a.steps, a.warmup, flush, others=others, cpu=cpu)), flush=True)


if __name__ == "__main__":
    main()
