"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one pass of the whole path over one batch: slot mapping of the new
tokens, their KV write through the slot mapping, then paged attention.  The
headline workload is the Llama-3-8B-shaped decode layer (64 sequences,
context U[512, 4096], 32 q / 8 kv heads, head_dim 128, block 16, bf16); its
value is KV bytes streamed per second over whole steps.  Every other workload
of the problem statement is a leg of the same run:

  C1 tiny fp32 decode (parity-sized), C2 the headline, C3 the mixed
  continuous-batching step (48 decodes + two 512-token chunks in one flattened
  batch: its prefill TFLOP/s), C4 the 70B-layer long-context decode, C5 the
  prefix-shared fp8-KV decode (plain and cascade, warm and with a 512 MB
  scratch write between steps),

plus the fp8-KV Llama-3-8B decode, long prompts (the steady-state prefill
rate), the sliding-window legs and a measured matrix-core peak.  Each of
C1-C5 gets a record with the step and kernel times (mean, median, min), the
algorithmic bytes or FLOPs and their rate against the MI355X peak, the HBM
rate from the committed rocprofv3 counters (when they were taken with the
current kernel sources), the oracle's time on a bounded sample of the same
batch on the host cores (CPU model and thread count stated) and the largest
error of the sampled GPU rows against the oracle, with the tolerance.

Prints one JSON line.  Inputs are seeded and synthetic and resident in HBM
before the timed region; two copies of the KV pool alternate between steps so
no step reads KV that the previous step left in the 256 MB last-level cache.

Device time of each kernel comes from HIP events that the library records on
its own launch stream around each kernel (pa_timing_enable), in a second pass
of the same steps, so the headline pass carries no extra events.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       [--only tiny|decode|mixed|cascade|window|long|copy]   (copy: a plain 1 GiB
       device copy, the reference for scaling the FETCH_SIZE / WRITE_SIZE counters)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores
METRIC = "paged decode KV GB/s (% of HBM peak) + prefill TFLOP/s at 1×MI355X"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "paged_kv_cache_418_amd", "csrc")
COPY_BYTES = 1 << 30
SCRATCH_BYTES = 512 << 20       # written between the cold-cache steps of C5 (twice the 256 MB MALL)
TOL = {"f32": 2e-3, "bf16": 1.5e-2, "fp8": 6e-2}
# the sources a kernel's measured counters depend on (a profile taken on other sources is stale)
DECODE_SOURCES = ["decode_kernels.hip", "decode_body.h", "pa_device.h", "pa_internal.h",
                  "abi.cpp"]  # abi.cpp: launch shape
PREFILL_SOURCES = ["prefill_kernels.hip", "prefill_body.h", "pa_device.h", "pa_internal.h", "abi.cpp"]
# the cascade launch holds the decode body and the prefill body (its prefix tiles)
CASCADE_SOURCES = DECODE_SOURCES + ["prefill_body.h", "prefill_kernels.hip", "fused_kernels.hip"]


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Step:
    """Device state of one workload and the calls of one step."""

    def __init__(self, w, copies: int = 2, cascade: bool = False, window: int = 0, fused_write: bool = False):
        import paged_kv_cache_418_amd as pk
        self.pk = pk
        self.w = w
        self.cascade = cascade
        self.window = window
        # a step as one call that also stores the new K/V (pa_decode_write*, pa_decode_cascade_write_fp8,
        # pa_prefill_varlen_write over bf16 pools)
        self.fused_write = fused_write and (w.is_decode or (not window and (cascade or w.kv_dtype != "fp8")))
        dev = "cuda"
        self.pools = [(w.k_cache.to(dev), w.v_cache.to(dev))]
        for _ in range(copies - 1):
            self.pools.append((self.pools[0][0].clone(), self.pools[0][1].clone()))
        self.bt = torch.from_numpy(w.block_tables).to(dev)
        self.sl = torch.from_numpy(w.seq_lens).to(dev)
        self.qsl = torch.from_numpy(w.query_start_loc).to(dev)
        self.q = w.query.to(dev)
        self.nk = w.new_k.to(dev)
        self.nv = w.new_v.to(dev)
        self.slots = torch.empty(w.num_tokens, dtype=torch.int32, device=dev)
        self.out = torch.empty_like(self.q)
        self.max_len = int(w.seq_lens.max())
        self.max_q = int(w.q_lens.max())
        if cascade:
            nb = pk.pa_decode_cascade_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                                      self.max_len, w.shared_prefix_blocks, 0)
        elif w.is_decode:
            nb = pk.pa_decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, self.max_len, 0)
        elif window:
            nb = pk.pa_prefill_varlen_window_workspace_bytes(w.query_start_loc, w.seq_lens, w.num_q_heads,
                                                             w.num_kv_heads, w.head_dim, window)
        elif w.kv_dtype == "fp8":
            nb = pk.pa_prefill_varlen_fp8_workspace_bytes(w.query_start_loc, w.seq_lens, w.num_q_heads,
                                                          w.num_kv_heads, w.head_dim, w.block_tables.shape[1])
        else:
            nb = pk.pa_prefill_varlen_workspace_bytes(w.query_start_loc, w.seq_lens, w.num_q_heads, w.num_kv_heads,
                                                      w.head_dim)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        self.i = 0
        for kc, vc in self.pools:  # the new tokens' slots hold their K/V before any timed call
            self.write(kc, vc)
        torch.cuda.synchronize()

    def write(self, kc, vc):
        """Slot mapping and KV write, one launch (the slot array is stored too)."""
        w, pk = self.w, self.pk
        scales = dict(k_scale=w.k_scale, v_scale=w.v_scale) if w.kv_dtype == "fp8" else {}
        pk.pa_write_kv(self.nk, self.nv, kc, vc, self.bt, self.sl, self.qsl, self.max_q, slot_mapping=self.slots,
                       **scales)

    def attend(self, kc, vc):
        w, pk = self.w, self.pk
        if self.cascade:
            pk.pa_decode_cascade_fp8(self.q, kc, vc, self.bt, self.sl, w.scale, w.k_scale, w.v_scale, self.max_len,
                                     w.shared_prefix_blocks, out=self.out, workspace=self.ws)
        elif self.window and w.is_decode:
            pk.pa_decode_window(self.q, kc, vc, self.bt, self.sl, w.scale, self.max_len, self.window, out=self.out,
                                workspace=self.ws)
        elif self.window:
            pk.pa_prefill_varlen_window(self.q, kc, vc, self.bt, self.sl, self.qsl, w.seq_lens, w.query_start_loc,
                                        w.scale, self.window, out=self.out, workspace=self.ws)
        elif w.is_decode:
            if w.kv_dtype == "fp8":
                pk.pa_decode_fp8(self.q, kc, vc, self.bt, self.sl, w.scale, w.k_scale, w.v_scale, self.max_len,
                                 out=self.out, workspace=self.ws)
            else:
                pk.pa_decode(self.q, kc, vc, self.bt, self.sl, w.scale, self.max_len, out=self.out, workspace=self.ws)
        elif w.kv_dtype == "fp8":
            pk.pa_prefill_varlen_fp8(self.q, kc, vc, self.bt, self.sl, self.qsl, w.seq_lens, w.query_start_loc,
                                     w.scale, w.k_scale, w.v_scale, out=self.out, workspace=self.ws)
        else:
            pk.pa_prefill_varlen(self.q, kc, vc, self.bt, self.sl, self.qsl, w.seq_lens, w.query_start_loc, w.scale,
                                 out=self.out, workspace=self.ws)

    def write_and_attend(self, kc, vc):
        """The step as one call that stores the new K/V and attends (pa_decode_write, pa_decode_cascade_write_fp8,
        pa_prefill_varlen_write)."""
        w, pk = self.w, self.pk
        if self.cascade:
            pk.pa_decode_cascade_write_fp8(self.q, self.nk, self.nv, kc, vc, self.bt, self.sl, w.scale, w.k_scale,
                                           w.v_scale, self.max_len, w.shared_prefix_blocks, out=self.out,
                                           workspace=self.ws)
        elif self.window:
            pk.pa_decode_window_write(self.q, self.nk, self.nv, kc, vc, self.bt, self.sl, w.scale, self.max_len,
                                      self.window, out=self.out, workspace=self.ws)
        elif not w.is_decode:
            pk.pa_prefill_varlen_write(self.q, self.nk, self.nv, kc, vc, self.bt, self.sl, self.qsl, w.seq_lens,
                                       w.query_start_loc, w.scale, out=self.out, workspace=self.ws)
        elif w.kv_dtype == "fp8":
            pk.pa_decode_write_fp8(self.q, self.nk, self.nv, kc, vc, self.bt, self.sl, w.scale, w.k_scale, w.v_scale,
                                   self.max_len, out=self.out, workspace=self.ws)
        else:
            pk.pa_decode_write(self.q, self.nk, self.nv, kc, vc, self.bt, self.sl, w.scale, self.max_len,
                               out=self.out, workspace=self.ws)

    def attend_next(self):
        kc, vc = self.pools[self.i % len(self.pools)]
        self.i += 1
        self.attend(kc, vc)

    def two_calls(self):
        """The step as the KV write's launch followed by the attention call."""
        kc, vc = self.pools[self.i % len(self.pools)]
        self.i += 1
        self.write(kc, vc)
        self.attend(kc, vc)

    def __call__(self):
        if not self.fused_write:
            return self.two_calls()
        kc, vc = self.pools[self.i % len(self.pools)]
        self.i += 1
        self.write_and_attend(kc, vc)


def _stats(ms_list) -> dict:
    return {"mean": round(float(np.mean(ms_list)), 5), "median": round(float(statistics.median(ms_list)), 5),
            "min": round(float(min(ms_list)), 5), "n": len(ms_list)}


# Untimed calls of the step before its warm-up: after the host-side workload generation the GPU
# has been idle for seconds and its clock has dropped; the first milliseconds of work run slower
# (the fp8 decode step: 60-61 us against 52-56 warm, whichever variant is measured first).
SETTLE_S = 0.3


def settle(fn, seconds: float = SETTLE_S):
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_steps(fn, steps: int, warmup: int, between=None):
    """Times `steps` calls of fn.

    Returns (ms, wall_s, per_call): ms is the mean over the calls bracketed by two events (the
    events of that pass enclose the calls only); per_call holds mean / median / min of the
    calls, from a second pass with an event pair around every call.  between(), when given,
    runs before every call outside the timed region (the cold-cache variant's scratch write);
    ms is then the mean of the second pass.  The warm-up follows SETTLE_S seconds of untimed
    calls."""
    settle(fn)
    for _ in range(warmup):
        if between:
            between()
        fn()
    torch.cuda.synchronize()
    ms, wall = None, None
    if between is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = e0.elapsed_time(e1) / steps
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for b, e in pairs:
        if between:
            between()
        b.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    per = [b.elapsed_time(e) for b, e in pairs]
    if ms is None:
        ms, wall = float(np.mean(per)), time.perf_counter() - t0
    return ms, wall, _stats(per)


def kernel_times(fn, steps: int, kernels, between=None):
    """Device ms per launch of each named kernel over `steps` calls, from the library's own events:
    {name: {"mean", "median", "min", "n"}} (None when the kernel did not run)."""
    import paged_kv_cache_418_amd as pk
    torch.cuda.synchronize()
    pk.timing_reset()
    pk.timing_enable(True)
    for _ in range(steps):
        if between:
            pk.timing_enable(False)
            between()
            pk.timing_enable(True)
        fn()
    torch.cuda.synchronize()
    pk.timing_enable(False)
    out = {}
    for k in kernels:
        v = pk._binding.timing_launches(k)
        out[k] = _stats(v) if v else None
    return out


def kmean(kt, name):
    return kt[name]["mean"] if kt.get(name) else None


def source_hash(*files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_profile(name: str, sources) -> dict:
    """The machine-readable 'key: value' lines of a committed counter summary (profiles/<name>.txt), with
    'valid' False when the kernel sources changed since the counters were taken (hash mismatch)."""
    path = os.path.join(PROFILES, name + ".txt")
    if not os.path.exists(path):
        return {"valid": False, "why": f"no {os.path.relpath(path, ROOT)}"}
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash(*sources):
        return {"valid": False, "why": "kernel source changed since the counters were taken"}
    kv["valid"] = True
    return kv


def read_traffic(name: str, sources) -> dict:
    """HBM bytes per launch of a kernel from its committed counter summary: FETCH_SIZE and WRITE_SIZE in KiB
    per dispatch, each scaled by what the same counter reads for a plain copy of known size."""
    kv = read_profile(name, sources)
    if not kv["valid"]:
        return {"bytes": None, "why": kv["why"]}
    try:
        fetch = float(kv["fetch_kib"]) * float(kv["fetch_bytes_per_kib"])
        write = float(kv["write_kib"]) * float(kv["write_bytes_per_kib"])
    except (KeyError, ValueError):
        return {"bytes": None, "why": f"incomplete profiles/{name}.txt"}
    return {"bytes": int(round(fetch + write)), "fetch_bytes": int(round(fetch)), "write_bytes": int(round(write))}


def fetch_rate(traffic: dict, kernel_ms):
    """FETCH_SIZE bytes per second of the kernel (GB/s), from the counters and the live kernel time."""
    if traffic.get("fetch_bytes") is None or not kernel_ms:
        return None
    return round(traffic["fetch_bytes"] / (kernel_ms * 1e-3) / 1e9, 1)


# ---- the oracle beside the GPU: a bounded sample of the same batch on the host cores

def oracle_check(w, out: torch.Tensor, rows, tol: float, work_bytes: int = 0, work_flops: int = 0, pools=None,
                 what: str = ""):
    """Times the oracle on the given rows of the batch (pools with the new tokens written) and compares the
    GPU's output rows with it.  Returns the oracle record and the parity record."""
    import oracle
    if pools is None:
        pools = oracle.written_pools(w)
    rows = [int(r) for r in rows]
    t0 = time.perf_counter()
    ref = oracle.attention_for(w, rows=rows, pools=pools)
    secs = time.perf_counter() - t0
    got = out[torch.tensor(rows, device=out.device)].float().cpu().double().numpy()
    finite = bool(np.all(np.isfinite(got)))
    err = float(np.max(np.abs(got - ref))) if finite else float("inf")
    rec = {"seconds": round(secs, 3), "rows": len(rows), "cores": oracle.num_threads(), "cpu_model": cpu_model(),
           "kind": "oracle (fp64 C, OpenMP over q heads)", "sample": what or f"{len(rows)} rows of {w.name}"}
    if work_bytes:
        rec["gbps"] = round(work_bytes / secs / 1e9, 4)
    if work_flops:
        rec["gflops"] = round(work_flops / secs / 1e9, 3)
    par = {"rows": len(rows), "max_abs_err": err, "tol": tol, "pass": bool(finite and err <= tol)}
    return rec, par


def rows_kv_bytes(w, rows) -> int:
    """KV bytes the oracle reads for some decode rows (their sequences' whole contexts)."""
    seq_of = np.searchsorted(w.query_start_loc, np.asarray(rows), side="right") - 1
    return int(sum(2 * int(w.seq_lens[s]) for s in seq_of) * w.num_kv_heads * w.head_dim * w.kv_elem_bytes)


def rows_pairs(w, rows) -> int:
    """(row, key) pairs some rows of a flattened batch see: row i of sequence s sees c_s + i + 1 keys."""
    qsl = w.query_start_loc
    seq_of = np.searchsorted(qsl, np.asarray(rows), side="right") - 1
    return int(sum(int(w.seq_lens[s]) - int(qsl[s + 1] - qsl[s]) + (r - int(qsl[s])) + 1
                   for r, s in zip(rows, seq_of)))


def decode_rows_sample(w, n: int):
    """n decode rows spread evenly over the batch (row index = sequence index for a decode batch)."""
    return sorted(set(int(x) for x in np.linspace(0, w.num_tokens - 1, n).round()))


def cpu_baseline(w, budget_s: float = 12.0):
    """The oracle on a bounded sample of the workload's sequences (repeated until the budget is spent)."""
    import oracle
    threads = oracle.num_threads()
    done_bytes, spent, n = 0, 0.0, 0
    s = 0
    while spent < budget_s:
        t0 = time.perf_counter()
        oracle.attention_for(w, rows=[int(w.query_start_loc[s])])
        spent += time.perf_counter() - t0
        done_bytes += 2 * int(w.seq_lens[s]) * w.num_kv_heads * w.head_dim * w.kv_elem_bytes
        n += 1
        s = (s + 1) % w.num_seqs
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": threads, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{n} single-sequence decode rows of {w.name} in turn (fp64 C oracle, OpenMP over q heads, "
                      f"{spent:.1f} s)"}


def decode_record(cfg, w, step_stats, kt, alg_bytes, traffic, oracle_rec, parity, kernel="decode"):
    k_ms = kmean(kt, kernel)
    rec = {"cfg": cfg, "workload": w.name, "bound": "hbm", "step_ms": step_stats, "kernel_ms": kt.get(kernel),
           "alg_bytes": alg_bytes}
    if k_ms:
        gbps = alg_bytes / (k_ms * 1e-3) / 1e9
        rec.update({"gbps": round(gbps, 1), "pct_hbm": round(100 * gbps / HBM_PEAK_GBPS, 2)})
    rec["fetch_size_gbps"] = fetch_rate(traffic, k_ms) if traffic else None
    rec["oracle"] = oracle_rec
    rec["parity"] = parity
    return rec


# ---- legs

def bench_tiny(args, result):
    """C1: the tiny fp32 decode (4 sequences of 1, 17, 33 and 100 tokens), checked whole against the oracle."""
    from paged_kv_cache_418_amd import workloads as wl
    w = wl.tiny_fp32_decode()
    st = Step(w, copies=1, fused_write=True)
    ms, _, per = time_steps(st, args.steps, args.warmup)
    kt = kernel_times(st, args.steps, ["reshape_and_cache", "decode", "decode_merge"])
    rec, par = (None, None)
    if not args.no_cpu:
        rec, par = oracle_check(w, st.out, range(w.num_tokens), TOL["f32"], work_bytes=wl.decode_kv_bytes(w),
                                what="the whole batch (4 rows)")
    result.setdefault("configs", {})["C1"] = decode_record("C1", w, per, kt, wl.decode_alg_bytes(w), None, rec, par)
    del st


def bench_decode(args, result):
    from paged_kv_cache_418_amd import workloads as wl
    _log("generating llama3_8b_decode_bf16 ...")
    w = wl.llama3_8b_decode_bf16()
    st = Step(w, fused_write=True)
    kv_bytes = wl.decode_kv_bytes(w)
    alg_bytes = wl.decode_write_alg_bytes(w)
    _log("timing decode steps ...")
    ms, wall, per = time_steps(st, args.steps, args.warmup)
    kt = kernel_times(st, args.steps, ["reshape_and_cache", "decode", "decode_merge"])
    # the same step as two calls (the KV write's own launch, then pa_decode), for reference
    ms2, _, per2 = time_steps(st.two_calls, args.steps, args.warmup)
    dec_ms = kmean(kt, "decode")
    att_gbps = alg_bytes / (dec_ms * 1e-3) / 1e9
    traffic = read_traffic("decode_bf16_d128_llama3_8b_traffic", DECODE_SOURCES)
    result.update({
        "metric": METRIC,
        "value": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_s": SETTLE_S,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama3_8b_decode_bf16", "num_seqs": w.num_seqs, "ctx": "U[512,4096]",
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "num_blocks": w.num_blocks, "kv_bytes": kv_bytes,
                   "num_splits": "auto"},
        "pct_hbm": round(100 * kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "wall_s": round(wall, 4),
        "step_ms": per,
        "step_two_calls_ms": per2,
        "roofline": {"kernel": "decode_mfma_kernel<128, bf16, write>", "bound": "hbm",
                     "achieved": round(att_gbps, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(att_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic["bytes"], "alg_bytes_per_launch": alg_bytes,
                     "launch_ms": round(dec_ms, 5), "launch_ms_median": kt["decode"]["median"],
                     "launch_ms_min": kt["decode"]["min"], "launches_timed": kt["decode"]["n"]},
        "step_kernels_ms": {k: (v["mean"] if v else None) for k, v in kt.items()},
    })
    if traffic["bytes"] is None:
        result["roofline"]["traffic_note"] = traffic["why"]
    else:
        result["roofline"]["traffic_over_alg"] = round(traffic["bytes"] / alg_bytes, 4)
        result["roofline"]["fetch_size_gbps"] = fetch_rate(traffic, dec_ms)
    rec, par = (None, None)
    if not args.no_cpu:
        rows = decode_rows_sample(w, 8)
        rec, par = oracle_check(w, st.out, rows, TOL["bf16"], work_bytes=rows_kv_bytes(w, rows),
                                what=f"{len(rows)} decode rows spread over the batch")
    result.setdefault("configs", {})["C2"] = decode_record("C2", w, per, kt, alg_bytes, traffic, rec, par)
    _log("generating llama3_8b_decode_fp8 ...")
    w8 = wl.llama3_8b_decode_fp8()
    st8 = Step(w8, fused_write=True)
    ms8, _, per8 = time_steps(st8, args.steps, args.warmup)
    kt8 = kernel_times(st8, args.steps, ["decode", "decode_merge"])
    _, _, per8_two = time_steps(st8.two_calls, args.steps, args.warmup)
    kv8 = wl.decode_kv_bytes(w8)
    d8 = kmean(kt8, "decode")
    result["fp8_kv_decode"] = {
        "workload": "llama3_8b_decode_fp8 (the same batch with E4M3 pools, K scale 0.05, V scale 0.04)",
        "kv_bytes": kv8, "ms_per_step": round(ms8, 5), "step_ms": per8, "step_two_calls_ms": per8_two,
        "decode_kernel_ms": round(d8, 5),
        "decode_kernel": kt8["decode"], "merge_kernel_ms": kmean(kt8, "decode_merge"),
        "kernel_gbps": round(kv8 / (d8 * 1e-3) / 1e9, 1),
        "kernel_frac_hbm": round(kv8 / (d8 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    del st8, w8
    if not args.no_cpu:
        _log("cpu baseline ...")
        result["cpu_baseline"] = cpu_baseline(w)
    del st
    torch.cuda.empty_cache()


def bench_mixed(args, result):
    from paged_kv_cache_418_amd import workloads as wl
    _log("generating mixed_step_bf16 ...")
    w = wl.mixed_step_bf16()
    st = Step(w, fused_write=True)
    ms, _, per = time_steps(st, args.steps, args.warmup)
    kt_step = kernel_times(st, args.steps, ["reshape_and_cache", "decode", "decode_merge", "prefill",
                                            "prefill_merge", "fused"])
    # the same step as two calls (the KV write's own launch, then pa_prefill_varlen), for reference
    _, _, per_two = time_steps(st.two_calls, args.steps, args.warmup)
    flops = wl.prefill_flops(w)
    rec, par = (None, None)
    if not args.no_cpu:
        # 6 decode rows and 16 rows of the two chunks (their first, last and spread positions)
        dec_rows = [int(x) for x in np.linspace(0, 47, 6).round()]
        chunk_rows = [int(x) for q0 in (48, 560) for x in np.linspace(q0, q0 + 511, 8).round()]
        rec, par = oracle_check(w, st.out, dec_rows + chunk_rows, TOL["bf16"],
                                work_flops=4 * w.num_q_heads * w.head_dim * rows_pairs(w, dec_rows + chunk_rows),
                                what="6 decode rows and 16 chunk rows (8 per chunk, first to last)")
    del st
    # the two chunks alone (prefill part) and the 48 decodes alone
    chunk_w = _sub(w, list(range(48, 50)))
    cs = Step(chunk_w, copies=1)
    pre_call_ms, _, pre_call = time_steps(cs.attend_next, args.steps, args.warmup)
    kt = kernel_times(cs.attend_next, args.steps, ["prefill", "prefill_merge"])
    pre_ms = kmean(kt, "prefill")
    del cs
    # the same two chunks over fp8 pools (the kernel converts the codes itself) + merge
    w8 = wl.mixed_step_bf16(kv_dtype="fp8")
    cs8 = Step(_sub(w8, list(range(48, 50))), copies=1)
    pre8_call_ms, _, _ = time_steps(cs8.attend_next, args.steps, args.warmup)
    kt8 = kernel_times(cs8.attend_next, args.steps, ["prefill"])
    del cs8, w8
    # steady state: long prompts, where launch, first tiles and tail are small next to the tile loop
    lw = wl.long_prefill_bf16()
    ls = Step(lw, copies=1)
    long_call_ms, _, long_call = time_steps(ls.attend_next, max(5, args.steps // 5), 2)
    ktl = kernel_times(ls.attend_next, max(5, args.steps // 5), ["prefill"])
    long_flops = wl.prefill_flops(lw)
    del ls, lw
    mfma_peak = pk_mod().probe_mfma_peak()
    dec_w = _sub(w, list(range(48)))
    ds = Step(dec_w, copies=2)
    dms, _, _ = time_steps(ds.attend_next, args.steps, args.warmup)
    dec_bytes = wl.decode_kv_bytes(dec_w)
    del ds
    tflops = flops / (pre_ms * 1e-3) / 1e12
    counters = read_profile("prefill_bf16_d128_counters", PREFILL_SOURCES)
    mfma_busy = {"chunks": float(counters["mfma_busy_chunks"]), "long": float(counters["mfma_busy_long"])} \
        if counters["valid"] and "mfma_busy_chunks" in counters else None
    # the shader clock the counters saw under the long prompts (the published peak assumes 2.4 GHz)
    clock_long = float(counters["clock_ghz_long"]) if counters["valid"] and "clock_ghz_long" in counters else None
    chunk_fetch = float(counters["fetch_bytes_chunks"]) if counters["valid"] and "fetch_bytes_chunks" in counters \
        else None
    mixed = {"workload": "mixed_step_bf16", "ms_per_step": round(ms, 5), "step_ms": per, "step_two_calls_ms": per_two,
             "step_kernels_ms": {k: (v["mean"] if v else None) for k, v in kt_step.items()},
             "prefill_gflop": round(flops / 1e9, 3),
             "prefill_kernel_ms": round(pre_ms, 5), "prefill_kernel": kt["prefill"],
             "prefill_merge_ms": kmean(kt, "prefill_merge"),
             "prefill_call_ms": round(pre_call_ms, 5), "prefill_call": pre_call,
             "prefill_tflops": round(tflops, 2),
             "prefill_pct_mfma": round(100 * tflops / BF16_MFMA_PEAK_TFLOPS, 2),
             "prefill_roofline": {"kernel": "prefill_kernel<128>", "bound": "mfma", "achieved": round(tflops, 2),
                                  "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                                  "peak_measured": round(mfma_peak, 1),
                                  "frac_of_measured": round(tflops / mfma_peak, 4),
                                  "alg_flops_per_launch": flops,
                                  "mfma_busy": mfma_busy,
                                  "fetch_size_gbps": round(chunk_fetch / (pre_ms * 1e-3) / 1e9, 1)
                                  if chunk_fetch else None},
             "prefill_long": {"workload": "long_prefill_bf16 (4 prompts x 4096 tokens, causal, empty caches)",
                              "gflop": round(long_flops / 1e9, 2), "call_ms": round(long_call_ms, 4),
                              "call": long_call,
                              "kernel_ms": round(kmean(ktl, "prefill"), 4), "kernel": ktl["prefill"],
                              "kernel_tflops": round(long_flops / (kmean(ktl, "prefill") * 1e-3) / 1e12, 1),
                              "kernel_frac_of_peak": round(long_flops / (kmean(ktl, "prefill") * 1e-3) / 1e12 /
                                                           BF16_MFMA_PEAK_TFLOPS, 4),
                              "call_tflops": round(long_flops / (long_call_ms * 1e-3) / 1e12, 1),
                              "call_frac_of_peak": round(long_flops / (long_call_ms * 1e-3) / 1e12 /
                                                         BF16_MFMA_PEAK_TFLOPS, 4),
                              "call_frac_of_measured_peak": round(long_flops / (long_call_ms * 1e-3) / 1e12 /
                                                                  mfma_peak, 4),
                              "counters_clock_ghz": clock_long,
                              "counters_mfma_busy": mfma_busy["long"] if mfma_busy else None},
             "mfma_measured_peak_tflops": round(mfma_peak, 1),
             "prefill_fp8": {"call_ms": round(pre8_call_ms, 5), "kernel_ms": kmean(kt8, "prefill"),
                             "call_tflops": round(flops / (pre8_call_ms * 1e-3) / 1e12, 2)},
             "decode_part_gbps": round(dec_bytes / (dms * 1e-3) / 1e9, 2),
             "decode_part_ms": round(dms, 5)}
    result.setdefault("configs", {})["C3"] = {
        "cfg": "C3", "workload": w.name, "bound": "hbm (decode rows) + mfma (chunks)", "step_ms": per,
        "alg_bytes_decode": dec_bytes, "alg_flops_prefill": flops,
        "decode_part_gbps": mixed["decode_part_gbps"], "decode_part_pct_hbm":
            round(100 * mixed["decode_part_gbps"] / HBM_PEAK_GBPS, 2),
        "prefill_kernel_ms": kt["prefill"], "prefill_tflops": mixed["prefill_tflops"],
        "prefill_pct_mfma": mixed["prefill_pct_mfma"], "mfma_busy": mfma_busy,
        "fetch_size_gbps": mixed["prefill_roofline"]["fetch_size_gbps"], "oracle": rec, "parity": par}
    if "metric" in result:
        result["mixed_step"] = mixed
    else:
        result.update({"metric": METRIC, "value": mixed["decode_part_gbps"], "unit": "GB/s", "n_gpus": 1,
                       "steps": args.steps, "warmup": args.warmup, "ms_per_step": mixed["ms_per_step"],
                       "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                       "data": "synthetic", "config": {"workload": "mixed_step_bf16"}, "mixed_step": mixed})
    torch.cuda.empty_cache()


def bench_cascade(args, result):
    """C5: prefix-shared fp8 decode (128 requests, a 2048-token shared prefix, suffixes U[128,1024]): whole steps
    with the plain decode and with the cascade decode, each one call that also stores the new K/V
    (pa_decode_write_fp8, pa_decode_cascade_write_fp8; step_two_calls_ms: the KV write's launch, then the decode); logical KV bytes (each request's whole context) and unique
    bytes (the prefix once) per second, warm and with a 512 MB scratch write before every step (so no step finds
    the previous step's KV in the 256 MB MALL)."""
    from paged_kv_cache_418_amd import workloads as wl
    _log("generating prefix_shared_fp8_decode ...")
    w = wl.prefix_shared_fp8_decode()
    logical = wl.decode_kv_bytes(w)
    pre_tok = w.shared_prefix_blocks * w.block_size
    unique = int(2 * (pre_tok + np.sum(w.seq_lens.astype(np.int64) - pre_tok)) * w.num_kv_heads * w.head_dim *
                 w.kv_elem_bytes)
    out = {"workload": "prefix_shared_fp8_decode", "num_seqs": w.num_seqs, "shared_prefix_tokens": pre_tok,
           "logical_kv_bytes": logical, "unique_kv_bytes": unique}
    scratch = torch.empty(SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    flush = lambda: scratch.fill_(7)  # noqa: E731  (a plain fill kernel: 512 MB written)
    casc_out = None
    for name, cascade in (("plain", False), ("cascade", True)):
        st = Step(w, cascade=cascade, fused_write=True)
        ms, _, per = time_steps(st, args.steps, args.warmup)
        kt = kernel_times(st, args.steps, ["decode", "decode_merge"])
        _, _, per2 = time_steps(st.two_calls, args.steps, args.warmup)
        cms, _, cper = time_steps(st, args.steps, args.warmup, between=flush)
        ktc = kernel_times(st, args.steps, ["decode", "decode_merge"], between=flush)
        d = kmean(kt, "decode")
        out[name] = {"ms_per_step": round(ms, 5), "step_ms": per, "step_two_calls_ms": per2,
                     "logical_gbps": round(logical / (ms * 1e-3) / 1e9, 1),
                     "unique_gbps": round(unique / (ms * 1e-3) / 1e9, 1),
                     "decode_kernel_ms": round(d, 5), "decode_kernel": kt["decode"],
                     "merge_kernel_ms": kmean(kt, "decode_merge"),
                     "kernel_unique_gbps": round(unique / (d * 1e-3) / 1e9, 1),
                     "kernel_unique_frac_hbm": round(unique / (d * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "cold": {"note": "512 MB scratch write before every step, outside the timed region",
                              "step_ms": cper, "decode_kernel": ktc["decode"],
                              "kernel_unique_gbps": round(unique / (kmean(ktc, "decode") * 1e-3) / 1e9, 1)}}
        if cascade:
            casc_out = st.out
            casc_step, casc_kt = per, kt
        del st
    out["speedup"] = round(out["plain"]["ms_per_step"] / out["cascade"]["ms_per_step"], 3)
    del scratch
    result["cascade_step"] = out
    traffic = read_traffic("cascade_fp8_prefix_shared_traffic", CASCADE_SOURCES)
    if traffic.get("fetch_bytes") is not None:  # the cascade launch's HBM reads against the unique KV bytes
        out["cascade"]["kernel_fetch_bytes"] = traffic["fetch_bytes"]
        out["cascade"]["kernel_fetch_over_unique"] = round(traffic["fetch_bytes"] / unique, 4)
    rec, par = (None, None)
    if not args.no_cpu:
        rows = decode_rows_sample(w, 8)
        rec, par = oracle_check(w, casc_out, rows, TOL["fp8"], work_bytes=rows_kv_bytes(w, rows),
                                what=f"{len(rows)} decode rows spread over the batch (cascade output)")
    c5 = decode_record("C5", w, casc_step, casc_kt, unique, traffic, rec, par)
    c5.update({"alg_bytes_note": "unique KV bytes (the shared prefix once); logical bytes are in cascade_step",
               "logical_bytes": logical, "cold_kernel_unique_gbps": out["cascade"]["cold"]["kernel_unique_gbps"]})
    result.setdefault("configs", {})["C5"] = c5
    torch.cuda.empty_cache()


def pk_mod():
    import paged_kv_cache_418_amd as pk
    return pk._binding


def bench_window(args, result):
    """Sliding-window attention on two of the workloads above: the Llama-3-8B decode layer with a 1024-token window
    (bytes of the windowed keys per second) and the mixed step's two prefill chunks with a 256-token window (FLOPs
    of the visible pairs per second)."""
    from paged_kv_cache_418_amd import workloads as wl
    window_dec, window_pre = 1024, 256
    _log("generating llama3_8b_decode_bf16 (window) ...")
    w = wl.llama3_8b_decode_bf16()
    st = Step(w, window=window_dec, fused_write=True)
    ms, _, per = time_steps(st, args.steps, args.warmup)
    kt = kernel_times(st, args.steps, ["decode", "decode_merge"])
    _, _, per_two = time_steps(st.two_calls, args.steps, args.warmup)
    kv = wl.decode_window_kv_bytes(w, window_dec)
    dec_ms = kmean(kt, "decode")
    out = {"decode": {"workload": "llama3_8b_decode_bf16", "window": window_dec, "window_kv_bytes": kv,
                      "ms_per_step": round(ms, 5), "step_ms": per, "step_two_calls_ms": per_two,
                      "decode_kernel_ms": round(dec_ms, 5),
                      "decode_kernel": kt["decode"], "merge_kernel_ms": kmean(kt, "decode_merge"),
                      "kernel_gbps": round(kv / (dec_ms * 1e-3) / 1e9, 1),
                      "kernel_frac_hbm": round(kv / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}}
    del st
    _log("generating mixed_step_bf16 chunks (window) ...")
    cw = _sub(wl.mixed_step_bf16(), [48, 49])
    cs = Step(cw, copies=1, window=window_pre)
    call_ms, _, _ = time_steps(cs.attend_next, args.steps, args.warmup)
    kt = kernel_times(cs.attend_next, args.steps, ["prefill", "prefill_merge"])
    flops = wl.prefill_flops(cw, window=window_pre)
    pre_ms = kmean(kt, "prefill")
    out["prefill"] = {"workload": "mixed_step_bf16 chunks 512@0 + 512@1536", "window": window_pre,
                      "gflop": round(flops / 1e9, 3), "call_ms": round(call_ms, 5), "kernel_ms": round(pre_ms, 5),
                      "kernel": kt["prefill"], "merge_ms": kmean(kt, "prefill_merge"),
                      "kernel_tflops": round(flops / (pre_ms * 1e-3) / 1e12, 2)}
    del cs
    result["window"] = out
    torch.cuda.empty_cache()


def bench_long(args, result):
    """C4: the 70B-layer long-context decode (8 sequences of 32k-128k tokens, 64 q / 8 kv heads): one pool copy is
    already ten times the 256 MB MALL."""
    from paged_kv_cache_418_amd import workloads as wl
    _log("generating long_ctx_70b_decode_bf16 ...")
    w = wl.long_ctx_70b_decode_bf16()
    st = Step(w, copies=1, fused_write=True)
    steps = max(5, args.steps // 5)
    ms, _, per = time_steps(st, steps, 2)
    kt = kernel_times(st, steps, ["decode", "decode_merge"])
    kv = wl.decode_kv_bytes(w)
    alg = wl.decode_write_alg_bytes(w)
    dec_ms = kmean(kt, "decode")
    traffic = read_traffic("long_ctx_70b_decode_traffic", DECODE_SOURCES)
    result["long_context"] = {"workload": "long_ctx_70b_decode_bf16", "kv_bytes": kv, "ms_per_step": round(ms, 4),
                              "step_ms": per, "step_gbps": round(kv / (ms * 1e-3) / 1e9, 1),
                              "decode_kernel_ms": round(dec_ms, 4), "decode_kernel": kt["decode"],
                              "merge_kernel_ms": kmean(kt, "decode_merge"),
                              "kernel_gbps": round(alg / (dec_ms * 1e-3) / 1e9, 1),
                              "kernel_frac_hbm": round(alg / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                              "traffic": traffic["bytes"],
                              "traffic_over_alg": round(traffic["bytes"] / alg, 4) if traffic["bytes"] else None}
    rec, par = (None, None)
    if not args.no_cpu:
        # the shortest and the longest sequence of the batch
        order = np.argsort(w.seq_lens)
        rows = sorted({int(order[0]), int(order[-1])})
        rec, par = oracle_check(w, st.out, rows, TOL["bf16"], work_bytes=rows_kv_bytes(w, rows),
                                what="the shortest and the longest sequence's decode rows")
    result.setdefault("configs", {})["C4"] = decode_record("C4", w, per, kt, alg, traffic, rec, par)
    del st, w
    torch.cuda.empty_cache()


def bench_copy(args, result):
    """A plain device-to-device copy of 1 GiB: the known-size reference for the HBM byte counters."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms, _, _ = time_steps(lambda: dst.copy_(src), args.steps, args.warmup)
    result.update({"workload": "copy_1GiB", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                   "ms_per_copy": round(ms, 5), "GBps_read_plus_write": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 2)})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle (baseline and parity samples)")
    ap.add_argument("--only", default="",
                    choices=["", "tiny", "decode", "mixed", "cascade", "window", "long", "copy"])
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this library's path runs on a single GPU and has no multi-GPU form; "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import paged_kv_cache_418_amd as pk
    pk.load()
    result = {}
    if args.only == "copy":
        bench_copy(args, result)
    else:
        if args.only in ("", "decode"):
            bench_decode(args, result)
        if args.only in ("", "tiny"):
            bench_tiny(args, result)
        if args.only in ("", "mixed"):
            bench_mixed(args, result)
        if args.only in ("", "cascade"):
            bench_cascade(args, result)
        if args.only in ("", "window"):
            bench_window(args, result)
        if args.only in ("", "long"):
            bench_long(args, result)
    if "configs" in result:
        result["configs"] = dict(sorted(result["configs"].items()))
    print(json.dumps(result), flush=True)


def _sub(w, seqs):
    """A workload restricted to some of its sequences (same pools and tables)."""
    import dataclasses
    ql = w.q_lens[seqs]
    qsl = np.zeros(len(seqs) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(ql)
    rows = np.concatenate([np.arange(w.query_start_loc[s], w.query_start_loc[s + 1]) for s in seqs])
    r = torch.from_numpy(rows)
    return dataclasses.replace(w, name=w.name + "_sub", seq_lens=w.seq_lens[seqs].copy(), query_start_loc=qsl,
                               block_tables=w.block_tables[seqs].copy(), query=w.query[r].contiguous(),
                               new_k=w.new_k[r].contiguous(), new_v=w.new_v[r].contiguous())


if __name__ == "__main__":
    main()
