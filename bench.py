"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one pass of the whole path over one batch: slot mapping, the KV
write of the new tokens, then paged attention (decode with split-context
partitions and the log-sum-exp merge).  The headline workload is the
Llama-3-8B-shaped decode layer (batch 64, context U[512, 4096], 32 q / 8 kv
heads, head_dim 128, block 16, bf16); its value is algorithmic KV bytes per
second.  The mixed continuous-batching step (48 decodes + two 512-token
chunks) is timed too and gives the prefill TFLOP/s.

Prints one JSON line.  Inputs are seeded and synthetic and resident in HBM
before the timed region; two copies of the KV pool alternate between steps so
no step reads KV that the previous step left in the 256 MB last-level cache.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
METRIC = "paged decode KV GB/s (% of HBM peak) + prefill TFLOP/s at 1×MI355X"


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


class Step:
    """Device state of one workload and the calls of one step."""

    def __init__(self, w, copies: int = 2):
        import paged_kv_cache_418_amd as pk
        self.pk = pk
        self.w = w
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
        if w.is_decode:
            nb = pk.pa_decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, self.max_len, 0)
        else:
            nb = pk.pa_prefill_varlen_workspace_bytes(w.query_start_loc, w.seq_lens, w.num_q_heads, w.num_kv_heads,
                                                      w.head_dim)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        self.i = 0
        for kc, vc in self.pools:  # the new tokens' slots hold their K/V before any timed call
            self.write(kc, vc)
        torch.cuda.synchronize()

    def attend_next(self):
        kc, vc = self.pools[self.i % len(self.pools)]
        self.i += 1
        self.attend(kc, vc)

    def write(self, kc, vc):
        w, pk = self.w, self.pk
        pk.pa_slot_mapping(self.bt, self.sl, self.qsl, w.num_tokens, w.block_size, out=self.slots)
        if w.kv_dtype == "fp8":
            pk.pa_reshape_and_cache_fp8(self.nk, self.nv, kc, vc, self.slots, w.k_scale, w.v_scale)
        else:
            pk.pa_reshape_and_cache(self.nk, self.nv, kc, vc, self.slots)

    def attend(self, kc, vc):
        w, pk = self.w, self.pk
        if w.is_decode:
            if w.kv_dtype == "fp8":
                pk.pa_decode_fp8(self.q, kc, vc, self.bt, self.sl, w.scale, w.k_scale, w.v_scale, self.max_len,
                                 out=self.out, workspace=self.ws)
            else:
                pk.pa_decode(self.q, kc, vc, self.bt, self.sl, w.scale, self.max_len, out=self.out, workspace=self.ws)
        else:
            pk.pa_prefill_varlen(self.q, kc, vc, self.bt, self.sl, self.qsl, w.seq_lens, w.query_start_loc, w.scale,
                                 out=self.out, workspace=self.ws)

    def __call__(self):
        kc, vc = self.pools[self.i % len(self.pools)]
        self.i += 1
        self.write(kc, vc)
        self.attend(kc, vc)


def time_steps(fn, steps: int, warmup: int):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def time_each(fn, reps: int):
    """Per-call durations (ms) from events recorded around each call on the current stream."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def cpu_baseline(w, budget_s: float = 12.0):
    """The oracle on a bounded sample of the workload's sequences: KV GB/s on the host cores."""
    import oracle
    from paged_kv_cache_418_amd import workloads as wl
    threads = oracle.num_threads()
    order = list(range(w.num_seqs))
    done_bytes, spent, n = 0, 0.0, 0
    B = w.block_size
    while order and spent < budget_s:
        s = order.pop(0)
        rows = [int(w.query_start_loc[s])]
        t0 = time.perf_counter()
        oracle.attention_for(w, rows=rows)
        spent += time.perf_counter() - t0
        done_bytes += 2 * int(w.seq_lens[s]) * w.num_kv_heads * w.head_dim * w.kv_elem_bytes
        n += 1
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {w.num_seqs} sequences of {w.name} (fp64 C oracle, {spent:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default="", help="decode | mixed (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path has no multi-GPU form in this library (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    from paged_kv_cache_418_amd import workloads as wl
    result = {}
    if args.only in ("", "decode"):
        _log("generating llama3_8b_decode_bf16 ...")
        w = wl.llama3_8b_decode_bf16()
        st = Step(w)
        kv_bytes = wl.decode_kv_bytes(w)
        alg_bytes = wl.decode_alg_bytes(w)
        _log("timing decode step ...")
        ms, wall = time_steps(st, args.steps, args.warmup)
        # attention launch alone (decode kernel + LSE merge), events around each call
        per = time_each(st.attend_next, max(args.steps, 20))
        att_ms = float(np.mean(per))
        att_gbps = alg_bytes / (att_ms * 1e-3) / 1e9
        result.update({
            "metric": METRIC,
            "value": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
            "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "llama3_8b_decode_bf16", "num_seqs": w.num_seqs, "ctx": "U[512,4096]",
                       "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128, "block_size": 16,
                       "num_blocks": w.num_blocks, "kv_bytes": kv_bytes, "partition_size": 512},
            "pct_hbm": round(100 * kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
            "wall_s": round(wall, 4),
            "roofline": {"kernel": "paged decode attention (decode_mfma_kernel + decode_merge_kernel)",
                         "bound": "hbm", "achieved": round(att_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(att_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                         "launch_ms": round(att_ms, 5), "alg_bytes_per_launch": alg_bytes},
        })
        if not args.no_cpu:
            _log("cpu baseline ...")
            result["cpu_baseline"] = cpu_baseline(w)
        del st
        torch.cuda.empty_cache()

    if args.only in ("", "mixed"):
        _log("generating mixed_step_bf16 ...")
        w = wl.mixed_step_bf16()
        st = Step(w)
        ms, _ = time_steps(st, args.steps, args.warmup)
        flops = wl.prefill_flops(w)
        # the two chunks alone (prefill part) and the 48 decodes alone
        del st
        chunk_w = _sub(w, list(range(48, 50)))
        dec_w = _sub(w, list(range(48)))
        cs = Step(chunk_w, copies=1)
        per_c = time_each(cs.attend_next, max(args.steps, 20))
        pre_ms = float(np.mean(per_c))
        del cs
        ds = Step(dec_w, copies=2)
        dms, _ = time_steps(ds.attend_next, args.steps, args.warmup)
        dec_bytes = wl.decode_kv_bytes(dec_w)
        mixed = {"workload": "mixed_step_bf16", "ms_per_step": round(ms, 5),
                 "prefill_tflops": round(flops / (pre_ms * 1e-3) / 1e12, 2),
                 "prefill_pct_mfma": round(100 * flops / (pre_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 2),
                 "prefill_ms": round(pre_ms, 5), "prefill_gflop": round(flops / 1e9, 3),
                 "decode_part_gbps": round(dec_bytes / (dms * 1e-3) / 1e9, 2),
                 "decode_part_ms": round(dms, 5)}
        if "metric" in result:
            result["mixed_step"] = mixed
        else:
            result.update({"metric": METRIC, "value": mixed["decode_part_gbps"], "unit": "GB/s", "n_gpus": 1,
                           "steps": args.steps, "warmup": args.warmup, "ms_per_step": mixed["ms_per_step"],
                           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                           "data": "synthetic", "config": {"workload": "mixed_step_bf16"}, "mixed_step": mixed})
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
