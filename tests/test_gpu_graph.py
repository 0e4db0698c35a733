"""The path under HIP graph capture, on the GPU through the C ABI.

A step (KV write through the block tables, then attention) is captured once and replayed
several times.  Before each replay the pools are reset from a pristine copy and the output
is poisoned, with other eager work and synchronisations in between; every replay must equal
the eager step bit for bit.  The library records no memset and takes its work list as kernel
arguments, so a captured step replays the plan made at capture.
"""
import pytest
import torch

import paged_kv_cache_418_amd as pk
from paged_kv_cache_418_amd import workloads as wl
from pa_gpu_util import DevWorkload, say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _check_replays(d: DevWorkload, attend, replays: int = 4):
    """attend(d) -> output tensor; the step is write_kv + attend on pools reset from a pristine copy."""
    w = d.w
    k0, v0 = d.k_cache.clone(), d.v_cache.clone()
    scales = dict(k_scale=w.k_scale, v_scale=w.v_scale) if w.kv_dtype == "fp8" else {}
    max_q = int(w.q_lens.max())

    def step():
        d.k_cache.copy_(k0)
        d.v_cache.copy_(v0)
        pk.pa_write_kv(d.new_k, d.new_v, d.k_cache, d.v_cache, d.block_tables, d.seq_lens, d.qsl, max_q, **scales)
        return attend(d)

    eager = step().clone()
    eager_k = d.k_cache.clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    for r in range(replays):
        out.fill_(float("nan"))
        d.k_cache.fill_(0)  # the replay's own copy must restore it
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"  replay {r}")
        assert torch.equal(_bits(out), _bits(eager)), f"replay {r}"
        assert torch.equal(_bits(d.k_cache), _bits(eager_k)), f"replay {r} pools"
        del junk


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_graph_replay_mixed_batch(kv):
    """Decode rows and chunked-prefill chunks in one varlen call (fp8: with the staging kernel)."""
    w = wl.random_case(991 if kv == "bf16" else 992, num_seqs=9, ctx_range=(1, 1500), chunk_range=(1, 400),
                       num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16", kv_dtype=kv, k_scale=0.05,
                       v_scale=0.04)
    say("graph mixed", kv, list(w.q_lens), list(w.seq_lens))
    _check_replays(DevWorkload(w), lambda d: d.prefill())


@pytest.mark.parametrize("num_splits", [0, 7])
def test_graph_replay_decode(num_splits):
    """Split decode with its merge launch."""
    w = wl.random_case(993 + num_splits, num_seqs=24, ctx_range=(1, 3000), num_q_heads=32, num_kv_heads=8,
                       head_dim=128, q_dtype="bf16", kv_dtype="bf16")
    say("graph decode", num_splits)
    _check_replays(DevWorkload(w), lambda d: d.decode(num_splits))


def test_graph_replay_cascade():
    w = wl.random_case(995, num_seqs=16, ctx_range=(16 * 6 + 1, 900), num_q_heads=32, num_kv_heads=8, head_dim=128,
                       q_dtype="bf16", kv_dtype="fp8", k_scale=0.05, v_scale=0.04, shared_prefix_tokens=16 * 6)
    say("graph cascade")
    _check_replays(DevWorkload(w), lambda d: d.cascade(6))
