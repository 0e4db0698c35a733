"""pa_decode_static (the decode entry point that allocates nothing) against pa_decode.

Both run the same kernels and the same work split; pa_decode_static's scratch is the
library's static device array instead of a caller workspace.  Two calls in a row, the
second on a smaller batch, each compared with pa_decode bit for bit and with the oracle
within the bf16 tolerance; then a batch too large for the static scratch is refused.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_418_amd as pk
from paged_kv_cache_418_amd import workloads as wl
from pa_gpu_util import TOL, DevWorkload, max_err, say

pytestmark = pytest.mark.gpu


def _static_then_workspace(w, num_splits):
    d = DevWorkload(w)
    d.write_new_tokens()  # the new tokens' slots hold NaN until they are written
    L = d.max_seq_len()
    got = pk.pa_decode_static(d.query, d.k_cache, d.v_cache, d.block_tables, d.seq_lens, w.scale, L, num_splits)
    torch.cuda.synchronize()
    ref_ws = pk.pa_decode(d.query, d.k_cache, d.v_cache, d.block_tables, d.seq_lens, w.scale, L, num_splits)
    torch.cuda.synchronize()
    return got, ref_ws


@pytest.mark.parametrize("num_splits", [0, 37])
def test_static_decode_two_calls_match_workspace_decode(num_splits):
    big = wl.random_case(4501, num_seqs=48, ctx_range=(300, 3000), num_q_heads=32, num_kv_heads=8, head_dim=128,
                         q_dtype="bf16", kv_dtype="bf16")
    small = wl.random_case(4502, num_seqs=5, ctx_range=(1, 700), num_q_heads=32, num_kv_heads=8, head_dim=128,
                           q_dtype="bf16", kv_dtype="bf16")
    for name, w in (("big", big), ("small", small)):
        say(f"static decode {name} (splits {num_splits})")
        got, ref_ws = _static_then_workspace(w, num_splits)
        assert torch.equal(got.view(torch.int16), ref_ws.view(torch.int16)), "differs from pa_decode"
        err = max_err(got, oracle.attention_for(w, pools=oracle.written_pools(w)))
        say(f"  max_abs_err={err:.3e}")
        assert err <= TOL["bf16"]


def test_static_decode_fp32_and_llama_layer():
    w = wl.random_case(4503, num_seqs=6, ctx_range=(1, 400), num_q_heads=8, num_kv_heads=2, head_dim=64,
                       q_dtype="f32", kv_dtype="f32")
    got, ref_ws = _static_then_workspace(w, 0)
    assert torch.equal(got, ref_ws)
    assert max_err(got, oracle.attention_for(w, pools=oracle.written_pools(w))) <= TOL["f32"]
    w = wl.llama3_8b_decode_bf16()
    say("static decode, Llama-3-8B layer")
    got, ref_ws = _static_then_workspace(w, 0)
    assert torch.equal(got.view(torch.int16), ref_ws.view(torch.int16))


def test_static_decode_refuses_batches_beyond_its_scratch():
    # 4096 sequences x 64 q heads x d 128 with 4096 shares per kv head: partials for 8192 pieces x 64 x 128 fp32
    # = 256 MiB, beyond the 32 MiB array; refused before any launch
    need = pk.pa_decode_workspace_bytes(4096, 64, 8, 128, 8192, 4096)
    assert need > 32 << 20
    lib = pk.load()
    fake = 0x10000
    st = lib.pa_decode_static(fake, fake, fake, fake, fake, 512, fake, 4096, 64, 8, 128, 16, 100000, 8192, 0.088,
                              pk.PA_BF16, 4096, None)
    assert st == 4
    assert b"static" in lib.pa_last_error()
