"""Metadata validation (pa_set_validate(1), the checks PA_VALIDATE=1 turns on): good metadata passes and gives the
same output as unchecked calls; each kind of bad metadata is refused with PA_ERR_SHAPE before anything is launched.
Every bad case is also one the kernels survive unchecked (ids clamped into the pool, positions past max_seq_len not
read, tiles planned from other lengths clamped to the device's), so nothing here can fault the GPU even if a check
were missing."""
import numpy as np
import pytest
import torch

import paged_kv_cache_418_amd as pk
from paged_kv_cache_418_amd import _binding as b
from paged_kv_cache_418_amd import workloads as wl
from pa_gpu_util import DevWorkload, say

pytestmark = pytest.mark.gpu

SHAPE = 2  # PA_ERR_SHAPE


@pytest.fixture
def validating():
    pk.set_validate(1)
    yield
    pk.set_validate(-1)


def _refused(fn, *args, **kw):
    with pytest.raises(b.PAError) as e:
        fn(*args, **kw)
    assert e.value.status == SHAPE, e.value
    assert "PA_VALIDATE" in e.value.message
    return e.value.message


def test_good_metadata_passes_with_the_same_output(validating):
    w = wl.random_case(801, num_seqs=6, ctx_range=(1, 300), chunk_range=(1, 80), num_q_heads=8, num_kv_heads=2,
                       head_dim=128, q_dtype="bf16", kv_dtype="bf16")
    say("validate good")
    d = DevWorkload(w)
    d.write_new_tokens()
    checked = d.prefill()
    pk.set_validate(0)
    unchecked = d.prefill()
    torch.cuda.synchronize()
    assert torch.equal(checked.view(torch.int16), unchecked.view(torch.int16))


def test_block_id_out_of_range_is_refused(validating):
    w = wl.llama3_8b_decode_bf16()
    say("validate bad block id")
    d = DevWorkload(w)
    d.block_tables[3, 0] = w.num_blocks  # one past the pool
    msg = _refused(d.decode)
    assert "block_tables[3][0]" in msg


def test_seq_len_past_max_seq_len_is_refused(validating):
    w = wl.llama3_8b_decode_bf16()
    say("validate long seq")
    d = DevWorkload(w)
    longest = int(np.argmax(w.seq_lens))
    d.seq_lens[longest] += 1  # past max_seq_len (taken from the host copy)
    _refused(d.decode)


def test_duplicate_slots_are_refused(validating):
    w = wl.random_case(803, num_seqs=4, ctx_range=(20, 100), chunk_range=(2, 10), num_q_heads=4, num_kv_heads=2,
                       head_dim=64, q_dtype="bf16", kv_dtype="bf16")
    say("validate duplicate slots")
    d = DevWorkload(w)
    slots = pk.pa_slot_mapping(d.block_tables, d.seq_lens, d.qsl, w.num_tokens)
    slots[1] = slots[0]
    _refused(pk.pa_reshape_and_cache, d.new_k, d.new_v, d.k_cache, d.v_cache, slots)


def test_non_monotone_query_start_loc_is_refused(validating):
    w = wl.random_case(804, num_seqs=4, ctx_range=(20, 100), chunk_range=(2, 10), num_q_heads=4, num_kv_heads=2,
                       head_dim=64, q_dtype="bf16", kv_dtype="bf16")
    say("validate qsl")
    d = DevWorkload(w)
    bad = d.qsl.clone()
    bad[2] = bad[1] - 1  # sequence 1 would have a negative q_len
    _refused(pk.pa_slot_mapping, d.block_tables, d.seq_lens, bad, w.num_tokens)


def test_host_and_device_metadata_must_agree(validating):
    w = wl.random_case(805, num_seqs=4, ctx_range=(50, 300), chunk_range=(2, 40), num_q_heads=8, num_kv_heads=2,
                       head_dim=128, q_dtype="bf16", kv_dtype="bf16")
    say("validate host/device")
    d = DevWorkload(w)
    host_sl = w.seq_lens.copy()
    host_sl[0] -= 1  # a plan for other lengths than the device holds
    _refused(pk.pa_prefill_varlen, d.query, d.k_cache, d.v_cache, d.block_tables, d.seq_lens, d.qsl, host_sl,
             w.query_start_loc, w.scale)


def test_cascade_tables_must_share_the_prefix(validating):
    w = wl.random_case(806, num_seqs=6, ctx_range=(100, 400), num_q_heads=8, num_kv_heads=2, head_dim=128,
                       q_dtype="bf16", kv_dtype="bf16", shared_prefix_tokens=64)
    say("validate cascade prefix")
    d = DevWorkload(w)
    d.block_tables[4, 2] = d.block_tables[4, 5]  # a valid block, but not the shared one
    _refused(d.cascade, 4)
