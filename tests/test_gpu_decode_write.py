"""The decode step that stores its own new K/V (pa_decode_write, pa_decode_write_fp8), on the GPU.

Its contract is pa_write_kv (one new row per sequence) followed by pa_decode: the output and every byte of both
pools must equal those of the two calls, run on copies of the same pools; the output is also checked against
the CPU oracle at the parity tolerance (max-abs 2e-3 fp32, 1.5e-2 bf16, 6e-2 fp8 KV).  The pools the
workloads hold before the step have NaN (or the fp8 NaN code) at every new row's slot, so a row that is not
stored, or not attended from the new values, shows.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_418_amd as pk
from paged_kv_cache_418_amd import workloads as wl
from pa_gpu_util import TOL, max_err, say

pytestmark = pytest.mark.gpu


class Step:
    """Device copies of a decode workload; run(fused) returns (out, key pool, value pool)."""

    def __init__(self, w, key=None, value=None, seq_lens=None, max_len=None, prefix=0):
        self.w = w
        self.prefix = prefix  # > 0: the cascade entry points over this many shared blocks
        self.kc = w.k_cache.cuda()
        self.vc = w.v_cache.cuda()
        self.bt = torch.from_numpy(w.block_tables).cuda()
        self.sl = torch.from_numpy(w.seq_lens if seq_lens is None else seq_lens).cuda()
        self.qsl = torch.from_numpy(w.query_start_loc).cuda()
        self.q = w.query.cuda()
        self.nk = w.new_k.cuda() if key is None else key
        self.nv = w.new_v.cuda() if value is None else value
        self.max_len = int(w.seq_lens.max()) if max_len is None else max_len

    def run(self, fused: bool, num_splits: int = 0):
        w = self.w
        kc, vc = self.kc.clone(), self.vc.clone()
        out = torch.zeros_like(self.q)  # rows of empty sequences are left as they are
        fp8 = w.kv_dtype == "fp8"
        if self.prefix:
            return self._run_cascade(fused, num_splits, kc, vc, out)
        if fused:
            if fp8:
                pk.pa_decode_write_fp8(self.q, self.nk, self.nv, kc, vc, self.bt, self.sl, w.scale, w.k_scale,
                                       w.v_scale, self.max_len, num_splits, out=out)
            else:
                pk.pa_decode_write(self.q, self.nk, self.nv, kc, vc, self.bt, self.sl, w.scale, self.max_len,
                                   num_splits, out=out)
        else:
            scales = dict(k_scale=w.k_scale, v_scale=w.v_scale) if fp8 else {}
            pk.pa_write_kv(self.nk, self.nv, kc, vc, self.bt, self.sl, self.qsl, 1, **scales)
            if fp8:
                pk.pa_decode_fp8(self.q, kc, vc, self.bt, self.sl, w.scale, w.k_scale, w.v_scale, self.max_len,
                                 num_splits, out=out)
            else:
                pk.pa_decode(self.q, kc, vc, self.bt, self.sl, w.scale, self.max_len, num_splits, out=out)
        torch.cuda.synchronize()
        return out, kc, vc

    def _run_cascade(self, fused, num_splits, kc, vc, out):
        w, P = self.w, self.prefix
        fp8 = w.kv_dtype == "fp8"
        if fused:
            if fp8:
                pk.pa_decode_cascade_write_fp8(self.q, self.nk, self.nv, kc, vc, self.bt, self.sl, w.scale, w.k_scale,
                                               w.v_scale, self.max_len, P, num_splits, out=out)
            else:
                pk.pa_decode_cascade_write(self.q, self.nk, self.nv, kc, vc, self.bt, self.sl, w.scale, self.max_len,
                                           P, num_splits, out=out)
        else:
            scales = dict(k_scale=w.k_scale, v_scale=w.v_scale) if fp8 else {}
            pk.pa_write_kv(self.nk, self.nv, kc, vc, self.bt, self.sl, self.qsl, 1, **scales)
            if fp8:
                pk.pa_decode_cascade_fp8(self.q, kc, vc, self.bt, self.sl, w.scale, w.k_scale, w.v_scale,
                                         self.max_len, P, num_splits, out=out)
            else:
                pk.pa_decode_cascade(self.q, kc, vc, self.bt, self.sl, w.scale, self.max_len, P, num_splits, out=out)
        torch.cuda.synchronize()
        return out, kc, vc


def _bytes(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.uint8)


def _same(a, b) -> bool:
    return all(torch.equal(_bytes(x), _bytes(y)) for x, y in zip(a, b))


def _check(w, step: Step, num_splits: int = 0, oracle_check: bool = True):
    fused = step.run(True, num_splits)
    ref = step.run(False, num_splits)
    assert torch.equal(_bytes(fused[1]), _bytes(ref[1])), "key pool differs from pa_write_kv's"
    assert torch.equal(_bytes(fused[2]), _bytes(ref[2])), "value pool differs from pa_write_kv's"
    assert torch.equal(_bytes(fused[0]), _bytes(ref[0])), "output differs from pa_decode's after the write"
    if oracle_check:
        want = oracle.attention_for(w, pools=oracle.written_pools(w))
        err = max_err(fused[0], want)
        tol = TOL[w.kv_dtype if w.kv_dtype == "fp8" else w.q_dtype]
        say(f"  {w.name} splits={num_splits} max_abs_err={err:.3e} tol={tol}")
        assert err <= tol
    return fused


@pytest.mark.parametrize("kinds", [("bf16", "bf16"), ("bf16", "fp8"), ("f32", "fp8"), ("f32", "f32")])
@pytest.mark.parametrize("heads", [(4, 2, 64), (32, 8, 128), (12, 4, 128), (48, 1, 64), (64, 2, 128)])
@pytest.mark.parametrize("num_splits", [0, 1, 7])
def test_decode_write_equals_write_then_decode(kinds, heads, num_splits):
    """Random lengths 1..700 (partly filled last blocks, sequences inside one block, pieces split across shares),
    head sizes 64 and 128, one to three q-head groups per kv head (48 and 64 q heads per kv head)."""
    Hq, Hkv, D = heads
    seed = 900 + Hq + 3 * Hkv + D + num_splits + len(kinds[0]) + 7 * len(kinds[1])
    w = wl.random_case(seed, num_seqs=7, ctx_range=(1, 700), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                       q_dtype=kinds[0], kv_dtype=kinds[1], k_scale=0.05, v_scale=0.04)
    say("decode_write", kinds, heads, num_splits, "seq_lens", w.seq_lens.tolist())
    _check(w, Step(w), num_splits)


@pytest.mark.parametrize("maker", [wl.llama3_8b_decode_bf16, wl.llama3_8b_decode_fp8])
def test_decode_write_llama3_8b_full(maker):
    """The bench's decode batches at full size (64 sequences x 3000-5000 tokens, 32 / 8 heads, head size 128):
    bit-identical to the two calls; oracle at the parity tolerance."""
    w = maker()
    say("decode_write full", w.name)
    _check(w, Step(w))


def test_decode_write_block_boundaries():
    """New rows at every offset of a block: lengths 1..33 (first row of a block, last row, second block)."""
    w = wl.build("boundaries", seed=931, ctx_lens=list(range(1, 34)), q_lens=[1] * 33, num_q_heads=8,
                 num_kv_heads=2, head_dim=128, q_dtype="bf16", kv_dtype="bf16")
    say("decode_write boundaries")
    _check(w, Step(w))
    _check(w, Step(w), num_splits=5)


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_decode_write_unaligned_rows_take_the_separate_write(kind):
    """key/value rows 2 bytes off 16-byte alignment: the KV write runs as its own launch; same bytes."""
    w = wl.random_case(941 + len(kind), num_seqs=5, ctx_range=(1, 300), num_q_heads=8, num_kv_heads=4, head_dim=64,
                       q_dtype="bf16", kv_dtype=kind, k_scale=0.05, v_scale=0.04)
    S, H, D = w.new_k.shape
    bufk = torch.empty(S * H * D + 8, dtype=torch.bfloat16, device="cuda")
    bufv = torch.empty_like(bufk)
    key = bufk[1:1 + S * H * D].view(S, H, D)
    value = bufv[1:1 + S * H * D].view(S, H, D)
    key.copy_(w.new_k.cuda())
    value.copy_(w.new_v.cuda())
    assert key.data_ptr() % 16 != 0
    say("decode_write unaligned", kind)
    _check(w, Step(w, key=key, value=value))


def test_decode_write_strided_rows():
    """key/value as views into a wider per-token buffer (a fused QKV projection's output): row stride
    (Hq + 2 Hkv) * D elements, still 16-byte aligned, so the decode launch stores the rows itself."""
    w = wl.random_case(951, num_seqs=6, ctx_range=(1, 400), num_q_heads=16, num_kv_heads=4, head_dim=128,
                       q_dtype="bf16", kv_dtype="bf16")
    S, H, D = w.new_k.shape
    qkv = torch.full((S, (16 + 2 * H) * D), float("nan"), dtype=torch.bfloat16, device="cuda")
    key = qkv[:, 16 * D:(16 + H) * D].view(S, H, D)
    value = qkv[:, (16 + H) * D:].view(S, H, D)
    key.copy_(w.new_k.cuda())
    value.copy_(w.new_v.cuda())
    say("decode_write strided rows")
    _check(w, Step(w, key=key, value=value))


def test_decode_write_cut_and_empty_sequences():
    """A sequence longer than max_seq_len is attended over its first max_seq_len positions and its row is not
    stored; a sequence of length 0 stores nothing and attends nothing; the others are stored and attended."""
    w = wl.random_case(961, num_seqs=6, ctx_range=(40, 300), num_q_heads=8, num_kv_heads=2, head_dim=128,
                       q_dtype="bf16", kv_dtype="bf16")
    sl = w.seq_lens.copy()
    max_len = int(np.sort(sl)[-2])  # the longest sequence alone is cut
    cut = int(np.argmax(sl))
    assert sl[cut] > max_len
    sl[0 if cut != 0 else 1] = 0
    say("decode_write cut / empty", sl.tolist(), max_len)
    step = Step(w, seq_lens=sl, max_len=max_len)
    out, kc, vc = step.run(True)
    ref_out, ref_kc, ref_vc = step.run(False)
    # the two calls store the cut sequence's row; the fused call leaves its slot as it was
    pos = int(sl[cut]) - 1
    blk, off = int(w.block_tables[cut, pos // 16]), pos % 16
    assert torch.equal(_bytes(kc[blk, off]), _bytes(step.kc[blk, off]))
    assert torch.equal(_bytes(vc[blk, off]), _bytes(step.vc[blk, off]))
    ref_kc[blk, off] = step.kc[blk, off]
    ref_vc[blk, off] = step.vc[blk, off]
    assert _same((kc, vc), (ref_kc, ref_vc))
    assert torch.equal(_bytes(out), _bytes(ref_out))


def test_decode_write_repeats_bit_identical():
    """The same step twice on the same pools (the second finds its rows already stored): same bytes."""
    w = wl.random_case(971, num_seqs=9, ctx_range=(1, 900), num_q_heads=32, num_kv_heads=8, head_dim=128,
                       q_dtype="bf16", kv_dtype="fp8", k_scale=0.05, v_scale=0.04)
    step = Step(w)
    first = step.run(True)
    step.kc, step.vc = first[1], first[2]
    second = step.run(True)
    assert _same(first, second)


# ---- the cascade decode step (pa_decode_cascade_write*): the same contract over a batch whose tables begin with
# the same physical blocks; the suffix waves of the prefix tiles' launch store the rows (bf16 queries over bf16 or
# fp8 pools), the other paths run the write first

@pytest.mark.parametrize("kinds", [("bf16", "bf16"), ("bf16", "fp8"), ("f32", "fp8"), ("f32", "f32")])
@pytest.mark.parametrize("heads", [(32, 8, 128), (4, 2, 64), (16, 1, 128)])
@pytest.mark.parametrize("num_splits", [0, 7])
def test_cascade_write_equals_write_then_cascade(kinds, heads, num_splits):
    """Shared prefixes of 3 blocks, suffixes 1..300 tokens (new rows at every block offset)."""
    Hq, Hkv, D = heads
    seed = 980 + Hq + 3 * Hkv + D + num_splits + len(kinds[0]) + 7 * len(kinds[1])
    w = wl.random_case(seed, num_seqs=9, ctx_range=(49, 348), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                       q_dtype=kinds[0], kv_dtype=kinds[1], k_scale=0.05, v_scale=0.04, shared_prefix_tokens=48)
    say("cascade_write", kinds, heads, num_splits, "seq_lens", w.seq_lens.tolist())
    _check(w, Step(w, prefix=3), num_splits)


def test_cascade_write_prefix_shared_fp8_full():
    """The bench's prefix-shared batch at full size (128 requests, a 2048-token shared prefix, suffixes
    U[128,1024], E4M3 pools): bit-identical to the two calls; oracle at the parity tolerance."""
    w = wl.prefix_shared_fp8_decode()
    say("cascade_write full", w.name)
    _check(w, Step(w, prefix=w.shared_prefix_blocks))


# ---- the mixed step (pa_prefill_varlen_write): decode rows and chunked-prefill chunks in one flattened batch;
# in one fused launch the decode waves store their rows and the chunks' tiles read their new keys from the input
# rows while one item per row tile stores them; otherwise the write runs first

def _varlen_check(w, key=None, value=None):
    kc0, vc0 = w.k_cache.cuda(), w.v_cache.cuda()
    bt = torch.from_numpy(w.block_tables).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    qsl = torch.from_numpy(w.query_start_loc).cuda()
    q = w.query.cuda()
    nk = w.new_k.cuda() if key is None else key
    nv = w.new_v.cuda() if value is None else value
    res = []
    for fused in (True, False):
        kc, vc = kc0.clone(), vc0.clone()
        out = torch.zeros_like(q)
        if fused:
            pk.pa_prefill_varlen_write(q, nk, nv, kc, vc, bt, sl, qsl, w.seq_lens, w.query_start_loc, w.scale,
                                       out=out)
        else:
            pk.pa_write_kv(nk, nv, kc, vc, bt, sl, qsl, int(w.q_lens.max()))
            pk.pa_prefill_varlen(q, kc, vc, bt, sl, qsl, w.seq_lens, w.query_start_loc, w.scale, out=out)
        torch.cuda.synchronize()
        res.append((out, kc, vc))
    (out, kc, vc), (rout, rkc, rvc) = res
    assert torch.equal(_bytes(kc), _bytes(rkc)), "key pool differs from pa_write_kv's"
    assert torch.equal(_bytes(vc), _bytes(rvc)), "value pool differs from pa_write_kv's"
    assert torch.equal(_bytes(out), _bytes(rout)), "output differs from pa_prefill_varlen's after the write"
    return out


def _mixed(seed, heads, num_seqs=10, q_dtype="bf16", kv="bf16"):
    Hq, Hkv, D = heads
    rng = np.random.default_rng(seed)
    q_lens = [1 if i % 2 == 0 else int(rng.integers(2, 300)) for i in range(num_seqs)]
    ctx = [int(q + rng.integers(0, 1500)) for q in q_lens]
    ctx[1] = q_lens[1]  # one chunk from an empty cache: its filler key is a new row
    return wl.build(f"mixed_write_{seed}", seed=seed, ctx_lens=ctx, q_lens=q_lens, num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=D, q_dtype=q_dtype, kv_dtype=kv)


@pytest.fixture
def fused_mode():
    def set_mode(mode):
        pk.set_fused(mode)
    yield set_mode
    pk.set_fused(-1)


@pytest.mark.parametrize("mode", [2, 0])
@pytest.mark.parametrize("seed,heads", [(991, (32, 8, 128)), (992, (8, 2, 64)), (993, (48, 1, 128)),
                                        (994, (12, 4, 128))])
def test_varlen_write_equals_write_then_prefill(fused_mode, mode, seed, heads):
    """Mixed batches (decode rows, chunks with and without cached tokens, partly filled blocks at both ends of a
    chunk) with the fused launch forced on (the rows stored inside it) and off (the write's own launch)."""
    fused_mode(mode)
    w = _mixed(seed, heads)
    say("varlen_write", mode, heads, "q_lens", w.q_lens.tolist())
    out = _varlen_check(w)
    want = oracle.attention_for(w, pools=oracle.written_pools(w))
    err = max_err(out, want)
    say(f"  max_abs_err={err:.3e}")
    assert err <= TOL["bf16"]


def test_varlen_write_fp32_takes_the_separate_write(fused_mode):
    """fp32 pools and activations (every chunk token a decode row of its own): the write runs first."""
    fused_mode(2)
    w = _mixed(995, (8, 2, 128), q_dtype="f32", kv="f32")
    say("varlen_write fp32")
    _varlen_check(w)


def test_varlen_write_unaligned_rows(fused_mode):
    """Rows 2 bytes off 16-byte alignment: the write runs as its own launch."""
    fused_mode(2)
    w = _mixed(996, (8, 2, 64))
    T, H, D = w.new_k.shape
    buf = torch.empty(2, T * H * D + 8, dtype=torch.bfloat16, device="cuda")
    key = buf[0, 1:1 + T * H * D].view(T, H, D)
    value = buf[1, 1:1 + T * H * D].view(T, H, D)
    key.copy_(w.new_k.cuda())
    value.copy_(w.new_v.cuda())
    _varlen_check(w, key, value)


def test_varlen_write_mixed_step_full(fused_mode):
    """The bench's mixed step at full size (48 decode rows + two 512-token chunks at 0 and 1536 cached tokens),
    fused launch forced: bit-identical to the two calls."""
    fused_mode(2)
    w = wl.mixed_step_bf16()
    say("varlen_write mixed step full")
    _varlen_check(w)


@pytest.mark.parametrize("shape", ["decode_rows_only", "chunks_only"])
def test_varlen_write_batches_that_do_not_fuse(fused_mode, shape):
    """A batch of decode rows only, and one of chunks only: no fused launch, so the write runs first; same bytes."""
    fused_mode(2)
    rng = np.random.default_rng(997)
    n = 7
    q_lens = [1] * n if shape == "decode_rows_only" else [int(rng.integers(2, 200)) for _ in range(n)]
    ctx = [int(q + rng.integers(0, 900)) for q in q_lens]
    w = wl.build(f"varlen_write_{shape}", seed=997, ctx_lens=ctx, q_lens=q_lens, num_q_heads=16, num_kv_heads=4,
                 head_dim=128, q_dtype="bf16", kv_dtype="bf16")
    say("varlen_write", shape)
    _varlen_check(w)


# ---- the sliding-window and chunked-local decode steps (pa_decode_window_write*, pa_decode_local_write*)

def _masked_run(w, mask, size, fused, num_splits):
    kc, vc = w.k_cache.cuda(), w.v_cache.cuda()
    bt = torch.from_numpy(w.block_tables).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    qsl = torch.from_numpy(w.query_start_loc).cuda()
    q, nk, nv = w.query.cuda(), w.new_k.cuda(), w.new_v.cuda()
    out = torch.zeros_like(q)
    L = int(w.seq_lens.max())
    fp8 = w.kv_dtype == "fp8"
    sc = (w.k_scale, w.v_scale) if fp8 else ()
    if fused:
        fn = {("window", False): pk.pa_decode_window_write, ("window", True): pk.pa_decode_window_write_fp8,
              ("local", False): pk.pa_decode_local_write, ("local", True): pk.pa_decode_local_write_fp8}[(mask, fp8)]
        fn(q, nk, nv, kc, vc, bt, sl, w.scale, *sc, L, size, num_splits, out=out)
    else:
        scales = dict(k_scale=w.k_scale, v_scale=w.v_scale) if fp8 else {}
        pk.pa_write_kv(nk, nv, kc, vc, bt, sl, qsl, 1, **scales)
        fn = {("window", False): pk.pa_decode_window, ("window", True): pk.pa_decode_window_fp8,
              ("local", False): pk.pa_decode_local, ("local", True): pk.pa_decode_local_fp8}[(mask, fp8)]
        fn(q, kc, vc, bt, sl, w.scale, *sc, L, size, num_splits, out=out)
    torch.cuda.synchronize()
    return out, kc, vc


@pytest.mark.parametrize("kinds", [("bf16", "bf16"), ("bf16", "fp8"), ("f32", "fp8"), ("f32", "f32")])
@pytest.mark.parametrize("mask,size", [("window", 1), ("window", 37), ("window", 200), ("window", 100000),
                                       ("local", 16), ("local", 100)])
@pytest.mark.parametrize("num_splits", [0, 7])
def test_masked_decode_write_equals_write_then_masked_decode(kinds, mask, size, num_splits):
    seed = 1100 + size % 97 + num_splits + len(kinds[0]) + 3 * len(kinds[1]) + (50 if mask == "local" else 0)
    w = wl.random_case(seed, num_seqs=7, ctx_range=(1, 700), num_q_heads=8, num_kv_heads=2, head_dim=128,
                       q_dtype=kinds[0], kv_dtype=kinds[1], k_scale=0.05, v_scale=0.04)
    say("masked decode_write", mask, size, kinds, num_splits)
    fused = _masked_run(w, mask, size, True, num_splits)
    ref = _masked_run(w, mask, size, False, num_splits)
    assert _same(fused[1:], ref[1:]), "pools differ from pa_write_kv's"
    assert torch.equal(_bytes(fused[0]), _bytes(ref[0])), "output differs from the masked decode's after the write"
