"""Seeded synthetic inputs for paged-KV attention.

This module only draws random numbers and lays them out; it performs none of
the attention, addressing or quantisation arithmetic.  Both the CPU oracle
(through the tests) and the HIP path consume what it produces.

Layout of what a :class:`Workload` holds (host memory, torch CPU tensors or
numpy arrays):

* ``k_cache`` / ``v_cache``: the physical block pool, ``[num_blocks, block_size,
  num_kv_heads, head_dim]``, dtype float32 / bfloat16 / uint8 (fp8 E4M3 codes).
  One pool per tensor, as in the page "vLLM 架构概述" §2 (a pool of physical
  blocks that per-request block tables point into).
* ``block_tables``: int32 ``[num_seqs, max_blocks_per_seq]``; columns past a
  sequence's last block point at a NaN-filled poison block.
* ``seq_lens``: int32 ``[num_seqs]``, tokens of each sequence *including* the
  new tokens of this step.
* ``query_start_loc``: int32 ``[num_seqs + 1]``; the batch is one flattened
  super-sequence of new tokens (reading note on "Inside vLLM", core point 2).
* ``query``: ``[num_tokens, num_q_heads, head_dim]``; ``new_k`` / ``new_v``:
  ``[num_tokens, num_kv_heads, head_dim]``, the K/V of the new tokens, to be
  written into the pool before attention.

Recipe (one ``numpy.random.default_rng(seed)`` per workload, fixed draw order):
context lengths, then the block permutation, then the K pool, V pool, query,
new K, new V, each ``standard_normal`` float32; bf16 by round-to-nearest-even
through torch; fp8 pools store torch ``float8_e4m3fn`` casts of N(0,1)/scale.
Every pool position not covered by a sequence's cached tokens is NaN (fp8:
code 0x7F), including the slots the new tokens will be written to, the tails
of last blocks and the unused blocks of the pool.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

FP8_NAN_CODE = 0x7F
BLOCK_SIZE = 16

# Generation of big pools is done in slabs of blocks so that the float32
# staging copy stays small.
_SLAB_BLOCKS = 2048


@dataclasses.dataclass
class Workload:
    name: str
    q_dtype: str            # "f32" | "bf16"
    kv_dtype: str           # "f32" | "bf16" | "fp8"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    seq_lens: np.ndarray          # int32 [S]
    query_start_loc: np.ndarray   # int32 [S+1]
    block_tables: np.ndarray      # int32 [S, max_blocks]
    k_cache: torch.Tensor         # [NB, B, Hkv, D]
    v_cache: torch.Tensor
    query: torch.Tensor           # [T, Hq, D]
    new_k: torch.Tensor           # [T, Hkv, D]
    new_v: torch.Tensor
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    poison_block: int = -1
    partition_size: int = 512
    shared_prefix_blocks: int = 0

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int32)

    @property
    def is_decode(self) -> bool:
        return bool(np.all(self.q_lens == 1))

    @property
    def kv_elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.kv_dtype]

    @property
    def q_elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2}[self.q_dtype]

    def copy_pools(self):
        return self.k_cache.clone(), self.v_cache.clone()


def _torch_dtype(kind: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[kind]


def _cast(x32: np.ndarray, kind: str, scale: float = 1.0) -> torch.Tensor:
    t = torch.from_numpy(x32)
    if kind == "f32":
        return t.clone()
    if kind == "bf16":
        return t.to(torch.bfloat16)
    if kind == "fp8":
        return (t / scale).to(torch.float8_e4m3fn).view(torch.uint8)
    raise ValueError(kind)


def _draw_pool(rng, nb, b, hkv, d, kind, scale, covered):
    """Draws one pool slab by slab and poisons positions where covered is False."""
    out = torch.empty((nb, b, hkv, d), dtype=_torch_dtype(kind))
    for s0 in range(0, nb, _SLAB_BLOCKS):
        s1 = min(nb, s0 + _SLAB_BLOCKS)
        x = rng.standard_normal((s1 - s0, b, hkv, d), dtype=np.float32)
        out[s0:s1] = _cast(x, kind, scale)
    mask = torch.from_numpy(~covered)  # [NB, B] True where poisoned
    if kind == "fp8":
        out[mask] = FP8_NAN_CODE
    else:
        out[mask] = float("nan")
    return out


def build(name: str, *, seed: int, ctx_lens: Sequence[int], q_lens: Sequence[int],
          num_q_heads: int, num_kv_heads: int, head_dim: int, q_dtype: str,
          kv_dtype: str, max_blocks: Optional[int] = None, num_blocks: Optional[int] = None,
          rng: Optional[np.random.Generator] = None, shared_prefix_tokens: int = 0,
          k_scale: float = 1.0, v_scale: float = 1.0, partition_size: int = 512,
          block_size: int = BLOCK_SIZE, pool_slack: float = 1.10) -> Workload:
    """Lays out a workload from context lengths that were already drawn.

    ``rng`` continues the stream that drew ``ctx_lens`` (a fresh one from
    ``seed`` if None).  ``shared_prefix_tokens`` (a multiple of the block size)
    makes every sequence's first blocks the same physical blocks.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)
    S = ctx.shape[0]
    assert ql.shape[0] == S and np.all(ql >= 1) and np.all(ctx >= ql)
    B = block_size
    assert shared_prefix_tokens % B == 0
    n_shared = shared_prefix_tokens // B
    nblk = (ctx + B - 1) // B
    if n_shared:
        assert np.all(ctx > shared_prefix_tokens)
        unique_needed = int(n_shared + np.sum(nblk - n_shared))
    else:
        unique_needed = int(np.sum(nblk))
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_slack * unique_needed))
    # at least one spare block serves as the poison target of unused columns
    assert num_blocks >= unique_needed + 1, (num_blocks, unique_needed)
    if max_blocks is None:
        max_blocks = int(nblk.max())
    assert max_blocks >= int(nblk.max())

    perm = rng.permutation(num_blocks).astype(np.int32)
    poison_block = int(perm[unique_needed])
    tables = np.full((S, max_blocks), poison_block, dtype=np.int32)
    covered = np.zeros((num_blocks, B), dtype=bool)
    cursor = n_shared
    for s in range(S):
        if n_shared:
            tables[s, :n_shared] = perm[:n_shared]
            own = int(nblk[s] - n_shared)
            tables[s, n_shared:n_shared + own] = perm[cursor:cursor + own]
        else:
            own = int(nblk[s])
            tables[s, :own] = perm[cursor:cursor + own]
        cursor += own
        cached = int(ctx[s] - ql[s])
        for j in range(int(nblk[s])):
            lo = j * B
            n_cov = min(B, max(0, cached - lo))
            if n_cov:
                covered[tables[s, j], :n_cov] = True
    assert cursor == unique_needed

    k_cache = _draw_pool(rng, num_blocks, B, num_kv_heads, head_dim, kv_dtype, k_scale, covered)
    v_cache = _draw_pool(rng, num_blocks, B, num_kv_heads, head_dim, kv_dtype, v_scale, covered)
    T = int(ql.sum())
    new_dtype = q_dtype  # new K/V arrive in the activation dtype
    query = _cast(rng.standard_normal((T, num_q_heads, head_dim), dtype=np.float32), q_dtype)
    new_k = _cast(rng.standard_normal((T, num_kv_heads, head_dim), dtype=np.float32), new_dtype)
    new_v = _cast(rng.standard_normal((T, num_kv_heads, head_dim), dtype=np.float32), new_dtype)
    qsl = np.zeros(S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(ql)
    return Workload(
        name=name, q_dtype=q_dtype, kv_dtype=kv_dtype, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=B, num_blocks=num_blocks,
        seq_lens=ctx.astype(np.int32), query_start_loc=qsl, block_tables=tables,
        k_cache=k_cache, v_cache=v_cache, query=query, new_k=new_k, new_v=new_v,
        scale=float(np.float32(1.0 / math.sqrt(head_dim))), k_scale=k_scale, v_scale=v_scale,
        poison_block=poison_block, partition_size=partition_size,
        shared_prefix_blocks=n_shared)


# --- the five named workloads -------------------------------------------------

SEED_BASE = 418_000


def tiny_fp32_decode() -> Workload:
    """4 sequences, context lengths {1,17,33,100}, GQA 4 q / 2 kv heads, D 64, fp32, 64-block pool."""
    rng = np.random.default_rng(SEED_BASE + 0)
    ctx = [1, 17, 33, 100]
    return build("tiny_fp32_decode", seed=SEED_BASE, rng=rng, ctx_lens=ctx, q_lens=[1] * 4,
                 num_q_heads=4, num_kv_heads=2, head_dim=64, q_dtype="f32", kv_dtype="f32",
                 num_blocks=64, max_blocks=7)


def llama3_8b_decode_bf16(num_seqs: int = 64) -> Workload:
    """Llama-3-8B layer shape decode: batch 64, ctx U[512,4096], 32 q / 8 kv heads, D 128, bf16."""
    rng = np.random.default_rng(SEED_BASE + 1)
    ctx = rng.integers(512, 4096, num_seqs, endpoint=True)
    return build("llama3_8b_decode_bf16", seed=SEED_BASE + 1, rng=rng, ctx_lens=ctx,
                 q_lens=[1] * num_seqs, num_q_heads=32, num_kv_heads=8, head_dim=128,
                 q_dtype="bf16", kv_dtype="bf16", max_blocks=256)


def llama3_8b_decode_fp8(num_seqs: int = 64) -> Workload:
    """The Llama-3-8B decode layer's batch with E4M3 pools (K scale 0.05, V scale 0.04) and bf16 queries."""
    rng = np.random.default_rng(SEED_BASE + 1)
    ctx = rng.integers(512, 4096, num_seqs, endpoint=True)
    return build("llama3_8b_decode_fp8", seed=SEED_BASE + 1, rng=rng, ctx_lens=ctx,
                 q_lens=[1] * num_seqs, num_q_heads=32, num_kv_heads=8, head_dim=128,
                 q_dtype="bf16", kv_dtype="fp8", max_blocks=256, k_scale=0.05, v_scale=0.04)


def mixed_step_bf16(num_decode: int = 48, chunk: int = 512, cached: Sequence[int] = (0, 1536),
                    kv_dtype: str = "bf16") -> Workload:
    """Mixed continuous-batching step: 48 decodes (ctx U[256,8192]) then two 512-token
    chunked-prefill chunks with 0 and 1536 cached tokens; 32 q / 8 kv heads, D 128, bf16
    (kv_dtype "fp8": the same step over E4M3 pools with scales K 0.05, V 0.04)."""
    rng = np.random.default_rng(SEED_BASE + 2)
    ctx_dec = rng.integers(256, 8192, num_decode, endpoint=True)
    ctx = list(ctx_dec) + [c + chunk for c in cached]
    ql = [1] * num_decode + [chunk] * len(cached)
    fp8 = kv_dtype == "fp8"
    return build("mixed_step_fp8" if fp8 else "mixed_step_bf16", seed=SEED_BASE + 2, rng=rng, ctx_lens=ctx,
                 q_lens=ql, num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16", kv_dtype=kv_dtype,
                 max_blocks=512, k_scale=0.05 if fp8 else 1.0, v_scale=0.04 if fp8 else 1.0)


def long_ctx_70b_decode_bf16(num_seqs: int = 8) -> Workload:
    """70B layer shape, long context: batch 8, ctx U[32768,131072], 64 q / 8 kv heads, D 128, bf16."""
    rng = np.random.default_rng(SEED_BASE + 3)
    ctx = rng.integers(32768, 131072, num_seqs, endpoint=True)
    return build("long_ctx_70b_decode_bf16", seed=SEED_BASE + 3, rng=rng, ctx_lens=ctx,
                 q_lens=[1] * num_seqs, num_q_heads=64, num_kv_heads=8, head_dim=128,
                 q_dtype="bf16", kv_dtype="bf16", max_blocks=8192, partition_size=512)


def prefix_shared_fp8_decode(num_seqs: int = 128) -> Workload:
    """128 requests sharing a 2048-token (128-block) prefix plus suffixes U[128,1024];
    fp8 E4M3 KV (K scale 0.05, V scale 0.04), bf16 Q, 32 q / 8 kv heads, D 128."""
    rng = np.random.default_rng(SEED_BASE + 4)
    suffix = rng.integers(128, 1024, num_seqs, endpoint=True)
    ctx = 2048 + suffix
    return build("prefix_shared_fp8_decode", seed=SEED_BASE + 4, rng=rng, ctx_lens=ctx,
                 q_lens=[1] * num_seqs, num_q_heads=32, num_kv_heads=8, head_dim=128,
                 q_dtype="bf16", kv_dtype="fp8", max_blocks=192, shared_prefix_tokens=2048,
                 k_scale=0.05, v_scale=0.04)


def long_prefill_bf16(num_seqs: int = 4, prompt: int = 4096) -> Workload:
    """Steady-state prefill: 4 prompts of 4096 tokens from empty caches (each a single chunk, causal), 32 q / 8
    kv heads, D 128, bf16 -- long enough that the kernel's fixed costs (launch, first tiles, tail) are small."""
    return build("long_prefill_bf16", seed=SEED_BASE + 5, ctx_lens=[prompt] * num_seqs, q_lens=[prompt] * num_seqs,
                 num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16", kv_dtype="bf16")


NAMED = {
    "tiny_fp32_decode": tiny_fp32_decode,
    "llama3_8b_decode_bf16": llama3_8b_decode_bf16,
    "llama3_8b_decode_fp8": llama3_8b_decode_fp8,
    "mixed_step_bf16": mixed_step_bf16,
    "long_ctx_70b_decode_bf16": long_ctx_70b_decode_bf16,
    "prefix_shared_fp8_decode": prefix_shared_fp8_decode,
    "long_prefill_bf16": long_prefill_bf16,
}


def random_case(seed: int, *, num_seqs: int, ctx_range=(1, 40), q_lens=None, num_q_heads=4,
                num_kv_heads=2, head_dim=8, q_dtype="f32", kv_dtype="f32", chunk_range=None,
                k_scale=1.0, v_scale=1.0, block_size=BLOCK_SIZE, extra_blocks=3,
                shared_prefix_tokens=0) -> Workload:
    """Small random case: context lengths U[ctx_range]; q_lens all 1 unless given,
    or drawn U[chunk_range] (capped by the context length) when chunk_range is set.
    shared_prefix_tokens (a multiple of the block size, below every context length):
    the sequences' tables begin with the same physical blocks."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ctx_range[0], ctx_range[1], num_seqs, endpoint=True)
    if q_lens is None:
        if chunk_range is None:
            q_lens = [1] * num_seqs
        else:
            q_lens = [int(min(c, rng.integers(chunk_range[0], chunk_range[1], endpoint=True))) for c in ctx]
    nblk = int(np.sum((ctx + block_size - 1) // block_size))
    return build(f"random_{seed}", seed=seed, rng=rng, ctx_lens=ctx, q_lens=q_lens,
                 num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                 q_dtype=q_dtype, kv_dtype=kv_dtype, num_blocks=nblk + extra_blocks,
                 k_scale=k_scale, v_scale=v_scale, block_size=block_size,
                 shared_prefix_tokens=shared_prefix_tokens)


# --- byte / flop accounting (sizes only; no attention arithmetic) ---------------

def decode_kv_bytes(w: Workload) -> int:
    """KV bytes one pass over the batch must read: every sequence reads its whole context, K and V."""
    return int(2 * np.sum(w.seq_lens.astype(np.int64)) * w.num_kv_heads * w.head_dim * w.kv_elem_bytes)


def decode_alg_bytes(w: Workload) -> int:
    """Algorithmic bytes of a decode pass: KV + Q + O + the block-table entries read + seq_lens."""
    B = w.block_size
    nblk = int(np.sum((w.seq_lens.astype(np.int64) + B - 1) // B))
    qo = 2 * w.num_tokens * w.num_q_heads * w.head_dim * w.q_elem_bytes
    return decode_kv_bytes(w) + qo + 4 * nblk + 4 * w.num_seqs


def decode_write_alg_bytes(w: Workload) -> int:
    """decode_alg_bytes plus the step's new K/V rows, read from the input and stored into the pools."""
    row = w.num_tokens * w.num_kv_heads * w.head_dim
    return decode_alg_bytes(w) + 2 * row * (w.q_elem_bytes + w.kv_elem_bytes)


def unique_kv_bytes(w: Workload) -> int:
    """KV bytes of distinct cached positions (shared prefix blocks counted once)."""
    B = w.block_size
    seen = set()
    n = 0
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        for j in range((L + B - 1) // B):
            blk = int(w.block_tables[s, j])
            if blk in seen:
                continue
            seen.add(blk)
            n += min(B, L - j * B)
    return int(2 * n * w.num_kv_heads * w.head_dim * w.kv_elem_bytes)


def visible_pairs(w: Workload, rows: Optional[np.ndarray] = None) -> int:
    """Number of (query row, key) pairs that causal attention sees."""
    total = 0
    ql = w.q_lens
    for s in range(w.num_seqs):
        c = int(w.seq_lens[s] - ql[s])
        q = int(ql[s])
        if q == 1:
            total += c + 1
        else:
            total += q * c + q * (q + 1) // 2
    return total


def prefill_flops(w: Workload, only_chunks: bool = True, window: int = 0) -> int:
    """4 * Hq * D flops per visible (row, key) pair (QK^T and PV, multiply+add each); with a sliding window the
    row at position p sees min(p + 1, window) keys."""
    ql = w.q_lens
    pairs = 0
    for s in range(w.num_seqs):
        q = int(ql[s])
        if only_chunks and q == 1:
            continue
        c = int(w.seq_lens[s] - q)
        if window > 0:
            pos = np.arange(c, c + q, dtype=np.int64)
            pairs += int(np.minimum(pos + 1, window).sum())
        else:
            pairs += q * c + q * (q + 1) // 2
    return 4 * w.num_q_heads * w.head_dim * pairs


def decode_window_kv_bytes(w: Workload, window: int) -> int:
    """K+V bytes of the keys a windowed decode row sees: min(seq_len, window) per sequence."""
    toks = np.minimum(w.seq_lens.astype(np.int64), window)
    return int(2 * toks.sum() * w.num_kv_heads * w.head_dim * w.kv_elem_bytes)
