"""Pure-Python brute-force paged attention for tiny inputs (TEST INFRASTRUCTURE ONLY).

An independent second evaluation of the same definition as the C oracle:
plain nested loops over Python floats, exact sums by math.fsum, its own
bf16 and fp8 decoding, and its own block-table addressing.  Used only to pin
the C oracle on tiny cases.

Definition (page "vLLM 架构概述" §2: per-request block table into a pool of
physical blocks; page "vLLM：从 KV Cache 到高吞吐推理服务", tutorial 3: logical
block, offset, physical block; reading note on "Inside vLLM", core point 2:
flattened batch, each sequence sees only its own tokens):

    for new row i of sequence s with c = seq_len - q_len cached tokens:
        keys 0 .. c + i of s; key j at pool[table[s][j // B]][j % B][h // G]
        out = sum_j softmax_j(scale * q . k_j) v_j
"""
from __future__ import annotations

import math
import struct
from typing import List

from . import fp8_ref


def _bf16_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def _value(flat, idx: int, kind: str, scale: float) -> float:
    raw = flat[idx]
    if kind == "f32":
        return float(raw)
    if kind == "bf16":
        return _bf16_to_float(int(raw))
    return fp8_ref.decode(int(raw)) * scale


def attention(query, q_kind, k_cache, v_cache, kv_kind, block_tables, seq_lens, query_start_loc,
              num_q_heads, num_kv_heads, head_dim, block_size, scale, k_scale=1.0, v_scale=1.0,
              window=0, chunk=0) -> List:
    """Inputs are flat Python lists (bf16 as uint16 bit patterns, fp8 as codes).
    window > 0: the row at position p sees only the keys p - window + 1 .. p (those >= 0).
    chunk > 0: the row at position p sees only the keys of its own chunk of positions,
    [chunk * (p // chunk), p].

    Returns out[t][h][d] as nested lists of floats."""
    G = num_q_heads // num_kv_heads
    S = len(seq_lens)
    out = []
    for s in range(S):
        q0, q1 = query_start_loc[s], query_start_loc[s + 1]
        cached = seq_lens[s] - (q1 - q0)
        for t in range(q0, q1):
            pos = cached + (t - q0)
            row = []
            for h in range(num_q_heads):
                kvh = h // G
                q = [_value(query, (t * num_q_heads + h) * head_dim + d, q_kind, 1.0) for d in range(head_dim)]
                keys = []
                for j in range(pos + 1):
                    if window and j <= pos - window:
                        continue
                    if chunk and j // chunk != pos // chunk:
                        continue
                    blk = block_tables[s][j // block_size]
                    base = ((blk * block_size + j % block_size) * num_kv_heads + kvh) * head_dim
                    keys.append(base)
                z = []
                for base in keys:
                    prods = [q[d] * _value(k_cache, base + d, kv_kind, k_scale) for d in range(head_dim)]
                    z.append(scale * math.fsum(prods))
                m = max(z)
                w = [math.exp(x - m) for x in z]
                l = math.fsum(w)
                o = []
                for d in range(head_dim):
                    o.append(math.fsum(w[j] * _value(v_cache, keys[j] + d, kv_kind, v_scale)
                                       for j in range(len(keys))) / l)
                row.append(o)
            out.append(row)
    return out


def from_workload(w, pools, window=0, chunk=0):
    """Runs attention() on a workload's tensors (converted to flat lists)."""
    import torch

    def flat(x):
        x = x.contiguous()
        if x.dtype == torch.bfloat16:
            return [int(v) & 0xFFFF for v in x.view(torch.int16).reshape(-1).tolist()]
        return x.reshape(-1).tolist()

    kc, vc = pools
    return attention(flat(w.query), w.q_dtype, flat(kc), flat(vc), w.kv_dtype,
                     [list(map(int, r)) for r in w.block_tables], [int(v) for v in w.seq_lens],
                     [int(v) for v in w.query_start_loc], w.num_q_heads, w.num_kv_heads, w.head_dim,
                     w.block_size, float(w.scale), float(w.k_scale), float(w.v_scale), window=window,
                     chunk=chunk)
