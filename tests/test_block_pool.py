"""The host block pool (pa_pool_*): the pages' worked numbers, the chained block hash, and random operation
sequences checked step by step against the plain Python model in pool_model.py.  Host code only (no GPU)."""
import numpy as np
import pytest

import paged_kv_cache_418_amd as pk
from paged_kv_cache_418_amd import _binding as b
from pool_model import BadState, NoSpace, PoolModel


def _fnv1a64(data: bytes) -> int:
    """FNV-1a, 64 bits, from its published definition (offset basis and prime of Fowler, Noll and Vo)."""
    h = 0xCBF29CE484222325
    for c in data:
        h = ((h ^ c) * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def test_fnv1a64_published_vectors():
    # test vectors published with the FNV definition
    assert _fnv1a64(b"") == 0xCBF29CE484222325
    assert _fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert _fnv1a64(b"foobar") == 0x85944171F73967E8


def _chain(tokens, bs, extra):
    out, parent = [], 0
    for i in range(len(tokens) // bs):
        data = parent.to_bytes(8, "little")
        data += b"".join(int(t).to_bytes(4, "little", signed=True) for t in tokens[i * bs:(i + 1) * bs])
        data += extra.to_bytes(8, "little")
        parent = _fnv1a64(data)
        out.append(parent)
    return out


def test_hash_chain():
    rng = np.random.default_rng(1)
    toks = rng.integers(-5, 50000, 70).astype(np.int32)
    h = pk.pool_hash_blocks(toks, 16, 7)
    assert len(h) == 4  # 70 tokens: 4 full blocks, the partial fifth has no hash
    assert [int(x) for x in h] == _chain(toks, 16, 7)
    # a block's hash depends on every token before it, and on nothing after
    t2 = toks.copy()
    t2[40] += 1
    h2 = pk.pool_hash_blocks(t2, 16, 7)
    assert list(h2[:2]) == list(h[:2]) and all(h2[i] != h[i] for i in (2, 3))
    t3 = toks.copy()
    t3[69] += 1
    assert list(pk.pool_hash_blocks(t3, 16, 7)) == list(h)
    # the extra identity (salt, adapter, ...) changes every hash
    assert all(x != y for x, y in zip(pk.pool_hash_blocks(toks, 16, 8), h))
    assert len(pk.pool_hash_blocks(toks[:15], 16, 0)) == 0


def test_allocate_slots_worked_example():
    """17 new tokens of 16-token blocks take ceil(17/16) = 2 blocks from the head of the free list."""
    p = pk.BlockPool(10, 16)
    assert p.num_free == 9 and p.free_queue() == list(range(1, 10))  # block 0 is the null block
    assert p.allocate_slots(1, 17) == 2
    assert p.block_table(1) == [1, 2] and p.num_free == 7
    assert p.allocate_slots(1, 32) == 2      # still fits in 2 blocks
    assert p.allocate_slots(1, 33) == 3      # one more token, one more block
    assert p.block_table(1) == [1, 2, 3]
    assert p.block_state(1) == (1, False, None)


def test_prefix_sharing_tables_A_and_B():
    """A's table [B0, B3, B7] and B's [B0, B3, B1, B5, B8]: B's first two blocks are A's, found by hash, ref 2."""
    p = pk.BlockPool(16, 16)
    rng = np.random.default_rng(2)
    prompt_a = rng.integers(0, 1000, 48).astype(np.int32)
    prompt_b = np.concatenate([prompt_a[:32], rng.integers(1000, 2000, 48).astype(np.int32)])
    ha = pk.pool_hash_blocks(prompt_a)
    assert p.find_longest_cache_hit(ha) == []
    p.allocate_slots(10, len(prompt_a))
    p.cache_blocks(10, ha, 3)
    hb = pk.pool_hash_blocks(prompt_b)
    hits = p.find_longest_cache_hit(hb)
    ta = p.block_table(10)
    assert hits == ta[:2]
    p.allocate_slots(11, len(prompt_b), hits)
    tb = p.block_table(11)
    assert tb[:2] == ta[:2] and len(tb) == 5 and not set(tb[2:]) & set(ta)
    assert [p.block_state(x)[0] for x in ta] == [2, 2, 1]
    # A finishes: its private block returns to the free list (cached), the shared ones stay held by B
    p.free(10)
    assert p.block_state(ta[2]) == (0, True, int(ha[2]))
    assert [p.block_state(x)[0] for x in ta[:2]] == [1, 1]
    # a third request with A's prompt hits all three blocks; the freed one leaves the free list again
    free_before = p.num_free
    p.allocate_slots(12, 48, p.find_longest_cache_hit(ha))
    assert p.block_table(12) == ta and p.num_free == free_before - 1
    assert p.block_state(ta[2]) == (1, False, int(ha[2]))


def test_eviction_and_physical_copies():
    p = pk.BlockPool(5, 4)  # 4 usable blocks of 4 tokens
    t = np.arange(8, dtype=np.int32)
    h = pk.pool_hash_blocks(t, 4)
    # two requests compute the same prefix without a hit: two physical copies of each hash
    p.allocate_slots(1, 8)
    p.allocate_slots(2, 8)
    p.cache_blocks(1, h, 2)
    p.cache_blocks(2, h, 2)
    t1, t2 = p.block_table(1), p.block_table(2)
    assert p.find_longest_cache_hit(h) == t1  # the oldest copy
    p.free(1)
    p.free(2)
    # released last block first: the free list holds 1's blocks reversed, then 2's
    assert p.free_queue() == [t1[1], t1[0], t2[1], t2[0]]
    # handing out the head evicts its hash; the other copy still serves hits
    p.allocate_slots(3, 4)
    assert p.block_table(3) == [t1[1]] and p.block_state(t1[1])[2] is None
    assert p.find_longest_cache_hit(h) == [t1[0], t2[1]]
    # every block handed out: the pool is full and refuses without changing anything
    p.allocate_slots(4, 12)
    assert p.num_free == 0
    with pytest.raises(b.PAError) as e:
        p.allocate_slots(5, 1)
    assert e.value.status == 7  # PA_ERR_NO_SPACE


def test_errors_leave_the_pool_unchanged():
    p = pk.BlockPool(6, 16)
    p.allocate_slots(1, 40)
    q, t = p.free_queue(), p.block_table(1)
    with pytest.raises(b.PAError):
        p.allocate_slots(2, 16 * 5)            # 5 blocks wanted, 2 free
    with pytest.raises(b.PAError):
        p.allocate_slots(1, 50, [t[0]])        # hits only on a request's first allocation
    with pytest.raises(b.PAError):
        p.allocate_slots(3, 40, [4])           # not a cached block
    with pytest.raises(b.PAError):
        p.free(99)
    with pytest.raises(b.PAError):
        p.cache_blocks(1, np.zeros(4, np.uint64), 4)  # more full blocks than the request holds
    assert p.free_queue() == q and p.block_table(1) == t
    with pytest.raises(b.PAError):
        pk.BlockPool(1, 16)


def test_sliding_window_release():
    p = pk.BlockPool(12, 16)
    p.allocate_slots(1, 100)                   # 7 blocks
    t = p.block_table(1)
    # window 40 and a next row at position 100: keys from 61 on are kept, blocks 0..2 (positions < 48) go
    p.release_before(1, 100 - 40 + 1)
    assert p.block_table(1) == [0, 0, 0] + t[3:]
    assert p.free_queue()[-3:] == t[:3]
    p.release_before(1, 100 - 40 + 1)          # idempotent
    p.free(1)
    assert p.num_free == 11


@pytest.mark.parametrize("seed", [11, 12, 13, 14])
def test_random_operations_match_the_model(seed):
    rng = np.random.default_rng(seed)
    nb, bs = int(rng.integers(20, 60)), int(rng.choice([4, 16]))
    pool, model = pk.BlockPool(nb, bs), PoolModel(nb, bs)
    prompts = [rng.integers(0, 50, int(rng.integers(1, 6 * bs))).astype(np.int32) for _ in range(4)]
    live = {}  # request id -> its tokens
    next_id = 0
    for step in range(600):
        op = rng.random()
        if op < 0.35 or not live:  # a new request: a stored prompt, maybe extended
            base = prompts[int(rng.integers(len(prompts)))]
            toks = np.concatenate([base, rng.integers(0, 50, int(rng.integers(0, 2 * bs))).astype(np.int32)])
            hashes = pk.pool_hash_blocks(toks, bs)
            hits = pool.find_longest_cache_hit(hashes)
            assert hits == model.find_longest_cache_hit([int(h) for h in hashes])
            if len(hits) * bs >= len(toks):  # keep at least one token to compute
                hits = hits[:max(0, (len(toks) - 1) // bs)]
            rid, next_id = next_id, next_id + 1
            try:
                model.allocate_slots(rid, len(toks), hits)
                ok = True
            except NoSpace:
                ok = False
            if ok:
                pool.allocate_slots(rid, len(toks), hits)
                pool.cache_blocks(rid, hashes, len(hashes))
                model.cache_blocks(rid, hashes, len(hashes))
                live[rid] = toks
            else:
                with pytest.raises(b.PAError):
                    pool.allocate_slots(rid, len(toks), hits)
        elif op < 0.7:  # decode steps: a running request grows
            rid = list(live)[int(rng.integers(len(live)))]
            toks = np.concatenate([live[rid], rng.integers(0, 50, int(rng.integers(1, bs + 2))).astype(np.int32)])
            try:
                model.allocate_slots(rid, len(toks))
                ok = True
            except NoSpace:
                ok = False
            if ok:
                pool.allocate_slots(rid, len(toks))
                hashes = pk.pool_hash_blocks(toks, bs)
                pool.cache_blocks(rid, hashes, len(hashes))
                model.cache_blocks(rid, hashes, len(hashes))
                live[rid] = toks
            else:
                with pytest.raises(b.PAError):
                    pool.allocate_slots(rid, len(toks))
        elif op < 0.8:  # sliding window
            rid = list(live)[int(rng.integers(len(live)))]
            pos = len(live[rid]) - int(rng.integers(1, 3 * bs))
            pool.release_before(rid, pos)
            model.release_before(rid, pos)
        else:
            rid = list(live)[int(rng.integers(len(live)))]
            pool.free(rid)
            model.free_request(rid)
            del live[rid]
        assert pool.free_queue() == model.free, step
        for rid in live:
            assert pool.block_table(rid) == model.req[rid][0]
        if step % 50 == 0:
            for blk in range(1, nb):
                ref, is_free, h = pool.block_state(blk)
                assert ref == model.ref[blk] and is_free == (blk in model.free) and h == model.hash[blk]
    for rid in list(live):
        pool.free(rid)
    assert pool.num_free == nb - 1


def test_model_refuses_like_the_pool():
    m = PoolModel(3, 16)
    m.allocate_slots(1, 20)
    with pytest.raises(NoSpace):
        m.allocate_slots(2, 1)
    with pytest.raises(BadState):
        m.free_request(7)
