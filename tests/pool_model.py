"""A plain Python model of the host block pool, written from the pages' description
(lists and dicts, O(n) operations, no cleverness), that the C pool is checked against.

"vLLM 架构概述" §5.1: a free list of blocks, a map from block hash to cached blocks,
a reference count and a hash per block.  Reading note on "Inside vLLM", core point 1:
allocate_slots takes ceil(tokens / block_size) blocks from the head of the free list
after checking that enough are free.  Block 0 is the null block; freed blocks go to
the tail with their hash (still hittable) and are evicted when handed out again; a
request's blocks are released from its last to its first.
"""


class NoSpace(Exception):
    pass


class BadState(Exception):
    pass


class PoolModel:
    def __init__(self, num_blocks: int, block_size: int):
        self.bs = block_size
        self.free = list(range(1, num_blocks))  # head first
        self.ref = [0] * num_blocks
        self.hash = [None] * num_blocks
        self.cached = {}  # hash -> [blocks], oldest copy first
        self.req = {}     # request id -> [blocks, number of leading blocks already cached]

    def _evict(self, b):
        h = self.hash[b]
        if h is None:
            return
        self.cached[h].remove(b)
        if not self.cached[h]:
            del self.cached[h]
        self.hash[b] = None

    def _release(self, b):
        if b == 0:
            return
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    def find_longest_cache_hit(self, hashes):
        out = []
        for h in hashes:
            if h not in self.cached:
                break
            out.append(self.cached[h][0])
        return out

    def allocate_slots(self, rid, num_tokens, hits=()):
        hits = list(hits)
        known = rid in self.req
        if known and hits:
            raise BadState
        have = len(self.req[rid][0]) if known else 0
        want = -(-num_tokens // self.bs)
        fresh = max(0, want - have - len(hits))
        hits_free = sum(1 for b in hits if b in self.free)
        if fresh + hits_free > len(self.free):
            raise NoSpace
        blocks, ncached = self.req.get(rid, [[], 0])
        for b in hits:
            if b in self.free:
                self.free.remove(b)
            self.ref[b] += 1
            blocks.append(b)
        if not known:
            ncached = len(hits)
        for _ in range(fresh):
            b = self.free.pop(0)
            self._evict(b)
            self.ref[b] = 1
            blocks.append(b)
        self.req[rid] = [blocks, ncached]
        return len(blocks)

    def cache_blocks(self, rid, hashes, num_full):
        if rid not in self.req:
            raise BadState
        blocks, ncached = self.req[rid]
        for i in range(ncached, num_full):
            b = blocks[i]
            if b == 0 or self.hash[b] is not None:
                continue
            self.hash[b] = int(hashes[i])
            self.cached.setdefault(int(hashes[i]), []).append(b)
        self.req[rid][1] = max(ncached, num_full)

    def release_before(self, rid, position):
        if rid not in self.req:
            raise BadState
        blocks = self.req[rid][0]
        for j in range(min(max(position, 0) // self.bs, len(blocks))):
            self._release(blocks[j])
            blocks[j] = 0

    def free_request(self, rid):
        if rid not in self.req:
            raise BadState
        for b in reversed(self.req[rid][0]):
            self._release(b)
        del self.req[rid]
