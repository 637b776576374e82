"""Plain model of the KV block manager (TEST INFRASTRUCTURE ONLY: see the
package docstring; nothing on the product path uses it).

What it follows ("vLLM 学习笔记 01"): section 1.5 -- blocks of 16 tokens,
one block table per request, a request takes one more block when it grows
and returns all of them when it ends, free blocks wait in a queue; section
1.4 -- the scheduler asks for slots and has to preempt when blocks run out;
section 2.2 -- prefix caching: a full block is identified by everything
before it and its own tokens (the pages key it by a hash chain; this model
keys it by the whole token prefix itself, which is what the hash chain
stands for), a new request reuses the longest cached run of full blocks from
its start, a released block keeps its content and key until it is taken for
new content, blocks are reference counted, partly filled blocks are never
cached.

Where the pages leave the choice open, this model takes the readings that
the C ABI header states (they are restated here so the model reads on its
own):

* new blocks are taken from the front of the free queue; released blocks
  are appended at its back, a request's blocks from its last block to its
  first;
* a request matches cached blocks only at its first allocation, and at most
  (known tokens - 1) // 16 of them, so at least one token is computed;
* a block is registered when an allocation makes it full; if the same key is
  already registered (to another block), the block stays unregistered;
* a request carries a salt that is part of every one of its keys (the pages'
  extra keys, e.g. an adapter id).

Everything is a Python list or dict, scanned plainly: the free queue is a
list (removal from the middle is ``list.remove``), so operations are O(n),
not O(1) -- this model is for checking, not for speed.

Parity status: pinned by ``tests/test_oracle_block_manager.py`` (the pages'
prefix-caching scenario and smaller cases worked by hand, invariants under
random operation sequences, and a brute-force longest-prefix check);
``tests/test_oracle_bm_mutations.py`` checks that planted mistakes in a copy
of this model fail those pins.
"""

BLOCK = 16


class BlockManagerModel:
    def __init__(self, num_blocks, prefix_caching=True):
        self.caching = bool(prefix_caching)
        self.free = list(range(num_blocks))      # front = next block handed out
        self.ref = [0] * num_blocks
        self.key = [None] * num_blocks           # the cache key a block is registered under
        self.cache = {}                          # key -> block id
        self.reqs = {}                           # id -> dict(tokens, table, computed, salt)

    # -- keys ---------------------------------------------------------------
    @staticmethod
    def _key(salt, tokens, b):
        """Key of full block b of a request: its salt and all tokens up to the
        end of block b."""
        return (salt, tuple(tokens[:(b + 1) * BLOCK]))

    def _match(self, r):
        """Block ids of the longest cached run of full blocks from the start."""
        if not self.caching:
            return []
        ids = []
        for b in range((len(r["tokens"]) - 1) // BLOCK):
            k = self._key(r["salt"], r["tokens"], b)
            if k not in self.cache:
                break
            ids.append(self.cache[k])
        return ids

    # -- requests -----------------------------------------------------------
    def add_request(self, req, tokens, salt=0):
        if req in self.reqs or len(tokens) < 1:
            raise ValueError("duplicate request or no tokens")
        self.reqs[req] = {"tokens": list(tokens), "table": [], "computed": 0, "salt": salt,
                          "registered": 0}

    def append_tokens(self, req, tokens):
        self.reqs[req]["tokens"].extend(tokens)

    def num_cached_tokens(self, req):
        r = self.reqs[req]
        if not r["table"] and r["computed"] == 0:
            return len(self._match(r)) * BLOCK
        return r["computed"]

    def allocate_slots(self, req, num_new):
        """Slots of the request's next num_new tokens, or None (nothing
        changed) when the free queue is too short."""
        r = self.reqs[req]
        first = not r["table"] and r["computed"] == 0
        hits = self._match(r) if first else []
        computed = len(hits) * BLOCK if first else r["computed"]
        end = computed + num_new
        if num_new < 0 or end > len(r["tokens"]):
            raise ValueError("allocation past the known tokens")
        blocks_needed = -(-end // BLOCK)
        need = max(0, blocks_needed - (len(r["table"]) + len(hits)))
        available = len(self.free) - sum(1 for b in hits if b in self.free)
        if need > available:
            return None
        for b in hits:
            if b in self.free:
                self.free.remove(b)
            self.ref[b] += 1
            r["table"].append(b)
        if first:
            r["computed"] = computed
            r["registered"] = len(hits)
        for _ in range(need):
            b = self.free.pop(0)
            if self.key[b] is not None:
                if self.cache.get(self.key[b]) == b:
                    del self.cache[self.key[b]]
                self.key[b] = None
            self.ref[b] = 1
            r["table"].append(b)
        slots = [r["table"][p // BLOCK] * BLOCK + p % BLOCK for p in range(computed, end)]
        r["computed"] = end
        if self.caching:
            while (r["registered"] + 1) * BLOCK <= r["computed"]:
                b = r["registered"]
                k = self._key(r["salt"], r["tokens"], b)
                blk = r["table"][b]
                if self.key[blk] is None and k not in self.cache:
                    self.cache[k] = blk
                    self.key[blk] = k
                r["registered"] += 1
        return slots

    def free_request(self, req):
        r = self.reqs.pop(req)
        for b in reversed(r["table"]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    def block_table(self, req):
        return list(self.reqs[req]["table"])

    def step_metadata(self, reqs, num_new, width):
        """block_tables [S, width] (-1 padded), cu_seqlens_q, seq_lens and
        slot_mapping of one step, in packing order."""
        tables, cu, lens, slots = [], [0], [], []
        for req, n in zip(reqs, num_new):
            r = self.reqs[req]
            L = r["computed"]
            if n < 0 or n > L or len(r["table"]) > width:
                raise ValueError("bad step")
            tables.append(r["table"] + [-1] * (width - len(r["table"])))
            cu.append(cu[-1] + n)
            lens.append(L)
            slots += [r["table"][p // BLOCK] * BLOCK + p % BLOCK for p in range(L - n, L)]
        return tables, cu, lens, slots

    def num_free_blocks(self):
        return len(self.free)

    def num_cached_blocks(self):
        return len(self.cache)
