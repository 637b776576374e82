"""Pins of the block-manager model (oracle/block_manager.py) against what the
pages fix ("vLLM 学习笔记 01", sections 1.4, 1.5, 2.2) and the readings
stated there: a prefix-caching scenario worked by hand, invariants that must
hold after every operation, and a brute-force longest-prefix search that
does not go through the model's cache dictionary."""

import numpy as np
import pytest

from oracle.block_manager import BLOCK, BlockManagerModel


def _slots(blocks_and_rows):
    return [b * BLOCK + r for b, r in blocks_and_rows]


def test_pages_scenario_by_hand():
    # 8 blocks; a 32-token system prompt shared by several requests
    m = BlockManagerModel(8)
    sys_prompt = list(range(1000, 1032))
    a = sys_prompt + list(range(8))                 # 40 tokens: 2 full blocks + 8
    m.add_request("A", a)
    assert m.num_cached_tokens("A") == 0
    assert m.allocate_slots("A", 40) == list(range(40))        # blocks 0, 1, 2 from the front
    assert m.block_table("A") == [0, 1, 2]
    assert m.num_cached_blocks() == 2                           # the partial block 2 is not cached
    assert m.free == [3, 4, 5, 6, 7]

    b = sys_prompt + [7, 7, 7, 7, 7]                            # 37 tokens
    m.add_request("B", b)
    assert m.num_cached_tokens("B") == 32                       # both prompt blocks hit
    assert m.allocate_slots("B", 5) == _slots([(3, r) for r in range(5)])
    assert m.block_table("B") == [0, 1, 3]
    assert m.ref[0] == m.ref[1] == 2 and m.ref[2] == m.ref[3] == 1

    m.free_request("A")                                         # last block first
    assert m.free == [4, 5, 6, 7, 2] and m.ref[0] == m.ref[1] == 1
    m.free_request("B")
    assert m.free == [4, 5, 6, 7, 2, 3, 1, 0]
    assert m.num_cached_blocks() == 2                           # content and keys kept

    c = sys_prompt + [9]                                        # 33 tokens
    m.add_request("C", c)
    assert m.num_cached_tokens("C") == 32
    assert m.allocate_slots("C", 1) == [4 * BLOCK]              # cached blocks leave the queue
    assert m.block_table("C") == [0, 1, 4] and m.free == [5, 6, 7, 2, 3]

    d = list(range(5000, 5080))                                 # 80 unique tokens: 5 blocks
    m.add_request("D", d)
    assert m.allocate_slots("D", 80) is not None
    assert m.block_table("D") == [5, 6, 7, 2, 3] and m.free == []
    assert m.num_cached_blocks() == 7

    e = list(range(6000, 6040))
    m.add_request("E", e)
    assert m.allocate_slots("E", 40) is None                    # no block left: nothing changes
    assert m.reqs["E"]["table"] == [] and m.free == []

    m.free_request("C")
    assert m.free == [4, 1, 0]
    assert m.allocate_slots("E", 40) is not None                # takes 4, 1, 0: evicts the prompt
    assert m.block_table("E") == [4, 1, 0]
    m.add_request("F", sys_prompt + [1])
    assert m.num_cached_tokens("F") == 0                        # the shared prompt is gone


def test_at_least_one_token_is_computed():
    m = BlockManagerModel(8)
    prompt = list(range(32))
    m.add_request(1, prompt)
    m.allocate_slots(1, 32)
    m.add_request(2, prompt)                       # the whole prompt is cached ...
    assert m.num_cached_tokens(2) == 16            # ... but its last block is recomputed
    assert m.allocate_slots(2, 16) == _slots([(2, r) for r in range(16)])


def test_salt_separates_keys():
    m = BlockManagerModel(8)
    prompt = list(range(40))
    m.add_request(1, prompt, salt=0)
    m.allocate_slots(1, 40)
    m.add_request(2, prompt, salt=5)
    assert m.num_cached_tokens(2) == 0
    m.add_request(3, prompt, salt=0)
    assert m.num_cached_tokens(3) == 32


def test_decode_growth_takes_one_block_per_16_tokens():
    m = BlockManagerModel(4, prefix_caching=False)
    m.add_request(1, list(range(15)))
    m.allocate_slots(1, 15)
    assert m.block_table(1) == [0]
    m.append_tokens(1, [99])
    assert m.allocate_slots(1, 1) == [15]
    assert m.block_table(1) == [0]
    m.append_tokens(1, [98])
    assert m.allocate_slots(1, 1) == [1 * BLOCK]   # token 16 opens the second block
    assert m.block_table(1) == [0, 1] and m.num_cached_blocks() == 0


def _check_invariants(m):
    nb = len(m.ref)
    assert len(set(m.free)) == len(m.free)
    for b in range(nb):
        held = sum(r["table"].count(b) for r in m.reqs.values())
        assert m.ref[b] == held, f"block {b}: ref {m.ref[b]} vs held {held}"
        assert (b in m.free) == (held == 0)
    for r in m.reqs.values():
        assert len(r["table"]) == -(-r["computed"] // BLOCK)
        assert len(set(r["table"])) == len(r["table"])
    for k, b in m.cache.items():
        assert m.key[b] == k
    for b in range(nb):
        if m.key[b] is not None:
            assert m.cache.get(m.key[b]) == b


def _brute_cached_tokens(m, salt, tokens):
    """Longest run of full blocks from the start whose content (salt and the
    whole token prefix) some registered block holds: found by scanning every
    block's key, not through the cache dictionary."""
    held = {m.key[b] for b in range(len(m.ref)) if m.key[b] is not None}
    nb = 0
    while nb < (len(tokens) - 1) // BLOCK and (salt, tuple(tokens[:(nb + 1) * BLOCK])) in held:
        nb += 1
    return nb * BLOCK


@pytest.mark.parametrize("seed", range(6))
def test_invariants_under_random_operations(seed):
    rng = np.random.default_rng([469, 60, seed])
    m = BlockManagerModel(int(rng.integers(12, 40)))
    prompts = [list(rng.integers(0, 50, size=int(rng.integers(16, 70)))) for _ in range(4)]
    live, next_id = [], 0
    for _ in range(300):
        op = rng.integers(0, 4)
        if op == 0 or not live:
            base = prompts[int(rng.integers(0, len(prompts)))]
            cut = int(rng.integers(1, len(base) + 1))
            toks = base[:cut] + list(rng.integers(0, 50, size=int(rng.integers(0, 20))))
            salt = int(rng.integers(0, 2))
            m.add_request(next_id, toks, salt=salt)
            assert m.num_cached_tokens(next_id) == _brute_cached_tokens(m, salt, toks)
            live.append(next_id)
            next_id += 1
        elif op == 1:
            req = live[int(rng.integers(0, len(live)))]
            r = m.reqs[req]
            if r["computed"] == len(r["tokens"]):
                m.append_tokens(req, [int(rng.integers(0, 50))])
            left = len(r["tokens"]) - m.num_cached_tokens(req)
            n = int(rng.integers(1, left + 1))
            before = (list(m.free), [list(x["table"]) for x in m.reqs.values()])
            slots = m.allocate_slots(req, n)
            if slots is None:
                assert before == (list(m.free), [list(x["table"]) for x in m.reqs.values()])
            else:
                t, c = r["table"], r["computed"]
                assert slots == [t[p // BLOCK] * BLOCK + p % BLOCK for p in range(c - n, c)]
        else:
            req = live.pop(int(rng.integers(0, len(live))))
            m.free_request(req)
        _check_invariants(m)


def test_step_metadata_by_hand():
    # one table per request, -1 padded; the new tokens are each request's
    # last n positions, packed in the order given (section 1.5)
    m = BlockManagerModel(6, prefix_caching=False)
    m.add_request(1, list(range(20)))
    m.add_request(2, list(range(5)))
    assert m.allocate_slots(1, 20) == list(range(20))          # blocks 0, 1
    assert m.allocate_slots(2, 3) == _slots([(2, 0), (2, 1), (2, 2)])   # a chunk of 3
    tables, cu, lens, slots = m.step_metadata([1, 2], [20, 3], 3)
    assert tables == [[0, 1, -1], [2, -1, -1]]
    assert cu == [0, 20, 23] and lens == [20, 3]
    assert slots == list(range(20)) + _slots([(2, 0), (2, 1), (2, 2)])
    m.append_tokens(1, [7])
    assert m.allocate_slots(1, 1) == _slots([(1, 4)])          # position 20
    assert m.allocate_slots(2, 2) == _slots([(2, 3), (2, 4)])
    tables, cu, lens, slots = m.step_metadata([2, 1], [2, 1], 3)
    assert tables == [[2, -1, -1], [0, 1, -1]]
    assert cu == [0, 2, 3] and lens == [5, 21]
    assert slots == _slots([(2, 3), (2, 4), (1, 4)])
    with pytest.raises(ValueError):
        m.step_metadata([2], [6], 3)                            # more new tokens than L
    with pytest.raises(ValueError):
        m.step_metadata([1], [1], 1)                            # table wider than the row


def test_cached_hits_in_the_free_queue_are_not_free():
    # a released, still-cached block that a request hits leaves the free
    # queue, so it cannot also be handed out as a new block (section 1.4:
    # the scheduler must preempt when blocks run out)
    m = BlockManagerModel(3)
    prompt = list(range(33))
    m.add_request(1, prompt)
    m.allocate_slots(1, 33)                        # blocks 0, 1 cached, 2 partial
    m.free_request(1)
    assert m.free == [2, 1, 0] and m.num_cached_blocks() == 2
    m.add_request(2, prompt[:32] + list(range(100, 117)))   # 49 tokens: 4 blocks
    assert m.num_cached_tokens(2) == 32
    assert m.allocate_slots(2, 17) is None         # 2 hits + 2 new > 3 blocks
    assert m.free == [2, 1, 0] and m.block_table(2) == []
    m.add_request(3, prompt[:32] + [5])
    assert m.allocate_slots(3, 1) == [2 * BLOCK]   # 2 hits + 1 new fits exactly
    assert m.free == []


def test_concurrent_prompts_match_once_and_register_once():
    # two requests with the same prompt, chunked side by side: the second
    # matched nothing at its first allocation and matches nothing later, and
    # a block filled with content already registered to another block stays
    # unregistered
    m = BlockManagerModel(8)
    prompt = list(range(40))
    m.add_request(1, prompt)
    m.add_request(2, prompt)
    assert m.allocate_slots(1, 10) == list(range(10))                  # block 0, partial
    assert m.allocate_slots(2, 16) == _slots([(1, r) for r in range(16)])
    assert m.key[1] is not None                                         # block 1 registered first
    assert m.allocate_slots(1, 30) == list(range(10, 16)) + list(range(32, 56))
    assert m.block_table(1) == [0, 2, 3]
    assert m.key[0] is None and m.num_cached_blocks() == 2              # same content as block 1
    assert m.num_cached_tokens(2) == 16                                 # no late matching
    assert m.allocate_slots(2, 24) == _slots([(4, r) for r in range(16)] + [(5, r) for r in range(8)])
    assert m.block_table(2) == [1, 4, 5]
    assert m.key[4] is None and m.num_cached_blocks() == 2
    m.add_request(3, prompt)
    assert m.num_cached_tokens(3) == 32 and m._match(m.reqs[3]) == [1, 2]
