"""Pins for the oracle's pool layout and KV write.

* Block bytes: the page's closed form (golden fixture with hand-multiplied
  values).
* Write: read back through an independent route (the pool viewed as a flat
  array of token slots, slot = block*16 + position), -1 skips, untouched
  memory keeps its poison, caller errors raise.
"""

import os

import numpy as np
import pytest

from oracle import paged

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_block_bytes_golden():
    rows = _fixture_rows("block_bytes.txt")
    assert rows
    for r in rows:
        bs, hkv, d, db, want = (int(x) for x in r[:5])
        assert paged.block_bytes(bs, hkv, d, db) == want


def test_block_bytes_is_pool_stride():
    pool = np.zeros((3, 2, 16, 8, 128), dtype=np.uint16)
    assert pool.strides[0] == paged.block_bytes(16, 8, 128, 2)


def _slot_view(pool):
    """The pool as [NB*16] K slots and [NB*16] V slots (independent route)."""
    nb, _, bs, hkv, d = pool.shape
    return (pool[:, 0].reshape(nb * bs, hkv, d), pool[:, 1].reshape(nb * bs, hkv, d))


def test_write_round_trip_and_poison():
    rng = np.random.default_rng(1)
    nb, hkv, d, t = 12, 2, 8, 70
    pool = np.full((nb, 2, 16, hkv, d), 0x7FC1, dtype=np.uint16)
    slots = rng.choice(nb * 16, size=t, replace=False).astype(np.int32)
    slots[[3, 17, 40]] = -1
    k = rng.integers(0, 1 << 16, (t, hkv, d)).astype(np.uint16)
    v = rng.integers(0, 1 << 16, (t, hkv, d)).astype(np.uint16)
    paged.kv_write(k, v, slots, pool)
    ks, vs = _slot_view(pool)
    live = slots != -1
    assert np.array_equal(ks[slots[live]], k[live])
    assert np.array_equal(vs[slots[live]], v[live])
    untouched = np.setdiff1d(np.arange(nb * 16), slots[live])
    assert np.all(ks[untouched] == 0x7FC1) and np.all(vs[untouched] == 0x7FC1)


def test_write_gather_round_trip():
    rng = np.random.default_rng(2)
    nb, hkv, d, length = 9, 3, 4, 37
    pool = np.full((nb, 2, 16, hkv, d), 0x7FC1, dtype=np.uint16)
    table = rng.permutation(nb)[:3].astype(np.int32)
    pos = np.arange(length)
    slots = table[pos // 16] * 16 + pos % 16
    k = rng.integers(0, 1 << 15, (length, hkv, d)).astype(np.uint16)
    v = rng.integers(0, 1 << 15, (length, hkv, d)).astype(np.uint16)
    paged.kv_write(k, v, slots, pool)
    gk, gv = paged.gather(pool, np.concatenate([table, [-1, -1]]), length)
    assert np.array_equal(gk, k) and np.array_equal(gv, v)


def test_gather_reads_only_live_entries():
    pool = np.zeros((4, 2, 16, 1, 2), dtype=np.uint16)
    # entries past ceil(L/16) are garbage on purpose and must not be touched
    gk, _ = paged.gather(pool, np.array([2, 99999, -5], dtype=np.int32), 16)
    assert gk.shape == (16, 1, 2)
    with pytest.raises(ValueError):
        paged.gather(pool, np.array([2, 99999], dtype=np.int32), 17)


@pytest.mark.parametrize("slots", [[0, 5, 5], [-2, 1, 2], [0, 1, 64]])
def test_write_rejects_bad_slots(slots):
    pool = np.zeros((4, 2, 16, 1, 2), dtype=np.uint16)
    k = np.zeros((3, 1, 2), dtype=np.uint16)
    with pytest.raises(ValueError):
        paged.kv_write(k, k, np.array(slots, dtype=np.int32), pool)


def test_write_all_skipped_is_noop():
    pool = np.full((2, 2, 16, 1, 2), 7, dtype=np.uint16)
    k = np.ones((4, 1, 2), dtype=np.uint16)
    paged.kv_write(k, k, np.full(4, -1, dtype=np.int32), pool)
    assert np.all(pool == 7)


def test_decode_advance_matches_block_manager_model():
    # the slot of each new decode token, from the block-manager model's own
    # allocation (an independent computation of block * 16 + position)
    from oracle.block_manager import BlockManagerModel
    rng = np.random.default_rng([469, 65, 0])
    m = BlockManagerModel(200, prefix_caching=False)
    lens = [int(x) for x in rng.integers(1, 120, size=9)]
    for r, n in enumerate(lens):
        m.add_request(r, [0] * n)
        m.allocate_slots(r, n)
    for _ in range(40):
        width = max(len(m.block_table(r)) for r in range(9)) + 1
        tables = np.full((9, width), -1, dtype=np.int32)
        for r in range(9):
            t = m.block_table(r)
            tables[r, :len(t)] = t
        want = []
        for r in range(9):
            m.append_tokens(r, [0])
            want += m.allocate_slots(r, 1)
        # the model took any new block already; the table above may lack it:
        # refresh the table with the model's blocks first, as a caller would
        for r in range(9):
            t = m.block_table(r)
            tables[r, :len(t)] = t
        new_lens, cu, slots = paged.decode_advance(tables, lens, 200)
        assert slots.tolist() == want
        assert cu.tolist() == list(range(10)) and new_lens.tolist() == [x + 1 for x in lens]
        lens = new_lens.tolist()


def test_decode_advance_edges():
    tables = np.array([[3, -1], [5, 7], [1, 2]], dtype=np.int32)
    lens, cu, slots = paged.decode_advance(tables, [16, 31, 32], num_blocks=6)
    # segment 0: position 16 -> entry 1 = -1; segment 1: position 31 -> block 7
    # is outside a 6-block pool; segment 2: position 32 is past the table
    assert slots.tolist() == [-1, -1, -1]
    lens, cu, slots = paged.decode_advance(tables, [15, 17, 0], num_blocks=8)
    assert slots.tolist() == [3 * 16 + 15, 7 * 16 + 1, 1 * 16 + 0]
    assert lens.tolist() == [16, 18, 1] and cu.tolist() == [0, 1, 2, 3]
