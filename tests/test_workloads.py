"""The seeded generators: determinism, structure and accounting."""

import numpy as np
import pytest

import workloads
from oracle import paged


def test_tiny_mixed_structure():
    wl = workloads.make("tiny_mixed")
    assert wl.cu_seqlens_q.tolist() == [0, 6, 7]
    assert wl.seq_lens.tolist() == [6, 38]
    assert wl.num_blocks == 64 and wl.group == 8
    t = wl.block_tables
    assert (t[0] >= 0).sum() == 1 and (t[1] >= 0).sum() == 3
    # B's new token sits at position 37: block 2 of its table, row 5
    assert wl.slot_mapping[6] == t[1, 2] * 16 + 5
    assert wl.slot_mapping[:6].tolist() == [t[0, 0] * 16 + i for i in range(6)]


def test_deterministic():
    a = workloads.make("decode_8b", num_requests=8)
    b = workloads.make("decode_8b", num_requests=8)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.q(), b.q())
    assert np.array_equal(a.request_kv(3)[0], b.request_kv(3)[0])


def _check_slots_cover(wl):
    slots = [wl.slot_mapping]
    for s, _, _ in wl.history_chunks():
        slots.append(s)
    allslots = np.concatenate(slots)
    assert np.unique(allslots).size == allslots.size
    assert allslots.min() >= 0 and allslots.max() < wl.num_blocks * 16
    # every position < L of every segment is written exactly once overall
    want = set()
    for s in range(wl.num_seqs):
        want.update(wl.slots_of(s, 0, int(wl.seq_lens[s])).tolist())
    assert set(allslots.tolist()) == want


@pytest.mark.parametrize("name,kw", [
    ("tiny_mixed", {}),
    ("decode_8b", {"num_requests": 10}),
    ("prefill_8b", {"num_prompts": 3, "lens": (20, 70)}),
    ("cb_step_8b", {"num_decodes": 6, "ctx": (40, 90), "shared": 3, "prefix": 32,
                    "chunk": 20, "chunk_history": 48}),
    ("cb_step_8b", {"num_decodes": 6, "ctx": (40, 90), "shared": 3, "prefix": 32,
                    "chunk": 20, "chunk_history": 48, "decode_first": False}),
    ("long_decode_70b", {"num_requests": 3, "ctx": (100, 300), "num_blocks": 5000}),
    ("spec_verify_8b", {"num_requests": 5, "ctx": (30, 90)}),
    ("spec_verify_70b", {"num_requests": 4, "ctx": (30, 90)}),
])
def test_structure(name, kw):
    wl = workloads.make(name, **kw)
    _check_slots_cover(wl)
    assert wl.block_tables.shape == (wl.num_seqs, wl.max_blocks_per_seq)
    k, v = wl.new_kv()
    assert k.shape == (wl.num_tokens, wl.num_kv_heads, wl.head_dim)
    assert wl.q().shape == (wl.num_tokens, wl.num_q_heads, wl.head_dim)


def test_shared_prefix_tables_and_values():
    wl = workloads.make("cb_step_8b", num_decodes=5, ctx=(40, 90), shared=3,
                        prefix=32, chunk=20, chunk_history=48)
    t = wl.block_tables
    assert np.array_equal(t[0, :2], t[1, :2]) and np.array_equal(t[0, :2], t[2, :2])
    assert not np.array_equal(t[3, :2], t[0, :2])
    k0, _ = wl.request_kv(0)
    k1, _ = wl.request_kv(1)
    assert np.array_equal(k0[:32], k1[:32]) and not np.array_equal(k0[32:40], k1[32:40])
    assert wl.kv_bytes_unique() == wl.kv_bytes_logical() - 2 * 32 * 4096


def test_host_pool_holds_every_request():
    # writing history + new tokens with the oracle gives back each request's K/V
    wl = workloads.make("cb_step_8b", num_decodes=4, ctx=(40, 60), shared=2,
                        prefix=32, chunk=17, chunk_history=16)
    pool = np.full((wl.num_blocks, 2, 16, 8, 128), 0x7FC1, dtype=np.uint16)
    for slots, k, v in wl.history_chunks():
        paged.kv_write(k, v, slots, pool)
    k, v = wl.new_kv()
    paged.kv_write(k, v, wl.slot_mapping, pool)
    for s in range(wl.num_seqs):
        gk, gv = paged.gather(pool, wl.block_tables[s], int(wl.seq_lens[s]))
        rk, rv = wl.request_kv(s)
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv)


def test_full_size_accounting():
    # the expected sizes of the five workloads (lengths only, no values)
    d2 = workloads.make("decode_8b")
    assert d2.num_seqs == 256 and d2.num_tokens == 256
    assert 2.2e9 < d2.kv_bytes_logical() < 2.6e9
    p3 = workloads.make("prefill_8b")
    assert 1.6e11 < p3.attention_flops() < 2.6e11
    c4 = workloads.make("cb_step_8b")
    assert c4.num_tokens == 192 + 2048 <= 8192
    assert c4.kv_bytes_logical() - c4.kv_bytes_unique() == 63 * 1024 * 4096
    assert c4.attention_flops(segments=[192]) == 4 * 128 * 32 * (2048 * 16384 + 2048 * 2049 // 2)
    assert workloads.make("tiny_mixed").kv_bytes_logical() == (6 + 38) * 1024
