"""Small builders for hand-made paged cases used by the oracle pin tests.

Test code only: lays dense per-request K/V into a paged pool with the
oracle's own write, so the pins can compare paged results with dense ones.
"""

import numpy as np

from oracle import bf16, paged


def bits(x):
    """float array -> bf16 bits (exact for values that are bf16 already)."""
    return bf16.from_f64(np.asarray(x, dtype=np.float64))


def paged_case(reqs, hkv, d, num_blocks, perm_seed=0, poison=0x7FC1, tables=None):
    """reqs: list of (k_bits [L,Hkv,D], v_bits, n_new).  Returns
    (pool, block_tables, cu_seqlens_q, seq_lens) with each request's blocks
    taken from a seeded permutation of the pool, unless ``tables`` is given."""
    rng = np.random.default_rng(perm_seed)
    pool = np.full((num_blocks, 2, 16, hkv, d), poison, dtype=np.uint16)
    lens = [k.shape[0] for k, _, _ in reqs]
    width = max(1, max((length + 15) // 16 for length in lens))
    if tables is None:
        perm = rng.permutation(num_blocks)
        tables = np.full((len(reqs), width), -1, dtype=np.int32)
        c = 0
        for s, length in enumerate(lens):
            nb = (length + 15) // 16
            tables[s, :nb] = perm[c:c + nb]
            c += nb
    for s, (k, v, _) in enumerate(reqs):
        length = k.shape[0]
        pos = np.arange(length)
        slots = tables[s][pos // 16].astype(np.int64) * 16 + pos % 16
        # a shared block is written once: skip slots already written by an
        # earlier request with the same data
        fresh = pool[slots // 16, 0, slots % 16, 0, 0] == poison
        paged.kv_write(k[fresh], v[fresh], slots[fresh], pool)
    cu = np.zeros(len(reqs) + 1, dtype=np.int32)
    cu[1:] = np.cumsum([n for _, _, n in reqs])
    return pool, tables, cu, np.array(lens, dtype=np.int32)


def random_req(rng, length, n, hkv, d, gain=1.0):
    k = bits(rng.standard_normal((length, hkv, d)) * gain)
    v = bits(rng.standard_normal((length, hkv, d)))
    return k, v, n


def new_rows(reqs):
    return sum(n for _, _, n in reqs)
