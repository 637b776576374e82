"""Pins for the oracle's paged attention.

Brute force (a scalar pure-Python twin) on tiny random cases; closed forms
that fix the scale, the softmax axis, the causal alignment and the GQA head
mapping; and the invariants the pages fix: paged == dense, invariance under
a permutation of physical blocks, shared prefix blocks == private copies,
segments isolated, decode token == last row of a full prefill, chunk rows ==
the matching rows of a full prefill.
"""

import math

import numpy as np
import pytest

from oracle import bf16, brute, paged
from oracle_cases import bits, new_rows, paged_case, random_req

SCALE64 = float(np.float32(1 / 8))


def _q(rng, t, hq, d, gain=1.0):
    return bits(rng.standard_normal((t, hq, d)) * gain)


def _run(q, case, scale):
    pool, tables, cu, lens = case
    return paged.attend(q, pool, tables, cu, lens, scale)


# ---------------------------------------------------------------- brute force

def _brute(q, case, scale):
    pool, tables, cu, lens = case
    qf = bf16.to_f64(q).tolist()
    pf = bf16.to_f64(pool).tolist()
    return np.array(brute.attend(qf, pf, tables.tolist(), cu.tolist(), lens.tolist(), scale))


@pytest.mark.parametrize("seed", range(12))
def test_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = int(rng.choice([1, 2, 4, 8]))
    reqs = []
    for _ in range(int(rng.integers(1, 5))):
        length = int(rng.integers(1, 41))
        n = int(rng.integers(0, length + 1))
        reqs.append(random_req(rng, length, n, hkv, d, gain=1.5))
    nb = sum((k.shape[0] + 15) // 16 for k, _, _ in reqs) + 2
    case = paged_case(reqs, hkv, d, nb, perm_seed=seed)
    q = _q(rng, new_rows(reqs), hq, d, gain=1.5)
    scale = float(np.float32(rng.uniform(0.1, 1.0)))
    got = _run(q, case, scale)
    want = _brute(q, case, scale)
    assert np.max(np.abs(got - want)) <= 1e-12


# ---------------------------------------------------------------- closed forms

def test_single_key_returns_its_value_exactly():
    rng = np.random.default_rng(3)
    k, v, _ = random_req(rng, 1, 1, 2, 8)
    case = paged_case([(k, v, 1)], 2, 8, 4)
    q = _q(rng, 1, 4, 8, gain=3.0)
    out = _run(q, case, 0.3)
    want = bf16.to_f64(v)[0]
    assert np.array_equal(out[0, :2], np.broadcast_to(want[0], (2, 8)))
    assert np.array_equal(out[0, 2:], np.broadcast_to(want[1], (2, 8)))


def test_zero_query_gives_causal_mean():
    rng = np.random.default_rng(4)
    length, n, hkv, d = 29, 5, 1, 4
    k, v, _ = random_req(rng, length, n, hkv, d)
    case = paged_case([(k, v, n)], hkv, d, 3)
    q = np.zeros((n, 2, d), dtype=np.uint16)
    out = _run(q, case, 0.5)
    vf = bf16.to_f64(v)[:, 0]
    h = length - n
    for i in range(n):
        assert np.allclose(out[i, 0], vf[:h + i + 1].mean(axis=0), rtol=0, atol=1e-13)


def test_index_valued_v_pins_causal_alignment():
    # V[j] = j and a zero query: row i averages keys 0..h+i, i.e. (h+i)/2.
    rng = np.random.default_rng(5)
    length, n, d = 40, 7, 2
    k = bits(rng.standard_normal((length, 1, d)))
    v = bits(np.repeat(np.arange(length, dtype=np.float64)[:, None, None], d, axis=2))
    case = paged_case([(k, v, n)], 1, d, 4)
    out = _run(np.zeros((n, 1, d), dtype=np.uint16), case, 1.0)
    h = length - n
    for i in range(n):
        assert abs(out[i, 0, 0] - (h + i) / 2) < 1e-12


def test_head_valued_v_pins_gqa_mapping():
    # V[:, g, :] = g: query head hq must read KV head hq // G.
    rng = np.random.default_rng(6)
    hkv, group, length, d = 4, 3, 20, 4
    k = bits(rng.standard_normal((length, hkv, d)))
    v = bits(np.broadcast_to(np.arange(hkv, dtype=np.float64)[None, :, None], (length, hkv, d)))
    case = paged_case([(k, v, 2)], hkv, d, 3)
    q = _q(rng, 2, hkv * group, d)
    out = _run(q, case, 0.7)
    for hq in range(hkv * group):
        assert np.max(np.abs(out[:, hq] - hq // group)) <= 1e-14


def test_two_keys_logistic_form():
    # q = e0, k0 = a e0, k1 = b e0: the second key's weight is
    # 1 / (1 + exp(scale * (a - b))); a prefill's first row sees key 0 only.
    a, b, scale, d = 1.5, -0.5, 0.375, 4
    k = np.zeros((2, 1, d))
    k[0, 0, 0], k[1, 0, 0] = a, b
    v = np.array([[[1.0, -2.0, 0.5, 3.0]], [[-1.0, 4.0, 0.25, 0.0]]])
    q1 = np.zeros((1, 1, d))
    q1[0, 0, 0] = 1.0
    w1 = 1.0 / (1.0 + math.exp(scale * (a - b)))
    want = (1 - w1) * v[0, 0] + w1 * v[1, 0]
    dec = paged_case([(bits(k), bits(v), 1)], 1, d, 2)
    assert np.allclose(_run(bits(q1), dec, scale)[0, 0], want, rtol=0, atol=1e-15)
    pre = paged_case([(bits(k), bits(v), 2)], 1, d, 2)
    out = _run(bits(np.concatenate([q1, q1])), pre, scale)
    assert np.array_equal(out[0, 0], v[0, 0])
    assert np.allclose(out[1, 0], want, rtol=0, atol=1e-15)


def test_dominant_key_only_when_visible():
    # one key aligned with a large query dominates rows that can see it and
    # has no effect on rows before it
    rng = np.random.default_rng(8)
    length, n, d = 24, 24, 8
    k = rng.standard_normal((length, 1, d)) * 0.1
    qv = np.zeros(d)
    qv[0] = 8.0
    k[10, 0] = 0
    k[10, 0, 0] = 8.0
    v = rng.standard_normal((length, 1, d))
    case = paged_case([(bits(k), bits(v), n)], 1, d, 3)
    q = bits(np.broadcast_to(qv, (n, 1, d)))
    out = _run(q, case, 1.0)
    vb = bf16.to_f64(bits(v))
    for i in range(n):
        if i >= 10:
            assert np.max(np.abs(out[i, 0] - vb[10, 0])) < 1e-9
        else:
            assert np.max(np.abs(out[i, 0] - vb[10, 0])) > 1e-3


# ---------------------------------------------------------------- invariants

def _mixed(rng, hkv=2, d=8, specs=((6, 6), (1, 38), (5, 45), (0, 12), (17, 33))):
    return [random_req(rng, length, n, hkv, d) for n, length in specs]


def test_paged_equals_dense():
    rng = np.random.default_rng(9)
    reqs = _mixed(rng)
    case = paged_case(reqs, 2, 8, 20, perm_seed=3)
    q = _q(rng, new_rows(reqs), 8, 8)
    out = _run(q, case, SCALE64)
    row = 0
    for k, v, n in reqs:
        if n:
            dense = paged.attend_dense(bf16.to_f64(q[row:row + n]), bf16.to_f64(k),
                                       bf16.to_f64(v), SCALE64, k.shape[0] - n)
            assert np.array_equal(out[row:row + n], dense)
        row += n


def test_block_permutation_invariance():
    rng = np.random.default_rng(10)
    reqs = _mixed(rng)
    q = _q(rng, new_rows(reqs), 8, 8)
    a = _run(q, paged_case(reqs, 2, 8, 20, perm_seed=1), SCALE64)
    b = _run(q, paged_case(reqs, 2, 8, 40, perm_seed=2), SCALE64)
    assert np.array_equal(a, b)


def test_shared_prefix_equals_private_copies():
    rng = np.random.default_rng(11)
    hkv, d, prefix = 2, 8, 32
    pk, pv, _ = random_req(rng, prefix, 0, hkv, d)
    reqs = []
    for length in (45, 33, 60):
        k, v, _ = random_req(rng, length, 1, hkv, d)
        k[:prefix], v[:prefix] = pk, pv
        reqs.append((k, v, 1))
    q = _q(rng, 3, 4, d)
    private = _run(q, paged_case(reqs, hkv, d, 16, perm_seed=4), SCALE64)
    tables = np.full((3, 4), -1, dtype=np.int32)
    tables[:, :2] = [7, 3]                      # the shared, refcounted blocks
    tables[0, 2:3] = [0]
    tables[1, 2:3] = [1]
    tables[2, 2:4] = [2, 5]
    shared = _run(q, paged_case(reqs, hkv, d, 8, tables=tables), SCALE64)
    assert np.array_equal(private, shared)


def test_segments_isolated():
    rng = np.random.default_rng(12)
    reqs = _mixed(rng)
    q = _q(rng, new_rows(reqs), 8, 8)
    base = _run(q, paged_case(reqs, 2, 8, 20), SCALE64)
    other = _mixed(np.random.default_rng(99))
    mixed = [reqs[0], other[1], reqs[2], other[3], other[4]]
    q2 = q.copy()
    rows = np.cumsum([0] + [n for _, _, n in reqs])
    q2[rows[1]:rows[2]] = _q(rng, 1, 8, 8)
    out = _run(q2, paged_case(mixed, 2, 8, 20), SCALE64)
    for s in (0, 2):
        assert np.array_equal(out[rows[s]:rows[s + 1]], base[rows[s]:rows[s + 1]])


def test_decode_is_last_row_of_full_prefill():
    rng = np.random.default_rng(13)
    length, hkv, d = 53, 2, 8
    k, v, _ = random_req(rng, length, 0, hkv, d)
    q = _q(rng, length, 8, 8)
    full = _run(q, paged_case([(k, v, length)], hkv, d, 4), SCALE64)
    dec = _run(q[-1:], paged_case([(k, v, 1)], hkv, d, 4), SCALE64)
    assert np.max(np.abs(dec[0] - full[-1])) <= 1e-13


def test_chunk_rows_equal_full_prefill_rows():
    rng = np.random.default_rng(14)
    length, chunk, hkv, d = 70, 21, 2, 8
    k, v, _ = random_req(rng, length, 0, hkv, d)
    q = _q(rng, length, 4, d)
    full = _run(q, paged_case([(k, v, length)], hkv, d, 5), SCALE64)
    # the chunk covers positions [30, 51): its request holds 51 tokens
    lo, hi = 30, 30 + chunk
    part = _run(q[lo:hi], paged_case([(k[:hi], v[:hi], chunk)], hkv, d, 5), SCALE64)
    assert np.max(np.abs(part - full[lo:hi])) <= 1e-13


def test_tail_and_padding_never_read():
    # NaN in the unused rows of the last block and garbage table padding
    rng = np.random.default_rng(15)
    reqs = _mixed(rng)
    case = paged_case(reqs, 2, 8, 20, poison=0x7FC1)
    pool, tables, cu, lens = case
    tables = tables.copy()
    for s, length in enumerate(lens):
        tables[s, (length + 15) // 16:] = 123456
    out = paged.attend(_q(rng, new_rows(reqs), 8, 8), pool, tables, cu, lens, SCALE64)
    assert np.all(np.isfinite(out))


def test_empty_segments_and_errors():
    rng = np.random.default_rng(16)
    k, v, _ = random_req(rng, 10, 0, 1, 2)
    case = paged_case([(k, v, 0)], 1, 2, 2)
    out = _run(np.zeros((0, 1, 2), dtype=np.uint16), case, 1.0)
    assert out.shape == (0, 1, 2)
    pool, tables, _, lens = case
    with pytest.raises(ValueError):      # more new tokens than the sequence
        paged.attend(np.zeros((11, 1, 2), np.uint16), pool, tables,
                     np.array([0, 11]), lens, 1.0)
    with pytest.raises(ValueError):      # decreasing segment bounds
        paged.attend(np.zeros((2, 1, 2), np.uint16), pool, tables,
                     np.array([0, 2, 1]), np.array([10, 10]), 1.0)
