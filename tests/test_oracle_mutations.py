"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that
the pins catch each one: a pin set that passes a broken oracle pins nothing."""

import importlib.util
import math
import os
import sys
import types

import numpy as np
import pytest

import oracle
from oracle import bf16, brute
from oracle_cases import bits, paged_case, random_req

SRC = os.path.join(os.path.dirname(oracle.__file__), "paged.py")


def _mutant(old, new):
    text = open(SRC).read()
    assert old in text, old
    mod = types.ModuleType("oracle._mutant")
    mod.__package__ = "oracle"
    exec(compile(text.replace(old, new, 1), SRC, "exec"), mod.__dict__)
    return mod


def _pins_pass(mod):
    """A compact run of the attention and write pins against ``mod``."""
    try:
        # brute force on mixed shapes
        for seed in range(4):
            rng = np.random.default_rng(500 + seed)
            hkv, hq, d = 2, 4, 4
            reqs = [random_req(rng, length, n, hkv, d, gain=1.5)
                    for n, length in ((3, 20), (1, 9), (5, 5))]
            pool, tables, cu, lens = paged_case(reqs, hkv, d, 8, perm_seed=seed)
            for (k, v, n), s in zip(reqs, range(3)):
                pos = np.arange(k.shape[0])
                slots = tables[s][pos // 16].astype(np.int64) * 16 + pos % 16
                fresh = np.full((8, 2, 16, hkv, d), 0x7FC1, np.uint16)
                mod.kv_write(k, v, slots, fresh)
                gk, gv = mod.gather(fresh, tables[s], k.shape[0])
                if not (np.array_equal(gk, k) and np.array_equal(gv, v)):
                    return False
            q = bits(rng.standard_normal((9, hq, d)) * 1.5)
            got = mod.attend(q, pool, tables, cu, lens, 0.375)
            want = np.array(brute.attend(bf16.to_f64(q).tolist(), bf16.to_f64(pool).tolist(),
                                         tables.tolist(), cu.tolist(), lens.tolist(), 0.375))
            if np.max(np.abs(got - want)) > 1e-12:
                return False
        # two-key logistic form (scale, sign, softmax axis)
        a, b, scale = 1.5, -0.5, 0.375
        k = np.zeros((2, 1, 2))
        k[0, 0, 0], k[1, 0, 0] = a, b
        v = np.array([[[1.0, -2.0]], [[-1.0, 4.0]]])
        q1 = np.zeros((1, 1, 2))
        q1[0, 0, 0] = 1.0
        w1 = 1.0 / (1.0 + math.exp(scale * (a - b)))
        pool, tables, cu, lens = paged_case([(bits(k), bits(v), 1)], 1, 2, 2)
        out = mod.attend(bits(q1), pool, tables, cu, lens, scale)
        if not np.allclose(out[0, 0], (1 - w1) * v[0, 0] + w1 * v[1, 0], rtol=0, atol=1e-15):
            return False
        # index-valued V (causal alignment) with a chunk over history
        vv = bits(np.repeat(np.arange(40.0)[:, None, None], 2, axis=2))
        kk = bits(np.random.default_rng(1).standard_normal((40, 1, 2)))
        pool, tables, cu, lens = paged_case([(kk, vv, 7)], 1, 2, 4)
        out = mod.attend(np.zeros((7, 1, 2), np.uint16), pool, tables, cu, lens, 1.0)
        if any(abs(out[i, 0, 0] - (33 + i) / 2) > 1e-12 for i in range(7)):
            return False
        # head-valued V (GQA mapping)
        kh = bits(np.random.default_rng(2).standard_normal((20, 4, 2)))
        vh = bits(np.broadcast_to(np.arange(4.0)[None, :, None], (20, 4, 2)))
        pool, tables, cu, lens = paged_case([(kh, vh, 2)], 4, 2, 3)
        qh = bits(np.random.default_rng(3).standard_normal((2, 12, 2)))
        out = mod.attend(qh, pool, tables, cu, lens, 0.7)
        if any(np.max(np.abs(out[:, h] - h // 3)) > 1e-14 for h in range(12)):
            return False
        return True
    except (ValueError, IndexError):
        return False


def test_unmutated_oracle_passes():
    spec = importlib.util.spec_from_file_location("oracle._clean", SRC)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    sys.modules["oracle._clean"] = mod
    spec.loader.exec_module(mod)
    assert _pins_pass(mod)


MUTATIONS = [
    ("causal off by one", "keys[None, :] <= (history", "keys[None, :] < (history"),
    ("history ignored", "(history + np.arange(i0, i1))", "(np.arange(i0, i1))"),
    ("scale dropped", "x = (sc * (qg @ kg.T))", "x = ((qg @ kg.T))"),
    ("scale squared", "x = (sc * (qg @ kg.T))", "x = (sc * sc * (qg @ kg.T))"),
    ("interleaved GQA heads", "qg = q[i0:i1, g * group:(g + 1) * group, :]",
     "qg = q[i0:i1, g::hkv, :]"),
    ("values read from keys", "vg = np.ascontiguousarray(v[:, g, :])",
     "vg = np.ascontiguousarray(k[:, g, :])"),
    ("normalised over heads", "num / w.sum(axis=2)[..., None]",
     "num / w.sum(axis=(1, 2))[:, None, None]"),
    ("missing max shift sign", "w = np.exp(x - m)", "w = np.exp(m - x)"),
    ("K/V halves swapped in write", "pool[b, 0, r] = k[t]", "pool[b, 1, r] = k[t]"),
    ("slot split with the wrong block size", "b, r = divmod(s, BLOCK_SIZE)",
     "b, r = divmod(s, 8)"),
    ("gather reads V from K", "v = pool[ids, 1]", "v = pool[ids, 0]"),
]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(name, old, new):
    assert not _pins_pass(_mutant(old, new)), name
