"""Plant plausible mistakes in copies of the block-manager model and of the
oracle's decode-step metadata (CPU only), and check that their pins catch
each one: every pin test of the module is run with the mutant swapped in,
and at least one must fail."""

import importlib.util
import inspect
import os
import types

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_DIR = os.path.dirname(oracle.__file__)


def _load(path, name, old=None, new=None):
    text = open(path).read()
    if old is not None:
        assert old in text, old
        text = text.replace(old, new, 1)
    mod = types.ModuleType(name)
    mod.__package__ = "oracle"
    mod.__file__ = path
    exec(compile(text, path, "exec"), mod.__dict__)
    return mod


def _pins_pass(pin_file, swap):
    """Run every test_* function of ``pin_file`` (parametrised seeds
    included) with the globals in ``swap`` replaced; True if all pass."""
    spec = importlib.util.spec_from_file_location("pins_" + os.path.basename(pin_file)[:-3],
                                                  os.path.join(HERE, pin_file))
    pins = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(pins)
    for k, v in swap.items():
        setattr(pins, k, v)
    for name, fn in vars(pins).items():
        if not name.startswith("test_") or not callable(fn):
            continue
        marks = getattr(fn, "pytestmark", [])
        cases = [{}]
        for mk in marks:
            if mk.name == "parametrize":
                arg, values = mk.args
                cases = [{arg: v} for v in values]
        params = inspect.signature(fn).parameters
        for case in cases:
            if set(params) - set(case):
                continue
            try:
                fn(**case)
            except Exception:      # an assertion, or a crash of the mutant
                return False
    return True


BM_SRC = os.path.join(ORACLE_DIR, "block_manager.py")


def _bm_pins_pass(old=None, new=None):
    mod = _load(BM_SRC, "oracle._bm_mutant", old, new)
    return _pins_pass("test_oracle_block_manager.py", {"BlockManagerModel": mod.BlockManagerModel})


def test_unmutated_block_manager_model_passes():
    assert _bm_pins_pass()


BM_MUTATIONS = [
    ("released blocks go to the front of the queue", "self.free.append(b)",
     "self.free.insert(0, b)"),
    ("blocks released first to last", "for b in reversed(r[\"table\"]):",
     "for b in r[\"table\"]:"),
    ("new blocks from the back of the queue", "b = self.free.pop(0)", "b = self.free.pop()"),
    ("whole prompt may hit the cache", "range((len(r[\"tokens\"]) - 1) // BLOCK)",
     "range(len(r[\"tokens\"]) // BLOCK)"),
    ("key holds only the block's own tokens", "tuple(tokens[:(b + 1) * BLOCK])",
     "tuple(tokens[b * BLOCK:(b + 1) * BLOCK])"),
    ("salt left out of the key", "return (salt, tuple(", "return (0, tuple("),
    ("partial blocks registered", "while (r[\"registered\"] + 1) * BLOCK <= r[\"computed\"]:",
     "while r[\"registered\"] * BLOCK < r[\"computed\"]:"),
    ("evicted block stays in the cache", "del self.cache[self.key[b]]", "pass"),
    ("hit does not add a reference", "self.ref[b] += 1", "self.ref[b] = 1"),
    ("hit stays in the free queue", "self.free.remove(b)", "pass"),
    ("hits not counted in blocks held", "(len(r[\"table\"]) + len(hits))", "len(r[\"table\"])"),
    ("hits in the queue counted as free", "available = len(self.free) - sum(",
     "available = len(self.free) + 0 * sum("),
    ("re-registration over an existing key", "if self.key[blk] is None and k not in self.cache:",
     "if self.key[blk] is None:"),
    ("cache matched again mid-request", "first = not r[\"table\"] and r[\"computed\"] == 0",
     "first = r[\"computed\"] % BLOCK == 0"),
    ("step slots shifted by one", "for p in range(L - n, L)]", "for p in range(L - n + 1, L + 1)]"),
    ("step tables not padded", "r[\"table\"] + [-1] * (width - len(r[\"table\"]))",
     "r[\"table\"] + [0] * (width - len(r[\"table\"]))"),
]


@pytest.mark.parametrize("name,old,new", BM_MUTATIONS, ids=[m[0] for m in BM_MUTATIONS])
def test_block_manager_pins_catch_mutation(name, old, new):
    assert not _bm_pins_pass(old, new), name


PAGED_SRC = os.path.join(ORACLE_DIR, "paged.py")


def _advance_pins_pass(old=None, new=None):
    mod = _load(PAGED_SRC, "oracle._paged_mutant", old, new)
    spec = importlib.util.spec_from_file_location("pins_write", os.path.join(HERE, "test_oracle_write.py"))
    pins = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(pins)
    pins.paged = mod
    try:
        pins.test_decode_advance_matches_block_manager_model()
        pins.test_decode_advance_edges()
    except Exception:
        return False
    return True


def test_unmutated_decode_advance_passes():
    assert _advance_pins_pass()


ADVANCE_MUTATIONS = [
    ("slot of the last known position", "pos = int(lens[s])", "pos = int(lens[s]) - 1"),
    ("block index from the wrong divisor", "b = int(tables[s, pos // BLOCK_SIZE])",
     "b = int(tables[s, pos // (BLOCK_SIZE + 1)])"),
    ("pool bound not checked", "if 0 <= b < num_blocks:", "if 0 <= b:"),
    ("table width off by one", "if 0 <= pos and pos // BLOCK_SIZE < width:",
     "if 0 <= pos and pos // BLOCK_SIZE <= width:"),
    ("lengths not advanced", "return ((lens + 1).astype(np.int32)", "return ((lens).astype(np.int32)"),
]


@pytest.mark.parametrize("name,old,new", ADVANCE_MUTATIONS, ids=[m[0] for m in ADVANCE_MUTATIONS])
def test_decode_advance_pins_catch_mutation(name, old, new):
    assert not _advance_pins_pass(old, new), name


def test_runner_runs_every_pin_case():
    # the runner must execute each parametrised seed of the invariant pins,
    # not skip the functions that take arguments
    mod = _load(BM_SRC, "oracle._bm_clean")
    calls = []

    class Counting(mod.BlockManagerModel):
        def __init__(self, *a, **k):
            calls.append(1)
            super().__init__(*a, **k)
    assert _pins_pass("test_oracle_block_manager.py", {"BlockManagerModel": Counting})
    # one model per plain pin, one per seed of the random-operation pin
    import test_oracle_block_manager as pins
    plain = [n for n in vars(pins) if n.startswith("test_")]
    assert len(calls) == len(plain) - 1 + 6
