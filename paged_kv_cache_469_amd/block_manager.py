"""ctypes binding of the host-side KV block manager declared in
``include/paged_block_manager.h`` (argument marshalling only; the manager
itself is C++ inside ``libpaged_attn.so``).

A ``BlockManager`` hands out 16-token blocks of one KV pool, keeps the
prefix cache and produces, for each step, the block tables, segment bounds,
sequence lengths and slot mapping that ``paged_kv_write`` and
``paged_attention`` take.
"""

import ctypes

import numpy as np

from ._lib import lib

OK = 0
EINVAL = 1
ENOSPACE = 4

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)

_SIGS = {
    "paged_bm_create": (ctypes.c_void_p, [ctypes.c_int64, ctypes.c_int32]),
    "paged_bm_destroy": (None, [ctypes.c_void_p]),
    "paged_bm_add_request": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, _i32p, ctypes.c_int32,
                                            ctypes.c_int64]),
    "paged_bm_append_tokens": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, _i32p, ctypes.c_int32]),
    "paged_bm_num_cached_tokens": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, _i32p]),
    "paged_bm_allocate_slots": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, _i32p]),
    "paged_bm_free_request": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64]),
    "paged_bm_block_table": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, _i32p, ctypes.c_int32,
                                            _i32p]),
    "paged_bm_step_metadata": (ctypes.c_int, [ctypes.c_void_p, _i64p, _i32p, ctypes.c_int32,
                                              ctypes.c_int32, _i32p, _i32p, _i32p, _i32p]),
    "paged_bm_num_free_blocks": (ctypes.c_int64, [ctypes.c_void_p]),
    "paged_bm_num_cached_blocks": (ctypes.c_int64, [ctypes.c_void_p]),
    "paged_bm_ref_count": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int64]),
    "paged_bm_free_queue": (ctypes.c_int64, [ctypes.c_void_p, _i32p, ctypes.c_int64]),
    "paged_bm_last_error": (ctypes.c_char_p, []),
}
_BOUND = None


def _c():
    global _BOUND
    if _BOUND is None:
        h = lib()
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _BOUND = h
    return _BOUND


class BlockManagerError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def _check(code):
    if code != OK:
        raise BlockManagerError(code, _c().paged_bm_last_error().decode())


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_i32p)


class BlockManager:
    """Blocks [0, num_blocks) of one pool; see the C header for the policies."""

    def __init__(self, num_blocks, prefix_caching=True):
        self._h = _c().paged_bm_create(int(num_blocks), 1 if prefix_caching else 0)
        if not self._h:
            raise BlockManagerError(EINVAL, _c().paged_bm_last_error().decode())
        self.num_blocks = int(num_blocks)

    def close(self):
        if self._h:
            _c().paged_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_request(self, req, tokens, salt=0):
        a, p = _i32(tokens)
        _check(_c().paged_bm_add_request(self._h, int(req), p, a.size, int(salt)))

    def append_tokens(self, req, tokens):
        a, p = _i32(tokens)
        _check(_c().paged_bm_append_tokens(self._h, int(req), p, a.size))

    def num_cached_tokens(self, req):
        out = ctypes.c_int32()
        _check(_c().paged_bm_num_cached_tokens(self._h, int(req), ctypes.byref(out)))
        return out.value

    def allocate_slots(self, req, num_new):
        """Slots (int32 array) of the request's next num_new tokens, or None
        when the free queue is too short (nothing changed)."""
        slots = np.empty(max(int(num_new), 0), dtype=np.int32)
        code = _c().paged_bm_allocate_slots(self._h, int(req), int(num_new),
                                            slots.ctypes.data_as(_i32p))
        if code == ENOSPACE:
            return None
        _check(code)
        return slots

    def free_request(self, req):
        _check(_c().paged_bm_free_request(self._h, int(req)))

    def block_table(self, req):
        n = ctypes.c_int32()
        _check(_c().paged_bm_block_table(self._h, int(req), None, 0, ctypes.byref(n)))
        out = np.empty(n.value, dtype=np.int32)
        _check(_c().paged_bm_block_table(self._h, int(req), out.ctypes.data_as(_i32p), n.value,
                                         ctypes.byref(n)))
        return out

    def step_metadata(self, reqs, num_new, width):
        """(block_tables [S, width], cu_seqlens_q [S+1], seq_lens [S],
        slot_mapping [sum num_new]) as int32 arrays, for requests that were
        just given num_new[s] slots, in packing order."""
        r = np.ascontiguousarray(reqs, dtype=np.int64)
        n, np_ = _i32(num_new)
        s = r.size
        tables = np.empty((s, width), dtype=np.int32)
        cu = np.empty(s + 1, dtype=np.int32)
        lens = np.empty(s, dtype=np.int32)
        slots = np.empty(int(n.sum()), dtype=np.int32)
        _check(_c().paged_bm_step_metadata(self._h, r.ctypes.data_as(_i64p), np_, s, int(width),
                                           tables.ctypes.data_as(_i32p), cu.ctypes.data_as(_i32p),
                                           lens.ctypes.data_as(_i32p),
                                           slots.ctypes.data_as(_i32p)))
        return tables, cu, lens, slots

    def num_free_blocks(self):
        return int(_c().paged_bm_num_free_blocks(self._h))

    def num_cached_blocks(self):
        return int(_c().paged_bm_num_cached_blocks(self._h))

    def ref_count(self, block):
        return int(_c().paged_bm_ref_count(self._h, int(block)))

    def free_queue(self):
        n = int(_c().paged_bm_free_queue(self._h, None, 0))
        out = np.empty(n, dtype=np.int32)
        _c().paged_bm_free_queue(self._h, out.ctypes.data_as(_i32p), n)
        return out
