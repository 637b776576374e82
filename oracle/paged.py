"""The oracle proper: paged KV write and paged attention, plain and in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

What is computed, and where the pages state it:

* Pool layout.  The KV cache is cut into fixed blocks of 16 token slots
  ([NOTES01] section 1.5: default block size 16).  One block holds, for one
  layer, both keys and values of its 16 slots for every KV head, so its size
  in bytes is 2 * block_size * kv_heads * head_size * dtype_bytes ([INSIDE],
  the block size formula of the engine-constructor part).  Here the pool is a
  uint16 (bf16 bit) array of shape [num_blocks, 2, 16, kv_heads, head_dim]:
  index 0 of axis 1 holds keys, index 1 values.

* Write ([NOTES01] section 1.6): the attention operator is told, for every
  new token, which block and which position inside it its K/V goes to (the
  slot mapping).  Reading taken: ``slot = block * 16 + position``; ``-1``
  means "no write"; any other value outside the pool, or a slot repeated
  within one call, is a caller error.

* Attention ([NOTES01] sections 1.4, 1.6, 2.1): all tokens of a step are
  packed end to end; the operator is told where each segment starts and ends
  and segments never see each other.  Each request has a number of computed
  tokens and a total; a step catches the first up to the second, so a segment
  with ``n`` new tokens and total length ``L`` has ``h = L - n`` tokens of
  history already in its blocks (decode: n = 1; prefill: h = 0; a chunk of a
  long prompt: both > 0).  Reading taken: query ``i`` of the segment sits at
  absolute position ``h + i`` and attends to keys ``0 .. h + i`` (causal,
  aligned to the end of the history).  The new tokens' K/V are written before
  attention runs, so they are read from the pool like the history.  Keys of
  KV head ``g`` serve query heads ``g*G .. g*G+G-1`` with ``G = Hq / Hkv``.
  Softmax scale is a caller-given float32; the oracle uses exactly that
  float32 value, widened to fp64.

* Unused table entries and the unfilled tail of the last block are never
  read ([NOTES01] section 1.5: a request wastes at most the unfilled part of
  its last block).

Parity status: every function below is pinned (``tests/test_oracle_*.py``):
block bytes by the page's closed form; write by round trips and poison
checks; the decode-step metadata by the block-manager model's slots for a
decode token and by its out-of-table and out-of-pool cases; attention by brute force on tiny inputs, by closed forms (single key,
zero query, index-valued V, head-valued V, two-key logistic form, one
dominant key) and by the invariants paged == dense, block permutation,
shared prefix == private copies, segment isolation, decode == last row of a
full prefill and chunk == matching rows of a full prefill.
"""

import numpy as np

BLOCK_SIZE = 16


def block_bytes(block_size, num_kv_heads, head_dim, dtype_bytes):
    """Bytes of one block for one layer: K and V, all KV heads ([INSIDE])."""
    return 2 * block_size * num_kv_heads * head_dim * dtype_bytes


def check_slots(slot_mapping, num_blocks):
    """Raise ValueError unless every slot is -1 or a unique in-pool slot."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = slots[slots != -1]
    if live.size and (live.min() < 0 or live.max() >= num_blocks * BLOCK_SIZE):
        raise ValueError("slot outside the pool")
    if np.unique(live).size != live.size:
        raise ValueError("slot written twice in one call")


def kv_write(k, v, slot_mapping, pool):
    """Scatter new tokens' K/V rows into the pool, in place, as a bit copy.

    k, v: uint16 [T, Hkv, D]; slot_mapping: int [T]; pool: uint16
    [NB, 2, 16, Hkv, D].  Token t with slot s != -1 goes to block s // 16,
    position s % 16 ([NOTES01] section 1.6, slot mapping).
    """
    k = np.asarray(k)
    v = np.asarray(v)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    if k.shape != v.shape or k.shape[0] != slots.shape[0]:
        raise ValueError("k, v and slot_mapping disagree on the token count")
    if k.shape[1:] != pool.shape[3:]:
        raise ValueError("k/v rows do not match the pool's [kv_heads, head_dim]")
    check_slots(slots, pool.shape[0])
    for t in range(slots.shape[0]):
        s = int(slots[t])
        if s == -1:
            continue
        b, r = divmod(s, BLOCK_SIZE)
        pool[b, 0, r] = k[t]
        pool[b, 1, r] = v[t]
    return pool


def decode_advance(block_tables, seq_lens, num_blocks):
    """Metadata of a decode step in which every segment gains one token
    ([NOTES01] sections 1.4 and 1.6).  The new token of segment s sits at
    position L = seq_lens[s]; returns (seq_lens + 1, cu_seqlens_q = 0..S,
    slot_mapping) with slot = table[s][L // 16] * 16 + L % 16, or -1 when
    that entry is past the table or outside [0, num_blocks)."""
    tables = np.asarray(block_tables, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    s_count, width = tables.shape
    slots = []
    for s in range(s_count):
        pos = int(lens[s])
        slot = -1
        if 0 <= pos and pos // BLOCK_SIZE < width:
            b = int(tables[s, pos // BLOCK_SIZE])
            if 0 <= b < num_blocks:
                slot = b * BLOCK_SIZE + pos % BLOCK_SIZE
        slots.append(slot)
    return ((lens + 1).astype(np.int32), np.arange(s_count + 1, dtype=np.int32),
            np.array(slots, dtype=np.int32))


def gather(pool, table_row, length):
    """Contiguous K, V (uint16 [L, Hkv, D]) of one request from its blocks.

    Only the first ceil(L / 16) table entries and the first L slots are
    touched ([NOTES01] section 1.5).
    """
    nb = -(-int(length) // BLOCK_SIZE)
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    if ids.size != nb:
        raise ValueError("block table shorter than the sequence")
    if nb and (ids.min() < 0 or ids.max() >= pool.shape[0]):
        raise ValueError("block id outside the pool")
    hkv, d = pool.shape[3], pool.shape[4]
    k = pool[ids, 0].reshape(nb * BLOCK_SIZE, hkv, d)[:length]
    v = pool[ids, 1].reshape(nb * BLOCK_SIZE, hkv, d)[:length]
    return k, v


def attend_dense(q, k, v, scale, history, max_elems=1 << 24):
    """Causal softmax attention of one segment over contiguous K/V, in fp64.

    q: float64 [n, Hq, D]; k, v: float64 [L, Hkv, D] with L = history + n;
    scale: the float32 softmax scale.  Query i may use key j iff
    j <= history + i.  Returns float64 [n, Hq, D].  Rows are processed in
    slices only to bound memory; each row is computed on its own.
    """
    n, hq, d = q.shape
    length, hkv, _ = k.shape
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    if length != history + n:
        raise ValueError("L must equal history + new tokens")
    group = hq // hkv
    sc = np.float64(np.float32(scale))
    out = np.empty((n, hq, d), dtype=np.float64)
    keys = np.arange(length)
    row_tile = max(1, max_elems // max(1, group * length))
    for g in range(hkv):
        kg = np.ascontiguousarray(k[:, g, :])        # [L, D]
        vg = np.ascontiguousarray(v[:, g, :])        # [L, D]
        for i0 in range(0, n, row_tile):
            i1 = min(n, i0 + row_tile)
            r = i1 - i0
            qg = q[i0:i1, g * group:(g + 1) * group, :].reshape(r * group, d)
            x = (sc * (qg @ kg.T)).reshape(r, group, length)        # logits
            allowed = keys[None, :] <= (history + np.arange(i0, i1))[:, None]
            x = np.where(allowed[:, None, :], x, -np.inf)
            m = x.max(axis=2, keepdims=True)
            w = np.exp(x - m)
            num = (w.reshape(r * group, length) @ vg).reshape(r, group, d)
            out[i0:i1, g * group:(g + 1) * group, :] = num / w.sum(axis=2)[..., None]
    return out


def attend(q, pool, block_tables, cu_seqlens_q, seq_lens, scale):
    """Paged attention over a packed batch, in fp64.

    q: uint16 [T, Hq, D] (bf16 bits); pool: uint16 [NB, 2, 16, Hkv, D];
    block_tables: int [S, W]; cu_seqlens_q: int [S+1]; seq_lens: int [S].
    Returns float64 [T, Hq, D]; rows of no segment stay zero.
    """
    from .bf16 import to_f64

    q = np.asarray(q)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    t_total = q.shape[0]
    if cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] > t_total:
        raise ValueError("cu_seqlens_q must start at 0, not decrease and stay within q")
    out = np.zeros(q.shape, dtype=np.float64)
    for s in range(lens.shape[0]):
        n = int(cu[s + 1] - cu[s])
        length = int(lens[s])
        if not 0 <= n <= length:
            raise ValueError("each segment needs 0 <= new tokens <= seq_len")
        if n == 0:
            continue
        k, v = gather(pool, block_tables[s], length)
        out[cu[s]:cu[s + 1]] = attend_dense(
            to_f64(q[cu[s]:cu[s + 1]]), to_f64(k), to_f64(v), scale, length - n)
    return out
