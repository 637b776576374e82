"""Scalar pure-Python twin of the oracle's attention, for tiny inputs only.

TEST INFRASTRUCTURE ONLY.  Written independently of ``paged.attend``: nested
loops, ``math.exp`` and ``math.fsum``, lists instead of arrays, and its own
slot-to-(block, position) walk instead of a gathered copy.  It follows the
same statements of the pages (see ``oracle.paged``): segments packed end to
end and isolated, query i of a segment with history h sees keys 0 .. h + i,
KV head g serves query heads g*G .. g*G+G-1, scale given as float32.

Inputs are plain nested lists of floats (already widened from bf16) so that
nothing here depends on numpy.
"""

import math
import struct


def _f32(x):
    """Round a Python float to the nearest float32 value."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def attend(q, pool, block_tables, cu_seqlens_q, seq_lens, scale, block_size=16):
    """q[t][hq][d]; pool[b][kv][row][g][d]; returns out[t][hq][d] (floats)."""
    t_total = len(q)
    hq = len(q[0]) if t_total else 0
    hkv = len(pool[0][0][0]) if pool else 0
    d = len(q[0][0]) if t_total else 0
    group = hq // hkv if hkv else 0
    sc = _f32(scale)
    out = [[[0.0] * d for _ in range(hq)] for _ in range(t_total)]
    for s in range(len(seq_lens)):
        start, stop = cu_seqlens_q[s], cu_seqlens_q[s + 1]
        n = stop - start
        length = seq_lens[s]
        hist = length - n
        for i in range(n):
            for h in range(hq):
                g = h // group
                logits = []
                rows = []
                for j in range(hist + i + 1):
                    blk = block_tables[s][j // block_size]
                    pos = j % block_size
                    kvec = pool[blk][0][pos][g]
                    logits.append(sc * math.fsum(q[start + i][h][e] * kvec[e] for e in range(d)))
                    rows.append(pool[blk][1][pos][g])
                top = max(logits)
                w = [math.exp(x - top) for x in logits]
                den = math.fsum(w)
                for e in range(d):
                    out[start + i][h][e] = math.fsum(w[j] * rows[j][e] for j in range(len(w))) / den
    return out
