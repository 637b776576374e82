"""Shared-prefix groups: consecutive single-token decode segments whose
leading full partitions list the same blocks read those partitions once per
group instead of once per segment.

Each case runs the same step three ways -- groups of the automatic size,
groups capped at three members, no groups -- and checks that:
* the outputs are bitwise the same (a row's MFMA products and softmax do not
  depend on the other rows of its tile, and a group reads the keys in the
  order the segment's own item would);
* the number of group items and of ordinary decode items the plan kernel
  made (read from the workspace header) equal what a plain Python model of
  the grouping rule gives;
* the output matches the CPU oracle within the parity bound.
Random sharing patterns (runs, prefix depths, copied blocks, segments of 0
or 2 new tokens, short contexts) are checked the same way.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_469_amd as pkv
import workloads
from gpu_harness import DeviceStep, check_close, down_u16, log, up
from oracle import bf16, paged
from workloads.synth import build

pytestmark = pytest.mark.gpu


def _expected(wl, part, members, limit=1024):
    """(group items, ordinary decode items) of the grouping rule: the
    segments with one new token, more than one partition and a valid first
    block id, sorted by (first block id, index); neighbours in that order
    link while their leading full partitions start and end with the same
    block ids;
    runs of links are cut into groups of `members`, and a group of two or
    more covers the partitions every neighbouring pair in it links.  Only
    the first `limit` segments are grouped.  (The decode kernel then compares
    each grouped partition's ids whole.)"""
    cu, lens, tables = wl.cu_seqlens_q, wl.seq_lens, wl.block_tables
    n = np.diff(cu)
    s_count = len(lens)
    npb = part // 16
    order = sorted((s for s in range(min(s_count, limit))
                    if n[s] == 1 and lens[s] > part and tables[s, 0] >= 0),
                   key=lambda s: (int(tables[s, 0]), s))
    link = [0] * len(order)
    for r in range(1, len(order)):
        a, b = order[r], order[r - 1]
        if tables[a, 0] == tables[b, 0]:
            full = min(lens[a], lens[b]) // part
            c = 0
            while (c < full and tables[a, c * npb] == tables[b, c * npb]
                   and tables[a, c * npb + npb - 1] == tables[b, c * npb + npb - 1]):
                c += 1
            link[r] = c
    cov = [0] * s_count
    groups = 0
    r = 0
    while r < len(order):
        e = r + 1
        while e < len(order) and link[e] > 0:
            e += 1
        for c0 in range(r, e, members):
            mem = list(range(c0, min(c0 + members, e)))
            if len(mem) >= 2:
                cnt = min(link[m] for m in mem[1:])
                groups += cnt
                for m in mem:
                    cov[order[m]] = cnt
        r = e
    max_n = min(8, 32 // (wl.num_q_heads // wl.num_kv_heads))
    items = sum(-(-int(lens[s]) // part) - cov[s] for s in range(s_count) if 1 <= n[s] <= max_n)
    return groups, items


def _header(ws):
    h = ws[:64].view(torch.int32).cpu().numpy()
    return int(h[12]), int(h[1])   # n_group, n_decode


def _run(st, members):
    pkv.paged_attention_set_group_members(members)
    try:
        out = st.attend()
    finally:
        pkv.paged_attention_set_group_members(0)
    return down_u16(out), _header(st.ws)


def _mixed_runs():
    """Sharers broken into runs by a 2-token segment and by a short decode of
    another request; a prefill chunk at the end."""
    rng = np.random.default_rng([469, 70, 0])
    segs, rids, sharers = [], [], []
    for kind, count in (("d", 5), ("spec", 1), ("d", 4), ("short", 1), ("d", 3), ("chunk", 1)):
        for _ in range(count):
            r = len(segs)
            if kind == "d":
                segs.append((1, int(rng.integers(1100, 2600))))
                sharers.append(r)
            elif kind == "spec":
                segs.append((2, int(rng.integers(1100, 2600))))
                sharers.append(r)
            elif kind == "short":
                segs.append((1, 200))
            else:
                segs.append((300, 1000))
            rids.append(r)
    return build("mixed_runs", 4, 32, 8, 128, segs, request_ids=rids, shared_prefix=1024,
                 shared_requests=tuple(sharers), num_blocks=2000)


CASES = {
    # 8B-shaped continuous-batching step: 19 sharers (groups of 8, 8, 3)
    "cb_8b_p256": (lambda: workloads.make("cb_step_8b", num_decodes=40, ctx=(1100, 3000), shared=19,
                                          prefix=1024, chunk=300, chunk_history=700), 256, None),
    "cb_8b_p1024": (lambda: workloads.make("cb_step_8b", num_decodes=30, ctx=(1100, 3000), shared=12,
                                           prefix=1024, chunk=300, chunk_history=700), 1024, None),
    # 70B-shaped heads (G = 8: groups of 4)
    "g8_70b": (lambda: build("g8_70b", 5, 64, 8, 128, [(1, 2100 + 37 * i) for i in range(11)],
                             shared_prefix=2048, shared_requests=tuple(range(9))), 512, None),
    # G = 1, head_dim 64: eight members in one column tile
    "g1_d64": (lambda: build("g1_d64", 4, 8, 8, 64, [(1, 700 + 13 * i) for i in range(12)],
                             shared_prefix=512, shared_requests=tuple(range(12))), 128, None),
    # G = 16: groups of two
    "g16": (lambda: build("g16", 4, 32, 2, 128, [(1, 600 + 5 * i) for i in range(7)],
                          shared_prefix=512, shared_requests=tuple(range(7))), 256, None),
    # sharers interleaved with other requests (every third segment shares)
    "interleaved": (lambda: build("interleaved", 4, 32, 8, 128, [(1, 1100 + 29 * i) for i in range(30)],
                                  shared_prefix=1024, shared_requests=tuple(range(0, 30, 3))), 256, None),
    # 1100 segments: every fifth shares, on both sides of segment 1024 (only
    # the first 1024 segments are grouped)
    "big_batch": (lambda: build("big_batch", 4, 8, 2, 64, [(1, 140 + (37 * i) % 160) for i in range(1100)],
                                shared_prefix=128, shared_requests=tuple(range(0, 1100, 5))), 64, None),
    # a shared prefix of 20 partitions: the plan compares 8 per round
    "long_prefix": (lambda: build("long_prefix", 2, 32, 8, 128, [(1, 2600 + 41 * i) for i in range(10)],
                                  shared_prefix=2560, shared_requests=tuple(range(10))), 128, None),
    # exactly 8 shared partitions and 8 full ones per member: a round boundary
    "round_edge": (lambda: build("round_edge", 2, 32, 8, 128, [(1, 1030 + 11 * i) for i in range(9)],
                                 shared_prefix=1024, shared_requests=tuple(range(9))), 128, None),
    # runs broken by a non-member; two members whose third partition holds a
    # copy of a shared block (same data, another id): at the partition's
    # first entry (the plan's links stop there) and inside it (the decode
    # kernel finds it and computes that member's partition on its own)
    "mixed_runs": (_mixed_runs, 256, [(11, 2 * 16), (7, 2 * 16 + 3)]),
    # a shared prefix that ends inside a partition (1024 tokens at P = 2048):
    # no partition is shared whole, so no group forms and each segment reads
    # its own (the plan compares a partition's last id too)
    "prefix_inside": (lambda: build("prefix_inside", 2, 32, 8, 128, [(1, 4200 + 97 * i) for i in range(9)],
                                    shared_prefix=1024, shared_requests=tuple(range(9))), 2048, None),
    # partitions of 2048 keys (128 blocks, two ids per lane): two shared
    # partitions; in the second case one member's entry 69 (upper half of the
    # first partition) points at a copy, which only the second id of a lane
    # reveals
    "p2048": (lambda: build("p2048", 2, 32, 8, 128, [(1, 4200 + 97 * i) for i in range(9)],
                            shared_prefix=4096, shared_requests=tuple(range(9))), 2048, None),
    "p2048_copy": (lambda: build("p2048_copy", 2, 32, 8, 128, [(1, 4200 + 97 * i) for i in range(9)],
                                 shared_prefix=4096, shared_requests=tuple(range(9)), num_blocks=2400),
                   2048, [(3, 69)]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_groups_bitwise_and_parity(name):
    make, part, copy = CASES[name]
    wl = make()
    st = DeviceStep(wl, host_pool=True)
    for s, idx in copy or []:   # point a member's table entry at a copy of its block
        used = set(int(x) for x in wl.block_tables[wl.block_tables >= 0].ravel())
        spare = next(b for b in range(wl.num_blocks) if b not in used)
        src = int(wl.block_tables[s, idx])
        st.pool[spare].copy_(st.pool[src])
        st.host[spare] = st.host[src]
        wl.block_tables[s, idx] = spare
        st.bt = torch.from_numpy(wl.block_tables).cuda()
    group = wl.num_q_heads // wl.num_kv_heads
    auto = min(8, 32 // group)
    log(f"case groups {name}: S={wl.num_seqs} T={wl.num_tokens} G={group} P={part}")
    pkv.paged_attention_set_partition_tokens(part)
    try:
        runs = {m: _run(st, m) for m in (0, 3, 1)}
    finally:
        pkv.paged_attention_set_partition_tokens(0)
    for m, (out, (n_group, n_decode)) in runs.items():
        want = _expected(wl, part, auto if m == 0 else min(auto, m))
        log(f"  members {m}: {n_group} group items, {n_decode} decode items (expected {want})")
        assert (n_group, n_decode) == want, f"members {m}"
        assert np.array_equal(out, runs[1][0]), f"members {m}: output differs from the ungrouped run"
    if name == "prefix_inside":
        assert runs[0][1][0] == 0, "a prefix that ends inside a partition must not group it"
    else:
        assert runs[0][1][0] > 0, "the case must form groups"
    assert pkv.paged_attention_device_status(st.ws) == 0
    ref = paged.attend(st.q_host, st.host, wl.block_tables, wl.cu_seqlens_q, wl.seq_lens, wl.scale)
    check_close(runs[0][0], ref, f"groups {name}")


def _random_step(seed, hq=32, hkv=8, d=128, part=128, shuffle=False):
    """Random sharing: runs of segments share a random number of leading
    blocks; some entries point at copies of the shared block (same data,
    another id); some segments have 0 or 2 new tokens or a short context.
    With ``shuffle`` the segments are packed in a random order, so requests
    that share a prefix are interleaved with others."""
    from types import SimpleNamespace
    rng = np.random.default_rng([469, 71, seed])
    s_count = int(rng.integers(20, 40))
    n = rng.choice([1, 1, 1, 1, 1, 1, 0, 2], size=s_count)
    lens = rng.integers(part // 2, 6 * part, size=s_count)
    lens = np.maximum(lens, n).astype(np.int32)
    width = int(-(-lens.max() // 16))
    tables = np.full((s_count, width), -1, dtype=np.int32)
    next_id = 0
    prefix = []
    copies = []   # (copy id, original id)
    for s in range(s_count):
        nblk = -(-int(lens[s]) // 16)
        if rng.random() < 0.25 or not prefix:   # a new run with a fresh shared prefix
            prefix = list(range(next_id, next_id + int(rng.integers(1, 30))))
            next_id += len(prefix)
        k = min(len(prefix), nblk)
        row = prefix[:k] + list(range(next_id, next_id + nblk - k))
        next_id += nblk - k
        for _ in range(int(rng.integers(0, 2))):   # a copied entry inside the shared part
            if k:
                i = int(rng.integers(0, k))
                copies.append((next_id, row[i]))
                row[i] = next_id
                next_id += 1
        tables[s, :nblk] = row
    if shuffle:
        perm = rng.permutation(s_count)
        n, lens, tables = n[perm], lens[perm], tables[perm]
    nb = next_id
    pool = bf16.f32_to_bf16(rng.standard_normal((nb, 2, 16, hkv, d)).astype(np.float32))
    for c, o in copies:
        pool[c] = pool[o]
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    q = bf16.f32_to_bf16(rng.standard_normal((int(cu[-1]), hq, d)).astype(np.float32))
    wl = SimpleNamespace(cu_seqlens_q=cu, seq_lens=lens, block_tables=tables, num_q_heads=hq,
                         num_kv_heads=hkv, scale=float(np.float32(1 / np.sqrt(d))))
    return wl, pool, q, part


@pytest.mark.parametrize("seed", range(8))
def test_groups_random_tables(seed):
    wl, pool, q, part = _random_step(seed, shuffle=seed >= 4)
    s_count, t = len(wl.seq_lens), int(wl.cu_seqlens_q[-1])
    log(f"case groups random seed {seed}: S={s_count} T={t} NB={pool.shape[0]}")
    dev = {k: up(v) for k, v in (("pool", pool), ("q", q), ("bt", wl.block_tables),
                                   ("cu", wl.cu_seqlens_q), ("lens", wl.seq_lens))}
    ws = torch.empty(pkv.paged_attention_workspace_size(s_count, t, wl.num_q_heads, wl.num_kv_heads,
                                                        pool.shape[-1], wl.block_tables.shape[1]),
                     dtype=torch.uint8, device="cuda")
    auto = min(8, 32 // (wl.num_q_heads // wl.num_kv_heads))
    outs = {}
    pkv.paged_attention_set_partition_tokens(part)
    try:
        for m in (0, 3, 1):
            pkv.paged_attention_set_group_members(m)
            o = pkv.paged_attention(dev["q"], dev["pool"], dev["bt"], dev["cu"], dev["lens"], wl.scale,
                                    workspace=ws)
            torch.cuda.synchronize()
            outs[m] = (down_u16(o), _header(ws))
            assert pkv.paged_attention_device_status(ws) == 0
    finally:
        pkv.paged_attention_set_group_members(0)
        pkv.paged_attention_set_partition_tokens(0)
    for m, (out, counts) in outs.items():
        want = _expected(wl, part, auto if m == 0 else min(auto, m))
        log(f"  members {m}: {counts[0]} group items, {counts[1]} decode items (expected {want})")
        assert counts == want
        assert np.array_equal(out, outs[1][0]), f"members {m}: output differs from the ungrouped run"
    ref = paged.attend(q, pool, wl.block_tables, wl.cu_seqlens_q, wl.seq_lens, wl.scale)
    check_close(outs[0][0], ref, f"groups random seed {seed}")
