"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

KV writes are compared bit for bit with the oracle's write of the same
inputs; attention element by element within 2e-2 + 1e-2*|ref| plus the
relative-RMS gate (see gpu_harness).  Sizes: every workload at a reduced
size the oracle finishes in seconds (all rows checked, several tiles and
partitions, ragged tails), and at full size with sampled segments and rows.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_469_amd as pkv
import workloads
from gpu_harness import DeviceStep, check_close, down_u16, log, oracle_rows, up
from oracle import bf16, paged

pytestmark = pytest.mark.gpu

REDUCED = [
    ("tiny_mixed", {}),
    ("decode_8b", dict(num_requests=24)),
    ("prefill_8b", dict(num_prompts=4, lens=(200, 700))),
    ("cb_step_8b", dict(num_decodes=12, ctx=(1024, 3000), shared=4, prefix=1024, chunk=300,
                        chunk_history=700)),
    ("cb_step_8b", dict(num_decodes=12, ctx=(1024, 3000), shared=4, prefix=1024, chunk=300,
                        chunk_history=700, decode_first=False)),
    ("long_decode_70b", dict(num_requests=3, ctx=(4000, 20000))),
]


@pytest.mark.parametrize("name,kw", REDUCED, ids=[f"{n}-{i}" for i, (n, _) in enumerate(REDUCED)])
def test_reduced_full_check(name, kw):
    wl = workloads.make(name, **kw)
    log(f"case {name} {kw}: S={wl.num_seqs} T={wl.num_tokens} NB={wl.num_blocks}")
    st = DeviceStep(wl, host_pool=True)
    out = st.attend()
    assert np.array_equal(down_u16(st.pool), st.host), "KV pool differs from the oracle's write"
    ref = paged.attend(st.q_host, st.host, wl.block_tables, wl.cu_seqlens_q, wl.seq_lens,
                       wl.scale)
    check_close(down_u16(out), ref, name)
    assert st.status() == 0


SHARP = [REDUCED[0], REDUCED[1], REDUCED[2], REDUCED[3], REDUCED[5]]


@pytest.mark.parametrize("name,kw", SHARP, ids=["tiny", "decode", "prefill", "cb", "long70b"])
def test_sharpened_queries(name, kw):
    # q x 4: logits with std 4, outputs O(0.1-1); correctness only
    wl = workloads.make(name, **kw)
    log(f"case sharpened {name}")
    st = DeviceStep(wl, q_gain=4.0)
    out = down_u16(st.attend())
    refs = oracle_rows(wl, st.q_host)
    rows = np.concatenate([r for r, _ in refs.values()])
    ref = np.concatenate([x for _, x in refs.values()])
    check_close(out[rows], ref, f"sharpened {name}")


def _custom(hq, hkv, d, segs, cfg=50, **kw):
    return workloads.build("custom", cfg, hq, hkv, d, segs, **kw)


EDGE = [
    ("mha_d64", dict(hq=8, hkv=8, d=64, segs=[(1, 1), (1, 16), (1, 17), (5, 5), (0, 9), (33, 80)])),
    ("g2_d128", dict(hq=16, hkv=8, d=128, segs=[(2, 2), (1, 1024), (1, 1025), (64, 64), (3, 700)])),
    ("g3_d128", dict(hq=6, hkv=2, d=128, segs=[(1, 300), (17, 17), (100, 260)])),
    ("g8_d64", dict(hq=32, hkv=4, d=64, segs=[(6, 6), (1, 38), (40, 40), (1, 2049)])),
    ("g16_d128", dict(hq=32, hkv=2, d=128, segs=[(1, 513), (70, 100)])),
    ("zero_len_segments", dict(hq=32, hkv=8, d=128, segs=[(0, 0), (1, 33), (0, 40), (7, 7)])),
    ("block_multiples", dict(hq=32, hkv=8, d=128, segs=[(1, 16), (1, 32), (1, 1024), (16, 16), (64, 128)])),
    # a few new tokens at the end of a long history (a speculative-decoding
    # verify step): n = 2..8, beside single-token decodes
    ("short_chunks", dict(hq=32, hkv=8, d=128, segs=[(2, 3001), (4, 5003), (1, 4000), (5, 1237),
                                                     (8, 8200), (3, 67)])),
]


@pytest.mark.parametrize("name,kw", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes(name, kw):
    wl = _custom(kw["hq"], kw["hkv"], kw["d"], kw["segs"], num_blocks=None)
    log(f"case edge {name}")
    st = DeviceStep(wl, host_pool=True)
    sentinel = torch.full((wl.num_tokens, wl.num_q_heads, wl.head_dim), 7.0,
                          dtype=torch.bfloat16, device="cuda")
    out = down_u16(st.attend(out=sentinel))
    assert np.array_equal(down_u16(st.pool), st.host)
    ref = paged.attend(st.q_host, st.host, wl.block_tables, wl.cu_seqlens_q, wl.seq_lens,
                       wl.scale)
    check_close(out, ref, name)


@pytest.mark.parametrize("tokens", [32, 64, 256, 1024, 2048])
def test_partition_sizes(tokens):
    wl = workloads.make("long_decode_70b", num_requests=3, ctx=(3000, 9000))
    log(f"case partition {tokens}")
    pkv.paged_attention_set_partition_tokens(tokens)
    try:
        st = DeviceStep(wl)
        out = down_u16(st.attend())
    finally:
        pkv.paged_attention_set_partition_tokens(0)
    refs = oracle_rows(wl, st.q_host)
    rows = np.concatenate([r for r, _ in refs.values()])
    check_close(out[rows], np.concatenate([x for _, x in refs.values()]), f"P={tokens}")


# Segments of a few new tokens over a history (one decode step, or a
# speculative-decoding check of n - 1 drafted tokens) take the split-context
# decode path when n * G <= 32 and n <= 8 (one or two column tiles of 16
# query rows), beside longer segments on the prefill path.  Small partitions give many partials per token, including
# last partitions none of whose keys some of the segment's tokens see.
MULTI = [
    ("g4_d128", dict(hq=32, hkv=8, d=128, segs=[(1, 97), (2, 2), (2, 1025), (3, 67), (4, 4),
                                               (4, 4097), (4, 3001), (3, 2050), (5, 700)])),
    ("g1_d64", dict(hq=8, hkv=8, d=64, segs=[(8, 8), (8, 2000), (7, 333), (6, 1024), (1, 1),
                                            (9, 40)])),
    ("g2_d128", dict(hq=16, hkv=8, d=128, segs=[(8, 1500), (2, 2), (5, 4100), (9, 9)])),
    ("g8_d64", dict(hq=32, hkv=4, d=64, segs=[(2, 2), (2, 3333), (1, 50), (3, 600)])),
    ("g3_d128", dict(hq=6, hkv=2, d=128, segs=[(5, 800), (4, 4), (2, 2049), (6, 90)])),
    # two column tiles of 16 rows: n * G in 17 .. 32
    ("g8_d128_70b", dict(hq=64, hkv=8, d=128, segs=[(4, 5000), (3, 2049), (2, 17), (4, 4),
                                                    (1, 3000), (5, 900)])),
    ("g4_d128_long", dict(hq=32, hkv=8, d=128, segs=[(8, 4100), (6, 2500), (7, 33), (8, 8),
                                                     (9, 300)])),
]


@pytest.mark.parametrize("tokens", [32, 256, 2048, 0])
@pytest.mark.parametrize("name,kw", MULTI, ids=[m[0] for m in MULTI])
def test_multi_token_decode(name, kw, tokens):
    wl = _custom(kw["hq"], kw["hkv"], kw["d"], kw["segs"], cfg=51, num_blocks=None)
    log(f"case multi-token decode {name} P={tokens}")
    pkv.paged_attention_set_partition_tokens(tokens)
    try:
        st = DeviceStep(wl, host_pool=True)
        out = down_u16(st.attend())
    finally:
        pkv.paged_attention_set_partition_tokens(0)
    ref = paged.attend(st.q_host, st.host, wl.block_tables, wl.cu_seqlens_q, wl.seq_lens,
                       wl.scale)
    check_close(out, ref, f"{name} P={tokens}")
    assert st.status() == 0


def test_multi_token_decode_sharpened():
    kw = MULTI[0][1]
    wl = _custom(kw["hq"], kw["hkv"], kw["d"], kw["segs"], cfg=51, num_blocks=None)
    log("case multi-token decode sharpened")
    pkv.paged_attention_set_partition_tokens(64)
    try:
        st = DeviceStep(wl, host_pool=True, q_gain=4.0)
        out = down_u16(st.attend())
    finally:
        pkv.paged_attention_set_partition_tokens(0)
    ref = paged.attend(st.q_host, st.host, wl.block_tables, wl.cu_seqlens_q, wl.seq_lens,
                       wl.scale)
    check_close(out, ref, "multi-token sharpened")


def test_running_maximum_jumps():
    # keys whose scores sit far above everything before them (by 17 and 58
    # log2 units, a third and nine tenths of the way through each sequence):
    # the lazy running maximum of both kernels has to move late in an item and
    # rescale O and l there (decode, a speculative check and a prompt)
    segs = [(1, 3000), (1, 5000), (4, 4100), (1, 700), (100, 400)]
    wl = _custom(32, 8, 128, segs, cfg=52, num_blocks=None)
    log("case running maximum jumps")
    st = DeviceStep(wl, host_pool=True)
    cu, lens, bt, g_ = wl.cu_seqlens_q, wl.seq_lens, wl.block_tables, wl.group
    qf = bf16.to_f64(st.q_host)
    pool16 = st.pool.view(torch.int16)
    for s in range(wl.num_seqs):
        length, tok = int(lens[s]), int(cu[s + 1]) - 1   # the segment's last query sees every key
        for frac, target in ((0.3, 12.0), (0.9, 40.0)):
            pos = int(frac * (length - 1))
            blk, row = int(bt[s, pos // 16]), pos % 16
            for g in range(wl.num_kv_heads):
                qv = qf[tok, g * g_]
                bits = bf16.from_f64(qv * (target / (wl.scale * float(qv @ qv))))   # logit = target
                st.host[blk, 0, row, g] = bits
                pool16[blk, 0, row, g] = torch.from_numpy(bits.view(np.int16)).cuda()
    ref = paged.attend(st.q_host, st.host, bt, cu, lens, wl.scale)
    for tokens in (0, 256):
        pkv.paged_attention_set_partition_tokens(tokens)
        try:
            out = down_u16(st.attend())
        finally:
            pkv.paged_attention_set_partition_tokens(0)
        check_close(out, ref, f"maximum jumps P={tokens}")
    assert st.status() == 0


def test_more_than_1024_segments():
    # the plan kernel walks segments in chunks of 1024 threads: decode items,
    # partial rows and prefill items of later chunks take its second path
    rng = np.random.default_rng([469, 52, 0])
    segs = []
    for i in range(1100):
        if i in (3, 700, 1030, 1090):
            n = int(rng.integers(65, 200))
            segs.append((n, n + int(rng.integers(0, 100))))
        elif i % 97 == 5:
            segs.append((int(rng.integers(2, 5)), int(rng.integers(40, 300))))
        else:
            segs.append((1, int(rng.integers(1, 120))))
    wl = _custom(32, 8, 128, segs, cfg=53, num_blocks=None)
    log(f"case 1100 segments: T={wl.num_tokens} NB={wl.num_blocks}")
    pkv.paged_attention_set_partition_tokens(64)   # several partitions per longer decode
    try:
        st = DeviceStep(wl, host_pool=True)
        out = down_u16(st.attend())
    finally:
        pkv.paged_attention_set_partition_tokens(0)
    assert np.array_equal(down_u16(st.pool), st.host)
    ref = paged.attend(st.q_host, st.host, wl.block_tables, wl.cu_seqlens_q, wl.seq_lens,
                       wl.scale)
    check_close(out, ref, "1100 segments")
    assert st.status() == 0


def test_permutation_invariance_and_determinism():
    kw = dict(num_decodes=10, ctx=(1024, 2500), shared=3, prefix=1024, chunk=130, chunk_history=300)
    a = workloads.make("cb_step_8b", **kw)
    b = workloads.make("cb_step_8b", num_blocks=a.num_blocks * 3, **kw)   # other placement
    log("case permutation/determinism")
    sa, sb = DeviceStep(a), DeviceStep(b)
    oa1 = down_u16(sa.attend())
    oa2 = down_u16(sa.attend())
    ob = down_u16(sb.attend())
    assert np.array_equal(oa1, oa2), "repeat run is not bitwise identical"
    same = np.array_equal(oa1, ob)
    log(f"  permuted pool bitwise identical: {same}")
    refs = oracle_rows(b, sb.q_host)
    rows = np.concatenate([r for r, _ in refs.values()])
    check_close(ob[rows], np.concatenate([x for _, x in refs.values()]), "permuted")


def test_write_strided_and_unaligned():
    rng = np.random.default_rng(3)
    t, hkv, d, nb = 37, 8, 128, 20
    slots = rng.choice(nb * 16, size=t, replace=False).astype(np.int32)
    slots[[2, 9]] = -1
    host = np.full((nb, 2, 16, hkv, d), 0x7FC1, dtype=np.uint16)
    for width in (hkv * d * 3, hkv * d + 4):    # 16-byte aligned stride, then not
        log(f"case write stride {width}")
        buf = rng.integers(0, 1 << 16, (t, width)).astype(np.uint16)
        dev = up(buf)
        k = dev[:, :hkv * d].view(t, hkv, d)
        v = dev[:, width - hkv * d:].view(t, hkv, d)
        pool = torch.empty((nb, 2, 16, hkv, d), dtype=torch.bfloat16, device="cuda")
        pool.view(torch.int16).fill_(0x7FC1)
        pkv.paged_kv_write(k, v, up(slots), pool)
        torch.cuda.synchronize()
        want = host.copy()
        paged.kv_write(buf[:, :hkv * d].reshape(t, hkv, d), buf[:, width - hkv * d:].reshape(t, hkv, d),
                       slots, want)
        assert np.array_equal(down_u16(pool), want)


def test_bad_metadata_is_skipped_and_flagged():
    wl = _custom(32, 8, 128, [(1, 100), (1, 200), (4, 50)], cfg=51)
    log("case bad metadata")
    st = DeviceStep(wl)
    good = down_u16(st.attend())
    bt = wl.block_tables.copy()
    bt[1, 3] = wl.num_blocks + 1000                      # outside the pool
    st.bt = up(bt)
    out = down_u16(st.attend())
    assert st.status() & pkv.STATUS_BAD_BLOCK
    assert np.array_equal(out[0], good[0]) and np.array_equal(out[2:], good[2:])
    st.bt = up(wl.block_tables)
    lens = wl.seq_lens.copy()
    lens[0] = wl.max_blocks_per_seq * 16 + 5             # longer than its table
    st.lens = up(lens)
    out = down_u16(st.attend())
    assert st.status() & pkv.STATUS_BAD_SEGMENT
    assert np.array_equal(out[1:], good[1:])
    with pytest.raises(pkv.PagedError):
        pkv.paged_validate(None, st.bt, st.cu, st.lens, wl.num_tokens, wl.num_blocks)
    st.lens = up(wl.seq_lens)
    pkv.paged_validate(st.slots, st.bt, st.cu, st.lens, wl.num_tokens, wl.num_blocks)
    dup = up(np.array([5, 5], dtype=np.int32))
    with pytest.raises(pkv.PagedError, match="twice"):
        pkv.paged_validate(dup, None, None, None, 0, wl.num_blocks)


def test_overlapping_segments_are_dropped_and_flagged():
    # cu_seqlens_q = [0, T, 0, T, ..., T - 1, T]: the even segments each claim
    # all T rows (malformed: the odd ones run backwards), so their prefill
    # items (T / 32 each at G = 8) add up to far more than the list holds
    # (and past 2^20).  The plan must flag the batch and drop every prefill
    # item without writing outside its lists; the last segment, a well-formed
    # single-token decode, is still computed.
    t, hq, hkv, d = 1 << 17, 8, 1, 64
    s_total = 1024
    w = t // 16
    nb = w + 8
    log(f"case overlapping segments: S={s_total} T={t}")
    cu = np.zeros(s_total + 1, dtype=np.int32)
    cu[1:-1] = np.where(np.arange(1, s_total) % 2 == 1, t, 0)
    cu[-2], cu[-1] = t - 1, t
    lens = np.full(s_total, t, dtype=np.int32)
    lens[-1] = 100
    bt = np.tile(np.arange(w, dtype=np.int32), (s_total, 1))
    rng = np.random.default_rng([469, 54])

    def normal_bf16(shape):
        x = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16)
        return x.view(torch.int16).numpy().view(np.uint16)

    k, v = normal_bf16((100, hkv, d)), normal_bf16((100, hkv, d))
    pool = torch.zeros((nb, 2, 16, hkv, d), dtype=torch.bfloat16, device="cuda")
    pkv.paged_kv_write(up(k), up(v), up(np.arange(100, dtype=np.int32)), pool)
    q_host = normal_bf16((t, hq, d))
    out = torch.full((t, hq, d), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(pkv.paged_attention_workspace_size(s_total, t, hq, hkv, d, w),
                     dtype=torch.uint8, device="cuda")
    pkv.paged_attention(up(q_host), pool, up(bt), up(cu), up(lens), 0.125, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert pkv.paged_attention_device_status(ws) & pkv.STATUS_BAD_SEGMENT
    got = down_u16(out)
    sentinel = np.full((hq, d), 0x40E0, dtype=np.uint16)   # bf16 7.0
    assert (got[:t - 1] == sentinel).all(), "a dropped prefill item wrote output rows"
    ref = paged.attend_dense(bf16.to_f64(q_host[t - 1:t]), bf16.to_f64(k), bf16.to_f64(v),
                             0.125, 99)
    check_close(got[t - 1:t], ref, "decode segment beside overlapping ones")


# ------------------------------------------------------------------ full size

def _full_sampled(wl, sample_segments, rows_per_segment=None, pool_blocks=None, fill_others=False,
                  ungrouped_equal=False, all_rows=()):
    """Full-size workload.  Each request's K/V is written with one
    paged_kv_write call over all its positions (the step's write order is
    covered by the reduced cases).  With ``fill_others`` only the sampled
    segments' values come from the host generator; the others are drawn on
    the GPU (seeded) and are not compared.  With ``ungrouped_equal`` the step
    is run again without shared-prefix groups and the whole output must be
    bitwise the same.  Segments in ``all_rows`` are compared on every row."""
    torch.cuda.empty_cache()
    hkv, d = wl.num_kv_heads, wl.head_dim
    nb = wl.num_blocks if pool_blocks is None else pool_blocks
    pool = torch.empty((nb, 2, 16, hkv, d), dtype=torch.bfloat16, device="cuda")
    pool.view(torch.int16).fill_(0x7FC1)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(469)
    sample = set(int(s) for s in sample_segments)
    for s in range(wl.num_seqs):
        length = int(wl.seq_lens[s])
        slots = up(wl.slots_of(s, 0, length))
        if s in sample or not fill_others:
            k, v = wl.request_kv(s)
            pkv.paged_kv_write(up(k), up(v), slots, pool)
        else:
            kv = torch.randn((2, length, hkv, d), generator=gen, device="cuda").to(torch.bfloat16)
            pkv.paged_kv_write(kv[0], kv[1], slots, pool)
            del kv
    q_host = wl.q()
    ws = torch.empty(pkv.paged_attention_workspace_size(
        wl.num_seqs, wl.num_tokens, wl.num_q_heads, hkv, d, wl.max_blocks_per_seq),
        dtype=torch.uint8, device="cuda")
    out = pkv.paged_attention(up(q_host), pool, up(wl.block_tables), up(wl.cu_seqlens_q),
                              up(wl.seq_lens), wl.scale, workspace=ws)
    torch.cuda.synchronize()
    assert pkv.paged_attention_device_status(ws) == 0
    if ungrouped_equal:
        pkv.paged_attention_set_group_members(1)
        try:
            again = pkv.paged_attention(up(q_host), pool, up(wl.block_tables), up(wl.cu_seqlens_q),
                                        up(wl.seq_lens), wl.scale, workspace=ws)
            torch.cuda.synchronize()
        finally:
            pkv.paged_attention_set_group_members(0)
        assert torch.equal(again.view(torch.int16), out.view(torch.int16)), "groups change the output"
    # write check on the sampled requests: their blocks hold exactly their K/V
    for s in sample:
        length = int(wl.seq_lens[s])
        ids = torch.from_numpy(wl.block_tables[s][:(length + 15) // 16].astype(np.int64)).cuda()
        blocks = pool.index_select(0, ids)
        got = blocks.view(torch.int16).cpu().numpy().view(np.uint16)
        gk = got[:, 0].reshape(-1, hkv, d)[:length]
        gv = got[:, 1].reshape(-1, hkv, d)[:length]
        rk, rv = wl.request_kv(s)
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv), f"segment {s} blocks"
    full = set(int(s) for s in all_rows)
    refs = oracle_rows(wl, q_host, segments=sorted(sample - full), rows_per_segment=rows_per_segment,
                       rng=np.random.default_rng(1))
    refs.update(oracle_rows(wl, q_host, segments=sorted(full)))
    got = down_u16(out)
    rows = np.concatenate([r for r, _ in refs.values()])
    ref = np.concatenate([x for _, x in refs.values()])
    return got[rows], ref


def test_full_decode_8b():
    wl = workloads.make("decode_8b")
    log(f"case full decode_8b: KV {wl.kv_bytes_logical() / 1e9:.2f} GB")
    sample = np.random.default_rng(2).choice(wl.num_seqs, 12, replace=False)
    got, ref = _full_sampled(wl, sample)
    check_close(got, ref, "decode_8b full (12 sampled requests)")


def test_full_prefill_8b():
    wl = workloads.make("prefill_8b")
    log(f"case full prefill_8b: T={wl.num_tokens}")
    longest = int(np.argmax(wl.new_tokens))
    sample = sorted({0, 5, 9, 15, longest})
    got, ref = _full_sampled(wl, sample, rows_per_segment=24, all_rows=[longest])
    check_close(got, ref, f"prefill_8b full (segments {sample} x 26 rows, all "
                          f"{int(wl.new_tokens[longest])} rows of the longest, {longest})")


def test_full_cb_step_8b():
    wl = workloads.make("cb_step_8b")
    log(f"case full cb_step_8b: T={wl.num_tokens}")
    chunk = wl.num_seqs - 1
    # segments 0, 1 and 63 share the cached prefix: grouped (and the whole
    # output equals the ungrouped run's, bit for bit)
    got, ref = _full_sampled(wl, [0, 1, 63, 64, 150, chunk], rows_per_segment=24,
                             ungrouped_equal=True)
    check_close(got, ref, "cb_step_8b full (5 decodes + 26 chunk rows)")


def test_full_long_decode_70b():
    free, _ = torch.cuda.mem_get_info()
    nb = int(0.92 * (free - (4 << 30)) // 65536)
    wl = workloads.make("long_decode_70b", num_blocks=nb)
    log(f"case full long_decode_70b: pool {nb} blocks ({nb * 16} tokens), "
        f"KV {wl.kv_bytes_logical() / 1e9:.1f} GB")
    # the longest request has more than 64 partitions of 1024 keys, so its
    # merge takes the second pass of the lanes over the partitions
    longest = int(np.argmax(wl.seq_lens))
    assert wl.seq_lens[longest] > 64 * 1024
    sample = sorted({3, 40, longest})
    got, ref = _full_sampled(wl, sample, pool_blocks=nb, fill_others=True)
    check_close(got, ref, f"long_decode_70b full (requests {sample}; longest L = "
                          f"{int(wl.seq_lens[longest])})")


def test_full_spec_verify_8b():
    wl = workloads.make("spec_verify_8b")
    log(f"case full spec_verify_8b: KV {wl.kv_bytes_logical() / 1e9:.2f} GB")
    sample = np.random.default_rng(3).choice(wl.num_seqs, 8, replace=False)
    got, ref = _full_sampled(wl, sample, fill_others=True)
    check_close(got, ref, "spec_verify_8b full (8 sampled requests)")


def _random_batch(seed):
    """A seeded mixed batch: a head layout (G from 1 to 8, head size 64 or
    128) and 1-12 segments, each a single-token decode, a few-token verify
    (2-8 new tokens), an empty segment or a prompt chunk (9-259 new tokens),
    over a history of 0-2999 cached tokens."""
    rng = np.random.default_rng([469, 77, seed])
    layouts = [(8, 8, 64), (16, 8, 128), (32, 8, 128), (32, 4, 64), (64, 8, 128), (6, 2, 128),
               (32, 4, 128)]
    hq, hkv, d = layouts[int(rng.integers(len(layouts)))]
    segs = []
    for _ in range(int(rng.integers(1, 13))):
        kind = rng.choice(4, p=[0.5, 0.2, 0.05, 0.25])
        n = [1, int(rng.integers(2, 9)), 0, int(rng.integers(9, 260))][kind]
        segs.append((n, int(rng.integers(0, 3000)) + n))
    if all(n == 0 for n, _ in segs):
        segs[0] = (1, segs[0][1] + 1)
    return hq, hkv, d, segs


@pytest.mark.parametrize("seed", range(24))
def test_random_batches(seed):
    hq, hkv, d, segs = _random_batch(seed)
    wl = _custom(hq, hkv, d, segs, cfg=60 + seed)
    log(f"case random {seed}: heads {hq}/{hkv}, d {d}, (n, L) {segs}")
    st = DeviceStep(wl, host_pool=True)
    out = down_u16(st.attend())
    assert np.array_equal(down_u16(st.pool), st.host)
    ref = paged.attend(st.q_host, st.host, wl.block_tables, wl.cu_seqlens_q, wl.seq_lens, wl.scale)
    check_close(out, ref, f"random batch {seed}")
