"""The block manager's step metadata driving the HIP path: a few steps of a
small engine loop (prompts that share a cached system prompt, one of them
chunked, then decode steps and a speculative-decoding check) run through
paged_kv_write and paged_attention on the GPU; the pool must equal the
oracle's write bit for bit and every output row the oracle's attention
within the parity bound."""

import numpy as np
import pytest
import torch

import paged_kv_cache_469_amd as pkv
from gpu_harness import check_close, down_u16, log, up
from oracle import bf16, paged
from oracle.block_manager import BlockManagerModel

pytestmark = pytest.mark.gpu


def test_engine_loop_through_block_manager():
    rng = np.random.default_rng([469, 64, 0])
    hq, hkv, d, nb, width = 32, 8, 128, 400, 160
    scale = float(np.float32(1 / np.sqrt(d)))
    bm, model = pkv.BlockManager(nb), BlockManagerModel(nb)
    pool = torch.empty((nb, 2, 16, hkv, d), dtype=torch.bfloat16, device="cuda")
    pool.view(torch.int16).fill_(0x7FC1)
    host = np.full(tuple(pool.shape), 0x7FC1, dtype=np.uint16)
    sys_prompt = [int(x) for x in rng.integers(0, 1000, size=600)]
    known = {r: sys_prompt + [int(x) for x in rng.integers(0, 1000, size=int(rng.integers(5, 400)))]
             for r in range(6)}
    for r, toks in known.items():
        bm.add_request(r, toks)
        model.add_request(r, toks)
    ws = None
    plan = [[(0, None), (1, 300)], [(1, None), (2, None), (3, None), (4, None), (5, None)],
            "decode", ("verify", 4), "decode"]
    for i, step in enumerate(plan):
        entries = []
        if step == "decode" or isinstance(step, tuple):
            n = 1 if step == "decode" else step[1]
            for r in known:
                t = [int(x) for x in rng.integers(0, 1000, size=n)]
                known[r] += t
                bm.append_tokens(r, t)
                model.append_tokens(r, t)
                a, b = bm.allocate_slots(r, n), model.allocate_slots(r, n)
                assert a is not None and a.tolist() == b
                entries.append((r, n))
        else:
            for r, n in step:
                # asked right before the request's allocation: requests
                # allocated earlier in the step may have cached its prefix
                left = len(known[r]) - bm.num_cached_tokens(r)
                n = left if n is None else min(n, left)
                a, b = bm.allocate_slots(r, n), model.allocate_slots(r, n)
                assert a is not None and a.tolist() == b
                entries.append((r, n))
        reqs = [r for r, _ in entries]
        news = [n for _, n in entries]
        tables, cu, lens, slots = bm.step_metadata(reqs, news, width)
        t = int(cu[-1])
        log(f"case engine step {i}: S={len(reqs)} T={t} L={lens.tolist()}")
        k = bf16.f32_to_bf16(rng.standard_normal((t, hkv, d)).astype(np.float32))
        v = bf16.f32_to_bf16(rng.standard_normal((t, hkv, d)).astype(np.float32))
        q = bf16.f32_to_bf16(rng.standard_normal((t, hq, d)).astype(np.float32))
        pkv.paged_kv_write(up(k), up(v), up(slots), pool)
        paged.kv_write(k, v, slots, host)
        need = pkv.paged_attention_workspace_size(len(reqs), t, hq, hkv, d, width)
        if ws is None or ws.numel() < need:
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        out = pkv.paged_attention(up(q), pool, up(tables), up(cu), up(lens), scale, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(down_u16(pool), host), f"step {i}: pool differs from the oracle's write"
        ref = paged.attend(q, host, tables, cu, lens, scale)
        check_close(down_u16(out), ref, f"engine step {i}")
        assert pkv.paged_attention_device_status(ws) == 0
    # the system prompt's full blocks are shared by all six requests
    assert bm.ref_count(bm.block_table(5)[0]) == 6
    bm.close()


def test_preemption_and_recompute():
    """Preemption by recompute ([NOTES01] §1.4, the scheduler's answer when
    the free queue runs dry; §2.2 for the cached blocks it leaves): request
    A is preempted so that B can grow, B's new tokens land in blocks A held,
    C then takes the blocks of A that stayed cached, and A is readmitted and
    recomputed into other blocks.  A decode
    step of A with the same query before and after gives the same output bit
    for bit (same keys, same values, same segment; only the block ids
    differ) and the oracle's within the bound; B's step over the reused
    blocks matches the oracle too, and every pool write is bit-exact."""
    rng = np.random.default_rng([469, 64, 1])
    hq, hkv, d, nb, width = 32, 8, 128, 24, 32
    scale = float(np.float32(1 / np.sqrt(d)))
    bm, model = pkv.BlockManager(nb), BlockManagerModel(nb)
    pool = torch.empty((nb, 2, 16, hkv, d), dtype=torch.bfloat16, device="cuda")
    pool.view(torch.int16).fill_(0x7FC1)
    host = np.full(tuple(pool.shape), 0x7FC1, dtype=np.uint16)
    # K/V of every token of a request, drawn once: a recompute writes them again
    kv = {}

    def kv_of(r, pos):
        if (r, pos) not in kv:
            kv[(r, pos)] = (bf16.f32_to_bf16(rng.standard_normal((hkv, d)).astype(np.float32)),
                            bf16.f32_to_bf16(rng.standard_normal((hkv, d)).astype(np.float32)))
        return kv[(r, pos)]

    toks = {0: [int(x) for x in rng.integers(0, 1000, size=150)],
            1: [int(x) for x in rng.integers(0, 1000, size=100)],
            2: [int(x) for x in rng.integers(0, 1000, size=80)]}
    ws = torch.empty(pkv.paged_attention_workspace_size(4, 512, hq, hkv, d, width),
                     dtype=torch.uint8, device="cuda")

    def step(entries, q=None, what=""):
        """entries: (req, first position, count); writes their K/V and runs
        attention; returns the outputs (bf16 bits)"""
        reqs = [r for r, _, _ in entries]
        news = [n for _, _, n in entries]
        tables, cu, lens, slots = bm.step_metadata(reqs, news, width)
        mt = model.step_metadata(reqs, news, width)
        assert all(np.array_equal(np.asarray(a), np.asarray(b)) for a, b in zip((tables, cu, lens, slots), mt))
        t = int(cu[-1])
        k = np.concatenate([np.stack([kv_of(r, p)[0] for p in range(p0, p0 + n)]) for r, p0, n in entries])
        v = np.concatenate([np.stack([kv_of(r, p)[1] for p in range(p0, p0 + n)]) for r, p0, n in entries])
        if q is None:
            q = bf16.f32_to_bf16(rng.standard_normal((t, hq, d)).astype(np.float32))
        log(f"case preemption {what}: S={len(reqs)} T={t} L={lens.tolist()}")
        pkv.paged_kv_write(up(k), up(v), up(slots), pool)
        paged.kv_write(k, v, slots, host)
        out = pkv.paged_attention(up(q), pool, up(tables), up(cu), up(lens), scale, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(down_u16(pool), host), f"{what}: pool differs from the oracle's write"
        got = down_u16(out)
        check_close(got, paged.attend(q, host, tables, cu, lens, scale), what)
        assert pkv.paged_attention_device_status(ws) == 0
        return got

    def admit(r, n):
        a, b = bm.allocate_slots(r, n), model.allocate_slots(r, n)
        assert (a is None) == (b is None)
        assert a is None or a.tolist() == b
        return a

    for r in (0, 1):
        bm.add_request(r, toks[r])
        model.add_request(r, toks[r])
        assert admit(r, len(toks[r])) is not None
    step([(0, 0, 150), (1, 0, 100)], what="prefill A and B")

    # A decodes one token with query qa: the output to reproduce
    t_a = int(rng.integers(0, 1000))
    qa = bf16.f32_to_bf16(rng.standard_normal((1, hq, d)).astype(np.float32))
    for m in (bm, model):
        m.append_tokens(0, [t_a])
    assert admit(0, 1) is not None
    before = step([(0, 150, 1)], q=qa, what="A decode before")
    old_a = bm.block_table(0).tolist()

    # B grows past what is free: preempt A (its blocks go back, its full
    # blocks stay cached until taken), then B's tokens take blocks A held
    grow = [int(x) for x in rng.integers(0, 1000, size=200)]
    for m in (bm, model):
        m.append_tokens(1, grow)
    assert admit(1, 200) is None, "the pool should be too small for B without preempting A"
    bm.free_request(0)
    model.free_request(0)
    assert admit(1, 200) is not None
    assert set(old_a) & set(bm.block_table(1).tolist()), "B should reuse blocks A held"
    step([(1, 100, 200)], what="B over A's blocks")

    # B finishes and C arrives, taking the blocks of A that were still
    # cached; A is readmitted with its prompt and recomputed into other
    # blocks, then decodes the same token again
    bm.free_request(1)
    model.free_request(1)
    for m in (bm, model):
        m.add_request(2, toks[2])
    assert admit(2, 80) is not None
    step([(2, 0, 80)], what="C prefill")
    for m in (bm, model):
        m.add_request(0, toks[0])
    cached = bm.num_cached_tokens(0)
    assert cached == model.num_cached_tokens(0) and cached < 150
    assert admit(0, 150 - cached) is not None
    step([(0, cached, 150 - cached)], what="A recompute")
    for m in (bm, model):
        m.append_tokens(0, [t_a])
    assert admit(0, 1) is not None
    new_a = bm.block_table(0).tolist()
    assert all(a != b for a, b in zip(old_a, new_a)), f"A should now sit in other blocks: {old_a} {new_a}"
    after = step([(0, 150, 1)], q=qa, what="A decode after")
    assert np.array_equal(before, after), "A's decode output changed across preemption"
    bm.close()
