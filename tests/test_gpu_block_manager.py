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
