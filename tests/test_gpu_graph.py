"""A whole step (KV write of the new tokens + attention) captured in a HIP
graph and replayed.

The calls make no host synchronisation, allocation or memset: the plan
kernel resets the workspace it uses on the device.  So a step can be
captured once and replayed.  Each replay is checked bit for bit against the
eager result of the same call (the kernels are deterministic: every work
item's result is independent of which workgroup takes it), with eager work
and synchronisations between the replays, and the eager result against the
CPU oracle.
"""

import time

import numpy as np
import pytest
import torch

import paged_kv_cache_469_amd as pkv
import workloads
from gpu_harness import DeviceStep, check_close, down_u16, log, up
from oracle import bf16, paged

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny_mixed", {}),
    ("cb_step_8b", dict(num_decodes=12, ctx=(1024, 3000), shared=4, prefix=1024, chunk=300,
                        chunk_history=700)),
]


def _step(st, k, v, out):
    pkv.paged_kv_write(k, v, st.slots, st.pool)
    pkv.paged_attention(st.q, st.pool, st.bt, st.cu, st.lens, st.wl.scale, out=out,
                        workspace=st.ws)


@pytest.mark.parametrize("name,kw", CASES, ids=[n for n, _ in CASES])
def test_graph_replay_matches_eager(name, kw):
    wl = workloads.make(name, **kw)
    log(f"case graph {name}: S={wl.num_seqs} T={wl.num_tokens}")
    st = DeviceStep(wl, host_pool=True)
    k, v = up(st.k_new), up(st.v_new)
    eager = torch.empty_like(st.q)
    _step(st, k, v, eager)   # rewrites the same new tokens: the pool is unchanged
    torch.cuda.synchronize()
    assert np.array_equal(down_u16(st.pool), st.host), "KV pool differs from the oracle's write"
    ref = paged.attend(st.q_host, st.host, wl.block_tables, wl.cu_seqlens_q, wl.seq_lens, wl.scale)
    check_close(down_u16(eager), ref, f"graph {name} eager")
    want = down_u16(eager)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph_out = torch.empty_like(st.q)
    with torch.cuda.stream(side):
        _step(st, k, v, graph_out)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(st, k, v, graph_out)
    torch.cuda.synchronize()

    scratch = torch.empty_like(st.q)
    for rep in range(4):
        graph_out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(down_u16(graph_out), want), f"replay {rep} differs from the eager call"
        assert st.status() == 0
        _step(st, k, v, scratch)   # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(down_u16(scratch), want)

    # launch overhead, reported (not asserted): eager step vs replayed graph
    n = 50
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        _step(st, k, v, scratch)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(n):
        g.replay()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    log(f"graph {name}: eager {1e6 * (t1 - t0) / n:.1f} us/step, replay {1e6 * (t2 - t1) / n:.1f} us/step")
    assert np.array_equal(down_u16(graph_out), want)


def test_decode_advance_matches_oracle():
    rng = np.random.default_rng([469, 66, 0])
    s, w, nb = 300, 40, 5000
    tables = rng.integers(-1, nb + 50, size=(s, w)).astype(np.int32)   # some entries invalid
    lens = rng.integers(0, w * 16 + 20, size=s).astype(np.int32)      # some past the table
    bt, sl = up(tables), up(lens)
    cu = torch.full((s + 1,), -7, dtype=torch.int32, device="cuda")
    slots = torch.full((s,), -7, dtype=torch.int32, device="cuda")
    pkv.paged_decode_advance(bt, sl, cu, slots, nb)
    torch.cuda.synchronize()
    want_lens, want_cu, want_slots = paged.decode_advance(tables, lens, nb)
    assert sl.cpu().numpy().tolist() == want_lens.tolist()
    assert cu.cpu().numpy().tolist() == want_cu.tolist()
    assert slots.cpu().numpy().tolist() == want_slots.tolist()


def test_graph_replayed_decode_loop():
    """A steady-state decode loop: each step is paged_decode_advance (metadata
    on the device), paged_kv_write and paged_attention, captured once in a
    graph and replayed N times.  Every replayed step must equal the same step
    run eagerly with metadata computed on the host (bit for bit), the pools
    must end equal, and the last step must match the oracle."""
    rng = np.random.default_rng([469, 67, 0])
    s, hq, hkv, d, steps = 24, 32, 8, 128, 20
    scale = float(np.float32(1 / np.sqrt(d)))
    L0 = rng.integers(100, 1200, size=s).astype(np.int32)
    room = steps + 60                     # positions the tables hold beyond L0 (timing included)
    nblk = (L0 + room + 15) // 16
    w = int(nblk.max())
    nb = int(nblk.sum()) + 7
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((s, w), -1, dtype=np.int32)
    c = 0
    for i in range(s):
        tables[i, :nblk[i]] = perm[c:c + nblk[i]]
        c += nblk[i]
    host = np.full((nb, 2, 16, hkv, d), 0x7FC1, dtype=np.uint16)
    for i in range(s):   # history of positions 0 .. L0 - 1
        pos = np.arange(L0[i])
        kv = bf16.f32_to_bf16(rng.standard_normal((2, L0[i], hkv, d)).astype(np.float32))
        paged.kv_write(kv[0], kv[1], tables[i][pos // 16] * 16 + pos % 16, host)
    ks = bf16.f32_to_bf16(rng.standard_normal((steps, s, hkv, d)).astype(np.float32))
    vs = bf16.f32_to_bf16(rng.standard_normal((steps, s, hkv, d)).astype(np.float32))
    qs = bf16.f32_to_bf16(rng.standard_normal((steps, s, hq, d)).astype(np.float32))
    log(f"case graph decode loop: S={s} steps={steps} NB={nb}")

    pool_e = up(host).view(torch.bfloat16).reshape(host.shape)
    pool_g = pool_e.clone()
    bt = up(tables)
    ks_d, vs_d, qs_d = up(ks), up(vs), up(qs)
    ws = torch.empty(pkv.paged_attention_workspace_size(s, s, hq, hkv, d, w), dtype=torch.uint8,
                     device="cuda")

    # eager: metadata from the host every step
    eager_out = []
    lens = L0.copy()
    for i in range(steps):
        new_lens, cu, slots = paged.decode_advance(tables, lens, nb)
        pkv.paged_kv_write(ks_d[i], vs_d[i], up(slots), pool_e)
        eager_out.append(pkv.paged_attention(qs_d[i], pool_e, bt, up(cu), up(new_lens), scale,
                                             workspace=ws))
        paged.kv_write(ks[i], vs[i], slots, host)
        lens = new_lens
        last_cu, last_lens = cu, new_lens
    torch.cuda.synchronize()
    eager_out = [down_u16(o) for o in eager_out]

    # graph: advance + write + attention, inputs in static buffers
    g_lens = up(L0.copy())
    g_cu = torch.zeros(s + 1, dtype=torch.int32, device="cuda")
    g_slots = torch.zeros(s, dtype=torch.int32, device="cuda")
    k_buf, v_buf, q_buf = ks_d[0].clone(), vs_d[0].clone(), qs_d[0].clone()
    out_buf = torch.empty_like(q_buf)
    ws_g = torch.empty_like(ws)

    def step():
        pkv.paged_decode_advance(bt, g_lens, g_cu, g_slots, nb)
        pkv.paged_kv_write(k_buf, v_buf, g_slots, pool_g)
        pkv.paged_attention(q_buf, pool_g, bt, g_cu, g_lens, scale, out=out_buf, workspace=ws_g)

    # the step allocates nothing, so it is captured directly; capture runs nothing
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    assert g_lens.cpu().numpy().tolist() == L0.tolist(), "capture must not run the step"
    for i in range(steps):
        k_buf.copy_(ks_d[i])
        v_buf.copy_(vs_d[i])
        q_buf.copy_(qs_d[i])
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(down_u16(out_buf), eager_out[i]), f"replayed step {i} differs"
    assert np.array_equal(down_u16(pool_g), down_u16(pool_e)), "pools differ"
    assert g_lens.cpu().numpy().tolist() == (L0 + steps).tolist()
    assert np.array_equal(down_u16(pool_e), host), "pool differs from the oracle's writes"
    ref = paged.attend(qs[-1], host, tables, last_cu, last_lens, scale)
    check_close(eager_out[-1], ref, "graph decode loop, last step")
    assert pkv.paged_attention_device_status(ws_g) == 0

    # per-step time, reported: eager with host metadata vs replay
    n = 50
    lens = (L0 + steps).astype(np.int32)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        new_lens, cu, slots = paged.decode_advance(tables, lens, nb)
        pkv.paged_kv_write(ks_d[0], vs_d[0], up(slots), pool_e)
        pkv.paged_attention(qs_d[0], pool_e, bt, up(cu), up(new_lens), scale, workspace=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(n):
        g.replay()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    log(f"graph decode loop: eager with host metadata {1e6 * (t1 - t0) / n:.1f} us/step, "
        f"replay {1e6 * (t2 - t1) / n:.1f} us/step")
