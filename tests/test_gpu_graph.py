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
from oracle import paged

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
