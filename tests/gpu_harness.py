"""Helpers for the GPU parity tests: put a seeded workload on the device
through the C ABI (history first, then the step's new tokens, then
attention), and compare with the CPU oracle on the same inputs.

The bar: KV writes bit-exact; attention per element
|gpu - ref| <= 2e-2 + 1e-2 * |ref| (gpu = bf16 output widened, ref = fp64
oracle), plus a relative RMS error <= 1e-2 gate, because with N(0,1) inputs
the outputs of long contexts are small enough that the element bound alone
would accept an all-zero output.
"""

import sys

import numpy as np
import torch

import paged_kv_cache_469_amd as pkv
from oracle import bf16, paged

ATOL = 2e-2
RTOL = 1e-2
REL_RMS = 1e-2
POISON = 0x7FC1


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def up(a, dev="cuda"):
    """numpy -> device tensor (uint16 arrays become bf16)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def down_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceStep:
    """A workload on the GPU: poisoned pool, history written, new tokens written."""

    def __init__(self, wl, host_pool=False, q_gain=None, num_blocks=None, poison=True):
        self.wl = wl
        hkv, d = wl.num_kv_heads, wl.head_dim
        nb = wl.num_blocks if num_blocks is None else num_blocks
        self.pool = torch.empty((nb, 2, 16, hkv, d), dtype=torch.bfloat16, device="cuda")
        if poison:
            self.pool.view(torch.int16).fill_(POISON)
        self.host = None
        if host_pool:
            self.host = np.full((nb, 2, 16, hkv, d), POISON, dtype=np.uint16)
        for slots, k, v in wl.history_chunks():
            pkv.paged_kv_write(up(k), up(v), up(slots), self.pool)
            if self.host is not None:
                paged.kv_write(k, v, slots, self.host)
        k, v = wl.new_kv()
        self.k_new, self.v_new = k, v
        self.slots = up(wl.slot_mapping)
        pkv.paged_kv_write(up(k), up(v), self.slots, self.pool)
        if self.host is not None:
            paged.kv_write(k, v, wl.slot_mapping, self.host)
        self.q_host = wl.q(gain=q_gain)
        self.q = up(self.q_host)
        self.bt = up(wl.block_tables)
        self.cu = up(wl.cu_seqlens_q)
        self.lens = up(wl.seq_lens)
        self.ws = torch.empty(pkv.paged_attention_workspace_size(
            wl.num_seqs, wl.num_tokens, wl.num_q_heads, hkv, d, wl.max_blocks_per_seq),
            dtype=torch.uint8, device="cuda")

    def attend(self, out=None):
        out = pkv.paged_attention(self.q, self.pool, self.bt, self.cu, self.lens,
                                  self.wl.scale, out=out, workspace=self.ws)
        torch.cuda.synchronize()
        return out

    def status(self):
        return pkv.paged_attention_device_status(self.ws)


def oracle_rows(wl, q_host, segments=None, rows_per_segment=None, rng=None):
    """fp64 oracle output for the chosen segments, from each request's own
    K/V (dense; the paged == dense identity is pinned on the CPU).
    Returns {segment: (row_indices_in_q, ref [r, Hq, D])}."""
    cu = wl.cu_seqlens_q
    res = {}
    segs = range(wl.num_seqs) if segments is None else segments
    for s in segs:
        n = int(wl.new_tokens[s])
        if n == 0:
            continue
        length = int(wl.seq_lens[s])
        k, v = wl.request_kv(s)
        rows = np.arange(n)
        if rows_per_segment is not None and n > rows_per_segment:
            rows = np.unique(np.concatenate([
                [0, n - 1], (rng or np.random.default_rng(0)).choice(n, rows_per_segment, replace=False)]))
        kf, vf = bf16.to_f64(k), bf16.to_f64(v)
        qf = bf16.to_f64(q_host[cu[s]:cu[s + 1]])
        h = length - n
        if rows.size == n:
            ref = paged.attend_dense(qf, kf, vf, wl.scale, h)
        else:
            ref = np.stack([paged.attend_dense(qf[i:i + 1], kf[:h + i + 1], vf[:h + i + 1],
                                               wl.scale, h + i)[0] for i in rows])
        res[s] = (cu[s] + rows, ref)
    return res


def check_close(got_u16, ref, what):
    got = bf16.to_f64(got_u16)
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    rms = np.sqrt(np.mean((got - ref) ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-300)
    floor = np.sqrt(np.mean((bf16.to_f64(bf16.from_f64(ref)) - ref) ** 2)) / max(
        np.sqrt(np.mean(ref ** 2)), 1e-300)
    log(f"  {what}: max|err| {err.max():.3e}, rel rms {rms:.3e} (bf16 floor {floor:.3e}), "
        f"{int(bad.sum())} of {err.size} outside the bound")
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside 2e-2 + 1e-2|ref|"
    assert rms <= REL_RMS, f"{what}: relative RMS error {rms:.3e} > {REL_RMS}"
    return err.max(), rms
