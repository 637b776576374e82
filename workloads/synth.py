"""Seeded synthetic workloads for paged KV write + paged attention.

The shapes follow the workloads the pages describe: a mixed step with a
6-token prefill beside a 1-token decode over cached history ("vLLM 学习笔记
01", section 1.6), decode batches over long cached contexts, prompts packed
end to end, a continuous-batching step under a token budget with one chunk of
a long prompt (section 2.1) and requests that share a cached system-prompt
prefix (section 2.2), a speculative-decoding check of a few drafted tokens
per request (section 2.4), and a pool sized to a fraction of free device
memory.

Every random draw comes from ``np.random.default_rng([469, cfg, purpose,
idx])`` with purpose 0 = lengths, 1 = block placement, 2 = q, 3 = k/v of
request ``idx``, 4 = the shared prefix's k/v.  Values are float32 standard
normals rounded to bf16 (round to nearest even, done by PyTorch's dtype
conversion) and held as uint16 bit patterns.  Lengths are integers uniform on
inclusive ranges.  Physical blocks are handed out in order from a seeded
random permutation of the pool; table padding is -1.

A segment is one request's share of the step: ``n`` new tokens at the end of
a sequence of ``L`` tokens, the first ``h = L - n`` of which are already
cached.  Segment index = packing position; each segment keeps the request id
that seeds its values, so packing orders can be permuted without changing
any request's data.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK = 16
POISON_BF16 = 0x7FC1          # a quiet NaN, used to fill unwritten pool memory


def _rng(cfg, purpose, idx=0):
    return np.random.default_rng([469, cfg, purpose, idx])


def _bf16_bits(f32):
    """float32 array -> uint16 bf16 bit patterns (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _normal_bf16(rng, shape, gain=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if gain != 1.0:
        x *= np.float32(gain)
    return _bf16_bits(x)


@dataclass
class Workload:
    name: str
    cfg: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    new_tokens: np.ndarray          # int32 [S]   n_s
    seq_lens: np.ndarray            # int32 [S]   L_s
    request_ids: np.ndarray         # int64 [S]   seeds of each segment's values
    block_tables: np.ndarray        # int32 [S, W], -1 padded
    shared_prefix: int = 0          # tokens of the shared prefix (multiple of 16)
    shared_requests: tuple = ()     # request ids that share it
    q_gain: float = 1.0
    _kv_cache: dict = field(default_factory=dict, repr=False)
    cache_values: bool = False

    # ---- shapes -----------------------------------------------------------
    @property
    def num_seqs(self):
        return int(self.seq_lens.shape[0])

    @property
    def cu_seqlens_q(self):
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        np.cumsum(self.new_tokens, out=cu[1:])
        return cu

    @property
    def num_tokens(self):
        return int(self.new_tokens.sum())

    @property
    def history(self):
        return (self.seq_lens - self.new_tokens).astype(np.int32)

    @property
    def max_blocks_per_seq(self):
        return int(self.block_tables.shape[1])

    @property
    def scale(self):
        return float(np.float32(1.0 / np.sqrt(self.head_dim)))

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    def slots_of(self, s, start, stop):
        """Slots of positions [start, stop) of segment s."""
        pos = np.arange(start, stop, dtype=np.int64)
        return (self.block_tables[s][pos // BLOCK].astype(np.int64) * BLOCK
                + pos % BLOCK).astype(np.int32)

    @property
    def slot_mapping(self):
        """Slots of the step's new tokens, in packing order."""
        parts = [self.slots_of(s, int(self.history[s]), int(self.seq_lens[s]))
                 for s in range(self.num_seqs)]
        if not parts:
            return np.zeros(0, dtype=np.int32)
        return np.concatenate(parts).astype(np.int32)

    # ---- values -----------------------------------------------------------
    def request_kv(self, s):
        """(k, v) uint16 [L_s, Hkv, D]: every token of segment s's request."""
        rid = int(self.request_ids[s])
        if rid in self._kv_cache:
            return self._kv_cache[rid]
        length = int(self.seq_lens[s])
        shape = (2, length, self.num_kv_heads, self.head_dim)
        kv = _normal_bf16(_rng(self.cfg, 3, rid), shape)
        if self.shared_prefix and rid in self.shared_requests:
            p = self.shared_prefix
            kv[:, :p] = _normal_bf16(
                _rng(self.cfg, 4, 0), (2, p, self.num_kv_heads, self.head_dim))
        out = (kv[0], kv[1])
        if self.cache_values:
            self._kv_cache[rid] = out
        return out

    def q(self, gain=None):
        """uint16 [T, Hq, D] bf16 bits of the step's queries."""
        g = self.q_gain if gain is None else gain
        return _normal_bf16(_rng(self.cfg, 2, 0),
                            (self.num_tokens, self.num_q_heads, self.head_dim), g)

    def new_kv(self):
        """(k, v) uint16 [T, Hkv, D] of the step's new tokens, packing order."""
        ks, vs = [], []
        for s in range(self.num_seqs):
            k, v = self.request_kv(s)
            h = int(self.history[s])
            ks.append(k[h:])
            vs.append(v[h:])
        if not ks:
            z = np.zeros((0, self.num_kv_heads, self.head_dim), dtype=np.uint16)
            return z, z.copy()
        return np.concatenate(ks), np.concatenate(vs)

    def history_chunks(self):
        """Yield (slots, k, v) writes that fill every segment's cached history.

        The shared prefix is written once, by the first sharing segment.
        """
        prefix_done = False
        for s in range(self.num_seqs):
            rid = int(self.request_ids[s])
            h = int(self.history[s])
            start = 0
            if self.shared_prefix and rid in self.shared_requests:
                if prefix_done:
                    start = min(h, self.shared_prefix)
                prefix_done = True
            if h > start:
                k, v = self.request_kv(s)
                yield self.slots_of(s, start, h), k[start:h], v[start:h]

    # ---- accounting -------------------------------------------------------
    def kv_bytes_logical(self):
        """K+V bytes attention must read, counted per segment (bf16)."""
        return int(self.seq_lens[self.new_tokens > 0].astype(np.int64).sum()
                   * 2 * self.num_kv_heads * self.head_dim * 2)

    def kv_bytes_unique(self):
        """As above, but shared prefix slots counted once."""
        total = self.kv_bytes_logical()
        live = [s for s in range(self.num_seqs)
                if self.new_tokens[s] > 0 and int(self.request_ids[s]) in self.shared_requests]
        if self.shared_prefix and len(live) > 1:
            total -= (len(live) - 1) * self.shared_prefix * 2 * self.num_kv_heads * self.head_dim * 2
        return int(total)

    def attention_pairs(self):
        """Unmasked (query, key) pairs: sum_s n_s*h_s + n_s(n_s+1)/2."""
        n = self.new_tokens.astype(np.int64)
        h = self.history.astype(np.int64)
        return int((n * h + n * (n + 1) // 2).sum())

    def attention_flops(self, segments=None):
        """4*D*Hq flop per unmasked pair (QK^T and PV, 2 flop per MAC)."""
        n = self.new_tokens.astype(np.int64)
        h = self.history.astype(np.int64)
        pairs = n * h + n * (n + 1) // 2
        if segments is not None:
            pairs = pairs[segments]
        return int(4 * self.head_dim * self.num_q_heads * pairs.sum())


def build(name, cfg, hq, hkv, d, segs, *, request_ids=None, shared_prefix=0,
          shared_requests=(), num_blocks=None, width=None, q_gain=1.0):
    """Lay out a workload.  ``segs`` = [(n, L)] in packing order."""
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    if shared_prefix % BLOCK:
        raise ValueError("a shared prefix is made of full blocks")
    s_count = len(segs)
    n_arr = np.array([n for n, _ in segs], dtype=np.int32).reshape(-1)
    l_arr = np.array([length for _, length in segs], dtype=np.int32).reshape(-1)
    if np.any(n_arr < 0) or np.any(n_arr > l_arr):
        raise ValueError("each segment needs 0 <= n <= L")
    rids = np.arange(s_count) if request_ids is None else np.asarray(request_ids)
    shared_requests = tuple(int(r) for r in shared_requests)
    nblk = (l_arr.astype(np.int64) + BLOCK - 1) // BLOCK
    shared_blocks = shared_prefix // BLOCK
    sharers = [s for s in range(s_count) if int(rids[s]) in shared_requests]
    for s in sharers:
        if l_arr[s] - n_arr[s] < shared_prefix:
            raise ValueError("a sharing request must hold the whole prefix as history")
    needed = int(nblk.sum()) - (max(0, len(sharers) - 1) * shared_blocks if sharers else 0)
    nb = needed if num_blocks is None else int(num_blocks)
    if nb < needed:
        raise ValueError(f"pool of {nb} blocks cannot hold {needed}")
    w = int(nblk.max()) if (width is None and s_count) else int(width or 1)
    w = max(w, 1)
    if s_count and w < nblk.max():
        raise ValueError("block table narrower than the longest sequence")
    rng = _rng(cfg, 1, 0)
    if nb <= 8 * needed:
        phys = rng.permutation(nb)[:needed]
    else:
        phys = rng.choice(nb, size=needed, replace=False)
    phys = phys.astype(np.int32)
    tables = np.full((s_count, w), -1, dtype=np.int32)
    cursor = 0
    shared_ids = None
    if sharers:
        shared_ids = phys[:shared_blocks]
        cursor = shared_blocks
    # private blocks are handed out in request-id order
    for s in sorted(range(s_count), key=lambda i: int(rids[i])):
        k = int(nblk[s])
        start = 0
        if shared_ids is not None and int(rids[s]) in shared_requests:
            tables[s, :shared_blocks] = shared_ids
            start = shared_blocks
        tables[s, start:k] = phys[cursor:cursor + (k - start)]
        cursor += k - start
    assert cursor == needed
    return Workload(name=name, cfg=cfg, num_q_heads=hq, num_kv_heads=hkv,
                    head_dim=d, num_blocks=nb, new_tokens=n_arr, seq_lens=l_arr,
                    request_ids=rids, block_tables=tables,
                    shared_prefix=shared_prefix, shared_requests=shared_requests,
                    q_gain=q_gain)


# --------------------------------------------------------------------------
# The five workloads.  Keyword arguments shrink them into parity twins that
# keep the structure (same seeds for lengths and values, fewer requests or
# shorter contexts).
# --------------------------------------------------------------------------

def tiny_mixed(**kw):
    """TinyLlama-shaped mixed step: a 6-token prefill beside a 1-token decode
    over 37 cached tokens; 32 q heads, 4 KV heads, head_dim 64, 64-block pool."""
    return build("tiny_mixed", 1, 32, 4, 64, [(6, 6), (1, 38)],
                 num_blocks=kw.pop("num_blocks", 64), **kw)


def decode_8b(num_requests=256, ctx=(512, 4096), **kw):
    """Llama-3-8B-shaped decode batch: 32/8 heads, head_dim 128, one new token
    per request over a cached context uniform in ``ctx``."""
    c = _rng(2, 0).integers(ctx[0], ctx[1] + 1, size=num_requests)
    return build("decode_8b", 2, 32, 8, 128, [(1, int(x) + 1) for x in c], **kw)


def prefill_8b(num_prompts=16, lens=(256, 2048), **kw):
    """8B-shaped prefill batch: prompts of length uniform in ``lens``, packed
    end to end, no history."""
    n = _rng(3, 0).integers(lens[0], lens[1] + 1, size=num_prompts)
    return build("prefill_8b", 3, 32, 8, 128, [(int(x), int(x)) for x in n], **kw)


def cb_step_8b(num_decodes=192, ctx=(1024, 8192), shared=64, prefix=1024,
               chunk=2048, chunk_history=16384, decode_first=True, **kw):
    """Continuous-batching step under an 8192-token budget: ``num_decodes``
    decodes (the first ``shared`` of them share a ``prefix``-token cached
    prefix) plus one ``chunk``-token chunk of a long prompt whose first
    ``chunk_history`` tokens are cached."""
    c = _rng(4, 0).integers(ctx[0], ctx[1] + 1, size=num_decodes)
    dec = [(1, int(x) + 1) for x in c]
    segs = dec + [(chunk, chunk_history + chunk)]
    rids = list(range(num_decodes + 1))
    if not decode_first:
        segs = segs[-1:] + segs[:-1]
        rids = rids[-1:] + rids[:-1]
    return build("cb_step_8b", 4, 32, 8, 128, segs, request_ids=rids,
                 shared_prefix=prefix if shared else 0,
                 shared_requests=tuple(range(min(shared, num_decodes))), **kw)


def long_decode_70b(num_requests=64, ctx=(32768, 131072), **kw):
    """70B-shaped single-layer share: 64 q heads, 8 KV heads, head_dim 128;
    decodes over cached contexts uniform in ``ctx``; the pool may be far
    larger than what the requests use (``num_blocks``)."""
    c = _rng(5, 0).integers(ctx[0], ctx[1] + 1, size=num_requests)
    return build("long_decode_70b", 5, 64, 8, 128, [(1, int(x) + 1) for x in c], **kw)


def spec_verify_8b(num_requests=128, drafts=3, ctx=(2048, 16384), **kw):
    """8B-shaped speculative-decoding check ("vLLM 学习笔记 01", section 2.4:
    k drafted tokens are checked by the large model in one forward pass):
    each request feeds its last accepted token and ``drafts`` drafted ones
    (n = drafts + 1 new tokens) over a cached context uniform in ``ctx``."""
    c = _rng(6, 0).integers(ctx[0], ctx[1] + 1, size=num_requests)
    n = drafts + 1
    return build("spec_verify_8b", 6, 32, 8, 128, [(n, int(x) + n) for x in c], **kw)


def spec_verify_70b(num_requests=64, drafts=3, ctx=(4096, 16384), **kw):
    """70B-shaped speculative-decoding check (64 q heads, 8 KV heads, head_dim
    128): each request feeds its last accepted token and ``drafts`` drafted
    ones over a cached context uniform in ``ctx``; n * G = 32 query rows per
    KV head."""
    c = _rng(7, 0).integers(ctx[0], ctx[1] + 1, size=num_requests)
    n = drafts + 1
    return build("spec_verify_70b", 7, 64, 8, 128, [(n, int(x) + n) for x in c], **kw)


NAMED = {
    "tiny_mixed": tiny_mixed,
    "decode_8b": decode_8b,
    "prefill_8b": prefill_8b,
    "cb_step_8b": cb_step_8b,
    "long_decode_70b": long_decode_70b,
    "spec_verify_8b": spec_verify_8b,
    "spec_verify_70b": spec_verify_70b,
}


def make(name, **kw):
    return NAMED[name](**kw)
