"""CPU oracle for the paged-KV hot path: KV block write and paged attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this package.  Its only users are ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``.  It shares no code with the HIP
path (no kernels, headers, helpers, tables or constants); it imports numpy and
the standard library only.

Sources (the web pages this follows, named by title):

* [NOTES01] "vLLM 学习笔记 01：一个请求在 vLLM 里的一生" (a reader's notes on a
  request's life in vLLM), sections 1.4 (scheduler: computed vs. total
  tokens), 1.5 (paged KV cache), 1.6 (forward pass over an unpadded batch),
  2.1 (chunked prefill) and 2.2 (prefix caching).
* [INSIDE] Chinese translation of "Inside vLLM: Anatomy of a High-Throughput
  LLM Inference System", the part on the LLM engine constructor that gives
  the per-layer KV block size formula.
* [ZSH] "从0开始的vLLM学习" (study notes), the prefill/decode paragraph: a
  decode step feeds only the newest token because earlier tokens' K/V are
  cached.

Modules:

* ``bf16``   -- bf16 <-> float bit helpers (numpy has no bf16 dtype here).
* ``paged``  -- the oracle proper: block bytes, write, gather, attention (fp64).
* ``brute``  -- a scalar pure-Python twin of the attention, for tiny inputs.
* ``block_manager`` -- a plain list/dict model of the KV block manager (free
  queue, reference counts, prefix cache, slot allocation), sections 1.4, 1.5
  and 2.2 of [NOTES01].

Every function is a plain definition: no blocking, fusion or reordering
beyond what the definition states.  Parity status of each function is given
in its docstring; every function here is pinned by ``tests/test_oracle_*.py``.
"""

from . import bf16, block_manager, brute, paged  # noqa: F401
