"""MI355X paged-KV hot path: KV block write and paged attention.

A thin ctypes binding over ``libpaged_attn.so`` (built from ``csrc/`` by
``build.py``).  It only marshals arguments: every step of the computation
runs in the library's HIP kernels.  PyTorch supplies device memory and the
current stream.  The names follow the C ABI in ``include/paged_attn.h``.

There is no fallback: if the library is missing, every call raises.
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    PagedError,
    lib,
    NOALLOC_SCRATCH_BYTES,
    paged_attention,
    paged_attention_noalloc,
    paged_attention_device_status,
    paged_attention_set_partition_tokens,
    paged_attention_set_group_members,
    paged_attention_set_stage_events,
    paged_attention_workspace_size,
    paged_decode_advance,
    paged_kv_block_bytes,
    paged_kv_write,
    paged_last_error,
    paged_validate,
    STATUS_BAD_BLOCK,
    STATUS_BAD_SEGMENT,
)
from .block_manager import BlockManager, BlockManagerError  # noqa: F401,E402
