"""PagedAttention decode (and paged prefill) on AMD Instinct MI355X (gfx950).

The work runs in ``libpkv.so`` (hand-written HIP kernels and a C++ block allocator behind the
C ABI in ``include/pkv.h``); this package only marshals arguments. Importing it fails if the
library has not been built (``python paged_kv_cache_459_amd/build.py``): there is no fallback.
"""

from ._lib import BF16, BLOCK_SHARED, F16, F32, STATUS, PkvError, lib  # noqa: F401
from .api import (BLOCK_SIZE, ENGINE_PLAN, BlockAllocator, Engine, alloc_caches, cache_bytes,  # noqa: F401
                  cache_shapes, pkv_copy_blocks, pkv_decode_append_attn, pkv_decode_append_merge,
                  pkv_decode_append_attn_noalloc,
                  pkv_decode_append_stream,
                  pkv_decode_attn, pkv_decode_kernel, pkv_decode_merge,
                  pkv_decode_num_workers, pkv_decode_plan, pkv_decode_planned,
                  pkv_decode_planned_launches, pkv_decode_planned_workspace_bytes,
                  pkv_decode_stream,
                  pkv_decode_stream_workspace_bytes,
                  pkv_decode_workspace_bytes, pkv_dtype, pkv_prefill_attn, pkv_prefill_plan,
                  pkv_prefill_workspace_bytes, pkv_probe_read, pkv_set_attn_kernel, pkv_write,
                  split_workspace)
