"""SegPagedAttention with head-aware KV reuse on AMD Instinct MI355X (gfx950).

The compute path is libsegpaged.so (include/segpaged.h): a host page-table
builder and hand-written HIP kernels for RoPE relocation, prefill attention and
split-K decode.  ``segpaged`` is its ctypes binding; ``workload`` and
``kvpool`` are device-memory glue built on torch.
"""
from . import segpaged  # noqa: F401

__all__ = ["segpaged"]
