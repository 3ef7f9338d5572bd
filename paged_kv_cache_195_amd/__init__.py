"""Paged attention over a block-table K/V cache for AMD MI355X (gfx950).

``decode``, ``prefill`` and ``combine`` call the HIP kernels of libpa.so
through its C ABI (include/pa.h).  Build the library with
``python -m paged_kv_cache_195_amd.build``.
"""

from .api import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    PaShape,
    combine,
    decode,
    decode_noalloc,
    describe_plan,
    load_library,
    make_shape,
    prefill,
    resolve_num_splits,
    split_views,
    strerror,
    workspace_bytes,
)
