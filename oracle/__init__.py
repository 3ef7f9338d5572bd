"""CPU oracle (test infrastructure only; see ``oracle.paged_attention``)."""

from .paged_attention import (  # noqa: F401
    attend,
    attention,
    check_pages,
    code_value,
    dequantize_cache,
    combine,
    gather_logical,
    key_limit,
    kv_head_of,
    pages_for,
    split_page_ranges,
    split_partials,
)
