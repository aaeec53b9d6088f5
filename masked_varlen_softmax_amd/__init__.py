"""masked_varlen_softmax_amd: fused masked softmax attention over packed
variable-length sequences for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libmvs.so`` built from ``csrc/``; this
package is its thin Python binding. The binding is loaded on first use of an
API name and raises if the library is missing: there is no CPU fallback.

``masked_varlen_softmax_amd.workloads`` (seeded synthetic inputs) imports
neither the library nor torch's device state. Useful-work counts come from the
library's own accounting functions (``prefill_useful_flops``,
``decode_useful_bytes``).
"""

_API = (
    "build_query_range_table",
    "build_query_range_table_device",
    "prefill_useful_flops",
    "decode_useful_bytes",
    "attn_varlen_fwd",
    "attn_varlen_fwd_paged",
    "attn_varlen_fwd_range_scan",
    "attn_paged_decode",
    "attn_paged_decode_workspace_size",
    "attn_paged_decode_noalloc",
    "lib",
    "library_path",
    "MvsError",
    "plan_key_tiles",
)


def __getattr__(name):
    if name in _API:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)


__all__ = list(_API)
