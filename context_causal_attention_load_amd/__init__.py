"""Load-balanced context-parallel causal attention and GQA decode for MI355X (gfx950).

The compute path is the HIP library ``libcpattn.so`` behind the C ABI declared in
``include/cpattn.h``; ``binding`` marshals torch tensors into that ABI. Nothing in this
package computes attention on the CPU: if the library is missing, every call raises.
"""

from .binding import (  # noqa: F401
    CpattnError,
    library_path,
    load_library,
    permute,
    unpermute,
    attention_fwd,
    attention_fwd_workspace_bytes,
    attention_bwd,
    attention_bwd_workspace_bytes,
    attention_bwd_split_workspace_bytes,
    decode,
    decode_noalloc,
    decode_merge,
    decode_int8,
    quantize_kv,
    decode_workspace_bytes,
    lb_source_index,
    lb_positions,
)
