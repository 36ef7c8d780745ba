"""libhla: MI355X (gfx950) kernels for the SANA-Video hybrid-attention token mixer.

The compute lives in ``libhla.so`` (hand-written HIP, C ABI declared in
``include/hla.h``); ``softmax_attention_relu_amd.hla`` is its ctypes binding.
Build with ``python -m softmax_attention_relu_amd.build``.
"""
from . import hla  # noqa: F401
from .hla import (  # noqa: F401
    HlaError,
    Rope3D,
    hla_attnres_route,
    hla_linear_attn,
    hla_linear_attn_chunked,
    hla_linear_attn_chunked_workspace,
    hla_linear_attn_workspace,
    hla_rope_table_host,
    hla_softmax_anchor,
    hla_softmax_anchor_workspace,
    hla_status_string,
)
