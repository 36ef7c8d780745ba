"""Plain fp64 CPU oracle for the hybrid-attention token-mixing path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this package: only the tests, the smoke check and the bench's CPU-baseline leg
use it. It shares no code with the HIP library (no kernels, headers, tables or
helpers); both sides only read the same seeded input bits.

Every function is the plain definition from the pages, in float64, with the
pages' order of operations:

* ``rope3d``      -- 3D rotary embedding (SANA-Video notes, section 3.2; the
                     band split, base and pairing are readings, see module).
* ``linear_attention`` -- bidirectional ReLU-kernel linear attention with RoPE
                     after the ReLU and a RoPE-free denominator (SANA-Video
                     notes, section 3.2, equation and pseudocode), with the
                     optional sigmoid output gate (the SANA-Video 2.0 abstract
                     describes the linear layers as gated).
* ``linear_attention_backward`` -- gradients of the bidirectional (gated)
                     variant, derived by hand from the definition.
* ``linear_attention_chunked_backward`` -- gradients of the block-causal
                     variant, including those of the carried and returned cache.
* ``linear_attention_causal`` -- token-causal variant (SANA-Video notes,
                     section 3.4, causal equation), with a carried state.
* ``linear_attention_chunked`` -- block-causal variant with the carried
                     cumulative state and key sum (SANA-Video notes, section
                     3.4, causal equation and Algorithm 1).
* ``softmax_anchor`` -- gated non-causal softmax attention (SANA-Video 2.0
                     abstract and summary, hybrid 3:1 design).
* ``softmax_anchor_backward`` -- gradients of the gated anchor, derived by
                     hand from its definition.
* ``softmax_anchor_lse`` -- the natural-log normaliser of every query row
                     (what a backward pass reuses instead of the forward).
* ``softmax_anchor_block_sparse`` -- the anchor restricted to caller-given
                     key blocks per query block (the pages name a sparse
                     anchor without its pattern: parity unpinned against them).
* ``attnres_route`` -- block attention-residual router (SANA-Video 2.0
                     summary, method section, router equation).

Pins: every function is checked in ``tests/test_oracle.py`` against brute
force on tiny inputs, closed forms, invariants and independent library
routines. One part is "parity unpinned" against the pages' own model: the
RoPE pairing and frequency convention (the pages do not define
``apply_3d_rope``); it is pinned only to the reading stated in ``rope3d``.
"""
from .rope3d import Rope3D, rope3d_angles, rope3d_rotate
from .linear_attention import (linear_attention, linear_attention_backward, linear_attention_causal,
                               linear_attention_chunked, linear_attention_chunked_backward)
from .softmax_anchor import softmax_anchor, softmax_anchor_backward, softmax_anchor_block_sparse, softmax_anchor_lse
from .attnres_router import attnres_route

__all__ = [
    "Rope3D",
    "rope3d_angles",
    "rope3d_rotate",
    "linear_attention",
    "linear_attention_backward",
    "linear_attention_causal",
    "linear_attention_chunked",
    "linear_attention_chunked_backward",
    "softmax_anchor",
    "softmax_anchor_block_sparse",
    "softmax_anchor_backward",
    "softmax_anchor_lse",
    "attnres_route",
]
