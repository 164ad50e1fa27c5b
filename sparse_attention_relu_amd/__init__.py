"""MI355X (gfx950) indexer-selected sparse MLA: HIP kernels behind a C ABI.

The four calls of the hot path -- indexer_score, topk_select,
mla_sparse_attn, layer_stack -- live in libsparse_mla.so; this package is a
thin binding (``api``) plus seeded synthetic inputs (``synth``).
"""
from .api import (LayerStack, indexer_score, layer_is_full, layer_stack, mla_sparse_attn,  # noqa: F401
                  topk_select, workspace)
