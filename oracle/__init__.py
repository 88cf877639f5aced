"""CPU oracle for block-sparse video-DiT attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct CPU statement of what the attention hot path
computes: the two mask builders (LVSA and Draft Attention), the Draft token
reorder, and softmax attention in float64 over an explicit key set.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package. The
product (the HIP library and its Python binding) never imports it, and this
package never imports the product: they share no code. Inputs come from the
seeded generators in ``video_diffusion_transformer_lvsa_amd.synth``, which
hold none of the method's arithmetic; the oracle itself only receives arrays.

Sources (cited by page title and section):

* "LVSA: Training-Free Sparse Attention for Long Video Diffusion"
  (gist.science explainer), technical summary §2 "Methodology": core
  mechanism A(t) = G ∪ W(t), rotating global anchors, expanding adaptive
  window, complexity.
* "科学家提出视频扩散模型加速方法，在H100实现一倍以上端到端加速"
  (163.com article on Draft Attention): [t, h, w] reshape and average
  pooling of Q and K into a low-resolution draft map, sparse mask from the
  draft map, the pool_h x pool_w = block_size constraint, and the reorder
  that makes the kept blocks contiguous.

Every function is pinned by ``tests/test_oracle_*.py`` (``-m "not gpu"``)
against closed forms, invariants, brute force and a library routine,
including the bfloat16 decode ``to_f64`` (fixed bit patterns, all 65536
codes against a decoder written from the format's fields, torch's own
conversion). The FP8 probability rounding is pinned by a derived bound and
a statistical match rather than element by element.
"""
from .lvsa import anchors, nearest_order, attend_set, lvsa_mask, lvsa_capacity
from .draft import (
    DraftGrid,
    draft_grid,
    draft_permutation,
    draft_pool,
    draft_scores,
    topk_count,
    draft_topk,
    draft_mask,
)
from .fp8 import E4M3_MAX, e4m3_decode_table, e4m3_encode, quantize_per_head, dequantize, attention_p_e4m3, p_rounding_bound
from .attention import (
    attention_keyset,
    attention_statistics,
    dense_attention,
    block_sparse_attention,
    draft_attention_original_order,
    to_f64,
)

__all__ = [
    "E4M3_MAX",
    "e4m3_decode_table",
    "e4m3_encode",
    "quantize_per_head",
    "dequantize",
    "attention_p_e4m3",
    "p_rounding_bound",
    "attention_statistics",
    "anchors",
    "nearest_order",
    "attend_set",
    "lvsa_mask",
    "lvsa_capacity",
    "DraftGrid",
    "draft_grid",
    "draft_permutation",
    "draft_pool",
    "draft_scores",
    "topk_count",
    "draft_topk",
    "draft_mask",
    "attention_keyset",
    "dense_attention",
    "block_sparse_attention",
    "draft_attention_original_order",
    "to_f64",
]
