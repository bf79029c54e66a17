"""CPU oracle for block-causal paged attention and the KV commit.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
baseline may import this package. The product path (the HIP library and its Python
binding) never imports, calls or links it, and it shares no code with them.

What it computes is the plain definition, densely, in float64 over a contiguous copy
of the cached K/V:

* block-causal mask: a token attends to every token of its own block, to every token
  of earlier blocks and to none of later blocks ("Inference for Interpretable
  Text-Diffusion Models", Background, block-causal diffusion decoding);
* the paged cache: each sequence's committed rows live in fixed-size pages that need
  not be contiguous, located through a page table (same page, section "Paged
  Attention");
* tiles of the mask are fully included, fully excluded or partial (same page, section
  "FlexAttention with Aligned Tiles" and the BlockMask tile figure);
* commit: once a block is finished its keys and values are written into the cache
  (same page, section "KV Cache", step 3);
* multi-canvas decoding: canvas i attends to the prompt cache, to earlier canvases and
  to itself, never to later canvases ("Inference: Fewer, smaller forwards",
  Advancement 1), with each cached entry carrying its own position tag (Advancements
  10 and 11).

Modules: numerics (bit widening), paging (translate, physical tile pages, gather),
mask (dense visibility), attention (softmax attention), tiles (tile classes by brute
force on the dense mask), commit (bitwise scatter into pages).
"""
from .numerics import widen
from .paging import translate, phys_page, gather
from .mask import dense_mask
from .attention import attention, attention_rows
from .tiles import tile_classes, TILE_SKIP, TILE_PARTIAL, TILE_FULL
from .commit import commit

__all__ = [
    "widen", "translate", "phys_page", "gather", "dense_mask", "attention", "attention_rows",
    "tile_classes", "TILE_SKIP", "TILE_PARTIAL", "TILE_FULL", "commit",
]
