"""CPU oracle for the pre-LayerNorm ViT encoder block (test infrastructure).

This package is the correctness reference, and nothing else. It is plain,
slow, float64 numpy (plus pure-Python loops for tiny cases), written step by
step from the pages that describe the block:

* "Phase 4: Hiera Backbone MLX Port" (corridorkey-mrp-mlx plan), sections
  "Architecture Summary", "MaskUnitAttention" and "MLP";
* the SigLIP-B/16 vision tower source (franken_ocr 0.8.0,
  ``vision_siglip.rs``), functions ``encoder_block`` and ``self_attention``;
* the SAM3 image model source (cortiq-engine 0.8.44, ``sam3.rs``),
  functions ``layer_norm_rows``, ``apply_rope``, ``run_attn`` and
  ``vit_windows`` and the trunk block loop.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The HIP library never does, and this package
imports nothing from the HIP side: the two share no code. Inputs reach both
from the seeded generator module, which holds none of the block's arithmetic.

Modules:
  block      -- the block forward with every intermediate ("seam")
  index_maps -- Hiera unroll/reroll token orders, mask-unit and spatial
                windows, the 2x2 pooling groups
  brute      -- pure-Python loop versions for tiny shapes (pins for block)

Parity pins: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle.py`` against page-printed values, closed forms,
invariants, library routines or brute force. The whole-block output has no
page-printed value for a known input; it is pinned only through its pinned
steps and the brute force (see the header of ``block``).
"""
