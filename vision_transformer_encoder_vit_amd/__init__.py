"""MI355X-native pre-LayerNorm ViT encoder block.

The block runs as hand-written HIP kernels for gfx950 behind a C ABI
(``include/vit_block.h``, built into ``libvitblock.so`` next to this file).
``binding`` is the thin ctypes layer over that ABI; it only marshals device
pointers, sizes and the stream. ``synth`` draws the seeded synthetic inputs,
``work`` counts the algorithmic FLOPs and bytes of a workload.

Nothing is imported eagerly, so ``synth`` and ``work`` load on a machine
without the built library or a GPU.
"""
