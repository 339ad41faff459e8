"""MI355X (gfx950) FlashAttention forward: a C-ABI HIP library and its thin Python binding.

Importing the package does not load the library; the first call through
``exact_io_aware_21_amd.attn`` does, and raises if the built library is missing.
"""
