"""gfx950 FlashAttention forward: Python binding of libattn.so (placeholder until the HIP library lands)."""
