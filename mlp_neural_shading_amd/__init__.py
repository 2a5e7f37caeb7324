"""Fused FP16 MLP inference on MI355X (gfx950): a C-ABI HIP library and its thin Python binding."""
