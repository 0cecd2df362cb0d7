"""MI355X (gfx950) fused attention forward: a C-ABI HIP library and its thin
Python binding."""
