"""MI355X-native MoE-layer hot path: C-ABI HIP library and its Python binding."""
