"""MI355X-native fused MoE layer: one GPU's share of an expert-parallel MoE.

The compute path is the HIP library ``libmoe.so`` (C ABI in ``include/moe.h``);
``mixture_experts_layer_layout_amd.api`` is its thin ctypes binding and
``mixture_experts_layer_layout_amd.synth`` draws seeded synthetic inputs.
Importing the package loads nothing; importing ``api`` loads the library and
fails loudly if it has not been built.
"""
