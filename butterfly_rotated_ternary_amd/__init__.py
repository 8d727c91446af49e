"""ButterflyMoE expert-layer forward for MI355X (gfx950).

The compute lives in ``libbmoe.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/bmoe.h``). ``butterfly_rotated_ternary_amd.bmoe`` is the
thin Python binding over it; ``workloads`` draws seeded synthetic inputs.
"""
