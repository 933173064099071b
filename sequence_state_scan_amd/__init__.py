"""MI355X-native chunkwise gated linear attention with ZeCO's segment decomposition.

The compute lives in ``libgla.so`` (hand-written HIP for gfx950, C ABI declared in
``include/gla.h``); ``sequence_state_scan_amd.gla`` is the thin ctypes binding over it.
``sequence_state_scan_amd.inputs`` draws the seeded synthetic workloads.
"""
