"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This package holds no step of the quantize / select / attend method. It draws
the random numbers both sides consume: a counter-based Philox4x32-10 stream
turned into approximately normal values, the per-cell and per-channel scale
factors, plans, sequence lengths and block tables. ``synth.philox`` is the
numpy implementation; ``synth/csrc/synth_kernel.hip`` implements the same
published generator on the GPU so that very large caches can be drawn in HBM
without materialising them on the host.
"""
