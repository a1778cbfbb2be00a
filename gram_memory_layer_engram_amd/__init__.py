"""Engram layer forward hot path for MI355X (gfx950): HIP kernels behind a C ABI.

The compute lives in ``libengram.so`` (built from ``csrc/``); ``engram`` holds
the thin ctypes binding. ``workloads`` draws seeded synthetic inputs.
"""
