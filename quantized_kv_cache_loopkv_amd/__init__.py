"""LoopKV loop-aware decode attention over a per-(loop, layer) mixed-precision KV cache, for MI355X.

The compute path is the HIP library ``libloopkv.so`` (C ABI in include/loopkv.h);
``quantized_kv_cache_loopkv_amd.loopkv`` is its ctypes binding.
"""
from .loopkv import (Context, StepGraph, LoopKVError, lib, plan_search, CELL_Q4, CELL_Q2, CELL_SHARE, F32, BF16,  # noqa: F401
                     LAYOUT_PLANES, LAYOUT_KIVI4, MAX_LEN, MAX_SPLIT, MAX_CELLS, EXPORTED)
