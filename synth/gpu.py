"""ctypes binding of synth/libloopkv_synth.so: the seeded generator drawn directly in HBM.

Produces the same bits as ``synth.philox`` (the tests check it) so that caches
too large for host memory can be built on the GPU.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libloopkv_synth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.synth_kv_bf16.argtypes = [vp, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
        L.synth_kv_bf16.restype = ctypes.c_int
        L.synth_normal.argtypes = [vp, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_int, vp]
        L.synth_normal.restype = ctypes.c_int
        L.synth_stream_read.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int, vp]
        L.synth_stream_read.restype = ctypes.c_int
        L.synth_chunk_read.argtypes = [vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
        L.synth_chunk_read.restype = ctypes.c_int
        _lib = L
    return _lib


def _s():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def kv_bf16(seed: int, stream: int, B: int, n_tok: int, t0: int, T: int, H: int, D: int,
            factors: torch.Tensor, out: torch.Tensor, t0s: torch.Tensor = None):
    """Fill out (bf16 [B][n_tok][H][D]) with stream values of tokens t0 + i (or t0s[b] + i)."""
    assert out.dtype == torch.bfloat16 and out.is_contiguous() and out.numel() == B * n_tok * H * D
    assert factors.dtype == torch.float32 and factors.is_cuda and factors.numel() == H * D
    r = lib().synth_kv_bf16(_s(), seed, stream, B, n_tok, t0, None if t0s is None else ctypes.c_void_p(t0s.data_ptr()),
                            T, H, D, ctypes.c_void_p(factors.data_ptr()), ctypes.c_void_p(out.data_ptr()))
    if r != 0:
        raise RuntimeError(f"synth_kv_bf16 failed: {r}")
    return out


def normal(seed: int, stream: int, offset: int, out: torch.Tensor):
    """Fill out (bf16 or float32, contiguous) with draws offset .. offset + numel - 1."""
    assert out.is_contiguous() and out.dtype in (torch.bfloat16, torch.float32)
    r = lib().synth_normal(_s(), seed, stream, offset, out.numel(), int(out.dtype == torch.bfloat16),
                           ctypes.c_void_p(out.data_ptr()))
    if r != 0:
        raise RuntimeError(f"synth_normal failed: {r}")
    return out


def read_ceiling(n_bytes: int = 16 << 30, record_bytes: int = 2560, chunk_bytes: int = 768, reps: int = 3) -> dict:
    """Practical HBM read rates on this device: a streaming read of ``n_bytes`` (contiguous
    spans per workgroup, nontemporal loads), and
    ``chunk_bytes`` reads at the starts of ``record_bytes`` records in a seeded random order
    (the shape of the decode's per-block reads). Returns GB/s for both."""
    buf = torch.empty(n_bytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    blocks = 256 * 32
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    L = lib()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sblocks = 4096   # contiguous spans of 4 MB per workgroup at 16 GiB
    L.synth_stream_read(_s(), ctypes.c_void_p(buf.data_ptr()), n_bytes // 16, sblocks, ctypes.c_void_p(out.data_ptr()))
    ev0.record()
    for _ in range(reps):
        L.synth_stream_read(_s(), ctypes.c_void_p(buf.data_ptr()), n_bytes // 16, sblocks,
                            ctypes.c_void_p(out.data_ptr()))
    ev1.record()
    torch.cuda.synchronize()
    stream_gbs = reps * n_bytes / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    n_chunks = n_bytes // record_bytes
    g = torch.Generator(device="cpu").manual_seed(0)
    order = torch.randperm(n_chunks, generator=g).to(torch.int32).cuda()
    L.synth_chunk_read(_s(), ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(order.data_ptr()), n_chunks, record_bytes,
                       chunk_bytes, blocks, ctypes.c_void_p(out.data_ptr()))
    ev0.record()
    for _ in range(reps):
        L.synth_chunk_read(_s(), ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(order.data_ptr()), n_chunks,
                           record_bytes, chunk_bytes, blocks, ctypes.c_void_p(out.data_ptr()))
    ev1.record()
    torch.cuda.synchronize()
    chunk_gbs = reps * n_chunks * chunk_bytes / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return {"stream_read_GBps": round(stream_gbs, 1), "record_chunk_read_GBps": round(chunk_gbs, 1),
            "chunk_bytes": chunk_bytes, "record_bytes": record_bytes, "buffer_GB": n_bytes / 1e9}
