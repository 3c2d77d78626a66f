"""Thin ctypes binding of libloopkv.so (include/loopkv.h).

Argument marshalling only: every step of append and decode runs in the HIP
kernels of the library. torch supplies device memory (tensors) and the stream
(``torch.cuda.current_stream()``). If the library is missing this module raises;
there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LOOPKV_LIB selects another build of the same library (the host-sanitized one, for CPU checks)
LIB_PATH = os.environ.get("LOOPKV_LIB") or os.path.join(_HERE, "libloopkv.so")

OK, ERR_INVALID_ARG, ERR_PLAN, ERR_WORKSPACE, ERR_CAPACITY, ERR_UNSUPPORTED, ERR_HIP = range(7)
CELL_Q4, CELL_Q2, CELL_SHARE = 0, 1, 2
F32, BF16 = 0, 1
LAYOUT_PLANES, LAYOUT_KIVI4 = 0, 1
MAX_LEN = 32768
MAX_CELLS = 128
MAX_SPLIT = 64
NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTED = ["loopkv_create", "loopkv_destroy", "loopkv_plan", "loopkv_workspace_bytes",
            "loopkv_bind_workspace", "loopkv_cell_storage", "loopkv_append", "loopkv_decode_attn",
            "loopkv_split_scratch_bytes", "loopkv_decode_attn_split", "loopkv_decode_attn_split_noalloc",
            "loopkv_decode_attn_skip", "loopkv_plan_search",
            "loopkv_step_graph_create", "loopkv_step_graph_launch", "loopkv_step_graph_destroy", "loopkv_last_error"]


class LoopKVError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"loopkv status {status}: {msg}")
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [("n_loops", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("group_size", ctypes.c_int32), ("block_tokens", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("max_seqs", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32)]


class _CellCost(ctypes.Structure):
    _fields_ = [("damage", ctypes.c_double * 3), ("reads", ctypes.c_double * 3), ("storage", ctypes.c_int64 * 3)]


_lib = None


def lib():
    """Load libloopkv.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    L.loopkv_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(vp)]
    L.loopkv_destroy.argtypes = [vp]
    L.loopkv_destroy.restype = None
    L.loopkv_plan.argtypes = [vp, ctypes.POINTER(ctypes.c_uint8)]
    L.loopkv_workspace_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    L.loopkv_bind_workspace.argtypes = [vp, vp, ctypes.c_size_t]
    L.loopkv_cell_storage.argtypes = [vp, i32, i32, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t),
                                      ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(i32)]
    L.loopkv_append.argtypes = [vp, vp, i32, i32, vp, vp, i32, i32, i32, vp, vp, i32, vp]
    L.loopkv_decode_attn.argtypes = [vp, vp, i32, i32, vp, i32, i32, vp, vp, i32, vp, i32, f32, f32, vp, i32, vp]
    L.loopkv_decode_attn_skip.argtypes = [vp, vp, i32, i32, vp, i32, i32, vp, vp, i32, vp, i32, f32, f32, vp, i32, vp]
    L.loopkv_split_scratch_bytes.argtypes = [vp, i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.loopkv_decode_attn_split.argtypes = [vp, vp, i32, i32, vp, i32, i32, vp, vp, i32, vp, i32, f32, f32, vp, i32,
                                           vp, i32, vp, ctypes.c_size_t]
    L.loopkv_decode_attn_split_noalloc.argtypes = [vp, vp, i32, i32, vp, i32, i32, vp, vp, i32, vp, i32, f32, f32,
                                                   vp, i32, vp, i32]
    L.loopkv_plan_search.argtypes = [i32, i32, ctypes.POINTER(_CellCost), ctypes.c_double, ctypes.c_int64,
                                     ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    L.loopkv_step_graph_create.argtypes = [vp, vp, vp, i32, vp, i32, i32, vp, vp, i32, vp, vp, i32, f32, f32, vp, i32,
                                           vp, i32, vp, ctypes.c_size_t, ctypes.POINTER(vp)]
    L.loopkv_step_graph_launch.argtypes = [vp, vp]
    L.loopkv_step_graph_destroy.argtypes = [vp]
    L.loopkv_step_graph_destroy.restype = None
    L.loopkv_last_error.restype = ctypes.c_char_p
    L.loopkv_last_error.argtypes = []
    for name in ["loopkv_create", "loopkv_plan", "loopkv_workspace_bytes", "loopkv_bind_workspace",
                 "loopkv_cell_storage", "loopkv_append", "loopkv_decode_attn", "loopkv_split_scratch_bytes",
                 "loopkv_decode_attn_split", "loopkv_decode_attn_split_noalloc", "loopkv_decode_attn_skip",
                 "loopkv_plan_search",
                 "loopkv_step_graph_create", "loopkv_step_graph_launch"]:
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int):
    if status != OK:
        raise LoopKVError(status, lib().loopkv_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _dev_i32(t: Optional[torch.Tensor], name: str, numel: Optional[int] = None):
    """A contiguous int32 tensor of at least ``numel`` elements (its device is checked by
    _on_device)."""
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t


def _block_table(bt: torch.Tensor, n_seqs: int):
    """The kernels read n_seqs rows of bt_stride entries: a 2-D table needs at least n_seqs rows;
    a 1-D table is one row, so it serves one sequence only. Returns (table, bt_stride)."""
    _dev_i32(bt, "block_table")
    if bt.dim() == 2:
        if bt.shape[0] < n_seqs or bt.shape[1] < 1:
            raise ValueError(f"block_table of shape {tuple(bt.shape)} has fewer than {n_seqs} rows")
        return bt, int(bt.shape[1])
    if bt.dim() == 1:
        if n_seqs > 1 or bt.numel() < 1:
            raise ValueError("a 1-D block_table is one sequence's row; pass [n_seqs][bt_stride] for more")
        return bt, int(bt.numel())
    raise ValueError("block_table must be [n_seqs][bt_stride] (or one row)")


def _on_device(device, **tensors):
    """Every given tensor must live on the GPU the context's workspace is on (any GPU before a
    workspace is bound): the library passes their addresses to kernels unchecked."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA tensor")
        if device is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, the workspace on {device}")


def plan_search(n_loops: int, n_layers: int, damage, reads, storage, damage_budget: float, storage_budget: int):
    """Least-reads kinds ([n_loops * n_layers] list of CELL_*) under the damage and storage budgets
    (loopkv_plan_search). damage, reads: [cells][3] floats; storage: [cells][3] ints (kind order
    Q4, Q2, SHARE). Returns (kinds, damage, reads, storage); raises LoopKVError (status ERR_PLAN)
    when no plan meets the budgets."""
    n = n_loops * n_layers
    arr = (_CellCost * n)()
    for c in range(n):
        for k in range(3):
            arr[c].damage[k] = float(damage[c][k])
            arr[c].reads[k] = float(reads[c][k])
            arr[c].storage[k] = int(storage[c][k])
    kinds = (ctypes.c_uint8 * n)()
    d, r, st = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
    _check(lib().loopkv_plan_search(n_loops, n_layers, arr, float(damage_budget), int(storage_budget), kinds,
                                    ctypes.byref(d), ctypes.byref(r), ctypes.byref(st)))
    return [int(k) for k in kinds], d.value, r.value, st.value


class Context:
    """One LoopKV cache: config, plan, caller-owned workspace."""

    def __init__(self, n_loops: int, n_layers: int, n_heads: int, head_dim: int, num_blocks: int,
                 max_seqs: int, layout: int = LAYOUT_PLANES, n_kv_heads: int = 0, block_tokens: int = 16,
                 group_size: int = 32):
        """n_kv_heads: KV heads (0: one per query head); query head h reads KV head
        h // (n_heads // n_kv_heads). block_tokens: tokens per page of the block table (16 or
        32); num_blocks counts pages. group_size: quantization group (32 or 64 tokens per K
        group and channels per V group)."""
        self.cfg = _Config(n_loops, n_layers, n_heads, head_dim, group_size, block_tokens, num_blocks, max_seqs,
                           layout, n_kv_heads)
        h = ctypes.c_void_p()
        _check(lib().loopkv_create(ctypes.byref(self.cfg), ctypes.byref(h)))
        self._h = h
        self.workspace = None
        self.kinds = None

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.loopkv_destroy(h)
            self._h = None

    @property
    def kv_heads(self) -> int:
        return self.cfg.n_kv_heads or self.cfg.n_heads

    @property
    def n_cells(self) -> int:
        return self.cfg.n_loops * self.cfg.n_layers

    def plan(self, kinds: Sequence[int]):
        arr = (ctypes.c_uint8 * self.n_cells)(*[int(k) for k in list(kinds)])
        if len(list(kinds)) != self.n_cells:
            raise ValueError(f"plan needs {self.n_cells} kinds")
        _check(lib().loopkv_plan(self._h, arr))
        self.kinds = [int(k) for k in kinds]
        self.workspace = None

    def workspace_bytes(self) -> int:
        n = ctypes.c_size_t()
        _check(lib().loopkv_workspace_bytes(self._h, ctypes.byref(n)))
        return n.value

    def bind(self, ws: torch.Tensor):
        if not ws.is_cuda:
            raise ValueError("workspace must be a CUDA tensor")
        _check(lib().loopkv_bind_workspace(self._h, _ptr(ws), ws.numel() * ws.element_size()))
        self.workspace = ws

    def cell_storage(self, loop: int, layer: int) -> dict:
        p, t, r = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        s = ctypes.c_int32()
        _check(lib().loopkv_cell_storage(self._h, loop, layer, ctypes.byref(p), ctypes.byref(t), ctypes.byref(r),
                                         ctypes.byref(s)))
        return {"pool_offset": p.value, "tail_offset": t.value, "record_bytes": r.value, "storage_cell": s.value}

    def _device(self):
        return None if self.workspace is None else self.workspace.device

    def _cell(self, cell):
        if cell is None:
            return -1, -1
        return int(cell[0]), int(cell[1])

    def append(self, k: torch.Tensor, v: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
               cell=None, seq_slots: Optional[torch.Tensor] = None):
        """k, v: [cells][n_seqs][n_new][H][D] (cell=None) or [n_seqs][n_new][H][D]."""
        loop, layer = self._cell(cell)
        if k.shape != v.shape or not k.is_contiguous() or not v.is_contiguous() or k.dtype != v.dtype:
            raise ValueError("k and v must be contiguous tensors of one shape and dtype")
        if cell is None:
            if k.dim() != 5 or k.shape[0] != self.n_cells:
                raise ValueError("whole-plan append needs k of shape [cells][n_seqs][n_new][H][D]")
            n_seqs, n_new = k.shape[1], k.shape[2]
        else:
            if k.dim() != 4:
                raise ValueError("single-cell append needs k of shape [n_seqs][n_new][H][D]")
            n_seqs, n_new = k.shape[0], k.shape[1]
        if k.shape[-2:] != (self.kv_heads, self.cfg.head_dim):
            raise ValueError("k trailing dims must be [KV heads][D]")
        bt, bt_stride = _block_table(block_table, n_seqs)
        _dev_i32(seq_lens, "seq_lens", n_seqs)
        _dev_i32(seq_slots, "seq_slots", n_seqs)
        _on_device(self._device(), k=k, v=v, block_table=bt, seq_lens=seq_lens, seq_slots=seq_slots)
        _check(lib().loopkv_append(self._h, _stream(), loop, layer, _ptr(k), _ptr(v), _dtype_code(k), n_seqs, n_new,
                                   _ptr(seq_slots), _ptr(bt), bt_stride, _ptr(seq_lens)))

    def split_scratch_bytes(self, n_seqs: int, max_len: int, n_split: int, cell=None) -> int:
        loop, layer = self._cell(cell)
        n = ctypes.c_size_t()
        _check(lib().loopkv_split_scratch_bytes(self._h, loop, layer, int(n_seqs), int(max_len), int(n_split),
                                                ctypes.byref(n)))
        return n.value

    def step_graph(self, k, v, q, block_table, lens_before, lens_after, max_len: int, tau: float, out,
                   sel_mask=None, n_split: int = 0, scratch=None, sm_scale=None, seq_slots=None) -> "StepGraph":
        """Capture one serving step of every cell (loopkv_step_graph_create): k, v [cells][B][1][KV
        heads][D]; q, out [cells][B][H][D]; lens_before / lens_after advance by one per launch."""
        return StepGraph(self, k, v, q, block_table, lens_before, lens_after, max_len, tau, out, sel_mask, n_split,
                         scratch, sm_scale, seq_slots)

    def decode(self, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor, max_len: int,
               tau: float, sm_scale: Optional[float] = None, cell=None, out_dtype=torch.float32,
               out: Optional[torch.Tensor] = None, sel_mask=False, seq_slots: Optional[torch.Tensor] = None,
               n_split: int = 0, scratch: Optional[torch.Tensor] = None, skip: bool = False,
               no_alloc: bool = False):
        """q: [cells][n_seqs][H][D] (cell=None) or [n_seqs][H][D]. Returns out (and sel_mask if asked).
        n_split > 0 splits each row over that many workgroups (loopkv_decode_attn_split); scratch is
        then a CUDA tensor of at least split_scratch_bytes() bytes (allocated here if None).
        skip=True runs the token-skipping ablation (loopkv_decode_attn_skip), not the method.
        no_alloc=True (with n_split > 0) runs loopkv_decode_attn_split_noalloc: the split scratch is
        the library's fixed device array (NOALLOC_SCRATCH_BYTES), nothing is allocated."""
        loop, layer = self._cell(cell)
        if not q.is_contiguous():
            raise ValueError("q must be contiguous")
        n_seqs = q.shape[1] if cell is None else q.shape[0]
        if (cell is None and (q.dim() != 4 or q.shape[0] != self.n_cells)) or (cell is not None and q.dim() != 3):
            raise ValueError("q has the wrong rank for this call")
        if q.shape[-2:] != (self.cfg.n_heads, self.cfg.head_dim):
            raise ValueError("q trailing dims must be [query heads][D]")
        D = self.cfg.head_dim
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(D)
        if out is None:
            out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
        if out.shape != q.shape or not out.is_contiguous():
            raise ValueError("out must be contiguous with q's shape")
        _dtype_code(q)
        _dtype_code(out)
        words = (int(max_len) + 31) // 32
        sm = None
        if sel_mask is True:
            sm = torch.zeros((*q.shape[:-1], words), dtype=torch.int32, device=q.device)
        elif isinstance(sel_mask, torch.Tensor):
            # the kernels write rows x ceil(max_len / 32) words
            sm = _dev_i32(sel_mask, "sel_mask", q.numel() // D * words)
        elif sel_mask not in (False, None):
            raise ValueError("sel_mask must be True, False/None or an int32 tensor")
        bt, bt_stride = _block_table(block_table, n_seqs)
        _dev_i32(seq_lens, "seq_lens", n_seqs)
        _dev_i32(seq_slots, "seq_slots", n_seqs)
        if scratch is not None and not scratch.is_contiguous():
            raise ValueError("scratch must be a contiguous CUDA tensor")
        _on_device(self._device(), q=q, out=out, sel_mask=sm, block_table=bt, seq_lens=seq_lens,
                   seq_slots=seq_slots, scratch=scratch)
        if no_alloc and (skip or not n_split):
            raise ValueError("no_alloc is the split decode's variant: give n_split > 0")
        if skip:
            if n_split:
                raise ValueError("the token-skipping ablation runs one workgroup per row (n_split=0)")
            _check(lib().loopkv_decode_attn_skip(self._h, _stream(), loop, layer, _ptr(q), _dtype_code(q), n_seqs,
                                                 _ptr(seq_slots), _ptr(bt), bt_stride, _ptr(seq_lens), int(max_len),
                                                 float(tau), float(sm_scale), _ptr(out), _dtype_code(out), _ptr(sm)))
        elif n_split and no_alloc:
            if scratch is not None:
                raise ValueError("no_alloc takes no scratch")
            _check(lib().loopkv_decode_attn_split_noalloc(self._h, _stream(), loop, layer, _ptr(q), _dtype_code(q),
                                                          n_seqs, _ptr(seq_slots), _ptr(bt), bt_stride,
                                                          _ptr(seq_lens), int(max_len), float(tau), float(sm_scale),
                                                          _ptr(out), _dtype_code(out), _ptr(sm), int(n_split)))
        elif n_split:
            if scratch is None:
                scratch = torch.empty(self.split_scratch_bytes(n_seqs, max_len, n_split, cell), dtype=torch.uint8,
                                      device=q.device)
            _check(lib().loopkv_decode_attn_split(self._h, _stream(), loop, layer, _ptr(q), _dtype_code(q), n_seqs,
                                                  _ptr(seq_slots), _ptr(bt), bt_stride, _ptr(seq_lens), int(max_len),
                                                  float(tau), float(sm_scale), _ptr(out), _dtype_code(out), _ptr(sm),
                                                  int(n_split), _ptr(scratch),
                                                  scratch.numel() * scratch.element_size()))
        else:
            _check(lib().loopkv_decode_attn(self._h, _stream(), loop, layer, _ptr(q), _dtype_code(q), n_seqs,
                                            _ptr(seq_slots), _ptr(bt), bt_stride, _ptr(seq_lens), int(max_len),
                                            float(tau), float(sm_scale), _ptr(out), _dtype_code(out), _ptr(sm)))
        if sm is not None:
            return out, sm
        return out


class StepGraph:
    """One serving step (every cell in order: append the token, decode the cell; then both
    length arrays advance by one) captured into a HIP graph by loopkv_step_graph_create.
    Holds the tensors it was built on; refill k, v and q between launches."""

    def __init__(self, ctx: "Context", k, v, q, block_table, lens_before, lens_after, max_len: int, tau: float,
                 out, sel_mask=None, n_split: int = 0, scratch=None, sm_scale=None, seq_slots=None):
        C, H, D, KVH = ctx.n_cells, ctx.cfg.n_heads, ctx.cfg.head_dim, ctx.kv_heads
        if q.dim() != 4:
            raise ValueError("q must be [cells][n_seqs][H][D]")
        n_seqs = q.shape[1]
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(D)
        # the captured launches stride k, v over every cell (a reuse cell's slice is unread) and q,
        # out, sel_mask over every cell
        if tuple(k.shape) != (C, n_seqs, 1, KVH, D) or tuple(v.shape) != tuple(k.shape):
            raise ValueError(f"k and v must be [{C} cells][{n_seqs}][1][{KVH}][{D}]")
        if tuple(q.shape) != (C, n_seqs, H, D) or tuple(out.shape) != tuple(q.shape):
            raise ValueError(f"q and out must be [{C} cells][n_seqs][{H}][{D}]")
        if k.dtype != v.dtype:
            raise ValueError("k and v must share a dtype")
        for name, t in (("k", k), ("v", v), ("q", q), ("out", out)):
            _dtype_code(t)
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        if sel_mask is not None:
            _dev_i32(sel_mask, "sel_mask", C * n_seqs * H * ((int(max_len) + 31) // 32))
        bt, bt_stride = _block_table(block_table, n_seqs)
        _dev_i32(lens_before, "lens_before", n_seqs)
        _dev_i32(lens_after, "lens_after", n_seqs)
        _dev_i32(seq_slots, "seq_slots", n_seqs)
        if scratch is not None and not scratch.is_contiguous():
            raise ValueError("scratch must be a contiguous CUDA tensor")
        _on_device(ctx._device(), k=k, v=v, q=q, out=out, sel_mask=sel_mask, block_table=bt,
                   lens_before=lens_before, lens_after=lens_after, seq_slots=seq_slots, scratch=scratch)
        if n_split and scratch is None:
            scratch = torch.empty(ctx.split_scratch_bytes(n_seqs, max_len, n_split, (0, 0)), dtype=torch.uint8,
                                  device=q.device)
        self._keep = (ctx, k, v, q, bt, lens_before, lens_after, out, sel_mask, scratch, seq_slots)
        h = ctypes.c_void_p()
        nbytes = 0 if scratch is None else scratch.numel() * scratch.element_size()
        _check(lib().loopkv_step_graph_create(ctx._h, _ptr(k), _ptr(v), _dtype_code(k), _ptr(q), _dtype_code(q),
                                              n_seqs, _ptr(seq_slots), _ptr(bt), bt_stride, _ptr(lens_before),
                                              _ptr(lens_after), int(max_len), float(tau), float(sm_scale), _ptr(out),
                                              _dtype_code(out), _ptr(sel_mask), int(n_split), _ptr(scratch), nbytes,
                                              ctypes.byref(h)))
        self._h = h

    def launch(self):
        _check(lib().loopkv_step_graph_launch(self._h, _stream()))

    def close(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.loopkv_step_graph_destroy(h)
        self._h = None

    def __del__(self):
        self.close()

