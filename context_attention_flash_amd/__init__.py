"""Python binding of libringattn.so (the ring-attention rank-share C ABI).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  PyTorch supplies device memory and streams.  If the
library has not been built, every call raises RuntimeError; there is no
fallback path.

The functions carry the names of the C entry points (include/ring_attn.h).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from .synth import BASIC, ZIGZAG, STRIPE, VARLEN_RING, LLAMA3, VARLEN_ZIGZAG, VARLEN_STRIPE  # noqa: F401

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libringattn.so")

RA_F32, RA_BF16 = 0, 1
RA_MERGE_FUSED, RA_MERGE_SEPARATE, RA_MERGE_STEPWISE = 0, 1, 2

ERRORS = {
    -1: "RA_E_NULL", -2: "RA_E_SHAPE", -3: "RA_E_WORLD", -4: "RA_E_DIVISIBILITY",
    -5: "RA_E_CU_SEQLENS", -6: "RA_E_HEADS", -7: "RA_E_UNSUPPORTED", -8: "RA_E_WORKSPACE",
    -9: "RA_E_LAYOUT", -10: "RA_E_HIP", -11: "RA_E_ARG", -12: "RA_E_NO_PLAN", -13: "RA_E_SCRATCH",
}


class RingAttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("seqlen", ctypes.c_int64), ("world", ctypes.c_int32),
        ("rank", ctypes.c_int32), ("causal", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("n_seqs", ctypes.c_int32),
        ("merge_mode", ctypes.c_int32), ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
    ]


class RingAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {ERRORS.get(code, code)} ({ring_attn_strerror(code)})")


_lib = None

_P = ctypes.c_void_p
_DP = ctypes.POINTER(RingAttnDesc)
_SIGS = {
    "ring_attn_workspace_bytes": (ctypes.c_int64, [_DP, ctypes.c_int]),
    "ring_attn_bwd_ds_bytes": (ctypes.c_int64, [_DP, _P]),
    "ring_attn_fwd_split_bytes": (ctypes.c_int64, [_DP]),
    "ring_attn_fwd": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "ring_attn_bwd": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     ctypes.c_size_t, _P]),
    "ring_attn_bwd_noalloc": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "ring_attn_noalloc_scratch_bytes": (ctypes.c_int64, []),
    "ring_attn_lse_merge": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, ctypes.c_int64,
                                           ctypes.c_int32, ctypes.c_int32, _P]),
    "ring_attn_positions": (ctypes.c_int, [_DP, _P, ctypes.c_int32, _P]),
    "ring_attn_kv_positions": (ctypes.c_int, [_DP, _P, ctypes.c_int32, _P]),
    "ring_attn_schedule": (ctypes.c_int, [_DP, _P, _P, _P, _P]),
    "ring_attn_tile_kinds": (ctypes.c_int, [_DP, _P, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, _P]),
    "ring_attn_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "ring_attn_timing_read": (ctypes.c_int, [ctypes.c_char_p, _P, _P]),
    "ring_attn_clear_cache": (ctypes.c_int, []),
    "ring_attn_plan_cache_limit": (ctypes.c_int, [ctypes.c_int32]),
    "ring_attn_plan_cache_info": (ctypes.c_int, [_P, _P]),
    "ring_attn_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "ring_attn_version": (ctypes.c_int, []),
}


def lib() -> ctypes.CDLL:
    """Load libringattn.so (built in-tree by build_lib.py); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m context_attention_flash_amd.build_lib`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc: int, where: str):
    if rc != 0:
        raise RingAttnError(rc, where)


def ring_attn_strerror(code: int) -> str:
    return lib().ring_attn_strerror(code).decode()


def ring_attn_version() -> int:
    return lib().ring_attn_version()


def make_desc(batch, heads_q, heads_kv, head_dim, seqlen, world, rank, causal, layout,
              dtype="bf16", softmax_scale=0.0, cu_seqlens: Optional[Sequence[int]] = None,
              merge_mode=RA_MERGE_FUSED, window=(-1, -1)) -> RingAttnDesc:
    d = RingAttnDesc()
    d.batch, d.heads_q, d.heads_kv, d.head_dim = batch, heads_q, heads_kv, head_dim
    d.seqlen, d.world, d.rank, d.causal, d.layout = seqlen, world, rank, int(causal), layout
    d.dtype = RA_BF16 if dtype in ("bf16", RA_BF16) else (RA_F32 if dtype in ("f32", RA_F32) else dtype)
    d.softmax_scale = float(softmax_scale)
    d.n_seqs = 0 if cu_seqlens is None else len(cu_seqlens) - 1
    d.merge_mode = merge_mode
    d.window_left, d.window_right = int(window[0]), int(window[1])
    return d


def desc_from_workload(w, rank=None, merge_mode=RA_MERGE_FUSED) -> RingAttnDesc:
    return make_desc(w.batch, w.heads_q, w.heads_kv, w.head_dim, w.seqlen, w.world,
                     w.rank if rank is None else rank, w.causal, w.layout, w.dtype,
                     cu_seqlens=w.cu_seqlens, merge_mode=merge_mode, window=w.window)


def _cu_arg(cu):
    if cu is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(cu, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def shard_sizes(desc: RingAttnDesc):
    """(S, Skv, n_blocks) of a descriptor."""
    S = desc.seqlen // desc.world
    if desc.layout == LLAMA3:
        return S, desc.seqlen, 1
    return S, S, desc.world


def ring_attn_workspace_bytes(desc: RingAttnDesc, is_bwd: bool) -> int:
    n = lib().ring_attn_workspace_bytes(ctypes.byref(desc), int(is_bwd))
    if n < 0:
        raise RingAttnError(int(n), "ring_attn_workspace_bytes")
    return int(n)


def ring_attn_fwd_split_bytes(desc: RingAttnDesc) -> int:
    """Extra forward workspace that lets long query-tile lists be split
    across CUs (0 when the descriptor's path never splits)."""
    n = lib().ring_attn_fwd_split_bytes(ctypes.byref(desc))
    if n < 0:
        raise RingAttnError(int(n), "ring_attn_fwd_split_bytes")
    return int(n)


def ring_attn_bwd_ds_bytes(desc: RingAttnDesc, cu_seqlens=None) -> int:
    keep, cu = _cu_arg(cu_seqlens)
    n = lib().ring_attn_bwd_ds_bytes(ctypes.byref(desc), cu)
    if n < 0:
        raise RingAttnError(int(n), "ring_attn_bwd_ds_bytes")
    return int(n)


# The binding gives the backward the dS tile store when it needs at most this
# many bytes (callers who pass their own workspace decide for themselves).
DS_STORE_LIMIT = 16 << 30


def ring_attn_positions(desc: RingAttnDesc, cu_seqlens=None, rank: Optional[int] = None) -> np.ndarray:
    S, _, _ = shard_sizes(desc)
    out = np.empty(S, np.int64)
    keep, cu = _cu_arg(cu_seqlens)
    _check(lib().ring_attn_positions(ctypes.byref(desc), cu, desc.rank if rank is None else rank,
                                     out.ctypes.data_as(ctypes.c_void_p)), "ring_attn_positions")
    return out


def ring_attn_kv_positions(desc: RingAttnDesc, cu_seqlens, block: int) -> np.ndarray:
    _, Skv, _ = shard_sizes(desc)
    out = np.empty(Skv, np.int64)
    keep, cu = _cu_arg(cu_seqlens)
    _check(lib().ring_attn_kv_positions(ctypes.byref(desc), cu, block,
                                        out.ctypes.data_as(ctypes.c_void_p)), "ring_attn_kv_positions")
    return out


def ring_attn_schedule(desc: RingAttnDesc, cu_seqlens=None):
    """[(step, block, pairs)] for desc.rank."""
    _, _, nb = shard_sizes(desc)
    blocks = np.zeros(max(nb, 1), np.int32)
    pairs = np.zeros(max(nb, 1), np.int64)
    n = ctypes.c_int32(0)
    keep, cu = _cu_arg(cu_seqlens)
    _check(lib().ring_attn_schedule(ctypes.byref(desc), cu, blocks.ctypes.data_as(ctypes.c_void_p),
                                    pairs.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n)),
           "ring_attn_schedule")
    return [(s, int(blocks[s]), int(pairs[s])) for s in range(n.value)]


def ring_attn_tile_kinds(desc: RingAttnDesc, cu_seqlens, step: int, tile_q: int, tile_k: int):
    S, Skv, _ = shard_sizes(desc)
    nqt, nkt = -(-S // tile_q), -(-Skv // tile_k)
    out = np.zeros((nqt, nkt), np.int8)
    keep, cu = _cu_arg(cu_seqlens)
    _check(lib().ring_attn_tile_kinds(ctypes.byref(desc), cu, step, tile_q, tile_k,
                                      out.ctypes.data_as(ctypes.c_void_p)), "ring_attn_tile_kinds")
    return out


# ---------------------------------------------------------------------------
# Device entry points (torch tensors -> pointers)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _expect(t, shape, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.data_ptr() % 16:
        raise ValueError(f"{name}: must be 16-byte aligned")
    return ctypes.c_void_p(t.data_ptr())


def _shapes(desc):
    S, Skv, nb = shard_sizes(desc)
    B, Hq, Hkv, d = desc.batch, desc.heads_q, desc.heads_kv, desc.head_dim
    return dict(q=(B, S, Hq, d), kv=(nb, B, Skv, Hkv, d), lse=(B, Hq, S))


def _elem_dtype(desc):
    torch = _torch()
    return torch.bfloat16 if desc.dtype == RA_BF16 else torch.float32


def alloc_workspace(desc: RingAttnDesc, is_bwd: bool, device="cuda", cu_seqlens=None,
                    ds_store: bool = True):
    """Workspace for the forward or the backward.  The forward one includes
    the part buffer that lets long query-tile lists be split across CUs; with
    ``ds_store`` the backward one includes the dS tile store, whole or (beyond
    DS_STORE_LIMIT) for as many kv heads at a time as fit the limit."""
    torch = _torch()
    n = ring_attn_workspace_bytes(desc, is_bwd)
    if not is_bwd:
        n += ring_attn_fwd_split_bytes(desc)
    if is_bwd and ds_store:
        full = ring_attn_bwd_ds_bytes(desc, cu_seqlens)
        per_kv_head = -(-full // desc.heads_kv)
        if full <= DS_STORE_LIMIT:
            n += full
        elif per_kv_head <= DS_STORE_LIMIT:   # kv heads in several passes
            n += DS_STORE_LIMIT // per_kv_head * per_kv_head
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def ring_attn_fwd(desc: RingAttnDesc, q, k, v, cu_seqlens=None, out=None, lse=None,
                  workspace=None, stream=None):
    """Forward of the rank share; returns (out, lse).  Allocates out, lse and
    the workspace with torch when they are not given."""
    torch = _torch()
    sh = _shapes(desc)
    dt = _elem_dtype(desc)
    if out is None:
        out = torch.empty(sh["q"], dtype=dt, device=q.device)
    if lse is None:
        lse = torch.empty(sh["lse"], dtype=torch.float32, device=q.device)
    args = [_expect(q, sh["q"], dt, "q"), _expect(k, sh["kv"], dt, "k"), _expect(v, sh["kv"], dt, "v"),
            _expect(out, sh["q"], dt, "out"), _expect(lse, sh["lse"], torch.float32, "lse")]
    if workspace is None:
        workspace = alloc_workspace(desc, False, q.device)
    keep, cu = _cu_arg(cu_seqlens)
    rc = lib().ring_attn_fwd(ctypes.byref(desc), *args[:3], cu, *args[3:],
                             ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                             _stream_ptr(stream))
    _check(rc, "ring_attn_fwd")
    return out, lse


def ring_attn_bwd(desc: RingAttnDesc, dout, q, k, v, out, lse, cu_seqlens=None, dq=None,
                  dk=None, dv=None, workspace=None, stream=None):
    """Backward of the rank share; dq is overwritten, dk/dv are accumulated
    (allocated zeroed when not given).  Returns (dq, dk, dv)."""
    torch = _torch()
    sh = _shapes(desc)
    dt = _elem_dtype(desc)
    f32 = torch.float32
    if dq is None:
        dq = torch.empty(sh["q"], dtype=f32, device=q.device)
    if dk is None:
        dk = torch.zeros(sh["kv"], dtype=f32, device=q.device)
    if dv is None:
        dv = torch.zeros(sh["kv"], dtype=f32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(desc, True, q.device, cu_seqlens)
    keep, cu = _cu_arg(cu_seqlens)
    rc = lib().ring_attn_bwd(ctypes.byref(desc), _expect(dout, sh["q"], dt, "dout"),
                             _expect(q, sh["q"], dt, "q"), _expect(k, sh["kv"], dt, "k"),
                             _expect(v, sh["kv"], dt, "v"), _expect(out, sh["q"], dt, "out"),
                             _expect(lse, sh["lse"], f32, "lse"), cu,
                             _expect(dq, sh["q"], f32, "dq"), _expect(dk, sh["kv"], f32, "dk"),
                             _expect(dv, sh["kv"], f32, "dv"),
                             ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                             _stream_ptr(stream))
    _check(rc, "ring_attn_bwd")
    return dq, dk, dv


def ring_attn_bwd_noalloc(desc: RingAttnDesc, dout, q, k, v, out, lse, dq, dk, dv,
                          cu_seqlens=None, stream=None):
    """ring_attn_bwd with the library's static scratch as workspace: allocates
    nothing (every tensor is the caller's); the shape's plan must exist."""
    torch = _torch()
    sh = _shapes(desc)
    dt = _elem_dtype(desc)
    f32 = torch.float32
    keep, cu = _cu_arg(cu_seqlens)
    rc = lib().ring_attn_bwd_noalloc(ctypes.byref(desc), _expect(dout, sh["q"], dt, "dout"),
                                     _expect(q, sh["q"], dt, "q"), _expect(k, sh["kv"], dt, "k"),
                                     _expect(v, sh["kv"], dt, "v"), _expect(out, sh["q"], dt, "out"),
                                     _expect(lse, sh["lse"], f32, "lse"), cu,
                                     _expect(dq, sh["q"], f32, "dq"), _expect(dk, sh["kv"], f32, "dk"),
                                     _expect(dv, sh["kv"], f32, "dv"), _stream_ptr(stream))
    _check(rc, "ring_attn_bwd_noalloc")
    return dq, dk, dv


def ring_attn_noalloc_scratch_bytes() -> int:
    return int(lib().ring_attn_noalloc_scratch_bytes())


def ring_attn_lse_merge(out, lse, out_j, lse_j, stream=None):
    """In-place LSE merge; out/out_j fp32 [B, S, H, d], lse/lse_j fp32 [B, H, S]."""
    torch = _torch()
    B, S, H, d = out.shape
    f32 = torch.float32
    rc = lib().ring_attn_lse_merge(_expect(out, (B, S, H, d), f32, "out"),
                                   _expect(lse, (B, H, S), f32, "lse"),
                                   _expect(out_j, (B, S, H, d), f32, "out_j"),
                                   _expect(lse_j, (B, H, S), f32, "lse_j"), B, S, H, d,
                                   _stream_ptr(stream))
    _check(rc, "ring_attn_lse_merge")
    return out, lse


def ring_attn_timing_enable(enable: bool):
    _check(lib().ring_attn_timing_enable(int(enable)), "ring_attn_timing_enable")


def ring_attn_timing_read(name: str):
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _check(lib().ring_attn_timing_read(name.encode(), ctypes.byref(n), ctypes.byref(ms)),
           "ring_attn_timing_read")
    return int(n.value), float(ms.value)


def ring_attn_clear_cache():
    _check(lib().ring_attn_clear_cache(), "ring_attn_clear_cache")


def ring_attn_plan_cache_limit(max_plans: int) -> int:
    """Set the most plans the library caches; returns the previous limit."""
    rc = lib().ring_attn_plan_cache_limit(int(max_plans))
    if rc < 0:
        raise RingAttnError(rc, "ring_attn_plan_cache_limit")
    return int(rc)


def ring_attn_plan_cache_info():
    """(number of cached plans, device bytes they hold)."""
    n = ctypes.c_int64(0)
    b = ctypes.c_int64(0)
    _check(lib().ring_attn_plan_cache_info(ctypes.byref(n), ctypes.byref(b)),
           "ring_attn_plan_cache_info")
    return int(n.value), int(b.value)
