"""Thin torch-facing wrappers over libmfa's C ABI.

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libmfa. torch supplies device memory and the current stream.
Function names follow the C entry points (mfa_qproj -> ``qproj`` ...).
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import _lib
from ._lib import (BLOCK_TOKENS, MFA_BF16, MFA_F32, MFA_FP8_E4M3, MFA_WEIGHTS_PACKED,
                   MFA_WEIGHTS_ROWMAJOR, check)

_DTYPES = {torch.float32: MFA_F32, torch.bfloat16: MFA_BF16}


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class KVCache:
    """One layer's KV cache in libmfa's block layout (see include/mfa.h).

    k and v hold num_blocks blocks of 64*d elements of the cache dtype (the
    element order inside a block is the library's, written only by
    ``kv_append``); FP8 caches add fp32 k_scale / v_scale [num_blocks][64].
    ``block_table`` [B][max_blocks_per_seq] int32 (None: contiguous,
    sequence b owns blocks b*max_blocks_per_seq ..).
    """

    def __init__(self, num_blocks: int, head_dim: int, dtype: str, max_blocks_per_seq: int,
                 block_table: Optional[torch.Tensor] = None, device="cuda", zero: bool = True):
        self.num_blocks = int(num_blocks)
        self.head_dim = int(head_dim)
        self.dtype = dtype
        self.max_blocks_per_seq = int(max_blocks_per_seq)
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[dtype]
        alloc = torch.zeros if zero else torch.empty
        self.k = alloc((self.num_blocks, BLOCK_TOKENS * self.head_dim), dtype=tdt, device=device)
        self.v = alloc((self.num_blocks, BLOCK_TOKENS * self.head_dim), dtype=tdt, device=device)
        if dtype == "fp8":
            self.k_scale = alloc((self.num_blocks, BLOCK_TOKENS), dtype=torch.float32, device=device)
            self.v_scale = alloc((self.num_blocks, BLOCK_TOKENS), dtype=torch.float32, device=device)
        else:
            self.k_scale = self.v_scale = None
        if block_table is not None:
            _dev(block_table, "block_table")
            if block_table.dtype != torch.int32:
                raise ValueError("block_table must be int32")
        self.block_table = block_table
        self._desc = None

    @property
    def mfa_dtype(self) -> int:
        return {"f32": MFA_F32, "bf16": MFA_BF16, "fp8": MFA_FP8_E4M3}[self.dtype]

    def desc(self) -> _lib.KVCacheDesc:
        d = _lib.KVCacheDesc()
        d.k = self.k.data_ptr()
        d.v = self.v.data_ptr()
        d.k_scale = self.k_scale.data_ptr() if self.k_scale is not None else None
        d.v_scale = self.v_scale.data_ptr() if self.v_scale is not None else None
        d.block_table = self.block_table.data_ptr() if self.block_table is not None else None
        d.num_blocks = self.num_blocks
        d.max_blocks_per_seq = self.max_blocks_per_seq
        d.head_dim = self.head_dim
        d.dtype = self.mfa_dtype
        return d


def qproj_workspace_bytes(batch: int, hidden: int, q_rank: int, heads: int, head_dim: int,
                          dtype: torch.dtype) -> int:
    lib = _lib.load()
    return int(lib.mfa_qproj_workspace_bytes(batch, hidden, q_rank, heads, head_dim,
                                             _DTYPES[dtype]))


def pack_weight(w: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Operand-order packed copy of a bf16 weight [N][K] (mfa_pack_weight).
    The result keeps the logical shape [N][K]; its element order is the
    library's."""
    lib = _lib.load()
    _dev(w, "w")
    N, K = w.shape
    if out is None:
        out = torch.empty_like(w)
    check("mfa_pack_weight", lib.mfa_pack_weight(_ptr(w), _ptr(out), N, K, _DTYPES[w.dtype],
                                                 _stream(w.device)))
    return out


def qproj(x: torch.Tensor, w_qdown: torch.Tensor, q_norm_w: torch.Tensor, w_qup: torch.Tensor,
          heads: int, head_dim: int, eps: float = 1e-6, out: Optional[torch.Tensor] = None,
          workspace: Optional[torch.Tensor] = None, packed: bool = False) -> torch.Tensor:
    """q [B][H][d] = RMSNorm(x W_qdown^T; g, eps) W_qup^T (mfa_qproj). With
    ``packed`` both weights come from ``pack_weight``."""
    lib = _lib.load()
    B, hidden = x.shape
    q_rank = w_qdown.shape[0]
    dt = _DTYPES[x.dtype]
    for t, n in ((x, "x"), (w_qdown, "w_qdown"), (q_norm_w, "q_norm_w"), (w_qup, "w_qup")):
        _dev(t, n)
    if out is None:
        out = torch.empty((B, heads, head_dim), dtype=x.dtype, device=x.device)
    need = int(lib.mfa_qproj_workspace_bytes(B, hidden, q_rank, heads, head_dim, dt))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    layout = MFA_WEIGHTS_PACKED if packed else MFA_WEIGHTS_ROWMAJOR
    check("mfa_qproj", lib.mfa_qproj(_ptr(x), _ptr(w_qdown), _ptr(q_norm_w), _ptr(w_qup),
                                     _ptr(out), _ptr(workspace), workspace.numel(), B, hidden,
                                     q_rank, heads, head_dim, eps, dt, layout,
                                     _stream(x.device)))
    return out


def kv_append(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor,
              pos: torch.Tensor) -> None:
    """Write k_new/v_new [B][n_new][d] (or [B][d]) at positions pos[b].. (mfa_kv_append)."""
    lib = _lib.load()
    if k_new.dim() == 2:
        k_new, v_new = k_new.unsqueeze(1), v_new.unsqueeze(1)
    B, n_new, _ = k_new.shape
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (pos, "pos")):
        _dev(t, n)
    if pos.dtype != torch.int32:
        raise ValueError("pos must be int32")
    desc = cache.desc()
    check("mfa_kv_append", lib.mfa_kv_append(_ptr(k_new), _ptr(v_new), _DTYPES[k_new.dtype],
                                             _ptr(pos), n_new, B, ctypes.byref(desc),
                                             _stream(k_new.device)))


def decode_plan_lens(heads: int, head_dim: int, seq_lens, kv_dtype: str):
    """(num_splits, chunk_tokens) the library picks for these host lengths
    (mfa_decode_plan_lens): the split plan, or (0, 0) for the balanced
    partition."""
    import numpy as np
    lib = _lib.load()
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    ns, ch = ctypes.c_int(), ctypes.c_int()
    check("mfa_decode_plan_lens", lib.mfa_decode_plan_lens(
        len(lens), heads, head_dim, lens.ctypes.data_as(ctypes.c_void_p),
        {"f32": MFA_F32, "bf16": MFA_BF16, "fp8": MFA_FP8_E4M3}[kv_dtype],
        ctypes.byref(ns), ctypes.byref(ch)))
    return ns.value, ch.value


def decode_plan(batch: int, heads: int, head_dim: int, max_seq_len: int, kv_dtype: str):
    """(num_splits, chunk_tokens) the library picks (mfa_decode_plan)."""
    lib = _lib.load()
    ns, ch = ctypes.c_int(), ctypes.c_int()
    check("mfa_decode_plan", lib.mfa_decode_plan(
        batch, heads, head_dim, max_seq_len,
        {"f32": MFA_F32, "bf16": MFA_BF16, "fp8": MFA_FP8_E4M3}[kv_dtype],
        ctypes.byref(ns), ctypes.byref(ch)))
    return ns.value, ch.value


BALANCED = 0   # num_splits value of the balanced (equal-work) partition


def _chunk(max_seq_len: int, num_splits: int) -> int:
    """Tokens per split for num_splits splits (0 for the balanced partition)."""
    if num_splits == BALANCED:
        return 0
    per = -(-max(max_seq_len, 1) // num_splits)
    return -(-per // BLOCK_TOKENS) * BLOCK_TOKENS


def decode_workspace_bytes(batch: int, heads: int, head_dim: int, num_splits: int) -> int:
    """Bytes of split workspace (mfa_decode_workspace_bytes)."""
    return int(_lib.load().mfa_decode_workspace_bytes(batch, heads, head_dim, num_splits))


split_workspace_bytes = decode_workspace_bytes


def decode_attn(q: torch.Tensor, cache: KVCache, seq_lens: torch.Tensor, max_seq_len: int,
                sm_scale: Optional[float] = None, num_splits: int = 1,
                chunk_tokens: Optional[int] = None, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                combine: bool = True) -> Optional[torch.Tensor]:
    """Attention of q [B][H][d] over the cache (mfa_decode_attn).

    num_splits 0 (``BALANCED``) runs the equal-work partition over all the
    batch's cached blocks. With num_splits != 1 and ``combine`` False, only
    the partials are written to ``workspace`` (run ``combine_splits``
    afterwards) and None is returned.
    """
    lib = _lib.load()
    B, H, d = q.shape
    _dev(q, "q")
    _dev(seq_lens, "seq_lens")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if chunk_tokens is None:
        chunk_tokens = _chunk(max_seq_len, num_splits)
    if out_dtype is None:
        out_dtype = q.dtype
    if out is None and (num_splits == 1 or combine):
        out = torch.empty((B, H, d), dtype=out_dtype, device=q.device)
    if num_splits != 1 and workspace is None:
        workspace = torch.empty(split_workspace_bytes(B, H, d, num_splits), dtype=torch.uint8,
                                device=q.device)
    desc = cache.desc()
    check("mfa_decode_attn", lib.mfa_decode_attn(
        _ptr(q), _DTYPES[q.dtype], B, H, ctypes.byref(desc), _ptr(seq_lens), int(max_seq_len),
        float(sm_scale), int(num_splits), int(chunk_tokens), _ptr(workspace),
        workspace.numel() if workspace is not None else 0,
        _ptr(out) if (num_splits == 1 or combine) else None, _DTYPES[out_dtype],
        _stream(q.device)))
    return out if (num_splits == 1 or combine) else None


def decode_attn_multi(q: torch.Tensor, cache: KVCache, seq_lens: torch.Tensor, max_seq_len: int,
                      sm_scale: Optional[float] = None, num_splits: int = 1,
                      chunk_tokens: Optional[int] = None, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None,
                      out_dtype: Optional[torch.dtype] = None,
                      combine: bool = True, fp8_queries: bool = False) -> Optional[torch.Tensor]:
    """Attention of q [B][q_len][H][d] (the last q_len tokens of every sequence,
    causal among themselves) over the cache (mfa_decode_attn_multi); out is
    [B][q_len][H][d]. Splits and ``combine`` as in ``decode_attn``, over the
    B * q_len rows. ``fp8_queries`` (FP8 caches): q quantized per (row, head)
    and Q.K^T on the FP8 matrix cores (mfa_decode_attn_q8)."""
    lib = _lib.load()
    B, T, H, d = q.shape
    _dev(q, "q")
    _dev(seq_lens, "seq_lens")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if chunk_tokens is None:
        chunk_tokens = _chunk(max_seq_len, num_splits)
    if out_dtype is None:
        out_dtype = q.dtype
    if out is None and (num_splits == 1 or combine):
        out = torch.empty((B, T, H, d), dtype=out_dtype, device=q.device)
    if num_splits != 1 and workspace is None:
        workspace = torch.empty(split_workspace_bytes(B * T, H, d, num_splits), dtype=torch.uint8,
                                device=q.device)
    desc = cache.desc()
    fn, name = ((lib.mfa_decode_attn_q8, "mfa_decode_attn_q8") if fp8_queries
                else (lib.mfa_decode_attn_multi, "mfa_decode_attn_multi"))
    check(name, fn(
        _ptr(q), _DTYPES[q.dtype], B, T, H, ctypes.byref(desc), _ptr(seq_lens), int(max_seq_len),
        float(sm_scale), int(num_splits), int(chunk_tokens), _ptr(workspace),
        workspace.numel() if workspace is not None else 0,
        _ptr(out) if (num_splits == 1 or combine) else None, _DTYPES[out_dtype],
        _stream(q.device)))
    return out if (num_splits == 1 or combine) else None


def out_proj(o: torch.Tensor, w_o: torch.Tensor, packed: bool = False, want_y: bool = True,
             want_fp8: bool = True, workspace: Optional[torch.Tensor] = None,
             out: Optional[tuple] = None):
    """Attention output projection y = o W_o^T (bf16) and its per-token FP8
    pack (mfa_out_proj). o [B][HD] (or [B][H][d]); w_o [hidden][HD].
    ``out`` = (y, codes, scales) preallocated (entries may be None).
    Returns (y or None, codes uint8 [B][hidden] or None, scales [B] or None)."""
    lib = _lib.load()
    o2 = o.reshape(o.shape[0], -1)
    _dev(o2, "o")
    _dev(w_o, "w_o")
    B, HD = o2.shape
    hidden = w_o.shape[0]
    dt = _DTYPES[o2.dtype]
    if workspace is None:
        nb = lib.mfa_out_proj_workspace_bytes(B, HD, hidden, dt)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=o.device)
    if out is not None:
        y, codes, scales = out
        for t, name in ((y, "y"), (codes, "codes"), (scales, "scales")):
            if t is not None:
                _dev(t, name)
    else:
        y = torch.empty((B, hidden), dtype=o2.dtype, device=o.device) if want_y else None
        codes = torch.empty((B, hidden), dtype=torch.uint8, device=o.device) if want_fp8 else None
        scales = torch.empty(B, dtype=torch.float32, device=o.device) if want_fp8 else None
    if y is not None and y.numel() != B * hidden:
        raise ValueError("y must hold B x hidden values")
    if codes is not None and (codes.numel() != B * hidden or scales is None or scales.numel() != B):
        raise ValueError("codes must hold B x hidden bytes and scales B floats")
    check("mfa_out_proj", lib.mfa_out_proj(
        _ptr(o2), _ptr(w_o), MFA_WEIGHTS_PACKED if packed else MFA_WEIGHTS_ROWMAJOR, B, HD,
        hidden, dt, _ptr(workspace), workspace.numel(), _ptr(y), _ptr(codes), _ptr(scales),
        _stream(o.device)))
    return y, codes, scales


def combine_splits(workspace: torch.Tensor, batch: int, heads: int, head_dim: int, num_splits: int,
                   out: Optional[torch.Tensor] = None,
                   out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Merge split partials into out [B][H][d] (mfa_combine)."""
    lib = _lib.load()
    _dev(workspace, "workspace")
    if out is None:
        out = torch.empty((batch, heads, head_dim), dtype=out_dtype, device=workspace.device)
    check("mfa_combine", lib.mfa_combine(_ptr(workspace), workspace.numel(), batch, heads,
                                         head_dim, num_splits, _ptr(out), _DTYPES[out.dtype],
                                         _stream(workspace.device)))
    return out


def decode_step(args: "_lib.StepArgs", device) -> None:
    """Run a prepared ``mfa_step_args`` (mfa_decode_step) on the current
    stream of ``device``. The caller keeps the tensors the struct points to
    alive."""
    lib = _lib.load()
    check("mfa_decode_step", lib.mfa_decode_step(ctypes.byref(args), _stream(device)))


def decode_attn_static(q: torch.Tensor, cache: KVCache, seq_lens: torch.Tensor, max_seq_len: int,
                       sm_scale: Optional[float] = None, num_splits: int = 1,
                       chunk_tokens: Optional[int] = None, out: Optional[torch.Tensor] = None,
                       out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """``decode_attn`` with the split partials in the library's own static
    scratch (mfa_decode_attn_static): no workspace is passed and the call
    allocates nothing when ``out`` is given."""
    lib = _lib.load()
    B, H, d = q.shape
    _dev(q, "q")
    _dev(seq_lens, "seq_lens")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if chunk_tokens is None:
        chunk_tokens = _chunk(max_seq_len, num_splits)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else q.dtype
    if out is None:
        out = torch.empty((B, H, d), dtype=out_dtype, device=q.device)
    _dev(out, "out")
    desc = cache.desc()
    check("mfa_decode_attn_static", lib.mfa_decode_attn_static(
        _ptr(q), _DTYPES[q.dtype], B, H, ctypes.byref(desc), _ptr(seq_lens), int(max_seq_len),
        float(sm_scale), int(num_splits), int(chunk_tokens), _ptr(out), _DTYPES[out_dtype],
        _stream(q.device)))
    return out
