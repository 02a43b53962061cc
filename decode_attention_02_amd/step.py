"""One MFA decode step through libmfa: query path, KV append, attention,
split combine, on the current stream. Marshalling only; each stage is one
C-ABI call (mfa_qproj, mfa_kv_append, mfa_decode_attn, mfa_combine).

Also fills a cache from prompt tokens (mfa_kv_append with n_new > 1).
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import _lib, api
from ._lib import check


class DecodeStep:
    """Pre-planned decode step for B sequences of at most ``max_seq_len`` tokens.
    With ``seq_lens_host`` (the lengths the step will attend) and no
    ``num_splits``, the library plans from the lengths (mfa_decode_plan_lens).

    Workspaces (query-path partials, split partials) and outputs are
    allocated once here, so calling the step allocates nothing.
    """

    def __init__(self, cache: api.KVCache, batch: int, heads: int, max_seq_len: int,
                 hidden: Optional[int] = None, q_rank: Optional[int] = None,
                 act_dtype: torch.dtype = torch.bfloat16, num_splits: Optional[int] = None,
                 chunk_tokens: Optional[int] = None, eps: float = 1e-6,
                 out_dtype: Optional[torch.dtype] = None, sm_scale: Optional[float] = None,
                 packed_weights: bool = False, device="cuda", seq_lens_host=None):
        self.cache = cache
        self.B, self.H, self.d = batch, heads, cache.head_dim
        self.max_seq_len = int(max_seq_len)
        self.hidden, self.q_rank = hidden, q_rank
        self.act_dtype = act_dtype
        self.eps = eps
        self.packed_weights = packed_weights
        self.sm_scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(self.d)
        if num_splits is None and seq_lens_host is not None:
            # the plan from the batch's lengths (balanced partition for mixed ones)
            num_splits, chunk_tokens = api.decode_plan_lens(heads, self.d, seq_lens_host,
                                                            cache.dtype)
        elif num_splits is None:
            num_splits, chunk_tokens = api.decode_plan(batch, heads, self.d, self.max_seq_len,
                                                       cache.dtype)
        elif chunk_tokens is None:
            chunk_tokens = api._chunk(self.max_seq_len, num_splits)
        self.num_splits, self.chunk_tokens = int(num_splits), int(chunk_tokens)
        self.out_dtype = out_dtype or act_dtype
        self.out = torch.empty((batch, heads, self.d), dtype=self.out_dtype, device=device)
        self.q = torch.empty((batch, heads, self.d), dtype=act_dtype, device=device)
        nbytes = api.split_workspace_bytes(batch, heads, self.d, self.num_splits)
        self.split_ws = (torch.empty(nbytes, dtype=torch.uint8, device=device)
                         if nbytes else None)
        self.qproj_ws = None
        if hidden is not None:
            nb = api.qproj_workspace_bytes(batch, hidden, q_rank, heads, self.d, act_dtype)
            self.qproj_ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=device)
        self._desc = cache.desc()
        self._lib = _lib.load()

    # -- stages ---------------------------------------------------------
    def query(self, x, w_qdown, g, w_qup):
        return api.qproj(x, w_qdown, g, w_qup, self.H, self.d, self.eps, out=self.q,
                         workspace=self.qproj_ws, packed=self.packed_weights)

    def append(self, k_new, v_new, pos):
        api.kv_append(self.cache, k_new, v_new, pos)

    def attend(self, q, seq_lens, combine_separately: bool = True):
        """Attention (+ combine). ``combine_separately`` runs mfa_combine as its
        own call; otherwise mfa_decode_attn merges into ``out`` itself."""
        if self.num_splits == 1:
            return api.decode_attn(q, self.cache, seq_lens, self.max_seq_len, self.sm_scale, 1,
                                   self.chunk_tokens, out=self.out)
        if combine_separately:
            api.decode_attn(q, self.cache, seq_lens, self.max_seq_len, self.sm_scale,
                            self.num_splits, self.chunk_tokens, workspace=self.split_ws,
                            combine=False)
            return api.combine_splits(self.split_ws, self.B, self.H, self.d, self.num_splits,
                                      out=self.out)
        return api.decode_attn(q, self.cache, seq_lens, self.max_seq_len, self.sm_scale,
                               self.num_splits, self.chunk_tokens, out=self.out,
                               workspace=self.split_ws)

    def __call__(self, k_new, v_new, pos, seq_lens, x=None, weights=None, q=None, w_kv=None):
        """q from x and weights=(w_qdown, g, w_qup) (or given), append, attend,
        as one mfa_decode_step call (the library shares launches between the
        stages). Returns ``out``.

        With ``w_kv`` ([2d][hidden], W_k over W_v; needs x), the appended
        token is the K/V projection of x; k_new / v_new are then optional
        outputs receiving it ([B][d] in the activation dtype, or None)."""
        args = _lib.StepArgs()
        args.B, args.H, args.d = self.B, self.H, self.d
        args.dtype = api._DTYPES[self.act_dtype]
        if q is None:
            w_qdown, g, w_qup = weights
            for t, n in ((x, "x"), (w_qdown, "w_qdown"), (g, "g"), (w_qup, "w_qup")):
                api._dev(t, n)
            args.x, args.w_qdown, args.w_qup = x.data_ptr(), w_qdown.data_ptr(), w_qup.data_ptr()
            args.q_norm_w = g.data_ptr()
            args.hidden, args.q_rank = self.hidden, self.q_rank
            args.weight_layout = (api.MFA_WEIGHTS_PACKED if self.packed_weights
                                  else api.MFA_WEIGHTS_ROWMAJOR)
            args.eps = self.eps
            args.qproj_workspace = self.qproj_ws.data_ptr()
            args.qproj_workspace_bytes = self.qproj_ws.numel()
            q = self.q
        if w_kv is not None:
            if x is None:
                raise ValueError("the K/V projection needs x")
            api._dev(w_kv, "w_kv")
            args.w_kv = w_kv.data_ptr()
            args.kv_in_dtype = args.dtype
            for t, n in ((k_new, "k_new"), (v_new, "v_new")):
                if t is not None:
                    api._dev(t, n)
                    if t.dtype != self.act_dtype:
                        raise ValueError(f"{n} must be {self.act_dtype} with the K/V projection")
            args.k_new = k_new.data_ptr() if k_new is not None else None
            args.v_new = v_new.data_ptr() if v_new is not None else None
        else:
            api._dev(k_new, "k_new")
            api._dev(v_new, "v_new")
            args.k_new, args.v_new = k_new.data_ptr(), v_new.data_ptr()
            args.kv_in_dtype = api._DTYPES[k_new.dtype]
        for t, n in ((q, "q"), (pos, "pos"), (seq_lens, "seq_lens")):
            api._dev(t, n)
        if pos.dtype != torch.int32 or seq_lens.dtype != torch.int32:
            raise ValueError("pos and seq_lens must be int32")
        args.q = q.data_ptr()
        args.pos = pos.data_ptr()
        args.cache = ctypes.pointer(self._desc)
        args.seq_lens = seq_lens.data_ptr()
        args.max_seq_len = self.max_seq_len
        args.sm_scale = self.sm_scale
        args.num_splits, args.chunk_tokens = self.num_splits, self.chunk_tokens
        if self.split_ws is not None:
            args.split_workspace = self.split_ws.data_ptr()
            args.split_workspace_bytes = self.split_ws.numel()
        args.out = self.out.data_ptr()
        args.out_dtype = api._DTYPES[self.out_dtype]
        api.decode_step(args, self.out.device)
        return self.out

    def staged(self, k_new, v_new, pos, seq_lens, x=None, weights=None, q=None):
        """The same step as four separate calls (mfa_qproj, mfa_kv_append,
        mfa_decode_attn, mfa_combine)."""
        if q is None:
            q = self.query(x, *weights)
        self.append(k_new, v_new, pos)
        return self.attend(q, seq_lens)


def prefill(cache: api.KVCache, k_rows: torch.Tensor, v_rows: torch.Tensor, offsets,
            lengths) -> None:
    """Write tokens 0..lengths[b]-1 of every sequence b from the packed rows
    k_rows/v_rows [sum(lengths)][d] (sequence-major, ``offsets`` host [B+1])."""
    lib = _lib.load()
    B = len(lengths)
    dev = k_rows.device
    dt = api._DTYPES[k_rows.dtype]
    if max(int(l) for l in lengths) == 0:
        return
    if all(int(l) == int(lengths[0]) for l in lengths) and int(lengths[0]) > 0:
        L = int(lengths[0])
        pos = torch.zeros(B, dtype=torch.int32, device=dev)
        api.kv_append(cache, k_rows.view(B, L, -1), v_rows.view(B, L, -1), pos)
        return
    if cache.block_table is None:
        # contiguous cache: every sequence owns its region, so pad to the
        # longest prompt; rows past a sequence's length land in its own
        # region beyond seq_len and are never attended
        L = max(int(l) for l in lengths)
        kp = torch.zeros((B, L, k_rows.shape[1]), dtype=k_rows.dtype, device=dev)
        vp = torch.zeros_like(kp)
        for b in range(B):
            n, o = int(lengths[b]), int(offsets[b])
            kp[b, :n] = k_rows[o:o + n]
            vp[b, :n] = v_rows[o:o + n]
        api.kv_append(cache, kp, vp, torch.zeros(B, dtype=torch.int32, device=dev))
        return
    zero = torch.zeros(1, dtype=torch.int32, device=dev)
    stride = cache.max_blocks_per_seq * 4
    for b in range(B):
        n = int(lengths[b])
        if n == 0:
            continue
        desc = cache.desc()
        desc.block_table = cache.block_table.data_ptr() + b * stride
        o = int(offsets[b])
        kb = k_rows[o:o + n].unsqueeze(0)
        vb = v_rows[o:o + n].unsqueeze(0)
        check("mfa_kv_append", lib.mfa_kv_append(
            ctypes.c_void_p(kb.data_ptr()), ctypes.c_void_p(vb.data_ptr()), dt,
            ctypes.c_void_p(zero.data_ptr()), n, 1, ctypes.byref(desc),
            ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)))
