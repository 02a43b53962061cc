"""MFA decode attention for one AMD Instinct MI355X (gfx950).

The compute lives in ``libmfa.so`` (hand-written HIP kernels behind the C ABI
of ``include/mfa.h``); this package is its thin torch-facing binding.
"""
from ._lib import BLOCK_TOKENS, MfaError, load  # noqa: F401
from .api import (BALANCED, KVCache, combine_splits, decode_attn, decode_attn_multi,  # noqa: F401
                  decode_attn_static, decode_plan, decode_plan_lens,
                  kv_append, out_proj, pack_weight, qproj, qproj_workspace_bytes,
                  decode_workspace_bytes, split_workspace_bytes)
