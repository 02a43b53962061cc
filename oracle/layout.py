"""The physical KV-cache layout that the MFA library documents, written out.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``). Used to check the
library's KV append bit for bit. The layout is the library's contract (its C
header states it); this module restates it from that statement:

* a cache block holds 64 consecutive logical tokens of one sequence;
* K blocks are token-major: element (block, token-in-block, dim);
* V blocks are dim-major (transposed): element (block, dim, token-in-block);
* FP8 caches keep one fp32 scale per token for K and for V:
  (block, token-in-block);
* without a block table, logical block j of sequence b is physical block
  b * max_blocks_per_seq + j.
"""
from __future__ import annotations

import numpy as np

BLOCK_TOKENS = 64


def k_blocks(token_rows: np.ndarray) -> np.ndarray:
    """Token-major rows [num_blocks*64][d] -> K block array [num_blocks][64][d]."""
    nb = token_rows.shape[0] // BLOCK_TOKENS
    return token_rows.reshape(nb, BLOCK_TOKENS, token_rows.shape[1])


def v_blocks(token_rows: np.ndarray) -> np.ndarray:
    """Token-major rows [num_blocks*64][d] -> V block array [num_blocks][d][64]."""
    nb = token_rows.shape[0] // BLOCK_TOKENS
    return np.ascontiguousarray(
        token_rows.reshape(nb, BLOCK_TOKENS, token_rows.shape[1]).transpose(0, 2, 1))


def scale_blocks(token_scales: np.ndarray) -> np.ndarray:
    """Per-token scales [num_blocks*64] -> [num_blocks][64]."""
    return token_scales.reshape(-1, BLOCK_TOKENS)
