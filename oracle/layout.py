"""The physical KV-cache block layout that the MFA library documents, written
out with numpy reshapes.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``). Used to check the
library's KV append and weight packing bit for bit. The layout is the library's contract (its C
header states it); this module restates it from that statement:

* a cache block holds 64 consecutive logical tokens of one sequence; without
  a block table, logical block j of sequence b is physical block
  b * max_blocks_per_seq + j; FP8 caches keep one fp32 scale per token for K
  and for V, indexed (block, token-in-block);
* fp32 blocks: K is token-major [64][d], V is feature-major [d][64];
* bf16 blocks are cut into 1 KB units of 64 lanes x 16 bytes:
  K: units ordered (token group t//16, dim group d//32); in a unit, lane
     (16*((d%32)//8) + t%16) holds the 8 values K[t][8*(d//8) .. +8];
  V: units ordered (feature group f//16, token half t//32); in a unit, lane
     (16*((t%32)//8) + f%16) holds the 8 values V[8*(t//8) .. +8][f];
* FP8 blocks, same idea with 16 one-byte codes per lane:
  K: units ordered (token group t//16, dim group d//64); lane
     (16*((d%64)//16) + t%16) holds K[t][16*(d//16) .. +16];
  V: units ordered (feature group f//16); lane (16*(t//16) + f%16) holds
     V[16*(t//16) .. +16][f].
"""
from __future__ import annotations

import numpy as np

BLOCK_TOKENS = 64


def _split(rows: np.ndarray) -> np.ndarray:
    nb = rows.shape[0] // BLOCK_TOKENS
    return rows.reshape(nb, BLOCK_TOKENS, rows.shape[1])


def k_blocks(token_rows: np.ndarray, dtype: str) -> np.ndarray:
    """Token-major rows [num_blocks*64][d] of stored values -> K blocks,
    flattened per block in storage order: [num_blocks][64*d]."""
    x = _split(token_rows)
    nb, _, d = x.shape
    if dtype == "f32":
        return x.reshape(nb, -1)
    if dtype == "bf16":
        # t = (tg, c); d = (s, g, j)  ->  order (tg, s, g, c, j)
        y = x.reshape(nb, 4, 16, d // 32, 4, 8).transpose(0, 1, 3, 4, 2, 5)
        return np.ascontiguousarray(y).reshape(nb, -1)
    if dtype == "fp8":
        # t = (tg, c); d = (u, g, j)  ->  order (tg, u, g, c, j)
        y = x.reshape(nb, 4, 16, d // 64, 4, 16).transpose(0, 1, 3, 4, 2, 5)
        return np.ascontiguousarray(y).reshape(nb, -1)
    raise ValueError(dtype)


def v_blocks(token_rows: np.ndarray, dtype: str) -> np.ndarray:
    """Token-major rows [num_blocks*64][d] -> V blocks [num_blocks][64*d]."""
    x = _split(token_rows)
    nb, _, d = x.shape
    if dtype == "f32":
        return np.ascontiguousarray(x.transpose(0, 2, 1)).reshape(nb, -1)
    if dtype == "bf16":
        # t = (s2, g, j); f = (fg, c)  ->  order (fg, s2, g, c, j)
        y = x.reshape(nb, 2, 4, 8, d // 16, 16).transpose(0, 4, 1, 2, 5, 3)
        return np.ascontiguousarray(y).reshape(nb, -1)
    if dtype == "fp8":
        # t = (g, j); f = (fg, c)  ->  order (fg, g, c, j)
        y = x.reshape(nb, 4, 16, d // 16, 16).transpose(0, 3, 1, 4, 2)
        return np.ascontiguousarray(y).reshape(nb, -1)
    raise ValueError(dtype)


def _inverse(fwd, blocks: np.ndarray, d: int, dtype: str) -> np.ndarray:
    """Undo a forward layout by pushing token/dim indices through it."""
    nb = blocks.shape[0]
    idx = np.arange(BLOCK_TOKENS * d, dtype=np.int64).reshape(BLOCK_TOKENS, d)
    pos = fwd(idx, dtype)[0]                     # pos[k] = flat (t*d + dd) stored at k
    rows = np.empty((nb, BLOCK_TOKENS * d), dtype=blocks.dtype)
    rows[:, pos] = blocks.reshape(nb, -1)
    return rows.reshape(nb * BLOCK_TOKENS, d)


def k_rows_from_blocks(blocks: np.ndarray, d: int, dtype: str) -> np.ndarray:
    """Storage-order K blocks [num_blocks][64*d] -> token-major rows."""
    return _inverse(k_blocks, blocks, d, dtype)


def v_rows_from_blocks(blocks: np.ndarray, d: int, dtype: str) -> np.ndarray:
    """Storage-order V blocks [num_blocks][64*d] -> token-major rows."""
    return _inverse(v_blocks, blocks, d, dtype)


def scale_blocks(token_scales: np.ndarray) -> np.ndarray:
    """Per-token scales [num_blocks*64] -> [num_blocks][64]."""
    return token_scales.reshape(-1, BLOCK_TOKENS)


def pack_weight(w: np.ndarray) -> np.ndarray:
    """Row-major weight [N][K] -> the library's packed operand order, flat.

    1 KB units (16 rows x 32 columns of bf16) ordered (row group n//16,
    column group k//32); in a unit, lane 16*((k%32)//8) + n%16 holds the 8
    values w[n][8*(k//8) .. +8].
    """
    N, K = w.shape
    # n = (nt, c); k = (kt, g, j)  ->  order (nt, kt, g, c, j)
    y = w.reshape(N // 16, 16, K // 32, 4, 8).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(y).reshape(-1)
