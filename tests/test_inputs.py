"""The seeded input generator: determinism, shapes, structure (CPU only)."""
import hashlib
import json
import os

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _digest(inp):
    h = hashlib.sha256()
    for key in sorted(inp):
        v = inp[key]
        if isinstance(v, np.ndarray):
            h.update(key.encode())
            h.update(np.ascontiguousarray(v).tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("idx,kw", [(1, {}), (2, dict(batch=2, context=100)),
                                    (3, dict(batch=5, context=300)), (4, dict(batch=2, context=130)),
                                    (5, dict(batch=1, context=200))])
def test_deterministic_and_shaped(idx, kw):
    a = workloads.make_inputs(idx, **kw)
    b = workloads.make_inputs(idx, **kw)
    assert _digest(a) == _digest(b)
    c = workloads.make_inputs(idx, seed=a["seed"] + 17, **kw)
    assert _digest(a) != _digest(c)
    w = a["workload"]
    B, d = w.batch, w.head_dim
    assert a["k_ctx"].shape == (int(a["prefill_lens"].sum()), d)
    assert a["k_new"].shape == (B, d)
    assert np.array_equal(a["seq_lens"], a["prefill_lens"] + 1)
    nblk = (a["seq_lens"] + 63) // 64
    assert a["max_blocks_per_seq"] == nblk.max()
    if w.paged:
        bt = a["block_table"]
        used = np.concatenate([bt[i, :nblk[i]] for i in range(B)])
        assert sorted(used.tolist()) == list(range(a["num_blocks"]))   # a permutation
        for i in range(B):
            assert np.all(bt[i, nblk[i]:] == -1)
    else:
        assert a["block_table"] is None
    if w.has_qproj:
        assert a["w_qup"].shape == (w.heads * w.head_dim, w.q_rank)
    else:
        assert a["q"].shape == (B, w.heads, w.head_dim)


def test_full_workload_shapes():
    W = workloads.WORKLOADS
    assert (W[2].batch, W[2].hidden, W[2].q_rank, W[2].heads, W[2].head_dim) == (32, 7168, 2048, 64, 256)
    assert W[5].num_splits == 32 and W[5].context == 65536
    assert W[4].kv_dtype == "fp8" and W[4].context == 32768 and W[4].paged
    assert W[3].context_range == (1024, 8192) and W[3].batch == 128


def test_hidden_size_matches_page_traffic_figures():
    """Batch 128 of FP8 (1 B) and BF16 (2 B) hidden states of width 7168 give
    the 896 KiB / 1.75 MiB one-way payloads printed on the StepMesh page."""
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        figs = {e["id"]: e["value"] for e in json.load(f)["figures"]}
    hidden = workloads.WORKLOADS[2].hidden
    assert 128 * hidden * 1 == figs["a2f_bytes_batch128"]
    assert 128 * hidden * 2 == figs["f2a_bytes_batch128"]


def test_bf16_cast_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], dtype=np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    # 1+2^-8 is a tie between 1 and 1+2^-7: goes to even (1.0); 1+3*2^-8 -> 1+2^-6
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1 + 2 ** -6)
    assert back[3] == -2.5
