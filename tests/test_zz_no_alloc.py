"""mfa_decode_attn_static (split partials in the library's static scratch,
no workspace, no allocation) against mfa_decode_attn with a caller-owned
workspace: two calls in a row on one GPU, the second with a smaller input."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import check_bf16_bars, say, setup, to_np
from oracle import run as orun

pytestmark = pytest.mark.gpu


def _case(lens, splits, seed):
    import dataclasses
    w = dataclasses.replace(workloads.WORKLOADS[3], batch=len(lens))
    inp = workloads.make_inputs(3, workload=w, prefill_lens=lens, seed=seed)
    maxlen = int(inp["seq_lens"].max())
    chunk = -(-(-(-maxlen // splits)) // 64) * 64
    T, cache, _ = setup(inp, num_splits=splits, chunk_tokens=chunk)
    import decode_attention_02_amd as mfa
    mfa.kv_append(cache, T["k_new"], T["v_new"], T["prefill_lens"])
    return inp, T, cache, maxlen, chunk


def test_static_scratch_matches_workspace_call(gpu_lib):
    import decode_attention_02_amd as mfa
    # first call: 7 ragged sequences, 5 splits; second: 3 shorter ones, 2 splits
    for lens, splits, seed in (([1, 62, 63, 64, 300, 777, 1500], 5, 201), ([10, 64, 130], 2, 202)):
        inp, T, cache, maxlen, chunk = _case(lens, splits, seed)
        say(f"static scratch: B={len(lens)} splits={splits}")
        ref = mfa.decode_attn(T["q"], cache, T["seq_lens"], maxlen, num_splits=splits,
                              chunk_tokens=chunk)
        out = torch.empty_like(ref)
        got = mfa.decode_attn_static(T["q"], cache, T["seq_lens"], maxlen, num_splits=splits,
                                     chunk_tokens=chunk, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        # the same kernels on the same inputs: bit-identical to the workspace call
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
        check_bf16_bars(to_np(got), orun.decode_step(inp)["o"], f"static B={len(lens)}")


def test_static_scratch_limit(gpu_lib):
    """Partials beyond the static scratch are refused before any launch."""
    import decode_attention_02_amd as mfa
    from decode_attention_02_amd._lib import MfaError
    inp, T, cache, maxlen, chunk = _case([100, 200], 2, 203)
    lib = mfa.load()
    need = lib.mfa_decode_workspace_bytes(2, 64, 256, 300)
    assert need > 32 << 20
    with pytest.raises(MfaError, match="TOO_LARGE"):
        mfa.decode_attn_static(T["q"], cache, T["seq_lens"], maxlen, num_splits=300,
                               chunk_tokens=64)
