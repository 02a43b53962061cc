"""GPU parity: libmfa (through its C ABI) against the fp64 oracle on the same
seeded inputs. Tolerances: bf16 and FP8-KV outputs rel-L2 <= 5e-3 and max
abs <= 2e-2; fp32 rel-L2 <= 1e-5; KV append bit-exact."""
import dataclasses

import numpy as np
import pytest
import torch

import pins
import workloads
from gpu_util import (MAX_ABS_BF16, REL_L2_BF16, REL_L2_F32, cache_rows, max_abs, rel_l2, run,
                      say, setup, to_np)
from oracle import mfa as omfa
from oracle import run as orun

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def small(base, **kw):
    return dataclasses.replace(W[base], **kw)


def check_bf16(got, want, what):
    r, m = rel_l2(got, want), max_abs(got, want)
    say(f"{what}: rel_l2={r:.3e} max_abs={m:.3e}")
    assert r <= REL_L2_BF16 and m <= MAX_ABS_BF16, (what, r, m)


# ---------------------------------------------------------------- small cases
# bf16 / fp8, paged and contiguous, ragged lengths spanning several blocks,
# 1, 2, 3, 7 splits (chunk chosen to leave empty and partial splits).
SMALL = [
    ("bf16-contig", 3, dict(paged=False), [0, 63, 200]),
    ("bf16-contig-tail", 3, dict(paged=False), [64, 129, 1]),
    ("bf16-paged", 3, dict(), [1, 62, 63, 64, 65, 127, 300, 777]),
    ("fp8-paged", 4, dict(), [0, 63, 64, 190, 513]),
    ("fp8-contig", 4, dict(paged=False), [255, 70, 3]),
    # 8 sequences: batch x splits is a multiple of 8 and at most 128, so every
    # split is walked as two halves (as for the 8 bf16-paged sequences)
    ("fp8-paged-8", 4, dict(), [0, 1, 63, 64, 65, 190, 513, 1000]),
]


@pytest.mark.parametrize("splits", [1, 2, 3, 7])
@pytest.mark.parametrize("name,base,over,lens", SMALL, ids=[s[0] for s in SMALL])
def test_small_parity(gpu_lib, name, base, over, lens, splits):
    w = small(base, **over)
    inp = workloads.make_inputs(base, workload=w, prefill_lens=lens, seed=101 + base)
    say(f"small {name} splits={splits} lens={lens}")
    maxlen = int(inp["seq_lens"].max())
    chunk = -(-maxlen // splits)
    chunk = -(-chunk // 64) * 64
    T, cache, step = setup(inp, num_splits=splits, chunk_tokens=chunk)
    _, out = run(T, step)
    want = orun.decode_step(inp)
    check_bf16(to_np(out), want["o"], f"{name}/S={splits}")


# Caches filled with 0xFF bytes (NaN in bf16, e4m3 and fp32) before the
# prefill: the slots past every sequence's end hold NaNs, which masking must
# keep out of the output. Lengths leave tail blocks with 1 .. 63 tokens.
POISON = [
    ("bf16-paged", 3, dict(), [1, 62, 65, 127, 300], False),
    ("bf16-contig", 3, dict(paged=False), [0, 63, 200], False),
    ("fp8-paged", 4, dict(), [0, 63, 190, 513], False),
    ("fp8-paged-8", 4, dict(), [0, 1, 63, 64, 65, 190, 513, 1000], False),
    ("fp8-contig", 4, dict(paged=False), [255, 70, 3], False),
    ("q8-paged", 4, dict(), [0, 63, 190, 513], True),
    ("q8-paged-8", 4, dict(), [0, 1, 63, 64, 65, 190, 513, 1000], True),
]


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("name,base,over,lens,q8", POISON, ids=[p[0] for p in POISON])
def test_poisoned_cache_tails(gpu_lib, name, base, over, lens, q8, splits):
    import decode_attention_02_amd as mfa
    w = small(base, **over)
    inp = workloads.make_inputs(base, workload=w, prefill_lens=lens, seed=151 + base)
    say(f"poisoned cache {name} splits={splits} lens={lens}")
    maxlen = int(inp["seq_lens"].max())
    chunk = -(-(-(-maxlen // splits)) // 64) * 64
    T, cache, step = setup(inp, num_splits=splits, chunk_tokens=chunk, zero_cache=False,
                           poison=True)
    if q8:
        mfa.kv_append(cache, T["k_new"], T["v_new"], T["prefill_lens"])
        out = mfa.decode_attn_multi(T["q"].unsqueeze(1), cache, T["seq_lens"], maxlen,
                                    num_splits=splits, chunk_tokens=chunk, fp8_queries=True)
        torch.cuda.synchronize()
        got, want = to_np(out)[:, 0], orun.decode_step(inp, fp8_queries=True)["o"]
    else:
        _, out = run(T, step)
        got, want = to_np(out), orun.decode_step(inp)["o"]
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    check_bf16(got, want, f"poisoned {name}/S={splits}")


# ---------------------------------------------------------------- balanced partition
# num_splits == 0: the rows' blocks are split evenly over 256 workgroups, so a
# workgroup walks across row boundaries (pieces), and rows with 0 or 1 block
# sit inside a workgroup's range.
def _ragged(n, seed, top=1500, head=(0, 1, 63, 64, 65)):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, top, size=n).tolist()
    lens[:len(head)] = list(head)
    return lens


BAL = [
    # few blocks (fewer than workgroups): one block per workgroup
    ("bf16-paged-few", 3, dict(), [1, 62, 65, 127, 300, 777]),
    ("bf16-contig-few", 3, dict(paged=False), [0, 63, 200]),
    # hundreds of blocks: ~3 blocks per workgroup, many boundaries
    ("bf16-paged-64", 3, dict(batch=64), _ragged(64, 91)),
    ("bf16-contig-48", 3, dict(batch=48, paged=False), _ragged(48, 92)),
    ("fp8-paged-40", 4, dict(batch=40), _ragged(40, 93)),
    ("fp8-contig-24", 4, dict(batch=24, paged=False), _ragged(24, 94, top=3000)),
    # long rows next to 1-token rows: pieces of one block between long ones
    ("bf16-paged-mix", 3, dict(batch=12), [5000, 0, 1, 3000, 63, 64, 1, 7000, 2, 130, 4000, 0]),
    # the most rows the partition takes (1024, two per setup thread), short
    # rows with empty ones, and one long row that spans many workgroups
    ("bf16-paged-1024", 3, dict(batch=1024), _ragged(1023, 95, top=300) + [9000]),
    ("fp8-paged-1024", 4, dict(batch=1024), [9000] + _ragged(1023, 96, top=300)),
]


@pytest.mark.parametrize("name,base,over,lens", BAL, ids=[b[0] for b in BAL])
def test_balanced_parity(gpu_lib, name, base, over, lens):
    w = small(base, **over)
    inp = workloads.make_inputs(base, workload=w, prefill_lens=lens, seed=301 + base)
    say(f"balanced {name} rows={len(lens)} blocks={int(np.sum((inp['seq_lens'] + 63) // 64))}")
    T, cache, step = setup(inp, num_splits=0)
    _, out = run(T, step)
    check_bf16(to_np(out), orun.decode_step(inp)["o"], f"balanced {name}")


@pytest.mark.parametrize("name,base,over,lens", [BAL[2], BAL[4], BAL[6]],
                         ids=["bf16-paged-64", "fp8-paged-40", "bf16-paged-mix"])
def test_balanced_poisoned(gpu_lib, name, base, over, lens):
    """The balanced walk on caches whose unwritten slots hold NaNs."""
    w = small(base, **over)
    inp = workloads.make_inputs(base, workload=w, prefill_lens=lens, seed=311 + base)
    say(f"balanced poisoned {name}")
    T, cache, step = setup(inp, num_splits=0, zero_cache=False, poison=True)
    _, out = run(T, step)
    got = to_np(out)
    assert np.all(np.isfinite(got))
    check_bf16(got, orun.decode_step(inp)["o"], f"balanced poisoned {name}")


@pytest.mark.parametrize("T", [2, 4])
@pytest.mark.parametrize("base", [3, 4], ids=["bf16", "fp8"])
def test_balanced_multi_token(gpu_lib, base, T):
    """Virtual rows (sequence, query token) in the balanced walk."""
    import decode_attention_02_amd as mfa
    lens = _ragged(20, 95, head=(0, 1, 2, 63, 64))
    w = small(base, batch=len(lens))
    inp = workloads.make_inputs(base, workload=w, seed=321, prefill_lens=lens, q_len=T)
    say(f"balanced multi-token base={base} T={T}")
    T_, cache, step = setup(inp)
    mfa.kv_append(cache, T_["k_new"], T_["v_new"], T_["prefill_lens"])
    maxlen = int(inp["seq_lens"].max())
    out = mfa.decode_attn_multi(T_["q_multi"], cache, T_["seq_lens"], maxlen, num_splits=0)
    torch.cuda.synchronize()
    check_bf16(to_np(out), orun.decode_step_multi(inp), f"balanced multi T={T}")


def _balanced_partition(lens, G=256, row_cost=6):
    """The balanced partition restated: rows' blocks (64 tokens) in row order,
    a block costing U units and an interior row start (not a cut of the plain
    even partition) row_cost more when there are at least 4 blocks per
    workgroup; workgroup w takes the blocks whose cost start lies in
    [floor(w TC / Geff), floor((w+1) TC / Geff)). Returns per row the
    (first workgroup, number of workgroups) that walk it (None: no blocks)."""
    nb = [(L + 63) // 64 for L in lens]
    NB = sum(nb)
    geff = min(G, NB)
    weighted = NB >= 4 * G
    U, RC = (4, row_cost) if weighted else (1, 0)
    pfx = np.concatenate([[0], np.cumsum(nb)])

    def interior(st):
        v = -(-st * geff // NB)
        return not (v < geff and v * NB // geff == st)
    cost, c = [], 0
    for r, n in enumerate(nb):
        rc = RC if (n > 0 and interior(int(pfx[r]))) else 0
        cost.append((c, rc))
        c += U * n + rc
    TC = c

    def wg_of(x):
        v = x * geff // TC
        return v + 1 if (v + 1) * TC // geff <= x else v
    out = []
    for r, n in enumerate(nb):
        if n == 0:
            out.append(None)
            continue
        c0 = cost[r][0] + cost[r][1]
        wf, wl = wg_of(c0), wg_of(c0 + U * (n - 1))
        out.append((wf, wl - wf + 1))
    return out


@pytest.mark.parametrize("name,n,top,seed", [("plain", 64, 1500, 96), ("weighted", 96, 12000, 98)])
def test_balanced_separate_combine(gpu_lib, name, n, top, seed):
    """Attention with out=NULL then mfa_combine(num_splits=0) equals the
    call that merges itself, bit for bit, and the per-row metadata (first
    slot = first workgroup + row, slot count) is the restated partition's,
    with fewer than 4 blocks per workgroup (plain cut) and with more
    (cost-weighted cut)."""
    import decode_attention_02_amd as mfa
    lens = _ragged(n, seed, top=top)
    w = small(3, batch=len(lens))
    inp = workloads.make_inputs(3, workload=w, seed=331, prefill_lens=lens)
    T, cache, step = setup(inp, num_splits=0)
    mfa.kv_append(cache, T["k_new"], T["v_new"], T["prefill_lens"])
    maxlen = int(inp["seq_lens"].max())
    B = len(lens)
    ws = torch.empty(mfa.decode_workspace_bytes(B, 64, 256, 0), dtype=torch.uint8, device="cuda")
    nblk = (inp["seq_lens"] + 63) // 64
    say(f"balanced {name}: separate combine, {int(nblk.sum())} blocks")
    fused = mfa.decode_attn(T["q"], cache, T["seq_lens"], maxlen, num_splits=0, workspace=ws)
    fused = fused.clone()
    mfa.decode_attn(T["q"], cache, T["seq_lens"], maxlen, num_splits=0, workspace=ws,
                    combine=False)
    sep = mfa.combine_splits(ws, B, 64, 256, 0)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), sep.view(torch.int16))
    assert (int(nblk.sum()) >= 1024) == (name == "weighted")
    # metadata: (first slot, count) per row at the end of the workspace
    rows = (256 + B) * 64
    off_ml = -(-rows * 256 * 4 // 256) * 256
    off_meta = -(-(off_ml + rows * 8) // 16) * 16
    meta = ws[off_meta:off_meta + B * 8].cpu().numpy().view(np.int32).reshape(B, 2)
    want = _balanced_partition([int(x) for x in inp["seq_lens"]])
    # pieces per workgroup: the first piece that ends inside a walk is held in
    # LDS to the end, later ones are stored at once; both cases are present
    per_wg = {}
    for p in want:
        for wg in (range(p[0], p[0] + p[1]) if p else ()):
            per_wg[wg] = per_wg.get(wg, 0) + 1
    assert max(per_wg.values()) >= (3 if name == "weighted" else 2)
    for r in range(B):
        if want[r] is None:
            assert meta[r, 1] == 0, r
        else:
            assert (meta[r, 0], meta[r, 1]) == (want[r][0] + r, want[r][1]), (r, meta[r], want[r])
    check_bf16(to_np(fused), orun.decode_step(inp)["o"], f"balanced {name} separate combine")


def test_balanced_static_and_graph(gpu_lib):
    """The balanced partition through mfa_decode_attn_static, and the whole
    step with it captured in a HIP graph (every replay bit-identical)."""
    import decode_attention_02_amd as mfa
    lens = _ragged(32, 97)
    w = small(3, batch=len(lens))
    inp = workloads.make_inputs(3, workload=w, seed=341, prefill_lens=lens)
    T, cache, step = setup(inp, num_splits=0)
    say("balanced: static scratch and graph replay")
    _, eager = run(T, step)
    eager = eager.clone()
    maxlen = int(inp["seq_lens"].max())
    st = mfa.decode_attn_static(T["q"], cache, T["seq_lens"], maxlen, num_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(st.view(torch.int16), eager.view(torch.int16))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(T["k_new"], T["v_new"], T["prefill_lens"], T["seq_lens"], q=T["q"])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step(T["k_new"], T["v_new"], T["prefill_lens"], T["seq_lens"], q=T["q"])
    for r in range(3):
        step.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
    check_bf16(to_np(eager), orun.decode_step(inp)["o"], "balanced graph step")


@pytest.mark.parametrize("base,over,lens,splits", [
    (3, dict(), [1, 62, 64, 300, 777, 2000], 3),
    (4, dict(), [0, 63, 190, 513, 1500], 4),
], ids=["bf16-split", "fp8-split"])
def test_graph_replay_append_in_attention(gpu_lib, base, over, lens, splits):
    """The step without a query path on a split plan (the KV append inside
    the attention launch) captured in a HIP graph: every replay, with eager
    work and synchronisations in between, equals the eager step bit for bit,
    output and cache."""
    w = small(base, **over)
    inp = workloads.make_inputs(base, workload=w, prefill_lens=lens, seed=359 + base)
    T, cache, step = setup(inp, num_splits=splits)
    say(f"graph replay, append in the attention launch, base={base} splits={splits}")
    _, eager = run(T, step)
    eager = eager.clone()
    rows = [r.copy() for r in cache_rows(cache)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(T["k_new"], T["v_new"], T["prefill_lens"], T["seq_lens"], q=T["q"])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step(T["k_new"], T["v_new"], T["prefill_lens"], T["seq_lens"], q=T["q"])
    for r in range(3):
        step.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
        for a_, b_ in zip(cache_rows(cache), rows):
            assert np.array_equal(a_, b_), f"replay {r} cache"
    check_bf16(to_np(eager), orun.decode_step(inp)["o"], "graph step, append in attention")


def test_small_f32_generic(gpu_lib):
    """fp32 cache and q on the vector-ALU kernel, ragged lengths, 1 and 3 splits."""
    w = small(1, hidden=None, q_rank=None)
    for splits in (1, 3):
        inp = workloads.make_inputs(1, workload=w, prefill_lens=[0, 5, 130], seed=7)
        say(f"f32 generic splits={splits}")
        T, cache, step = setup(inp, num_splits=splits)
        _, out = run(T, step)
        want = orun.decode_step(inp)
        r = rel_l2(to_np(out), want["o"])
        say(f"f32 generic S={splits}: rel_l2={r:.3e}")
        assert r <= REL_L2_F32


@pytest.mark.parametrize("base,over", [(3, dict()), (4, dict())], ids=["bf16-paged", "fp8-paged"])
def test_waves_of_workgroups(gpu_lib, base, over):
    """More (sequence, split) pairs than compute units (64 ragged sequences x
    8 splits = 512 workgroups, so they run in waves), empty tail splits
    included."""
    rng = np.random.default_rng(71)
    lens = rng.integers(0, 1500, size=64).tolist()
    lens[:4] = [0, 1, 63, 1499]
    w = small(base, batch=64, **over)
    inp = workloads.make_inputs(base, workload=w, seed=72, prefill_lens=lens)
    say(f"waves of workgroups {w.kv_dtype}: 64 x 8 splits")
    T, cache, step = setup(inp, num_splits=8, chunk_tokens=192)
    _, out = run(T, step)
    check_bf16(to_np(out), orun.decode_step(inp)["o"], f"64 x 8 splits {w.kv_dtype}")


def test_single_token_returns_v_exactly(gpu_lib):
    """Context of one token: the output is V bit for bit (bf16 cache, bf16 out)."""
    w = small(3, paged=False)
    inp = workloads.make_inputs(3, workload=w, prefill_lens=[0, 0, 0], seed=3)
    say("single token")
    T, cache, step = setup(inp, num_splits=1)
    _, out = run(T, step)
    v = T["v_new"].view(3, 1, 256).expand(3, 64, 256)
    assert torch.equal(out.cpu(), v.cpu())


def test_physical_block_permutation_bit_identical(gpu_lib):
    """Same logical tokens under two different block tables: identical bits."""
    w = small(3)
    lens = [100, 400, 250]
    outs = []
    for seed in (11, 12):          # seeds differ only in the block permutation
        inp = workloads.make_inputs(3, workload=w, prefill_lens=lens, seed=10)
        rng = np.random.default_rng(seed)
        nblk = (inp["seq_lens"] + 63) // 64
        perm = rng.permutation(inp["num_blocks"]).astype(np.int32)
        bt = np.full_like(inp["block_table"], -1)
        p = 0
        for b in range(3):
            bt[b, :nblk[b]] = perm[p:p + nblk[b]]
            p += nblk[b]
        inp["block_table"] = bt
        say(f"block permutation seed={seed}")
        T, cache, step = setup(inp, num_splits=2)
        _, out = run(T, step)
        outs.append(out.cpu())
    assert torch.equal(outs[0], outs[1])


def test_split_counts_agree(gpu_lib):
    w = small(3)
    inp = workloads.make_inputs(3, workload=w, prefill_lens=[2047, 1000], seed=5)
    want = orun.decode_step(inp)["o"]
    res = {}
    for s in (1, 2, 7, 32):
        say(f"split count {s}")
        T, cache, step = setup(inp, num_splits=s)
        _, out = run(T, step)
        res[s] = to_np(out)
        check_bf16(res[s], want, f"splits={s}")
    for s in (2, 7, 32):
        assert rel_l2(res[s], res[1]) <= 2 * REL_L2_BF16


@pytest.mark.parametrize("out_dtype,S,H,d", [("f32", 20, 64, 256), ("bf16", 20, 64, 256),
                                             ("f32", 2, 64, 256), ("f32", 9, 64, 256),
                                             ("bf16", 64, 64, 256), ("f32", 20, 4, 64),
                                             ("f32", 9, 8, 128), ("f32", 33, 32, 256)])
def test_combine_standalone(gpu_lib, out_dtype, S, H, d):
    """mfa_combine on drawn fp32 partials (some splits empty) against the
    oracle's log-sum-exp merge, into fp32 and bf16 outputs. Three rows fill
    few workgroups, so 9 and more splits are shared by four thread groups
    per head (9: runs of 3, 3, 3 and none; 20: 5 each; 33: 9, 9, 9, 6; 64: 16
    each), also at head widths 64 and 128 (16 and 32 threads per head)."""
    import decode_attention_02_amd as mfa
    rng = np.random.default_rng(77 + S + d)
    B = 3
    o = rng.standard_normal((B, S, H, d)).astype(np.float32)
    m = (rng.standard_normal((B, S, H)) * 3).astype(np.float32)
    l = rng.uniform(0.5, 40, size=(B, S, H)).astype(np.float32)
    empty = rng.random((B, S, H)) < 0.3
    empty[0, :, 0] = True                      # a head with every split empty
    m[empty], l[empty], o[empty] = -np.inf, 0.0, 0.0
    nbytes = mfa.decode_workspace_bytes(B, H, d, S)
    ws = np.zeros(nbytes, dtype=np.uint8)
    rows = B * S * H
    off = -(-rows * d * 4 // 256) * 256
    ws[:rows * d * 4] = o.reshape(-1).view(np.uint8)
    ws[off:off + rows * 8] = np.stack([m, l], axis=-1).reshape(-1).view(np.uint8)
    say(f"combine standalone {out_dtype}")
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out = mfa.combine_splits(torch.from_numpy(ws).cuda(), B, H, d, S, out_dtype=tdt)
    torch.cuda.synchronize()
    got = to_np(out)
    tol = 1e-6 if out_dtype == "f32" else 4e-3    # bf16: the output rounding alone
    for b in range(B):
        want = omfa.combine([(o[b, s], m[b, s], l[b, s]) for s in range(S)])
        assert rel_l2(got[b], want) <= tol
    assert np.all(got[0, 0] == 0)


def test_combine_output_type_free(gpu_lib):
    """Attention with out=NULL (bf16 out_dtype) leaves fp32 partials; the
    combine may then write fp32 or bf16, and the bf16 result is the bf16
    rounding of the fp32 one."""
    import decode_attention_02_amd as mfa
    w = small(3, batch=3)
    inp = workloads.make_inputs(3, workload=w, seed=81, prefill_lens=[100, 700, 3])
    T, cache, step = setup(inp, num_splits=3)
    mfa.kv_append(cache, T["k_new"], T["v_new"], T["prefill_lens"])
    maxlen = int(inp["seq_lens"].max())
    ws = torch.empty(mfa.decode_workspace_bytes(3, 64, 256, 3), dtype=torch.uint8, device="cuda")
    say("combine output types")
    mfa.decode_attn(T["q"], cache, T["seq_lens"], maxlen, num_splits=3, workspace=ws,
                    out_dtype=torch.bfloat16, combine=False)
    o32 = mfa.combine_splits(ws, 3, 64, 256, 3, out_dtype=torch.float32)
    o16 = mfa.combine_splits(ws, 3, 64, 256, 3, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))
    check_bf16(to_np(o16), orun.decode_step(inp)["o"], "combine after attention")


# ---------------------------------------------------------------- KV append
@pytest.mark.parametrize("base,over,lens", [
    (3, dict(), [10, 64, 130]),
    (3, dict(paged=False), [5, 64, 70]),
    (4, dict(), [10, 64, 200]),
    (1, dict(hidden=None, q_rank=None), [3, 66]),
])
def test_append_bit_exact(gpu_lib, base, over, lens):
    """Prefill + one appended token, then read back every token's stored
    bytes (and FP8 scales) and compare with the oracle's codec and layout."""
    w = small(base, **over)
    inp = workloads.make_inputs(base, workload=w, prefill_lens=lens, seed=41)
    say(f"append bit-exact base={base} {over} {lens}")
    T, cache, step = setup(inp, num_splits=1)
    run(T, step)
    exp, owned = orun.expected_cache_rows(inp, range(len(lens)))
    kg, vg = cache_rows(cache)
    for b, rows in owned.items():
        assert np.array_equal(kg[rows].view(np.uint8), exp["k"][rows].view(np.uint8)), b
        assert np.array_equal(vg[rows].view(np.uint8), exp["v"][rows].view(np.uint8)), b
        if w.kv_dtype == "fp8":
            ks = cache.k_scale.cpu().numpy().reshape(-1)
            vs = cache.v_scale.cpu().numpy().reshape(-1)
            assert np.array_equal(ks[rows].view(np.uint32), exp["k_scale"][rows].view(np.uint32))
            assert np.array_equal(vs[rows].view(np.uint32), exp["v_scale"][rows].view(np.uint32))


def test_fp8_codec_bit_exact_random_scales(gpu_lib):
    """Quantise many random bf16 tokens at several magnitudes (incl. tiny and
    zero rows) through mfa_kv_append; codes and scales equal the oracle's."""
    import decode_attention_02_amd as mfa
    rng = np.random.default_rng(9)
    n, d = 512, 256
    x = rng.standard_normal((n, d)).astype(np.float32)
    x *= (10.0 ** rng.uniform(-6, 3, size=(n, 1))).astype(np.float32)
    x[5] = 0.0
    x[6, :] = -np.abs(x[6])
    bits = workloads.f32_to_bf16_bits(x)
    # row 7: the hand-worked row of the oracle pins (zeros past its 8 values)
    bits[7] = 0
    bits[7, :8] = pins.FP8_WORKED_ROW_BITS
    xb = omfa.bf16_bits_to_f64(bits)
    kc, ks = omfa.quantize_tokens(xb)
    cache = mfa.KVCache(8, d, "fp8", 8)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda().view(1, n, d)
    say("fp8 codec random")
    mfa.kv_append(cache, t, t, torch.zeros(1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    got, gv = cache_rows(cache)
    assert np.array_equal(got, kc)
    assert np.array_equal(cache.k_scale.cpu().numpy().reshape(n).view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(gv, kc)
    assert int(cache.k_scale.cpu().numpy().reshape(n).view(np.uint32)[7]) == pins.FP8_WORKED_SCALE_BITS
    assert got[7, :8].tolist() == pins.FP8_WORKED_CODES and not got[7, 8:].any()


# ---------------------------------------------------------------- query path
def test_qproj_small_bf16(gpu_lib):
    import decode_attention_02_amd as mfa
    w = dataclasses.replace(W[2], batch=5, hidden=512, q_rank=256, heads=64, head_dim=256,
                            context=65)
    inp = workloads.make_inputs(2, workload=w, seed=21)
    T = workloads.to_torch(inp)
    say("qproj small bf16")
    q = mfa.qproj(T["x"], T["w_qdown"], T["g"], T["w_qup"], 64, 256)
    torch.cuda.synchronize()
    check_bf16(to_np(q), orun.query(inp), "qproj small")


def test_pack_weight_bit_exact(gpu_lib):
    """mfa_pack_weight puts every bf16 weight where the documented packed
    order says (checked against the oracle's restatement of that order)."""
    import decode_attention_02_amd as mfa
    from oracle import layout
    rng = np.random.default_rng(12)
    w = workloads.f32_to_bf16_bits(rng.standard_normal((96, 320)).astype(np.float32))
    t = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    say("pack weight")
    pk = mfa.pack_weight(t)
    torch.cuda.synchronize()
    got = pk.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1)
    assert np.array_equal(got, layout.pack_weight(w))


@pytest.mark.parametrize("B", [5, 32, 70])
def test_qproj_packed_matches_oracle(gpu_lib, B):
    import decode_attention_02_amd as mfa
    w = dataclasses.replace(W[2], batch=B, hidden=1024, q_rank=512, context=65)
    inp = workloads.make_inputs(2, workload=w, seed=22)
    T = workloads.to_torch(inp)
    say(f"qproj packed B={B}")
    wd, wu = mfa.pack_weight(T["w_qdown"]), mfa.pack_weight(T["w_qup"])
    q = mfa.qproj(T["x"], wd, T["g"], wu, 64, 256, packed=True)
    q_rm = mfa.qproj(T["x"], T["w_qdown"], T["g"], T["w_qup"], 64, 256)
    torch.cuda.synchronize()
    check_bf16(to_np(q), orun.query(inp), f"qproj packed B={B}")
    check_bf16(to_np(q_rm), orun.query(inp), f"qproj row-major B={B}")


def test_qproj_max_batch(gpu_lib):
    """The largest batch the query path takes (256 rows: four passes of 64),
    Step-3's query shape on a smaller hidden width."""
    import decode_attention_02_amd as mfa
    w = dataclasses.replace(W[2], batch=256, hidden=1024, context=65)
    inp = workloads.make_inputs(2, workload=w, seed=23)
    T = workloads.to_torch(inp)
    say("qproj B=256")
    q = mfa.qproj(T["x"], T["w_qdown"], T["g"], T["w_qup"], 64, 256)
    torch.cuda.synchronize()
    check_bf16(to_np(q), orun.query(inp), "qproj B=256")


def test_qproj_split_k_and_reuse(gpu_lib):
    """A query shape whose up-projection is split over K (partials summed by
    the reduction kernel) and whose down-projection is not; repeated calls on
    one workspace are bit-identical (no state carried between calls)."""
    import decode_attention_02_amd as mfa
    w = dataclasses.replace(W[2], batch=3, hidden=256, q_rank=2048, heads=4, head_dim=64,
                            context=65)
    inp = workloads.make_inputs(2, workload=w, seed=23)
    T = workloads.to_torch(inp)
    ws = torch.zeros(mfa.qproj_workspace_bytes(3, 256, 2048, 4, 64, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    say("qproj split-K up-projection, workspace reuse")
    outs = [mfa.qproj(T["x"], T["w_qdown"], T["g"], T["w_qup"], 4, 64, workspace=ws)
            for _ in range(3)]
    torch.cuda.synchronize()
    check_bf16(to_np(outs[0]), orun.query(inp), "qproj split-K up")
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    # the same workspace then serves a smaller batch of another shape
    w2 = dataclasses.replace(W[2], batch=2, hidden=512, q_rank=256, heads=64, head_dim=256,
                             context=65)
    inp2 = workloads.make_inputs(2, workload=w2, seed=24)
    T2 = workloads.to_torch(inp2)
    ws2 = torch.zeros(mfa.qproj_workspace_bytes(2, 512, 256, 64, 256, torch.bfloat16),
                      dtype=torch.uint8, device="cuda")
    a = mfa.qproj(T2["x"], T2["w_qdown"], T2["g"], T2["w_qup"], 64, 256, workspace=ws2)
    b = mfa.qproj(T2["x"], T2["w_qdown"], T2["g"], T2["w_qup"], 64, 256, workspace=ws2)
    torch.cuda.synchronize()
    check_bf16(to_np(a), orun.query(inp2), "qproj reuse")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_graph_replay_matches_eager(gpu_lib):
    """The whole step (query path, append, attention, combine) captured in a
    HIP graph: every replay, with eager work and synchronisations in between,
    equals the eager step bit for bit."""
    w = dataclasses.replace(W[2], batch=4, hidden=1024, q_rank=512, context=300)
    inp = workloads.make_inputs(2, workload=w, seed=25)
    T, cache, step = setup(inp, num_splits=3)
    say("graph replay vs eager")
    _, eager = run(T, step)
    eager = eager.clone()
    wts = (T["w_qdown"], T["g"], T["w_qup"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(T["k_new"], T["v_new"], T["prefill_lens"], T["seq_lens"], x=T["x"], weights=wts)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step(T["k_new"], T["v_new"], T["prefill_lens"], T["seq_lens"], x=T["x"], weights=wts)
    for r in range(3):
        step.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
    check_bf16(to_np(eager), orun.decode_step(inp)["o"], "graph step")


def test_graph_replay_multi_q8_out_proj(gpu_lib):
    """KV append of the new token, FP8-query multi-token attention over the
    last 2 tokens of every sequence (3 splits, combine) and the output
    projection with its FP8 pack, captured in one HIP graph: every replay,
    with eager work and synchronisations in between, equals the eager run
    bit for bit."""
    import decode_attention_02_amd as mfa
    w = small(4, batch=5)
    inp = workloads.make_inputs(4, workload=w, seed=26, prefill_lens=[1, 63, 64, 200, 700],
                                q_len=2, out_proj=True)
    T, cache, step = setup(inp)
    say("graph replay: append + q8 multi + out_proj")
    B, d = 5, 256
    maxlen = int(inp["seq_lens"].max())
    chunk = -(-(-(-maxlen // 3)) // 64) * 64
    wo = mfa.pack_weight(T["w_o"])
    ws = torch.empty(mfa.split_workspace_bytes(B * 2, 64, d, 3), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, 2, 64, d), dtype=torch.bfloat16, device="cuda")
    hid = T["w_o"].shape[0]
    wsp = torch.empty(max(mfa.load().mfa_out_proj_workspace_bytes(B * 2, 64 * d, hid, 1), 16),
                      dtype=torch.uint8, device="cuda")
    outs = (torch.empty((B * 2, hid), dtype=torch.bfloat16, device="cuda"),
            torch.empty((B * 2, hid), dtype=torch.uint8, device="cuda"),
            torch.empty(B * 2, dtype=torch.float32, device="cuda"))

    def work():
        mfa.kv_append(cache, T["k_new"], T["v_new"], T["prefill_lens"])
        mfa.decode_attn_multi(T["q_multi"], cache, T["seq_lens"], maxlen, num_splits=3,
                              chunk_tokens=chunk, out=o, workspace=ws, fp8_queries=True)
        mfa.out_proj(o.view(B * 2, -1), wo, packed=True, workspace=wsp, out=outs)

    work()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (o,) + outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for r in range(3):
        for t in (o,) + outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((o,) + outs, eager):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {r}"
    check_bf16(to_np(eager[0]), orun.decode_step_multi(inp, fp8_queries=True), "graph q8 multi")


@pytest.mark.parametrize("idx,shrink", [(2, dict(batch=6, hidden=1024, q_rank=512, context=300)),
                                        (4, dict(batch=3, context=400)),
                                        (1, {})])
def test_fused_step_matches_staged(gpu_lib, idx, shrink):
    """mfa_decode_step (KV append inside the query down-projection launch on
    the bf16 path) gives bit-identical outputs and cache contents to the four
    separate calls."""
    w = dataclasses.replace(W[idx], **shrink)
    inp = workloads.make_inputs(idx, workload=w, seed=26)
    say(f"fused vs staged: {w.name} {shrink}")
    outs, caches = [], []
    for mode in ("fused", "staged"):
        T, cache, step = setup(inp, num_splits=3 if w.context and w.context > 256 else None)
        fn = step if mode == "fused" else step.staged
        if w.has_qproj:
            out = fn(T["k_new"], T["v_new"], T["prefill_lens"], T["seq_lens"], x=T["x"],
                     weights=(T["w_qdown"], T["g"], T["w_qup"]))
        else:
            out = fn(T["k_new"], T["v_new"], T["prefill_lens"], T["seq_lens"], q=T["q"])
        torch.cuda.synchronize()
        outs.append(out.detach().cpu().clone())
        rows = list(cache_rows(cache))
        if cache.dtype == "fp8":
            rows += [cache.k_scale.cpu().numpy(), cache.v_scale.cpu().numpy()]
        caches.append(rows)
    assert torch.equal(outs[0].view(torch.uint8), outs[1].view(torch.uint8))
    for a, b in zip(*caches):
        assert np.array_equal(a, b)


# The step without a query path (KV append, then attention and combine)
# against the separate calls, with the new token either the last attended
# one ("next": seq_len = pos + 1) or not attended ("behind": seq_len = pos,
# so the token lands in a walked block past the length, or, when pos is a
# multiple of 64 or the row is empty, in a block no workgroup reads).
STEP_POSITIONS = [
    ("bf16-paged-bal", 3, dict(batch=12), [5000, 0, 1, 3000, 63, 64, 1, 7000, 2, 130, 4000, 0],
     "next", 0),
    ("bf16-paged-bal-behind", 3, dict(batch=12),
     [5000, 0, 1, 3000, 63, 64, 1, 7000, 2, 128, 4000, 0], "behind", 0),
    ("bf16-paged-bal-1024", 3, dict(batch=1024), _ragged(1023, 97, top=300) + [9000], "next", 0),
    ("bf16-paged-bal-empty", 3, dict(batch=5), [0, 0, 0, 0, 0], "behind", 0),
    ("bf16-contig-split", 3, dict(paged=False), [0, 63, 200], "next", 3),
    ("bf16-contig-split-behind", 3, dict(paged=False), [0, 64, 200], "behind", 3),
    ("bf16-paged-unsplit", 3, dict(), [1, 62, 63, 64, 65, 127, 300, 777], "next", 1),
    ("fp8-paged-split", 4, dict(), [0, 63, 64, 190, 513], "next", 3),
    ("fp8-paged-bal", 4, dict(batch=40), _ragged(40, 98), "next", 0),
    ("fp8-contig-split-behind", 4, dict(paged=False), [64, 70, 3, 128], "behind", 2),
    ("bf16-paged-split-behind", 3, dict(), [0, 64, 128, 200, 4095, 4096], "behind", 4),
    ("bf16-paged-split-8", 3, dict(), [5, 1000, 3000, 9000], "next", 8),
    ("fp8-paged-split-8", 4, dict(), [1, 700, 4000, 8191], "next", 8),
    # balanced: workgroups holding many whole rows, rows shared by several
    # workgroups, empty rows among the others (the combine in the attention
    # launch against the separate combine)
    ("bf16-paged-bal-short-rows", 3, dict(batch=1024), [20000] + [1, 0, 70] * 341, "next", 0),
    ("bf16-paged-bal-empty-mix", 3, dict(batch=300), [0, 5000, 0, 64, 1] * 60, "behind", 0),
    ("fp8-paged-bal-1024", 4, dict(batch=1024), _ragged(1023, 97, top=300) + [9000], "next", 0),
]


@pytest.mark.parametrize("name,base,over,lens,mode,splits", STEP_POSITIONS,
                         ids=[c[0] for c in STEP_POSITIONS])
def test_step_positions_match_staged(gpu_lib, name, base, over, lens, mode, splits):
    """mfa_decode_step without a query path against the separate calls
    (mfa_kv_append, then attention and combine): bit-identical outputs and
    cache contents (codes and scales); with the token attended, also within
    the bars of the oracle step."""
    w = small(base, **over)
    inp = workloads.make_inputs(base, workload=w, prefill_lens=lens, seed=331 + base)
    say(f"step positions {name} mode={mode} splits={splits}")
    outs, caches = [], []
    for fused in (True, False):
        T, cache, step = setup(inp, num_splits=splits)
        seq = T["seq_lens"] if mode == "next" else T["prefill_lens"].clone()
        fn = step if fused else step.staged
        out = fn(T["k_new"], T["v_new"], T["prefill_lens"], seq, q=T["q"])
        torch.cuda.synchronize()
        outs.append(out.detach().cpu().clone())
        rows = list(cache_rows(cache))
        if cache.dtype == "fp8":
            rows += [cache.k_scale.cpu().numpy(), cache.v_scale.cpu().numpy()]
        caches.append(rows)
    assert torch.equal(outs[0].view(torch.uint8), outs[1].view(torch.uint8))
    for a, b in zip(*caches):
        assert np.array_equal(a, b)
    if mode == "next":
        check_bf16(to_np(outs[0]), orun.decode_step(inp)["o"], f"step positions {name}")


def test_step_balanced_f32_out(gpu_lib):
    """The balanced step with an fp32 output (the combine in the attention
    launch writes fp32) against the separate calls, bit for bit, and within
    the bars of the oracle."""
    lens = _ragged(48, 97, top=3000) + [0, 1, 64]
    w = small(3, batch=len(lens))
    inp = workloads.make_inputs(3, workload=w, prefill_lens=lens, seed=353)
    say("balanced step, fp32 output")
    outs = []
    for fused in (True, False):
        T, cache, step = setup(inp, num_splits=0, out_dtype=torch.float32)
        fn = step if fused else step.staged
        outs.append(fn(T["k_new"], T["v_new"], T["prefill_lens"], T["seq_lens"], q=T["q"]).clone())
        torch.cuda.synchronize()
    assert outs[0].dtype == torch.float32
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    check_bf16(to_np(outs[0]), orun.decode_step(inp)["o"], "balanced step fp32 out")


@pytest.mark.parametrize("idx,shrink,packed", [
    (2, dict(batch=6, hidden=1024, q_rank=512, context=300), False),
    (2, dict(batch=6, hidden=1024, q_rank=512, context=300), True),
    (2, dict(batch=70, hidden=512, q_rank=256, context=130), True),     # two row passes
    (2, dict(batch=5, hidden=512, q_rank=256, context=200, kv_dtype="fp8", paged=True), True),
    (5, dict(batch=3, context=300), True),                              # 80-column tiles, 16 rows
    (2, dict(batch=24, context=130), True),                             # 80-column tiles, 32 rows
    (2, dict(batch=48, context=130), True),                             # 64-column tiles x 4 K slices
    (1, {}, False),                                                     # fp32 path
], ids=["bf16", "bf16-packed", "bf16-two-passes", "fp8-paged", "split", "full-width",
        "full-width-48", "f32"])
def test_kv_projection_step(gpu_lib, idx, shrink, packed):
    """The K/V projection fused into the step (w_kv): the new token equals
    the oracle's x W_k^T, x W_v^T rounded to the activation dtype; the cache
    holds exactly what mfa_kv_append writes from the step's k/v outputs; the
    attention output matches the oracle step with the projected token."""
    import decode_attention_02_amd as mfa
    w = dataclasses.replace(W[idx], **shrink)
    inp = workloads.make_inputs(idx, workload=w, seed=31, kv_proj=True)
    say(f"kv projection: {w.name} {shrink} packed={packed}")
    act = torch.float32 if w.act_dtype == "f32" else torch.bfloat16
    res = {}
    for mode in ("fused", "staged"):
        T, cache, step = setup(inp, num_splits=3 if (w.context or 0) > 256 else None)
        wts = (T["w_qdown"], T["g"], T["w_qup"])
        wkv = T["w_kv"]
        if packed:
            step.packed_weights = True
            wts = (mfa.pack_weight(wts[0]), wts[1], mfa.pack_weight(wts[2]))
            wkv = mfa.pack_weight(wkv)
        if mode == "fused":
            k_out = torch.empty((w.batch, w.head_dim), dtype=act, device="cuda")
            v_out = torch.empty_like(k_out)
            out = step(k_out, v_out, T["prefill_lens"], T["seq_lens"], x=T["x"], weights=wts,
                       w_kv=wkv)
            torch.cuda.synchronize()
            res["k"], res["v"] = k_out.clone(), v_out.clone()
        else:
            out = step.staged(res["k"], res["v"], T["prefill_lens"], T["seq_lens"], x=T["x"],
                              weights=wts)
            torch.cuda.synchronize()
        rows = list(cache_rows(cache))
        if cache.dtype == "fp8":
            rows += [cache.k_scale.cpu().numpy(), cache.v_scale.cpu().numpy()]
        res[mode] = (out.detach().cpu().clone(), rows)
    # 1. the projected token against the oracle's exact projection
    kx, vx = omfa.kv_projection(omfa.stored_to_f64(inp["x"], w.act_dtype),
                                omfa.stored_to_f64(inp["w_kv"], w.act_dtype), w.head_dim)
    for got, want, n in ((to_np(res["k"]), kx, "k"), (to_np(res["v"]), vx, "v")):
        r = rel_l2(got, want)
        if w.act_dtype == "f32":
            say(f"projected {n}: rel_l2={r:.3e}")
            assert r <= REL_L2_F32
        else:
            # one bf16 rounding of a value that differs from the exact one by
            # the fp32 accumulation only: within one unit in the 8th bit
            err = np.abs(got - want) / np.maximum(np.abs(want), 1e-30)
            say(f"projected {n}: rel_l2={r:.3e} max rel={err.max():.3e}")
            assert r <= REL_L2_BF16 and np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -7 + 1e-6)
    # 2. fused cache == append of the step's own k/v outputs (bit for bit);
    # the outputs are not compared bit for bit: with the K/V columns the
    # down-projection may split K differently, so q can differ in its last bits
    for a, b in zip(res["fused"][1], res["staged"][1]):
        assert np.array_equal(a, b)
    # 3. attention output against the oracle step with the projected token
    want = orun.decode_step(inp)["o"]
    got = to_np(res["fused"][0])
    if w.act_dtype == "f32":
        r = rel_l2(got, want)
        say(f"kv projection f32 step: rel_l2={r:.3e}")
        assert r <= REL_L2_F32
    else:
        check_bf16(got, want, "kv projection step")


MULTI = [
    ("bf16-paged", 3, dict(), [3, 62, 63, 64, 65, 200, 777]),
    ("fp8-paged", 4, dict(), [2, 64, 129, 513]),
    ("bf16-contig", 3, dict(paged=False), [130, 5, 64]),
    ("f32-valu", 3, dict(paged=False, kv_dtype="f32", act_dtype="f32", heads=4, head_dim=64),
     [7, 100, 64]),
]


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("T", [2, 4])
@pytest.mark.parametrize("name,base,over,lens", MULTI, ids=[m[0] for m in MULTI])
def test_multi_token_decode(gpu_lib, name, base, over, lens, T, splits):
    """T new tokens per sequence attending causally (mfa_decode_attn_multi)
    against the oracle; sequences shorter than T included (their early
    queries see nothing or only part of the new tokens)."""
    import decode_attention_02_amd as mfa
    w = small(base, batch=len(lens), **over)
    inp = workloads.make_inputs(base, workload=w, seed=41, prefill_lens=lens, q_len=T)
    say(f"multi-token {name} T={T} splits={splits}")
    T_, cache, step = setup(inp)
    mfa.kv_append(cache, T_["k_new"], T_["v_new"], T_["prefill_lens"])
    maxlen = int(inp["seq_lens"].max())
    chunk = -(-(-(-maxlen // splits)) // 64) * 64 if splits > 1 else None
    out = mfa.decode_attn_multi(T_["q_multi"], cache, T_["seq_lens"], maxlen,
                                num_splits=splits, chunk_tokens=chunk)
    torch.cuda.synchronize()
    want = orun.decode_step_multi(inp)
    got = to_np(out)
    if w.act_dtype == "f32":
        r = rel_l2(got, want)
        say(f"multi-token f32: rel_l2={r:.3e}")
        assert r <= REL_L2_F32
    else:
        check_bf16(got, want, f"multi-token {name} T={T}")


@pytest.mark.parametrize("seed", range(16))
def test_random_sweep(gpu_lib, seed):
    """Seeded random configurations against the oracle: cache type (bf16 or
    FP8), layout (paged or contiguous), 1..24 sequences with a length mix
    that includes empty, one-token, one-block and block-edge rows, the plan
    (the library's from the lengths, the balanced partition, or a fixed
    split count) and 1..3 query tokens."""
    import decode_attention_02_amd as mfa
    rng = np.random.default_rng(7000 + seed)
    base = int(rng.choice([3, 4]))
    paged = bool(rng.integers(0, 2))
    B = int(rng.integers(1, 25))
    top = int(rng.choice([200, 1500, 3000]))
    lens = [int(x) for x in rng.integers(0, top, size=B)]
    for e in (0, 1, 63, 64, 65):
        if rng.random() < 0.3:
            lens[int(rng.integers(0, B))] = e
    plan = str(rng.choice(["lib", "balanced", "fixed"]))
    T = int(rng.choice([1, 1, 2, 3]))
    w = small(base, batch=B, **({} if paged else dict(paged=False)))
    inp = workloads.make_inputs(base, workload=w, seed=7100 + seed, prefill_lens=lens, q_len=T)
    maxlen = int(inp["seq_lens"].max())
    if plan == "balanced":
        ns, chunk = 0, None
    elif plan == "fixed":
        ns = int(rng.choice([1, 2, 3, 5, 8]))
        chunk = -(-(-(-max(maxlen, 1) // ns)) // 64) * 64
    else:
        ns, chunk = None, None
    say(f"sweep seed={seed}: base={base} paged={paged} B={B} T={T} plan={plan} ns={ns} "
        f"lens={lens}")
    if T == 1:
        T_, cache, step = setup(inp, num_splits=ns, chunk_tokens=chunk)
        _, out = run(T_, step)
        got, want = to_np(out), orun.decode_step(inp)["o"]
    else:
        T_, cache, step = setup(inp)
        mfa.kv_append(cache, T_["k_new"], T_["v_new"], T_["prefill_lens"])
        if ns is None:
            vl = (np.asarray(inp["seq_lens"]).reshape(B, 1) - (T - 1) + np.arange(T)).reshape(-1)
            ns, chunk = mfa.decode_plan_lens(64, 256, np.maximum(vl, 0), w.kv_dtype)
            chunk = chunk or None
        out = mfa.decode_attn_multi(T_["q_multi"], cache, T_["seq_lens"], maxlen,
                                    num_splits=ns, chunk_tokens=chunk)
        torch.cuda.synchronize()
        got, want = to_np(out), orun.decode_step_multi(inp)
    assert np.all(np.isfinite(got))
    check_bf16(got, want, f"sweep seed={seed}")


@pytest.mark.parametrize("seed", range(8))
def test_random_sweep_vector_kernel(gpu_lib, seed):
    """Seeded random configurations of the fp32 path (the vector-ALU kernel):
    head count and width, paged or contiguous, 1..12 sequences with planted
    edge lengths, the library's plan or fixed splits, 1..2 query tokens;
    fp32 bar against the oracle."""
    import decode_attention_02_amd as mfa
    rng = np.random.default_rng(7500 + seed)
    H, d = [(4, 64), (8, 128), (64, 64), (16, 256), (32, 256)][int(rng.integers(0, 5))]
    paged = bool(rng.integers(0, 2))
    B = int(rng.integers(1, 13))
    lens = [int(x) for x in rng.integers(0, int(rng.choice([150, 700])), size=B)]
    for e in (0, 1, 31, 32, 63, 64, 65):
        if rng.random() < 0.3:
            lens[int(rng.integers(0, B))] = e
    T = int(rng.choice([1, 2]))
    fixed = bool(rng.integers(0, 2))
    w = small(3, batch=B, kv_dtype="f32", act_dtype="f32", heads=H, head_dim=d,
              **({} if paged else dict(paged=False)))
    inp = workloads.make_inputs(3, workload=w, seed=7600 + seed, prefill_lens=lens, q_len=T)
    maxlen = int(inp["seq_lens"].max())
    ns, chunk = None, None
    if fixed:
        ns = int(rng.choice([2, 3, 5]))
        chunk = -(-(-(-max(maxlen, 1) // ns)) // 64) * 64
    say(f"vector sweep seed={seed}: H={H} d={d} paged={paged} B={B} T={T} ns={ns} lens={lens}")
    T_, cache, step = setup(inp)
    mfa.kv_append(cache, T_["k_new"], T_["v_new"], T_["prefill_lens"])
    if ns is None:
        ns, chunk = mfa.decode_plan(B * T, H, d, max(maxlen, 1), "f32")
    out = mfa.decode_attn_multi(T_["q_multi"] if T > 1 else T_["q"].unsqueeze(1), cache,
                                T_["seq_lens"], maxlen, num_splits=ns, chunk_tokens=chunk)
    torch.cuda.synchronize()
    got = to_np(out)
    want = orun.decode_step_multi(inp) if T > 1 else orun.decode_step(inp)["o"][:, None]
    r = rel_l2(got, want)
    say(f"vector sweep seed={seed}: rel_l2={r:.3e}")
    assert np.all(np.isfinite(got)) and r <= REL_L2_F32, (seed, r)


def test_multi_token_max_query_tokens(gpu_lib):
    """q_len = 16, the most the library takes, with sequences shorter than
    q_len (their first queries see nothing), 2 splits."""
    import decode_attention_02_amd as mfa
    lens = [0, 5, 15, 16, 200]
    w = small(3, batch=len(lens))
    inp = workloads.make_inputs(3, workload=w, seed=43, prefill_lens=lens, q_len=16)
    say("multi-token q_len=16")
    T_, cache, step = setup(inp)
    mfa.kv_append(cache, T_["k_new"], T_["v_new"], T_["prefill_lens"])
    maxlen = int(inp["seq_lens"].max())
    out = mfa.decode_attn_multi(T_["q_multi"], cache, T_["seq_lens"], maxlen, num_splits=2,
                                chunk_tokens=-(-(-(-maxlen // 2)) // 64) * 64)
    torch.cuda.synchronize()
    want = orun.decode_step_multi(inp)
    got = to_np(out)
    # query token j of sequence b sees L_b - (15 - j) tokens; none: zeros
    for b, L in enumerate(inp["seq_lens"]):
        for j in range(16):
            if L - (15 - j) <= 0:
                assert not np.any(got[b, j]), (b, j)
    check_bf16(got, want, "multi-token q_len=16")


def test_multi_token_one_is_single_token(gpu_lib):
    """q_len = 1 through mfa_decode_attn_multi is bit-identical to mfa_decode_attn."""
    import decode_attention_02_amd as mfa
    w = small(3, batch=5)
    inp = workloads.make_inputs(3, workload=w, seed=42, prefill_lens=[1, 63, 64, 300, 129])
    T_, cache, step = setup(inp)
    mfa.kv_append(cache, T_["k_new"], T_["v_new"], T_["prefill_lens"])
    maxlen = int(inp["seq_lens"].max())
    for splits in (1, 2):
        chunk = -(-(-(-maxlen // splits)) // 64) * 64
        a = mfa.decode_attn(T_["q"], cache, T_["seq_lens"], maxlen, num_splits=splits,
                            chunk_tokens=chunk)
        b = mfa.decode_attn_multi(T_["q"].unsqueeze(1), cache, T_["seq_lens"], maxlen,
                                  num_splits=splits, chunk_tokens=chunk)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.squeeze(1).view(torch.int16))


# ---------------------------------------------------------------- FP8 queries
# FP8 caches; 5 and 3 sequences run one workgroup per split, 8 sequences (and
# 4 x q_len 2) walk each split as two halves; q_len 1, 2 and 4; 1 and 3 splits.
Q8_CASES = [
    ("paged", dict(), [0, 63, 64, 190, 513], 1),
    ("contig", dict(paged=False), [255, 70, 3], 1),
    ("paged-8", dict(), [0, 1, 63, 64, 65, 190, 513, 1000], 1),
    ("paged-T2", dict(), [2, 64, 129, 513], 2),
    ("contig-T4", dict(paged=False), [3, 64, 300], 4),
]


def run_q8(inp, T, splits, cache, T_):
    import decode_attention_02_amd as mfa
    mfa.kv_append(cache, T_["k_new"], T_["v_new"], T_["prefill_lens"])
    maxlen = int(inp["seq_lens"].max())
    chunk = -(-(-(-maxlen // splits)) // 64) * 64 if splits > 1 else None
    q = T_["q_multi"] if T > 1 else T_["q"].unsqueeze(1)
    return mfa.decode_attn_multi(q, cache, T_["seq_lens"], maxlen, num_splits=splits,
                                 chunk_tokens=chunk, fp8_queries=True)


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("name,over,lens,T", Q8_CASES, ids=[c[0] for c in Q8_CASES])
def test_fp8_queries(gpu_lib, name, over, lens, T, splits):
    """mfa_decode_attn_q8 against the oracle with the same per-(row, head)
    e4m3 queries; the output is also closer to that reading than to
    attention with the unquantised queries (the quantisation really runs)."""
    w = small(4, batch=len(lens), **over)
    inp = workloads.make_inputs(4, workload=w, seed=61, prefill_lens=lens, q_len=T)
    say(f"fp8 queries {name} T={T} splits={splits}")
    T_, cache, step = setup(inp)
    out = run_q8(inp, T, splits, cache, T_)
    torch.cuda.synchronize()
    got = to_np(out) if T > 1 else to_np(out)[:, 0]
    if T > 1:
        want, plain = (orun.decode_step_multi(inp, fp8_queries=True),
                       orun.decode_step_multi(inp))
    else:
        want, plain = (orun.decode_step(inp, fp8_queries=True)["o"], orun.decode_step(inp)["o"])
    check_bf16(got, want, f"fp8 queries {name}")
    rq, rp = rel_l2(got, want), rel_l2(got, plain)
    say(f"fp8 queries {name}: rel_l2 vs e4m3-q oracle {rq:.3e}, vs bf16-q oracle {rp:.3e}")
    assert rq < rp


def test_fp8_queries_rejects_bf16_cache(gpu_lib):
    import decode_attention_02_amd as mfa
    from decode_attention_02_amd._lib import MfaError
    w = small(3, batch=2)
    inp = workloads.make_inputs(3, workload=w, seed=62, prefill_lens=[10, 70])
    T_, cache, step = setup(inp)
    with pytest.raises(MfaError, match="UNSUPPORTED"):
        mfa.decode_attn_multi(T_["q"].unsqueeze(1), cache, T_["seq_lens"], 71, fp8_queries=True)


# ---------------------------------------------------------------- output projection
def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def check_a2f(y, codes, scales, want, what):
    """y within the bf16 bars of the fp64 projection; the FP8 pack is a
    deterministic function of the library's own bf16 row, so the oracle's
    pack of exactly that row (oracle.mfa.a2f_pack) must equal the library's
    codes and scales bit for bit, on every row."""
    check_bf16(to_np(y), want["y"], f"{what} y")
    yb = bf16_bits(y)
    cg, sg = codes.cpu().numpy(), scales.cpu().numpy()
    oc, os_ = omfa.a2f_pack(yb)
    say(f"{what}: y bits equal to the oracle's rounding {np.mean(yb == want['y_bits']):.5f}")
    assert np.array_equal(sg.view(np.uint32), os_.view(np.uint32)), f"{what}: scales differ"
    assert np.array_equal(cg, oc), f"{what}: codes differ"
    deq = omfa.dequantize_tokens(cg, sg)
    r = rel_l2(deq, want["y"])
    say(f"{what}: dequantised pack rel_l2={r:.3e}")
    assert r <= 0.04                    # e4m3 keeps 3 mantissa bits: rms error ~2^-6


OUTPROJ = [
    # (B, heads*head_dim via heads, hidden, packed)
    (1, 4, 512, False),
    (256, 4, 8192, True),           # the limits: two passes of 128 rows, hidden 8192
    (5, 64, 7168, False),
    (32, 64, 7168, True),           # 112-column tiles x 4 K slices: 256 workgroups
    (64, 4, 1024, True),
    (70, 64, 2048, False),
    (128, 64, 7168, True),
    (128, 64, 7168, False),
]


@pytest.mark.parametrize("B,heads,hidden,packed", OUTPROJ)
def test_out_proj(gpu_lib, B, heads, hidden, packed):
    """y = o W_o^T and its per-token FP8 pack (mfa_out_proj) against the
    oracle; 128 tokens of Step-3's shape is the page's A2F payload (the last
    two cases). Up to 32 rows at 7168 columns run 112-column tiles; 65 to
    128 rows with packed weights run the row-split kernel; B = 256 takes two
    passes of 128 rows."""
    import decode_attention_02_amd as mfa
    w = small(2, batch=B, heads=heads, hidden=hidden, context=65)
    inp = workloads.make_inputs(2, workload=w, seed=51, out_proj=True)
    T = workloads.to_torch(inp)
    say(f"out_proj B={B} HD={heads * 256} hidden={hidden} packed={packed}")
    wo = mfa.pack_weight(T["w_o"]) if packed else T["w_o"]
    y, codes, scales = mfa.out_proj(T["o_attn"], wo, packed=packed)
    torch.cuda.synchronize()
    want = orun.output_projection(inp)
    check_a2f(y, codes, scales, want, f"out_proj B={B}")
    # y alone and the pack alone give the same bytes as both together
    y2, _, _ = mfa.out_proj(T["o_attn"], wo, packed=packed, want_fp8=False)
    _, c3, s3 = mfa.out_proj(T["o_attn"], wo, packed=packed, want_y=False)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(codes, c3) and torch.equal(scales, s3)


def test_out_proj_zero_rows(gpu_lib):
    """A zero attention output row projects to zeros, packs with scale 1 and
    all-zero codes, next to non-zero rows."""
    import decode_attention_02_amd as mfa
    w = small(2, batch=6, heads=4, hidden=512, context=65)
    inp = workloads.make_inputs(2, workload=w, seed=52, out_proj=True)
    inp["o_attn"][[0, 4]] = 0
    T = workloads.to_torch(inp)
    say("out_proj zero rows")
    y, codes, scales = mfa.out_proj(T["o_attn"], T["w_o"])
    torch.cuda.synchronize()
    sc = scales.cpu().numpy()
    assert sc[0] == 1.0 and sc[4] == 1.0
    assert not codes[[0, 4]].any() and not y[[0, 4]].float().abs().sum()
    check_a2f(y, codes, scales, orun.output_projection(inp), "out_proj zero rows")


def test_step_then_out_proj(gpu_lib):
    """The decode step's attention output fed to the output projection
    against the oracle's chained fp64 result (errors of both stages add)."""
    import decode_attention_02_amd as mfa
    w = small(3, batch=6)
    inp = workloads.make_inputs(3, workload=w, seed=53, prefill_lens=[0, 63, 64, 200, 700, 129],
                                out_proj=True)
    say("step then out_proj")
    T, cache, step = setup(inp)
    _, o = run(T, step)
    y, codes, scales = mfa.out_proj(o, T["w_o"])
    torch.cuda.synchronize()
    res = orun.decode_step(inp)
    want = orun.output_projection(inp, res["o"])
    check_a2f(y, codes, scales, want, "step -> out_proj")


# ---------------------------------------------------------------- full sizes
def test_full_tiny_f32(gpu_lib):
    inp = workloads.make_inputs(1)
    say("full tiny f32")
    T, cache, step = setup(inp)
    q, out = run(T, step)
    want = orun.decode_step(inp)
    rq, ro = rel_l2(to_np(q), want["q"]), rel_l2(to_np(out), want["o"])
    say(f"tiny f32: q rel_l2={rq:.3e} o rel_l2={ro:.3e}")
    assert rq <= REL_L2_F32 and ro <= REL_L2_F32


def test_full_step3_bf16(gpu_lib):
    inp = workloads.make_inputs(2)
    say("full step3 bf16 4k")
    T, cache, step = setup(inp)
    say(f"plan: splits={step.num_splits} chunk={step.chunk_tokens}")
    q, out = run(T, step)
    want = orun.decode_step(inp)
    check_bf16(to_np(q), want["q"], "step3 q")
    check_bf16(to_np(out), want["o"], "step3 o")


def test_full_paged_mixed(gpu_lib):
    """The full paged mixed-length workload on the split plan for its longest
    row (the lengths-aware plan picks the balanced partition, tested below)."""
    import decode_attention_02_amd as mfa
    inp = workloads.make_inputs(3)
    say("full paged mixed, split plan")
    ns, ch = mfa.decode_plan(128, 64, 256, int(inp["seq_lens"].max()), "bf16")
    T, cache, step = setup(inp, num_splits=ns, chunk_tokens=ch)
    say(f"plan: splits={step.num_splits} chunk={step.chunk_tokens}")
    _, out = run(T, step)
    want = orun.decode_step(inp)
    check_bf16(to_np(out), want["o"], "paged mixed")


def test_full_paged_mixed_balanced(gpu_lib):
    """The full paged mixed-length workload with the plan from its lengths:
    the balanced partition."""
    inp = workloads.make_inputs(3)
    say("full paged mixed, balanced")
    T, cache, step = setup(inp)
    assert step.num_splits == 0
    _, out = run(T, step)
    want = orun.decode_step(inp)
    check_bf16(to_np(out), want["o"], "paged mixed balanced")


def test_full_fp8_32k_sampled(gpu_lib):
    inp = workloads.make_inputs(4)
    say("full fp8 32k")
    T, cache, step = setup(inp)
    say(f"plan: splits={step.num_splits} chunk={step.chunk_tokens}")
    _, out = run(T, step)
    seqs = [0, 7, 15]
    want = orun.decode_step(inp, seqs=seqs)
    check_bf16(to_np(out)[seqs], want["o"], "fp8 32k sampled")
    # stored codes and scales of every token of the sampled sequences
    exp, owned = orun.expected_cache_rows(inp, seqs)
    kg, vg = cache_rows(cache)
    ks = cache.k_scale.cpu().numpy().reshape(-1)
    for b, rows in owned.items():
        assert np.array_equal(kg[rows], exp["k"][rows])
        assert np.array_equal(vg[rows], exp["v"][rows])
        assert np.array_equal(ks[rows].view(np.uint32), exp["k_scale"][rows].view(np.uint32))


def test_full_fp8_32k_fp8_queries_sampled(gpu_lib):
    """FP8 queries at full size (16 sequences of 32K, the library's split
    plan), sampled sequences against the oracle."""
    import decode_attention_02_amd as mfa
    inp = workloads.make_inputs(4)
    say("full fp8 32k, fp8 queries")
    T, cache, step = setup(inp)
    mfa.kv_append(cache, T["k_new"], T["v_new"], T["prefill_lens"])
    out = mfa.decode_attn_multi(T["q"].unsqueeze(1), cache, T["seq_lens"], step.max_seq_len,
                                num_splits=step.num_splits, chunk_tokens=step.chunk_tokens,
                                fp8_queries=True)
    torch.cuda.synchronize()
    seqs = [0, 7, 15]
    want = orun.decode_step(inp, seqs=seqs, fp8_queries=True)
    check_bf16(to_np(out)[seqs, 0], want["o"], "fp8 32k fp8-queries sampled")


def test_full_split32_64k(gpu_lib):
    inp = workloads.make_inputs(5)
    say("full split32 64k")
    T, cache, step = setup(inp)
    assert step.num_splits == 32
    q, out = run(T, step)
    want = orun.decode_step(inp)
    check_bf16(to_np(q), want["q"], "split32 q")
    check_bf16(to_np(out), want["o"], "split32 o")
