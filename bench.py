"""Benchmark of one MFA decode step on one MI355X.

A step is the whole hot path over one batch: query path (down-projection,
RMSNorm, up-projection; workloads that have one), KV append of the new
token, split-KV decode attention, split combine -- each one libmfa C-ABI
call on one stream. Default workload: the largest one, paged bf16 decode of
128 sequences with mixed contexts (uniform in 1024..8192 tokens before the
append, 64-token blocks at permuted physical ids; 64 heads x 256 sharing one
KV head; 620 MB of KV per step). Inputs are seeded and synthetic and
resident in HBM before timing;
``--rotate`` independent copies of cache and weights are cycled so that the
256 MB last-level cache cannot hold a step's working set.

The steps are captured once into HIP graphs (no allocation happens inside a
step) and replayed, so the GPU runs them back to back. Prints one JSON line:
throughput in decode tokens/s over K timed steps; the attention kernel's
roofline (algorithmic KV bytes per launch / its average duration, from HIP
events around K back-to-back attention launches on the same buffers); the
spread of single-step times; a pure read stream of the attention's bytes on
the same device, for reference (libmfa_probe.so); and the fp64 oracle timed
on the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3,
                    help="workload index 1..5 (default 3: the largest, paged mixed lengths)")
    ap.add_argument("--rotate", type=int, default=0, help="buffer sets cycled (0: auto)")
    ap.add_argument("--splits", type=int, default=-1,
                    help="override the split count (0: the balanced partition; -1: the plan)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-ceiling", action="store_true",
                    help="skip the pure read-stream reference measurement")
    ap.add_argument("--q-len", type=int, default=1,
                    help="new tokens per sequence decoded together (multi-token decode, "
                         "workloads without a query path)")
    ap.add_argument("--kv-proj", action="store_true",
                    help="compute the new token's K/V from x in the step (w_kv) instead of "
                         "reading it (query-path workloads)")
    ap.add_argument("--out-proj", action="store_true",
                    help="the step also projects the attention output (W_o, hidden 7168 for "
                         "workloads without a query path) and packs it to FP8 (mfa_out_proj)")
    ap.add_argument("--fp8-queries", action="store_true",
                    help="FP8-cache workloads: queries quantized per head and Q.K^T on the FP8 "
                         "matrix cores (mfa_decode_attn_q8)")
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of HIP graphs")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (reference for HBM counters)")
    return ap.parse_args()


def kv_bytes_per_token(w) -> int:
    """K row + V row (+ one fp32 scale each for FP8): 2*d*b (+8)."""
    elem = {"f32": 4, "bf16": 2, "fp8": 1}[w.kv_dtype]
    return 2 * w.head_dim * elem + (8 if w.kv_dtype == "fp8" else 0)


def counters_for(workload_name: str, kernel_sig: str):
    """HBM traffic per launch from a committed rocprofv3 counter summary,
    only if it was taken on the current attention kernel source."""
    path = os.path.join(PROFILE_DIR, f"attn_counters_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_source_sha256") != kernel_sig:
        return None
    return c.get("hbm_bytes_per_launch")


def code_text(src: str) -> str:
    """Source text without // comments, trailing blanks and empty lines: the
    signature follows the code, not its commentary."""
    import re
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in src.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_sig() -> str:
    """sha256 over the code of the attention kernel's sources."""
    import hashlib
    h = hashlib.sha256()
    for name in ("attn_mfma.hip", "device_common.h", "kernels.h"):
        with open(os.path.join(ROOT, "decode_attention_02_amd", "csrc", name)) as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or the platform's processor."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(inp, min_seconds: float = 10.0, fp8_queries: bool = False,
                 one_thread_seconds: float = 4.0):
    """fp64 oracle on the same inputs: the whole batch (query path, cache
    fill, attention of every sequence, and the output projection with its FP8
    pack when the inputs hold W_o), repeated until ``min_seconds`` of
    host time have passed, on the BLAS threads the host gives; then the same
    oracle on one thread over the first sequences of the batch (at most 16),
    repeated for ``one_thread_seconds``. Returns the record."""
    import numpy as np  # noqa: F401
    from oracle import run as orun
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = len(os.sched_getaffinity(0))
    w = inp["workload"]
    multi = "q_multi" in inp
    tq = inp["q_multi"].shape[1] if multi else 1

    def timed(seqs, seconds):
        runs, total = 0, 0.0
        while total < seconds and runs < 50:
            t0 = time.perf_counter()
            if multi:
                orun.decode_step_multi(inp, fp8_queries=fp8_queries, seqs=seqs)
            else:
                res = orun.decode_step(inp, seqs=seqs, fp8_queries=fp8_queries)
                if "w_o" in inp and seqs is None:
                    orun.output_projection(inp, res["o"])
            total += time.perf_counter() - t0
            runs += 1
        return total / runs, runs

    dt, runs = timed(None, min_seconds)
    toks = int(inp["seq_lens"].sum())
    rec = {"value": w.batch * tq / dt, "unit": "decode tokens/s", "cores": int(threads),
           "kind": "oracle", "cpu_model": cpu_model(),
           "kv_tokens_per_s": toks / dt,
           "sample": f"whole batch of workload {w.name} ({w.batch} sequences, {toks} cached "
                     f"tokens{', with output projection' if 'w_o' in inp else ''}), fp64 numpy, "
                     f"{threads} BLAS threads, mean of {runs} runs ({dt:.2f} s each)"}
    if threadpool_limits is not None:
        nseq = min(16, w.batch)
        seqs = list(range(nseq))
        with threadpool_limits(1):
            dt1, runs1 = timed(seqs, one_thread_seconds)
        toks1 = int(inp["seq_lens"][:nseq].sum())
        rec["one_thread"] = {
            "value": nseq * tq / dt1, "unit": "decode tokens/s", "cores": 1,
            "kv_tokens_per_s": toks1 / dt1,
            "sample": f"sequences 0..{nseq - 1} of {w.name} ({toks1} cached tokens; the query "
                      f"path of the whole batch included), fp64 numpy on 1 thread, mean of "
                      f"{runs1} runs ({dt1:.2f} s each)"}
    return rec


def stream_ceiling(device, nbytes: int = 134217728, copies: int = 4, reps: int = 20) -> dict:
    """Read bandwidth of a pure stream of nbytes (16-byte non-temporal loads,
    one workgroup per compute unit) over `copies` rotating buffers, so the
    last-level cache cannot hold them: the same bytes the 4K attention reads,
    streamed with nothing else to do."""
    import ctypes

    import torch
    from decode_attention_02_amd import build as mbuild
    lib = ctypes.CDLL(mbuild.PROBE)
    lib.mfa_probe_stream.restype = ctypes.c_int
    lib.mfa_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device=device) for _ in range(copies)]
    sink = torch.empty(512 * 16, dtype=torch.uint8, device=device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)

    def launch(i):
        rc = lib.mfa_probe_stream(ctypes.c_void_p(bufs[i % copies].data_ptr()), nbytes, 256, 1,
                                  ctypes.c_void_p(sink.data_ptr()), stream)
        if rc != 0:
            raise RuntimeError(f"stream probe failed ({rc})")
    for i in range(copies * 2):
        launch(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del bufs
    return {"GBps": nbytes / (us * 1e-6) / 1e9, "bytes": nbytes, "us": us,
            "kind": "non-temporal 16-byte loads, 256 workgroups, 4 rotating buffers"}


def copy_calibration(mib: int) -> None:
    """Five device-to-device copies of exactly ``mib`` MiB each: a kernel whose
    HBM traffic is known (mib MiB read, mib MiB written per launch), so that
    rocprofv3's FETCH_SIZE / WRITE_SIZE readings can be scaled to bytes."""
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    pad = torch.empty(1 << 27, dtype=torch.float32, device="cuda:0")
    for _ in range(5):
        pad.fill_(0.0)           # evict src/dst from the 256 MB last-level cache
        torch.mul(src, 1.0, out=dst)   # one elementwise kernel: n bytes in, n bytes out
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import decode_attention_02_amd as mfa
    import workloads
    from decode_attention_02_amd.step import DecodeStep, prefill

    mfa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.WORKLOADS[args.config]
    if args.kv_proj and not w.has_qproj:
        print("--kv-proj needs a workload with a query path (configs 1, 2, 5)", file=sys.stderr)
        sys.exit(2)
    TQ = args.q_len
    if TQ > 1 and w.has_qproj:
        print("--q-len > 1 needs a workload whose queries are drawn (configs 3, 4)", file=sys.stderr)
        sys.exit(2)
    if args.fp8_queries and (w.kv_dtype != "fp8" or w.has_qproj):
        print("--fp8-queries needs an FP8-cache workload (config 4)", file=sys.stderr)
        sys.exit(2)
    MULTI = TQ > 1 or args.fp8_queries          # append + mfa_decode_attn_multi / _q8 per step
    if args.out_proj and (TQ > 1 or w.act_dtype != "bf16"):
        print("--out-proj needs a single-token bf16 workload (configs 2..5)", file=sys.stderr)
        sys.exit(2)
    inp = workloads.make_inputs(args.config, kv_proj=args.kv_proj, q_len=TQ,
                                out_proj=args.out_proj)
    T = workloads.to_torch(inp, dev)
    act = torch.float32 if w.act_dtype == "f32" else torch.bfloat16
    B = w.batch
    maxlen = int(inp["seq_lens"].max())
    kvb = kv_bytes_per_token(w)
    kv_bytes = int(inp["seq_lens"].sum()) * kvb
    w_bytes = 0
    if w.has_qproj:
        w_bytes = (T["w_qdown"].numel() + T["w_qup"].numel()) * T["w_qup"].element_size()
        if args.kv_proj:
            w_bytes += T["w_kv"].numel() * T["w_kv"].element_size()
    if args.out_proj:
        hid = T["w_o"].shape[0]
        HDo = T["w_o"].shape[1]
        w_bytes += T["w_o"].numel() * 2
        # algorithmic bytes of one output projection: W_o, o, y, FP8 codes, scales
        op_bytes = hid * HDo * 2 + B * HDo * 2 + B * hid * 2 + B * hid + B * 4
    # at least 4 sets, and together at least twice the 256 MB last-level cache
    rotate = args.rotate or max(4, min(8, -(-2 * 256 * 2 ** 20 // max(kv_bytes + w_bytes, 1))))

    sets = []
    for r in range(rotate):
        cache = mfa.KVCache(inp["num_blocks"], w.head_dim, w.kv_dtype, inp["max_blocks_per_seq"],
                            block_table=T["block_table"], device=dev, zero=False)
        prefill(cache, T["k_ctx"], T["v_ctx"], inp["ctx_offsets"], inp["prefill_lens"])
        ns = args.splits if args.splits >= 0 else w.num_splits
        packed = w.has_qproj and w.act_dtype == "bf16"
        step = DecodeStep(cache, B, w.heads, maxlen, hidden=w.hidden, q_rank=w.q_rank,
                          act_dtype=act, num_splits=ns, packed_weights=packed, device=dev,
                          seq_lens_host=inp["seq_lens"])
        wts, wkv = None, None
        if w.has_qproj:
            # weights are static: packed once into operand order, like a load step
            if packed:
                wts = (mfa.pack_weight(T["w_qdown"]), T["g"].clone(), mfa.pack_weight(T["w_qup"]))
                wkv = mfa.pack_weight(T["w_kv"]) if args.kv_proj else None
            else:
                wts = (T["w_qdown"].clone(), T["g"].clone(), T["w_qup"].clone())
                wkv = T["w_kv"].clone() if args.kv_proj else None
        sets.append((step, wts, wkv))
    torch.cuda.synchronize()
    ops = []
    if args.out_proj:
        nb = mfa.load().mfa_out_proj_workspace_bytes(B, HDo, hid, 1)
        for r in range(rotate):
            ops.append((mfa.pack_weight(T["w_o"]),
                        torch.empty(max(nb, 16), dtype=torch.uint8, device=dev),
                        (torch.empty((B, hid), dtype=torch.bfloat16, device=dev),
                         torch.empty((B, hid), dtype=torch.uint8, device=dev),
                         torch.empty(B, dtype=torch.float32, device=dev))))
        torch.cuda.synchronize()

    def project(i):
        step = sets[i % rotate][0]
        wo, ws, outs = ops[i % rotate]
        mfa.out_proj(step.out, wo, packed=True, workspace=ws, out=outs)

    if MULTI:
        # multi-token decode: the step appends TQ tokens per sequence (the last TQ
        # positions) and attends with the TQ queries of each, causal among them
        # (TQ = 1 with FP8 queries: the single-token step through the same call)
        ns_m, ch_m = mfa.decode_plan(B * TQ, w.heads, w.head_dim, maxlen, w.kv_dtype)
        if args.splits >= 0:
            ns_m = args.splits
            ch_m = mfa.api._chunk(maxlen, ns_m)
        k_m = T["k_new"].unsqueeze(1).expand(B, TQ, w.head_dim).contiguous()
        v_m = T["v_new"].unsqueeze(1).expand(B, TQ, w.head_dim).contiguous()
        pos_m = (T["seq_lens"] - TQ).to(torch.int32)
        q_m = T["q_multi"] if TQ > 1 else T["q"].unsqueeze(1)
        multi = []
        for r in range(rotate):
            nb = mfa.split_workspace_bytes(B * TQ, w.heads, w.head_dim, ns_m)
            multi.append((torch.empty(max(nb, 16), dtype=torch.uint8, device=dev),
                          torch.empty((B, TQ, w.heads, w.head_dim), dtype=act, device=dev)))

    def attention_multi(i, combine):
        step = sets[i % rotate][0]
        ws, out = multi[i % rotate]
        mfa.decode_attn_multi(q_m, step.cache, T["seq_lens"], maxlen, step.sm_scale,
                              ns_m, ch_m, out=out if combine else None, workspace=ws,
                              combine=combine, fp8_queries=args.fp8_queries)

    def attention(i, q):
        if MULTI:
            attention_multi(i, combine=ns_m == 1)
            return
        step = sets[i % rotate][0]
        if step.num_splits != 1:
            mfa.decode_attn(q, step.cache, T["seq_lens"], step.max_seq_len, step.sm_scale,
                            step.num_splits, step.chunk_tokens, workspace=step.split_ws,
                            combine=False)
        else:
            step.attend(q, T["seq_lens"])

    def one(i):
        """One decode step on buffer set i % rotate (DecodeStep: query path,
        KV append, attention, split combine)."""
        step, wts, wkv = sets[i % rotate]
        if MULTI:
            mfa.kv_append(step.cache, k_m, v_m, pos_m)
            attention_multi(i, combine=True)
            return
        if w.has_qproj:
            step(T["k_new"], T["v_new"], T["prefill_lens"], T["seq_lens"], x=T["x"], weights=wts,
                 w_kv=wkv)
        else:
            step(T["k_new"], T["v_new"], T["prefill_lens"], T["seq_lens"], q=T["q"])
        if args.out_proj:
            project(i)

    q_fixed = [sets[r][0].q if w.has_qproj else T["q"] for r in range(rotate)]

    def capture(fn):
        """HIP graph of fn's launches (one graph launch replays them back to back)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    use_graph = not args.eager
    if use_graph:
        g_ones = [capture(lambda r=r: one(r)) for r in range(rotate)]
        g_warm = capture(lambda: [one(i) for i in range(args.warmup)])
        g_steps = capture(lambda: [one(i) for i in range(args.steps)])
        g_attn = capture(lambda: [attention(i, q_fixed[i % rotate]) for i in range(args.steps)])
        if args.out_proj:
            g_op = capture(lambda: [project(i) for i in range(args.steps)])
    # warmup
    if use_graph:
        g_warm.replay()
    else:
        for i in range(args.warmup):
            one(i)
    torch.cuda.synchronize()
    # timed region 1: K whole steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    if use_graph:
        g_steps.replay()
    else:
        for i in range(args.steps):
            one(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    # timed region 2: K attention launches back to back (same buffers, same
    # rotation), bracketed by HIP events on the launching stream
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    if use_graph:
        g_attn.replay()
    else:
        for i in range(args.steps):
            attention(i, q_fixed[i % rotate])
    a1.record()
    torch.cuda.synchronize()
    attn_avg = a0.elapsed_time(a1) / args.steps
    # per-step spread: one step at a time (same buffer rotation), events around each
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        if use_graph:
            g_ones[i % rotate].replay()
        else:
            one(i)
        e1.record()
    torch.cuda.synchronize()
    per_step = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)

    def pct(q):
        return per_step[min(len(per_step) - 1, int(q * (len(per_step) - 1) + 0.5))]
    op_rec = None
    if args.out_proj:
        # timed region 3: K output projections back to back
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record()
        if use_graph:
            g_op.replay()
        else:
            for i in range(args.steps):
                project(i)
        p1.record()
        torch.cuda.synchronize()
        op_avg = p0.elapsed_time(p1) / args.steps
        op_ach = op_bytes / (op_avg * 1e-3) / 1e9
        op_rec = {"bound": "hbm", "achieved": op_ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": op_ach / HBM_PEAK_GBS, "kernels": "gemm_skinny_kernel+outproj_pack_kernel",
                  "call_avg_us": op_avg * 1e3, "algorithmic_bytes_per_call": op_bytes,
                  "hidden": hid, "tokens": B}
    achieved = kv_bytes / (attn_avg * 1e-3) / 1e9
    step0 = sets[0][0]
    traffic = counters_for(w.name, kernel_source_sig())
    rec = {
        "metric": "MFA decode-attention tokens/s and achieved KV HBM GB/s (% of peak), 1xMI355X",
        "value": B * TQ / (ms * 1e-3),
        "unit": "decode tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else (
            ("fp8-qk/bf16-pv" if args.fp8_queries else "fp8-kv/bf16") if w.kv_dtype == "fp8"
            else "f32"),
        "data": "synthetic (seeded N(0,1) K/V, N(0,1/fan_in) weights, random-init)",
        "config": {"workload": w.name, "batch": B, "context": maxlen, "heads": w.heads,
                   "head_dim": w.head_dim, "kv_dtype": w.kv_dtype, "hidden": w.hidden,
                   "q_rank": w.q_rank, "paged": w.paged,
                   "num_splits": ns_m if MULTI else step0.num_splits,
                   "chunk_tokens": ch_m if MULTI else step0.chunk_tokens, "rotate": rotate,
                   "q_len": TQ, "fp8_queries": bool(args.fp8_queries),
                   "step": (("qproj+kv_proj+kv_append+decode_attn+combine" if args.kv_proj
                             else "qproj+kv_append+decode_attn+combine") if w.has_qproj
                            else ("kv_append(q_len)+decode_attn_q8+combine" if args.fp8_queries
                                  else "kv_append(q_len)+decode_attn_multi+combine" if TQ > 1
                                  else "kv_append+decode_attn+combine"))
                   + ("+out_proj+fp8_pack" if args.out_proj else "")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (traffic / (attn_avg * 1e-3) / 1e9) if traffic else None,
                     "traffic_bytes_per_launch": traffic,
                     "kernel": ("mfa_decode_mfma_kernel"
                                if (w.heads == 64 and w.head_dim == 256 and w.kv_dtype != "f32")
                                else "mfa_decode_valu_kernel"),
                     "kernel_avg_us": attn_avg * 1e3,
                     "algorithmic_bytes_per_launch": kv_bytes},
        "step_kv_plus_weights_GBps": (kv_bytes + w_bytes) / (ms * 1e-3) / 1e9,
        "kv_tokens_per_s": int(inp["seq_lens"].sum()) / (ms * 1e-3),
        "step_us_single": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9),
                           "note": "one step per replay, events around each (adds the per-replay "
                                   "launch); value/ms_per_step time K steps in one replay"},
    }
    if not args.no_stream_ceiling:
        ceil = stream_ceiling(dev)
        ceil["attention_frac_of_ceiling"] = achieved / ceil["GBps"]
        rec["stream_ceiling"] = ceil
    if op_rec is not None:
        rec["out_proj_roofline"] = op_rec
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(inp, fp8_queries=args.fp8_queries)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
