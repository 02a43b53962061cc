"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/mfa.h declares, and rejects malformed calls on the host before
anything is launched. Fake device pointers are only ever passed to calls
that fail validation, so no kernel runs."""
import ctypes
import os
import re

import pytest

from decode_attention_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mfa.h")

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS = 0, 1, 2, 3, 4, 5, 6
F32, BF16, FP8 = 0, 1, 2
P = 0x10000          # fake, 16-byte aligned, never dereferenced
PM = 0x10008         # fake, misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mfa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmfa.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    decl = declared_functions()
    assert decl, "no declarations parsed"
    assert sorted(_lib.SIGNATURES) == decl, "binding signatures differ from the header"
    for name in decl:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.mfa_abi_version() == _lib.ABI_VERSION == 3
    for s in range(8):
        assert lib.mfa_status_str(s)
    assert lib.mfa_status_str(99) == b"unknown status"


def _cache(**kw):
    d = _lib.KVCacheDesc()
    d.k, d.v = P, P + 4096
    d.k_scale = d.v_scale = None
    d.block_table = None
    d.num_blocks, d.max_blocks_per_seq, d.head_dim, d.dtype = 64, 16, 256, BF16
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _attn(lib, cache, q=P, qdt=BF16, B=4, H=64, seq=P, maxlen=512, ns=1, chunk=512, ws=None,
          wsb=0, out=P, odt=BF16, scale=0.0625):
    return lib.mfa_decode_attn(q, qdt, B, H, ctypes.byref(cache), seq, maxlen, scale, ns, chunk,
                               ws, wsb, out, odt, None)


def test_decode_attn_validation(lib):
    c = _cache()
    assert _attn(lib, c, q=None) == NULL
    assert _attn(lib, c, seq=None) == NULL
    assert _attn(lib, c, q=PM) == ALIGN
    assert _attn(lib, _cache(k=PM)) == ALIGN
    assert _attn(lib, _cache(dtype=7)) == DTYPE
    assert _attn(lib, c, maxlen=16 * 64 + 1) == SHAPE            # beyond capacity
    assert _attn(lib, c, ns=-1) == SHAPE
    assert _attn(lib, c, ns=0) == WS                              # balanced: needs a workspace
    assert _attn(lib, c, chunk=100) == SHAPE                     # not a multiple of 64
    assert _attn(lib, c, ns=2, chunk=64, maxlen=512) == SHAPE    # splits do not cover
    assert _attn(lib, c, ns=8, chunk=64, ws=None) == WS
    assert _attn(lib, c, ns=8, chunk=64, ws=P, wsb=16) == WS
    assert _attn(lib, c, qdt=F32) == DTYPE                       # bf16 cache, f32 q on MFMA path
    assert _attn(lib, c, out=None) == NULL
    assert _attn(lib, c, odt=FP8) == DTYPE
    assert _attn(lib, c, B=5) == SHAPE                           # contiguous cache too small
    assert _attn(lib, _cache(dtype=FP8)) == NULL                 # fp8 without scales
    assert _attn(lib, _cache(dtype=FP8, k_scale=P, v_scale=P), H=32) == UNSUP
    assert _attn(lib, _cache(head_dim=96)) == SHAPE
    for bad in (0.0, -0.0625, float("inf"), float("nan")):
        assert _attn(lib, c, scale=bad) == SHAPE                 # scale must be positive, finite


def test_decode_attn_q8_validation(lib):
    def q8(cache, **kw):
        return lib.mfa_decode_attn_q8(kw.get("q", P), kw.get("qdt", BF16), 4, kw.get("ql", 1), 64,
                                      ctypes.byref(cache), P, 512, 0.0625, 1, 512, None, 0, P,
                                      BF16, None)
    fp8 = _cache(dtype=FP8, k_scale=P, v_scale=P)
    assert q8(_cache()) == UNSUP                                   # bf16 cache
    assert q8(fp8, qdt=F32) == DTYPE
    assert q8(fp8, ql=0) == SHAPE
    assert q8(fp8, ql=17) == SHAPE
    assert q8(fp8, q=None) == NULL
    assert q8(fp8, q=PM) == ALIGN


def test_kv_append_validation(lib):
    c = _cache()
    ap = lambda **kw: lib.mfa_kv_append(kw.get("k", P), kw.get("v", P), kw.get("dt", BF16),
                                        kw.get("pos", P), kw.get("n", 1), kw.get("B", 4),
                                        ctypes.byref(kw.get("cache", c)), None)
    assert ap(k=None) == NULL
    assert ap(pos=None) == NULL
    assert ap(v=PM) == ALIGN
    assert ap(n=0) == SHAPE
    assert ap(n=16 * 64 + 1) == SHAPE
    assert ap(dt=F32) == DTYPE                                   # bf16 cache, f32 input
    assert ap(dt=FP8) == DTYPE
    assert ap(B=5) == SHAPE
    assert lib.mfa_kv_append(P, P, BF16, P, 1, 4, None, None) == NULL


def test_qproj_validation_and_workspace(lib):
    q = lambda **kw: lib.mfa_qproj(kw.get("x", P), P, P, P, P, kw.get("ws", P),
                                   kw.get("wsb", 1 << 30), kw.get("B", 32), kw.get("hid", 7168),
                                   kw.get("r", 2048), 64, 256, 1e-6, kw.get("dt", BF16),
                                   kw.get("lay", 0), None)
    assert q(x=None) == NULL
    assert q(x=PM) == ALIGN
    assert q(B=0) == SHAPE
    assert q(B=257) == SHAPE
    assert q(hid=7000) == SHAPE
    assert q(dt=FP8) == DTYPE
    assert q(ws=None) == WS
    assert q(lay=2) == SHAPE                                     # unknown weight layout
    assert q(lay=1, dt=F32, hid=256, r=128) == DTYPE             # packed weights are bf16 only
    need = lib.mfa_qproj_workspace_bytes(32, 7168, 2048, 64, 256, BF16)
    assert need > 0
    assert q(wsb=need - 1) == WS
    assert lib.mfa_qproj_workspace_bytes(32, 7000, 2048, 64, 256, BF16) == 0
    assert lib.mfa_qproj_workspace_bytes(2, 256, 128, 4, 64, F32) > 0


def test_pack_weight_validation(lib):
    assert lib.mfa_pack_weight(None, P, 64, 64, BF16, None) == NULL
    assert lib.mfa_pack_weight(P, P, 64, 64, F32, None) == DTYPE
    assert lib.mfa_pack_weight(P, P, 60, 64, BF16, None) == SHAPE
    assert lib.mfa_pack_weight(P, P, 64, 48, BF16, None) == SHAPE
    assert lib.mfa_pack_weight(PM, P, 64, 64, BF16, None) == ALIGN


def test_out_proj_validation_and_workspace(lib):
    def op(**kw):
        return lib.mfa_out_proj(kw.get("o", P), kw.get("w", P), kw.get("lay", 0), kw.get("B", 128),
                                kw.get("HD", 16384), kw.get("hid", 7168), kw.get("dt", BF16),
                                kw.get("ws", P), kw.get("wsb", 1 << 30), kw.get("y", P),
                                kw.get("codes", P), kw.get("sc", P), None)
    assert op(o=None) == NULL
    assert op(y=None, codes=None, sc=None) == NULL               # nothing to write
    assert op(codes=None) == NULL                                # codes and scales go together
    assert op(sc=None) == NULL
    assert op(B=0) == SHAPE
    assert op(B=257) == SHAPE
    assert op(HD=1000) == SHAPE
    assert op(hid=7000) == SHAPE
    assert op(hid=8256) == SHAPE                                 # above 8192
    assert op(dt=F32) == DTYPE
    assert op(lay=2) == SHAPE
    assert op(o=PM) == ALIGN
    assert op(codes=PM) == ALIGN
    assert op(sc=P + 2) == ALIGN
    assert op(ws=None) == WS
    need = lib.mfa_out_proj_workspace_bytes(128, 16384, 7168, BF16)
    assert need > 0 and need % 256 == 0
    assert op(wsb=need - 1) == WS
    assert lib.mfa_out_proj_workspace_bytes(128, 16384, 7000, BF16) == 0
    assert lib.mfa_out_proj_workspace_bytes(128, 16384, 7168, F32) == 0


def test_plan_and_split_workspace(lib):
    ns, ch = ctypes.c_int(), ctypes.c_int()
    for B, L in ((32, 4096), (128, 8193), (16, 32768), (4, 65536), (1, 1), (2, 0)):
        assert lib.mfa_decode_plan(B, 64, 256, L, BF16, ctypes.byref(ns), ctypes.byref(ch)) == OK
        assert ns.value >= 1 and ch.value % 64 == 0 and ns.value * ch.value >= L
    assert lib.mfa_decode_plan(0, 64, 256, 10, BF16, ctypes.byref(ns), ctypes.byref(ch)) == SHAPE
    # the matrix-core kernel gets splits of two blocks, the vector kernel of one
    for B, L, H, d, dt, want in ((2, 129, 4, 64, F32, (3, 64)), (2, 129, 64, 256, BF16, (1, 256)),
                                 (1, 4096, 64, 256, BF16, (32, 128)), (1, 4096, 8, 128, F32, (64, 64))):
        assert lib.mfa_decode_plan(B, H, d, L, dt, ctypes.byref(ns), ctypes.byref(ch)) == OK
        assert (ns.value, ch.value) == want, (B, L, H, d, dt, ns.value, ch.value)
    assert lib.mfa_decode_workspace_bytes(4, 64, 256, 1) == 0
    rows = 16 * 16 * 64                          # 16 rows x 16 splits: one partial per split
    assert lib.mfa_decode_workspace_bytes(16, 64, 256, 16) == rows * 256 * 4 + rows * 2 * 4
    # 4 rows x 32 splits leave half the chip idle: each split is walked as two
    # halves, so the workspace holds 64 partials per row
    rows = 4 * 64 * 64
    assert lib.mfa_decode_workspace_bytes(4, 64, 256, 32) == rows * 256 * 4 + rows * 2 * 4
    rows = 3 * 5 * 7
    off_ml = -(-rows * 64 * 4 // 256) * 256
    assert lib.mfa_decode_workspace_bytes(3, 7, 64, 5) == off_ml + rows * 2 * 4
    for args in ((4, 64, 256, 32), (3, 7, 64, 5), (1, 1, 1, 1)):
        assert lib.mfa_split_workspace_bytes(*args) == lib.mfa_decode_workspace_bytes(*args)
    assert lib.mfa_combine(None, 0, 4, 64, 256, 32, P, BF16, None) == NULL
    assert lib.mfa_combine(P, 16, 4, 64, 256, 32, P, BF16, None) == WS
    assert lib.mfa_combine(P, 1 << 30, 4, 64, 256, 1, P, BF16, None) == SHAPE


def test_static_scratch_refuses_oversize(lib):
    """mfa_decode_attn_static refuses partials beyond its static scratch on the
    host, before any HIP call (so it runs without a GPU)."""
    desc = _lib.KVCacheDesc(k=P, v=P, num_blocks=1 << 20, max_blocks_per_seq=4096, head_dim=256,
                            dtype=BF16)
    too_many = 300                      # 2 x 300 splits x 64 KB of partials > 32 MiB
    assert lib.mfa_decode_workspace_bytes(2, 64, 256, too_many) > 32 << 20
    rc = lib.mfa_decode_attn_static(P, BF16, 2, 64, ctypes.byref(desc), P, 64 * too_many,
                                    0.0625, too_many, 64, P, BF16, None)
    assert rc == 8 and lib.mfa_status_str(8) == b"request needs more than the library's static scratch"
    assert lib.mfa_decode_attn_static(P, BF16, 2, 64, ctypes.byref(desc), P, 100, 0.0625, 2, 64,
                                      None, BF16, None) == NULL


def test_balanced_partition_limits(lib):
    """num_splits == 0 (balanced partition): workspace for 256 + B slots plus
    per-row metadata; more than 1024 rows is a shape error, before any HIP
    call."""
    rows = (256 + 100) * 64
    off_ml = rows * 256 * 4
    off_meta = -(-(off_ml + rows * 8) // 16) * 16
    assert lib.mfa_decode_workspace_bytes(100, 64, 256, 0) == off_meta + 100 * 8
    assert lib.mfa_decode_workspace_bytes(1025, 64, 256, 0) == 0
    desc = _lib.KVCacheDesc(k=P, v=P, num_blocks=1 << 20, max_blocks_per_seq=64, head_dim=256,
                            dtype=BF16)
    big = lib.mfa_decode_workspace_bytes(1024, 64, 256, 0)
    assert lib.mfa_decode_attn(P, BF16, 1025, 64, ctypes.byref(desc), P, 100, 0.0625, 0, 0, P,
                               big, P, BF16, None) == SHAPE
    # the balanced partition needs the matrix-core kernel (64 heads of 256)
    d64 = _lib.KVCacheDesc(k=P, v=P, num_blocks=1 << 20, max_blocks_per_seq=64, head_dim=64,
                           dtype=F32)
    assert lib.mfa_decode_attn(P, F32, 4, 4, ctypes.byref(d64), P, 100, 0.125, 0, 0, P,
                               1 << 30, P, F32, None) == UNSUP
    assert lib.mfa_combine(P, 16, 1025, 64, 256, 0, P, BF16, None) == SHAPE


def _c_layout(struct, fields):
    """sizeof and offsetof of a struct of mfa.h, from a C program built by gcc."""
    import shutil
    import subprocess
    import tempfile
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    body = "".join(f'  printf("%zu\\n", offsetof({struct}, {f}));\n' for f in fields)
    src = ("#include <stdio.h>\n#include <stddef.h>\n#include \"mfa.h\"\nint main(void) {\n"
           f'  printf("%zu\\n", sizeof({struct}));\n{body}  return 0;\n}}\n')
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "t.c"), os.path.join(d, "t")
        with open(c, "w") as f:
            f.write(src)
        subprocess.check_call(["gcc", "-I", os.path.dirname(HEADER), "-o", exe, c])
        return [int(v) for v in subprocess.check_output([exe]).split()]


@pytest.mark.parametrize("struct,mirror", [("mfa_kv_cache", _lib.KVCacheDesc),
                                            ("mfa_step_args", _lib.StepArgs)])
def test_struct_layout_matches_header(struct, mirror):
    names = [f[0] for f in mirror._fields_]
    got = _c_layout(struct, names)
    assert got[0] == ctypes.sizeof(mirror)
    for n, off in zip(names, got[1:]):
        assert getattr(mirror, n).offset == off, n


def test_decode_step_validation(lib):
    assert lib.mfa_decode_step(None, None) == NULL
    c = _cache()
    a = _lib.StepArgs()
    a.B, a.H, a.d, a.dtype = 4, 64, 256, BF16
    a.q, a.k_new, a.v_new, a.kv_in_dtype, a.pos = P, P, P, BF16, P
    a.cache = ctypes.pointer(c)
    a.seq_lens, a.max_seq_len, a.sm_scale = P, 512, 0.0625
    a.num_splits, a.chunk_tokens = 1, 512
    a.out, a.out_dtype = P, BF16
    ok = lambda: lib.mfa_decode_step(ctypes.byref(a), None)
    a.k_new = None
    assert ok() == NULL                                          # append arguments checked
    a.k_new = P
    a.sm_scale = -1.0
    assert ok() == SHAPE                                         # attention arguments checked
    a.sm_scale = 0.0625
    a.d = 128
    assert ok() == SHAPE                                         # d must be the cache's
    a.d = 256
    a.x, a.w_qdown, a.w_qup, a.q_norm_w = P, P, P, P
    a.hidden, a.q_rank = 7000, 2048
    assert ok() == SHAPE                                         # query-path arguments checked
    a.hidden = 7168
    a.qproj_workspace, a.qproj_workspace_bytes = None, 0
    assert ok() == WS
    # K/V projection: needs x, an aligned weight, kv_in_dtype == dtype; k_new, v_new optional
    a.qproj_workspace, a.qproj_workspace_bytes = P, 1 << 30
    a.w_kv = PM
    assert ok() == ALIGN
    a.w_kv = P
    a.kv_in_dtype = F32
    assert ok() == DTYPE
    a.kv_in_dtype = BF16
    a.k_new = a.v_new = None
    a.pos = None
    assert ok() == NULL                                          # pos still required
    a.pos = P
    a.x = None
    assert ok() == NULL                                          # projection without x


def test_plan_from_lengths(lib):
    """mfa_decode_plan_lens: uniform lengths keep the split plan; mixed ones
    whose longest split walks clearly more than the chip's even share get the
    balanced partition; shapes without the matrix-core kernel never do."""
    import numpy as np
    ns, ch = ctypes.c_int(), ctypes.c_int()

    def plan(lens, H=64, d=256, dt=BF16):
        a = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
        rc = lib.mfa_decode_plan_lens(len(a), H, d, a.ctypes.data_as(ctypes.c_void_p), dt,
                                      ctypes.byref(ns), ctypes.byref(ch))
        assert rc == OK
        return ns.value, ch.value
    assert plan([4096] * 32) == (8, 512)                  # the 4K workload: as mfa_decode_plan
    assert plan([32768] * 16, dt=FP8)[0] == 16
    rng = np.random.default_rng(2)
    mixed = rng.integers(1025, 8194, size=128)
    assert plan(mixed) == (0, 0)                          # mixed lengths: balanced
    assert plan(mixed, H=4, d=64, dt=F32)[0] >= 1         # VALU shapes: split plan only
    assert plan([0] * 8)[0] >= 1                          # nothing to walk: split plan
    big = np.full(1025, 3000)
    assert plan(big)[0] >= 1                              # more rows than the balanced walk takes
    assert lib.mfa_decode_plan_lens(4, 64, 256, None, BF16, ctypes.byref(ns),
                                    ctypes.byref(ch)) == NULL
