"""The C ABI library loads, exports every function include/attn_fp4.h declares,
and rejects bad arguments on the host (no GPU work is launched by these calls)."""

import ctypes
import os
import re

import pytest

import precision_attention_forward_amd as paf
from precision_attention_forward_amd import _binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "attn_fp4.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(paf.LIB_PATH):
        pytest.fail("libattnfp4.so is not built (run __graft_entry__.build())")
    return paf.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert "attn_fwd_directp" in names and "attn_quant_nvfp4" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in attn_fp4.h but not exported"
    assert set(names) == set(B.EXPORTS), "binding and header disagree"


def test_product_library_has_no_phase_trace(lib):
    # The forward's phase-trace stamps exist only in the diagnostic build
    # (libattnfp4_trace.so); the product library compiles them out.
    assert not hasattr(lib, "attn_fwd_phase_trace_read")
    from precision_attention_forward_amd.build import TRACE_LIB
    if os.path.exists(TRACE_LIB):
        assert hasattr(ctypes.CDLL(TRACE_LIB), "attn_fwd_phase_trace_read")


def test_struct_layout_matches_header():
    # attn_fwd_args as laid out by the compiler for the C declaration
    assert ctypes.sizeof(B.FwdArgs) == 4 * 6 + 8 * 2 + 8 * 2 + 4 + 4 + 24 * 2 + 32 + 8 + 4 + 4 + 8 + 8 + 8 + 8 + 8 + 4 + 4 + 8 + 8


def _c_offsets(struct, fields):
    """sizeof and offsetof of a header struct, from a C program compiled with gcc."""
    import shutil
    import subprocess
    import tempfile
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    lines = [f'printf("%zu\\n", sizeof({struct}));']
    lines += [f'printf("%zu\\n", offsetof({struct}, {f}));' for f in fields]
    src = "#include <stddef.h>\n#include <stdio.h>\n#include \"attn_fp4.h\"\nint main(void) {\n" + "\n".join(lines) + "\nreturn 0; }\n"
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "t.c"), os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", inc, c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()
    return [int(x) for x in out]


@pytest.mark.parametrize("cls,cname", [(B.FwdArgs, "attn_fwd_args"), (B.BwdArgs, "attn_bwd_args"),
                                       (B.DecodeArgs, "attn_decode_args")])
def test_ctypes_struct_matches_c_layout(cls, cname):
    fields = [f for f, _ in cls._fields_]
    got = _c_offsets(cname, fields)
    assert got[0] == ctypes.sizeof(cls)
    for f, off in zip(fields, got[1:]):
        assert getattr(cls, f).offset == off, f


def test_status_strings_and_constants(lib):
    assert lib.attn_status_str(0) == b"ok"
    assert lib.attn_status_str(1) == b"invalid argument"
    assert lib.attn_status_str(3) == b"workspace missing or too small"
    assert lib.attn_quant_ws_bytes() >= 2048
    assert lib.attn_version().startswith(b"attn_fp4")


def test_v_cols(lib):
    assert lib.attn_v_cols(2, 300, 0, 0) == 2 * 384
    assert lib.attn_v_cols(1, 32760, 0, 0) == 32768
    assert lib.attn_v_cols(3, 100, 1000, 1) == 128 * (8 + 3)
    # every varlen sequence fits: start 128*(cu//128 + s), length roundup(len, 128)
    import numpy as np
    rng = np.random.default_rng(0)
    for _ in range(200):
        lens = rng.integers(0, 700, size=rng.integers(1, 9))
        cu = np.concatenate([[0], np.cumsum(lens)])
        cols = lib.attn_v_cols(len(lens), int(lens.max()), int(cu[-1]), 1)
        ends = [128 * (cu[s] // 128 + s) + (lens[s] + 127) // 128 * 128 for s in range(len(lens))]
        starts = [128 * (cu[s] // 128 + s) for s in range(len(lens))]
        assert max(ends) <= cols
        assert all(ends[s] <= starts[s + 1] for s in range(len(lens) - 1))


def test_quant_rejects_bad_arguments_without_launching(lib):
    ws = ctypes.create_string_buffer(4096)
    ts = ctypes.c_float()
    # D not a multiple of 16
    assert lib.attn_quant_nvfp4(None, 4, 24, None, None, ctypes.byref(ts), ws, 4096, None) == 1
    # missing input pointer for a non-empty tensor
    assert lib.attn_quant_nvfp4(None, 4, 64, None, None, ctypes.byref(ts), ws, 4096, None) == 1
    # workspace too small
    fake = ctypes.c_void_p(1 << 20)
    assert lib.attn_quant_nvfp4(fake, 4, 64, fake, fake, ctypes.byref(ts), ws, 16, None) == 3
    # V: unsupported head dim, bad format
    assert lib.attn_quant_v(fake, 1, 8, 1, 96, None, 0, 0, fake, None, ctypes.byref(ts), ws, 4096, None) == 1
    assert lib.attn_quant_v(fake, 1, 8, 1, 64, None, 0, 7, fake, None, ctypes.byref(ts), ws, 4096, None) == 1
    # decode V cache: capacity in whole 128-key tiles, head dim, format, MXFP4 scales, workspace
    qc = lib.attn_quant_v_cache
    assert qc(fake, 1, 200, 1, 64, 0, fake, None, ctypes.byref(ts), ws, 4096, None) == 1
    assert qc(fake, 1, 128, 1, 96, 0, fake, None, ctypes.byref(ts), ws, 4096, None) == 1
    assert qc(fake, 1, 128, 1, 64, 7, fake, None, ctypes.byref(ts), ws, 4096, None) == 1
    assert qc(fake, 1, 128, 1, 64, 0, fake, None, None, ws, 4096, None) == 1             # FP8 needs its scale slot
    assert qc(fake, 1, 128, 1, 64, 1, fake, None, None, ws, 4096, None) == 1             # MXFP4 needs scales
    assert qc(None, 1, 128, 1, 64, 0, fake, None, ctypes.byref(ts), ws, 4096, None) == 1
    assert qc(fake, 1, 128, 1, 64, 0, fake, None, ctypes.byref(ts), ws, 16, None) == 3


def _args(**kw):
    a = B.FwdArgs()
    a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.D = 1, 4, 2, 256, 256, 128
    a.softmax_scale = 0.125
    p = 1 << 24
    a.q = B._NvTensor(p, p, p)
    a.k = B._NvTensor(p, p, p)
    a.v = B._VTensor(0, p, p, p)
    a.o = p
    a.o_dtype = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_fwd_validation(lib):
    a = _args()
    need = lib.attn_fwd_ws_bytes(ctypes.byref(a))
    # K fp16 operand tiles (2 KV heads x 256 keys x 128), 2 bytes each; Q is decoded in the kernel
    assert need == 2 * 128 * (2 * 256) + 256
    a.ws, a.ws_bytes = 1 << 24, need
    assert lib.attn_fwd_directp(ctypes.byref(_args(D=96, ws=1 << 24, ws_bytes=need)), None) == 1
    assert lib.attn_fwd_directp(ctypes.byref(_args(Hkv=3, ws=1 << 24, ws_bytes=need)), None) == 1
    assert lib.attn_fwd_directp(ctypes.byref(_args(causal=1, ws=1 << 24, ws_bytes=need)), None) == 2
    assert lib.attn_fwd_fp8pv(ctypes.byref(_args(causal=1, Nk=128, ws=1 << 24, ws_bytes=need)), None) == 1
    assert lib.attn_fwd_fp8pv(ctypes.byref(_args(v=B._VTensor(1, 1 << 24, 1 << 24, 1 << 24), ws=1 << 24,
                                                 ws_bytes=need)), None) == 2
    assert lib.attn_fwd_directp(ctypes.byref(_args(ws=1 << 24, ws_bytes=need - 1)), None) == 3
    assert lib.attn_fwd_directp(ctypes.byref(_args(softmax_scale=0.0, ws=1 << 24, ws_bytes=need)), None) == 1
    assert lib.attn_fwd_directp(ctypes.byref(_args(o=None, ws=1 << 24, ws_bytes=need)), None) == 1
    assert lib.attn_fwd_directp(None, None) == 1
    # the exp-free entry points share the checks of the exact ones
    assert lib.attn_fwd_directp_efq(ctypes.byref(_args(causal=1, ws=1 << 24, ws_bytes=need)), None) == 2
    assert lib.attn_fwd_directp_efq(ctypes.byref(_args(D=96, ws=1 << 24, ws_bytes=need)), None) == 1
    assert lib.attn_fwd_directp_efq(ctypes.byref(_args(ws=1 << 24, ws_bytes=need - 1)), None) == 3
    assert lib.attn_fwd_fp8pv_cast(ctypes.byref(_args(v=B._VTensor(1, 1 << 24, 1 << 24, 1 << 24), ws=1 << 24,
                                                      ws_bytes=need)), None) == 2
    assert lib.attn_fwd_fp8pv_cast(ctypes.byref(_args(causal=1, Nk=128, ws=1 << 24, ws_bytes=need)), None) == 1
    assert lib.attn_fwd_fp8pv_cast(None, None) == 1
    # backward: shapes, V format, workspace
    bw = B.BwdArgs()
    bw.B, bw.Hq, bw.Hkv, bw.N, bw.D, bw.softmax_scale, bw.causal = 2, 4, 2, 256, 128, 0.1, 1
    need_b = lib.attn_bwd_ws_bytes(ctypes.byref(bw))
    nq_b, nk_b = 2 * 4 * 256 * 128, 2 * 2 * 256 * 128   # elements of Q / dO and of K / V
    # bf16 Q^ and K^, E4M3 V, E5M2 dO^ row-major and transposed
    assert need_b > 2 * nq_b + 2 * nk_b + nk_b + nq_b
    bw.D = 96
    assert lib.attn_bwd_ws_bytes(ctypes.byref(bw)) == 0 and lib.attn_bwd_fp8(ctypes.byref(bw), None) == 1
    bw.D, bw.Hkv = 128, 3
    assert lib.attn_bwd_fp8(ctypes.byref(bw), None) == 1
    bw.Hkv = 2
    bw.v = B._VTensor(1, 1 << 24, 1 << 24, 1 << 24)
    assert lib.attn_bwd_fp8(ctypes.byref(bw), None) == 2
    bw.v = B._VTensor(0, 1 << 24, None, 1 << 24)
    assert lib.attn_bwd_fp8(ctypes.byref(bw), None) == 1          # null operand pointers
    assert lib.attn_bwd_fp8(None, None) == 1
    # varlen needs both cu_seqlens
    assert lib.attn_fwd_directp(ctypes.byref(_args(cu_seqlens_q=1 << 24, ws=1 << 24, ws_bytes=need)), None) == 1
    # bf16 baseline argument checks
    assert lib.attn_fwd_bf16(None, None, None, None, None, 1, 4, 3, 16, 16, 128, 0.1, 0, None) == 1
    assert lib.attn_fwd_bf16(None, None, None, None, None, 1, 4, 4, 16, 16, 80, 0.1, 0, None) == 1


def test_fwd_offset_limits(lib):
    # The forward reads one KV head's V^T rows with 32-bit per-lane byte
    # offsets d * cols: FP8 V needs D * cols < 2^32, MXFP4 V D * cols / 2 <
    # 2^32.  Past the limit the call returns UNSUPPORTED before any launch (the
    # fake pointers are never touched); just below it, validation goes on to
    # the next check (here: no workspace).
    D = 128
    fp8_over = (1 << 32) // D                  # cols = 2^25: D * cols = 2^32
    fp8_under = fp8_over - 128
    big = dict(B=1, Hq=1, Hkv=1, Nq=256)
    v_fp8, v_mx = B._VTensor(0, 1 << 24, None, 1 << 24), B._VTensor(1, 1 << 24, 1 << 24, None)
    for fn in (lib.attn_fwd_directp, lib.attn_fwd_fp8pv, lib.attn_fwd_directp_efq, lib.attn_fwd_fp8pv_mxqk):
        assert fn(ctypes.byref(_args(Nk=fp8_over, v=v_fp8, **big)), None) == 2
        assert fn(ctypes.byref(_args(Nk=fp8_under, v=v_fp8, **big)), None) == 3
    # MXFP4 V: half a byte per key
    assert lib.attn_fwd_directp(ctypes.byref(_args(Nk=2 * fp8_over, v=v_mx, **big)), None) == 2
    assert lib.attn_fwd_directp(ctypes.byref(_args(Nk=2 * fp8_over - 128, v=v_mx, **big)), None) == 3
    # one packed sequence past the limit (FP8 V): cols = 128 * (ceil(total_k / 128) + B)
    pk = _args(Nk=fp8_over, v=v_fp8, cu_seqlens_q=1 << 24, cu_seqlens_k=1 << 24, total_q=256, total_k=fp8_over,
               **big)
    assert lib.attn_fwd_fp8pv(ctypes.byref(pk), None) == 2
    # BF16 baseline: the rows of a 128-key tile are addressed with 32-bit byte
    # offsets (128 * Hkv * D * 2 < 2^31)
    fake = ctypes.c_void_p(1 << 24)
    assert lib.attn_fwd_bf16(fake, fake, fake, fake, None, 1, 1 << 16, 1 << 16, 16, 16, 128, 0.1, 0, None) == 2


def _dec_args(**kw):
    a = B.DecodeArgs()
    a.B, a.Hq, a.Hkv, a.nq, a.Nk, a.D = 2, 8, 2, 1, 1024, 128
    a.softmax_scale = 0.125
    p = 1 << 24
    a.q = B._NvTensor(p, p, p)
    a.k = B._NvTensor(p, p, p)
    a.v = B._VTensor(0, p, p, p)
    a.o = p
    a.o_dtype = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_decode_validation(lib):
    # every case below fails on the host, so the fake pointers are never used
    d = lambda **kw: lib.attn_decode_directp(ctypes.byref(_dec_args(**kw)), None)
    assert d(D=96) == 1
    assert d(Hkv=3) == 1
    assert d(nq=0) == 1
    assert d(Nk=-1) == 1
    assert d(Nk=1000) == 1                                         # capacity in whole 128-key tiles
    assert d(softmax_scale=0.0) == 1
    assert d(softmax_scale=float("nan")) == 1
    assert d(o=None) == 1
    assert d(o_dtype=5) == 1
    assert d(v=B._VTensor(7, 1 << 24, 1 << 24, 1 << 24)) == 1
    assert d(v=B._VTensor(1, 1 << 24, None, 1 << 24)) == 1          # MXFP4 V needs its scales
    assert d(k=B._NvTensor(1 << 24, None, 1 << 24)) == 1
    assert d(q=B._NvTensor((1 << 24) + 4, 1 << 24, 1 << 24)) == 1  # misaligned codes
    assert d(seqlens_k=(1 << 24) + 2) == 1
    assert d(dbg_p_codes=1 << 24, dbg_b=2) == 1
    assert d(dbg_p_codes=1 << 24) == 1                             # Direct-P dump needs the scale buffer
    # the grid (one workgroup per sequence, KV head and 16 query rows) stays below 2^31
    assert d(B=1 << 30) == 2
    # FP8-P/V takes FP8 V only
    assert lib.attn_decode_fp8pv(ctypes.byref(_dec_args(v=B._VTensor(1, 1 << 24, 1 << 24, 1 << 24))), None) == 2
    assert lib.attn_decode_directp(None, None) == 1 and lib.attn_decode_fp8pv(None, None) == 1


def test_mx_qk_entry_points_reject_bad_arguments(lib):
    fake = ctypes.c_void_p(1 << 20)
    # D must be a multiple of 32; non-empty tensors need their pointers; codes 16-byte aligned
    assert lib.attn_quant_mxfp4(fake, 4, 48, fake, fake, None) == 1
    assert lib.attn_quant_mxfp4(None, 4, 64, fake, fake, None) == 1
    assert lib.attn_quant_mxfp4(fake, 4, 64, ctypes.c_void_p((1 << 20) + 8), fake, None) == 1
    assert lib.attn_quant_mxfp4(None, 0, 64, None, None, None) == 0      # empty: nothing to do
    a = _args()
    need = lib.attn_fwd_ws_bytes(ctypes.byref(a))
    # tensor scales are not used: NULL is accepted past validation only with everything else valid,
    # so check the rejections that come first
    noscale = dict(q=B._NvTensor(1 << 24, 1 << 24, None), k=B._NvTensor(1 << 24, 1 << 24, None))
    assert lib.attn_fwd_directp_mxqk(ctypes.byref(_args(causal=1, ws=1 << 24, ws_bytes=need, **noscale)), None) == 2
    assert lib.attn_fwd_directp_mxqk(ctypes.byref(_args(D=96, ws=1 << 24, ws_bytes=need, **noscale)), None) == 1
    assert lib.attn_fwd_directp_mxqk(ctypes.byref(_args(ws=1 << 24, ws_bytes=need - 1, **noscale)), None) == 3
    misaligned = dict(q=B._NvTensor((1 << 24) + 8, 1 << 24, None), k=B._NvTensor(1 << 24, 1 << 24, None))
    assert lib.attn_fwd_directp_mxqk(ctypes.byref(_args(ws=1 << 24, ws_bytes=need, **misaligned)), None) == 1
    assert lib.attn_fwd_directp_mxqk(None, None) == 1
    # the FP8-P/V variant takes causal inputs but needs FP8 V
    assert lib.attn_fwd_fp8pv_mxqk(ctypes.byref(_args(causal=1, Nk=128, ws=1 << 24, ws_bytes=need, **noscale)),
                                   None) == 1
    assert lib.attn_fwd_fp8pv_mxqk(ctypes.byref(_args(v=B._VTensor(1, 1 << 24, 1 << 24, 1 << 24), ws=1 << 24,
                                                      ws_bytes=need, **noscale)), None) == 2
    assert lib.attn_fwd_fp8pv_mxqk(None, None) == 1
    # the exp-free MX entry point is Direct-P only: noncausal
    assert lib.attn_fwd_directp_efq_mxqk(ctypes.byref(_args(causal=1, ws=1 << 24, ws_bytes=need, **noscale)), None) == 2
    assert lib.attn_fwd_directp_efq_mxqk(None, None) == 1
    assert lib.attn_fwd_fp8pv_cast_mxqk(ctypes.byref(_args(v=B._VTensor(1, 1 << 24, 1 << 24, 1 << 24), ws=1 << 24,
                                                           ws_bytes=need, **noscale)), None) == 2
    assert lib.attn_fwd_fp8pv_cast_mxqk(None, None) == 1


def test_noalloc_validation(lib):
    # The forward without a caller workspace keeps the K operand tiles in a
    # fixed device array of ATTN_NOALLOC_SCRATCH_BYTES: past it the call
    # returns ATTN_ERR_WORKSPACE; its other checks are attn_fwd_directp's.  All
    # of these fail on the host before the array or the GPU is touched.
    cap = (64 << 20) + 4096
    fn = lambda **kw: lib.attn_fwd_directp_noalloc(ctypes.byref(_args(**kw)), None)
    over = _args(B=4, Hq=32, Hkv=8, Nq=8192, Nk=8192 + 128)
    assert lib.attn_fwd_ws_bytes(ctypes.byref(over)) > cap
    assert lib.attn_fwd_directp_noalloc(ctypes.byref(over), None) == 3
    assert lib.attn_fwd_ws_bytes(ctypes.byref(_args(B=4, Hq=32, Hkv=8, Nq=8192, Nk=8192))) <= cap
    assert fn(causal=1) == 2
    assert fn(D=96) == 1
    assert fn(o=None) == 1
    assert lib.attn_fwd_directp_noalloc(None, None) == 1


def test_probe_entry_points_reject_bad_arguments(lib):
    # the issue-rate diagnostics: kinds are counted by the library; bad kinds
    # and null or misaligned pointers are rejected before any launch
    assert lib.attn_probe_kinds() == 34
    units = ctypes.c_longlong(-1)
    grid = ctypes.c_int(-1)
    for kind in (-1, 34, 1000):
        assert lib.attn_probe_issue_rates(kind, 1 << 20, ctypes.byref(units), ctypes.byref(grid), None) == 1
    assert lib.attn_probe_issue_rates(0, None, ctypes.byref(units), ctypes.byref(grid), None) == 1
    assert lib.attn_probe_issue_rates(0, (1 << 20) + 4, ctypes.byref(units), ctypes.byref(grid), None) == 1
    assert lib.attn_probe_issue_rates(0, 1 << 20, None, ctypes.byref(grid), None) == 1
    assert lib.attn_probe_issue_rates(0, 1 << 20, ctypes.byref(units), None, None) == 1
    assert units.value == -1 and grid.value == -1
