"""ctypes binding of libattnfp4.so (the C ABI in include/attn_fp4.h).

Argument marshalling only: torch provides device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if the shared library is missing or fails to load,
every entry point raises.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattnfp4.so")

ATTN_OK = 0
V_FP8 = 0
V_MXFP4 = 1
OUT_BF16 = 0
OUT_F32 = 1

_lib = None


class AttnError(RuntimeError):
    pass


class _NvTensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("tensor_scale", ctypes.c_void_p)]


class _VTensor(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p)]


class FwdArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Nq", ctypes.c_int32), ("Nk", ctypes.c_int32), ("D", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
        ("total_q", ctypes.c_int64), ("total_k", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32),
        ("q", _NvTensor), ("k", _NvTensor), ("v", _VTensor),
        ("o", ctypes.c_void_p), ("o_dtype", ctypes.c_int32), ("lse", ctypes.c_void_p),
        ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
        ("dbg_p_codes", ctypes.c_void_p), ("dbg_p_scales", ctypes.c_void_p),
        ("dbg_b", ctypes.c_int32), ("dbg_h", ctypes.c_int32),
        ("prof_event_begin", ctypes.c_void_p), ("prof_event_end", ctypes.c_void_p),
    ]


class BwdArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("N", ctypes.c_int32), ("D", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32),
        ("q", _NvTensor), ("k", _NvTensor), ("v", _VTensor),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("dout", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
        ("dbg_p_codes", ctypes.c_void_p), ("dbg_p_exps", ctypes.c_void_p),
        ("dbg_dsk_codes", ctypes.c_void_p), ("dbg_dsk_exps", ctypes.c_void_p),
        ("dbg_dsq_codes", ctypes.c_void_p), ("dbg_dsq_exps", ctypes.c_void_p),
        ("dbg_b", ctypes.c_int32), ("dbg_h", ctypes.c_int32),
        ("prof_event_begin", ctypes.c_void_p), ("prof_event_end", ctypes.c_void_p),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("nq", ctypes.c_int32), ("Nk", ctypes.c_int32), ("D", ctypes.c_int32),
        ("seqlens_k", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32),
        ("q", _NvTensor), ("k", _NvTensor), ("v", _VTensor),
        ("o", ctypes.c_void_p), ("o_dtype", ctypes.c_int32), ("lse", ctypes.c_void_p),
        ("dbg_p_codes", ctypes.c_void_p), ("dbg_p_scales", ctypes.c_void_p),
        ("dbg_b", ctypes.c_int32), ("dbg_h", ctypes.c_int32),
        ("prof_event_begin", ctypes.c_void_p), ("prof_event_end", ctypes.c_void_p),
    ]


EXPORTS = {
    "attn_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_last_hip_error": (ctypes.c_int, []),
    "attn_version": (ctypes.c_char_p, []),
    "attn_quant_ws_bytes": (ctypes.c_size_t, []),
    "attn_quant_nvfp4": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]),
    "attn_quant_nvfp4_46": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]),
    "attn_quant_mxfp4": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]),
    "attn_quant_mxfp4_had": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]),
    "attn_v_cols": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]),
    "attn_quant_v": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "attn_quant_v_cache": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "attn_fwd_ws_bytes": (ctypes.c_size_t, [ctypes.POINTER(FwdArgs)]),
    "attn_fwd_directp": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "attn_fwd_directp_noalloc": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "attn_fwd_fp8pv": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "attn_fwd_directp_efq": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "attn_fwd_fp8pv_cast": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "attn_fwd_directp_mxqk": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "attn_fwd_fp8pv_mxqk": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "attn_fwd_directp_efq_mxqk": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "attn_fwd_fp8pv_cast_mxqk": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "attn_decode_directp": (ctypes.c_int, [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]),
    "attn_decode_fp8pv": (ctypes.c_int, [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]),
    "attn_bwd_ws_bytes": (ctypes.c_size_t, [ctypes.POINTER(BwdArgs)]),
    "attn_bwd_fp8": (ctypes.c_int, [ctypes.POINTER(BwdArgs), ctypes.c_void_p]),
    "attn_fwd_bf16": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                     ctypes.c_void_p]),
    "attn_probe_kinds": (ctypes.c_int, []),
    "attn_probe_issue_rates": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_longlong),
                                              ctypes.POINTER(ctypes.c_int), ctypes.c_void_p]),
}


def load_library(path=None):
    """Load libattnfp4.so (raises if it is missing) and declare signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise AttnError(f"{path} is missing: build it with `python -m precision_attention_forward_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != ATTN_OK:
        lib = load_library()
        msg = lib.attn_status_str(status).decode()
        if status == 4:
            msg += f" (hipError {lib.attn_last_hip_error()})"
        raise AttnError(f"attn library returned {status}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise AttnError("tensors must be contiguous and on the GPU")


def quant_nvfp4(x, four_six=False):
    """NVFP4-quantize a bf16 tensor along its last axis (D).  Returns
    (codes uint8 [..., D/2], scales uint8 [..., D/16], tensor_scale float32 [1]).
    ``four_six`` selects the Four Over Six adaptive block scale
    (attn_quant_nvfp4_46); the output format is the same."""
    lib = load_library()
    _need_cuda(x)
    if x.dtype != torch.bfloat16:
        raise AttnError("quant_nvfp4 expects bfloat16")
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    codes = torch.empty(x.shape[:-1] + (D // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (D // 16,), dtype=torch.uint8, device=x.device)
    ts = torch.empty(1, dtype=torch.float32, device=x.device)
    ws = torch.empty(lib.attn_quant_ws_bytes(), dtype=torch.uint8, device=x.device)
    fn = lib.attn_quant_nvfp4_46 if four_six else lib.attn_quant_nvfp4
    _check(fn(_ptr(x), rows, D, _ptr(codes), _ptr(scales), _ptr(ts), _ptr(ws), ws.numel(), _stream()))
    return codes, scales, ts


def quant_mxfp4(x, hadamard=False):
    """MXFP4-quantize a bf16 tensor along its last axis (D, a multiple of 32),
    the MX-native Q/K format of fwd_directp_mxqk.  Returns (codes uint8
    [..., D/2], E8M0 scales uint8 [..., D/32], None) -- the None stands where
    the NVFP4 tuples carry their tensor scale.  ``hadamard`` rotates each
    32-element block by the 32-point Hadamard matrix first
    (attn_quant_mxfp4_had); Q and K rotated alike need softmax_scale / 32."""
    lib = load_library()
    _need_cuda(x)
    if x.dtype != torch.bfloat16:
        raise AttnError("quant_mxfp4 expects bfloat16")
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    codes = torch.empty(x.shape[:-1] + (D // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (D // 32,), dtype=torch.uint8, device=x.device)
    fn = lib.attn_quant_mxfp4_had if hadamard else lib.attn_quant_mxfp4
    _check(fn(_ptr(x), rows, D, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales, None


def v_cols(B, Nk, total_k=0, varlen=False):
    return load_library().attn_v_cols(B, Nk, total_k, 1 if varlen else 0)


def quant_v(v, fmt, cu_seqlens=None, max_seqlen=None):
    """Quantize V (bf16 [B, Nk, Hkv, D] or packed [T, Hkv, D] with device
    cu_seqlens) to FP8 E4M3 (fmt=V_FP8) or MXFP4 (fmt=V_MXFP4), transposed to
    [Hkv, D, cols] with keys contiguous.  Returns (codes, scales|None, tensor_scale|None, cols)."""
    lib = load_library()
    _need_cuda(v, cu_seqlens)
    if v.dtype != torch.bfloat16:
        raise AttnError("quant_v expects bfloat16")
    if cu_seqlens is None:
        B, Nk, Hkv, D = v.shape
        total = B * Nk
    else:
        total, Hkv, D = v.shape
        B = cu_seqlens.numel() - 1
        Nk = int(max_seqlen)
    cols = lib.attn_v_cols(B, Nk, total, 0 if cu_seqlens is None else 1)
    # dense: the library writes every column (zeros past Nk in the last tile);
    # packed: the columns between sequences are never written, so they are zeroed
    alloc = torch.empty if cu_seqlens is None else torch.zeros
    if fmt == V_FP8:
        codes = alloc((Hkv, D, cols), dtype=torch.uint8, device=v.device)
        scales = None
        ts = torch.empty(1, dtype=torch.float32, device=v.device)
    else:
        codes = alloc((Hkv, D, cols // 2), dtype=torch.uint8, device=v.device)
        scales = alloc((Hkv, D, cols // 32), dtype=torch.uint8, device=v.device)
        ts = None
    ws = torch.empty(lib.attn_quant_ws_bytes(), dtype=torch.uint8, device=v.device)
    _check(lib.attn_quant_v(_ptr(v), B, Nk, Hkv, D, _ptr(cu_seqlens), total, fmt, _ptr(codes), _ptr(scales),
                            _ptr(ts), _ptr(ws), ws.numel(), _stream()))
    return codes, scales, ts, cols


def quant_v_cache(v, fmt):
    """Quantize a decode step's V cache (bf16 [B, Nk, Hkv, D], Nk a multiple
    of 128) to FP8 E4M3 or MXFP4 with the values of quant_v, stored as the
    decode kernels read it: one block of D key-contiguous rows per (sequence,
    KV head, 128-key tile).  Returns (codes [B, Hkv, Nk/128, D, 128 or 64],
    scales [B, Hkv, Nk/128, D, 4]|None, tensor_scale|None)."""
    lib = load_library()
    _need_cuda(v)
    if v.dtype != torch.bfloat16:
        raise AttnError("quant_v_cache expects bfloat16")
    B, Nk, Hkv, D = v.shape
    nt = Nk // 128
    if fmt == V_FP8:
        codes = torch.empty((B, Hkv, nt, D, 128), dtype=torch.uint8, device=v.device)
        scales = None
        ts = torch.empty(1, dtype=torch.float32, device=v.device)
    else:
        codes = torch.empty((B, Hkv, nt, D, 64), dtype=torch.uint8, device=v.device)
        scales = torch.empty((B, Hkv, nt, D, 4), dtype=torch.uint8, device=v.device)
        ts = None
    ws = torch.empty(lib.attn_quant_ws_bytes(), dtype=torch.uint8, device=v.device)
    _check(lib.attn_quant_v_cache(_ptr(v), B, Nk, Hkv, D, fmt, _ptr(codes), _ptr(scales), _ptr(ts), _ptr(ws),
                                  ws.numel(), _stream()))
    return codes, scales, ts


class Workspace:
    """A reusable device byte buffer that grows on demand."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes, device):
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(device):
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


_default_ws = Workspace()


def make_fwd_args(q, k, v, *, B, Hq, Hkv, Nq, Nk, D, softmax_scale, causal=False, cu_seqlens_q=None,
                  cu_seqlens_k=None, total_q=0, total_k=0, o=None, o_dtype=OUT_F32, lse=None, ws=None,
                  dbg_codes=None, dbg_scales=None, dbg_b=0, dbg_h=0):
    """q/k: (codes, scales, tensor_scale); v: (format, codes, scales|None, tensor_scale|None)."""
    a = FwdArgs()
    a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.D = B, Hq, Hkv, Nq, Nk, D
    a.cu_seqlens_q = None if cu_seqlens_q is None else cu_seqlens_q.data_ptr()
    a.cu_seqlens_k = None if cu_seqlens_k is None else cu_seqlens_k.data_ptr()
    a.total_q, a.total_k = total_q, total_k
    a.softmax_scale = softmax_scale
    a.causal = 1 if causal else 0
    a.q = _NvTensor(q[0].data_ptr(), q[1].data_ptr(), None if q[2] is None else q[2].data_ptr())
    a.k = _NvTensor(k[0].data_ptr(), k[1].data_ptr(), None if k[2] is None else k[2].data_ptr())
    a.v = _VTensor(v[0], v[1].data_ptr(), None if v[2] is None else v[2].data_ptr(),
                   None if v[3] is None else v[3].data_ptr())
    a.o = None if o is None else o.data_ptr()
    a.o_dtype = o_dtype
    a.lse = None if lse is None else lse.data_ptr()
    a.ws = None if ws is None else ws.data_ptr()
    a.ws_bytes = 0 if ws is None else ws.numel()
    a.dbg_p_codes = None if dbg_codes is None else dbg_codes.data_ptr()
    a.dbg_p_scales = None if dbg_scales is None else dbg_scales.data_ptr()
    a.dbg_b, a.dbg_h = dbg_b, dbg_h
    return a


def _fwd_lowp(entry, q, k, v, *, Hq, Hkv, D, softmax_scale, causal=False, B=None, Nq=None, Nk=None,
              cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
              out_dtype=torch.float32, want_lse=True, workspace=None, debug=None, events=None, out=None):
    """Shared driver of the low-precision forward entry points.  Returns (O, LSE, dbg)."""
    lib = load_library()
    dev = q[0].device
    varlen = cu_seqlens_q is not None
    if varlen:
        B = cu_seqlens_q.numel() - 1
        total_q = q[0].shape[0]
        total_k = k[0].shape[0]
        Nq, Nk = int(max_seqlen_q), int(max_seqlen_k)
        oshape = (total_q, Hq, D)
        lshape = (Hq, total_q)
    else:
        total_q, total_k = B * Nq, B * Nk
        oshape = (B, Nq, Hq, D)
        lshape = (B, Hq, Nq)
    if out is not None:
        o, lse = out
    else:
        o = torch.empty(oshape, dtype=out_dtype, device=dev)
        lse = torch.empty(lshape, dtype=torch.float32, device=dev) if want_lse else None
    dbg_codes = dbg_scales = None
    dbg_b = dbg_h = 0
    if debug is not None:
        dbg_b, dbg_h = debug
        nq_dbg = Nq
        nk_pad = (Nk + 127) // 128 * 128
        if entry in ("attn_fwd_directp", "attn_fwd_directp_noalloc", "attn_fwd_directp_efq", "attn_fwd_directp_mxqk",
                     "attn_fwd_directp_efq_mxqk"):
            dbg_codes = torch.zeros((nq_dbg, nk_pad // 2), dtype=torch.uint8, device=dev)
            dbg_scales = torch.zeros((nq_dbg, nk_pad // 32), dtype=torch.uint8, device=dev)
        else:
            dbg_codes = torch.zeros((nq_dbg, nk_pad), dtype=torch.uint8, device=dev)
    a = make_fwd_args(q, k, v, B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, D=D, softmax_scale=softmax_scale, causal=causal,
                      cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, total_q=total_q, total_k=total_k, o=o,
                      o_dtype=OUT_F32 if out_dtype == torch.float32 else OUT_BF16, lse=lse,
                      dbg_codes=dbg_codes, dbg_scales=dbg_scales, dbg_b=dbg_b, dbg_h=dbg_h)
    if entry != "attn_fwd_directp_noalloc":      # (that one keeps its K tiles in the library's own array)
        need = lib.attn_fwd_ws_bytes(ctypes.byref(a))
        ws = (workspace or _default_ws).get(need, dev)
        a.ws, a.ws_bytes = ws.data_ptr(), ws.numel()
    if events is not None:
        a.prof_event_begin = events[0].cuda_event
        a.prof_event_end = events[1].cuda_event
    _check(getattr(lib, entry)(ctypes.byref(a), _stream()))
    return o, lse, (dbg_codes, dbg_scales)


def fwd_directp(q, k, v, **kw):
    """Direct-P forward: MXFP4 P, V FP8 or MXFP4 (noncausal)."""
    return _fwd_lowp("attn_fwd_directp", q, k, v, **kw)


def fwd_directp_noalloc(q, k, v, **kw):
    """attn_fwd_directp without a caller workspace: the library keeps the K
    operand tiles in a fixed device array (ATTN_NOALLOC_SCRATCH_BYTES per GPU)
    and the call allocates nothing.  Calls that overlap on one GPU race."""
    return _fwd_lowp("attn_fwd_directp_noalloc", q, k, v, **kw)


def fwd_fp8pv(q, k, v, **kw):
    """FP8-P/V forward (causal allowed)."""
    return _fwd_lowp("attn_fwd_fp8pv", q, k, v, **kw)


def fwd_directp_efq(q, k, v, **kw):
    """Exp-free Direct-P: E2M1 codes by the log-linear cast (noncausal)."""
    return _fwd_lowp("attn_fwd_directp_efq", q, k, v, **kw)


def fwd_fp8pv_cast(q, k, v, **kw):
    """Exp-free FP8-P/V: E4M3 codes by the one-FMA log-linear cast (causal allowed)."""
    return _fwd_lowp("attn_fwd_fp8pv_cast", q, k, v, **kw)


def fwd_directp_mxqk(q, k, v, **kw):
    """Direct-P with MX-native Q/K (opt-in): q/k from quant_mxfp4, Q.K^T on
    the block-scaled FP4 matrix instruction (noncausal)."""
    return _fwd_lowp("attn_fwd_directp_mxqk", q, k, v, **kw)


def fwd_fp8pv_mxqk(q, k, v, **kw):
    """FP8-P/V with MX-native Q/K (opt-in; causal allowed)."""
    return _fwd_lowp("attn_fwd_fp8pv_mxqk", q, k, v, **kw)


def fwd_directp_efq_mxqk(q, k, v, **kw):
    """Exp-free Direct-P with MX-native Q/K (opt-in; noncausal)."""
    return _fwd_lowp("attn_fwd_directp_efq_mxqk", q, k, v, **kw)


def fwd_fp8pv_cast_mxqk(q, k, v, **kw):
    """Exp-free FP8-P/V with MX-native Q/K (opt-in; causal allowed)."""
    return _fwd_lowp("attn_fwd_fp8pv_cast_mxqk", q, k, v, **kw)


def _decode(entry, q, k, v, *, B, Hq, Hkv, nq, Nk, D, softmax_scale, causal=False, seqlens_k=None,
            out_dtype=torch.float32, want_lse=True, debug=None, events=None, out=None):
    """Shared driver of the decode entry points.  q: NVFP4 (codes, scales,
    tensor_scale) of a [B, nq, Hq, D] tensor; k: the same of the head-major
    K cache [B, Hkv, Nk, D]; v: (format, codes, scales|None,
    tensor_scale|None) from quant_v_cache of the [B, Nk, Hkv, D] V cache;
    seqlens_k: optional device int32 [B].  Returns (O [B, nq, Hq, D],
    LSE [B, Hq, nq], (dump codes, dump scales))."""
    lib = load_library()
    _need_cuda(q[0], k[0], v[1], seqlens_k)
    dev = q[0].device
    if out is not None:
        o, lse = out
    else:
        o = torch.empty((B, nq, Hq, D), dtype=out_dtype, device=dev)
        lse = torch.empty((B, Hq, nq), dtype=torch.float32, device=dev) if want_lse else None
    a = DecodeArgs()
    a.B, a.Hq, a.Hkv, a.nq, a.Nk, a.D = B, Hq, Hkv, nq, Nk, D
    a.seqlens_k = None if seqlens_k is None else seqlens_k.data_ptr()
    a.softmax_scale = softmax_scale
    a.causal = 1 if causal else 0
    a.q = _NvTensor(q[0].data_ptr(), q[1].data_ptr(), None if q[2] is None else q[2].data_ptr())
    a.k = _NvTensor(k[0].data_ptr(), k[1].data_ptr(), None if k[2] is None else k[2].data_ptr())
    a.v = _VTensor(v[0], v[1].data_ptr(), None if v[2] is None else v[2].data_ptr(),
                   None if v[3] is None else v[3].data_ptr())
    a.o = o.data_ptr()
    a.o_dtype = OUT_F32 if o.dtype == torch.float32 else OUT_BF16
    a.lse = None if lse is None else lse.data_ptr()
    dbg_codes = dbg_scales = None
    if debug is not None:
        a.dbg_b, a.dbg_h = debug
        nk_pad = (Nk + 127) // 128 * 128
        if entry == "attn_decode_directp":
            dbg_codes = torch.zeros((nq, nk_pad // 2), dtype=torch.uint8, device=dev)
            dbg_scales = torch.zeros((nq, nk_pad // 32), dtype=torch.uint8, device=dev)
            a.dbg_p_scales = dbg_scales.data_ptr()
        else:
            dbg_codes = torch.zeros((nq, nk_pad), dtype=torch.uint8, device=dev)
        a.dbg_p_codes = dbg_codes.data_ptr()
    if events is not None:
        a.prof_event_begin = events[0].cuda_event
        a.prof_event_end = events[1].cuda_event
    _check(getattr(lib, entry)(ctypes.byref(a), _stream()))
    return o, lse, (dbg_codes, dbg_scales)


def decode_directp(q, k, v, **kw):
    """Decode-shaped Direct-P forward (MXFP4 P, V FP8 or MXFP4)."""
    return _decode("attn_decode_directp", q, k, v, **kw)


def decode_fp8pv(q, k, v, **kw):
    """Decode-shaped FP8-P/V forward."""
    return _decode("attn_decode_fp8pv", q, k, v, **kw)


def bwd_fp8(q, k, v, o, lse, dout, *, softmax_scale, causal=True, workspace=None, events=None, debug=None):
    """Backward of the FP8-P/V forward on its saved quantized operands.
    q, k: (codes, scales, tensor_scale) from quant_nvfp4; v: (V_FP8, codes,
    None, tensor_scale) from quant_v; o: bf16 [B, N, Hq, D] forward output;
    lse: float32 [B, Hq, N]; dout: bf16 [B, N, Hq, D].  Returns float32
    (dq [B, N, Hq, D], dk [B, N, Hkv, D], dv [B, N, Hkv, D]) and, with
    ``debug=(b, h)``, a dict of the E4M3 operand dumps of that (batch, query
    head) as a fourth element."""
    lib = load_library()
    _need_cuda(o, lse, dout, q[0], k[0], v[1])
    if o.dtype != torch.bfloat16 or dout.dtype != torch.bfloat16 or lse.dtype != torch.float32:
        raise AttnError("bwd_fp8 expects bf16 o/dout and float32 lse")
    B, N, Hq, D = dout.shape
    Hkv = k[0].shape[-2]
    dev = dout.device
    dq = torch.empty((B, N, Hq, D), dtype=torch.float32, device=dev)
    dk = torch.empty((B, N, Hkv, D), dtype=torch.float32, device=dev)
    dv = torch.empty((B, N, Hkv, D), dtype=torch.float32, device=dev)
    a = BwdArgs()
    a.B, a.Hq, a.Hkv, a.N, a.D = B, Hq, Hkv, N, D
    a.softmax_scale = softmax_scale
    a.causal = 1 if causal else 0
    a.q = _NvTensor(q[0].data_ptr(), q[1].data_ptr(), None if q[2] is None else q[2].data_ptr())
    a.k = _NvTensor(k[0].data_ptr(), k[1].data_ptr(), None if k[2] is None else k[2].data_ptr())
    a.v = _VTensor(v[0], v[1].data_ptr(), None if v[2] is None else v[2].data_ptr(),
                   None if v[3] is None else v[3].data_ptr())
    a.o, a.lse, a.dout = o.data_ptr(), lse.data_ptr(), dout.data_ptr()
    a.dq, a.dk, a.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    dumps = None
    if debug is not None:
        npad = (N + 127) // 128 * 128
        dumps = {"p_codes": torch.zeros((npad, npad), dtype=torch.uint8, device=dev),
                 "p_exps": torch.zeros((npad // 32, npad), dtype=torch.uint8, device=dev),
                 "dsk_codes": torch.zeros((npad, npad), dtype=torch.uint8, device=dev),
                 "dsk_exps": torch.zeros((npad // 32, npad), dtype=torch.uint8, device=dev),
                 "dsq_codes": torch.zeros((npad, npad), dtype=torch.uint8, device=dev),
                 "dsq_exps": torch.zeros((npad, npad // 32), dtype=torch.uint8, device=dev)}
        a.dbg_p_codes, a.dbg_p_exps = dumps["p_codes"].data_ptr(), dumps["p_exps"].data_ptr()
        a.dbg_dsk_codes, a.dbg_dsk_exps = dumps["dsk_codes"].data_ptr(), dumps["dsk_exps"].data_ptr()
        a.dbg_dsq_codes, a.dbg_dsq_exps = dumps["dsq_codes"].data_ptr(), dumps["dsq_exps"].data_ptr()
        a.dbg_b, a.dbg_h = debug
    need = lib.attn_bwd_ws_bytes(ctypes.byref(a))
    ws = (workspace or _default_ws).get(need, dev)
    a.ws, a.ws_bytes = ws.data_ptr(), ws.numel()
    if events is not None:
        a.prof_event_begin = events[0].cuda_event
        a.prof_event_end = events[1].cuda_event
    _check(lib.attn_bwd_fp8(ctypes.byref(a), _stream()))
    if debug is not None:
        return dq, dk, dv, dumps
    return dq, dk, dv


def fwd_bf16(q, k, v, softmax_scale, causal=False, want_lse=True):
    """BF16 baseline forward on dense [B, N, H, D] bf16 tensors."""
    lib = load_library()
    _need_cuda(q, k, v)
    B, Nq, Hq, D = q.shape
    _, Nk, Hkv, _ = k.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if want_lse else None
    _check(lib.attn_fwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, D, softmax_scale,
                             1 if causal else 0, _stream()))
    return o, lse


def probe_issue_rates(kind):
    """Diagnostics: one launch of issue-rate micro-kernel ``kind`` on the
    current stream (see attn_probe_issue_rates in include/attn_fp4.h).
    Returns (mean cycles per workgroup, units of work per launch, grid)."""
    lib = load_library()
    cycles = torch.zeros(512, dtype=torch.int64, device="cuda")
    units = ctypes.c_longlong(0)
    grid = ctypes.c_int(0)
    _check(lib.attn_probe_issue_rates(int(kind), cycles.data_ptr(), ctypes.byref(units), ctypes.byref(grid),
                                      _stream()))
    torch.cuda.synchronize()
    return float(cycles[:grid.value].double().mean()), int(units.value), int(grid.value)
