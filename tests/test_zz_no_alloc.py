"""attn_fwd_directp_noalloc (the forward for callers that cannot allocate)
against attn_fwd_directp on the same inputs, through the C ABI: the two run
the same kernels, so O and LSE must agree bit for bit.  Two calls in a row,
the second with a smaller input, so the second reads the library's array
after a larger call has filled it."""

import ctypes

import pytest
import torch

from precision_attention_forward_amd import synth

pytestmark = pytest.mark.gpu


def _quantized(gpu, wl):
    inp = synth.generate(wl, "cpu")
    q, k = gpu.quant_nvfp4(inp.q.cuda()), gpu.quant_nvfp4(inp.k.cuda())
    vf = gpu.V_FP8 if wl.v_format == "fp8" else gpu.V_MXFP4
    vq = gpu.quant_v(inp.v.cuda(), vf)
    return inp, q, k, (vf, vq[0], vq[1], vq[2])


def _both(gpu, wl):
    inp, q, k, v = _quantized(gpu, wl)
    kw = dict(B=wl.B, Nq=wl.N, Nk=wl.N, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, softmax_scale=inp.sigma)
    o_ref, l_ref, _ = gpu.fwd_directp(q, k, v, **kw)
    torch.cuda.synchronize()
    o, l, _ = gpu.fwd_directp_noalloc(q, k, v, **kw)
    torch.cuda.synchronize()
    return o, l, o_ref, l_ref


CASES = [
    # the array's capacity exactly: 8 KV heads x 4 x 8192 keys at D = 128 (MXFP4 P, FP8 V)
    ("at_capacity", synth.WORKLOADS[4].with_(causal=False, p_format="mxfp4", seed=401)),
    # then a smaller call: the Wan recipe with MXFP4 V on 2 heads of 700 keys (a ragged last tile)
    ("smaller", synth.WORKLOADS[2].with_(Hq=2, Hkv=2, N=700, seed=402)),
]


def test_noalloc_matches_workspace_entry_point(gpu):
    lib = gpu.load_library()
    for name, wl in CASES:
        print(f"[case] noalloc {name}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} N={wl.N} D={wl.D} V={wl.v_format}",
              flush=True)
        a = gpu.make_fwd_args(*(_quantized(gpu, wl)[1:]), B=wl.B, Hq=wl.Hq, Hkv=wl.Hkv, Nq=wl.N, Nk=wl.N, D=wl.D,
                              softmax_scale=wl.D ** -0.5)
        assert lib.attn_fwd_ws_bytes(ctypes.byref(a)) <= (64 << 20) + 4096
        o, l, o_ref, l_ref = _both(gpu, wl)
        assert torch.equal(o, o_ref), f"{name}: O differs from attn_fwd_directp"
        assert torch.equal(l, l_ref), f"{name}: LSE differs from attn_fwd_directp"


def test_noalloc_rejects_beyond_capacity(gpu):
    # one KV column past the array: refused before any launch
    lib = gpu.load_library()
    wl = synth.WORKLOADS[4].with_(B=1, causal=False, p_format="mxfp4", N=4 * 8192 + 128)
    a = gpu.make_fwd_args(*(_quantized(gpu, wl.with_(N=128))[1:]), B=1, Hq=wl.Hq, Hkv=wl.Hkv, Nq=wl.N, Nk=wl.N,
                          D=wl.D, softmax_scale=0.1, o=torch.empty(16, device="cuda"))
    assert lib.attn_fwd_ws_bytes(ctypes.byref(a)) > (64 << 20) + 4096
    assert lib.attn_fwd_directp_noalloc(ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 3
