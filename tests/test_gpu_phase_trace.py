"""The forward's phase-trace diagnostic build (libattnfp4_trace.so: the product
sources with -DATTN_FWD_PHASE_TRACE) computes exactly what the product library
computes, and fills its per-wave phase table.  Skipped when the diagnostic
library has not been built."""

import ctypes
import os

import numpy as np
import pytest
import torch

from precision_attention_forward_amd import _binding as B, synth
from precision_attention_forward_amd.build import TRACE_LIB

pytestmark = pytest.mark.gpu


def _forward(wl, inp):
    q, k = B.quant_nvfp4(inp.q), B.quant_nvfp4(inp.k)
    vq = B.quant_v(inp.v, B.V_MXFP4)
    v = (B.V_MXFP4, vq[0], vq[1], vq[2])
    o, lse, _ = B.fwd_directp(q, k, v, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, softmax_scale=inp.sigma, causal=False,
                              out_dtype=torch.float32, B=wl.B, Nq=wl.N, Nk=wl.N)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def test_phase_trace_build_matches_product(gpu):
    if not os.path.exists(TRACE_LIB):
        pytest.skip("libattnfp4_trace.so is not built (python -m precision_attention_forward_amd.build --phase-trace)")
    # the Wan recipe (MXFP4 P and V, outlier channels) at 2 heads x 1000 keys:
    # 8 key tiles, the last one ragged
    wl = synth.WORKLOADS[2].with_(Hq=2, Hkv=2, N=1000, seed=21)
    inp = synth.generate(wl, "cuda")
    product = B.load_library()
    o_p, l_p = _forward(wl, inp)
    traced = ctypes.CDLL(TRACE_LIB)
    for name, (res, args) in B.EXPORTS.items():
        getattr(traced, name).restype = res
        getattr(traced, name).argtypes = args
    traced.attn_fwd_phase_trace_read.restype = ctypes.c_int
    traced.attn_fwd_phase_trace_read.argtypes = [ctypes.c_void_p]
    B._lib = traced
    try:
        o_t, l_t = _forward(wl, inp)
    finally:
        B._lib = product
    print(f"trace build vs product: O max |diff| {float((o_t - o_p).abs().max()):.3e}", flush=True)
    assert torch.equal(o_t, o_p) and torch.equal(l_t, l_p), "the phase-trace build changed the results"
    table = np.zeros((8, 8), dtype=np.uint64)
    assert traced.attn_fwd_phase_trace_read(table.ctypes.data_as(ctypes.c_void_p)) == 0
    n_tiles = (wl.N + 127) // 128
    for w in range(8):
        assert int(table[w, 5]) == n_tiles, (w, table[w])
        phases = [int(x) for x in table[w, :5]]
        assert all(p > 0 for p in phases[:4]), (w, phases)
        # every wave's iterations together span about the same time
        assert 0.5 < sum(phases) / sum(int(x) for x in table[0, :5]) < 2.0, (w, phases)
