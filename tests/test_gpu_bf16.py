"""The in-library BF16 attention forward (the comparison baseline) against
textbook softmax attention in float64 on the same bf16 inputs.

Tolerance from the arithmetic: P is rounded to bf16 (relative error <= 2**-9
per probability) and O to bf16 (another 2**-9), with float32 accumulation;
a relative L2 error of 1e-2 bounds both with margin.  The LSE sums unrounded
float32 probabilities, so it is held to 1e-4 absolute."""

import numpy as np
import pytest
import torch

from oracle import attention as OA
from precision_attention_forward_amd import synth

pytestmark = pytest.mark.gpu

CASES = [
    ("d64", dict(B=1, Hq=2, Hkv=2, N=300, D=64, causal=False)),
    ("d128_gqa", dict(B=2, Hq=4, Hkv=2, N=513, D=128, causal=False)),
    ("d128_causal", dict(B=1, Hq=2, Hkv=1, N=700, D=128, causal=True)),
    ("short", dict(B=1, Hq=1, Hkv=1, N=17, D=128, causal=False)),
]


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c[0] for c in CASES])
def test_bf16_forward(gpu, idx):
    name, shape = CASES[idx]
    print(f"[case] bf16 {name}", flush=True)
    wl = synth.WORKLOADS[1].with_(B=shape["B"], Hq=shape["Hq"], Hkv=shape["Hkv"], N=shape["N"], D=shape["D"],
                                  causal=shape["causal"], seed=900 + idx)
    inp = synth.generate(wl, "cpu")
    o, lse = gpu.fwd_bf16(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sigma, causal=wl.causal)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    g = wl.Hq // wl.Hkv
    for b in range(wl.B):
        for h in range(wl.Hq):
            q = inp.q[b, :, h].double().numpy()
            k = inp.k[b, :, h // g].double().numpy()
            v = inp.v[b, :, h // g].double().numpy()
            oe, le = OA.attn_exact_head(q, k, v, inp.sigma, wl.causal)
            rel = np.linalg.norm(o[b, :, h] - oe) / np.linalg.norm(oe)
            assert rel < 1e-2, (b, h, rel)
            assert np.max(np.abs(lse[b, h] - le)) < 1e-4


def test_bf16_forward_full_size_sampled(gpu):
    # the Wan2.1-14B shape the benchmark times (B=1, H=40, N=32760, D=128):
    # 48 sampled query rows of the first and the last head, all keys
    print("[case] bf16 full-size wan14b", flush=True)
    wl = synth.WORKLOADS[2]
    inp = synth.generate(wl, "cuda")
    o, lse = gpu.fwd_bf16(inp.q, inp.k, inp.v, inp.sigma, causal=False)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(5).integers(0, wl.N, 44), [0, 255, 256, wl.N - 1]]))
    ridx = torch.as_tensor(rows, device="cuda")
    for h in (0, wl.Hq - 1):
        q = inp.q[0, ridx, h].double().cpu().numpy()
        k = inp.k[0, :, h].double().cpu().numpy()
        v = inp.v[0, :, h].double().cpu().numpy()
        oe, le = OA.attn_exact_head(q, k, v, inp.sigma, q_index=rows)
        og = o[0, ridx, h].float().cpu().numpy()
        rel = np.linalg.norm(og - oe) / np.linalg.norm(oe)
        assert rel < 1e-2, (h, rel)
        assert np.max(np.abs(lse[0, h, ridx].cpu().numpy() - le)) < 1e-4
    del inp, o, lse
    torch.cuda.empty_cache()
