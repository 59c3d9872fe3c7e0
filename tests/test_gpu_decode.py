"""GPU decode-shaped forward (attn_decode_directp / attn_decode_fp8pv) vs the
oracle on the same seeded inputs.

A decode step runs the oracle's tiled forward for the nq new tokens of each
(sequence, head) against that sequence's valid cache entries: K quantized
over the whole cache tensor (its amax), V quantized over the whole cache
(MXFP4 V blocks of 32 keys from key 0 of the sequence, as stored), new token
i at position L - nq + i for the causal mask.

Bar (as for the prefill forward): every probability code or block exponent
in which the kernel's dump differs from the oracle must be a float32
rounding near-tie, at most 1e-4 of the live codes; O within relative L2
1e-3 and max abs 5e-3, LSE within 1e-4 relative, against the oracle's own
outputs, widened on a row only by the oracle-only bound of what its near-tie
codes could move; where a tie went the other way, also against the oracle
run on the kernel's codes.  The dump build must reproduce the production
outputs bit for bit.
"""

import numpy as np
import pytest
import torch

from helpers import (PureCompare, assert_close_outputs, check_code_choices, f32, gpu_codes, oracle_v_head, p_mismatch,
                     tie_flip_bound, P_MISMATCH_MAX)
from oracle import attention as OA
from oracle import quant as OQ
from precision_attention_forward_amd import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _amax(x, chunk=1 << 26):
    flat = x.reshape(-1)
    return max(float(flat[i:i + chunk].to("cpu").abs().max()) for i in range(0, flat.numel(), chunk))


class _Prepared:
    """Quantized operands of a decode step (the cache quantized once, as a
    prefill would have stored it)."""

    def __init__(self, gpu, inp):
        wl = inp.wl
        self.q = gpu.quant_nvfp4(inp.q.cuda())
        self.k = gpu.quant_nvfp4(inp.k.cuda())
        self.vf = gpu.V_FP8 if wl.v_format == "fp8" else gpu.V_MXFP4
        vq = gpu.quant_v_cache(inp.v.cuda(), self.vf)
        self.v = (self.vf, vq[0], vq[1], vq[2])
        self.seqlens = inp.seqlens.cuda()


def _run(gpu, inp, prep, debug=None):
    wl = inp.wl
    fn = gpu.decode_directp if wl.p_format == "mxfp4" else gpu.decode_fp8pv
    o, lse, dbg = fn(prep.q, prep.k, prep.v, B=wl.B, Hq=wl.Hq, Hkv=wl.Hkv, nq=inp.q.shape[1], Nk=wl.N, D=wl.D,
                     softmax_scale=inp.sigma, causal=wl.causal, seqlens_k=prep.seqlens, debug=debug)
    torch.cuda.synchronize()
    return o, lse, dbg


def _check(gpu, inp, pairs=None):
    """Compare every (sequence, head) in ``pairs`` (default: all) with the
    oracle: O and LSE against the oracle's own outputs (helpers.PureCompare,
    widened only by the oracle-only bound of its near-tie codes); every code
    or block exponent of the dump that differs from the oracle's must be a
    rounding near-tie; where one went the other way, O and LSE must also
    meet the plain bars against the oracle run on the kernel's codes."""
    wl = inp.wl
    prep = _Prepared(gpu, inp)
    o, lse, _ = _run(gpu, inp, prep)
    nq = inp.q.shape[1]
    G = wl.Hq // wl.Hkv
    amax_q, amax_k, amax_v = _amax(inp.q), _amax(inp.k), _amax(inp.v)
    if pairs is None:
        pairs = [(b, h) for b in range(wl.B) for h in range(wl.Hq)]
    pure = PureCompare(f"{wl.name} decode vs the oracle")
    tight = [0.0, 0.0, 0.0]
    n_mis = n_tot = n_e = n_c = 0
    vcache = {}
    for (b, h) in pairs:
        L = int(inp.seqlens[b])
        hk = h // G
        q_index = (L - nq + np.arange(nq)) if wl.causal else None
        qc, qs, gq = OQ.quant_nvfp4(f32(inp.q[b, :, h]), amax=amax_q)
        kc, ks, gk = OQ.quant_nvfp4(f32(inp.k[b, hk, :L]), amax=amax_k)
        if (b, hk) not in vcache:
            vcache[(b, hk)] = oracle_v_head(f32(inp.v[b, :, hk]), wl.v_format, amax_v)[:L]
        args = (OQ.dequant_nvfp4_raw(qc, qs), OQ.dequant_nvfp4_raw(kc, ks), gq, gk, vcache[(b, hk)], inp.sigma,
                wl.p_format, wl.causal)
        od, ld, (dc, ds) = _run(gpu, inp, prep, debug=(b, h))
        assert torch.equal(od, o) and torch.equal(ld, lse), "the dump build computes other outputs"
        og, lg = f32(o[b, :, h]).astype(np.float64), f32(lse[b, h]).astype(np.float64)
        O, Lr, oc, oe, pre, xmax, tiles = OA.attn_lowp_head(*args, q_index=q_index, return_pre=True,
                                                             return_tiles=True)
        ob, lb = np.zeros_like(O), np.zeros(nq)
        if L > 0:
            dcn = dc.cpu().numpy()
            dsn = None if ds is None else ds.cpu().numpy()
            gc, ge = gpu_codes(dcn, dsn, wl.p_format, L)
            live = (np.arange(L)[None, :] <= q_index[:, None]) if wl.causal else np.ones((nq, L), bool)
            e1, c1 = check_code_choices(gc, ge, oc, oe, pre, xmax, wl.p_format, "exact", live)
            mis, tot = p_mismatch(dcn, dsn, oc, oe, wl.p_format, L, live)
            n_mis, n_tot, n_e, n_c = n_mis + mis, n_tot + tot, n_e + e1, n_c + c1
            ob, lb, _ = tie_flip_bound(pre, oc, oe, xmax, tiles, O, vcache[(b, hk)], wl.p_format, "exact", live)
            if e1 or c1:
                O2, L2 = OA.attn_lowp_head(*args, q_index=q_index, p_given=(gc, ge))
                t = assert_close_outputs(og, lg, O2, L2, f"seq {b} head {h} on the kernel's codes")
                tight = [max(x, y) for x, y in zip(tight, t)]
        pure.add(og, lg, O, Lr, ob, lb)
    rel = pure.finish()
    assert n_mis <= P_MISMATCH_MAX * max(n_tot, 1), f"P codes: {n_mis} of {n_tot} differ"
    print(f"  P codes: {n_mis} of {n_tot} live codes differ; near-ties taken the other way: {n_e} exponents, "
          f"{n_c} codes; against the oracle: O rel L2 {rel:.2e}, max abs {pure.max_abs:.2e}, LSE rel "
          f"{pure.lse_rel:.2e} ({pure.rows_with_ties} of {pure.rows} rows with near-tie candidates, "
          f"{pure.rows_widened} past the plain bar)", flush=True)
    if n_e or n_c:
        print(f"  on the kernel's codes: O rel L2 {tight[0]:.2e}, max abs {tight[1]:.2e}, LSE rel {tight[2]:.2e}",
              flush=True)
    return o, lse


W = synth.WORKLOADS[6]
SMALL = [
    # Direct-P, FP8 V, one new token, ragged cache lengths, GQA 4
    ("directp_fp8v_nq1", W.with_(B=3, Hq=8, Hkv=2, N=1024, seed=61, extra={"nq": 1, "ragged": True})),
    # four new tokens with the causal mask among them (16 query rows per KV head)
    ("directp_nq4_causal", W.with_(B=2, Hq=8, Hkv=2, N=768, seed=62, extra={"nq": 4, "ragged": True})),
    # FP8 P/V, D = 64, no GQA, three causal tokens
    ("fp8pv_d64_nq3", W.with_(B=2, Hq=4, Hkv=4, N=640, D=64, p_format="fp8", seed=63,
                              extra={"nq": 3, "ragged": True})),
    # Direct-P with MXFP4 V, noncausal (every new token sees the whole cache)
    ("directp_mxfp4v_noncausal", W.with_(B=2, Hq=4, Hkv=1, N=896, causal=False, v_format="mxfp4", seed=64,
                                         extra={"nq": 2, "ragged": True})),
    # 48 query rows per KV head: two workgroups (query groups) per KV head
    ("directp_two_query_groups", W.with_(B=1, Hq=16, Hkv=1, N=384, seed=65, extra={"nq": 3})),
    # MXFP4 V with D = 64
    ("directp_mxfp4v_d64", W.with_(B=2, Hq=2, Hkv=2, N=384, D=64, v_format="mxfp4", seed=66,
                                   extra={"nq": 1, "ragged": True})),
]


@pytest.mark.parametrize("name,wl", SMALL, ids=[s[0] for s in SMALL])
def test_decode_small_all_heads(gpu, name, wl):
    _say(f"decode {name}")
    _check(gpu, synth.generate_decode(wl))


@pytest.mark.parametrize("name,wl", [SMALL[1], SMALL[2]], ids=[SMALL[1][0], SMALL[2][0]])
def test_decode_wide_score_range(gpu, name, wl):
    # new-token rows scaled by powers of two 2^-3 .. 2^6 (per sequence, row and
    # head): blocks of the cache underflow to the E8M0 floor beside flat rows
    _say(f"decode wide score range {name}")
    inp = synth.generate_decode(wl)
    g = torch.Generator().manual_seed(wl.seed + 1000)
    f = torch.exp2(torch.randint(-3, 7, tuple(inp.q.shape[:-1]), generator=g).float())
    inp.q = (inp.q.float() * f[..., None]).to(torch.bfloat16)
    _check(gpu, inp)


def test_decode_length_edges(gpu):
    # valid lengths at and around the block (32) and tile (128) edges, a full
    # cache, an empty one, and caches shorter than the new tokens (causal rows
    # with no visible key: O = 0, LSE = -inf)
    wl = W.with_(B=10, Hq=4, Hkv=2, N=384, seed=67, extra={"nq": 2})
    inp = synth.generate_decode(wl)
    inp.seqlens = torch.tensor([0, 1, 2, 63, 64, 65, 128, 129, 257, 384], dtype=torch.int32)
    _say("decode length edges")
    o, lse = _check(gpu, inp)
    assert float(o[0].abs().max()) == 0.0 and bool(torch.isinf(lse[0]).all())
    assert bool(torch.isinf(lse[1, :, 0]).all())          # L = 1, token 0 sits at position -1


def test_decode_full_size_sampled(gpu):
    # the benchmark's workload and launch configuration: B = 64, Hq = 32,
    # Hkv = 8, 8192 cached keys, one new token; sampled (sequence, head) pairs
    wl = synth.WORKLOADS[6]
    _say(f"decode full-size {wl.name}")
    inp = synth.generate_decode(wl)
    pairs = [(0, 0), (0, 31), (17, 5), (63, 0), (63, 30)]
    o, lse = _check(gpu, inp, pairs=pairs)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    torch.cuda.empty_cache()


def test_decode_bf16_output(gpu):
    # the bf16 output is the float32 output rounded to nearest even, element
    # for element; LSE is the same; without an LSE buffer O is unchanged
    wl = W.with_(B=2, Hq=8, Hkv=2, N=512, seed=68, extra={"nq": 2, "ragged": True})
    inp = synth.generate_decode(wl)
    prep = _Prepared(gpu, inp)
    kw = dict(B=wl.B, Hq=wl.Hq, Hkv=wl.Hkv, nq=2, Nk=wl.N, D=wl.D, softmax_scale=inp.sigma, causal=True,
              seqlens_k=prep.seqlens)
    _say("decode bf16 output")
    o32, l32, _ = gpu.decode_directp(prep.q, prep.k, prep.v, **kw)
    o16, l16, _ = gpu.decode_directp(prep.q, prep.k, prep.v, out_dtype=torch.bfloat16, **kw)
    o_nolse, none, _ = gpu.decode_directp(prep.q, prep.k, prep.v, want_lse=False, **kw)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(l16, l32) and torch.equal(o_nolse, o32)


def test_decode_step_graph_replays(gpu):
    # a decode step (Q quantization + decode kernel) captured as a HIP graph:
    # every replay, with eager library work and synchronizations between the
    # replays, reproduces the eager step's outputs bit for bit
    wl = W.with_(B=4, Hq=8, Hkv=2, N=512, seed=69, extra={"nq": 1, "ragged": True})
    inp = synth.generate_decode(wl)
    prep = _Prepared(gpu, inp)
    qb = inp.q.cuda()
    kw = dict(B=wl.B, Hq=wl.Hq, Hkv=wl.Hkv, nq=1, Nk=wl.N, D=wl.D, softmax_scale=inp.sigma, causal=True,
              seqlens_k=prep.seqlens)
    _say("decode step as a replayed graph")
    out = gpu.decode_directp(gpu.quant_nvfp4(qb), prep.k, prep.v, **kw)[:2]
    torch.cuda.synchronize()
    ref = [t.clone() for t in out]

    def step():
        gpu.decode_directp(gpu.quant_nvfp4(qb), prep.k, prep.v, out=out, **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = (qb.float() * 2).to(torch.bfloat16)
    for r in range(4):
        for t in out:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(out, ref):
            assert torch.equal(x, y), f"replay {r}"
        # eager work between replays: another step on other inputs and outputs
        o2 = gpu.decode_directp(gpu.quant_nvfp4(other), prep.k, prep.v, **kw)[0]
        torch.cuda.synchronize()
        assert bool(torch.isfinite(o2).all())
