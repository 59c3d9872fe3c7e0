"""GPU forward (Direct-P and FP8-P/V, exact and exp-free encoders) vs the
oracle on the same seeded inputs.

Bar: probability codes (debug dump of each compared (batch, head)) may
differ from the oracle's in at most 1e-4 of the live elements, and only at
rounding near-ties; O within relative L2 1e-3 and max abs 5e-3, LSE within
1e-4 relative, of the oracle's own outputs -- widened on a row only by the
oracle-only bound of what its near-tie codes could move.  Small shapes are
compared on every output; the full-size workloads, in the launch
configuration the benchmark times, on every head's first 256 query rows plus
seeded later rows, and on one complete head.
"""

import math
import os
import shutil
import tempfile
import time

import numpy as np
import pytest
import torch

import oracle_pool
from helpers import PureCompare, assert_close_outputs, f32, oracle_head, P_MISMATCH_MAX
from precision_attention_forward_amd import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


ENTRY = {("mxfp4", "exact"): "fwd_directp", ("fp8", "exact"): "fwd_fp8pv",
         ("mxfp4", "loglin"): "fwd_directp_efq", ("fp8", "loglin"): "fwd_fp8pv_cast"}


def _gpu_run(gpu, inp, debug=None, out_dtype=torch.float32, encoder="exact", four_six=False, qk="nvfp4"):
    wl = inp.wl
    sigma = inp.sigma
    if qk in ("mxfp4", "mxfp4_had"):
        had = qk == "mxfp4_had"
        q, k = gpu.quant_mxfp4(inp.q, hadamard=had), gpu.quant_mxfp4(inp.k, hadamard=had)
        sigma = sigma / 32.0 if had else sigma      # rotated Q.K is 32 times the original
    else:
        q = gpu.quant_nvfp4(inp.q, four_six=four_six)
        k = gpu.quant_nvfp4(inp.k, four_six=four_six)
    vf = gpu.V_FP8 if wl.v_format == "fp8" else gpu.V_MXFP4
    kw = dict(Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, softmax_scale=sigma, causal=wl.causal, out_dtype=out_dtype,
              debug=debug)
    if inp.cu_seqlens is None:
        vq = gpu.quant_v(inp.v, vf)
        kw.update(B=wl.B, Nq=wl.N, Nk=wl.N)
    else:
        cu = inp.cu_seqlens.cuda()
        mx = int(inp.seqlens.max())
        vq = gpu.quant_v(inp.v, vf, cu_seqlens=cu, max_seqlen=mx)
        kw.update(cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=mx, max_seqlen_k=mx)
    v = (vf, vq[0], vq[1], vq[2])
    fn = getattr(gpu, ENTRY[(wl.p_format, encoder)] + ("_mxqk" if qk.startswith("mxfp4") else ""))
    o, lse, dbg = fn(q, k, v, **kw)
    torch.cuda.synchronize()
    return o, lse, dbg


def _amax(x, chunk=1 << 26):
    flat = x.reshape(-1)
    return max(float(flat[i:i + chunk].to("cpu").abs().max()) for i in range(0, flat.numel(), chunk))


def _seq_slices(inp):
    wl = inp.wl
    if inp.cu_seqlens is None:
        return [(b, b * wl.N, wl.N) for b in range(wl.B)]
    cu = inp.cu_seqlens.numpy()
    return [(s, int(cu[s]), int(cu[s + 1] - cu[s])) for s in range(len(cu) - 1)]


def _chunk_rows(nk):
    return int(min(512, max(32, (1 << 24) // max(nk, 1))))


def _jobs(inp, heads=None, seqs=None, rows=None, max_rows=None):
    """(sequence, head, query rows) triples from the older selection arguments."""
    wl = inp.wl
    out = []
    for (s, t0, L) in _seq_slices(inp):
        if (seqs is not None and s not in seqs) or L == 0:
            continue
        for h in (range(wl.Hq) if heads is None else heads):
            r = np.arange(L) if rows is None else np.asarray(sorted(set(int(x) for x in rows if x < L)))
            if max_rows is not None and len(r) > max_rows:
                r = r[np.linspace(0, len(r) - 1, max_rows).astype(int)]
            out.append((s, h, r))
    return out


def _check(gpu, inp, heads=None, seqs=None, rows=None, dumps=True, max_rows=None, encoder="exact", four_six=False,
           qk="nvfp4", jobs=None):
    """Run the production kernel once and compare the selected (sequence,
    head, query rows) -- ``jobs``, or the product of heads / seqs / rows --
    with the oracle.

    O and LSE are held to the oracle's own outputs (helpers.PureCompare):
    max abs 5e-3 and LSE 1e-4 relative per element, rel L2 1e-3 over all
    compared rows, each widened only by the oracle-only bound of what its
    near-tie codes could move (helpers.tie_flip_bound).  With ``dumps``, the
    build with the probability dump also runs once per compared (sequence,
    head): its O and LSE must equal the production kernel's bit for bit; every
    probability code or block exponent in which it differs from the oracle
    must be a rounding near-tie (helpers.check_code_choices), at most
    P_MISMATCH_MAX of the live codes; and where a tie went the other way, O
    and LSE must also meet the plain bars against the oracle run on the
    kernel's codes (the tight check)."""
    wl = inp.wl
    o, lse, _ = _gpu_run(gpu, inp, encoder=encoder, four_six=four_six, qk=qk)
    amax_q, amax_k, amax_v = _amax(inp.q), _amax(inp.k), _amax(inp.v)
    varlen = inp.cu_seqlens is not None
    group = wl.Hq // wl.Hkv
    slices = {s: (t0, L) for (s, t0, L) in _seq_slices(inp)}
    if jobs is None:
        jobs = _jobs(inp, heads, seqs, rows, max_rows)
    stats = []
    n_ties = [0, 0]
    tight = [0.0, 0.0, 0.0]
    pure = PureCompare(f"{wl.name} vs the oracle")

    def seq_views(s, h):
        t0, L = slices[s]
        hk = h // group
        if varlen:
            return L, inp.q[t0:t0 + L, h], inp.k[t0:t0 + L, hk], inp.v[t0:t0 + L, hk], o[t0:t0 + L, h], lse[h, t0:t0 + L]
        return L, inp.q[s, :, h], inp.k[s, :, hk], inp.v[s, :, hk], o[s, :, h], lse[s, h]

    # 1. on the GPU, in order: the dump build per compared (sequence, head),
    #    and the host copies of the rows to compare
    host = []
    for (s, h, r) in jobs:
        r = np.asarray(r)
        L, qh, kh, vh, o_g, l_g = seq_views(s, h)
        ridx = torch.as_tensor(r, device=o.device)
        rec = dict(s=s, h=h, r=r, L=L, q=f32(qh[ridx]), og=f32(o_g[ridx]).astype(np.float64),
                   lg=f32(l_g[ridx]).astype(np.float64), dc=None, ds=None)
        if dumps:
            od, ld, (dc, ds) = _gpu_run(gpu, inp, debug=(s, h), encoder=encoder, four_six=four_six, qk=qk)
            assert torch.equal(od, o) and torch.equal(ld, lse), "the dump build computes other outputs"
            rec["dc"] = dc[ridx].cpu().numpy()
            rec["ds"] = None if ds is None else ds[ridx].cpu().numpy()
            del od, ld, dc, ds
        host.append(rec)
    t_start = time.time()
    if len(jobs) > 8:
        print(f"  GPU runs and copies done for {len(jobs)} jobs", flush=True)
    # 2. the oracle, in worker processes (tests/oracle_pool.py): each
    #    (sequence, KV head) goes to them once as a file of its K / V rows
    tmp = tempfile.mkdtemp(prefix="attn_parity_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        kv_path = {}
        for (s, hk) in sorted({(rec["s"], rec["h"] // group) for rec in host}):
            _, _, kh, vh, _, _ = seq_views(s, hk * group)
            kv_path[(s, hk)] = os.path.join(tmp, f"kv_{s}_{hk}.npz")
            np.savez(kv_path[(s, hk)], k=f32(kh), v=f32(vh))
        kv_params = dict(amax_k=amax_k, amax_v=amax_v, v_format=wl.v_format, four_six=four_six, qk=qk)
        q_params = dict(amax_q=amax_q, sigma=inp.sigma, four_six=four_six, qk=qk)
        futs = []
        for j, rec in enumerate(host):
            step = _chunk_rows(rec["L"])
            for c0 in range(0, len(rec["r"]), step):
                c1 = min(c0 + step, len(rec["r"]))
                task = dict(kv_path=kv_path[(rec["s"], rec["h"] // group)], kv_params=kv_params,
                            q=rec["q"][c0:c1], q_params=q_params, rows=rec["r"][c0:c1], L=rec["L"],
                            p_format=wl.p_format, encoder=encoder, causal=wl.causal,
                            og=rec["og"][c0:c1], lg=rec["lg"][c0:c1],
                            dc=None if rec["dc"] is None else rec["dc"][c0:c1],
                            ds=None if rec["ds"] is None else rec["ds"][c0:c1],
                            what=f"seq {rec['s']} head {rec['h']}")
                futs.append((j, c0, c1, oracle_pool.pool().submit(oracle_pool.fwd_chunk, task)))
        per_job = [[0, 0] for _ in host]
        t_say = time.time()
        for i_f, (j, c0, c1, f) in enumerate(futs):
            out = f.result()
            if time.time() - t_say > 20:
                t_say = time.time()
                print(f"  oracle chunks {i_f + 1} of {len(futs)} compared ({t_say - t_start:.0f} s)", flush=True)
            rec = host[j]
            pure.add(rec["og"][c0:c1], rec["lg"][c0:c1], out["O"], out["L"], out["ob"], out["lb"])
            n_ties[0] += out["n_e"]
            n_ties[1] += out["n_c"]
            per_job[j][0] += out["mis"]
            per_job[j][1] += out["tot"]
            if out["tight"] is not None:
                tight = [max(a_, b_) for a_, b_ in zip(tight, out["tight"])]
        for j, rec in enumerate(host):
            if rec["dc"] is not None:
                mis, tot = per_job[j]
                stats.append((mis, tot))
                assert mis <= P_MISMATCH_MAX * tot, f"seq {rec['s']} head {rec['h']}: P codes: {mis} of {tot} differ"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    rel = pure.finish()
    if stats:
        tot = sum(t for _, t in stats)
        print(f"  P codes: {sum(m for m, _ in stats)} of {tot} live codes differ; rounding near-ties taken the "
              f"other way: {n_ties[0]} block exponents, {n_ties[1]} element codes", flush=True)
    print(f"  against the oracle: O rel L2 {rel:.2e}, O max abs {pure.max_abs:.2e}, LSE rel {pure.lse_rel:.2e} over "
          f"{pure.rows} rows ({pure.rows_with_ties} with near-tie candidates, {pure.rows_widened} past the plain bar)",
          flush=True)
    if n_ties[0] or n_ties[1]:
        print(f"  on the kernel's codes: O rel L2 {tight[0]:.2e}, max abs {tight[1]:.2e}, LSE rel {tight[2]:.2e}",
              flush=True)
    return o, lse, stats


SMALL = [
    ("tiny", synth.WORKLOADS[1], None),
    ("wan_recipe_small", synth.WORKLOADS[2].with_(Hq=2, Hkv=2, N=1000, seed=21), None),
    ("wan_d64_small", synth.WORKLOADS[3].with_(Hq=3, Hkv=3, N=700, seed=31), None),
    ("llama_causal_small", synth.WORKLOADS[4].with_(B=2, Hq=4, Hkv=2, N=600, seed=41), None),
    ("llama_noncausal_d64", synth.WORKLOADS[4].with_(B=1, Hq=4, Hkv=1, N=333, D=64, causal=False, seed=42), None),
    ("directp_mxfp4v_d64", synth.WORKLOADS[3].with_(Hq=2, Hkv=2, N=520, v_format="mxfp4", seed=33), None),
    ("directp_fp8v_d128_gqa", synth.WORKLOADS[2].with_(Hq=4, Hkv=1, N=384, v_format="fp8", seed=22), None),
    ("varlen_small", synth.WORKLOADS[5].with_(Hq=2, Hkv=2, varlen=(5, 1, 700), seed=51), None),
    ("varlen_causal_fp8", synth.WORKLOADS[4].with_(B=0, Hq=2, Hkv=1, varlen=(4, 1, 400), seed=52), None),
    ("llama_causal_d64", synth.WORKLOADS[4].with_(B=1, Hq=2, Hkv=1, N=450, D=64, seed=43), None),
]


@pytest.mark.parametrize("name,wl,_", SMALL, ids=[s[0] for s in SMALL])
def test_small_shapes_all_outputs(gpu, name, wl, _):
    _say(f"fwd small {name}")
    inp = synth.generate(wl, "cpu")
    inp.q, inp.k, inp.v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    o, lse, stats = _check(gpu, inp)
    assert stats, "probability dump not compared"


def test_edge_single_key_and_short(gpu):
    for N in (1, 2, 31, 128, 129):
        _say(f"fwd edge N={N}")
        wl = synth.WORKLOADS[1].with_(N=N, seed=100 + N)
        inp = synth.generate(wl, "cpu")
        inp.q, inp.k, inp.v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
        o, lse, _ = _check(gpu, inp)
        if N == 1:
            # one key: every query's O is the same dequantized V row
            assert torch.equal(o[0, :1].expand_as(o[0]), o[0])


@pytest.mark.parametrize("qk", ["nvfp4", "mxfp4", "mxfp4_had"])
def test_varlen_with_empty_sequences(gpu, qk):
    # packed batch whose second and fourth sequences are empty: their
    # workgroups must write nothing and the neighbours must be unaffected
    # (4 sequences x 2 heads: the launch order that groups query blocks of
    # one (sequence, head) per XCD, with its padding workgroups)
    wl = synth.WORKLOADS[5].with_(Hq=2, Hkv=1, varlen=(4, 0, 300), seed=53)
    lens = torch.tensor([257, 0, 130, 0], dtype=torch.int32)
    T = int(lens.sum())
    g = torch.Generator().manual_seed(53)
    q = torch.randn(T, 2, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(T, 1, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(T, 1, 128, generator=g).to(torch.bfloat16).cuda()
    cu = torch.zeros(5, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0)
    inp = synth.Inputs(wl, q, k, v, lens, cu, None)
    _say(f"varlen lengths [257, 0, 130, 0], Q/K {qk}")
    _check(gpu, inp, qk=qk)


@pytest.mark.parametrize("nseq,H,Hkv,causal", [(24, 2, 1, False), (24, 2, 2, True), (7, 1, 1, False)],
                         ids=["48pairs_gqa", "48pairs_causal", "7pairs"])
def test_varlen_many_short_sequences(gpu, nseq, H, Hkv, causal):
    # many short sequences (0 .. 300 keys, with 128 and 129 among them): most
    # query-block slots of the packed launch are empty or padding.  48 (batch,
    # head) pairs take the launch order that groups query blocks per XCD, 7
    # pairs the plain order
    g = torch.Generator().manual_seed(900 + nseq + H + int(causal))
    lens = torch.randint(0, 301, (nseq,), generator=g, dtype=torch.int32)
    lens[0], lens[1], lens[2] = 128, 0, 129
    T = int(lens.sum())
    wl = synth.WORKLOADS[5].with_(Hq=H, Hkv=Hkv, causal=causal, p_format="fp8" if causal else "mxfp4",
                                  varlen=(nseq, 0, 300), seed=900 + nseq)
    q = torch.randn(T, H, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(T, Hkv, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(T, Hkv, 128, generator=g).to(torch.bfloat16).cuda()
    cu = torch.zeros(nseq + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0)
    inp = synth.Inputs(wl, q, k, v, lens, cu, None)
    _say(f"varlen {nseq} short sequences, {H} heads / {Hkv} KV heads, causal {causal}, total {T} tokens")
    _check(gpu, inp)


@pytest.mark.parametrize("qk", ["nvfp4", "mxfp4", "mxfp4_had"])
def test_edge_zero_queries_closed_form(gpu, qk):
    # Q = 0: every probability code is 4.0 with e = -2 (p = 1), so O is the mean
    # of the dequantized V rows and LSE = ln(Nk).
    _say(f"fwd Q=0 closed form, Q/K {qk}")
    wl = synth.WORKLOADS[1].with_(N=300, seed=7)
    inp = synth.generate(wl, "cpu")
    inp.q = torch.zeros_like(inp.q)
    inp.q, inp.k, inp.v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    o, lse, _ = _gpu_run(gpu, inp, qk=qk)
    np.testing.assert_allclose(f32(lse), math.log(300), rtol=1e-6)
    o, lse, _ = _check(gpu, inp, dumps=False, qk=qk)


WIDE = [
    ("wan_recipe_wide", synth.WORKLOADS[2].with_(Hq=2, Hkv=2, N=700, seed=81), "nvfp4", "exact"),
    ("llama_causal_gqa_wide", synth.WORKLOADS[4].with_(B=1, Hq=4, Hkv=2, N=520, seed=82), "nvfp4", "exact"),
    ("wan_recipe_wide_mxqk_had", synth.WORKLOADS[2].with_(Hq=2, Hkv=2, N=700, seed=83), "mxfp4_had", "exact"),
    ("llama_causal_wide_mxqk", synth.WORKLOADS[4].with_(B=1, Hq=2, Hkv=1, N=400, seed=84), "mxfp4", "exact"),
    ("wan_recipe_wide_cast", synth.WORKLOADS[2].with_(Hq=2, Hkv=2, N=700, seed=85), "nvfp4", "loglin"),
    ("llama_causal_wide_cast_mxqk", synth.WORKLOADS[4].with_(B=1, Hq=2, Hkv=1, N=400, seed=86), "mxfp4_had",
     "loglin"),
]


@pytest.mark.parametrize("name,wl,qk,encoder", WIDE, ids=[w[0] for w in WIDE])
def test_wide_score_range(gpu, name, wl, qk, encoder):
    # Q rows scaled by powers of two 2^-3 .. 2^6 (per batch, row and head):
    # rows whose scaled scores span hundreds of binades sit beside near-flat
    # ones, so whole 32-key blocks underflow (block exponent at its floor, all
    # codes 0) and the running max jumps far enough to take alpha to 0
    _say(f"fwd wide score range {name}, Q/K {qk}, encoder {encoder}")
    inp = synth.generate(wl, "cpu")
    g = torch.Generator().manual_seed(wl.seed + 1000)
    f = torch.exp2(torch.randint(-3, 7, tuple(inp.q.shape[:-1]), generator=g).float())
    inp.q = (inp.q.float() * f[..., None]).to(torch.bfloat16)
    # the inputs are what the case claims: some row of (batch 0, head 0)
    # spans more than 200 binades between its largest and smallest live score
    x = (inp.q[0, :, 0].float() @ inp.k[0, :, 0].float().T) * inp.sigma * math.log2(math.e)
    live = torch.ones_like(x, dtype=torch.bool)
    if wl.causal:
        live = live.tril()
    span = x.masked_fill(~live, -math.inf).amax(1) - x.masked_fill(~live, math.inf).amin(1)
    assert float(span.max()) > 200.0
    inp.q, inp.k, inp.v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    _check(gpu, inp, qk=qk, encoder=encoder)


def test_bf16_output_mode(gpu):
    _say("fwd bf16 output")
    wl = synth.WORKLOADS[3].with_(Hq=2, Hkv=2, N=500, seed=61)
    inp = synth.generate(wl, "cpu")
    inp.q, inp.k, inp.v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    o32, l32, _ = _gpu_run(gpu, inp)
    o16, l16, _ = _gpu_run(gpu, inp, out_dtype=torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16), o16)
    assert torch.equal(l32, l16)


def test_determinism(gpu):
    _say("fwd determinism")
    wl = synth.WORKLOADS[2].with_(Hq=2, Hkv=2, N=777, seed=71)
    inp = synth.generate(wl, "cpu")
    inp.q, inp.k, inp.v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    a = _gpu_run(gpu, inp)
    b = _gpu_run(gpu, inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _full_size_jobs(inp, seed):
    """The full-size parity subset: every (batch, head) on query rows 0..255
    plus 8 seeded rows from the rest of the sequence, and one complete head;
    for a packed batch, every head of the shortest and the longest sequence
    that way (each also complete on one head), and head 0 of every other
    sequence on its first 256 rows."""
    wl = inp.wl
    rng = np.random.default_rng(seed)

    def rows(L):
        extra = rng.integers(256, L, 8) if L > 256 else []
        return np.unique(np.concatenate([np.arange(min(256, L)), extra]).astype(np.int64))

    if inp.cu_seqlens is None:
        jobs = [(b, h, rows(wl.N)) for b in range(wl.B) for h in range(wl.Hq)]
        jobs[-1] = (wl.B - 1, wl.Hq - 1, np.arange(wl.N))
        return jobs
    lens = inp.seqlens.numpy()
    s_min, s_max = int(np.argmin(lens)), int(np.argmax(lens))
    jobs = []
    for s in range(len(lens)):
        if s in (s_min, s_max):
            jobs += [(s, h, rows(int(lens[s]))) for h in range(wl.Hq)]
        elif lens[s] > 0:
            jobs.append((s, 0, np.arange(min(256, int(lens[s])))))
    i_min = next(i for i, j in enumerate(jobs) if j[0] == s_min and j[1] == 0)
    i_max = next(i for i, j in enumerate(jobs) if j[0] == s_max and j[1] == wl.Hq - 1)
    jobs[i_min] = (s_min, 0, np.arange(int(lens[s_min])))
    jobs[i_max] = (s_max, wl.Hq - 1, np.arange(int(lens[s_max])))
    return jobs


@pytest.mark.parametrize("k", [2, 3, 4, 5], ids=[f"workload{k}" for k in (2, 3, 4, 5)])
def test_full_size_parity_subset(gpu, k):
    # the workloads at their full sizes, in the launch configuration the
    # benchmark times (NVFP4 Q/K, exact encoder)
    wl = synth.WORKLOADS[k]
    inp = synth.generate(wl, "cuda")
    jobs = _full_size_jobs(inp, seed=k)
    n_rows = sum(len(j[2]) for j in jobs)
    _say(f"fwd full-size {wl.name}: {len(jobs)} (sequence, head) jobs, {n_rows} query rows")
    o, lse, stats = _check(gpu, inp, jobs=jobs)
    assert len(stats) == len(jobs)
    del inp, o, lse
    torch.cuda.empty_cache()


# ---- exp-free encoders (log-linear casts): same bar against the oracle's
# encoder="loglin" forward

@pytest.mark.parametrize("name,wl,_", SMALL, ids=[s[0] for s in SMALL])
def test_expfree_small_shapes_all_outputs(gpu, name, wl, _):
    _say(f"fwd exp-free small {name}")
    inp = synth.generate(wl, "cpu")
    inp.q, inp.k, inp.v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    o, lse, stats = _check(gpu, inp, encoder="loglin")
    assert stats, "probability dump not compared"


def test_expfree_edge_short_and_zero_query(gpu):
    for N in (1, 31, 129):
        _say(f"fwd exp-free edge N={N}")
        wl = synth.WORKLOADS[1].with_(N=N, seed=300 + N)
        inp = synth.generate(wl, "cpu")
        inp.q, inp.k, inp.v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
        _check(gpu, inp, encoder="loglin")
    # Q = 0: y = 2 in every block, code 6 (4.0) -> p = 1 as in Direct-P
    wl = synth.WORKLOADS[1].with_(N=300, seed=8)
    inp = synth.generate(wl, "cpu")
    inp.q = torch.zeros_like(inp.q)
    inp.q, inp.k, inp.v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    o, lse, _ = _gpu_run(gpu, inp, encoder="loglin")
    np.testing.assert_allclose(f32(lse), math.log(300), rtol=1e-6)


EXPFREE_FULL = [(2, [0, 39], 32), (4, [0, 31], 32)]


@pytest.mark.parametrize("k,heads,nrows", EXPFREE_FULL, ids=[f"workload{f[0]}" for f in EXPFREE_FULL])
def test_expfree_full_size_sampled(gpu, k, heads, nrows):
    wl = synth.WORKLOADS[k]
    _say(f"fwd exp-free full-size {wl.name}")
    inp = synth.generate(wl, "cuda")
    L = wl.N
    seqs = [0, wl.B - 1]
    rng = np.random.default_rng(100 + k)
    rows = np.unique(np.concatenate([rng.integers(0, L, nrows), [0, 1, 255, 256, L - 1]]))
    o, lse, stats = _check(gpu, inp, heads=heads, seqs=seqs, rows=rows, encoder="loglin")
    assert stats
    del inp
    torch.cuda.empty_cache()


# ---- Q and K quantized with the Four Over Six block scale: the forward
# consumes the same format; parity against the oracle on the same quantizer

FOUR_SIX = [SMALL[1], SMALL[3], SMALL[7]]


@pytest.mark.parametrize("name,wl,_", FOUR_SIX, ids=[s[0] for s in FOUR_SIX])
def test_four_six_quantized_forward(gpu, name, wl, _):
    _say(f"fwd 4/6-quantized Q/K {name}")
    inp = synth.generate(wl, "cpu")
    inp.q, inp.k, inp.v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    o, lse, stats = _check(gpu, inp, four_six=True)
    assert stats


@pytest.mark.parametrize("entry", ["fwd_directp", "fwd_fp8pv"])
def test_no_keys_gives_empty_softmax(gpu, entry):
    # Rows that see no key have an empty softmax: O = 0 and LSE = -inf (the
    # oracle's value), and the kernel must read nothing of K or V, whose
    # buffers are then empty.  Dense Nk = 0, then a packed batch whose second
    # sequence has queries but no keys, beside sequences that have both.
    _say(f"{entry}: Nk = 0 and an empty key sequence")
    vf = gpu.V_FP8
    D, Hq, Hkv = 128, 4, 2
    g = torch.Generator().manual_seed(77)
    q = torch.randn(1, 300, Hq, D, generator=g).to(torch.bfloat16).cuda()
    k = torch.empty(1, 0, Hkv, D, dtype=torch.bfloat16, device="cuda")
    qq, kq = gpu.quant_nvfp4(q), gpu.quant_nvfp4(k)
    vq = gpu.quant_v(torch.empty(1, 0, Hkv, D, dtype=torch.bfloat16, device="cuda"), vf)
    fn = getattr(gpu, entry)
    for out_dtype in (torch.float32, torch.bfloat16):
        o, lse, _ = fn(qq, kq, (vf, vq[0], vq[1], vq[2]), B=1, Nq=300, Nk=0, Hq=Hq, Hkv=Hkv, D=D,
                       softmax_scale=D ** -0.5, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert not o.float().any()
        assert bool(torch.isneginf(lse).all())
    # packed: query lengths [200, 130, 70], key lengths [180, 0, 300]
    lq, lk = [200, 130, 70], [180, 0, 300]
    cu_q = torch.tensor([0] + np.cumsum(lq).tolist(), dtype=torch.int32)
    cu_k = torch.tensor([0] + np.cumsum(lk).tolist(), dtype=torch.int32)
    qp = torch.randn(sum(lq), Hq, D, generator=g).to(torch.bfloat16)
    kp = torch.randn(sum(lk), Hkv, D, generator=g).to(torch.bfloat16)
    vp = torch.randn(sum(lk), Hkv, D, generator=g).to(torch.bfloat16)
    qq, kq = gpu.quant_nvfp4(qp.cuda()), gpu.quant_nvfp4(kp.cuda())
    vq = gpu.quant_v(vp.cuda(), vf, cu_seqlens=cu_k.cuda(), max_seqlen=max(lk))
    o, lse, _ = fn(qq, kq, (vf, vq[0], vq[1], vq[2]), Hq=Hq, Hkv=Hkv, D=D, softmax_scale=D ** -0.5,
                   cu_seqlens_q=cu_q.cuda(), cu_seqlens_k=cu_k.cuda(), max_seqlen_q=max(lq), max_seqlen_k=max(lk))
    torch.cuda.synchronize()
    o, lse = f32(o), f32(lse)
    qf, kf, vf32 = qp.float().numpy(), kp.float().numpy(), vp.float().numpy()
    amax = [float(np.abs(x).max()) for x in (qf, kf, vf32)]
    p_format = "mxfp4" if entry == "fwd_directp" else "fp8"
    for s in range(3):
        q0, q1, k0, k1 = int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1])
        for h in range(Hq):
            O, L = oracle_head(qf[q0:q1, h], kf[k0:k1, h // 2], vf32[k0:k1, h // 2], amax_q=amax[0], amax_k=amax[1],
                               amax_v=amax[2], sigma=D ** -0.5, p_format=p_format, v_format="fp8", causal=False)
            if k1 == k0:
                assert not o[q0:q1, h].any() and bool(np.isneginf(lse[h, q0:q1]).all())
                assert not O.any() and bool(np.isneginf(L).all())
            else:
                assert_close_outputs(o[q0:q1, h], lse[h, q0:q1], O, L, f"seq {s} head {h}")


# ---- cross attention: Nq != Nk (non-causal; causal needs Nq == Nk) -------------
# Dense cases take Q from the first Nq tokens and K / V from the first Nk tokens
# of one draw of the workload's recipe (so the Wan recipe's outlier channels
# agree); packed cases draw the query and the key sequences from two seeds with
# the same number of sequences.
CROSS = [
    ("dense_mxfp4_q_lt_k", synth.WORKLOADS[2].with_(Hq=2, Hkv=2, seed=91), 300, 700, None),
    ("dense_mxfp4_q_gt_k_gqa", synth.WORKLOADS[2].with_(Hq=2, Hkv=1, seed=92), 650, 200, None),
    ("dense_fp8_d64_gqa", synth.WORKLOADS[4].with_(B=2, Hq=4, Hkv=2, D=64, causal=False, seed=93), 129, 383, None),
    ("varlen_fp8_gqa", synth.WORKLOADS[5].with_(Hq=2, Hkv=1, p_format="fp8", seed=94), 0, 0, (4, 300, 520)),
    ("varlen_mxfp4", synth.WORKLOADS[5].with_(Hq=2, Hkv=2, v_format="mxfp4", seed=95), 0, 0, (3, 450, 140)),
]


def _cross_inputs(wl, nq, nk, varlen):
    if varlen is None:
        inp = synth.generate(wl.with_(N=max(nq, nk)), "cpu")
        return (inp.q[:, :nq].contiguous(), inp.k[:, :nk].contiguous(), inp.v[:, :nk].contiguous(), None, None,
                inp.sigma)
    n, qhi, khi = varlen
    iq = synth.generate(wl.with_(varlen=(n, 1, qhi)), "cpu")
    ik = synth.generate(wl.with_(varlen=(n, 1, khi), seed=wl.seed + 1000), "cpu")
    return iq.q, ik.k, ik.v, iq.cu_seqlens, ik.cu_seqlens, iq.sigma


@pytest.mark.parametrize("name,wl,nq,nk,varlen", CROSS, ids=[c[0] for c in CROSS])
def test_cross_attention(gpu, name, wl, nq, nk, varlen):
    """Every output of every (sequence, head) against the oracle run on the
    query rows and the other key sequence, with the P-code dump checks."""
    _say(f"fwd cross {name}")
    qb, kb, vb, cu_q, cu_k, sigma = _cross_inputs(wl, nq, nk, varlen)
    qb, kb, vb = qb.cuda(), kb.cuda(), vb.cuda()
    q, k = gpu.quant_nvfp4(qb), gpu.quant_nvfp4(kb)
    vf = gpu.V_FP8 if wl.v_format == "fp8" else gpu.V_MXFP4
    kw = dict(Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, softmax_scale=sigma, causal=False, out_dtype=torch.float32)
    if cu_q is None:
        vq = gpu.quant_v(vb, vf)
        kw.update(B=wl.B, Nq=nq, Nk=nk)
        seqs = [(b, b * nq, nq, b * nk, nk) for b in range(wl.B)]
    else:
        mq, mk = int((cu_q[1:] - cu_q[:-1]).max()), int((cu_k[1:] - cu_k[:-1]).max())
        vq = gpu.quant_v(vb, vf, cu_seqlens=cu_k.cuda(), max_seqlen=mk)
        kw.update(cu_seqlens_q=cu_q.cuda(), cu_seqlens_k=cu_k.cuda(), max_seqlen_q=mq, max_seqlen_k=mk)
        seqs = [(s, int(cu_q[s]), int(cu_q[s + 1] - cu_q[s]), int(cu_k[s]), int(cu_k[s + 1] - cu_k[s]))
                for s in range(len(cu_q) - 1)]
    v = (vf, vq[0], vq[1], vq[2])
    fn = getattr(gpu, ENTRY[(wl.p_format, "exact")])
    o, lse, _ = fn(q, k, v, **kw)
    torch.cuda.synchronize()
    group = wl.Hq // wl.Hkv
    amax_q, amax_k, amax_v = _amax(qb), _amax(kb), _amax(vb)
    pure = PureCompare(f"{name} vs the oracle")
    mis_all = tot_all = 0
    tmp = tempfile.mkdtemp(prefix="attn_cross_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        futs = []
        for (s, q0, lq, k0, lk) in seqs:
            if lq == 0:
                continue
            for h in range(wl.Hq):
                hk = h // group
                if cu_q is None:
                    qh, kh, vh = qb[s, :, h], kb[s, :, hk], vb[s, :, hk]
                    og, lg = o[s, :, h], lse[s, h]
                else:
                    qh, kh, vh = qb[q0:q0 + lq, h], kb[k0:k0 + lk, hk], vb[k0:k0 + lk, hk]
                    og, lg = o[q0:q0 + lq, h], lse[h, q0:q0 + lq]
                od, ld, (dc, ds) = fn(q, k, v, debug=(s, h), **kw)
                assert torch.equal(od, o) and torch.equal(ld, lse), "the dump build computes other outputs"
                path = os.path.join(tmp, f"kv_{s}_{h}.npz")
                np.savez(path, k=f32(kh), v=f32(vh))
                task = dict(kv_path=path, kv_params=dict(amax_k=amax_k, amax_v=amax_v, v_format=wl.v_format,
                                                         four_six=False, qk="nvfp4"),
                            q=f32(qh), q_params=dict(amax_q=amax_q, sigma=sigma, four_six=False, qk="nvfp4"),
                            rows=np.arange(lq), L=lk, p_format=wl.p_format, encoder="exact", causal=False,
                            og=f32(og).astype(np.float64), lg=f32(lg).astype(np.float64),
                            dc=dc[:lq].cpu().numpy(), ds=None if ds is None else ds[:lq].cpu().numpy(),
                            what=f"seq {s} head {h}")
                futs.append((task["og"], task["lg"], oracle_pool.pool().submit(oracle_pool.fwd_chunk, task)))
        for og, lg, f in futs:
            out = f.result()
            pure.add(og, lg, out["O"], out["L"], out["ob"], out["lb"])
            mis_all += out["mis"]
            tot_all += out["tot"]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    rel = pure.finish()
    assert tot_all > 0 and mis_all <= P_MISMATCH_MAX * tot_all, f"P codes: {mis_all} of {tot_all} differ"
    print(f"  P codes: {mis_all} of {tot_all} differ; O rel L2 {rel:.2e}, max abs {pure.max_abs:.2e}, "
          f"LSE rel {pure.lse_rel:.2e} over {pure.rows} rows", flush=True)
