"""GPU quantizers vs the oracle: codes, block scales and tensor scales must be
bit-exact (NVFP4 Q/K, FP8 E4M3 V, MXFP4 V), on small ragged shapes, the
degenerate cases, and sampled rows of the full-size workloads."""

import numpy as np
import pytest
import torch

from oracle import quant as OQ
from oracle import formats as OF
from precision_attention_forward_amd import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _bf16_cpu(x):
    return x.detach().to("cpu").contiguous()


def _amax_cpu(x_gpu, chunk=1 << 26):
    """max |x| of a bf16 GPU tensor, computed on the CPU in chunks."""
    flat = x_gpu.reshape(-1)
    m = 0.0
    for i in range(0, flat.numel(), chunk):
        m = max(m, float(flat[i:i + chunk].to("cpu").abs().max()))
    return m


def _check_nvfp4(gpu, x_gpu, rows=None, amax=None, four_six=False):
    D = x_gpu.shape[-1]
    codes, scales, ts = gpu.quant_nvfp4(x_gpu, four_six=four_six)
    torch.cuda.synchronize()
    x2 = x_gpu.reshape(-1, D)
    c2, s2 = codes.reshape(-1, D // 2), scales.reshape(-1, D // 16)
    if rows is not None:
        x2, c2, s2 = x2[rows], c2[rows], s2[rows]
    xc = _bf16_cpu(x2).float().numpy()
    oc, os_, og = (OQ.quant_nvfp4_46 if four_six else OQ.quant_nvfp4)(xc, amax=amax)
    np.testing.assert_array_equal(c2.cpu().numpy(), oc)
    np.testing.assert_array_equal(s2.cpu().numpy(), os_)
    assert ts.item() == float(og)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("rows", [1, 37, 1000])
def test_nvfp4_small_bitexact(gpu, D, rows):
    _say(f"nvfp4 D={D} rows={rows}")
    g = torch.Generator().manual_seed(rows * 7 + D)
    x = torch.randn((rows, D), generator=g) * torch.exp2(torch.randint(-8, 8, (rows, 1), generator=g).float())
    x[:, 3] *= 16
    _check_nvfp4(gpu, x.to(torch.bfloat16).cuda())


def test_nvfp4_degenerate_cases(gpu):
    _say("nvfp4 zeros / underflow / tiny / negative zero")
    _check_nvfp4(gpu, torch.zeros((5, 64), dtype=torch.bfloat16, device="cuda"))
    x = torch.zeros((2, 64))
    x[0, 0] = 1000.0
    x[1, 16:32] = -1e-6
    x[1, 40] = -0.0
    _check_nvfp4(gpu, x.to(torch.bfloat16).cuda())
    tiny = torch.full((3, 64), 1e-37) * torch.randn((3, 64), generator=torch.Generator().manual_seed(0))
    _check_nvfp4(gpu, tiny.to(torch.bfloat16).cuda())
    # E2M1 rounding ties and saturation inside one block (amax_t = 6 -> enc 1)
    t = torch.tensor([[6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 0.0, -0.0, 4.5, 5.5, 1.0, 2.0]])
    _check_nvfp4(gpu, t.to(torch.bfloat16).cuda())


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_nvfp4_full_size_sampled(gpu, k):
    wl = synth.WORKLOADS[k]
    _say(f"nvfp4 full-size workload {wl.name}")
    inp = synth.generate(wl, "cuda")
    for name, x in (("q", inp.q), ("k", inp.k)):
        D = x.shape[-1]
        nrows = x.numel() // D
        rng = np.random.default_rng(k)
        rows = torch.from_numpy(np.unique(np.concatenate([rng.integers(0, nrows, 2000), [0, nrows - 1]]))).cuda()
        _check_nvfp4(gpu, x, rows=rows, amax=_amax_cpu(x))
    del inp
    torch.cuda.empty_cache()


# ---- Four Over Six (adaptive block scale): the same bar

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("rows", [1, 37, 1000])
def test_nvfp4_46_small_bitexact(gpu, D, rows):
    _say(f"nvfp4 4/6 D={D} rows={rows}")
    g = torch.Generator().manual_seed(rows * 11 + D)
    x = torch.randn((rows, D), generator=g) * torch.exp2(torch.randint(-8, 8, (rows, 1), generator=g).float())
    x[:, 5] *= 16
    _check_nvfp4(gpu, x.to(torch.bfloat16).cuda(), four_six=True)


def test_nvfp4_46_degenerate_and_hand_derived(gpu):
    _say("nvfp4 4/6 zeros / tiny / hand-derived blocks / tie")
    _check_nvfp4(gpu, torch.zeros((5, 64), dtype=torch.bfloat16, device="cuda"), four_six=True)
    tiny = torch.full((3, 64), 1e-37) * torch.randn((3, 64), generator=torch.Generator().manual_seed(1))
    _check_nvfp4(gpu, tiny.to(torch.bfloat16).cuda(), four_six=True)
    # amax_t = 7 (S_enc 256): block [7, 5.25] takes max 4; block [6] ties and keeps max 6;
    # block [6, 1] with max 6 wins over max 4; then a block of rounding ties
    x = torch.zeros((1, 64))
    x[0, 0], x[0, 1] = 7.0, 5.25
    x[0, 16] = 6.0
    x[0, 32], x[0, 33] = 6.0, 1.0
    x[0, 48:64] = torch.tensor([5.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, -5.0, 4.5, 5.5, 1.0, 2.0, -0.0, 0.0, 3.0, -3.0])
    _check_nvfp4(gpu, x.to(torch.bfloat16).cuda(), four_six=True)
    codes, scales, ts = gpu.quant_nvfp4(x.to(torch.bfloat16).cuda(), four_six=True)
    assert scales[0, 0].item() == 0x7E and scales[0, 1].item() == 0x78 and ts.item() == 1.0 / 256.0


@pytest.mark.parametrize("k", [2, 4])
def test_nvfp4_46_full_size_sampled(gpu, k):
    wl = synth.WORKLOADS[k]
    _say(f"nvfp4 4/6 full-size workload {wl.name}")
    inp = synth.generate(wl, "cuda")
    for name, x in (("q", inp.q), ("k", inp.k)):
        D = x.shape[-1]
        nrows = x.numel() // D
        rng = np.random.default_rng(100 + k)
        rows = torch.from_numpy(np.unique(np.concatenate([rng.integers(0, nrows, 2000), [0, nrows - 1]]))).cuda()
        _check_nvfp4(gpu, x, rows=rows, amax=_amax_cpu(x), four_six=True)
    del inp
    torch.cuda.empty_cache()


def _oracle_v(v_cpu_f32, fmt, cu=None, amax=None):
    """Oracle V codes per sequence in the logical layout."""
    seqs = []
    if cu is None:
        for b in range(v_cpu_f32.shape[0]):
            seqs.append(v_cpu_f32[b])
    else:
        for s in range(len(cu) - 1):
            seqs.append(v_cpu_f32[cu[s]:cu[s + 1]])
    out = []
    for vs in seqs:
        if fmt == "fp8":
            out.append(OQ.quant_v_fp8(vs, amax=amax))
        else:
            out.append(OQ.quant_v_mxfp4(vs))
    return out


def _compare_v(gpu_codes, gpu_scales, gpu_ts, oracle_out, fmt, lens, starts, heads=None, chans=None):
    codes = gpu_codes.cpu().numpy()
    scales = None if gpu_scales is None else gpu_scales.cpu().numpy()
    for s, (o, L, c0) in enumerate(zip(oracle_out, lens, starts)):
        hs = range(codes.shape[0]) if heads is None else heads
        for h in hs:
            ds = range(codes.shape[1]) if chans is None else chans
            for d in ds:
                if fmt == "fp8":
                    oc, s_v = o
                    np.testing.assert_array_equal(codes[h, d, c0:c0 + L], oc[:, h, d], err_msg=f"seq {s} h {h} d {d}")
                    pad = (-L) % 128
                    assert not codes[h, d, c0 + L:c0 + L + pad].any()
                else:
                    oc, oe = o
                    got = OF.unpack_nibbles(codes[h, d, c0 // 2:c0 // 2 + (L + 1) // 2])[:L]
                    np.testing.assert_array_equal(got, oc[:, h, d], err_msg=f"seq {s} h {h} d {d}")
                    nb = (L + 31) // 32
                    np.testing.assert_array_equal(scales[h, d, c0 // 32:c0 // 32 + nb], oe[:, h, d])
        if fmt == "fp8":
            assert gpu_ts.item() == float(o[1])


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("D", [64, 128])
def test_v_dense_small(gpu, fmt, D):
    _say(f"quant_v dense fmt={fmt} D={D}")
    g = torch.Generator().manual_seed(D)
    B, Nk, H = 2, 300, 3
    v = (torch.randn((B, Nk, H, D), generator=g) * 3).to(torch.bfloat16)
    v[0, 5:37, 1, 7] = 0          # an all-zero MX block
    f = gpu.V_FP8 if fmt == "fp8" else gpu.V_MXFP4
    codes, scales, ts, cols = gpu.quant_v(v.cuda(), f)
    torch.cuda.synchronize()
    vf = v.float().numpy()
    ora = _oracle_v(vf, fmt, amax=np.abs(vf).max())
    nk_pad = (Nk + 127) // 128 * 128
    _compare_v(codes, scales, ts, ora, fmt, [Nk] * B, [b * nk_pad for b in range(B)])


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_v_varlen_small(gpu, fmt):
    _say(f"quant_v varlen fmt={fmt}")
    lens = [1, 129, 64, 300, 31]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    g = torch.Generator().manual_seed(3)
    v = torch.randn((int(cu[-1]), 2, 64), generator=g).to(torch.bfloat16)
    f = gpu.V_FP8 if fmt == "fp8" else gpu.V_MXFP4
    cu_d = torch.from_numpy(cu).cuda()
    codes, scales, ts, cols = gpu.quant_v(v.cuda(), f, cu_seqlens=cu_d, max_seqlen=max(lens))
    torch.cuda.synchronize()
    vf = v.float().numpy()
    ora = _oracle_v(vf, fmt, cu=cu, amax=np.abs(vf).max())
    starts = [128 * (int(cu[s]) // 128 + s) for s in range(len(lens))]
    _compare_v(codes, scales, ts, ora, fmt, lens, starts)


def test_v_fp8_scale_non_power_of_two_amax(gpu):
    # the hand-derived FP8 V fixture of the oracle's pins (amax = 49/32): the
    # kernel's stored scale and codes must equal the literals bit for bit
    from test_oracle_quant import FP8V_AMAX_PIN
    _say("quant_v fp8, amax 49/32 fixture")
    vals = torch.tensor(FP8V_AMAX_PIN["values"], dtype=torch.float32)
    n = vals.numel()
    v = torch.zeros((1, n, 1, 64), dtype=torch.float32)
    v[0, :, 0, 0] = vals
    v[0, :, 0, 5] = vals.flip(0) * 0.5
    vb = v.to(torch.bfloat16)
    assert torch.equal(vb.float(), v), "fixture values must be bf16-representable"
    codes, scales, ts, cols = gpu.quant_v(vb.cuda(), gpu.V_FP8)
    torch.cuda.synchronize()
    assert ts.cpu().view(torch.int32).item() == FP8V_AMAX_PIN["s_v_bits"]
    assert codes[0, 0, :n].cpu().tolist() == FP8V_AMAX_PIN["codes"]
    vf = vb.float().numpy()
    _compare_v(codes, scales, ts, _oracle_v(vf, "fp8", amax=np.abs(vf).max()), "fp8", [n], [0])


@pytest.mark.parametrize("k", [2, 3, 5])
def test_v_full_size_sampled(gpu, k):
    wl = synth.WORKLOADS[k]
    _say(f"quant_v full-size workload {wl.name} fmt={wl.v_format}")
    inp = synth.generate(wl, "cuda")
    f = gpu.V_FP8 if wl.v_format == "fp8" else gpu.V_MXFP4
    amax = _amax_cpu(inp.v)
    if inp.cu_seqlens is None:
        codes, scales, ts, cols = gpu.quant_v(inp.v, f)
        seq_ids = [0]
        lens = [wl.N]
        starts = [0]
        seqs = [inp.v[0]]
    else:
        cu = inp.cu_seqlens.numpy()
        codes, scales, ts, cols = gpu.quant_v(inp.v, f, cu_seqlens=inp.cu_seqlens.cuda(),
                                              max_seqlen=int(inp.seqlens.max()))
        seq_ids = [int(np.argmin(inp.seqlens)), int(np.argmax(inp.seqlens))]
        lens = [int(inp.seqlens[s]) for s in seq_ids]
        starts = [128 * (int(cu[s]) // 128 + s) for s in seq_ids]
        seqs = [inp.v[int(cu[s]):int(cu[s + 1])] for s in seq_ids]
    torch.cuda.synchronize()
    heads, chans = [0, wl.Hkv - 1], [0, 5, wl.D - 1]
    ora = []
    for sv in seqs:
        vf = sv[:, heads].to("cpu").float().numpy()
        if wl.v_format == "fp8":
            ora.append(OQ.quant_v_fp8(vf, amax=amax))
        else:
            ora.append(OQ.quant_v_mxfp4(vf))
    sub_codes = codes[heads][:, chans]
    sub_scales = None if scales is None else scales[heads][:, chans]
    # re-index: oracle arrays are [N, len(heads), D]; compare selected channels
    ora_sel = []
    for o in ora:
        if wl.v_format == "fp8":
            ora_sel.append((o[0][:, :, chans], o[1]))
        else:
            ora_sel.append((o[0][:, :, chans], o[1][:, :, chans]))
    _compare_v(sub_codes, sub_scales, ts, ora_sel, wl.v_format, lens, starts)
    del inp
    torch.cuda.empty_cache()


def _compare_v_cache(codes, scales, ts, ora, fmt, seqs, heads, chans):
    """Decode-cache V (blocks [B, Hkv, Nk/128, D, row]) against the oracle's
    codes of the listed sequences (ora[i] covers sequence seqs[i], heads and
    channels indexed as given)."""
    codes = codes.cpu().numpy()
    scales = None if scales is None else scales.cpu().numpy()
    for i, b in enumerate(seqs):
        oc = ora[i][0]
        N = oc.shape[0]
        for hi, h in enumerate(heads):
            for ci, d in enumerate(chans):
                if fmt == "fp8":
                    got = codes[b, h, :, d, :].reshape(-1)
                else:
                    got = OF.unpack_nibbles(codes[b, h, :, d, :].reshape(-1))
                    np.testing.assert_array_equal(scales[b, h, :, d, :].reshape(-1), ora[i][1][:, hi, ci],
                                                  err_msg=f"scales seq {b} h {h} d {d}")
                np.testing.assert_array_equal(got[:N], oc[:, hi, ci], err_msg=f"codes seq {b} h {h} d {d}")
        if fmt == "fp8":
            assert ts.item() == float(ora[i][1])


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("D", [64, 128])
def test_v_cache_small(gpu, fmt, D):
    # the decode cache layout holds the oracle's V codes of every key, head and channel
    _say(f"quant_v_cache fmt={fmt} D={D}")
    g = torch.Generator().manual_seed(10 + D)
    B, Nk, H = 2, 256, 3
    v = (torch.randn((B, Nk, H, D), generator=g) * 3).to(torch.bfloat16)
    v[1, 130:162, 2, 9] = 0       # an all-zero MX block
    f = gpu.V_FP8 if fmt == "fp8" else gpu.V_MXFP4
    codes, scales, ts = gpu.quant_v_cache(v.cuda(), f)
    torch.cuda.synchronize()
    vf = v.float().numpy()
    ora = _oracle_v(vf, fmt, amax=np.abs(vf).max())
    _compare_v_cache(codes, scales, ts, ora, fmt, list(range(B)), list(range(H)), list(range(D)))


def test_v_cache_full_size_sampled(gpu):
    # the decode workload's cache (64 sequences x 8192 keys x 8 KV heads, FP8):
    # first and last sequence, first and last head, three channels
    wl = synth.WORKLOADS[6]
    _say(f"quant_v_cache full-size workload {wl.name} fmt={wl.v_format}")
    inp = synth.generate_decode(wl, "cuda")
    f = gpu.V_FP8 if wl.v_format == "fp8" else gpu.V_MXFP4
    amax = _amax_cpu(inp.v)
    codes, scales, ts = gpu.quant_v_cache(inp.v, f)
    torch.cuda.synchronize()
    seqs, heads, chans = [0, wl.B - 1], [0, wl.Hkv - 1], [0, 5, wl.D - 1]
    ora = []
    for b in seqs:
        vf = inp.v[b][:, heads][:, :, chans].to("cpu").float().numpy()
        ora.append(OQ.quant_v_fp8(vf, amax=amax) if wl.v_format == "fp8" else OQ.quant_v_mxfp4(vf))
    _compare_v_cache(codes, scales, ts, ora, wl.v_format, seqs, heads, chans)
    del inp
    torch.cuda.empty_cache()
