#!/usr/bin/env python3
"""Throughput of the Direct-P FP4 attention forward on one MI355X.

One step is the whole hot path over one batch of synthetic inputs already
resident in HBM: NVFP4 quantization of Q and K, quantization of V, and the
forward (Q/K expansion pre-pass + attention kernel).  Default workload: the
Wan2.1-14B-shaped video self-attention (B=1, H=40, N=32760, D=128,
noncausal, MXFP4 P and V).  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload 1..5]
  python bench.py --backward      causal-training backward (Llama-3.1-8B shape)
  python bench.py --backward --noncausal   the same shape without the causal mask
  python bench.py --decode        decode step against a resident KV cache
"""

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MXFP4_PEAK_TFLOPS = 10066.3        # MI355X dense MXFP4/MXFP6 MFMA peak
FP8_PEAK_TFLOPS = 5033.2
BF16_PEAK_TFLOPS = 2516.6


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=None,
                    help="1..5 (default 2: Wan2.1-14B shape; 4: Llama-3.1-8B shape with --backward)")
    ap.add_argument("--encoder", choices=("exact", "loglin"), default="exact",
                    help="probability encoder: exact (RNE of 2^y) or the exp-free log-linear cast")
    ap.add_argument("--four-six", action="store_true",
                    help="quantize Q and K with the Four Over Six adaptive block scale (attn_quant_nvfp4_46)")
    ap.add_argument("--qk", choices=("nvfp4", "mxfp4", "mxfp4_had"), default="nvfp4",
                    help="Q/K format: nvfp4 (the method's; Q.K^T on the FP16 MFMA, exact) or the opt-in "
                         "MX-native mxfp4 (E8M0 per 32 along D; Q.K^T on the scaled FP4 MFMA, "
                         "attn_fwd_directp_mxqk / attn_fwd_fp8pv_mxqk); mxfp4_had rotates each 32-element block "
                         "of Q and K by the Hadamard matrix first (attn_quant_mxfp4_had, softmax scale / 32)")
    ap.add_argument("--backward", action="store_true",
                    help="time the causal-training backward (attn_bwd_fp8) instead of the forward; its own JSON line")
    ap.add_argument("--noncausal", action="store_true",
                    help="with --backward: the same shape without the causal mask")
    ap.add_argument("--decode", action="store_true",
                    help="time a decode step (workload 6: new tokens against a resident NVFP4/FP8 KV cache); "
                         "its own JSON line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=16384, help="query rows of the oracle sample")
    ap.add_argument("--cpu-rows-bwd", type=int, default=8192, help="rows of the backward oracle sample")
    ap.add_argument("--cpu-seqs-dec", type=int, default=8, help="sequences of the decode oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (HBM counter calibration) and exit")
    ap.add_argument("--issue-rates", action="store_true",
                    help="print the per-instruction costs measured by the library's issue-rate micro-kernels")
    ap.add_argument("--phase-trace", action="store_true",
                    help="run the Wan-shape forward on the phase-trace library (libattnfp4_trace.so, built by "
                         "`python -m precision_attention_forward_amd.build --phase-trace`) and print each wave's "
                         "shader-clock cycles per key-loop iteration in five phases, then exit")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="only time torch's bf16 and fp16 matrix products (n = 8192, 16384) on this GPU, the "
                         "vendor-library reference for the BF16 attention's matrix rate, and exit")
    return ap.parse_args()


# Sources the forward attention kernel is compiled from; a traffic figure
# measured by hardware counters is reported only while they are unchanged.
KERNEL_SOURCES = ["fwd_lowp.hip", "common.h", "pipeline.h", "fwd_params.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_lowp_kernel_hbm_traffic.md")
DEC_KERNEL_SOURCES = ["decode.hip", "common.h", "dec_params.h", "fwd_params.h", "pipeline.h"]
DEC_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_llama8b_decode.md")
HBM_PEAK_GBS = 8000.0


def kernel_source_hash(sources=None):
    import hashlib
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, "precision_attention_forward_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, path=TRAFFIC_FILE, sources=None, qk="nvfp4"):
    """HBM bytes per launch of the attention kernel for `workload` (and Q/K
    mode `qk`), from the counter summary (FETCH_SIZE + WRITE_SIZE, each scaled
    by the factor a plain copy of known size reads for the same counter), or
    None when there is no figure for this workload or the kernel sources
    changed since it was taken."""
    if not os.path.exists(path):
        return None
    src = kernel_source_hash(sources)
    for line in open(path):
        m = re.match(r"\s*traffic:\s+workload=(\d+)(?:\s+qk=(\w+))?\s+source=([0-9a-f]+)\s+bytes_per_launch=([0-9.eE+]+)",
                     line)
        if m and int(m.group(1)) == workload and (m.group(2) or "nvfp4") == qk and m.group(3) == src:
            return float(m.group(4))
    return None


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "launches": 3}), flush=True)


def gemm_reference():
    """Square bf16 / fp16 products through torch (the vendor BLAS): the
    matrix rate a plain library GEMM reaches on this GPU, printed as one JSON
    line per (dtype, n)."""
    import torch
    torch.manual_seed(0)
    for dt in (torch.bfloat16, torch.float16):
        for n in (8192, 16384):
            a = torch.randn(n, n, device="cuda:0", dtype=dt)
            b = torch.randn(n, n, device="cuda:0", dtype=dt)
            for _ in range(3):
                c = a @ b
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            reps = 10 if n == 8192 else 4
            e0.record()
            for _ in range(reps):
                c = a @ b
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            print(json.dumps({"gemm": str(dt).replace("torch.", ""), "n": n, "ms": round(ms, 3),
                              "tflops": round(2 * n ** 3 / ms / 1e9, 1)}), flush=True)
            del a, b, c


PROBE_NAMES = ("v_fma_f32", "v_exp_f32", "v_med3_f32", "v_cvt_scalef32_pk_fp8_f32 (two values)", "v_max3_f32",
               "v_mfma_f32_32x32x16_bf16", "v_mfma_scale_f32_32x32x64_f8f6f4 FP8", "v_mfma_scale_f32_32x32x64_f8f6f4 FP4",
               "bf16 MFMA wave + v_fma_f32 wave", "bf16 MFMA wave + v_exp_f32 wave",
               "2 v_fma_f32 per MFMA, two waves", "4 v_fma_f32 per MFMA, two waves", "8 v_fma_f32 per MFMA, two waves",
               "ds_read_b128", "ds_read_b64", "ds_read_b64_tr_b16", "ds_write_b128", "ds_write_b32",
               "v_cvt_scalef32_pk_fp4_f32 (two values)",
               "v_exp_f32 + 1 v_fma_f32", "v_exp_f32 + 3 v_fma_f32", "v_exp_f32 + 1 v_max3_f32",
               "v_exp_f32 + 1 v_cvt_scalef32_pk_fp4_f32", "4 v_exp_f32 + 4 v_fma_f32 (per 4 steps)",
               "v_fma_f32, four waves per SIMD", "8 v_fma_f32 per MFMA, four waves", "16 v_fma_f32 per MFMA, two waves",
               "bf16 MFMA wave + 3x v_fma_f32 wave", "bf16 MFMA wave + 4x v_fma_f32 wave",
               "bf16 MFMA wave + 2x v_exp_f32 wave",
               "forward tile mix, interleaved", "forward tile mix, ping-pong with barriers",
               "forward tile mix, encode chains in one slot", "forward tile mix, encode chains over three slots")


def issue_rates():
    """The library's issue-rate micro-kernels (attn_probe_issue_rates): one
    JSON line per kind with cycles per instruction per SIMD, or bytes per
    clock per CU for the LDS kinds; for the MFMA + vector kinds, the time
    relative to the MFMA issue alone (32 cycles per bf16 32x32x16); for the
    exponential + other kinds, cycles per step (one exponential and its
    partners) per SIMD."""
    import torch  # noqa: F401
    import precision_attention_forward_amd as paf
    n = paf.load_library().attn_probe_kinds()
    assert n == len(PROBE_NAMES), (n, len(PROBE_NAMES))
    for kind in range(n):
        paf.probe_issue_rates(kind)                      # warm-up (clocks, code load)
        cyc, units, grid = paf.probe_issue_rates(kind)
        line = {"probe": kind, "what": PROBE_NAMES[kind], "cycles_per_workgroup": round(cyc)}
        if 13 <= kind <= 17:
            line["bytes_per_clock_per_cu"] = round(units / cyc, 1)
        elif 19 <= kind <= 23:
            line["cycles_per_exp_step_per_simd"] = round(cyc / units, 2)
        elif 8 <= kind <= 12 or 25 <= kind <= 29:
            line["mfma_per_simd"] = units
            line["time_over_mfma_alone"] = round(cyc / (32.0 * units), 3)
        elif kind >= 30:
            line["cycles_per_wave_tile_per_simd"] = round(cyc / units, 1)
            line["time_over_mfma_alone"] = round(cyc / units / (42 * 32.0), 3)
        else:
            line["cycles_per_instruction_per_simd"] = round(cyc / units, 2)
        print(json.dumps(line), flush=True)


PHASE_NAMES = ("before the slots", "slots 0-9 (P.V, statistics)", "slots 10-25 (S sub-tiles 0-1)",
               "slots 26-41 (S sub-tiles 2-3; waves 4-7's barrier)", "after the slots (waves 0-3's barrier)")


def phase_trace(steps=5):
    """The forward attention kernel's key-loop phases on the Wan shape
    (workload 2, MXFP4 P / MXFP4 V, NVFP4 Q/K): the diagnostic library's
    workgroup 0 records, per wave, the shader-clock cycles spent in each phase
    summed over its iterations (see the phase trace in csrc/fwd_lowp.hip).
    Prints one JSON line per wave (cycles per iteration) and a summary line
    with the call time, which includes the stamps' own cost."""
    import ctypes
    import numpy as np
    import torch
    import precision_attention_forward_amd as paf
    from precision_attention_forward_amd import synth
    from precision_attention_forward_amd.build import TRACE_LIB
    if not os.path.exists(TRACE_LIB):
        print(f"{TRACE_LIB} is missing: build it with `python -m precision_attention_forward_amd.build --phase-trace`",
              file=sys.stderr)
        sys.exit(2)
    lib = paf.load_library(TRACE_LIB)
    lib.attn_fwd_phase_trace_read.restype = ctypes.c_int
    lib.attn_fwd_phase_trace_read.argtypes = [ctypes.c_void_p]
    wl = synth.WORKLOADS[2]
    inp = synth.generate(wl, "cuda")
    q, k = paf.quant_nvfp4(inp.q), paf.quant_nvfp4(inp.k)
    vq = paf.quant_v(inp.v, paf.V_MXFP4)
    v = (paf.V_MXFP4, vq[0], vq[1], vq[2])
    kw = dict(Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, softmax_scale=inp.sigma, causal=False, out_dtype=torch.bfloat16,
              B=1, Nq=wl.N, Nk=wl.N)
    ws = paf.Workspace()
    o, lse, _ = paf.fwd_directp(q, k, v, workspace=ws, **kw)
    for _ in range(2):
        paf.fwd_directp(q, k, v, workspace=ws, out=(o, lse), **kw)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        paf.fwd_directp(q, k, v, workspace=ws, out=(o, lse), **kw)
    ev1.record()
    torch.cuda.synchronize()
    buf = np.zeros((8, 8), dtype=np.uint64)
    st = lib.attn_fwd_phase_trace_read(buf.ctypes.data_as(ctypes.c_void_p))
    if st != 0:
        raise RuntimeError(f"attn_fwd_phase_trace_read failed: hip error {st}")
    totals = []
    for w in range(8):
        iters = int(buf[w, 5]) + 1                   # the key loop runs n_tiles + 1 iterations
        per = [float(buf[w, j]) / iters for j in range(5)]
        totals.append(sum(per))
        print(json.dumps({"wave": w, "iterations": iters,
                          "cycles_per_iteration": {n: round(x, 1) for n, x in zip(PHASE_NAMES, per)},
                          "total": round(sum(per), 1)}), flush=True)
    print(json.dumps({"phase_trace": "fwd_lowp_kernel wan14b (MXFP4 P, MXFP4 V, NVFP4 Q/K)",
                      "call_ms_with_stamps": round(ev0.elapsed_time(ev1) / steps, 4),
                      "cycles_per_iteration_mean": round(sum(totals) / 8, 1)}), flush=True)


def cpu_baseline(inp, rows, encoder="exact", four_six=False, qk="nvfp4"):
    """Time the CPU oracle (as it stands) on a bounded sample: one (batch,
    head), `rows` query rows against all keys, including the sample's
    quantization.  Returns a dict for the JSON line."""
    import numpy as np
    from oracle import attention as OA, quant as OQ
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    wl = inp.wl
    if inp.cu_seqlens is None:
        Nk = wl.N
        qh, kh, vh = inp.q[0, :, 0], inp.k[0, :, 0], inp.v[0, :, 0]
    else:
        s = int(np.argmax(inp.seqlens))
        t0, Nk = int(inp.cu_seqlens[s]), int(inp.seqlens[s])
        qh, kh, vh = inp.q[t0:t0 + Nk, 0], inp.k[t0:t0 + Nk, 0], inp.v[t0:t0 + Nk, 0]
    R = min(rows, qh.shape[0])
    idx = np.linspace(0, qh.shape[0] - 1, R).astype(np.int64)
    qf = qh.float().cpu().numpy()[idx]
    kf = kh.float().cpu().numpy()
    vf = vh.float().cpu().numpy()
    t = time.perf_counter()
    sigma = inp.sigma
    if qk in ("mxfp4", "mxfp4_had"):
        had = qk == "mxfp4_had"
        qc, qe = OQ.quant_mxfp4(qf, hadamard=had)
        kc, ke = OQ.quant_mxfp4(kf, hadamard=had)
        q_raw, k_raw, gq, gk = OQ.dequant_mxfp4(qc, qe), OQ.dequant_mxfp4(kc, ke), 1.0, 1.0
        sigma = sigma / 32.0 if had else sigma
    else:
        qfn = OQ.quant_nvfp4_46 if four_six else OQ.quant_nvfp4
        qc, qs, gq = qfn(qf)
        kc, ks, gk = qfn(kf)
        q_raw, k_raw = OQ.dequant_nvfp4_raw(qc, qs), OQ.dequant_nvfp4_raw(kc, ks)
    if wl.v_format == "fp8":
        vcodes, s_v = OQ.quant_v_fp8(vf)
        vhat = OQ.dequant_v_fp8(vcodes, s_v)
    else:
        vcodes, ve = OQ.quant_v_mxfp4(vf[:, None, :])
        vhat = OQ.dequant_v_mxfp4(vcodes, ve)[:, 0, :]
    OA.attn_lowp_head(q_raw, k_raw, gq, gk, vhat, sigma, wl.p_format, wl.causal, q_index=idx, encoder=encoder)
    dt = time.perf_counter() - t
    live = sum(min(int(i) + 1, Nk) for i in idx) if wl.causal else R * Nk
    flops = 4.0 * live * wl.D
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"1 head, {R} query rows x {Nk} keys of workload {wl.name} ({qk.upper()}/V quantization of the "
                      f"sample included), {dt:.1f} s; numpy float64, BLAS threads = cores"}


def accuracy_sample(inp, o, lse, rows=64):
    """Error of the low-precision forward against softmax attention computed
    in float64 on the unquantized (bf16) inputs, for `rows` evenly spaced
    query rows of head 0 of the first batch entry (the longest sequence of a
    packed batch), all keys.  Not the parity check (that compares with the
    oracle); this measures what the quantized path costs in accuracy."""
    import numpy as np
    wl = inp.wl
    if inp.cu_seqlens is None:
        t0, L = 0, wl.N
        qh, kh, vh = inp.q[0, :, 0], inp.k[0, :, 0], inp.v[0, :, 0]
        og, lg = o[0, :, 0], lse[0, 0]
    else:
        s = int(np.argmax(inp.seqlens))
        t0, L = int(inp.cu_seqlens[s]), int(inp.seqlens[s])
        qh, kh, vh = inp.q[t0:t0 + L, 0], inp.k[t0:t0 + L, 0], inp.v[t0:t0 + L, 0]
        og, lg = o[t0:t0 + L, 0], lse[0, t0:t0 + L]
    idx = np.linspace(0, L - 1, min(rows, L)).astype(np.int64)
    q = qh.float().cpu().numpy().astype(np.float64)[idx]
    k = kh.float().cpu().numpy().astype(np.float64)
    v = vh.float().cpu().numpy().astype(np.float64)
    sc = inp.sigma * (q @ k.T)
    if wl.causal:
        sc = np.where(np.arange(L)[None, :] <= idx[:, None], sc, -np.inf)
    mx = sc.max(axis=1, keepdims=True)
    p = np.exp(sc - mx)
    den = p.sum(axis=1, keepdims=True)
    o_ref = (p @ v) / den
    lse_ref = (mx + np.log(den))[:, 0]
    got = og.float().cpu().numpy()[idx].astype(np.float64)
    lse_got = lg.float().cpu().numpy()[idx].astype(np.float64)
    return {"o_rel_l2_vs_softmax": float(np.linalg.norm(got - o_ref) / np.linalg.norm(o_ref)),
            "lse_max_abs_vs_softmax": float(np.abs(lse_got - lse_ref).max()),
            "sample": f"{len(idx)} evenly spaced query rows of head 0, all {L} keys; float64 softmax attention "
                      "on the bf16 inputs"}


class HipEvents:
    """Raw hipEvent_t pairs (the library records them itself, so torch's
    Event bookkeeping does not apply)."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(a)) == 0 and self.hip.hipEventCreate(ctypes.byref(b)) == 0
            self.pairs.append((a, b))

    def handles(self, i):
        class _E:
            def __init__(self, h):
                self.cuda_event = h.value
        return (_E(self.pairs[i][0]), _E(self.pairs[i][1]))

    def times_ms(self):
        ms = self.ct.c_float()
        out = []
        for a, b in self.pairs:
            assert self.hip.hipEventSynchronize(b) == 0
            assert self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) == 0
            out.append(ms.value)
        return out

    def mean_ms(self):
        t = self.times_ms()
        return sum(t) / len(t)

    def median_ms(self):
        t = sorted(self.times_ms())
        n = len(t)
        return t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])


def cpu_baseline_bwd(inp, dout, o, lse, rows):
    """The oracle backward (as it stands) on a bounded sample: one (batch,
    head), ``rows`` query rows of dQ and ``rows`` key rows of dK/dV, including
    the quantization of the head.  Returns a dict for the JSON line."""
    import numpy as np
    from oracle import backward as OB, quant as OQ
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    wl = inp.wl
    N = wl.N
    qf = inp.q[0, :, 0].float().cpu().numpy()
    kf = inp.k[0, :, 0].float().cpu().numpy()
    vf = inp.v[0, :, 0].float().cpu().numpy()
    df = dout[0, :, 0].float().cpu().numpy()
    of = o[0, :, 0].float().cpu().numpy()
    lf = lse[0, 0].float().cpu().numpy()
    R = min(rows, N)
    idx = np.linspace(0, N - 1, R).astype(np.int64)
    t = time.perf_counter()
    qc, qs, gq = OQ.quant_nvfp4(qf)
    kc, ks, gk = OQ.quant_nvfp4(kf)
    vcodes, s_v = OQ.quant_v_fp8(vf)
    dcodes, s_do = OB.quant_do_e5m2(df)
    OB.attn_bwd_head(OQ.dequant_nvfp4_raw(qc, qs), OQ.dequant_nvfp4_raw(kc, ks), gq, gk, OQ.dequant_v_fp8(vcodes, s_v),
                     of, OB.dequant_do_e5m2(dcodes, s_do), lf, inp.sigma, wl.causal, q_rows=idx, k_rows=idx)
    dt = time.perf_counter() - t
    # algorithmic work of the sample: dQ rows see their visible keys, dK/dV rows their visible queries
    vis_q = sum(min(int(i) + 1, N) for i in idx) if wl.causal else R * N
    vis_k = sum(N - int(j) for j in idx) if wl.causal else R * N
    flops = 2.0 * wl.D * (3 * vis_q + 4 * vis_k)   # dQ rows: S, dP, dQ; dK/dV rows: S, dP, dV, dK
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"1 head, {R} dQ rows and {R} dK/dV rows of workload {wl.name} (quantization of the head "
                      f"included), {dt:.1f} s; numpy float64, BLAS threads = cores"}


def backward_main(args, torch, paf, synth):
    """One step = attn_bwd_fp8 on resident forward outputs (quantized Q/K/V,
    O, LSE) and dO.  Flops: 5 matrix products of 2 N^2 D per (batch, head),
    halved for causal (the usual backward count, 2.5x the forward's)."""
    wl = synth.WORKLOADS[args.workload]
    if args.noncausal:
        wl = wl.with_(causal=False)
    if wl.varlen is not None:
        print("the backward takes dense batches only", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.generate(wl, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed + 7)
    dout = torch.randn(inp.q.shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    q = paf.quant_nvfp4(inp.q)
    k = paf.quant_nvfp4(inp.k)
    vc, vs, vt, _ = paf.quant_v(inp.v, paf.V_FP8)
    v = (paf.V_FP8, vc, None, vt)
    B, N, Hq, D = inp.q.shape
    Hkv = inp.k.shape[2]
    o, lse, _ = paf.fwd_fp8pv(q, k, v, Hq=Hq, Hkv=Hkv, D=D, softmax_scale=inp.sigma, causal=wl.causal, B=B, Nq=N,
                              Nk=N, out_dtype=torch.bfloat16)
    ws = paf.Workspace()
    kev = HipEvents(args.steps)
    flops = 2.5 * synth.flops(wl)

    def step(i=None):
        return paf.bwd_fp8(q, k, v, o, lse, dout, softmax_scale=inp.sigma, causal=wl.causal, workspace=ws,
                           events=None if i is None else kev.handles(i))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    a.record()
    for i in range(args.steps):
        step(i)
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = a.elapsed_time(b) / args.steps
    kern_ms = kev.mean_ms()
    kern_median_ms = kev.median_ms()
    value = flops / (ms * 1e-3) / 1e12
    kern_tflops = flops / (kern_ms * 1e-3) / 1e12
    # three of the five products run on the bf16 MFMA (S, dK, dQ: NVFP4 values need 6 bits), two on FP8 (dP, dV)
    ceiling = 1.0 / (0.6 / BF16_PEAK_TFLOPS + 0.4 / FP8_PEAK_TFLOPS)
    cpu = None if args.no_cpu_baseline else cpu_baseline_bwd(inp, dout, o, lse, args.cpu_rows_bwd)
    out = {
        "metric": "attn bwd (causal training path, FP8 gradient operands) TFLOP/s on 1 MI355X",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8+bf16", "data": "synthetic (seeded Gaussian, the workload's recipe)",
        "config": {"workload": f"{wl.name}: B={B} N={N} Hq={Hq} Hkv={Hkv} D={D} "
                               f"{'causal' if wl.causal else 'noncausal'}, backward of the FP8-P/V forward",
                   "B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "D": D, "causal": wl.causal, "flops_per_step": flops,
                   "parallelism": "single GPU"},
        "bwd_kernels_tflops": round(kern_tflops, 2),
        "bwd_kernels_ms": {"mean": round(kern_ms, 4), "median": round(kern_median_ms, 4)},
        "prep_ms": round(ms - kern_ms, 4),
        "precision": "NVFP4 Q/K (exact values on the bf16 MFMA), E5M2 dO, FP8 E4M3 V, MX E4M3 P~ and dS~, "
                     "FP32 accumulation",
        "roofline": {"bound": "mfma", "achieved": round(kern_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(kern_tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "bwd_dkdv_kernel + bwd_dq_kernel", "kernel_ms": round(kern_ms, 4),
                     "mixed_ceiling_tflops": round(ceiling, 1), "frac_of_mixed_ceiling": round(kern_tflops / ceiling, 4)},
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_dec(inp, seqs):
    """The oracle (as it stands) on a bounded sample of a decode step: every
    head of the first ``seqs`` sequences, including the quantization of their
    cache.  Value in GB/s of cache entries processed (the metric's unit)."""
    import numpy as np
    from oracle import attention as OA, quant as OQ
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    wl = inp.wl
    nq = inp.q.shape[1]
    G = wl.Hq // wl.Hkv
    S = min(seqs, wl.B)
    amax_q = float(inp.q.abs().max())
    amax_k = float(inp.k.abs().max())
    amax_v = float(inp.v.abs().max())
    qf = inp.q[:S].float().cpu().numpy()
    kf = inp.k[:S].float().cpu().numpy()
    vf = inp.v[:S].float().cpu().numpy()
    keys = 0
    t = time.perf_counter()
    for b in range(S):
        L = int(inp.seqlens[b])
        keys += L
        q_index = (L - nq + np.arange(nq)) if wl.causal else None
        for hk in range(wl.Hkv):
            kc, ks, gk = OQ.quant_nvfp4(kf[b, hk, :L], amax=amax_k)
            vcodes, s_v = OQ.quant_v_fp8(vf[b, :, hk], amax=amax_v)
            vhat = OQ.dequant_v_fp8(vcodes, s_v)[:L]
            kraw = OQ.dequant_nvfp4_raw(kc, ks)
            for h in range(hk * G, hk * G + G):
                qc, qs, gq = OQ.quant_nvfp4(qf[b, :, h], amax=amax_q)
                OA.attn_lowp_head(OQ.dequant_nvfp4_raw(qc, qs), kraw, gq, gk, vhat, inp.sigma, wl.p_format,
                                  wl.causal, q_index=q_index)
    dt = time.perf_counter() - t
    from precision_attention_forward_amd import synth
    by = synth.decode_bytes(wl.with_(B=S), inp.seqlens[:S])
    return {"value": by / dt / 1e9, "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"all {wl.Hq} heads of the first {S} sequences of workload {wl.name} ({keys} cached keys "
                      f"per head; quantization of their cache included), {dt:.1f} s; numpy float64, "
                      f"BLAS threads = cores"}


def decode_main(args, torch, paf, synth):
    """One step = NVFP4 quantization of the new tokens' Q and the decode
    kernel against the resident quantized KV cache (written once, as a
    prefill leaves it).  The metric is bandwidth: the bytes a decode step must
    move at least (every valid cache entry once, Q, O, LSE) per second."""
    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.generate_decode(wl, dev)
    nq = inp.q.shape[1]
    k = paf.quant_nvfp4(inp.k)
    vf = paf.V_FP8 if wl.v_format == "fp8" else paf.V_MXFP4
    vq = paf.quant_v_cache(inp.v, vf)
    v = (vf, vq[0], vq[1], vq[2])
    seqlens = inp.seqlens.to(dev)
    fn = paf.decode_directp if wl.p_format == "mxfp4" else paf.decode_fp8pv
    kw = dict(B=wl.B, Hq=wl.Hq, Hkv=wl.Hkv, nq=nq, Nk=wl.N, D=wl.D, softmax_scale=inp.sigma, causal=wl.causal,
              seqlens_k=seqlens)
    q = paf.quant_nvfp4(inp.q)
    out = fn(q, k, v, **kw)[:2]
    kev = HipEvents(args.steps)

    def step(i=None):
        qq = paf.quant_nvfp4(inp.q)
        return fn(qq, k, v, out=out, events=None if i is None else kev.handles(i), **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    a.record()
    for i in range(args.steps):
        step(i)
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = a.elapsed_time(b) / args.steps
    # the kernel alone: back-to-back launches between two events (the
    # per-call events above also hold the gap before each launch, which is a
    # few percent of a 0.2 ms kernel)
    q = paf.quant_nvfp4(inp.q)
    torch.cuda.synchronize()
    a.record()
    for i in range(args.steps):
        fn(q, k, v, out=out, **kw)
    b.record()
    torch.cuda.synchronize()
    kern_ms = a.elapsed_time(b) / args.steps
    call_ms = kev.mean_ms()
    by = synth.decode_bytes(wl, inp.seqlens)
    fl = synth.decode_flops(wl, inp.seqlens)
    value = by / (ms * 1e-3) / 1e9
    kern_gbs = by / (kern_ms * 1e-3) / 1e9
    traffic = measured_traffic(args.workload, DEC_TRAFFIC_FILE, DEC_KERNEL_SOURCES)
    cpu = None if args.no_cpu_baseline else cpu_baseline_dec(inp, args.cpu_seqs_dec)
    pf = "MXFP4 P (Direct-P)" if wl.p_format == "mxfp4" else "FP8 E4M3 P"
    vfn = "FP8 E4M3 V" if wl.v_format == "fp8" else "MXFP4 V"
    out_line = {
        "metric": "Direct-P decode attention bandwidth (KV cache + Q + O bytes per second) on 1 MI355X",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4+fp8", "data": "synthetic (seeded Gaussian Q, K cache and V cache)",
        "config": {"workload": f"{wl.name}: B={wl.B} sequences x {nq} new token(s), Hq={wl.Hq} Hkv={wl.Hkv} "
                               f"D={wl.D}, {wl.N} cached keys each; NVFP4 Q/K, {pf}, {vfn}",
                   "B": wl.B, "nq": nq, "Hq": wl.Hq, "Hkv": wl.Hkv, "cached_keys": wl.N, "D": wl.D,
                   "bytes_per_step": by, "flops_per_step": fl, "parallelism": "single GPU"},
        "kernel_tflops": round(fl / (kern_ms * 1e-3) / 1e12, 2),
        "kernel_call_ms": round(call_ms, 4),
        "q_quant_ms": round(ms - call_ms, 4),
        "roofline": {"bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "decode_kernel", "kernel_ms": round(kern_ms, 4)},
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out_line), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.issue_rates:
        issue_rates()
        return
    if args.gemm_reference:
        gemm_reference()
        return
    if args.phase_trace:
        phase_trace()
        return
    import torch
    import precision_attention_forward_amd as paf
    from precision_attention_forward_amd import synth

    paf.load_library()
    if args.workload is None:
        args.workload = 6 if args.decode else (4 if args.backward else 2)
    if args.decode:
        if "nq" not in synth.WORKLOADS[args.workload].extra:
            print("--decode takes a decode workload (6)", file=sys.stderr)
            sys.exit(2)
        decode_main(args, torch, paf, synth)
        return
    if "nq" in synth.WORKLOADS[args.workload].extra:
        print(f"workload {args.workload} is a decode step: use --decode", file=sys.stderr)
        sys.exit(2)
    if args.backward:
        backward_main(args, torch, paf, synth)
        return
    wl = synth.WORKLOADS[args.workload]
    mxqk = args.qk in ("mxfp4", "mxfp4_had")
    had = args.qk == "mxfp4_had"
    if mxqk and args.four_six:
        print("--qk mxfp4 takes no Four Over Six", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.generate(wl, dev)
    varlen = inp.cu_seqlens is not None
    vfmt = paf.V_FP8 if wl.v_format == "fp8" else paf.V_MXFP4
    fwd = {("mxfp4", "exact"): paf.fwd_directp, ("fp8", "exact"): paf.fwd_fp8pv,
           ("mxfp4", "loglin"): paf.fwd_directp_efq, ("fp8", "loglin"): paf.fwd_fp8pv_cast}[(wl.p_format,
                                                                                          args.encoder)]
    if mxqk:
        fwd = {("mxfp4", "exact"): paf.fwd_directp_mxqk, ("fp8", "exact"): paf.fwd_fp8pv_mxqk,
               ("mxfp4", "loglin"): paf.fwd_directp_efq_mxqk,
               ("fp8", "loglin"): paf.fwd_fp8pv_cast_mxqk}[(wl.p_format, args.encoder)]
    # (Q and K rotated alike by the 32-point Hadamard matrix: every Q.K is 32 times the original)
    kw = dict(Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, softmax_scale=inp.sigma / 32.0 if had else inp.sigma, causal=wl.causal,
              out_dtype=torch.bfloat16)
    if varlen:
        cu = inp.cu_seqlens.to(dev)
        mx = int(inp.seqlens.max())
        kw.update(cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=mx, max_seqlen_k=mx)
    else:
        kw.update(B=wl.B, Nq=wl.N, Nk=wl.N)
    flops = synth.flops(wl, inp.seqlens)
    ws = paf.Workspace()
    kev = HipEvents(args.steps)

    def quantize():
        if mxqk:
            q, k = paf.quant_mxfp4(inp.q, hadamard=had), paf.quant_mxfp4(inp.k, hadamard=had)
        else:
            q = paf.quant_nvfp4(inp.q, four_six=args.four_six)
            k = paf.quant_nvfp4(inp.k, four_six=args.four_six)
        if varlen:
            vc, vs, vt, _ = paf.quant_v(inp.v, vfmt, cu_seqlens=kw["cu_seqlens_k"], max_seqlen=kw["max_seqlen_k"])
        else:
            vc, vs, vt, _ = paf.quant_v(inp.v, vfmt)
        return q, k, (vfmt, vc, vs, vt)

    def step():
        q, k, v = quantize()
        return fwd(q, k, v, workspace=ws, **kw)

    def timed(fn, n):
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    for _ in range(args.warmup):
        step()
    # (1) the whole step: quantize Q, K, V + forward
    wall0 = time.perf_counter()
    ms_step = timed(lambda i: step(), args.steps)
    wall = time.perf_counter() - wall0
    value = flops / (ms_step * 1e-3) / 1e12
    # (2) the forward call alone on stored quantized operands, with HIP events
    #     around the attention kernel inside it (same stream)
    qkv = quantize()
    fwd_ms = timed(lambda i: fwd(*qkv, workspace=ws, events=kev.handles(i), **kw), args.steps)
    kern_ms = kev.mean_ms()
    kern_median_ms = kev.median_ms()
    fwd_tflops = flops / (fwd_ms * 1e-3) / 1e12
    kern_tflops = flops / (kern_ms * 1e-3) / 1e12
    o_out, lse_out, _ = fwd(*qkv, workspace=ws, **kw)
    acc = accuracy_sample(inp, o_out, lse_out)

    # the in-library BF16 forward on the same bf16 inputs (dense layouts only)
    bf16 = None
    if not args.no_bf16 and not varlen:
        for _ in range(2):
            paf.fwd_bf16(inp.q, inp.k, inp.v, inp.sigma, causal=wl.causal, want_lse=True)
        torch.cuda.synchronize()
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record()
        nb = max(3, args.steps // 2)
        for _ in range(nb):
            paf.fwd_bf16(inp.q, inp.k, inp.v, inp.sigma, causal=wl.causal, want_lse=True)
        b1.record()
        torch.cuda.synchronize()
        bf_ms = b0.elapsed_time(b1) / nb
        bf16 = {"ms": bf_ms, "tflops": flops / (bf_ms * 1e-3) / 1e12}

    # dominant kernel roofline: the attention kernel is MFMA bound
    pv_peak = MXFP4_PEAK_TFLOPS if wl.v_format == "mxfp4" else FP8_PEAK_TFLOPS
    # mixed ceiling: QK^T runs on the FP16 MFMA (exact NVFP4) or, MX-native, on the FP4 rate; P.V at the P/V
    # format rate
    qk_rate = MXFP4_PEAK_TFLOPS if mxqk else BF16_PEAK_TFLOPS
    pv_rate = pv_peak if wl.p_format == "mxfp4" else FP8_PEAK_TFLOPS
    ceiling = 1.0 / (0.5 / qk_rate + 0.5 / pv_rate)
    roofline = {"bound": "mfma", "achieved": round(kern_tflops, 2), "peak": MXFP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(kern_tflops / MXFP4_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(args.workload, qk=args.qk) if args.encoder == "exact" else None,
                "kernel": "fwd_lowp_kernel", "kernel_ms": round(kern_ms, 4),
                "mixed_ceiling_tflops": round(ceiling, 1), "frac_of_mixed_ceiling": round(kern_tflops / ceiling, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_rows, args.encoder, args.four_six, args.qk)

    cfg = {"workload": f"{wl.name}: " + (f"{wl.varlen[0]} packed sequences" if varlen else
                                         f"B={wl.B} N={wl.N}") +
           f" Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} {'causal' if wl.causal else 'noncausal'}, "
           f"P={wl.p_format.upper()} V={wl.v_format.upper()}" +
           ("" if args.encoder == "exact" else ", exp-free log-linear P encoder") +
           (", Four Over Six Q/K block scales" if args.four_six else "") +
           (", MX-native MXFP4 Q/K (opt-in)" if mxqk else "") +
           (" after a 32-point block Hadamard rotation" if had else ""),
           "encoder": args.encoder, "four_six": args.four_six, "qk": args.qk,
           "B": wl.B if not varlen else int(len(inp.seqlens)), "Hq": wl.Hq, "Hkv": wl.Hkv,
           "N": wl.N if not varlen else int(inp.seqlens.max()), "D": wl.D, "causal": wl.causal,
           "flops_per_step": flops, "parallelism": "single GPU"}
    out = {
        "metric": "Direct-P attn fwd TFLOP/s on 1 MI355X; % of MXFP4 MFMA peak; x BF16 attn",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4", "data": "synthetic (seeded Gaussian, the workload's outlier recipe)", "config": cfg,
        "fwd_call_tflops": round(fwd_tflops, 2),
        "fwd_kernel_tflops": round(kern_tflops, 2),
        "fwd_kernel_ms": {"mean": round(kern_ms, 4), "median": round(kern_median_ms, 4)},
        "quantize_ms": round(ms_step - fwd_ms, 4),
        "pct_mxfp4_peak": round(100 * value / MXFP4_PEAK_TFLOPS, 2),
        "pct_mxfp4_peak_fwd_call": round(100 * fwd_tflops / MXFP4_PEAK_TFLOPS, 2),
        "pct_mxfp4_peak_fwd_kernel": round(100 * kern_tflops / MXFP4_PEAK_TFLOPS, 2),
        "x_bf16": None if bf16 is None else round(fwd_tflops / bf16["tflops"], 3),
        "x_bf16_incl_quantize": None if bf16 is None else round(value / bf16["tflops"], 3),
        "bf16_tflops": None if bf16 is None else round(bf16["tflops"], 2),
        "precision": (("MX-native MXFP4 Q/K (E8M0 per 32 along D" +
                       ("; 32-point block Hadamard rotation first" if had else "") +
                       "; contracted on the scaled FP4 MFMA), ") if mxqk else
                      "NVFP4 Q/K (exact, contracted on the FP16 MFMA), ") +
                     ("MXFP4 E2M1 P (Direct-P)" if wl.p_format == "mxfp4" else "FP8 E4M3 P") +
                     ("" if args.encoder == "exact" else " by the exp-free log-linear cast") +
                     f", {wl.v_format.upper()} V, FP32 accumulation",
        "roofline": roofline,
        "accuracy": acc,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
