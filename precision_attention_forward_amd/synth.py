"""Seeded synthetic inputs shaped like the workloads of the Direct-P pages.

This module draws random numbers only; it holds none of the method's
arithmetic, so both the HIP path and the CPU oracle may take their inputs
from it.  Workloads (the pages use Wan2.1 video diffusion and a Llama-3.1-style
8B model; their weights, prompts and data are not available, so seeded
Gaussian tensors of the same shapes stand in for them):

  tiny      B=1, H=2, N=256, D=64, noncausal; MXFP4 P, FP8 V
  wan14b    B=1, H=40, N=32760, D=128, noncausal; Q, K with 4 of the 128
            channels scaled x8 (shared by Q and K and by every head);
            MXFP4 P, MXFP4 V
  wan_d64   B=1, H=80, N=16384, D=64, noncausal; same outlier recipe on 4 of
            64 channels; MXFP4 P, FP8 V
  llama8b   B=4, Hq=32, Hkv=8, N=8192, D=128, causal prefill; FP8 P and V
  varlen16  16 sequences, N_i ~ U{1024..65536}, packed with cu_seqlens,
            H=32, D=128, noncausal; 1% of token rows of Q and (independently)
            of K scaled x16; MXFP4 P, FP8 V
  llama8b_decode  a decode step of the Llama-3.1-style model: B=64
            sequences, Hq=32, Hkv=8, D=128, nq=1 new token per sequence
            against a KV cache of N=8192 keys; MXFP4 P, FP8 V (generate_decode)

Draw order for a seed: sequence lengths (varlen only), then Q, K, V as
float32 standard normals cast to bfloat16, then the outlier choice.
"""

from dataclasses import dataclass, field, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int                      # Nq = Nk (dense); ignored for varlen
    D: int
    causal: bool
    p_format: str               # "mxfp4" (Direct-P) or "fp8"
    v_format: str               # "fp8" or "mxfp4"
    outlier: Optional[tuple] = None   # ("channels", count, factor) | ("tokens", prob, factor)
    varlen: Optional[tuple] = None    # (num_seqs, min_len, max_len)
    seed: int = 0
    extra: dict = field(default_factory=dict)

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    1: Workload("tiny", 1, 2, 2, 256, 64, False, "mxfp4", "fp8", None, None, 1),
    2: Workload("wan14b", 1, 40, 40, 32760, 128, False, "mxfp4", "mxfp4",
                ("channels", 4, 8.0), None, 2),
    3: Workload("wan_d64", 1, 80, 80, 16384, 64, False, "mxfp4", "fp8",
                ("channels", 4, 8.0), None, 3),
    4: Workload("llama8b", 4, 32, 8, 8192, 128, True, "fp8", "fp8", None, None, 4),
    5: Workload("varlen16", 16, 32, 32, 0, 128, False, "mxfp4", "fp8",
                ("tokens", 0.01, 16.0), (16, 1024, 65536), 5),
    6: Workload("llama8b_decode", 64, 32, 8, 8192, 128, True, "mxfp4", "fp8", None, None, 6,
                {"nq": 1}),
}


@dataclass
class Inputs:
    wl: Workload
    q: torch.Tensor            # bf16 [B, N, Hq, D] or [T, Hq, D]
    k: torch.Tensor            # bf16 [B, N, Hkv, D] or [T, Hkv, D]
    v: torch.Tensor            # bf16 like k
    seqlens: Optional[torch.Tensor] = None      # int32 CPU [num_seqs] (varlen)
    cu_seqlens: Optional[torch.Tensor] = None   # int32 CPU [num_seqs + 1] (varlen)
    outlier_channels: Optional[torch.Tensor] = None

    @property
    def sigma(self):
        return 1.0 / float(self.wl.D) ** 0.5


def generate(wl: Workload, device="cpu") -> Inputs:
    """Draw the inputs of ``wl`` from ``torch.Generator(device)`` seeded with
    ``wl.seed``.  Values differ between devices (different generators)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    seqlens = cu = None
    if wl.varlen is not None:
        nseq, lo, hi = wl.varlen
        seqlens = torch.randint(lo, hi + 1, (nseq,), generator=gen, device=dev).to("cpu", torch.int32)
        cu = torch.zeros(nseq + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(seqlens, 0).to(torch.int32)
        qshape = (int(cu[-1]), wl.Hq, wl.D)
        kshape = (int(cu[-1]), wl.Hkv, wl.D)
    else:
        qshape = (wl.B, wl.N, wl.Hq, wl.D)
        kshape = (wl.B, wl.N, wl.Hkv, wl.D)

    def draw(shape):
        return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

    q = draw(qshape)
    k = draw(kshape)
    v = draw(kshape)
    chans = None
    if wl.outlier is not None:
        kind, amount, factor = wl.outlier
        if kind == "channels":
            chans = torch.randperm(wl.D, generator=gen, device=dev)[:amount]
            q[..., chans] = (q[..., chans].float() * factor).to(torch.bfloat16)
            k[..., chans] = (k[..., chans].float() * factor).to(torch.bfloat16)
        elif kind == "tokens":
            tok_shape = qshape[:-2]
            mq = torch.rand(tok_shape, generator=gen, device=dev) < amount
            mk = torch.rand(tok_shape, generator=gen, device=dev) < amount
            q[mq] = (q[mq].float() * factor).to(torch.bfloat16)
            k[mk] = (k[mk].float() * factor).to(torch.bfloat16)
        else:
            raise ValueError(kind)
    return Inputs(wl, q, k, v, seqlens, cu, chans)


@dataclass
class DecodeInputs:
    wl: Workload
    q: torch.Tensor            # bf16 [B, nq, Hq, D], the new tokens
    k: torch.Tensor            # bf16 [B, Hkv, N, D], head-major K cache
    v: torch.Tensor            # bf16 [B, N, Hkv, D], V cache
    seqlens: torch.Tensor      # int32 CPU [B], valid cache entries per sequence

    @property
    def sigma(self):
        return 1.0 / float(self.wl.D) ** 0.5


def generate_decode(wl: Workload, device="cpu") -> DecodeInputs:
    """Inputs of a decode step: ``wl.N`` is the cache capacity (whole
    128-key tiles), ``extra["nq"]``
    the new tokens per sequence and ``extra["ragged"]`` (optional) draws the
    valid lengths from U{1..N} instead of taking N for every sequence.
    Draw order: lengths (ragged only), then Q, K, V as float32 standard
    normals cast to bfloat16."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    nq = int(wl.extra.get("nq", 1))
    if wl.extra.get("ragged"):
        seqlens = torch.randint(1, wl.N + 1, (wl.B,), generator=gen, device=dev).to("cpu", torch.int32)
    else:
        seqlens = torch.full((wl.B,), wl.N, dtype=torch.int32)

    def draw(shape):
        return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

    q = draw((wl.B, nq, wl.Hq, wl.D))
    k = draw((wl.B, wl.Hkv, wl.N, wl.D))
    v = draw((wl.B, wl.N, wl.Hkv, wl.D))
    return DecodeInputs(wl, q, k, v, seqlens)


def decode_bytes(wl: Workload, seqlens) -> float:
    """Bytes a decode step must move at least: every valid cache entry once
    (NVFP4 K: D/2 + D/16 bytes per key and KV head; V: D bytes (FP8) or
    D/2 + D/32 (MXFP4)), the NVFP4 Q and the float32 O and LSE."""
    D = wl.D
    per_key = D / 2 + D / 16 + (D if wl.v_format == "fp8" else D / 2 + D / 32)
    keys = float(sum(int(n) for n in seqlens))
    nq = int(wl.extra.get("nq", 1))
    q = wl.B * nq * wl.Hq * (D / 2 + D / 16)
    o = wl.B * nq * wl.Hq * (4 * D + 4)
    return keys * wl.Hkv * per_key + q + o


def decode_flops(wl: Workload, seqlens) -> float:
    """4 * Hq * nq * D flops per valid cached key (2 D for Q.K and 2 D for
    P.V per query row).  The causal mask among the nq new tokens removes
    only nq (nq - 1) / 2 pairs per head; the kernel computes them anyway, so
    they are counted."""
    nq = int(wl.extra.get("nq", 1))
    return 4.0 * wl.Hq * nq * wl.D * float(sum(int(n) for n in seqlens))


def flops(wl: Workload, seqlens=None) -> float:
    """Attention flops counted as 4 * B * H * Nq * Nk * D, halved for causal."""
    if wl.varlen is not None:
        assert seqlens is not None
        tot = sum(int(n) * int(n) for n in seqlens)
        f = 4.0 * wl.Hq * wl.D * tot
    else:
        f = 4.0 * wl.B * wl.Hq * wl.N * wl.N * wl.D
    return f / 2 if wl.causal else f
