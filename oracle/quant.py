"""Quantizers of the oracle.  TEST INFRASTRUCTURE ONLY.

The pages ("Hardware-Aware FP4 FlashAttention-4", summary page, "What the
paper found") say only that Q and K stay in NVFP4, that P is MXFP4 E2M1 in
Direct-P, and that V is FP4 or FP8 (FP8 P/V is the stable training variant).
They print no recipe.  The readings below are the plain NVFP4 / OCP MX
conventions, written out step by step in float32 so that the GPU quantizers
can be required to match bit for bit.
"""

import numpy as np

from .formats import (e2m1_encode, e2m1_decode, e4m3_encode, e4m3_decode,
                      pack_nibbles, unpack_nibbles, e8m0_decode)

F32 = np.float32
FLT_MAX = np.finfo(np.float32).max
NVFP4_BLOCK = 16
MX_BLOCK = 32


def _enc_scale(amax, top):
    """float32 ``top / amax`` (``1`` when amax is 0), clamped to FLT_MAX when
    the quotient overflows (only for amax below ~7.9e-36)."""
    amax = F32(amax)
    if amax == 0:
        return F32(1.0)
    with np.errstate(over="ignore"):
        s = F32(F32(top) / amax)
    return F32(FLT_MAX) if not np.isfinite(s) else s


def quant_nvfp4(x, amax=None):
    """NVFP4 quantization of a tensor whose last axis is D (multiple of 16).

    Reading (the pages give the format name only):
      1. amax_t = max |x| over the whole tensor (one FP32 scale per tensor).
      2. S_enc = fl(2688 / amax_t) (2688 = 448 * 6), or 1 when amax_t = 0.
      3. g = fl(1 / S_enc) is the stored tensor scale.
      4. For each run of 16 consecutive elements along D: amax_b = max |x|,
         s = E4M3(fl(fl(amax_b / 6) * S_enc)).
      5. If s decodes to 0 every code of the block is 0; otherwise
         enc = fl(S_enc / s) and code_i = E2M1(fl(x_i * enc)).
    Dequantized value: E2M1(code) * E4M3(s) * g.

    Returns (codes_packed uint8 [..., D/2], scales uint8 [..., D/16], g float32).
    Element 2k of a row sits in the low nibble of byte k.

    ``amax`` lets a caller quantize a slice of a larger tensor: pass the max
    |x| of the whole tensor (step 1) and the rows of interest.
    """
    x = np.asarray(x, dtype=F32)
    D = x.shape[-1]
    assert D % NVFP4_BLOCK == 0
    lead = x.shape[:-1]
    xb = x.reshape(-1, D // NVFP4_BLOCK, NVFP4_BLOCK)
    if amax is None:
        amax = np.max(np.abs(xb)) if xb.size else 0.0
    amax_t = F32(amax)
    s_enc = _enc_scale(amax_t, 2688.0)
    g = F32(F32(1.0) / s_enc)
    amax_b = np.max(np.abs(xb), axis=-1) if xb.size else np.zeros(xb.shape[:-1], F32)
    s_f = (amax_b / F32(6.0)).astype(F32) * s_enc
    s_code = e4m3_encode(s_f.astype(F32))
    s_val = e4m3_decode(s_code).astype(F32)
    with np.errstate(divide="ignore"):
        enc = np.where(s_val > 0, s_enc / np.where(s_val > 0, s_val, F32(1)), F32(0)).astype(F32)
    y = (xb * enc[..., None]).astype(F32)
    codes = e2m1_encode(y)
    codes = np.where((s_val > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    codes = codes.reshape(lead + (D,))
    return pack_nibbles(codes), s_code.reshape(lead + (D // NVFP4_BLOCK,)), g


def quant_nvfp4_46(x, amax=None, return_choice=False, candidates=(6.0, 4.0)):
    """NVFP4 quantization with the Four Over Six adaptive block scale.

    The method is listed beside the arXiv entry of the pages' paper (arXiv
    listing 2609.04105v1, "Related papers": "Four Over Six: More Accurate
    NVFP4 Quantization with Adaptive Block Scaling"), abstract only: each
    block evaluates two scale factors, and for some blocks scaling the block
    maximum to the smaller FP4 value 4 instead of 6 represents the block
    better.  Reading taken (same float32 operation order as quant_nvfp4):
      1. amax_t as in quant_nvfp4; S_enc = fl(1792 / amax_t) (1792 = 448 * 4,
         so that a block scale that maps the block max to 4 still fits E4M3),
         or 1 when amax_t = 0; g = fl(1 / S_enc).
      2. For M in (6, 4): s_M = E4M3(fl(fl(amax_b / M) * S_enc)) and codes_M
         as step 5 of quant_nvfp4 with s_M.
      3. err_M = sum over the block's 16 elements, in element order, of
         fl(d * d) with d = fl(fl(x_i * S_enc) - E2M1(code_i) * s_M), summed
         in float32 from 0 (the squared error in units of g).
      4. The block keeps M = 4 when err_4 < err_6, else M = 6.
    Dequantized value: E2M1(code) * E4M3(s) * g, as for quant_nvfp4.

    Returns (codes_packed, scales, g) like quant_nvfp4 and, with
    ``return_choice``, a bool array [..., D/16] that is True where M = 4.
    ``candidates`` restricts the block maxima tried (one value forces it).
    """
    x = np.asarray(x, dtype=F32)
    D = x.shape[-1]
    assert D % NVFP4_BLOCK == 0
    lead = x.shape[:-1]
    xb = x.reshape(-1, D // NVFP4_BLOCK, NVFP4_BLOCK)
    if amax is None:
        amax = np.max(np.abs(xb)) if xb.size else 0.0
    s_enc = _enc_scale(F32(amax), 1792.0)
    g = F32(F32(1.0) / s_enc)
    amax_b = np.max(np.abs(xb), axis=-1) if xb.size else np.zeros(xb.shape[:-1], F32)
    xs = (xb * s_enc).astype(F32)
    cand = []
    for M in candidates:
        s_code = e4m3_encode(((amax_b / F32(M)).astype(F32) * s_enc).astype(F32))
        s_val = e4m3_decode(s_code).astype(F32)
        with np.errstate(divide="ignore"):
            enc = np.where(s_val > 0, s_enc / np.where(s_val > 0, s_val, F32(1)), F32(0)).astype(F32)
        codes = e2m1_encode((xb * enc[..., None]).astype(F32))
        codes = np.where((s_val > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
        q = (e2m1_decode(codes).astype(F32) * s_val[..., None]).astype(F32)
        d = (xs - q).astype(F32)
        sq = (d * d).astype(F32)
        err = np.zeros(xb.shape[:-1], F32)
        for i in range(NVFP4_BLOCK):
            err = (err + sq[..., i]).astype(F32)
        cand.append((s_code, codes, err))
    if len(cand) == 1:
        four = np.full(xb.shape[:-1], candidates[0] == 4.0)
        s_code, codes = cand[0][0], cand[0][1].reshape(lead + (D,))
    else:
        four = cand[1][2] < cand[0][2]
        s_code = np.where(four, cand[1][0], cand[0][0]).astype(np.uint8)
        codes = np.where(four[..., None], cand[1][1], cand[0][1]).astype(np.uint8).reshape(lead + (D,))
    out = (pack_nibbles(codes), s_code.reshape(lead + (D // NVFP4_BLOCK,)), g)
    if return_choice:
        return out + (four.reshape(lead + (D // NVFP4_BLOCK,)),)
    return out


def dequant_nvfp4_raw(codes_packed, scales):
    """E2M1(code) * E4M3(scale) without the tensor scale, float64 [..., D].

    Each value has at most 6 significant bits, so it is exact in float64 and
    any product of two of them is exact too."""
    c = unpack_nibbles(codes_packed)
    D = c.shape[-1]
    s = e4m3_decode(scales)
    return e2m1_decode(c) * np.repeat(s, NVFP4_BLOCK, axis=-1)[..., :D]


def dequant_nvfp4(codes_packed, scales, g):
    """Full NVFP4 dequantization E2M1(code) * E4M3(scale) * g, float64."""
    return dequant_nvfp4_raw(codes_packed, scales) * np.float64(g)


def quant_v_fp8(v, amax=None):
    """FP8 E4M3 V with one FP32 scale per tensor.

    Reading: enc = fl(448 / amax_v) (1 when amax_v = 0), stored scale
    s_v = fl(1 / enc), code = E4M3(fl(v * enc)); dequantized value
    E4M3(code) * s_v.  Returns (codes uint8 same shape as v, s_v float32).
    ``amax`` (max |v| of the whole tensor) allows quantizing a slice.
    """
    v = np.asarray(v, dtype=F32)
    if amax is None:
        amax = np.max(np.abs(v)) if v.size else 0.0
    amax = F32(amax)
    enc = _enc_scale(amax, 448.0)
    s_v = F32(F32(1.0) / enc)
    codes = e4m3_encode((v * enc).astype(F32))
    return codes, s_v


def dequant_v_fp8(codes, s_v):
    return e4m3_decode(codes) * np.float64(s_v)


def mx_block_exponent(amax):
    """OCP MX shared exponent for E2M1 elements:
    e = clamp(floor(log2(amax)) - 2, -127, 127), and -127 for an all-zero
    block (2 is the exponent of E2M1's largest normal, 6 = 1.5 * 2**2)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, k = np.frexp(amax)                    # amax = f * 2**k, f in [0.5, 1)
    e = k.astype(np.int64) - 1 - 2
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127)


def quant_v_mxfp4(v):
    """MXFP4 V for one sequence: v float [Nk, H, D].

    Blocks are 32 consecutive keys (aligned to key 0 of the sequence) for each
    (head, channel); the last block may be short.  Each block gets the OCP MX
    E8M0 exponent e (see :func:`mx_block_exponent`) and codes
    E2M1(v * 2**-e).  Returns (codes uint8 [Nk, H, D] one code per element,
    e8m0 uint8 [ceil(Nk/32), H, D]).
    """
    v = np.asarray(v, dtype=F32)
    Nk = v.shape[0]
    nblk = (Nk + MX_BLOCK - 1) // MX_BLOCK
    pad = nblk * MX_BLOCK - Nk
    vp = np.concatenate([v, np.zeros((pad,) + v.shape[1:], F32)], axis=0)
    vb = vp.reshape((nblk, MX_BLOCK) + v.shape[1:]).astype(np.float64)
    e = mx_block_exponent(np.max(np.abs(vb), axis=1))          # [nblk, H, D]
    codes = e2m1_encode(vb * np.ldexp(1.0, -e)[:, None])
    codes = codes.reshape((nblk * MX_BLOCK,) + v.shape[1:])[:Nk]
    return codes.astype(np.uint8), (e + 127).astype(np.uint8)


def dequant_v_mxfp4(codes, e8m0):
    Nk = codes.shape[0]
    s = np.repeat(e8m0_decode(e8m0), MX_BLOCK, axis=0)[:Nk]
    return e2m1_decode(codes) * s


def hadamard32(x):
    """Unnormalized 32-point Walsh-Hadamard transform of each block of 32
    consecutive elements along the last axis, in float32: the block rotation
    read from "Bridging the Gap Between Promise and Performance for
    Microscaling FP4 Quantization" (listed beside the arXiv entry of the
    pages' paper; abstract only: rotations within microscaling blocks before
    FP4 quantization).  H is the Sylvester matrix (entries +-1, H H^T = 32 I),
    so rotating both Q and K multiplies every Q.K by exactly 32.

    Fixed float32 order: stages of stride 1, 2, 4, 8, 16; in each, the pair
    (i, i + s) with bit s of i clear becomes (x_i + x_{i+s}, x_i - x_{i+s}).
    """
    x = np.asarray(x, dtype=F32)
    D = x.shape[-1]
    assert D % MX_BLOCK == 0
    y = x.reshape(x.shape[:-1] + (D // MX_BLOCK, MX_BLOCK)).copy()
    s = 1
    while s < MX_BLOCK:
        idx = np.array([i for i in range(MX_BLOCK) if not i & s])
        a, b = y[..., idx], y[..., idx + s]
        y[..., idx] = a + b                     # float32 + float32 -> float32, RNE
        y[..., idx + s] = a - b
        s *= 2
    return y.reshape(x.shape)


def quant_mxfp4(x, hadamard=False):
    """MXFP4 quantization along the last axis (D, a multiple of 32): the
    MX-native Q/K format, an opt-in alternative to NVFP4 whose blocks the
    gfx950 scaled matrix instruction can apply directly.

    The pages keep Q and K in NVFP4 ("Hardware-Aware FP4 FlashAttention-4",
    summary page, "What the paper found") and use MXFP4 -- E2M1 elements with
    one E8M0 exponent per 32 -- for P and V; this applies that same OCP MX
    rule to Q/K rows: per 32 consecutive elements along D,
    e = clamp(floor(log2 amax) - 2, -127, 127) (-127 for an all-zero block)
    and code = E2M1(x * 2**-e).  No tensor scale.

    With ``hadamard``, each 32-element block is first rotated by
    :func:`hadamard32` (float32), and the quantized values are those of the
    rotated rows.

    Returns (codes uint8 [..., D/2], element 2k in the low nibble of byte k;
    e8m0 uint8 [..., D/32]).
    """
    x = np.asarray(x, dtype=F32)
    if hadamard:
        x = hadamard32(x)
    D = x.shape[-1]
    assert D % MX_BLOCK == 0
    xb = x.reshape(x.shape[:-1] + (D // MX_BLOCK, MX_BLOCK)).astype(np.float64)
    e = mx_block_exponent(np.max(np.abs(xb), axis=-1))              # [..., D/32]
    codes = e2m1_encode(xb * np.ldexp(1.0, -e)[..., None])          # exact scaling by 2**-e
    codes = codes.reshape(x.shape).astype(np.uint8)
    return pack_nibbles(codes), (e + 127).astype(np.uint8)


def dequant_mxfp4(codes_packed, e8m0):
    """E2M1(code) * 2**e per 32-element block along the last axis, float64."""
    c = unpack_nibbles(codes_packed)
    s = np.repeat(e8m0_decode(e8m0), MX_BLOCK, axis=-1)
    return e2m1_decode(c) * s
