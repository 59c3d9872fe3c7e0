/*
 * attn_fp4.h -- C ABI of the MI355X (gfx950) Direct-P FP4 attention forward.
 *
 * The method is the one described on the pages "Hardware-Aware FP4
 * FlashAttention-4" (summary page, section "What the paper found"; arXiv
 * listing 2609.04105v1, abstract): Q and K stay in NVFP4, the row-max-shifted
 * log2 scores are mapped directly to MXFP4 E2M1 probability codes with one
 * E8M0 scale per 32 keys, the softmax denominator is summed from the same
 * rounded probabilities that the P.V product consumes, and a causal path
 * keeps FP8 E4M3 probabilities and values.  The forward saves the
 * log-sum-exp (LSE) per query row.
 *
 * Conventions shared by every entry point:
 *  - All pointers except `args` structs and `cu_seqlens_*_host` are DEVICE
 *    pointers on the current HIP device.  The caller owns every buffer; the
 *    library never allocates, frees or synchronizes, and keeps no state.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work; they return before the work finishes.
 *  - Arguments are validated on the host before any work is enqueued.  On
 *    any status other than ATTN_OK nothing has been enqueued and no output
 *    has been written.  Data-dependent conditions (NaN/Inf inputs, a
 *    cu_seqlens array that is not non-decreasing, lengths that disagree with
 *    the totals) are not detected and give unspecified outputs.
 *  - bf16 inputs are contiguous and row-major.  A "row" is the D values of
 *    one (token, head): dense tensors are [B, N, H, D], packed variable-length
 *    ("varlen") tensors are [T, H, D] with sequence s occupying tokens
 *    cu_seqlens[s] .. cu_seqlens[s+1]-1.
 *  - Minimum alignments: 16 bytes for every tensor pointer, 4 bytes for
 *    scalars.
 */
#ifndef ATTN_FP4_H
#define ATTN_FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, bad layout */
  ATTN_ERR_UNSUPPORTED = 2,      /* valid request this library does not implement */
  ATTN_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
  ATTN_ERR_HIP = 4               /* a HIP launch failed; see attn_last_hip_error() */
} attn_status;

typedef enum attn_v_format {
  ATTN_V_FP8_E4M3 = 0, /* E4M3 codes and one FP32 scale per tensor */
  ATTN_V_MXFP4 = 1     /* E2M1 codes and one E8M0 scale per (channel, 32 keys) */
} attn_v_format;

typedef enum attn_out_dtype {
  ATTN_OUT_BF16 = 0, /* O rounded to nearest-even bfloat16 */
  ATTN_OUT_F32 = 1   /* O in float32 */
} attn_out_dtype;

/* Human-readable name of a status code (static storage). */
const char* attn_status_str(attn_status s);
/* The hipError_t (as int) of the last ATTN_ERR_HIP in this thread, else 0. */
int attn_last_hip_error(void);
/* Library version string. */
const char* attn_version(void);

/* ------------------------------------------------------------------------
 * Quantization
 * --------------------------------------------------------------------- */

/* Bytes of device workspace every quantizer needs (a fixed, small size). */
size_t attn_quant_ws_bytes(void);

/*
 * NVFP4 quantization of Q or K (the pages keep "NVFP4 for Q and K": summary
 * page, "What the paper found").  x_bf16 is a [rows, D] bf16 matrix, D a
 * multiple of 16 (64 and 128 are what the forward accepts).
 *
 * Rule (one FP32 scale per tensor, one E4M3 scale per 16 consecutive
 * elements along D, every step an IEEE float32 operation rounded to nearest
 * even):
 *   amax_t = max |x| over the tensor
 *   S_enc  = 2688 / amax_t  (1 if amax_t == 0; FLT_MAX if the quotient overflows)
 *   g      = 1 / S_enc                                -> *tensor_scale
 *   per block: s = E4M3_sat((amax_b / 6) * S_enc)     -> scales
 *              code_i = E2M1_sat(x_i * (S_enc / s)), all 0 when s == 0
 * E2M1/E4M3 encoders round to nearest even, keep the sign (so -0 and values
 * that round to zero from below are code 8 / 0x80) and saturate.
 *
 * Outputs: codes [rows, D/2] (element 2k in the low nibble of byte k),
 * scales [rows, D/16] (E4M3 bytes), tensor_scale (one float).
 * ws: at least attn_quant_ws_bytes() bytes, no alignment beyond 16.
 * rows == 0 is valid and writes only *tensor_scale (= 1).
 */
attn_status attn_quant_nvfp4(const void* x_bf16, int64_t rows, int32_t D,
                             uint8_t* codes, uint8_t* scales, float* tensor_scale,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * NVFP4 quantization with the Four Over Six adaptive block scale, a related
 * method listed beside the arXiv entry of the pages' paper (2609.04105v1,
 * "Related papers": "Four Over Six: More Accurate NVFP4 Quantization with
 * Adaptive Block Scaling"; abstract only): each block evaluates two scale
 * factors, one mapping the block maximum to 6 and one mapping it to 4.
 * Reading implemented (float32, RNE, same order as attn_quant_nvfp4):
 *   S_enc = 1792 / amax_t   (448 * 4, so that both candidate scales fit E4M3)
 *   g     = 1 / S_enc                                -> *tensor_scale
 *   per block, for M in {6, 4}: s_M = E4M3_sat((amax_b / M) * S_enc),
 *     codes_M = E2M1_sat(x_i * (S_enc / s_M)) (all 0 when s_M == 0),
 *     err_M = sum over i = 0..15 in order of (x_i * S_enc - E2M1(code_i) * s_M)^2
 *   the block keeps M = 4 when err_4 < err_6, else M = 6.
 * The output format, arguments, workspace and errors are those of
 * attn_quant_nvfp4, so the forward entry points take its output unchanged.
 */
attn_status attn_quant_nvfp4_46(const void* x_bf16, int64_t rows, int32_t D,
                                uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * MXFP4 quantization of Q or K for the opt-in MX-native Q/K forward
 * (attn_fwd_directp_mxqk).  The pages keep Q and K in NVFP4 and use MXFP4 --
 * E2M1 elements with one E8M0 exponent per 32 -- for P and V (summary page,
 * "What the paper found"); this applies the same OCP MX rule along D so that
 * Q.K^T can run on gfx950's block-scaled FP4 matrix instruction, whose scales
 * are E8M0 per 32 elements (NVFP4's E4M3 scale per 16 is not one of them).
 *   per 32 consecutive elements along D: e = clamp(floor(log2 amax) - 2,
 *   -127, 127) (-127 when the block max is 0 or subnormal), code =
 *   E2M1_sat(x * 2^-e) rounded to nearest even (sign kept), byte = e + 127
 * x_bf16: [rows, D] bf16, D a multiple of 32 (the forward takes 64 and 128),
 * 16-byte aligned.  Outputs: codes [rows, D/2] (element 2k in the low nibble
 * of byte k, 16-byte aligned), scales [rows, D/32] E8M0 bytes.  No tensor
 * scale and no workspace.  rows == 0 is valid and writes nothing.
 * Errors: ATTN_ERR_INVALID_ARGUMENT (bad size, null or misaligned pointer),
 * ATTN_ERR_HIP.
 */
attn_status attn_quant_mxfp4(const void* x_bf16, int64_t rows, int32_t D,
                             uint8_t* codes, uint8_t* scales, void* stream);

/*
 * attn_quant_mxfp4 after a block rotation: each 32-element block of a row is
 * multiplied by the unnormalized 32-point Hadamard (Sylvester) matrix H
 * (entries +-1, H H^T = 32 I) before the MX rule above.  This is the
 * micro-rotation of "Bridging the Gap Between Promise and Performance for
 * Microscaling FP4 Quantization" (listed beside the pages' arXiv entry,
 * 2609.04105v1): it spreads an outlier channel over its block.  Every step
 * is a float32 operation in a fixed order: butterfly stages of stride 1, 2,
 * 4, 8, 16, where the pair (i, i + s) becomes (x_i + x_{i+s}, x_i - x_{i+s}).
 * Rotating Q and K alike multiplies every Q.K by 32, so the forward on the
 * result takes softmax_scale = sigma / 32.  Arguments, output format and
 * errors as for attn_quant_mxfp4.  Inputs whose rotated values overflow
 * float32 (|x| above about 1e37) give undefined codes.
 */
attn_status attn_quant_mxfp4_had(const void* x_bf16, int64_t rows, int32_t D,
                                 uint8_t* codes, uint8_t* scales, void* stream);

/*
 * Number of key columns of the transposed V layout used by attn_quant_v and
 * the forward.  Sequence s starts at column
 *     dense : s * roundup(Nk, 128)
 *     varlen: 128 * (cu_seqlens_k[s] / 128 + s)
 * and the columns past its end up to the next 128-multiple hold zeros.
 * dense (varlen == 0): B * roundup(Nk, 128); varlen: 128 * (ceil(total_k/128) + B).
 */
int64_t attn_v_cols(int32_t B, int32_t Nk, int64_t total_k, int32_t varlen);

/*
 * Quantize V (FP8 E4M3 or MXFP4; the pages pair FP4 or FP8 P with FP4 or FP8
 * V: summary page, "What the paper found") and transpose it so that keys are
 * contiguous, which is the operand order the P.V product reads.
 *   v_bf16 : [B, Nk, Hkv, D] (dense) or [total_k, Hkv, D] (varlen)
 *   cu_seqlens_k : device int32 [B+1] for varlen, NULL for dense
 *   FP8  : enc = fl(448 / amax_v) (1 if amax_v == 0), *tensor_scale =
 *          s_v = fl(1 / enc), code = E4M3_sat(fl(v * enc)), all float32 with
 *          round-to-nearest-even (the NVFP4 tensor scale's pattern; s_v is
 *          not fl(amax_v / 448): for amax_v = 49/32 that would be 7/2048,
 *          while fl(1 / fl(448 / amax_v)) is one ulp below it)
 *   MXFP4: per (head, channel, 32 keys from the start of the sequence):
 *          e = clamp(floor(log2 amax) - 2, -127, 127) (-127 if all zero),
 *          code = E2M1_sat(v * 2^-e), scale byte = e + 127
 * Outputs (cols = attn_v_cols(...)):
 *   codes : FP8 [Hkv, D, cols] bytes; MXFP4 [Hkv, D, cols/2] (key 2k in the
 *           low nibble of byte k)
 *   scales: MXFP4 only, [Hkv, D, cols/32] E8M0 bytes (may be NULL for FP8)
 *   tensor_scale: FP8 only (may be NULL for MXFP4)
 * Padding columns receive code 0 and (MXFP4) scale byte 0.
 */
attn_status attn_quant_v(const void* v_bf16, int32_t B, int32_t Nk, int32_t Hkv, int32_t D,
                         const int32_t* cu_seqlens_k, int64_t total_k, int32_t format,
                         uint8_t* codes, uint8_t* scales, float* tensor_scale,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * Quantize a decode step's V cache: the same codes, E8M0 bytes and FP8
 * tensor scale as attn_quant_v of the same dense tensor (summary page, "What
 * the paper found": FP4 or FP8 V), stored as the decode kernels read it
 * (the cached keys and values of the Colfax Research feed's post on
 * FlashAttention-4 decode): one block of D key-contiguous rows per
 * (sequence, KV head, 128-key tile), the tiles of one (sequence, head) in
 * order, so that every tile is one contiguous read.
 *   v_bf16 : dense [B, Nk, Hkv, D]; Nk is the cache capacity, a multiple of
 *            128 (ATTN_ERR_INVALID_ARGUMENT otherwise)
 * Outputs, with t = (b * Hkv + h) * (Nk / 128) + key / 128 and j = key % 128:
 *   FP8  : codes [B, Hkv, Nk/128, D, 128]: code of (b, key, h, d) at byte
 *          (t * D + d) * 128 + j; tensor_scale as attn_quant_v
 *   MXFP4: codes [B, Hkv, Nk/128, D, 64]: byte (t * D + d) * 64 + j / 2, key
 *          j even in the low nibble; scales [B, Hkv, Nk/128, D, 4]: E8M0 of
 *          keys 32 i .. 32 i + 31 of the tile at byte (t * D + d) * 4 + i
 * ws as attn_quant_v (attn_quant_ws_bytes()).  Nothing is read past the
 * input and nothing written past these sizes.
 */
attn_status attn_quant_v_cache(const void* v_bf16, int32_t B, int32_t Nk, int32_t Hkv, int32_t D,
                               int32_t format, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                               void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Forward
 * --------------------------------------------------------------------- */

typedef struct attn_nvfp4_tensor {
  const uint8_t* codes;       /* [rows, D/2] as written by attn_quant_nvfp4 */
  const uint8_t* scales;      /* [rows, D/16] */
  const float* tensor_scale;  /* one float */
} attn_nvfp4_tensor;

typedef struct attn_v_tensor {
  int32_t format;             /* attn_v_format */
  const uint8_t* codes;       /* as written by attn_quant_v */
  const uint8_t* scales;      /* MXFP4 only */
  const float* tensor_scale;  /* FP8 only */
} attn_v_tensor;

typedef struct attn_fwd_args {
  /* Shapes.  Dense: B batches of Nq queries and Nk keys.  Varlen: B
   * sequences, Nq/Nk are the longest query/key lengths, total_q/total_k the
   * packed token counts, and cu_seqlens_q/k (device int32 [B+1]) the
   * offsets; the forward requires identical query and key lengths per
   * sequence only when causal. */
  int32_t B, Hq, Hkv, Nq, Nk, D;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int64_t total_q, total_k;
  float softmax_scale;        /* sigma; scores are sigma * Q.K */
  int32_t causal;             /* key j visible to query i iff j <= i (needs Nq == Nk) */
  attn_nvfp4_tensor q;        /* rows ordered like the bf16 Q: [B, Nq, Hq] / [total_q, Hq] */
  attn_nvfp4_tensor k;        /* [B, Nk, Hkv] / [total_k, Hkv] */
  attn_v_tensor v;
  void* o;                    /* [B, Nq, Hq, D] / [total_q, Hq, D] */
  int32_t o_dtype;            /* attn_out_dtype */
  float* lse;                 /* nullable; [B, Hq, Nq] / [Hq, total_q], natural log */
  void* ws;                   /* at least attn_fwd_ws_bytes(args) bytes */
  size_t ws_bytes;
  /* Optional probability dump for one (batch or sequence dbg_b, head dbg_h):
   * P codes [Nq, roundup(Nk,128)/2] (MXFP4, key 2k in the low nibble) or
   * [Nq, roundup(Nk,128)] (FP8), and E8M0 bytes [Nq, roundup(Nk,128)/32]
   * (MXFP4).  Codes of masked keys are 0.  NULL disables the dump. */
  uint8_t* dbg_p_codes;
  uint8_t* dbg_p_scales;
  int32_t dbg_b, dbg_h;
  /* Optional profiling: hipEvent_t handles (NULL to skip) recorded on
   * `stream` immediately before and after the attention kernel itself (after
   * the K expansion pre-pass), so callers can time the dominant kernel. */
  void* prof_event_begin;
  void* prof_event_end;
} attn_fwd_args;

/* Bytes of device workspace the forward needs for these shapes: the exact
 * float16 expansion of the NVFP4 K payload (E2M1 * E4M3, 6 significant
 * bits, exact in float16), arranged in 128-key operand tiles, i.e.
 * 2 * D * Hkv * kcols + 256 with kcols = B * roundup(Nk, 128), or
 * 128 * (ceil(total_k / 128) + B) for packed batches.  (Q is decoded from
 * its NVFP4 codes inside the attention kernel.)  Returns 0 for invalid
 * shapes. */
size_t attn_fwd_ws_bytes(const attn_fwd_args* a);

/*
 * Direct-P forward (noncausal inference path of the pages; summary page,
 * "What the paper found"): S = Q.K^T on the exact NVFP4 values, per tile of
 * 128 keys the running max m' of t = sigma*log2(e)*S is updated, each
 * 32-key block gets the E8M0 exponent e = max(floor(max(t) - m') - 2, -127)
 * and codes E2M1(2^(t - m' - e)), the denominator l and O accumulate the
 * dequantized codes times V, and finally O = o / l (times the FP8 V tensor
 * scale) and LSE = ln2 * (m + log2 l).  V may be FP8 or MXFP4.
 * D in {64, 128}; Hq % Hkv == 0; causal must be 0 (ATTN_ERR_UNSUPPORTED).
 */
attn_status attn_fwd_directp(const attn_fwd_args* a, void* stream);

/*
 * attn_fwd_directp for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, kernels, results and errors as attn_fwd_directp, except
 * that a->ws and a->ws_bytes are ignored: the float16 K operand tiles that
 * attn_fwd_directp keeps in the caller's workspace go to a fixed device
 * array inside the library, ATTN_NOALLOC_SCRATCH_BYTES per GPU, which every
 * GPU the library runs on holds until the process ends.  The call itself
 * allocates nothing (no hipMalloc, no hipFree, no allocating library call).
 * Limit: attn_fwd_ws_bytes(a) <= ATTN_NOALLOC_SCRATCH_BYTES, i.e. Hkv * kcols
 * <= 262159 at D = 128 (2 x 262159 at D = 64), e.g. 8 KV heads x 4 x 8192
 * keys; beyond it the call returns ATTN_ERR_WORKSPACE and launches nothing.
 * The array's address on a device is looked up once, on the first call on
 * that device (the device of `stream`).  All calls on one GPU share its
 * array, which keeps the last call's contents (each call writes every tile
 * it reads before reading it, so nothing needs clearing): calls that overlap
 * on one GPU -- on different streams, or from different host threads without
 * ordering -- race and give undefined results.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (((size_t)64 << 20) + 4096)
attn_status attn_fwd_directp_noalloc(const attn_fwd_args* a, void* stream);

/*
 * FP8-P/V forward (the variant the pages keep for stable causal training;
 * summary page, "What the paper found"): identical to attn_fwd_directp
 * except that each probability is E4M3(2^(t - m')) with unit scale and V is
 * FP8 E4M3.  Causal or not.  D in {64, 128}; Hq % Hkv == 0.
 */
attn_status attn_fwd_fp8pv(const attn_fwd_args* a, void* stream);

/*
 * Exp-free variants.  Two related methods listed beside the arXiv entry of
 * the pages' paper (2609.04105v1, "Related papers") map log2-domain scores
 * to probability codes without an exponential: "VC-Attention: Value
 * Smoothing and Softmax Casting for Low-bit Attention" (E4M3 codes from one
 * fused multiply-add) and "EFQ-Softmax: Exp-Free Quantization for Softmax"
 * (block-scaled E2M1).  Only their abstracts are available; the reading
 * implemented is the log-linear cast: a minifloat code read as an integer is
 * a fixed-point log2 of its value, so with y the log2 of the probability the
 * code is clamp(RNE(2^M (y + b)), 0, top) -- M mantissa bits and exponent
 * bias b of the code format, top its largest finite code.  The decoded value
 * is Mitchell's piecewise-linear 2^y (to M fraction bits) in the normal range.
 * Running max, block exponents, denominator (from the same decoded codes),
 * P.V, O and LSE are those of the exact entry points; only the element map
 * changes, so the results are approximations of the exact ones, not equal to
 * them.  Arguments, workspace, errors and the debug dump are as for the exact
 * entry point named.
 *
 * attn_fwd_directp_efq: as attn_fwd_directp, code = min(RNE(2 (t - m' - e) + 2), 7)
 *                       (E2M1: M = 1, b = 1), same E8M0 exponent e per 32 keys.
 * attn_fwd_fp8pv_cast:  as attn_fwd_fp8pv, code = max(RNE(8 (t - m') + 56), 0)
 *                       (E4M3: M = 3, b = 7), unit scale.  Causal or not.
 */
attn_status attn_fwd_directp_efq(const attn_fwd_args* a, void* stream);
attn_status attn_fwd_fp8pv_cast(const attn_fwd_args* a, void* stream);

/*
 * Direct-P forward with MX-native Q/K (opt-in; not the pages' format).  The
 * arithmetic is that of attn_fwd_directp -- running max per 128-key tile,
 * E8M0 exponent and E2M1 codes per 32 keys, denominator from the same codes,
 * O = o / l, LSE = ln2 (m + log2 l) -- except that Q^ and K^ are the MXFP4
 * values E2M1(code) * 2^e written by attn_quant_mxfp4, so that
 * t = sigma * log2(e) * (Q^ . K^) and Q.K^T runs as a block-scaled FP4
 * contraction.  Arguments as for attn_fwd_directp, with:
 *   q, k: codes [rows, D/2] (16-byte aligned) and scales [rows, D/32] E8M0
 *         bytes (aligned to D/32 bytes); tensor_scale is ignored (may be NULL)
 *   ws  : at least attn_fwd_ws_bytes(args) bytes (this entry point uses
 *         64 D + 512 bytes per 128-key tile and KV head of it)
 * Noncausal (ATTN_ERR_UNSUPPORTED otherwise); D in {64, 128}; V FP8 or
 * MXFP4.  Errors as for attn_fwd_directp.
 *
 * attn_fwd_fp8pv_mxqk: the same MX-native Q/K with the FP8-P/V arithmetic of
 * attn_fwd_fp8pv (E4M3(2^(t - m')) with unit scale, FP8 V, causal or not).
 *
 * attn_fwd_directp_efq_mxqk: MX-native Q/K with the exp-free E2M1 cast of
 * attn_fwd_directp_efq (code = min(RNE(2 (t - m' - e) + 2), 7)) in place of
 * RNE(2^(t - m' - e)); noncausal.
 *
 * attn_fwd_fp8pv_cast_mxqk: MX-native Q/K with the exp-free E4M3 cast of
 * attn_fwd_fp8pv_cast (code = max(RNE(8 (t - m') + 56), 0)); FP8 V, causal
 * or not.
 */
attn_status attn_fwd_directp_mxqk(const attn_fwd_args* a, void* stream);
attn_status attn_fwd_fp8pv_mxqk(const attn_fwd_args* a, void* stream);
attn_status attn_fwd_directp_efq_mxqk(const attn_fwd_args* a, void* stream);
attn_status attn_fwd_fp8pv_cast_mxqk(const attn_fwd_args* a, void* stream);

/*
 * BF16 fused attention forward, the baseline the pages compare against
 * (BF16 FlashAttention-4 on the summary page, "Key results"): O =
 * softmax(sigma Q K^T) V with bf16 operands, float32 accumulation and
 * probabilities rounded to bf16 for the P.V product.
 *   q: [B, Nq, Hq, D] bf16, k/v: [B, Nk, Hkv, D] bf16 (dense only),
 *   o: [B, Nq, Hq, D] bf16, lse: nullable [B, Hq, Nq].
 * D in {64, 128}.  No workspace.
 */
attn_status attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                          int32_t B, int32_t Hq, int32_t Hkv, int32_t Nq, int32_t Nk, int32_t D,
                          float softmax_scale, int32_t causal, void* stream);

/* ------------------------------------------------------------------------
 * Decode-shaped forward
 * --------------------------------------------------------------------- */

/*
 * Forward of a decode step: nq new query tokens per sequence attend to a KV
 * cache of up to Nk keys (the workload of the Colfax Research feed's post on
 * FlashAttention-4 decode, which generates one or a few tokens per step from
 * the cached keys and values).  The arithmetic is exactly that of
 * attn_fwd_directp / attn_fwd_fp8pv (128-key tiles of the running max from
 * key 0, E8M0 per 32 keys, l from the rounded probabilities), so a decode
 * call and a prefill call over the same quantized operands give the same
 * probability codes up to float32 rounding near-ties.  The kernel reads the
 * compact cache directly; it needs no workspace.
 *
 *   q     : NVFP4 Q of the new tokens, rows ordered [B, nq, Hq]
 *           (attn_quant_nvfp4 of a bf16 [B, nq, Hq, D] tensor)
 *   k     : NVFP4 K cache, head-major: rows ordered [B, Hkv, Nk]
 *           (attn_quant_nvfp4 of a bf16 [B, Hkv, Nk, D] tensor)
 *   v     : V cache as attn_quant_v_cache writes it for a dense bf16
 *           [B, Nk, Hkv, D] tensor (one contiguous block per sequence, KV
 *           head and 128-key tile)
 *   seqlens_k : nullable device int32 [B], the number of valid cache
 *           entries of each sequence (values are clamped to [0, Nk]); NULL
 *           means Nk for every sequence.  The kernel reads whole 128-key
 *           tiles: cache entries past a sequence's valid length up to the
 *           next multiple of 128 are read and masked, so they must hold
 *           finite codes (zeros, or stale entries written by the quantizers)
 *   causal: new token i (0-based) of a sequence with L valid keys sits at
 *           position L - nq + i and sees keys 0 .. L - nq + i (the new
 *           tokens are the last nq entries of the cache); otherwise every
 *           new token sees all L keys.  With nq == 1 both are the same.
 *   o     : [B, nq, Hq, D] (o_dtype); lse: nullable float [B, Hq, nq]
 * A row with no visible key gets O = 0 and LSE = -inf.
 * Limits: D in {64, 128}; Hq % Hkv == 0; 1 <= nq; the cache capacity Nk a
 * multiple of 128 (ATTN_ERR_INVALID_ARGUMENT otherwise); B * Hkv *
 * ceil(Hq / Hkv * nq / 16) below 2^31 (ATTN_ERR_UNSUPPORTED otherwise).
 * attn_decode_fp8pv requires FP8 V.  Optional probability dump
 * of (dbg_b, dbg_h): codes [nq, roundup(Nk,128)/2] (MXFP4 P) or
 * [nq, roundup(Nk,128)] (FP8 P), E8M0 bytes [nq, roundup(Nk,128)/32].
 * prof_event_begin/end (hipEvent_t, nullable) are recorded around the kernel.
 */
typedef struct attn_decode_args {
  int32_t B, Hq, Hkv, nq, Nk, D;
  const int32_t* seqlens_k;
  float softmax_scale;
  int32_t causal;
  attn_nvfp4_tensor q;
  attn_nvfp4_tensor k;
  attn_v_tensor v;
  void* o;
  int32_t o_dtype;
  float* lse;
  uint8_t* dbg_p_codes;
  uint8_t* dbg_p_scales;
  int32_t dbg_b, dbg_h;
  void* prof_event_begin;
  void* prof_event_end;
} attn_decode_args;

/* Direct-P decode: MXFP4 P (E8M0 per 32 keys), V FP8 or MXFP4. */
attn_status attn_decode_directp(const attn_decode_args* a, void* stream);
/* FP8-P/V decode: E4M3 P with unit scale, FP8 V. */
attn_status attn_decode_fp8pv(const attn_decode_args* a, void* stream);

/* ------------------------------------------------------------------------
 * Backward (causal training path)
 * --------------------------------------------------------------------- */

/*
 * Backward of the FP8-P/V forward, the path the pages train with (summary
 * page, "What the paper found": the forward keeps its quantized Q/K payloads,
 * scales and LSE; the backward rebuilds the probabilities from them and uses
 * FP8 gradient operands, with E5M2 output gradients).  The pages give no
 * formulas; the operation implemented, per (batch, head), is:
 *   dO^ = E5M2_sat(dO * S) * s with S = 57344 / amax(dO) (one scale per tensor), s = 1 / S
 *   D_i = sum_d dO^_id O_id
 *   P   = 2^(t - LSE log2 e), t = sigma log2(e) g_q g_k Q_raw . K_raw (as in the forward)
 *   dP  = dO^ V^T,  dS = P (dP - D)
 *   dV  = P~^T dO^, dK = sigma dS~^T Q^, dQ = sigma dS~ K^
 * with Q^ = Q_raw g_q, K^ = K_raw g_k the exact NVFP4 values, V^ the FP8
 * values, and P~, dS~ rounded to E4M3 with one E8M0 exponent per 32 elements
 * along the contraction axis of their product (OCP MX rule, e = floor(log2
 * amax) - 8): along queries for dV and dK, along keys for dQ.  GQA sums the
 * query heads of a group into dK and dV.  Causal: key j is visible to query
 * i iff j <= i.
 *
 * Dense batches only (Nq == Nk == N).  D in {64, 128}; Hq % Hkv == 0;
 * 2 * D * roundup(N, 128) below 2^31 (N up to 8 388 480 at D = 128).
 *   q, k   : the forward's NVFP4 operands (attn_quant_nvfp4 output)
 *   v      : the forward's FP8 V (attn_quant_v, ATTN_V_FP8_E4M3; MXFP4 V is
 *            ATTN_ERR_UNSUPPORTED)
 *   o      : bf16 [B, N, Hq, D], the forward output
 *   lse    : float [B, Hq, N], the forward LSE (natural log)
 *   dout   : bf16 [B, N, Hq, D]
 *   dq     : float [B, N, Hq, D];  dk, dv : float [B, N, Hkv, D] (written)
 *   ws     : attn_bwd_ws_bytes(args) bytes, 256-byte aligned: the prepared
 *            operands (bf16 Q^/K^ row-major, E5M2 dO^ row-major,
 *            key-major V codes, D and LSE log2 e per row)
 * Argument errors are found before any launch.  prof_event_begin/end
 * (hipEvent_t, nullable) are recorded around the dK/dV and dQ kernels.
 */
typedef struct attn_bwd_args {
  int32_t B, Hq, Hkv, N, D;
  float softmax_scale;
  int32_t causal;
  attn_nvfp4_tensor q;
  attn_nvfp4_tensor k;
  attn_v_tensor v;
  const void* o;
  const float* lse;
  const void* dout;
  float* dq;
  float* dk;
  float* dv;
  void* ws;
  size_t ws_bytes;
  /* Optional dump of the E4M3 operands of one (batch dbg_b, query head
   * dbg_h), each buffer caller-allocated and zero-filled, NPAD = roundup(N,
   * 128): P~ and dS~K codes [NPAD, NPAD] (query row, key column) with their
   * E8M0 bytes [NPAD/32, NPAD] (32-query block, key); dS~Q codes [NPAD, NPAD]
   * with E8M0 bytes [NPAD, NPAD/32] (query, 32-key block).  All six NULL
   * disables the dump; otherwise all six must be given. */
  uint8_t* dbg_p_codes;
  uint8_t* dbg_p_exps;
  uint8_t* dbg_dsk_codes;
  uint8_t* dbg_dsk_exps;
  uint8_t* dbg_dsq_codes;
  uint8_t* dbg_dsq_exps;
  int32_t dbg_b, dbg_h;
  void* prof_event_begin;
  void* prof_event_end;
} attn_bwd_args;

size_t attn_bwd_ws_bytes(const attn_bwd_args* a);
attn_status attn_bwd_fp8(const attn_bwd_args* a, void* stream);

/* ---- diagnostics ---------------------------------------------------------
 * For the measurement script that derives the per-instruction costs behind
 * the kernels' roofline notes; not part of the attention path.
 *
 * attn_probe_kinds: the number of issue-rate micro-kernels.
 * attn_probe_issue_rates launches micro-kernel `kind` (0 .. attn_probe_kinds()
 * - 1) on `stream` as 256 workgroups of 96 KB LDS (one per CU).  Each
 * workgroup writes its cycle count (s_memtime, from a barrier before its
 * waves start to a barrier after all finish) to cycles[workgroup].
 * `cycles` is a device buffer of 512 int64, 8-byte aligned, owned by the
 * caller: entries 256 .. 511 belong to a store that keeps the kernels'
 * results live and that no launch takes in practice.  *units receives the work of one launch: instructions per SIMD
 * (vector and matrix kinds) or bytes per CU (LDS kinds); *grid receives 256.
 * Kinds: 0 v_fma_f32, 1 v_exp_f32, 2 v_med3_f32, 3 v_cvt_scalef32_pk_fp8_f32,
 * 4 v_max3_f32 (two waves per SIMD, eight independent chains each);
 * 5 v_mfma_f32_32x32x16_bf16, 6 the scaled 32x32x64 MFMA on FP8, 7 on FP4
 * (one wave per SIMD, four accumulators); 8 and 9: one MFMA wave (bf16) and
 * one v_fma_f32 (8) or v_exp_f32 (9) wave per SIMD, units = MFMA per SIMD;
 * 10, 11, 12: two waves per SIMD, each issuing 2, 4 or 8 v_fma_f32 per MFMA,
 * units = MFMA per SIMD; 13 ds_read_b128, 14 ds_read_b64, 15
 * ds_read_b64_tr_b16, 16 ds_write_b128, 17 ds_write_b32 (eight waves,
 * lane-contiguous, conflict-free; units = bytes per CU); 18
 * v_cvt_scalef32_pk_fp4_f32 (as 0-4); 19-22: two waves per SIMD, each step
 * one v_exp_f32 followed by independent work: 19 one v_fma_f32, 20 three
 * v_fma_f32, 21 one v_max3_f32, 22 one v_cvt_scalef32_pk_fp4_f32, 23 as
 * 19 in runs of four exponentials and four FMAs (units = steps per SIMD);
 * 24 v_fma_f32 at four waves per SIMD (1024 threads); 25 as 12 at four
 * waves per SIMD; 26 as 12 with 16 v_fma_f32 per MFMA (units = MFMA per
 * SIMD for 25 and 26); 27, 28: as 8 with 3 and 4 times the FMAs, 29: as 9
 * with twice the exponentials (units = MFMA per SIMD); 30-33: the forward
 * key loop's instruction mix per 128-key tile (42 bf16 MFMA, 64 v_exp_f32,
 * 32 FP4 conversions, 36 v_max3_f32, the rest v_fma_f32) -- 30 interleaved
 * one MFMA per slot, 31 as two-phase ping-pong with a barrier per phase, 32
 * and 33 with the encode as dependent fma -> exp -> conversion chains, in
 * one slot (32) or spread over three (33); units = wave-tiles per SIMD.
 * Errors: ATTN_ERR_INVALID_ARGUMENT (kind out of range, null or misaligned
 * pointer), ATTN_ERR_HIP.
 */
int attn_probe_kinds(void);
attn_status attn_probe_issue_rates(int kind, long long* cycles, long long* units, int* grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FP4_H */
