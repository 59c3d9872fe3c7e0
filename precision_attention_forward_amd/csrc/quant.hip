// Quantizers of the Direct-P attention forward (gfx950).
//
// NVFP4 for Q and K and FP8 E4M3 / MXFP4 for V, following "Hardware-Aware FP4
// FlashAttention-4" (summary page, "What the paper found": NVFP4 Q/K, FP4 or
// FP8 P/V).  The page gives only the format names; the rules implemented here
// are the NVFP4 and OCP MX conventions stated in include/attn_fp4.h, with
// every step an IEEE float32 operation so the codes are reproducible bit for
// bit.  All kernels are HBM-bound: each reads its bf16 input once for the
// per-tensor amax and once for the encode.  Element codes come from gfx950's
// conversions (v_cvt_scalef32_pk_fp4_f32: round to nearest even, saturating,
// sign kept; v_cvt_pk_fp8_f32: round to nearest even) applied to the same
// float32 products fl(x * enc) the rules define; block scales use the
// integer E4M3 encoder of common.h.
#include "common.h"

namespace attn {

constexpr int AMAX_THREADS = 256;
constexpr int AMAX_MAX_PARTIALS = 2048;
constexpr int AMAX_UNROLL = 4;      // 16-byte loads in flight per thread

// Pass 1: per-workgroup max |x| over a bf16 array of n elements (n % 8 == 0).
__global__ void __launch_bounds__(AMAX_THREADS) amax_partials_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                                     float* __restrict__ partials) {
  float m = 0.0f;
  const int64_t n8 = n / 8;
  const u32x4* x8 = reinterpret_cast<const u32x4*>(x);
  const int64_t stride = (int64_t)gridDim.x * AMAX_THREADS;
  int64_t i = blockIdx.x * (int64_t)AMAX_THREADS + threadIdx.x;
  for (; i + (AMAX_UNROLL - 1) * stride < n8; i += AMAX_UNROLL * stride) {
    u32x4 v[AMAX_UNROLL];
#pragma unroll
    for (int u = 0; u < AMAX_UNROLL; ++u) v[u] = __builtin_nontemporal_load(&x8[i + u * stride]);
#pragma unroll
    for (int u = 0; u < AMAX_UNROLL; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m = __builtin_fmaxf(m, __builtin_fabsf(bf16_bits_to_f32(v[u][j] & 0xFFFFu)));
        m = __builtin_fmaxf(m, __builtin_fabsf(bf16_bits_to_f32(v[u][j] >> 16)));
      }
  }
  for (; i < n8; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(&x8[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = __builtin_fmaxf(m, __builtin_fabsf(bf16_bits_to_f32(v[j] & 0xFFFFu)));
      m = __builtin_fmaxf(m, __builtin_fabsf(bf16_bits_to_f32(v[j] >> 16)));
    }
  }
  m = wave_max(m);
  __shared__ float red[AMAX_THREADS / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < AMAX_THREADS / 64; ++w) r = __builtin_fmaxf(r, red[w]);
    partials[blockIdx.x] = r;
  }
}

// Reduce the pass-1 partials (every workgroup of pass 2 does this itself; at
// most AMAX_MAX_PARTIALS floats, read from L2).
__device__ inline float reduce_partials(const float* partials, int np) {
  __shared__ float red[8];
  float m = 0.0f;
  for (int i = threadIdx.x; i < np; i += blockDim.x) m = __builtin_fmaxf(m, partials[i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = __builtin_fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// top / amax, 1 for amax == 0, FLT_MAX when the quotient overflows.
__device__ inline float encode_scale(float amax, float top) {
  if (amax == 0.0f) return 1.0f;
  float s = top / amax;
  return __builtin_isinf(s) ? 3.40282347e+38f : s;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// One NVFP4 block for a block maximum mapped to M (6 in the standard recipe):
// s = E4M3((amax_b / M) * S_enc), codes E2M1(x * (S_enc / s)) (element 2k in
// the low nibble of byte k), all 0 when s decodes to 0.  Returns the scale code.
__device__ inline uint32_t nvfp4_block(const float (&v)[16], float amax_b, float s_enc, float M, u32x2& out,
                                       float& sv) {
  const float sf = (amax_b / M) * s_enc;
  const uint32_t sc = e4m3_encode(sf);
  sv = e4m3_decode(sc);
  out = u32x2{0u, 0u};
  if (sv > 0.0f) {
    const float enc = s_enc / sv;
    float y[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) y[j] = v[j] * enc;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      uint32_t w = 0u;
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[8 * h2 + 0], y[8 * h2 + 1], 1.0f, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[8 * h2 + 2], y[8 * h2 + 3], 1.0f, 1);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[8 * h2 + 4], y[8 * h2 + 5], 1.0f, 2);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[8 * h2 + 6], y[8 * h2 + 7], 1.0f, 3);
      out[h2] = w;
    }
  }
  return sc;
}

// Squared error of a block candidate in units of the tensor scale:
// sum over j in order of (x_j S_enc - E2M1(code_j) s)^2, float32, no contraction.
// The codes are decoded two at a time by the hardware FP4 -> F32 conversion
// (unit scale; element 2k from the low nibble of byte k), then multiplied by s
// (exact: at most 2 x 4 significant bits).
__device__ inline float nvfp4_block_err(const float (&xs)[16], const u32x2& w, float sv) {
  float q[16];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[h2], 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[h2], 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[h2], 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[h2], 1.0f, 3);
    q[8 * h2 + 0] = p0[0]; q[8 * h2 + 1] = p0[1];
    q[8 * h2 + 2] = p1[0]; q[8 * h2 + 3] = p1[1];
    q[8 * h2 + 4] = p2[0]; q[8 * h2 + 5] = p2[1];
    q[8 * h2 + 6] = p3[0]; q[8 * h2 + 7] = p3[1];
  }
  float err = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float d = xs[j] - q[j] * sv;
    err = err + d * d;
  }
  return err;
}

// Pass 2 (NVFP4): one thread per 16-element block along D.  FOUR_SIX: the
// Four Over Six variant (related method listed beside the arXiv entry of the
// pages' paper, "Four Over Six: More Accurate NVFP4 Quantization with Adaptive
// Block Scaling"): S_enc = 1792 / amax_t, and each block keeps the block
// maximum mapped to 4 instead of 6 when that gives the smaller squared error.
template <bool FOUR_SIX>
__global__ void __launch_bounds__(256) quant_nvfp4_kernel(const uint16_t* __restrict__ x, int64_t nblocks,
                                                          const float* __restrict__ partials, int np,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                          float* __restrict__ tensor_scale) {
  const float amax_t = reduce_partials(partials, np);
  const float s_enc = encode_scale(amax_t, FOUR_SIX ? 1792.0f : 2688.0f);
  if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = 1.0f / s_enc;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nblocks; i += (int64_t)gridDim.x * blockDim.x) {
    const u32x4* p = reinterpret_cast<const u32x4*>(x + 16 * i);
    u32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_bits_to_f32(a[j] & 0xFFFFu);
      v[2 * j + 1] = bf16_bits_to_f32(a[j] >> 16);
      v[8 + 2 * j] = bf16_bits_to_f32(b[j] & 0xFFFFu);
      v[8 + 2 * j + 1] = bf16_bits_to_f32(b[j] >> 16);
    }
    float amax_b = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax_b = __builtin_fmaxf(amax_b, __builtin_fabsf(v[j]));
    u32x2 out;
    float sv;
    uint32_t sc = nvfp4_block(v, amax_b, s_enc, 6.0f, out, sv);
    if (FOUR_SIX) {
      float xs[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) xs[j] = v[j] * s_enc;
      u32x2 out4;
      float sv4;
      const uint32_t sc4 = nvfp4_block(v, amax_b, s_enc, 4.0f, out4, sv4);
      if (nvfp4_block_err(xs, out4, sv4) < nvfp4_block_err(xs, out, sv)) {
        out = out4;
        sc = sc4;
      }
    }
    *reinterpret_cast<u32x2*>(codes + 8 * i) = out;
    scales[i] = (uint8_t)sc;
  }
}

// Pass 2 (V): one workgroup per (128-key tile, kv head, sequence).  The tile
// is staged in LDS, then each thread encodes one (channel, 32-key block) and
// writes it key-contiguous.  FMT 0 = FP8 E4M3 (per-tensor scale), 1 = MXFP4.
// LAYOUT 0: the transposed layout [Hkv][D][cols] of the forward; LAYOUT 1:
// the decode cache, one block of D key-contiguous rows per (sequence, KV
// head, 128-key tile), tiles of a (sequence, head) consecutive (dense input,
// nk_pad = Nk).
template <int FMT, int D, int LAYOUT>
__global__ void __launch_bounds__(256) quant_v_kernel(const uint16_t* __restrict__ v, int Nk, int Hkv,
                                                      const int32_t* __restrict__ cu_k, int64_t nk_pad, int64_t cols,
                                                      const float* __restrict__ partials, int np,
                                                      uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                      float* __restrict__ tensor_scale) {
  // Head fastest in dispatch order: a key's row holds all KV heads side by
  // side (Hkv * D * 2 bytes), so the workgroups dispatched together read
  // neighbouring head slices of the same keys instead of one head's slice of
  // keys far apart.  1.06x (MXFP4) and 1.09x (FP8) against tile-fastest order
  // on the Wan shape.
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int h = lin % gridDim.y, tile = (lin / gridDim.y) % gridDim.x, s = lin / (gridDim.x * gridDim.y);
  const bool varlen = cu_k != nullptr;
  const int64_t tok0 = varlen ? cu_k[s] : (int64_t)s * Nk;
  const int len = varlen ? cu_k[s + 1] - cu_k[s] : Nk;
  float enc = 1.0f;
  if (FMT == 0) {
    const float amax = reduce_partials(partials, np);
    enc = encode_scale(amax, 448.0f);
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *tensor_scale = 1.0f / enc;
  }
  if (tile * KEY_TILE >= len) return;
  __shared__ uint16_t tileb[KEY_TILE * D];
  // stage: 128 keys x D bf16, zero beyond the end of the sequence
  constexpr int CH = KEY_TILE * D / 8;  // 16-byte chunks
  for (int c = threadIdx.x; c < CH; c += 256) {
    const int key = c / (D / 8), part = c % (D / 8);
    u32x4 val = {0u, 0u, 0u, 0u};
    const int kg = tile * KEY_TILE + key;
    if (kg < len) val = *reinterpret_cast<const u32x4*>(v + ((tok0 + kg) * Hkv + h) * (int64_t)D + part * 8);
    *reinterpret_cast<u32x4*>(&tileb[key * D + part * 8]) = val;
  }
  __syncthreads();
  const int64_t col0 = kcol_offset(varlen, s, tok0, nk_pad) + (int64_t)tile * KEY_TILE;
  // one thread per (channel d, 32-key block); consecutive lanes take
  // consecutive channels, so each LDS read of a wave covers 128 contiguous bytes
  for (int p = threadIdx.x; p < D * 4; p += 256) {
    const int d = p % D, blk = p / D;
    float x[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] = bf16_bits_to_f32(tileb[(blk * 32 + j) * D + d]);
    const int64_t row = (int64_t)h * D + d;
    // destinations of this (channel, block): 32 FP8 codes / 16 MXFP4 code bytes and one scale byte
    uint8_t* cdst;
    uint8_t* sdst = nullptr;
    if (LAYOUT == 0) {
      cdst = FMT == 0 ? codes + row * cols + col0 + blk * 32 : codes + (row * cols + col0 + blk * 32) / 2;
      if (FMT == 1) sdst = scales + row * (cols / 32) + (col0 + blk * 32) / 32;
    } else {
      const int64_t t = ((int64_t)s * Hkv + h) * (nk_pad / KEY_TILE) + tile;
      cdst = FMT == 0 ? codes + (t * D + d) * 128 + blk * 32 : codes + (t * D + d) * 64 + blk * 16;
      if (FMT == 1) sdst = scales + (t * D + d) * 4 + blk;
    }
    float mul = enc;
    if (FMT == 1) {
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[j]));
      const uint32_t ab = __float_as_uint(amax);
      const int E = (int)(ab >> 23) - 127;              // floor(log2 amax) for normal amax
      int e = (ab >> 23) == 0 ? -127 : E - 2;           // zero/subnormal block max -> -127
      e = e < -127 ? -127 : e;
      mul = __builtin_amdgcn_ldexpf(1.0f, -e);          // exact: x * 2^-e
      *sdst = (uint8_t)(e + 127);
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] *= mul;
    if (FMT == 0) {
      u32x4 o[2];
#pragma unroll
      for (int k = 0; k < 8; ++k) {   // value 4k + i in byte i of word k
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * k], x[4 * k + 1], 0, false);
        o[k >> 2][k & 3] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[4 * k + 2], x[4 * k + 3], lo, true);
      }
      u32x4* dst = reinterpret_cast<u32x4*>(cdst);
      dst[0] = o[0];
      dst[1] = o[1];
    } else {
      u32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) {   // value 8k + 2i (+1) in byte i of word k, low nibble first
        uint32_t w = 0u;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[8 * k + 0], x[8 * k + 1], 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[8 * k + 2], x[8 * k + 3], 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[8 * k + 4], x[8 * k + 5], 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[8 * k + 6], x[8 * k + 7], 1.0f, 3);
        o[k] = w;
      }
      *reinterpret_cast<u32x4*>(cdst) = o;
    }
  }
}

// MXFP4 Q/K (opt-in MX-native format; the OCP MX rule the V quantizer
// applies along keys, here along D).  Four consecutive lanes share one
// 32-element block, eight elements (16 bytes) each, so a wave reads 1 KB of
// contiguous input per load; the block max is combined with two lane
// exchanges inside the group of four.  e = floor(log2 amax) - 2 (-127 for a
// zero or subnormal block max, below the E8M0 range), codes E2M1(x * 2^-e)
// by the hardware RNE conversion (x * 2^-e is exact), element 2k in the low
// nibble of byte k.  No tensor scale and no amax pass: one read of the input.
//
// HAD: each block is first rotated by the unnormalized 32-point Hadamard
// (Sylvester) matrix, the micro-rotation of "Bridging the Gap Between Promise
// and Performance for Microscaling FP4 Quantization" (listed beside the
// pages' arXiv entry), in float32 butterfly stages of stride 1, 2, 4 (inside
// a lane's eight elements) and 8, 16 (with lanes ^1, ^2): the pair (i, i + s)
// becomes (x_i + x_{i+s}, x_i - x_{i+s}).  Rotating Q and K alike multiplies
// every Q.K by 32.
template <bool HAD>
__global__ void __launch_bounds__(256) quant_mxfp4_kernel(const uint16_t* __restrict__ x, int64_t nblocks,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t nparts = nblocks * 4;            // 8-element parts; a block's four parts share a lane group
  const int64_t stride = (int64_t)gridDim.x * 256;
  // (stride and the start are multiples of 4, so a lane group is entirely in or out of range)
  for (int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x; i < nparts; i += stride) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + i);
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
      f[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
    }
    if (HAD) {
#pragma unroll
      for (int st = 1; st < 8; st *= 2)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (!(j & st)) {
            const float a = f[j], c = f[j + st];
            f[j] = a + c;
            f[j + st] = a - c;
          }
#pragma unroll
      for (int lm = 1; lm < 4; lm *= 2) {          // strides 8 and 16: lanes lm apart in the group
        const bool upper = (i & lm) != 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float other = __shfl_xor(f[j], lm, 64);
          f[j] = upper ? other - f[j] : f[j] + other;
        }
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[j]));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2, 64));
    const uint32_t ab = __float_as_uint(amax);
    int e = (ab >> 23) == 0 ? -127 : (int)(ab >> 23) - 127 - 2;
    e = e < -127 ? -127 : e;
    const float mul = __builtin_amdgcn_ldexpf(1.0f, -e);
    uint32_t c = 0u;
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[0] * mul, f[1] * mul, 1.0f, 0);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[2] * mul, f[3] * mul, 1.0f, 1);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[4] * mul, f[5] * mul, 1.0f, 2);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[6] * mul, f[7] * mul, 1.0f, 3);
    reinterpret_cast<uint32_t*>(codes)[i] = c;
    if ((i & 3) == 0) scales[i >> 2] = (uint8_t)(e + 127);
  }
}

// ---- host launchers (called from api.cpp) ----
hipError_t launch_amax(const void* x, int64_t n, float* partials, int* np_out, hipStream_t st) {
  int64_t want = (n / 8 + AMAX_THREADS * 16 - 1) / (AMAX_THREADS * 16);
  int np = (int)(want < 1 ? 1 : (want > AMAX_MAX_PARTIALS ? AMAX_MAX_PARTIALS : want));
  *np_out = np;
  hipLaunchKernelGGL(amax_partials_kernel, dim3(np), dim3(AMAX_THREADS), 0, st, (const uint16_t*)x, n, partials);
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const void* x, int64_t rows, int D, const float* partials, int np, uint8_t* codes,
                              uint8_t* scales, float* tensor_scale, bool four_six, hipStream_t st) {
  int64_t nblocks = rows * (D / 16);
  int64_t want = (nblocks + 255) / 256;
  int grid = (int)(want < 1 ? 1 : (want > 4096 ? 4096 : want));
  if (four_six)
    hipLaunchKernelGGL(quant_nvfp4_kernel<true>, dim3(grid), dim3(256), 0, st, (const uint16_t*)x, nblocks, partials,
                       np, codes, scales, tensor_scale);
  else
    hipLaunchKernelGGL(quant_nvfp4_kernel<false>, dim3(grid), dim3(256), 0, st, (const uint16_t*)x, nblocks, partials,
                       np, codes, scales, tensor_scale);
  return hipGetLastError();
}

template <int F, int DD>
static void launch_quant_v_t(dim3 grid, hipStream_t st, const void* v, int Nk, int Hkv, const int32_t* cu_k,
                             int64_t nk_pad, int64_t cols, const float* partials, int np, uint8_t* codes,
                             uint8_t* scales, float* tensor_scale, bool cache_layout) {
  if (cache_layout)
    hipLaunchKernelGGL((quant_v_kernel<F, DD, 1>), grid, dim3(256), 0, st, (const uint16_t*)v, Nk, Hkv, cu_k, nk_pad,
                       cols, partials, np, codes, scales, tensor_scale);
  else
    hipLaunchKernelGGL((quant_v_kernel<F, DD, 0>), grid, dim3(256), 0, st, (const uint16_t*)v, Nk, Hkv, cu_k, nk_pad,
                       cols, partials, np, codes, scales, tensor_scale);
}

hipError_t launch_quant_v(const void* v, int B, int Nk, int Hkv, int D, const int32_t* cu_k, int max_len, int64_t cols,
                          int fmt, const float* partials, int np, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                          bool cache_layout, hipStream_t st) {
  const int64_t nk_pad = roundup(Nk, KEY_TILE);
  dim3 grid((unsigned)((max_len + KEY_TILE - 1) / KEY_TILE), (unsigned)Hkv, (unsigned)B);
  if (grid.x == 0) grid.x = 1;
  auto go = fmt == 0 ? (D == 64 ? launch_quant_v_t<0, 64> : launch_quant_v_t<0, 128>)
                     : (D == 64 ? launch_quant_v_t<1, 64> : launch_quant_v_t<1, 128>);
  go(grid, st, v, Nk, Hkv, cu_k, nk_pad, cols, partials, np, codes, scales, tensor_scale, cache_layout);
  return hipGetLastError();
}

hipError_t launch_quant_mxfp4(const void* x, int64_t rows, int D, uint8_t* codes, uint8_t* scales, bool hadamard,
                              hipStream_t st) {
  const int64_t nblocks = rows * (D / 32);
  if (nblocks == 0) return hipSuccess;
  const int64_t want = (nblocks * 4 + 255) / 256;
  const int grid = (int)(want > 16384 ? 16384 : want);
  if (hadamard)
    hipLaunchKernelGGL(quant_mxfp4_kernel<true>, dim3(grid), dim3(256), 0, st, (const uint16_t*)x, nblocks, codes,
                       scales);
  else
    hipLaunchKernelGGL(quant_mxfp4_kernel<false>, dim3(grid), dim3(256), 0, st, (const uint16_t*)x, nblocks, codes,
                       scales);
  return hipGetLastError();
}

}  // namespace attn
