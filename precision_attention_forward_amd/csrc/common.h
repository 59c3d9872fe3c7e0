// Shared device helpers for the gfx950 kernels: vector types, bit-exact
// E2M1 / E4M3 encoders, decoders, and the tile geometry of the forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Tiles of the forward: 128 keys per tile (the running-max granularity of the
// method's online softmax), 32 queries per wave, 8 waves per workgroup.
constexpr int KEY_TILE = 128;
constexpr int WAVE_Q = 32;
constexpr int WG_WAVES = 8;
constexpr int WG_Q = WAVE_Q * WG_WAVES;  // 256

__host__ __device__ inline int64_t roundup(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Start column of sequence s in the transposed V / tiled K layouts.
__host__ __device__ inline int64_t kcol_offset(bool varlen, int s, int64_t cu_k_s, int64_t nk_pad) {
  return varlen ? 128 * (cu_k_s / 128 + s) : (int64_t)s * nk_pad;
}

// bf16 bits -> float (exact).
__device__ inline float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// E4M3 (fn) encoder: round to nearest even, saturate to +-448, keep the sign.
__device__ inline uint32_t e4m3_encode(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = __builtin_fabsf(v);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7Eu;
  } else if (a < 0x1p-6f) {          // subnormal range: multiples of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);   // exact scaling; 8 == 2^-6
  } else {
    uint32_t ab = __float_as_uint(a);
    uint32_t r = ab + 0x7FFFFu + ((ab >> 20) & 1u);  // round at mantissa bit 20
    code = (r >> 20) - (120u << 3);                  // rebias exponent 127 -> 7
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  return code | sign;
}

// E2M1 encoder: round to nearest even, saturate to +-6, keep the sign.
__device__ inline uint32_t e2m1_encode(float v) {
  uint32_t sign = (__float_as_uint(v) >> 28) & 0x8u;
  float a = __builtin_fabsf(v);
  uint32_t code;
  if (!(a < 6.0f)) {
    code = 7u;
  } else if (a < 1.0f) {             // 0, 0.5, 1.0 are codes 0, 1, 2
    code = (uint32_t)__builtin_rintf(a * 2.0f);
  } else {
    uint32_t ab = __float_as_uint(a);
    uint32_t r = ab + 0x1FFFFFu + ((ab >> 22) & 1u);  // round at mantissa bit 22
    code = (r >> 22) - (126u << 1);                  // rebias exponent 127 -> 1
    code = code > 7u ? 7u : code;
  }
  return code | sign;
}

__device__ inline float e4m3_decode(uint32_t c) {
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

__device__ inline float e2m1_decode(uint32_t c) {
  uint32_t e = (c >> 1) & 3u, m = c & 1u;
  float mag = e == 0 ? (float)m * 0.5f : __uint_as_float(((e + 126u) << 23) | (m << 22));
  return (c & 8u) ? -mag : mag;
}

// IEEE-2019 maximum of two / three floats (v_maximum3_f32 on gfx950): the
// larger operand, NaN if either is NaN.  Unlike fmax, its operands need no
// canonicalizing, which matters for matrix-instruction results.
__device__ inline float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ inline float fmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Wave-wide max (DPP/permute based; 64 lanes).
__device__ inline float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace attn
