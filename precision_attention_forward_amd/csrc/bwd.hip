// Attention backward of the causal training path for gfx950.
//
// Method: "Hardware-Aware FP4 FlashAttention-4" (summary page, "What the paper
// found"; arXiv listing 2609.04105v1, abstract): the forward keeps its
// quantized Q/K payloads, their scales and the LSE; the backward rebuilds
// the probabilities from them and uses FP8 gradient operands, the output
// gradient in E5M2.  Operations (per batch and head, t = c Q_raw.K_raw with
// c = sigma log2(e) g_q g_k as in the forward):
//   dO^ = E5M2(dO * S) * s (one scale per tensor), D_i = sum_d dO^_id O_id
//   P = 2^(t - LSE log2 e), dP = dO^ V^T, dS = P (dP - D)
//   dV = P~^T dO^, dK = sigma dS~^T Q^, dQ = sigma dS~ K^
// where P~ and dS~ are E4M3 with one E8M0 exponent per 32 elements along the
// contraction axis of their product (the OCP MX rule, e = floor(log2 amax) - 8):
// along queries for dV and dK, along keys for dQ.
//
// gfx950 mapping:
//  * Preparation kernels write the exact NVFP4 values of Q and K as bf16 (at
//    most 6 significant bits: exact) row-major, dO^ as E5M2 codes row-major
//    and transposed, V as key-major E4M3 codes, and the per row D and
//    LSE log2 e.
//  * dK/dV: one workgroup of 8 waves per 128 keys of a KV head, one key per
//    lane (32 keys per pair of waves on one SIMD); it walks the query heads
//    of its group and the query chunks of 64.  One wave of a pair computes
//    S = Q^ K^T (v_mfma_f32_32x32x16_bf16), P, P~ and dV, its partner dP =
//    dO^ V^T (scaled FP8 MFMA, E5M2 x E4M3), dS, dS~ and dK one chunk
//    behind, with P passed through LDS.  The query rows of Q^ / dO^ are read
//    in the order that makes each S sub-tile one 32-query MX block split
//    16/16 between a lane and lane^32 -- the k-blocks of the FP8 32x32x64
//    operand -- so P~^T is directly the A operand of the dV MFMA with its
//    E8M0 exponents as scale_a; dS~ (rounded to E4M3 and rescaled, exact in
//    bf16) feeds dK on the bf16 MFMA against Q^^T, read from the row-major
//    Q^ tile by transposing LDS reads.
//  * dQ: one workgroup of 8 waves per 256 queries of a head, one query per
//    lane as in the forward; every wave computes S^T, P, dP^T, dS, dS~ and
//    dQ^T for its 32 queries.  K^ / V rows are read so that a lane half
//    holds 32 consecutive keys, which makes the MX blocks of dS~ lane-local;
//    dQ^T accumulates on the bf16 MFMA against K^^T (transposing reads of the
//    row-major K^ tile).
#include <type_traits>

#include "common.h"
#include "bwd_params.h"

namespace attn {

typedef float f32x2 __attribute__((ext_vector_type(2)));

namespace {

constexpr int BWD_ROWS = 128;      // rows (keys or queries) per workgroup
constexpr int BWD_CHUNK = 64;      // rows of the other side per inner step

__device__ inline float bwd_reduce_partials(const float* partials, int np) {
  __shared__ float red[8];
  float m = 0.0f;
  for (int i = threadIdx.x; i < np; i += blockDim.x) m = __builtin_fmaxf(m, partials[i]);
  for (int o = 32; o > 0; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = __builtin_fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// MX E4M3 exponent of a block with maximum magnitude a: floor(log2 a) - 8,
// at least -127; -127 for an empty (all-zero) block.
__device__ inline int mx_e4m3_exponent(float a) {
  if (!(a > 0.0f)) return -127;
  const int e = __builtin_amdgcn_frexp_expf(a) - 1 - 8;   // a = f 2^k, f in [0.5, 1): floor(log2 a) = k - 1
  return e < -127 ? -127 : e;
}

// The float32 whose exponent field is the E8M0 byte e + 127 (2^e; for
// e = -127 the field is 0).  gfx950's scaled conversions take only the
// exponent field of their scale operand.
__device__ inline float e8m0_scale(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// Two values of an MX E4M3 block to codes, written into half HI of w (the
// other half is kept): E4M3 of x 2^-e, rounded to nearest even, saturated at
// +-448 (the MX rule saturates block maxima with a significand of 1.75 +
// 1/16 or more).  v_cvt_scalef32_pk_fp8_f32 divides by the scale and rounds
// but does not saturate, so x is first clamped to +-448 2^e (exact); lim and
// scale are 448 2^e and e8m0_scale(e).
typedef short s16x2 __attribute__((ext_vector_type(2)));
template <bool HI>
__device__ inline s16x2 mx_e4m3_pair(s16x2 w, float x0, float x1, float lim, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, __builtin_amdgcn_fmed3f(x0, -lim, lim),
                                                  __builtin_amdgcn_fmed3f(x1, -lim, lim), scale, HI);
}
// The same into the low half of a new word whose high half is left as
// whatever the register held (the clamped x0: a dead value, so no copy).
__device__ inline s16x2 mx_e4m3_pair_lo(float x0, float x1, float lim, float scale) {
  const float c0 = __builtin_amdgcn_fmed3f(x0, -lim, lim);
  return __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(s16x2, c0), c0,
                                                  __builtin_amdgcn_fmed3f(x1, -lim, lim), scale, false);
}

// The two block values E4M3(code) 2^e of the low pair of w, as two bf16 in
// one word (exact: four significant bits).
__device__ inline uint32_t mx_e4m3_pair_bf16(s16x2 w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(__builtin_bit_cast(uint32_t, w),
                                                                                scale, false));
}

}  // namespace

// ---------------------------------------------------------------------------
// Preparation 1: exact bf16 values of NVFP4 rows (without the tensor scale),
// row-major.  One workgroup per (64 rows, head, batch).
template <int D>
__global__ void __launch_bounds__(256) bwd_expand_kernel(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales, int H, int N,
                                                         int64_t npad, __bf16* __restrict__ rm) {
  constexpr int G8 = D / 8;
  const int r0 = blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z;
  const int64_t head = (int64_t)b * H + h;
  for (int it = threadIdx.x; it < 64 * G8; it += 256) {
    const int row = it / G8, g = it % G8, n = r0 + row;
    bf16x8 val;
    if (n < N) {
      const int64_t src = ((int64_t)b * N + n) * H + h;
      const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + src * (D / 2) + 4 * g);
      const float sv = e4m3_decode(scales[src * (D / 16) + g / 2]);
#pragma unroll
      for (int j = 0; j < 8; ++j) val[j] = (__bf16)(e2m1_decode((cw >> (4 * j)) & 0xFu) * sv);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) val[j] = (__bf16)0.0f;
    }
    *reinterpret_cast<bf16x8*>(rm + (head * npad + n) * D + 8 * g) = val;
  }
}

// Preparation 2: dO^ (E5M2, one scale per tensor), row-major, D = sum_d dO^ O
// and LSE log2 e per row.  One workgroup per (64 rows, head,
// batch); the tensor amax comes from the shared amax pass.
template <int D>
__global__ void __launch_bounds__(256) bwd_do_kernel(const uint16_t* __restrict__ dout, const uint16_t* __restrict__ o,
                                                     const float* __restrict__ lse, const float* __restrict__ partials,
                                                     int np, int H, int N, int64_t npad, uint8_t* __restrict__ drm,
                                                     float* __restrict__ dvec,
                                                     float* __restrict__ lvec, float* __restrict__ sdo) {
  constexpr int G8 = D / 8;
  __shared__ float part[64][G8 + 1];
  const float amax = bwd_reduce_partials(partials, np);
  float enc = amax == 0.0f ? 1.0f : 57344.0f / amax;
  if (__builtin_isinf(enc)) enc = 3.40282347e+38f;
  const float s = 1.0f / enc;
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *sdo = s;
  const int r0 = blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z;
  const int64_t head = (int64_t)b * H + h;
  for (int it = threadIdx.x; it < 64 * G8; it += 256) {
    const int row = it / G8, g = it % G8, n = r0 + row;
    uint32_t w0 = 0u, w1 = 0u;
    float acc = 0.0f;
    if (n < N) {
      const int64_t src = (((int64_t)b * N + n) * H + h) * D + 8 * g;
      const u32x4 dv = *reinterpret_cast<const u32x4*>(dout + src);
      const u32x4 ov = *reinterpret_cast<const u32x4*>(o + src);
      float y[8], ox[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[2 * j] = bf16_bits_to_f32(dv[j] & 0xFFFFu) * enc;
        y[2 * j + 1] = bf16_bits_to_f32(dv[j] >> 16) * enc;
        ox[2 * j] = bf16_bits_to_f32(ov[j] & 0xFFFFu);
        ox[2 * j + 1] = bf16_bits_to_f32(ov[j] >> 16);
      }
      // |y| <= 57344 up to one rounding, so the round-to-nearest-even E5M2
      // conversion cannot reach infinity
      w0 = __builtin_amdgcn_cvt_pk_bf8_f32(y[0], y[1], w0, false);
      w0 = __builtin_amdgcn_cvt_pk_bf8_f32(y[2], y[3], w0, true);
      w1 = __builtin_amdgcn_cvt_pk_bf8_f32(y[4], y[5], w1, false);
      w1 = __builtin_amdgcn_cvt_pk_bf8_f32(y[6], y[7], w1, true);
      const f32x2 d0 = __builtin_amdgcn_cvt_pk_f32_bf8(w0, false), d1 = __builtin_amdgcn_cvt_pk_f32_bf8(w0, true);
      const f32x2 d2 = __builtin_amdgcn_cvt_pk_f32_bf8(w1, false), d3 = __builtin_amdgcn_cvt_pk_f32_bf8(w1, true);
      const float dq[8] = {d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = acc + (dq[j] * s) * ox[j];
    }
    *reinterpret_cast<u32x2*>(drm + (head * npad + n) * D + 8 * g) = u32x2{w0, w1};
    part[row][g] = acc;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int row = threadIdx.x, n = r0 + row;
    float acc = 0.0f;
    for (int g = 0; g < G8; ++g) acc = acc + part[row][g];
    dvec[head * npad + n] = n < N ? acc : 0.0f;
    lvec[head * npad + n] = n < N ? lse[head * N + n] * 1.4426950408889634f : __builtin_inff();
  }
}

// Preparation 3: V codes from the forward's [Hkv][D][cols] layout (cols =
// B * roundup(N, 128)) to key-major [B][Hkv][NPAD][D].
template <int D>
__global__ void __launch_bounds__(256) bwd_v_kernel(const uint8_t* __restrict__ v, int Hkv, int64_t cols,
                                                    int64_t npad, uint8_t* __restrict__ vrm) {
  __shared__ uint8_t tile[D][64 + 16];
  const int r0 = blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z;
  for (int it = threadIdx.x; it < D * 4; it += 256) {
    const int d = it / 4, rg = it % 4;
    const u32x4 w = *reinterpret_cast<const u32x4*>(v + ((int64_t)h * D + d) * cols + (int64_t)b * npad + r0 + 16 * rg);
#pragma unroll
    for (int j = 0; j < 16; ++j) tile[d][16 * rg + j] = (uint8_t)(w[j / 4] >> (8 * (j % 4)));
  }
  __syncthreads();
  const int64_t head = (int64_t)b * Hkv + h;
  for (int it = threadIdx.x; it < 64 * (D / 16); it += 256) {
    const int row = it / (D / 16), g = it % (D / 16);
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)tile[16 * g + 4 * j][row] | ((uint32_t)tile[16 * g + 4 * j + 1][row] << 8) |
             ((uint32_t)tile[16 * g + 4 * j + 2][row] << 16) | ((uint32_t)tile[16 * g + 4 * j + 3][row] << 24);
    *reinterpret_cast<u32x4*>(vrm + (head * npad + r0 + row) * D + 16 * g) = w;
  }
}

// ---------------------------------------------------------------------------
// LDS chunk tiles of the main kernels: 64 rows of the other side (queries for
// dK/dV, keys for dQ) row-major, and their transposes (one row per channel d),
// copied straight from global memory by 1 KB global->LDS copies.  The 16-byte
// chunks of each row are XOR-swizzled instead of padding the rows (a copy
// fills 1 KB of LDS contiguously): chunk c of row R sits at c ^ f(R), with f
// a linear map of the row bits chosen so that every operand read of the
// kernels (16 lanes at a time over 256 bytes, 8 at a time over 128 bytes)
// touches distinct 16-byte bank groups.
//
// dK/dV: A-operand rows R = query perm(m) + 32 s2 of the chunk, with
// perm(m) = 16 ((m>>2)&1) + 4 (m>>3) + (m&3) (bits 0-4 of R vary across a read).
template <int RB>                      // row bytes: 256 (16 chunks), 128 (8), 64 (4)
__device__ __host__ inline int swz_qrows(int R) {
  if (RB == 256) return (R & 3) | (((R >> 4) & 1) << 2) | (((R >> 2) & 1) << 3);
  if (RB == 128) return ((R >> 4) & 1) | (((R >> 1) & 1) << 1) | (((R ^ (R >> 2)) & 1) << 2);
  return ((R >> 4) & 1) | ((((R >> 1) ^ (R >> 2)) & 1) << 1);
}
// The Q^ tile of the dK/dV kernel (rows of 2D bytes) is also read through
// transposing reads (4 consecutive rows x 32 bytes per 16 lanes), which this
// swizzle spreads over the banks as well.
template <int D>
__device__ __host__ inline int swz_qtile(int R) {
  if (D == 128) return (R & 3) | ((((R >> 2) ^ R) & 1) << 2) | ((((R >> 4) ^ (R >> 1)) & 1) << 3);
  return ((R >> 1) & 1) | (((R >> 2) & 1) << 1) | ((((R >> 4) ^ (R >> 1)) & 1) << 2);
}
// transposed tiles: row d = 32 dt + ln read by lanes ln = 0..31 (bits 0-3 vary
// across 16 lanes); 128-byte rows (bf16 x 64) and 64-byte rows (8-bit x 64)
__device__ __host__ inline int swz_drows128(int d) {
  return ((d >> 1) & 1) | (((d >> 2) & 1) << 1) | ((((d >> 3) ^ d) & 1) << 2);
}
__device__ __host__ inline int swz_drows64(int d) { return ((d >> 2) & 1) | ((((d >> 3) ^ (d >> 1)) & 1) << 1); }

// Copy 16 bytes per lane from global memory straight into LDS (lane i writes
// LDS bytes [lds + 16 i, lds + 16 i + 16)); `base` and `lds` wave-uniform,
// `off` a per-lane byte offset below 4 GiB.  Inline assembly, so that the
// compiler inserts no wait for it before unrelated LDS reads; completion is
// awaited with an explicit vmcnt wait.
__device__ inline void bwd_dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(base)
               : "memory");
}
__device__ inline void bwd_dma4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(base)
               : "memory");
}
__device__ inline uint32_t bwd_lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Makes the compiler wait, once, for registers loaded before a step loop.
// The loops' chunk copies are asm, invisible to the compiler's wait counting:
// left pending at the loop header, a pre-loop load would get a vmcnt wait in
// every iteration, which also waits for the copies of the next chunk that the
// iteration has just issued.
template <int N>
__device__ inline void bwd_settle(const u32x4 (&r)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(r[i]));
}
// 16 bytes, and (transposing read) 4 bf16, at an LDS byte address
__device__ inline u32x4 bwd_lds16(uint32_t a) {
  return *(__attribute__((address_space(3))) const u32x4*)(uintptr_t)a;
}

// ---------------------------------------------------------------------------
// dK / dV.  Workgroup: 8 waves for 128 keys kb*128 + 32*kw + (lane & 31) of KV
// head hk, two waves per 32-key block kw, on one SIMD (waves kw and kw + 4):
//   dP side (waves 0-3): dP = dO^ V^T, dS = P (dP - D), dS~ and dK += dS~^T Q^
//   S side (waves 4-7):  S = Q^ K^T, P = 2^(t - L), P~ and dV += P~^T dO^
// The dP side runs one 64-query chunk behind: in step s the S side takes
// chunk s and the dP side chunk s - 1, whose P the S side left in LDS as
// float32 (the dP side's lane l needs exactly the 32 values lane l of its
// partner computed).  One barrier per step, so one wave's matrix products
// overlap its partner's vector work; each wave holds one accumulator and one
// resident operand (K^ or V), so the two fit on one SIMD.  The dP side takes
// the older waves, which win the SIMD's issue arbitration (measured faster
// than the other assignment, when the dP side also issued only its share of
// the copies).
//   LDS: the Q^ chunk row-major in a ring of three (chunk x in slot x % 3:
//   the S side's chunk, the dP side's chunk and the next), read straight for
//   S and through transposing reads (ds_read_b64_tr_b16) as the Q^T operand of
//   dK; dO^ row-major in two buffers, read straight for dP and through 8-bit
//   transposing reads (ds_read_b64_tr_b8) as the dO^ operand of dV; L and P in
//   two buffers each, D in a ring of three.
// S / dP sub-tile s2 of a chunk: accumulator (lane half hh, register r) holds
// query 32*s2 + 16*hh + r of the chunk; A row m of the S / dP products is
// therefore query 32*s2 + 16*((m>>2)&1) + 4*(m>>3) + (m&3).
typedef short s16x4 __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ inline s16x4 bwd_lds_tr8(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)a);
}
// 8-bit transposing read: a 16-lane group reads 8 rows of 16 bytes (row j from
// the addresses of lanes 2j and 2j + 1, 8 bytes each); lane c receives byte c
// of every row
typedef int i32x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2v lds_i32x2;
__device__ inline u32x2 bwd_lds_tr_b8(uint32_t a) {
  const i32x2v r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(uintptr_t)a);
  return u32x2{(uint32_t)r[0], (uint32_t)r[1]};
}

template <int D, bool CAUSAL, bool DEBUG>
__global__ void __launch_bounds__(512, 1) bwd_dkdv_kernel(BwdParams p) {
  constexpr int KS = D / 16, DT = D / 32, KK = D / 64;
  // bytes of one buffer of each chunk tile
  constexpr int QB = BWD_CHUNK * D * 2, DOB = BWD_CHUNK * D;
  constexpr int NQC = QB / 1024, NDOC = DOB / 1024;
  __shared__ __attribute__((aligned(1024))) uint8_t sQ[3][QB];
  __shared__ __attribute__((aligned(1024))) uint8_t sDO[2][DOB];
  __shared__ __attribute__((aligned(16))) float sL[2][BWD_CHUNK];   // read as 16-byte vectors
  __shared__ __attribute__((aligned(16))) float sD[3][BWD_CHUNK];   // chunk x in slot x % 3
  __shared__ __attribute__((aligned(16))) f32x4 sP[2][4][2][4][64];  // [buffer][key block][s2][r / 4][lane]
  int kb = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  if (CAUSAL) {
    // Causal: a key block's work falls with kb.  Dispatch (which follows the
    // linear block index) takes the longest blocks of every head first, kb
    // major; the (batch, KV head) index varies fastest, so with 8 KV heads
    // each XCD (dispatch is round-robin over 8) keeps one KV head.
    const int nh = gridDim.y * gridDim.z;
    const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    kb = lin / nh;
    hk = (lin % nh) % gridDim.y;
    b = (lin % nh) / gridDim.y;
  }
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, ln = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool s_side = wave >= 4;                // uniform
  const int kw = wave & 3;
  const int key = kb * BWD_ROWS + kw * 32 + ln;
  const int G = p.Hq / p.Hkv;
  const int64_t npad = p.npad;
  const int64_t krow = ((int64_t)b * p.Hkv + hk) * npad + key;
  // resident operand, in one register array for both sides (a wave keeps
  // one side for the whole kernel, but the compiler cannot know that): K^ as
  // KS bf16x8 (S side, B operand of S) or V as KK i32x8 (dP side, B operand of dP)
  u32x4 res[KS];
  if (s_side) {
#pragma unroll
    for (int s = 0; s < KS; ++s) res[s] = *reinterpret_cast<const u32x4*>(p.krm + krow * D + 16 * s + 8 * hh);
  } else {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      res[2 * kk] = *reinterpret_cast<const u32x4*>(p.vrm + krow * D + 64 * kk + 16 * hh);
      res[2 * kk + 1] = *reinterpret_cast<const u32x4*>(p.vrm + krow * D + 64 * kk + 32 + 16 * hh);
    }
  }
  auto kop = [&](int st) { return __builtin_bit_cast(bf16x8, res[st]); };
  auto vop = [&](int kk) {
    const u32x4 lo = res[2 * kk], hi = res[2 * kk + 1];
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  f32x16 acc[DT];                               // dV (S side) or dK (dP side)
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x16{};
  const float cc = (float)((double)p.sigma * 1.4426950408889634 * (double)(*p.gq) * (double)(*p.gk));
  const float sdo = *p.sdo;
  const float sdv = sdo * *p.sv;
  const int nchunks = (int)(npad / BWD_CHUNK);
  const int c0 = CAUSAL ? (kb * BWD_ROWS) / BWD_CHUNK : 0;
  const int nch = nchunks - c0;                 // >= 2: the key block's own chunks
  const int total = G * nch;                    // (query head, query chunk) steps of each side
  const int m = ln;

  // ---- chunk copies, issued by the dP side only: wave w < 4 issues copies
  // j = w + 4 t of each tile.  A wave that issues copies stalls until the
  // vector memory path has taken them (32 KB per step and workgroup, at about
  // 64 bytes per clock); with the copies spread over all eight waves the dP
  // side waited at the barrier for the S side every step, so it takes them
  // all (4 % faster than all eight waves issuing).  The per-lane source
  // offsets within a tile are loop invariant.
  constexpr int CW = 4;
  constexpr int NQW = (NQC + CW - 1) / CW, NDOW = (NDOC + CW - 1) / CW;
  uint32_t oqc[NQW], odc[NDOW];
#pragma unroll
  for (int t = 0; t < NQW; ++t) {                          // Q rows: 2D bytes, 1024 / 2D rows per copy
    const int j = kw + CW * t;
    const int r = j * (1024 / (2 * D)) + (16 * lane) / (2 * D), c = ((16 * lane) % (2 * D)) / 16;
    oqc[t] = (uint32_t)(r * 2 * D + 16 * (c ^ swz_qtile<D>(r)));
  }
#pragma unroll
  for (int t = 0; t < NDOW; ++t) {                         // dO rows: D bytes
    const int j = kw + CW * t;
    const int r = j * (1024 / D) + (16 * lane) / D, c = ((16 * lane) % D) / 16;
    odc[t] = (uint32_t)(r * D + 16 * (c ^ swz_qrows<D>(r)));
  }
  auto chunk_row = [&](int g, int c) { return ((int64_t)b * p.Hq + hk * G + g) * npad + (int64_t)c * BWD_CHUNK; };
  // the S side's tiles of chunk (g, c): Q^ -> ring slot, L -> buffer
  auto copy_s = [&](int g, int c, int slot, int buf) {
    const int64_t q0 = chunk_row(g, c);
    const uint8_t* qb0 = reinterpret_cast<const uint8_t*>(p.qrm + q0 * D);
#pragma unroll
    for (int t = 0; t < NQW; ++t) {
      const int j = kw + CW * t;
      if (j < NQC) bwd_dma16(qb0, oqc[t], bwd_lds_address(&sQ[slot][0]) + 1024 * j);
    }
    if (wave == 0) bwd_dma4(p.lv + q0, (uint32_t)(4 * lane), bwd_lds_address(&sL[buf][0]));
  };
  // the dP side's tiles of chunk (g, c): dO^ -> buffer, D -> ring slot
  auto copy_d = [&](int g, int c, int buf, int slot) {
    const int64_t q0 = chunk_row(g, c);
    const uint8_t* db0 = p.dorm + q0 * D;
#pragma unroll
    for (int t = 0; t < NDOW; ++t) {
      const int j = kw + CW * t;
      if (j < NDOC) bwd_dma16(db0, odc[t], bwd_lds_address(&sDO[buf][0]) + 1024 * j);
    }
    if (wave == 1) bwd_dma4(p.dv + q0, (uint32_t)(4 * lane), bwd_lds_address(&sD[slot][0]));
  };
  // per-lane operand read offsets within a tile, as one per-lane base per
  // operand XOR a constant (the chunk index of a read is the swizzle XOR a
  // sum of disjoint bit fields; the tiles are 1024-byte aligned, so the XOR
  // may be applied to the LDS address).  Two bases per side, sharing two
  // registers:
  //   S side  b0: Q row R0, k-step ks: b0 ^ 32 ks (chunk 2 ks + hh)
  //           b1: transposing dO read (t, dt): (b1 + (8 (t & 1) + 32 (t >> 1)) D) ^ 32 dt
  //   dP side b0: dO row R0, (kk, lh): b0 ^ (64 kk + 32 lh) (chunk 4 kk + 2 lh + hh)
  //           b1: transposing Q read (dt, half): lane (g, c) of a 16-lane
  //           group reads 4 bf16 of row 16 (g >> 1) + 4 half + (c >> 2) (+ 32
  //           s2 + r0, which leave the swizzle unchanged) at channel 32 dt + 16
  //           (g & 1) + 4 (c & 3), and the transpose hands it channel 32 dt + 16
  //           (g & 1) + c of 4 rows: (b1 + 8 D half) ^ (64 dt) ^ (half ?
  //           swizzle bit of row bit 2 : 0)
  const int R0 = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);   // A row of the S / dP products
  uint32_t b0, b1;
  if (s_side) {
    b0 = (uint32_t)(R0 * 2 * D + 16 * (hh ^ swz_qtile<D>(R0)));
    // transposing 8-bit reads of the row-major dO^ tile: lane (g, c) of a
    // 16-lane group gives the address of row 16 (g >> 1) + (c >> 1) (+ 8 t0 +
    // 32 t1, which leave the swizzle unchanged), bytes 8 (c & 1) of chunk
    // 2 dt + (g & 1); the transpose hands lane c channel 32 dt + 16 (g & 1) + c
    // of 8 consecutive queries
    const int g4 = lane >> 4, c16 = lane & 15;
    const int R = 16 * (g4 >> 1) + (c16 >> 1);
    b1 = (uint32_t)(R * D + 16 * ((g4 & 1) ^ swz_qrows<D>(R)) + 8 * (c16 & 1));
  } else {
    b0 = (uint32_t)(R0 * D + 16 * (hh ^ swz_qrows<D>(R0)));
    const int g4 = lane >> 4, c16 = lane & 15;
    const int R = 16 * (g4 >> 1) + (c16 >> 2);
    const int byte = 2 * (16 * (g4 & 1) + 4 * (c16 & 3));
    b1 = (uint32_t)(R * 2 * D + 16 * ((byte / 16) ^ swz_qtile<D>(R)) + (byte % 16));
  }
  constexpr uint32_t TR_HALF_X = D == 128 ? 64 : 32;   // 16 x (the swizzle bit that row bit 2 flips)

  const int wkey_last = kb * BWD_ROWS + kw * 32 + 31;
  // prologue: the tiles of chunk 0
  bwd_settle(res);
  if (!s_side) {
    copy_s(0, c0, 0, 0);
    copy_d(0, c0, 0, 0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // Each side runs its own copy of the step loop (one side per wave for the
  // whole kernel; separate loops keep each side's accumulator in place).
  // Both loops take the same number of barriers.  Per step: the copies of
  // chunk step + 1, this side's work, then a barrier once this wave's copies
  // have landed and its LDS writes are done.
  // (g, c): the S side's chunk of step s; (gp, cp): the dP side's (s - 1)
  int g = 0, c = c0, gp = 0, cp = c0;
  auto step_begin = [&](int step, int& gn, int& cn) {
    gn = g;
    cn = c + 1;
    if (cn == nchunks) { cn = c0; ++gn; }
    if (!s_side && step + 1 < total) {
      copy_s(gn, cn, (step + 1) % 3, (step + 1) & 1);
      copy_d(gn, cn, (step + 1) & 1, (step + 1) % 3);
    }
  };
  auto step_end = [&](int gn, int cn) {
    // the copies for step + 1 (this wave's) have landed and this wave's LDS
    // writes are done; after the barrier every wave's are, and the tiles of
    // step - 1 may be overwritten
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    gp = g;
    cp = c;
    g = gn;
    c = cn;
  };
  if (s_side) {
    for (int step = 0; step <= total; ++step) {
      int gn, cn;
      step_begin(step, gn, cn);
      if (step < total) {

        const int buf = step & 1, slot = step % 3;
        const int h = hk * G + g;
        const bool dump = DEBUG && b == p.dbg_b && h == p.dbg_h;
        float pv[2][16];
        float amx[2];
        {
          f32x16 s[2];
          // S of both 32-query sub-tiles: the two accumulation chains
          // alternate, each A operand read from LDS two matrix instructions
          // ahead (fenced); each chain sums its k-steps in order
          const uint32_t qa = bwd_lds_address(&sQ[slot][0]) + b0;
          auto lda = [&](int i) {    // operand i: k-step i / 2 of sub-tile i % 2
            return __builtin_bit_cast(bf16x8, bwd_lds16((qa ^ (32u * (uint32_t)(i >> 1))) + 32 * 2 * D * (i & 1)));
          };
          bf16x8 op[3];
          op[0] = lda(0);
          op[1] = lda(1);
#pragma unroll
          for (int i = 0; i < 2 * KS; ++i) {
            if (i + 2 < 2 * KS) op[(i + 2) % 3] = lda(i + 2);
            const int st = i >> 1, s2 = i & 1;
            s[s2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % 3], kop(st), st == 0 ? f32x16{} : s[s2], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
          // P of (query 32 s2 + 16 hh + r, this lane's key).  Padded query rows
          // have L = +inf (P = 0); keys past the sequence and (causal) keys after
          // the query are masked, which only the block's boundary chunks need.
          const bool all_live = wkey_last < p.N && (!CAUSAL || wkey_last <= c * BWD_CHUNK);
          auto elements = [&](auto masked) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              amx[s2] = 0.0f;
              // query 32 s2 + 16 hh + r is live for this key when r >= thr
              const int thr = key >= p.N ? 16 : (CAUSAL ? key - (c * BWD_CHUNK + 32 * s2 + 16 * hh) : 0);
              f32x4 lr[4];           // the 16 rows' L as four 16-byte reads, issued together
#pragma unroll
              for (int v = 0; v < 4; ++v) lr[v] = *reinterpret_cast<const f32x4*>(&sL[buf][32 * s2 + 16 * hh + 4 * v]);
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[s2][r], cc, -lr[r >> 2][r & 3]));
                if (decltype(masked)::value) pr = r >= thr ? pr : 0.0f;
                pv[s2][r] = pr;
                amx[s2] = __builtin_fmaxf(amx[s2], pr);
              }
            }
          };
          if (all_live) elements(std::false_type{});
          else elements(std::true_type{});
        }
        // P for the dP side (next step)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            sP[buf][kw][s2][v][lane] = f32x4{pv[s2][4 * v], pv[s2][4 * v + 1], pv[s2][4 * v + 2], pv[s2][4 * v + 3]};
        // P~^T as the A operand of dV: bytes 0..15 sub-tile 0, bytes 16..31
        // sub-tile 1 (the k-blocks of the FP8 operand); block maxima over the 32
        // queries of each sub-tile (this lane's 16 and lane^32's 16); lane half
        // hh supplies the exponent of block hh
        int ep[2];
        float limp[2], scp[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const auto wp = __builtin_amdgcn_permlane32_swap(__float_as_uint(amx[s2]), __float_as_uint(amx[s2]), false, false);
          ep[s2] = mx_e4m3_exponent(__builtin_fmaxf(__uint_as_float(wp[0]), __uint_as_float(wp[1])));
          limp[s2] = __builtin_ldexpf(448.0f, ep[s2]);
          scp[s2] = e8m0_scale(ep[s2]);
        }
        i32x8 pa;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int s2 = w >> 2, r = 4 * (w & 3);
          s16x2 t = mx_e4m3_pair_lo(pv[s2][r], pv[s2][r + 1], limp[s2], scp[s2]);
          t = mx_e4m3_pair<true>(t, pv[s2][r + 2], pv[s2][r + 3], limp[s2], scp[s2]);
          pa[w] = __builtin_bit_cast(int, t);
        }
        const int scale_p = (hh ? ep[1] : ep[0]) + 127;
        if (dump) {
#pragma unroll
          for (int w = 0; w < 8; ++w)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int qi = c * BWD_CHUNK + 32 * (w >> 2) + 16 * hh + 4 * (w & 3) + j;
              p.dbg_pt[(int64_t)qi * npad + key] = (uint8_t)((uint32_t)pa[w] >> (8 * j));
            }
          if (hh == 0)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) p.dbg_pt_e[(int64_t)(2 * c + s2) * npad + key] = (uint8_t)(ep[s2] + 127);
        }
        const uint32_t ta = bwd_lds_address(&sDO[buf][0]) + b1;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          // queries 16 hh + [0, 16) and 32 + 16 hh + [0, 16) of channel 32 dt + ln
          u32x2 w[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            w[t] = bwd_lds_tr_b8((ta + (uint32_t)((8 * (t & 1) + 32 * (t >> 1)) * D)) ^ (32u * (uint32_t)dt));
          const i32x8 bb = {(int)w[0][0], (int)w[0][1], (int)w[1][0], (int)w[1][1],
                            (int)w[2][0], (int)w[2][1], (int)w[3][0], (int)w[3][1]};
          // A: P~ (E4M3, format 0) with its block exponents, B: dO^ codes (E5M2, format 1)
          acc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa, bb, acc[dt], 0, 1, 0, scale_p, 0, 127);
        }
      }
      step_end(gn, cn);
    }
  } else {
    // The dP side orders its step vector work first, matrix work last, so that
    // it runs opposite its partner (S products first, then P): step s takes
    // dS, dS~ and dK of chunk s - 1 (with the dP of that chunk, made at the
    // end of step s - 1 and kept in registers), then dP of chunk s.
    f32x16 dp[2];
    for (int step = 0; step <= total; ++step) {
      int gn, cn;
      step_begin(step, gn, cn);
      if (step > 0) {
        // chunk (gp, cp) of step - 1
        const int buf = (step - 1) & 1, slot = (step - 1) % 3;
        const int h = hk * G + gp;
        const bool dump = DEBUG && b == p.dbg_b && h == p.dbg_h;
        float pv[2][16];
        float amx[2];
        // dS = P (dP s - D) of (query 32 s2 + 16 hh + r, this lane's key)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          amx[s2] = 0.0f;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const f32x4 dr = *reinterpret_cast<const f32x4*>(&sD[slot][32 * s2 + 16 * hh + 4 * v]);
            const f32x4 pp = sP[buf][kw][s2][v][lane];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float ds = pp[j] * __builtin_fmaf(dp[s2][4 * v + j], sdv, -dr[j]);
              pv[s2][4 * v + j] = ds;
              amx[s2] = __builtin_fmaxf(amx[s2], __builtin_fabsf(ds));
            }
          }
        }
        // dS~: E4M3 of dS 2^-e (blocks of 32 queries, as for P~), back to
        // float, times 2^e: exact in bf16
        int es[2];
        float lims[2], scs[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const auto ws = __builtin_amdgcn_permlane32_swap(__float_as_uint(amx[s2]), __float_as_uint(amx[s2]), false, false);
          es[s2] = mx_e4m3_exponent(__builtin_fmaxf(__uint_as_float(ws[0]), __uint_as_float(ws[1])));
          lims[s2] = __builtin_ldexpf(448.0f, es[s2]);
          scs[s2] = e8m0_scale(es[s2]);
        }
        if (dump && hh == 0)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) p.dbg_dsk_e[(int64_t)(2 * cp + s2) * npad + key] = (uint8_t)(es[s2] + 127);
        uint32_t dsq[2][8];                       // bf16 pairs
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const s16x2 q2 = mx_e4m3_pair_lo(pv[s2][r], pv[s2][r + 1], lims[s2], scs[s2]);
            dsq[s2][r / 2] = mx_e4m3_pair_bf16(q2, scs[s2]);
            if (dump) {
              const uint32_t wq = __builtin_bit_cast(uint32_t, q2);
              const int qi = cp * BWD_CHUNK + 32 * s2 + 16 * hh + r;
              p.dbg_dsk[(int64_t)qi * npad + key] = (uint8_t)wq;
              p.dbg_dsk[(int64_t)(qi + 1) * npad + key] = (uint8_t)(wq >> 8);
            }
          }
        // dK: k-step j takes queries 32 (j/2) + 16 hh + 8 (j%2) + [0, 8) in both
        // operands; the Q^T operand comes from the row-major Q^ tile by two
        // transposing reads of 4 queries each
        const uint32_t xa = bwd_lds_address(&sQ[slot][0]) + b1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int s2 = j >> 1, r0 = 8 * (j & 1);
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{dsq[s2][r0 / 2], dsq[s2][r0 / 2 + 1],
                                                            dsq[s2][r0 / 2 + 2], dsq[s2][r0 / 2 + 3]});
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const uint32_t rowoff = (32 * s2 + r0) * 2 * D;
            const s16x4 r1 = bwd_lds_tr8((xa ^ (64u * dt)) + rowoff);
            const s16x4 r2 = bwd_lds_tr8(((xa + 8 * D) ^ ((64u * dt) ^ TR_HALF_X)) + rowoff);
            const u32x2 w1 = __builtin_bit_cast(u32x2, r1), w2 = __builtin_bit_cast(u32x2, r2);
            const bf16x8 bq = __builtin_bit_cast(bf16x8, u32x4{w1[0], w1[1], w2[0], w2[1]});
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq, acc[dt], 0, 0, 0);
          }
        }
      }
      if (step < total) {
        // dP of chunk (g, c), both sub-tiles: the two chains alternate, operands one ahead
        const uint32_t da = bwd_lds_address(&sDO[step & 1][0]) + b0;
        auto ldd = [&](int i) {    // operand i: k-step i / 2 of sub-tile i % 2 (two 16-byte halves)
          const int kk = i >> 1, s2 = i & 1;
          const u32x4 lo = bwd_lds16((da ^ (64u * kk)) + 32 * D * s2);
          const u32x4 hi = bwd_lds16((da ^ (64u * kk + 32u)) + 32 * D * s2);
          return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        };
        i32x8 op[2];
        op[0] = ldd(0);
#pragma unroll
        for (int i = 0; i < 2 * KK; ++i) {
          if (i + 1 < 2 * KK) op[(i + 1) & 1] = ldd(i + 1);
          const int kk = i >> 1, s2 = i & 1;
          // A: dO^ codes (E5M2, format 1), B: V codes (E4M3, format 0), unit scales
          dp[s2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op[i & 1], vop(kk), kk == 0 ? f32x16{} : dp[s2], 1,
                                                                  0, 0, 127, 0, 127);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      step_end(gn, cn);
    }
  }
  // C[key row][d]: lane holds d = 32 dt + ln, register r holds key row out_row(r, hh)
  const float f = s_side ? sdo : p.sigma * *p.gq;
  float* out = s_side ? p.dv_out : p.dk_out;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kb * BWD_ROWS + kw * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (kr < p.N) out[(((int64_t)b * p.N + kr) * p.Hkv + hk) * D + 32 * dt + ln] = acc[dt][r] * f;
    }
}

// ---------------------------------------------------------------------------
// dQ tiles: the K^ chunk (rows = keys, 2D bytes) is read straight as the A
// operand of S^T and through transposing reads as the K^T operand of dQ; the V
// chunk (rows = keys, D bytes) straight as the A operand of dP^T.  A rows are
// keys kr0(m) + 16 s2 with kr0(m) = 32 ((m>>2)&1) + 4 (m>>3) + (m&3).
template <int D>
__device__ __host__ inline int swz_ktile(int R) {
  if (D == 128) return (R & 3) | ((((R >> 2) ^ R) & 1) << 2) | ((((R >> 5) ^ (R >> 1)) & 1) << 3);
  return ((R >> 1) & 1) | (((R >> 2) & 1) << 1) | ((((R >> 5) ^ (R >> 1)) & 1) << 2);
}
template <int D>
__device__ __host__ inline int swz_vtile(int R) {
  if (D == 128) return ((R >> 1) & 1) | (((R >> 2) & 1) << 1) | (((R >> 5) & 1) << 2);
  return ((R >> 2) & 1) | (((R >> 5) & 1) << 1);
}

// dQ.  Workgroup: 8 waves for 256 queries qb*256 + 32*w + (lane & 31) of head
// h.  Every wave takes, for its 32 queries and each 64-key chunk,
//   S^T = K^ Q^T, P = 2^(t - L), dP^T = V dO^T, dS = P (dP - D), dS~ and
//   dQ^T += K^T dS~^T,
// with P and dS in its own registers (a lane holds one query and 32 keys of
// it per lane half, so the MX blocks of dS~ are lane-local).  The two waves
// of a SIMD (w and w + 4) run half a step apart: waves 4-7 take the S^T / dP^T
// products of chunk s first, then its vector work and dQ products; waves 0-3
// take the vector work and dQ products of chunk s - 1 first, then the S^T /
// dP^T products of chunk s.  So the vector phase of one wave runs beside the
// matrix phase of the other, with one barrier per step; the waves that start
// with vector work are the older ones, which win the SIMD's issue
// arbitration (about 7 % faster than the other assignment).
// LDS: K^ in a ring of three (chunks s - 1, s and the copy of s + 1), read
// straight (A operand of S^T) and through transposing reads (the K^T operand
// of dQ); V in two buffers.  S^T sub-tile s2 of a 64-key chunk: accumulator
// (lane half hh, register r) holds key 32*hh + 16*s2 + r of the chunk; A row m
// of the S^T / dP^T products is therefore key
// 32*((m>>2)&1) + 16*s2 + 4*(m>>3) + (m&3).
constexpr int BWD_QROWS = 256;     // queries per dQ workgroup

template <int D, bool CAUSAL, bool DEBUG>
__global__ void __launch_bounds__(512, 1) bwd_dq_kernel(BwdParams p) {
  constexpr int KS = D / 16, DT = D / 32, KK = D / 64;
  constexpr int KB = BWD_CHUNK * D * 2, VB = BWD_CHUNK * D;        // bytes of one K^ / V chunk
  constexpr int NKC = KB / 1024, NVC = VB / 1024;
  constexpr int CW = 4;
  constexpr int NKW = (NKC + CW - 1) / CW, NVW = (NVC + CW - 1) / CW;
  __shared__ __attribute__((aligned(1024))) uint8_t sK[3][KB];
  __shared__ __attribute__((aligned(1024))) uint8_t sV[2][VB];
  int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (CAUSAL) {
    // Causal: a query block's work grows with qb.  Dispatch takes the longest
    // blocks first, qb major from the last; within one qb the linear index r
    // = g (B Hkv) + b Hkv + hk puts the query heads g of one KV head's group
    // at the same residue mod 8, i.e. on one XCD, where they share its K / V.
    const int nh = gridDim.y * gridDim.z, G = p.Hq / p.Hkv;
    const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    qb = (int)gridDim.x - 1 - lin / nh;
    const int r = lin % nh, per_g = (int)gridDim.z * p.Hkv;
    const int g = r / per_g;
    b = (r % per_g) / p.Hkv;
    h = ((r % per_g) % p.Hkv) * G + g;
  }
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, ln = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lead = wave >= 4;                  // uniform: matrix products of a chunk first
  const int64_t npad = p.npad;
  const int wq_first = qb * BWD_QROWS + wave * 32;
  const bool wave_live = wq_first < npad;       // the last block may reach past the padded rows
  const int q = wq_first + ln;
  const int hk = h / (p.Hq / p.Hkv);
  const int64_t qrow = ((int64_t)b * p.Hq + h) * npad + (wave_live ? q : 0);
  // resident operands: Q^ as KS bf16x8 (B operand of S^T), dO^ as KK i32x8
  // (B operand of dP^T); L log2 e and D of the lane's query
  u32x4 qres[KS], dres[2 * KK];
  float lrow = 0.0f, drow = 0.0f;
  if (wave_live) {
#pragma unroll
    for (int s = 0; s < KS; ++s) qres[s] = *reinterpret_cast<const u32x4*>(p.qrm + qrow * D + 16 * s + 8 * hh);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      dres[2 * kk] = *reinterpret_cast<const u32x4*>(p.dorm + qrow * D + 64 * kk + 16 * hh);
      dres[2 * kk + 1] = *reinterpret_cast<const u32x4*>(p.dorm + qrow * D + 64 * kk + 32 + 16 * hh);
    }
    lrow = p.lv[qrow];
    drow = p.dv[qrow];
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qres[s] = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 2 * KK; ++s) dres[s] = u32x4{0, 0, 0, 0};
  }
  auto qop = [&](int st) { return __builtin_bit_cast(bf16x8, qres[st]); };
  auto dop = [&](int kk) {
    const u32x4 lo = dres[2 * kk], hi = dres[2 * kk + 1];
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  const float cc = (float)((double)p.sigma * 1.4426950408889634 * (double)(*p.gq) * (double)(*p.gk));
  const float sdv = *p.sdo * *p.sv;
  const int64_t khead = (int64_t)b * p.Hkv + hk;
  int nchunks = (int)(npad / BWD_CHUNK);
  if (CAUSAL) nchunks = min(nchunks, (qb * BWD_QROWS + BWD_QROWS) / BWD_CHUNK);
  // chunks this wave contributes to (causal: keys up to its last query)
  int wchunks = wave_live ? nchunks : 0;
  if (CAUSAL && wave_live) wchunks = min(nchunks, (wq_first + 31) / BWD_CHUNK + 1);
  const int m = ln;

  // ---- chunk copies, issued by waves 0-3 only (copies j = w + 4 t), the
  // waves that start each step with vector work: measured 1 % faster than all
  // eight waves issuing, while waves 4-7 alone (matrix products first) were
  // 23 % slower
  uint32_t okc[NKW], ovc[NVW];
#pragma unroll
  for (int t = 0; t < NKW; ++t) {
    const int j = (wave & 3) + CW * t;
    const int r = j * (1024 / (2 * D)) + (16 * lane) / (2 * D), c = ((16 * lane) % (2 * D)) / 16;
    okc[t] = (uint32_t)(r * 2 * D + 16 * (c ^ swz_ktile<D>(r)));
  }
#pragma unroll
  for (int t = 0; t < NVW; ++t) {
    const int j = (wave & 3) + CW * t;
    const int r = j * (1024 / D) + (16 * lane) / D, c = ((16 * lane) % D) / 16;
    ovc[t] = (uint32_t)(r * D + 16 * (c ^ swz_vtile<D>(r)));
  }
  auto copy_chunk = [&](int c, int slot, int buf) {
    const int64_t k0 = khead * npad + (int64_t)c * BWD_CHUNK;
    const uint8_t* kb0 = reinterpret_cast<const uint8_t*>(p.krm + k0 * D);
    const uint8_t* vb0 = p.vrm + k0 * D;
#pragma unroll
    for (int t = 0; t < NKW; ++t) {
      const int j = (wave & 3) + CW * t;
      if (j < NKC) bwd_dma16(kb0, okc[t], bwd_lds_address(&sK[slot][0]) + 1024 * j);
    }
#pragma unroll
    for (int t = 0; t < NVW; ++t) {
      const int j = (wave & 3) + CW * t;
      if (j < NVC) bwd_dma16(vb0, ovc[t], bwd_lds_address(&sV[buf][0]) + 1024 * j);
    }
  };
  // per-lane operand read offsets within a tile.  The 16-byte chunk index of
  // a read is the swizzle XOR a sum of disjoint bit fields, so each offset is
  // one per-lane base XOR a constant (the tiles are 1024-byte aligned, so the
  // XOR may be applied to the LDS address):
  //   K^ row R0, k-step ks:  kofs ^ 32 ks  (chunk 2 ks + hh)
  //   V row R0, (kk, lh):    vofs ^ (64 kk + 32 lh)  (chunk 4 kk + 2 lh + hh)
  //   transposing K^ read (dt, half): lane (g, c) of a 16-lane group reads 4
  //   bf16 of key row 32 (g >> 1) + 4 half + (c >> 2) (+ 16 s2 + r0, which
  //   leave the swizzle unchanged) at channel 32 dt + 16 (g & 1) + 4 (c & 3),
  //   and the transpose hands it channel 32 dt + 16 (g & 1) + c of 4 keys:
  //   (tofs + 8 D half) ^ (64 dt) ^ (half ? swizzle bit of row bit 2 : 0)
  const int R0 = 32 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);   // A row of the S^T / dP^T products
  const uint32_t kofs = (uint32_t)(R0 * 2 * D + 16 * (hh ^ swz_ktile<D>(R0)));
  const uint32_t vofs = (uint32_t)(R0 * D + 16 * (hh ^ swz_vtile<D>(R0)));
  uint32_t tofs;
  {
    const int g4 = lane >> 4, c16 = lane & 15;
    const int R = 32 * (g4 >> 1) + (c16 >> 2);
    const int byte = 2 * (16 * (g4 & 1) + 4 * (c16 & 3));
    tofs = (uint32_t)(R * 2 * D + 16 * ((byte / 16) ^ swz_ktile<D>(R)) + (byte % 16));
  }
  constexpr uint32_t TR_HALF_X = D == 128 ? 64 : 32;   // 16 x (the swizzle bit that row bit 2 flips)

  // S^T and dP^T of chunk c, both 16-key sub-tiles each: the chains of a
  // product alternate, operands read ahead
  f32x16 s[2], dp[2];
  auto products = [&](int c) {
    const uint32_t ka = bwd_lds_address(&sK[c % 3][0]) + kofs;
    auto lda = [&](int i) {    // operand i: k-step i / 2 of sub-tile i % 2
      return __builtin_bit_cast(bf16x8, bwd_lds16((ka ^ (32u * (uint32_t)(i >> 1))) + 16 * 2 * D * (i & 1)));
    };
    bf16x8 op[3];
    op[0] = lda(0);
    op[1] = lda(1);
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      if (i + 2 < 2 * KS) op[(i + 2) % 3] = lda(i + 2);
      const int st = i >> 1, s2 = i & 1;
      s[s2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % 3], qop(st), st == 0 ? f32x16{} : s[s2], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    const uint32_t va = bwd_lds_address(&sV[c & 1][0]) + vofs;
    auto ldv = [&](int i) {    // operand i: k-step i / 2 of sub-tile i % 2 (two 16-byte halves)
      const int kk = i >> 1, s2 = i & 1;
      const u32x4 lo = bwd_lds16((va ^ (64u * kk)) + 16 * D * s2);
      const u32x4 hi = bwd_lds16((va ^ (64u * kk + 32u)) + 16 * D * s2);
      return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    i32x8 ov[2];
    ov[0] = ldv(0);
#pragma unroll
    for (int i = 0; i < 2 * KK; ++i) {
      if (i + 1 < 2 * KK) ov[(i + 1) & 1] = ldv(i + 1);
      const int kk = i >> 1, s2 = i & 1;
      // A: V codes (E4M3, format 0), B: dO^ codes (E5M2, format 1), unit scales
      dp[s2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ov[i & 1], dop(kk), kk == 0 ? f32x16{} : dp[s2], 0, 1,
                                                              0, 127, 0, 127);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // P, dS, dS~ of chunk c and dQ^T += K^T dS~^T
  f32x16 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x16{};
  auto update = [&](int c) {
    // dS of (this lane's query, key 32 hh + 16 s2 + r); keys past the sequence
    // and (causal) after the query have P = 0, which only the last chunks need
    const bool all_live = c * BWD_CHUNK + BWD_CHUNK <= p.N && (!CAUSAL || c * BWD_CHUNK + BWD_CHUNK - 1 <= wq_first);
    // (dS overwrites dP in place); key 32 hh + 16 s2 + r of the chunk is live
    // when 16 s2 + r < lim
    float am = 0.0f;
    auto elements = [&](auto masked) {
      const int lim = (CAUSAL ? min(p.N, q + 1) : p.N) - (c * BWD_CHUNK + 32 * hh);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[s2][r], cc, -lrow));
          if (decltype(masked)::value) pr = 16 * s2 + r < lim ? pr : 0.0f;
          const float ds = pr * __builtin_fmaf(dp[s2][r], sdv, -drow);
          dp[s2][r] = ds;
          am = __builtin_fmaxf(am, __builtin_fabsf(ds));
        }
    };
    if (all_live) elements(std::false_type{});
    else elements(std::true_type{});
    // dS~: one MX block per lane half
    const int e = mx_e4m3_exponent(am);
    const float lim = __builtin_ldexpf(448.0f, e), sc = e8m0_scale(e);
    const bool dump = DEBUG && b == p.dbg_b && h == p.dbg_h;
    if (dump) p.dbg_dsq_e[(int64_t)q * (npad / 32) + 2 * c + hh] = (uint8_t)(e + 127);
    uint32_t dsq[2][8];                         // bf16 pairs
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const s16x2 q2 = mx_e4m3_pair_lo(dp[s2][r], dp[s2][r + 1], lim, sc);
        dsq[s2][r / 2] = mx_e4m3_pair_bf16(q2, sc);
        if (dump) {
          const uint32_t wq = __builtin_bit_cast(uint32_t, q2);
          const int kj = c * BWD_CHUNK + 32 * hh + 16 * s2 + r;
          p.dbg_dsq[(int64_t)q * npad + kj] = (uint8_t)wq;
          p.dbg_dsq[(int64_t)q * npad + kj + 1] = (uint8_t)(wq >> 8);
        }
      }
    // dQ^T: k-step j takes keys 32 hh + 16 (j/2) + 8 (j%2) + [0, 8) in both
    // operands; K^T from the row-major K^ tile by two transposing reads of 4 keys
    const uint32_t kt = bwd_lds_address(&sK[c % 3][0]) + tofs;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s2 = j >> 1, r0 = 8 * (j & 1);
      const bf16x8 bv = __builtin_bit_cast(bf16x8, u32x4{dsq[s2][r0 / 2], dsq[s2][r0 / 2 + 1],
                                                         dsq[s2][r0 / 2 + 2], dsq[s2][r0 / 2 + 3]});
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint32_t rowoff = (16 * s2 + r0) * 2 * D;
        const s16x4 r1 = bwd_lds_tr8((kt ^ (64u * dt)) + rowoff);
        const s16x4 r2 = bwd_lds_tr8(((kt + 8 * D) ^ ((64u * dt) ^ TR_HALF_X)) + rowoff);
        const u32x2 w1 = __builtin_bit_cast(u32x2, r1), w2 = __builtin_bit_cast(u32x2, r2);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{w1[0], w1[1], w2[0], w2[1]});
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc[dt], 0, 0, 0);
      }
    }
  };

  bwd_settle(qres);
  bwd_settle(dres);
  asm volatile("" ::"v"(lrow), "v"(drow));
  if (!lead) copy_chunk(0, 0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  auto step_end = [&]() {
    // this wave's copies for the next step have landed and its LDS writes are
    // done; after the barrier every wave's are, and the tiles of step - 2 may
    // be overwritten
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // Each group runs its own copy of the step loop (separate loops keep the
  // accumulators in place); both take nchunks + 1 barriers.
  if (lead) {
    for (int c = 0; c <= nchunks; ++c) {
      if (c < wchunks) {
        products(c);
        update(c);
      }
      step_end();
    }
  } else {
    for (int c = 0; c <= nchunks; ++c) {
      if (c + 1 < nchunks) copy_chunk(c + 1, (c + 1) % 3, (c + 1) & 1);
      if (c > 0 && c - 1 < wchunks) update(c - 1);
      if (c < wchunks) products(c);
      step_end();
    }
  }
  // C[d row][query]: lane holds the query, register r holds d = 32 dt + out_row(r, hh)
  if (wave_live && q < p.N) {
    const float fq = p.sigma * *p.gk;
    float* out = p.dq_out + (((int64_t)b * p.N + q) * p.Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) out[32 * dt + 8 * (r >> 2) + 4 * hh + (r & 3)] = acc[dt][r] * fq;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_bwd_prep(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                           const uint8_t* k_scales, const uint8_t* v_codes, int64_t v_cols, const void* dout,
                           const void* o, const float* lse, const float* partials, int np, int B, int Hq, int Hkv,
                           int N, int D, int64_t npad, __bf16* qrm, __bf16* krm,
                           uint8_t* vrm, uint8_t* drm, float* dvec, float* lvec, float* sdo, hipStream_t st) {
  const dim3 gq((unsigned)(npad / 64), (unsigned)Hq, (unsigned)B), gk((unsigned)(npad / 64), (unsigned)Hkv, (unsigned)B);
  if (D == 64) {
    hipLaunchKernelGGL(bwd_expand_kernel<64>, gq, dim3(256), 0, st, q_codes, q_scales, Hq, N, npad, qrm);
    hipLaunchKernelGGL(bwd_expand_kernel<64>, gk, dim3(256), 0, st, k_codes, k_scales, Hkv, N, npad, krm);
    hipLaunchKernelGGL(bwd_v_kernel<64>, gk, dim3(256), 0, st, v_codes, Hkv, v_cols, npad, vrm);
    hipLaunchKernelGGL(bwd_do_kernel<64>, gq, dim3(256), 0, st, (const uint16_t*)dout, (const uint16_t*)o, lse,
                       partials, np, Hq, N, npad, drm, dvec, lvec, sdo);
  } else {
    hipLaunchKernelGGL(bwd_expand_kernel<128>, gq, dim3(256), 0, st, q_codes, q_scales, Hq, N, npad, qrm);
    hipLaunchKernelGGL(bwd_expand_kernel<128>, gk, dim3(256), 0, st, k_codes, k_scales, Hkv, N, npad, krm);
    hipLaunchKernelGGL(bwd_v_kernel<128>, gk, dim3(256), 0, st, v_codes, Hkv, v_cols, npad, vrm);
    hipLaunchKernelGGL(bwd_do_kernel<128>, gq, dim3(256), 0, st, (const uint16_t*)dout, (const uint16_t*)o, lse,
                       partials, np, Hq, N, npad, drm, dvec, lvec, sdo);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_main(const BwdParams& p, int D, bool causal, bool debug, hipStream_t st) {
  const dim3 gkv((unsigned)(p.npad / BWD_ROWS), (unsigned)p.Hkv, (unsigned)p.B);
  const dim3 gq((unsigned)((p.npad + BWD_QROWS - 1) / BWD_QROWS), (unsigned)p.Hq, (unsigned)p.B);
#define BWD_LAUNCH(DD, C, G)                                                         \
  do {                                                                               \
    hipLaunchKernelGGL((bwd_dkdv_kernel<DD, C, G>), gkv, dim3(512), 0, st, p);       \
    hipLaunchKernelGGL((bwd_dq_kernel<DD, C, G>), gq, dim3(512), 0, st, p);          \
  } while (0)
  if (debug) {
    if (D == 64) {
      if (causal) BWD_LAUNCH(64, true, true); else BWD_LAUNCH(64, false, true);
    } else {
      if (causal) BWD_LAUNCH(128, true, true); else BWD_LAUNCH(128, false, true);
    }
  } else {
    if (D == 64) {
      if (causal) BWD_LAUNCH(64, true, false); else BWD_LAUNCH(64, false, false);
    } else {
      if (causal) BWD_LAUNCH(128, true, false); else BWD_LAUNCH(128, false, false);
    }
  }
#undef BWD_LAUNCH
  return hipGetLastError();
}

}  // namespace attn
