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
//    most 6 significant bits: exact) row-major and transposed, dO^ as E5M2
//    codes row-major and transposed, V as key-major E4M3 codes, and the per
//    row D and LSE log2 e.
//  * dK/dV: one workgroup of 4 waves per 128 keys of a KV head, one key per
//    lane (32 keys per wave); it walks the query heads of its group and the
//    query chunks of 64.  S = Q^ K^T runs on v_mfma_f32_32x32x16_bf16 and
//    dP = dO^ V^T on the scaled FP8 MFMA (E5M2 x E4M3), with the query rows
//    of Q^ / dO^ read in the order that makes each S sub-tile one 32-query MX
//    block split 16/16 between a lane and lane^32 -- the k-blocks of the
//    FP8 32x32x64 operand.  P~^T is then directly the A operand of the dV
//    MFMA with its E8M0 exponents as scale_a; dS~ (rounded to E4M3 and
//    rescaled, exact in bf16) feeds dK on the bf16 MFMA against Q^^T.
//  * dQ: one workgroup of 4 waves per 128 queries of a head, one query per
//    lane as in the forward; K^ / V rows are read so that a lane half holds
//    32 consecutive keys, which makes the MX blocks of dS~ lane-local; dQ^T
//    accumulates on the bf16 MFMA against K^^T.
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

// 16 bytes at base + off: base wave-uniform, off a per-lane byte offset below
// 4 GiB (a scalar base plus a 32-bit vector offset in the load).
__device__ inline u32x4 load16(const void* base, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(base) + off);
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

// The two block values E4M3(code) 2^e of the low pair of w, as two bf16 in
// one word (exact: four significant bits).
__device__ inline uint32_t mx_e4m3_pair_bf16(s16x2 w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(__builtin_bit_cast(uint32_t, w),
                                                                                scale, false));
}

}  // namespace

// ---------------------------------------------------------------------------
// Preparation 1: exact bf16 values of NVFP4 rows (without the tensor scale),
// row-major and transposed.  One workgroup per (64 rows, head, batch).
template <int D>
__global__ void __launch_bounds__(256) bwd_expand_kernel(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales, int H, int N,
                                                         int64_t npad, __bf16* __restrict__ rm,
                                                         __bf16* __restrict__ tr) {
  constexpr int G8 = D / 8;
  __shared__ __bf16 tile[64][D + 8];
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
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[row][8 * g + j] = val[j];
  }
  __syncthreads();
  for (int it = threadIdx.x; it < D * 8; it += 256) {
    const int d = it / 8, rg = it % 8;
    bf16x8 val;
#pragma unroll
    for (int j = 0; j < 8; ++j) val[j] = tile[8 * rg + j][d];
    *reinterpret_cast<bf16x8*>(tr + (head * D + d) * npad + r0 + 8 * rg) = val;
  }
}

// Preparation 2: dO^ (E5M2, one scale per tensor), row-major and transposed,
// D = sum_d dO^ O and LSE log2 e per row.  One workgroup per (64 rows, head,
// batch); the tensor amax comes from the shared amax pass.
template <int D>
__global__ void __launch_bounds__(256) bwd_do_kernel(const uint16_t* __restrict__ dout, const uint16_t* __restrict__ o,
                                                     const float* __restrict__ lse, const float* __restrict__ partials,
                                                     int np, int H, int N, int64_t npad, uint8_t* __restrict__ drm,
                                                     uint8_t* __restrict__ dtr, float* __restrict__ dvec,
                                                     float* __restrict__ lvec, float* __restrict__ sdo) {
  constexpr int G8 = D / 8;
  __shared__ uint8_t tile[64][D + 16];
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
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[row][8 * g + j] = (uint8_t)(w0 >> (8 * j));
      tile[row][8 * g + 4 + j] = (uint8_t)(w1 >> (8 * j));
    }
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
  for (int it = threadIdx.x; it < D * 4; it += 256) {
    const int d = it / 4, rg = it % 4;
    u32x4 val;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      val[j] = (uint32_t)tile[16 * rg + 4 * j][d] | ((uint32_t)tile[16 * rg + 4 * j + 1][d] << 8) |
               ((uint32_t)tile[16 * rg + 4 * j + 2][d] << 16) | ((uint32_t)tile[16 * rg + 4 * j + 3][d] << 24);
    *reinterpret_cast<u32x4*>(dtr + (head * D + d) * npad + r0 + 16 * rg) = val;
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
// dK / dV.  Workgroup: 4 waves, keys kb*128 + 32*wave + (lane & 31) of KV
// head hk.  S sub-tile s2 of a 64-query chunk: accumulator (lane half hh,
// register r) holds query 32*s2 + 16*hh + r of the chunk; A row m of the S /
// dP products is therefore query 32*s2 + 16*((m>>2)&1) + 4*(m>>3) + (m&3).
template <int D, bool CAUSAL, bool DEBUG>
__global__ void __launch_bounds__(256, 1) bwd_dkdv_kernel(BwdParams p) {
  constexpr int KS = D / 16, DT = D / 32, KK = D / 64;
  // LDS rows padded by 16 bytes (row strides of 256k + 16 bytes spread the
  // permuted-row operand reads over all banks)
  constexpr int QS = D + 8, QTS = BWD_CHUNK + 8;          // bf16 elements
  constexpr int DS = D + 16, DTS = BWD_CHUNK + 16;        // bytes
  __shared__ __attribute__((aligned(16))) __bf16 sQ[2][BWD_CHUNK * QS];
  __shared__ __attribute__((aligned(16))) __bf16 sQT[2][D * QTS];
  __shared__ __attribute__((aligned(16))) uint8_t sDO[2][BWD_CHUNK * DS];
  __shared__ __attribute__((aligned(16))) uint8_t sDOT[2][D * DTS];
  __shared__ __attribute__((aligned(16))) float sL[2][BWD_CHUNK];   // read as 16-byte vectors
  __shared__ __attribute__((aligned(16))) float sD[2][BWD_CHUNK];
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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5, ln = lane & 31;
  const int key = kb * BWD_ROWS + wave * 32 + ln;
  const int G = p.Hq / p.Hkv;
  const int64_t npad = p.npad;
  const int64_t krow = ((int64_t)b * p.Hkv + hk) * npad + key;
  bf16x8 kreg[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) kreg[s] = *reinterpret_cast<const bf16x8*>(p.krm + krow * D + 16 * s + 8 * hh);
  i32x8 vreg[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(p.vrm + krow * D + 64 * kk + 16 * hh);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(p.vrm + krow * D + 64 * kk + 32 + 16 * hh);
    vreg[kk] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  f32x16 dv[DT], dk[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) { dv[i] = f32x16{}; dk[i] = f32x16{}; }
  const float cc = (float)((double)p.sigma * 1.4426950408889634 * (double)(*p.gq) * (double)(*p.gk));
  const float sdo = *p.sdo;
  const float sdv = sdo * *p.sv;
  const int nchunks = (int)(npad / BWD_CHUNK);
  const int c0 = CAUSAL ? (kb * BWD_ROWS) / BWD_CHUNK : 0;
  const int nch = nchunks - c0;                 // >= 2: the key block's own chunks
  const int total = G * nch;                    // (query head, query chunk) steps
  const int m = ln;
  // Chunk copies are double-buffered through registers: the global loads of
  // step it + 1 are issued before the matrix work of step it and stored to
  // the other LDS buffer after it (one barrier per step).
  constexpr int NQ = BWD_CHUNK * D / 8 / 256, NQT = D * (BWD_CHUNK / 8) / 256;
  constexpr int NDO = BWD_CHUNK * D / 16 / 256, NDOT = D * (BWD_CHUNK / 16) / 256;
  u32x4 pq[NQ], pqt[NQT], pdo[NDO], pdot[NDOT];
  float pl = 0.0f, pd = 0.0f;
  // per-lane byte offsets of the chunk copies (loop invariant; the chunk and
  // head go into the wave-uniform base of each load)
  uint32_t oq[NQ], oqt[NQT], odo[NDO], odot[NDOT];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int it = tid + 256 * i, row = it / (D / 8), g8 = it % (D / 8);
    oq[i] = (uint32_t)(row * D + 8 * g8) * 2u;
  }
#pragma unroll
  for (int i = 0; i < NQT; ++i) {
    const int it = tid + 256 * i, d = it / (BWD_CHUNK / 8), r8 = it % (BWD_CHUNK / 8);
    oqt[i] = ((uint32_t)d * (uint32_t)npad + 8u * r8) * 2u;
  }
#pragma unroll
  for (int i = 0; i < NDO; ++i) {
    const int it = tid + 256 * i, row = it / (D / 16), g16 = it % (D / 16);
    odo[i] = (uint32_t)(row * D + 16 * g16);
  }
#pragma unroll
  for (int i = 0; i < NDOT; ++i) {
    const int it = tid + 256 * i, d = it / (BWD_CHUNK / 16), r16 = it % (BWD_CHUNK / 16);
    odot[i] = (uint32_t)d * (uint32_t)npad + 16u * r16;
  }
  auto fetch = [&](int step) {
    const int g = step / nch, c = c0 + step % nch;
    const int64_t qhead = (int64_t)b * p.Hq + hk * G + g;
    const int64_t q0 = qhead * npad + (int64_t)c * BWD_CHUNK;
    const __bf16* qb0 = p.qrm + q0 * D;
    const __bf16* qtb0 = p.qt + qhead * D * npad + (int64_t)c * BWD_CHUNK;
    const uint8_t* db0 = p.dorm + q0 * D;
    const uint8_t* dtb0 = p.dot + qhead * D * npad + (int64_t)c * BWD_CHUNK;
#pragma unroll
    for (int i = 0; i < NQ; ++i) pq[i] = load16(qb0, oq[i]);
#pragma unroll
    for (int i = 0; i < NQT; ++i) pqt[i] = load16(qtb0, oqt[i]);
#pragma unroll
    for (int i = 0; i < NDO; ++i) pdo[i] = load16(db0, odo[i]);
#pragma unroll
    for (int i = 0; i < NDOT; ++i) pdot[i] = load16(dtb0, odot[i]);
    if (tid < BWD_CHUNK) {
      pl = p.lv[q0 + tid];
      pd = p.dv[q0 + tid];
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int it = tid + 256 * i, row = it / (D / 8), g8 = it % (D / 8);
      *reinterpret_cast<u32x4*>(&sQ[buf][row * QS + 8 * g8]) = pq[i];
    }
#pragma unroll
    for (int i = 0; i < NQT; ++i) {
      const int it = tid + 256 * i, d = it / (BWD_CHUNK / 8), r8 = it % (BWD_CHUNK / 8);
      *reinterpret_cast<u32x4*>(&sQT[buf][d * QTS + 8 * r8]) = pqt[i];
    }
#pragma unroll
    for (int i = 0; i < NDO; ++i) {
      const int it = tid + 256 * i, row = it / (D / 16), g16 = it % (D / 16);
      *reinterpret_cast<u32x4*>(&sDO[buf][row * DS + 16 * g16]) = pdo[i];
    }
#pragma unroll
    for (int i = 0; i < NDOT; ++i) {
      const int it = tid + 256 * i, d = it / (BWD_CHUNK / 16), r16 = it % (BWD_CHUNK / 16);
      *reinterpret_cast<u32x4*>(&sDOT[buf][d * DTS + 16 * r16]) = pdot[i];
    }
    if (tid < BWD_CHUNK) {
      sL[buf][tid] = pl;
      sD[buf][tid] = pd;
    }
  };
  fetch(0);
  store(0);
  __syncthreads();
  for (int step = 0; step < total; ++step) {
    const int g = step / nch, c = c0 + step % nch, buf = step & 1;
    const int h = hk * G + g;
    fetch(step + 1 < total ? step + 1 : step);
    {
      f32x16 s[2], dp[2];
      // S of both 32-query sub-tiles: the two accumulation chains alternate,
      // and each A operand is read from LDS two matrix instructions ahead
      // (fenced), so that no read's latency is waited out right before its
      // use; each chain still sums its k-steps in order
      {
        const __bf16* qa = &sQ[buf][(16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3)) * QS + 8 * hh];
        auto lda = [&](int i) {    // operand i: k-step i / 2 of sub-tile i % 2
          return *reinterpret_cast<const bf16x8*>(qa + 32 * (i & 1) * QS + 16 * (i >> 1));
        };
        bf16x8 op[3];
        op[0] = lda(0);
        op[1] = lda(1);
#pragma unroll
        for (int i = 0; i < 2 * KS; ++i) {
          if (i + 2 < 2 * KS) op[(i + 2) % 3] = lda(i + 2);
          const int st = i >> 1, s2 = i & 1;
          s[s2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % 3], kreg[st], st == 0 ? f32x16{} : s[s2], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // dP likewise: the two sub-tiles' chains alternate, operands one ahead
      {
        const uint8_t* da = &sDO[buf][(16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3)) * DS + 16 * hh];
        auto ldd = [&](int i) {    // operand i: k-step i / 2 of sub-tile i % 2 (two 16-byte halves)
          const uint8_t* r = da + 32 * (i & 1) * DS + 64 * (i >> 1);
          const u32x4 lo = *reinterpret_cast<const u32x4*>(r);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(r + 32);
          return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        };
        i32x8 op[2];
        op[0] = ldd(0);
#pragma unroll
        for (int i = 0; i < 2 * KK; ++i) {
          if (i + 1 < 2 * KK) op[(i + 1) & 1] = ldd(i + 1);
          const int kk = i >> 1, s2 = i & 1;
          // A: dO^ codes (E5M2, format 1), B: V codes (E4M3, format 0), unit scales
          dp[s2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op[i & 1], vreg[kk], kk == 0 ? f32x16{} : dp[s2], 1,
                                                                  0, 0, 127, 0, 127);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // P and dS of (query 32 s2 + 16 hh + r, this lane's key).  Padded query
      // rows have L = +inf (P = 0); keys past the sequence and (causal) keys
      // after the query are masked, which only the wave's boundary chunks need.
      float pv[2][16], dsv[2][16];
      float amp[2], ams[2];
      const int wkey_last = kb * BWD_ROWS + wave * 32 + 31;
      const bool all_live = wkey_last < p.N && (!CAUSAL || wkey_last <= c * BWD_CHUNK);
      auto elements = [&](auto masked) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          amp[s2] = 0.0f;
          ams[s2] = 0.0f;
          // the 16 rows' L and D as four 16-byte reads each, issued together
          f32x4 lr[4], dr[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            lr[v] = *reinterpret_cast<const f32x4*>(&sL[buf][32 * s2 + 16 * hh + 4 * v]);
            dr[v] = *reinterpret_cast<const f32x4*>(&sD[buf][32 * s2 + 16 * hh + 4 * v]);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ql = 32 * s2 + 16 * hh + r, qi = c * BWD_CHUNK + ql;
            float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[s2][r], cc, -lr[r >> 2][r & 3]));
            if (decltype(masked)::value) pr = (key < p.N && (!CAUSAL || key <= qi)) ? pr : 0.0f;
            const float ds = pr * __builtin_fmaf(dp[s2][r], sdv, -dr[r >> 2][r & 3]);
            pv[s2][r] = pr;
            dsv[s2][r] = ds;
            amp[s2] = __builtin_fmaxf(amp[s2], pr);
            ams[s2] = __builtin_fmaxf(ams[s2], __builtin_fabsf(ds));
          }
        }
      };
      if (all_live) elements(std::false_type{});
      else elements(std::true_type{});
      // block maxima over the 32 queries of each sub-tile: this lane's 16 and lane^32's 16
      int ep[2], es[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const auto wp = __builtin_amdgcn_permlane32_swap(__float_as_uint(amp[s2]), __float_as_uint(amp[s2]), false, false);
        const auto ws = __builtin_amdgcn_permlane32_swap(__float_as_uint(ams[s2]), __float_as_uint(ams[s2]), false, false);
        ep[s2] = mx_e4m3_exponent(__builtin_fmaxf(__uint_as_float(wp[0]), __uint_as_float(wp[1])));
        es[s2] = mx_e4m3_exponent(__builtin_fmaxf(__uint_as_float(ws[0]), __uint_as_float(ws[1])));
      }
      // P~^T as the A operand of dV: bytes 0..15 sub-tile 0, bytes 16..31 sub-tile 1 (the
      // k-blocks of the FP8 operand); lane half hh supplies the exponent of block hh
      i32x8 pa;
      float limp[2], scp[2], lims[2], scs[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        limp[s2] = __builtin_ldexpf(448.0f, ep[s2]);
        scp[s2] = e8m0_scale(ep[s2]);
        lims[s2] = __builtin_ldexpf(448.0f, es[s2]);
        scs[s2] = e8m0_scale(es[s2]);
      }
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int s2 = w >> 2, r = 4 * (w & 3);
        s16x2 t = {0, 0};
        t = mx_e4m3_pair<false>(t, pv[s2][r], pv[s2][r + 1], limp[s2], scp[s2]);
        t = mx_e4m3_pair<true>(t, pv[s2][r + 2], pv[s2][r + 3], limp[s2], scp[s2]);
        pa[w] = __builtin_bit_cast(int, t);
      }
      const int scale_p = (hh ? ep[1] : ep[0]) + 127;
      const bool dump = DEBUG && b == p.dbg_b && h == p.dbg_h;
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
          for (int s2 = 0; s2 < 2; ++s2) {
            p.dbg_pt_e[(int64_t)(2 * c + s2) * npad + key] = (uint8_t)(ep[s2] + 127);
            p.dbg_dsk_e[(int64_t)(2 * c + s2) * npad + key] = (uint8_t)(es[s2] + 127);
          }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 32 * dt + ln;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(&sDOT[buf][d * DTS + 16 * hh]);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(&sDOT[buf][d * DTS + 32 + 16 * hh]);
        const i32x8 bb = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        // A: P~ (E4M3, format 0) with its block exponents, B: dO^ codes (E5M2, format 1)
        dv[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa, bb, dv[dt], 0, 1, 0, scale_p, 0, 127);
      }
      // dS~: E4M3 of dS 2^-e (same blocks), back to float, times 2^e: exact in bf16
      uint32_t dsq[2][8];                       // bf16 pairs
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const s16x2 q2 = mx_e4m3_pair<false>(s16x2{0, 0}, dsv[s2][r], dsv[s2][r + 1], lims[s2], scs[s2]);
          dsq[s2][r / 2] = mx_e4m3_pair_bf16(q2, scs[s2]);
          if (dump) {
            const uint32_t wq = __builtin_bit_cast(uint32_t, q2);
            const int qi = c * BWD_CHUNK + 32 * s2 + 16 * hh + r;
            p.dbg_dsk[(int64_t)qi * npad + key] = (uint8_t)wq;
            p.dbg_dsk[(int64_t)(qi + 1) * npad + key] = (uint8_t)(wq >> 8);
          }
        }
      // dK: k-step j takes queries 32 (j/2) + 16 hh + 8 (j%2) + [0, 8) in both operands
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s2 = j >> 1, r0 = 8 * (j & 1);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{dsq[s2][r0 / 2], dsq[s2][r0 / 2 + 1],
                                                          dsq[s2][r0 / 2 + 2], dsq[s2][r0 / 2 + 3]});
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int d = 32 * dt + ln;
          const bf16x8 bq = *reinterpret_cast<const bf16x8*>(&sQT[buf][d * QTS + 32 * s2 + 16 * hh + r0]);
          dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq, dk[dt], 0, 0, 0);
        }
      }
    }
    store(buf ^ 1);
    __syncthreads();
  }
  // C[key row][d]: lane holds d = 32 dt + ln, register r holds key row out_row(r, hh)
  const float fk = p.sigma * *p.gq;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kb * BWD_ROWS + wave * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (kr < p.N) {
        const int64_t o = (((int64_t)b * p.N + kr) * p.Hkv + hk) * D + 32 * dt + ln;
        p.dv_out[o] = dv[dt][r] * sdo;
        p.dk_out[o] = dk[dt][r] * fk;
      }
    }
}

// ---------------------------------------------------------------------------
// dQ.  Workgroup: 4 waves, queries qb*128 + 32*wave + (lane & 31) of head h.
// S^T sub-tile s2 of a 64-key chunk: accumulator (lane half hh, register r)
// holds key 32*hh + 16*s2 + r of the chunk; A row m of the S^T / dP^T
// products is therefore key 32*((m>>2)&1) + 16*s2 + 4*(m>>3) + (m&3).
template <int D, bool CAUSAL, bool DEBUG>
__global__ void __launch_bounds__(256, 1) bwd_dq_kernel(BwdParams p) {
  constexpr int KS = D / 16, DT = D / 32, KK = D / 64;
  constexpr int KSR = D + 8, KTS = BWD_CHUNK + 8;         // padded row strides (bf16 elements)
  constexpr int VS = D + 16;                              // bytes
  __shared__ __attribute__((aligned(16))) __bf16 sK[2][BWD_CHUNK * KSR];
  __shared__ __attribute__((aligned(16))) __bf16 sKT[2][D * KTS];
  __shared__ __attribute__((aligned(16))) uint8_t sV[2][BWD_CHUNK * VS];
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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5, ln = lane & 31;
  const int q = qb * BWD_ROWS + wave * 32 + ln;
  const int hk = h / (p.Hq / p.Hkv);
  const int64_t npad = p.npad;
  const int64_t qrow = ((int64_t)b * p.Hq + h) * npad + q;
  bf16x8 qreg[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(p.qrm + qrow * D + 16 * s + 8 * hh);
  i32x8 doreg[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(p.dorm + qrow * D + 64 * kk + 16 * hh);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(p.dorm + qrow * D + 64 * kk + 32 + 16 * hh);
    doreg[kk] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  const float lq = p.lv[qrow], dq_d = p.dv[qrow];
  f32x16 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x16{};
  const float cc = (float)((double)p.sigma * 1.4426950408889634 * (double)(*p.gq) * (double)(*p.gk));
  const float sdv = *p.sdo * *p.sv;
  const int64_t khead = (int64_t)b * p.Hkv + hk;
  int nchunks = (int)(npad / BWD_CHUNK);
  if (CAUSAL) nchunks = min(nchunks, (qb * BWD_ROWS + BWD_ROWS) / BWD_CHUNK);
  const int m = ln;
  // chunk copies double-buffered through registers, as in the dK/dV kernel
  constexpr int NK = BWD_CHUNK * D / 8 / 256, NKT = D * (BWD_CHUNK / 8) / 256, NV = BWD_CHUNK * D / 16 / 256;
  u32x4 pk[NK], pkt[NKT], pv4[NV];
  uint32_t ok[NK], okt[NKT], ov[NV];               // per-lane byte offsets (loop invariant)
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int it = tid + 256 * i, row = it / (D / 8), g8 = it % (D / 8);
    ok[i] = (uint32_t)(row * D + 8 * g8) * 2u;
  }
#pragma unroll
  for (int i = 0; i < NKT; ++i) {
    const int it = tid + 256 * i, d = it / (BWD_CHUNK / 8), r8 = it % (BWD_CHUNK / 8);
    okt[i] = ((uint32_t)d * (uint32_t)npad + 8u * r8) * 2u;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int it = tid + 256 * i, row = it / (D / 16), g16 = it % (D / 16);
    ov[i] = (uint32_t)(row * D + 16 * g16);
  }
  auto fetch = [&](int c) {
    const int64_t k0 = khead * npad + (int64_t)c * BWD_CHUNK;
    const __bf16* kb0 = p.krm + k0 * D;
    const __bf16* ktb0 = p.kt + khead * D * npad + (int64_t)c * BWD_CHUNK;
    const uint8_t* vb0 = p.vrm + k0 * D;
#pragma unroll
    for (int i = 0; i < NK; ++i) pk[i] = load16(kb0, ok[i]);
#pragma unroll
    for (int i = 0; i < NKT; ++i) pkt[i] = load16(ktb0, okt[i]);
#pragma unroll
    for (int i = 0; i < NV; ++i) pv4[i] = load16(vb0, ov[i]);
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int it = tid + 256 * i, row = it / (D / 8), g8 = it % (D / 8);
      *reinterpret_cast<u32x4*>(&sK[buf][row * KSR + 8 * g8]) = pk[i];
    }
#pragma unroll
    for (int i = 0; i < NKT; ++i) {
      const int it = tid + 256 * i, d = it / (BWD_CHUNK / 8), r8 = it % (BWD_CHUNK / 8);
      *reinterpret_cast<u32x4*>(&sKT[buf][d * KTS + 8 * r8]) = pkt[i];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int it = tid + 256 * i, row = it / (D / 16), g16 = it % (D / 16);
      *reinterpret_cast<u32x4*>(&sV[buf][row * VS + 16 * g16]) = pv4[i];
    }
  };
  fetch(0);
  store(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    fetch(c + 1 < nchunks ? c + 1 : c);

    f32x16 s[2], dp[2];
    // S^T and dP^T of both 16-key sub-tiles, as in the dK/dV kernel: the two
    // accumulation chains alternate and each A operand is read from LDS ahead
    // of its matrix instruction (fenced); each chain sums its k-steps in order
    {
      const int kr0 = 32 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
      const __bf16* ka = &sK[buf][kr0 * KSR + 8 * hh];
      auto lda = [&](int i) {      // operand i: k-step i / 2 of sub-tile i % 2
        return *reinterpret_cast<const bf16x8*>(ka + 16 * (i & 1) * KSR + 16 * (i >> 1));
      };
      bf16x8 op[3];
      op[0] = lda(0);
      op[1] = lda(1);
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) {
        if (i + 2 < 2 * KS) op[(i + 2) % 3] = lda(i + 2);
        const int st = i >> 1, s2 = i & 1;
        s[s2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % 3], qreg[st], st == 0 ? f32x16{} : s[s2], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      const uint8_t* va = &sV[buf][kr0 * VS + 16 * hh];
      auto ldv = [&](int i) {      // operand i: k-step i / 2 of sub-tile i % 2 (two 16-byte halves)
        const uint8_t* r = va + 16 * (i & 1) * VS + 64 * (i >> 1);
        const u32x4 lo = *reinterpret_cast<const u32x4*>(r);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(r + 32);
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      };
      i32x8 ov[2];
      ov[0] = ldv(0);
#pragma unroll
      for (int i = 0; i < 2 * KK; ++i) {
        if (i + 1 < 2 * KK) ov[(i + 1) & 1] = ldv(i + 1);
        const int kk = i >> 1, s2 = i & 1;
        // A: V codes (E4M3, format 0), B: dO^ codes (E5M2, format 1), unit scales
        dp[s2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ov[i & 1], doreg[kk], kk == 0 ? f32x16{} : dp[s2], 0,
                                                                1, 0, 127, 0, 127);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // dS of (this lane's query, key 32 hh + 16 s2 + r): one MX block per lane half
    // (keys past the sequence and, causal, after the wave's first query are
    // masked; only the last chunks need it)
    float dsv[2][16];
    float am = 0.0f;
    const int wq_first = qb * BWD_ROWS + wave * 32;
    const bool all_live = c * BWD_CHUNK + BWD_CHUNK <= p.N && (!CAUSAL || c * BWD_CHUNK + BWD_CHUNK - 1 <= wq_first);
    auto elements = [&](auto masked) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = c * BWD_CHUNK + 32 * hh + 16 * s2 + r;
          float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[s2][r], cc, -lq));
          if (decltype(masked)::value) pr = (kj < p.N && (!CAUSAL || kj <= q)) ? pr : 0.0f;
          const float ds = pr * __builtin_fmaf(dp[s2][r], sdv, -dq_d);
          dsv[s2][r] = ds;
          am = __builtin_fmaxf(am, __builtin_fabsf(ds));
        }
    };
    if (all_live) elements(std::false_type{});
    else elements(std::true_type{});
    const int e = mx_e4m3_exponent(am);
    const float lim = __builtin_ldexpf(448.0f, e), sc = e8m0_scale(e);
    const bool dump = DEBUG && b == p.dbg_b && h == p.dbg_h;
    if (dump) p.dbg_dsq_e[(int64_t)q * (npad / 32) + 2 * c + hh] = (uint8_t)(e + 127);
    uint32_t dsq[2][8];                         // bf16 pairs
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const s16x2 q2 = mx_e4m3_pair<false>(s16x2{0, 0}, dsv[s2][r], dsv[s2][r + 1], lim, sc);
        dsq[s2][r / 2] = mx_e4m3_pair_bf16(q2, sc);
        const uint32_t wq = __builtin_bit_cast(uint32_t, q2);
        if (dump) {
          const int kj = c * BWD_CHUNK + 32 * hh + 16 * s2 + r;
          p.dbg_dsq[(int64_t)q * npad + kj] = (uint8_t)wq;
          p.dbg_dsq[(int64_t)q * npad + kj + 1] = (uint8_t)(wq >> 8);
        }
      }
    // dQ^T: k-step j takes keys 32 hh + 16 (j/2) + 8 (j%2) + [0, 8) in both operands
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s2 = j >> 1, r0 = 8 * (j & 1);
      const bf16x8 bv = __builtin_bit_cast(bf16x8, u32x4{dsq[s2][r0 / 2], dsq[s2][r0 / 2 + 1],
                                                         dsq[s2][r0 / 2 + 2], dsq[s2][r0 / 2 + 3]});
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 32 * dt + ln;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sKT[buf][d * KTS + 32 * hh + 16 * s2 + r0]);
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc[dt], 0, 0, 0);
      }
    }
    store(buf ^ 1);
    __syncthreads();
  }
  // C[d row][query]: lane holds the query, register r holds d = 32 dt + out_row(r, hh)
  if (q < p.N) {
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
                           int N, int D, int64_t npad, __bf16* qrm, __bf16* qt, __bf16* krm, __bf16* kt,
                           uint8_t* vrm, uint8_t* drm, uint8_t* dtr, float* dvec, float* lvec, float* sdo,
                           hipStream_t st) {
  const dim3 gq((unsigned)(npad / 64), (unsigned)Hq, (unsigned)B), gk((unsigned)(npad / 64), (unsigned)Hkv, (unsigned)B);
  if (D == 64) {
    hipLaunchKernelGGL(bwd_expand_kernel<64>, gq, dim3(256), 0, st, q_codes, q_scales, Hq, N, npad, qrm, qt);
    hipLaunchKernelGGL(bwd_expand_kernel<64>, gk, dim3(256), 0, st, k_codes, k_scales, Hkv, N, npad, krm, kt);
    hipLaunchKernelGGL(bwd_v_kernel<64>, gk, dim3(256), 0, st, v_codes, Hkv, v_cols, npad, vrm);
    hipLaunchKernelGGL(bwd_do_kernel<64>, gq, dim3(256), 0, st, (const uint16_t*)dout, (const uint16_t*)o, lse,
                       partials, np, Hq, N, npad, drm, dtr, dvec, lvec, sdo);
  } else {
    hipLaunchKernelGGL(bwd_expand_kernel<128>, gq, dim3(256), 0, st, q_codes, q_scales, Hq, N, npad, qrm, qt);
    hipLaunchKernelGGL(bwd_expand_kernel<128>, gk, dim3(256), 0, st, k_codes, k_scales, Hkv, N, npad, krm, kt);
    hipLaunchKernelGGL(bwd_v_kernel<128>, gk, dim3(256), 0, st, v_codes, Hkv, v_cols, npad, vrm);
    hipLaunchKernelGGL(bwd_do_kernel<128>, gq, dim3(256), 0, st, (const uint16_t*)dout, (const uint16_t*)o, lse,
                       partials, np, Hq, N, npad, drm, dtr, dvec, lvec, sdo);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_main(const BwdParams& p, int D, bool causal, bool debug, hipStream_t st) {
  const dim3 gkv((unsigned)(p.npad / BWD_ROWS), (unsigned)p.Hkv, (unsigned)p.B);
  const dim3 gq((unsigned)(p.npad / BWD_ROWS), (unsigned)p.Hq, (unsigned)p.B);
#define BWD_LAUNCH(DD, C, G)                                                         \
  do {                                                                               \
    hipLaunchKernelGGL((bwd_dkdv_kernel<DD, C, G>), gkv, dim3(256), 0, st, p);       \
    hipLaunchKernelGGL((bwd_dq_kernel<DD, C, G>), gq, dim3(256), 0, st, p);          \
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
