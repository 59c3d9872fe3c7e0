// BF16 fused attention forward for gfx950: the baseline the Direct-P pages
// compare against ("Hardware-Aware FP4 FlashAttention-4", summary page, "Key
// results": throughput relative to BF16 FlashAttention-4).
//
// Same tiling as the low-precision forward (256 queries per workgroup, 32 per
// wave, 128-key tiles double-buffered in LDS, S^T = K Q^T with one query per
// lane), but every operand is bf16: S^T on v_mfma_f32_32x32x16_bf16, online
// softmax in float32 with v_exp_f32, P rounded to bf16, O^T += V^T P^T on the
// same MFMA.  The key rows of K are permuted so that each lane's 16 S values
// of a sub-tile are exactly the 8 + 8 keys its P operand needs for two
// 16-key MFMA steps; V is transposed into key-contiguous rows while staging.
#include "common.h"

namespace attn {

// key within a 128-key tile of S^T sub-tile st, register v, lane half hh
__device__ inline int bf_key(int st, int v, int hh) { return 32 * st + 16 * (v >> 3) + 8 * hh + (v & 7); }
__device__ inline int bf_out_row(int v, int hh) { return 8 * (v >> 2) + 4 * hh + (v & 3); }

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1) fwd_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                                                          float* __restrict__ lse, int B, int Hq, int Hkv, int Nq,
                                                          int Nk, int QB, float sigma) {
  constexpr int KS = D / 16, DT = D / 32, HALF = D / 2;
  constexpr int K_BYTES = KEY_TILE * D * 2, V_BYTES = KEY_TILE * D * 2, STAGE = K_BYTES + V_BYTES;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int nwg = gridDim.x;
  int lin = blockIdx.x;
  if ((nwg & 7) == 0) lin = (lin & 7) * (nwg >> 3) + (lin >> 3);
  int qb = lin % QB;
  const int h = (lin / QB) % Hq;
  const int b = lin / (QB * Hq);
  if (CAUSAL) qb = QB - 1 - qb;
  const int hk = h / (Hq / Hkv);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, ql = lane & 31;
  const int q0 = qb * WG_Q + wave * WAVE_Q, my_q = q0 + ql;
  const bool wave_active = q0 < Nq;
  int n_tiles = (Nk + KEY_TILE - 1) / KEY_TILE;
  if (CAUSAL) n_tiles = min(n_tiles, (min(qb * WG_Q + WG_Q, Nq) - 1) / KEY_TILE + 1);
  const float cc = sigma * 1.44269504088896341f;

  bf16x8 qf[KS];
  {
    const bool ok = my_q < Nq;
    const uint16_t* src = q + (((int64_t)b * Nq + my_q) * Hq + h) * D + hh * HALF;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (ok) w = *reinterpret_cast<const u32x4*>(src + 8 * ks);
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // staging: K as (st, kh, ks, r) 16-byte units; V transposed as (ks2, dt, hh, r) units
  constexpr int K_UNITS = K_BYTES / 16, K_PER = K_UNITS / 512;
  constexpr int V_ITERS = (KEY_TILE / 8) * (D / 2) / 512;   // (8 keys x 2 channels) per thread per iter
  u32x4 kreg[K_PER];
  uint32_t vreg[V_ITERS][8];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < K_PER; ++i) {
      const int u = i * 512 + tid;
      const int key = u / (D / 8), part = u % (D / 8);
      const int kg = t * KEY_TILE + key;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (kg < Nk) w = *reinterpret_cast<const u32x4*>(k + (((int64_t)b * Nk + kg) * Hkv + hk) * D + 8 * part);
      kreg[i] = w;
    }
#pragma unroll
    for (int it = 0; it < V_ITERS; ++it) {
      const int idx = it * 512 + tid;
      const int dp = idx % (D / 2), kgrp = idx / (D / 2);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kg = t * KEY_TILE + kgrp * 8 + j;
        vreg[it][j] = kg < Nk ? *reinterpret_cast<const uint32_t*>(v + (((int64_t)b * Nk + kg) * Hkv + hk) * D + 2 * dp) : 0u;
      }
    }
  };
  auto store_tile = [&](int stage) {
    uint8_t* base = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < K_PER; ++i) {
      const int u = i * 512 + tid;
      const int key = u / (D / 8), part = u % (D / 8);
      const int d0 = 8 * part, kh = d0 / HALF, ks = (d0 % HALF) / 8;
      const int st = key >> 5, w = key & 31;
      const int vv = 8 * (w >> 4) + (w & 7), hq = (w >> 3) & 1;
      const int r = bf_out_row(vv, hq);
      *reinterpret_cast<u32x4*>(base + ((((st * 2 + kh) * KS + ks) * 32 + r) * 16)) = kreg[i];
    }
#pragma unroll
    for (int it = 0; it < V_ITERS; ++it) {
      const int idx = it * 512 + tid;
      const int dp = idx % (D / 2), kgrp = idx / (D / 2);
      u32x4 lo, hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo[j] = __builtin_amdgcn_perm(vreg[it][2 * j + 1], vreg[it][2 * j], 0x05040100u);
        hi[j] = __builtin_amdgcn_perm(vreg[it][2 * j + 1], vreg[it][2 * j], 0x07060302u);
      }
      const int kk = 8 * kgrp, ks2 = kk >> 4, hq = (kk >> 3) & 1;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int d = 2 * dp + x, dt = d >> 5, r = d & 31;
        *reinterpret_cast<u32x4*>(base + K_BYTES + ((((ks2 * DT + dt) * 2 + hq) * 32 + r) * 16)) = x ? hi : lo;
      }
    }
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};
  float l_run = 0.0f, m_run = -__builtin_inff();

  if (n_tiles > 0) { load_tile(0); store_tile(0); }
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int stage = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);
    const uint8_t* sK = smem + stage * STAGE;
    const uint8_t* sV = sK + K_BYTES;
    const int key0 = t * KEY_TILE;
    bool wave_work = wave_active;
    if (CAUSAL) wave_work = wave_work && key0 <= q0 + WAVE_Q - 1;
    if (wave_work) {
      f32x16 s[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        s[st] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + ((((st * 2 + hh) * KS + ks) * 32 + ql) * 16));
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[st], 0, 0, 0);
        }
      }
      if (key0 + KEY_TILE > Nk || (CAUSAL && key0 + KEY_TILE - 1 > q0)) {
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int vv = 0; vv < 16; ++vv) {
            const int key = key0 + bf_key(st, vv, hh);
            if (key >= Nk || (CAUSAL && key > my_q)) s[st][vv] = -__builtin_inff();
          }
      }
      float rmax = s[0][0];
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) rmax = __builtin_fmaxf(rmax, s[st][vv]);
      rmax = __builtin_fmaxf(rmax, __shfl_xor(rmax, 32, 64));
      const float m_new = __builtin_fmaxf(m_run, rmax * cc);
      const bool dead = m_new == -__builtin_inff();
      const float alpha = dead ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      const float ms = dead ? 0.0f : m_new;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int i = 0; i < DT; ++i) oacc[i] *= alpha;
      }
      // P for one 16-key step at a time (keeps only 4 VGPRs of bf16 P live)
      float psum = 0.0f;
#pragma unroll
      for (int ks2 = 0; ks2 < 8; ++ks2) {
        bf16x8 pb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[ks2 >> 1][8 * (ks2 & 1) + j], cc, -ms));
          psum += pv;
          pb[j] = (__bf16)pv;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sV + ((((ks2 * DT + dt) * 2 + hh) * 32 + ql) * 16));
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[dt], 0, 0, 0);
        }
      }
      psum += __shfl_xor(psum, 32, 64);
      l_run = l_run * alpha + psum;
      m_run = m_new;
    }
    if (t + 1 < n_tiles) store_tile(stage ^ 1);
    __syncthreads();
  }
  if (!wave_active || my_q >= Nq) return;
  const bool empty = !(l_run > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / l_run;
  const int64_t orow = (((int64_t)b * Nq + my_q) * Hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * dt + 8 * j + 4 * hh;
      uint32_t u[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        uint32_t bits = __float_as_uint(oacc[dt][4 * j + x] * inv);
        u[x] = (bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16;
      }
      *reinterpret_cast<u32x2*>(o + orow + d) = u32x2{u[0] | (u[1] << 16), u[2] | (u[3] << 16)};
    }
  if (lse != nullptr && hh == 0)
    lse[((int64_t)b * Hq + h) * Nq + my_q] = empty ? -__builtin_inff() : 0.6931471805599453f * (m_run + __builtin_log2f(l_run));
}

template <int D, bool CAUSAL>
static hipError_t launch_bf16_t(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                                int Hkv, int Nq, int Nk, float sigma, hipStream_t st) {
  const int QB = (Nq + WG_Q - 1) / WG_Q;
  const int nwg = B * Hq * QB;
  if (nwg == 0) return hipSuccess;
  auto kern = fwd_bf16_kernel<D, CAUSAL>;
  const int lds = 2 * (KEY_TILE * D * 2 * 2);
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(512), lds, st, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                     (uint16_t*)o, lse, B, Hq, Hkv, Nq, Nk, QB, sigma);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                           int Nq, int Nk, int D, float sigma, bool causal, hipStream_t st) {
  if (D == 64) return causal ? launch_bf16_t<64, true>(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, sigma, st)
                             : launch_bf16_t<64, false>(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, sigma, st);
  return causal ? launch_bf16_t<128, true>(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, sigma, st)
                : launch_bf16_t<128, false>(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, sigma, st);
}

}  // namespace attn
