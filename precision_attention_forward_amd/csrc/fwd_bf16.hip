// BF16 fused attention forward for gfx950: the baseline the Direct-P pages
// compare against ("Hardware-Aware FP4 FlashAttention-4", summary page, "Key
// results": throughput relative to BF16 FlashAttention-4).
//
// Same pipeline as the low-precision forward (256 queries per workgroup, 32
// per wave, two ping-pong groups of four waves, 128-key tiles copied straight
// into double-buffered LDS, S^T = K Q^T with one query per lane), but every
// operand is bf16: S^T on v_mfma_f32_32x32x16_bf16, online softmax in
// float32 with v_exp_f32, P rounded to bf16, O^T += V^T P^T on the same MFMA.
// The key rows of K are permuted so that each lane's 16 S values of a
// sub-tile are exactly the 8 + 8 keys its P operand needs for two 16-key MFMA
// steps; V stays key-major in LDS and is read transposed (ds_read_b64_tr_b16).
#include "common.h"
#include "pipeline.h"

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
  const int grp = wave >> 2;
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
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[ks]));
  }

  // Stage j (slot j % 2): K tile j in MFMA-operand order; V tile j-1 as
  // [32-channel slice][key][32 channels] (64 bytes per key and slice), so the
  // four keys x 32 channels a transposing read of one P.V operand touches are
  // 256 contiguous bytes.  Rows past the end of the sequence re-read the last
  // row (their probabilities are zero).
  const uint32_t lds0 = lds_address(smem);
  const uint16_t* kbase = k + ((int64_t)b * Nk * Hkv + hk) * D;
  const uint16_t* vbase = v + ((int64_t)b * Nk * Hkv + hk) * D;
  const int rstride = Hkv * D;
  auto issue_stage = [&](int j) {
    const uint32_t slot = lds0 + (uint32_t)((j & 1) * STAGE);
    if (j < n_tiles) {
#pragma unroll
      for (int i = 0; i < K_BYTES / 16 / 512; ++i) {
        const int u0 = i * 512 + wave * 64, u = u0 + lane;
        const int r = u & 31, ks = (u >> 5) % KS, kh = (u >> 5) / KS % 2, st = (u >> 5) / KS / 2;
        const int hq = (r >> 2) & 1, vv = ((r >> 3) << 2) | (r & 3);
        const int key = min(j * KEY_TILE + 32 * st + 16 * (vv >> 3) + 8 * hq + (vv & 7), Nk - 1);
        dma16(kbase, (uint32_t)((key * rstride + kh * HALF + 8 * ks) * 2), slot + u0 * 16);
      }
    }
    if (j >= 1) {
      const int t = j - 1;
#pragma unroll
      for (int i = 0; i < V_BYTES / 16 / 512; ++i) {
        const int u0 = i * 512 + wave * 64, u = u0 + lane;
        const int c4 = u & 3, kr = (u >> 2) & 127, dt = u >> 9;
        const int key = min(t * KEY_TILE + kr, Nk - 1);
        dma16(vbase, (uint32_t)((key * rstride + 32 * dt + 8 * c4) * 2), slot + K_BYTES + u0 * 16);
      }
    }
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};
  float l_run = 0.0f, m_run = -__builtin_inff();
  f32x16 s[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) s[st] = f32x16{};
  bf16x8 pb[8];
  bool have_s = false, have_p = false;

  auto mfma_phase = [&](int j) {
    const uint8_t* sK = smem + (j & 1) * STAGE;
    const uint8_t* sV = sK + K_BYTES;
    if (have_p) {
      const int g = lane >> 4, i = lane & 15;
#pragma unroll
      for (int ks2 = 0; ks2 < 8; ++ks2) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          // transposing reads: lane (g, i) gets V[kb + 0..3][d] and V[kb + 4..7][d], d = 32dt + 16(g&1) + i
          const int k1 = 16 * ks2 + 8 * (g >> 1) + (i >> 2);
          const int dl = 16 * (g & 1) + 4 * (i & 3);        // channel within the 32-channel slice
          typedef short s16x4 __attribute__((__vector_size__(8)));
          typedef __attribute__((address_space(3))) s16x4 lds_s4;
          const uint8_t* a1 = sV + (dt * KEY_TILE + k1) * 64 + dl * 2;
          const uint8_t* a2 = a1 + 4 * 64;
          const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(__attribute__((address_space(3))) const void*)a1);
          const s16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(__attribute__((address_space(3))) const void*)a2);
          typedef short short8 __attribute__((ext_vector_type(8)));
          const short8 av = {r1[0], r1[1], r1[2], r1[3], r2[0], r2[1], r2[2], r2[3]};
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb[ks2], oacc[dt], 0, 0, 0);
        }
      }
      have_p = false;
    }
    have_s = false;
    if (j < n_tiles) {
      bool work = wave_active;
      if (CAUSAL) work = work && (j * KEY_TILE <= q0 + WAVE_Q - 1);
      if (work) {
        const uint8_t* kb = sK + (hh * KS * 32 + ql) * 16;
        bf16x8 a[4], an[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          s[st] = f32x16{};
          a[st] = *reinterpret_cast<const bf16x8*>(kb + st * 2 * KS * 32 * 16);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + 1 < KS) {
#pragma unroll
            for (int st = 0; st < 4; ++st)
              an[st] = *reinterpret_cast<const bf16x8*>(kb + (st * 2 * KS + ks + 1) * 32 * 16);
          }
#pragma unroll
          for (int st = 0; st < 4; ++st) s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[st], qf[ks], s[st], 0, 0, 0);
          if (ks + 1 < KS) {
#pragma unroll
            for (int st = 0; st < 4; ++st) a[st] = an[st];
          }
        }
        have_s = true;
      }
    }
  };

  auto valu_phase = [&](int j) {
    if (!have_s) return;
    const int key0 = j * KEY_TILE;
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
    float psum = 0.0f;
#pragma unroll
    for (int ks2 = 0; ks2 < 8; ++ks2)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[ks2 >> 1][8 * (ks2 & 1) + jj], cc, -ms));
        psum += pv;
        pb[ks2][jj] = (__bf16)pv;
      }
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    have_p = true;
  };

  issue_stage(0);
  dma_wait();
  phase_barrier();
  const int nph = 2 * n_tiles + 2;
  for (int ph = 0; ph < nph; ++ph) {
    if ((ph & 1) == 0 && (ph >> 1) + 1 <= n_tiles) issue_stage((ph >> 1) + 1);
    const int my = ph - grp;
    if (my >= 0 && my <= 2 * n_tiles) {
      if ((my & 1) == 0) mfma_phase(my >> 1);
      else valu_phase(my >> 1);
    }
    if (ph & 1) dma_wait();
    phase_barrier();
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
