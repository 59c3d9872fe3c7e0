// BF16 fused attention forward for gfx950: the baseline the Direct-P pages
// compare against ("Hardware-Aware FP4 FlashAttention-4", summary page, "Key
// results": throughput relative to BF16 FlashAttention-4).
//
// Online softmax over 128-key tiles in float32 (v_exp_f32), P rounded to
// bf16, both products on v_mfma_f32_32x32x16_bf16.  256 queries per
// workgroup of 8 waves, 32 per wave; S^T = K Q^T puts one query per lane.
// The key rows of K are permuted so that each lane's 16 S values of a
// sub-tile are exactly the 8 + 8 keys its P operand needs for two 16-key
// steps of O^T += V^T P^T; V stays key-major in LDS and its operand is read
// transposed (ds_read_b64_tr_b16).
//
// Software pipeline (one wave): iteration t issues, one matrix instruction per
// slot, P(t-2).V(t-2) and then S(t) = K(t) Q^T, and beside them the softmax of
// S(t-1): row max, running max m', alpha = 2^(m - m'), P(t-1) = 2^(t - m')
// rounded to bf16 pairs, and the row sum of the float32 probabilities.  P has one
// buffer: each 32-key sub-tile of P(t-1) is written after the P.V steps that
// read the same registers and before S(t) overwrites that sub-tile of S.  The
// O / l rescale by alpha(t-2) runs at the head of iteration t, only in waves
// where some row max moved.  K tiles sit in a ring of three LDS slots and V
// tiles in a ring of two, copied from HBM by buffer loads straight into LDS
// (keys past the end of the tensor read zeros); one workgroup barrier per
// iteration, taken by the two groups of four waves (one wave of each per
// SIMD) one S sub-tile (D/16 slots) apart.
#include "common.h"
#include "pipeline.h"

namespace attn {

// key within a 128-key tile of S^T sub-tile st, register v, lane half hh
__host__ __device__ inline int bf_key(int st, int v, int hh) { return 32 * st + 16 * (v >> 3) + 8 * hh + (v & 7); }

// Raw buffer resource (gfx9 layout): base address, byte count, default flags.
// Loads at or past the byte count return zeros instead of touching memory.
__device__ inline i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)(uint32_t)(a >> 32);
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from a buffer straight into LDS: lane i reads the buffer
// at byte `off` and writes LDS bytes [lds + 16 i, lds + 16 i + 16).
__device__ inline void dma16_buf(i32x4 rsrc, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(rsrc)
               : "memory");
}

#ifndef ATTN_BF16_G1B
#define ATTN_BF16_G1B (NS - KS)
#endif

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1) fwd_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                                                          float* __restrict__ lse, int B, int Hq, int Hkv, int Nq,
                                                          int Nk, int QB, float sigma) {
  constexpr int KS = D / 16;             // k-steps of an S sub-tile
  constexpr int DT = D / 32;             // 32-channel tiles of O^T
  constexpr int HALF = D / 2;
  constexpr int K_BYTES = KEY_TILE * D * 2, V_BYTES = KEY_TILE * D * 2;
  constexpr int K_RING = 3, V_RING = 2;
  constexpr int V_BASE = K_RING * K_BYTES;
  constexpr int NPV = 8 * DT;            // P.V instructions per tile: 8 steps of 16 keys x DT
  constexpr int NS = NPV + 4 * KS;       // slots per iteration
  constexpr int NK_DMA = K_BYTES / 16 / 512, NV_DMA = V_BYTES / 16 / 512;
  constexpr int G1B = ATTN_BF16_G1B;     // slot after which the second group takes its barrier
  static_assert(G1B >= NPV && G1B <= NS, "the V ring of two needs the second group past its P.V slots");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // ---- workgroup -> (batch, head, query block): the query blocks of one
  // head run on one XCD (workgroups are dealt round-robin over the 8 XCDs);
  // causal launches take the longest rows first
  const int nwg = gridDim.x;
  int lin = blockIdx.x;
  if ((nwg & 7) == 0) lin = (lin & 7) * (nwg >> 3) + (lin >> 3);
  int qb = lin % QB;
  const int h = __builtin_amdgcn_readfirstlane((lin / QB) % Hq);
  const int b = __builtin_amdgcn_readfirstlane(lin / (QB * Hq));
  if (CAUSAL) qb = QB - 1 - qb;
  qb = __builtin_amdgcn_readfirstlane(qb);
  const int hk = h / (Hq / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, ql = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int q0 = qb * WG_Q + wave * WAVE_Q, my_q = q0 + ql;
  const bool wave_active = q0 < Nq;
  int n_tiles = (Nk + KEY_TILE - 1) / KEY_TILE;
  if (CAUSAL) n_tiles = min(n_tiles, (min(qb * WG_Q + WG_Q, Nq) - 1) / KEY_TILE + 1);
  const int64_t orow = (((int64_t)b * Nq + my_q) * Hq + h) * D;
  if (n_tiles == 0) {                    // no key: O = 0, LSE = -inf, nothing of K / V is read
    if (wave_active && my_q < Nq) {
#pragma unroll
      for (int d = 0; d < HALF; d += 8)
        *reinterpret_cast<u32x4*>(o + orow + hh * HALF + d) = u32x4{0u, 0u, 0u, 0u};
      if (lse != nullptr && hh == 0) lse[((int64_t)b * Hq + h) * Nq + my_q] = -__builtin_inff();
    }
    return;
  }
  const float cc = sigma * 1.44269504088896341f;

  // ---- Q operand (B of S^T): lane holds query ql, d = hh*D/2 + 8 ks + j at k-step ks
  bf16x8 qf[KS];
  {
    const bool ok = my_q < Nq;
    const uint16_t* src = q + (((int64_t)b * Nq + (ok ? my_q : 0)) * Hq + h) * D + hh * HALF;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (ok) w = *reinterpret_cast<const u32x4*>(src + 8 * ks);
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[ks]));
  }

  // ---- copies.  K tile j in MFMA-operand order (16-byte unit (st, kh, ks, r)
  // holds key bf_key(st, .) of A-operand row r, channels kh*D/2 + 8 ks + [0, 8));
  // V tile j as [32-channel slice][key][32 channels] (64 bytes per key and
  // slice), so that the four keys x 32 channels one transposing read of a P.V
  // operand touches are 256 contiguous bytes.  Per-lane offsets are loop
  // invariant; the tile moves the buffer's base.
  const uint32_t lds0 = lds_address(smem);
  const int rstride = Hkv * D;
  const uint16_t* kbase = k + ((int64_t)b * Nk * Hkv + hk) * D;
  const uint16_t* vbase = v + ((int64_t)b * Nk * Hkv + hk) * D;
  // a tile spans 128 rows of Hkv * D elements; only the last batch entry's
  // partial last tile reaches past the tensor's end: there the buffer ends
  // with the tensor
  const uint32_t tile_bytes = (uint32_t)(KEY_TILE * rstride * 2);
  const int tail_tile = Nk / KEY_TILE;
  const uint32_t tail_bytes = (uint32_t)(((Nk - tail_tile * KEY_TILE) * Hkv - hk) * D * 2);
  const bool last_batch = b == B - 1;
  uint32_t koff[NK_DMA], voff[NV_DMA];
#pragma unroll
  for (int i = 0; i < NK_DMA; ++i) {
    const int u = i * 512 + wave * 64 + lane;
    const int r = u & 31, ks = (u >> 5) % KS, kh = (u >> 5) / KS % 2, st = (u >> 5) / KS / 2;
    const int hq = (r >> 2) & 1, vv = ((r >> 3) << 2) | (r & 3);   // inverse of the accumulator row map
    koff[i] = (uint32_t)((bf_key(st, vv, hq) * rstride + kh * HALF + 8 * ks) * 2);
  }
#pragma unroll
  for (int i = 0; i < NV_DMA; ++i) {
    const int u = i * 512 + wave * 64 + lane;
    const int c4 = u & 3, kr = (u >> 2) & 127, dt = u >> 9;
    voff[i] = (uint32_t)((kr * rstride + 32 * dt + 8 * c4) * 2);
  }
  auto tile_rsrc = [&](const uint16_t* base, int j) {
    return buffer_rsrc(reinterpret_cast<const uint8_t*>(base) + (uint64_t)j * tile_bytes,
                       last_batch && j == tail_tile ? tail_bytes : tile_bytes);
  };
  auto copy_k_part = [&](int slot, int j, int i) {
    dma16_buf(tile_rsrc(kbase, j), koff[i], lds0 + (uint32_t)(slot * K_BYTES + (i * 512 + wave * 64) * 16));
  };
  auto copy_v_part = [&](int slot, int j, int i) {
    dma16_buf(tile_rsrc(vbase, j), voff[i], lds0 + (uint32_t)(V_BASE + slot * V_BYTES + (i * 512 + wave * 64) * 16));
  };

  // ---- accumulators and per-wave state
  f32x16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};
  f32x16 s[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) s[st] = f32x16{};
  u32x4 pb[8];                           // P: k-step ks, bf16 pairs (keys 16 ks + 8 hh + [0, 8))
#pragma unroll
  for (int i = 0; i < 8; ++i) pb[i] = u32x4{0u, 0u, 0u, 0u};
  float m_run = -__builtin_inff(), negm = 0.0f, alpha_pend = 1.0f, alpha_prev = 1.0f;
  float lsum = 0.0f, lt = 0.0f, lt_prev = 0.0f;
  bool rescale_any = false;
  float bmp = 0.0f, bmn = 0.0f;          // max of S sub-tiles 0..2 of the tile being encoded / the next

  auto tile_max = [&](int st) {
    const float a = fmax3(s[st][0], s[st][1], s[st][2]);
    const float b2 = fmax3(s[st][3], s[st][4], s[st][5]);
    const float c = fmax3(s[st][6], s[st][7], s[st][8]);
    const float d = fmax3(s[st][9], s[st][10], s[st][11]);
    const float e = fmax3(s[st][12], s[st][13], s[st][14]);
    return fmax3(fmax3(a, b2, c), fmax3(d, e, s[st][15]), -__builtin_inff());
  };
  auto mask = [&](int j) {
    const int key0 = j * KEY_TILE;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int key = key0 + bf_key(st, vv, hh);
        if (key >= Nk || (CAUSAL && key > my_q)) s[st][vv] = -__builtin_inff();
      }
  };

  // ---- slot machinery.  Slot i issues: i < NPV: O^T += V^T P^T for 16-key
  // step i / DT and channel tile i % DT; else S sub-tile (i - NPV) / KS,
  // k-step (i - NPV) % KS.  Operands are read from LDS two slots ahead.
  typedef short s16x4 __attribute__((__vector_size__(8)));
  typedef __attribute__((address_space(3))) s16x4 lds_s4;
  u32x4 opa[3];
  auto load_op = [&](int i, const uint8_t* sK, const uint8_t* sV) {
    const int bs = i % 3;
    if (i < NPV) {
      const int ks2 = i / DT, dt = i % DT;
      // transposing reads: lane (g, c) gets V[kb + 0..3][d] and V[kb + 4..7][d], d = 32 dt + 16 (g & 1) + c
      const int g = lane >> 4, c = lane & 15;
      const int k1 = 16 * ks2 + 8 * (g >> 1) + (c >> 2);
      const int dl = 16 * (g & 1) + 4 * (c & 3);
      const uint8_t* a1 = sV + (dt * KEY_TILE + k1) * 64 + dl * 2;
      const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(__attribute__((address_space(3))) const void*)a1);
      const s16x4 r2 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(__attribute__((address_space(3))) const void*)(a1 + 4 * 64));
      const u32x2 w1 = __builtin_bit_cast(u32x2, r1), w2 = __builtin_bit_cast(u32x2, r2);
      opa[bs] = u32x4{w1[0], w1[1], w2[0], w2[1]};
    } else {
      const int st = (i - NPV) / KS, ks = (i - NPV) % KS;
      opa[bs] = *reinterpret_cast<const u32x4*>(sK + ((st * 2 + hh) * KS * 32 + ks * 32 + ql) * 16);
    }
  };
  auto mfma_slot = [&](int i) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, opa[i % 3]);
    if (i < NPV) {
      const int ks2 = i / DT, dt = i % DT;
      oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pb[ks2]), oacc[dt], 0, 0, 0);
    } else {
      const int st = (i - NPV) / KS, ks = (i - NPV) % KS;
      s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], ks == 0 ? f32x16{} : s[st], 0, 0, 0);
    }
  };
  // Vector units of tile t-1: 0 = its row max (sub-tile 3 joins the maxima of
  // sub-tiles 0..2 taken an iteration earlier) and m', alpha; 1..32 = encode
  // scores 2k, 2k+1 of sub-tile st (unit 1 + 8 st + k); 33..35 = maxima of S(t)
  // sub-tiles 0..2 for the next iteration.
  constexpr int ENC_FIRST = 2 * DT;                  // P of k-steps 0, 1 consumed by then
  constexpr int ENC_SPAN = NPV + 3 * KS - 2 * DT;    // sub-tile 3 done before S(t) sub-tile 3
  auto unit_slot = [&](int u) -> int {
    if (u == 0) return 0;
    if (u <= 32) return ENC_FIRST + ((u - 1) * ENC_SPAN) / 32;
    return NPV + KS * (u - 32) + 1;                  // one slot after sub-tile u - 33 of S(t) is issued
  };
  auto vunit = [&](int u) {
    if (u == 0) {
      float rmax = fmax2(bmp, tile_max(3));
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rmax), __float_as_uint(rmax), false, false);
      rmax = fmax2(__uint_as_float(sw[0]), __uint_as_float(sw[1]));   // max with lane ^ 32
      // every row sees a live key in its first tile, so m' is finite from then on
      const float m_new = fmax2(m_run, rmax * cc);
      alpha_pend = __builtin_amdgcn_exp2f(m_run - m_new);
      rescale_any = __builtin_amdgcn_ballot_w64(alpha_pend != 1.0f) != 0;
      m_run = m_new;
      negm = -m_new;
      lt = 0.0f;
    } else if (u <= 32) {
      const int n = u - 1, st = n >> 3, kk = n & 7, vv = 2 * kk;
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][vv], cc, negm));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][vv + 1], cc, negm));
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
      const uint32_t w = __builtin_bit_cast(uint32_t, pp);
      pb[2 * st + (kk >> 2)][kk & 3] = w;
      lt += p0 + p1;                     // the row sum of the float32 probabilities
    } else {
      const int st = u - 33;
      if (st == 0) bmn = tile_max(0);
      else bmn = fmax2(bmn, tile_max(st));
    }
  };

  // ---- prologue: zero the LDS rings (keys past the tensor's end may leave
  // their bytes unwritten), K(0) and K(1), S(0)
  for (int i = tid; i < (K_RING * K_BYTES + V_RING * V_BYTES) / 16; i += 512)
    *reinterpret_cast<u32x4*>(smem + i * 16) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NK_DMA; ++i) copy_k_part(0, 0, i);
  dma_wait();
  __syncthreads();
  if (n_tiles > 1) {
#pragma unroll
    for (int i = 0; i < NK_DMA; ++i) copy_k_part(1, 1, i);
  }
  {
    const uint8_t* sK = smem;
#pragma unroll
    for (int i = NPV; i < NS; ++i) {
      load_op(i, sK, smem);
      mfma_slot(i);
    }
    bmp = fmax2(fmax2(tile_max(0), tile_max(1)), tile_max(2));
  }
  dma_wait();
  phase_barrier();

  for (int t = 1; t <= n_tiles + 1; ++t) {
    const int rk = t % 3, rk1 = (t + 1) % 3;           // K(t), K(t+1)
    const int rv = t & 1;                              // V(t-2); V(t-1) goes to the other slot
    const int last = n_tiles - 1;
    const int src_k = min(t + 1, last), src_v = min(t - 1, last);
    // O / l rescale by alpha(t-2), set while S(t-2) was encoded in the
    // previous iteration: after P(t-3).V, before P(t-2).V; then l takes the
    // row sum of P(t-2), which is at the new scale
    if (rescale_any) {
#pragma unroll
      for (int i = 0; i < DT; ++i) oacc[i] *= alpha_pend;
    }
    alpha_prev = alpha_pend;
    lt_prev = lt;
    lsum = __builtin_fmaf(lsum, alpha_prev, lt_prev);
    const int j = t - 1;                               // tile being encoded
    if (j * KEY_TILE + KEY_TILE > Nk || (CAUSAL && j * KEY_TILE + KEY_TILE - 1 > q0)) {
      mask(j);
      bmp = fmax2(fmax2(tile_max(0), tile_max(1)), tile_max(2));
    }
    const uint8_t* sK = smem + rk * K_BYTES;
    const uint8_t* sV = smem + V_BASE + rv * V_BYTES;
    load_op(0, sK, sV);
    load_op(1, sK, sV);
    __builtin_amdgcn_sched_barrier(0);
#pragma clang loop unroll(full)
    for (int i = 0; i < NS; ++i) {
      // copies of K(t+1) and V(t-1), spread over the slots before the second group's barrier
#pragma unroll
      for (int c = 0; c < NK_DMA + NV_DMA; ++c)
        if (i == (c * (G1B - 2)) / (NK_DMA + NV_DMA)) {
          if (c < NK_DMA) copy_k_part(rk1, src_k, c);
          else copy_v_part(rv ^ 1, src_v, c - NK_DMA);
        }
      if (i + 2 < NS) load_op(i + 2, sK, sV);
      mfma_slot(i);
#pragma unroll
      for (int u = 0; u < 36; ++u)
        if (unit_slot(u) == i) vunit(u);
      __builtin_amdgcn_sched_barrier(0);
      if (i == G1B - 1 && G1B < NS) dma_wait_barrier_if(group);
    }
    bmp = bmn;
    dma_wait_barrier_if(G1B >= NS ? 1 : group ^ 1);
  }
  lsum = __builtin_fmaf(lsum, alpha_pend, lt);

  // ---- epilogue: l from both lane halves, O = o / l, LSE = ln2 * (m + log2 l)
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (!wave_active || my_q >= Nq) return;
  const bool empty = !(lsum > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / lsum;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d = 32 * dt + 8 * jj + 4 * hh;
      uint32_t u[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t bits = __float_as_uint(oacc[dt][4 * jj + x] * inv);
        u[x] = (bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16;
      }
      *reinterpret_cast<u32x2*>(o + orow + d) = u32x2{u[0] | (u[1] << 16), u[2] | (u[3] << 16)};
    }
  if (lse != nullptr && hh == 0)
    lse[((int64_t)b * Hq + h) * Nq + my_q] = empty ? -__builtin_inff() : 0.6931471805599453f * (m_run + __builtin_log2f(lsum));
}

template <int D, bool CAUSAL>
static hipError_t launch_bf16_t(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                                int Hkv, int Nq, int Nk, float sigma, hipStream_t st) {
  const int QB = (Nq + WG_Q - 1) / WG_Q;
  const int nwg = B * Hq * QB;
  if (nwg == 0) return hipSuccess;
  auto kern = fwd_bf16_kernel<D, CAUSAL>;
  const int lds = (3 + 2) * KEY_TILE * D * 2;
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
