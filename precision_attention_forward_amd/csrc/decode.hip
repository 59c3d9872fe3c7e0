// Decode-shaped Direct-P / FP8-P forward for gfx950: a few new query tokens
// per sequence against a long quantized KV cache.
//
// Method: the same tiled low-precision softmax as the prefill forward
// ("Hardware-Aware FP4 FlashAttention-4", summary page, "What the paper
// found"): NVFP4 Q and K, the running row max m' updated once per tile of 128
// keys, Direct-P E2M1 probability codes with one E8M0 exponent per 32 keys (or
// E4M3 codes with a unit scale), the denominator summed from the rounded
// probabilities, O = o / l and LSE = ln2 (m + log2 l).  The decode workload
// is the one of the Colfax Research feed's post on FlashAttention-4 decode
// (abstract only): each step generates one or a few tokens per sequence from
// the keys and values cached by the prefill.
//
// gfx950 mapping:
//  * A decode step reads every cached key once for only G * nq query rows per
//    KV head (G query heads per KV head, nq new tokens), so it is bound by HBM
//    bandwidth.  The kernel streams the compact cache itself -- NVFP4 K (D/2
//    code bytes and D/16 E4M3 scales per key) and FP8 or MXFP4 V -- and
//    decodes K to exact FP16 in registers (v_cvt_scalef32_pk_f16_fp4, then a
//    packed FP16 multiply by the block scale: E2M1 x E4M3 has at most 6
//    significant bits), where the prefill path expands K in HBM once and
//    re-reads it for every query block.
//  * One workgroup of four waves per (sequence, KV head, 32 query rows): the
//    G * nq query rows of a KV head are the columns of S^T = K Q^T, so the
//    cache is read once for the whole GQA group.  Waves take interleaved
//    64-key chunks (step s: wave w takes chunk 4s + w, i.e. two 128-key tiles
//    per step), keep their own O / l partials, and exchange per-chunk row
//    maxima through LDS once per step, so that every wave encodes with the
//    running max m' of its own tile: the codes of one sequential pass, which
//    splitting the keys over independent workgroups would not give.
//  * Each wave loads its chunks from HBM straight into registers two steps
//    ahead (no LDS staging: no other wave reads them).
//  * At the end the four partials are rescaled to the final max and summed
//    through LDS.
//  * S^T, P.V and l use the operand layouts of the prefill kernel: S^T on
//    v_mfma_f32_32x32x16_f16 with one query per lane, each lane holding the 32
//    keys of one P block (MXFP4) or the 32 keys the FP8 operand wants; P.V on
//    v_mfma_scale_f32_32x32x64_f8f6f4; l on one 16x16x128 scaled MFMA per chunk
//    against a constant 0/1 operand.
#include "common.h"
#include "dec_params.h"
#include "fwd_params.h"

namespace attn {

constexpr int DEC_WAVES = 4;
constexpr int DEC_CHUNK = 64;

// Key (0..63) of a 64-key chunk held by S^T sub-tile s2 (0, 1), accumulator
// register v (0..15), lane half hh.  MXFP4 P: lane half hh holds the 32 keys
// of one P block; FP8 P: the k order of the FP8 operand of the 32x32x64 MFMA
// (k-block 0 = bytes 0-15 of both lane halves).
template <int PF>
__host__ __device__ inline int dec_key(int s2, int v, int hh) {
  return PF == PF_MXFP4 ? 32 * hh + 16 * s2 + v : 32 * s2 + 16 * hh + v;
}

// Operands of one 64-key chunk, as one lane holds them.
template <int D, int VF>
struct DecBuf {
  u32x4 kc[2][D / 64];                       // K codes of the lane's key, its D/2 channels, per sub-tile
  uint32_t ks[2];                            // their E4M3 block scales (D/32 bytes)
  u32x4 va[D / 32][VF == VF_FP8 ? 2 : 1];    // V^T operand per 32 channels
  uint32_t vs[VF == VF_MXFP4 ? D / 32 : 1];  // MXFP4 V: E8M0 bytes of the tile's 4 blocks
};

template <int D, int PF, int VF, bool CAUSAL, bool DEBUG>
__global__ void __launch_bounds__(256, 1) decode_kernel(DecParams p) {
  constexpr int KS = D / 16;     // k-steps of the S MFMA
  constexpr int DT = D / 32;     // 32-row tiles of O^T
  constexpr int HALF = D / 2;    // code bytes per row
  constexpr int LB = D / 4;      // code bytes of one lane half (D/2 channels)
  constexpr int LS = D / 32;     // scale bytes of one lane half
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* sM = reinterpret_cast<float*>(smem);                       // [2][DEC_WAVES][32] chunk maxima
  float* sO = sM + 2 * DEC_WAVES * 32;                              // [DEC_WAVES][DT][16][64] partial O
  float* sL = sO + DEC_WAVES * DT * 16 * 64;                        // [DEC_WAVES][64] partial l

  // ---- workgroup -> (sequence, KV head, query group)
  int lin = blockIdx.x;
  int qg = lin % p.QG;
  int hk = (lin / p.QG) % p.Hkv;
  int b = lin / (p.QG * p.Hkv);
  qg = __builtin_amdgcn_readfirstlane(qg);
  hk = __builtin_amdgcn_readfirstlane(hk);
  b = __builtin_amdgcn_readfirstlane(b);
  int len_k = p.seqlens != nullptr ? p.seqlens[b] : p.Nk;
  len_k = len_k < 0 ? 0 : (len_k > p.Nk ? p.Nk : len_k);          // reads stay inside the cache
  len_k = __builtin_amdgcn_readfirstlane(len_k);
  const int G = p.Hq / p.Hkv;
  const int R = G * p.nq;                                            // query rows of this KV head

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, ql = lane & 31;
  // query row of this lane's S^T column: row r = token i * G + head g
  const int my_r = 32 * qg + ql;
  const bool row_ok = my_r < R;
  const int my_i = row_ok ? my_r / G : 0;
  const int my_h = hk * G + (row_ok ? my_r % G : 0);
  const int my_pos = len_k - p.nq + my_i;                            // absolute position (causal)

  const int n_chunks = (len_k + DEC_CHUNK - 1) / DEC_CHUNK;
  const int n_steps = (n_chunks + DEC_WAVES - 1) / DEC_WAVES;

  const float cc = (float)((double)p.sigma * 1.4426950408889634 * (double)(*p.gq) * (double)(*p.gk));
  const float vscale = VF == VF_FP8 ? *p.sv : 1.0f;

  // ---- Q operand (B of S^T): lane holds query row my_r, channels
  // [hh D/2, hh D/2 + D/2), decoded from NVFP4 (exact in FP16)
  f16x8 qf[KS];
  {
    const int64_t row = row_ok ? ((int64_t)b * p.nq + my_i) * p.Hq + my_h : 0;
    const uint8_t* qc = p.q_codes + row * HALF + hh * LB;
    const uint8_t* qs = p.q_scales + row * (D / 16) + hh * LS;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t cw = row_ok ? *reinterpret_cast<const uint32_t*>(qc + 4 * ks) : 0u;
      const float sv = e4m3_decode(row_ok ? qs[ks >> 1] : 0u);
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[ks][j] = (_Float16)(e2m1_decode((cw >> (4 * j)) & 0xFu) * sv);
    }
  }

  // ---- per-lane load offsets (bytes, below 2^31; the host checks D * cols)
  // A operand of S^T: lane (r, hh) reads the key of accumulator row r of
  // sub-tile s2 (rows of the 32x32 output: r = 8 (v / 4) + 4 hh' + v % 4),
  // channels [hh D/2, hh D/2 + D/2).
  const int rr = lane & 31;
  const int kl0 = dec_key<PF>(0, 4 * (rr >> 3) + (rr & 3), (rr >> 2) & 1);
  const int kl1 = dec_key<PF>(1, 4 * (rr >> 3) + (rr & 3), (rr >> 2) & 1);
  const uint8_t* khead = p.k_codes + ((int64_t)b * p.Hkv + hk) * p.Nk * HALF;
  const uint8_t* shead = p.k_scales + ((int64_t)b * p.Hkv + hk) * p.Nk * (D / 16);
  const int64_t col0 = (int64_t)b * p.nk_pad;
  const uint8_t* vhead = VF == VF_MXFP4 ? p.v_codes + (int64_t)hk * D * (p.cols / 2) + col0 / 2
                                        : p.v_codes + (int64_t)hk * D * p.cols + col0;
  const uint8_t* vshead = VF == VF_MXFP4 ? p.v_scales + (int64_t)hk * D * (p.cols / 32) + col0 / 32 : nullptr;

  auto load = [&](DecBuf<D, VF>& bf, int s) {
    int jc = s * DEC_WAVES + wave;
    jc = jc < n_chunks ? jc : n_chunks - 1;      // past the end: the last chunk again (a cache hit)
    const int key0 = jc * DEC_CHUNK;
    const uint8_t* kb = khead + (int64_t)key0 * HALF;
    const uint8_t* sb = shead + (int64_t)key0 * (D / 16);
    const int last = len_k - 1 - key0;           // keys past the sequence read its last key instead
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int kl = s2 == 0 ? kl0 : kl1;
      const int kr = kl <= last ? kl : last;
      const uint32_t ko = (uint32_t)(kr * HALF + hh * LB);
      const uint32_t so = (uint32_t)(kr * (D / 16) + hh * LS);
#pragma unroll
      for (int c = 0; c < D / 64; ++c) bf.kc[s2][c] = *reinterpret_cast<const u32x4*>(kb + ko + 16 * c);
      if (D == 128) bf.ks[s2] = *reinterpret_cast<const uint32_t*>(sb + so);
      else bf.ks[s2] = *reinterpret_cast<const uint16_t*>(sb + so);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t d = (uint32_t)(32 * dt + ql);
      if (VF == VF_FP8) {
        const uint8_t* vb = vhead + key0;
        bf.va[dt][0] = *reinterpret_cast<const u32x4*>(vb + d * (uint32_t)p.cols + 16 * hh);
        bf.va[dt][VF == VF_FP8 ? 1 : 0] = *reinterpret_cast<const u32x4*>(vb + d * (uint32_t)p.cols + 16 * hh + 32);
      } else {
        const uint8_t* vb = vhead + key0 / 2;
        bf.va[dt][0] = *reinterpret_cast<const u32x4*>(vb + d * (uint32_t)(p.cols / 2) + 16 * hh);
        const uint8_t* vsb = vshead + (key0 / 128) * 4;
        bf.vs[VF == VF_MXFP4 ? dt : 0] = *reinterpret_cast<const uint32_t*>(vsb + d * (uint32_t)(p.cols / 32));
      }
    }
  };

  // constant 0/1 operand of the row-sum MFMA (16x16x128, FP4 1.0 = code 2):
  // lane l of the accumulator ends up with the sum of query l % 32
  i32x8 ones = {0, 0, 0, 0, 0, 0, 0, 0};
  {
    const int row = lane & 15, g = lane >> 4;
    const bool r0 = (row == 0 || row == 8), r1 = (row == 4 || row == 12);
    if (PF == PF_MXFP4) {
      // rows 0/8 sum k-blocks {0,2}, rows 4/12 k-blocks {1,3}; lane holds k = 32g + [0,32)
      const bool on = (r0 && (g == 0 || g == 2)) || (r1 && (g == 1 || g == 3));
      if (on) { ones[0] = ones[1] = ones[2] = ones[3] = 0x22222222; }
    } else {
      // FP8 P: rows 0/8 sum k with k%32 < 16, rows 4/12 k%32 >= 16
      if (r0) { ones[0] = ones[1] = 0x22222222; }
      if (r1) { ones[2] = ones[3] = 0x22222222; }
    }
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();   // running max after the last tile (same in every wave)
  float m_w = -__builtin_inff();     // max the wave's partial O / l refer to

  // ---- one step: chunk j = 4 s + wave
  auto body = [&](int s, const DecBuf<D, VF>& bf) {
    const int j = s * DEC_WAVES + wave;
    const bool live = j < n_chunks;            // wave-uniform
    f32x16 sacc[2];
    float bm = -__builtin_inff();
    if (live) {
      // S^T = K Q^T for the chunk's two 32-key sub-tiles
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const f16x2 sc01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bf.ks[s2], 1.0f, false);
        const f16x2 sc23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bf.ks[s2], 1.0f, true);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint32_t w = bf.kc[s2][ks >> 2][ks & 3];
          const int blk = ks >> 1;               // block of 16 channels within the lane's half
          const _Float16 sc = blk == 0 ? sc01[0] : blk == 1 ? sc01[1] : blk == 2 ? sc23[0] : sc23[1];
          const f16x2 s2v = {sc, sc};
          const f16x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2v;
          const f16x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2v;
          const f16x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2v;
          const f16x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2v;
          const f16x8 a = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
          sacc[s2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[ks], ks == 0 ? f32x16{} : sacc[s2], 0, 0, 0);
        }
      }
      // mask keys past the sequence and (causal) past each row's position
      const int key0 = j * DEC_CHUNK;
      if (key0 + DEC_CHUNK > len_k || (CAUSAL && key0 + DEC_CHUNK - 1 > len_k - p.nq)) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = key0 + dec_key<PF>(s2, v, hh);
            const bool dead = key >= len_k || (CAUSAL && key > my_pos);
            if (dead) sacc[s2][v] = -__builtin_inff();
          }
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int v = 0; v < 16; ++v) bm = __builtin_fmaxf(bm, sacc[s2][v]);
    }
    // chunk max of the lane's query (both lane halves), through LDS to every wave
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    const float cmax = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    float* slot = sM + (s & 1) * DEC_WAVES * 32;
    if (hh == 0) slot[wave * 32 + ql] = cmax;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // running max after each of the step's two tiles; this wave's tile is wave / 2
    float m_tile = m_run;
#pragma unroll
    for (int t = 0; t < DEC_WAVES / 2; ++t) {
      const float tmax = __builtin_fmaxf(slot[(2 * t) * 32 + ql], slot[(2 * t + 1) * 32 + ql]) * cc;
      m_run = __builtin_fmaxf(m_run, tmax);
      if (t == (wave >> 1)) m_tile = m_run;
    }
    if (!live) return;

    // ---- encode the chunk with m' of its tile
    const bool row_dead = m_tile == -__builtin_inff();
    int psc;
    float me;
    if (PF == PF_MXFP4) {
      const float xmax = bm * cc - m_tile;       // fl(fl(S*c) - m')
      const float fl = __builtin_floorf(xmax);
      const int e = (row_dead || !(fl >= -125.0f)) ? -127 : (int)fl - 2;   // -127 also for no live key
      psc = e + 127;
      me = row_dead ? 0.0f : m_tile + (float)e;
    } else {
      psc = 127;
      me = row_dead ? 0.0f : m_tile;
    }
    i32x8 pw = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int v = 2 * k;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[s2][v], cc, -me));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[s2][v + 1], cc, -me));
        if (PF == PF_MXFP4) {
          const int word = 2 * s2 + (k >> 2), byte = k & 3;   // key 16 s2 + v of the lane's block
          uint32_t w = (uint32_t)pw[word];
          if (byte == 0) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p0, p1, 1.0f, 0);
          else if (byte == 1) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p0, p1, 1.0f, 1);
          else if (byte == 2) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p0, p1, 1.0f, 2);
          else w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p0, p1, 1.0f, 3);
          pw[word] = (int)w;
        } else {
          const int word = 4 * s2 + (k >> 1);
          if (k & 1) pw[word] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pw[word], true);
          else pw[word] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pw[word], false);
        }
      }
    if (DEBUG && b == p.dbg_b && my_h == p.dbg_h && row_ok) {
      const int64_t row = (int64_t)my_i * p.dbg_ld;
      const int key0 = j * DEC_CHUNK;
      if (PF == PF_MXFP4) {
        const int key = key0 + 32 * hh;
        *reinterpret_cast<u32x4*>(p.dbg_codes + (row + key) / 2) =
            u32x4{(uint32_t)pw[0], (uint32_t)pw[1], (uint32_t)pw[2], (uint32_t)pw[3]};
        p.dbg_scales[(row + key) / 32] = (uint8_t)psc;
      } else {
        const int key = key0 + 16 * hh;
        *reinterpret_cast<u32x4*>(p.dbg_codes + row + key) =
            u32x4{(uint32_t)pw[0], (uint32_t)pw[1], (uint32_t)pw[2], (uint32_t)pw[3]};
        *reinterpret_cast<u32x4*>(p.dbg_codes + row + key + 32) =
            u32x4{(uint32_t)pw[4], (uint32_t)pw[5], (uint32_t)pw[6], (uint32_t)pw[7]};
      }
    }

    // ---- bring the wave's partial to the tile's max, then accumulate
    const float alpha = row_dead ? 1.0f : __builtin_amdgcn_exp2f(m_w - m_tile);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
      lacc[0] *= alpha;
    }
    m_w = m_tile;
    lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pw, lacc, 4, PF == PF_MXFP4 ? 4 : 0, 0, 127, 0,
                                                            psc);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      if (VF == VF_MXFP4) {
        const i32x8 a = {(int)bf.va[dt][0][0], (int)bf.va[dt][0][1], (int)bf.va[dt][0][2], (int)bf.va[dt][0][3],
                         0, 0, 0, 0};
        const int vsc = (int)(bf.vs[VF == VF_MXFP4 ? dt : 0] >> (8 * hh));   // byte 2c: block (c, hh)
        if (wave & 1)
          oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pw, oacc[dt], 4, PF == PF_MXFP4 ? 4 : 0, 2,
                                                                     vsc, 0, psc);
        else
          oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pw, oacc[dt], 4, PF == PF_MXFP4 ? 4 : 0, 0,
                                                                     vsc, 0, psc);
      } else {
        const u32x4 x = bf.va[dt][0], y = bf.va[dt][VF == VF_FP8 ? 1 : 0];
        const i32x8 a = {(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
        oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pw, oacc[dt], 0, PF == PF_MXFP4 ? 4 : 0, 0, 127,
                                                                   0, psc);
      }
    }
  };

  // ---- the key loop: three register buffers, loads two steps ahead
  if (n_steps > 0) {
    DecBuf<D, VF> b0, b1, b2;
    load(b0, 0);
    load(b1, 1);
    int s = 0;
    for (;;) {
      load(b2, s + 2);
      body(s, b0);
      if (++s == n_steps) break;
      load(b0, s + 2);
      body(s, b1);
      if (++s == n_steps) break;
      load(b1, s + 2);
      body(s, b2);
      if (++s == n_steps) break;
    }
  }

  // ---- combine the four partials at the final max, O = o / l, LSE
  const float f = m_w == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_w - m_run);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) sO[((wave * DT + dt) * 16 + v) * 64 + lane] = oacc[dt][v] * f;
  sL[wave * 64 + lane] = lacc[0] * f;
  __syncthreads();
  if (wave >= DT || !row_ok) return;
  float l = 0.0f;
#pragma unroll
  for (int w = 0; w < DEC_WAVES; ++w) l += sL[w * 64 + lane];
  const bool empty = !(l > 0.0f);
  const float inv = empty ? 0.0f : vscale / l;
  const int dt = wave;
  const int64_t orow = (((int64_t)b * p.nq + my_i) * p.Hq + my_h) * (int64_t)D;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int d = 32 * dt + 8 * jj + 4 * hh;
    float o4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < DEC_WAVES; ++w) acc += sO[((w * DT + dt) * 16 + 4 * jj + k) * 64 + lane];
      o4[k] = acc * inv;
    }
    if (p.o_f32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + orow + d) = f32x4{o4[0], o4[1], o4[2], o4[3]};
    } else {
      uint32_t u[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t x = __float_as_uint(o4[k]);
        u[k] = (x + 0x7FFFu + ((x >> 16) & 1u)) >> 16;   // round to nearest even
      }
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.o) + orow + d) =
          u32x2{u[0] | (u[1] << 16), u[2] | (u[3] << 16)};
    }
  }
  if (p.lse != nullptr && dt == 0 && hh == 0) {
    const float lse = empty ? -__builtin_inff() : 0.6931471805599453f * (m_run + __builtin_log2f(l));
    p.lse[((int64_t)b * p.Hq + my_h) * p.nq + my_i] = lse;
  }
}

template <int D, int VF>
constexpr int dec_lds_bytes() {
  return (2 * DEC_WAVES * 32 + DEC_WAVES * (D / 32) * 16 * 64 + DEC_WAVES * 64) * 4;
}

template <int D, int PF, int VF, bool CAUSAL, bool DEBUG>
static hipError_t launch_dec_t(const DecParams& p, int nwg, hipStream_t st) {
  auto kern = decode_kernel<D, PF, VF, CAUSAL, DEBUG>;
  const int lds = dec_lds_bytes<D, VF>();
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(64 * DEC_WAVES), lds, st, p);
  return hipGetLastError();
}

template <int D, int PF, int VF>
static hipError_t launch_dec_c(const DecParams& p, int nwg, bool causal, bool debug, hipStream_t st) {
  if (causal)
    return debug ? launch_dec_t<D, PF, VF, true, true>(p, nwg, st) : launch_dec_t<D, PF, VF, true, false>(p, nwg, st);
  return debug ? launch_dec_t<D, PF, VF, false, true>(p, nwg, st) : launch_dec_t<D, PF, VF, false, false>(p, nwg, st);
}

template <int D>
static hipError_t launch_dec_d(const DecParams& p, int nwg, int pf, int vf, bool causal, bool debug, hipStream_t st) {
  if (pf == PF_MXFP4)
    return vf == VF_MXFP4 ? launch_dec_c<D, PF_MXFP4, VF_MXFP4>(p, nwg, causal, debug, st)
                          : launch_dec_c<D, PF_MXFP4, VF_FP8>(p, nwg, causal, debug, st);
  return launch_dec_c<D, PF_FP8, VF_FP8>(p, nwg, causal, debug, st);
}

hipError_t launch_decode(const DecParams& p, int D, int pf, int vf, bool causal, bool debug, hipStream_t st) {
  const int nwg = p.B * p.Hkv * p.QG;
  if (nwg == 0) return hipSuccess;
  return D == 64 ? launch_dec_d<64>(p, nwg, pf, vf, causal, debug, st)
                 : launch_dec_d<128>(p, nwg, pf, vf, causal, debug, st);
}

}  // namespace attn
