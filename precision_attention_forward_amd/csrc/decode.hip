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
//  * One workgroup of four waves per (sequence, KV head, 16 query rows): the
//    G * nq query rows of a KV head are the columns of S^T = K Q^T, so the
//    cache is read once for the whole GQA group.  With so few rows the 16x16
//    matrix instructions waste least: S^T on v_mfma_f32_16x16x32_f16, P.V and
//    the row sum l on v_mfma_scale_f32_16x16x128_f8f6f4 (l against a constant
//    0/1 operand, so it sums exactly the rounded probabilities).  The key rows
//    of each 16-key S^T sub-tile are permuted so that every group of 16 lanes
//    ends up holding, for its query, the 32 keys its probability operand
//    needs: one E8M0 block for MXFP4 P, whose block max, exponent and codes
//    are then lane-local.
//  * Waves take interleaved 128-key tiles (step s: wave w takes tile 4s + w),
//    keep their own O / l partials, and exchange per-tile row maxima through
//    LDS once per step, so that every wave encodes with the running max m' of
//    its own tile: the codes of one sequential pass, which splitting the keys
//    over independent workgroups would not give.
//  * Each wave streams its own tiles.  K codes and scales go by direct
//    global->LDS copies into two buffers of the wave, two steps ahead; the
//    16-byte chunks of each code row are XOR-swizzled so that the 16 rows of
//    one operand read fall on distinct banks.  V goes straight into registers
//    one step ahead (issued as soon as the step's P.V has read the previous
//    tile), from the decode cache layout in which each (sequence, KV head,
//    128-key tile) is one contiguous block: the V^T rows of a tile in the
//    forward's layout lie a whole cache row apart, and reading such 128-byte
//    pieces streams far below the rate of contiguous blocks.  The K copies
//    carry the non-temporal hint (the cache is read once per step).  At most 256 registers and ~75 KB of LDS per workgroup let two
//    workgroups share a CU, i.e. two waves per SIMD, so that one wave's
//    matrix products overlap the other's K decode and softmax.
//  * At the end the four partials are rescaled to the final max and summed
//    through LDS.
#include "common.h"
#include "dec_params.h"
#include "fwd_params.h"
#include "pipeline.h"

namespace attn {

constexpr int DEC_WAVES = 4;
constexpr int DEC_Q = 16;          // query rows per workgroup (columns of S^T)

// Key (0..127) of a 128-key tile at S^T sub-tile st (0..7), output row r
// (0..15) of the 16x16 MFMA: lane group g = r / 4 ends up holding, over the
// eight sub-tiles, exactly the 32 keys its probability operand needs in the
// 16x16x128 scaled MFMA -- MXFP4: keys 32 g + [0, 32) (one P block); FP8:
// keys 16 g + [0, 16) and 64 + 16 g + [0, 16) (the FP8 operand order) --
// with element 4 st + (r % 4) in operand order.
template <int PF>
__host__ __device__ inline int dec_key(int st, int r) {
  const int g = r >> 2, i = r & 3;
  if (PF == PF_MXFP4) return 32 * g + 4 * st + i;
  return st < 4 ? 16 * g + 4 * st + i : 64 + 16 * g + 4 * (st - 4) + i;
}

// LDS bytes of one K tile: 128 rows of D/2 code bytes, then 128 rows of D/16
// E4M3 block-scale bytes.
template <int D>
constexpr int dec_ktile_bytes() {
  return KEY_TILE * (D / 2 + D / 16);
}
// Copy instructions per K tile (1 KB of codes each; the scales in one 1 KB
// copy at D = 128, two 256-byte copies at D = 64) and load instructions per V
// tile (per 16 rows of V^T: two 16-byte loads for FP8, one 16-byte code load
// and one 4-byte scale load for MXFP4).
template <int D>
constexpr int dec_k_copies() {
  return D / 16 + (D == 128 ? 1 : 2);
}
template <int D>
constexpr int dec_v_loads() {
  return 2 * (D / 16);
}
// Position of 16-byte chunk c of K code row k (D = 128: four 64-byte rows
// per 256 bytes) in LDS: c ^ kswz(k).  The 16 lanes of one operand read take
// keys 32 j + 4 st + i (MXFP4 P) or 16 j + 4 st + i (FP8 P), i, j in 0..3;
// kswz sends the four values of j to four different chunks, so the 16 reads
// hit 16 different 16-byte bank groups of a 256-byte window.  (A variant that
// also separated them within 128-byte windows counted more bank conflicts on
// gfx950 and ran no faster.)
__host__ __device__ constexpr int dec_kswz(int k) { return ((k >> 4) ^ (k >> 5)) & 3; }

template <int D, int PF, int VF, bool CAUSAL, bool DEBUG>
__global__ void __launch_bounds__(256, 2) decode_kernel(DecParams p) {
  constexpr int KS = D / 32;     // k-steps (32 channels) of the S MFMA
  constexpr int DT = D / 16;     // 16-row tiles of O^T
  constexpr int HALF = D / 2;    // code bytes per row
  constexpr int GC = D / 4;      // channels of one lane group
  constexpr int KT = dec_ktile_bytes<D>();
  constexpr int KSC = KEY_TILE * HALF;                              // scale rows within a K tile
  constexpr int NK = dec_k_copies<D>(), NV = dec_v_loads<D>();
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* sM = reinterpret_cast<float*>(smem);                       // [2][DEC_WAVES][16] tile maxima
  float* sL = sM + 2 * DEC_WAVES * DEC_Q;                           // [DEC_WAVES][64] partial l
  uint8_t* sKall = smem + (2 * DEC_WAVES * DEC_Q + DEC_WAVES * 64) * 4;   // [DEC_WAVES][2][KT] K tiles
  float* sO = reinterpret_cast<float*>(sKall);                      // [DEC_WAVES][DT][4][64] partial O, after the loop
  static_assert(DEC_WAVES * DT * 4 * 64 * 4 <= DEC_WAVES * 2 * KT, "the partial O fits the K tiles");

  // ---- workgroup -> (sequence, KV head, query group)
  const int lin = blockIdx.x;
  const int qg = __builtin_amdgcn_readfirstlane(lin % p.QG);
  const int hk = __builtin_amdgcn_readfirstlane((lin / p.QG) % p.Hkv);
  const int b = __builtin_amdgcn_readfirstlane(lin / (p.QG * p.Hkv));
  int len_k = p.seqlens != nullptr ? p.seqlens[b] : p.Nk;
  len_k = len_k < 0 ? 0 : (len_k > p.Nk ? p.Nk : len_k);          // reads stay inside the cache
  len_k = __builtin_amdgcn_readfirstlane(len_k);
  const int G = p.Hq / p.Hkv;
  const int R = G * p.nq;                                            // query rows of this KV head

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  // query row of this lane's S^T column: row r = token i * G + head
  const int my_r = DEC_Q * qg + n;
  const bool row_ok = my_r < R;
  const int my_i = row_ok ? my_r / G : 0;
  const int my_h = hk * G + (row_ok ? my_r % G : 0);
  const int my_pos = len_k - p.nq + my_i;                            // absolute position (causal)

  const int n_tiles = (len_k + KEY_TILE - 1) / KEY_TILE;
  const int n_steps = (n_tiles + DEC_WAVES - 1) / DEC_WAVES;

  const float cc = (float)((double)p.sigma * 1.4426950408889634 * (double)(*p.gq) * (double)(*p.gk));
  const float vscale = VF == VF_FP8 ? *p.sv : 1.0f;

  // ---- Q operand (B of S^T, 16x16x32): lane (n, g) holds query row my_r,
  // channels GC g + 8 ks + [0, 8) in k-step ks, decoded from NVFP4 (exact in FP16)
  f16x8 qf[KS];
  {
    const int64_t row = row_ok ? ((int64_t)b * p.nq + my_i) * p.Hq + my_h : 0;
    const uint8_t* qc = p.q_codes + row * HALF + g * (GC / 2);
    const uint8_t* qs = p.q_scales + row * (D / 16) + g * (GC / 16);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t cw = row_ok ? *reinterpret_cast<const uint32_t*>(qc + 4 * ks) : 0u;
      const float sv = e4m3_decode(row_ok ? qs[ks >> 1] : 0u);
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[ks][j] = (_Float16)(e2m1_decode((cw >> (4 * j)) & 0xFu) * sv);
    }
  }

  // ---- tile bases (64-bit) and per-lane offsets within a tile
  const int rr = lane & 15;
  const uint8_t* khead = p.k_codes + ((int64_t)b * p.Hkv + hk) * p.Nk * HALF;
  const uint8_t* shead = p.k_scales + ((int64_t)b * p.Hkv + hk) * p.Nk * (D / 16);
  // V cache: one block of D key-contiguous rows (V^T) per (sequence, KV head, 128-key tile)
  constexpr int VROWB = VF == VF_MXFP4 ? KEY_TILE / 2 : KEY_TILE;       // code bytes of a block row
  const int64_t vtile0 = ((int64_t)b * p.Hkv + hk) * (p.Nk / KEY_TILE);
  auto tile_of = [&](int s) { return s * DEC_WAVES + wave; };   // loaded only while below n_tiles

  // K tiles: copied into two LDS buffers of this wave, two steps ahead.
  // Keys past the sequence but inside its cache (the capacity is whole
  // 128-key tiles) are read and masked later.
  uint8_t* sK = sKall + wave * 2 * KT;
  const uint32_t sK_lds = lds_address(sK);
  // D = 128: lane l of copy i writes key 16 i + l / 4, LDS chunk l % 4, which
  // holds its chunk (l % 4) ^ kswz(key); kswz(16 i + r) = kswz(16 i) for r < 16.
  uint32_t kcp_off[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) kcp_off[f] = (uint32_t)((lane >> 2) * HALF + 16 * ((lane & 3) ^ f));
  auto copy_k = [&](int s, int buf) {
    const int key0 = tile_of(s) * KEY_TILE;
    const uint8_t* kb = khead + (int64_t)key0 * HALF;
    const uint8_t* sb = shead + (int64_t)key0 * (D / 16);
    const uint32_t dst = sK_lds + buf * KT;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      // copy i: 1 KB of code rows (16 keys at D = 128, 32 at D = 64)
      const uint32_t off = D == 128 ? kcp_off[dec_kswz(16 * i)] : (uint32_t)(16 * lane);
      dma16_nt(kb + 1024 * i, off, dst + 1024 * i);
    }
    if (D == 128) {
      dma16_nt(sb, (uint32_t)(16 * lane), dst + KSC);
    } else {
      dma4_nt(sb, (uint32_t)(4 * lane), dst + KSC);
      dma4_nt(sb + 256, (uint32_t)(4 * lane), dst + KSC + 256);
    }
  };
  // the lane's operand reads of sub-tile st within a K tile (loop invariant)
  uint32_t kr_off[8], sr_off[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    const int kl = dec_key<PF>(st, rr);
    kr_off[st] = D == 128 ? (uint32_t)(kl * HALF + 16 * (g ^ dec_kswz(kl))) : (uint32_t)(kl * HALF + 8 * g);
    sr_off[st] = (uint32_t)(KSC + kl * (D / 16) + g * (GC / 16));
  }

  // V tile: straight into registers, one step ahead
  u32x4 va[DT][VF == VF_FP8 ? 2 : 1];    // V^T operand per 16 channels
  uint32_t vs[VF == VF_MXFP4 ? DT : 1];  // MXFP4 V: E8M0 bytes of the tile's four blocks
  const uint32_t voff = (uint32_t)(rr * VROWB + 16 * g);   // row rr of a 16-row group, the lane's 16 bytes
  auto load_v = [&](int s) {
    const int64_t t = vtile0 + tile_of(s);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint8_t* vb = p.v_codes + t * (D * VROWB) + 16 * dt * VROWB;
      va[dt][0] = *reinterpret_cast<const u32x4*>(vb + voff);
      if (VF == VF_FP8)
        va[dt][VF == VF_FP8 ? 1 : 0] = *reinterpret_cast<const u32x4*>(vb + voff + 64);
      else
        vs[VF == VF_MXFP4 ? dt : 0] = *reinterpret_cast<const uint32_t*>(p.v_scales + (t * D + 16 * dt + rr) * 4);
    }
  };

  // constant 0/1 operand of the row-sum MFMA (16x16x128, FP4 1.0 = code 2):
  // rows 0, 4, 8, 12 sum all 128 keys, so register 0 of every lane holds l of its query
  i32x8 ones = {0, 0, 0, 0, 0, 0, 0, 0};
  if ((rr & 3) == 0) { ones[0] = ones[1] = ones[2] = ones[3] = 0x22222222; }

  f32x4 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();   // running max after the last tile (same in every wave)
  float m_w = -__builtin_inff();     // max the wave's partial O / l refer to

  // ---- one step: tile j = 4 s + wave
  auto body = [&](int s) {
    const int j = s * DEC_WAVES + wave;
    const bool live = j < n_tiles;             // wave-uniform
    f32x4 sacc[8];
    float bm = -__builtin_inff();
    if (live) {
      // S^T = K Q^T, eight 16-key sub-tiles, K from this wave's LDS tile
      const uint8_t* kt = sK + (s & 1) * KT;
      u32x4 kc_next;
      uint32_t ksc_next;
      auto read_k = [&](int st) {   // operands of sub-tile st, read one sub-tile ahead
        if (D == 128) {
          kc_next = *reinterpret_cast<const u32x4*>(kt + kr_off[st]);
          ksc_next = *reinterpret_cast<const uint16_t*>(kt + sr_off[st]);
        } else {
          const u32x2 w = *reinterpret_cast<const u32x2*>(kt + kr_off[st]);
          kc_next = u32x4{w[0], w[1], 0u, 0u};
          ksc_next = kt[sr_off[st]];
        }
      };
      read_k(0);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x4 kc = kc_next;
        const uint32_t ksc = ksc_next;
        if (st < 7) read_k(st + 1);
        const f16x2 scp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ksc, 1.0f, false);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint32_t w = kc[ks];
          const _Float16 sc = (ks >> 1) == 0 ? scp[0] : scp[1];   // block of 16 channels
          const f16x2 s2v = {sc, sc};
          const f16x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2v;
          const f16x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2v;
          const f16x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2v;
          const f16x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2v;
          const f16x8 a = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
          sacc[st] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qf[ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[st],
                                                            0, 0, 0);
        }
      }
      // mask keys past the sequence and (causal) past each row's position
      const int key0 = j * KEY_TILE;
      if (key0 + KEY_TILE > len_k || (CAUSAL && key0 + KEY_TILE - 1 > len_k - p.nq)) {
        // live keys of the lane's row: key < lim (one compare per score)
        const int lim = (CAUSAL ? min(len_k, my_pos + 1) : len_k) - key0;
#pragma unroll
        for (int st = 0; st < 8; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sacc[st][i] = dec_key<PF>(st, 4 * g + i) < lim ? sacc[st][i] : -__builtin_inff();
      }
#pragma unroll
      for (int st = 0; st < 8; ++st)
        bm = __builtin_fmaxf(bm, __builtin_fmaxf(__builtin_fmaxf(sacc[st][0], sacc[st][1]),
                                                 __builtin_fmaxf(sacc[st][2], sacc[st][3])));
    }
    // tile max of the lane's query (its four lane groups), through LDS to every wave
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    float tm = __builtin_fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tm), __float_as_uint(tm), false, false);
    tm = __builtin_fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
    float* slot = sM + (s & 1) * DEC_WAVES * DEC_Q;
    if (g == 0) slot[wave * DEC_Q + n] = tm;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // running max after each of the step's four tiles; this wave's tile is the wave-th
    float m_tile = m_run;
#pragma unroll
    for (int t = 0; t < DEC_WAVES; ++t) {
      m_run = __builtin_fmaxf(m_run, slot[t * DEC_Q + n] * cc);
      if (t == wave) m_tile = m_run;
    }
    if (!live) return;

    // ---- encode the tile with m' (its running max)
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
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[st][2 * h2], cc, -me));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[st][2 * h2 + 1], cc, -me));
        if (PF == PF_MXFP4) {
          // element 4 st + 2 h2 (+1): word st / 2, byte 2 (st % 2) + h2
          const int word = st >> 1, byte = 2 * (st & 1) + h2;
          uint32_t w = (uint32_t)pw[word];
          if (byte == 0) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p0, p1, 1.0f, 0);
          else if (byte == 1) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p0, p1, 1.0f, 1);
          else if (byte == 2) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p0, p1, 1.0f, 2);
          else w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p0, p1, 1.0f, 3);
          pw[word] = (int)w;
        } else {
          // element 4 st + 2 h2 (+1): word st, bytes 2 h2, 2 h2 + 1
          if (h2) pw[st] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pw[st], true);
          else pw[st] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pw[st], false);
        }
      }
    if (DEBUG && b == p.dbg_b && my_h == p.dbg_h && row_ok) {
      const int64_t row = (int64_t)my_i * p.dbg_ld;
      const int key0 = j * KEY_TILE;
      if (PF == PF_MXFP4) {
        const int key = key0 + 32 * g;
        *reinterpret_cast<u32x4*>(p.dbg_codes + (row + key) / 2) =
            u32x4{(uint32_t)pw[0], (uint32_t)pw[1], (uint32_t)pw[2], (uint32_t)pw[3]};
        p.dbg_scales[(row + key) / 32] = (uint8_t)psc;
      } else {
        *reinterpret_cast<u32x4*>(p.dbg_codes + row + key0 + 16 * g) =
            u32x4{(uint32_t)pw[0], (uint32_t)pw[1], (uint32_t)pw[2], (uint32_t)pw[3]};
        *reinterpret_cast<u32x4*>(p.dbg_codes + row + key0 + 64 + 16 * g) =
            u32x4{(uint32_t)pw[4], (uint32_t)pw[5], (uint32_t)pw[6], (uint32_t)pw[7]};
      }
    }

    // ---- bring the wave's partial to the tile's max, then accumulate
    const float alpha = row_dead ? 1.0f : __builtin_amdgcn_exp2f(m_w - m_tile);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[dt][i] *= alpha;
      lacc[0] *= alpha;
    }
    m_w = m_tile;
    lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pw, lacc, 4, PF == PF_MXFP4 ? 4 : 0, 0, 127, 0,
                                                            psc);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      if (VF == VF_MXFP4) {
        const u32x4 x = va[dt][0];
        const i32x8 a = {(int)x[0], (int)x[1], (int)x[2], (int)x[3], 0, 0, 0, 0};
        const int vsc = (int)(vs[VF == VF_MXFP4 ? dt : 0] >> (8 * g));   // block g of the tile
        oacc[dt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, pw, oacc[dt], 4, PF == PF_MXFP4 ? 4 : 0, 0,
                                                                    vsc, 0, psc);
      } else {
        const u32x4 x = va[dt][0], y = va[dt][VF == VF_FP8 ? 1 : 0];
        const i32x8 a = {(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
        oacc[dt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, pw, oacc[dt], 0, PF == PF_MXFP4 ? 4 : 0, 0, 127,
                                                                    0, psc);
      }
    }
  };

  // ---- the key loop.  Per step the wave issues, in this order, the V loads
  // of the next step (into the registers the step's P.V has just read) and
  // the K copies of the step after (into the LDS buffer the step's S has
  // read).  Memory operations complete in order, so at the top of step s the
  // K tile of s has landed once no more than NV + NK loads are outstanding
  // (those of V(s) and K(s + 1)); the compiler waits for V(s) itself before
  // the P.V products.
  // Only tiles the wave takes are loaded (live(s): tile 4 s + wave exists;
  // live(s + 1) implies live(s)), so the count also drops NK when the
  // next K tile is not loaded.
  auto live_step = [&](int s) { return s * DEC_WAVES + wave < n_tiles; };
  if (n_steps > 0) {
    if (live_step(0)) {
      copy_k(0, 0);
      load_v(0);
    }
    if (live_step(1)) copy_k(1, 1);
    for (int s = 0; s < n_steps; ++s) {
      if (live_step(s + 1))
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NV + NK) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NV) : "memory");
      body(s);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the step's LDS reads are done
      if (live_step(s + 1)) load_v(s + 1);
      if (live_step(s + 2)) copy_k(s + 2, s & 1);
    }
  }
  // no copy may still be writing the K tiles, which the partial O reuses
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ---- combine the four partials at the final max, O = o / l, LSE
  const float f = m_w == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_w - m_run);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *reinterpret_cast<f32x4*>(sO + ((wave * DT + dt) * 64 + lane) * 4) =
        f32x4{oacc[dt][0] * f, oacc[dt][1] * f, oacc[dt][2] * f, oacc[dt][3] * f};
  sL[wave * 64 + lane] = lacc[0] * f;
  __syncthreads();
  if (!row_ok) return;
  float l = 0.0f;
#pragma unroll
  for (int w = 0; w < DEC_WAVES; ++w) l += sL[w * 64 + lane];
  const bool empty = !(l > 0.0f);
  const float inv = empty ? 0.0f : vscale / l;
  const int64_t orow = (((int64_t)b * p.nq + my_i) * p.Hq + my_h) * (int64_t)D;
#pragma unroll
  for (int k = 0; k < DT / DEC_WAVES; ++k) {
    const int dt = wave * (DT / DEC_WAVES) + k;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) acc += *reinterpret_cast<const f32x4*>(sO + ((w * DT + dt) * 64 + lane) * 4);
    const f32x4 o4 = acc * inv;
    const int d = 16 * dt + 4 * g;
    if (p.o_f32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + orow + d) = o4;
    } else {
      uint32_t u[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t x = __float_as_uint(o4[q]);
        u[q] = (x + 0x7FFFu + ((x >> 16) & 1u)) >> 16;   // round to nearest even
      }
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.o) + orow + d) =
          u32x2{u[0] | (u[1] << 16), u[2] | (u[3] << 16)};
    }
  }
  if (p.lse != nullptr && wave == 0 && g == 0) {
    const float lse = empty ? -__builtin_inff() : 0.6931471805599453f * (m_run + __builtin_log2f(l));
    p.lse[((int64_t)b * p.Hq + my_h) * p.nq + my_i] = lse;
  }
}

template <int D>
constexpr int dec_lds_bytes() {
  return (2 * DEC_WAVES * DEC_Q + DEC_WAVES * 64) * 4 + DEC_WAVES * 2 * dec_ktile_bytes<D>();
}

template <int D, int PF, int VF, bool CAUSAL, bool DEBUG>
static hipError_t launch_dec_t(const DecParams& p, int nwg, hipStream_t st) {
  auto kern = decode_kernel<D, PF, VF, CAUSAL, DEBUG>;
  const int lds = dec_lds_bytes<D>();
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
