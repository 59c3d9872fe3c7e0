// Direct-P FP4 attention forward and its FP8-P/V variant for gfx950.
//
// Method: "Hardware-Aware FP4 FlashAttention-4" (summary page, "What the paper
// found"; arXiv listing 2609.04105v1, abstract).  NVFP4 Q and K; per tile of
// 128 keys the running row max m' of the log2-domain scores is updated, the
// shifted scores are mapped straight to E2M1 probability codes with one E8M0
// exponent per 32 keys (Direct-P) or to E4M3 codes with a unit scale (FP8 P);
// the denominator is summed from the same rounded probabilities the P.V
// product consumes; O = o / l and LSE = ln2 * (m + log2 l).
//
// Exp-free variants (ENC = 1), from two related methods listed beside the
// arXiv entry ("VC-Attention: Value Smoothing and Softmax Casting for Low-bit
// Attention" for E4M3, "EFQ-Softmax: Exp-Free Quantization for Softmax" for
// block-scaled E2M1; abstracts only): a minifloat code read as an integer is
// a fixed-point log2 of its value (M mantissa bits, exponent bias b), so the
// code of 2^y is taken as clamp(RNE(2^M (y + b)), 0, top) -- one FMA of the
// raw score with per-row constants, then v_cvt_pk_u8_f32 (round to nearest
// even, clamped to [0, 255]) -- instead of exp2 and a format conversion.
// Same running max, block exponents, denominator and P.V as ENC = 0.
//
// gfx950 mapping (the pages' Blackwell pipeline is prior art, not copied):
//  * NVFP4 blocks carry an E4M3 scale per 16 elements; the scaled MFMA takes
//    one E8M0 scale per 32, so Q.K^T is run as an FP16 MFMA on the exact
//    dequantized values (E2M1 x E4M3 has at most 6 significant bits).  A
//    pre-pass expands K once into 128-key FP16 tiles laid out in the order
//    the MFMA operand is read; Q is decoded into FP16 operand registers at
//    the start of each workgroup.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_f16 puts one query per lane; the key
//    rows of K are permuted so that each lane ends up holding exactly the 32
//    keys of one P block (MXFP4) or the 32 keys the FP8 operand layout wants.
//    Block max, E8M0 exponent and E2M1/E4M3 encoding are then lane-local; the
//    row max needs one exchange with lane l^32.
//  * O^T += V^T P^T on v_mfma_scale_f32_32x32x64_f8f6f4 (P as the B operand,
//    its E8M0 block exponent as scale_b; MXFP4 V brings its own scale_a).
//  * l = sum of the dequantized P is computed by one 16x16x128 scaled MFMA
//    per 64 keys against a constant 0/1 operand, so it sums exactly the
//    rounded probabilities without any VALU work.
#include "common.h"
#include "fwd_params.h"
#include "pipeline.h"

namespace attn {


// Key (0..127) of S^T sub-tile st (0..3), accumulator register v (0..15), lane half hh.
// MXFP4 P: lane half hh of chunk c = st/2 owns keys 64c + 32hh + [0, 32).
// FP8 P  : lane half hh owns keys 64c + 16hh + [0,16) and 64c + 32 + 16hh + [0,16)
//          (the k order of the FP8 operand of the 32x32x64 MFMA).
template <int PF>
__host__ __device__ inline int s_key(int st, int v, int hh) {
  const int c = st >> 1, s2 = st & 1;
  return PF == PF_MXFP4 ? 64 * c + 32 * hh + 16 * s2 + v : 64 * c + 32 * s2 + 16 * hh + v;
}
// Accumulator row r (0..31) of a 32x32 MFMA output held by lane half hh, register v.
__host__ __device__ inline int out_row(int v, int hh) { return 8 * (v >> 2) + 4 * hh + (v & 3); }

// ---------------------------------------------------------------------------
// Pre-pass: exact FP16 expansion of NVFP4 K into the operand tile order.
//   K tile (128 keys, D): element (st, kh, ks, r, j) at (((st*2+kh)*KS+ks)*32+r)*8+j,
//     holding K[key = s_key(st, v(r), hh(r))][d = kh*D/2 + 8*ks + j], KS = D/16.
// The tile's code rows (D/2 bytes per key) and scale rows (D/16 bytes) are
// first staged in LDS with row-contiguous loads (consecutive keys of one head
// lie H rows apart); then each thread writes whole 16-byte chunks in output
// order (coalesced), gathering the 4 code bytes and the scale of its 8
// elements from LDS.  Keys past the end of the sequence are written as zeros.
template <int D, int PF>
__global__ void __launch_bounds__(256) expand_k_kernel(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales, int H, int N,
                                                       const int32_t* __restrict__ cu, int64_t n_pad, int64_t cols,
                                                       _Float16* __restrict__ out) {
  const int tile = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const bool varlen = cu != nullptr;
  const int64_t tok0 = varlen ? cu[s] : (int64_t)s * N;
  const int len = varlen ? cu[s + 1] - cu[s] : N;
  if (tile * KEY_TILE >= len) return;
  constexpr int KS = D / 16, HALF = D / 2, CHUNKS = KEY_TILE * D / 8;
  constexpr int CW = HALF / 4, SB = D / 16;          // code words and scale bytes per key
  __shared__ uint32_t scode[KEY_TILE][CW + 1];
  __shared__ uint8_t sscale[KEY_TILE][SB];
  for (int i = threadIdx.x; i < KEY_TILE * (CW / 2); i += 256) {   // 8-byte pieces of the code rows
    const int key = i / (CW / 2), c = i % (CW / 2);
    const int idx = tile * KEY_TILE + key;
    u32x2 w = {0u, 0u};
    if (idx < len) w = *reinterpret_cast<const u32x2*>(codes + ((tok0 + idx) * H + h) * HALF + 8 * c);
    scode[key][2 * c] = w[0];
    scode[key][2 * c + 1] = w[1];
  }
  for (int i = threadIdx.x; i < KEY_TILE * SB; i += 256) {
    const int key = i / SB, c = i % SB;
    const int idx = tile * KEY_TILE + key;
    sscale[key][c] = idx < len ? scales[((tok0 + idx) * H + h) * SB + c] : (uint8_t)0;
  }
  __syncthreads();
  _Float16* tb = out + ((int64_t)h * cols + kcol_offset(varlen, s, tok0, n_pad) + (int64_t)tile * KEY_TILE) * D;
  for (int u = threadIdx.x; u < CHUNKS; u += 256) {
    const int r = u & 31, ks = (u >> 5) % KS, kh = ((u >> 5) / KS) & 1, st = (u >> 5) / (2 * KS);
    const int hh = (r >> 2) & 1, v = 4 * (r >> 3) + (r & 3);   // inverse of out_row
    const int key = s_key<PF>(st, v, hh);
    const int d0 = kh * HALF + 8 * ks;
    const uint32_t cw = scode[key][d0 / 8];
    const float sv = e4m3_decode(sscale[key][d0 / 16]);
    f16x8 val;
#pragma unroll
    for (int j = 0; j < 8; ++j) val[j] = (_Float16)(e2m1_decode((cw >> (4 * j)) & 0xFu) * sv);
    *reinterpret_cast<f16x8*>(tb + u * 8) = val;
  }
}

// Pre-pass of the MX Q/K mode: MXFP4 K codes rearranged into 128-key operand
// tiles of the scaled FP4 S MFMA (no decoding).  Tile layout (K_BYTES =
// 64 D + 512 bytes): 16-byte unit (st, ks, kh, r) at ((st*KS + ks)*2 + kh)*32 + r
// holds the codes of d in 64 ks + 32 kh + [0, 32) of key s_key(st, v(r), hh(r))
// (KS = D/64), then one dword per (st, r) at 64 D + 4 (32 st + r) holding
// that key's D/32 E8M0 bytes (byte b = block b).  Keys past the end of the
// sequence get zero codes and zero bytes.
template <int D, int PF>
__global__ void __launch_bounds__(256) pack_k_mx_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales, int H, int N,
                                                        const int32_t* __restrict__ cu, int64_t n_pad, int64_t cols,
                                                        uint8_t* __restrict__ out) {
  const int tile = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const bool varlen = cu != nullptr;
  const int64_t tok0 = varlen ? cu[s] : (int64_t)s * N;
  const int len = varlen ? cu[s + 1] - cu[s] : N;
  if (tile * KEY_TILE >= len) return;
  constexpr int KS = D / 64, KC = KEY_TILE * D / 2, UNITS = KC / 16;
  uint8_t* tb = out + ((int64_t)h * (cols / KEY_TILE) + kcol_offset(varlen, s, tok0, n_pad) / KEY_TILE + tile) *
                          (int64_t)(KC + 512);
  for (int u = threadIdx.x; u < UNITS + 128; u += 256) {
    const bool is_code = u < UNITS;
    const int w = is_code ? u : u - UNITS;
    const int r = w & 31;
    const int kh = (w >> 5) & 1, ks = (w >> 6) % KS, st = is_code ? (w >> 6) / KS : w >> 5;
    const int hh = (r >> 2) & 1, v = 4 * (r >> 3) + (r & 3);   // inverse of out_row
    const int idx = tile * KEY_TILE + s_key<PF>(st, v, hh);
    const int64_t row = (tok0 + idx) * H + h;
    if (is_code) {
      u32x4 val = {0u, 0u, 0u, 0u};
      if (idx < len) val = *reinterpret_cast<const u32x4*>(codes + row * (D / 2) + 32 * ks + 16 * kh);
      *reinterpret_cast<u32x4*>(tb + u * 16) = val;
    } else {
      uint32_t val = 0u;
      if (idx < len)
        val = D == 128 ? *reinterpret_cast<const uint32_t*>(scales + row * 4)
                       : (uint32_t)*reinterpret_cast<const uint16_t*>(scales + row * 2);
      *reinterpret_cast<uint32_t*>(tb + KC + w * 4) = val;
    }
  }
}

// First vector unit of slot i of the key loop: slots [0, NPV) carry units
// [3, 13) (statistics and the encode of sub-tile 0); then each group of KS
// slots carries 8 units (encode of the next sub-tile; in the last group the
// rescale units, which run elsewhere).
template <int NPV, int KS>
__host__ __device__ constexpr int slot_unit_begin(int i) {
  return i < NPV ? 3 + (i * 10) / NPV : 13 + 8 * ((i - NPV) / KS) + (((i - NPV) % KS) * 8) / KS;
}

// Query blocks of one (sequence, head) dispatched to one XCD in a row in
// packed variable-length launches (see the kernel's workgroup order).
constexpr int VARLEN_QGROUP = 16;

// Slot after which the second wave group of a workgroup takes its barrier
// (the first group takes it after the last slot); see the key loop.
#ifndef ATTN_G1_BARRIER
#define ATTN_G1_BARRIER (NS - KS)
#endif
#ifndef ATTN_PRIO_MODE
#define ATTN_PRIO_MODE 1
#endif
#ifndef ATTN_PRIO_END
#define ATTN_PRIO_END (NPV - 1)
#endif

// K tile: FP16 operand tile (QK = 0), or (QK = 1) the MXFP4 codes in
// operand order followed by one E8M0 dword per (sub-tile, A-operand row).
template <int D, int VF, int QK = 0>
struct LdsLayout {
  static constexpr int KC_BYTES = QK ? KEY_TILE * D / 2 : KEY_TILE * D * 2;
  static constexpr int K_BYTES = KC_BYTES + (QK ? 4 * 32 * 4 : 0);
  static constexpr int V_BYTES = VF == VF_MXFP4 ? KEY_TILE * D / 2 : KEY_TILE * D;
  static constexpr int VS_BYTES = VF == VF_MXFP4 ? D * 4 : 0;              // E8M0 V scales
  static constexpr int V_SLOT = V_BYTES + VS_BYTES;
  static constexpr int RING = 3;                                            // tiles in flight
  static constexpr int V_BASE = RING * K_BYTES;
  static constexpr int TOTAL = RING * K_BYTES + RING * V_SLOT;
};

// Software pipeline of one wave (32 queries).  Iteration t of the key loop:
//   A: O^T += V(t-2)^T P(t-2)^T and l += sum P(t-2)      (matrix)
//      row max of S(t-1), m', alpha, block exponents,
//      encode keys 0..63 of S(t-1) -> P(t-1)            (vector)
//   B: S(t) sub-tiles 0,1 = K(t) Q^T                      (matrix)
//      encode keys 64..127 of S(t-1) -> P(t-1)           (vector)
//   C: S(t) sub-tiles 2,3                                 (matrix)
//      O *= alpha(t-1), l *= alpha(t-1)                   (vector)
// so every matrix step has independent vector work beside it in the same
// wave.  S sub-tiles are overwritten only after they have been encoded;
// P is double-buffered (P(t-2) is read while P(t-1) is written).  The
// 8 waves share K(t) / V(t-2) tiles in LDS; tiles for iteration t+1 are
// copied during iteration t and one barrier per iteration separates them.
//
// QK = 1 is the opt-in MX-native Q/K mode: Q and K carry MXFP4 codes with one
// E8M0 exponent per 32 elements along D, and each S sub-tile is D/64 scaled
// FP4 MFMAs (v_mfma_scale_f32_32x32x64_f8f6f4, both operands E2M1, the block
// exponents as scale_a / scale_b) instead of D/16 FP16 ones.  The S^T layout,
// and with it everything from the row max on, is unchanged.
// Phase trace (a diagnostic build only: compiled with -DATTN_FWD_PHASE_TRACE
// into its own library, libattnfp4_trace.so; the product library has none of
// it).  Workgroup 0 of a launch writes, per wave, the shader-clock cycles
// (s_memtime) that the wave spent in five phases of the key loop, summed over
// its iterations, and its tile count:
//   [0] from the previous iteration's end to the first slot (rescale, mask,
//       scale and operand loads), [1] slots 0 .. NPV-1, [2] slots
//       NPV .. NPV+2KS-1, [3] the remaining slots (waves 4-7 take their
//       barrier there), [4] after the last slot (waves 0-3 take theirs there);
//   [5] the number of key tiles.
// Each stamp is fenced by scheduling barriers, which perturbs the schedule a
// little.  attn_fwd_phase_trace_read copies the 8 x 8 table to the host.
#ifdef ATTN_FWD_PHASE_TRACE
__device__ unsigned long long g_fwd_phase_trace[8][8];
extern "C" hipError_t attn_fwd_phase_trace_read(unsigned long long* host_dst) {
  return hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(g_fwd_phase_trace), sizeof(g_fwd_phase_trace), 0,
                             hipMemcpyDeviceToHost);
}
#define FWD_PHASE_STAMP(k)                      \
  do {                                          \
    __builtin_amdgcn_sched_barrier(0);          \
    tstamp[k] = __builtin_amdgcn_s_memtime();   \
    __builtin_amdgcn_sched_barrier(0);          \
  } while (0)
#else
#define FWD_PHASE_STAMP(k) do {} while (0)
#endif

template <int D, int PF, int VF, bool CAUSAL, bool DEBUG, int ENC, int QK>
__global__ void __launch_bounds__(512, 1) fwd_lowp_kernel(FwdParams p) {
  constexpr int KS = QK ? D / 64 : D / 16;   // k-steps of the S MFMA per sub-tile
  constexpr int DT = D / 32;           // 32-row tiles of O^T
  constexpr int HALF = D / 2;
  using L = LdsLayout<D, VF, QK>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // ---- workgroup -> (batch, head, query block).
  // Dense batches: XCD-grouped, so that the query blocks of one head run on
  // one XCD and share its L2 copy of the head's K / V tiles (workgroups are
  // dispatched round-robin over the 8 XCDs).
  // Packed variable-length batches: sequences differ in length, so grouping
  // them by XCD would leave XCDs unevenly loaded; there the order is query
  // block major, from the last block down (only long sequences have high
  // blocks, and their workgroups are the longest-running).  Within that
  // order, VARLEN_QGROUP consecutive query blocks of one (sequence, head) go
  // to the same XCD one after another, so the workgroups running together
  // there stream the same K / V tiles through its L2; the (sequence, head)
  // pairs are dealt to XCDs by pair index mod 8, which gives every XCD the
  // same share of every sequence.  The grid is padded to whole groups
  // (workgroups with qb < 0 exit).
  const int nwg = gridDim.x;
  int lin = blockIdx.x;
  int qb, h, b;
  if (p.cu_q != nullptr) {
    const int npairs = p.B * p.Hq;
    if ((npairs & 7) == 0) {
      const int j = lin >> 3, np8 = npairs >> 3;
      const int t = j / VARLEN_QGROUP;
      const int pair = (t % np8) * 8 + (lin & 7);
      qb = p.QB - 1 - ((t / np8) * VARLEN_QGROUP + j % VARLEN_QGROUP);
      h = pair % p.Hq;
      b = pair / p.Hq;
    } else {
      qb = p.QB - 1 - lin / npairs;
      h = lin % p.Hq;
      b = (lin / p.Hq) % p.B;
    }
  } else {
    if ((nwg & 7) == 0) lin = (lin & 7) * (nwg >> 3) + (lin >> 3);
    qb = lin % p.QB;
    h = (lin / p.QB) % p.Hq;
    b = lin / (p.QB * p.Hq);
    if (CAUSAL) qb = p.QB - 1 - qb;    // longest rows first
  }
  // (uniform: keep them, and everything derived, in scalar registers)
  qb = __builtin_amdgcn_readfirstlane(qb);
  h = __builtin_amdgcn_readfirstlane(h);
  b = __builtin_amdgcn_readfirstlane(b);
  const bool varlen = p.cu_q != nullptr;
  const int64_t tq0 = varlen ? p.cu_q[b] : (int64_t)b * p.Nq;
  const int64_t tk0 = varlen ? p.cu_k[b] : (int64_t)b * p.Nk;
  const int len_q = varlen ? p.cu_q[b + 1] - p.cu_q[b] : p.Nq;
  const int len_k = varlen ? p.cu_k[b + 1] - p.cu_k[b] : p.Nk;
  if (qb < 0 || qb * WG_Q >= len_q) return;
  const int hk = h / (p.Hq / p.Hkv);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: kept in a scalar register
  const int hh = lane >> 5, ql = lane & 31;
  const int q0 = qb * WG_Q + wave * WAVE_Q;     // first query of this wave
  const int my_q = q0 + ql;
  const bool wave_active = q0 < len_q;

  int n_tiles = (len_k + KEY_TILE - 1) / KEY_TILE;
  if (CAUSAL) {
    const int last_q = min(qb * WG_Q + WG_Q, len_q) - 1;
    n_tiles = min(n_tiles, last_q / KEY_TILE + 1);
  }
  // No key at all (Nk = 0, or an empty key sequence of a packed batch): every
  // row has an empty softmax, O = 0 and LSE = -inf, and nothing of K or V
  // may be read (their buffers can be empty).  Uniform per workgroup, before
  // any barrier.
  if (n_tiles == 0) {
    if (wave_active && my_q < len_q) {
      const int64_t orow = ((tq0 + my_q) * p.Hq + h) * (int64_t)D + hh * HALF;
      if (p.o_f32) {
#pragma unroll
        for (int d = 0; d < HALF; d += 4)
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + orow + d) = f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
#pragma unroll
        for (int d = 0; d < HALF; d += 8)
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.o) + orow + d) = u32x4{0u, 0u, 0u, 0u};
      }
      if (p.lse != nullptr && hh == 0) {
        if (varlen) p.lse[(int64_t)h * (p.cu_q[p.B]) + tq0 + my_q] = -__builtin_inff();
        else p.lse[((int64_t)b * p.Hq + h) * p.Nq + my_q] = -__builtin_inff();
      }
    }
    return;
  }

  // ---- scalars: c = sigma * log2(e) * gq * gk
  // (MX Q/K: no tensor scales, the E8M0 block exponents are applied by the MFMA)
  const float cc = QK ? (float)((double)p.sigma * 1.4426950408889634)
                      : (float)((double)p.sigma * 1.4426950408889634 * (double)(*p.gq) * (double)(*p.gk));
  const float vscale = VF == VF_FP8 ? *p.sv : 1.0f;
  // exp-free cast: 2^M, and 2^M * b, of the code format (E2M1: M = 1, b = 1;
  // E4M3: M = 3, b = 7); ccl = 2^M c is exact
  constexpr float CAST_MUL = PF == PF_MXFP4 ? 2.0f : 8.0f;
  constexpr float CAST_BIAS = PF == PF_MXFP4 ? 2.0f : 56.0f;
  const float ccl = cc * CAST_MUL;

  // ---- Q operand (B of S^T): lane holds query ql, d in [hh*D/2, hh*D/2 + D/2),
  // decoded here from the NVFP4 codes (E2M1 * E4M3 is exact in FP16); once per
  // workgroup, so a separate expansion pass for Q is not needed
  f16x8 qf[QK ? 1 : KS];
  // MX Q/K: lane (ql, hh) holds the FP4 codes of d in 64 ks + 32 hh + [0, 32)
  // for each k-step, and the row's E8M0 bytes shifted so that byte 2 ks is
  // block (ks, hh) -- the B operand of the scaled MFMA and its scale_b
  u32x4 qm[QK ? KS : 1];
  uint32_t qsc = 0u;
  if constexpr (QK) {
    const bool live = wave_active && my_q < len_q;
    const int64_t row = live ? (tq0 + my_q) * p.Hq + h : 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qm[ks] = live ? *reinterpret_cast<const u32x4*>(p.q_codes + row * HALF + 32 * ks + 16 * hh) : u32x4{0u, 0u, 0u, 0u};
    uint32_t sw = 0u;
    if (live) sw = D == 128 ? *reinterpret_cast<const uint32_t*>(p.q_scales + row * 4)
                            : (uint32_t)*reinterpret_cast<const uint16_t*>(p.q_scales + row * 2);
    qsc = sw >> (8 * hh);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qm[ks]));
    asm volatile("" : "+v"(qsc));
  } else {
    const bool live = wave_active && my_q < len_q;
    const int64_t row = live ? (tq0 + my_q) * p.Hq + h : 0;
    const uint8_t* qc = p.q_codes + row * HALF + hh * (HALF / 2);
    const uint8_t* qs = p.q_scales + row * (D / 16) + hh * (HALF / 16);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t cw = live ? *reinterpret_cast<const uint32_t*>(qc + 4 * ks) : 0u;
      const float sv = e4m3_decode(live ? qs[ks >> 1] : 0u);
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[ks][j] = (_Float16)(e2m1_decode((cw >> (4 * j)) & 0xFu) * sv);
    }
    // make the Q loads complete here, so no vector-memory wait is left for the
    // pipeline below (it would also wait for the in-flight LDS copies)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[ks]));
  }

  // ---- LDS: K slots 0/1 then V slots 0/1 (codes + scales).  Iteration t reads
  // K(t) from K slot t%2 and V(t-2) from V slot t%2.
  const int64_t kcol0 = kcol_offset(varlen, b, tk0, p.nk_pad);
  // K tiles of this head in the workspace, L::K_BYTES each (kcols and kcol0
  // are multiples of the tile)
  const uint8_t* ksrc = reinterpret_cast<const uint8_t*>(p.khat) +
                        ((int64_t)hk * (p.kcols / KEY_TILE) + kcol0 / KEY_TILE) * L::K_BYTES;
  const uint32_t lds0 = lds_address(smem);
  // per-head bases (per-lane offsets below stay under 4 GiB)
  const uint8_t* vhead = p.v_codes + (VF == VF_MXFP4 ? (int64_t)hk * D * p.kcols / 2 : (int64_t)hk * D * p.kcols);
  const uint8_t* shead = VF == VF_MXFP4 ? p.v_scales + (int64_t)hk * D * (p.kcols / 32) : nullptr;
  constexpr int K_UNITS = L::KC_BYTES / 16;
  constexpr int V_UNITS = L::V_BYTES / 16;
  static_assert(QK || K_UNITS % 512 == 0, "K tile must split evenly over the workgroup");
  static_assert(!QK || K_UNITS % 256 == 0, "MX K codes must split over whole waves");
  // Copies are split into parts of one instruction per wave (1 KB of K or V,
  // or the V block exponents) so that the key loop can spread them over its
  // slots: a burst of copies at one point would fill the address queue and
  // stall the issuing waves' matrix work behind it.
  // (MX K: the codes, then one part for the 512 bytes of block exponents)
  constexpr int NK_DMA = QK ? (K_UNITS + 511) / 512 + 1 : K_UNITS / 512;
  constexpr int NV_DMA = (V_UNITS + 511) / 512 + (VF == VF_MXFP4 ? 1 : 0);
  // part i of K(src) -> K ring slot rs
  // (tile and part offsets go into the scalar base, so that the per-lane
  // offsets are loop invariant)
  auto copy_k_part = [&](int rs, int src, int i) {
    const uint32_t slot = lds0 + (uint32_t)(rs * L::K_BYTES);
    if (QK && i == NK_DMA - 1) {               // E8M0 dwords: two waves' worth, the others repeat them
      const int w = wave & 1;
      dma4(ksrc + (int64_t)src * L::K_BYTES + L::KC_BYTES + w * 256, (uint32_t)(lane * 4),
           slot + L::KC_BYTES + w * 256);
      return;
    }
    // (MX K at D=64: 256 units, so waves 4-7 repeat the copies of waves 0-3)
    const int u0 = QK ? (i * 512 + wave * 64) % K_UNITS : i * 512 + wave * 64;
    dma16(ksrc + (int64_t)src * L::K_BYTES + u0 * 16, (uint32_t)(lane * 16), slot + u0 * 16);
  };
  // part i of V(src) -> V ring slot rs
  auto copy_v_part = [&](int rs, int src, int i) {
    const uint32_t slot = lds0 + (uint32_t)(L::V_BASE + rs * L::V_SLOT);
    const int64_t col = kcol0 + (int64_t)src * KEY_TILE;
    // No branches here (these copies sit inside the key loop's slots): waves
    // beyond the ones a part needs copy the same bytes to the same place again.
    if (VF == VF_MXFP4 && i == NV_DMA - 1) {         // E8M0 exponents, one dword per d
      const int w = wave % (D / 64);
      const int d = w * 64 + lane;
      dma4(shead + col / 32, (uint32_t)(d * (p.kcols / 32)), slot + L::V_BYTES + w * 256);
      return;
    }
    const int u0 = (i * 512 + wave * 64) % V_UNITS;
    const int u = u0 + lane;
    int c, dt, kh, r, part = 0;
    if (VF == VF_MXFP4) { r = u & 31; kh = (u >> 5) & 1; dt = (u >> 6) % DT; c = (u >> 6) / DT; }
    else { r = u & 31; kh = (u >> 5) & 1; part = (u >> 6) & 1; dt = (u >> 7) % DT; c = (u >> 7) / DT; }
    const int d = 32 * dt + r;
    if (VF == VF_MXFP4)   // col and the per-lane key offset are even
      dma16(vhead + col / 2, (uint32_t)((d * p.kcols + 64 * c + 32 * kh) / 2), slot + u0 * 16);
    else
      dma16(vhead + col, (uint32_t)(d * p.kcols + 64 * c + 16 * kh + 32 * part), slot + u0 * 16);
  };
  auto copy_k = [&](int t) {                 // K(t) -> ring slot t (prologue, t < 3)
#pragma unroll
    for (int i = 0; i < NK_DMA; ++i) copy_k_part(t, t, i);
  };

  // ---- accumulators and per-wave state
  f32x16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float alpha_pend = 1.0f;
  bool rescale_any = false;
  f32x16 s[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) s[st] = f32x16{};
  i32x8 pw[2], pr[2];                  // probabilities being written / read by P.V
  int psw[2] = {127, 127}, psr[2] = {127, 127};
  float bm[2] = {0.f, 0.f};            // block maxima of S(t-1) (raw scores)
  float bmp[2] = {0.f, 0.f};           // S(t-1): max of sub-tiles 0,1 / of sub-tile 2 (set a tile ahead)
  float bmn[2] = {0.f, 0.f};           // the same for S(t), built during iteration t
  float me[2] = {0.f, 0.f};            // exact encode: m' + e per block
  float mb[2] = {0.f, 0.f};            // exp-free cast: 2^M (b - m' - e) per block
  uint32_t cev = 0, cod = 0;           // exp-free E2M1: even / odd key codes, one byte each
  pw[0] = pw[1] = pr[0] = pr[1] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};

  // constant 0/1 operand of the row-sum MFMA (16x16x128, FP4 1.0 = code 2)
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

  // ---- pipeline pieces --------------------------------------------------
  // S^T sub-tiles st0, st0+1 of K(t) Q^T (K in slot ks_)
  // MX Q/K: one scaled FP4 MFMA of S^T sub-tile st, k-step ks; ka holds the
  // lane's 32 K codes (A operand row ql, k-half hh), ksw the key row's E8M0
  // bytes shifted so that byte 2 ks is block (ks, hh)
  auto mx_mfma = [&](int st, int ks, const u32x4& ka, uint32_t ksw) {
    const i32x8 a = {(int)ka[0], (int)ka[1], (int)ka[2], (int)ka[3], 0, 0, 0, 0};
    const i32x8 bq = {(int)qm[ks][0], (int)qm[ks][1], (int)qm[ks][2], (int)qm[ks][3], 0, 0, 0, 0};
    if (ks == 0)
      s[st] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bq, f32x16{}, 4, 4, 0, (int)ksw, 0, (int)qsc);
    else
      s[st] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bq, s[st], 4, 4, 2, (int)ksw, 2, (int)qsc);
  };
  auto qk2 = [&](int kslot, int st0) {
    if constexpr (QK) {
      const uint8_t* kbm = smem + kslot * L::K_BYTES + lane * 16;
      const uint32_t* kw = reinterpret_cast<const uint32_t*>(smem + kslot * L::K_BYTES + L::KC_BYTES);
#pragma unroll
      for (int st = st0; st < st0 + 2; ++st) {
        const uint32_t ksw = kw[st * 32 + ql] >> (8 * hh);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          mx_mfma(st, ks, *reinterpret_cast<const u32x4*>(kbm + (st * KS + ks) * 64 * 16), ksw);
      }
      return;
    }
    const uint8_t* kb = smem + kslot * L::K_BYTES + (hh * KS * 32 + ql) * 16;
    f16x8 a0 = *reinterpret_cast<const f16x8*>(kb + (st0 * 2 * KS) * 32 * 16);
    f16x8 a1 = *reinterpret_cast<const f16x8*>(kb + ((st0 + 1) * 2 * KS) * 32 * 16);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      f16x8 n0, n1;
      if (ks + 1 < KS) {
        n0 = *reinterpret_cast<const f16x8*>(kb + (st0 * 2 * KS + ks + 1) * 32 * 16);
        n1 = *reinterpret_cast<const f16x8*>(kb + ((st0 + 1) * 2 * KS + ks + 1) * 32 * 16);
      }
      s[st0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, qf[ks], ks == 0 ? f32x16{} : s[st0], 0, 0, 0);
      s[st0 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, qf[ks], ks == 0 ? f32x16{} : s[st0 + 1], 0, 0, 0);
      if (ks + 1 < KS) { a0 = n0; a1 = n1; }
    }
  };
  // max of the 16 scores of S sub-tile st, as a shallow tree (short dependency
  // chains).  IEEE-2019 maximum (v_maximum3_f32): the scores hold no NaN, and
  // unlike fmax it needs no canonicalizing copies of the matrix results.
  auto tile_max = [&](int st) {
    const float a = fmax3(s[st][0], s[st][1], s[st][2]);
    const float b = fmax3(s[st][3], s[st][4], s[st][5]);
    const float c = fmax3(s[st][6], s[st][7], s[st][8]);
    const float d = fmax3(s[st][9], s[st][10], s[st][11]);
    const float e = fmax3(s[st][12], s[st][13], s[st][14]);
    return fmax3(fmax3(a, b, c), fmax3(d, e, s[st][15]), -__builtin_inff());
  };
  // masking of S (tail of the sequence, causal diagonal) for tile j
  auto mask = [&](int j) {
    const int key0 = j * KEY_TILE;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = key0 + s_key<PF>(st, v, hh);
        const bool dead = key >= len_k || (CAUSAL && key > my_q);
        if (dead) s[st][v] = -__builtin_inff();
      }
  };
  auto dump = [&](int j, const i32x8 (&pk)[2], const int (&psc)[2]) {
    if (DEBUG && b == p.dbg_b && h == p.dbg_h && my_q < len_q) {
      const int key0 = j * KEY_TILE;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int64_t row = (int64_t)my_q * p.dbg_ld;
        if (PF == PF_MXFP4) {
          const int key = key0 + 64 * c + 32 * hh;
          *reinterpret_cast<u32x4*>(p.dbg_codes + (row + key) / 2) =
              u32x4{(uint32_t)pk[c][0], (uint32_t)pk[c][1], (uint32_t)pk[c][2], (uint32_t)pk[c][3]};
          p.dbg_scales[(row + key) / 32] = (uint8_t)psc[c];
        } else {
          const int key = key0 + 64 * c + 16 * hh;
          *reinterpret_cast<u32x4*>(p.dbg_codes + row + key) =
              u32x4{(uint32_t)pk[c][0], (uint32_t)pk[c][1], (uint32_t)pk[c][2], (uint32_t)pk[c][3]};
          *reinterpret_cast<u32x4*>(p.dbg_codes + row + key + 32) =
              u32x4{(uint32_t)pk[c][4], (uint32_t)pk[c][5], (uint32_t)pk[c][6], (uint32_t)pk[c][7]};
        }
      }
    }
  };
  // ---- one iteration as NS slots ----------------------------------------
  // Slot i issues one matrix instruction -- P.V / row-sum of tile t-2 for
  // i < NPV, then S(t) = K(t) Q^T sub-tile by sub-tile -- and a fixed share of
  // the vector units of tile t-1, with a scheduling fence after each slot so
  // that matrix and vector work stay interleaved in the instruction stream
  // (one wave issues in order: a run of matrix instructions would otherwise
  // stall its vector work).  LDS operands are read two slots ahead.
  //   unit  3       : block maxima of S(t-1): sub-tile 3 joins the maxima of
  //                   sub-tiles 0..2, taken beside the previous iteration's
  //                   later slots (units 45..47, one phase after each sub-tile)
  //   unit  4       : row max, m', alpha, block exponents
  //   units [5, 37) : encode two scores (sub-tile (u-5)/8, registers 2k, 2k+1)
  //   units [37, 45): O / l rescale, one eighth each (run at the head of the
  //                   next iteration, and only when some row max of the wave moved)
  // Sub-tile st of S(t-1) is fully encoded before the slot that overwrites it.
  constexpr int NPV = 2 * (DT + 1);
  constexpr int NS = NPV + 4 * KS;
  u32x4 opa[3], opb[3];
  uint32_t vsc[DT];
  uint32_t ksc[4];                     // MX K: E8M0 words of K(t), one per S sub-tile
  auto load_op = [&](int i, const uint8_t* sV, const uint8_t* kb) {
    const int bs = i % 3;
    if (i < NPV) {
      const int c = i / (DT + 1), dt = i % (DT + 1);
      if (dt == DT) return;                      // row-sum: constant operand
      if (VF == VF_MXFP4) {
        opa[bs] = *reinterpret_cast<const u32x4*>(sV + ((((c * DT + dt) * 2 + hh) * 32 + ql) * 16));
      } else {
        opa[bs] = *reinterpret_cast<const u32x4*>(sV + ((((c * DT + dt) * 2 + 0) * 2 + hh) * 32 + ql) * 16);
        opb[bs] = *reinterpret_cast<const u32x4*>(sV + ((((c * DT + dt) * 2 + 1) * 2 + hh) * 32 + ql) * 16);
      }
    } else {
      const int q = i - NPV, st = q / KS, ks = q % KS;
      if (QK) opa[bs] = *reinterpret_cast<const u32x4*>(kb + (st * KS + ks) * 64 * 16);
      else opa[bs] = *reinterpret_cast<const u32x4*>(kb + (st * 2 * KS + ks) * 32 * 16);
    }
  };
  auto mfma_slot = [&](int i) {
    const int bs = i % 3;
    if (i < NPV) {
      const int c = i / (DT + 1), dt = i % (DT + 1);
      if (dt == DT) {
        lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pr[c], lacc, 4, PF == PF_MXFP4 ? 4 : 0, 0, 127,
                                                               0, psr[c]);
      } else if (VF == VF_MXFP4) {
        const i32x8 a = {(int)opa[bs][0], (int)opa[bs][1], (int)opa[bs][2], (int)opa[bs][3], 0, 0, 0, 0};
        // byte 2c of the lane's shifted scale word is its block (c, hh)
        if (c == 0)
          oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pr[c], oacc[dt], 4, PF == PF_MXFP4 ? 4 : 0,
                                                                     0, (int)vsc[dt], 0, psr[c]);
        else
          oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pr[c], oacc[dt], 4, PF == PF_MXFP4 ? 4 : 0,
                                                                     2, (int)vsc[dt], 0, psr[c]);
      } else {
        const i32x8 a = {(int)opa[bs][0], (int)opa[bs][1], (int)opa[bs][2], (int)opa[bs][3],
                         (int)opb[bs][0], (int)opb[bs][1], (int)opb[bs][2], (int)opb[bs][3]};
        oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pr[c], oacc[dt], 0, PF == PF_MXFP4 ? 4 : 0, 0,
                                                                   127, 0, psr[c]);
      }
    } else {
      const int q = i - NPV, st = q / KS, ks = q % KS;
      if constexpr (QK) {
        mx_mfma(st, ks, opa[bs], ksc[st]);
      } else {
        const f16x8 a = __builtin_bit_cast(f16x8, opa[bs]);
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[ks], ks == 0 ? f32x16{} : s[st], 0, 0, 0);
      }
    }
  };
  // Exact MXFP4-P encode at D=128 with NVFP4 Q/K, where slots 2 .. NPV + 3 KS - 1
  // carry one encode unit each: a unit's conversion to codes is issued one slot
  // after its exponentials (it would otherwise wait on the transcendental
  // unit's result within the slot); the probabilities wait in pend0 / pend1.
  // Measured 0.6 % faster on the Wan shape; with FP8 P it was 1.2 % slower, so
  // that path keeps the conversion in the slot.
  constexpr bool SKEW = !ENC && !QK && D == 128 && PF == PF_MXFP4;
  float pend0 = 0.0f, pend1 = 0.0f;
  auto encode_codes = [&](int u) {
    const int st = (u - 5) >> 3, k = (u - 5) & 7, c = st >> 1, s2 = st & 1;
    if (PF == PF_MXFP4) {
      const int word = 2 * s2 + (k >> 2), byte = k & 3;   // key 16*s2 + 2k of the lane's block
      uint32_t w = (uint32_t)pw[c][word];
      if (byte == 0) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, pend0, pend1, 1.0f, 0);
      else if (byte == 1) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, pend0, pend1, 1.0f, 1);
      else if (byte == 2) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, pend0, pend1, 1.0f, 2);
      else w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, pend0, pend1, 1.0f, 3);
      pw[c][word] = (int)w;
    } else {
      const int word = 4 * s2 + (k >> 1);
      if (k & 1) pw[c][word] = __builtin_amdgcn_cvt_pk_fp8_f32(pend0, pend1, pw[c][word], true);
      else pw[c][word] = __builtin_amdgcn_cvt_pk_fp8_f32(pend0, pend1, pw[c][word], false);
    }
  };
  static_assert(!SKEW || (slot_unit_begin<NPV, KS>(2) == 5 && slot_unit_begin<NPV, KS>(NPV + 3 * KS) == 37 &&
                          NPV + 3 * KS - 2 == 32),
                "one encode unit per slot in slots 2 .. NPV + 3 KS - 1");
  auto vunit = [&](int u) {
    if (u < 4) {                                 // block maxima of S(t-1): sub-tile 3 joins the
      if (u == 3) {                              // maxima of sub-tiles 0..2 taken a tile earlier
        bm[0] = bmp[0];
        bm[1] = fmax2(bmp[1], tile_max(3));
      }
    } else if (u == 4) {                         // row statistics
      float rmax = fmax2(bm[0], bm[1]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rmax), __float_as_uint(rmax), false, false);
      rmax = fmax2(__uint_as_float(sw[0]), __uint_as_float(sw[1]));   // max with lane ^ 32
      const float tmax = rmax * cc;              // max of fl(S*c) (c > 0)
      // Every row sees a live key in its first tile (the key-less case exits
      // before the loop; causal rows always see key 0), so m' is finite from
      // the first tile on, and alpha = 2^(m - m') is 0 there (m = -inf).
      const float m_new = fmax2(m_run, tmax);
      alpha_pend = __builtin_amdgcn_exp2f(m_run - m_new);
      // alpha is exactly 1 wherever the running max did not move; the rescale
      // is skipped when that holds for the whole wave
      rescale_any = __builtin_amdgcn_ballot_w64(alpha_pend != 1.0f) != 0;
      m_run = m_new;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (PF == PF_MXFP4) {
          const float xmax = bm[c] * cc - m_new;   // fl(fl(S*c) - m'), no contraction
          // e = max(floor(xmax) - 2, -127); a block without a live key has
          // xmax = -inf and gets -127
          const float ef = fmax2(__builtin_floorf(xmax), -125.0f) - 2.0f;
          psw[c] = (int)ef + 127;
          me[c] = m_new + ef;
        } else {
          psw[c] = 127;
          me[c] = m_new;
        }
        if (ENC) mb[c] = CAST_BIAS - CAST_MUL * me[c];   // 2^M me is exact
      }
    } else if (u < 37 && ENC) {                  // exp-free cast of scores 2k, 2k+1 of sub-tile st
      const int st = (u - 5) >> 3, k = (u - 5) & 7, c = st >> 1, s2 = st & 1, v = 2 * k;
      const float y0 = __builtin_fmaf(s[st][v], ccl, mb[c]);       // -inf on masked keys -> code 0
      const float y1 = __builtin_fmaf(s[st][v + 1], ccl, mb[c]);
      if (PF == PF_MXFP4) {
        // E2M1 codes of keys 16*s2 + v, v+1 go to the low / high nibble of
        // byte k&3 of word 2*s2 + k/4; even and odd keys are gathered one
        // byte each, then merged once per word
        const float a0 = __builtin_fminf(y0, 7.0f), a1 = __builtin_fminf(y1, 7.0f);
        const int byte = k & 3;
        if (byte == 0) { cev = __builtin_amdgcn_cvt_pk_u8_f32(a0, 0, cev); cod = __builtin_amdgcn_cvt_pk_u8_f32(a1, 0, cod); }
        else if (byte == 1) { cev = __builtin_amdgcn_cvt_pk_u8_f32(a0, 1, cev); cod = __builtin_amdgcn_cvt_pk_u8_f32(a1, 1, cod); }
        else if (byte == 2) { cev = __builtin_amdgcn_cvt_pk_u8_f32(a0, 2, cev); cod = __builtin_amdgcn_cvt_pk_u8_f32(a1, 2, cod); }
        else {
          cev = __builtin_amdgcn_cvt_pk_u8_f32(a0, 3, cev);
          cod = __builtin_amdgcn_cvt_pk_u8_f32(a1, 3, cod);
          pw[c][2 * s2 + (k >> 2)] = (int)((cod << 4) | cev);
        }
      } else {
        // E4M3 codes (at most 56 here: y <= 56 up to rounding) of keys v, v+1
        // go to bytes 2(k&1), 2(k&1)+1 of word 4*s2 + k/2
        const int word = 4 * s2 + (k >> 1);
        uint32_t w = (uint32_t)pw[c][word];
        if (k & 1) { w = __builtin_amdgcn_cvt_pk_u8_f32(y0, 2, w); w = __builtin_amdgcn_cvt_pk_u8_f32(y1, 3, w); }
        else { w = __builtin_amdgcn_cvt_pk_u8_f32(y0, 0, w); w = __builtin_amdgcn_cvt_pk_u8_f32(y1, 1, w); }
        pw[c][word] = (int)w;
      }
    } else if (u < 37 && SKEW) {                 // scores 2k, 2k+1 of sub-tile st -> pending probabilities
      const int st = (u - 5) >> 3, k = (u - 5) & 7, c = st >> 1, v = 2 * k;
      pend0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][v], cc, -me[c]));
      pend1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][v + 1], cc, -me[c]));
    } else if (u < 37) {                         // encode scores 2k, 2k+1 of sub-tile st
      const int st = (u - 5) >> 3, k = (u - 5) & 7, c = st >> 1, s2 = st & 1, v = 2 * k;
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][v], cc, -me[c]));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][v + 1], cc, -me[c]));
      if (PF == PF_MXFP4) {
        const int word = 2 * s2 + (k >> 2), byte = k & 3;   // key 16*s2 + v of the lane's block
        uint32_t w = (uint32_t)pw[c][word];
        if (byte == 0) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p0, p1, 1.0f, 0);
        else if (byte == 1) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p0, p1, 1.0f, 1);
        else if (byte == 2) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p0, p1, 1.0f, 2);
        else w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p0, p1, 1.0f, 3);
        pw[c][word] = (int)w;
      } else {
        const int word = 4 * s2 + (k >> 1);
        if (k & 1) pw[c][word] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pw[c][word], true);
        else pw[c][word] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pw[c][word], false);
      }
    } else if (u >= 45) {                        // maxima of S(t) sub-tiles 0..2 for the next tile
      if (u == 45) bmn[0] = tile_max(0);
      else if (u == 46) bmn[0] = fmax2(bmn[0], tile_max(1));
      else bmn[1] = tile_max(2);
    } else {                                     // rescale slice
      const int r = u - 37;
#pragma unroll
      for (int e = r * 2 * DT; e < (r + 1) * 2 * DT; ++e) oacc[e >> 4][e & 15] *= alpha_pend;
      if (r == 7) lacc[0] *= alpha_pend;
    }
  };

  // ---- the key loop.  Prologue: K(0) and S(0).  Iteration t = 1..n+1 runs
  // P.V of tile t-2, the softmax/encode of tile t-1 and Q.K^T of tile t.
  // Out-of-range pieces run on harmless data instead of branching: P of the
  // tile before 0 is all-zero codes against a zeroed V slot, and the tile
  // after the last is masked completely (all its probabilities are 0), so the
  // steady body has no branches between its matrix and vector work.
  //
  // K and V tiles sit in rings of three LDS slots (tile x in slot x mod 3).
  // Iteration t copies K(t+1) and V(t-1) in its first NS/2 slots; every wave
  // waits for its own copies and then joins one workgroup barrier per
  // iteration.  Waves 0-3 take it after their last slot, waves 4-7 after
  // slot G1B: the two waves of a SIMD (one of each group) then run G1B slots
  // apart instead of in step, so the vector-heavy first slots of one meet
  // the matrix-only last slots of the other.  With three slots a tile is
  // overwritten only two barriers after the last iteration that reads it,
  // which covers the lag of the second group.
  constexpr int G1B = ATTN_G1_BARRIER;
  static_assert(G1B >= NS / 2, "the second group's barrier must follow its copies");
  const int group = wave >> 2;
  {
    // zero the V slots once (P(-1) = 0 meets V(-1) = slot 2 in iteration 1)
    for (int i = tid; i < L::RING * L::V_SLOT / 16; i += 512)
      *reinterpret_cast<u32x4*>(smem + L::V_BASE + i * 16) = u32x4{0u, 0u, 0u, 0u};
  }
  copy_k(0);
  dma_wait();
  __syncthreads();
  if (n_tiles > 1) copy_k(1);
  qk2(0, 0);
  qk2(0, 2);
  bmp[0] = fmax2(tile_max(0), tile_max(1));
  bmp[1] = tile_max(2);
  dma_wait();
  phase_barrier();
#ifdef ATTN_FWD_PHASE_TRACE
  unsigned long long tacc[5] = {0, 0, 0, 0, 0}, tstamp[5];
  unsigned long long tprev = __builtin_amdgcn_s_memtime();
#endif
  int rk = 1;                                  // ring slot of K(t) = t mod 3
  for (int t = 1; t <= n_tiles + 1; ++t) {
    const int rk1 = rk == 2 ? 0 : rk + 1, rk2 = rk1 == 2 ? 0 : rk1 + 1;   // (t+1), (t+2) = (t-1) mod 3
    // sources of the copies of this iteration, K(t+1) and V(t-1); past the
    // last tile the last tile is copied again (into a slot whose contents
    // only meet all-zero probabilities), which keeps the loop free of branches
    const int last = n_tiles > 0 ? n_tiles - 1 : 0;
    const int src_k = min(t + 1, last), src_v = min(t - 1, last);
    // O / l rescale by alpha(t-2), set while S(t-2) was encoded in the
    // previous iteration: after P(t-3).V, before P(t-2).V.  Only waves where
    // some row max moved do it (alpha is exactly 1 elsewhere); as a branch
    // inside the slots it would split them, so it runs before them.
    if (rescale_any) {
#pragma unroll
      for (int u = 37; u < 45; ++u) vunit(u);
    }
    const int j = t - 1;                       // tile being encoded
    if (j * KEY_TILE + KEY_TILE > len_k || (CAUSAL && j * KEY_TILE + KEY_TILE - 1 > q0)) {
      mask(j);
      bmp[0] = fmax2(tile_max(0), tile_max(1));   // maxima taken before the mask
      bmp[1] = tile_max(2);
    }
    const uint8_t* sV = smem + L::V_BASE + rk1 * L::V_SLOT;                   // V(t-2): (t-2) mod 3 = (t+1) mod 3
    const uint8_t* kb = smem + rk * L::K_BYTES + (QK ? lane : hh * KS * 32 + ql) * 16;   // K(t)
    if constexpr (QK) {
      const uint32_t* kw = reinterpret_cast<const uint32_t*>(smem + rk * L::K_BYTES + L::KC_BYTES);
#pragma unroll
      for (int st = 0; st < 4; ++st) ksc[st] = kw[st * 32 + ql] >> (8 * hh);
    }
    if (VF == VF_MXFP4) {
      const uint32_t* sVS = reinterpret_cast<const uint32_t*>(sV + L::V_BYTES);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vsc[dt] = sVS[32 * dt + ql] >> (8 * hh);   // blocks (c, hh) at bytes 2c
    }
    load_op(0, sV, kb);
    load_op(1, sV, kb);
#if ATTN_PRIO_MODE == 1 || ATTN_PRIO_MODE == 2
    setprio_if<2>(group);
#endif
    __builtin_amdgcn_sched_barrier(0);
    FWD_PHASE_STAMP(0);
#pragma clang loop unroll(full)
    for (int i = 0; i < NS; ++i) {
      // copies for the next iterations, K(t+1) and V(t-1), spread over the
      // first half of the slots
#pragma unroll
      for (int q = 0; q < NK_DMA + NV_DMA; ++q)
        if (i == (q * (NS / 2)) / (NK_DMA + NV_DMA)) {
          if (q < NK_DMA) copy_k_part(rk1, src_k, q);
          else copy_v_part(rk2, src_v, q - NK_DMA);
        }
      if (i + 2 < NS) load_op(i + 2, sV, kb);
      mfma_slot(i);
      if (SKEW && i >= 3 && i <= NPV + 3 * KS) encode_codes(slot_unit_begin<NPV, KS>(i - 1));
#pragma unroll
      for (int u = slot_unit_begin<NPV, KS>(i); u < slot_unit_begin<NPV, KS>(i + 1); ++u)
        if (u < 37) vunit(u);
      if (i == NPV + 2 * KS - 1) vunit(45);      // S(t) sub-tile 0, finished one phase ago
      if (i == NPV + 3 * KS - 1) vunit(46);      // sub-tile 1
      if (i == NS - 1) vunit(47);                // sub-tile 2
      __builtin_amdgcn_sched_barrier(0);
#if ATTN_PRIO_MODE == 1
      if (i == ATTN_PRIO_END) setprio_if<0>(group);
#endif
      if (i == G1B - 1 && G1B < NS) dma_wait_barrier_if(group);
      if (i == NPV - 1) FWD_PHASE_STAMP(1);
      if (i == NPV + 2 * KS - 1) FWD_PHASE_STAMP(2);
      if (i == NS - 1) FWD_PHASE_STAMP(3);
    }

    if (j < n_tiles) dump(j, pw, psw);
    pr[0] = pw[0]; pr[1] = pw[1]; psr[0] = psw[0]; psr[1] = psw[1];
    bmp[0] = bmn[0]; bmp[1] = bmn[1];
    dma_wait_barrier_if(G1B >= NS ? 1 : group ^ 1);
#ifdef ATTN_FWD_PHASE_TRACE
    FWD_PHASE_STAMP(4);
    tacc[0] += tstamp[0] - tprev;
#pragma unroll
    for (int k = 1; k < 5; ++k) tacc[k] += tstamp[k] - tstamp[k - 1];
    tprev = tstamp[4];
#endif
    rk = rk1;
  }
#ifdef ATTN_FWD_PHASE_TRACE
  if (blockIdx.x == 0 && lane < 6) {
    unsigned long long v = (unsigned long long)n_tiles;
#pragma unroll
    for (int k = 0; k < 5; ++k) v = lane == k ? tacc[k] : v;
    g_fwd_phase_trace[wave][lane] = v;
  }
#endif

  // ---- epilogue: O = o / l (x FP8 V tensor scale), LSE = ln2 * (m + log2 l)
  if (!wave_active || my_q >= len_q) return;
  const float l = lacc[0];
  const bool empty = !(l > 0.0f);
  const float inv = empty ? 0.0f : vscale / l;
  const int64_t orow = ((tq0 + my_q) * p.Hq + h) * (int64_t)D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * dt + 8 * j + 4 * hh;
      f32x4 v = {oacc[dt][4 * j] * inv, oacc[dt][4 * j + 1] * inv, oacc[dt][4 * j + 2] * inv, oacc[dt][4 * j + 3] * inv};
      if (p.o_f32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + orow + d) = v;
      } else {
        uint32_t u[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t x = __float_as_uint(v[k]);
          u[k] = (x + 0x7FFFu + ((x >> 16) & 1u)) >> 16;   // round to nearest even
        }
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.o) + orow + d) = u32x2{u[0] | (u[1] << 16), u[2] | (u[3] << 16)};
      }
    }
  if (p.lse != nullptr && hh == 0) {
    const float lse = empty ? -__builtin_inff() : 0.6931471805599453f * (m_run + __builtin_log2f(l));
    if (varlen) p.lse[(int64_t)h * (p.cu_q[p.B]) + tq0 + my_q] = lse;
    else p.lse[((int64_t)b * p.Hq + h) * p.Nq + my_q] = lse;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_expand_k(const uint8_t* codes, const uint8_t* scales, int H, int B, int N, int max_len,
                           const int32_t* cu, int64_t n_pad, int64_t cols, int D, int pf, _Float16* out,
                           hipStream_t st) {
  dim3 grid((unsigned)((max_len + KEY_TILE - 1) / KEY_TILE), (unsigned)H, (unsigned)B);
  if (grid.x == 0 || B == 0) return hipSuccess;
#define EX(DD, P) \
  hipLaunchKernelGGL((expand_k_kernel<DD, P>), grid, dim3(256), 0, st, codes, scales, H, N, cu, n_pad, cols, out)
  if (pf == PF_MXFP4) {
    if (D == 64) EX(64, 0); else EX(128, 0);
  } else {
    if (D == 64) EX(64, 1); else EX(128, 1);
  }
#undef EX
  return hipGetLastError();
}

// Workgroups of a forward launch (packed batches: padded to whole query-block
// groups, see the kernel's workgroup order).
static int fwd_grid(const FwdParams& p) {
  const int qb = p.cu_q != nullptr ? (p.QB + VARLEN_QGROUP - 1) / VARLEN_QGROUP * VARLEN_QGROUP : p.QB;
  return p.B * p.Hq * qb;
}

template <int D, int PF, int VF, bool CAUSAL, bool DEBUG, int ENC, int QK = 0>
static hipError_t launch_fwd_t(const FwdParams& p, int nwg, hipStream_t st) {
  auto kern = fwd_lowp_kernel<D, PF, VF, CAUSAL, DEBUG, ENC, QK>;
  const int lds = LdsLayout<D, VF, QK>::TOTAL;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(512), lds, st, p);
  return hipGetLastError();
}

template <int D, int PF, int VF, bool CAUSAL, int ENC>
static hipError_t launch_fwd_d(const FwdParams& p, int nwg, bool debug, hipStream_t st) {
  return debug ? launch_fwd_t<D, PF, VF, CAUSAL, true, ENC>(p, nwg, st)
               : launch_fwd_t<D, PF, VF, CAUSAL, false, ENC>(p, nwg, st);
}

template <int ENC>
static hipError_t launch_fwd_e(const FwdParams& p, int nwg, int D, int pf, int vf, bool causal, bool debug,
                               hipStream_t st) {
  if (pf == PF_MXFP4) {
    if (vf == VF_MXFP4)
      return D == 64 ? launch_fwd_d<64, 0, 1, false, ENC>(p, nwg, debug, st)
                     : launch_fwd_d<128, 0, 1, false, ENC>(p, nwg, debug, st);
    return D == 64 ? launch_fwd_d<64, 0, 0, false, ENC>(p, nwg, debug, st)
                   : launch_fwd_d<128, 0, 0, false, ENC>(p, nwg, debug, st);
  }
  if (causal)
    return D == 64 ? launch_fwd_d<64, 1, 0, true, ENC>(p, nwg, debug, st)
                   : launch_fwd_d<128, 1, 0, true, ENC>(p, nwg, debug, st);
  return D == 64 ? launch_fwd_d<64, 1, 0, false, ENC>(p, nwg, debug, st)
                 : launch_fwd_d<128, 1, 0, false, ENC>(p, nwg, debug, st);
}

hipError_t launch_fwd_lowp(const FwdParams& p, int D, int pf, int vf, bool causal, bool debug, int enc,
                           hipStream_t st) {
  const int nwg = fwd_grid(p);
  if (nwg == 0) return hipSuccess;
  return enc ? launch_fwd_e<1>(p, nwg, D, pf, vf, causal, debug, st)
             : launch_fwd_e<0>(p, nwg, D, pf, vf, causal, debug, st);
}

// MX Q/K mode: Direct-P (MXFP4 P; V FP8 or MXFP4; noncausal) or FP8-P/V
// (causal or not), each with the exact encode or (enc = 1) the exp-free cast.
// The K tiles follow the P format's key order.
hipError_t launch_pack_k_mx(const uint8_t* codes, const uint8_t* scales, int H, int B, int N, int max_len,
                            const int32_t* cu, int64_t n_pad, int64_t cols, int D, int pf, uint8_t* out,
                            hipStream_t st) {
  dim3 grid((unsigned)((max_len + KEY_TILE - 1) / KEY_TILE), (unsigned)H, (unsigned)B);
  if (grid.x == 0 || B == 0) return hipSuccess;
#define PK(DD, P) \
  hipLaunchKernelGGL((pack_k_mx_kernel<DD, P>), grid, dim3(256), 0, st, codes, scales, H, N, cu, n_pad, cols, out)
  if (pf == PF_MXFP4) {
    if (D == 64) PK(64, PF_MXFP4); else PK(128, PF_MXFP4);
  } else {
    if (D == 64) PK(64, PF_FP8); else PK(128, PF_FP8);
  }
#undef PK
  return hipGetLastError();
}

hipError_t launch_fwd_mx(const FwdParams& p, int D, int pf, int vf, bool causal, bool debug, int enc,
                         hipStream_t st) {
  const int nwg = fwd_grid(p);
  if (nwg == 0) return hipSuccess;
#define MXL(DD, PP, VV, CC)                                                     \
  (debug ? launch_fwd_t<DD, PP, VV, CC, true, 0, 1>(p, nwg, st)                  \
         : launch_fwd_t<DD, PP, VV, CC, false, 0, 1>(p, nwg, st))
#define MXE(DD, PP, VV, CC)                                                     \
  (debug ? launch_fwd_t<DD, PP, VV, CC, true, 1, 1>(p, nwg, st)                  \
         : launch_fwd_t<DD, PP, VV, CC, false, 1, 1>(p, nwg, st))
  if (enc) {
    if (pf == PF_FP8) {
      if (causal) return D == 64 ? MXE(64, PF_FP8, VF_FP8, true) : MXE(128, PF_FP8, VF_FP8, true);
      return D == 64 ? MXE(64, PF_FP8, VF_FP8, false) : MXE(128, PF_FP8, VF_FP8, false);
    }
    if (causal) return hipErrorInvalidValue;
    if (vf == VF_MXFP4) return D == 64 ? MXE(64, PF_MXFP4, VF_MXFP4, false) : MXE(128, PF_MXFP4, VF_MXFP4, false);
    return D == 64 ? MXE(64, PF_MXFP4, VF_FP8, false) : MXE(128, PF_MXFP4, VF_FP8, false);
  }
#undef MXE
  if (pf == PF_FP8) {
    if (causal) return D == 64 ? MXL(64, PF_FP8, VF_FP8, true) : MXL(128, PF_FP8, VF_FP8, true);
    return D == 64 ? MXL(64, PF_FP8, VF_FP8, false) : MXL(128, PF_FP8, VF_FP8, false);
  }
  if (vf == VF_MXFP4) return D == 64 ? MXL(64, PF_MXFP4, VF_MXFP4, false) : MXL(128, PF_MXFP4, VF_MXFP4, false);
  return D == 64 ? MXL(64, PF_MXFP4, VF_FP8, false) : MXL(128, PF_MXFP4, VF_FP8, false);
#undef MXL
}

}  // namespace attn
