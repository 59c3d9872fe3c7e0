// Kernel parameter block of the decode-shaped forward (shared by the host
// launcher and the kernel).
#pragma once
#include <stdint.h>

namespace attn {

struct DecParams {
  const uint8_t* q_codes;   // NVFP4 Q: E2M1 codes [B][nq][Hq][D/2], E4M3 scales [B][nq][Hq][D/16]
  const uint8_t* q_scales;
  const uint8_t* k_codes;   // NVFP4 K cache, head-major: [B][Hkv][Nk][D/2], scales [B][Hkv][Nk][D/16]
  const uint8_t* k_scales;
  const uint8_t* v_codes;   // V cache: [B][Hkv][Nk/128] blocks of D key-contiguous rows (FP8 128 bytes,
  const uint8_t* v_scales;  // MXFP4 64 bytes per row; MXFP4 scales [B][Hkv][Nk/128][D][4])
  const float* gq;
  const float* gk;
  const float* sv;
  const int32_t* seqlens;   // [B] valid cache lengths (clamped to [0, Nk] in the kernel), or null = Nk
  void* o;                  // [B][nq][Hq][D]
  int o_f32;
  float* lse;               // [B][Hq][nq] or null
  int B, Hq, Hkv, nq, Nk, QG;
  int64_t nk_pad;
  float sigma;
  uint8_t* dbg_codes;       // probability dump of (dbg_b, dbg_h): [nq][dbg_ld] codes, [nq][dbg_ld/32] E8M0
  uint8_t* dbg_scales;
  int dbg_b, dbg_h;
  int64_t dbg_ld;
};

}  // namespace attn
