// Kernel parameter block of the low-precision forward (shared by the host
// launcher and the kernels).
#pragma once
#include <stdint.h>

namespace attn {

enum { PF_MXFP4 = 0, PF_FP8 = 1 };
enum { VF_FP8 = 0, VF_MXFP4 = 1 };

struct FwdParams {
  const uint8_t* q_codes;              // NVFP4 Q: E2M1 codes [rows][D/2], E4M3 scales [rows][D/16]
  const uint8_t* q_scales;
  const _Float16* khat;                // exact FP16 expansion of K in operand tiles
  int64_t kcols;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  const float* gq;
  const float* gk;
  const float* sv;
  void* o;
  int o_f32;
  float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int B, Hq, Hkv, Nq, Nk, QB;
  int64_t nk_pad;
  float sigma;
  uint8_t* dbg_codes;
  uint8_t* dbg_scales;
  int dbg_b, dbg_h;
  int64_t dbg_ld;
};

}  // namespace attn
