// Kernel parameter block of the attention backward (shared by the host
// launcher and the kernels).  All operand layouts are head-major and padded
// to NPAD = roundup(N, 128) rows, written by the backward's preparation
// kernels into the caller's workspace.
#pragma once
#include <stdint.h>

namespace attn {

struct BwdParams {
  const __bf16* qrm;      // [B][Hq][NPAD][D]   exact NVFP4 Q values without tensor scale (bf16)
  const __bf16* krm;      // [B][Hkv][NPAD][D]
  const uint8_t* vrm;     // [B][Hkv][NPAD][D]  FP8 E4M3 V codes, key-major
  const uint8_t* dorm;    // [B][Hq][NPAD][D]   E5M2 dO codes
  const float* lv;        // [B][Hq][NPAD]      LSE * log2 e (+inf on padded rows)
  const float* dv;        // [B][Hq][NPAD]      D = sum_d dO^ O
  const float* gq;        // device scalars: tensor scales of Q, K, V and dO
  const float* gk;
  const float* sv;
  const float* sdo;
  float* dq_out;          // [B][N][Hq][D]
  float* dk_out;          // [B][N][Hkv][D]
  float* dv_out;          // [B][N][Hkv][D]
  int B, Hq, Hkv, N;
  int64_t npad;
  float sigma;
  // optional dump of the E4M3 operands of one (batch dbg_b, query head dbg_h):
  // codes [NPAD][NPAD] (query row, key column); exponents (E8M0 bytes) of P~
  // and dS~K per (32-query block, key) [NPAD/32][NPAD], of dS~Q per (query,
  // 32-key block) [NPAD][NPAD/32]
  uint8_t* dbg_pt;
  uint8_t* dbg_pt_e;
  uint8_t* dbg_dsk;
  uint8_t* dbg_dsk_e;
  uint8_t* dbg_dsq;
  uint8_t* dbg_dsq_e;
  int dbg_b, dbg_h;
};

}  // namespace attn
