// C ABI of the Direct-P FP4 attention library (declared in include/attn_fp4.h).
// Host-side argument validation and launch sequencing only; every step of the
// computation runs in the HIP kernels of quant.hip, fwd_lowp.hip, fwd_bf16.hip,
// decode.hip and bwd.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/attn_fp4.h"
#include "common.h"

namespace attn {
hipError_t launch_amax(const void* x, int64_t n, float* partials, int* np_out, hipStream_t st);
hipError_t launch_quant_nvfp4(const void* x, int64_t rows, int D, const float* partials, int np, uint8_t* codes,
                              uint8_t* scales, float* tensor_scale, bool four_six, hipStream_t st);
hipError_t launch_quant_v(const void* v, int B, int Nk, int Hkv, int D, const int32_t* cu_k, int max_len, int64_t cols,
                          int fmt, const float* partials, int np, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                          bool cache_layout, hipStream_t st);
hipError_t launch_expand_k(const uint8_t* codes, const uint8_t* scales, int H, int B, int N, int max_len,
                           const int32_t* cu, int64_t n_pad, int64_t cols, int D, int pf, _Float16* out,
                           hipStream_t st);
hipError_t launch_quant_mxfp4(const void* x, int64_t rows, int D, uint8_t* codes, uint8_t* scales, bool hadamard,
                              hipStream_t st);
hipError_t launch_pack_k_mx(const uint8_t* codes, const uint8_t* scales, int H, int B, int N, int max_len,
                            const int32_t* cu, int64_t n_pad, int64_t cols, int D, int pf, uint8_t* out,
                            hipStream_t st);
struct FwdParams;
hipError_t launch_fwd_mx(const FwdParams& p, int D, int pf, int vf, bool causal, bool debug, int enc,
                         hipStream_t st);
hipError_t launch_fwd_lowp(const FwdParams& p, int D, int pf, int vf, bool causal, bool debug, int enc,
                           hipStream_t st);
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                           int Nq, int Nk, int D, float sigma, bool causal, hipStream_t st);
hipError_t launch_bwd_prep(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                           const uint8_t* k_scales, const uint8_t* v_codes, int64_t v_cols, const void* dout,
                           const void* o, const float* lse, const float* partials, int np, int B, int Hq, int Hkv,
                           int N, int D, int64_t npad, __bf16* qrm, __bf16* krm,
                           uint8_t* vrm, uint8_t* drm, float* dvec, float* lvec, float* sdo,
                           hipStream_t st);
struct BwdParams;
hipError_t launch_bwd_main(const BwdParams& p, int D, bool causal, bool debug, hipStream_t st);
struct DecParams;
hipError_t launch_decode(const DecParams& p, int D, int pf, int vf, bool causal, bool debug, hipStream_t st);
hipError_t launch_probe_kind(int kind, long long* cycles, int64_t* units, int* grid, hipStream_t st);
int probe_kind_count();
}  // namespace attn

#include "fwd_params.h"
#include "bwd_params.h"
#include "dec_params.h"

using namespace attn;

static thread_local int g_last_hip_error = 0;
static const size_t QUANT_WS = 8192;   // >= 2048 partial maxima

static attn_status hip_status(hipError_t e) {
  if (e == hipSuccess) return ATTN_OK;
  g_last_hip_error = (int)e;
  return ATTN_ERR_HIP;
}
static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

extern "C" {

const char* attn_status_str(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int attn_last_hip_error(void) { return g_last_hip_error; }
const char* attn_version(void) { return "attn_fp4 0.1 gfx950"; }
size_t attn_quant_ws_bytes(void) { return QUANT_WS; }

static attn_status run_quant_nvfp4(const void* x_bf16, int64_t rows, int32_t D, uint8_t* codes, uint8_t* scales,
                                   float* tensor_scale, void* ws, size_t ws_bytes, void* stream, bool four_six) {
  if (rows < 0 || D <= 0 || D % 16 != 0 || tensor_scale == nullptr || !aligned(tensor_scale, 4))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (rows > 0 && (x_bf16 == nullptr || codes == nullptr || scales == nullptr || !aligned(x_bf16, 16) ||
                   !aligned(codes, 8)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (ws == nullptr || ws_bytes < QUANT_WS || !aligned(ws, 16)) return ATTN_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  int np = 0;
  float* partials = (float*)ws;
  hipError_t e = launch_amax(x_bf16, rows * (int64_t)D, partials, &np, st);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_quant_nvfp4(x_bf16, rows, D, partials, np, codes, scales, tensor_scale, four_six, st));
}

attn_status attn_quant_nvfp4(const void* x_bf16, int64_t rows, int32_t D, uint8_t* codes, uint8_t* scales,
                             float* tensor_scale, void* ws, size_t ws_bytes, void* stream) {
  return run_quant_nvfp4(x_bf16, rows, D, codes, scales, tensor_scale, ws, ws_bytes, stream, false);
}

attn_status attn_quant_nvfp4_46(const void* x_bf16, int64_t rows, int32_t D, uint8_t* codes, uint8_t* scales,
                                float* tensor_scale, void* ws, size_t ws_bytes, void* stream) {
  return run_quant_nvfp4(x_bf16, rows, D, codes, scales, tensor_scale, ws, ws_bytes, stream, true);
}

static attn_status run_quant_mxfp4(const void* x_bf16, int64_t rows, int32_t D, uint8_t* codes, uint8_t* scales,
                                   bool hadamard, void* stream) {
  if (rows < 0 || D <= 0 || D % 32 != 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (rows > 0 && (x_bf16 == nullptr || codes == nullptr || scales == nullptr || !aligned(x_bf16, 16) ||
                   !aligned(codes, 16)))
    return ATTN_ERR_INVALID_ARGUMENT;
  return hip_status(launch_quant_mxfp4(x_bf16, rows, D, codes, scales, hadamard, (hipStream_t)stream));
}

attn_status attn_quant_mxfp4(const void* x_bf16, int64_t rows, int32_t D, uint8_t* codes, uint8_t* scales,
                             void* stream) {
  return run_quant_mxfp4(x_bf16, rows, D, codes, scales, false, stream);
}

attn_status attn_quant_mxfp4_had(const void* x_bf16, int64_t rows, int32_t D, uint8_t* codes, uint8_t* scales,
                                 void* stream) {
  return run_quant_mxfp4(x_bf16, rows, D, codes, scales, true, stream);
}

int64_t attn_v_cols(int32_t B, int32_t Nk, int64_t total_k, int32_t varlen) {
  if (B < 0 || Nk < 0 || total_k < 0) return -1;
  if (varlen) return 128 * ((total_k + 127) / 128 + B);
  return (int64_t)B * roundup(Nk, 128);
}

attn_status attn_quant_v(const void* v_bf16, int32_t B, int32_t Nk, int32_t Hkv, int32_t D,
                         const int32_t* cu_seqlens_k, int64_t total_k, int32_t format, uint8_t* codes,
                         uint8_t* scales, float* tensor_scale, void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || Nk < 0 || Hkv <= 0 || (D != 64 && D != 128)) return ATTN_ERR_INVALID_ARGUMENT;
  if (format != ATTN_V_FP8_E4M3 && format != ATTN_V_MXFP4) return ATTN_ERR_INVALID_ARGUMENT;
  const bool varlen = cu_seqlens_k != nullptr;
  if (varlen && total_k < 0) return ATTN_ERR_INVALID_ARGUMENT;
  const int64_t tokens = varlen ? total_k : (int64_t)B * Nk;
  if (format == ATTN_V_FP8_E4M3 && (tensor_scale == nullptr || !aligned(tensor_scale, 4)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (tokens > 0 && (v_bf16 == nullptr || codes == nullptr || !aligned(v_bf16, 16) || !aligned(codes, 16)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (tokens > 0 && format == ATTN_V_MXFP4 && (scales == nullptr || !aligned(scales, 4)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (ws == nullptr || ws_bytes < QUANT_WS || !aligned(ws, 16)) return ATTN_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int64_t cols = attn_v_cols(B, Nk, total_k, varlen);
  float* partials = (float*)ws;
  int np = 0;
  hipError_t e;
  if (format == ATTN_V_FP8_E4M3) {
    e = launch_amax(v_bf16, tokens * Hkv * (int64_t)D, partials, &np, st);
    if (e != hipSuccess) return hip_status(e);
  }
  if (B == 0) return ATTN_OK;
  return hip_status(launch_quant_v(v_bf16, B, Nk, Hkv, D, cu_seqlens_k, Nk, cols, format, partials, np, codes, scales,
                                   tensor_scale, false, st));
}

attn_status attn_quant_v_cache(const void* v_bf16, int32_t B, int32_t Nk, int32_t Hkv, int32_t D, int32_t format,
                               uint8_t* codes, uint8_t* scales, float* tensor_scale, void* ws, size_t ws_bytes,
                               void* stream) {
  if (B < 0 || Nk < 0 || Nk % 128 != 0 || Hkv <= 0 || (D != 64 && D != 128)) return ATTN_ERR_INVALID_ARGUMENT;
  if (format != ATTN_V_FP8_E4M3 && format != ATTN_V_MXFP4) return ATTN_ERR_INVALID_ARGUMENT;
  const int64_t tokens = (int64_t)B * Nk;
  if (format == ATTN_V_FP8_E4M3 && (tensor_scale == nullptr || !aligned(tensor_scale, 4)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (tokens > 0 && (v_bf16 == nullptr || codes == nullptr || !aligned(v_bf16, 16) || !aligned(codes, 16)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (tokens > 0 && format == ATTN_V_MXFP4 && (scales == nullptr || !aligned(scales, 4)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (ws == nullptr || ws_bytes < QUANT_WS || !aligned(ws, 16)) return ATTN_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  float* partials = (float*)ws;
  int np = 0;
  hipError_t e;
  if (format == ATTN_V_FP8_E4M3) {
    e = launch_amax(v_bf16, tokens * Hkv * (int64_t)D, partials, &np, st);
    if (e != hipSuccess) return hip_status(e);
  }
  if (B == 0) return ATTN_OK;
  return hip_status(launch_quant_v(v_bf16, B, Nk, Hkv, D, nullptr, Nk, (int64_t)B * Nk, format, partials, np, codes,
                                   scales, tensor_scale, true, st));
}

// Workspace of the forward: the K fp16 operand tiles, kcols columns per KV head.
static int64_t fwd_kcols(const attn_fwd_args* a) {
  if (a->cu_seqlens_q != nullptr) return 128 * ((a->total_k + 127) / 128 + a->B);
  return (int64_t)a->B * roundup(a->Nk, 128);
}

size_t attn_fwd_ws_bytes(const attn_fwd_args* a) {
  if (a == nullptr || a->B < 0 || a->Hq <= 0 || a->Hkv <= 0 || (a->D != 64 && a->D != 128)) return 0;
  return (size_t)(2 * a->D) * (size_t)(a->Hkv * fwd_kcols(a)) + 256;
}

static attn_status validate_fwd(const attn_fwd_args* a, bool allow_causal, int pf, bool mx = false,
                                bool own_ws = false) {
  if (a == nullptr) return ATTN_ERR_INVALID_ARGUMENT;
  if (a->B < 0 || a->Hq <= 0 || a->Hkv <= 0 || a->Nq < 0 || a->Nk < 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (a->D != 64 && a->D != 128) return ATTN_ERR_INVALID_ARGUMENT;
  if (a->Hq % a->Hkv != 0) return ATTN_ERR_INVALID_ARGUMENT;
  if ((a->cu_seqlens_q == nullptr) != (a->cu_seqlens_k == nullptr)) return ATTN_ERR_INVALID_ARGUMENT;
  const bool varlen = a->cu_seqlens_q != nullptr;
  if (varlen && (a->total_q < 0 || a->total_k < 0 || !aligned(a->cu_seqlens_q, 4) || !aligned(a->cu_seqlens_k, 4)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (!(a->softmax_scale > 0.0f) || a->softmax_scale != a->softmax_scale) return ATTN_ERR_INVALID_ARGUMENT;
  if (a->causal && !allow_causal) return ATTN_ERR_UNSUPPORTED;
  if (a->causal && a->Nq != a->Nk) return ATTN_ERR_INVALID_ARGUMENT;
  if (a->v.format != ATTN_V_FP8_E4M3 && a->v.format != ATTN_V_MXFP4) return ATTN_ERR_INVALID_ARGUMENT;
  if (pf == 1 && a->v.format != ATTN_V_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
  if (a->o_dtype != ATTN_OUT_BF16 && a->o_dtype != ATTN_OUT_F32) return ATTN_ERR_INVALID_ARGUMENT;
  const int64_t nq = varlen ? a->total_q : (int64_t)a->B * a->Nq;
  const int64_t nk = varlen ? a->total_k : (int64_t)a->B * a->Nk;
  const attn_nvfp4_tensor* t[2] = {&a->q, &a->k};
  const int64_t n[2] = {nq, nk};
  for (int i = 0; i < 2; ++i) {
    if (!mx && (t[i]->tensor_scale == nullptr || !aligned(t[i]->tensor_scale, 4))) return ATTN_ERR_INVALID_ARGUMENT;
    if (n[i] > 0 && (t[i]->codes == nullptr || t[i]->scales == nullptr || !aligned(t[i]->codes, mx ? 16 : 8)))
      return ATTN_ERR_INVALID_ARGUMENT;
    if (mx && n[i] > 0 && !aligned(t[i]->scales, a->D == 128 ? 4 : 2)) return ATTN_ERR_INVALID_ARGUMENT;
  }
  if (nk > 0 && (a->v.codes == nullptr || !aligned(a->v.codes, 16))) return ATTN_ERR_INVALID_ARGUMENT;
  if (nk > 0 && a->v.format == ATTN_V_MXFP4 && (a->v.scales == nullptr || !aligned(a->v.scales, 4)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (a->v.format == ATTN_V_FP8_E4M3 && (a->v.tensor_scale == nullptr || !aligned(a->v.tensor_scale, 4)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (nq > 0 && (a->o == nullptr || !aligned(a->o, 16))) return ATTN_ERR_INVALID_ARGUMENT;
  if (a->lse != nullptr && !aligned(a->lse, 4)) return ATTN_ERR_INVALID_ARGUMENT;
  if (a->dbg_p_codes != nullptr) {
    if (a->dbg_b < 0 || a->dbg_b >= a->B || a->dbg_h < 0 || a->dbg_h >= a->Hq || !aligned(a->dbg_p_codes, 16))
      return ATTN_ERR_INVALID_ARGUMENT;
    if (pf == 0 && a->dbg_p_scales == nullptr) return ATTN_ERR_INVALID_ARGUMENT;
  }
  // The kernels address one KV head's V^T rows with 32-bit per-lane byte
  // offsets d * cols (FP8: one byte per key; MXFP4: half a byte), and index
  // workgroups with 32-bit integers.
  const int64_t kcols = fwd_kcols(a);
  const int64_t vrow_bytes = a->v.format == ATTN_V_MXFP4 ? (int64_t)a->D * kcols / 2 : (int64_t)a->D * kcols;
  if (vrow_bytes >= ((int64_t)1 << 32)) return ATTN_ERR_UNSUPPORTED;
  // (query blocks of 256 rows; packed batches pad them to whole groups of 16)
  const int64_t qb = ((int64_t)a->Nq + WG_Q - 1) / WG_Q + 16;
  if ((int64_t)a->B * a->Hq * qb >= ((int64_t)1 << 31)) return ATTN_ERR_UNSUPPORTED;
  const size_t need = attn_fwd_ws_bytes(a);
  if (own_ws) return need <= ATTN_NOALLOC_SCRATCH_BYTES ? ATTN_OK : ATTN_ERR_WORKSPACE;
  if (a->ws == nullptr || a->ws_bytes < need || !aligned(a->ws, 256)) return ATTN_ERR_WORKSPACE;
  return ATTN_OK;
}

// Scratch of attn_fwd_directp_noalloc: a fixed device array in place of the
// caller's workspace for the float16 K operand tiles.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and only
// that address is passed to the kernels.
static __device__ __align__(256) uint8_t scratch[ATTN_NOALLOC_SCRATCH_BYTES];
constexpr int SCRATCH_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[SCRATCH_MAX_DEVICES];

static attn_status scratch_address(hipStream_t st, void** out) {
  int dev = 0, cur = 0;
  hipError_t e = hipStreamGetDevice(st, &dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_status(e);
    if (ptr == nullptr) return hip_status(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

// mx: the MX-native Q/K mode (MXFP4 Q/K codes with E8M0 bytes, no tensor
// scales; exact encoders), whose K pre-pass packs FP4 operand tiles instead
// of expanding K to FP16.
static attn_status run_fwd_lowp(const attn_fwd_args* a, void* stream, int pf, int enc, bool mx = false,
                                bool own_ws = false) {
  attn_status s = validate_fwd(a, pf == 1, pf, mx, own_ws);
  if (s != ATTN_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const bool varlen = a->cu_seqlens_q != nullptr;
  const int64_t kcols = fwd_kcols(a);
  void* ws = a->ws;
  if (own_ws && (s = scratch_address(st, &ws)) != ATTN_OK) return s;
  _Float16* khat = (_Float16*)ws;
  const int64_t nk_pad = roundup(a->Nk, 128);
  hipError_t e = mx ? launch_pack_k_mx(a->k.codes, a->k.scales, a->Hkv, a->B, a->Nk, a->Nk, a->cu_seqlens_k, nk_pad,
                                       kcols, a->D, pf, (uint8_t*)ws, st)
                    : launch_expand_k(a->k.codes, a->k.scales, a->Hkv, a->B, a->Nk, a->Nk, a->cu_seqlens_k, nk_pad,
                                      kcols, a->D, pf, khat, st);
  if (e != hipSuccess) return hip_status(e);
  FwdParams p;
  memset(&p, 0, sizeof(p));
  p.q_codes = a->q.codes;
  p.q_scales = a->q.scales;
  p.khat = khat;
  p.kcols = kcols;
  p.v_codes = a->v.codes;
  p.v_scales = a->v.scales;
  p.gq = a->q.tensor_scale;
  p.gk = a->k.tensor_scale;
  p.sv = a->v.tensor_scale;
  p.o = a->o;
  p.o_f32 = a->o_dtype == ATTN_OUT_F32;
  p.lse = a->lse;
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.Nq = a->Nq;
  p.Nk = a->Nk;
  p.QB = (a->Nq + WG_Q - 1) / WG_Q;
  p.nk_pad = nk_pad;
  p.sigma = a->softmax_scale;
  p.dbg_codes = a->dbg_p_codes;
  p.dbg_scales = a->dbg_p_scales;
  p.dbg_b = a->dbg_b;
  p.dbg_h = a->dbg_h;
  p.dbg_ld = nk_pad;
  (void)varlen;
  if (a->prof_event_begin != nullptr) {
    e = hipEventRecord((hipEvent_t)a->prof_event_begin, st);
    if (e != hipSuccess) return hip_status(e);
  }
  e = mx ? launch_fwd_mx(p, a->D, pf, a->v.format == ATTN_V_MXFP4 ? 1 : 0, a->causal != 0, a->dbg_p_codes != nullptr,
                         enc, st)
         : launch_fwd_lowp(p, a->D, pf, a->v.format == ATTN_V_MXFP4 ? 1 : 0, a->causal != 0,
                           a->dbg_p_codes != nullptr, enc, st);
  if (e != hipSuccess) return hip_status(e);
  if (a->prof_event_end != nullptr) e = hipEventRecord((hipEvent_t)a->prof_event_end, st);
  return hip_status(e);
}

attn_status attn_fwd_directp(const attn_fwd_args* a, void* stream) { return run_fwd_lowp(a, stream, 0, 0); }
attn_status attn_fwd_directp_noalloc(const attn_fwd_args* a, void* stream) {
  return run_fwd_lowp(a, stream, 0, 0, false, true);
}
attn_status attn_fwd_fp8pv(const attn_fwd_args* a, void* stream) { return run_fwd_lowp(a, stream, 1, 0); }
attn_status attn_fwd_directp_efq(const attn_fwd_args* a, void* stream) { return run_fwd_lowp(a, stream, 0, 1); }
attn_status attn_fwd_fp8pv_cast(const attn_fwd_args* a, void* stream) { return run_fwd_lowp(a, stream, 1, 1); }
attn_status attn_fwd_directp_mxqk(const attn_fwd_args* a, void* stream) {
  return run_fwd_lowp(a, stream, 0, 0, true);
}
attn_status attn_fwd_fp8pv_mxqk(const attn_fwd_args* a, void* stream) { return run_fwd_lowp(a, stream, 1, 0, true); }
attn_status attn_fwd_directp_efq_mxqk(const attn_fwd_args* a, void* stream) {
  return run_fwd_lowp(a, stream, 0, 1, true);
}
attn_status attn_fwd_fp8pv_cast_mxqk(const attn_fwd_args* a, void* stream) {
  return run_fwd_lowp(a, stream, 1, 1, true);
}

attn_status attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B, int32_t Hq,
                          int32_t Hkv, int32_t Nq, int32_t Nk, int32_t D, float softmax_scale, int32_t causal,
                          void* stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Nq < 0 || Nk < 0 || (D != 64 && D != 128) || Hq % Hkv != 0)
    return ATTN_ERR_INVALID_ARGUMENT;
  if (!(softmax_scale > 0.0f)) return ATTN_ERR_INVALID_ARGUMENT;
  if (causal && Nq != Nk) return ATTN_ERR_INVALID_ARGUMENT;
  const int64_t nq = (int64_t)B * Nq, nk = (int64_t)B * Nk;
  if (nq > 0 && (q == nullptr || o == nullptr || !aligned(q, 16) || !aligned(o, 16))) return ATTN_ERR_INVALID_ARGUMENT;
  if (nk > 0 && (k == nullptr || v == nullptr || !aligned(k, 16) || !aligned(v, 16))) return ATTN_ERR_INVALID_ARGUMENT;
  if (lse != nullptr && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARGUMENT;
  // the rows of one 128-key tile are addressed with 32-bit byte offsets from the tile's base
  if ((int64_t)KEY_TILE * Hkv * D * 2 >= ((int64_t)1 << 31)) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq * ((Nq + WG_Q - 1) / WG_Q) >= ((int64_t)1 << 31)) return ATTN_ERR_UNSUPPORTED;
  return hip_status(launch_fwd_bf16(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, D, softmax_scale, causal != 0,
                                    (hipStream_t)stream));
}


// ---- backward -------------------------------------------------------------
struct BwdLayout {
  int64_t npad, qrm, krm, vrm, drm, dvec, lvec, sdo, partials, total;
};

static bool bwd_shapes_ok(const attn_bwd_args* a) {
  // the supported range: one head's bf16 operand rows (2 D NPAD bytes) below 2^31 bytes
  return a != nullptr && a->B >= 0 && a->N >= 0 && a->Hq > 0 && a->Hkv > 0 && a->Hq % a->Hkv == 0 &&
         (a->D == 64 || a->D == 128) && 2 * (int64_t)a->D * roundup(a->N, 128) < ((int64_t)1 << 31);
}

static BwdLayout bwd_layout(const attn_bwd_args* a) {
  BwdLayout L;
  auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
  L.npad = roundup(a->N, 128);
  const int64_t nq = (int64_t)a->B * a->Hq * L.npad * a->D, nk = (int64_t)a->B * a->Hkv * L.npad * a->D;
  int64_t off = 0;
  L.qrm = off; off += al(2 * nq);
  L.krm = off; off += al(2 * nk);
  L.vrm = off; off += al(nk);
  L.drm = off; off += al(nq);
  L.dvec = off; off += al(4 * (int64_t)a->B * a->Hq * L.npad);
  L.lvec = off; off += al(4 * (int64_t)a->B * a->Hq * L.npad);
  L.sdo = off; off += 256;
  L.partials = off; off += (int64_t)QUANT_WS;
  L.total = off;
  return L;
}

size_t attn_bwd_ws_bytes(const attn_bwd_args* a) {
  if (!bwd_shapes_ok(a)) return 0;
  return (size_t)bwd_layout(a).total + 256;
}

attn_status attn_bwd_fp8(const attn_bwd_args* a, void* stream) {
  if (!bwd_shapes_ok(a) || !(a->softmax_scale > 0.0f)) return ATTN_ERR_INVALID_ARGUMENT;
  if (a->v.format != ATTN_V_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
  if (a->N > 0) {
    const void* need[] = {a->q.codes, a->q.scales, a->q.tensor_scale, a->k.codes, a->k.scales, a->k.tensor_scale,
                          a->v.codes, a->v.tensor_scale, a->o, a->lse, a->dout, a->dq, a->dk, a->dv};
    for (const void* x : need)
      if (x == nullptr) return ATTN_ERR_INVALID_ARGUMENT;
    if (!aligned(a->o, 16) || !aligned(a->dout, 16) || !aligned(a->q.codes, 4) || !aligned(a->k.codes, 4) ||
        !aligned(a->v.codes, 16) || !aligned(a->lse, 4) || !aligned(a->dq, 4) || !aligned(a->dk, 4) ||
        !aligned(a->dv, 4))
      return ATTN_ERR_INVALID_ARGUMENT;
  }
  const uint8_t* dumps[] = {a->dbg_p_codes, a->dbg_p_exps, a->dbg_dsk_codes, a->dbg_dsk_exps, a->dbg_dsq_codes,
                           a->dbg_dsq_exps};
  int ndump = 0;
  for (const uint8_t* x : dumps) ndump += x != nullptr;
  const bool debug = ndump == 6;
  if (ndump != 0 && (!debug || a->dbg_b < 0 || a->dbg_b >= a->B || a->dbg_h < 0 || a->dbg_h >= a->Hq))
    return ATTN_ERR_INVALID_ARGUMENT;
  const BwdLayout L = bwd_layout(a);
  if (a->ws == nullptr || a->ws_bytes < (size_t)L.total || !aligned(a->ws, 256)) return ATTN_ERR_WORKSPACE;
  if (a->N == 0 || a->B == 0) return ATTN_OK;
  hipStream_t st = (hipStream_t)stream;
  uint8_t* w = (uint8_t*)a->ws;
  int np = 0;
  float* partials = (float*)(w + L.partials);
  hipError_t e = launch_amax(a->dout, (int64_t)a->B * a->N * a->Hq * a->D, partials, &np, st);
  if (e != hipSuccess) return hip_status(e);
  float* sdo = (float*)(w + L.sdo);
  e = launch_bwd_prep(a->q.codes, a->q.scales, a->k.codes, a->k.scales, a->v.codes, (int64_t)a->B * L.npad, a->dout,
                      a->o, a->lse, partials, np, a->B, a->Hq, a->Hkv, a->N, a->D, L.npad, (__bf16*)(w + L.qrm),
                      (__bf16*)(w + L.krm), w + L.vrm, w + L.drm, (float*)(w + L.dvec), (float*)(w + L.lvec), sdo,
                      st);
  if (e != hipSuccess) return hip_status(e);
  BwdParams p;
  memset(&p, 0, sizeof(p));
  p.qrm = (const __bf16*)(w + L.qrm);
  p.krm = (const __bf16*)(w + L.krm);
  p.vrm = w + L.vrm;
  p.dorm = w + L.drm;
  p.lv = (const float*)(w + L.lvec);
  p.dv = (const float*)(w + L.dvec);
  p.gq = a->q.tensor_scale;
  p.gk = a->k.tensor_scale;
  p.sv = a->v.tensor_scale;
  p.sdo = sdo;
  p.dq_out = a->dq;
  p.dk_out = a->dk;
  p.dv_out = a->dv;
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.N = a->N;
  p.npad = L.npad;
  p.sigma = a->softmax_scale;
  p.dbg_pt = a->dbg_p_codes;
  p.dbg_pt_e = a->dbg_p_exps;
  p.dbg_dsk = a->dbg_dsk_codes;
  p.dbg_dsk_e = a->dbg_dsk_exps;
  p.dbg_dsq = a->dbg_dsq_codes;
  p.dbg_dsq_e = a->dbg_dsq_exps;
  p.dbg_b = a->dbg_b;
  p.dbg_h = a->dbg_h;
  if (a->prof_event_begin != nullptr) {
    e = hipEventRecord((hipEvent_t)a->prof_event_begin, st);
    if (e != hipSuccess) return hip_status(e);
  }
  e = launch_bwd_main(p, a->D, a->causal != 0, debug, st);
  if (e != hipSuccess) return hip_status(e);
  if (a->prof_event_end != nullptr) e = hipEventRecord((hipEvent_t)a->prof_event_end, st);
  return hip_status(e);
}

// ---- decode-shaped forward ----
static attn_status validate_decode(const attn_decode_args* a, int pf) {
  if (a == nullptr) return ATTN_ERR_INVALID_ARGUMENT;
  if (a->B < 0 || a->Hq <= 0 || a->Hkv <= 0 || a->nq < 1 || a->Nk < 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (a->D != 64 && a->D != 128) return ATTN_ERR_INVALID_ARGUMENT;
  if (a->Nk % 128 != 0) return ATTN_ERR_INVALID_ARGUMENT;   // cache capacity in whole 128-key tiles
  if (a->Hq % a->Hkv != 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (!(a->softmax_scale > 0.0f) || a->softmax_scale != a->softmax_scale) return ATTN_ERR_INVALID_ARGUMENT;
  if (a->v.format != ATTN_V_FP8_E4M3 && a->v.format != ATTN_V_MXFP4) return ATTN_ERR_INVALID_ARGUMENT;
  if (pf == 1 && a->v.format != ATTN_V_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
  if (a->o_dtype != ATTN_OUT_BF16 && a->o_dtype != ATTN_OUT_F32) return ATTN_ERR_INVALID_ARGUMENT;
  // one workgroup per (sequence, KV head, 16 query rows): the grid's x size
  const int64_t qg = ((int64_t)(a->Hq / a->Hkv) * a->nq + 15) / 16;
  if ((int64_t)a->B * a->Hkv * qg >= ((int64_t)1 << 31)) return ATTN_ERR_UNSUPPORTED;
  if (a->seqlens_k != nullptr && !aligned(a->seqlens_k, 4)) return ATTN_ERR_INVALID_ARGUMENT;
  const int64_t nq = (int64_t)a->B * a->nq, nk = (int64_t)a->B * a->Nk;
  const attn_nvfp4_tensor* t[2] = {&a->q, &a->k};
  const int64_t n[2] = {nq, nk};
  for (int i = 0; i < 2; ++i) {
    if (t[i]->tensor_scale == nullptr || !aligned(t[i]->tensor_scale, 4)) return ATTN_ERR_INVALID_ARGUMENT;
    if (n[i] > 0 && (t[i]->codes == nullptr || t[i]->scales == nullptr || !aligned(t[i]->codes, 16) ||
                     !aligned(t[i]->scales, 4)))
      return ATTN_ERR_INVALID_ARGUMENT;
  }
  if (nk > 0 && (a->v.codes == nullptr || !aligned(a->v.codes, 16))) return ATTN_ERR_INVALID_ARGUMENT;
  if (nk > 0 && a->v.format == ATTN_V_MXFP4 && (a->v.scales == nullptr || !aligned(a->v.scales, 4)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (a->v.format == ATTN_V_FP8_E4M3 && (a->v.tensor_scale == nullptr || !aligned(a->v.tensor_scale, 4)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (nq > 0 && (a->o == nullptr || !aligned(a->o, 16))) return ATTN_ERR_INVALID_ARGUMENT;
  if (a->lse != nullptr && !aligned(a->lse, 4)) return ATTN_ERR_INVALID_ARGUMENT;
  if (a->dbg_p_codes != nullptr) {
    if (a->dbg_b < 0 || a->dbg_b >= a->B || a->dbg_h < 0 || a->dbg_h >= a->Hq || !aligned(a->dbg_p_codes, 16))
      return ATTN_ERR_INVALID_ARGUMENT;
    if (pf == 0 && a->dbg_p_scales == nullptr) return ATTN_ERR_INVALID_ARGUMENT;
  }
  return ATTN_OK;
}

static attn_status run_decode(const attn_decode_args* a, void* stream, int pf) {
  attn_status s = validate_decode(a, pf);
  if (s != ATTN_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  DecParams p;
  memset(&p, 0, sizeof(p));
  p.q_codes = a->q.codes;
  p.q_scales = a->q.scales;
  p.k_codes = a->k.codes;
  p.k_scales = a->k.scales;
  p.v_codes = a->v.codes;
  p.v_scales = a->v.scales;
  p.gq = a->q.tensor_scale;
  p.gk = a->k.tensor_scale;
  p.sv = a->v.tensor_scale;
  p.seqlens = a->seqlens_k;
  p.o = a->o;
  p.o_f32 = a->o_dtype == ATTN_OUT_F32;
  p.lse = a->lse;
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.nq = a->nq;
  p.Nk = a->Nk;
  p.QG = (int)(((int64_t)(a->Hq / a->Hkv) * a->nq + 15) / 16);   // 16 query rows per workgroup
  p.nk_pad = roundup(a->Nk, 128);
  p.sigma = a->softmax_scale;
  p.dbg_codes = a->dbg_p_codes;
  p.dbg_scales = a->dbg_p_scales;
  p.dbg_b = a->dbg_b;
  p.dbg_h = a->dbg_h;
  p.dbg_ld = p.nk_pad;
  hipError_t e;
  if (a->prof_event_begin != nullptr) {
    e = hipEventRecord((hipEvent_t)a->prof_event_begin, st);
    if (e != hipSuccess) return hip_status(e);
  }
  // with one new token the causal mask hides nothing (the token is the last key)
  const bool causal = a->causal != 0 && a->nq > 1;
  e = launch_decode(p, a->D, pf, a->v.format == ATTN_V_MXFP4 ? 1 : 0, causal, a->dbg_p_codes != nullptr, st);
  if (e != hipSuccess) return hip_status(e);
  if (a->prof_event_end != nullptr) e = hipEventRecord((hipEvent_t)a->prof_event_end, st);
  return hip_status(e);
}

attn_status attn_decode_directp(const attn_decode_args* a, void* stream) { return run_decode(a, stream, 0); }
attn_status attn_decode_fp8pv(const attn_decode_args* a, void* stream) { return run_decode(a, stream, 1); }

// ---- diagnostics ------------------------------------------------------------
int attn_probe_kinds(void) { return probe_kind_count(); }

attn_status attn_probe_issue_rates(int kind, long long* cycles, long long* units, int* grid, void* stream) {
  if (kind < 0 || kind >= probe_kind_count() || cycles == nullptr || units == nullptr || grid == nullptr ||
      !aligned(cycles, 8))
    return ATTN_ERR_INVALID_ARGUMENT;
  int64_t u = 0;
  int g = 0;
  const hipError_t e = launch_probe_kind(kind, cycles, &u, &g, (hipStream_t)stream);
  *units = (long long)u;
  *grid = g;
  return hip_status(e);
}

}  // extern "C"
