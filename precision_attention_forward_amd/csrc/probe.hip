// Issue-rate micro-kernels of gfx950: the per-instruction costs that the
// kernels' roofline notes rest on (vector ALU, transcendental, the MX
// conversions, the matrix instructions, LDS reads and writes, and how much
// vector issue fits beside the matrix pipe).  Not part of the attention
// path: a diagnostics entry point for the measurement script.
//
// Each launch is 256 workgroups with 96 KB of LDS each (one per CU), of 512
// threads (two waves per SIMD) unless a kind says otherwise.  Every
// wave of a workgroup starts after a barrier and the span ends after a second
// barrier, so the cycle count (s_memtime) covers every wave's work.
#include "common.h"

namespace attn {
namespace {

constexpr int PROBE_GRID = 256;
constexpr int PROBE_ITERS = 4096;
constexpr int PROBE_LDS = 96 * 1024;

typedef short p16x4 __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) p16x4 lds_p16x4;

enum ProbeKind {
  P_FMA = 0, P_EXP, P_MED3, P_CVT_FP8, P_MAX3,          // 8 waves per CU, 8 independent chains each
  P_MFMA_BF16, P_MFMA_FP8, P_MFMA_FP4,                  // 4 waves per CU (one per SIMD), 4 chains
  P_MFMA_AND_FMA, P_MFMA_AND_EXP,                       // waves 0-3 MFMA, waves 4-7 vector
  P_MIX2, P_MIX4, P_MIX8,                               // 8 waves: k FMA per MFMA in each wave
  P_LDS_R128, P_LDS_R64, P_LDS_TR64, P_LDS_W128, P_LDS_W32,
  P_CVT_FP4,                                            // 8 waves per CU, 8 chains, like the vector kinds
  P_EXP_FMA, P_EXP_FMA3, P_EXP_MAX3, P_EXP_CVT_FP4,     // 8 waves: v_exp_f32 chains interleaved with others
  P_EXP_FMA_G4,                                         // as P_EXP_FMA, in runs of four of each
  P_FMA_4W, P_MIX8_4W,                                  // 16 waves per CU (four per SIMD)
  P_MIX16,                                              // 8 waves: 16 FMA per MFMA in each wave
  P_MFMA_FMA3, P_MFMA_FMA4, P_MFMA_EXP2,                // as P_MFMA_AND_FMA / EXP with 3x, 4x, 2x the vector work
  P_FWD_INTER, P_FWD_PPB, P_FWD_DEP, P_FWD_SKEW,        // the forward key loop's instruction mix per 128-key tile
  P_COUNT
};

// The forward mix per wave and 128-key tile: 42 bf16 32x32x16 MFMA and 228
// vector instructions (64 v_exp_f32, 32 FP4 conversions, 36 v_max3_f32, 96
// v_fma_f32), all independent (FX_*), or with the encode as dependent chains.
#define FX_MFMA(c) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc[(c) & 3]) : "v"(opb), "v"(opb))
#define FX_EXP(i) asm volatile("v_exp_f32 %0, %0" : "+v"(x[(i) & 7]))
#define FX_FMA(i) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(y[(i) & 7]) : "v"(a), "v"(b))
#define FX_MAX3(i) asm volatile("v_max3_f32 %0, %0, |%1|, |%2|" : "+v"(z[(i) & 3]) : "v"(a), "v"(b))
#define FX_CVT(i) asm volatile("v_cvt_scalef32_pk_fp4_f32 %0, %1, %1, %2" : "+v"(w[(i) & 3]) : "v"(y[((i) + 3) & 7]), "v"(one))
#define FX_VUNIT(u) do { const int uu = (u); \
    if (uu % 57 < 16) FX_EXP(uu); else if (uu % 57 < 24) FX_CVT(uu); else if (uu % 57 < 33) FX_MAX3(uu); else FX_FMA(uu); } while (0)

template <int KIND>
__global__ void __launch_bounds__(1024) probe_kernel(long long* cycles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[PROBE_LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float x[8], y[8], z[4], w[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = 0.001f * (float)(tid + i);
    y[i] = 0.002f * (float)(tid + i);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[i] = 0.1f * (float)(tid + i);
    w[i] = 0.0f;
  }
  const float a = 1.0001f, b = 0.5f, one = 1.0f;
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  bf16x8 opb;
  i32x8 op8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    opb[i] = (__bf16)(0.01f * (float)(tid + i));
    op8[i] = 0x3a3a3a3a + tid + i;
  }
  for (int i = tid; i < PROBE_LDS / 16; i += blockDim.x)
    reinterpret_cast<u32x4*>(lds)[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  u32x4 lacc = {0, 0, 0, 0};
  __syncthreads();
  const long long t0 = __builtin_readcyclecounter();
  if (KIND >= P_MFMA_FMA3 && KIND <= P_MFMA_EXP2) {
    // waves 0-3: 4 MFMA per iteration; waves 4-7: N x 8 FMA or exponentials
    constexpr int N = KIND == P_MFMA_FMA3 ? 3 : KIND == P_MFMA_FMA4 ? 4 : 2;
    if (wave < 4) {
      for (int it = 0; it < PROBE_ITERS; ++it) {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opb, opb, acc[c & 1], 0, 0, 0);
      }
    } else {
      for (int it = 0; it < PROBE_ITERS; ++it) {
#pragma unroll
        for (int r = 0; r < N; ++r)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (KIND == P_MFMA_EXP2) asm volatile("v_exp_f32 %0, %0" : "+v"(x[i]));
            else asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(a), "v"(b));
          }
      }
    }
  } else if (KIND == P_FWD_INTER || KIND == P_FWD_PPB) {
    constexpr int T = PROBE_ITERS / 32;   // tiles per wave
    if (KIND == P_FWD_INTER) {
      // every wave: 42 slots of one MFMA and its share of the 228 vector instructions
      for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int sl = 0; sl < 42; ++sl) {
          FX_MFMA(sl);
#pragma unroll
          for (int u = (sl * 228) / 42; u < ((sl + 1) * 228) / 42; ++u) FX_VUNIT(u);
        }
      }
    } else {
      // ping-pong: each wave alternates the 42 MFMA and the 228 vector
      // instructions; waves 4-7 start with a vector phase, so the two waves of a
      // SIMD are in opposite phases, with a workgroup barrier after every phase
      if (wave >= 4) {
#pragma unroll
        for (int u = 0; u < 228; ++u) FX_VUNIT(u);
        __builtin_amdgcn_s_barrier();
      }
      for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int sl = 0; sl < 42; ++sl) FX_MFMA(sl);
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int u = 0; u < 228; ++u) FX_VUNIT(u);
        __builtin_amdgcn_s_barrier();
      }
      if (wave < 4) {
#pragma unroll
        for (int sl = 0; sl < 42; ++sl) FX_MFMA(sl);
        __builtin_amdgcn_s_barrier();
      }
    }
  } else if (KIND == P_FWD_DEP || KIND == P_FWD_SKEW) {
    // the encode as dependent chains: per unit of two scores t = fma(s, c, -m),
    // p = exp(t), codes = cvt(p0, p1); 32 units per tile, one starting in each
    // of slots 0-31, beside 100 further vector instructions (36 max3, 64 fma);
    // 260 vector instructions per tile.  DEP: a unit's whole chain in its slot;
    // SKEW: its fma in slot i, its exponentials in slot i+1, its conversion in
    // slot i+2.
    constexpr int T = PROBE_ITERS / 32;
    float sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = 0.01f * (float)(tid + i);
    float t0[3], t1[3], p0[3], p1[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) t0[i] = t1[i] = p0[i] = p1[i] = 0.0f;
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int sl = 0; sl < 42; ++sl) {
        FX_MFMA(sl);
        if (KIND == P_FWD_DEP) {
          if (sl < 32) {
            const float a0 = sv[(2 * sl) & 7], a1 = sv[(2 * sl + 1) & 7];
            asm volatile("v_fma_f32 %0, %1, %2, %3" : "=v"(t0[0]) : "v"(a0), "v"(a), "v"(b));
            asm volatile("v_fma_f32 %0, %1, %2, %3" : "=v"(t1[0]) : "v"(a1), "v"(a), "v"(b));
            asm volatile("v_exp_f32 %0, %1" : "=v"(p0[0]) : "v"(t0[0]));
            asm volatile("v_exp_f32 %0, %1" : "=v"(p1[0]) : "v"(t1[0]));
            asm volatile("v_cvt_scalef32_pk_fp4_f32 %0, %1, %2, %3" : "+v"(w[sl & 3]) : "v"(p0[0]), "v"(p1[0]), "v"(one));
          }
        } else {
          if (sl >= 2 && sl < 34) {
            const int k2 = (sl - 2) % 3;
            asm volatile("v_cvt_scalef32_pk_fp4_f32 %0, %1, %2, %3" : "+v"(w[sl & 3]) : "v"(p0[k2]), "v"(p1[k2]), "v"(one));
          }
          if (sl >= 1 && sl < 33) {
            const int k1 = (sl - 1) % 3;
            asm volatile("v_exp_f32 %0, %1" : "=v"(p0[k1]) : "v"(t0[k1]));
            asm volatile("v_exp_f32 %0, %1" : "=v"(p1[k1]) : "v"(t1[k1]));
          }
          if (sl < 32) {
            const int k = sl % 3;
            const float a0 = sv[(2 * sl) & 7], a1 = sv[(2 * sl + 1) & 7];
            asm volatile("v_fma_f32 %0, %1, %2, %3" : "=v"(t0[k]) : "v"(a0), "v"(a), "v"(b));
            asm volatile("v_fma_f32 %0, %1, %2, %3" : "=v"(t1[k]) : "v"(a1), "v"(a), "v"(b));
          }
        }
#pragma unroll
        for (int u = (sl * 100) / 42; u < ((sl + 1) * 100) / 42; ++u) {
          if (u % 25 < 9) FX_MAX3(u);
          else FX_FMA(u);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) x[i] += t0[i] + t1[i] + p0[i] + p1[i];
  } else if (KIND == P_CVT_FP4) {
    for (int it = 0; it < PROBE_ITERS; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        asm volatile("v_cvt_scalef32_pk_fp4_f32 %0, %1, %1, %2" : "+v"(x[i]) : "v"(x[(i + 1) & 7]), "v"(one));
    }
  } else if (KIND == P_EXP_FMA_G4) {
    for (int it = 0; it < PROBE_ITERS; ++it) {
#pragma unroll
      for (int g = 0; g < 8; g += 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("v_exp_f32 %0, %0" : "+v"(x[g + i]));
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(y[g + i]) : "v"(a), "v"(b));
      }
    }
  } else if (KIND == P_FMA_4W) {
    for (int it = 0; it < PROBE_ITERS; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(a), "v"(b));
    }
  } else if (KIND > P_CVT_FP4 && KIND <= P_EXP_CVT_FP4) {
    // one v_exp_f32 per step on x[i], followed by independent work on y
    for (int it = 0; it < PROBE_ITERS; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        asm volatile("v_exp_f32 %0, %0" : "+v"(x[i]));
        if (KIND == P_EXP_FMA) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(y[i]) : "v"(a), "v"(b));
        if (KIND == P_EXP_FMA3) {
          asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(y[i]) : "v"(a), "v"(b));
          asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(y[(i + 3) & 7]) : "v"(a), "v"(b));
          asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(y[(i + 6) & 7]) : "v"(a), "v"(b));
        }
        if (KIND == P_EXP_MAX3) asm volatile("v_max3_f32 %0, %0, |%1|, |%2|" : "+v"(y[i]) : "v"(a), "v"(b));
        if (KIND == P_EXP_CVT_FP4)
          asm volatile("v_cvt_scalef32_pk_fp4_f32 %0, %1, %1, %2" : "+v"(y[i]) : "v"(y[(i + 1) & 7]), "v"(one));
      }
    }
  } else if (KIND <= P_MAX3) {
    for (int it = 0; it < PROBE_ITERS; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (KIND == P_FMA) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(a), "v"(b));
        if (KIND == P_EXP) asm volatile("v_exp_f32 %0, %0" : "+v"(x[i]));
        if (KIND == P_MED3) asm volatile("v_med3_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(a), "v"(b));
        if (KIND == P_MAX3) asm volatile("v_max3_f32 %0, %0, |%1|, |%2|" : "+v"(x[i]) : "v"(a), "v"(b));
        if (KIND == P_CVT_FP8)
          asm volatile("v_cvt_scalef32_pk_fp8_f32 %0, %1, %1, %2" : "+v"(x[i]) : "v"(x[(i + 1) & 7]), "v"(one));
      }
    }
  } else if (KIND <= P_MFMA_FP4) {
    for (int it = 0; it < PROBE_ITERS; ++it) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (KIND == P_MFMA_BF16) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opb, opb, acc[c], 0, 0, 0);
        if (KIND == P_MFMA_FP8)
          acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op8, op8, acc[c], 0, 0, 0, 127, 0, 127);
        if (KIND == P_MFMA_FP4)
          acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op8, op8, acc[c], 4, 4, 0, 127, 0, 127);
      }
    }
  } else if (KIND <= P_MFMA_AND_EXP) {
    if (wave < 4) {
      for (int it = 0; it < PROBE_ITERS; ++it) {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opb, opb, acc[c & 1], 0, 0, 0);
      }
    } else {
      for (int it = 0; it < PROBE_ITERS; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (KIND == P_MFMA_AND_FMA) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(a), "v"(b));
          else asm volatile("v_exp_f32 %0, %0" : "+v"(x[i]));
        }
      }
    }
  } else if (KIND <= P_MIX8 || KIND == P_MIX8_4W || KIND == P_MIX16) {
    constexpr int K = KIND == P_MIX2 ? 2 : KIND == P_MIX4 ? 4 : KIND == P_MIX16 ? 16 : 8;
    for (int it = 0; it < PROBE_ITERS; ++it) {
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opb, opb, acc[0], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < K; ++i) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[i & 7]) : "v"(a), "v"(b));
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opb, opb, acc[1], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < K; ++i) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[(i + 4) & 7]) : "v"(a), "v"(b));
    }
  } else {
    // LDS: each wave streams 8 accesses per iteration over a 64 KB window,
    // lane-contiguous (no bank conflicts); 16, 8 or 4 bytes per lane
    constexpr int BPL = (KIND == P_LDS_R128 || KIND == P_LDS_W128) ? 16 : (KIND == P_LDS_W32 ? 4 : 8);
    const uint32_t lb = (uint32_t)lane * BPL;
    for (int it = 0; it < PROBE_ITERS; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t ad = (lb + (uint32_t)((it * 8 + j + wave * 8) * 64 * BPL)) & 65535u;
        uint8_t* pa = lds + ad;
        if (KIND == P_LDS_R128) lacc ^= *reinterpret_cast<const u32x4*>(pa);
        if (KIND == P_LDS_R64) {
          const u32x2 v = *reinterpret_cast<const u32x2*>(pa);
          lacc[0] ^= v[0];
          lacc[1] ^= v[1];
        }
        if (KIND == P_LDS_TR64) {
          const p16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_p16x4*)(__attribute__((address_space(3))) void*)pa);
          lacc[0] ^= (uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16);
          lacc[1] ^= (uint32_t)(uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16);
        }
        if (KIND == P_LDS_W128) *reinterpret_cast<u32x4*>(pa) = u32x4{(uint32_t)it, (uint32_t)j, 0u, 0u};
        if (KIND == P_LDS_W32) *reinterpret_cast<uint32_t*>(pa) = (uint32_t)(it + j);
      }
    }
  }
  __syncthreads();
  const long long t1 = __builtin_readcyclecounter();
  // keep every result live: a store that no input can trigger
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i] + y[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) s += z[i] + w[i];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  lacc[0] ^= reinterpret_cast<const uint32_t*>(lds)[tid];
  // a hash of every result against a value the compiler cannot know (it
  // depends on the clock): the store, in bounds, almost never happens
  const uint32_t hsh = __float_as_uint(s) ^ lacc[0] ^ lacc[1] ^ lacc[2] ^ lacc[3];
  if (hsh == 0x5a5a0000u + (uint32_t)(t1 & 0xffff)) cycles[PROBE_GRID + blockIdx.x] = hsh;
  if (tid == 0) cycles[blockIdx.x] = t1 - t0;
}

// threads per workgroup and the work one launch puts on a SIMD (instructions)
// or, for the LDS kinds, on a CU (bytes)
void probe_shape(int kind, int* threads, int64_t* units) {
  const int64_t it = PROBE_ITERS;
  switch (kind) {
    case P_FMA: case P_EXP: case P_MED3: case P_MAX3: *threads = 512; *units = 2 * it * 8; break;
    case P_CVT_FP8: *threads = 512; *units = 2 * it * 8; break;
    case P_MFMA_BF16: case P_MFMA_FP8: case P_MFMA_FP4: *threads = 256; *units = it * 4; break;
    case P_MFMA_AND_FMA: case P_MFMA_AND_EXP: *threads = 512; *units = it * 4; break;   // MFMA per SIMD
    case P_MIX2: case P_MIX4: case P_MIX8: *threads = 512; *units = 2 * it * 2; break;   // MFMA per SIMD
    case P_LDS_R128: case P_LDS_W128: *threads = 512; *units = 8 * it * 8 * 64 * 16; break;
    case P_LDS_R64: case P_LDS_TR64: *threads = 512; *units = 8 * it * 8 * 64 * 8; break;
    case P_CVT_FP4: *threads = 512; *units = 2 * it * 8; break;
    case P_EXP_FMA: case P_EXP_FMA3: case P_EXP_MAX3: case P_EXP_CVT_FP4: case P_EXP_FMA_G4:
      *threads = 512; *units = 2 * it * 8; break;                    // exponentials per SIMD
    case P_FMA_4W: *threads = 1024; *units = 4 * it * 8; break;
    case P_MIX8_4W: *threads = 1024; *units = 4 * it * 2; break;     // MFMA per SIMD
    case P_MIX16: *threads = 512; *units = 2 * it * 2; break;        // MFMA per SIMD
    case P_MFMA_FMA3: case P_MFMA_FMA4: case P_MFMA_EXP2: *threads = 512; *units = it * 4; break;   // MFMA per SIMD
    case P_FWD_INTER: case P_FWD_PPB: case P_FWD_DEP: case P_FWD_SKEW:
      *threads = 512; *units = 2 * (it / 32); break;                 // wave-tiles per SIMD
    default: *threads = 512; *units = 8 * it * 8 * 64 * 4; break;
  }
}

template <int KIND>
hipError_t launch_probe(int threads, long long* cycles, hipStream_t st) {
  hipLaunchKernelGGL(probe_kernel<KIND>, dim3(PROBE_GRID), dim3(threads), 0, st, cycles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_probe_kind(int kind, long long* cycles, int64_t* units, int* grid, hipStream_t st) {
  int threads;
  probe_shape(kind, &threads, units);
  *grid = PROBE_GRID;
  switch (kind) {
    case P_FMA: return launch_probe<P_FMA>(threads, cycles, st);
    case P_EXP: return launch_probe<P_EXP>(threads, cycles, st);
    case P_MED3: return launch_probe<P_MED3>(threads, cycles, st);
    case P_CVT_FP8: return launch_probe<P_CVT_FP8>(threads, cycles, st);
    case P_MAX3: return launch_probe<P_MAX3>(threads, cycles, st);
    case P_MFMA_BF16: return launch_probe<P_MFMA_BF16>(threads, cycles, st);
    case P_MFMA_FP8: return launch_probe<P_MFMA_FP8>(threads, cycles, st);
    case P_MFMA_FP4: return launch_probe<P_MFMA_FP4>(threads, cycles, st);
    case P_MFMA_AND_FMA: return launch_probe<P_MFMA_AND_FMA>(threads, cycles, st);
    case P_MFMA_AND_EXP: return launch_probe<P_MFMA_AND_EXP>(threads, cycles, st);
    case P_MIX2: return launch_probe<P_MIX2>(threads, cycles, st);
    case P_MIX4: return launch_probe<P_MIX4>(threads, cycles, st);
    case P_MIX8: return launch_probe<P_MIX8>(threads, cycles, st);
    case P_LDS_R128: return launch_probe<P_LDS_R128>(threads, cycles, st);
    case P_LDS_R64: return launch_probe<P_LDS_R64>(threads, cycles, st);
    case P_LDS_TR64: return launch_probe<P_LDS_TR64>(threads, cycles, st);
    case P_LDS_W128: return launch_probe<P_LDS_W128>(threads, cycles, st);
    case P_LDS_W32: return launch_probe<P_LDS_W32>(threads, cycles, st);
    case P_CVT_FP4: return launch_probe<P_CVT_FP4>(threads, cycles, st);
    case P_EXP_FMA: return launch_probe<P_EXP_FMA>(threads, cycles, st);
    case P_EXP_FMA3: return launch_probe<P_EXP_FMA3>(threads, cycles, st);
    case P_EXP_MAX3: return launch_probe<P_EXP_MAX3>(threads, cycles, st);
    case P_EXP_CVT_FP4: return launch_probe<P_EXP_CVT_FP4>(threads, cycles, st);
    case P_EXP_FMA_G4: return launch_probe<P_EXP_FMA_G4>(threads, cycles, st);
    case P_FMA_4W: return launch_probe<P_FMA_4W>(threads, cycles, st);
    case P_MIX8_4W: return launch_probe<P_MIX8_4W>(threads, cycles, st);
    case P_MIX16: return launch_probe<P_MIX16>(threads, cycles, st);
    case P_MFMA_FMA3: return launch_probe<P_MFMA_FMA3>(threads, cycles, st);
    case P_MFMA_FMA4: return launch_probe<P_MFMA_FMA4>(threads, cycles, st);
    case P_MFMA_EXP2: return launch_probe<P_MFMA_EXP2>(threads, cycles, st);
    case P_FWD_INTER: return launch_probe<P_FWD_INTER>(threads, cycles, st);
    case P_FWD_PPB: return launch_probe<P_FWD_PPB>(threads, cycles, st);
    case P_FWD_DEP: return launch_probe<P_FWD_DEP>(threads, cycles, st);
    case P_FWD_SKEW: return launch_probe<P_FWD_SKEW>(threads, cycles, st);
    default: return hipErrorInvalidValue;
  }
}

int probe_kind_count() { return P_COUNT; }

}  // namespace attn
