// Device helpers shared by the libvc kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vc.h"

namespace vc {

typedef _Float16 f16;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;          // head dimension
constexpr int GROUP = 32;       // KIVI group size
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int COUNTER_BYTES = 4096;  // ticket counters at the head of a draft workspace

// ---------------------------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(f16, (uint16_t)b);
}
__device__ __forceinline__ uint16_t f16_bits(f16 h) { return __builtin_bit_cast(uint16_t, h); }

// Element i of a VC_F32 / VC_F16 / VC_BF16 array as float (exact).
__device__ __forceinline__ float load_as_f32(const void* p, int64_t i, int dtype) {
  if (dtype == VC_F32) return static_cast<const float*>(p)[i];
  const uint16_t b = static_cast<const uint16_t*>(p)[i];
  return dtype == VC_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

// Largest fp16 value <= x, as float.
__device__ __forceinline__ float f16_round_down(float x) {
  f16 h = (f16)x;  // round to nearest even
  if ((float)h > x) {
    uint16_t b = f16_bits(h);
    b = (b == 0x0000u) ? 0x8001u : ((b & 0x8000u) ? (uint16_t)(b + 1) : (uint16_t)(b - 1));
    h = __builtin_bit_cast(f16, b);
  }
  return (float)h;
}

// Smallest fp16 value >= x, as float.
__device__ __forceinline__ float f16_round_up(float x) {
  f16 h = (f16)x;
  if ((float)h < x) {
    uint16_t b = f16_bits(h);
    b = (b == 0x8000u) ? 0x0001u : ((b & 0x8000u) ? (uint16_t)(b - 1) : (uint16_t)(b + 1));
    h = __builtin_bit_cast(f16, b);
  }
  return (float)h;
}

// Pack two floats into an f16x2 word (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return (uint32_t)f16_bits((f16)lo) | ((uint32_t)f16_bits((f16)hi) << 16);
}

// ---------------------------------------------------------------------------------------------
// cross-lane helpers (wave64)
// ---------------------------------------------------------------------------------------------
// Value of the neighbouring lane within each lane pair (lane ^ 1) via DPP quad_perm [1,0,3,2].
__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

// Reductions over the four 16-lane rows that hold the same column (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float max_over_rows(float x) {
  x = fmaxf(x, shfl_xor(x, 16));
  return fmaxf(x, shfl_xor(x, 32));
}
__device__ __forceinline__ float sum_over_rows(float x) {
  x += shfl_xor(x, 16);
  return x + shfl_xor(x, 32);
}
__device__ __forceinline__ float wave_max(float x) {
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int m = 32; m >= 1; m >>= 1) x += shfl_xor(x, m);
  return x;
}

// Order this wave's LDS writes before its following LDS reads of other lanes' data (a wave's LDS
// instructions execute in order; the fences keep the compiler from moving memory operations).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// ---------------------------------------------------------------------------------------------
// matrix-core wrappers: D = A(16x32) * B(32x16) + C, fp32 accumulate.
// Lane l supplies A[l%16][8*(l/16)+e] and B[8*(l/16)+e][l%16] (e = 0..7) and holds
// D[4*(l/16)+r][l%16] (r = 0..3).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                               __builtin_bit_cast(half8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------------------------
// split partials and their log-sum-exp merge (natural-log units)
// part_o [rows][S][D], part_ml [rows][S][2] = (m, l)
// ---------------------------------------------------------------------------------------------
// Merge the S partials of one row; called by 64 lanes of one wave, lane handles channels
// 2*lane, 2*lane+1. Writes out[row][D] (normalised) and lse[row] (if non-null).
__device__ __forceinline__ void merge_row_wave(const float* __restrict__ part_o,
                                              const float* __restrict__ part_ml, int S,
                                              float* __restrict__ out, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
  for (int s = lane; s < S; s += 64) {
    const float ms = part_ml[2 * s], ls = part_ml[2 * s + 1];
    if (ls > 0.f) m = fmaxf(m, ms);
  }
  m = wave_max(m);
  float o0 = 0.f, o1 = 0.f, l = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float ls = part_ml[2 * s + 1];
      if (!(ls > 0.f)) continue;
      const float w = __expf(part_ml[2 * s] - m);
      const float2 po = reinterpret_cast<const float2*>(part_o + (int64_t)s * D)[lane];
      o0 += w * po.x;
      o1 += w * po.y;
      l += w * ls;
    }
  }
  float2 res;
  if (l > 0.f) {
    const float inv = 1.0f / l;
    res = make_float2(o0 * inv, o1 * inv);
  } else {
    res = make_float2(0.f, 0.f);
  }
  reinterpret_cast<float2*>(out)[lane] = res;
  if (lse && lane == 0) *lse = (l > 0.f) ? m + __logf(l) : -INFINITY;
}

}  // namespace vc
