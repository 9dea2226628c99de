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

// Elements i .. i+7 of a VC_F32 / VC_F16 / VC_BF16 array (i a multiple of 8, array 16-byte
// aligned), fetched with 16-byte loads as raw words (load8_raw) and converted to float later
// (cvt8), so the loads can be issued well ahead of their use.
struct Raw8 {
  u32x4 a, b;  // VC_F32: 8 floats; 16-bit types: a holds all 8
};
__device__ __forceinline__ Raw8 load8_raw(const void* p, int64_t i, int dtype) {
  // branch-free: a 16-bit type loads its 16 bytes twice
  const int esz = dtype == VC_F32 ? 4 : 2;
  const uint8_t* b = static_cast<const uint8_t*>(p) + i * esz;
  Raw8 r;
  r.a = *reinterpret_cast<const u32x4*>(b);
  r.b = *reinterpret_cast<const u32x4*>(b + (esz == 4 ? 16 : 0));
  return r;
}
// As load8_raw, but issued as inline assembly the compiler does not track: the caller must wait
// for it explicitly (s_waitcnt vmcnt) through raw8_wait_* before reading the registers. Lets a
// kernel keep these loads in flight across direct-to-LDS copies it waits for itself.
__device__ __forceinline__ Raw8 load8_raw_untracked(const void* p, int64_t i, int dtype) {
  const int esz = dtype == VC_F32 ? 4 : 2;
  const uint8_t* b = static_cast<const uint8_t*>(p) + i * esz;
  const uint8_t* b2 = b + (esz == 4 ? 16 : 0);
  Raw8 r;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r.a) : "v"(b) : "memory");
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r.b) : "v"(b2) : "memory");
  return r;
}

__device__ __forceinline__ void cvt8(const Raw8& r, int dtype, float* out) {
#pragma unroll
  for (int z = 0; z < 4; ++z) {
    if (dtype == VC_F32) {
      out[z] = __uint_as_float(r.a[z]);
      out[4 + z] = __uint_as_float(r.b[z]);
    } else if (dtype == VC_BF16) {
      out[2 * z] = bf16_bits_to_f32(r.a[z] & 0xffffu);
      out[2 * z + 1] = bf16_bits_to_f32(r.a[z] >> 16);
    } else {
      out[2 * z] = f16_bits_to_f32(r.a[z] & 0xffffu);
      out[2 * z + 1] = f16_bits_to_f32(r.a[z] >> 16);
    }
  }
}
__device__ __forceinline__ void load8_as_f32(const void* p, int64_t i, int dtype, float* out) {
  cvt8(load8_raw(p, i, dtype), dtype, out);
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

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Pack two floats into an f16x2 word, round to nearest even (one v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t{lo, hi}), half2_t));
}

// ---------------------------------------------------------------------------------------------
// mixed-precision FMAs (v_fma_mix*): f32 operands combined with fp16 halves of packed words,
// results written straight into fp16 halves. Word b holds an fp16 pair (lo, hi).
// ---------------------------------------------------------------------------------------------
// (fp16(a0 * b0.lo), fp16(a1 * b1.lo)) as one packed word
__device__ __forceinline__ uint32_t mix_mul_pair(float a0, uint32_t b0, float a1, uint32_t b1) {
  uint32_t d;  // the low half is written first, the high half second
  asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=&v"(d) : "v"(a0), "v"(b0));
  asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "+v"(d) : "v"(a1), "v"(b1));
  return d;
}
// (fp16(a0 * b0.lo - h.lo), fp16(a1 * b1.lo - h.hi)): the rounding remainders of mix_mul_pair
__device__ __forceinline__ uint32_t mix_rem_pair(float a0, uint32_t b0, float a1, uint32_t b1,
                                                 uint32_t h) {
  uint32_t d;
  asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel_hi:[0,1,1]" : "=&v"(d) : "v"(a0), "v"(b0), "v"(h));
  asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,1,1]"
      : "+v"(d) : "v"(a1), "v"(b1), "v"(h));
  return d;
}
// (fp16(a0 * w.lo), fp16(a1 * w.hi)) for a packed fp16 pair w
__device__ __forceinline__ uint32_t mix_mul2(float a0, float a1, uint32_t w) {
  uint32_t d;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=&v"(d) : "v"(a0), "v"(w));
  asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(d) : "v"(a1), "v"(w));
  return d;
}
// (fp16(a0 * w.lo - h.lo), fp16(a1 * w.hi - h.hi)): the rounding remainders of mix_mul2
__device__ __forceinline__ uint32_t mix_rem2(float a0, float a1, uint32_t w, uint32_t h) {
  uint32_t d;
  asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel_hi:[0,1,1]" : "=&v"(d) : "v"(a0), "v"(w), "v"(h));
  asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,1,1] op_sel_hi:[0,1,1]"
      : "+v"(d) : "v"(a1), "v"(w), "v"(h));
  return d;
}
// acc + a * b.hi
__device__ __forceinline__ float mix_fma_hi(float a, uint32_t b, float acc) {
  asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(acc) : "v"(a), "v"(b));
  return acc;
}

// ---------------------------------------------------------------------------------------------
// cross-lane helpers (wave64)
// ---------------------------------------------------------------------------------------------
// Value of the neighbouring lane within each lane pair (lane ^ 1) via DPP quad_perm [1,0,3,2].
__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

// Reductions over the four 16-lane rows that hold the same column (lanes l, l^16, l^32, l^48),
// with gfx950's row-swap permutes (no LDS round trip): permlane16_swap(x, x) returns x with odd and
// even rows exchanged between its two results, permlane32_swap likewise for the two wave halves.
__device__ __forceinline__ float max_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Recursive-halving reduction of S * 2 values per lane across the 64 lanes of a wave (S = 32: 64
// values): after the step of lane bit b (S = 2^b), a lane keeps the half of its values selected by
// that bit, summed with its partner's copy of the same half; lane l ends with the wave total of
// value l. No LDS: the bit-5 and bit-4 steps exchange whole registers between wave halves / odd
// and even rows (permlane32_swap / permlane16_swap: after swapping (r[i], r[i + S]) a lane holds
// its own and its partner's copy of the half it keeps, so one add finishes the step); the bit-3 ..
// bit-0 steps read the partner through DPP (row_mirror pairs lanes l and 15 - l, row_half_mirror
// l and 7 - l, quad permutes l ^ 2 and l ^ 1: each pair differs in the step's bit and agrees in
// the bits above it, which is all a halving step needs).
template <int S>
__device__ __forceinline__ void wave_halve(float* r, int lane) {
  if constexpr (S >= 16) {
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const auto p = S == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(r[i]), __float_as_uint(r[i + S]), false, false)
                             : __builtin_amdgcn_permlane16_swap(__float_as_uint(r[i]), __float_as_uint(r[i + S]), false, false);
      r[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
    wave_halve<S / 2>(r, lane);
  } else if constexpr (S >= 1) {
    constexpr int CTRL = S == 8 ? 0x140 : S == 4 ? 0x141 : S == 2 ? 0x4E : 0xB1;
    const bool up = lane & S;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const float send = up ? r[i] : r[i + S];
      const float keep = up ? r[i + S] : r[i];
      r[i] = keep + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), CTRL, 0xF, 0xF, false));
    }
    wave_halve<S / 2>(r, lane);
  }
}
__device__ __forceinline__ float wave_max(float x) {
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int m = 32; m >= 1; m >>= 1) x += shfl_xor(x, m);
  return x;
}

// Wait until at most N vector-memory operations of this wave are outstanding (s_waitcnt vmcnt).
// Direct-to-LDS copies count like loads and complete in order, so this is how a kernel knows
// which of its copies have landed; the memory clobbers keep the compiler from moving LDS reads
// across the wait (it does not track direct-to-LDS copies itself).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Direct global -> LDS copy (global_load_lds_dwordx4): lane l's 16 bytes from g land at
// lds + 16 l, where lds is the wave's common base. Completion is counted by vmcnt; the compiler
// does not order LDS reads after it, so callers wait explicitly. (The host pass of this file has
// no such instruction; the body exists for the device pass only.)
template <int AUX>
__device__ __forceinline__ void copy16_to_lds(const void* g, void* lds) {
#if __HIP_DEVICE_COMPILE__
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, AUX);
#endif
}

// Compiler-only ordering of this wave's LDS accesses: the hardware already runs one wave's LDS
// instructions in order, so a later read sees an earlier write of another lane of the same wave.
// (No fence: a fence would also wait for outstanding global loads and direct-to-LDS copies.)
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

// Order this wave's LDS writes before its following LDS reads of other lanes' data, with fences
// that also keep the compiler from moving memory operations (and wait for outstanding loads).
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
// Merge the S partials of one row; called by the 64 lanes of one wave, lane handles channels
// 2*lane, 2*lane+1. Writes out[row][D] (normalised) and lse[row] (if non-null). Lane s reads split
// s's (m, l), so every partial load of the row is in flight at once. COHERENT reads bypass the
// non-coherent caches (device-scope relaxed atomic loads), for partials written by other
// workgroups of the same kernel.
// ---------------------------------------------------------------------------------------------
// Device-scope store that writes through the non-coherent caches (read back by load_f32<true>).
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <bool COHERENT>
__device__ __forceinline__ float load_f32(const float* p) {
  if constexpr (COHERENT)
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}
template <bool COHERENT>
__device__ __forceinline__ float2 load_f32x2(const float* p) {
  if constexpr (COHERENT) {
    const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
  } else {
    return *reinterpret_cast<const float2*>(p);
  }
}

template <bool COHERENT>
__device__ __forceinline__ void merge_row_wave(const float* __restrict__ part_o,
                                              const float* __restrict__ part_ml, int S,
                                              float* __restrict__ out, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
  float o0 = 0.f, o1 = 0.f, l = 0.f;
  if (S <= 16) {
    // every load of the row in one round trip (splits past S re-read split S-1 and weigh 0)
    const float2 ml = load_f32x2<COHERENT>(part_ml + 2 * min(lane, S - 1));
    float2 po[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) po[s] = load_f32x2<COHERENT>(part_o + (int64_t)min(s, S - 1) * D + 2 * lane);
    const bool live = lane < S && ml.y > 0.f;
    m = wave_max(live ? ml.x : -INFINITY);
    const float w = (live && m != -INFINITY) ? __expf(ml.x - m) : 0.f;
    l = w * ml.y;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s));
      o0 += ws * po[s].x;
      o1 += ws * po[s].y;
    }
  } else {
  for (int s = lane; s < S; s += 64) {
    const float2 ml = load_f32x2<COHERENT>(part_ml + 2 * s);
    if (ml.y > 0.f) m = fmaxf(m, ml.x);
  }
  m = wave_max(m);
  if (m != -INFINITY) {
    for (int s0 = 0; s0 < S; s0 += 64) {
      // lane s0 + i holds split (s0 + i)'s weight; empty splits weigh 0 (their o is 0)
      float w = 0.f;
      if (s0 + lane < S) {
        const float2 ml = load_f32x2<COHERENT>(part_ml + 2 * (s0 + lane));
        if (ml.y > 0.f) {
          w = __expf(ml.x - m);
          l += w * ml.y;
        }
      }
      // sixteen splits per step, their loads in flight together; steps past the last split read
      // split S - 1 again with the weight 0 that lanes past S hold
      const int n = min(64, S - s0);
      for (int i = 0; i < n; i += 16) {
        float2 po[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          po[u] = load_f32x2<COHERENT>(part_o + (int64_t)min(s0 + i + u, S - 1) * D + 2 * lane);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), i + u));
          o0 += wi * po[u].x;
          o1 += wi * po[u].y;
        }
      }
    }
  }
  }
  l = wave_sum(l);
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
