// Greedy accept: per-row argmax, first disagreement with the drafts, correction / bonus token.
//
// "VeriCache: making lossy KV compression exact", The Core Idea (the accept step, Figure 1 and
// the worked example): drafts are accepted left to right until the first one that differs from
// the full-cache prediction; the full-cache token is emitted there, or the extra prediction when
// every draft matches. Ties in the argmax go to the lowest token id.
//
// One workgroup of 1024 threads (16 waves) per batch row: the L rows one after the other, each
// scanned by all 16 waves (a slice each) with 16-byte loads, a shuffle reduction of (value, index)
// pairs per wave and an LDS reduction over the waves; then one thread walks the L argmax values to
// find the first disagreement. No atomics, no inter-workgroup traffic.
#include "common.h"
#include "kernels.h"

namespace vc {

namespace {

constexpr int WAVES = 16;
constexpr int MAX_L = 64;

// (a_val, a_idx) beats (b_val, b_idx): larger value, or equal value with lower index.
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

__global__ void __launch_bounds__(1024) accept_kernel(const float* __restrict__ logits,
                                                      const int32_t* __restrict__ drafts, int L,
                                                      int V, int32_t* __restrict__ accept_len,
                                                      int32_t* __restrict__ next_token,
                                                      int32_t* __restrict__ argmax_out) {
  __shared__ int s_arg[MAX_L];
  __shared__ float s_bv[WAVES];
  __shared__ int s_bi[WAVES];
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool vec = (V % 4) == 0;
  // Rows one after the other, each spread over all 16 waves (wave w scans a 1/16 slice of the
  // row), so a single row (a greedy step) still has 1024 threads' loads in flight.
  for (int row = 0; row < L; ++row) {
    const float* z = logits + ((int64_t)b * L + row) * V;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    if (vec) {
      // UNROLL 16-byte loads per lane in flight at a time (lanes past the slice re-read its last
      // float4 and lose every comparison: an equal value at a higher index never wins)
      constexpr int UNROLL = 4;
      const float4* z4 = reinterpret_cast<const float4*>(z);
      const int n4 = V / 4;
      const int per = (n4 + WAVES - 1) / WAVES;
      const int s0 = min(wave * per, n4), s1 = min(s0 + per, n4);
      for (int i0 = s0; i0 < s1; i0 += 64 * UNROLL) {
        float4 t[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) t[u] = z4[min(i0 + 64 * u + lane, s1 - 1)];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int base = 4 * min(i0 + 64 * u + lane, s1 - 1);
          if (better(t[u].x, base + 0, bv, bi)) { bv = t[u].x; bi = base + 0; }
          if (better(t[u].y, base + 1, bv, bi)) { bv = t[u].y; bi = base + 1; }
          if (better(t[u].z, base + 2, bv, bi)) { bv = t[u].z; bi = base + 2; }
          if (better(t[u].w, base + 3, bv, bi)) { bv = t[u].w; bi = base + 3; }
        }
      }
    } else {
      for (int i = threadIdx.x; i < V; i += 64 * WAVES) {
        const float t = z[i];
        if (better(t, i, bv, bi)) { bv = t; bi = i; }
      }
    }
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const int oi = __shfl_xor(bi, m, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) {
      s_bv[wave] = bv;
      s_bi[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float v = s_bv[0];
      int ix = s_bi[0];
      for (int w = 1; w < WAVES; ++w)
        if (better(s_bv[w], s_bi[w], v, ix)) { v = s_bv[w]; ix = s_bi[w]; }
      s_arg[row] = ix;
      if (argmax_out) argmax_out[(int64_t)b * L + row] = ix;
    }
    __syncthreads();  // s_bv / s_bi are reused by the next row
  }
  if (threadIdx.x == 0) {
    int a = L - 1;
    for (int i = 0; i < L - 1; ++i) {
      if (drafts[(int64_t)b * (L - 1) + i] != s_arg[i]) {
        a = i;
        break;
      }
    }
    accept_len[b] = a;
    next_token[b] = s_arg[a];
  }
}

__global__ void __launch_bounds__(256) merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    int64_t rows, int S, float* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  merge_row_wave<false>(part_o + row * S * D, part_ml + row * S * 2, S, out + row * D,
                 lse ? lse + row : nullptr);
}

}  // namespace

hipError_t launch_accept(const float* logits, const int32_t* drafts, int B, int L, int V,
                         int32_t* accept_len, int32_t* next_token, int32_t* argmax, hipStream_t s) {
  hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(1024), 0, s, logits, drafts, L, V, accept_len,
                     next_token, argmax);
  return hipGetLastError();
}

hipError_t launch_merge(const float* part_o, const float* part_ml, int64_t rows, int S, float* out,
                        float* lse, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, part_o,
                     part_ml, rows, S, out, lse);
  return hipGetLastError();
}

}  // namespace vc
