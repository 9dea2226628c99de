// Greedy accept: per-row argmax, first disagreement with the drafts, correction / bonus token.
//
// "VeriCache: making lossy KV compression exact", The Core Idea (the accept step, Figure 1 and
// the worked example): drafts are accepted left to right until the first one that differs from
// the full-cache prediction; the full-cache token is emitted there, or the extra prediction when
// every draft matches. Ties in the argmax go to the lowest token id.
//
// One workgroup of 1024 threads (16 waves) per batch row: wave w scans rows w, w+16, ... with
// 16-byte loads and a shuffle reduction of (value, index) pairs, then one thread walks the L
// argmax values to find the first disagreement. No atomics, no inter-workgroup traffic.
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
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool vec = (V % 4) == 0;
  for (int row = wave; row < L; row += WAVES) {
    const float* z = logits + ((int64_t)b * L + row) * V;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    if (vec) {
      // UNROLL 16-byte loads per lane in flight at a time (lanes past the row re-read its last
      // float4 and lose every comparison: an equal value at a higher index never wins)
      constexpr int UNROLL = 8;
      const float4* z4 = reinterpret_cast<const float4*>(z);
      const int n4 = V / 4;
      for (int i0 = 0; i0 < n4; i0 += 64 * UNROLL) {
        float4 t[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) t[u] = z4[min(i0 + 64 * u + lane, n4 - 1)];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int base = 4 * min(i0 + 64 * u + lane, n4 - 1);
          if (better(t[u].x, base + 0, bv, bi)) { bv = t[u].x; bi = base + 0; }
          if (better(t[u].y, base + 1, bv, bi)) { bv = t[u].y; bi = base + 1; }
          if (better(t[u].z, base + 2, bv, bi)) { bv = t[u].z; bi = base + 2; }
          if (better(t[u].w, base + 3, bv, bi)) { bv = t[u].w; bi = base + 3; }
        }
      }
    } else {
      for (int i = lane; i < V; i += 64) {
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
      s_arg[row] = bi;
      if (argmax_out) argmax_out[(int64_t)b * L + row] = bi;
    }
  }
  __syncthreads();
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
