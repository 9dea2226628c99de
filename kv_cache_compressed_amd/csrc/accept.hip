// Greedy accept: per-row argmax, first disagreement with the drafts, correction / bonus token.
//
// "VeriCache: making lossy KV compression exact", The Core Idea (the accept step, Figure 1 and
// the worked example): drafts are accepted left to right until the first one that differs from
// the full-cache prediction; the full-cache token is emitted there, or the extra prediction when
// every draft matches. Ties in the argmax go to the lowest token id.
//
// One workgroup of 1024 threads (16 waves) per batch row. The waves are dealt over the L rows so
// that all 16 keep loads in flight whatever L is: WPR = 16 / L waves per row (a power of two, at
// least 1), each scanning a slice of its row with 16-byte loads, rows taken 16 / WPR at a time; a
// shuffle reduction of (value, index) pairs per wave and an LDS reduction over a row's waves give
// its argmax; then one thread walks the L argmax values to find the first disagreement. No
// atomics, no inter-workgroup traffic.
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
  int wpr = WAVES;  // waves per row: the largest power of two with wpr * L <= WAVES, at least 1
  while (wpr > 1 && wpr * L > WAVES) wpr >>= 1;
  const int conc = WAVES / wpr;  // rows in flight at a time
  const int sub = wave % wpr;
  for (int r0 = 0; r0 < L; r0 += conc) {
    const int row = r0 + wave / wpr;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    if (row < L) {
      const float* z = logits + ((int64_t)b * L + row) * V;
      if (vec) {
        // UNROLL 16-byte loads per lane in flight at a time (lanes past the slice re-read its
        // last float4 and lose every comparison: an equal value at a higher index never wins)
        constexpr int UNROLL = 8;
        const float4* z4 = reinterpret_cast<const float4*>(z);
        const int n4 = V / 4;
        const int per = (n4 + wpr - 1) / wpr;
        const int s0 = min(sub * per, n4), s1 = min(s0 + per, n4);
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
        for (int i = sub * 64 + lane; i < V; i += 64 * wpr) {
          const float t = z[i];
          if (better(t, i, bv, bi)) { bv = t; bi = i; }
        }
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
    if (lane == 0 && sub == 0 && row < L) {  // the row's first wave combines its wpr waves
      float v = s_bv[wave];
      int ix = s_bi[wave];
      for (int w = wave + 1; w < wave + wpr; ++w)
        if (better(s_bv[w], s_bi[w], v, ix)) { v = s_bv[w]; ix = s_bi[w]; }
      s_arg[row] = ix;
      if (argmax_out) argmax_out[(int64_t)b * L + row] = ix;
    }
    __syncthreads();  // s_bv / s_bi are reused by the next rows; s_arg complete after the last
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

// Top-2 margin of each logits row: gap[r] = z_best - z_second over distinct indices (0 when the
// best value occurs twice). One 256-thread workgroup per row.
__global__ void __launch_bounds__(256) margin_kernel(const float* __restrict__ logits, int V,
                                                     float* __restrict__ gap) {
  __shared__ float s1[4], s2[4];
  const float* z = logits + (int64_t)blockIdx.x * V;
  float b1 = -INFINITY, b2 = -INFINITY;  // best and second best of this thread's elements
  for (int i = threadIdx.x; i < V; i += 256) {
    const float t = z[i];
    if (t > b1) {
      b2 = b1;
      b1 = t;
    } else if (t > b2) {
      b2 = t;
    }
  }
  auto merge = [](float& a1, float& a2, float c1, float c2) {
    const float hi = fmaxf(a1, c1), lo = fminf(a1, c1);
    a1 = hi;
    a2 = fmaxf(lo, fmaxf(a2, c2));
  };
  for (int m = 32; m >= 1; m >>= 1) {
    const float c1 = __shfl_xor(b1, m, 64), c2 = __shfl_xor(b2, m, 64);
    merge(b1, b2, c1, c2);
  }
  if ((threadIdx.x & 63) == 0) {
    s1[threadIdx.x >> 6] = b1;
    s2[threadIdx.x >> 6] = b2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float a1 = s1[0], a2 = s2[0];
    for (int w = 1; w < 4; ++w) merge(a1, a2, s1[w], s2[w]);
    gap[blockIdx.x] = V > 1 ? a1 - a2 : INFINITY;
  }
}

// Plain streaming read of n16 16-byte words (the HBM read ceiling a bandwidth-bound kernel is
// compared with): workgroups stride over the buffer with four 16-byte loads per thread in flight,
// fold what they read with XOR and write one word per thread, so no load can be dropped.
__global__ void __launch_bounds__(256) read_stream_kernel(const uint4* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
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

hipError_t launch_margins(const float* logits, int64_t rows, int V, float* gap, hipStream_t s) {
  hipLaunchKernelGGL(margin_kernel, dim3((unsigned)rows), dim3(256), 0, s, logits, V, gap);
  return hipGetLastError();
}

hipError_t launch_read_stream(const void* src, int64_t n16, uint32_t* sink, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const uint4*>(src), n16, sink);
  return hipGetLastError();
}

hipError_t launch_merge(const float* part_o, const float* part_ml, int64_t rows, int S, float* out,
                        float* lse, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, part_o,
                     part_ml, rows, S, out, lse);
  return hipGetLastError();
}

}  // namespace vc
