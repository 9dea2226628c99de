// Keep-list selection of a token-dropping drafter: for each (batch row, kv head) the ascending list
// of kept positions = the first `sinks` positions, the last `recent` ones, and the `take`
// highest-scoring positions of the middle (equal scores prefer the lower position).
//
// "VeriCache: making lossy KV compression exact", The Tradeoff VeriCache Is Trying to Escape
// (token-dropping compressors keep attention sinks and recent tokens, or score cached entries and
// evict the least useful); "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference", Key
// Contributions (the compressor interface exposes which positions are dropped) and Limitations
// (the same number of dropped tokens in every head).
//
// One workgroup of 1024 threads per row. Scores map to order-preserving 32-bit keys (NaN below
// every number, -0 equal to +0). A radix select over the middle finds the threshold key T and how
// many keys equal to T are taken (the lowest positions among them): three passes on 11, 11 and 10
// key bits, each a histogram over the keys that match the digits found so far (8 LDS copies of the
// 2048 bins, two waves per copy, to spread atomic conflicts) followed by a search from the top bin
// by wave 0. A last pass walks positions 0..n-1 in order, 16384 per step, and writes every kept
// position at its rank: one block-wide scan per step of packed (ties, other kept) counts gives
// each thread how many kept positions and ties precede it. Rows are re-read from L2 by every pass;
// float4 loads, eight in flight per thread in the histogram passes, the next step's four during a
// step of the last pass.
#include "common.h"
#include "kernels.h"

namespace vc {

namespace {

constexpr int ST = 1024;        // threads per workgroup
constexpr int SW = ST / 64;     // waves
constexpr int NB = 2048;        // bins of an 11-bit digit
constexpr int NSUB = 8;         // LDS histogram copies
constexpr int UNROLL = 8;       // float4 loads in flight per thread (histogram passes)

struct SArgs {
  const float* s;       // row r at s + r * s_stride
  int64_t s_stride;     // multiple of 4, >= n rounded up to a multiple of 4
  int32_t* idx;         // row r at idx + r * idx_stride
  int64_t idx_stride;
  int64_t n, lo, hi, take;  // middle [lo, hi), take <= hi - lo
  int64_t count;            // kept positions per row (= lo + n - hi + take); writes stay below it
};

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: below every number (no number maps to 0)
  if (u == 0x80000000u) u = 0u;                     // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// Workgroup barrier for LDS data: waits for this wave's LDS operations (lgkmcnt) but not for its
// outstanding global loads, so prefetched loads stay in flight across it (a fence would wait for
// them too). The memory clobbers keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Exclusive scan of one value per thread over the workgroup; `total` gets the sum. Two LDS
// barriers.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* s_w, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_w[wave] = incl;
  lds_barrier();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SW; ++w) {
    const uint32_t t = s_w[w];
    before += w < wave ? t : 0u;
    tot += t;
  }
  lds_barrier();  // s_w is rewritten by the next scan
  total = tot;
  return before + incl - x;
}

__global__ void __launch_bounds__(ST) select_keep_kernel(SArgs a) {
  __shared__ uint32_t hist[NSUB * NB];  // 64 KB
  __shared__ uint32_t s_w[SW];
  __shared__ uint32_t s_digit, s_above;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* row = a.s + (int64_t)blockIdx.x * a.s_stride;
  int32_t* out = a.idx + (int64_t)blockIdx.x * a.idx_stride;
  const int64_t lo = a.lo, hi = a.hi, m = hi - lo;

  // ---- threshold key T and the number r of keys equal to T that are taken ------------------
  uint32_t T;
  int64_t r;
  if (a.take == 0) {
    T = 0xffffffffu;  // above every key: nothing of the middle is kept
    r = 0;
  } else if (a.take >= m) {
    T = 0u;  // every number is above it and the NaNs tie at it, all taken
    r = m;
  } else {
    uint32_t prefix = 0u, mask = 0u;
    int64_t remaining = a.take;
    const int64_t a0 = lo & ~(int64_t)3;
    uint32_t* h = hist + (wave % NSUB) * NB;
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t dm = pass == 2 ? 0x3ffu : 0x7ffu;
      for (int i = tid; i < NSUB * NB; i += ST) hist[i] = 0u;
      __syncthreads();
      for (int64_t j0 = a0 + 4 * (int64_t)tid; j0 < hi; j0 += (int64_t)4 * ST * UNROLL) {
        float4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int64_t j = j0 + (int64_t)4 * ST * u;
          v[u] = j < hi ? load4(row + j) : float4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int64_t j = j0 + (int64_t)4 * ST * u;
          const float e4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t p = j + e;
            if (p < lo || p >= hi) continue;
            const uint32_t k = order_key(e4[e]);
            if ((k & mask) == prefix) atomicAdd(&h[(k >> shift) & dm], 1u);
          }
        }
      }
      __syncthreads();
      for (int b = tid; b < NB; b += ST) {  // bin b is owned by one thread: sum in place
        uint32_t c = 0u;
#pragma unroll
        for (int w = 0; w < NSUB; ++w) c += hist[w * NB + b];
        hist[b] = c;
      }
      __syncthreads();
      if (wave == 0) {
        // lane l owns bins 32 l .. 32 l + 31; find the digit d with
        // (count above d) < remaining <= (count above d) + count(d)
        uint32_t c[32];
        uint32_t sum = 0u;
#pragma unroll
        for (int b = 0; b < 32; ++b) {
          c[b] = hist[32 * lane + b];
          sum += c[b];
        }
        uint32_t incl = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t y = __shfl_up(incl, off, 64);
          if (lane >= off) incl += y;
        }
        const uint32_t total = __shfl(incl, 63, 64);
        int64_t above = (int64_t)(total - incl);  // candidates in bins of higher lanes
        if (above < remaining && remaining <= above + (int64_t)sum) {
          for (int b = 31; b >= 0; --b) {
            if (above + (int64_t)c[b] >= remaining) {
              s_digit = (uint32_t)(32 * lane + b);
              s_above = (uint32_t)above;
              break;
            }
            above += c[b];
          }
        }
      }
      __syncthreads();
      remaining -= (int64_t)s_above;
      prefix |= s_digit << shift;
      mask |= dm << shift;
      __syncthreads();  // s_digit / s_above are rewritten by the next pass
    }
    T = prefix;
    r = remaining;
  }

  // ---- positions 0..n-1 in order: keep, and write at the rank --------------------------------
  // Each step covers 16 ST positions, 16 consecutive ones per thread; the next step's loads are
  // issued before this step's scan (whose barriers wait for LDS only), so they stay in flight.
  constexpr int PT = 16;
  int64_t g_other = 0, g_ties = 0;  // kept non-tie positions and ties before this step
  float4 cur[PT / 4];
  auto load_step = [&](int64_t c0, float4* v) {
#pragma unroll
    for (int u = 0; u < PT / 4; ++u) {
      const int64_t p = c0 + (int64_t)PT * tid + 4 * u;
      v[u] = p < a.n ? load4(row + p) : float4{0.f, 0.f, 0.f, 0.f};
    }
  };
  load_step(0, cur);
  for (int64_t c0 = 0; c0 < a.n; c0 += (int64_t)PT * ST) {
    float4 nxt[PT / 4];
    if (c0 + (int64_t)PT * ST < a.n) load_step(c0 + (int64_t)PT * ST, nxt);
    const int64_t p0 = c0 + (int64_t)PT * tid;
    uint32_t kinds = 0u;  // 2 bits per position: 0 dropped, 1 kept, 2 tie at the threshold
    uint32_t nk = 0u, nt = 0u;
#pragma unroll
    for (int u = 0; u < PT / 4; ++u) {
      const float e4[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t p = p0 + 4 * u + e;
        uint32_t kd = 0u;
        if (p < a.n) {
          if (p < lo || p >= hi) {
            kd = 1u;
          } else {
            const uint32_t k = order_key(e4[e]);
            kd = k > T ? 1u : (k == T ? 2u : 0u);
          }
        }
        kinds |= kd << (2 * (4 * u + e));
        nk += kd == 1u;
        nt += kd == 2u;
      }
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((nt << 16) | nk, s_w, tot);  // counts <= 16384 per step
    int64_t ties_before = g_ties + (ex >> 16);
    int64_t base = g_other + (ex & 0xffffu) + (ties_before < r ? ties_before : r);
#pragma unroll
    for (int e = 0; e < PT; ++e) {
      const uint32_t kd = (kinds >> (2 * e)) & 3u;
      const bool take_it = kd == 1u || (kd == 2u && ties_before < r);
      if (take_it && base < a.count) out[base] = (int32_t)(p0 + e);
      base += take_it;
      ties_before += kd == 2u;
    }
    g_other += tot & 0xffffu;
    g_ties += tot >> 16;
#pragma unroll
    for (int u = 0; u < PT / 4; ++u) cur[u] = nxt[u];
  }
}

}  // namespace

hipError_t launch_select_keep(const float* scores, int64_t s_stride, int rows, int64_t n, int64_t lo,
                              int64_t hi, int64_t take, int32_t* idx, int64_t idx_stride,
                              hipStream_t s) {
  SArgs a;
  a.count = lo + (n - hi) + take;
  a.s = scores;
  a.s_stride = s_stride;
  a.idx = idx;
  a.idx_stride = idx_stride;
  a.n = n;
  a.lo = lo;
  a.hi = hi;
  a.take = take;
  select_keep_kernel<<<dim3((unsigned)rows), ST, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace vc
