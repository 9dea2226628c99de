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
// many keys equal to T are taken (the lowest positions among them), on 11, 11 and 10 key bits:
// the first digit from a histogram of the whole middle (8 LDS copies of the 2048 bins, two waves
// per copy, to spread atomic conflicts; wave 0 searches from the top bin); then the keys of the
// chosen bin (about 4% of a row of normal scores) are gathered into LDS, when they fit, and the two
// other digits come from histograms of those candidates alone (otherwise from two more passes
// over the row). A last pass walks positions 0..n-1 in order, 16384 per step, and writes every kept
// position at its rank: one block-wide scan per step of packed (ties, other kept) counts gives
// each thread how many kept positions and ties precede it; a thread's 16 positions that all lie in
// the middle skip the per-position range checks. float4 loads: eight in flight per thread in the
// row passes, the next step's four during a step of the last pass.
#include "common.h"
#include "kernels.h"

namespace vc {

namespace {

constexpr int ST = 1024;        // threads per workgroup
constexpr int SW = ST / 64;     // waves
constexpr int NB = 2048;        // bins of an 11-bit digit
constexpr int NSUB = 8;         // LDS histogram copies
constexpr int UNROLL = 8;       // float4 loads in flight per thread (row passes)
constexpr int PT = 16;          // positions per thread per step of the last pass
constexpr int CAND = 16384;     // candidate keys gathered in LDS

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

struct Shared {
  uint32_t hist[NSUB * NB];  // 64 KB
  uint32_t cand[CAND];       // 64 KB
  uint32_t s_w[SW];
  uint32_t digit, above, bin, ncand;
};

// After the histogram copies are filled: sum them into hist[0 .. NB) and let wave 0 find the digit
// d with (count above d) < remaining <= (count above d) + count(d) (lane l owns bins 32 l .. 32 l
// + 31). Leaves the digit, the count above it and the count in its bin in shared memory.
__device__ void find_digit(Shared& sh, int64_t remaining) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __syncthreads();
  for (int b = tid; b < NB; b += ST) {  // bin b is owned by one thread: sum in place
    uint32_t c = 0u;
#pragma unroll
    for (int w = 0; w < NSUB; ++w) c += sh.hist[w * NB + b];
    sh.hist[b] = c;
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t c[32];
    uint32_t sum = 0u;
#pragma unroll
    for (int b = 0; b < 32; ++b) {
      c[b] = sh.hist[32 * lane + b];
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
          sh.digit = (uint32_t)(32 * lane + b);
          sh.above = (uint32_t)above;
          sh.bin = c[b];
          break;
        }
        above += c[b];
      }
    }
  }
  __syncthreads();
}

__global__ void __launch_bounds__(ST) select_keep_kernel(SArgs a) {
  __shared__ Shared sh;
  const int tid = threadIdx.x, wave = tid >> 6;
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
    uint32_t* h = sh.hist + (wave % NSUB) * NB;
    const int m32 = (int)m;
    auto clear = [&]() {
      for (int i = tid; i < NSUB * NB; i += ST) sh.hist[i] = 0u;
      __syncthreads();
    };
    // f(key) for every middle position of the row, 4 positions per float4 group
    auto for_row = [&](auto f) {
      for (int64_t j0 = (lo & ~(int64_t)3) + 4 * (int64_t)tid; j0 < hi; j0 += (int64_t)4 * ST * UNROLL) {
        float4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int64_t j = j0 + (int64_t)4 * ST * u;
          v[u] = j < hi ? load4(row + j) : float4{0.f, 0.f, 0.f, 0.f};
        }
        // position j + e is in the middle iff (j + e - lo) as unsigned < hi - lo (32-bit: n < 2^31)
        const int rel0 = (int)(j0 - lo);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int rel = rel0 + 4 * ST * u;
          const float e4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) f(order_key(e4[e]), (unsigned)(rel + e) < (unsigned)m32);
        }
      }
    };
    auto take_digit = [&](int shift, uint32_t dm) {
      find_digit(sh, remaining);
      remaining -= (int64_t)sh.above;
      prefix |= sh.digit << shift;
      mask |= dm << shift;
    };
    // digit 1: bits 31..21 over the whole middle
    clear();
    for_row([&](uint32_t k, bool in) {
      if (in) atomicAdd(&h[k >> 21], 1u);
    });
    take_digit(21, 0x7ffu);
    const uint32_t nbin = sh.bin;  // keys that share the first digit: the candidates
    __syncthreads();               // every thread has read the digit before it is rewritten
    if (nbin <= (uint32_t)CAND) {
      // gather the candidates' keys into LDS (a slot per candidate from an LDS counter; their
      // order is irrelevant to the histograms)
      if (tid == 0) sh.ncand = 0u;
      __syncthreads();
      for_row([&](uint32_t k, bool in) {
        if (in && (k & mask) == prefix) {
          const uint32_t slot = atomicAdd(&sh.ncand, 1u);
          if (slot < (uint32_t)CAND) sh.cand[slot] = k;
        }
      });
      __syncthreads();
      const int nc = (int)min(sh.ncand, (uint32_t)CAND);
      // digits 2 (bits 20..10) and 3 (bits 9..0) over the candidates
      clear();
      for (int i = tid; i < nc; i += ST) {
        const uint32_t k = sh.cand[i];
        atomicAdd(&h[(k >> 10) & 0x7ffu], 1u);  // every candidate matches the first digit
      }
      take_digit(10, 0x7ffu);
      __syncthreads();
      clear();
      for (int i = tid; i < nc; i += ST) {
        const uint32_t k = sh.cand[i];
        if ((k & mask) == prefix) atomicAdd(&h[k & 0x3ffu], 1u);
      }
      take_digit(0, 0x3ffu);
    } else {
      // too many keys share the first digit: two more passes over the row
      clear();
      for_row([&](uint32_t k, bool in) {
        if (in && (k & mask) == prefix) atomicAdd(&h[(k >> 10) & 0x7ffu], 1u);
      });
      take_digit(10, 0x7ffu);
      __syncthreads();
      clear();
      for_row([&](uint32_t k, bool in) {
        if (in && (k & mask) == prefix) atomicAdd(&h[k & 0x3ffu], 1u);
      });
      take_digit(0, 0x3ffu);
    }
    T = prefix;
    r = remaining;
  }

  // ---- positions 0..n-1 in order: keep, and write at the rank --------------------------------
  // Each step covers 16 ST positions, 16 consecutive ones per thread; the next step's loads are
  // issued before this step's scan (whose barriers wait for LDS only), so they stay in flight.
  int g_other = 0, g_ties = 0;  // kept non-tie positions and ties before this step (< 2^31)
  const int rr = (int)r, cnt = (int)a.count;
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
    const bool inside = p0 >= lo && p0 + PT <= hi;  // all 16 positions in the middle (hi <= n)
    uint32_t kinds = 0u;  // 2 bits per position: 0 dropped, 1 kept, 2 tie at the threshold
    uint32_t nk = 0u, nt = 0u;
#pragma unroll
    for (int u = 0; u < PT / 4; ++u) {
      const float e4[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t kd;
        const uint32_t k = order_key(e4[e]);
        const uint32_t by_key = k > T ? 1u : (k == T ? 2u : 0u);
        if (inside) {
          kd = by_key;
        } else {
          const int64_t p = p0 + 4 * u + e;
          kd = p >= a.n ? 0u : ((p < lo || p >= hi) ? 1u : by_key);
        }
        kinds |= kd << (2 * (4 * u + e));
        nk += kd == 1u;
        nt += kd == 2u;
      }
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((nt << 16) | nk, sh.s_w, tot);  // counts <= 16384 per step
    int ties_before = g_ties + (int)(ex >> 16);
    int base = g_other + (int)(ex & 0xffffu) + (ties_before < rr ? ties_before : rr);
    const int q0 = (int)p0;  // positions are below n < 2^31
#pragma unroll
    for (int e = 0; e < PT; ++e) {
      const uint32_t kd = (kinds >> (2 * e)) & 3u;
      const bool take_it = kd == 1u || (kd == 2u && ties_before < rr);
      if (take_it && base < cnt) out[base] = q0 + e;
      base += take_it;
      ties_before += kd == 2u;
    }
    g_other += (int)(tot & 0xffffu);
    g_ties += (int)(tot >> 16);
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
