// Logits projection with a fused greedy argmax: z[b][i][v] = sum_{h,c} W[v][128 h + c] o[b][h][i][c]
// (W fp32, or bf16 widened exactly to fp32; fp32 products and accumulation either way).
//
// The round turns each attention output into a token by a greedy decision over logits ("VeriCache:
// making lossy KV compression exact", The Core Idea and Figure 1: the draft model's greedy token
// at every drafted position; the full-cache prediction that the accept step compares against).
// A single attention layer has no model head, so the logits are a fixed fp32 projection of the
// concatenated head outputs; this kernel is that projection, and for draft steps it also takes
// the argmax (lowest index on ties), so no logits round trip and no second launch are needed.
//
// Memory bound on W (V x Hq*128 fp32) for few rows (below TILED_MIN_ROWS; more rows take the tiled
// matrix-core form further down). Workgroup = 512 threads on VT = 8 vocabulary
// rows and MT = 8 output rows (grid.y covers more rows); thread t owns channels 4t .. 4t+3 of each
// 2048-channel chunk, so every W row is read with coalesced 16-byte loads, all VT rows of a chunk
// in flight at once and the next chunk's loads issued before this chunk's FMAs. The VT x MT dot
// products are reduced across the wave by recursive halving (each lane ends with one of the 64
// sums) and across the 8 waves through LDS. For the argmax each workgroup folds its best (value,
// index) per row into one 64-bit slot per row with an atomic max (the value in an order-preserving
// encoding above the complemented index, so the maximum is the largest value at its lowest index);
// the last workgroup of a row tile (ticket counter) reads the slots out and clears them.
#include "common.h"
#include "kernels.h"

namespace vc {

namespace {

constexpr int PT = 512;         // threads per workgroup
constexpr int PW = PT / 64;     // waves
constexpr int VT = 8;           // vocabulary rows per workgroup
constexpr int MT = 8;           // output rows per workgroup
constexpr int CHUNK = 4 * PT;   // channels per chunk
static_assert(PW == MT, "one wave per row in the final reduction");

struct PArgs {
  const void* W;        // [V][Dm], fp32 or bf16 (template parameter of the kernel)
  const float* o;       // [B][Hq][L][128]
  int V, Dm, Hq, L, M;  // M = B * L output rows, row m = (b, i) = (m / L, m % L)
  int nvt;              // vocabulary tiles (grid.x)
  float* z;             // [M][V] or null
  int32_t* idx;         // row (b, i) at idx[b * idx_b_stride + i], or null
  int64_t idx_b_stride;
  unsigned* counters;   // one per row tile (grid.y); zero between calls
  unsigned long long* slot;  // [M] packed (value, index) maxima; zero between calls
};

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// (value, index) as one unsigned 64-bit key ordered like better() for finite values: the float's
// bits mapped to an unsigned order (negative: all bits flipped; positive: sign bit set; -0 counts
// as +0) above 0xffffffff - index. Every key is nonzero, so zero marks an empty slot.
__device__ __forceinline__ unsigned long long argmax_key(float v, int i) {
  uint32_t u = __float_as_uint(v + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (0xffffffffu - (uint32_t)i);
}

// Four consecutive weights of a row as fp32: one 16-byte load (fp32 rows) or one 8-byte load
// widened exactly (bf16 rows).
template <bool WBF16>
__device__ __forceinline__ f32x4 load_w4(const void* row, int d) {
  if constexpr (WBF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(row) + d);
    return f32x4{bf16_bits_to_f32(u.x & 0xffffu), bf16_bits_to_f32(u.x >> 16),
                 bf16_bits_to_f32(u.y & 0xffffu), bf16_bits_to_f32(u.y >> 16)};
  } else {
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(row) + d);
  }
}

template <bool WBF16>
__global__ void __launch_bounds__(PT) project_kernel(PArgs a) {
  static_assert(VT * MT == 64, "one reduced value per lane");
  __shared__ float s_red[PW][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v0 = blockIdx.x * VT, m0 = blockIdx.y * MT;
  const int64_t wbytes = WBF16 ? 2 : 4;

  // Row pointers (rows past the end read the last row and are never written).
  const void* wrow[VT];
#pragma unroll
  for (int v = 0; v < VT; ++v)
    wrow[v] = static_cast<const char*>(a.W) + (int64_t)min(v0 + v, a.V - 1) * a.Dm * wbytes;
  int64_t orow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int mm = min(m0 + m, a.M - 1);
    const int b = mm / a.L, i = mm % a.L;
    orow[m] = ((int64_t)b * a.Hq * a.L + i) * 128;
  }
  // channel d = 128 h + c of row (b, i) is at o[orow + h * L * 128 + c]
  auto load_chunk = [&](int d0, f32x4* w, f32x4* x) {
    const int d = min(d0 + 4 * tid, a.Dm - 4);  // past the end: re-read, weighed by 0 below
    const int64_t od = (int64_t)(d >> 7) * a.L * 128 + (d & 127);
#pragma unroll
    for (int v = 0; v < VT; ++v) w[v] = load_w4<WBF16>(wrow[v], d);
#pragma unroll
    for (int m = 0; m < MT; ++m) x[m] = *reinterpret_cast<const f32x4*>(a.o + orow[m] + od);
  };

  float acc[VT * MT];
#pragma unroll
  for (int k = 0; k < VT * MT; ++k) acc[k] = 0.f;
  f32x4 w[VT], x[MT];
  load_chunk(0, w, x);
  for (int d0 = 0; d0 < a.Dm; d0 += CHUNK) {
    f32x4 wn[VT], xn[MT];
    if (d0 + CHUNK < a.Dm) load_chunk(d0 + CHUNK, wn, xn);
    const float live = d0 + 4 * tid < a.Dm ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < MT; ++m) x[m] *= live;
#pragma unroll
    for (int v = 0; v < VT; ++v)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float s = acc[v * MT + m];
        s = fmaf(w[v][0], x[m][0], s);
        s = fmaf(w[v][1], x[m][1], s);
        s = fmaf(w[v][2], x[m][2], s);
        s = fmaf(w[v][3], x[m][3], s);
        acc[v * MT + m] = s;
      }
    if (d0 + CHUNK < a.Dm) {
#pragma unroll
      for (int v = 0; v < VT; ++v) w[v] = wn[v];
#pragma unroll
      for (int m = 0; m < MT; ++m) x[m] = xn[m];
    }
  }

  wave_halve<32>(acc, lane);
  s_red[wave][lane] = acc[0];
  __syncthreads();
  __shared__ int s_last;
  if (wave == 0) {
    float zv = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < PW; ++w2) zv += s_red[w2][lane];
    const int v = v0 + lane / MT, m = m0 + lane % MT;  // lane = v_local * MT + m_local
    const bool ok = v < a.V && m < a.M;
    if (a.z && ok) a.z[(int64_t)m * a.V + v] = zv;
    if (a.idx) {
      // best (value, index) of this tile per row: lanes m_local + MT k
      float bv = ok ? zv : -INFINITY;
      int bi = ok ? v : 0x7fffffff;
#pragma unroll
      for (int off = MT; off < 64; off <<= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      // The device-scope atomic max has been performed (its old value returned) before the
      // ticket is taken; the last ticket holder reads the slots with device-coherent loads.
      // (Release / acquire fences would write back and invalidate the whole L2 instead, costing
      // microseconds per call.) One counter per row tile: a two-level ticket (group counters,
      // then a top counter) spreads the contention but adds a round trip, and measured ~0.8 us
      // slower per call at 256 vocabulary tiles.
      if (lane < MT && m < a.M && bi != 0x7fffffff) {
        const unsigned long long old = __hip_atomic_fetch_max(a.slot + m, argmax_key(bv, bi),
                                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("" ::"v"(old));  // use the returned value: wait for the atomic itself
      }
      if (lane == 0) {
        unsigned* cnt = a.counters + blockIdx.y;
        const int last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                         (unsigned)(a.nvt - 1);
        if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = last;
      }
    }
  }
  if (!a.idx) return;
  __syncthreads();
  if (!s_last) return;

  // Last workgroup of this row tile: thread t < MT reads row m0 + t's slot, clears it and writes
  // the index.
  const int row = m0 + tid;
  if (tid >= MT || row >= a.M) return;
  const unsigned long long key = __hip_atomic_load(a.slot + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(a.slot + row, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  a.idx[(int64_t)(row / a.L) * a.idx_b_stride + row % a.L] = (int32_t)(0xffffffffu - (uint32_t)key);
}

// ---------------------------------------------------------------------------------------------
// Many rows (the verify block's B*L rows): a tiled product on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: exact fp32 products, fp32 accumulation). Workgroup = 4 waves on TMT = 32
// output rows x TVT = 64 vocabulary rows; wave w owns vocabulary rows 16w .. 16w + 15 against all
// 32 output rows (two 16 x 16 tiles). K goes through two LDS slots in chunks of KC = 64 (the next
// chunk stored to one slot while the current one is multiplied from the other, the two after it in
// flight in registers). Within a group of four
// MFMA steps a lane of k-slot s takes the real channels 4s .. 4s + 3 of the group's 16 (the same
// remap for both operands), so each operand read is one 16-byte LDS load per four steps. The
// argmax (when asked for) goes through per-row slots (atomic max of the same 64-bit keys) and a
// row-tile ticket.
// ---------------------------------------------------------------------------------------------
constexpr int TMT = 32;
constexpr int TVT = 64;
constexpr int KC = 64;
constexpr int KCP = KC + 4;  // padded LDS row (floats)

template <bool WBF16>
__global__ void __launch_bounds__(256) project_tiled_kernel(PArgs a) {
  __shared__ __attribute__((aligned(16))) float s_a[2][TMT * KCP];  // two chunk slots
  __shared__ __attribute__((aligned(16))) float s_b[2][TVT * KCP];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * TMT, v0 = blockIdx.x * TVT;

  // staging: A rows (t / 8, two 16-byte pieces), B rows (t / 4, four 16-byte pieces)
  const int ar = tid >> 3, ap = tid & 7;
  const int am = min(m0 + ar, a.M - 1);
  const int64_t abase = ((int64_t)(am / a.L) * a.Hq * a.L + am % a.L) * 128;  // head 0 of row am
  const int br = tid >> 2, bp = tid & 3;
  const int64_t brow = (int64_t)min(v0 + br, a.V - 1) * a.Dm;
  // Staging ring: chunk k is multiplied from LDS slot k % 2 while chunk k + 1 is stored to the other
  // slot and the loads of chunks k + 2 .. k + NB - 1 are in flight in registers (a load past the
  // last chunk re-reads the last one, so every step issues the same loads and waits for exactly the
  // chunk it stores); one barrier per chunk.
  constexpr int NB = 4;
  const int nch = a.Dm / KC;
  f32x4 ra[NB][2], rb[NB][4];
  auto load = [&](int c, f32x4* qa, f32x4* qb) {
    const int k0 = min(c, nch - 1) * KC;
    const int64_t ao = abase + (int64_t)(k0 >> 7) * a.L * 128 + (k0 & 127);  // k0 % 64 == 0
#pragma unroll
    for (int z = 0; z < 2; ++z) qa[z] = *reinterpret_cast<const f32x4*>(a.o + ao + 4 * ap + 32 * z);
#pragma unroll
    for (int z = 0; z < 4; ++z) {
      const int64_t d = brow + k0 + 16 * bp + 4 * z;
      if constexpr (WBF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.W) + d);
        qb[z] = f32x4{bf16_bits_to_f32(u.x & 0xffffu), bf16_bits_to_f32(u.x >> 16),
                      bf16_bits_to_f32(u.y & 0xffffu), bf16_bits_to_f32(u.y >> 16)};
      } else {
        qb[z] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.W) + d);
      }
    }
  };
  auto store = [&](int slot, const f32x4* qa, const f32x4* qb) {
#pragma unroll
    for (int z = 0; z < 2; ++z) *reinterpret_cast<f32x4*>(s_a[slot] + ar * KCP + 4 * ap + 32 * z) = qa[z];
#pragma unroll
    for (int z = 0; z < 4; ++z) *reinterpret_cast<f32x4*>(s_b[slot] + br * KCP + 16 * bp + 4 * z) = qb[z];
  };

  const int i16 = lane & 15, ks = lane >> 4;
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int c = 0; c < NB - 1; ++c) load(c, ra[c], rb[c]);
  store(0, ra[0], rb[0]);
  __syncthreads();
  for (int c0 = 0; c0 < nch; c0 += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int k = c0 + u;
      load(k + NB - 1, ra[(u + NB - 1) % NB], rb[(u + NB - 1) % NB]);
      // chunk k + 1 into the other slot (last read by chunk k - 1, before the previous barrier;
      // past the end: unused)
      store((u + 1) % 2, ra[(u + 1) % NB], rb[(u + 1) % NB]);
      if (k < nch) {
        const float* sa = s_a[u % 2];
        const float* sb = s_b[u % 2];
#pragma unroll
        for (int g = 0; g < KC / 16; ++g) {
          const f32x4 bv = *reinterpret_cast<const f32x4*>(sb + (16 * wave + i16) * KCP + 16 * g + 4 * ks);
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(sa + (16 * r + i16) * KCP + 16 * g + 4 * ks);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], acc[r], 0, 0, 0);
          }
        }
      }
      __syncthreads();
    }
  }
  wait_vm<0>();  // the ring's last loads (past the end) have landed

  // lane holds C[m0 + 16 r + 4 ks + e][v0 + 16 wave + i16]
  const int v = v0 + 16 * wave + i16;
  if (a.z && v < a.V) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 16 * r + 4 * ks + e;
        if (m < a.M) a.z[(int64_t)m * a.V + v] = acc[r][e];
      }
  }
  if (!a.idx) return;
  // tile-local argmax per row through LDS (the staging space is free after the loop's last barrier)
  float* s_t = s_a[0];  // [TMT][TVT + 1]
  static_assert(TMT * (TVT + 1) <= TMT * KCP, "argmax staging");
  float* s_tt = s_a[0];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      s_tt[(16 * r + 4 * ks + e) * (TVT + 1) + 16 * wave + i16] = v < a.V ? acc[r][e] : -INFINITY;
  __syncthreads();
  if (tid < TMT) {
    const int m = m0 + tid;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int c = 0; c < TVT; ++c) {
      const float x = s_t[tid * (TVT + 1) + c];
      if (v0 + c < a.V && better(x, v0 + c, bv, bi)) { bv = x; bi = v0 + c; }
    }
    if (m < a.M && bi != 0x7fffffff) {
      const unsigned long long old = __hip_atomic_fetch_max(a.slot + m, argmax_key(bv, bi),
                                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("" ::"v"(old));  // the atomic has been performed before the ticket below
    }
  }
  __syncthreads();
  if (tid == 0) {
    unsigned* cnt = a.counters + blockIdx.y;
    const int last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     (unsigned)(a.nvt - 1);
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  const int row = m0 + tid;
  if (tid >= TMT || row >= a.M) return;
  const unsigned long long key = __hip_atomic_load(a.slot + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(a.slot + row, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  a.idx[(int64_t)(row / a.L) * a.idx_b_stride + row % a.L] = (int32_t)(0xffffffffu - (uint32_t)key);
}

}  // namespace

ProjectPlan plan_project(int M, int V) {
  ProjectPlan p;
  p.tiled = M >= TILED_MIN_ROWS;
  p.nvt = p.tiled ? (V + TVT - 1) / TVT : (V + VT - 1) / VT;
  p.nmt = p.tiled ? (M + TMT - 1) / TMT : (M + MT - 1) / MT;
  const size_t counters = ((size_t)p.nmt * sizeof(unsigned) + 255) & ~(size_t)255;
  p.counter_bytes = counters;
  p.ws_bytes = counters + (size_t)M * sizeof(unsigned long long);
  return p;
}

hipError_t launch_project(const void* W, int w_dtype, int V, const float* o, int B, int Hq, int L,
                          float* z, int32_t* idx, int64_t idx_b_stride, void* ws,
                          const ProjectPlan& plan, hipStream_t s) {
  PArgs a;
  a.W = W;
  a.o = o;
  a.V = V;
  a.Dm = Hq * 128;
  a.Hq = Hq;
  a.L = L;
  a.M = B * L;
  a.nvt = plan.nvt;
  a.z = z;
  a.idx = idx;
  a.idx_b_stride = idx_b_stride;
  a.counters = static_cast<unsigned*>(ws);
  a.slot = idx ? reinterpret_cast<unsigned long long*>(static_cast<uint8_t*>(ws) + plan.counter_bytes)
               : nullptr;
  if (plan.tiled) {
    if (w_dtype == VC_BF16)
      project_tiled_kernel<true><<<dim3(plan.nvt, plan.nmt), 256, 0, s>>>(a);
    else
      project_tiled_kernel<false><<<dim3(plan.nvt, plan.nmt), 256, 0, s>>>(a);
  } else if (w_dtype == VC_BF16) {
    project_kernel<true><<<dim3(plan.nvt, plan.nmt), PT, 0, s>>>(a);
  } else {
    project_kernel<false><<<dim3(plan.nvt, plan.nmt), PT, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace vc
