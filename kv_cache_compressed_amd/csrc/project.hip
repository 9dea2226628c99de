// Logits projection with a fused greedy argmax: z[b][i][v] = sum_{h,c} W[v][128 h + c] o[b][h][i][c].
//
// The round turns each attention output into a token by a greedy decision over logits ("VeriCache:
// making lossy KV compression exact", The Core Idea and Figure 1: the draft model's greedy token
// at every drafted position; the full-cache prediction that the accept step compares against).
// A single attention layer has no model head, so the logits are a fixed fp32 projection of the
// concatenated head outputs; this kernel is that projection, and for draft steps it also takes
// the argmax (lowest index on ties), so no logits round trip and no second launch are needed.
//
// Memory bound on W (V x Hq*128 fp32) for few rows. Workgroup = 512 threads on VT = 8 vocabulary
// rows and MT = 8 output rows (grid.y covers more rows); thread t owns channels 4t .. 4t+3 of each
// 2048-channel chunk, so every W row is read with coalesced 16-byte loads, all VT rows of a chunk
// in flight at once and the next chunk's loads issued before this chunk's FMAs. The VT x MT dot
// products are reduced across the wave by recursive halving (each lane ends with one of the 64
// sums) and across the 8 waves through LDS. For the argmax each workgroup writes its best (value,
// index) per row; the last workgroup of a row tile (ticket counter) reduces them.
#include "common.h"
#include "kernels.h"

namespace vc {

namespace {

constexpr int PT = 512;         // threads per workgroup
constexpr int PW = PT / 64;     // waves
constexpr int VT = 8;           // vocabulary rows per workgroup
constexpr int MT = 8;           // output rows per workgroup
constexpr int CHUNK = 4 * PT;   // channels per chunk
constexpr int TG = 8;           // ticket groups per row tile
static_assert(PW == MT, "one wave per row in the final reduction");

struct PArgs {
  const float* W;       // [V][Dm]
  const float* o;       // [B][Hq][L][128]
  int V, Dm, Hq, L, M;  // M = B * L output rows, row m = (b, i) = (m / L, m % L)
  int nvt;              // vocabulary tiles (grid.x)
  float* z;             // [M][V] or null
  int32_t* idx;         // row (b, i) at idx[b * idx_b_stride + i], or null
  int64_t idx_b_stride;
  unsigned* counters;   // TG + 1 per row tile (grid.y); zero between calls
  float* part;          // [M][nvt][2]: (value, index bits) per vocabulary tile
};

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// Recursive-halving reduction of N values per lane across the 64 lanes of a wave: after the
// step of lane bit k, a lane keeps the half of its values selected by that bit, summed with the
// partner lane's copy of the same half; lane l ends with the wave total of value l (N == 64).
template <int S>
__device__ __forceinline__ void halve(float* r, int lane) {
  if constexpr (S >= 1) {
    const bool up = lane & S;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const float send = up ? r[i] : r[i + S];
      const float keep = up ? r[i + S] : r[i];
      r[i] = keep + __shfl_xor(send, S, 64);
    }
    halve<S / 2>(r, lane);
  }
}

__global__ void __launch_bounds__(PT) project_kernel(PArgs a) {
  static_assert(VT * MT == 64, "one reduced value per lane");
  __shared__ float s_red[PW][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v0 = blockIdx.x * VT, m0 = blockIdx.y * MT;

  // Row pointers (rows past the end read the last row and are never written).
  const float* wrow[VT];
#pragma unroll
  for (int v = 0; v < VT; ++v) wrow[v] = a.W + (int64_t)min(v0 + v, a.V - 1) * a.Dm;
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
    for (int v = 0; v < VT; ++v) w[v] = *reinterpret_cast<const f32x4*>(wrow[v] + d);
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

  halve<32>(acc, lane);
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
      // Candidates go out as device-coherent stores and have completed before the ticket is
      // taken; the last ticket holder reads them back with device-coherent loads. (Release /
      // acquire fences would write back and invalidate the whole L2 instead, costing
      // microseconds per call.) Two-level ticket: the tiles of a row tile count in TG group
      // counters (tile t in group t % TG), the last of each group in a top counter, so no
      // counter sees more than ~nvt/TG contending atomics.
      if (lane < MT && m < a.M) {
        float* p = a.part + ((int64_t)m * a.nvt + blockIdx.x) * 2;
        store_coherent(p, bv);
        store_coherent(p + 1, __int_as_float(bi));
      }
      wait_vm<0>();
      if (lane == 0) {
        unsigned* cnt = a.counters + blockIdx.y * (TG + 1);
        const int grp = blockIdx.x % TG, ngrp = min(TG, a.nvt);
        const unsigned in_grp = (unsigned)((a.nvt - grp + TG - 1) / TG);
        int last = 0;
        if (__hip_atomic_fetch_add(cnt + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == in_grp - 1) {
          __hip_atomic_store(cnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (__hip_atomic_fetch_add(cnt + TG, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(ngrp - 1)) {
            __hip_atomic_store(cnt + TG, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = 1;
          }
        }
        s_last = last;
      }
    }
  }
  if (!a.idx) return;
  __syncthreads();
  if (!s_last) return;

  // Last workgroup of this row tile: wave w reduces the candidates of row m0 + w (4 loads per
  // lane in flight per batch of 256 tiles).
  const int row = m0 + wave;
  if (row >= a.M) return;
  float cv = -INFINITY;
  int ci = 0x7fffffff;
  for (int t0 = 0; t0 < a.nvt; t0 += 256) {
    float2 pv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = min(t0 + lane + 64 * k, a.nvt - 1);  // past the end: re-read, no effect
      pv[k] = load_f32x2<true>(a.part + ((int64_t)row * a.nvt + t) * 2);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int pi = __float_as_int(pv[k].y);
      if (better(pv[k].x, pi, cv, ci)) { cv = pv[k].x; ci = pi; }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(cv, off, 64);
    const int oi = __shfl_xor(ci, off, 64);
    if (better(ov, oi, cv, ci)) { cv = ov; ci = oi; }
  }
  if (lane == 0) a.idx[(int64_t)(row / a.L) * a.idx_b_stride + row % a.L] = ci;
}

}  // namespace

ProjectPlan plan_project(int M, int V) {
  ProjectPlan p;
  p.nvt = (V + VT - 1) / VT;
  p.nmt = (M + MT - 1) / MT;
  const size_t counters = ((size_t)p.nmt * (TG + 1) * sizeof(unsigned) + 255) & ~(size_t)255;
  p.counter_bytes = counters;
  p.ws_bytes = counters + (size_t)M * p.nvt * 2 * sizeof(float);
  return p;
}

hipError_t launch_project(const float* W, int V, const float* o, int B, int Hq, int L, float* z,
                          int32_t* idx, int64_t idx_b_stride, void* ws, const ProjectPlan& plan,
                          hipStream_t s) {
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
  a.part = idx ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + plan.counter_bytes) : nullptr;
  project_kernel<<<dim3(plan.nvt, plan.nmt), PT, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace vc
