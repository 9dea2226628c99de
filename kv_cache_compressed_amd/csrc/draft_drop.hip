// Draft attention over the kept positions of a token-dropping compressor.
//
// "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference", Key Contributions (token
// dropping drafters; the compressor interface exposes the dropped positions) and Limitations
// (identical drop counts for every layer/head); "VeriCache: making lossy KV compression exact",
// The Tradeoff VeriCache Is Trying to Escape (dropping keeps only part of the positions) and
// Verifying Without Giving Back the Speedup (drafting is bound by GPU memory bandwidth).
//
// Workgroup = 4 waves on one (b, kv head) and one range of the kept list; wave w takes every 4th
// block of 32 kept entries. Keys are gathered straight into the matrix-core row operand (each kept
// row is one contiguous 256-byte span: four 16-byte loads per lane); values are gathered into a
// per-wave LDS tile transposed to channel-major token pairs. QK^T and PV run on
// v_mfma_f32_16x16x32_bf16; columns j = 2h + hl carry query head h twice so that the PV product
// can take the softmax weight as a bf16 hi (hl = 0) + lo (hl = 1) pair without moving data across
// lanes. Split partials are merged by a small second kernel.
#include "common.h"
#include "kernels.h"

namespace vc {

namespace {

constexpr int WAVES = 4;
constexpr int THREADS = 64 * WAVES;
constexpr int BLK = 32;                 // kept entries per block
constexpr int VT_STRIDE = BLK / 2 + 4;  // dwords per transposed value row

struct DDArgs {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  const uint16_t* q;
  float* out;
  float* lse;
  float* part_o;
  float* part_ml;
  int64_t tok_cap, n_keep, idx_cap;
  int Hkv, Hq, G, splits;
  float qscale;
};

__global__ void __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(3, 3))) draft_drop_kernel(DDArgs a) {
  // per-wave transposed value tiles; reused for the cross-wave merge after the main loop
  __shared__ uint32_t s_raw[WAVES * D * VT_STRIDE];
  __shared__ float s_m[WAVES][8], s_l[WAVES][8];
  float(*s_o)[8][D] = reinterpret_cast<float(*)[8][D]>(s_raw);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, gq = lane >> 4;
  const int h = j >> 1, hl = j & 1;
  const bool active = h < a.G;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int hq = kvh * a.G + h;

  // Q^T operand (exact bf16): lane holds channels 32kb + 8gq + 0..7 of head h (both hl lanes).
  u32x4 qop[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    qop[kb] = active ? *reinterpret_cast<const u32x4*>(a.q + ((int64_t)b * a.Hq + hq) * D + 32 * kb + 8 * gq)
                     : u32x4{0u, 0u, 0u, 0u};

  const int64_t nblk = (a.n_keep + BLK - 1) / BLK;
  const int64_t blk_begin = nblk * split / a.splits, blk_end = nblk * (split + 1) / a.splits;
  const int32_t* ilist = a.idx + (int64_t)bh * a.idx_cap;
  const uint16_t* kbase = a.k + (int64_t)bh * a.tok_cap * D;
  const uint16_t* vbase = a.v + (int64_t)bh * a.tok_cap * D;
  uint32_t* vt = s_raw + wave * D * VT_STRIDE;

  float m_run = -INFINITY, l_lane = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Progress-based wave priority: every wave starts at the top level and steps down at 1/3, 2/3
  // and 5/6 of its share, so waves that started early yield to later ones and the waves of a CU
  // finish closer together.
  const int nmine = __builtin_amdgcn_readfirstlane(
      (int)(blk_begin + wave < blk_end ? (blk_end - blk_begin - wave + WAVES - 1) / WAVES : 0));
  const int q1 = nmine / 3, q2 = 2 * nmine / 3, q3 = 5 * nmine / 6;
  __builtin_amdgcn_s_setprio(3);
  int it = 0;
  for (int64_t blk = blk_begin + wave; blk < blk_end; blk += WAVES, ++it) {
    if (it == q1) __builtin_amdgcn_s_setprio(2);
    if (it == q2) __builtin_amdgcn_s_setprio(1);
    if (it == q3) __builtin_amdgcn_s_setprio(0);
    const int64_t e0 = blk * BLK;
    // ---- gather keys into the row operand: lane (token 16tb + j, quarter gq) ----------------
    u32x4 kop[2][4];
    bool valid[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int64_t e = e0 + 16 * tb + j;
      int32_t pos = (e < a.n_keep) ? ilist[e] : -1;
      valid[tb] = pos >= 0 && pos < a.tok_cap;
      const uint16_t* kr = kbase + (int64_t)(valid[tb] ? pos : 0) * D;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        kop[tb][kb] = valid[tb] ? *reinterpret_cast<const u32x4*>(kr + 32 * kb + 8 * gq)
                                : u32x4{0u, 0u, 0u, 0u};
    }
    // ---- gather values, transposed: lane (token pair tp = lane % 16, channel quarter cq) -----
    {
      const int tp = lane & 15, cq = lane >> 4;
      u32x4 v0[4], v1[4];
#pragma unroll
      for (int z = 0; z < 2; ++z) {
        const int64_t e = e0 + 2 * tp + z;
        const int32_t pos = (e < a.n_keep) ? ilist[e] : -1;
        const bool ok = pos >= 0 && pos < a.tok_cap;
        const uint16_t* vr = vbase + (int64_t)(ok ? pos : 0) * D + 32 * cq;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const u32x4 t = ok ? *reinterpret_cast<const u32x4*>(vr + 8 * w) : u32x4{0u, 0u, 0u, 0u};
          if (z == 0) v0[w] = t; else v1[w] = t;
        }
      }
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int zz = 0; zz < 4; ++zz) {
          const int c = 32 * cq + 8 * w + 2 * zz;
          vt[c * VT_STRIDE + tp] = __builtin_amdgcn_perm(v1[w][zz], v0[w][zz], 0x05040100u);
          vt[(c + 1) * VT_STRIDE + tp] = __builtin_amdgcn_perm(v1[w][zz], v0[w][zz], 0x07060302u);
        }
    }
    // ---- QK^T ------------------------------------------------------------------------------
    f32x4 s[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) c = mfma_bf16(kop[tb][kb], qop[kb], c);
      s[tb] = c;
    }
    // ---- online softmax (entry 16tb + 4gq + r of the block; invalid entries masked) ---------
    float sc[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t ent = e0 + 16 * (e >> 2) + 4 * gq + (e & 3);
      int32_t pos = (ent < a.n_keep) ? ilist[ent] : -1;
      const bool ok = pos >= 0 && pos < a.tok_cap;
      const float v = ok ? s[e >> 2][e & 3] * a.qscale : -INFINITY;
      sc[e] = v;
      mx = fmaxf(mx, v);
    }
    mx = max_over_rows(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    uint32_t pw[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float p0 = (m_new == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[e] - m_new);
      float p1 = (m_new == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[e + 1] - m_new);
      psum += p0 + p1;
      const float h0 = __uint_as_float(__float_as_uint(p0) & 0xffff0000u);
      const float h1 = __uint_as_float(__float_as_uint(p1) & 0xffff0000u);
      // hi lanes carry the truncated bf16 part, lo lanes the (truncated) remainder
      const float x0 = hl ? (p0 - h0) : h0;
      const float x1 = hl ? (p1 - h1) : h1;
      pw[e / 2] = (__float_as_uint(x0) >> 16) | (__float_as_uint(x1) & 0xffff0000u);
    }
    l_lane = l_lane * alpha + psum;
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] *= alpha;
    const u32x4 pop = active ? u32x4{pw[0], pw[1], pw[2], pw[3]} : u32x4{0u, 0u, 0u, 0u};
    // ---- PV (values from the wave's LDS tile; same wave wrote it, LDS is in order) ---------
    wave_lds_sync();  // the transposed writes of every lane come before the operand reads
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t* vr = vt + (16 * t + j) * VT_STRIDE;
      const u32x2 lo2 = *reinterpret_cast<const u32x2*>(vr + 2 * gq);
      const u32x2 hi2 = *reinterpret_cast<const u32x2*>(vr + 8 + 2 * gq);
      acc[t] = mfma_bf16(u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}, pop, acc[t]);
    }
    wave_lds_sync();  // operand reads finish before the next block overwrites the tile
  }

  __builtin_amdgcn_s_setprio(3);  // the partial stores end the workgroup's share
  // ---- wave result -> LDS (column 2h holds the hi sum, 2h+1 the lo sum) ---------------------
  const float l_tot = sum_over_rows(l_lane);
  __syncthreads();  // every wave is done with its value tile before s_o reuses the storage
  float osum[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) osum[t][r] = acc[t][r] + dpp_xor1(acc[t][r]);
  if (active && hl == 0) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_o[wave][h][16 * t + 4 * gq + r] = osum[t][r];
    if (gq == 0) {
      s_m[wave][h] = m_run * LN2;
      s_l[wave][h] = l_tot;
    }
  }
  __syncthreads();
  for (int id = tid; id < a.G * D; id += THREADS) {
    const int hh = id / D, c = id % D;
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
      if (s_l[w][hh] > 0.f) m = fmaxf(m, s_m[w][hh]);
    float o = 0.f, l = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        if (s_l[w][hh] > 0.f) {
          const float f = __expf(s_m[w][hh] - m);
          o += f * s_o[w][hh][c];
          l += f * s_l[w][hh];
        }
      }
    }
    const int64_t row = (int64_t)b * a.Hq + kvh * a.G + hh;
    a.part_o[(row * a.splits + split) * D + c] = o;
    if (c == 0) {
      a.part_ml[(row * a.splits + split) * 2 + 0] = m;
      a.part_ml[(row * a.splits + split) * 2 + 1] = l;
    }
  }

}

}  // namespace

DraftDropPlan plan_draft_drop(int B, int Hkv, int Hq, int64_t n_keep) {
  DraftDropPlan p;
  const int64_t units = (int64_t)B * Hkv;
  const int64_t nblk = (n_keep + BLK - 1) / BLK;
  int64_t s = std::max<int64_t>(1, 768 / units);  // one resident round at 3 workgroups per CU
  s = std::min<int64_t>(s, std::max<int64_t>(1, nblk / 8));
  p.splits = (int)std::max<int64_t>(1, s);
  p.ws_bytes = (size_t)B * Hq * p.splits * (D + 2) * sizeof(float);
  return p;
}

hipError_t launch_draft_drop(const void* k, const void* v, int kv_dtype, int B, int Hkv,
                             int64_t tok_cap, const int32_t* idx, int64_t n_keep, int64_t idx_cap,
                             const void* q, int Hq, float sm_scale, float* out, float* lse,
                             void* ws, const DraftDropPlan& plan, hipStream_t s) {
  (void)kv_dtype;  // VC_BF16 (validated by the caller)
  DDArgs a;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.idx = idx;
  a.q = static_cast<const uint16_t*>(q);
  a.out = out;
  a.lse = lse;
  const size_t rows = (size_t)B * Hq;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = a.part_o + rows * plan.splits * D;
  a.tok_cap = tok_cap;
  a.n_keep = n_keep;
  a.idx_cap = idx_cap;
  a.Hkv = Hkv;
  a.Hq = Hq;
  a.G = Hq / Hkv;
  a.splits = plan.splits;
  a.qscale = sm_scale * LOG2E;
  hipLaunchKernelGGL(draft_drop_kernel, dim3(plan.splits, (unsigned)(B * Hkv)), dim3(THREADS), 0,
                     s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_merge(a.part_o, a.part_ml, (int64_t)rows, plan.splits, out, lse, s);
}

}  // namespace vc
