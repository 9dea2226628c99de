// Draft attention over the KIVI cache: one query per (b, query head), keys/values dequantised on
// the fly from packed 2/4-bit codes, plus the full-precision residual.
//
// "VeriCache: making lossy KV compression exact", The Core Idea (the drafter decodes each token
// over the compressed cache) and Verifying Without Giving Back the Speedup (drafting is bound by
// GPU memory bandwidth); "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference", Key
// Contributions (drafting reads the compressed KV from HBM).
//
// Algebra. Keys are quantised per channel over 32-token groups, so for a group g
//   q.k_t = sum_c (q_c s_gc) code_tc + sum_c q_c m_gc
// and values per token over 32-channel groups, so for channel c in channel group cg
//   sum_t p_t v_tc = sum_t (p_t s_tcg) code_tc + sum_t p_t m_tcg.
// Both code sums run on the matrix cores (v_mfma_f32_16x16x32_f16): a 2/4-bit code is turned into
// an exact fp16 operand by masking it into the mantissa of a half (a subnormal equal to
// code * 4^p * 2^-24 for the slot position p), which costs one AND per two codes; the power of
// four of the slot position is divided out of the other operand. The other operand (q_c s_gc in
// the QK product, p_t s_tcg in the PV product) is prepared once per 32-token group. q s is carried
// as an fp16 hi + lo pair in two matrix columns so that the scores keep ~22 significant bits; p s
// is carried as one fp16 (11 bits) since the softmax weights enter the output linearly.
//
// Work split. Workgroup = 4 waves on one (b, kv head) and one contiguous range of groups (a
// split); wave w takes every 4th group of the range. Lane l of a wave is (column j = l % 16,
// row block gq = l / 16); column j = 2h + hl carries query head h (hl = 0: hi part, 1: lo part),
// so up to 8 query heads share each code load. The scores of a 16-token tile come back in the
// layout the PV product needs as its B operand, so softmax weights never cross lanes. The
// residual tokens (n_q .. n_q+r-1, fp16/fp32 ring) form one extra split computed on the vector
// ALUs. Each split writes an unnormalised partial (o, m, l); the last split of a (b, kv head) to
// finish (ticket counter) merges them with log-sum-exp and writes the output.
#include "common.h"
#include "kernels.h"

namespace vc {

namespace {

constexpr int WAVES = 4;
constexpr int THREADS = 64 * WAVES;
constexpr int RES_MAX = 512;           // residual ring slots handled by the residual split
constexpr float SCALE_QK = 256.0f;     // 2^8: magnitude headroom of the fp16 QK operand
constexpr float SCALE_PV = 256.0f;     // 2^8: same for the PV operand
constexpr float SUBNORMAL = 16777216.0f;  // 2^24: one fp16 subnormal step is 2^-24

struct DQArgs {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const void* k_meta;
  const void* v_meta;
  const void* k_res;
  const void* v_res;
  const void* q;
  float* out;
  float* lse;
  float* part_o;
  float* part_ml;
  unsigned* counters;
  int64_t tok_cap, n_q;
  int r, res_cap, res_dtype, q_dtype;
  int Hkv, Hq, G;
  int ngroups, splits, total_splits;
  float qscale;  // sm_scale * log2(e): scores are kept in log2 units inside the kernel
};

// Reciprocal of the slot-position power carried by unpacked element e of an operand.
template <int BITS>
__device__ __forceinline__ constexpr float cls_inv(int e) {
  return BITS == 2 ? (e < 2 ? 1.f : e < 4 ? 0.25f : e < 6 ? 0.0625f : 0.015625f)
                   : (((e >> 1) & 1) ? 0.0625f : 1.f);
}

// Codes of one operand (8 elements, 4 f16x2 words) from a packed word.
__device__ __forceinline__ u32x4 unpack2(uint32_t w, int hb) {
  const uint32_t x = hb ? (w >> 8) : w;
  return u32x4{x & 0x00030003u, x & 0x000C000Cu, x & 0x00300030u, x & 0x00C000C0u};
}
__device__ __forceinline__ u32x4 unpack4(uint32_t w) {
  const uint32_t x = w >> 8;
  return u32x4{w & 0x000F000Fu, w & 0x00F000F0u, x & 0x000F000Fu, x & 0x00F000F0u};
}

// (scale, min) of key channel c of group g.
template <bool META_F16>
__device__ __forceinline__ float2 kmeta(const void* base, int64_t idx) {
  if (META_F16) {
    const uint32_t w = static_cast<const uint32_t*>(base)[idx];
    return make_float2(f16_bits_to_f32(w & 0xffffu), f16_bits_to_f32(w >> 16));
  }
  return static_cast<const float2*>(base)[idx];
}

template <int BITS, bool META_F16>
__device__ void quant_split(const DQArgs& a, int bh, int split, float* smem) {
  constexpr int WPL = 2 * BITS;        // packed words per lane per block
  constexpr int ROW_BYTES = D * BITS / 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, gq = lane >> 4;
  const int h = j >> 1, hl = j & 1;
  const bool active = h < a.G;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int hq = kvh * a.G + h;

  // Query values of this lane's 32 channels (c = 32 kb + 8 gq + e), pre-scaled to log2 units.
  float qb[32];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 32 * kb + 8 * gq + e;
      qb[kb * 8 + e] = active ? load_as_f32(a.q, ((int64_t)b * a.Hq + hq) * D + c, a.q_dtype) * a.qscale : 0.f;
    }
  const float mk = hl ? 1.f : 0.f;  // lo lanes subtract the hi part

  const int g_begin = (int)((int64_t)a.ngroups * split / a.splits);
  const int g_end = (int)((int64_t)a.ngroups * (split + 1) / a.splits);
  const int64_t ngcap = a.tok_cap / GROUP;

  float m_run = -INFINITY, l_lane = 0.f;
  float bv[4] = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int g = g_begin + wave; g < g_end; g += WAVES) {
    const int64_t blk = (int64_t)bh * a.tok_cap + (int64_t)g * GROUP;
    // ---- loads --------------------------------------------------------------------------
    const u32x4* kp = reinterpret_cast<const u32x4*>(a.k_codes + blk * ROW_BYTES) + lane * (WPL / 4);
    const u32x4* vp = reinterpret_cast<const u32x4*>(a.v_codes + blk * ROW_BYTES) + lane * (WPL / 4);
    uint32_t kw[WPL], vw[WPL];
#pragma unroll
    for (int u = 0; u < WPL / 4; ++u) {
      const u32x4 tk = __builtin_nontemporal_load(kp + u);
      const u32x4 tv = __builtin_nontemporal_load(vp + u);
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        kw[4 * u + z] = tk[z];
        vw[4 * u + z] = tv[z];
      }
    }
    // ---- QK operand: q_c * s_gc as hi/lo fp16, and the bias sum_c q_c m_gc ----------------
    u32x4 bq[4];
    float bias = 0.f;
    const int64_t kmb = ((int64_t)bh * ngcap + g) * D;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float vals[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 sm = kmeta<META_F16>(a.k_meta, kmb + 32 * kb + 8 * gq + e);
        const float qt = qb[kb * 8 + e] * sm.x * (SCALE_QK * cls_inv<BITS>(e));
        const float hi = (float)(f16)qt;
        vals[e] = qt - mk * hi;
        bias += qb[kb * 8 + e] * sm.y;
      }
      bq[kb] = u32x4{pack_f16x2(vals[0], vals[1]), pack_f16x2(vals[2], vals[3]),
                     pack_f16x2(vals[4], vals[5]), pack_f16x2(vals[6], vals[7])};
    }
    bias = sum_over_rows(bias);
    // ---- QK on the matrix cores: two 16-token tiles x four 32-channel blocks -----------
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const u32x4 av = BITS == 2 ? unpack2(kw[2 * tb + kb / 2], kb & 1) : unpack4(kw[4 * tb + kb]);
        s[tb] = mfma_f16(av, bq[kb], s[tb]);
      }
    // ---- scores (log2 units) and online softmax ------------------------------------------
    float sc[8];
    float mx = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float raw = s[tb][r] + dpp_xor1(s[tb][r]);  // hi column + lo column
        const float v = raw * (SUBNORMAL / SCALE_QK) + bias;
        sc[tb * 4 + r] = v;
        mx = fmaxf(mx, v);
      }
    mx = max_over_rows(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sc[e] = exp2f(sc[e] - m_new);
      psum += sc[e];
    }
    l_lane = l_lane * alpha + psum;
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] *= alpha;
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) bv[cg] *= alpha;
    // ---- PV operand: p_t * s_tcg (fp16, hi columns only) and the bias sum_t p_t m_tcg ----
    // Element e of this lane's B operand is token 16*(e/4) + 4*gq + e%4 = sc[e]'s token.
    u32x4 bp[4];
    {
      float pv[4][8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = 16 * (e >> 2) + 4 * gq + (e & 3);
        const int64_t vmi = (blk + tok) * 4;
        float svals[4], mvals[4];
        if (META_F16) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint32_t*>(a.v_meta) + vmi);
#pragma unroll
          for (int cg = 0; cg < 4; ++cg) {
            svals[cg] = f16_bits_to_f32(w[cg] & 0xffffu);
            mvals[cg] = f16_bits_to_f32(w[cg] >> 16);
          }
        } else {
          const float4* p4 = reinterpret_cast<const float4*>(static_cast<const float2*>(a.v_meta) + vmi);
          const float4 w0 = p4[0], w1 = p4[1];
          svals[0] = w0.x; mvals[0] = w0.y; svals[1] = w0.z; mvals[1] = w0.w;
          svals[2] = w1.x; mvals[2] = w1.y; svals[3] = w1.z; mvals[3] = w1.w;
        }
        const float pe = (hl == 0 && active) ? sc[e] : 0.f;
#pragma unroll
        for (int cg = 0; cg < 4; ++cg) {
          pv[cg][e] = pe * svals[cg] * (SCALE_PV * cls_inv<BITS>(e));
          bv[cg] += pe * mvals[cg];
        }
      }
#pragma unroll
      for (int cg = 0; cg < 4; ++cg)
        bp[cg] = u32x4{pack_f16x2(pv[cg][0], pv[cg][1]), pack_f16x2(pv[cg][2], pv[cg][3]),
                       pack_f16x2(pv[cg][4], pv[cg][5]), pack_f16x2(pv[cg][6], pv[cg][7])};
    }
    // ---- PV on the matrix cores: eight 16-channel tiles, K = the group's 32 tokens ------
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const u32x4 av = BITS == 2 ? unpack2(vw[t / 2], t & 1) : unpack4(vw[t]);
      acc[t] = mfma_f16(av, bp[t / 2], acc[t]);
    }
  }

  // ---- wave result -> LDS: m [WAVES][8], l [WAVES][8], o [WAVES][8][D] --------------------
  float* s_m = smem;
  float* s_l = smem + WAVES * 8;
  float* s_o = smem + 2 * WAVES * 8;
  const float l_tot = sum_over_rows(l_lane);
  float bvt[4];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) bvt[cg] = sum_over_rows(bv[cg]);
  if (active && hl == 0) {
    if (gq == 0) {
      s_m[wave * 8 + h] = m_run * LN2;  // natural-log units from here on
      s_l[wave * 8 + h] = l_tot;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 16 * t + 4 * gq + r;
        s_o[(wave * 8 + h) * D + c] = acc[t][r] * (SUBNORMAL / SCALE_PV) + bvt[c / GROUP];
      }
  }
  __syncthreads();
  // ---- merge the four waves into this split's partial -----------------------------------
  for (int idx = tid; idx < a.G * D; idx += THREADS) {
    const int hh = idx / D, c = idx % D;
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
      if (s_l[w * 8 + hh] > 0.f) m = fmaxf(m, s_m[w * 8 + hh]);
    float o = 0.f, l = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float lw = s_l[w * 8 + hh];
        if (lw > 0.f) {
          const float f = __expf(s_m[w * 8 + hh] - m);
          o += f * s_o[(w * 8 + hh) * D + c];
          l += f * lw;
        }
      }
    }
    const int64_t row = (int64_t)b * a.Hq + kvh * a.G + hh;
    a.part_o[(row * a.total_splits + split) * D + c] = o;
    if (c == 0) {
      a.part_ml[(row * a.total_splits + split) * 2 + 0] = m;
      a.part_ml[(row * a.total_splits + split) * 2 + 1] = l;
    }
  }
}

// Residual tokens n_q .. n_q+r-1 from the fp16/fp32 ring, on the vector ALUs.
__device__ void residual_split(const DQArgs& a, int bh, int split, float* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int G = a.G, r = a.r;
  float* s_q = smem;                  // [8][D]
  float* s_p = smem + 8 * D;          // [8][RES_MAX]
  float* s_ml = s_p + 8 * RES_MAX;    // [8][2]
  for (int idx = tid; idx < G * D; idx += THREADS) {
    const int hh = idx / D, c = idx % D;
    s_q[idx] = load_as_f32(a.q, ((int64_t)b * a.Hq + kvh * G + hh) * D + c, a.q_dtype) * a.qscale;
  }
  __syncthreads();
  const int64_t res_base = (int64_t)bh * a.res_cap;
  for (int t = tid; t < r; t += THREADS) {
    const int64_t slot = (a.n_q + t) % a.res_cap;
    const int64_t rowi = (res_base + slot) * D;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < D; ++c) {
      const float kx = load_as_f32(a.k_res, rowi + c, a.res_dtype);
#pragma unroll
      for (int hh = 0; hh < 8; ++hh)
        if (hh < G) acc[hh] += s_q[hh * D + c] * kx;
    }
#pragma unroll
    for (int hh = 0; hh < 8; ++hh)
      if (hh < G) s_p[hh * RES_MAX + t] = acc[hh];
  }
  __syncthreads();
  for (int hh = wave; hh < G; hh += WAVES) {
    float m = -INFINITY;
    for (int t = lane; t < r; t += 64) m = fmaxf(m, s_p[hh * RES_MAX + t]);
    m = wave_max(m);
    float l = 0.f;
    for (int t = lane; t < r; t += 64) {
      const float p = exp2f(s_p[hh * RES_MAX + t] - m);
      s_p[hh * RES_MAX + t] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) {
      s_ml[2 * hh] = (r > 0) ? m * LN2 : -INFINITY;
      s_ml[2 * hh + 1] = l;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += THREADS) {
    const int hh = idx / D, c = idx % D;
    float o = 0.f;
    for (int t = 0; t < r; ++t) {
      const int64_t slot = (a.n_q + t) % a.res_cap;
      o += s_p[hh * RES_MAX + t] * load_as_f32(a.v_res, (res_base + slot) * D + c, a.res_dtype);
    }
    const int64_t row = (int64_t)b * a.Hq + kvh * G + hh;
    a.part_o[(row * a.total_splits + split) * D + c] = o;
    if (c == 0) {
      a.part_ml[(row * a.total_splits + split) * 2 + 0] = s_ml[2 * hh];
      a.part_ml[(row * a.total_splits + split) * 2 + 1] = s_ml[2 * hh + 1];
    }
  }
}

template <int BITS, bool META_F16>
__global__ void __launch_bounds__(THREADS) draft_quant_kernel(DQArgs a) {
  __shared__ float smem[8 * D + 8 * RES_MAX + 16];
  __shared__ int s_last;
  const int split = blockIdx.x;
  const int bh = blockIdx.y;
  if (split < a.splits)
    quant_split<BITS, META_F16>(a, bh, split, smem);
  else
    residual_split(a, bh, split, smem);

  // ---- ticket: the last split of this (b, kv head) merges every partial -----------------
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(a.counters + bh, 1u) == (unsigned)(a.total_splits - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  for (int hh = threadIdx.x >> 6; hh < a.G; hh += WAVES) {
    const int64_t row = (int64_t)b * a.Hq + kvh * a.G + hh;
    merge_row_wave(a.part_o + row * a.total_splits * D, a.part_ml + row * a.total_splits * 2,
                   a.total_splits, a.out + row * D, a.lse ? a.lse + row : nullptr);
  }
  if (threadIdx.x == 0) a.counters[bh] = 0u;
}

}  // namespace

DraftQuantPlan plan_draft_quant(const vc_kivi& c, int64_t n_q, int Hq) {
  DraftQuantPlan p;
  const int64_t ngroups = n_q / GROUP;
  const int64_t units = (int64_t)c.B * c.Hkv;
  int64_t s = (1024 + units - 1) / units;       // aim at ~1024 workgroups
  s = std::min<int64_t>(s, std::max<int64_t>(1, ngroups / 8));  // >= 2 groups per wave
  if (ngroups == 0) s = 0;
  p.splits = (int)s;
  p.total_splits = p.splits + 1;
  const size_t rows = (size_t)c.B * Hq;
  p.ws_bytes = COUNTER_BYTES + rows * p.total_splits * (D + 2) * sizeof(float);
  return p;
}

hipError_t launch_draft_quant(const vc_kivi& c, int64_t n_q, int r, const void* q, int q_dtype,
                              int Hq, float sm_scale, float* out, float* lse, void* ws,
                              const DraftQuantPlan& plan, hipStream_t s) {
  DQArgs a;
  a.k_codes = static_cast<const uint8_t*>(c.k_codes);
  a.v_codes = static_cast<const uint8_t*>(c.v_codes);
  a.k_meta = c.k_meta;
  a.v_meta = c.v_meta;
  a.k_res = c.k_res;
  a.v_res = c.v_res;
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.counters = static_cast<unsigned*>(ws);
  const size_t rows = (size_t)c.B * Hq;
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(ws) + COUNTER_BYTES);
  a.part_ml = a.part_o + rows * plan.total_splits * D;
  a.tok_cap = c.tok_cap;
  a.n_q = n_q;
  a.r = r;
  a.res_cap = c.res_cap;
  a.res_dtype = c.res_dtype;
  a.q_dtype = q_dtype;
  a.Hkv = c.Hkv;
  a.Hq = Hq;
  a.G = Hq / c.Hkv;
  a.ngroups = (int)(n_q / GROUP);
  a.splits = plan.splits;
  a.total_splits = plan.total_splits;
  a.qscale = sm_scale * LOG2E;
  dim3 grid((unsigned)plan.total_splits, (unsigned)(c.B * c.Hkv));
  const bool f16m = c.meta_dtype == VC_F16;
  if (c.bits == 2) {
    if (f16m) hipLaunchKernelGGL((draft_quant_kernel<2, true>), grid, dim3(THREADS), 0, s, a);
    else hipLaunchKernelGGL((draft_quant_kernel<2, false>), grid, dim3(THREADS), 0, s, a);
  } else {
    if (f16m) hipLaunchKernelGGL((draft_quant_kernel<4, true>), grid, dim3(THREADS), 0, s, a);
    else hipLaunchKernelGGL((draft_quant_kernel<4, false>), grid, dim3(THREADS), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace vc
