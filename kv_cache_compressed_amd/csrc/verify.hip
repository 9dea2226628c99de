// Verify attention: L <= 32 query rows per query head attend causally over the full cache.
//
// "VeriCache: making lossy KV compression exact", The Core Idea (one pass over the full cache
// scores every drafted position plus one) and Verifying Without Giving Back the Speedup (the full
// cache may sit in CPU memory and is brought to the GPU only for verification, loading the
// interconnect; the verifier checks several positions at once, so it uses compute differently
// from one-token decoding); "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference", Key
// Contributions (verification is bound by the interconnect and FLOPs).
//
// bf16 path (matrix cores). Workgroup = G waves on one (b, kv head) and one range of 32-token
// key tiles; wave w owns query head kvh*G + w and its L rows (two 16-row column tiles). Each key
// tile is staged once in LDS for all G waves: keys row-major (bf16), values transposed to
// channel-major token pairs (bf16x2) so that the PV product reads its operand with 8-byte LDS
// loads. QK^T uses v_mfma_f32_16x16x32_bf16 with the keys as the row operand, so each lane gets the
// scores of 8 tokens for one query row in exactly the layout the PV product wants for its B
// operand. The softmax weights are carried as a bf16 hi + lo pair (two accumulations), which keeps
// ~16 significant bits in the weights at the cost of a second PV product; the fp32 accumulators
// are exact enough that the logits keep their argmax.
//
// fp32 path (vector ALUs): one workgroup per (row, split) with a thread per key.
//
// Both paths write unnormalised split partials (o, m, l); the past is split into ranges (or
// streamed chunk by chunk from pinned host memory through two device stages), the causal block
// is one more split, and a log-sum-exp merge produces the output.
#include "common.h"
#include "kernels.h"

namespace vc {

namespace {

constexpr int TK = 32;             // keys per tile
constexpr int K_STRIDE = D + 8;    // bf16 elements per staged key row (16-byte pad)
constexpr int VT_STRIDE = TK / 2 + 4;  // dwords per staged transposed value row

struct VArgs {
  const uint16_t* q;       // [B][Hq][L][D] bf16
  const uint16_t* k;       // source keys: element (bh, t, c) at (bh*bh_stride + t)*D + c
  const uint16_t* v;
  int64_t bh_stride;       // tokens between consecutive (b, kv head) source rows
  int64_t ntok;            // tokens in this source
  int splits;              // workgroups per (b, kv head) for this source
  int split_offset;        // partial index of this launch's split 0
  int causal;              // source is the round's block: row i sees tokens 0..i
  int L, Hq, Hkv, G, total_splits;
  float qscale;            // sm_scale * log2(e)
  float* part_o;
  float* part_ml;
};

__device__ __forceinline__ uint32_t bf16_pack_rne(float lo, float hi) {
  const uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
  const uint32_t ra = (a + 0x7fffu + ((a >> 16) & 1u)) >> 16;
  const uint32_t rb = (b + 0x7fffu + ((b >> 16) & 1u)) & 0xffff0000u;
  return ra | rb;
}

__global__ void __launch_bounds__(512) verify_bf16_kernel(VArgs a) {
  __shared__ uint16_t s_k[TK * K_STRIDE];
  __shared__ uint32_t s_vt[D * VT_STRIDE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthreads = blockDim.x;
  const int j = lane & 15, gq = lane >> 4;
  const int bh = blockIdx.y, split = blockIdx.x;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int hq = kvh * a.G + wave;

  // tile range of this split
  const int64_t ntiles = (a.ntok + TK - 1) / TK;
  const int64_t t_begin = ntiles * split / a.splits;
  const int64_t t_end = ntiles * (split + 1) / a.splits;

  // Q^T operand: column tile ct holds rows 16ct + j; lane holds channels 32kb + 8gq + 0..7.
  u32x4 qop[2][4];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int row = 16 * ct + j;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (row < a.L) {
        const int64_t off = (((int64_t)b * a.Hq + hq) * a.L + row) * D + 32 * kb + 8 * gq;
        qop[ct][kb] = *reinterpret_cast<const u32x4*>(a.q + off);
      } else {
        qop[ct][kb] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  float m_run[2] = {-INFINITY, -INFINITY};
  float l_lane[2] = {0.f, 0.f};
  f32x4 acc[2][8];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[ct][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* kbase = a.k + (int64_t)bh * a.bh_stride * D;
  const uint16_t* vbase = a.v + (int64_t)bh * a.bh_stride * D;

  for (int64_t tile = t_begin; tile < t_end; ++tile) {
    const int64_t tok0 = tile * TK;
    const int tlen = (int)min<int64_t>(TK, a.ntok - tok0);
    __syncthreads();  // previous tile fully consumed
    // ---- stage keys (row-major) ---------------------------------------------------------
    for (int idx = tid; idx < TK * (D / 8); idx += nthreads) {
      const int t = idx / (D / 8), c8 = idx % (D / 8);
      u32x4 val = u32x4{0u, 0u, 0u, 0u};
      if (t < tlen) val = *reinterpret_cast<const u32x4*>(kbase + (tok0 + t) * D + c8 * 8);
      *reinterpret_cast<u32x4*>(s_k + t * K_STRIDE + c8 * 8) = val;
    }
    // ---- stage values transposed: s_vt[c][tp] = (v[2tp][c], v[2tp+1][c]) -------------------
    for (int idx = tid; idx < (TK / 2) * (D / 8); idx += nthreads) {
      const int tp = idx % (TK / 2), c8 = idx / (TK / 2);
      u32x4 v0 = u32x4{0u, 0u, 0u, 0u}, v1 = u32x4{0u, 0u, 0u, 0u};
      if (2 * tp < tlen) v0 = *reinterpret_cast<const u32x4*>(vbase + (tok0 + 2 * tp) * D + c8 * 8);
      if (2 * tp + 1 < tlen) v1 = *reinterpret_cast<const u32x4*>(vbase + (tok0 + 2 * tp + 1) * D + c8 * 8);
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        // channels 8c8 + 2z (low halves) and 8c8 + 2z + 1 (high halves)
        s_vt[(c8 * 8 + 2 * z) * VT_STRIDE + tp] = __builtin_amdgcn_perm(v1[z], v0[z], 0x05040100u);
        s_vt[(c8 * 8 + 2 * z + 1) * VT_STRIDE + tp] = __builtin_amdgcn_perm(v1[z], v0[z], 0x07060302u);
      }
    }
    __syncthreads();
    // ---- QK^T: S^T[token][row] ------------------------------------------------------------
    f32x4 s[2][2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      u32x4 kop[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        kop[kb] = *reinterpret_cast<const u32x4*>(s_k + (16 * tb + j) * K_STRIDE + 32 * kb + 8 * gq);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) c = mfma_bf16(kop[kb], qop[ct][kb], c);
        s[tb][ct] = c;
      }
    }
    // ---- masked online softmax per query row --------------------------------------------
    u32x4 phi[2], plo[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int row = 16 * ct + j;
      float sc[8];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = 16 * (e >> 2) + 4 * gq + (e & 3);
        bool ok = tok < tlen;
        if (a.causal) ok = ok && (tok0 + tok <= row);
        const float v = ok ? s[e >> 2][ct][e & 3] * a.qscale : -INFINITY;
        sc[e] = v;
        mx = fmaxf(mx, v);
      }
      mx = max_over_rows(mx);
      const float m_new = fmaxf(m_run[ct], mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[ct] - m_new);
      m_run[ct] = m_new;
      float psum = 0.f, hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = (m_new == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[e] - m_new);
        psum += p;
        hi[e] = __uint_as_float(__float_as_uint(p) & 0xffff0000u);  // truncated: exact split
        lo[e] = p - hi[e];
      }
      l_lane[ct] = l_lane[ct] * alpha + psum;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[ct][t] *= alpha;
      phi[ct] = u32x4{(__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xffff0000u),
                      (__float_as_uint(hi[2]) >> 16) | (__float_as_uint(hi[3]) & 0xffff0000u),
                      (__float_as_uint(hi[4]) >> 16) | (__float_as_uint(hi[5]) & 0xffff0000u),
                      (__float_as_uint(hi[6]) >> 16) | (__float_as_uint(hi[7]) & 0xffff0000u)};
      plo[ct] = u32x4{bf16_pack_rne(lo[0], lo[1]), bf16_pack_rne(lo[2], lo[3]),
                      bf16_pack_rne(lo[4], lo[5]), bf16_pack_rne(lo[6], lo[7])};
    }
    // ---- PV: O^T[c][row] += V^T[c][tok] P^T[tok][row] ----------------------------------------
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t* vr = s_vt + (16 * t + j) * VT_STRIDE;
      const u32x2 lo2 = *reinterpret_cast<const u32x2*>(vr + 2 * gq);
      const u32x2 hi2 = *reinterpret_cast<const u32x2*>(vr + 8 + 2 * gq);
      const u32x4 vop = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        acc[ct][t] = mfma_bf16(vop, phi[ct], acc[ct][t]);
        acc[ct][t] = mfma_bf16(vop, plo[ct], acc[ct][t]);
      }
    }
  }

  // ---- write this wave's partial rows ------------------------------------------------------
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int row = 16 * ct + j;
    const float l = sum_over_rows(l_lane[ct]);
    if (row < a.L) {
      const int64_t prow = ((int64_t)b * a.Hq + hq) * a.L + row;
      const int sidx = a.split_offset + split;
      float* po = a.part_o + (prow * a.total_splits + sidx) * D;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        *reinterpret_cast<f32x4*>(po + 16 * t + 4 * gq) = acc[ct][t];
      if (gq == 0) {
        a.part_ml[(prow * a.total_splits + sidx) * 2 + 0] = (l > 0.f) ? m_run[ct] * LN2 : -INFINITY;
        a.part_ml[(prow * a.total_splits + sidx) * 2 + 1] = l;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// fp32 path: one workgroup per (query row, split) with one thread per key.
// ---------------------------------------------------------------------------------------------
struct VF32Args {
  const float* q;       // [B][Hq][L][D]
  const float* k_past;  // element (bh, t, c) at (bh*past_stride + t)*D + c
  const float* v_past;
  const float* k_blk;   // [B][Hkv][L][D]
  const float* v_blk;
  int64_t past_stride, n;
  int L, Hq, Hkv, G, splits;
  float qscale;
  float* part_o;
  float* part_ml;
};

__global__ void __launch_bounds__(256) verify_f32_kernel(VF32Args a) {
  __shared__ float s_q[D];
  __shared__ float s_p[256];
  __shared__ float s_red[8];
  __shared__ float s_o[2][D];
  const int tid = threadIdx.x;
  const int64_t prow = blockIdx.y;  // (b*Hq + hq)*L + i
  const int split = blockIdx.x;
  const int i = (int)(prow % a.L);
  const int64_t bhq = prow / a.L;
  const int b = (int)(bhq / a.Hq), hq = (int)(bhq % a.Hq);
  const int bh = b * a.Hkv + hq / a.G;
  const int64_t nkeys = a.n + i + 1;
  const int64_t k_begin = nkeys * split / a.splits, k_end = nkeys * (split + 1) / a.splits;
  if (tid < D) s_q[tid] = a.q[prow * D + tid] * a.qscale;
  __syncthreads();
  float m_run = -INFINITY, l_run = 0.f, o_acc = 0.f;
  const int c = tid & (D - 1), half = tid >> 7;
  for (int64_t k0 = k_begin; k0 < k_end; k0 += 256) {
    const int64_t key = k0 + tid;
    float s = -INFINITY;
    if (key < k_end) {
      const float* kr = key < a.n ? a.k_past + ((int64_t)bh * a.past_stride + key) * D
                                  : a.k_blk + ((int64_t)bh * a.L + (key - a.n)) * D;
      float acc = 0.f;
      for (int cc = 0; cc < D; ++cc) acc += s_q[cc] * kr[cc];
      s = acc;
    }
    const float mx_w = wave_max(s);
    if ((tid & 63) == 0) s_red[tid >> 6] = mx_w;
    __syncthreads();
    const float mx = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float p = (key < k_end) ? __builtin_amdgcn_exp2f(s - m_new) : 0.f;
    s_p[tid] = p;
    const float ps = wave_sum(p);
    __syncthreads();
    if ((tid & 63) == 0) s_red[4 + (tid >> 6)] = ps;
    __syncthreads();
    l_run = l_run * alpha + (s_red[4] + s_red[5] + s_red[6] + s_red[7]);
    m_run = m_new;
    o_acc *= alpha;
    const int nk = (int)min<int64_t>(256, k_end - k0);
    for (int t = half; t < nk; t += 2) {
      const int64_t key2 = k0 + t;
      const float* vr = key2 < a.n ? a.v_past + ((int64_t)bh * a.past_stride + key2) * D
                                   : a.v_blk + ((int64_t)bh * a.L + (key2 - a.n)) * D;
      o_acc += s_p[t] * vr[c];
    }
    __syncthreads();
  }
  s_o[half][c] = o_acc;
  __syncthreads();
  if (tid < D) {
    a.part_o[(prow * a.splits + split) * D + tid] = s_o[0][tid] + s_o[1][tid];
    if (tid == 0) {
      a.part_ml[(prow * a.splits + split) * 2 + 0] = (l_run > 0.f) ? m_run * LN2 : -INFINITY;
      a.part_ml[(prow * a.splits + split) * 2 + 1] = l_run;
    }
  }
}

}  // namespace

VerifyPlan plan_verify(int B, int Hq, int Hkv, int L, int64_t n, int past_on_host,
                       int64_t chunk_tokens, int dtype) {
  VerifyPlan p{};
  const int64_t units = (int64_t)B * Hkv;
  if (dtype == VC_F32) {
    p.past_splits = (int)std::max<int64_t>(1, std::min<int64_t>(16, (n + L + 1023) / 1024));
    p.chunks = 0;
    p.chunk_tokens = 0;
    p.total_splits = p.past_splits;
    p.stage_bytes = 0;
  } else if (!past_on_host) {
    const int64_t tiles = (n + TK - 1) / TK;
    int64_t s = (512 + units - 1) / units;
    s = std::min<int64_t>(s, std::max<int64_t>(1, tiles / 4));
    if (n == 0) s = 0;
    p.past_splits = (int)s;
    p.chunks = 0;
    p.chunk_tokens = 0;
    p.total_splits = p.past_splits + 1;
    p.stage_bytes = 0;
  } else {
    const int64_t ct = std::min<int64_t>(chunk_tokens, std::max<int64_t>(n, 1));
    p.chunk_tokens = ct;
    p.chunks = (int)((n + ct - 1) / ct);
    const int64_t tiles = (ct + TK - 1) / TK;
    int64_t s = (512 + units - 1) / units;
    s = std::min<int64_t>(s, std::max<int64_t>(1, tiles / 4));
    p.past_splits = (int)s;
    p.total_splits = p.chunks * p.past_splits + 1;
    p.stage_bytes = (size_t)units * ct * D * 2 * 2;  // keys + values, bf16
  }
  const size_t rows = (size_t)B * Hq * L;
  p.part_bytes = rows * p.total_splits * (D + 2) * sizeof(float);
  p.part_bytes = (p.part_bytes + 255) & ~(size_t)255;
  p.ws_bytes = p.part_bytes + 2 * p.stage_bytes;
  return p;
}

hipError_t launch_verify(const void* q, const void* k_blk, const void* v_blk, int L,
                         const void* k_past, const void* v_past, int64_t past_stride, int64_t n,
                         int past_on_host, int dtype, int B, int Hq, int Hkv, float sm_scale,
                         float* out, float* lse, void* ws, const VerifyPlan& plan,
                         hipStream_t compute, hipStream_t copy) {
  const size_t rows = (size_t)B * Hq * L;
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o + rows * plan.total_splits * D;
  const int G = Hq / Hkv;
  const float qscale = sm_scale * LOG2E;
  hipError_t err;

  if (dtype == VC_F32) {
    VF32Args a;
    a.q = static_cast<const float*>(q);
    a.k_past = static_cast<const float*>(k_past);
    a.v_past = static_cast<const float*>(v_past);
    a.k_blk = static_cast<const float*>(k_blk);
    a.v_blk = static_cast<const float*>(v_blk);
    a.past_stride = past_stride;
    a.n = n;
    a.L = L;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = G;
    a.splits = plan.total_splits;
    a.qscale = qscale;
    a.part_o = part_o;
    a.part_ml = part_ml;
    hipLaunchKernelGGL(verify_f32_kernel, dim3(plan.total_splits, (unsigned)rows), dim3(256), 0,
                       compute, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    return launch_merge(part_o, part_ml, (int64_t)rows, plan.total_splits, out, lse, compute);
  }

  VArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.L = L;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.total_splits = plan.total_splits;
  a.qscale = qscale;
  a.part_o = part_o;
  a.part_ml = part_ml;
  const dim3 block(64 * G);
  const unsigned units = (unsigned)(B * Hkv);

  if (!past_on_host) {
    if (plan.past_splits > 0) {
      a.k = static_cast<const uint16_t*>(k_past);
      a.v = static_cast<const uint16_t*>(v_past);
      a.bh_stride = past_stride;
      a.ntok = n;
      a.splits = plan.past_splits;
      a.split_offset = 0;
      a.causal = 0;
      hipLaunchKernelGGL(verify_bf16_kernel, dim3(plan.past_splits, units), block, 0, compute, a);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  } else {
    // Stream the past chunk by chunk: copies on `copy` into stage c % 2, compute on `compute`.
    char* stage_base = static_cast<char*>(ws) + plan.part_bytes;
    uint16_t* stage_k[2];
    uint16_t* stage_v[2];
    for (int z = 0; z < 2; ++z) {
      stage_k[z] = reinterpret_cast<uint16_t*>(stage_base + z * plan.stage_bytes);
      stage_v[z] = stage_k[z] + (size_t)units * plan.chunk_tokens * D;
    }
    hipEvent_t ready[2], done[2], start;
    bool made = true;
    for (int z = 0; z < 2 && made; ++z) {
      made = hipEventCreateWithFlags(&ready[z], hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&done[z], hipEventDisableTiming) == hipSuccess;
    }
    if (!made || hipEventCreateWithFlags(&start, hipEventDisableTiming) != hipSuccess)
      return hipErrorOutOfMemory;
    // the copy stream must not overwrite stages before earlier work on `compute` is ordered
    err = hipEventRecord(start, compute);
    if (err == hipSuccess) err = hipStreamWaitEvent(copy, start, 0);
    const size_t src_pitch = (size_t)past_stride * D * 2;
    for (int c = 0; c < plan.chunks && err == hipSuccess; ++c) {
      const int z = c % 2;
      const int64_t t0 = (int64_t)c * plan.chunk_tokens;
      const int64_t len = std::min<int64_t>(plan.chunk_tokens, n - t0);
      if (c >= 2) err = hipStreamWaitEvent(copy, done[z], 0);
      const size_t width = (size_t)len * D * 2;
      const size_t dpitch = (size_t)plan.chunk_tokens * D * 2;
      if (err == hipSuccess)
        err = hipMemcpy2DAsync(stage_k[z], dpitch, static_cast<const char*>(k_past) + t0 * D * 2,
                               src_pitch, width, units, hipMemcpyHostToDevice, copy);
      if (err == hipSuccess)
        err = hipMemcpy2DAsync(stage_v[z], dpitch, static_cast<const char*>(v_past) + t0 * D * 2,
                               src_pitch, width, units, hipMemcpyHostToDevice, copy);
      if (err == hipSuccess) err = hipEventRecord(ready[z], copy);
      if (err == hipSuccess) err = hipStreamWaitEvent(compute, ready[z], 0);
      if (err != hipSuccess) break;
      a.k = stage_k[z];
      a.v = stage_v[z];
      a.bh_stride = plan.chunk_tokens;
      a.ntok = len;
      a.splits = plan.past_splits;
      a.split_offset = c * plan.past_splits;
      a.causal = 0;
      hipLaunchKernelGGL(verify_bf16_kernel, dim3(plan.past_splits, units), block, 0, compute, a);
      if ((err = hipGetLastError()) != hipSuccess) break;
      err = hipEventRecord(done[z], compute);
    }
    // make `compute` wait for the copy stream's last command (covers every copy)
    if (err == hipSuccess) err = hipEventRecord(ready[0], copy);
    if (err == hipSuccess) err = hipStreamWaitEvent(compute, ready[0], 0);
    for (int z = 0; z < 2; ++z) {
      (void)hipEventDestroy(ready[z]);
      (void)hipEventDestroy(done[z]);
    }
    (void)hipEventDestroy(start);
    if (err != hipSuccess) return err;
  }
  // the causal block: one more split
  a.k = static_cast<const uint16_t*>(k_blk);
  a.v = static_cast<const uint16_t*>(v_blk);
  a.bh_stride = L;
  a.ntok = L;
  a.splits = 1;
  a.split_offset = plan.total_splits - 1;
  a.causal = 1;
  hipLaunchKernelGGL(verify_bf16_kernel, dim3(1, units), block, 0, compute, a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_merge(part_o, part_ml, (int64_t)rows, plan.total_splits, out, lse, compute);
}

}  // namespace vc
