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

constexpr float LAZY = 2.0f;  // log2 slack before a row's reference max is moved

// One key/value tile (32 tokens x 128 channels) in flight in registers: KI 16-byte key chunks and
// VI token pairs of 16-byte value chunks per thread.
template <int NT>
struct TileRegs {
  static constexpr int KI = (TK * (D / 8) + NT - 1) / NT;
  static constexpr int VI = ((TK / 2) * (D / 8) + NT - 1) / NT;
  u32x4 k[KI];
  u32x4 v0[VI], v1[VI];
};

// Issue the loads of tile `tile` through buffer resources whose size is the source's ntok rows,
// so rows past the end read as zero with no per-row checks; each thread's byte offsets are fixed
// and the tile offset is a uniform scalar.
constexpr int RSRC_WORD3 = 0x00020000;  // raw buffer, 32-bit data format
template <int NT>
__device__ __forceinline__ void tile_load(TileRegs<NT>& r, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                          int64_t tile, bool live) {
  const int tid = threadIdx.x;
  const int sbase = live ? (int)(tile * TK * D * 2) : 0x7fffff00;  // dead tiles: out of range -> 0
  // Every load is unconditional (threads past an item range re-read a valid item and do not store
  // it), so the loads form straight-line code the compiler can count precisely.
#pragma unroll
  for (int z = 0; z < TileRegs<NT>::KI; ++z) {
    const int idx = (tid + z * NT) % (TK * (D / 8));
    const int t = idx / (D / 8), c8 = idx % (D / 8);
    r.k[z] = __builtin_amdgcn_raw_buffer_load_b128(rk, t * D * 2 + c8 * 16, sbase, 0);
  }
#pragma unroll
  for (int z = 0; z < TileRegs<NT>::VI; ++z) {
    const int idx = (tid + z * NT) % ((TK / 2) * (D / 8));
    const int tp = idx % (TK / 2), c8 = idx / (TK / 2);
    r.v0[z] = __builtin_amdgcn_raw_buffer_load_b128(rv, 2 * tp * D * 2 + c8 * 16, sbase, 0);
    r.v1[z] = __builtin_amdgcn_raw_buffer_load_b128(rv, (2 * tp + 1) * D * 2 + c8 * 16, sbase, 0);
  }
}

// Write a loaded tile to LDS: keys row-major (padded rows), values transposed to channel-major
// token pairs: s_vt[c][tp] = (v[2tp][c], v[2tp+1][c]).
template <int NT>
__device__ __forceinline__ void tile_store(const TileRegs<NT>& r, uint16_t* s_k, uint32_t* s_vt) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int z = 0; z < TileRegs<NT>::KI; ++z) {
    const int idx = tid + z * NT;
    const int t = idx / (D / 8), c8 = idx % (D / 8);
    if (idx < TK * (D / 8)) *reinterpret_cast<u32x4*>(s_k + t * K_STRIDE + c8 * 8) = r.k[z];
  }
#pragma unroll
  for (int z = 0; z < TileRegs<NT>::VI; ++z) {
    const int idx = tid + z * NT;
    const int tp = idx % (TK / 2), c8 = idx / (TK / 2);
    if (idx < (TK / 2) * (D / 8)) {
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        s_vt[(c8 * 8 + 2 * y) * VT_STRIDE + tp] = __builtin_amdgcn_perm(r.v1[z][y], r.v0[z][y], 0x05040100u);
        s_vt[(c8 * 8 + 2 * y + 1) * VT_STRIDE + tp] = __builtin_amdgcn_perm(r.v1[z][y], r.v0[z][y], 0x07060302u);
      }
    }
  }
}

// Workgroup = NW waves (NW >= G) on one (b, kv head) and one range of 32-token tiles; wave w < G
// owns query head kvh*G + w and its L rows (two 16-row column tiles); all NW waves stage tiles.
// Tiles are double-buffered in LDS and loaded two tiles ahead into registers, so each tile costs
// one barrier and its loads overlap the two tiles before it.
template <int NW>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) verify_bf16_kernel(VArgs a) {
  constexpr int NT = 64 * NW;
  __shared__ uint16_t s_k[2][TK * K_STRIDE];
  __shared__ uint32_t s_vt[2][D * VT_STRIDE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, gq = lane >> 4;
  const int bh = blockIdx.y, split = blockIdx.x;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const bool computes = wave < a.G;
  const int hq = kvh * a.G + min(wave, a.G - 1);

  // tile range of this split
  const int64_t ntiles = (a.ntok + TK - 1) / TK;
  const int64_t t_begin = ntiles * split / a.splits;
  const int64_t t_end = ntiles * (split + 1) / a.splits;
  const int nbytes = (int)(a.ntok * D * 2);  // this (b, kv head)'s source rows
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.k + (int64_t)bh * a.bh_stride * D), (short)0, nbytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.v + (int64_t)bh * a.bh_stride * D), (short)0, nbytes, RSRC_WORD3);

  TileRegs<NT> ra, rb;
  tile_load<NT>(ra, rk, rv, t_begin, t_begin < t_end);
  tile_load<NT>(rb, rk, rv, t_begin + 1, t_begin + 1 < t_end);

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

  tile_store<NT>(ra, s_k[0], s_vt[0]);
  __syncthreads();

  // One tile: compute `tile` from LDS buffer `cur`; `ahead` holds tile+1 (loaded), `free` is
  // reloaded with tile+2, then `ahead` goes to the other buffer.
  auto step = [&](int64_t tile, int cur, TileRegs<NT>& free, TileRegs<NT>& ahead) {
    tile_load<NT>(free, rk, rv, tile + 2, tile + 2 < t_end);
    if (computes && tile < t_end) {
      const int64_t tok0 = tile * TK;
      const int tlen = (int)min<int64_t>(TK, a.ntok - tok0);
      const uint16_t* sk = s_k[cur];
      const uint32_t* svt = s_vt[cur];
      // ---- QK^T: S^T[token][row] ----------------------------------------------------------
      f32x4 s[2][2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        u32x4 kop[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          kop[kb] = *reinterpret_cast<const u32x4*>(sk + (16 * tb + j) * K_STRIDE + 32 * kb + 8 * gq);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) c = mfma_bf16(kop[kb], qop[ct][kb], c);
          s[tb][ct] = c;
        }
      }
      // ---- masked online softmax per query row, lazily moved reference max ------------------
      // (scores are scaled inside the exponent: the max is taken on the raw products)
      const bool masked = a.causal || tlen < TK;
      u32x4 phi[2], plo[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int row = 16 * ct + j;
        float raw[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) raw[e] = s[e >> 2][ct][e & 3];
        if (masked) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int tok = 16 * (e >> 2) + 4 * gq + (e & 3);
            bool ok = tok < tlen;
            if (a.causal) ok = ok && (tok0 + tok <= row);
            raw[e] = ok ? raw[e] : -INFINITY;
          }
        }
        const float mraw = fmaxf(fmaxf(fmaxf(raw[0], raw[1]), fmaxf(raw[2], raw[3])),
                                 fmaxf(fmaxf(raw[4], raw[5]), fmaxf(raw[6], raw[7])));
        const float mx = max_over_rows(mraw) * a.qscale;
        const bool move = mx > m_run[ct] + LAZY;
        if (__builtin_amdgcn_ballot_w64(move)) {
          const float m_new = move ? mx : m_run[ct];
          const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[ct] - m_new);
          m_run[ct] = m_new;
          l_lane[ct] *= alpha;
#pragma unroll
          for (int t = 0; t < 8; ++t) acc[ct][t] *= alpha;
        }
        const float nref = m_run[ct] == -INFINITY ? 0.f : -m_run[ct];
        float p[8], lo[8];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(fmaf(raw[e], a.qscale, nref));  // masked: exp2(-inf) = 0
          psum += p[e];
          lo[e] = p[e] - __uint_as_float(__float_as_uint(p[e]) & 0xffff0000u);  // exact remainder
        }
        l_lane[ct] += psum;
        // bf16 hi = truncated p; bf16 lo = truncated remainder (the pair keeps ~16 bits)
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          phi[ct][e2] = __builtin_amdgcn_perm(__float_as_uint(p[2 * e2 + 1]), __float_as_uint(p[2 * e2]), 0x07060302u);
          plo[ct][e2] = __builtin_amdgcn_perm(__float_as_uint(lo[2 * e2 + 1]), __float_as_uint(lo[2 * e2]), 0x07060302u);
        }
      }
      // ---- PV: O^T[c][row] += V^T[c][tok] P^T[tok][row] ---------------------------------------
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t* vr = svt + (16 * t + j) * VT_STRIDE;
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
    tile_store<NT>(ahead, s_k[cur ^ 1], s_vt[cur ^ 1]);  // a tile past the range stores zeros
    __syncthreads();
  };
  // tiles in pairs; a pair's second tile past the range loads zeros and computes nothing
  for (int64_t tile = t_begin; tile < t_end; tile += 2) {
    step(tile, 0, ra, rb);
    step(tile + 1, 1, rb, ra);
  }

  // ---- write this wave's partial rows ------------------------------------------------------
  if (!computes) return;
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
  const int NW = G <= 4 ? 4 : 8;
  const dim3 block(64 * NW);
  const unsigned units = (unsigned)(B * Hkv);
  auto launch_bf16 = [&](dim3 grid) {
    if (NW == 4)
      hipLaunchKernelGGL(verify_bf16_kernel<4>, grid, block, 0, compute, a);
    else
      hipLaunchKernelGGL(verify_bf16_kernel<8>, grid, block, 0, compute, a);
  };

  if (!past_on_host) {
    if (plan.past_splits > 0) {
      a.k = static_cast<const uint16_t*>(k_past);
      a.v = static_cast<const uint16_t*>(v_past);
      a.bh_stride = past_stride;
      a.ntok = n;
      a.splits = plan.past_splits;
      a.split_offset = 0;
      a.causal = 0;
      launch_bf16(dim3(plan.past_splits, units));
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
      launch_bf16(dim3(plan.past_splits, units));
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
  launch_bf16(dim3(1, units));
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_merge(part_o, part_ml, (int64_t)rows, plan.total_splits, out, lse, compute);
}

}  // namespace vc
