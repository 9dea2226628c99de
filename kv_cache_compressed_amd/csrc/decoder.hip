// Decoder-layer products for few rows (a draft step of a batch: one row per request): the layer's
// weight-bound matrix-vector products with the work around them fused in, so a layer's one-row
// step is a handful of launches instead of a chain of small elementwise kernels.
//
// "VeriCache: making lossy KV compression exact", The Core Idea: the drafter is the same model run
// over the compressed cache, one token at a time, so every draft step also runs the model's layers
// for one row per request; these kernels are that work for Llama-form layers (pre-norm RMSNorm,
// rotary positions on queries and keys, SwiGLU MLP), the published layer of the model families the
// pages evaluate ("VeriCache: Turning Lossy KV Cache into Lossless LLM Inference", Methodology).
//
// One kernel, four epilogues. Y[m][n] = s_m * sum_k X[m][k] g[k] W[n][k] with W [N][K] fp32 or bf16
// (bf16 widened exactly), fp32 products and accumulation, s_m = 1 / sqrt(mean_k X[m][k]^2 + eps)
// and g the norm gain when the norm is fused (else s_m = 1, g = 1). The sum of squares is gathered
// from the same loads as the product, so the norm costs no extra pass. Workgroup = 256 threads on
// 4 output columns and 16 rows; thread t owns k = 4t .. 4t+3 of every 1024-wide chunk; the 64 dot
// products are reduced across each wave by recursive halving and across the 4 waves through LDS.
// The 4 columns are two pairs taken P columns apart (c, c+1 and c+P, c+P+1), so the epilogues that
// combine column c with column c+P find both in one workgroup:
//   STORE   Y -> out (fp32)
//   ADD     out += Y (the residual stream)
//   ROPE    Y holds [q | k | v] heads of 128: q and k are rotated (channel i with i + 64, angle
//           (pos[m] + pos_add) * theta^(-i/64) from the cos/sin tables) and q, k, v are written to
//           their own arrays in the output dtype (fp32 or bf16, round to nearest even)
//   SWIGLU  Y holds [gate | up] (F columns each): out[m][c] = silu(gate) * up
#include "common.h"
#include "kernels.h"

namespace vc {

namespace {

constexpr int GT = 256;        // threads (1 wave per SIMD: 3 workgroups fit a CU)
constexpr int GW = GT / 64;    // waves
constexpr int GV = 4;          // output columns per workgroup (two groups of 2, P apart)
constexpr int GM = 16;         // rows per workgroup (a draft step's batch in one tile: each weight
                               // is read once per 16 rows)
constexpr int GCHUNK = 4 * GT; // k per chunk

struct GArgs {
  const void* W;       // [N][K]
  const float* X;      // [M][K] fp32 (row stride K)
  const float* g;      // [K] norm gain, or null (no norm)
  float eps;
  int M, K, N;
  int P;               // partner distance of the column groups
  int period;          // columns per pairing period: 2P (ROPE: 128), or N (SWIGLU: P = N / 2)
  int epi;             // DEC_STORE / DEC_ADD / DEC_ROPE / DEC_SWIGLU
  float* out;          // STORE [M][N], ADD [M][N] (in place), SWIGLU [M][N/2]
  // ROPE
  void* q_out;         // [M][Hq][128]
  void* k_out;         // [M][Hkv][128]
  void* v_out;         // [M][Hkv][128]
  int out_bf16;
  int Hq, Hkv;
  const float* cos_t;  // [positions][64]
  const float* sin_t;
  const int32_t* pos;  // [M]
  int pos_add;
  int n_pos;           // rows of the cos/sin tables (positions are clamped into them)
};

template <bool WBF16>
__device__ __forceinline__ f32x4 w4(const void* row, int k) {
  if constexpr (WBF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(row) + k);
    return f32x4{bf16_bits_to_f32(u.x & 0xffffu), bf16_bits_to_f32(u.x >> 16),
                 bf16_bits_to_f32(u.y & 0xffffu), bf16_bits_to_f32(u.y >> 16)};
  } else {
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(row) + k);
  }
}

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

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);  // finite inputs
}

// First column of this workgroup's first group.
__device__ __forceinline__ int first_col(const GArgs& a, int w) {
  const int per = a.P / 2;  // workgroups per pairing period
  return (w / per) * a.period + (w % per) * 2;
}

template <bool WBF16>
__global__ void __launch_bounds__(GT) dec_gemv_kernel(GArgs a) {
  static_assert(GV * GM == 64, "one reduced value per lane");
  __shared__ float s_red[GW][64];
  __shared__ float s_ss[GW][GM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = first_col(a, blockIdx.x), m0 = blockIdx.y * GM;
  const int64_t wb = WBF16 ? 2 : 4;
  const void* wrow[GV];
#pragma unroll
  for (int v = 0; v < GV; ++v) {
    const int col = c0 + (v & 1) + (v >> 1) * a.P;
    wrow[v] = static_cast<const char*>(a.W) + (int64_t)min(col, a.N - 1) * a.K * wb;
  }
  const float* xrow[GM];
#pragma unroll
  for (int m = 0; m < GM; ++m) xrow[m] = a.X + (int64_t)min(m0 + m, a.M - 1) * a.K;

  float acc[GV * GM];
#pragma unroll
  for (int i = 0; i < GV * GM; ++i) acc[i] = 0.f;
  float ss[GM];
#pragma unroll
  for (int m = 0; m < GM; ++m) ss[m] = 0.f;
  for (int k0 = 0; k0 < a.K; k0 += GCHUNK) {
    const int k = k0 + 4 * tid;
    if (k < a.K) {  // K is a multiple of 4
      f32x4 w[GV], x[GM];
#pragma unroll
      for (int v = 0; v < GV; ++v) w[v] = w4<WBF16>(wrow[v], k);
#pragma unroll
      for (int m = 0; m < GM; ++m) x[m] = *reinterpret_cast<const f32x4*>(xrow[m] + k);
      if (a.g) {
        const f32x4 gg = *reinterpret_cast<const f32x4*>(a.g + k);
#pragma unroll
        for (int m = 0; m < GM; ++m) {
          ss[m] = fmaf(x[m][0], x[m][0], fmaf(x[m][1], x[m][1], fmaf(x[m][2], x[m][2], fmaf(x[m][3], x[m][3], ss[m]))));
          x[m] *= gg;
        }
      }
#pragma unroll
      for (int v = 0; v < GV; ++v)
#pragma unroll
        for (int m = 0; m < GM; ++m) {
          float s = acc[v * GM + m];
          s = fmaf(w[v][0], x[m][0], s);
          s = fmaf(w[v][1], x[m][1], s);
          s = fmaf(w[v][2], x[m][2], s);
          s = fmaf(w[v][3], x[m][3], s);
          acc[v * GM + m] = s;
        }
    }
  }
  halve<32>(acc, lane);
  s_red[wave][lane] = acc[0];
  if (a.g) {
#pragma unroll
    for (int m = 0; m < GM; ++m) ss[m] = wave_sum(ss[m]);
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < GM; ++m) s_ss[wave][m] = ss[m];
    }
  }
  __syncthreads();
  if (wave != 0) return;
  // lane = v * GM + m: column pair v >> 1, column offset v & 1, row m
  const int v = lane / GM, m = lane % GM;
  float y = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < GW; ++w2) y += s_red[w2][lane];
  if (a.g) {
    float t = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < GW; ++w2) t += s_ss[w2][m];
    y *= 1.0f / sqrtf(t / (float)a.K + a.eps);
  }
  const float partner = __shfl_xor(y, 2 * GM, 64);  // same row, the other column pair
  const int row = m0 + m;
  const int col = c0 + (v & 1) + (v >> 1) * a.P;
  const bool first = v < 2;
  if (row >= a.M || col >= a.N) return;
  switch (a.epi) {
    case DEC_STORE:
      a.out[(int64_t)row * a.N + col] = y;
      break;
    case DEC_ADD:
      a.out[(int64_t)row * a.N + col] += y;
      break;
    case DEC_SWIGLU:
      if (first) a.out[(int64_t)row * (a.N / 2) + col] = y / (1.f + __expf(-y)) * partner;
      break;
    case DEC_ROPE: {
      const int head = col / 128, ch = col % 128;
      float r = y;
      if (head < a.Hq + a.Hkv) {  // q and k heads rotate: channel i < 64 pairs with i + 64
        const int i = ch & 63;
        const int pp = min(max(a.pos[row] + a.pos_add, 0), a.n_pos - 1);
        const int64_t p = (int64_t)pp * 64 + i;
        const float cs = a.cos_t[p], sn = a.sin_t[p];
        r = first ? y * cs - partner * sn : y * cs + partner * sn;
      }
      void* dst;
      int64_t off;
      if (head < a.Hq) {
        dst = a.q_out;
        off = ((int64_t)row * a.Hq + head) * 128 + ch;
      } else if (head < a.Hq + a.Hkv) {
        dst = a.k_out;
        off = ((int64_t)row * a.Hkv + head - a.Hq) * 128 + ch;
      } else {
        dst = a.v_out;
        off = ((int64_t)row * a.Hkv + head - a.Hq - a.Hkv) * 128 + ch;
      }
      if (a.out_bf16)
        static_cast<uint16_t*>(dst)[off] = bf16_rne(r);
      else
        static_cast<float*>(dst)[off] = r;
      break;
    }
  }
}

// Row-wise RMS norm with gain: Y[m] = X[m] * g / sqrt(mean(X[m]^2) + eps), one workgroup per row.
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float* X, const float* g, float eps, int K,
                                                      float* Y) {
  __shared__ float s[4];
  const float* x = X + (int64_t)blockIdx.x * K;
  float t = 0.f;
  for (int k = threadIdx.x; k < K; k += 256) t = fmaf(x[k], x[k], t);
  t = wave_sum(t);
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = t;
  __syncthreads();
  const float inv = 1.0f / sqrtf((s[0] + s[1] + s[2] + s[3]) / (float)K + eps);
  float* y = Y + (int64_t)blockIdx.x * K;
  for (int k = threadIdx.x; k < K; k += 256) y[k] = x[k] * inv * g[k];
}

// Embedding rows: out[m] = E[tok[m * tok_stride]] (fp32 rows of K), one workgroup per row; ids
// outside [0, V) give a zero row.
__global__ void __launch_bounds__(256) embed_kernel(const float* E, int V, int K, const int32_t* tok,
                                                    int64_t tok_stride, float* out) {
  const int m = blockIdx.x;
  const int t = tok[(int64_t)m * tok_stride];
  float* o = out + (int64_t)m * K;
  const bool ok = t >= 0 && t < V;
  const float* e = E + (int64_t)(ok ? t : 0) * K;
  for (int k = threadIdx.x; k < K; k += 256) o[k] = ok ? e[k] : 0.f;
}

}  // namespace

hipError_t launch_dec_gemv(const DecGemv& d, hipStream_t s) {
  GArgs a;
  a.W = d.W;
  a.X = d.X;
  a.g = d.g;
  a.eps = d.eps;
  a.M = d.M;
  a.K = d.K;
  a.N = d.N;
  a.epi = d.epi;
  a.out = d.out;
  a.q_out = d.q_out;
  a.k_out = d.k_out;
  a.v_out = d.v_out;
  a.out_bf16 = d.out_bf16;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.cos_t = d.cos_t;
  a.sin_t = d.sin_t;
  a.pos = d.pos;
  a.pos_add = d.pos_add;
  a.n_pos = d.n_pos;
  unsigned groups;
  if (d.epi == DEC_ROPE) {  // heads of 128: columns c and c + 64
    a.P = 64;
    a.period = 128;
    groups = (unsigned)(d.N / GV);
  } else if (d.epi == DEC_SWIGLU) {  // gate column c with up column c + N/2
    a.P = d.N / 2;
    a.period = d.N;
    groups = (unsigned)(d.N / GV);
  } else {  // plain: consecutive pairs, the partner pair right after
    a.P = 2;
    a.period = 4;
    groups = (unsigned)((d.N + GV - 1) / GV);
  }
  const dim3 grid(groups, (unsigned)((d.M + GM - 1) / GM));
  if (d.w_bf16)
    hipLaunchKernelGGL(dec_gemv_kernel<true>, grid, dim3(GT), 0, s, a);
  else
    hipLaunchKernelGGL(dec_gemv_kernel<false>, grid, dim3(GT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_embed(const float* E, int V, int K, const int32_t* tok, int64_t tok_stride, int M,
                        float* out, hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3((unsigned)M), dim3(256), 0, s, E, V, K, tok, tok_stride, out);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* X, const float* g, float eps, int M, int K, float* Y,
                          hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)M), dim3(256), 0, s, X, g, eps, K, Y);
  return hipGetLastError();
}

}  // namespace vc
