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
#include <algorithm>

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
  // matrix-core form only
  int S;               // slices of K per column group
  int groups;          // column groups
  unsigned* counters;  // [row tiles][groups] tickets, zero between calls
  float* part;         // [row tiles][groups][S][MSLOT] slice partials
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

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);  // finite inputs
}

// First column of this workgroup's first group.
__device__ __forceinline__ int first_col(const GArgs& a, int w) {
  const int per = a.P / 2;  // workgroups per pairing period
  return (w / per) * a.period + (w % per) * 2;
}

// Column col of row row: y (normed), partner = the same row's column col + P (first) or col - P.
__device__ __forceinline__ void dec_epilogue(const GArgs& a, int row, int col, float y, float partner,
                                             bool first) {
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
  wave_halve<32>(acc, lane);
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
  dec_epilogue(a, row, col, y, partner, first);
}

// ---------------------------------------------------------------------------------------------
// Matrix-core form (bf16 weights, K % 32 == 0): the same products on v_mfma_f32_16x16x32_bf16.
// X (times the gain) is split exactly into three bf16 pieces, x = hi + mid + lo, each the
// round-to-nearest-even of what the pieces before it leave (hi takes the leading 8 significant bits,
// mid the next 8 or so, and the rest, at most 8 bits, fits lo exactly), so every term W[n][k] x[m][k]
// enters as three exact bf16 x bf16 products summed in fp32: the result is an fp32 sum of the exact
// terms, as in the vector form, in another order.
// Workgroup = 8 waves on 128 columns (two blocks of 64 columns P apart, as above) x 16 rows x one
// slice of K (at most 512). The slice of X is loaded, split and stored in LDS once, behind one
// barrier; then each wave streams its 16 columns' weights with no further barrier: the weights are
// the row operand (lane: one column, 8 consecutive k, 16 bytes straight from the weight row), eight
// 32-wide k-blocks in flight per wave (a block's registers are refilled with the block 8 ahead as
// soon as its products are issued), the X pieces from LDS the column operand. When the column
// groups alone would not fill the chip, K is cut into S slices (split-K): each slice's 128 x 16
// tile and its rows' sums of squares go to the workspace with device-scope stores, and the last
// slice of the column group to finish (a ticket, returned to zero) reads the S tiles (all loads of
// a thread in flight together) and adds them in slice order, then runs the epilogue, so the result
// does not depend on which slice finishes first.
// ---------------------------------------------------------------------------------------------
constexpr int MC = 128;            // columns per workgroup
constexpr int MWV = 8;             // waves
constexpr int MTH = 64 * MWV;      // threads
constexpr int MKMAX = 512;         // largest slice of K
constexpr int MROW = MKMAX + 8;    // LDS row pitch in bf16 (1040 bytes: rows start 4 banks apart)
constexpr int MWIN = 8;            // k-blocks in flight per wave
constexpr int MTILE = MC * 16;     // one slice's partial tile (floats)
constexpr int MSLOT = MTILE + 16;  // + the rows' sums of squares
constexpr int MTARGET = 512;       // workgroups a launch aims for (2 resident per CU)
constexpr int MSMAX = 32;          // most slices
// Workspace layout, the same for every shape so that products of different shapes can share one
// workspace: MUNITS ticket counters (zero between calls), then the slice partials.
constexpr int MUNITS = 4096;       // most column groups x row tiles
constexpr size_t MPART_OFF = (size_t)MUNITS * 4;

// First column of column group w (two blocks of 64 columns, P apart).
__device__ __forceinline__ int first_col_m(const GArgs& a, int w) {
  const int per = a.P / 64;  // column groups per pairing period
  return (w / per) * a.period + (w % per) * 64;
}

__global__ void __launch_bounds__(MTH) dec_gemv_mfma_kernel(GArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[3][16][MROW];
  __shared__ float s_y[MC][17];  // the tile: [column][row], padded
  __shared__ float s_ss[16];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = blockIdx.x / a.S, slice = blockIdx.x % a.S;
  const int rt = blockIdx.y, m0 = rt * 16;
  const int c0 = first_col_m(a, grp);
  const int nkb = a.K / 32;
  const int kb0 = (int)((int64_t)nkb * slice / a.S), kb1 = (int)((int64_t)nkb * (slice + 1) / a.S);
  const int klen = 32 * (kb1 - kb0);

  // X slice: thread t takes row t / 32 and k = 4 (t % 32) + 128 j of the slice (loads first, so
  // that waiting for them does not wait for the weight window issued after them)
  const int xr = tid >> 5, xk = 4 * (tid & 31);
  const bool xok = m0 + xr < a.M;
  const float* xsrc = a.X + (int64_t)min(m0 + xr, a.M - 1) * a.K + 32 * kb0 + xk;
  f32x4 xv[MKMAX / 128], gv[MKMAX / 128];
#pragma unroll
  for (int j = 0; j < MKMAX / 128; ++j) {
    const bool in = xk + 128 * j < klen;
    xv[j] = in ? *reinterpret_cast<const f32x4*>(xsrc + 128 * j) : f32x4{0.f, 0.f, 0.f, 0.f};
    gv[j] = (in && a.g) ? *reinterpret_cast<const f32x4*>(a.g + 32 * kb0 + xk + 128 * j)
                        : f32x4{1.f, 1.f, 1.f, 1.f};
  }
  // the weight window: k-blocks kb0 .. kb0 + 7 of this lane's column (clamped into the slice)
  const int wcol = min(c0 + (wave >> 2) * a.P + (wave & 3) * 16 + (lane & 15), a.N - 1);
  const uint16_t* wrow = static_cast<const uint16_t*>(a.W) + (int64_t)wcol * a.K + 8 * (lane >> 4);
  auto wload = [&](int kb) { return *reinterpret_cast<const u32x4*>(wrow + (int64_t)min(kb, kb1 - 1) * 32); };
  u32x4 w[MWIN];
#pragma unroll
  for (int i = 0; i < MWIN; ++i) w[i] = wload(kb0 + i);

  // split X into LDS; the rows' sums of squares from the same values
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MKMAX / 128; ++j) {
    f32x4 x = xok ? xv[j] : f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.g) {
      ss = fmaf(x[0], x[0], fmaf(x[1], x[1], fmaf(x[2], x[2], fmaf(x[3], x[3], ss))));
      x *= gv[j];
    }
    uint32_t p[3][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t h = bf16_rne(x[e]);
      const float r1 = x[e] - bf16_bits_to_f32(h);  // exact
      const uint32_t m = bf16_rne(r1);
      const float r2 = r1 - bf16_bits_to_f32(m);    // exact, at most 8 significant bits
      p[0][e] = h;
      p[1][e] = m;
      p[2][e] = bf16_rne(r2);
    }
    if (xk + 128 * j < klen) {
#pragma unroll
      for (int pc = 0; pc < 3; ++pc)
        *reinterpret_cast<uint2*>(&xs[pc][xr][xk + 128 * j]) =
            make_uint2(p[pc][0] | (p[pc][1] << 16), p[pc][2] | (p[pc][3] << 16));
    }
  }
  // row xr's k are the 32 lanes of one half-wave
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((lane & 31) == 0) s_ss[xr] = ss;
  __syncthreads();

  f32x4 acc[3];
#pragma unroll
  for (int pc = 0; pc < 3; ++pc) acc[pc] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* xb = &xs[0][lane & 15][8 * (lane >> 4)];
  for (int base = kb0; base < kb1; base += MWIN) {
#pragma unroll
    for (int i = 0; i < MWIN; ++i) {
      const int kb = base + i;
      if (kb < kb1) {
        const int kk = 32 * (kb - kb0);
#pragma unroll
        for (int pc = 0; pc < 3; ++pc)
          acc[pc] = mfma_bf16(w[i], *reinterpret_cast<const u32x4*>(xb + pc * 16 * MROW + kk), acc[pc]);
        if (kb + MWIN < kb1) w[i] = wload(kb + MWIN);
      }
    }
  }
  // the wave's 16 x 16 tile: lane holds columns 4 (lane / 16) + r, row lane % 16
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int cl = (wave >> 2) * 64 + (wave & 3) * 16 + 4 * (lane >> 4) + r;
    s_y[cl][lane & 15] = acc[0][r] + (acc[1][r] + acc[2][r]);
  }
  __syncthreads();

  if (a.S > 1) {
    float* mine = a.part + (((int64_t)rt * a.groups + grp) * a.S + slice) * MSLOT;
#pragma unroll
    for (int i = 0; i < MTILE / MTH; ++i) {
      const int o = tid + MTH * i;
      store_coherent(mine + o, s_y[o >> 4][o & 15]);
    }
    if (tid < 16) store_coherent(mine + MTILE + tid, s_ss[tid]);
    wait_vm<0>();
    __syncthreads();
    if (tid == 0) {
      unsigned* cnt = a.counters + rt * a.groups + grp;
      const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = old == (unsigned)(a.S - 1);
      if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    // last slice: thread t takes outputs t + 512 i of every slice, 8 slices' loads at a time
    const float* base = a.part + ((int64_t)rt * a.groups + grp) * a.S * MSLOT;
    float t[MTILE / MTH + 1];
#pragma unroll
    for (int i = 0; i <= MTILE / MTH; ++i) t[i] = 0.f;
    for (int s0 = 0; s0 < a.S; s0 += 8) {
      float v[8][MTILE / MTH + 1];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* sl = base + (int64_t)min(s0 + u, a.S - 1) * MSLOT;
#pragma unroll
        for (int i = 0; i < MTILE / MTH; ++i) v[u][i] = load_f32<true>(sl + tid + MTH * i);
        v[u][MTILE / MTH] = tid < 16 ? load_f32<true>(sl + MTILE + tid) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < a.S) {
#pragma unroll
          for (int i = 0; i <= MTILE / MTH; ++i) t[i] += v[u][i];
        }
    }
#pragma unroll
    for (int i = 0; i < MTILE / MTH; ++i) {
      const int o = tid + MTH * i;
      s_y[o >> 4][o & 15] = t[i];
    }
    if (tid < 16) s_ss[tid] = t[MTILE / MTH];
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < MTILE / MTH; ++i) {
    const int o = tid + MTH * i;
    const int cl = o >> 4, row = o & 15;
    const float inv = a.g ? 1.0f / sqrtf(s_ss[row] / (float)a.K + a.eps) : 1.f;
    const float y = s_y[cl][row] * inv, partner = s_y[cl ^ 64][row] * inv;
    const int col = c0 + (cl >= 64 ? a.P + cl - 64 : cl);
    if (m0 + row < a.M && col < a.N) dec_epilogue(a, m0 + row, col, y, partner, cl < 64);
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

DecPlan plan_dec_gemv(int epi, int w_bf16, int N, int K, int M) {
  DecPlan p{};
  const int P = epi == DEC_SWIGLU ? N / 2 : 64;
  p.mfma = w_bf16 && K % 32 == 0 && P % 64 == 0 && (epi != DEC_SWIGLU || N % 128 == 0);
  if (!p.mfma) return p;
  p.groups = (epi == DEC_STORE || epi == DEC_ADD) ? (N + MC - 1) / MC : N / MC;
  p.row_tiles = (M + 15) / 16;
  const int units = p.groups * p.row_tiles, nkb = K / 32;
  const int s_min = (nkb + MKMAX / 32 - 1) / (MKMAX / 32);  // slices of at most 512
  const int s_max = std::max(s_min, nkb / 8);                 // and, by choice, at least 256
  p.S = std::min(std::max((MTARGET + units - 1) / units, s_min), s_max);
  if (p.S > MSMAX) {  // K too long for the slices the kernel handles
    p.mfma = false;
    return p;
  }
  if (units > MUNITS) {
    p.mfma = false;
    return p;
  }
  p.ws_bytes = MPART_OFF + (p.S > 1 ? (size_t)units * p.S * MSLOT * 4 : 0);
  return p;
}

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
  const DecPlan p = plan_dec_gemv(d.epi, d.w_bf16, d.N, d.K, d.M);
  if (p.mfma && d.ws != nullptr) {
    a.P = d.epi == DEC_SWIGLU ? d.N / 2 : 64;
    a.period = d.epi == DEC_SWIGLU ? d.N : 128;
    a.S = p.S;
    a.groups = p.groups;
    a.counters = static_cast<unsigned*>(d.ws);
    a.part = reinterpret_cast<float*>(static_cast<char*>(d.ws) + MPART_OFF);
    hipLaunchKernelGGL(dec_gemv_mfma_kernel, dim3((unsigned)(p.groups * p.S), (unsigned)p.row_tiles),
                       dim3(MTH), 0, s, a);
    return hipGetLastError();
  }
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
