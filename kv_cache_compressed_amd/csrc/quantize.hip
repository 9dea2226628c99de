// KIVI-style quantisation of cached keys/values and residual appends.
//
// Compressor step of the method: the quantising drafter keeps every cached position and stores
// each entry with fewer bits ("VeriCache: making lossy KV compression exact", The Tradeoff
// VeriCache Is Trying to Escape; "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference",
// Key Contributions and Limitations). Keys: per channel over 32-token groups; values: per token
// over 32-channel groups; asymmetric min/max with round-half-even codes. Each arithmetic step is
// one correctly rounded float32 operation (division included), so the codes and metadata are
// bit-reproducible.
//
// One workgroup quantises one 32-token x 128-channel block of one (b, kv head) for both keys and
// values: the block is staged in LDS, 128 threads derive the per-channel key statistics and 128
// the per-(token, channel-group) value statistics, then every thread assembles whole packed
// words of the documented block layout (no atomics, no read-modify-write of codes).
#include "common.h"
#include "kernels.h"

namespace vc {

namespace {

struct QuantArgs {
  const void* k;
  const void* v;
  int64_t src_bh_stride;  // elements between consecutive (b, h) source slices
  int64_t t0;             // first token (multiple of 32)
  int src_dtype, meta_dtype, Hkv;
  int64_t tok_cap;
  uint8_t* k_codes;
  uint8_t* v_codes;
  void* k_meta;
  void* v_meta;
};

struct Stats {
  float scale, mn;
};

__device__ __forceinline__ Stats group_stats(float lo, float hi, float levels, bool meta_f16) {
  const float mn = meta_f16 ? f16_round_down(lo) : lo;
  float sc = __fdiv_rn(__fsub_rn(hi, mn), levels);
  if (meta_f16) sc = f16_round_up(sc);
  return {sc, mn};
}

__device__ __forceinline__ uint32_t code_of(float x, Stats st, float levels) {
  if (st.scale == 0.f) return 0u;
  float t = rintf(__fdiv_rn(__fsub_rn(x, st.mn), st.scale));
  t = fminf(fmaxf(t, 0.f), levels);
  return (uint32_t)t;
}

__device__ __forceinline__ void store_meta(void* base, int64_t idx, Stats st, bool meta_f16) {
  if (meta_f16) {
    reinterpret_cast<uint32_t*>(base)[idx] = pack_f16x2(st.scale, st.mn);  // exact: fp16 values
  } else {
    reinterpret_cast<float2*>(base)[idx] = make_float2(st.scale, st.mn);
  }
}

template <int BITS>
__global__ void __launch_bounds__(256) quantize_kernel(QuantArgs a) {
  constexpr int WORDS_PER_LANE = 2 * BITS;          // 32-bit words per lane of a block
  constexpr int BLOCK_WORDS = 64 * WORDS_PER_LANE;  // 256 (2-bit) or 512 (4-bit)
  constexpr int SLOTS = 16 / BITS;                  // codes per 16-bit half
  constexpr float LEVELS = (float)((1 << BITS) - 1);
  constexpr int ROW_BYTES = D * BITS / 8;

  __shared__ float sk[GROUP][D + 1];
  __shared__ float sv[GROUP][D + 1];
  __shared__ Stats kst[D];
  __shared__ Stats vst[GROUP][D / GROUP];

  const int tid = threadIdx.x;
  const int bh = blockIdx.y;
  const int64_t g = a.t0 / GROUP + blockIdx.x;           // absolute group index
  const int64_t src_base = (int64_t)bh * a.src_bh_stride + (int64_t)blockIdx.x * GROUP * D;
  const bool meta_f16 = a.meta_dtype == VC_F16;

  for (int e = tid; e < GROUP * D; e += 256) {
    const int t = e / D, c = e % D;
    sk[t][c] = load_as_f32(a.k, src_base + e, a.src_dtype);
    sv[t][c] = load_as_f32(a.v, src_base + e, a.src_dtype);
  }
  __syncthreads();

  if (tid < D) {  // key statistics: one channel over the group's 32 tokens
    float lo = sk[0][tid], hi = lo;
    for (int t = 1; t < GROUP; ++t) {
      lo = fminf(lo, sk[t][tid]);
      hi = fmaxf(hi, sk[t][tid]);
    }
    const Stats st = group_stats(lo, hi, LEVELS, meta_f16);
    kst[tid] = st;
    // key metadata is planar per group: 128 scales, then 128 mins
    const int64_t base = ((int64_t)bh * (a.tok_cap / GROUP) + g) * 2 * D;
    if (meta_f16) {
      static_cast<f16*>(a.k_meta)[base + tid] = (f16)st.scale;  // exact: fp16 values
      static_cast<f16*>(a.k_meta)[base + D + tid] = (f16)st.mn;
    } else {
      static_cast<float*>(a.k_meta)[base + tid] = st.scale;
      static_cast<float*>(a.k_meta)[base + D + tid] = st.mn;
    }
  } else {  // value statistics: one token over one 32-channel group
    const int t = (tid - D) / 4, cg = (tid - D) % 4;
    float lo = sv[t][cg * GROUP], hi = lo;
    for (int c = 1; c < GROUP; ++c) {
      lo = fminf(lo, sv[t][cg * GROUP + c]);
      hi = fmaxf(hi, sv[t][cg * GROUP + c]);
    }
    const Stats st = group_stats(lo, hi, LEVELS, meta_f16);
    vst[t][cg] = st;
    store_meta(a.v_meta, ((int64_t)bh * a.tok_cap + g * GROUP + t) * 4 + cg, st, meta_f16);
  }
  __syncthreads();

  uint32_t* kw = reinterpret_cast<uint32_t*>(a.k_codes + ((int64_t)bh * a.tok_cap + g * GROUP) * ROW_BYTES);
  uint32_t* vw = reinterpret_cast<uint32_t*>(a.v_codes + ((int64_t)bh * a.tok_cap + g * GROUP) * ROW_BYTES);
  for (int w = tid; w < BLOCK_WORDS; w += 256) {
    const int lane = w / WORDS_PER_LANE, u = w % WORDS_PER_LANE;
    const int i = lane % 16, gq = lane / 16;
    uint32_t kword = 0, vword = 0;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const int shift = 16 * hf + BITS * s;
        // keys
        int kt, kb, p;
        if (BITS == 2) {
          kt = 16 * (u / 2) + i;
          kb = 2 * (u % 2) + s / 4;
          p = s % 4;
        } else {
          kt = 16 * (u / 4) + i;
          kb = u % 4;
          p = s;
        }
        const int kc = 32 * kb + 8 * gq + 2 * p + hf;
        kword |= code_of(sk[kt][kc], kst[kc], LEVELS) << shift;
        // values
        int tile, pv;
        if (BITS == 2) {
          tile = 2 * u + s / 4;
          pv = s % 4;
        } else {
          tile = u;
          pv = s;
        }
        const int vc_ = 16 * tile + i;
        const int vt = 16 * (pv / 2) + 4 * gq + 2 * (pv % 2) + hf;
        vword |= code_of(sv[vt][vc_], vst[vt][vc_ / GROUP], LEVELS) << shift;
      }
    }
    kw[w] = kword;
    vw[w] = vword;
  }
}

struct AppendArgs {
  const void* k;
  const void* v;
  int64_t src_bh_stride, t0;
  int src_dtype, res_dtype, res_cap;
  void* k_res;
  void* v_res;
};

// One workgroup per (token, b*h); 128 threads = channels.
__global__ void __launch_bounds__(128) append_kernel(AppendArgs a) {
  const int c = threadIdx.x;
  const int i = blockIdx.x;
  const int bh = blockIdx.y;
  const int64_t src = (int64_t)bh * a.src_bh_stride + (int64_t)i * D + c;
  const int64_t slot = (a.t0 + i) % a.res_cap;
  const int64_t dst = ((int64_t)bh * a.res_cap + slot) * D + c;
  const float kx = load_as_f32(a.k, src, a.src_dtype);
  const float vx = load_as_f32(a.v, src, a.src_dtype);
  if (a.res_dtype == VC_F32) {
    static_cast<float*>(a.k_res)[dst] = kx;
    static_cast<float*>(a.v_res)[dst] = vx;
  } else {
    static_cast<f16*>(a.k_res)[dst] = (f16)kx;
    static_cast<f16*>(a.v_res)[dst] = (f16)vx;
  }
}

}  // namespace

hipError_t launch_quantize(const vc_kivi& c, const void* k, const void* v, int src_dtype,
                           int64_t src_bh_stride, int64_t t0, int64_t ntok, hipStream_t s) {
  QuantArgs a;
  a.k = k;
  a.v = v;
  a.src_bh_stride = src_bh_stride;
  a.t0 = t0;
  a.src_dtype = src_dtype;
  a.meta_dtype = c.meta_dtype;
  a.Hkv = c.Hkv;
  a.tok_cap = c.tok_cap;
  a.k_codes = static_cast<uint8_t*>(c.k_codes);
  a.v_codes = static_cast<uint8_t*>(c.v_codes);
  a.k_meta = c.k_meta;
  a.v_meta = c.v_meta;
  dim3 grid((unsigned)(ntok / GROUP), (unsigned)(c.B * c.Hkv));
  if (c.bits == 2)
    hipLaunchKernelGGL(quantize_kernel<2>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(quantize_kernel<4>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append(const vc_kivi& c, const void* k, const void* v, int src_dtype,
                         int64_t src_bh_stride, int64_t t0, int64_t ntok, hipStream_t s) {
  AppendArgs a;
  a.k = k;
  a.v = v;
  a.src_bh_stride = src_bh_stride;
  a.t0 = t0;
  a.src_dtype = src_dtype;
  a.res_dtype = c.res_dtype;
  a.res_cap = c.res_cap;
  a.k_res = c.k_res;
  a.v_res = c.v_res;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)ntok, (unsigned)(c.B * c.Hkv)), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace vc
