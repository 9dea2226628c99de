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
// the QK product, p_t s_tcg in the PV product) is prepared once per 32-token group: q s as an fp16
// hi + lo pair (scores keep ~22 significant bits), p s as one fp16 (the weights enter the output
// linearly).
//
// Work split. Workgroup = 4 waves on one (b, kv head) and one contiguous range of 32-token groups
// (a split); wave w takes every 4th group of the range and streams them through its own LDS ring
// with direct global -> LDS copies (several groups in flight, no registers held). With fp16
// metadata and up to 4 query heads per kv head, QK^T runs transposed against an LDS table of the
// group's q*s operands so each lane owns one head's scores (quant_split_t); the general form keeps
// a head's scores in CPH identical columns (quant_split). The residual tokens (n_q .. n_q+r-1, an
// fp16 or fp32 ring) form one extra split, run by the last workgroup of each (b, kv head) before a
// correspondingly smaller share of the groups, so every workgroup carries about the same work.
// Each split writes an unnormalised partial (o, m, l)
// with device-scope stores; the last workgroup of the (b, kv head) to finish (a ticket counter in
// the workspace) merges them with log-sum-exp, so one kernel does the whole call and no
// cache-wide fence is needed.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"

// Scratch of the no-allocation draft call (vc_draft_attn_quant_noalloc): the ticket counters and
// split partials a caller-owned workspace holds otherwise. One copy per GPU, held until the process
// ends; host code reaches it only through the address hipGetSymbolAddress returns per device.
static __device__ __align__(256) unsigned char scratch[vc::DRAFT_NOALLOC_SCRATCH_BYTES];

namespace vc {

namespace {

constexpr int WAVES = 4;
constexpr int THREADS = 64 * WAVES;
constexpr int RES_MAX = 512;           // residual ring slots handled by the residual split
constexpr int RES_UNITS = 5;           // work of one 32-token residual block, in quantised groups
constexpr float SCALE_QK = 256.0f;     // 2^8: magnitude headroom of the fp16 QK operand
constexpr float SCALE_PV = 256.0f;     // 2^8: same for the PV operand
constexpr float SUBNORMAL = 16777216.0f;  // 2^24: one fp16 subnormal step is 2^-24
constexpr float LAZY = 2.0f;           // log2 slack before the running max is moved
// Workgroups resident per CU (= waves per SIMD); the LDS of a CU (160 KB) is shared among them.
// 2-bit groups (3 KB) carry more compute per byte and need a third wave per SIMD to cover it;
// 4-bit groups (5 KB) stream faster with two waves and the deeper ring that leaves room for.
constexpr int wg_per_cu(int bits) { return bits == 2 ? 3 : 2; }
constexpr int NUM_CUS = 256;
constexpr int ring_wave_bytes(int bits) { return (160 * 1024 / wg_per_cu(bits) / WAVES) / 1024 * 1024; }
// LDS: residual split [q 8xD | p 8xRES_MAX | ml 16 | reduction WAVESx8xD] floats; the quantised
// split uses it for one 12 KB ring per wave and, after its loop, the wave merge.
constexpr int RES_SMEM_FLOATS = 8 * D + 8 * RES_MAX + 16 + WAVES * 8 * D;

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
  unsigned* counters;  // one ticket per (b, kv head); zero between calls
  int64_t tok_cap, n_q;
  int r, res_cap, res_dtype, q_dtype;
  int Hkv, Hq, G;
  int ngroups, splits, total_splits;  // splits = quantised-only workgroups; partials = splits + 2
  int nwg;                             // workgroups per (b, kv head) = splits + 1
  int64_t units;                       // work units: quantised groups + RES_UNITS per residual block
  float qscale;  // sm_scale * log2(e): scores are kept in log2 units inside the kernel
  const void* k_new;  // null, or residual token n_q + r - 1 to store before attending
  const void* v_new;
  int new_dtype;
  int64_t new_b_stride;   // elements between batch rows of k_new / v_new
  int64_t new_h_stride;   // elements between the kv heads of one batch row
  // Per batch row lengths (vc_draft_attn_quant_rows), in device memory: row b's quantised tokens
  // row_nq[b] and residual tokens row_r[b] + row_radd, clamped into the cache; null: the scalars.
  const int64_t* row_nq;
  const int32_t* row_r;
  int row_radd;
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


// Per-wave LDS ring for the quantised split: slot size, 16-byte-per-lane copies per slot, depth,
// and a small per-wave scratch area after the slots.
constexpr int DMA_NT = 2;  // cache policy of the ring copies: non-temporal (streamed once)
constexpr int WAVE_SCRATCH = 1024;
template <int BITS, bool META_F16>
struct RingPlan {
  static constexpr int CB = GROUP * D * BITS / 8;      // one group's key (or value) codes
  static constexpr int MB = META_F16 ? 512 : 1024;     // one group's key (or value) metadata
  static constexpr int SLOT = 2 * CB + 2 * MB;
  static constexpr int LOADS = SLOT / 1024;
  static constexpr int DEPTH = std::max(2, (ring_wave_bytes(BITS) - WAVE_SCRATCH) / SLOT);
  static constexpr int BYTES = DEPTH * SLOT + WAVE_SCRATCH;  // per wave
  static_assert(SLOT % 1024 == 0, "ring plan");
};

// Wait until at most `ahead` groups' copies (LOADS each) are still in flight: the copies of the
// group issued before them have then landed in LDS (see wait_vm).
template <int LOADS, int DEPTH>
__device__ __forceinline__ void wait_dma(int ahead) {
  if (DEPTH > 3 && ahead >= 3) wait_vm<3 * LOADS>();
  else if (DEPTH > 2 && ahead >= 2) wait_vm<2 * LOADS>();
  else if (ahead >= 1) wait_vm<LOADS>();
  else wait_vm<0>();
}

// The groups of one wave (g_begin + wave, + WAVES, ...) streamed through its LDS ring. A slot holds
// one group: key codes (CB bytes), value codes (CB), key metadata (MB), value metadata (MB), filled
// by LOADS 16-byte-per-lane copies; copy z lands at slot + 1024 z + 16 lane. Lane l's operand word
// u comes from source bytes 16 (l WPL/4 + u), so each lane reads its own words back from
// consecutive 16-byte LDS cells (no bank conflicts).
template <int BITS, bool META_F16>
struct GroupRing {
  using RP = RingPlan<BITS, META_F16>;
  static constexpr int WPL = 2 * BITS;  // packed code words per lane per group
  uint8_t* ring;
  const uint8_t* src[RP::LOADS];
  int64_t step[RP::LOADS];
  int g0, n;  // first group of this wave, number of groups

  __device__ GroupRing(const DQArgs& a, int bh, int g_begin, int g_end, float* smem, int wave, int lane) {
    ring = reinterpret_cast<uint8_t*>(smem) + wave * RP::BYTES;
    g0 = g_begin + wave;
    n = __builtin_amdgcn_readfirstlane(g0 < g_end ? (g_end - g0 + WAVES - 1) / WAVES : 0);  // wave-uniform
    const int64_t blk0 = (int64_t)bh * a.tok_cap;  // token 0 of this (b, kv head)
    constexpr int ROW_BYTES = D * BITS / 8;
    const uint8_t* kc = a.k_codes + blk0 * ROW_BYTES + lane * 16 * (WPL / 4);
    const uint8_t* vc = a.v_codes + blk0 * ROW_BYTES + lane * 16 * (WPL / 4);
    const uint8_t* km = static_cast<const uint8_t*>(a.k_meta) + (int64_t)bh * (a.tok_cap / GROUP) * RP::MB;
    const uint8_t* vm = static_cast<const uint8_t*>(a.v_meta) + blk0 * (RP::MB / GROUP);
#pragma unroll
    for (int u = 0; u < WPL / 4; ++u) {
      src[u] = kc + 16 * u;
      src[WPL / 4 + u] = vc + 16 * u;
      step[u] = step[WPL / 4 + u] = RP::CB;
    }
    if (META_F16) {  // one copy: lanes 0-31 key metadata, lanes 32-63 value metadata
      src[WPL / 2] = lane < 32 ? km + lane * 16 : vm + (lane - 32) * 16;
      step[WPL / 2] = RP::MB;
    } else {
      src[WPL / 2] = km + lane * 16;
      src[WPL / 2 + 1] = vm + lane * 16;
      step[WPL / 2] = step[WPL / 2 + 1] = RP::MB;
    }
  }
  __device__ uint8_t* slot(int i) const { return ring + (i % RP::DEPTH) * RP::SLOT; }
  __device__ uint8_t* scratch() const { return ring + RP::DEPTH * RP::SLOT; }
  // Copy local group gi into the slot of local group i.
  __device__ void issue(int i, int gi) {
    const int g = g0 + WAVES * gi;
    uint8_t* dst = slot(i);
#pragma unroll
    for (int z = 0; z < RP::LOADS; ++z) copy16_to_lds<DMA_NT>(src[z] + g * step[z], dst + 1024 * z);
  }
  __device__ void issue(int i) { issue(i, i); }
  // The first DEPTH-1 groups, as straight-line code (a wave with fewer groups re-copies its last
  // one into the spare slots), so that the compiler can count the copies in flight; then wait
  // until only those copies are outstanding: everything loaded before start() has arrived.
  __device__ void start() {
    if (n == 0) {  // nothing to copy: only the loads issued before start() are outstanding
      wait_vm<0>();
      return;
    }
#pragma unroll
    for (int i = 0; i < RP::DEPTH - 1; ++i) issue(i, min(i, n - 1));
    wait_vm<(RP::DEPTH - 1) * RP::LOADS>();
  }
  // Refill the slot freed by group i-1, wait for group i's copies, return its slot.
  __device__ uint8_t* acquire(int i) {
    if (i + RP::DEPTH - 1 < n) issue(i + RP::DEPTH - 1);
    wait_dma<RP::LOADS, RP::DEPTH>(min(RP::DEPTH - 1, n - 1 - i));
    return slot(i);
  }
  // This lane's packed key and value code words of the group in slot sl.
  __device__ void codes(const uint8_t* sl, int lane, uint32_t* kwd, uint32_t* vwd) const {
#pragma unroll
    for (int u = 0; u < WPL / 4; ++u) {
      const u32x4 kv4 = *reinterpret_cast<const u32x4*>(sl + 1024 * u + 16 * lane);
      const u32x4 vv4 = *reinterpret_cast<const u32x4*>(sl + 1024 * (WPL / 4 + u) + 16 * lane);
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        kwd[4 * u + z] = kv4[z];
        vwd[4 * u + z] = vv4[z];
      }
    }
  }
};

// Progress-based wave priority. Waves issue oldest first, so with equal shares the waves that
// started early race ahead and the CU's last waves run alone at the end, with too few loads in
// flight to keep HBM busy. Every wave starts at the top level and steps down as it works through
// its share (at 1/3, 2/3 and 5/6), so early starters yield to late ones and the waves of a CU
// finish close together.
struct ProgressPriority {
  int q1, q2, q3;
  __device__ explicit ProgressPriority(int n) : q1(n / 3), q2(2 * n / 3), q3(5 * n / 6) {}
  __device__ void step(int i) const {
    if (i == q1) __builtin_amdgcn_s_setprio(2);
    if (i == q2) __builtin_amdgcn_s_setprio(1);
    if (i == q3) __builtin_amdgcn_s_setprio(0);
  }
};

// The four waves' results, staged in LDS as m [WAVES][8] (natural log), l [WAVES][8] and
// o [WAVES][8][D], merged into this split's partial (device-scope stores, read back by the merge).
__device__ void write_split_partial(const DQArgs& a, int bh, int split, const float* smem) {
  const float* s_m = smem;
  const float* s_l = smem + WAVES * 8;
  const float* s_o = smem + 2 * WAVES * 8;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  for (int idx = threadIdx.x; idx < a.G * D; idx += THREADS) {
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
    store_coherent(a.part_o + (row * a.total_splits + split) * D + c, o);
    if (c == 0) {
      store_coherent(a.part_ml + (row * a.total_splits + split) * 2 + 0, m);
      store_coherent(a.part_ml + (row * a.total_splits + split) * 2 + 1, l);
    }
  }
}

// One split of quantised groups, general form (fp32 metadata, or up to 8 query heads per kv head).
// Every column of a query head h carries the same scores (the head's CPH columns j = CPH*h ..
// CPH*h + CPH-1 get identical QK operands), so no lane ever needs another lane's score. q*s enters
// the QK product as an fp16 hi part and an fp16 lo part, in two matrix products accumulated into
// the same registers (scores keep ~22 significant bits; a single fp16 would move them by up to
// ~1e-3 in log2 units at outlier channels).
//   CPH == 4 (G <= 4): PV column CPH*h + cg carries p * s_cg for value channel group cg, so one PV
//                      operand serves all eight channel tiles (each lane prepares 8 products).
//   CPH == 2 (G <= 8): PV uses one operand per channel group (both columns of the head alike).
// With fp16 metadata the key bias sum_c q_c m_gc is a matrix product too: q (bf16/fp16 values are
// exact in fp16) against the group's fp16 mins, exact products accumulated in fp32.
template <int BITS, bool META_F16, int CPH>
__device__ void quant_split(const DQArgs& a, int bh, int g_begin, int g_end, int split, float* smem) {
  constexpr int WPL = 2 * BITS;
  constexpr int MB = RingPlan<BITS, META_F16>::MB;
  constexpr int NBP = CPH == 4 ? 1 : 4;  // PV B operands per group
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, gq = lane >> 4;
  const int h = j / CPH, k = j % CPH;  // query head of this column, slot within the head
  const bool active = h < a.G;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int hq = kvh * a.G + h;

  // Query of this lane's 32 channels (c = 32 kb + 8 gq + e) in log2 units, pre-multiplied by the
  // fp16 headroom scale and divided by the slot-position power of element e; and, for the bias
  // product, the raw query as fp16 pairs.
  float qs[32];
  u32x4 qh[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    float qv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 32 * kb + 8 * gq + e;
      qv[e] = active ? load_as_f32(a.q, ((int64_t)b * a.Hq + hq) * D + c, a.q_dtype) : 0.f;
      qs[kb * 8 + e] = qv[e] * a.qscale * (SCALE_QK * cls_inv<BITS>(e));
    }
    qh[kb] = u32x4{pack_f16x2(qv[0], qv[1]), pack_f16x2(qv[2], qv[3]), pack_f16x2(qv[4], qv[5]),
                   pack_f16x2(qv[6], qv[7])};
  }

  float m_run = -INFINITY, l_lane = 0.f;
  float bv[4] = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  GroupRing<BITS, META_F16> gr(a, bh, g_begin, g_end, smem, wave, lane);
  gr.start();
  const ProgressPriority prio(gr.n);
  for (int i = 0; i < gr.n; ++i) {
    prio.step(i);
    const uint8_t* sl = gr.acquire(i);
    const uint8_t* mb = sl + 2 * RingPlan<BITS, META_F16>::CB;
    uint32_t kwd[WPL], vwd[WPL];
    gr.codes(sl, lane, kwd, vwd);
    // ---- key bias and QK -------------------------------------------------------------------
    // key metadata in LDS: scales at [c * ESZ], mins at [(D + c) * ESZ]
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    float bias;
    if constexpr (META_F16) {
      f32x4 sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const u32x4 mn = *reinterpret_cast<const u32x4*>(mb + (D + 32 * kb + 8 * gq) * 2);
        sb = mfma_f16(mn, qh[kb], sb);  // every row: sum_c m_c q_c (exact products)
      }
      bias = sb[0] * a.qscale;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        u32x4 bhi, blo;
        const u32x4 sc = *reinterpret_cast<const u32x4*>(mb + (32 * kb + 8 * gq) * 2);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float q0 = qs[kb * 8 + 2 * e2], q1 = qs[kb * 8 + 2 * e2 + 1];
          bhi[e2] = mix_mul2(q0, q1, sc[e2]);
          blo[e2] = mix_rem2(q0, q1, sc[e2], bhi[e2]);
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const u32x4 av = BITS == 2 ? unpack2(kwd[2 * tb + kb / 2], kb & 1) : unpack4(kwd[4 * tb + kb]);
          s[tb] = mfma_f16(av, bhi, s[tb]);
          s[tb] = mfma_f16(av, blo, s[tb]);
        }
      }
    } else {
      float bias_e[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float4* sp = reinterpret_cast<const float4*>(mb + (32 * kb + 8 * gq) * 4);
        const float4* mp = reinterpret_cast<const float4*>(mb + (D + 32 * kb + 8 * gq) * 4);
        const float4 s0 = sp[0], s1 = sp[1], m0 = mp[0], m1 = mp[1];
        const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const float mn[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        float hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float qt = qs[kb * 8 + e] * sc[e];
          hi[e] = (float)(f16)qt;
          lo[e] = qt - hi[e];
          bias_e[e] += qs[kb * 8 + e] * mn[e];
        }
        const u32x4 bhi = u32x4{pack_f16x2(hi[0], hi[1]), pack_f16x2(hi[2], hi[3]),
                                pack_f16x2(hi[4], hi[5]), pack_f16x2(hi[6], hi[7])};
        const u32x4 blo = u32x4{pack_f16x2(lo[0], lo[1]), pack_f16x2(lo[2], lo[3]),
                                pack_f16x2(lo[4], lo[5]), pack_f16x2(lo[6], lo[7])};
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const u32x4 av = BITS == 2 ? unpack2(kwd[2 * tb + kb / 2], kb & 1) : unpack4(kwd[4 * tb + kb]);
          s[tb] = mfma_f16(av, bhi, s[tb]);
          s[tb] = mfma_f16(av, blo, s[tb]);
        }
      }
      bias = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) bias += bias_e[e] * (1.0f / (SCALE_QK * cls_inv<BITS>(e)));
      bias = sum_over_rows(bias);
    }
    // ---- scores (log2 units) and online softmax with a lazily moved reference max -----------
    // score = s * 2^16 + bias is monotonic in s, so the column max is taken on the raw sums
    constexpr float KS = SUBNORMAL / SCALE_QK;
    const float sraw = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                             fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    const float mx = fmaf(max_over_rows(sraw), KS, bias);
    // The reference max moves only when a score exceeds it by more than LAZY (log2 units), so
    // weights stay <= 2^LAZY and most groups skip the rescale of the accumulators.
    const bool move = mx > m_run + LAZY;
    if (__builtin_amdgcn_ballot_w64(move)) {
      const float m_new = move ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_lane *= alpha;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] *= alpha;
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) bv[cg] *= alpha;
    }
    // weights (columns of absent heads carry finite junk that is never written out)
    float sc[8];
    const float off = bias - m_run;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sc[e] = __builtin_amdgcn_exp2f(fmaf(s[e >> 2][e & 3], KS, off));
      psum += sc[e];
    }
    l_lane += psum;
    // ---- PV operand(s) and value bias --------------------------------------------------------
    // Element e of this lane's B operand is token 16*(e/4) + 4*gq + e%4 = sc[e]'s token.
    u32x4 bp[NBP];
    if (CPH == 4) {
      const int cg = k;  // this column's value channel group
      if (META_F16) {
        uint32_t wv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tok = 16 * (e >> 2) + 4 * gq + (e & 3);
          wv[e] = *reinterpret_cast<const uint32_t*>(mb + MB + tok * 16 + cg * 4);
          bv[0] = mix_fma_hi(sc[e], wv[e], bv[0]);
        }
        uint32_t pw[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          pw[e2] = mix_mul_pair(sc[2 * e2] * (SCALE_PV * cls_inv<BITS>(2 * e2)), wv[2 * e2],
                                sc[2 * e2 + 1] * (SCALE_PV * cls_inv<BITS>(2 * e2 + 1)), wv[2 * e2 + 1]);
        bp[0] = u32x4{pw[0], pw[1], pw[2], pw[3]};
      } else {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tok = 16 * (e >> 2) + 4 * gq + (e & 3);
          const float2 w = *reinterpret_cast<const float2*>(mb + MB + tok * 32 + cg * 8);
          pv[e] = sc[e] * w.x * (SCALE_PV * cls_inv<BITS>(e));
          bv[0] += sc[e] * w.y;
        }
        bp[0] = u32x4{pack_f16x2(pv[0], pv[1]), pack_f16x2(pv[2], pv[3]),
                      pack_f16x2(pv[4], pv[5]), pack_f16x2(pv[6], pv[7])};
      }
    } else {
      float pv[4][8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = 16 * (e >> 2) + 4 * gq + (e & 3);
        float svals[4], mvals[4];
        if (META_F16) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(mb + MB + tok * 16);
#pragma unroll
          for (int cg = 0; cg < 4; ++cg) {
            svals[cg] = f16_bits_to_f32(w[cg] & 0xffffu);
            mvals[cg] = f16_bits_to_f32(w[cg] >> 16);
          }
        } else {
          const float4* p4 = reinterpret_cast<const float4*>(mb + MB + tok * 32);
          const float4 w0 = p4[0], w1 = p4[1];
          svals[0] = w0.x; mvals[0] = w0.y; svals[1] = w0.z; mvals[1] = w0.w;
          svals[2] = w1.x; mvals[2] = w1.y; svals[3] = w1.z; mvals[3] = w1.w;
        }
        const float pes = sc[e] * (SCALE_PV * cls_inv<BITS>(e));
#pragma unroll
        for (int cg = 0; cg < 4; ++cg) {
          pv[cg][e] = pes * svals[cg];
          bv[cg] += sc[e] * mvals[cg];
        }
      }
#pragma unroll
      for (int cg = 0; cg < NBP; ++cg)
        bp[cg] = u32x4{pack_f16x2(pv[cg][0], pv[cg][1]), pack_f16x2(pv[cg][2], pv[cg][3]),
                       pack_f16x2(pv[cg][4], pv[cg][5]), pack_f16x2(pv[cg][6], pv[cg][7])};
    }
    // ---- PV on the matrix cores: eight 16-channel tiles, K = the group's 32 tokens ------
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const u32x4 av = BITS == 2 ? unpack2(vwd[t / 2], t & 1) : unpack4(vwd[t]);
      acc[t] = mfma_f16(av, bp[CPH == 4 ? 0 : t / 2], acc[t]);
    }
  }

  // ---- wave result -> LDS: m [WAVES][8], l [WAVES][8], o [WAVES][8][D] --------------------
  __syncthreads();  // every wave is done with its ring
  float* s_m = smem;
  float* s_l = smem + WAVES * 8;
  float* s_o = smem + 2 * WAVES * 8;
  const float l_tot = sum_over_rows(l_lane);
  float bvt[4];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) bvt[cg] = sum_over_rows(bv[cg]);
  if (active && k == 0 && gq == 0) {
    s_m[wave * 8 + h] = m_run * LN2;  // natural-log units from here on
    s_l[wave * 8 + h] = l_tot;
  }
  if (CPH == 4) {
    // lane (head h, column group cg = k) owns channel tiles 2cg and 2cg + 1
    if (active) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t / 2 != k) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = 16 * t + 4 * gq + r;
          s_o[(wave * 8 + h) * D + c] = acc[t][r] * (SUBNORMAL / SCALE_PV) + bvt[0];
        }
      }
    }
  } else if (active && k == 0) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 16 * t + 4 * gq + r;
        s_o[(wave * 8 + h) * D + c] = acc[t][r] * (SUBNORMAL / SCALE_PV) + bvt[c / GROUP];
      }
  }
  __syncthreads();
  write_split_partial(a, bh, split, smem);
}

// Row reductions over the 16 lanes of a DPP row (lanes 16 gq .. 16 gq + 15).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Max over the row for values that are never NaN (scores: finite, or -inf for no token): four
// DPP-operand maxima. Written out because the fmaxf form compiles to a DPP move, a quieting max
// and the max per step (12 instructions); each DPP read of a register a vector instruction just
// wrote needs two wait states (the s_nop 1).
__device__ __forceinline__ float row16_max(float x) {
  float y;
  asm("s_nop 1\n\t"
      "v_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf"
      : "=&v"(y)
      : "v"(x));
  return y;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x124>(x);
  return x + dpp_mov<0x128>(x);
}

// One split of quantised groups, fast form for fp16 metadata and up to 4 query heads per kv head.
// QK^T is computed transposed: the q*s operand is the row operand, with row 4h + r carrying head
// h's fp16 hi part (r even) or lo part (r odd), built once per (head, channel) per group by the
// wave into an LDS table; the key codes are the column operand (column = token). Lane (j, gq) then
// holds head gq's hi and lo sums for token j of each 16-token tile, so a score costs one add and no
// lane computes another lane's softmax work. The weights go through a 512-byte LDS exchange into
// the PV operand layout (column 4h + cg carries p * s_cg of value channel group cg), the same PV
// product as the general form.
template <int BITS>
__device__ void quant_split_t(const DQArgs& a, int bh, int g_begin, int g_end, int split, float* smem) {
  constexpr int WPL = 2 * BITS;
  constexpr int MB = RingPlan<BITS, true>::MB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, gq = lane >> 4;
  const int hp = j >> 2, cg = j & 3;  // PV layout: column j = 4 hp + cg
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int64_t qrow0 = (int64_t)b * a.Hq + kvh * a.G;  // query row of head 0 of this kv head

  // The query loads go out first, then the first groups' copies; both are in flight together.
  const int th = lane >> 4, tc = lane & 15;  // table lane: head th, 8-channel chunk tc
  // (lanes of absent heads read head G-1 and zero it afterwards)
  // The query loads are untracked by the compiler; start() waits for them explicitly while the
  // ring copies stay in flight (the register dependence below keeps every read after that wait).
  Raw8 qraw[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    qraw[kb] = load8_raw_untracked(a.q, (qrow0 + min(hp, a.G - 1)) * D + 32 * kb + 8 * gq, a.q_dtype);
  Raw8 traw = load8_raw_untracked(a.q, (qrow0 + min(th, a.G - 1)) * D + 8 * tc, a.q_dtype);
  GroupRing<BITS, true> gr(a, bh, g_begin, g_end, smem, wave, lane);
  gr.start();
  // tie the query registers to the wait that retired their loads
  asm volatile("" : "+v"(qraw[0].a), "+v"(qraw[0].b), "+v"(qraw[1].a), "+v"(qraw[1].b), "+v"(qraw[2].a),
               "+v"(qraw[2].b), "+v"(qraw[3].a), "+v"(qraw[3].b), "+v"(traw.a), "+v"(traw.b));
  float qv[4][8], qt[8];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    cvt8(qraw[kb], a.q_dtype, qv[kb]);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[kb][e] = hp < a.G ? qv[kb][e] : 0.f;
  }
  cvt8(traw, a.q_dtype, qt);
#pragma unroll
  for (int e = 0; e < 8; ++e) qt[e] = th < a.G ? qt[e] : 0.f;

  // Bias operand: row j carries head j/4's query (channels 32 kb + 8 gq + e) as fp16.
  u32x4 qh[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    qh[kb] = u32x4{pack_f16x2(qv[kb][0], qv[kb][1]), pack_f16x2(qv[kb][2], qv[kb][3]),
                   pack_f16x2(qv[kb][4], qv[kb][5]), pack_f16x2(qv[kb][6], qv[kb][7])};
  // Table operand source: query in log2 units times the fp16 headroom scale over the
  // slot-position power of element e.
  float qs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qs[e] = qt[e] * a.qscale * (SCALE_QK * cls_inv<BITS>(e));

  float m_run = -INFINITY;  // head gq
  float l_lane = 0.f;       // head gq, this lane's tokens
  float bv = 0.f;           // PV layout: value bias of column j
  f32x4 acc[8];             // PV layout
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // [4 heads][SP_PITCH] weights (32 tokens, padded so the four heads' rows start in different
  // banks), then [4] rescale factors
  constexpr int SP_PITCH = 36;
  float* s_p = reinterpret_cast<float*>(gr.scratch());
  float* s_alpha = s_p + 4 * SP_PITCH;
  // q*s table cells (16 bytes): head h, part (0 hi, 1 lo), 8-channel chunk c at
  // 16 (4 part + h) + (c ^ (4 part + h)): the eight (head, part) rows a QK operand read touches
  // for one chunk land in eight different bank groups
  const int trow_s = 4 * (j & 1) + (j >> 2);
  int tcell[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) tcell[kb] = 16 * trow_s + ((4 * kb + gq) ^ trow_s);
  const ProgressPriority prio(gr.n);
  // One group in the slot sl.
  auto group = [&](uint8_t* sl) {
    const uint8_t* mb = sl + 2 * RingPlan<BITS, true>::CB;
    uint32_t kwd[WPL], vwd[WPL];
    gr.codes(sl, lane, kwd, vwd);
    // ---- key bias: rows 4h.. carry head h's sum_c q_c m_c (exact products) -------------------
    f32x4 sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const u32x4 mn = *reinterpret_cast<const u32x4*>(mb + (D + 32 * kb + 8 * gq) * 2);
      sb = mfma_f16(qh[kb], mn, sb);
    }
    const float bias = sb[0] * a.qscale;  // head gq
    // ---- q*s table over this slot's code words (already in registers; the slot is refilled
    // only after this group), cells as above (hi parts in rows 0-3, lo parts in rows 4-7)
    u32x4* tbl = reinterpret_cast<u32x4*>(sl);
    {
      const u32x4 sc = *reinterpret_cast<const u32x4*>(mb + (lane & 15) * 16);
      u32x4 thi, tlo;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        thi[e2] = mix_mul2(qs[2 * e2], qs[2 * e2 + 1], sc[e2]);
        tlo[e2] = mix_rem2(qs[2 * e2], qs[2 * e2 + 1], sc[e2], thi[e2]);
      }
      tbl[16 * th + (tc ^ th)] = thi;
      tbl[64 + 16 * th + (tc ^ (4 + th))] = tlo;
      wave_lds_order();
    }
    // ---- QK^T transposed: s[tb][r] = head gq, part r, token 16 tb + j -------------------------
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};

#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const u32x4 aq = tbl[tcell[kb]];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const u32x4 bk = BITS == 2 ? unpack2(kwd[2 * tb + kb / 2], kb & 1) : unpack4(kwd[4 * tb + kb]);
        s[tb] = mfma_f16(aq, bk, s[tb]);
      }
    }
    // ---- scores (log2 units), lazily moved reference max, weights ----------------------------
    constexpr float KS = SUBNORMAL / SCALE_QK;
    const float z0 = s[0][0] + s[0][1], z1 = s[1][0] + s[1][1];
    const float mx = fmaf(row16_max(fmaxf(z0, z1)), KS, bias);  // score is monotonic in z
    const bool move = mx > m_run + LAZY;
    if (__builtin_amdgcn_ballot_w64(move)) {
      const float m_new = move ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_lane *= alpha;
      if (j == 0) s_alpha[gq] = alpha;
      wave_lds_order();
      const float ap = s_alpha[hp];
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] *= ap;
      bv *= ap;
    }
    const float off = bias - m_run;
    const float p0 = __builtin_amdgcn_exp2f(fmaf(z0, KS, off));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(z1, KS, off));
    l_lane += p0 + p1;
    s_p[gq * SP_PITCH + j] = p0;
    s_p[gq * SP_PITCH + 16 + j] = p1;
    wave_lds_order();
    // ---- PV operand: element e = token 16 (e/4) + 4 gq + e%4 of head hp ----------------------
    const float4 pa = *reinterpret_cast<const float4*>(s_p + hp * SP_PITCH + 4 * gq);
    const float4 pb = *reinterpret_cast<const float4*>(s_p + hp * SP_PITCH + 16 + 4 * gq);
    const float pe[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
    uint32_t wv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tok = 16 * (e >> 2) + 4 * gq + (e & 3);
      wv[e] = *reinterpret_cast<const uint32_t*>(mb + MB + tok * 16 + cg * 4);
      bv = mix_fma_hi(pe[e], wv[e], bv);
    }
    uint32_t pw[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2)
      pw[e2] = mix_mul_pair(pe[2 * e2] * (SCALE_PV * cls_inv<BITS>(2 * e2)), wv[2 * e2],
                            pe[2 * e2 + 1] * (SCALE_PV * cls_inv<BITS>(2 * e2 + 1)), wv[2 * e2 + 1]);
    const u32x4 bp = u32x4{pw[0], pw[1], pw[2], pw[3]};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const u32x4 av = BITS == 2 ? unpack2(vwd[t / 2], t & 1) : unpack4(vwd[t]);
      acc[t] = mfma_f16(av, bp, acc[t]);
    }
  };
  // Whole turns of the ring with the slot fixed at compile time (LDS addresses as immediate
  // offsets: i is a multiple of DEPTH there, so group i + u sits in slot u), then the remaining
  // groups.
  constexpr int DEPTH = RingPlan<BITS, true>::DEPTH;
  int i = 0;
  for (; i + DEPTH <= gr.n; i += DEPTH) {
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      prio.step(i + u);
      gr.acquire(i + u);
      group(gr.ring + u * RingPlan<BITS, true>::SLOT);
    }
  }
  for (; i < gr.n; ++i) {
    prio.step(i);
    group(gr.acquire(i));
  }

  // ---- wave result -> LDS: m [WAVES][8], l [WAVES][8], o [WAVES][8][D] --------------------
  __syncthreads();  // every wave is done with its ring
  float* s_m = smem;
  float* s_l = smem + WAVES * 8;
  float* s_o = smem + 2 * WAVES * 8;
  const float l_tot = row16_sum(l_lane);
  const float bvt = sum_over_rows(bv);
  if (j == 0 && gq < a.G) {
    s_m[wave * 8 + gq] = m_run * LN2;  // natural-log units from here on
    s_l[wave * 8 + gq] = l_tot;
  }
  // lane (head hp, column group cg) owns channel tiles 2cg and 2cg + 1
  if (hp < a.G) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t / 2 != cg) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s_o[(wave * 8 + hp) * D + 16 * t + 4 * gq + r] = acc[t][r] * (SUBNORMAL / SCALE_PV) + bvt;
    }
  }
  __syncthreads();
  write_split_partial(a, bh, split, smem);
}

// Residual tokens n_q .. n_q+r-1 from an fp16 ring, on the matrix cores: wave w takes every 4th
// block of 32 ring tokens. Keys go straight from their ring rows into the row operand of QK^T
// (fp16 keys times fp16-exact queries: exact products, fp32 sums); values are staged in LDS as
// channel-major token pairs for the PV product; softmax weights enter as fp16 hi + lo.
constexpr int RVT = 17;  // dwords per staged value row (16 token pairs + 1 pad)
static_assert(WAVES * D * RVT <= RES_SMEM_FLOATS && 2 * WAVES * 8 + WAVES * 8 * D <= RES_SMEM_FLOATS,
              "residual LDS");

__device__ void residual_split_mfma(const DQArgs& a, int bh, int split, float* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, gq = lane >> 4;
  const int cph = a.G <= 4 ? 4 : 2;
  const int h = j / cph, k = j % cph;
  const bool active = h < a.G;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int hq = kvh * a.G + min(h, a.G - 1);  // absent heads read head G-1, zeroed below
  u32x4 qh[4];
  Raw8 qraw[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) qraw[kb] = load8_raw(a.q, ((int64_t)b * a.Hq + hq) * D + 32 * kb + 8 * gq, a.q_dtype);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    float qv[8];
    cvt8(qraw[kb], a.q_dtype, qv);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = active ? qv[e] : 0.f;
    qh[kb] = u32x4{pack_f16x2(qv[0], qv[1]), pack_f16x2(qv[2], qv[3]), pack_f16x2(qv[4], qv[5]),
                   pack_f16x2(qv[6], qv[7])};
  }
  const f16* kres = static_cast<const f16*>(a.k_res) + (int64_t)bh * a.res_cap * D;
  const f16* vres = static_cast<const f16*>(a.v_res) + (int64_t)bh * a.res_cap * D;
  const int base = (int)(a.n_q % a.res_cap);
  uint32_t* vt = reinterpret_cast<uint32_t*>(smem) + wave * D * RVT;
  float m_run = -INFINITY, l_lane = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nblk = (a.r + 31) / 32;
  for (int blk = wave; blk < nblk; blk += WAVES) {
    const int t0 = blk * 32;
    // keys of tokens t0 + 16 tb + j into the row operand
    u32x4 kop[2][4];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int tt = t0 + 16 * tb + j;
      int slot = base + tt;
      if (slot >= a.res_cap) slot -= a.res_cap;
      const bool ok = tt < a.r;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        kop[tb][kb] = ok ? *reinterpret_cast<const u32x4*>(kres + (int64_t)slot * D + 32 * kb + 8 * gq)
                         : u32x4{0u, 0u, 0u, 0u};
    }
    // values, transposed to token pairs: lane (pair tp = lane % 16, channel quarter cq)
    {
      const int tp = lane & 15, cq = lane >> 4;
      u32x4 v0[4], v1[4];
#pragma unroll
      for (int z = 0; z < 2; ++z) {
        const int tt = t0 + 2 * tp + z;
        int slot = base + tt;
        if (slot >= a.res_cap) slot -= a.res_cap;
        const bool ok = tt < a.r;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          const u32x4 t = ok ? *reinterpret_cast<const u32x4*>(vres + (int64_t)slot * D + 32 * cq + 8 * w4)
                             : u32x4{0u, 0u, 0u, 0u};
          if (z == 0) v0[w4] = t; else v1[w4] = t;
        }
      }
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4)
#pragma unroll
        for (int zz = 0; zz < 4; ++zz) {
          const int c = 32 * cq + 8 * w4 + 2 * zz;
          vt[c * RVT + tp] = __builtin_amdgcn_perm(v1[w4][zz], v0[w4][zz], 0x05040100u);
          vt[(c + 1) * RVT + tp] = __builtin_amdgcn_perm(v1[w4][zz], v0[w4][zz], 0x07060302u);
        }
    }
    f32x4 s[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) c = mfma_f16(kop[tb][kb], qh[kb], c);
      s[tb] = c;
    }
    float sc[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tt = t0 + 16 * (e >> 2) + 4 * gq + (e & 3);
      const float v = tt < a.r ? s[e >> 2][e & 3] * a.qscale : -INFINITY;
      sc[e] = v;
      mx = fmaxf(mx, v);
    }
    mx = max_over_rows(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_lane *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] *= alpha;
    float hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = (m_new == -INFINITY || !active) ? 0.f : __builtin_amdgcn_exp2f(sc[e] - m_new);
      l_lane += p;
      hi[e] = (float)(f16)p;
      lo[e] = p - hi[e];
    }
    const u32x4 phi = u32x4{pack_f16x2(hi[0], hi[1]), pack_f16x2(hi[2], hi[3]), pack_f16x2(hi[4], hi[5]),
                            pack_f16x2(hi[6], hi[7])};
    const u32x4 plo = u32x4{pack_f16x2(lo[0], lo[1]), pack_f16x2(lo[2], lo[3]), pack_f16x2(lo[4], lo[5]),
                            pack_f16x2(lo[6], lo[7])};
    wave_lds_sync();  // every lane's transposed value writes land before the operand reads
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t* vr = vt + (16 * t + j) * RVT;
      const u32x4 vop = u32x4{vr[2 * gq], vr[2 * gq + 1], vr[8 + 2 * gq], vr[8 + 2 * gq + 1]};
      acc[t] = mfma_f16(vop, phi, acc[t]);
      acc[t] = mfma_f16(vop, plo, acc[t]);
    }
    wave_lds_sync();  // operand reads finish before the next block overwrites the tile
  }
  // ---- waves -> LDS -> this split's partial ----------------------------------------------
  __syncthreads();
  float* s_m = smem;
  float* s_l = smem + WAVES * 8;
  float* s_o = smem + 2 * WAVES * 8;
  const float l_tot = sum_over_rows(l_lane);
  if (active && k == 0) {
    if (gq == 0) {
      s_m[wave * 8 + h] = m_run * LN2;
      s_l[wave * 8 + h] = l_tot;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) s_o[(wave * 8 + h) * D + 16 * t + 4 * gq + rr] = acc[t][rr];
  }
  __syncthreads();
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
    store_coherent(a.part_o + (row * a.total_splits + split) * D + c, o);
    if (c == 0) {
      store_coherent(a.part_ml + (row * a.total_splits + split) * 2 + 0, m);
      store_coherent(a.part_ml + (row * a.total_splits + split) * 2 + 1, l);
    }
  }
}

// Residual tokens n_q .. n_q+r-1 from the fp16/fp32 ring, on the vector ALUs: one thread per
// token for the scores (whole 16-byte row loads), then each wave takes every 4th token for the
// weighted value sum (two channels per lane, coalesced rows), reduced across waves in LDS.
template <bool RES_F16>
__device__ void residual_split(const DQArgs& a, int bh, int split, float* smem) {
  using RT = typename std::conditional<RES_F16, f16, float>::type;
  constexpr int PER16 = 16 / sizeof(RT);  // ring elements per 16-byte load
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int G = a.G, r = a.r;
  float* s_q = smem;                        // [8][D]
  float* s_p = smem + 8 * D;                // [8][RES_MAX]
  float* s_ml = s_p + 8 * RES_MAX;          // [8][2]
  float* s_red = s_ml + 16;                 // [WAVES][8][D]
  for (int idx = tid; idx < G * D; idx += THREADS) {
    const int hh = idx / D, c = idx % D;
    s_q[idx] = load_as_f32(a.q, ((int64_t)b * a.Hq + kvh * G + hh) * D + c, a.q_dtype) * a.qscale;
  }
  __syncthreads();
  const RT* kres = static_cast<const RT*>(a.k_res) + (int64_t)bh * a.res_cap * D;
  const RT* vres = static_cast<const RT*>(a.v_res) + (int64_t)bh * a.res_cap * D;
  const int base = (int)(a.n_q % a.res_cap);
  for (int t = tid; t < r; t += THREADS) {
    int slot = base + t;
    if (slot >= a.res_cap) slot -= a.res_cap;
    const u32x4* row = reinterpret_cast<const u32x4*>(kres + (int64_t)slot * D);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int z0 = 0; z0 < D / PER16; z0 += 4) {  // 4 x 16 bytes of the key row at a time
      u32x4 kv[4];
#pragma unroll
      for (int z = 0; z < 4; ++z) kv[z] = row[z0 + z];
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        float kx[PER16];
        if (RES_F16) {
#pragma unroll
          for (int y = 0; y < 4; ++y) {
            kx[2 * y] = f16_bits_to_f32(kv[z][y] & 0xffffu);
            kx[2 * y + 1] = f16_bits_to_f32(kv[z][y] >> 16);
          }
        } else {
#pragma unroll
          for (int y = 0; y < 4; ++y) kx[y] = __uint_as_float(kv[z][y]);
        }
        const int c0 = (z0 + z) * PER16;
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
          if (hh < G) {
#pragma unroll
            for (int y = 0; y < PER16; ++y) acc[hh] += s_q[hh * D + c0 + y] * kx[y];
          }
        }
      }
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
      const float p = __builtin_amdgcn_exp2f(s_p[hh * RES_MAX + t] - m);
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
  {
    float o[8][2];
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) o[hh][0] = o[hh][1] = 0.f;
#pragma unroll 4
    for (int t = wave; t < r; t += WAVES) {
      int slot = base + t;
      if (slot >= a.res_cap) slot -= a.res_cap;
      float v0, v1;
      if (RES_F16) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(vres + (int64_t)slot * D)[lane];
        v0 = f16_bits_to_f32(w & 0xffffu);
        v1 = f16_bits_to_f32(w >> 16);
      } else {
        const float2 w = reinterpret_cast<const float2*>(vres + (int64_t)slot * D)[lane];
        v0 = w.x;
        v1 = w.y;
      }
#pragma unroll
      for (int hh = 0; hh < 8; ++hh) {
        if (hh < G) {
          const float p = s_p[hh * RES_MAX + t];
          o[hh][0] += p * v0;
          o[hh][1] += p * v1;
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
      if (hh < G) {
        s_red[(wave * 8 + hh) * D + 2 * lane] = o[hh][0];
        s_red[(wave * 8 + hh) * D + 2 * lane + 1] = o[hh][1];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += THREADS) {
    const int hh = idx / D, c = idx % D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) o += s_red[(w * 8 + hh) * D + c];
    const int64_t row = (int64_t)b * a.Hq + kvh * G + hh;
    store_coherent(a.part_o + (row * a.total_splits + split) * D + c, o);
    if (c == 0) {
      store_coherent(a.part_ml + (row * a.total_splits + split) * 2 + 0, s_ml[2 * hh]);
      store_coherent(a.part_ml + (row * a.total_splits + split) * 2 + 1, s_ml[2 * hh + 1]);
    }
  }
}

// Ticket: the last workgroup of a (b, kv head) to finish merges every split's partial (read back
// past the non-coherent caches) and returns the ticket to zero. Partials are written with
// device-scope stores and waited for before the ticket is taken, so no cache-wide fence is needed.
__device__ void merge_if_last(const DQArgs& a, int bh, float* smem) {
  wait_vm<0>();
  __syncthreads();
  int* s_last = reinterpret_cast<int*>(smem);
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(a.counters + bh, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == (unsigned)(a.nwg - 1);
    if (last) __hip_atomic_store(a.counters + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_last = last;
  }
  __syncthreads();
  if (!*s_last) return;
  const int wave = threadIdx.x >> 6;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  for (int hh = wave; hh < a.G; hh += WAVES) {
    const int64_t row = (int64_t)b * a.Hq + kvh * a.G + hh;
    merge_row_wave<true>(a.part_o + row * a.total_splits * D, a.part_ml + row * a.total_splits * 2,
                         a.total_splits, a.out + row * D, a.lse ? a.lse + row : nullptr);
  }
}

// The step's own key/value (residual token n_q + r - 1) into its ring slot, converted to the
// residual dtype with round-half-even (as an append would store it): threads 0..127 take the
// key's channels, 128..255 the value's. Only the workgroup that runs the residual split reads the
// ring in this launch, and it does so after a barrier.
__device__ void append_new_token(const DQArgs& a, int bh) {
  static_assert(THREADS == 2 * D, "one thread per key or value channel");
  const int c = threadIdx.x & (D - 1);
  const bool val = threadIdx.x >= D;
  const int64_t src = (int64_t)(bh / a.Hkv) * a.new_b_stride + (int64_t)(bh % a.Hkv) * a.new_h_stride + c;
  const float x = load_as_f32(val ? a.v_new : a.k_new, src, a.new_dtype);
  if (a.n_q + a.r < 1) return;  // a row with no residual position (per-row lengths)
  const int64_t slot = (a.n_q + a.r - 1) % a.res_cap;
  const int64_t off = ((int64_t)bh * a.res_cap + slot) * D + c;
  void* dst = const_cast<void*>(val ? a.v_res : a.k_res);
  if (a.res_dtype == VC_F32)
    static_cast<float*>(dst)[off] = x;
  else
    static_cast<f16*>(dst)[off] = (f16)x;
}

template <int BITS, bool META_F16, bool RES_F16, int CPH>
__global__ void __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(wg_per_cu(BITS), wg_per_cu(BITS)))) draft_quant_kernel(DQArgs a0) {
  __shared__ float smem[std::max(WAVES * RingPlan<BITS, META_F16>::BYTES / 4, RES_SMEM_FLOATS)];
  static_assert(wg_per_cu(BITS) * sizeof(smem) <= 160 * 1024, "the workgroups per CU must fit its LDS");
  const int split = blockIdx.x;
  const int bh = blockIdx.y;
  DQArgs a = a0;
  if (a.row_nq) {  // this batch row's lengths (the splits and partial layout stay the launch's)
    const int b = bh / a.Hkv;
    const int64_t nq = a.row_nq[b];
    a.n_q = min(max(nq, (int64_t)0), a.tok_cap) / GROUP * GROUP;
    a.r = min(max(a.row_r[b] + a.row_radd, 0), a.res_cap);
    a.ngroups = (int)(a.n_q / GROUP);
    a.units = a.ngroups + (int64_t)RES_UNITS * ((a.r + GROUP - 1) / GROUP);
  }
  __builtin_amdgcn_s_setprio(3);  // lowered step by step as the wave's share is worked off
  // Work units: the quantised groups, then RES_UNITS per 32-token residual block; workgroup w
  // takes units [U w / nwg, U (w+1) / nwg). The last workgroup also runs the residual split
  // (partial index splits + 1) before its share of quantised groups (partial index w).
  const int g_begin = (int)std::min<int64_t>(a.ngroups, a.units * split / a.nwg);
  const int g_end = (int)std::min<int64_t>(a.ngroups, a.units * (split + 1) / a.nwg);
  if (split == a.nwg - 1) {
    if (a.k_new) {
      append_new_token(a, bh);
      __syncthreads();  // the residual split below reads the slot back
    }
    if (RES_F16 && a.q_dtype != VC_F32)
      residual_split_mfma(a, bh, a.splits + 1, smem);
    else
      residual_split<RES_F16>(a, bh, a.splits + 1, smem);
    __syncthreads();  // the residual split's LDS is free again
  }
  if constexpr (META_F16 && CPH == 4)
    quant_split_t<BITS>(a, bh, g_begin, g_end, split, smem);
  else
    quant_split<BITS, META_F16, CPH>(a, bh, g_begin, g_end, split, smem);
  __builtin_amdgcn_s_setprio(3);  // the merge is on the launch's critical path
  merge_if_last(a, bh, smem);
}

}  // namespace

DraftQuantPlan plan_draft_quant(const vc_kivi& c, int64_t n_q, int Hq) {
  DraftQuantPlan p;
  const int64_t ngroups = n_q / GROUP;
  const int64_t units = (int64_t)c.B * c.Hkv;
  // One resident round of workgroups: 256 CUs x the workgroups per CU the kernel is built for
  // (its waves per SIMD), splits + 1 per (b, kv head); at least 2 groups per wave.
  int64_t s = std::max<int64_t>(1, NUM_CUS * wg_per_cu(c.bits) / units - 1);
  s = std::min<int64_t>(s, std::max<int64_t>(1, ngroups / 8));
  if (ngroups == 0) s = 0;
  p.splits = (int)s;
  p.total_splits = p.splits + 2;  // partials: one per workgroup + the residual split's
  const size_t rows = (size_t)c.B * Hq;
  p.ws_bytes = DRAFT_COUNTER_BYTES + rows * p.total_splits * (D + 2) * sizeof(float);
  return p;
}

namespace {

hipError_t launch_draft_quant_impl(const vc_kivi& c, int64_t n_q, int r, const int64_t* row_nq,
                                   const int32_t* row_r, int row_radd,
                                   const void* k_new, const void* v_new, int new_dtype,
                                   int64_t new_b_stride, int64_t new_h_stride, const void* q, int q_dtype, int Hq,
                                   float sm_scale, float* out, float* lse, void* ws,
                                   const DraftQuantPlan& plan, hipStream_t s) {
  DQArgs a;
  a.row_nq = row_nq;
  a.row_r = row_r;
  a.row_radd = row_radd;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_dtype = new_dtype;
  a.new_b_stride = new_b_stride;
  a.new_h_stride = new_h_stride;
  a.k_codes = static_cast<const uint8_t*>(c.k_codes);
  a.v_codes = static_cast<const uint8_t*>(c.v_codes);
  a.k_meta = c.k_meta;
  a.v_meta = c.v_meta;
  a.k_res = c.k_res;
  a.v_res = c.v_res;
  a.q = q;
  a.out = out;
  a.lse = lse;
  const size_t rows = (size_t)c.B * Hq;
  a.counters = static_cast<unsigned*>(ws);
  a.part_o = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + DRAFT_COUNTER_BYTES);
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
  a.nwg = plan.splits + 1;
  a.units = a.ngroups + (int64_t)RES_UNITS * ((r + GROUP - 1) / GROUP);
  a.qscale = sm_scale * LOG2E;
  dim3 grid((unsigned)(plan.splits + 1), (unsigned)(c.B * c.Hkv));
  const bool f16m = c.meta_dtype == VC_F16, f16r = c.res_dtype == VC_F16;
  const bool wide = a.G <= 4;
#define VC_DQ_LAUNCH(BITS, MF, RF)                                                              \
  do {                                                                                          \
    if (wide) hipLaunchKernelGGL((draft_quant_kernel<BITS, MF, RF, 4>), grid, dim3(THREADS), 0, s, a); \
    else hipLaunchKernelGGL((draft_quant_kernel<BITS, MF, RF, 2>), grid, dim3(THREADS), 0, s, a);      \
  } while (0)
  if (c.bits == 2) {
    if (f16m) { if (f16r) VC_DQ_LAUNCH(2, true, true); else VC_DQ_LAUNCH(2, true, false); }
    else { if (f16r) VC_DQ_LAUNCH(2, false, true); else VC_DQ_LAUNCH(2, false, false); }
  } else {
    if (f16m) { if (f16r) VC_DQ_LAUNCH(4, true, true); else VC_DQ_LAUNCH(4, true, false); }
    else { if (f16r) VC_DQ_LAUNCH(4, false, true); else VC_DQ_LAUNCH(4, false, false); }
  }
#undef VC_DQ_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_draft_quant(const vc_kivi& c, int64_t n_q, int r, const void* k_new,
                              const void* v_new, int new_dtype, int64_t new_bh_stride, const void* q,
                              int q_dtype, int Hq, float sm_scale, float* out, float* lse, void* ws,
                              const DraftQuantPlan& plan, hipStream_t s) {
  return launch_draft_quant_impl(c, n_q, r, nullptr, nullptr, 0, k_new, v_new, new_dtype,
                                 new_bh_stride * c.Hkv, new_bh_stride, q, q_dtype, Hq, sm_scale, out,
                                 lse, ws, plan, s);
}

hipError_t launch_draft_quant_rows(const vc_kivi& c, const int64_t* n_q, const int32_t* r, int r_add,
                                   int64_t n_q_max, int r_max, const void* k_new, const void* v_new,
                                   int new_dtype, int64_t new_b_stride, int64_t new_h_stride,
                                   const void* q, int q_dtype, int Hq, float sm_scale, float* out,
                                   float* lse, void* ws, const DraftQuantPlan& plan, hipStream_t s) {
  return launch_draft_quant_impl(c, n_q_max, r_max, n_q, r, r_add, k_new, v_new, new_dtype,
                                 new_b_stride, new_h_stride, q, q_dtype, Hq, sm_scale, out, lse, ws,
                                 plan, s);
}

namespace {

__global__ void clear_counters_kernel(unsigned* counters, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) counters[i] = 0u;
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // per device ordinal: the device address of `scratch`

}  // namespace

hipError_t draft_scratch_pointer(void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_draft_quant_noalloc(const vc_kivi& c, int64_t n_q, int r, const void* k_new,
                                      const void* v_new, int new_dtype, int64_t new_bh_stride,
                                      const void* q, int q_dtype, int Hq, float sm_scale, float* out,
                                      float* lse, const DraftQuantPlan& plan, hipStream_t s) {
  void* ws = nullptr;
  hipError_t err = draft_scratch_pointer(&ws);
  if (err != hipSuccess) return err;
  // the tickets start at zero on every call (a fill kernel, not a memset node, so the call can be
  // captured into a graph); the partials are written before they are read
  const int units = c.B * c.Hkv;
  hipLaunchKernelGGL(clear_counters_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s,
                     static_cast<unsigned*>(ws), units);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_draft_quant(c, n_q, r, k_new, v_new, new_dtype, new_bh_stride, q, q_dtype, Hq,
                            sm_scale, out, lse, ws, plan, s);
}

}  // namespace vc
