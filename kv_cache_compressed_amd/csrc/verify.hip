// Verify attention: L <= 32 query rows per query head attend causally over the full cache.
//
// "VeriCache: making lossy KV compression exact", The Core Idea (one pass over the full cache
// scores every drafted position plus one) and Verifying Without Giving Back the Speedup (the full
// cache may sit in CPU memory and cross the host link only to be verified; verification is an
// L-row block per query head, so it is matrix-core work rather than a bandwidth-bound one-row
// product); "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference", Key Contributions
// (verification is bound by the interconnect and FLOPs).
//
// bf16 path (matrix cores). Workgroup = 4 waves on one (b, kv head), up to 4 of its query heads
// (ceil(G / 4) workgroups per tile range when G > 4) and one range of 32-token key tiles; wave w
// owns one query head and its L rows (two 16-row column tiles). Tiles reach LDS through direct buffer -> LDS copies into a 3-stage ring (two tiles in
// flight), row-major with swizzled 16-byte chunks, one workgroup barrier per tile. QK^T uses
// v_mfma_f32_16x16x32_bf16 with the keys as the row operand (S^T), so each lane holds 8 token
// scores of one query row, which is the layout of the PV product's column operand; the values
// reach the PV row operand through the LDS transpose read. The softmax weights are carried as a
// bf16 hi + lo pair (two accumulations), which keeps ~16 significant bits in the weights at the
// cost of a second PV product (bf16 weights alone move the logits by ~1e-2, enough to flip
// near-tied tokens); the fp32 accumulators keep the logits' argmax.
//
// fp32 path (vector ALUs): one workgroup per (row, split) with a thread per key.
//
// Both paths write unnormalised split partials (o, m, l); the past is split into ranges (or
// streamed chunk by chunk from pinned host memory through two device stages), the causal block
// is one more split, and a log-sum-exp merge produces the output.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace vc {

namespace {

constexpr int TK = 32;             // keys per tile (one ring stage)
constexpr int NTB = TK / 16;       // 16-token row tiles of QK^T per tile
constexpr int NHF = TK / 32;       // 32-token PV contraction blocks per tile
constexpr int WG_PER_CU = 3;       // resident workgroups per CU (waves per SIMD for G <= 4)
constexpr int RING = 3;            // tile stages per workgroup (RING - 1 in flight)
constexpr int TILE_BYTES = TK * D * 2;  // one tile of keys (or values), bf16
constexpr int NUM_CUS = 256;
// Relative tile share of a workgroup by dispatch tier (see tile_start), in hundredths.
constexpr int TIER_W0 = 105, TIER_W1 = 100, TIER_W2 = 95;

struct VArgs {
  const uint16_t* q;       // [B][Hq][L][D] bf16
  const uint16_t* k;       // source keys: element (bh, t, c) at (bh*bh_stride + t)*D + c
  const uint16_t* v;
  int64_t bh_stride;       // tokens between consecutive (b, kv head) source rows
  int64_t ntok;            // tokens in this source
  int splits;              // workgroups per (b, kv head) for this source
  int split_offset;        // partial index of this launch's split 0
  int causal;              // source is the round's block: row i sees tokens 0..i
  const uint16_t* k_blk;   // null, or the round's block [B][Hkv][L][D] as one more split
  const uint16_t* v_blk;   //   (the last split's workgroup runs it), causal, to partial blk_index
  int blk_index;
  int L, Hq, Hkv, G, total_splits;
  int Gw;                  // query heads per workgroup: G, or 4 when G > 4 (then ceil(G / 4)
                           //   workgroups per (b, kv head) and tile range, heads 4 z .. 4 z + 3)
  int gsplits, units, gz;  // logical grid: gsplits tile ranges x units (b, kv head) x gz head slices
                           //   (the launch is one-dimensional; see logical_block)
  int tiered;              // one resident round (not prefill): unit fastest, shares by tier
  float qscale;            // sm_scale * log2(e)
  float* part_o;
  float* part_ml;
  // prefill form only: causal self-attention of n rows; unit = (row block, b, kv head), row
  // block rb = rows 32 rb .. over key tiles 0 .. rb (the diagonal tile masked), heaviest first
  int n_rows;              // n
  int bh_units;            // B * Hkv
  int rblocks;             // ceil(n / 32)
};

constexpr float LAZY = 2.0f;  // log2 slack before a row's reference max is moved
constexpr int RSRC_WORD3 = 0x00020000;  // raw buffer, 32-bit data format

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Tiles live in LDS row-major (256 bytes per token row) with their 16-byte chunks swizzled,
// chunk c of row r at position r*16 + (c ^ (r & 15)), so that the 16 rows a matrix-core operand
// read touches fall in different banks.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }

// Values row operand: two LDS transpose reads (ds_read_b64_tr_b16), rows `addr` and 16 rows
// further (4096 bytes), issued as inline asm. The builtin form is compiled with a wait for every
// buffer -> LDS copy in flight (the compiler cannot tell which LDS bytes those copies target),
// which would stall every tile on the copies of the tiles behind it. The compiler does not track
// these reads either: tr16_wait() must run before the registers are used.
template <int OFF>
__device__ __forceinline__ u32x4 tr16_issue(unsigned addr) {
  static_assert(OFF >= 0 && OFF + 4096 <= 65535, "ds offset field");
  u32x2 r0, r1;
  // early clobber: the second read must not find its address register overwritten by the first
  asm volatile("ds_read_b64_tr_b16 %0, %2 offset:%3\n\tds_read_b64_tr_b16 %1, %2 offset:%4"
               : "=&v"(r0), "=&v"(r1)
               : "v"(addr), "n"(OFF), "n"(OFF + 4096));
  return u32x4{r0[0], r0[1], r1[0], r1[1]};
}
__device__ __forceinline__ void tr16_wait(u32x4& r) { asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r)); }

// Copy tile `tile` of one (b, kv head) source into ring slot `slot` (keys, then values): each of
// the NW waves copies TK*16/(64*NW) 16-byte chunks per operand with buffer -> LDS loads; the
// buffer resources span the source's ntok rows, so rows past the end (and whole tiles past the
// range) arrive as zeros.
template <int NW>
constexpr int COPY_PER_WAVE = TK * 16 / (64 * NW);  // 16-byte chunks per lane per operand

// This lane's buffer offsets within a tile (fixed for the whole loop): copy z of wave w lands at
// LDS position p = 64 (w * COPY_PER_WAVE + z) + lane, which holds chunk (p & 15) ^ (row & 15) of
// row p >> 4.
template <int NW>
__device__ __forceinline__ void tile_offsets(unsigned* voff) {
  static_assert(COPY_PER_WAVE<NW> >= 1 && TK * 16 % (64 * NW) == 0, "tile copy split");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int z = 0; z < COPY_PER_WAVE<NW>; ++z) {
    const int p = (wave * COPY_PER_WAVE<NW> + z) * 64 + lane;
    const int row = p >> 4, chunk = (p & 15) ^ (row & 15);
    voff[z] = (unsigned)(row * 256 + chunk * 16);
  }
}

template <int NW>
__device__ __forceinline__ void tile_copy(uint8_t* ring, int slot, __amdgpu_buffer_rsrc_t rk,
                                          __amdgpu_buffer_rsrc_t rv, const unsigned* voff, int tile,
                                          bool live) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // LDS bases in scalar registers
  const unsigned sbase = live ? (unsigned)tile * TILE_BYTES : 0x7ffff000u;  // dead: out of range
  uint8_t* kdst = ring + slot * 2 * TILE_BYTES;
  uint8_t* vdst = kdst + TILE_BYTES;
#pragma unroll
  for (int z = 0; z < COPY_PER_WAVE<NW>; ++z) {
    const int base = (wave * COPY_PER_WAVE<NW> + z) * 64;  // first LDS position of this copy
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(kdst + base * 16), 16,
                                             voff[z], sbase, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(vdst + base * 16), 16,
                                             voff[z], sbase, 0, 0);
  }
}

// Logical block (split, unit, z) of linear workgroup W. The hardware deals workgroups to the 8 XCDs
// in turn by linear id (XCD = W mod 8), and each XCD has its own L2. With two head slices per tile
// range (G > 4) both slices must stream the same tiles through the same L2 at the same time, or
// each tile is fetched from HBM twice: slice 0 of pair P runs as W = 16 (P / 8) + P % 8 and slice 1
// as W + 8 (same XCD, dispatched right after). The grid is padded to whole groups of 16; padding
// workgroups return at once. With one slice, W is the pair index itself. Pair P is split
// P / units of unit P % units when the launch is tiered (see tile_start), else split P % gsplits
// of unit P / gsplits (the prefill's heaviest-first unit order).
struct LogicalBlock {
  int split, unit, z;
  bool live;
};
__device__ __forceinline__ LogicalBlock logical_block(const VArgs& a) {
  const int W = (int)blockIdx.x;
  int P = W, z = 0;
  if (a.gz == 2) {
    P = (W >> 4) * 8 + (W & 7);
    z = (W >> 3) & 1;
  }
  LogicalBlock lb;
  lb.live = P < a.gsplits * a.units;
  if (a.tiered) {  // consecutive pairs take the same split of consecutive units
    lb.split = P / a.units;
    lb.unit = P % a.units;
  } else {
    lb.split = P % a.gsplits;
    lb.unit = P / a.gsplits;
  }
  lb.z = z;
  return lb;
}

// First tile of split s (of nsplit) of a unit's ntiles. Untiered: equal shares. Tiered (the grid
// fits one resident round): the hardware deals workgroups W < 256 to the CUs' first slots, then
// the second, then the third, and a later tier starts its copies behind the earlier tiers' and
// its waves issue behind older ones (its loop ran ~11% longer on equal work); pair P = s * units
// + unit is in tier W / 256 = P / (256 / gz), so every unit's splits cover all tiers and a split's
// share follows its tier's weight. The ranges depend on the launch shape only (deterministic).
__device__ int tile_start(const VArgs& a, int unit, int s, int nsplit, int ntiles) {
  if (!a.tiered) return (int)((int64_t)ntiles * s / nsplit);
  const int w[3] = {TIER_W0, TIER_W1, TIER_W2};
  const int per = NUM_CUS / a.gz;  // pairs per tier
  int64_t cum = 0, tot = 0;
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int lo = per * t - unit, hi = per * (t + 1) - unit;
    const int f0 = t == 0 ? 0 : min(nsplit, max(0, (lo + a.units - 1) / a.units));
    const int f1 = t == 2 ? nsplit : min(nsplit, max(0, (hi + a.units - 1) / a.units));
    const int n = max(0, f1 - f0);
    tot += (int64_t)w[t] * n;
    cum += (int64_t)w[t] * min(n, max(0, s - f0));
  }
  return tot > 0 ? (int)((int64_t)ntiles * cum / tot) : 0;
}

// Workgroup = NW waves on one (b, kv head), heads Gw z .. Gw z + Gw - 1 of its group (z: the
// logical head slice) and one range of 32-token tiles; wave w < Gw owns one of them and its L rows (two
// 16-row column tiles); all NW waves copy tiles.
// Tiles stream through a RING-stage LDS ring (RING - 1 in flight) with direct buffer -> LDS
// copies, one barrier per tile. Keys feed QK^T as the row operand; values are read straight into
// the PV row operand with the LDS transpose read (ds_read_b64_tr_b16): source lane s of a
// 16-lane block supplies 4 consecutive channels of one token row and result lane i receives
// element e from source lane 4e + i/4, so no transposed copy of the values is ever written.
template <int NW, bool PREFILL>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 4 ? WG_PER_CU : 2))) verify_bf16_kernel(VArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int COPIES = 2 * TK * 16 / NT;  // buffer -> LDS copies per lane per tile
  __shared__ __attribute__((aligned(16))) uint8_t ring[RING * 2 * TILE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, gq = lane >> 4;
  const LogicalBlock lb = logical_block(a);
  if (!lb.live) return;  // grid padding
  // prefill: this unit's row block (the longest first) and its rows' positions
  const int rb = PREFILL ? a.rblocks - 1 - lb.unit / a.bh_units : 0;
  const int pos0 = PREFILL ? 32 * rb : 0;                          // position of row 0
  const int Lu = PREFILL ? min(32, a.n_rows - pos0) : a.L;         // this unit's rows
  const int qrows = PREFILL ? a.n_rows : a.L;                      // rows per (b, head) in q / out
  const int bh = PREFILL ? lb.unit % a.bh_units : lb.unit;
  // Jobs of this workgroup: split lb.split of the launch's source (if lb.split < splits),
  // then, for the last workgroup of the row and when the round's block is given, the block as one
  // more causal split (it is one tile: a workgroup of its own would not fit the resident round).
  const bool do_past = lb.split < a.splits;
  const bool do_blk = a.k_blk != nullptr && lb.split == max(a.splits, 1) - 1;
  auto run_job = [&](const bool blk) {
  const uint16_t* const src_k = blk ? a.k_blk : a.k;
  const uint16_t* const src_v = blk ? a.v_blk : a.v;
  const int64_t src_stride = blk ? a.L : a.bh_stride, src_ntok = blk ? a.L : PREFILL ? pos0 + Lu : a.ntok;
  const int src_splits = blk ? 1 : a.splits, split = blk ? 0 : lb.split;
  const bool causal = blk || a.causal || PREFILL;
  const int sidx = blk ? a.blk_index : a.split_offset + split;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int hg = lb.z * a.Gw + wave;  // head within the kv group
  const bool computes = wave < a.Gw && hg < a.G;
  const int hq = kvh * a.G + min(hg, a.G - 1);

  // tile range of this split
  const int ntiles = (int)((src_ntok + TK - 1) / TK);  // < 2^18: src_ntok * 256 bytes < 2^31
  const int t_begin = blk ? 0 : tile_start(a, lb.unit, split, src_splits, ntiles);
  const int t_end = blk ? ntiles : tile_start(a, lb.unit, split + 1, src_splits, ntiles);
  unsigned voff[COPY_PER_WAVE<NW>];
  tile_offsets<NW>(voff);
  const int nbytes = (int)(src_ntok * D * 2);  // this (b, kv head)'s source rows
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(src_k + (int64_t)bh * src_stride * D), (short)0, nbytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(src_v + (int64_t)bh * src_stride * D), (short)0, nbytes, RSRC_WORD3);

  // the first RING - 1 tiles go out before anything else
#pragma unroll
  for (int z = 0; z < RING - 1; ++z) tile_copy<NW>(ring, z, rk, rv, voff, t_begin + z, t_begin + z < t_end);

  // Q^T operand: column tile ct holds rows 16ct + j; lane holds channels 32kb + 8gq + 0..7.
  u32x4 qop[2][4];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int row = pos0 + min(16 * ct + j, Lu - 1);  // rows past L read row L-1, never written
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int64_t off = (((int64_t)b * a.Hq + hq) * qrows + row) * D + 32 * kb + 8 * gq;
      qop[ct][kb] = *reinterpret_cast<const u32x4*>(a.q + off);
    }
  }

  float m_run[2] = {-INFINITY, -INFINITY};
  float nref[2] = {0.f, 0.f};  // -m_run, 0 while no key has been seen
  float l_lane[2] = {0.f, 0.f};
  f32x4 acc[2][8];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[ct][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Progress-based wave priority (waves issue oldest first; with equal shares the workgroups that
  // started early would finish early and leave the CU to the late ones at the end): start at the
  // top level and step down at 1/3, 2/3 and 5/6 of this workgroup's tiles.
  __builtin_amdgcn_s_setprio(3);
  const int q1 = t_begin + (t_end - t_begin) / 3, q2 = t_begin + 2 * (t_end - t_begin) / 3,
            q3 = t_begin + 5 * (t_end - t_begin) / 6;
  // One tile; the ring slot is a compile-time constant (the loop below is unrolled by RING), so
  // every LDS address of the tile is a per-lane base plus an immediate offset.
  auto step = [&](const int tile, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    if (tile == q1) __builtin_amdgcn_s_setprio(2);
    if (tile == q2) __builtin_amdgcn_s_setprio(1);
    if (tile == q3) __builtin_amdgcn_s_setprio(0);
    // this tile's copies have landed (only the RING - 2 later tiles' may be in flight), every
    // wave's share of them is visible, and every wave is done with the slot refilled below
    wait_vm<(RING - 2) * COPIES>();
    __syncthreads();
    tile_copy<NW>(ring, (slot + RING - 1) % RING, rk, rv, voff, tile + RING - 1, tile + RING - 1 < t_end);
    if (computes) {
      const int64_t tok0 = tile * TK;
      const int tlen = (int)min<int64_t>(TK, src_ntok - tok0);
      const uint8_t* sk = ring + slot * 2 * TILE_BYTES;
      // ---- QK^T: S^T[token][row]: s[tb][ct][r] = token 16 tb + 4 gq + r, row 16 ct + j -------
      f32x4 s[NTB][2];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        u32x4 kop[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          kop[kb] = *reinterpret_cast<const u32x4*>(sk + swz(16 * tb + j, 4 * kb + gq) * 16);
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
      // (prefill: only the diagonal tile masks; the tiles before it are whole)
      const bool masked = (causal && (!PREFILL || tok0 + TK > pos0)) || tlen < TK;
      u32x4 phi[2][NHF], plo[2][NHF];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int row = 16 * ct + j;
        float raw[4 * NTB];
#pragma unroll
        for (int e = 0; e < 4 * NTB; ++e) raw[e] = s[e >> 2][ct][e & 3];
        if (masked) {
          asm volatile("");  // keep this rarely taken path a branch (no if-conversion)
          // tokens of this tile that row sees: tok < lim (row at position pos0 + row)
          const int lim = causal ? (int)min<int64_t>(tlen, pos0 + row + 1 - tok0) : tlen;
#pragma unroll
          for (int e = 0; e < 4 * NTB; ++e) {
            const int tok = 16 * (e >> 2) + 4 * gq + (e & 3);
            raw[e] = tok < lim ? raw[e] : -INFINITY;
          }
        }
        // The reference max moves only when the row's max exceeds it by LAZY: a lane compares its
        // own 8 scores first, and only when some lane is over (rare after the first tile) is the
        // row max formed across the row's 4 lanes and the row rescaled.
        float mraw = raw[0];
#pragma unroll
        for (int e = 1; e < 4 * NTB; ++e) mraw = fmaxf(mraw, raw[e]);
        if (__builtin_amdgcn_ballot_w64(mraw * a.qscale > m_run[ct] + LAZY)) {
          asm volatile("");  // keep this rarely taken path a branch (no if-conversion)
          const float mx = max_over_rows(mraw) * a.qscale;
          const bool move = mx > m_run[ct] + LAZY;
          const float m_new = move ? mx : m_run[ct];
          const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[ct] - m_new);
          m_run[ct] = m_new;
          nref[ct] = m_new == -INFINITY ? 0.f : -m_new;
          l_lane[ct] *= alpha;
#pragma unroll
          for (int t = 0; t < 8; ++t) acc[ct][t] *= alpha;
        }
        float psum = 0.f;
#pragma unroll
        for (int hf = 0; hf < NHF; ++hf) {
          float p[8], lo[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(fmaf(raw[8 * hf + e], a.qscale, nref[ct]));  // masked: 0
            psum += p[e];
            lo[e] = p[e] - __uint_as_float(__float_as_uint(p[e]) & 0xffff0000u);  // exact remainder
          }
          // bf16 hi = truncated p; bf16 lo = truncated remainder (the pair keeps ~16 bits)
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            phi[ct][hf][e2] = __builtin_amdgcn_perm(__float_as_uint(p[2 * e2 + 1]), __float_as_uint(p[2 * e2]), 0x07060302u);
            plo[ct][hf][e2] = __builtin_amdgcn_perm(__float_as_uint(lo[2 * e2 + 1]), __float_as_uint(lo[2 * e2]), 0x07060302u);
          }
        }
        l_lane[ct] += psum;
      }
      // ---- PV: O^T[c][row] += V^T[c][tok] P^T[tok][row] ---------------------------------------
      // Row operand of channel tile t: lane (channel 16t + j, gq) needs tokens 4gq + e (e < 4) and
      // 16 + 4gq + e; source lane s = j of block gq supplies channels 16t + 4(s&3) .. +3 of token
      // 16h + 4gq + (s>>2) for the transpose read h.
      // The reads of step k + 1 are in flight while step k's products run.
      // (the ring's LDS base goes into the lane address, the slot's offset into the immediate)
      const unsigned ring_lds = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)ring;
      constexpr int VOFF = slot * 2 * TILE_BYTES + TILE_BYTES;
      auto vaddr = [&](int k) {  // step k = (channel tile t, contraction block hf)
        const int t = k / NHF, hf = k % NHF;
        const int row = 32 * hf + 4 * gq + (j >> 2);
        const int byte = (16 * t + 4 * (j & 3)) * 2;  // within the row
        return ring_lds + (unsigned)(swz(row, byte >> 4) * 16 + (byte & 15));
      };
      u32x4 vop = tr16_issue<VOFF>(vaddr(0));
#pragma unroll
      for (int k = 0; k < 8 * NHF; ++k) {
        const int t = k / NHF, hf = k % NHF;
        tr16_wait(vop);
        const u32x4 cur = vop;
        if (k + 1 < 8 * NHF) vop = tr16_issue<VOFF>(vaddr(k + 1));
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          acc[ct][t] = mfma_bf16(cur, phi[ct][hf], acc[ct][t]);
          acc[ct][t] = mfma_bf16(cur, plo[ct][hf], acc[ct][t]);
        }
      }
    }
  };
  static_assert(RING == 3, "the tile loop is unrolled by the ring depth");
  for (int tile = t_begin; tile < t_end; tile += RING) {
    step(tile, std::integral_constant<int, 0>{});
    if (tile + 1 < t_end) step(tile + 1, std::integral_constant<int, 1>{});
    if (tile + 2 < t_end) step(tile + 2, std::integral_constant<int, 2>{});
  }
  wait_vm<0>();  // no copy may still target LDS when the job (and the workgroup) ends

  // ---- write this wave's partial rows ------------------------------------------------------
  if (computes) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int row = 16 * ct + j;
      const float l = sum_over_rows(l_lane[ct]);
      if (row < Lu) {
        const int64_t prow = ((int64_t)b * a.Hq + hq) * qrows + pos0 + row;
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
  };
  if (do_past) run_job(false);
  if (do_blk) {
    if (do_past) __syncthreads();  // the block's copies refill the ring
    run_job(true);
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

// fp32 path. Workgroup = 256 threads on one (b, kv head), one chunk of up to RWF of its G*L query
// rows (row r: head r / L, block row r % L) and one range of the concatenated key sequence
// [past ; block]. Key tiles of TKF keys and their values are staged in LDS once and serve every row
// of the chunk. Scores: thread (row group g = tid / 32, key k = tid % 32) takes rows 4g .. 4g+3
// against key k (the 32 lanes of a row group share its online-softmax state through shuffles);
// PV: thread (channel tid % 128, row half tid / 128) accumulates 16 rows of one output channel.
constexpr int TKF = 32;  // keys per tile
constexpr int RWF = 32;  // query rows per workgroup

__global__ void __launch_bounds__(256) verify_f32_kernel(VF32Args a) {
  // rows padded by 16 bytes: 16-byte reads stay aligned and the 32 key lanes' reads of one column
  // block spread over the banks
  __shared__ float s_q[RWF][D + 4];
  __shared__ float s_k[TKF][D + 4];
  __shared__ float s_v[TKF][D];
  __shared__ float s_p[RWF][TKF + 4];
  __shared__ float s_alpha[RWF];
  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int R = a.G * a.L;
  const int rchunks = (R + RWF - 1) / RWF;
  const int unit = blockIdx.y / rchunks, r0 = (blockIdx.y % rchunks) * RWF;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int nrows = min(RWF, R - r0);
  const int64_t nkeys = a.n + a.L;
  const int64_t k_begin = nkeys * split / a.splits, k_end = nkeys * (split + 1) / a.splits;
  auto prow_of = [&](int r) {  // global query row of chunk row r
    const int rr = r0 + r;
    return ((int64_t)b * a.Hq + kvh * a.G + rr / a.L) * a.L + rr % a.L;
  };
  for (int e = tid; e < RWF * D; e += 256) {
    const int r = e / D, c = e % D;
    s_q[r][c] = r < nrows ? a.q[prow_of(r) * D + c] * a.qscale : 0.f;
  }
  const int kk = tid & 31, rg = tid >> 5;    // score mapping
  const int cc = tid & (D - 1), h2 = tid >> 7;  // PV mapping
  float m_run[4], l_run[4];
  int64_t lim[4];  // last visible key of each score row (row i sees keys 0 .. n + i)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
    const int r = rg * 4 + j;
    lim[j] = r < nrows ? a.n + (r0 + r) % a.L : -1;
  }
  float o[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) o[r] = 0.f;

  for (int64_t kt = k_begin; kt < k_end; kt += TKF) {
    __syncthreads();  // the previous tile's LDS reads are done (and s_q is written)
    for (int e = tid; e < TKF * D / 4; e += 256) {
      const int t = e / (D / 4), c4 = (e % (D / 4)) * 4;
      const int64_t key = kt + t;
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (key < k_end) {
        const int64_t off = key < a.n ? ((int64_t)unit * a.past_stride + key) * D
                                      : ((int64_t)unit * a.L + (key - a.n)) * D;
        const float* kb = key < a.n ? a.k_past : a.k_blk;
        const float* vb = key < a.n ? a.v_past : a.v_blk;
        kv = *reinterpret_cast<const f32x4*>(kb + off + c4);
        vv = *reinterpret_cast<const f32x4*>(vb + off + c4);
      }
      *reinterpret_cast<f32x4*>(&s_k[t][c4]) = kv;
      *reinterpret_cast<f32x4*>(&s_v[t][c4]) = vv;
    }
    __syncthreads();
    const int64_t key = kt + kk;
    float sc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int c = 0; c < D; c += 4) {
      const f32x4 k4 = *reinterpret_cast<const f32x4*>(&s_k[kk][c]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 q4 = *reinterpret_cast<const f32x4*>(&s_q[rg * 4 + j][c]);
        sc[j] = fmaf(q4[0], k4[0], sc[j]);
        sc[j] = fmaf(q4[1], k4[1], sc[j]);
        sc[j] = fmaf(q4[2], k4[2], sc[j]);
        sc[j] = fmaf(q4[3], k4[3], sc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = key < k_end && key <= lim[j];
      float mx = ok ? sc[j] : -INFINITY;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
      const float m_new = fmaxf(m_run[j], mx);
      const float p = ok ? __builtin_amdgcn_exp2f(sc[j] - m_new) : 0.f;
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[j] - m_new);
      float ps = p;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) ps += __shfl_xor(ps, off, 64);
      l_run[j] = l_run[j] * alpha + ps;
      m_run[j] = m_new;
      s_p[rg * 4 + j][kk] = p;
      if (kk == 0) s_alpha[rg * 4 + j] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = h2 * 16 + r;
      float acc = o[r] * s_alpha[row];
#pragma unroll 2
      for (int t = 0; t < TKF; t += 4) {
        const f32x4 p4 = *reinterpret_cast<const f32x4*>(&s_p[row][t]);
        acc = fmaf(p4[0], s_v[t][cc], acc);
        acc = fmaf(p4[1], s_v[t + 1][cc], acc);
        acc = fmaf(p4[2], s_v[t + 2][cc], acc);
        acc = fmaf(p4[3], s_v[t + 3][cc], acc);
      }
      o[r] = acc;
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = h2 * 16 + r;
    if (row < nrows) a.part_o[(prow_of(row) * a.splits + split) * D + cc] = o[r];
  }
  if (kk == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = rg * 4 + j;
      if (row < nrows) {
        const int64_t pr = prow_of(row);
        a.part_ml[(pr * a.splits + split) * 2 + 0] = l_run[j] > 0.f ? m_run[j] * LN2 : -INFINITY;
        a.part_ml[(pr * a.splits + split) * 2 + 1] = l_run[j];
      }
    }
  }
}

}  // namespace

VerifyPlan plan_verify(int B, int Hq, int Hkv, int L, int64_t n, int past_on_host,
                       int64_t chunk_tokens, int dtype) {
  VerifyPlan p{};
  const int64_t units = (int64_t)B * Hkv;
  if (dtype == VC_F32) {
    // enough (split, unit, row chunk) workgroups to fill the chip, at least one key tile each
    const int64_t tiles = (n + L + TKF - 1) / TKF;
    const int64_t wgs = units * ((int64_t)(Hq / Hkv) * L + RWF - 1) / RWF;
    p.past_splits = (int)std::max<int64_t>(1, std::min<int64_t>(tiles, (512 + wgs - 1) / wgs));
    p.chunks = 0;
    p.chunk_tokens = 0;
    p.total_splits = p.past_splits;
    p.stage_bytes = 0;
  } else if (!past_on_host) {
    const int64_t tiles = (n + TK - 1) / TK;
    const int64_t wunits = units * ((Hq / Hkv + 3) / 4);  // workgroups per tile range
    int64_t s = (256 * WG_PER_CU + wunits - 1) / wunits;
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
    const int64_t wunits = units * ((Hq / Hkv + 3) / 4);  // workgroups per tile range
    int64_t s = (256 * WG_PER_CU + wunits - 1) / wunits;
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

namespace {

// The two chunk stages behind the partials in the workspace: keys then values, [units][ct][128].
void stage_pointers(void* ws, const VerifyPlan& plan, int64_t units, uint16_t** sk, uint16_t** sv) {
  char* base = static_cast<char*>(ws) + plan.part_bytes;
  for (int z = 0; z < 2; ++z) {
    sk[z] = reinterpret_cast<uint16_t*>(base + z * plan.stage_bytes);
    sv[z] = sk[z] + (size_t)units * plan.chunk_tokens * D;
  }
}

// Host -> device copies of chunk c's keys and values (rows [c ct, min(n, (c + 1) ct)) of every
// (b, kv head)) into one stage, on `copy`.
hipError_t copy_chunk(const void* k_past, const void* v_past, int64_t past_stride, int64_t n,
                      int64_t units, const VerifyPlan& plan, int c, uint16_t* sk, uint16_t* sv,
                      hipStream_t copy) {
  const int64_t t0 = (int64_t)c * plan.chunk_tokens;
  const int64_t len = std::min<int64_t>(plan.chunk_tokens, n - t0);
  const size_t src_pitch = (size_t)past_stride * D * 2;
  const size_t width = (size_t)len * D * 2;
  const size_t dpitch = (size_t)plan.chunk_tokens * D * 2;
  hipError_t err = hipMemcpy2DAsync(sk, dpitch, static_cast<const char*>(k_past) + t0 * D * 2,
                                    src_pitch, width, units, hipMemcpyHostToDevice, copy);
  if (err == hipSuccess)
    err = hipMemcpy2DAsync(sv, dpitch, static_cast<const char*>(v_past) + t0 * D * 2, src_pitch,
                           width, units, hipMemcpyHostToDevice, copy);
  return err;
}

}  // namespace

hipError_t launch_verify_prefetch(const void* k_past, const void* v_past, int64_t past_stride,
                                  int64_t n, int B, int Hkv, void* ws, const VerifyPlan& plan,
                                  hipStream_t compute, hipStream_t copy, hipEvent_t* done) {
  *done = nullptr;
  const int64_t units = (int64_t)B * Hkv;
  uint16_t* stage_k[2];
  uint16_t* stage_v[2];
  stage_pointers(ws, plan, units, stage_k, stage_v);
  hipEvent_t start;
  if (hipEventCreateWithFlags(&start, hipEventDisableTiming) != hipSuccess) return hipErrorOutOfMemory;
  // the stages are free once the work already on `compute` (earlier verifies) has run
  hipError_t err = hipEventRecord(start, compute);
  if (err == hipSuccess) err = hipStreamWaitEvent(copy, start, 0);
  for (int c = 0; c < std::min(2, plan.chunks) && err == hipSuccess; ++c)
    err = copy_chunk(k_past, v_past, past_stride, n, units, plan, c, stage_k[c], stage_v[c], copy);
  (void)hipEventDestroy(start);
  if (err == hipSuccess) err = hipEventCreateWithFlags(done, hipEventDisableTiming);
  if (err == hipSuccess) err = hipEventRecord(*done, copy);
  if (err != hipSuccess && *done) {
    (void)hipEventDestroy(*done);
    *done = nullptr;
  }
  return err;
}

hipError_t launch_verify_copies(const void* k_past, const void* v_past, int64_t past_stride,
                                int64_t n, int B, int Hkv, void* ws, const VerifyPlan& plan,
                                hipStream_t copy) {
  const int64_t units = (int64_t)B * Hkv;
  uint16_t* stage_k[2];
  uint16_t* stage_v[2];
  stage_pointers(ws, plan, units, stage_k, stage_v);
  hipError_t err = hipSuccess;
  for (int c = 0; c < plan.chunks && err == hipSuccess; ++c)
    err = copy_chunk(k_past, v_past, past_stride, n, units, plan, c, stage_k[c % 2], stage_v[c % 2], copy);
  return err;
}

PrefillPlan plan_prefill(int B, int Hq, int Hkv, int64_t n) {
  PrefillPlan p{};
  const int64_t rblocks = (n + TK - 1) / TK;
  const int64_t wunits = (int64_t)B * Hkv * rblocks * ((Hq / Hkv + 3) / 4);
  // one tile range per row block unless that leaves the chip short of workgroups
  p.splits = (int)std::max<int64_t>(1, std::min<int64_t>((256 * WG_PER_CU + wunits - 1) / wunits,
                                                         std::max<int64_t>(1, rblocks / 8)));
  const size_t rows = (size_t)B * Hq * n;
  p.ws_bytes = (rows * p.splits * (D + 2) * sizeof(float) + 255) & ~(size_t)255;
  return p;
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, int64_t kv_stride, int64_t n,
                          int B, int Hq, int Hkv, float sm_scale, float* out, float* lse, void* ws,
                          const PrefillPlan& plan, hipStream_t s) {
  const size_t rows = (size_t)B * Hq * n;
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o + rows * plan.splits * D;
  const int G = Hq / Hkv;
  VArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.bh_stride = kv_stride;
  a.ntok = n;
  a.splits = plan.splits;
  a.split_offset = 0;
  a.causal = 1;
  a.k_blk = nullptr;
  a.v_blk = nullptr;
  a.blk_index = 0;
  a.L = 32;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.total_splits = plan.splits;
  a.Gw = G <= 4 ? G : 4;
  a.qscale = sm_scale * LOG2E;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.n_rows = (int)n;
  a.bh_units = B * Hkv;
  a.rblocks = (int)((n + TK - 1) / TK);
  constexpr int NW = 4;
  const int gz = (G + 3) / 4;
  a.units = a.bh_units * a.rblocks;
  a.gz = gz;
  a.gsplits = plan.splits;
  a.tiered = 0;  // row blocks go out heaviest first (split fastest)
  unsigned wgs = (unsigned)(a.gsplits * a.units * gz);
  if (gz == 2) wgs = (wgs + 15) / 16 * 16;  // whole groups of 16 (see logical_block)
  hipLaunchKernelGGL((verify_bf16_kernel<NW, true>), dim3(wgs), dim3(64 * NW), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_merge(part_o, part_ml, (int64_t)rows, plan.splits, out, lse, s);
}

hipError_t launch_verify(const void* q, const void* k_blk, const void* v_blk, int L,
                         const void* k_past, const void* v_past, int64_t past_stride, int64_t n,
                         int past_on_host, int dtype, int B, int Hq, int Hkv, float sm_scale,
                         float* out, float* lse, void* ws, const VerifyPlan& plan,
                         hipStream_t compute, hipStream_t copy, hipEvent_t prefetched) {
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
    const unsigned rchunks = (unsigned)((G * L + RWF - 1) / RWF);
    hipLaunchKernelGGL(verify_f32_kernel, dim3(plan.total_splits, (unsigned)(B * Hkv) * rchunks),
                       dim3(256), 0, compute, a);
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
  // G > 4 runs as ceil(G / 4) 4-wave workgroups per (b, kv head) and tile range (grid.z), each
  // on up to 4 of the heads: 3 workgroups per CU instead of one 8-wave workgroup at 2 waves per
  // SIMD; the other workgroups' reads of the same tiles mostly hit L2
  constexpr int NW = 4;
  a.Gw = G <= 4 ? G : 4;
  const unsigned gz = (unsigned)((G + 3) / 4);
  const dim3 block(64 * NW);
  const unsigned units = (unsigned)(B * Hkv);
  a.units = (int)units;
  a.gz = (int)gz;
  auto launch_bf16 = [&](dim3 grid) {  // grid.x tile ranges x grid.y units x grid.z head slices
    a.gsplits = (int)grid.x;
    unsigned n = grid.x * grid.y * grid.z;
    if (gz == 2) n = (n + 15) / 16 * 16;  // whole groups of 16 (see logical_block)
    a.tiered = n <= (unsigned)(NUM_CUS * WG_PER_CU);
    hipLaunchKernelGGL((verify_bf16_kernel<NW, false>), dim3(n), block, 0, compute, a);
  };

  a.k_blk = nullptr;
  a.v_blk = nullptr;
  a.blk_index = plan.total_splits - 1;
  if (!past_on_host) {
    // the past's splits and the causal block (one more split) in one launch
    a.k = static_cast<const uint16_t*>(k_past);
    a.v = static_cast<const uint16_t*>(v_past);
    a.bh_stride = past_stride;
    a.ntok = n;
    a.splits = plan.past_splits;
    a.split_offset = 0;
    a.causal = 0;
    a.k_blk = static_cast<const uint16_t*>(k_blk);
    a.v_blk = static_cast<const uint16_t*>(v_blk);
    launch_bf16(dim3(std::max(plan.past_splits, 1), units, gz));
    if ((err = hipGetLastError()) != hipSuccess) return err;
    return launch_merge(part_o, part_ml, (int64_t)rows, plan.total_splits, out, lse, compute);
  } else {
    // Stream the past chunk by chunk: copies on `copy` into stage c % 2, compute on `compute`.
    // With a prefetch (past_on_host == 2) the first two chunks' copies are already on `copy`.
    const int first = past_on_host == 2 ? std::min(2, plan.chunks) : 0;
    uint16_t* stage_k[2];
    uint16_t* stage_v[2];
    stage_pointers(ws, plan, units, stage_k, stage_v);
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
    // prefetched chunks: `compute` waits for the prefetch's own copies (recorded right after
    // them), not for whatever later calls have queued on `copy` since
    if (first > 0 && err == hipSuccess) err = hipStreamWaitEvent(compute, prefetched, 0);
    for (int c = 0; c < plan.chunks && err == hipSuccess; ++c) {
      const int z = c % 2;
      const int64_t t0 = (int64_t)c * plan.chunk_tokens;
      const int64_t len = std::min<int64_t>(plan.chunk_tokens, n - t0);
      if (c >= first) {
        if (c >= 2) err = hipStreamWaitEvent(copy, done[z], 0);
        if (err == hipSuccess)
          err = copy_chunk(k_past, v_past, past_stride, n, units, plan, c, stage_k[z], stage_v[z], copy);
        if (err == hipSuccess) err = hipEventRecord(ready[z], copy);
        if (err == hipSuccess) err = hipStreamWaitEvent(compute, ready[z], 0);
        if (err != hipSuccess) break;
      }
      a.k = stage_k[z];
      a.v = stage_v[z];
      a.bh_stride = plan.chunk_tokens;
      a.ntok = len;
      a.splits = plan.past_splits;
      a.split_offset = c * plan.past_splits;
      a.causal = 0;
      launch_bf16(dim3(plan.past_splits, units, gz));
      if ((err = hipGetLastError()) != hipSuccess) break;
      err = hipEventRecord(done[z], compute);
    }
    // every copy of this call is now behind a wait on `compute`: the prefetched chunks behind
    // `prefetched`, each later chunk behind its ready event before its kernel
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
  launch_bf16(dim3(1, units, gz));
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_merge(part_o, part_ml, (int64_t)rows, plan.total_splits, out, lse, compute);
}

}  // namespace vc
