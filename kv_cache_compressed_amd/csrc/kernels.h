// Host-side launchers of the libvc kernels (validated arguments only; see api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vc.h"

namespace vc {

hipError_t launch_quantize(const vc_kivi& c, const void* k, const void* v, int src_dtype,
                           int64_t src_bh_stride, int64_t t0, int64_t ntok, hipStream_t s);
hipError_t launch_append(const vc_kivi& c, const void* k, const void* v, int src_dtype,
                         int64_t src_bh_stride, int64_t t0, int64_t ntok, hipStream_t s);

hipError_t launch_margins(const float* logits, int64_t rows, int V, float* gap, hipStream_t s);
hipError_t launch_read_stream(const void* src, int64_t n16, uint32_t* sink, int blocks, hipStream_t s);
hipError_t launch_accept(const float* logits, const int32_t* drafts, int B, int L, int V,
                         int32_t* accept_len, int32_t* next_token, int32_t* argmax, hipStream_t s);

hipError_t launch_merge(const float* part_o, const float* part_ml, int64_t rows, int S,
                        float* out, float* lse, hipStream_t s);

// Draft over the quantised cache.
// Ticket counters at the start of a draft workspace: one per (b, kv head), at most 16384.
constexpr size_t DRAFT_COUNTER_BYTES = 65536;
struct DraftQuantPlan {
  int splits;        // quantised-token splits per (b, kv head)
  int total_splits;  // partials per row: splits + 1 workgroups' groups + the residual split
  size_t ws_bytes;
};
DraftQuantPlan plan_draft_quant(const vc_kivi& c, int64_t n_q, int Hq);
hipError_t launch_draft_quant(const vc_kivi& c, int64_t n_q, int r, const void* k_new,
                              const void* v_new, int new_dtype, int64_t new_bh_stride, const void* q,
                              int q_dtype, int Hq, float sm_scale, float* out, float* lse, void* ws,
                              const DraftQuantPlan& plan, hipStream_t s);

// The same with n_q[b] and r[b] + r_add per batch row (device arrays, clamped into the cache);
// plan for n_q_max.
hipError_t launch_draft_quant_rows(const vc_kivi& c, const int64_t* n_q, const int32_t* r, int r_add,
                                   int64_t n_q_max, int r_max, const void* k_new, const void* v_new,
                                   int new_dtype, int64_t new_b_stride, int64_t new_h_stride,
                                   const void* q, int q_dtype, int Hq, float sm_scale, float* out,
                                   float* lse, void* ws, const DraftQuantPlan& plan, hipStream_t s);

// The same call with its workspace in a per-device static scratch array (no allocation):
// counters cleared by a fill kernel on every call, then the same kernel as above.
constexpr size_t DRAFT_NOALLOC_SCRATCH_BYTES = (size_t)4 << 20;
hipError_t draft_scratch_pointer(void** ptr);
hipError_t launch_draft_quant_noalloc(const vc_kivi& c, int64_t n_q, int r, const void* k_new,
                                      const void* v_new, int new_dtype, int64_t new_bh_stride,
                                      const void* q, int q_dtype, int Hq, float sm_scale, float* out,
                                      float* lse, const DraftQuantPlan& plan, hipStream_t s);

// Draft over kept positions.
struct DraftDropPlan {
  int splits;
  size_t ws_bytes;
};
DraftDropPlan plan_draft_drop(int B, int Hkv, int Hq, int64_t n_keep);
hipError_t launch_draft_drop(const void* k, const void* v, int kv_dtype, int B, int Hkv,
                             int64_t tok_cap, const int32_t* idx, int64_t n_keep, int64_t idx_cap,
                             const void* q, int Hq, float sm_scale, float* out, float* lse,
                             void* ws, const DraftDropPlan& plan, hipStream_t s);

// Verify.
struct VerifyPlan {
  int past_splits;      // splits over the device-resident past (or per streamed chunk)
  int chunks;           // streamed chunks (0 when the past is device resident)
  int64_t chunk_tokens;
  int total_splits;     // partials per row
  size_t part_bytes;    // partial buffers
  size_t stage_bytes;   // one chunk stage (K and V), 0 when resident
  size_t ws_bytes;
};
VerifyPlan plan_verify(int B, int Hq, int Hkv, int L, int64_t n, int past_on_host,
                       int64_t chunk_tokens, int dtype);
// Prefill: causal self-attention of n rows (bf16), one launch plus the merge.
struct PrefillPlan {
  int splits;       // tile ranges per row block (partials per row)
  size_t ws_bytes;
};
PrefillPlan plan_prefill(int B, int Hq, int Hkv, int64_t n);
hipError_t launch_prefill(const void* q, const void* k, const void* v, int64_t kv_stride, int64_t n,
                          int B, int Hq, int Hkv, float sm_scale, float* out, float* lse, void* ws,
                          const PrefillPlan& plan, hipStream_t s);
hipError_t launch_verify(const void* q, const void* k_blk, const void* v_blk, int L,
                         const void* k_past, const void* v_past, int64_t past_stride, int64_t n,
                         int past_on_host, int dtype, int B, int Hq, int Hkv, float sm_scale,
                         float* out, float* lse, void* ws, const VerifyPlan& plan,
                         hipStream_t compute, hipStream_t copy, hipEvent_t prefetched);
// Copies of the first two streamed chunks into the workspace stages (past_on_host == 1 plan);
// *done is recorded on `copy` right after them (the caller owns it: the verify that consumes the
// prefetch waits on it, so it never waits for copies enqueued later for other calls).
hipError_t launch_verify_prefetch(const void* k_past, const void* v_past, int64_t past_stride,
                                  int64_t n, int B, int Hkv, void* ws, const VerifyPlan& plan,
                                  hipStream_t compute, hipStream_t copy, hipEvent_t* done);

// Every chunk copy of a host-streamed verify (chunk c into stage c % 2), with no compute.
hipError_t launch_verify_copies(const void* k_past, const void* v_past, int64_t past_stride,
                                int64_t n, int B, int Hkv, void* ws, const VerifyPlan& plan,
                                hipStream_t copy);

// Logits projection (+ argmax).
// Row count from which the projection runs as a tiled fp32 matrix-core product (fewer rows: a
// weight-streaming kernel with the reduction across lanes).
constexpr int TILED_MIN_ROWS = 32;
struct ProjectPlan {
  bool tiled;            // the tiled matrix-core form (M >= TILED_MIN_ROWS)
  int nvt, nmt;          // vocabulary tiles, row tiles
  size_t counter_bytes;  // ticket counters at the start of the workspace (one per row tile)
  size_t ws_bytes;
};
ProjectPlan plan_project(int M, int V);
hipError_t launch_project(const void* W, int w_dtype, int V, const float* o, int B, int Hq, int L,
                          float* z, int32_t* idx, int64_t idx_b_stride, void* ws,
                          const ProjectPlan& plan, hipStream_t s);

// Decoder-layer products for few rows (decoder.hip).
enum { DEC_STORE = 0, DEC_ADD = 1, DEC_ROPE = 2, DEC_SWIGLU = 3 };
struct DecGemv {
  int epi;
  const void* W;
  int w_bf16;
  int N, K, M;
  const float* X;
  const float* g;  // norm gain or null
  float eps;
  float* out;
  void* q_out;
  void* k_out;
  void* v_out;
  int out_bf16;
  int Hq, Hkv;
  const float* cos_t;
  const float* sin_t;
  int n_pos;
  const int32_t* pos;
  int pos_add;
  void* ws;  // null: the vector form; else the matrix-core form's workspace (when it applies)
};
// The matrix-core form of a product: whether it applies (bf16 weights, K % 32 == 0, paired blocks
// of 64 columns), its split of K and the workspace it needs (tickets + slice partials).
struct DecPlan {
  bool mfma;
  int groups, row_tiles, S;
  size_t ws_bytes;
};
DecPlan plan_dec_gemv(int epi, int w_bf16, int N, int K, int M);
hipError_t launch_dec_gemv(const DecGemv& d, hipStream_t s);
hipError_t launch_rmsnorm(const float* X, const float* g, float eps, int M, int K, float* Y,
                          hipStream_t s);
hipError_t launch_embed(const float* E, int V, int K, const int32_t* tok, int64_t tok_stride, int M,
                        float* out, hipStream_t s);

// Keep-list selection (token-dropping drafter).
hipError_t launch_select_keep(const float* scores, int64_t s_stride, int rows, int64_t n, int64_t lo,
                              int64_t hi, int64_t take, int32_t* idx, int64_t idx_stride,
                              hipStream_t s);

}  // namespace vc
