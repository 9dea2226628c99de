/*
 * vc.h -- C ABI of libvc, the MI355X (gfx950) draft/verify attention path of VeriCache.
 *
 * The method (pages: "VeriCache: making lossy KV compression exact", a blog walk-through;
 * "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference", a knowledge-base summary of
 * the paper): a compressed KV cache in GPU memory drafts x tokens one at a time; one pass of the
 * same model over the full KV cache then predicts every drafted position plus one more; the
 * drafts are accepted up to the first disagreement, where the full-cache token is emitted
 * instead. This library holds the attention and accept steps of that round:
 *
 *   vc_quantize_kv       KIVI-style b-bit quantisation of cached keys/values   (compressor)
 *   vc_kivi_append       append full-precision tokens to the KIVI residual     (compressor)
 *   vc_draft_attn_quant  one-query decode attention over the quantised cache  (draft)
 *   vc_draft_attn_quant_rows  the same with a context length per batch row     (draft)
 *   vc_draft_attn_drop   one-query decode attention over kept positions       (draft)
 *   vc_verify_attn       L-query causal block attention over the full cache   (verify)
 *   vc_verify_prefetch   first chunk copies of a host-streamed verify, issued early (verify)
 *   vc_prefill_attn      causal self-attention of a prompt's rows, one launch   (prefill)
 *   vc_verify_stream_copies  a host-streamed verify's copies alone (its link ceiling) (measurement)
 *   vc_lse_merge         log-sum-exp merge of split partials                  (verify / draft)
 *   vc_accept            per-row argmax, first disagreement, correction token (accept)
 *   vc_logit_margins     top-2 logit gap per row (near-ties, for token comparisons) (harness)
 *   vc_hbm_read_stream   a plain streaming read (the HBM read ceiling)           (measurement)
 *   vc_select_keep       kept positions of a token-dropping drafter           (compressor)
 *   vc_project_logits    logits of the attention outputs (+ greedy argmax): the
 *                        single layer's stand-in for a model head              (harness)
 *   vc_decoder_gemv      fused norm / product / rotation / SwiGLU / residual of
 *   vc_rmsnorm           a decoder layer's few-row steps (the draft step's model) (harness)
 *   vc_embed_rows        embedding rows of a block entry's tokens               (harness)
 *   vc_workspace_bytes   workspace size of any of the calls above               (host only)
 *
 * Conventions (all calls):
 *   - Every buffer is owned by the caller. Device pointers are HIP device memory; the library
 *     allocates nothing and keeps no pointer after the stream work ends.
 *   - Calls are asynchronous on the given stream (a hipStream_t passed as void*, NULL = the
 *     default stream) and re-entrant; the only mutable global state is the host-side record of
 *     pending vc_verify_prefetch calls (one per workspace, behind a mutex).
 *   - Every argument is checked on the host before anything is enqueued; on any error nothing is
 *     enqueued and a status != VC_OK is returned, with a detail string in vc_last_error()
 *     (thread-local). HIP runtime failures return VC_ERR_HIP. No C++ exception crosses the ABI.
 *   - Device pointers must be 16-byte aligned. Head dimension d is 128 everywhere.
 *   - Query head h reads kv head h / (Hq / Hkv) (grouped-query attention, contiguous groups).
 *   - sm_scale multiplies q.k before the softmax (1/sqrt(128) for the pages' models).
 */
#ifndef VC_H
#define VC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t vc_status;
enum {
  VC_OK = 0,
  VC_ERR_INVALID = 1,     /* bad argument (null pointer, shape, alignment, range)          */
  VC_ERR_UNSUPPORTED = 2, /* valid combination that this build does not implement           */
  VC_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the matching *_workspace()   */
  VC_ERR_HIP = 4          /* a HIP runtime call failed; vc_last_error() names it            */
};

enum { VC_F32 = 0, VC_F16 = 1, VC_BF16 = 2 };

/* Where the verify's past lives (vc_verify_attn's past_on_host). */
enum { VC_PAST_DEVICE = 0, VC_PAST_HOST = 1, VC_PAST_HOST_PREFETCHED = 2 };

/*
 * One attention layer's KIVI cache ("VeriCache: Turning Lossy KV Cache into Lossless LLM
 * Inference", Key Contributions: KIVI is one of the quantising drafters; the compressor interface
 * exposes bits per element; Limitations: one uniform bit width). Keys are quantised per channel
 * over groups of 32 consecutive tokens, values per token over groups of 32 consecutive channels;
 * the most recent tokens stay in a full-precision residual ring.
 *
 * Per group of 32 values: min m and max M; stored min m^ = m (fp32 metadata) or the largest fp16
 * <= m (fp16 metadata); stored scale s^ = fl32(fl32(M - m^) / (2^b - 1)), rounded up to fp16 for
 * fp16 metadata; code = 0 if s^ == 0, else clamp(rint_even(fl32(fl32(x - m^) / s^)), 0, 2^b-1);
 * x_hat = code * s^ + m^. Every step is one correctly rounded IEEE operation, so codes and
 * metadata are reproducible bit for bit.
 *
 * Code layout. Codes of each (b, h) form blocks of 32 tokens x 128 channels; block g holds
 * tokens 32g..32g+31 and occupies bytes [32g, 32g+32) x row_bytes of the [tok_cap][row_bytes]
 * buffer (row_bytes = 128*bits/8), i.e. 32*row_bytes contiguous bytes. A block is 64 "lanes" of
 * 2*bits little-endian 32-bit words; word u of lane l is word l*(2*bits)+u of the block. A word
 * has two 16-bit halves hf in {0,1}; half hf holds 16/bits slots s, slot s at bits
 * [16*hf + bits*s, 16*hf + bits*s + bits). With i = l % 16 and gq = l / 16:
 *   keys,   2-bit: token = 16*(u/2) + i,  kb = 2*(u%2) + s/4,  p = s%4
 *   keys,   4-bit: token = 16*(u/4) + i,  kb = u%4,            p = s
 *           both:  channel = 32*kb + 8*gq + 2*p + hf
 *   values, 2-bit: tile = 2*u + s/4,  p = s%4
 *   values, 4-bit: tile = u,          p = s
 *           both:  channel = 16*tile + i,  token = 16*(p/2) + 4*gq + 2*(p%2) + hf
 * (The layout puts the codes one 64-lane matrix-core operand needs into one lane's words.)
 */
typedef struct vc_kivi {
  int32_t bits;       /* 2 or 4                                                         */
  int32_t group;      /* 32                                                             */
  int32_t meta_dtype; /* VC_F32 or VC_F16: storage of (scale, min) pairs                */
  int32_t res_dtype;  /* VC_F32 or VC_F16: storage of residual keys/values              */
  int32_t B, Hkv, d;  /* batch, kv heads, head dim (128)                                 */
  int32_t res_cap;    /* residual ring slots per (b, h); multiple of 32, >= 32          */
  int64_t tok_cap;    /* quantised-token capacity per (b, h); multiple of 32            */
  void *k_codes;      /* [B][Hkv][tok_cap][128*bits/8] uint8, layout above              */
  void *v_codes;      /* [B][Hkv][tok_cap][128*bits/8] uint8, layout above              */
  void *k_meta;       /* [B][Hkv][tok_cap/32][2][128]: per group 128 scales then 128 mins */
  void *v_meta;       /* [B][Hkv][tok_cap][4][2]      (scale, min) in meta_dtype         */
  void *k_res;        /* [B][Hkv][res_cap][128] in res_dtype; token t in slot t % res_cap */
  void *v_res;        /* [B][Hkv][res_cap][128] in res_dtype                             */
} vc_kivi;

/*
 * Quantise tokens t0 .. t0+ntok-1 of every (b, h) into the cache's codes and metadata.
 * Source element (b, h, i, c) (token t0+i) is read at k[((b*Hkv + h)*src_bh_stride) + i*128 + c]
 * (likewise v), src_dtype VC_F32 | VC_F16 | VC_BF16, device memory. t0 and ntok are multiples of
 * 32, t0 + ntok <= tok_cap, src_bh_stride >= ntok*128. Used at prefill (source: the full cache)
 * and to flush 32 residual tokens (source: the ring slots of those tokens).
 * Pages: compressors keep every position at fewer bits ("VeriCache: making lossy KV compression
 * exact", The Tradeoff VeriCache Is Trying to Escape).
 */
vc_status vc_quantize_kv(const vc_kivi *c, const void *k, const void *v, int32_t src_dtype,
                         int64_t src_bh_stride, int64_t t0, int64_t ntok, void *stream);

/*
 * Write tokens t0 .. t0+ntok-1 (same source addressing as vc_quantize_kv) into the residual ring
 * slots (t0+i) % res_cap, converted to res_dtype with round-half-even. 1 <= ntok <= res_cap.
 */
vc_status vc_kivi_append(const vc_kivi *c, const void *k, const void *v, int32_t src_dtype,
                         int64_t src_bh_stride, int64_t t0, int64_t ntok, void *stream);

/*
 * Draft attention over the KIVI cache ("VeriCache: making lossy KV compression exact", The Core
 * Idea: the model drafts each token over the compressed cache; Verifying Without Giving Back the
 * Speedup: drafting is bound by GPU memory bandwidth).
 * For every (b, query head h): keys/values = dequantised tokens 0..n_q-1 followed by residual
 * tokens n_q..n_q+r-1 (ring slots); s_t = sm_scale * q.k_t; out = softmax(s) . V;
 * lse = log-sum-exp of s (natural log).
 *   k_new, v_new  NULL, or the drafting step's own key/value: residual token n_q + r - 1 (r >= 1),
 *        rows of 128 for each (b, kv head), new_bh_stride elements apart, in new_dtype, device.
 *        It is stored into ring slot (n_q + r - 1) % res_cap (as vc_kivi_append would store it)
 *        before the attention reads the residual, which saves a separate append launch per step.
 *   q    [B][Hq][128] in q_dtype (VC_F32 | VC_BF16 | VC_F16), device
 *   out  [B][Hq][128] fp32, device;  lse [B][Hq] fp32 or NULL
 *   n_q  multiple of 32, <= tok_cap;  0 <= r <= res_cap;  n_q + r >= 1;  Hq % Hkv == 0,
 *        Hq/Hkv <= 8;  B*Hkv <= 16384
 *   ws   device workspace of at least vc_draft_quant_workspace() bytes: its first 64 KB hold one
 *        ticket counter per (b, kv head), the rest the split partials. Zero-fill the workspace
 *        once after allocating it; every call leaves the counters at zero again, so a workspace
 *        can then be reused for any later call (any shape). Calls that overlap in time must not
 *        share a workspace. The splits and their log-sum-exp merge run in one kernel.
 */
vc_status vc_draft_attn_quant(const vc_kivi *c, int64_t n_q, int32_t r, const void *k_new,
                              const void *v_new, int32_t new_dtype, int64_t new_bh_stride,
                              const void *q, int32_t q_dtype, int32_t Hq, float sm_scale, float *out,
                              float *lse, void *ws, size_t ws_bytes, void *stream);
vc_status vc_draft_quant_workspace(const vc_kivi *c, int64_t n_q, int32_t r, int32_t Hq,
                                   size_t *bytes);
/*
 * vc_draft_attn_quant with a context length per batch row: batch row b attends over its own
 * quantised tokens and residual tokens ("VeriCache: making lossy KV compression exact", The Core
 * Idea: each request of a batch accepts its own number of drafts per round, so the requests' cached
 * lengths drift apart; one launch then serves the whole batch).
 *   n_q, r   device arrays of c->B int64 / int32 entries: row b has n_q[b] quantised tokens and
 *            r[b] + r_add residual tokens (r_add lets one array serve every draft step of a round,
 *            e.g. r = n - n_q and r_add = j + 1 at step j). Values are read by the kernel, so they
 *            are not checked: each row's n_q is clamped to [0, tok_cap] and rounded down to a
 *            multiple of 32, its residual count clamped to [0, res_cap]; a row left with no key gets
 *            out = 0, lse = -inf.
 *   n_q_max, r_max  host bounds of every row's values (they size the launch and the workspace,
 *            vc_draft_quant_workspace(c, n_q_max, r_max, Hq) bytes)
 *   k_new, v_new  NULL, or (b, kv head)'s row of 128 at b * new_b_stride + h * new_h_stride elements
 *            (any batch-row stride, e.g. the k part of a fused q/k/v row), stored at each row's own
 *            residual position before attending (each row's residual count must then be >= 1)
 *   other arguments as for vc_draft_attn_quant. The lengths live in device memory so a captured
 *   graph of a draft phase stays valid from round to round while the caller updates them.
 * Results per row equal the scalar call's on that row alone up to fp32 summation order (the split of
 * the work follows n_q_max).
 */
vc_status vc_draft_attn_quant_rows(const vc_kivi *c, const int64_t *n_q, const int32_t *r,
                                   int32_t r_add, int64_t n_q_max, int32_t r_max, const void *k_new,
                                   const void *v_new, int32_t new_dtype, int64_t new_b_stride,
                                   int64_t new_h_stride, const void *q, int32_t q_dtype, int32_t Hq,
                                   float sm_scale, float *out, float *lse, void *ws, size_t ws_bytes,
                                   void *stream);

/*
 * vc_draft_attn_quant for callers that cannot allocate device memory: code being captured into a
 * HIP graph, tight serving loops, harnesses that forbid hipMalloc. Same arguments, same kernels and
 * the same results, without the workspace: the ticket counters and split partials live in a static
 * scratch array of VC_DRAFT_NOALLOC_SCRATCH_BYTES (4 MiB) that the library holds on every GPU it
 * runs on until the process ends. Calls whose workspace (vc_draft_quant_workspace) would exceed it
 * return VC_ERR_WORKSPACE and enqueue nothing (the c2 shape, B 8, 8 kv heads, 32 query heads,
 * needs ~1.7 MB). Each call first clears the counters it uses with a fill kernel on `stream`. All
 * calls on one GPU share that GPU's scratch: calls that overlap in time on one GPU (concurrent
 * streams, threads) race and must be serialised by the caller. Allocates nothing.
 */
#define VC_DRAFT_NOALLOC_SCRATCH_BYTES (4u << 20)
vc_status vc_draft_attn_quant_noalloc(const vc_kivi *c, int64_t n_q, int32_t r, const void *k_new,
                                      const void *v_new, int32_t new_dtype, int64_t new_bh_stride,
                                      const void *q, int32_t q_dtype, int32_t Hq, float sm_scale,
                                      float *out, float *lse, void *stream);

/*
 * Draft attention over kept positions of a token-dropping compressor ("VeriCache: Turning Lossy KV
 * Cache into Lossless LLM Inference", Key Contributions: the interface exposes dropped positions;
 * Limitations: identical drop counts for every head).
 * For every (b, query head h, kv head g = h/(Hq/Hkv)): keys/values = rows idx[b][g][0..n_keep-1]
 * of k/v[b][g]; same attention as above.
 *   k, v  [B][Hkv][tok_cap][128] bf16 (kv_dtype must be VC_BF16; other dtypes return
 *         VC_ERR_UNSUPPORTED), device
 *   idx   [B][Hkv][idx_cap] int32 positions; entries outside [0, tok_cap) contribute nothing
 *   q     [B][Hq][128] bf16; out [B][Hq][128] fp32; lse [B][Hq] or NULL
 *   1 <= n_keep <= idx_cap;  ws as for vc_draft_attn_quant (vc_draft_drop_workspace() bytes).
 */
vc_status vc_draft_attn_drop(const void *k, const void *v, int32_t kv_dtype, int32_t B,
                             int32_t Hkv, int64_t tok_cap, const int32_t *idx, int64_t n_keep,
                             int64_t idx_cap, const void *q, int32_t Hq, float sm_scale,
                             float *out, float *lse, void *ws, size_t ws_bytes, void *stream);
vc_status vc_draft_drop_workspace(int32_t B, int32_t Hkv, int32_t Hq, int64_t n_keep,
                                  size_t *bytes);

/*
 * Verify attention ("VeriCache: making lossy KV compression exact", The Core Idea: one pass over
 * the full cache yields a prediction for every drafted position plus one; Verifying Without Giving
 * Back the Speedup: the full cache may live in CPU memory and be brought in only to verify).
 * Row i (0 <= i < L) of query head h is at position n+i and attends over past tokens 0..n-1 and
 * block tokens 0..i (causal). Split-K partials over the past (and over the block) are merged with
 * log-sum-exp.
 *   q            [B][Hq][L][128] in dtype, device
 *   k_blk, v_blk [B][Hkv][L][128] in dtype, device (keys/values of positions n..n+L-1)
 *   k_past, v_past  element (b, h, t, c) at [((b*Hkv + h)*past_stride + t)*128 + c], dtype;
 *                device memory (past_on_host = VC_PAST_DEVICE), or pinned host memory
 *                (VC_PAST_HOST: streamed in chunks of chunk_tokens tokens through the workspace,
 *                copies on `copy`, compute on `compute`; pageable host memory is rejected; or
 *                VC_PAST_HOST_PREFETCHED: the same, with the first two chunks' copies already
 *                issued by vc_verify_prefetch with identical past, sizes and workspace, which this
 *                call consumes; VC_ERR_INVALID without a matching prefetch). past_stride >= n.
 *   out          [B][Hq][L][128] fp32; lse [B][Hq][L] fp32 or NULL
 *   dtype        VC_BF16 (matrix-core path) or VC_F32 (vector path; device-resident past only)
 *   1 <= L <= 32, n >= 0, Hq % Hkv == 0, Hq/Hkv <= 8; VC_BF16: at most 8388607 tokens per
 *   (b, kv head) in a resident past or in one streamed chunk (else VC_ERR_UNSUPPORTED).
 *   ws           vc_verify_workspace() bytes (partials, plus two chunk stages when streaming).
 * The host past must stay valid until `compute` has passed this call: `compute` waits for every
 * copy, so synchronising `compute` suffices.
 */
vc_status vc_verify_attn(const void *q, const void *k_blk, const void *v_blk, int32_t L,
                         const void *k_past, const void *v_past, int64_t past_stride, int64_t n,
                         int32_t past_on_host, int64_t chunk_tokens, int32_t dtype, int32_t B,
                         int32_t Hq, int32_t Hkv, float sm_scale, float *out, float *lse, void *ws,
                         size_t ws_bytes, void *compute_stream, void *copy_stream);
/*
 * Prefill attention: causal self-attention of a prompt's n rows, the pass that fills the caches
 * before the first round ("VeriCache: making lossy KV compression exact", The Core Idea: both the
 * full and the compressed cache hold the prompt's keys and values before drafting starts). Row i
 * (position i) of query head h attends over tokens 0..i of kv head h / (Hq/Hkv); the same
 * arithmetic as the bf16 verify (bf16 products on the matrix cores, fp32 scores, the softmax
 * weights as a bf16 hi + lo pair, split partials merged with log-sum-exp): 32-row blocks, each
 * over the key tiles up to its own (the diagonal tile masked), the longest blocks first, all in
 * one launch plus the merge.
 *   q      [B][Hq][n][128] bf16, device
 *   k, v   element (b, h, t, c) at [((b*Hkv + h)*kv_stride + t)*128 + c], bf16, device;
 *          kv_stride >= n
 *   out    [B][Hq][n][128] fp32; lse [B][Hq][n] fp32 (natural log) or NULL
 *   n >= 1 (at most 8388607), Hq % Hkv == 0, Hq/Hkv <= 8 (else VC_ERR_UNSUPPORTED),
 *   B*Hkv*ceil(n/32) <= 2^24; ws: vc_prefill_workspace() bytes (split partials).
 */
vc_status vc_prefill_attn(const void *q, const void *k, const void *v, int64_t kv_stride, int64_t n,
                          int32_t B, int32_t Hq, int32_t Hkv, float sm_scale, float *out, float *lse,
                          void *ws, size_t ws_bytes, void *stream);
vc_status vc_prefill_workspace(int32_t B, int32_t Hq, int32_t Hkv, int64_t n, size_t *bytes);

/*
 * Prefetch of a host-streamed verify ("VeriCache: making lossy KV compression exact", Verifying
 * Without Giving Back the Speedup: the full cache is brought in from CPU memory only to verify; the
 * committed past of a round is known before its drafts are, so its first chunks can cross the link
 * while the draft steps run). Issues on `copy`, after the work already enqueued on `compute`, the
 * host-to-device copies of the first two chunks of the past into the workspace's chunk stages,
 * exactly as vc_verify_attn with VC_PAST_HOST would, and records (host side) that the workspace
 * holds them. The next vc_verify_attn on this workspace with VC_PAST_HOST_PREFETCHED and the same
 * k_past, v_past, past_stride, n, chunk_tokens, B, Hq, Hkv and L skips those copies; any other
 * verify on the workspace discards the record. The caller must not write past rows < n, nor use
 * the workspace for anything else, between the two calls, and must use the same copy stream.
 * Arguments as for vc_verify_attn (VC_BF16 past in pinned host memory, n >= 1).
 */
vc_status vc_verify_prefetch(const void *k_past, const void *v_past, int64_t past_stride, int64_t n,
                             int64_t chunk_tokens, int32_t B, int32_t Hq, int32_t Hkv, int32_t L,
                             void *ws, size_t ws_bytes, void *compute_stream, void *copy_stream);
vc_status vc_verify_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t L, int64_t n,
                              int32_t past_on_host, int64_t chunk_tokens, int32_t dtype,
                              size_t *bytes);
/*
 * The transfer of a host-streamed verify on its own ("VeriCache: making lossy KV compression exact",
 * Verifying Without Giving Back the Speedup: the full cache crosses the CPU-GPU link to be
 * verified; the copy is the bound of that verify). Issues on `copy` exactly the host-to-device copies
 * vc_verify_attn with VC_PAST_HOST issues for the same arguments (chunk c of every (b, kv head) into
 * workspace stage c % 2, one 2-D copy per chunk per tensor) and nothing else: no compute, no waits
 * between chunks. It measures the link's rate for the verify's own transfer pattern (the ceiling
 * a streamed verify is compared against). The stages' contents are unspecified afterwards; a pending
 * vc_verify_prefetch on the workspace is discarded. Arguments as for vc_verify_prefetch.
 */
vc_status vc_verify_stream_copies(const void *k_past, const void *v_past, int64_t past_stride,
                                  int64_t n, int64_t chunk_tokens, int32_t B, int32_t Hq,
                                  int32_t Hkv, int32_t L, void *ws, size_t ws_bytes,
                                  void *copy_stream);

/*
 * Log-sum-exp merge of S split partials per row (the pages are silent on how split work is
 * combined; this is the exact recombination of softmax partials):
 *   part_o  [rows][S][d] fp32: o_s = sum_t e^{s_t - m_s} v_t over split s
 *   part_ml [rows][S][2] fp32: (m_s, l_s = sum_t e^{s_t - m_s}); l_s == 0 marks an empty split
 *   m = max m_s;  out = sum_s o_s e^{m_s - m} / sum_s l_s e^{m_s - m};  lse = m + ln(sum ...)
 *   out [rows][d] fp32, lse [rows] or NULL. A row with no live split gets out = 0, lse = -inf.
 *   1 <= S <= 4096, d == 128.
 */
vc_status vc_lse_merge(const float *part_o, const float *part_ml, int64_t rows, int32_t S,
                       int32_t d, float *out, float *lse, void *stream);

/*
 * Greedy accept ("VeriCache: making lossy KV compression exact", The Core Idea, Figure 1 and the
 * worked example): v_i = argmax logits[b][i] (lowest index on ties) for i < L; a = first i < L-1
 * with drafts[b][i] != v_i, or L-1 if none; next = v_a (the correction, or the bonus token).
 * With L == 1 this is plain greedy argmax (drafts may be NULL).
 *   logits     [B][L][V] fp32, finite; drafts [B][L-1] int32
 *   accept_len [B] int32 (a);  next_token [B] int32;  argmax [B][L] int32 or NULL
 *   1 <= L <= 64, 1 <= V <= 2^30.
 */
vc_status vc_accept(const float *logits, const int32_t *drafts, int32_t B, int32_t L, int32_t V,
                    int32_t *accept_len, int32_t *next_token, int32_t *argmax, void *stream);

/*
 * Top-2 margins of logits rows, for comparing two decodings token by token: a row whose two best
 * logits lie within a tolerance is a near-tie, where two correct computations may pick different
 * tokens. Not part of the round.
 *   gap[r] = z_best - z_second over distinct indices of logits[r][0..V-1] (0 when the best value
 *   occurs twice; +inf when V == 1); logits [rows][V] fp32 finite, gap [rows] fp32, device.
 */
vc_status vc_logit_margins(const float *logits, int64_t rows, int32_t V, float *gap, void *stream);

/*
 * Plain streaming read of `bytes` of device memory (measurement: the HBM read rate a
 * bandwidth-bound kernel is set against, beside the 8 TB/s peak; not part of the round).
 * `blocks` workgroups of 256 threads stride over src with 16-byte loads and each thread writes
 * the XOR of what it read to sink[blocks * 256] (uint32, device), so every load is kept.
 * bytes a positive multiple of 16, src 16-byte aligned, 1 <= blocks <= 65536.
 */
vc_status vc_hbm_read_stream(const void *src, size_t bytes, uint32_t *sink, int32_t blocks, void *stream);

/*
 * Logits projection, the round's stand-in for a model's output head (a single attention layer has
 * none): z[b][i][v] = sum_{h < Hq, c < 128} W[v][128 h + c] * o[b][h][i][c], fp32 with fp32
 * accumulation, optionally fused with the greedy argmax of every row ("VeriCache: making lossy KV
 * compression exact", The Core Idea and Figure 1: the draft's greedy token at every drafted
 * position). Not one of the five calls of the path; it turns their outputs into tokens.
 *   W      [V][Hq*128], device, w_dtype VC_F32 or VC_BF16 (bf16 weights are widened exactly, so
 *          bf16-valued weights give the same result in either dtype);  o [B][Hq][L][128] fp32,
 *          device (the attention outputs: draft steps have L == 1, the verify block L rows; any
 *          row of Hq*128 values, so one-row calls are plain weight-bound GEMVs)
 *   logits [B][L][V] fp32 or NULL
 *   argmax row (b, i) written to argmax[b * argmax_b_stride + i] (lowest index on ties; -0 and +0
 *          tie; logits are expected finite), or NULL
 *   ws     device, >= vc_project_workspace bytes, 16-byte aligned; zero-filled once before first
 *          use (ticket counters and per-row argmax slots; every call leaves them zero); may be
 *          NULL when argmax is NULL.
 *          Calls that share a workspace must not overlap.
 *   1 <= B*L <= 2^20, 1 <= V <= 2^24, 1 <= Hq <= 1024, Hq*128*V < 2^31.
 */
vc_status vc_project_workspace(int32_t B, int32_t L, int32_t V, size_t *bytes);
vc_status vc_project_logits(const void *W, int32_t w_dtype, int32_t V, const float *o, int32_t B,
                            int32_t Hq, int32_t L, float *logits, int32_t *argmax,
                            int64_t argmax_b_stride, void *ws, size_t ws_bytes, void *stream);

/*
 * Keep-list selection of a token-dropping drafter ("VeriCache: making lossy KV compression exact",
 * The Tradeoff VeriCache Is Trying to Escape: token-dropping compressors keep attention sinks and
 * recent tokens, or score cached entries and evict the least useful; "VeriCache: Turning Lossy KV
 * Cache into Lossless LLM Inference", Key Contributions: the compressor interface exposes the
 * dropped positions; Limitations: the same number dropped in every head). The pages give no
 * scoring rule; scores are an input. For each of `rows` rows (one per (batch row, kv head)):
 *   lo = min(sinks, n), hi = max(lo, n - recent), fixed = lo + (n - hi),
 *   take = min(max(0, keep - fixed), hi - lo),
 *   kept = [0, lo) + the take highest-scoring positions of [lo, hi) + [hi, n), ascending;
 *   ranking: larger score first, equal scores (-0 == +0) by lower position, NaN below every
 *   number. The count lo + (n - hi) + take is the same for every row and is returned in *n_keep
 *   (host memory, written before the launch).
 *   scores  fp32 device, row r at scores + r * score_row_stride; score_row_stride a multiple of 4
 *           and >= n rounded up to a multiple of 4 (the buffer holds rows * score_row_stride floats:
 *           the kernel reads whole 16-byte groups)
 *   idx     int32 device, row r's kept positions at idx + r * idx_row_stride (idx_row_stride >=
 *           *n_keep); entries past *n_keep are not written
 *   1 <= rows <= 65535, 1 <= n <= 2^31 - 1, sinks, recent, keep >= 0.
 */
vc_status vc_select_keep(const float *scores, int64_t score_row_stride, int32_t rows, int64_t n,
                         int64_t sinks, int64_t recent, int64_t keep, int32_t *idx,
                         int64_t idx_row_stride, int64_t *n_keep, void *stream);

/*
 * Decoder-layer products for few rows: the layer work of a draft step around its attention, for a
 * decoder whose drafter and verifier are the same model ("VeriCache: making lossy KV compression
 * exact", The Core Idea: the drafter decodes each draft token with the full model over the
 * compressed cache). Llama-form layers (pre-norm RMSNorm, rotary q/k, SwiGLU MLP). Not one of the
 * path's five calls: they feed it.
 *   Y[m][n] = s_m * sum_k X[m][k] g[k] W[n][k], m < M, n < N, k < K (K % 4 == 0), fp32 products and
 *   sums; W [N][K] fp32 or bf16 (widened exactly), X [M][K] fp32 device, g = norm_gain [K] or NULL;
 *   with a gain s_m = 1 / sqrt(mean_k X[m][k]^2 + eps) (the row's RMS norm), else s_m = 1, g = 1.
 *   epilogue VC_DEC_STORE   out [M][N] = Y
 *            VC_DEC_ADD     out [M][N] += Y (a residual stream)
 *            VC_DEC_ROPE    Y = [q | k | v] heads of 128 (N = (Hq + 2 Hkv) 128); q and k heads are
 *                           rotated, channel i < 64 with i + 64 at angle index p = pos[m] + pos_add:
 *                           (y_i c - y_{i+64} s, y_{i+64} c + y_i s), c = cos_t[p][i], s = sin_t[p][i]
 *                           (tables [n_pos][64] fp32; p is clamped to [0, n_pos)); q_out [M][Hq][128],
 *                           k_out/v_out [M][Hkv][128] in out_dtype (VC_F32, or VC_BF16 rounded to
 *                           nearest even)
 *            VC_DEC_SWIGLU  Y = [gate | up] (N = 2F, N % 8 == 0): out [M][F] = silu(gate) * up
 *   Unused pointers may be NULL.
 *   ws: NULL selects the vector form (each weight read once per 16 rows; X re-read per 4 columns).
 *   Otherwise, for bf16 weights with K % 32 == 0 (and for VC_DEC_SWIGLU N % 128 == 0), the
 *   matrix-core form runs: X (times the gain) split exactly into three bf16 pieces, bf16 products
 *   (exact) summed in fp32, K cut into slices whose partial tiles are added in slice order by the
 *   last slice to finish (deterministic). ws then holds >= vc_decoder_gemv_workspace() bytes of
 *   device memory, zero-filled before its first use; its layout (16 KB of tickets, then the slice
 *   partials) is the same for every shape, and every completed call leaves its tickets at zero
 *   again, so one workspace sized for the largest of several products serves them all. Calls that
 *   share a workspace must not overlap (same stream, or ordered). Where the matrix-core form does
 *   not apply, ws is ignored. VC_ERR_INVALID if ws_bytes is too small.
 * vc_decoder_gemv_workspace: that size (0 where the matrix-core form does not apply), host only.
 * vc_rmsnorm: Y[m] = X[m] * g / sqrt(mean(X[m]^2) + eps), X, Y [M][K] fp32 (may alias).
 * vc_embed_rows: out[m] = E[tok[m * tok_stride]] for m < M, E [V][K] fp32, tok int32 (device, any
 *   stride, e.g. one block entry of every request); an id outside [0, V) gives a zero row.
 */
enum { VC_DEC_STORE = 0, VC_DEC_ADD = 1, VC_DEC_ROPE = 2, VC_DEC_SWIGLU = 3 };
vc_status vc_decoder_gemv(int32_t epilogue, const void *W, int32_t w_dtype, int32_t N, int32_t K,
                          const float *X, int32_t M, const float *norm_gain, float eps, float *out,
                          void *q_out, void *k_out, void *v_out, int32_t out_dtype, int32_t Hq,
                          int32_t Hkv, const float *cos_t, const float *sin_t, int32_t n_pos,
                          const int32_t *pos, int32_t pos_add, void *ws, size_t ws_bytes,
                          void *stream);
vc_status vc_decoder_gemv_workspace(int32_t epilogue, int32_t w_dtype, int32_t N, int32_t K, int32_t M,
                                    size_t *bytes);
vc_status vc_rmsnorm(const float *X, const float *g, float eps, int32_t M, int32_t K, float *Y,
                     void *stream);
vc_status vc_embed_rows(const float *E, int32_t V, int32_t K, const int32_t *tok, int64_t tok_stride,
                        int32_t M, float *out, void *stream);

/*
 * Workspace size of any call that takes one, by operation code and its size arguments (the same
 * values as the per-operation queries, which it forwards to; host only, nothing enqueued):
 *   VC_OP_DRAFT_QUANT  dims {B, Hkv, Hq, n_q}                                (vc_draft_attn_quant;
 *                      the size for 2-bit codes, which is also enough for 4-bit ones)
 *   VC_OP_DRAFT_DROP   dims {B, Hkv, Hq, n_keep}                             (vc_draft_attn_drop)
 *   VC_OP_VERIFY       dims {B, Hq, Hkv, L, n, past_on_host, chunk_tokens, dtype}  (vc_verify_attn,
 *                      vc_verify_prefetch, vc_verify_stream_copies)
 *   VC_OP_PROJECT      dims {B, L, V}                                        (vc_project_logits)
 *   VC_OP_DECODER      dims {epilogue, w_dtype, N, K, M}                     (vc_decoder_gemv)
 *   VC_OP_PREFILL      dims {B, Hq, Hkv, n}                                  (vc_prefill_attn)
 * A wrong count of dims or an unknown op returns VC_ERR_INVALID. The pages give the calls of the
 * path, not their memory; the caller owns every workspace ("VeriCache: Turning Lossy KV Cache into
 * Lossless LLM Inference", Key Contributions: one interface for every compressor).
 */
enum { VC_OP_DRAFT_QUANT = 1, VC_OP_DRAFT_DROP = 2, VC_OP_VERIFY = 3, VC_OP_PROJECT = 4, VC_OP_DECODER = 5,
       VC_OP_PREFILL = 6 };
vc_status vc_workspace_bytes(int32_t op, const int64_t *dims, int32_t ndims, size_t *bytes);

const char *vc_status_string(vc_status s);
const char *vc_last_error(void);
int32_t vc_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* VC_H */
