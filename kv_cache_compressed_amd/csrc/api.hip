// C ABI of libvc: host-side argument validation and launch orchestration.
//
// Every argument is checked before anything is enqueued; on error nothing is enqueued and the
// reason is kept in a thread-local string for vc_last_error(). No exception crosses the ABI.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "kernels.h"

static_assert(vc::DRAFT_NOALLOC_SCRATCH_BYTES == VC_DRAFT_NOALLOC_SCRATCH_BYTES,
              "scratch size in vc.h and kernels.h differ");

namespace {

thread_local std::string g_err;

vc_status fail(vc_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

vc_status hip_fail(hipError_t e, const char* where) {
  (void)hipGetLastError();  // clear the sticky launch error of this thread
  return fail(VC_ERR_HIP, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

vc_status ok() {
  g_err.clear();
  return VC_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, ...)                                  \
  do {                                                      \
    if (!(cond)) return fail(VC_ERR_INVALID, __VA_ARGS__);  \
  } while (0)
#define REQUIRE_PTR(p)                                                                \
  do {                                                                                \
    if ((p) == nullptr) return fail(VC_ERR_INVALID, "%s is null", #p);              \
    if (!aligned16(p)) return fail(VC_ERR_INVALID, "%s is not 16-byte aligned", #p); \
  } while (0)

bool valid_dtype(int32_t t) { return t == VC_F32 || t == VC_F16 || t == VC_BF16; }

vc_status check_kivi(const vc_kivi* c) {
  REQUIRE(c != nullptr, "kivi descriptor is null");
  REQUIRE(c->bits == 2 || c->bits == 4, "bits must be 2 or 4 (got %d)", c->bits);
  REQUIRE(c->group == 32, "group must be 32 (got %d)", c->group);
  REQUIRE(c->meta_dtype == VC_F32 || c->meta_dtype == VC_F16, "meta_dtype must be VC_F32 or VC_F16");
  REQUIRE(c->res_dtype == VC_F32 || c->res_dtype == VC_F16, "res_dtype must be VC_F32 or VC_F16");
  REQUIRE(c->B >= 1 && c->Hkv >= 1, "B and Hkv must be >= 1");
  REQUIRE(c->d == 128, "head dim must be 128 (got %d)", c->d);
  REQUIRE(c->res_cap >= 32 && c->res_cap % 32 == 0, "res_cap must be a positive multiple of 32");
  REQUIRE(c->tok_cap >= 0 && c->tok_cap % 32 == 0, "tok_cap must be a non-negative multiple of 32");
  REQUIRE((int64_t)c->B * c->Hkv <= 65535, "B*Hkv must be <= 65535");
  REQUIRE_PTR(c->k_res);
  REQUIRE_PTR(c->v_res);
  if (c->tok_cap > 0) {
    REQUIRE_PTR(c->k_codes);
    REQUIRE_PTR(c->v_codes);
    REQUIRE_PTR(c->k_meta);
    REQUIRE_PTR(c->v_meta);
  }
  return VC_OK;
}

}  // namespace

extern "C" {

int32_t vc_abi_version(void) { return 1; }

const char* vc_last_error(void) { return g_err.c_str(); }

const char* vc_status_string(vc_status s) {
  switch (s) {
    case VC_OK: return "VC_OK";
    case VC_ERR_INVALID: return "VC_ERR_INVALID";
    case VC_ERR_UNSUPPORTED: return "VC_ERR_UNSUPPORTED";
    case VC_ERR_WORKSPACE: return "VC_ERR_WORKSPACE";
    case VC_ERR_HIP: return "VC_ERR_HIP";
    default: return "VC_ERR_UNKNOWN";
  }
}

vc_status vc_quantize_kv(const vc_kivi* c, const void* k, const void* v, int32_t src_dtype,
                         int64_t src_bh_stride, int64_t t0, int64_t ntok, void* stream) {
  if (vc_status st = check_kivi(c)) return st;
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE(valid_dtype(src_dtype), "src_dtype must be VC_F32, VC_F16 or VC_BF16");
  REQUIRE(t0 >= 0 && t0 % 32 == 0, "t0 must be a non-negative multiple of 32");
  REQUIRE(ntok >= 0 && ntok % 32 == 0, "ntok must be a non-negative multiple of 32");
  REQUIRE(t0 + ntok <= c->tok_cap, "t0 + ntok (%lld) exceeds tok_cap (%lld)", (long long)(t0 + ntok),
          (long long)c->tok_cap);
  REQUIRE(src_bh_stride >= ntok * 128, "src_bh_stride must be >= ntok*128");
  if (ntok == 0) return ok();
  hipError_t e = vc::launch_quantize(*c, k, v, src_dtype, src_bh_stride, t0, ntok,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_quantize_kv launch");
  return ok();
}

vc_status vc_kivi_append(const vc_kivi* c, const void* k, const void* v, int32_t src_dtype,
                         int64_t src_bh_stride, int64_t t0, int64_t ntok, void* stream) {
  if (vc_status st = check_kivi(c)) return st;
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE(valid_dtype(src_dtype), "src_dtype must be VC_F32, VC_F16 or VC_BF16");
  REQUIRE(t0 >= 0, "t0 must be >= 0");
  REQUIRE(ntok >= 1 && ntok <= c->res_cap, "ntok must be in [1, res_cap]");
  REQUIRE(src_bh_stride >= ntok * 128, "src_bh_stride must be >= ntok*128");
  hipError_t e = vc::launch_append(*c, k, v, src_dtype, src_bh_stride, t0, ntok,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_kivi_append launch");
  return ok();
}

vc_status vc_draft_quant_workspace(const vc_kivi* c, int64_t n_q, int32_t r, int32_t Hq,
                                   size_t* bytes) {
  if (vc_status st = check_kivi(c)) return st;
  REQUIRE(bytes != nullptr, "bytes is null");
  REQUIRE(n_q >= 0 && n_q % 32 == 0 && n_q <= c->tok_cap, "n_q must be a multiple of 32 in [0, tok_cap]");
  REQUIRE(Hq >= 1 && Hq % c->Hkv == 0, "Hq must be a positive multiple of Hkv");
  (void)r;
  *bytes = vc::plan_draft_quant(*c, n_q, Hq).ws_bytes;
  return ok();
}

vc_status vc_draft_attn_quant(const vc_kivi* c, int64_t n_q, int32_t r, const void* k_new,
                              const void* v_new, int32_t new_dtype, int64_t new_bh_stride,
                              const void* q, int32_t q_dtype, int32_t Hq, float sm_scale, float* out,
                              float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (vc_status st = check_kivi(c)) return st;
  REQUIRE(n_q >= 0 && n_q % 32 == 0 && n_q <= c->tok_cap, "n_q must be a multiple of 32 in [0, tok_cap]");
  REQUIRE(r >= 0 && r <= c->res_cap, "r must be in [0, res_cap]");
  REQUIRE(n_q + r >= 1, "no keys: n_q + r must be >= 1");
  REQUIRE(Hq >= 1 && Hq % c->Hkv == 0, "Hq must be a positive multiple of Hkv");
  REQUIRE(valid_dtype(q_dtype), "q_dtype must be VC_F32, VC_F16 or VC_BF16");
  REQUIRE_PTR(q);
  REQUIRE_PTR(out);
  REQUIRE((k_new == nullptr) == (v_new == nullptr), "k_new and v_new must both be given or both be null");
  if (k_new) {
    REQUIRE(r >= 1, "r must be >= 1 when the step's key/value is passed (it is token n_q + r - 1)");
    REQUIRE(valid_dtype(new_dtype), "new_dtype must be VC_F32, VC_F16 or VC_BF16");
    REQUIRE(new_bh_stride >= 128, "new_bh_stride must be >= 128");
  }
  if (Hq / c->Hkv > 8) return fail(VC_ERR_UNSUPPORTED, "Hq/Hkv > 8 is not supported");
  if (c->res_cap > 512) return fail(VC_ERR_UNSUPPORTED, "res_cap > 512 is not supported");
  if ((int64_t)c->B * c->Hkv > (int64_t)(vc::DRAFT_COUNTER_BYTES / 4))
    return fail(VC_ERR_UNSUPPORTED, "B*Hkv > %d is not supported", (int)(vc::DRAFT_COUNTER_BYTES / 4));
  const vc::DraftQuantPlan plan = vc::plan_draft_quant(*c, n_q, Hq);
  if (ws == nullptr || ws_bytes < plan.ws_bytes || !aligned16(ws))
    return fail(VC_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", plan.ws_bytes,
                ws ? ws_bytes : (size_t)0);
  hipError_t e = vc::launch_draft_quant(*c, n_q, r, k_new, v_new, new_dtype, new_bh_stride, q, q_dtype,
                                        Hq, sm_scale, out, lse, ws, plan, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_draft_attn_quant launch");
  return ok();
}

vc_status vc_draft_attn_quant_rows(const vc_kivi* c, const int64_t* n_q, const int32_t* r,
                                   int32_t r_add, int64_t n_q_max, int32_t r_max, const void* k_new,
                                   const void* v_new, int32_t new_dtype, int64_t new_b_stride,
                                   int64_t new_h_stride, const void* q, int32_t q_dtype, int32_t Hq,
                                   float sm_scale, float* out, float* lse, void* ws, size_t ws_bytes,
                                   void* stream) {
  if (vc_status st = check_kivi(c)) return st;
  REQUIRE(n_q != nullptr && r != nullptr, "n_q and r (device arrays of B entries) are required");
  REQUIRE(n_q_max >= 0 && n_q_max % 32 == 0 && n_q_max <= c->tok_cap,
          "n_q_max must be a multiple of 32 in [0, tok_cap]");
  REQUIRE(r_max >= 1 && r_max <= c->res_cap, "r_max must be in [1, res_cap]");
  REQUIRE(Hq >= 1 && Hq % c->Hkv == 0, "Hq must be a positive multiple of Hkv");
  REQUIRE(valid_dtype(q_dtype), "q_dtype must be VC_F32, VC_F16 or VC_BF16");
  REQUIRE_PTR(q);
  REQUIRE_PTR(out);
  REQUIRE((k_new == nullptr) == (v_new == nullptr), "k_new and v_new must both be given or both be null");
  if (k_new) {
    REQUIRE(valid_dtype(new_dtype), "new_dtype must be VC_F32, VC_F16 or VC_BF16");
    REQUIRE(new_h_stride >= 128 && new_b_stride >= 0, "new_h_stride must be >= 128, new_b_stride >= 0");
  }
  if (Hq / c->Hkv > 8) return fail(VC_ERR_UNSUPPORTED, "Hq/Hkv > 8 is not supported");
  if (c->res_cap > 512) return fail(VC_ERR_UNSUPPORTED, "res_cap > 512 is not supported");
  if ((int64_t)c->B * c->Hkv > (int64_t)(vc::DRAFT_COUNTER_BYTES / 4))
    return fail(VC_ERR_UNSUPPORTED, "B*Hkv > %d is not supported", (int)(vc::DRAFT_COUNTER_BYTES / 4));
  const vc::DraftQuantPlan plan = vc::plan_draft_quant(*c, n_q_max, Hq);
  if (ws == nullptr || ws_bytes < plan.ws_bytes || !aligned16(ws))
    return fail(VC_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", plan.ws_bytes,
                ws ? ws_bytes : (size_t)0);
  hipError_t e = vc::launch_draft_quant_rows(*c, n_q, r, r_add, n_q_max, r_max, k_new, v_new, new_dtype,
                                             new_b_stride, new_h_stride, q, q_dtype, Hq, sm_scale, out,
                                             lse, ws, plan, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_draft_attn_quant_rows launch");
  return ok();
}

vc_status vc_draft_attn_quant_noalloc(const vc_kivi* c, int64_t n_q, int32_t r, const void* k_new,
                                      const void* v_new, int32_t new_dtype, int64_t new_bh_stride,
                                      const void* q, int32_t q_dtype, int32_t Hq, float sm_scale,
                                      float* out, float* lse, void* stream) {
  if (vc_status st = check_kivi(c)) return st;
  REQUIRE(n_q >= 0 && n_q % 32 == 0 && n_q <= c->tok_cap, "n_q must be a multiple of 32 in [0, tok_cap]");
  REQUIRE(r >= 0 && r <= c->res_cap, "r must be in [0, res_cap]");
  REQUIRE(n_q + r >= 1, "no keys: n_q + r must be >= 1");
  REQUIRE(Hq >= 1 && Hq % c->Hkv == 0, "Hq must be a positive multiple of Hkv");
  REQUIRE(valid_dtype(q_dtype), "q_dtype must be VC_F32, VC_F16 or VC_BF16");
  REQUIRE_PTR(q);
  REQUIRE_PTR(out);
  REQUIRE((k_new == nullptr) == (v_new == nullptr), "k_new and v_new must both be given or both be null");
  if (k_new) {
    REQUIRE(r >= 1, "r must be >= 1 when the step's key/value is passed (it is token n_q + r - 1)");
    REQUIRE(valid_dtype(new_dtype), "new_dtype must be VC_F32, VC_F16 or VC_BF16");
    REQUIRE(new_bh_stride >= 128, "new_bh_stride must be >= 128");
  }
  if (Hq / c->Hkv > 8) return fail(VC_ERR_UNSUPPORTED, "Hq/Hkv > 8 is not supported");
  if (c->res_cap > 512) return fail(VC_ERR_UNSUPPORTED, "res_cap > 512 is not supported");
  if ((int64_t)c->B * c->Hkv > (int64_t)(vc::DRAFT_COUNTER_BYTES / 4))
    return fail(VC_ERR_UNSUPPORTED, "B*Hkv > %d is not supported", (int)(vc::DRAFT_COUNTER_BYTES / 4));
  const vc::DraftQuantPlan plan = vc::plan_draft_quant(*c, n_q, Hq);
  if (plan.ws_bytes > vc::DRAFT_NOALLOC_SCRATCH_BYTES)
    return fail(VC_ERR_WORKSPACE,
                "this shape needs %zu bytes of scratch; the no-allocation call has %zu (use "
                "vc_draft_attn_quant with a workspace)", plan.ws_bytes, vc::DRAFT_NOALLOC_SCRATCH_BYTES);
  hipError_t e = vc::launch_draft_quant_noalloc(*c, n_q, r, k_new, v_new, new_dtype, new_bh_stride, q,
                                                q_dtype, Hq, sm_scale, out, lse, plan,
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_draft_attn_quant_noalloc");
  return ok();
}

vc_status vc_draft_drop_workspace(int32_t B, int32_t Hkv, int32_t Hq, int64_t n_keep, size_t* bytes) {
  REQUIRE(bytes != nullptr, "bytes is null");
  REQUIRE(B >= 1 && Hkv >= 1 && Hq >= 1 && Hq % Hkv == 0, "bad head/batch sizes");
  REQUIRE(n_keep >= 1, "n_keep must be >= 1");
  *bytes = vc::plan_draft_drop(B, Hkv, Hq, n_keep).ws_bytes;
  return ok();
}

vc_status vc_draft_attn_drop(const void* k, const void* v, int32_t kv_dtype, int32_t B,
                             int32_t Hkv, int64_t tok_cap, const int32_t* idx, int64_t n_keep,
                             int64_t idx_cap, const void* q, int32_t Hq, float sm_scale,
                             float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(q);
  REQUIRE_PTR(out);
  REQUIRE(valid_dtype(kv_dtype), "kv_dtype must be VC_F32, VC_F16 or VC_BF16");
  REQUIRE(B >= 1 && Hkv >= 1, "B and Hkv must be >= 1");
  REQUIRE(Hq >= 1 && Hq % Hkv == 0, "Hq must be a positive multiple of Hkv");
  REQUIRE(tok_cap >= 1, "tok_cap must be >= 1");
  REQUIRE(n_keep >= 1 && n_keep <= idx_cap, "n_keep must be in [1, idx_cap]");
  REQUIRE((int64_t)B * Hkv <= 65535, "B*Hkv must be <= 65535");
  if (kv_dtype != VC_BF16) return fail(VC_ERR_UNSUPPORTED, "only VC_BF16 keys/values are supported");
  if (Hq / Hkv > 8) return fail(VC_ERR_UNSUPPORTED, "Hq/Hkv > 8 is not supported");
  const vc::DraftDropPlan plan = vc::plan_draft_drop(B, Hkv, Hq, n_keep);
  if (ws == nullptr || ws_bytes < plan.ws_bytes || !aligned16(ws))
    return fail(VC_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", plan.ws_bytes,
                ws ? ws_bytes : (size_t)0);
  hipError_t e = vc::launch_draft_drop(k, v, kv_dtype, B, Hkv, tok_cap, idx, n_keep, idx_cap, q, Hq,
                                       sm_scale, out, lse, ws, plan, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_draft_attn_drop launch");
  return ok();
}

vc_status vc_verify_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t L, int64_t n,
                              int32_t past_on_host, int64_t chunk_tokens, int32_t dtype,
                              size_t* bytes) {
  REQUIRE(bytes != nullptr, "bytes is null");
  REQUIRE(B >= 1 && Hkv >= 1 && Hq >= 1 && Hq % Hkv == 0, "bad head/batch sizes");
  REQUIRE(L >= 1 && L <= 32, "L must be in [1, 32]");
  REQUIRE(n >= 0, "n must be >= 0");
  REQUIRE(dtype == VC_BF16 || dtype == VC_F32, "dtype must be VC_BF16 or VC_F32");
  if (past_on_host) REQUIRE(chunk_tokens >= 32, "chunk_tokens must be >= 32 when streaming");
  *bytes = vc::plan_verify(B, Hq, Hkv, L, n, past_on_host, chunk_tokens, dtype).ws_bytes;
  return ok();
}

vc_status vc_prefill_workspace(int32_t B, int32_t Hq, int32_t Hkv, int64_t n, size_t* bytes) {
  REQUIRE(bytes != nullptr, "bytes is null");
  REQUIRE(B >= 1 && Hkv >= 1 && Hq >= 1 && Hq % Hkv == 0, "bad head/batch sizes");
  REQUIRE(n >= 1, "n must be >= 1");
  *bytes = vc::plan_prefill(B, Hq, Hkv, n).ws_bytes;
  return ok();
}

vc_status vc_prefill_attn(const void* q, const void* k, const void* v, int64_t kv_stride, int64_t n,
                          int32_t B, int32_t Hq, int32_t Hkv, float sm_scale, float* out, float* lse,
                          void* ws, size_t ws_bytes, void* stream) {
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(out);
  REQUIRE(n >= 1, "n must be >= 1");
  REQUIRE(kv_stride >= n, "kv_stride must be >= n");
  REQUIRE(B >= 1 && Hkv >= 1 && Hq >= 1 && Hq % Hkv == 0, "Hq must be a positive multiple of Hkv");
  if (Hq / Hkv > 8) return fail(VC_ERR_UNSUPPORTED, "Hq/Hkv > 8 is not supported");
  // keys of one (b, kv head) are addressed through a buffer resource of < 2^31 bytes
  if (n > (int64_t)8388607) return fail(VC_ERR_UNSUPPORTED, "more than 8388607 tokens per (b, kv head)");
  REQUIRE((int64_t)B * Hkv * ((n + 31) / 32) <= (int64_t)1 << 24, "B*Hkv*ceil(n/32) must be <= 2^24");
  const vc::PrefillPlan plan = vc::plan_prefill(B, Hq, Hkv, n);
  if (ws == nullptr || ws_bytes < plan.ws_bytes || !aligned16(ws))
    return fail(VC_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", plan.ws_bytes,
                ws ? ws_bytes : (size_t)0);
  hipError_t e = vc::launch_prefill(q, k, v, kv_stride, n, B, Hq, Hkv, sm_scale, out, lse, ws, plan,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_prefill_attn launch");
  return ok();
}

namespace {

// Prefetches issued by vc_verify_prefetch and not yet consumed, one per workspace.
struct PendingPrefetch {
  const void* ws;
  const void* k;
  const void* v;
  int64_t stride, n, chunk;
  int32_t B, Hq, Hkv, L;
  hipEvent_t done;  // recorded on the copy stream right after the prefetch's copies
  bool operator==(const PendingPrefetch& o) const {
    return ws == o.ws && k == o.k && v == o.v && stride == o.stride && n == o.n && chunk == o.chunk &&
           B == o.B && Hq == o.Hq && Hkv == o.Hkv && L == o.L;
  }
};
std::mutex g_prefetch_mu;
std::vector<PendingPrefetch> g_prefetch;

// Removes the record of workspace ws; returns whether it equalled `want` (when given). On a match
// the record's event passes to *done (the caller destroys it); otherwise it is destroyed here.
bool take_prefetch(const void* ws, const PendingPrefetch* want, hipEvent_t* done = nullptr) {
  std::lock_guard<std::mutex> lock(g_prefetch_mu);
  for (size_t i = 0; i < g_prefetch.size(); ++i) {
    if (g_prefetch[i].ws != ws) continue;
    const bool match = want && g_prefetch[i] == *want;
    if (match && done)
      *done = g_prefetch[i].done;
    else if (g_prefetch[i].done)
      (void)hipEventDestroy(g_prefetch[i].done);
    g_prefetch.erase(g_prefetch.begin() + i);
    return match;
  }
  return false;
}

vc_status check_pinned(const void* k_past, const void* v_past) {
  for (const void* p : {k_past, v_past}) {
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      return fail(VC_ERR_INVALID, "past_on_host needs pinned host memory (hipHostMalloc); got pageable or device memory");
    }
  }
  return VC_OK;
}

}  // namespace

vc_status vc_verify_prefetch(const void* k_past, const void* v_past, int64_t past_stride, int64_t n,
                             int64_t chunk_tokens, int32_t B, int32_t Hq, int32_t Hkv, int32_t L,
                             void* ws, size_t ws_bytes, void* compute_stream, void* copy_stream) {
  REQUIRE_PTR(k_past);
  REQUIRE_PTR(v_past);
  REQUIRE(L >= 1 && L <= 32, "L must be in [1, 32] (got %d)", L);
  REQUIRE(n >= 1, "a host-streamed past needs n >= 1");
  REQUIRE(past_stride >= n, "past_stride must be >= n");
  REQUIRE(B >= 1 && Hkv >= 1 && Hq >= 1 && Hq % Hkv == 0, "Hq must be a positive multiple of Hkv");
  REQUIRE((int64_t)B * Hkv <= 65535, "B*Hkv must be <= 65535");
  REQUIRE(chunk_tokens >= 32, "chunk_tokens must be >= 32 when streaming");
  if (Hq / Hkv > 8) return fail(VC_ERR_UNSUPPORTED, "Hq/Hkv > 8 is not supported");
  if (std::min<int64_t>(chunk_tokens, n) > (int64_t)8388607)
    return fail(VC_ERR_UNSUPPORTED, "more than 8388607 past tokens per (b, kv head) in one chunk (use a smaller chunk_tokens)");
  const vc_status pin = check_pinned(k_past, v_past);
  if (pin != VC_OK) return pin;
  const vc::VerifyPlan plan = vc::plan_verify(B, Hq, Hkv, L, n, 1, chunk_tokens, VC_BF16);
  if (ws == nullptr || ws_bytes < plan.ws_bytes || !aligned16(ws))
    return fail(VC_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", plan.ws_bytes,
                ws ? ws_bytes : (size_t)0);
  (void)take_prefetch(ws, nullptr);
  hipEvent_t done = nullptr;
  hipError_t e = vc::launch_verify_prefetch(k_past, v_past, past_stride, n, B, Hkv, ws, plan,
                                            static_cast<hipStream_t>(compute_stream),
                                            static_cast<hipStream_t>(copy_stream), &done);
  if (e != hipSuccess) return hip_fail(e, "vc_verify_prefetch");
  std::lock_guard<std::mutex> lock(g_prefetch_mu);
  g_prefetch.push_back({ws, k_past, v_past, past_stride, n, chunk_tokens, B, Hq, Hkv, L, done});
  return ok();
}

vc_status vc_verify_stream_copies(const void* k_past, const void* v_past, int64_t past_stride,
                                  int64_t n, int64_t chunk_tokens, int32_t B, int32_t Hq, int32_t Hkv,
                                  int32_t L, void* ws, size_t ws_bytes, void* copy_stream) {
  REQUIRE_PTR(k_past);
  REQUIRE_PTR(v_past);
  REQUIRE(L >= 1 && L <= 32, "L must be in [1, 32] (got %d)", L);
  REQUIRE(n >= 1, "a host-streamed past needs n >= 1");
  REQUIRE(past_stride >= n, "past_stride must be >= n");
  REQUIRE(B >= 1 && Hkv >= 1 && Hq >= 1 && Hq % Hkv == 0, "Hq must be a positive multiple of Hkv");
  REQUIRE((int64_t)B * Hkv <= 65535, "B*Hkv must be <= 65535");
  REQUIRE(chunk_tokens >= 32, "chunk_tokens must be >= 32 when streaming");
  const vc_status pin = check_pinned(k_past, v_past);
  if (pin != VC_OK) return pin;
  const vc::VerifyPlan plan = vc::plan_verify(B, Hq, Hkv, L, n, 1, chunk_tokens, VC_BF16);
  if (ws == nullptr || ws_bytes < plan.ws_bytes || !aligned16(ws))
    return fail(VC_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", plan.ws_bytes,
                ws ? ws_bytes : (size_t)0);
  (void)take_prefetch(ws, nullptr);  // the stages are overwritten: any pending prefetch is gone
  hipError_t e = vc::launch_verify_copies(k_past, v_past, past_stride, n, B, Hkv, ws, plan,
                                          static_cast<hipStream_t>(copy_stream));
  if (e != hipSuccess) return hip_fail(e, "vc_verify_stream_copies");
  return ok();
}

vc_status vc_verify_attn(const void* q, const void* k_blk, const void* v_blk, int32_t L,
                         const void* k_past, const void* v_past, int64_t past_stride, int64_t n,
                         int32_t past_on_host, int64_t chunk_tokens, int32_t dtype, int32_t B,
                         int32_t Hq, int32_t Hkv, float sm_scale, float* out, float* lse, void* ws,
                         size_t ws_bytes, void* compute_stream, void* copy_stream) {
  REQUIRE_PTR(q);
  REQUIRE_PTR(k_blk);
  REQUIRE_PTR(v_blk);
  REQUIRE_PTR(out);
  REQUIRE(L >= 1 && L <= 32, "L must be in [1, 32] (got %d)", L);
  REQUIRE(n >= 0, "n must be >= 0");
  REQUIRE(past_stride >= n, "past_stride must be >= n");
  REQUIRE(B >= 1 && Hkv >= 1 && Hq >= 1 && Hq % Hkv == 0, "Hq must be a positive multiple of Hkv");
  REQUIRE(dtype == VC_BF16 || dtype == VC_F32, "dtype must be VC_BF16 or VC_F32");
  REQUIRE((int64_t)B * Hkv <= 65535, "B*Hkv must be <= 65535");
  if (n > 0) {
    REQUIRE_PTR(k_past);
    REQUIRE_PTR(v_past);
  }
  if (Hq / Hkv > 8) return fail(VC_ERR_UNSUPPORTED, "Hq/Hkv > 8 is not supported");
  if (dtype == VC_F32) {
    if (past_on_host) return fail(VC_ERR_UNSUPPORTED, "host-streamed past needs VC_BF16");
    if ((int64_t)B * Hq * L > 65535) return fail(VC_ERR_UNSUPPORTED, "VC_F32 verify needs B*Hq*L <= 65535");
  }
  if (dtype == VC_BF16) {
    // one source of the matrix-core kernel (the resident past, or one streamed chunk) is addressed
    // through a buffer resource of at most 2^31 - 1 bytes per (b, kv head): 256 bytes per token
    const int64_t span = past_on_host ? std::min<int64_t>(chunk_tokens, n) : n;
    if (span > (int64_t)8388607)
      return fail(VC_ERR_UNSUPPORTED, "more than 8388607 past tokens per (b, kv head) in one %s",
                  past_on_host ? "chunk (use a smaller chunk_tokens)" : "device-resident past (stream it)");
  }
  REQUIRE(past_on_host == VC_PAST_DEVICE || past_on_host == VC_PAST_HOST ||
              past_on_host == VC_PAST_HOST_PREFETCHED,
          "past_on_host must be VC_PAST_DEVICE, VC_PAST_HOST or VC_PAST_HOST_PREFETCHED");
  if (past_on_host) {
    REQUIRE(chunk_tokens >= 32, "chunk_tokens must be >= 32 when streaming");
    REQUIRE(n >= 1, "a host-streamed past needs n >= 1");
    const vc_status pin = check_pinned(k_past, v_past);
    if (pin != VC_OK) return pin;
  }
  const vc::VerifyPlan plan = vc::plan_verify(B, Hq, Hkv, L, n, past_on_host, chunk_tokens, dtype);
  if (ws == nullptr || ws_bytes < plan.ws_bytes || !aligned16(ws))
    return fail(VC_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", plan.ws_bytes,
                ws ? ws_bytes : (size_t)0);
  // a verify on this workspace consumes (or, without VC_PAST_HOST_PREFETCHED, discards) its prefetch
  const PendingPrefetch want{ws, k_past, v_past, past_stride, n, chunk_tokens, B, Hq, Hkv, L, nullptr};
  hipEvent_t prefetched = nullptr;
  if (!take_prefetch(ws, &want, &prefetched) && past_on_host == VC_PAST_HOST_PREFETCHED)
    return fail(VC_ERR_INVALID, "VC_PAST_HOST_PREFETCHED without a matching vc_verify_prefetch on this workspace");
  if (past_on_host != VC_PAST_HOST_PREFETCHED && prefetched) {  // a prefetch this call does not use
    (void)hipEventDestroy(prefetched);
    prefetched = nullptr;
  }
  hipError_t e = vc::launch_verify(q, k_blk, v_blk, L, k_past, v_past, past_stride, n, past_on_host,
                                   dtype, B, Hq, Hkv, sm_scale, out, lse, ws, plan,
                                   static_cast<hipStream_t>(compute_stream),
                                   static_cast<hipStream_t>(copy_stream), prefetched);
  if (prefetched) (void)hipEventDestroy(prefetched);  // the wait on it is enqueued
  if (e != hipSuccess) return hip_fail(e, "vc_verify_attn");
  return ok();
}

vc_status vc_lse_merge(const float* part_o, const float* part_ml, int64_t rows, int32_t S, int32_t d,
                       float* out, float* lse, void* stream) {
  REQUIRE_PTR(part_o);
  REQUIRE_PTR(part_ml);
  REQUIRE_PTR(out);
  REQUIRE(rows >= 1, "rows must be >= 1");
  REQUIRE(S >= 1 && S <= 4096, "S must be in [1, 4096]");
  REQUIRE(d == 128, "d must be 128");
  REQUIRE((rows + 3) / 4 <= 2147483647LL, "too many rows");
  hipError_t e = vc::launch_merge(part_o, part_ml, rows, S, out, lse, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_lse_merge launch");
  return ok();
}

vc_status vc_accept(const float* logits, const int32_t* drafts, int32_t B, int32_t L, int32_t V,
                    int32_t* accept_len, int32_t* next_token, int32_t* argmax, void* stream) {
  REQUIRE_PTR(logits);
  REQUIRE(accept_len != nullptr, "accept_len is null");
  REQUIRE(next_token != nullptr, "next_token is null");
  REQUIRE(B >= 1, "B must be >= 1");
  REQUIRE(L >= 1 && L <= 64, "L must be in [1, 64] (got %d)", L);
  REQUIRE(V >= 1 && V <= (1 << 30), "V must be in [1, 2^30]");
  if (L > 1) REQUIRE(drafts != nullptr, "drafts is null (needed when L > 1)");
  hipError_t e = vc::launch_accept(logits, drafts, B, L, V, accept_len, next_token, argmax,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_accept launch");
  return ok();
}

vc_status vc_logit_margins(const float* logits, int64_t rows, int32_t V, float* gap, void* stream) {
  REQUIRE_PTR(logits);
  REQUIRE(gap != nullptr, "gap is null");
  REQUIRE(rows >= 1 && rows <= ((int64_t)1 << 31) - 1, "rows must be in [1, 2^31 - 1]");
  REQUIRE(V >= 1 && V <= (1 << 30), "V must be in [1, 2^30]");
  hipError_t e = vc::launch_margins(logits, rows, V, gap, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_logit_margins launch");
  return ok();
}

vc_status vc_hbm_read_stream(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
  REQUIRE_PTR(src);
  REQUIRE(sink != nullptr, "sink is null");
  REQUIRE(bytes >= 16 && bytes % 16 == 0, "bytes must be a positive multiple of 16");
  REQUIRE(blocks >= 1 && blocks <= 65536, "blocks must be in [1, 65536]");
  hipError_t e = vc::launch_read_stream(src, (int64_t)(bytes / 16), sink, blocks,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_hbm_read_stream launch");
  return ok();
}

vc_status vc_project_workspace(int32_t B, int32_t L, int32_t V, size_t* bytes) {
  REQUIRE(bytes != nullptr, "bytes is null");
  REQUIRE(B >= 1 && L >= 1 && (int64_t)B * L <= (1 << 20), "B*L must be in [1, 2^20]");
  REQUIRE(V >= 1 && V <= (1 << 24), "V must be in [1, 2^24]");
  *bytes = vc::plan_project(B * L, V).ws_bytes;
  return ok();
}

vc_status vc_project_logits(const void* W, int32_t w_dtype, int32_t V, const float* o, int32_t B,
                            int32_t Hq, int32_t L, float* logits, int32_t* argmax,
                            int64_t argmax_b_stride, void* ws, size_t ws_bytes, void* stream) {
  REQUIRE_PTR(W);
  REQUIRE_PTR(o);
  REQUIRE(w_dtype == VC_F32 || w_dtype == VC_BF16, "w_dtype must be VC_F32 or VC_BF16");
  REQUIRE(B >= 1 && L >= 1 && (int64_t)B * L <= (1 << 20), "B*L must be in [1, 2^20]");
  REQUIRE(V >= 1 && V <= (1 << 24), "V must be in [1, 2^24]");
  REQUIRE(Hq >= 1 && Hq <= 1024, "Hq must be in [1, 1024]");
  REQUIRE((int64_t)Hq * 128 * V < ((int64_t)1 << 31), "Hq*128*V must be < 2^31");
  REQUIRE(logits != nullptr || argmax != nullptr, "nothing to write: logits and argmax are null");
  if (argmax != nullptr) {
    REQUIRE(argmax_b_stride >= L, "argmax_b_stride must be >= L");
    const vc::ProjectPlan plan = vc::plan_project(B * L, V);
    if (ws == nullptr || ws_bytes < plan.ws_bytes || !aligned16(ws))
      return fail(VC_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu",
                  plan.ws_bytes, ws ? ws_bytes : (size_t)0);
  }
  const vc::ProjectPlan plan = vc::plan_project(B * L, V);
  hipError_t e = vc::launch_project(W, w_dtype, V, o, B, Hq, L, logits, argmax, argmax_b_stride, ws,
                                    plan, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_project_logits launch");
  return ok();
}

vc_status vc_decoder_gemv(int32_t epilogue, const void* W, int32_t w_dtype, int32_t N, int32_t K,
                          const float* X, int32_t M, const float* norm_gain, float eps, float* out,
                          void* q_out, void* k_out, void* v_out, int32_t out_dtype, int32_t Hq,
                          int32_t Hkv, const float* cos_t, const float* sin_t, int32_t n_pos,
                          const int32_t* pos, int32_t pos_add, void* ws, size_t ws_bytes,
                          void* stream) {
  REQUIRE(epilogue == VC_DEC_STORE || epilogue == VC_DEC_ADD || epilogue == VC_DEC_ROPE ||
              epilogue == VC_DEC_SWIGLU,
          "unknown epilogue %d", epilogue);
  REQUIRE_PTR(W);
  REQUIRE_PTR(X);
  REQUIRE(w_dtype == VC_F32 || w_dtype == VC_BF16, "w_dtype must be VC_F32 or VC_BF16");
  REQUIRE(M >= 1 && M <= 4096, "M must be in [1, 4096]");
  REQUIRE(K >= 4 && K % 4 == 0, "K must be a positive multiple of 4");
  REQUIRE(N >= 1, "N must be >= 1");
  REQUIRE((int64_t)N * K < ((int64_t)1 << 31), "N*K must be < 2^31");
  if (norm_gain) {
    REQUIRE_PTR(norm_gain);
    REQUIRE(eps >= 0.f, "eps must be >= 0");
  }
  if (epilogue == VC_DEC_ROPE) {
    REQUIRE(Hq >= 1 && Hkv >= 1 && N == (Hq + 2 * Hkv) * 128, "ROPE: N must be (Hq + 2 Hkv) * 128");
    REQUIRE_PTR(q_out);
    REQUIRE_PTR(k_out);
    REQUIRE_PTR(v_out);
    REQUIRE(out_dtype == VC_F32 || out_dtype == VC_BF16, "out_dtype must be VC_F32 or VC_BF16");
    REQUIRE_PTR(cos_t);
    REQUIRE_PTR(sin_t);
    REQUIRE(pos != nullptr, "pos is null");
    REQUIRE(n_pos >= 1, "n_pos must be >= 1");
  } else {
    REQUIRE_PTR(out);
    if (epilogue == VC_DEC_SWIGLU) REQUIRE(N % 8 == 0, "SWIGLU: N (gate and up columns) must be a multiple of 8");
  }
  vc::DecGemv d{};
  d.epi = epilogue;
  d.W = W;
  d.w_bf16 = w_dtype == VC_BF16;
  d.N = N;
  d.K = K;
  d.M = M;
  d.X = X;
  d.g = norm_gain;
  d.eps = eps;
  d.out = out;
  d.q_out = q_out;
  d.k_out = k_out;
  d.v_out = v_out;
  d.out_bf16 = out_dtype == VC_BF16;
  d.Hq = Hq;
  d.Hkv = Hkv;
  d.cos_t = cos_t;
  d.sin_t = sin_t;
  d.n_pos = n_pos;
  d.pos = pos;
  d.pos_add = pos_add;
  if (ws) {
    const vc::DecPlan p = vc::plan_dec_gemv(epilogue, d.w_bf16, N, K, M);
    REQUIRE_PTR(ws);
    REQUIRE(!p.mfma || ws_bytes >= p.ws_bytes, "ws_bytes %zu < vc_decoder_gemv_workspace() = %zu",
            ws_bytes, p.ws_bytes);
    d.ws = p.mfma ? ws : nullptr;
  }
  hipError_t e = vc::launch_dec_gemv(d, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_decoder_gemv launch");
  return ok();
}

vc_status vc_decoder_gemv_workspace(int32_t epilogue, int32_t w_dtype, int32_t N, int32_t K, int32_t M,
                                    size_t* bytes) {
  REQUIRE(bytes != nullptr, "bytes is null");
  REQUIRE(epilogue == VC_DEC_STORE || epilogue == VC_DEC_ADD || epilogue == VC_DEC_ROPE ||
              epilogue == VC_DEC_SWIGLU,
          "unknown epilogue %d", epilogue);
  REQUIRE(w_dtype == VC_F32 || w_dtype == VC_BF16, "w_dtype must be VC_F32 or VC_BF16");
  REQUIRE(M >= 1 && M <= 4096 && K >= 4 && K % 4 == 0 && N >= 1, "M in [1, 4096], K a positive multiple of 4, N >= 1");
  const vc::DecPlan p = vc::plan_dec_gemv(epilogue, w_dtype == VC_BF16, N, K, M);
  *bytes = p.mfma ? p.ws_bytes : 0;
  return ok();
}

vc_status vc_rmsnorm(const float* X, const float* g, float eps, int32_t M, int32_t K, float* Y,
                     void* stream) {
  REQUIRE_PTR(X);
  REQUIRE_PTR(g);
  REQUIRE_PTR(Y);
  REQUIRE(M >= 1 && M <= 65535, "M must be in [1, 65535]");
  REQUIRE(K >= 1, "K must be >= 1");
  REQUIRE(eps >= 0.f, "eps must be >= 0");
  hipError_t e = vc::launch_rmsnorm(X, g, eps, M, K, Y, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_rmsnorm launch");
  return ok();
}

vc_status vc_embed_rows(const float* E, int32_t V, int32_t K, const int32_t* tok, int64_t tok_stride,
                        int32_t M, float* out, void* stream) {
  REQUIRE_PTR(E);
  REQUIRE_PTR(out);
  REQUIRE(tok != nullptr, "tok is null");
  REQUIRE(V >= 1 && K >= 1 && M >= 1 && M <= 65535, "V, K >= 1 and M in [1, 65535]");
  REQUIRE(tok_stride >= 1, "tok_stride must be >= 1");
  hipError_t e = vc::launch_embed(E, V, K, tok, tok_stride, M, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_embed_rows launch");
  return ok();
}

vc_status vc_workspace_bytes(int32_t op, const int64_t* dims, int32_t ndims, size_t* bytes) {
  REQUIRE(bytes != nullptr, "bytes is null");
  REQUIRE(dims != nullptr || ndims == 0, "dims is null");
  auto need = [&](int k) { return ndims == k; };
  auto fits32 = [&](int k) {
    for (int i = 0; i < k; ++i)
      if (dims[i] < INT32_MIN || dims[i] > INT32_MAX) return false;
    return true;
  };
  switch (op) {
    case VC_OP_DRAFT_QUANT: {  // {B, Hkv, Hq, n_q}
      REQUIRE(need(4), "VC_OP_DRAFT_QUANT takes 4 dims {B, Hkv, Hq, n_q} (got %d)", ndims);
      REQUIRE(fits32(3), "B, Hkv and Hq must fit int32");
      const int64_t B = dims[0], Hkv = dims[1], Hq = dims[2], n_q = dims[3];
      REQUIRE(B >= 1 && Hkv >= 1 && B * Hkv <= 65535, "B, Hkv >= 1 and B*Hkv <= 65535");
      REQUIRE(Hq >= 1 && Hq % Hkv == 0, "Hq must be a positive multiple of Hkv");
      REQUIRE(n_q >= 0 && n_q % 32 == 0, "n_q must be a non-negative multiple of 32");
      vc_kivi c{};
      c.B = (int32_t)B;
      c.Hkv = (int32_t)Hkv;
      c.bits = 2;  // 2-bit caches split the context most finely: the size covers either width
      *bytes = vc::plan_draft_quant(c, n_q, (int)Hq).ws_bytes;
      return ok();
    }
    case VC_OP_DRAFT_DROP:  // {B, Hkv, Hq, n_keep}
      REQUIRE(need(4), "VC_OP_DRAFT_DROP takes 4 dims {B, Hkv, Hq, n_keep} (got %d)", ndims);
      REQUIRE(fits32(3), "B, Hkv and Hq must fit int32");
      return vc_draft_drop_workspace((int32_t)dims[0], (int32_t)dims[1], (int32_t)dims[2], dims[3], bytes);
    case VC_OP_VERIFY:  // {B, Hq, Hkv, L, n, past_on_host, chunk_tokens, dtype}
      REQUIRE(need(8), "VC_OP_VERIFY takes 8 dims {B, Hq, Hkv, L, n, past_on_host, chunk_tokens, dtype} (got %d)",
              ndims);
      REQUIRE(fits32(4) && dims[5] >= INT32_MIN && dims[5] <= INT32_MAX && dims[7] >= INT32_MIN &&
                  dims[7] <= INT32_MAX,
              "B, Hq, Hkv, L, past_on_host and dtype must fit int32");
      return vc_verify_workspace((int32_t)dims[0], (int32_t)dims[1], (int32_t)dims[2], (int32_t)dims[3],
                                 dims[4], (int32_t)dims[5], dims[6], (int32_t)dims[7], bytes);
    case VC_OP_PROJECT:  // {B, L, V}
      REQUIRE(need(3), "VC_OP_PROJECT takes 3 dims {B, L, V} (got %d)", ndims);
      REQUIRE(fits32(3), "B, L and V must fit int32");
      return vc_project_workspace((int32_t)dims[0], (int32_t)dims[1], (int32_t)dims[2], bytes);
    case VC_OP_PREFILL:  // {B, Hq, Hkv, n}
      REQUIRE(need(4), "VC_OP_PREFILL takes 4 dims {B, Hq, Hkv, n} (got %d)", ndims);
      REQUIRE(fits32(3), "B, Hq and Hkv must fit int32");
      return vc_prefill_workspace((int32_t)dims[0], (int32_t)dims[1], (int32_t)dims[2], dims[3], bytes);
    case VC_OP_DECODER:  // {epilogue, w_dtype, N, K, M}
      REQUIRE(need(5), "VC_OP_DECODER takes 5 dims {epilogue, w_dtype, N, K, M} (got %d)", ndims);
      REQUIRE(fits32(5), "epilogue, w_dtype, N, K and M must fit int32");
      return vc_decoder_gemv_workspace((int32_t)dims[0], (int32_t)dims[1], (int32_t)dims[2],
                                       (int32_t)dims[3], (int32_t)dims[4], bytes);
    default:
      return fail(VC_ERR_INVALID, "unknown op %d", op);
  }
}

vc_status vc_select_keep(const float* scores, int64_t score_row_stride, int32_t rows, int64_t n,
                         int64_t sinks, int64_t recent, int64_t keep, int32_t* idx,
                         int64_t idx_row_stride, int64_t* n_keep, void* stream) {
  REQUIRE(n_keep != nullptr, "n_keep is null");
  REQUIRE_PTR(scores);
  REQUIRE_PTR(idx);
  REQUIRE(rows >= 1 && rows <= 65535, "rows must be in [1, 65535] (got %d)", rows);
  REQUIRE(n >= 1 && n <= 0x7fffffffLL, "n must be in [1, 2^31 - 1]");
  REQUIRE(sinks >= 0 && recent >= 0 && keep >= 0, "sinks, recent and keep must be >= 0");
  const int64_t n4 = (n + 3) & ~(int64_t)3;
  REQUIRE(score_row_stride >= n4 && score_row_stride % 4 == 0,
          "score_row_stride must be a multiple of 4 and >= n rounded up to a multiple of 4 (%lld)",
          (long long)n4);
  const int64_t lo = sinks < n ? sinks : n;
  const int64_t hi = (n - recent > lo) ? n - recent : lo;
  const int64_t fixed = lo + (n - hi);
  int64_t take = keep - fixed;
  if (take < 0) take = 0;
  if (take > hi - lo) take = hi - lo;
  const int64_t count = fixed + take;
  REQUIRE(idx_row_stride >= count, "idx_row_stride must be >= the kept count %lld", (long long)count);
  *n_keep = count;
  hipError_t e = vc::launch_select_keep(scores, score_row_stride, rows, n, lo, hi, take, idx,
                                        idx_row_stride, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "vc_select_keep launch");
  return ok();
}

}  // extern "C"
