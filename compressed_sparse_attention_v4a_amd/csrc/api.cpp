// C ABI of libv4a.so: argument validation, workspace sizing, dispatch.
// Declarations and their documentation are in include/v4a.h.
#include "../../include/v4a.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.h"

namespace {

thread_local char g_err[512] = "";
std::atomic<int> g_policy{0};

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return V4A_OK;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(V4A_EIO, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

int check_attn_common(const void* q, const void* kv_comp, const void* out, int n_h, int c,
                      int rope_dims, int w, v4a_dtype dt, int batch, float eps) {
  REQUIRE(q && kv_comp && out, V4A_EINVAL, "null q, kv_comp or out");
  REQUIRE(batch >= 1, V4A_EINVAL, "batch must be >= 1 (got %d)", batch);
  REQUIRE(n_h >= 1, V4A_EINVAL, "n_h must be >= 1 (got %d)", n_h);
  REQUIRE(c >= 2 && c % 2 == 0, V4A_EINVAL, "c must be even and >= 2 (got %d)", c);
  REQUIRE(c <= 1024, V4A_ENOTSUP, "c > 1024 is not supported (got %d)", c);
  REQUIRE(rope_dims >= 0 && rope_dims % 2 == 0 && rope_dims <= c, V4A_EINVAL,
          "rope_dims must be even and in [0, c] (got %d)", rope_dims);
  REQUIRE(rope_dims <= v4a::kMaxRopeDims, V4A_ENOTSUP, "rope_dims > %d is not supported",
          v4a::kMaxRopeDims);
  REQUIRE(w >= 1, V4A_EINVAL, "w must be >= 1 (got %d)", w);
  REQUIRE(dt == V4A_F32 || dt == V4A_BF16, V4A_ENOTSUP, "attention dtype must be F32 or BF16");
  REQUIRE(eps >= 0.0f && std::isfinite(eps), V4A_EINVAL, "eps must be finite and >= 0");
  return V4A_OK;
}

}  // namespace

namespace v4a {
int report_error(int code, const char* msg) { return fail(code, "%s", msg); }

void rope_table(RopeTab& tab, int rope_dims, float rope_base) {
  for (int i = 0; i < kMaxRopeDims / 2; ++i)
    tab.inv_freq[i] = (2 * i < rope_dims) ? std::pow((double)rope_base, -2.0 * (double)i / (double)rope_dims)
                                           : 0.0;
}
}  // namespace v4a

extern "C" {

const char* v4a_last_error(void) { return g_err; }

const char* v4a_version(void) { return "v4a 0.1.0 gfx950"; }

int v4a_set_kernel_policy(int policy) {
  if (policy != 0 && policy != 1) return g_policy.load();
  return g_policy.exchange(policy);
}

int v4a_visibility(int64_t t0, int T, int m, int k, int w, int32_t* E, int32_t* cnt,
                   int32_t* win_lo, int32_t* win_len, void* stream) {
  REQUIRE(t0 >= 0 && T >= 0, V4A_EINVAL, "t0 and T must be >= 0");
  REQUIRE(m >= 1 && w >= 1, V4A_EINVAL, "m and w must be >= 1");
  REQUIRE(t0 + T <= INT32_MAX, V4A_EINVAL, "t0 + T must fit int32");
  return hip_status(v4a::launch_visibility(t0, T, m, k, w, E, cnt, win_lo, win_len,
                                           (hipStream_t)stream),
                    "v4a_visibility");
}

}  // extern "C"

// Validation and internal arguments of v4a_compress (shared with the decode step).
static int compress_prepare(const void* C, const void* Z, v4a_dtype in_dt, const float* B,
                            int batch, int64_t n_buf, int64_t tok_base, int64_t t0, int T, int c,
                            int m, int overlap, const float* gamma, float eps, int rope_dims,
                            float rope_base, void* out, void* out_scale, v4a_dtype out_dt,
                            int64_t E_cap, v4a::CompressArgs& a) {
  REQUIRE(C && Z && B && out, V4A_EINVAL, "null C, Z, B or out");
  REQUIRE(batch >= 1, V4A_EINVAL, "batch must be >= 1");
  REQUIRE(c >= 2 && c % 2 == 0, V4A_EINVAL, "c must be even and >= 2 (got %d)", c);
  REQUIRE(m >= 1, V4A_EINVAL, "m must be >= 1");
  REQUIRE(overlap == 0 || overlap == 1, V4A_EINVAL, "overlap must be 0 or 1");
  REQUIRE(T >= 0 && t0 >= 0 && n_buf >= 0 && tok_base >= 0, V4A_EINVAL,
          "T, t0, n_buf, tok_base must be >= 0");
  REQUIRE(rope_dims >= 0 && rope_dims % 2 == 0 && rope_dims <= c, V4A_EINVAL,
          "rope_dims must be even and in [0, c]");
  REQUIRE(rope_dims <= v4a::kMaxRopeDims, V4A_ENOTSUP, "rope_dims > %d is not supported",
          v4a::kMaxRopeDims);
  REQUIRE(rope_dims == 0 || (std::isfinite(rope_base) && rope_base > 0.0f), V4A_EINVAL,
          "rope_base must be finite and > 0");
  REQUIRE(eps >= 0.0f && std::isfinite(eps), V4A_EINVAL, "eps must be finite and >= 0");
  REQUIRE(in_dt == V4A_F32 || in_dt == V4A_BF16, V4A_ENOTSUP, "in_dt must be F32 or BF16");
  const int vec = in_dt == V4A_F32 ? 4 : 8;
  REQUIRE(c % vec == 0, V4A_ENOTSUP, "c must be a multiple of %d for this input dtype", vec);
  REQUIRE(c / vec <= 256, V4A_ENOTSUP, "c too large (max %d for this input dtype)", 256 * vec);
  REQUIRE(out_dt == V4A_F32 || out_dt == V4A_BF16 || out_dt == V4A_FP8_E4M3 ||
              out_dt == V4A_MXFP4 || out_dt == V4A_KV576,
          V4A_ENOTSUP, "unknown out_dt");
  REQUIRE(out_dt != V4A_MXFP4 || c % 32 == 0, V4A_EINVAL, "MXFP4 output needs c %% 32 == 0");
  REQUIRE(out_dt != V4A_KV576 || (rope_dims % vec == 0 && rope_dims < c), V4A_EINVAL,
          "KV576 output needs rope_dims a multiple of %d and below c", vec);
  REQUIRE((out_dt != V4A_FP8_E4M3 && out_dt != V4A_MXFP4 && out_dt != V4A_KV576) || out_scale,
          V4A_EINVAL, "out_scale is required for FP8/MXFP4/KV576 output");
  REQUIRE(aligned(C, 16) && aligned(Z, 16), V4A_EINVAL, "C and Z must be 16-byte aligned");
  const int64_t i_begin = t0 / m, i_end = (t0 + T) / m;
  REQUIRE(E_cap >= i_end, V4A_EINVAL, "E_cap (%lld) < last entry + 1 (%lld)", (long long)E_cap,
          (long long)i_end);
  if (i_end > i_begin) {
    const int64_t first = (overlap && i_begin > 0) ? (int64_t)m * (i_begin - 1) : (int64_t)m * i_begin;
    REQUIRE(tok_base <= first, V4A_EINVAL,
            "buffer starts at position %lld but entry %lld pools position %lld", (long long)tok_base,
            (long long)i_begin, (long long)first);
    REQUIRE(tok_base + n_buf >= (int64_t)m * i_end, V4A_EINVAL,
            "buffer ends at position %lld but entry %lld needs position %lld",
            (long long)(tok_base + n_buf), (long long)(i_end - 1), (long long)(m * i_end - 1));
  }
  a = v4a::CompressArgs{};
  a.C = C; a.Z = Z; a.B = B; a.gamma = gamma; a.out = out; a.out_scale = out_scale;
  a.n_buf = n_buf; a.tok_base = tok_base; a.i_begin = i_begin; a.E_cap = E_cap;
  a.n_entries = (int)(i_end - i_begin); a.batch = batch; a.c = c; a.m = m; a.overlap = overlap;
  a.rope_dims = rope_dims; a.in_dt = in_dt; a.out_dt = out_dt; a.eps = eps; a.rope_base = rope_base;
  v4a::rope_table(a.rope, rope_dims, rope_base);
  return V4A_OK;
}

extern "C" {

int v4a_compress(const void* C, const void* Z, v4a_dtype in_dt, const float* B, int batch,
                 int64_t n_buf, int64_t tok_base, int64_t t0, int T, int c, int m, int overlap,
                 const float* gamma, float eps, int rope_dims, float rope_base, void* out,
                 void* out_scale, v4a_dtype out_dt, int64_t E_cap, void* stream) {
  v4a::CompressArgs a;
  const int rc = compress_prepare(C, Z, in_dt, B, batch, n_buf, tok_base, t0, T, c, m, overlap,
                                  gamma, eps, rope_dims, rope_base, out, out_scale, out_dt, E_cap, a);
  if (rc != V4A_OK) return rc;
  return hip_status(v4a::launch_compress(a, (hipStream_t)stream), "v4a_compress");
}

static int indexer_check(const void* qI, const void* qI_scale, const void* KI,
                         const void* KI_scale, v4a_dtype dt, const float* wI, int batch, int T,
                         int64_t t0, int n_hI, int cI, int m, int k, int64_t E_cap,
                         const int32_t* idx, const int32_t* cnt) {
  REQUIRE(qI && KI && wI && idx && cnt, V4A_EINVAL, "null qI, KI, wI, topk_idx or topk_cnt");
  REQUIRE(batch >= 1 && T >= 1, V4A_EINVAL, "batch and T must be >= 1");
  REQUIRE(t0 >= 0 && t0 + T <= INT32_MAX, V4A_EINVAL, "t0 out of range");
  REQUIRE(n_hI >= 1 && cI >= 1 && m >= 1 && k >= 1, V4A_EINVAL, "n_hI, cI, m, k must be >= 1");
  REQUIRE(dt == V4A_F32 || dt == V4A_BF16 || dt == V4A_FP8_E4M3 || dt == V4A_MXFP4, V4A_ENOTSUP,
          "unknown indexer dtype");
  REQUIRE(cI <= 1024 && (int64_t)n_hI * cI <= 16384, V4A_ENOTSUP,
          "indexer query too large (cI <= 1024, n_hI*cI <= 16384)");
  REQUIRE(dt != V4A_MXFP4 || cI % 32 == 0, V4A_EINVAL, "MXFP4 needs cI %% 32 == 0");
  REQUIRE((dt != V4A_FP8_E4M3 && dt != V4A_MXFP4) || (qI_scale && KI_scale), V4A_EINVAL,
          "scales are required for FP8/MXFP4");
  REQUIRE(E_cap >= (t0 + T) / m, V4A_EINVAL, "E_cap smaller than the visible entries");
  return V4A_OK;
}

size_t v4a_indexer_topk_workspace(int batch, int T, int64_t t0, int n_hI, int cI, int m, int k,
                                  v4a_dtype dt) {
  if (batch < 1 || T < 1 || m < 1 || k < 1 || t0 < 0) return 0;
  return v4a::indexer_plan(batch, T, t0, n_hI, cI, m, k, dt, g_policy.load()).total;
}

int v4a_indexer_topk(const void* qI, const void* qI_scale, const void* KI, const void* KI_scale,
                     v4a_dtype dt, const float* wI, int batch, int T, int64_t t0, int n_hI, int cI,
                     int m, int k, int64_t E_cap, int32_t* topk_idx, int32_t* topk_cnt,
                     float* topk_score, void* ws, size_t ws_bytes, void* stream) {
  int rc = indexer_check(qI, qI_scale, KI, KI_scale, dt, wI, batch, T, t0, n_hI, cI, m, k, E_cap,
                         topk_idx, topk_cnt);
  if (rc != V4A_OK) return rc;
  const v4a::IndexerPlan p = v4a::indexer_plan(batch, T, t0, n_hI, cI, m, k, dt, g_policy.load());
  REQUIRE(ws_bytes >= p.total, V4A_ENOSPC, "workspace too small: %zu < %zu", ws_bytes, p.total);
  REQUIRE(p.total == 0 || (ws && aligned(ws, 256)), V4A_EINVAL, "workspace must be 256-byte aligned");
  v4a::IndexerArgs a{};
  a.qI = qI; a.qI_scale = qI_scale; a.KI = KI; a.KI_scale = KI_scale; a.wI = wI;
  a.topk_idx = topk_idx; a.topk_cnt = topk_cnt; a.topk_score = topk_score;
  a.t0 = t0; a.E_cap = E_cap; a.batch = batch; a.T = T; a.n_hI = n_hI; a.cI = cI; a.m = m;
  a.k = k; a.dt = dt;
  return hip_status(v4a::launch_indexer_topk(a, p, ws, (hipStream_t)stream), "v4a_indexer_topk");
}

static v4a::AttnArgs attn_args(const void* q, const void* kv_comp, const void* kv_local,
                               void* kv_ring, const void* kv_new, const int32_t* idx,
                               const int32_t* cnt, const float* sink, const float* q_gamma,
                               const float* kv_gamma, float eps, int rope_dims, float rope_base,
                               float scale, int batch, int64_t t0, int T, int n_h, int c, int k,
                               int w, int m_prime, int64_t E_cap, int64_t loc_base, int64_t n_loc,
                               void* out, v4a_dtype dt, int mode, int num_splits) {
  v4a::AttnArgs a{};
  a.q = q; a.kv_comp = kv_comp; a.kv_local = kv_local; a.kv_ring = kv_ring; a.kv_new = kv_new;
  a.idx = idx; a.cnt = cnt; a.sink = sink; a.q_gamma = q_gamma; a.kv_gamma = kv_gamma;
  a.out = out; a.loc_base = loc_base; a.n_loc = n_loc; a.t0 = t0; a.E_cap = E_cap;
  a.batch = batch; a.T = T; a.n_h = n_h; a.c = c; a.k = k; a.w = w; a.m_prime = m_prime;
  a.rope_dims = rope_dims; a.dt = dt; a.mode = mode; a.num_splits = num_splits;
  a.eps = eps; a.rope_base = rope_base; a.scale = scale > 0.0f ? scale : 1.0f / std::sqrt((float)c);
  v4a::rope_table(a.rope, rope_dims, rope_base);
  return a;
}

size_t v4a_sparse_mqa_prefill_workspace(int batch, int64_t t0, int T, int64_t loc_base,
                                        int64_t n_loc, int n_h, int c, int k, int w, v4a_dtype dt) {
  v4a::AttnArgs a = attn_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr, nullptr, nullptr, 0, 0, 0, 0, batch, t0, T, n_h, c, k, w, 0,
                              0, loc_base, n_loc, nullptr, dt, v4a::kModeCSA, 1);
  return v4a::attn_workspace(a, g_policy.load());
}

int v4a_sparse_mqa_prefill(const void* q, const void* kv_comp, const void* kv_local,
                           int64_t loc_base, int64_t n_loc, const int32_t* topk_idx,
                           const int32_t* topk_cnt, const float* sink, const float* q_gamma,
                           const float* kv_gamma, float eps, int rope_dims, float rope_base,
                           float scale, int batch, int64_t t0, int T, int n_h, int c, int k, int w,
                           int64_t E_cap, void* out, v4a_dtype dt, void* ws, size_t ws_bytes,
                           void* stream) {
  int rc = check_attn_common(q, kv_comp, out, n_h, c, rope_dims, w, dt, batch, eps);
  if (rc != V4A_OK) return rc;
  REQUIRE(kv_local && topk_idx && topk_cnt, V4A_EINVAL, "null kv_local, topk_idx or topk_cnt");
  REQUIRE(T >= 1 && t0 >= 0 && k >= 1 && E_cap >= 1, V4A_EINVAL, "T, k, E_cap must be >= 1");
  const int64_t need_lo = t0 - w + 1 > 0 ? t0 - w + 1 : 0;
  REQUIRE(loc_base >= 0 && loc_base <= need_lo && loc_base + n_loc >= t0 + T, V4A_EINVAL,
          "local rows [%lld, %lld) do not cover the windows [%lld, %lld)", (long long)loc_base,
          (long long)(loc_base + n_loc), (long long)need_lo, (long long)(t0 + T));
  v4a::AttnArgs a = attn_args(q, kv_comp, kv_local, nullptr, nullptr, topk_idx, topk_cnt, sink,
                              q_gamma, kv_gamma, eps, rope_dims, rope_base, scale, batch, t0, T,
                              n_h, c, k, w, 0, E_cap, loc_base, n_loc, out, dt, v4a::kModeCSA, 1);
  const size_t need = v4a::attn_workspace(a, g_policy.load());
  REQUIRE(ws_bytes >= need, V4A_ENOSPC, "workspace too small: %zu < %zu", ws_bytes, need);
  REQUIRE(need == 0 || (ws && aligned(ws, 256)), V4A_EINVAL, "workspace must be 256-byte aligned");
  return hip_status(v4a::launch_attention(a, ws, g_policy.load(), (hipStream_t)stream),
                    "v4a_sparse_mqa_prefill");
}

static int decode_splits(int batch, int n_h, int num_splits, int k, int w) {
  if (num_splits > 0) return num_splits;
  // about one workgroup per CU over batch x head groups x splits, but every split at least
  // two 64-candidate chunks long: the partial states (c + 2 floats per head and split)
  // are written and merged again, so splitting short lists costs more than it gains
  const int groups = batch * ((n_h + 63) / 64);
  int s = 1;
  while (groups * 2 * s <= 256 && 2 * s * 128 <= k + w) s *= 2;
  return s;
}

size_t v4a_sparse_mqa_decode_workspace(int batch, int n_h, int c, int k, int w, int num_splits,
                                       v4a_dtype dt) {
  v4a::AttnArgs a = attn_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr, nullptr, nullptr, 0, 0, 0, 0, batch, 0, 1, n_h, c, k, w, 0,
                              0, 0, 0, nullptr, dt, v4a::kModeDecode,
                              decode_splits(batch, n_h, num_splits, k, w));
  return v4a::attn_workspace(a, g_policy.load());
}

int v4a_sparse_mqa_decode(const void* q, const void* kv_comp, void* kv_ring, const void* kv_new,
                          int64_t t, const int32_t* topk_idx, const int32_t* topk_cnt,
                          const float* sink, const float* q_gamma, const float* kv_gamma,
                          float eps, int rope_dims, float rope_base, float scale, int batch,
                          int n_h, int c, int k, int w, int64_t E_cap, int num_splits, void* out,
                          v4a_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_attn_common(q, kv_comp, out, n_h, c, rope_dims, w, dt, batch, eps);
  if (rc != V4A_OK) return rc;
  REQUIRE(kv_ring && topk_idx && topk_cnt, V4A_EINVAL, "null kv_ring, topk_idx or topk_cnt");
  REQUIRE(t >= 0 && k >= 1 && E_cap >= 1, V4A_EINVAL, "t must be >= 0, k and E_cap >= 1");
  REQUIRE(num_splits >= 0 && num_splits <= 64, V4A_EINVAL, "num_splits must be in [0, 64]");
  const int ns = decode_splits(batch, n_h, num_splits, k, w);
  v4a::AttnArgs a = attn_args(q, kv_comp, kv_ring, kv_ring, kv_new, topk_idx, topk_cnt, sink,
                              q_gamma, kv_gamma, eps, rope_dims, rope_base, scale, batch, t, 1, n_h,
                              c, k, w, 0, E_cap, 0, 0, out, dt, v4a::kModeDecode, ns);
  const size_t need = v4a::attn_workspace(a, g_policy.load());
  REQUIRE(ws_bytes >= need, V4A_ENOSPC, "workspace too small: %zu < %zu", ws_bytes, need);
  REQUIRE(need == 0 || (ws && aligned(ws, 256)), V4A_EINVAL, "workspace must be 256-byte aligned");
  return hip_status(v4a::launch_attention(a, ws, g_policy.load(), (hipStream_t)stream),
                    "v4a_sparse_mqa_decode");
}

size_t v4a_hca_attn_workspace(int batch, int64_t t0, int T, int64_t loc_base, int64_t n_loc,
                              int n_h, int c, int m_prime, int w, v4a_dtype dt) {
  v4a::AttnArgs a = attn_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr, nullptr, nullptr, 0, 0, 0, 0, batch, t0, T, n_h, c, 0, w,
                              m_prime, 0, loc_base, n_loc, nullptr, dt, v4a::kModeHCA, 1);
  return v4a::attn_workspace(a, g_policy.load());
}

int v4a_hca_attn(const void* q, const void* kv_comp, const void* kv_local, int64_t loc_base,
                 int64_t n_loc, const float* sink, const float* q_gamma, const float* kv_gamma,
                 float eps, int rope_dims, float rope_base, float scale, int batch, int64_t t0,
                 int T, int n_h, int c, int m_prime, int w, int64_t E_cap, void* out, v4a_dtype dt,
                 void* ws, size_t ws_bytes, void* stream) {
  int rc = check_attn_common(q, kv_comp, out, n_h, c, rope_dims, w, dt, batch, eps);
  if (rc != V4A_OK) return rc;
  REQUIRE(kv_local, V4A_EINVAL, "null kv_local");
  REQUIRE(T >= 1 && t0 >= 0 && m_prime >= 1, V4A_EINVAL, "T, m_prime must be >= 1, t0 >= 0");
  REQUIRE(E_cap >= (t0 + T) / m_prime, V4A_EINVAL, "E_cap smaller than the visible entries");
  const int64_t need_lo = t0 - w + 1 > 0 ? t0 - w + 1 : 0;
  REQUIRE(loc_base >= 0 && loc_base <= need_lo && loc_base + n_loc >= t0 + T, V4A_EINVAL,
          "local rows do not cover the windows");
  v4a::AttnArgs a = attn_args(q, kv_comp, kv_local, nullptr, nullptr, nullptr, nullptr, sink,
                              q_gamma, kv_gamma, eps, rope_dims, rope_base, scale, batch, t0, T,
                              n_h, c, 0, w, m_prime, E_cap, loc_base, n_loc, out, dt,
                              v4a::kModeHCA, 1);
  const size_t need = v4a::attn_workspace(a, g_policy.load());
  REQUIRE(ws_bytes >= need, V4A_ENOSPC, "workspace too small: %zu < %zu", ws_bytes, need);
  REQUIRE(need == 0 || (ws && aligned(ws, 256)), V4A_EINVAL, "workspace must be 256-byte aligned");
  return hip_status(v4a::launch_attention(a, ws, g_policy.load(), (hipStream_t)stream),
                    "v4a_hca_attn");
}

// ---- decode step: the whole CSA decode of one token per sequence in one call ----

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static bool serving(const v4a_decode_step* d) { return d->t_seq || d->page_table; }

static v4a::IndexerPlan step_plan(const v4a_decode_step* d) {
  return v4a::indexer_plan(d->batch, 1, d->t, d->n_hI, d->cI, d->m, d->k, d->index_dt,
                           g_policy.load(), serving(d));
}

static v4a::AttnArgs step_attn(const v4a_decode_step* d) {
  return attn_args(d->q, d->kv_comp, d->kv_ring, d->kv_ring, d->kv_new, d->topk_idx, d->topk_cnt,
                   d->sink, d->q_gamma, d->kv_gamma, d->eps, d->rope_dims, d->rope_base, d->scale,
                   d->batch, d->t, 1, d->n_h, d->c, d->k, d->w, 0, d->E_cap, 0, 0, d->out,
                   d->attn_dt, v4a::kModeDecode,
                   decode_splits(d->batch, d->n_h, d->num_splits, d->k, d->w));
}

// pool rows of the selected entries (paged bf16 steps), or the bf16 staging of the
// selected production-format rows (kv576 steps), after the indexer workspace
static size_t step_phys_bytes(const v4a_decode_step* d) {
  if (d->kv576) return align256((size_t)d->batch * d->k * (size_t)d->c * 2);
  return d->page_table ? align256((size_t)d->batch * d->k * sizeof(int32_t)) : 0;
}

// attention of a kv576 step: dense over the staged rows (cnt[b] of them), then the window
static v4a::AttnArgs step_attn_staged(const v4a_decode_step* d, void* staged) {
  v4a::AttnArgs a = attn_args(d->q, staged, d->kv_ring, d->kv_ring, d->kv_new, nullptr, d->topk_cnt,
                              d->sink, d->q_gamma, d->kv_gamma, d->eps, d->rope_dims, d->rope_base,
                              d->scale, d->batch, d->t, 1, d->n_h, d->c, d->k, d->w, 1, d->k, 0, 0,
                              d->out, d->attn_dt, v4a::kModeHCADecode,
                              decode_splits(d->batch, d->n_h, d->num_splits, d->k, d->w));
  a.dense_cnt = d->topk_cnt;
  return a;
}

static int log2_exact(int64_t x) {
  int s = 0;
  while (((int64_t)1 << s) < x) ++s;
  return ((int64_t)1 << s) == x ? s : -1;
}

// Validation of the serving fields shared by the CSA and HCA decode steps.
static int check_serving(const int64_t* t_seq, const int32_t* page_table, int64_t max_pages,
                         int64_t pool_rows, int page_entries, int64_t E_cap, bool mfma,
                         v4a::SeqState& st) {
  st = v4a::SeqState{};
  if (!t_seq && !page_table) return V4A_OK;
  REQUIRE(mfma, V4A_ENOTSUP,
          "per-sequence positions and paged caches need bf16 rows of 512 channels, heads in "
          "groups of 64 and RoPE 0 or 64");
  st.tpos = t_seq;
  if (page_table) {
    const int sh = log2_exact(page_entries);
    REQUIRE(page_entries >= 1 && sh >= 0, V4A_EINVAL, "page_entries must be a power of two");
    REQUIRE(max_pages >= 1 && E_cap == max_pages * page_entries, V4A_EINVAL,
            "E_cap must equal max_pages * page_entries");
    REQUIRE(pool_rows >= page_entries && pool_rows <= INT32_MAX && pool_rows % page_entries == 0,
            V4A_EINVAL, "pool_rows must be a positive multiple of page_entries below 2^31");
    st.pages = page_table;
    st.max_pages = max_pages;
    st.page_shift = sh;
  }
  return V4A_OK;
}

int v4a_decode_step_layout(size_t* off, int n, size_t* size) {
#define V4A_OFF(f) offsetof(v4a_decode_step, f)
  const size_t o[] = {
      V4A_OFF(t), V4A_OFF(E_cap), V4A_OFF(n_buf), V4A_OFF(tok_base), V4A_OFF(batch), V4A_OFF(n_h),
      V4A_OFF(c), V4A_OFF(n_hI), V4A_OFF(cI), V4A_OFF(m), V4A_OFF(k), V4A_OFF(w),
      V4A_OFF(num_splits), V4A_OFF(rope_dims), V4A_OFF(rope_dims_I), V4A_OFF(rope_base),
      V4A_OFF(eps), V4A_OFF(scale), V4A_OFF(tail_dt), V4A_OFF(index_dt), V4A_OFF(attn_dt),
      V4A_OFF(C), V4A_OFF(Z), V4A_OFF(B), V4A_OFF(gamma), V4A_OFF(CI), V4A_OFF(ZI), V4A_OFF(BI),
      V4A_OFF(gammaI), V4A_OFF(kv_comp), V4A_OFF(KI), V4A_OFF(KI_scale), V4A_OFF(qI),
      V4A_OFF(qI_scale), V4A_OFF(wI), V4A_OFF(q), V4A_OFF(sink), V4A_OFF(q_gamma),
      V4A_OFF(kv_gamma), V4A_OFF(kv_ring), V4A_OFF(kv_new), V4A_OFF(topk_idx), V4A_OFF(topk_cnt),
      V4A_OFF(topk_score), V4A_OFF(out), V4A_OFF(t_seq), V4A_OFF(page_table), V4A_OFF(max_pages),
      V4A_OFF(pool_rows), V4A_OFF(page_entries), V4A_OFF(kv576), V4A_OFF(kv_scale)};
#undef V4A_OFF
  const int nf = (int)(sizeof(o) / sizeof(o[0]));
  for (int i = 0; i < nf && i < n && off; ++i) off[i] = o[i];
  if (size) *size = sizeof(v4a_decode_step);
  return nf;
}

size_t v4a_csa_decode_step_workspace(const v4a_decode_step* d) {
  if (!d || d->batch < 1 || d->m < 1 || d->k < 1 || d->t < 0 || d->n_h < 1 || d->c < 2 ||
      d->num_splits < 0 || d->num_splits > 64)
    return 0;
  return align256(step_plan(d).total) + step_phys_bytes(d) +
         v4a::attn_workspace(d->kv576 ? step_attn_staged(d, nullptr) : step_attn(d), g_policy.load());
}

int v4a_csa_decode_step(const v4a_decode_step* d, void* ws, size_t ws_bytes, void* stream) {
  return v4a::decode_step_run(d, ws, ws_bytes, stream);
}

}  // extern "C"

// The decode step with a given workspace (the caller's, or the fixed device scratch of
// v4a_csa_decode_step_noalloc).
int v4a::decode_step_run(const v4a_decode_step* d, void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(d, V4A_EINVAL, "null step description");
  REQUIRE(d->t >= 0 && d->t < INT32_MAX, V4A_EINVAL, "t out of range");
  REQUIRE(d->num_splits >= 0 && d->num_splits <= 64, V4A_EINVAL, "num_splits must be in [0, 64]");
  REQUIRE(d->attn_dt == V4A_F32 || d->attn_dt == V4A_BF16, V4A_ENOTSUP,
          "attention dtype must be F32 or BF16");
  const bool ragged = d->t_seq != nullptr;
  // the stages' own checks, as the separate calls make them (per-sequence tails: the
  // fixed two-block buffer of every sequence, checked against the bound t)
  REQUIRE(!ragged || d->n_buf == 2 * (int64_t)d->m, V4A_EINVAL,
          "with t_seq the tail buffers hold 2m rows per sequence (n_buf = %d)", 2 * d->m);
  const int64_t tb = ragged ? (int64_t)d->m * (d->t / d->m) - d->m : d->tok_base;
  const bool kv576 = d->kv576 != 0;
  REQUIRE(!kv576 || d->kv_scale, V4A_EINVAL, "kv576 needs kv_scale");
  v4a::CompressArgs cm, ci;
  int rc = compress_prepare(d->C, d->Z, d->tail_dt, d->B, d->batch, d->n_buf,
                            ragged ? (tb > 0 ? tb : 0) : d->tok_base, ragged ? 0 : d->t,
                            ragged ? 0 : 1, d->c, d->m, 1, d->gamma, d->eps, d->rope_dims,
                            d->rope_base, d->kv_comp, kv576 ? d->kv_scale : nullptr,
                            kv576 ? V4A_KV576 : d->attn_dt, d->E_cap, cm);
  if (rc != V4A_OK) return rc;
  rc = compress_prepare(d->CI, d->ZI, d->tail_dt, d->BI, d->batch, d->n_buf,
                        ragged ? (tb > 0 ? tb : 0) : d->tok_base, ragged ? 0 : d->t, ragged ? 0 : 1,
                        d->cI, d->m, 1, d->gammaI, d->eps, d->rope_dims_I, d->rope_base, d->KI,
                        d->KI_scale, d->index_dt, d->E_cap, ci);
  if (rc != V4A_OK) return rc;
  rc = indexer_check(d->qI, d->qI_scale, d->KI, d->KI_scale, d->index_dt, d->wI, d->batch, 1, d->t,
                     d->n_hI, d->cI, d->m, d->k, d->E_cap, d->topk_idx, d->topk_cnt);
  if (rc != V4A_OK) return rc;
  rc = check_attn_common(d->q, d->kv_comp, d->out, d->n_h, d->c, d->rope_dims, d->w, d->attn_dt,
                         d->batch, d->eps);
  if (rc != V4A_OK) return rc;
  REQUIRE(d->kv_ring, V4A_EINVAL, "null kv_ring");
  const v4a::IndexerPlan p = step_plan(d);
  v4a::AttnArgs aa = step_attn(d);
  const int policy = g_policy.load();
  v4a::SeqState st;
  rc = check_serving(d->t_seq, d->page_table, d->max_pages, d->pool_rows, d->page_entries, d->E_cap,
                     policy == 0 && v4a::attn_mfma_supported(aa), st);
  if (rc != V4A_OK) return rc;
  REQUIRE(!kv576 || (policy == 0 && v4a::attn_mfma_supported(aa) && d->c == 512), V4A_ENOTSUP,
          "kv576 caches need bf16 rows of 512 channels, heads in groups of 64, RoPE 0 or 64");
  const size_t ws_i = align256(p.total), ws_p = step_phys_bytes(d);
  if (kv576) {
    aa = step_attn_staged(d, reinterpret_cast<char*>(ws) + ws_i);
    aa.seq = v4a::SeqState{};
    aa.seq.tpos = st.tpos;  // the staged list is contiguous; positions stay per sequence
  }
  const size_t need = ws_i + ws_p + v4a::attn_workspace(aa, policy);
  REQUIRE(ws_bytes >= need, V4A_ENOSPC, "workspace too small: %zu < %zu", ws_bytes, need);
  REQUIRE(ws && aligned(ws, 256), V4A_EINVAL, "workspace must be 256-byte aligned");
  int32_t* phys = (d->page_table && !kv576) ? reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + ws_i)
                                             : nullptr;
  if (ragged) {
    // one entry slot per sequence: emitted or not by the sequence's own position
    cm.seq = st;
    ci.seq = st;
    cm.n_entries = ci.n_entries = 1;
  } else if (d->page_table) {
    cm.seq = st;
    ci.seq = st;
  }
  v4a::IndexerArgs ia{};
  ia.qI = d->qI; ia.qI_scale = d->qI_scale; ia.KI = d->KI; ia.KI_scale = d->KI_scale; ia.wI = d->wI;
  ia.topk_idx = d->topk_idx; ia.topk_cnt = d->topk_cnt; ia.topk_score = d->topk_score;
  ia.t0 = d->t; ia.E_cap = d->E_cap; ia.batch = d->batch; ia.T = 1; ia.n_hI = d->n_hI;
  ia.cI = d->cI; ia.m = d->m; ia.k = d->k; ia.dt = d->index_dt;
  ia.seq = st;
  ia.phys = phys;
  if (!kv576) aa.seq = st;
  if (phys) aa.idx = phys;  // the attention gathers pool rows
  hipStream_t s = (hipStream_t)stream;
  void* ws_a = reinterpret_cast<char*>(ws) + ws_i + ws_p;
  hipError_t e = hipSuccess;
  const bool front = v4a::decode_front_supported(cm, ci, aa, policy);
  if (front && p.filter && v4a::indexer_fuses_compress(p, ci)) {
    // the scan compresses the index entry itself; the main entry, the window prep and the
    // ring insert ride in the top-k final launch (a few workgroups, latency-bound), so no
    // launch of their own precedes the scan
    v4a::FrontArgs fa;
    e = v4a::decode_front_args(cm, aa, ws_a, fa);
    if (e == hipSuccess) e = v4a::launch_indexer_topk(ia, p, ws, s, &ci, &fa);
    aa.prep_done = 1;
  } else {
    if (front) {
      // tail compressions, window prep and ring insert in one launch
      e = v4a::launch_decode_front(cm, ci, aa, ws_a, s);
      aa.prep_done = 1;
    } else {
      e = v4a::launch_compress(cm, s);
      if (e == hipSuccess) e = v4a::launch_compress(ci, s);
    }
    if (e == hipSuccess) e = v4a::launch_indexer_topk(ia, p, ws, s);
  }
  if (e == hipSuccess && kv576)
    e = v4a::launch_kv576_gather(d->kv_comp, d->kv_scale, d->topk_idx, d->topk_cnt, st, d->E_cap,
                                 d->batch, d->k, d->rope_dims, reinterpret_cast<char*>(ws) + ws_i, s);
  if (e == hipSuccess) e = v4a::launch_attention(aa, ws_a, policy, s);
  return hip_status(e, "v4a_csa_decode_step");
}

// ---- HCA decode step ---------------------------------------------------------------

static v4a::AttnArgs hca_step_attn(const v4a_hca_step* d) {
  // candidate list of the latest position: every completed entry plus the window
  const int64_t N = (d->t + 1) / (d->m_prime > 0 ? d->m_prime : 1) + d->w;
  return attn_args(d->q, d->kv_comp, d->kv_ring, d->kv_ring, d->kv_new, nullptr, nullptr, d->sink,
                   d->q_gamma, d->kv_gamma, d->eps, d->rope_dims, d->rope_base, d->scale, d->batch,
                   d->t, 1, d->n_h, d->c, 0, d->w, d->m_prime, d->E_cap, 0, 0, d->out, d->attn_dt,
                   v4a::kModeHCADecode,
                   decode_splits(d->batch, d->n_h, d->num_splits, (int)(N - d->w), d->w));
}

extern "C" {

int v4a_hca_decode_step_layout(size_t* off, int n, size_t* size) {
#define V4A_OFF(f) offsetof(v4a_hca_step, f)
  const size_t o[] = {
      V4A_OFF(t), V4A_OFF(E_cap), V4A_OFF(n_buf), V4A_OFF(tok_base), V4A_OFF(batch), V4A_OFF(n_h),
      V4A_OFF(c), V4A_OFF(m_prime), V4A_OFF(w), V4A_OFF(num_splits), V4A_OFF(rope_dims),
      V4A_OFF(rope_base), V4A_OFF(eps), V4A_OFF(scale), V4A_OFF(tail_dt), V4A_OFF(attn_dt),
      V4A_OFF(C), V4A_OFF(Z), V4A_OFF(B), V4A_OFF(gamma), V4A_OFF(kv_comp), V4A_OFF(q),
      V4A_OFF(sink), V4A_OFF(q_gamma), V4A_OFF(kv_gamma), V4A_OFF(kv_ring), V4A_OFF(kv_new),
      V4A_OFF(out), V4A_OFF(t_seq), V4A_OFF(page_table), V4A_OFF(max_pages), V4A_OFF(pool_rows),
      V4A_OFF(page_entries)};
#undef V4A_OFF
  const int nf = (int)(sizeof(o) / sizeof(o[0]));
  for (int i = 0; i < nf && i < n && off; ++i) off[i] = o[i];
  if (size) *size = sizeof(v4a_hca_step);
  return nf;
}

size_t v4a_hca_decode_step_workspace(const v4a_hca_step* d) {
  if (!d || d->batch < 1 || d->m_prime < 1 || d->t < 0 || d->n_h < 1 || d->c < 2 || d->w < 1 ||
      d->num_splits < 0 || d->num_splits > 64)
    return 0;
  return v4a::attn_workspace(hca_step_attn(d), g_policy.load());
}

int v4a_hca_decode_step(const v4a_hca_step* d, void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(d, V4A_EINVAL, "null step description");
  REQUIRE(d->t >= 0 && d->t < INT32_MAX, V4A_EINVAL, "t out of range");
  REQUIRE(d->m_prime >= 1, V4A_EINVAL, "m_prime must be >= 1");
  REQUIRE(d->num_splits >= 0 && d->num_splits <= 64, V4A_EINVAL, "num_splits must be in [0, 64]");
  int rc = check_attn_common(d->q, d->kv_comp, d->out, d->n_h, d->c, d->rope_dims, d->w, d->attn_dt,
                             d->batch, d->eps);
  if (rc != V4A_OK) return rc;
  REQUIRE(d->kv_ring, V4A_EINVAL, "null kv_ring");
  const bool ragged = d->t_seq != nullptr;
  REQUIRE(!ragged || d->n_buf == d->m_prime, V4A_EINVAL,
          "with t_seq the tail buffers hold m' rows per sequence (n_buf = %d)", d->m_prime);
  REQUIRE(d->E_cap >= (d->t + 1) / d->m_prime && d->E_cap >= 1, V4A_EINVAL,
          "E_cap smaller than the visible entries");
  v4a::AttnArgs aa = hca_step_attn(d);
  const int policy = g_policy.load();
  REQUIRE(policy == 0 && v4a::attn_mfma_supported(aa), V4A_ENOTSUP,
          "HCA decode needs bf16 rows of 512 channels, heads in groups of 64 and RoPE 0 or 64");
  v4a::SeqState st;
  rc = check_serving(d->t_seq, d->page_table, d->max_pages, d->pool_rows, d->page_entries, d->E_cap,
                     true, st);
  if (rc != V4A_OK) return rc;
  const int64_t tb = ragged ? (int64_t)d->m_prime * (d->t / d->m_prime) : d->tok_base;
  v4a::CompressArgs cm;
  rc = compress_prepare(d->C, d->Z, d->tail_dt, d->B, d->batch, d->n_buf, ragged ? tb : d->tok_base,
                        ragged ? 0 : d->t, ragged ? 0 : 1, d->c, d->m_prime, 0, d->gamma, d->eps,
                        d->rope_dims, d->rope_base, d->kv_comp, nullptr, d->attn_dt, d->E_cap, cm);
  if (rc != V4A_OK) return rc;
  const size_t need = v4a::attn_workspace(aa, policy);
  REQUIRE(ws_bytes >= need, V4A_ENOSPC, "workspace too small: %zu < %zu", ws_bytes, need);
  REQUIRE(ws && aligned(ws, 256), V4A_EINVAL, "workspace must be 256-byte aligned");
  cm.seq = st;
  if (ragged) cm.n_entries = 1;
  aa.seq = st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = v4a::launch_compress(cm, s);  // the entry a completed block emits
  if (e == hipSuccess) e = v4a::launch_attention(aa, ws, policy, s);
  return hip_status(e, "v4a_hca_decode_step");
}

}  // extern "C"
