/*
 * v4a.h -- C ABI of libv4a.so: the MI355X (gfx950) hot path of DeepSeek-V4
 * compressed sparse attention (CSA) and heavily compressed attention (HCA).
 *
 * Operations are defined on the page "CSA And HCA: Definition, State, And
 * Cost Model" (cited as [Def] with its section numbers).
 *
 * Conventions for every entry point
 *   - Pointers named as device buffers must point to GPU memory (hipMalloc or
 *     torch CUDA tensors); all are row-major and densely packed as stated.
 *   - The caller allocates and owns every buffer, including workspaces.  The
 *     library never allocates device memory, never frees, and keeps no pointer
 *     after a call returns (the one exception is the fixed scratch array of
 *     v4a_csa_decode_step_noalloc, part of the loaded library itself).  Buffers must stay alive until the work queued on
 *     `stream` completes.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *     Calls are asynchronous: they validate arguments on the host, enqueue
 *     kernels and return.
 *   - Return value: V4A_OK (0) or a negative V4A_E* code.  On error nothing has
 *     been enqueued (validation errors) or the launch failed (V4A_EIO); the
 *     message is available from v4a_last_error() on the calling thread.  No
 *     call prints, aborts or throws across the ABI.
 *   - Results are bitwise reproducible run to run for identical inputs (no
 *     floating-point atomics; fixed split and merge order).
 *   - Token positions are absolute and zero-based; compressed entry i covers
 *     tokens [r*i, r*(i+1)) for ratio r.  Query t sees entries
 *     s < floor((t+1)/r) ([Def] section 1) and the window
 *     j in [max(0, t-w+1), t] ([Def] section 5.1).
 *   - Batches: the prefill and separate decode calls take one position (t0, T, t) for
 *     every sequence of the call; the decode steps (v4a_csa_decode_step,
 *     v4a_hca_decode_step) also take per-sequence positions and paged caches.
 */
#ifndef V4A_H
#define V4A_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define V4A_API __attribute__((visibility("default")))
#else
#define V4A_API
#endif

#define V4A_OK 0
#define V4A_EINVAL (-22)  /* invalid argument (shape, range, null pointer, alignment) */
#define V4A_ENOTSUP (-95) /* valid but unsupported combination (dtype, size) */
#define V4A_ENOSPC (-28)  /* workspace too small */
#define V4A_EIO (-5)      /* a HIP launch or runtime call failed */

/* Element formats.
 *   V4A_F32      : IEEE float32.
 *   V4A_BF16     : bfloat16.
 *   V4A_FP8_E4M3 : OCP FP8 E4M3 (bias 7, no infinities, max 448) codes, one byte
 *                  per element, with one float32 scale per row (value = code * scale).
 *   V4A_MXFP4    : OCP MX v1.0 MXFP4: E2M1 codes packed two per byte (element 2j
 *                  in the low nibble of byte j) with one E8M0 scale byte per 32
 *                  consecutive elements of a row (value = code * 2^(scale-127)).
 *   V4A_KV576    : the production main-cache row of [Def] section 8: the c - rope_dims
 *                  leading channels as E4M3 codes (one float32 scale per row, scale =
 *                  max|x| / 448 over those channels, codes round to nearest even and
 *                  saturate), then the rope_dims rotated channels as bf16; c + rope_dims
 *                  bytes per row (576 at c = 512, rope_dims = 64).  Compressor output
 *                  and decode-step cache format only.
 */
/* V4A_DTYPE_RANGE_ only widens the enumeration to every 32-bit value, so that a caller's
 * out-of-range code reaches the library's validation (V4A_ENOTSUP) as a valid value of the
 * type; it is not a data type. */
typedef enum {
  V4A_F32 = 0, V4A_BF16 = 1, V4A_FP8_E4M3 = 2, V4A_MXFP4 = 3, V4A_KV576 = 4,
  V4A_DTYPE_RANGE_ = 0x7fffffff
} v4a_dtype;

/* Thread-local message of the last failed call on this thread ("" if none). */
V4A_API const char* v4a_last_error(void);

/* Library version string. */
V4A_API const char* v4a_version(void);

/* Kernel policy: 0 = automatic (MFMA kernels where the shape allows, the
 * general kernels otherwise), 1 = general kernels only.  Process-wide; for
 * testing and diagnosis.  Returns the previous policy. */
V4A_API int v4a_set_kernel_policy(int policy);

/*
 * v4a_visibility -- per-query sets for queries t = t0 .. t0+T-1
 * ([Def] section 1 completed entries, section 5.1 window; section 6 table).
 *   E[j]       = floor((t+1)/m)               visible completed entries
 *   cnt[j]     = min(k, E[j]) (k <= 0: E[j])  compressed candidates attended
 *   win_lo[j]  = max(0, t-w+1), win_len[j] = min(w, t+1)
 * Outputs: device int32 arrays of T elements each (any may be NULL).
 * Errors: V4A_EINVAL if t0 < 0, T < 0, m < 1, w < 1 or t0+T > 2^31-1.
 */
V4A_API int v4a_visibility(int64_t t0, int T, int m, int k, int w, int32_t* E, int32_t* cnt,
                   int32_t* win_lo, int32_t* win_len, void* stream);

/*
 * v4a_compress -- the learned feature-wise gated compressor
 * ([Def] section 2.1 for CSA with overlap = 1, section 2.2 for HCA with
 * overlap = 0; RMSNorm and partial RoPE of the emitted entry per section 5.2).
 *
 * For every sequence b < batch and entry i in [floor(t0/m), floor((t0+T)/m)):
 *   per channel ch, one softmax over positions of the logits
 *     Z^a[p][ch] + B^a[p - m*i][ch]           for p in [m*i, m*(i+1))      (stream a)
 *     Z^b[p][ch] + B^b[p - m*(i-1)][ch]       for p in [m*(i-1), m*i)      (stream b,
 *                                              only when overlap = 1 and i > 0)
 *   weights the matching C rows; the entry is their weighted sum (float32 math).
 *   If gamma != NULL: x <- x / sqrt(mean(x^2) + eps) * gamma.
 *   If rope_dims > 0: channels [c-rope_dims, c) are rotated in adjacent pairs
 *     (2i, 2i+1) by angle (m*i) * rope_base^(-2i/rope_dims).
 * Only completed blocks are emitted: with T tokens arriving at t0 the call emits
 * exactly the entries whose last token lies in [t0, t0+T); an incomplete final
 * block emits nothing and is never padded.
 *
 *   C, Z      : device [batch][n_buf][width] of in_dt (V4A_F32 or V4A_BF16),
 *               width = 2c when overlap = 1 (stream a in columns [0,c), stream b
 *               in [c,2c)), width = c when overlap = 0.  Row r of a sequence holds
 *               absolute token position tok_base + r.  Must contain every row the
 *               emitted entries pool.
 *   B         : device float32 [(1+overlap)*m][c]: rows 0..m-1 = B^a (or B),
 *               rows m..2m-1 = B^b.
 *   gamma     : device float32 [c] or NULL (no RMSNorm).
 *   out       : device [batch][E_cap][...]: entry i is written to row i.
 *               V4A_F32 / V4A_BF16: rows of c elements.
 *               V4A_FP8_E4M3: rows of c codes; out_scale = float32 [batch][E_cap]
 *                 (scale = max|x|/448, codes round to nearest even, saturating).
 *               V4A_MXFP4: rows of c/2 bytes; out_scale = uint8 E8M0
 *                 [batch][E_cap][c/32] (shared exponent floor(log2 max|x|) - 2,
 *                 codes round to nearest even, saturate at 6).
 * Errors: V4A_EINVAL for null pointers, c < 2 or odd, c % 32 != 0 with MXFP4
 *   output, m < 1, overlap not 0/1, rope_dims odd or > c, T < 0, tok_base or
 *   n_buf not covering the pooled rows, E_cap < floor((t0+T)/m);
 *   V4A_ENOTSUP for other dtype combinations or c > 2048.
 */
V4A_API int v4a_compress(const void* C, const void* Z, v4a_dtype in_dt, const float* B, int batch,
                 int64_t n_buf, int64_t tok_base, int64_t t0, int T, int c, int m, int overlap,
                 const float* gamma, float eps, int rope_dims, float rope_base, void* out,
                 void* out_scale, v4a_dtype out_dt, int64_t E_cap, void* stream);

/*
 * v4a_indexer_topk -- CSA lightning indexer and top-k ([Def] section 3.1).
 *
 * For each sequence b and query t = t0 + j (j < T), over the visible entries
 * s < E_t = floor((t+1)/m):
 *   I[t][s] = sum_h wI[t][h] * max(0, qI[t][h] . KI[s])     (no scale term)
 * and selects the min(k, E_t) entries with the largest I; ties go to the lower
 * entry index.  Scores are computed in float32 from the stored operands.
 *
 *   qI       : device [batch][T][n_hI][cI] of dt.
 *   qI_scale : dt = V4A_FP8_E4M3: float32 [batch][T][n_hI] (one per head row);
 *              dt = V4A_MXFP4: uint8 E8M0 [batch][T][n_hI][cI/32]; else NULL.
 *   KI       : device [batch][E_cap][cI] of dt (MXFP4: [batch][E_cap][cI/2]).
 *   KI_scale : FP8: float32 [batch][E_cap]; MXFP4: uint8 [batch][E_cap][cI/32].
 *   wI       : device float32 [batch][T][n_hI].
 *   topk_idx : device int32 [batch][T][k]: selected entries in ascending order,
 *              then -1 padding.
 *   topk_cnt : device int32 [batch][T]: min(k, E_t).
 *   topk_score: device float32 [batch][T][k] or NULL: I of the selected entries,
 *              aligned with topk_idx (0 in padding slots).
 *   ws       : device workspace of at least v4a_indexer_topk_workspace(...) bytes
 *              (256-byte aligned).
 * Errors: V4A_EINVAL for null pointers, T < 1, n_hI < 1, cI < 1, cI % 32 with
 *   MXFP4, m < 1, k < 1, E_cap < floor((t0+T)/m); V4A_ENOSPC if ws_bytes is too
 *   small; V4A_ENOTSUP for dt outside F32/BF16/FP8_E4M3/MXFP4 or cI > 1024.
 */
V4A_API size_t v4a_indexer_topk_workspace(int batch, int T, int64_t t0, int n_hI, int cI, int m, int k,
                                  v4a_dtype dt);
V4A_API int v4a_indexer_topk(const void* qI, const void* qI_scale, const void* KI, const void* KI_scale,
                     v4a_dtype dt, const float* wI, int batch, int T, int64_t t0, int n_hI, int cI,
                     int m, int k, int64_t E_cap, int32_t* topk_idx, int32_t* topk_cnt,
                     float* topk_score, void* ws, size_t ws_bytes, void* stream);

/*
 * Shared-KV MQA core attention, common to the three attention calls
 * ([Def] sections 3.2, 4 and 5.1-5.3).  For query t and head h:
 *   q'  = RoPE_t(RMSNorm_{q_gamma}(q[t][h]))         (norm skipped if q_gamma NULL)
 *   candidates, one list:  compressed entries as stored (already normalised and
 *     rotated by v4a_compress)  ||  local rows j of the window, each
 *     RoPE_j(RMSNorm_{kv_gamma}(local[j]))            (norm skipped if kv_gamma NULL)
 *   z_u = scale * q' . v_u;   a_u = exp(z_u) / (sum_v exp(z_v) + exp(sink[h]))
 *     (the sink term only when sink != NULL)
 *   out[t][h] = RoPE_{-t}( sum_u a_u v_u )           (inverse RoPE at t)
 * Each candidate row is both key and value for all n_h heads.  RoPE rotates
 * channels [c-rope_dims, c) in adjacent pairs with angle pos*rope_base^(-2i/rope_dims).
 * scale = 0 selects 1/sqrt(c).  float32 softmax and accumulation; bf16 inputs
 * enter the matrix cores as bf16.
 */

/*
 * v4a_sparse_mqa_prefill -- CSA attention for a chunk of queries [t0, t0+T).
 *   q        : device [batch][T][n_h][c] of dt (V4A_F32 or V4A_BF16).
 *   kv_comp  : device [batch][E_cap][c] of dt, compressed entries as stored.
 *   kv_local : device [batch][n_loc][c] of dt, raw local rows; row r holds
 *              position loc_base + r and must cover [max(0,t0-w+1), t0+T).
 *   topk_idx, topk_cnt : device int32 [batch][T][k], [batch][T] as produced by
 *              v4a_indexer_topk (entries >= 0 and < E_cap; order irrelevant).
 *   sink     : device float32 [n_h] or NULL.
 *   q_gamma, kv_gamma : device float32 [c] or NULL.
 *   out      : device [batch][T][n_h][c] of dt.
 *   ws       : device workspace of v4a_sparse_mqa_prefill_workspace(...) bytes.
 * Errors: V4A_EINVAL for null pointers, bad sizes, local rows not covering the
 *   windows; V4A_ENOSPC; V4A_ENOTSUP for c > 1024 or dt outside F32/BF16.
 */
V4A_API size_t v4a_sparse_mqa_prefill_workspace(int batch, int64_t t0, int T, int64_t loc_base,
                                        int64_t n_loc, int n_h, int c, int k, int w, v4a_dtype dt);
V4A_API int v4a_sparse_mqa_prefill(const void* q, const void* kv_comp, const void* kv_local,
                           int64_t loc_base, int64_t n_loc, const int32_t* topk_idx,
                           const int32_t* topk_cnt, const float* sink, const float* q_gamma,
                           const float* kv_gamma, float eps, int rope_dims, float rope_base,
                           float scale, int batch, int64_t t0, int T, int n_h, int c, int k, int w,
                           int64_t E_cap, void* out, v4a_dtype dt, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * v4a_sparse_mqa_decode -- CSA attention for one new token per sequence at
 * position t, with the window read from a w-slot ring ([Def] section 7, steps 1
 * and 5).
 *   q        : device [batch][n_h][c] of dt.
 *   kv_comp  : device [batch][E_cap][c] of dt.
 *   kv_ring  : device [batch][w][c] of dt; token j lives in slot j % w.
 *   kv_new   : device [batch][c] of dt or NULL.  When given, it is token t's raw
 *              local row: the call writes it into slot t % w (step 1) and
 *              attends over it.  When NULL the ring must already hold token t.
 *   topk_idx, topk_cnt : device int32 [batch][k], [batch].
 *   num_splits: 0 = automatic; otherwise the candidate list of each sequence is
 *              split into this many parts whose partial softmax states are merged
 *              (result identical up to float32 rounding).
 *   out      : device [batch][n_h][c] of dt.
 *   ws       : device workspace of v4a_sparse_mqa_decode_workspace(...) bytes.
 * Errors: as for prefill.
 */
V4A_API size_t v4a_sparse_mqa_decode_workspace(int batch, int n_h, int c, int k, int w, int num_splits,
                                       v4a_dtype dt);
V4A_API int v4a_sparse_mqa_decode(const void* q, const void* kv_comp, void* kv_ring, const void* kv_new,
                          int64_t t, const int32_t* topk_idx, const int32_t* topk_cnt,
                          const float* sink, const float* q_gamma, const float* kv_gamma,
                          float eps, int rope_dims, float rope_base, float scale, int batch,
                          int n_h, int c, int k, int w, int64_t E_cap, int num_splits, void* out,
                          v4a_dtype dt, void* ws, size_t ws_bytes, void* stream);

/*
 * v4a_hca_attn -- HCA attention for queries [t0, t0+T): the compressed part is
 * every completed entry s < floor((t+1)/m_prime), read densely ([Def] section 4).
 *   q, kv_local, out : as for v4a_sparse_mqa_prefill.
 *   kv_comp  : device [batch][E_cap][c], E_cap >= floor((t0+T)/m_prime).
 * Errors: as for prefill.
 */
V4A_API size_t v4a_hca_attn_workspace(int batch, int64_t t0, int T, int64_t loc_base, int64_t n_loc,
                              int n_h, int c, int m_prime, int w, v4a_dtype dt);
V4A_API int v4a_hca_attn(const void* q, const void* kv_comp, const void* kv_local, int64_t loc_base,
                 int64_t n_loc, const float* sink, const float* q_gamma, const float* kv_gamma,
                 float eps, int rope_dims, float rope_base, float scale, int batch, int64_t t0,
                 int T, int n_h, int c, int m_prime, int w, int64_t E_cap, void* out, v4a_dtype dt,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * v4a_csa_decode_step -- one CSA decode step for every sequence of the batch
 * (new token at position t), as one call: [Def] section 7, steps 1, 4 and 5.
 * The result is that of the sequence
 *   v4a_compress(C, Z, tail_dt, B, batch, n_buf, tok_base, t, 1, c, m, 1, gamma,
 *                eps, rope_dims, rope_base, kv_comp, NULL, attn_dt, E_cap)
 *   v4a_compress(CI, ZI, tail_dt, BI, batch, n_buf, tok_base, t, 1, cI, m, 1,
 *                gammaI, eps, rope_dims_I, rope_base, KI, KI_scale, index_dt, E_cap)
 *   v4a_indexer_topk(qI, qI_scale, KI, KI_scale, index_dt, wI, batch, 1, t, n_hI,
 *                    cI, m, k, E_cap, topk_idx, topk_cnt, topk_score)
 *   v4a_sparse_mqa_decode(q, kv_comp, kv_ring, kv_new, t, topk_idx, topk_cnt, sink,
 *                         q_gamma, kv_gamma, eps, rope_dims, rope_base, scale,
 *                         batch, n_h, c, k, w, E_cap, num_splits, out, attn_dt)
 * (bit for bit), with the same arguments, layouts and errors; workspaces are
 * replaced by one.  Where the shapes allow (bf16 tails and attention rows of 512
 * channels, heads in groups of 64), the step needs fewer launches: the two tail
 * compressions and the window-row preparation run as one launch ahead of the index
 * scan, or, when the top-k takes its threshold filter (one query over E >= 32 k
 * entries), the index scan emits the new index entry itself and the main entry,
 * window rows and ring insert run inside the final top-k launch.  When
 * (t+1) % m != 0 no entry is emitted and the compressor inputs are not read.
 *   d        : host pointer to the description below (read during the call only).
 *   ws       : device workspace of v4a_csa_decode_step_workspace(d) bytes,
 *              256-byte aligned.
 */
typedef struct v4a_decode_step {
  int64_t t;                 /* position of the new token (all sequences), 0 <= t < 2^31 - 1 */
  int64_t E_cap;             /* rows of kv_comp and KI per sequence */
  int64_t n_buf, tok_base;   /* tail buffers: n_buf rows, row r = position tok_base + r */
  int batch, n_h, c, n_hI, cI, m, k, w;
  int num_splits;            /* 0 = automatic */
  int rope_dims, rope_dims_I;
  float rope_base, eps, scale;
  v4a_dtype tail_dt;         /* C, Z, CI, ZI: F32 or BF16 */
  v4a_dtype index_dt;        /* qI, KI */
  v4a_dtype attn_dt;         /* q, kv_comp, kv_ring, kv_new, out: F32 or BF16 */
  const void* C;             /* main compressor: [batch][n_buf][2c] */
  const void* Z;
  const float* B;            /* [2m][c] */
  const float* gamma;        /* [c] or NULL */
  const void* CI;            /* index compressor: [batch][n_buf][2cI] */
  const void* ZI;
  const float* BI;           /* [2m][cI] */
  const float* gammaI;       /* [cI] or NULL */
  void* kv_comp;             /* [batch][E_cap][c], entry floor((t+1)/m) - 1 appended */
  void* KI;                  /* [batch][E_cap][cI] (index_dt layout), appended likewise */
  void* KI_scale;
  const void* qI;            /* [batch][n_hI][cI] */
  const void* qI_scale;
  const float* wI;           /* [batch][n_hI] */
  const void* q;             /* [batch][n_h][c] */
  const float* sink;         /* [n_h] or NULL */
  const float* q_gamma;      /* [c] or NULL */
  const float* kv_gamma;     /* [c] or NULL */
  void* kv_ring;             /* [batch][w][c], token j in slot j % w */
  const void* kv_new;        /* [batch][c] or NULL */
  int32_t* topk_idx;         /* [batch][k] */
  int32_t* topk_cnt;         /* [batch] */
  float* topk_score;         /* [batch][k] or NULL */
  void* out;                 /* [batch][n_h][c] */
  /* Serving state ([Def] section 7: every request owns its state), all optional.
   * t_seq      : device int64 [batch], the position of each sequence's new token
   *              (ragged batches); t is then an upper bound (t >= every t_seq[b]).  The
   *              tail buffers C, Z, CI, ZI become [batch][2m][2c] (resp. 2cI): row 0 is
   *              position m*(t_seq[b]/m) - m (the preceding block, then the current one;
   *              n_buf must be 2m, tok_base is ignored); sequence b emits an entry exactly
   *              when (t_seq[b]+1) % m == 0.
   * page_table : device int32 [batch][max_pages]: paged caches.  Entry s of sequence b is
   *              row page_table[b][s / page_entries] * page_entries + s % page_entries of
   *              the pools kv_comp [pool_rows][c], KI [pool_rows][...] and KI_scale
   *              [pool_rows][...]; E_cap must equal max_pages * page_entries.  With 128-token
   *              pages (page_entries = 128/m) the CSA and HCA caches of a layer share one
   *              page granularity (lcm(m, m') = 128 tokens).
   * Both need the matrix-core attention shapes (bf16 rows of 512 channels, heads in
   * groups of 64, RoPE 0 or 64); otherwise V4A_ENOTSUP. */
  const int64_t* t_seq;
  const int32_t* page_table;
  int64_t max_pages;
  int64_t pool_rows;
  int page_entries;          /* a power of two */
  /* Production cache rows ([Def] section 8): kv576 != 0 stores kv_comp as V4A_KV576 rows
   * ([batch][E_cap][c + rope_dims] bytes, or the pool) with kv_scale float32 [batch][E_cap]
   * (or [pool_rows]); the emitted entry is written in that format and the selected rows
   * are dequantised to bf16 when gathered.  q, the ring and out stay bf16.  Needs the
   * matrix-core shapes with c = 512. */
  int kv576;
  float* kv_scale;
} v4a_decode_step;

/* Byte offsets of the fields of v4a_decode_step in declaration order, for bindings
 * that mirror the struct: writes min(n, number of fields) offsets to off and
 * returns the number of fields; sizeof(v4a_decode_step) goes to *size if non-NULL. */
V4A_API int v4a_decode_step_layout(size_t* off, int n, size_t* size);
V4A_API size_t v4a_csa_decode_step_workspace(const v4a_decode_step* d);
V4A_API int v4a_csa_decode_step(const v4a_decode_step* d, void* ws, size_t ws_bytes, void* stream);

/*
 * v4a_hca_decode_step -- one HCA decode step for every sequence of the batch ([Def]
 * section 7 with the HCA state: ring, main cache appended every m' tokens, no
 * indexer; section 4 for the attention): the new token at position t goes into ring
 * slot t % w (from kv_new, when given); if (t+1) % m' == 0 the completed block's
 * entry (t+1)/m' - 1 is emitted (one-stream compressor of section 2.2, RMSNorm with
 * gamma, RoPE at m' i) into kv_comp; then one softmax per head over every completed
 * entry s < (t+1)/m' joined with the window, with sink, RMSNorm and RoPE as for the
 * CSA calls.  Equivalent to
 *   v4a_compress(C, Z, tail_dt, B, batch, n_buf, tok_base, t, 1, c, m_prime, 0, gamma,
 *                eps, rope_dims, rope_base, kv_comp, NULL, attn_dt, E_cap)
 * followed by the dense attention of v4a_hca_attn for the single query t, with the
 * window read from the ring.  Needs the matrix-core shapes (bf16 rows of 512
 * channels, heads in groups of 64, RoPE 0 or 64); V4A_ENOTSUP otherwise.  Serving
 * state (t_seq, page_table, ...) as in v4a_decode_step; with t_seq the tail buffers
 * are [batch][m'][c] whose row 0 is position m' * (t_seq[b] / m').
 */
typedef struct v4a_hca_step {
  int64_t t;                 /* position of the new token (upper bound with t_seq) */
  int64_t E_cap;             /* rows of kv_comp per sequence (logical capacity when paged) */
  int64_t n_buf, tok_base;   /* tail buffers: n_buf rows, row r = position tok_base + r */
  int batch, n_h, c, m_prime, w;
  int num_splits;            /* 0 = automatic */
  int rope_dims;
  float rope_base, eps, scale;
  v4a_dtype tail_dt;         /* C, Z: F32 or BF16 */
  v4a_dtype attn_dt;         /* q, kv_comp, kv_ring, kv_new, out: BF16 */
  const void* C;             /* [batch][n_buf][c] */
  const void* Z;
  const float* B;            /* [m_prime][c] */
  const float* gamma;        /* [c] or NULL */
  void* kv_comp;             /* [batch][E_cap][c] (or the pool when paged) */
  const void* q;             /* [batch][n_h][c] */
  const float* sink;         /* [n_h] or NULL */
  const float* q_gamma;      /* [c] or NULL */
  const float* kv_gamma;     /* [c] or NULL */
  void* kv_ring;             /* [batch][w][c], token j in slot j % w */
  const void* kv_new;        /* [batch][c] or NULL */
  void* out;                 /* [batch][n_h][c] */
  const int64_t* t_seq;      /* serving state, as in v4a_decode_step */
  const int32_t* page_table;
  int64_t max_pages;
  int64_t pool_rows;
  int page_entries;
} v4a_hca_step;

V4A_API int v4a_hca_decode_step_layout(size_t* off, int n, size_t* size);
V4A_API size_t v4a_hca_decode_step_workspace(const v4a_hca_step* d);
V4A_API int v4a_hca_decode_step(const v4a_hca_step* d, void* ws, size_t ws_bytes, void* stream);

/*
 * v4a_linear -- a plain projection Y = X W^T of the layer around the attention path
 * (the query, indexer and compressor projections of [Def] sections 2.1, 3.1, 3.2
 * and 5.1): Y[t][n] = sum_k X[t][k] W[n][k], bf16 operands, float32 accumulation.
 *   X   : device bf16 [T][K];  W : device bf16 [N][K] (row n = output feature n).
 *   Y   : device [T][N] of out_dt (V4A_BF16 or V4A_F32).
 *   ws  : device workspace of v4a_linear_workspace(T, K, N) bytes, 16-byte aligned.
 * Errors: V4A_EINVAL for null pointers or sizes < 1; V4A_ENOTSUP if K or N is not a
 *   multiple of 8 or out_dt is another type; V4A_ENOSPC for a small workspace;
 *   V4A_EIO if the GEMM library fails.
 */
V4A_API size_t v4a_linear_workspace(int T, int K, int N);
V4A_API int v4a_linear(const void* X, const void* W, int T, int K, int N, void* Y, v4a_dtype out_dt,
               void* ws, size_t ws_bytes, void* stream);

/*
 * v4a_grouped_out_proj -- the grouped output projection ([Def] section 5.4):
 *   out[t] = W_B [ W_A[0] o^G[t][0]; ... ; W_A[g-1] o^G[t][g-1] ]
 * where o^G[t][i] is the concatenation of the c-wide outputs of heads
 * i n_h/g .. (i+1) n_h/g - 1 of query t (a contiguous block of its output row).
 *   o    : device bf16 [T][n_h][c], the attention output.
 *   W_A  : device bf16 [g][d_g][c n_h/g].
 *   W_B  : device bf16 [d][g d_g].
 *   out  : device bf16 [T][d].
 *   ws   : device workspace of v4a_grouped_out_proj_workspace(...) bytes, 256-byte
 *          aligned; it also holds the intermediate [T][g d_g] (rounded to bf16).
 * Float32 accumulation.  Errors: V4A_EINVAL for null pointers, sizes < 1 or n_h not
 *   a multiple of g; V4A_ENOTSUP unless c n_h/g, d_g and d are multiples of 8;
 *   V4A_ENOSPC; V4A_EIO.
 */
V4A_API size_t v4a_grouped_out_proj_workspace(int T, int n_h, int c, int g, int d_g, int d);
V4A_API int v4a_grouped_out_proj(const void* o, const void* W_A, const void* W_B, int T, int n_h,
                         int c, int g, int d_g, int d, void* out, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * v4a_csa_decode_step_noalloc -- v4a_csa_decode_step for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops or harnesses
 * that forbid allocation).  Same description `d`, same results bit for bit, same
 * errors; the workspace is a fixed device array inside the library of
 * V4A_NOALLOC_SCRATCH_BYTES (64 MiB), one copy per GPU, held until the process
 * ends.  The call allocates and frees nothing.
 *   - V4A_ENOSPC (with a message naming both sizes) when
 *     v4a_csa_decode_step_workspace(d) exceeds the array.  64 MiB covers batch 64 at
 *     128K context with the V4-Flash shapes (about 32 MiB at batch 32) and batch 4 at
 *     1M context with the V4-Pro shapes (about 21 MiB).
 *   - Every call on one GPU uses that GPU's array, which keeps the last call's
 *     contents (nothing in it needs clearing between calls).  Calls that overlap in
 *     time on one GPU (several streams or threads) race on it: serialise them.
 */
#define V4A_NOALLOC_SCRATCH_BYTES (64u << 20)
V4A_API int v4a_csa_decode_step_noalloc(const v4a_decode_step* d, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* V4A_H */
