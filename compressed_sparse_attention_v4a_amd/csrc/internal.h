// Host-side launcher interface between the C ABI layer (api.cpp) and the
// kernel translation units.  Arguments are validated before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct v4a_decode_step;

namespace v4a {

// The whole decode step of v4a_csa_decode_step with the workspace `ws` (validation,
// launches, error reporting).
int decode_step_run(const v4a_decode_step* d, void* ws, size_t ws_bytes, void* stream);
// Sets the calling thread's v4a_last_error() message; returns code.
int report_error(int code, const char* msg);

enum Dt : int { kF32 = 0, kBF16 = 1, kFP8 = 2, kMXFP4 = 3, kKV576 = 4 };

// Production main-cache row (kKV576): the c - rope_dims leading channels as E4M3 codes
// scaled by one float32 per row, then the rope_dims rotated channels as bf16
// (c = 512, rope_dims = 64: 448 + 128 = 576 bytes).
__host__ __device__ inline int kv576_row_bytes(int c, int rope_dims) { return c + rope_dims; }

// RoPE inverse frequencies base^(-2i/rope_dims), i < rope_dims/2 (rope_dims <= 64).
constexpr int kMaxRopeDims = 64;
struct RopeTab {
  double inv_freq[kMaxRopeDims / 2];
};
void rope_table(RopeTab& tab, int rope_dims, float rope_base);

// Serving state shared by the decode kernels (all optional):
//   tpos   : per-sequence positions of the new token (device [batch]); NULL = the
//            uniform position of the call.
//   pages  : block table (device [batch][max_pages]) of paged caches: entry s of
//            sequence b lives in pool row pages[b][s >> page_shift] << page_shift |
//            (s & (2^page_shift - 1)); NULL = contiguous [batch][E_cap] caches.
struct SeqState {
  const int64_t* tpos;
  const int32_t* pages;
  int64_t max_pages;
  int page_shift;
};

// Row of entry s of sequence b in a cache of E_cap rows per sequence (or in the pool).
__host__ __device__ inline int64_t cache_row(const SeqState& st, int64_t E_cap, int b, int64_t s) {
  if (st.pages) {
    const int64_t pg = st.pages[(int64_t)b * st.max_pages + (s >> st.page_shift)];
    return (pg << st.page_shift) | (s & (((int64_t)1 << st.page_shift) - 1));
  }
  return (int64_t)b * E_cap + s;
}

struct CompressArgs {
  const void* C;
  const void* Z;
  const float* B;
  const float* gamma;
  void* out;
  void* out_scale;
  int64_t n_buf, tok_base, i_begin, E_cap;
  int n_entries, batch, c, m, overlap, rope_dims;
  int in_dt, out_dt;
  float eps, rope_base;
  RopeTab rope;
  // Per-sequence decode (seq.tpos set): sequence b emits entry tpos[b] / m when
  // (tpos[b] + 1) % m == 0, from a tail buffer whose row 0 is position
  // m * (tpos[b] / m) - (overlap ? m : 0) (the preceding block, then the current one).
  SeqState seq;
};

// Window-row preparation (attention prep kernel, fused decode front).
struct LocalPrepArgs {
  const uint16_t* src;   // prefill: kv_local [batch][n_loc][512]; decode: ring [batch][w][512]
  uint16_t* ring;        // decode: ring to insert kv_new into (may alias src)
  const uint16_t* kv_new;
  const float* gamma;
  uint16_t* ws;          // [batch][n_lrows][512]
  int64_t lrow_base, loc_base, n_loc, n_lrows, t;
  int w, rope_dims, decode;
  float eps, rope_base;
  RopeTab rope;
  const int64_t* tpos;   // decode: per-sequence position of the new token (or NULL: t)
};

struct IndexerArgs {
  const void* qI;
  const void* qI_scale;
  const void* KI;
  const void* KI_scale;
  const float* wI;
  int32_t* topk_idx;
  int32_t* topk_cnt;
  float* topk_score;
  int64_t t0, E_cap;
  int batch, T, n_hI, cI, m, k, dt;
  SeqState seq;      // decode: per-sequence positions and paged key rows
  int32_t* phys;     // paged decode: the selected entries' pool rows, aligned with topk_idx
};

// Workspace plan of the indexer: scores [batch][T][ld] f32 and stage-A candidates.
struct IndexerPlan {
  int64_t ld;        // score row stride (>= max visible entries of the chunk)
  int tile;          // entries per top-k stage-A tile
  int n_tiles;       // tiles per query
  int kc;            // candidates kept per tile = min(k, tile)
  bool fused;        // MFMA fused score + top-k path (no score buffer)
  bool mfma_scan;    // MFMA score scan into the score buffer (else the general kernel)
  bool filter;       // decode: threshold filter + final selection instead of tiles + merge
  int gshift;        // filter: group maxima over 16 << gshift entries
  int n_slices;      // filter: 4096-entry slices per query
  int64_t ng_ld;     // filter: group maxima per query row (padded)
  size_t score_bytes, cand_bytes, total;
};

struct AttnArgs {
  const void* q;
  const void* kv_comp;
  const void* kv_local;  // prefill / HCA: raw local rows; decode: ring
  void* kv_ring;
  const void* kv_new;
  const int32_t* idx;
  const int32_t* cnt;
  const float* sink;
  const float* q_gamma;
  const float* kv_gamma;
  void* out;
  int64_t loc_base, n_loc, t0, E_cap;
  int batch, T, n_h, c, k, w, m_prime, rope_dims, dt, mode, num_splits;
  int prep_done;  // window rows already prepared (fused decode front kernel)
  float eps, rope_base, scale;
  RopeTab rope;
  SeqState seq;   // decode: per-sequence positions and paged rows (idx then holds pool rows)
  const int32_t* dense_cnt;  // kModeHCADecode over a staged list: cnt[b] rows per sequence
};

// kModeHCADecode: one new token per sequence, every completed entry (ratio m_prime) and
// the ring window.
// Position of query j of sequence b (per-sequence decode positions when given).
__device__ inline int64_t query_pos(const IndexerArgs& a, int b, int j) {
  return a.seq.tpos ? a.seq.tpos[b] + j : a.t0 + j;
}

enum AttnMode : int { kModeCSA = 0, kModeDecode = 1, kModeHCA = 2, kModeHCADecode = 3 };

// launchers (return hipSuccess or the launch error)
hipError_t launch_visibility(int64_t t0, int T, int m, int k, int w, int32_t* E, int32_t* cnt,
                             int32_t* lo, int32_t* len, hipStream_t s);
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);

// serving: per-sequence positions or paged keys (the all-in-LDS fused kernels, which
// assume neither, are not planned)
IndexerPlan indexer_plan(int batch, int T, int64_t t0, int n_hI, int cI, int m, int k, int dt,
                         int policy, bool serving = false);
// Decode-step work that rides in the top-k final launch of the threshold-filter path
// (extra workgroups per sequence): the main-cache tail compression, the window-row prep
// and the ring insert, which the attention needs but the index scan does not.
struct FrontArgs {
  CompressArgs cm;     // main instance (n_entries 0: nothing to emit)
  LocalPrepArgs lp;    // window rows into the attention workspace, new token into the ring
  int n_comp, n_prep;  // workgroups per sequence of each role
  int gm;              // lanes per main entry, c / 8 (16, 32 or 64)
};

// ci (decode step, or NULL): the index-cache entry that the step's new token completes is
// compressed inside the scan (indexer_fuses_compress(p, *ci) must hold).  front (or NULL,
// threshold-filter plans only): run with the final selection.
hipError_t launch_indexer_topk(const IndexerArgs& a, const IndexerPlan& p, void* ws,
                               hipStream_t s, const CompressArgs* ci = nullptr,
                               const FrontArgs* front = nullptr);
bool indexer_fuses_compress(const IndexerPlan& p, const CompressArgs& ci);

size_t attn_workspace(const AttnArgs& a, int policy);
bool attn_mfma_supported(const AttnArgs& a);  // the matrix-core kernels take this shape
// Selected production-format rows (kKV576, c = 512) of a decode step -> bf16 staging
// [batch][k][512].
hipError_t launch_kv576_gather(const void* kv, const float* kv_scale, const int32_t* idx,
                               const int32_t* cnt, const SeqState& seq, int64_t E_cap, int batch,
                               int k, int rope_dims, void* staged, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, void* ws, int policy, hipStream_t s);

// Fused decode front (one launch: main and index tail compression, window-row prep and
// ring insert).  Supported when the attention takes the matrix-core path and both
// compressor instances take the register-resident path with bf16 inputs.
bool decode_front_supported(const CompressArgs& cm, const CompressArgs& ci, const AttnArgs& a,
                            int policy);
hipError_t launch_decode_front(const CompressArgs& cm, const CompressArgs& ci, const AttnArgs& a,
                               void* attn_ws, hipStream_t s);
// The same front work minus the index instance, described for the top-k final launch.
hipError_t decode_front_args(const CompressArgs& cm, const AttnArgs& a, void* attn_ws,
                             FrontArgs& out);

}  // namespace v4a
