// Host-side launcher interface between the C ABI layer (api.cpp) and the
// kernel translation units.  Arguments are validated before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace v4a {

enum Dt : int { kF32 = 0, kBF16 = 1, kFP8 = 2, kMXFP4 = 3 };

// RoPE inverse frequencies base^(-2i/rope_dims), i < rope_dims/2 (rope_dims <= 64).
constexpr int kMaxRopeDims = 64;
struct RopeTab {
  double inv_freq[kMaxRopeDims / 2];
};
void rope_table(RopeTab& tab, int rope_dims, float rope_base);

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
};

// Window-row preparation (attention prep kernel, fused decode front).
struct LocalPrepArgs {
  const uint16_t* src;   // prefill: kv_local [batch][n_loc][512]; decode: ring [batch][w][512]
  uint16_t* ring;        // decode: ring to insert kv_new into (may alias src)
  const uint16_t* kv_new;
  const float* gamma;
  uint16_t* ws;          // [batch][n_lrows][512]
  int* redo;             // count of the recomputation list, cleared here
  int64_t lrow_base, loc_base, n_loc, n_lrows, t;
  int w, rope_dims, decode;
  float eps, rope_base;
  RopeTab rope;
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
};

enum AttnMode : int { kModeCSA = 0, kModeDecode = 1, kModeHCA = 2 };

// launchers (return hipSuccess or the launch error)
hipError_t launch_visibility(int64_t t0, int T, int m, int k, int w, int32_t* E, int32_t* cnt,
                             int32_t* lo, int32_t* len, hipStream_t s);
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);

IndexerPlan indexer_plan(int batch, int T, int64_t t0, int n_hI, int cI, int m, int k, int dt,
                         int policy);
hipError_t launch_indexer_topk(const IndexerArgs& a, const IndexerPlan& p, void* ws,
                               hipStream_t s);

size_t attn_workspace(const AttnArgs& a, int policy);
hipError_t launch_attention(const AttnArgs& a, void* ws, int policy, hipStream_t s);

// Fused decode front (one launch: main and index tail compression, window-row prep and
// ring insert).  Supported when the attention takes the matrix-core path and both
// compressor instances take the register-resident path with bf16 inputs.
bool decode_front_supported(const CompressArgs& cm, const CompressArgs& ci, const AttnArgs& a,
                            int policy);
hipError_t launch_decode_front(const CompressArgs& cm, const CompressArgs& ci, const AttnArgs& a,
                               void* attn_ws, hipStream_t s);

}  // namespace v4a
