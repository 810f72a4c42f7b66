// Lightning indexer score and per-query top-k ("CSA And HCA: Definition,
// State, And Cost Model", section 3.1):
//   I[t][s] = sum_h wI[t][h] * max(0, qI[t][h] . KI[s])   for s < floor((t+1)/m)
// followed by TopK over those s, ties to the lower index.
//
// General path (any dtype and shape):
//   1. index_scores_kernel: one lane per entry s, all heads of one query; the
//      query's decoded rows sit in LDS and are read as broadcasts.  Scores go to
//      a float32 workspace [batch][T][ld].
//   2. topk_tile_kernel: per (query, tile of entries) an exact radix select in
//      LDS-resident histograms keeps min(k, tile) candidates (key + index, in
//      index order).  With one tile per query this writes the final result.
//   3. topk_merge_kernel: per query, the same select over the tiles' candidates.
// The MFMA paths for the production shapes live in indexer_mfma.hip and reuse
// the two top-k kernels.
#include "compress_rows.h"
#include "device_common.h"
#include "internal.h"
#include "topk.h"
#include "window_prep.h"

namespace v4a {

namespace {

// Selected entry e (or -1 padding) into slot pos of query row q, and, for paged caches,
// its pool row into the parallel list the attention gathers from.
__device__ __forceinline__ void write_sel(const IndexerArgs& a, int b, int64_t q, int pos, int32_t e) {
  a.topk_idx[q * a.k + pos] = e;
  if (a.phys) a.phys[q * a.k + pos] = e >= 0 ? (int32_t)cache_row(a.seq, a.E_cap, b, e) : -1;
}

constexpr int kScoreThreads = 256;
constexpr int kHeadChunk = 32;

__device__ __forceinline__ float load_elem(const void* base, int64_t i, int dt) {
  if (dt == kF32) return reinterpret_cast<const float*>(base)[i];
  if (dt == kBF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
  if (dt == kFP8) return e4m3_to_f32(reinterpret_cast<const uint8_t*>(base)[i]);
  const uint8_t byte = reinterpret_cast<const uint8_t*>(base)[i >> 1];
  return e2m1_to_f32((i & 1) ? (byte >> 4) : (byte & 15u));
}

// One block per (entry tile, query, sequence).
__global__ __launch_bounds__(kScoreThreads) void index_scores_kernel(IndexerArgs a, float* scores,
                                                                      int64_t ld) {
  extern __shared__ float sq[];  // [n_hI][cI] decoded query, then [n_hI] weights
  const int j = blockIdx.x, b = blockIdx.z;
  const int64_t t = query_pos(a, b, j);
  const int64_t E = (t + 1) / a.m;
  const int64_t s = (int64_t)blockIdx.y * kScoreThreads + threadIdx.x;
  const int nh = a.n_hI, cI = a.cI;
  float* sw = sq + (size_t)nh * cI;
  const int64_t qrow0 = ((int64_t)b * a.T + j) * nh;
  if ((int64_t)blockIdx.y * kScoreThreads >= E) {
    // whole tile beyond the visible entries: nothing to score
    return;
  }
  for (int e = threadIdx.x; e < nh * cI; e += kScoreThreads) {
    const int h = e / cI, d = e % cI;
    const int64_t qi = (qrow0 + h) * cI + d;
    float v = load_elem(a.qI, qi, a.dt);
    if (a.dt == kFP8) v *= reinterpret_cast<const float*>(a.qI_scale)[qrow0 + h];
    if (a.dt == kMXFP4)
      v *= e8m0_to_f32(reinterpret_cast<const uint8_t*>(a.qI_scale)[(qrow0 + h) * (cI / 32) + d / 32]);
    sq[e] = v;
  }
  for (int h = threadIdx.x; h < nh; h += kScoreThreads) sw[h] = a.wI[qrow0 + h];
  __syncthreads();
  if (s >= E) return;
  const int64_t krow = cache_row(a.seq, a.E_cap, b, s);
  float ks = 1.0f;
  if (a.dt == kFP8) ks = reinterpret_cast<const float*>(a.KI_scale)[krow];
  float score = 0.0f;
  for (int h0 = 0; h0 < nh; h0 += kHeadChunk) {
    float acc[kHeadChunk];
#pragma unroll
    for (int h = 0; h < kHeadChunk; ++h) acc[h] = 0.0f;
    for (int d = 0; d < cI; ++d) {
      float kv = load_elem(a.KI, krow * cI + d, a.dt);
      if (a.dt == kMXFP4)
        kv *= e8m0_to_f32(reinterpret_cast<const uint8_t*>(a.KI_scale)[krow * (cI / 32) + d / 32]);
#pragma unroll
      for (int h = 0; h < kHeadChunk; ++h)
        if (h0 + h < nh) acc[h] = fmaf(sq[(h0 + h) * cI + d], kv, acc[h]);
    }
#pragma unroll
    for (int h = 0; h < kHeadChunk; ++h)
      if (h0 + h < nh) score = fmaf(sw[h0 + h], fmaxf(acc[h] * ks, 0.0f), score);
  }
  scores[((int64_t)b * a.T + j) * ld + s] = score;
}

struct TopkOut {
  int32_t* idx;
  int32_t* cnt;
  float* score;
};

// Stage A: per (tile, query, sequence).  n_tiles == 1: final output.
__global__ __launch_bounds__(256) void topk_tile_kernel(IndexerArgs a, const float* scores,
                                                        int64_t ld, int tile, int n_tiles, int kc,
                                                        uint32_t* cand_key, int32_t* cand_idx) {
  __shared__ uint32_t hist[768];
  __shared__ int sh[16];
  const int j = blockIdx.x, tl = blockIdx.y, b = blockIdx.z;
  const int64_t t = query_pos(a, b, j);
  const int64_t E = (t + 1) / a.m;
  const int64_t s0 = (int64_t)tl * tile;
  const int N = (int)max((int64_t)0, min((int64_t)tile, E - s0));
  const int64_t q = (int64_t)b * a.T + j;
  const float* srow = scores + q * ld + s0;
  auto get = [&](int i) { return score_key(srow[i]); };
  if (n_tiles == 1) {
    const int k = a.k;
    float* osc = a.topk_score ? a.topk_score + q * k : nullptr;
    auto emit = [&](int pos, int i, uint32_t key) {
      write_sel(a, b, q, pos, (int32_t)(s0 + i));
      if (osc) osc[pos] = key_score(key);
    };
    const int n = min(N, k);
    if (N <= k) {
      block_emit_all(get, N, emit);
    } else {
      const Selection sel = block_radix_select(get, N, k, hist, sh);
      block_select_emit(get, N, k, sel, sh, emit);
    }
    for (int p = n + threadIdx.x; p < k; p += blockDim.x) {
      write_sel(a, b, q, p, -1);
      if (osc) osc[p] = 0.0f;
    }
    if (threadIdx.x == 0) a.topk_cnt[q] = n;
    return;
  }
  uint32_t* ck = cand_key + (q * n_tiles + tl) * kc;
  int32_t* ci = cand_idx + (q * n_tiles + tl) * kc;
  auto emit = [&](int pos, int i, uint32_t key) {
    ck[pos] = key;
    ci[pos] = (int32_t)(s0 + i);
  };
  const int n = min(N, kc);
  if (N <= kc) {
    block_emit_all(get, N, emit);
  } else {
    const Selection sel = block_radix_select(get, N, kc, hist, sh);
    block_select_emit(get, N, kc, sel, sh, emit);
  }
  for (int p = n + threadIdx.x; p < kc; p += blockDim.x) {
    ck[p] = 0u;  // below every real score's key
    ci[p] = -1;
  }
}

// Stage B: per (query, sequence): select among n_tiles * kc candidates.
__global__ __launch_bounds__(1024) void topk_merge_kernel(IndexerArgs a, int n_tiles, int kc,
                                                          const uint32_t* cand_key,
                                                          const int32_t* cand_idx) {
  __shared__ uint32_t hist[768];
  __shared__ int sh[40];
  const int j = blockIdx.x, b = blockIdx.y;
  const int64_t t = query_pos(a, b, j);
  const int64_t E = (t + 1) / a.m;
  const int64_t q = (int64_t)b * a.T + j;
  const int k = a.k;
  const int n = (int)min((int64_t)k, E);
  const int N = n_tiles * kc;
  const uint32_t* ck = cand_key + q * N;
  const int32_t* ci = cand_idx + q * N;
  float* osc = a.topk_score ? a.topk_score + q * k : nullptr;
  auto get = [&](int i) { return ck[i]; };
  auto emit = [&](int pos, int i, uint32_t key) {
    write_sel(a, b, q, pos, ci[i]);
    if (osc) osc[pos] = key_score(key);
  };
  if (n > 0) {
    // exactly n real candidates are wanted; padding keys (0) rank below all of them
    const Selection sel = block_radix_select(get, N, n, hist, sh);
    block_select_emit(get, N, n, sel, sh, emit);
  }
  for (int p = n + threadIdx.x; p < k; p += blockDim.x) {
    write_sel(a, b, q, p, -1);
    if (osc) osc[p] = 0.0f;
  }
  if (threadIdx.x == 0) a.topk_cnt[q] = n;
}

// Register forms of the two stages (keys loaded once, contiguous per thread; see topk.h).
// Stage A over tiles of 16 * THREADS entries (4096 or 16384).
template <int THREADS>
__global__ __launch_bounds__(THREADS) void topk_tile_reg_kernel(IndexerArgs a, const float* scores,
                                                            int64_t ld, int n_tiles, int kc,
                                                            uint32_t* cand_key, int32_t* cand_idx) {
  constexpr int PER = 16, kRegTile = PER * THREADS;
  __shared__ uint32_t hist[768];
  __shared__ int sh[40];
  const int j = blockIdx.x, tl = blockIdx.y, b = blockIdx.z;
  const int64_t t = query_pos(a, b, j);
  const int64_t E = (t + 1) / a.m;
  const int64_t s0 = (int64_t)tl * kRegTile;
  const int N = (int)max((int64_t)0, min((int64_t)kRegTile, E - s0));
  const int64_t q = (int64_t)b * a.T + j;
  const float* srow = scores + q * ld + s0;
  const int base = threadIdx.x * PER;
  uint32_t key[PER];
  if (N == kRegTile) {
#pragma unroll
    for (int v = 0; v < PER; v += 4) {
      const float4 f = *reinterpret_cast<const float4*>(srow + base + v);
      key[v] = score_key(f.x); key[v + 1] = score_key(f.y);
      key[v + 2] = score_key(f.z); key[v + 3] = score_key(f.w);
    }
  } else {
#pragma unroll
    for (int v = 0; v < PER; ++v) key[v] = base + v < N ? score_key(srow[base + v]) : 0u;
  }
  const bool final_out = n_tiles == 1;
  const int want = final_out ? a.k : kc;
  const int n = min(N, want);
  float* osc = a.topk_score ? a.topk_score + q * a.k : nullptr;
  uint32_t* ck = cand_key + (q * n_tiles + tl) * kc;
  int32_t* ci = cand_idx + (q * n_tiles + tl) * kc;
  auto emit = [&](int pos, int i, uint32_t kk) {
    if (final_out) {
      write_sel(a, b, q, pos, (int32_t)(s0 + i));
      if (osc) osc[pos] = key_score(kk);
    } else {
      ck[pos] = kk;
      ci[pos] = (int32_t)(s0 + i);
    }
  };
  // N <= want: every element, in order (the selection "all keys > 0 or == 0" with need_eq
  // equal to the number of zero keys among the first N is the same as taking all)
  Selection sel{0u, kRegTile};
  if (N > want) sel = reg_radix_select(key, N, want, hist, sh);
  reg_select_emit(key, N, sel, sh, emit);
  for (int p = n + threadIdx.x; p < want; p += blockDim.x) {
    if (final_out) {
      write_sel(a, b, q, p, -1);
      if (osc) osc[p] = 0.0f;
    } else {
      ck[p] = 0u;  // below every real score's key
      ci[p] = -1;
    }
  }
  if (final_out && threadIdx.x == 0) a.topk_cnt[q] = n;
}

// Stage B over N = n_tiles * kc <= 1024 * PER candidates with 1024 threads.
template <int PER>
__global__ __launch_bounds__(1024) void topk_merge_reg_kernel(IndexerArgs a, int n_tiles, int kc,
                                                              const uint32_t* cand_key,
                                                              const int32_t* cand_idx) {
  __shared__ uint32_t hist[768];
  __shared__ int sh[40];
  const int j = blockIdx.x, b = blockIdx.y;
  const int64_t t = query_pos(a, b, j);
  const int64_t E = (t + 1) / a.m;
  const int64_t q = (int64_t)b * a.T + j;
  const int k = a.k;
  const int n = (int)min((int64_t)k, E);
  const int N = n_tiles * kc;
  const uint32_t* ck = cand_key + q * N;
  const int32_t* ci = cand_idx + q * N;
  float* osc = a.topk_score ? a.topk_score + q * k : nullptr;
  const int base = threadIdx.x * PER;
  uint32_t key[PER];
  if (base + PER <= N && (N & 3) == 0) {
#pragma unroll
    for (int v = 0; v < PER; v += 4) {
      const uint4 u = *reinterpret_cast<const uint4*>(ck + base + v);
      key[v] = u.x; key[v + 1] = u.y; key[v + 2] = u.z; key[v + 3] = u.w;
    }
  } else {
#pragma unroll
    for (int v = 0; v < PER; ++v) key[v] = base + v < N ? ck[base + v] : 0u;
  }
  if (n > 0) {
    // exactly n real candidates are wanted; padding keys (0) rank below all of them
    const Selection sel = reg_radix_select(key, N, n, hist, sh);
    auto emit = [&](int pos, int i, uint32_t kk) {
      write_sel(a, b, q, pos, ci[i]);
      if (osc) osc[pos] = key_score(kk);
    };
    reg_select_emit(key, N, sel, sh, emit);
  }
  for (int p = n + threadIdx.x; p < k; p += blockDim.x) {
    write_sel(a, b, q, p, -1);
    if (osc) osc[p] = 0.0f;
  }
  if (threadIdx.x == 0) a.topk_cnt[q] = n;
}

// ---- decode top-k by threshold filter (one query row over E >> k entries) ----------
// The scan also records the maximum order key of every group of Gs = 16 << gshift
// consecutive entries.  Any K of those maxima are keys of K distinct entries, so the K-th
// largest group maximum is at most the K-th largest key T of the row; its top 16 bits
// (2 radix passes), low bits cleared, give a lower bound L <= T.  Every entry with key
// >= L is a candidate; they include every selected entry.  With n_g = 2k .. 4k groups the
// candidates number about k (1 + k Gs / 2E) plus the entries sharing T's top 16 bits.
//   filter: workgroup (slice, query) recomputes L from the group maxima, then compacts its
//           4096 entries with key >= L, in index order, into the slice's own region.
//   final : one workgroup per query selects the k largest candidates exactly (ties to
//           the lower index) and writes them in ascending index order: from registers
//           up to 4096 candidates, else streaming them from the workspace.  In a decode
//           step (GM > 0) the launch also carries the step's front work in workgroups
//           1.. of each sequence's row (FrontArgs): the final selection is a few
//           latency-bound workgroups, so the front runs beside it instead of in a launch
//           of its own ahead of the scan.
constexpr int kFiltSlice = 4096;      // entries per filter workgroup (256 threads x 16)
constexpr int kFiltGroups = 4096;     // group maxima per query at most (256 threads x 16)
constexpr int kFinalThreads = 256;    // final kernel: few waves keep its barriers and scans short
constexpr int kFinalPer = 16;         // candidates per thread held in registers (x 256)

__global__ __launch_bounds__(256) void topk_filter_kernel(IndexerArgs a, const float* scores,
                                                          int64_t ld, const uint32_t* gmax,
                                                          int64_t ng_ld, int gshift, int n_slices,
                                                          int* counts, uint32_t* cand_key,
                                                          int32_t* cand_idx) {
  __shared__ uint32_t hist[768];
  __shared__ int sh[40];
  const int sl = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int64_t t = query_pos(a, b, j);
  const int64_t E = (t + 1) / a.m;
  const int64_t q = (int64_t)b * a.T + j;
  // lower bound L from the group maxima (every workgroup of the row computes the same)
  const int ng = (int)((E + (16 << gshift) - 1) >> (4 + gshift));
  // every load first (group maxima and this slice's scores), from clamped addresses with
  // the absent elements masked afterwards, so that no load waits behind a branch
  constexpr int GP = kFiltGroups / 256;
  uint32_t gk[GP];
  const uint32_t* gq = gmax + q * ng_ld;
  // group maxima spread evenly over the threads (multiples of 4 for 16-byte loads)
  const int gper = ((ng + 255) / 256 + 3) & ~3;
  const int gb = threadIdx.x * gper;
#pragma unroll
  for (int v = 0; v < GP; v += 4) {
    const uint4 x = *reinterpret_cast<const uint4*>(gq + ((v < gper && gb + v < ng_ld) ? gb + v : 0));
    gk[v] = x.x; gk[v + 1] = x.y; gk[v + 2] = x.z; gk[v + 3] = x.w;
  }
  const int64_t s0 = (int64_t)sl * kFiltSlice;
  const int N = (int)max((int64_t)0, min((int64_t)kFiltSlice, E - s0));
  const float* srow = scores + q * ld + s0;
  const int base = threadIdx.x * 16;
  float f[16];
#pragma unroll
  for (int v = 0; v < 16; v += 4) {
    // the row has ld >= E entries allocated: clamp the slice into it
    const int64_t o = s0 + base + v + 4 <= ld ? base + v : 0;
    const float4 x = *reinterpret_cast<const float4*>(srow + o);
    f[v] = x.x; f[v + 1] = x.y; f[v + 2] = x.z; f[v + 3] = x.w;
  }
#pragma unroll
  for (int v = 0; v < GP; ++v) gk[v] = (v < gper && gb + v < ng) ? gk[v] : 0u;
  uint32_t key[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) key[v] = base + v < N ? score_key(f[v]) : 0u;
  // lower bound L from the group maxima (every workgroup of the row computes the same)
  uint32_t L = 0u;
  if (ng >= a.k) L = reg_radix_select(gk, ng, a.k, hist, sh, 16, gper).kth;
  int mine = 0;
#pragma unroll
  for (int v = 0; v < 16; ++v) mine += (base + v < N && key[v] >= L) ? 1 : 0;
  int tot;
  int pos = block_excl_sum(mine, sh, &tot);
  const int64_t reg = (q * n_slices + sl) * kFiltSlice;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    if (base + v < N && key[v] >= L) {
      cand_key[reg + pos] = key[v];
      cand_idx[reg + pos] = (int32_t)(s0 + base + v);
      ++pos;
    }
  }
  if (threadIdx.x == 0) counts[q * n_slices + sl] = tot;
}

template <int GM>
__global__ __launch_bounds__(kFinalThreads) void topk_final_kernel(IndexerArgs a, int n_slices,
                                                          const int* counts,
                                                          const uint32_t* cand_key,
                                                          const int32_t* cand_idx, FrontArgs f) {
  if constexpr (GM > 0) {
    if (blockIdx.x > 0) {  // front work of sequence blockIdx.y (T == 1: block 0 selects)
      const int blk = (int)blockIdx.x - 1, b = blockIdx.y;
      if (blk >= f.n_comp) {
        window_prep_block<kFrontRows / 4>(f.lp, blk - f.n_comp, b, threadIdx.x);
        return;
      }
      const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
      if (wv == 0 && (int64_t)blk * (64 / GM) < f.cm.n_entries)
        compress_rows_body<uint16_t, GM>(f.cm, blk, b, lane);
      return;
    }
  }
  __shared__ uint32_t hist[768];
  __shared__ int sh[40];
  __shared__ int pre[65];  // candidate offset of every slice (n_slices <= 64)
  const int j = blockIdx.x, b = blockIdx.y;
  const int64_t t = query_pos(a, b, j);
  const int64_t E = (t + 1) / a.m;
  const int64_t q = (int64_t)b * a.T + j;
  const int k = a.k;
  if (threadIdx.x < 64) {
    // slice counts loaded by one wave at once, then an inclusive scan across its lanes
    const int lane = threadIdx.x;
    const int c = lane < n_slices ? counts[q * n_slices + lane] : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    if (lane < n_slices) pre[lane + 1] = incl;
    if (lane == 0) pre[0] = 0;
  }
  __syncthreads();
  const int total = pre[n_slices];
  // candidates >= min(k, E) by construction; the minimum keeps the selection in range
  const int n = (int)min(min((int64_t)k, E), (int64_t)total);
  float* osc = a.topk_score ? a.topk_score + q * k : nullptr;
  // candidate p of the row (slice order = index order)
  auto at = [&](int p) -> int64_t {
    int lo = 0, hi = n_slices;  // pre[lo] <= p < pre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= p) lo = mid; else hi = mid;
    }
    return (q * n_slices + lo) * kFiltSlice + (p - pre[lo]);
  };
  if (total <= kFinalThreads * kFinalPer) {
    uint32_t key[kFinalPer];
    int32_t ix[kFinalPer];
    // the list spread evenly over the threads (thread t owns [t per, t per + per))
    const int per = (total + kFinalThreads - 1) / kFinalThreads;
    const int base = threadIdx.x * per;
    if (base < total) {
      // every load first, from clamped positions; absent elements masked afterwards.  The
      // thread's candidates are consecutive, so after one search the slice only advances.
      int64_t off[kFinalPer];
      {
        int lo = 0, hi = n_slices;  // pre[lo] <= base < pre[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (pre[mid] <= base) lo = mid; else hi = mid;
        }
        int sl = lo;
#pragma unroll
        for (int v = 0; v < kFinalPer; ++v) {
          const int p = (v < per && base + v < total) ? base + v : total - 1;
          while (pre[sl + 1] <= p) ++sl;
          off[v] = (q * n_slices + sl) * kFiltSlice + (p - pre[sl]);
        }
      }
#pragma unroll
      for (int v = 0; v < kFinalPer; ++v) {
        key[v] = cand_key[off[v]];
        ix[v] = cand_idx[off[v]];
      }
#pragma unroll
      for (int v = 0; v < kFinalPer; ++v) {
        key[v] = (v < per && base + v < total) ? key[v] : 0u;
        ix[v] = (v < per && base + v < total) ? ix[v] : -1;
      }
    } else {
#pragma unroll
      for (int v = 0; v < kFinalPer; ++v) {
        key[v] = 0u;
        ix[v] = -1;
      }
    }
    Selection sel{0u, kFinalThreads * kFinalPer};  // every candidate (total == n)
    if (total > n) sel = reg_radix_select(key, total, n, hist, sh, 0, per);
    reg_select_emit_slot(key, total, sel, sh, [&](int pos, int v, uint32_t kk) {
      write_sel(a, b, q, pos, ix[v]);
      if (osc) osc[pos] = key_score(kk);
    }, per);
  } else {
    // many candidates (keys concentrated near the bound): select while streaming them
    auto get = [&](int p) -> uint32_t { return cand_key[at(p)]; };
    const Selection sel = block_radix_select(get, total, n, hist, sh);
    block_select_emit(get, total, n, sel, sh, [&](int pos, int p, uint32_t kk) {
      write_sel(a, b, q, pos, cand_idx[at(p)]);
      if (osc) osc[pos] = key_score(kk);
    });
  }
  for (int p = n + threadIdx.x; p < k; p += blockDim.x) {
    write_sel(a, b, q, p, -1);
    if (osc) osc[p] = 0.0f;
  }
  if (threadIdx.x == 0) a.topk_cnt[q] = n;
}

}  // namespace

// MFMA paths (indexer_mfma.hip)
bool indexer_fused_supported(int64_t Emax, int T, int n_hI, int cI, int k, int dt);
hipError_t launch_indexer_fused(const IndexerArgs& a, int64_t Emax, hipStream_t s);
bool indexer_mfma_supported(int T, int n_hI, int cI, int dt);
hipError_t launch_indexer_scores_mfma(const IndexerArgs& a, float* scores, int64_t ld,
                                      uint32_t* gmax, int64_t ng_ld, int gshift, hipStream_t s,
                                      const CompressArgs* ci);

bool indexer_fuses_compress(const IndexerPlan& p, const CompressArgs& ci) {
  // the scan runs (matrix-core scan, not the all-in-LDS prefill kernel) and the entry is a
  // short-window bf16 entry of 128 channels: 2 channels per lane of one wave
  const int npos = ci.overlap ? 2 * ci.m : ci.m;
  return p.mfma_scan && !p.fused && ci.in_dt == kBF16 && ci.c == 128 && npos <= 8;
}

IndexerPlan indexer_plan(int batch, int T, int64_t t0, int n_hI, int cI, int m, int k, int dt,
                         int policy, bool serving) {
  IndexerPlan p{};
  const int64_t Emax = (t0 + T) / m;
  p.ld = (Emax + 63) / 64 * 64;
  if (p.ld < 64) p.ld = 64;
  // register-resident tile stage: 4096-entry tiles (256 threads) while the merge stays at
  // most 8192 candidates per query, otherwise 16384-entry tiles (1024 threads)
  p.tile = 4096;
  if ((Emax + 4095) / 4096 * (int64_t)(k < 4096 ? k : 4096) > 8192) p.tile = 16384;
  if (k > p.tile) p.tile = (k + 4095) / 4096 * 4096;
  p.n_tiles = (int)((Emax + p.tile - 1) / p.tile);
  if (p.n_tiles < 1) p.n_tiles = 1;
  p.kc = k < p.tile ? k : p.tile;
  p.fused = policy == 0 && !serving && indexer_fused_supported(Emax, T, n_hI, cI, k, dt);
  p.mfma_scan = policy == 0 && indexer_mfma_supported(T, n_hI, cI, dt);
  if (p.fused) {
    p.score_bytes = p.cand_bytes = p.total = 0;
    return p;
  }
  p.score_bytes = ((size_t)batch * T * p.ld * sizeof(float) + 255) / 256 * 256;
  // one decode query over E >= 32 k entries: threshold filter with 2k .. 4k group maxima
  // (the largest groups that keep at least 2k of them: fewer reductions in the scan)
  p.filter = false;
  if (p.mfma_scan && T == 1 && Emax >= 32 * (int64_t)k && Emax <= 64 * (int64_t)kFiltSlice) {
    int gs = 0;
    while (gs < 4 && (Emax + (32 << gs) - 1) / (32 << gs) >= 2 * (int64_t)k) ++gs;
    const int64_t ng = (Emax + (16 << gs) - 1) / (16 << gs);
    if (ng <= kFiltGroups && ng >= 2 * (int64_t)k) {
      p.filter = true;
      p.gshift = gs;
      p.ng_ld = (ng + 63) / 64 * 64;
      p.n_slices = (int)((Emax + kFiltSlice - 1) / kFiltSlice);
    }
  }
  if (p.filter) {
    const size_t rows = (size_t)batch * T;
    const size_t gm = (rows * p.ng_ld * 4 + 255) / 256 * 256;
    const size_t cn = (rows * p.n_slices * 4 + 255) / 256 * 256;
    p.cand_bytes = gm + cn + rows * p.n_slices * kFiltSlice * 8;
  } else {
    p.cand_bytes = p.n_tiles > 1 ? (size_t)batch * T * p.n_tiles * p.kc * 8 : 0;
  }
  p.total = p.score_bytes + p.cand_bytes;
  return p;
}

hipError_t launch_indexer_topk(const IndexerArgs& a, const IndexerPlan& p, void* ws,
                               hipStream_t s, const CompressArgs* cfuse, const FrontArgs* front) {
  float* scores = reinterpret_cast<float*>(ws);
  uint32_t* ck = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) + p.score_bytes);
  int32_t* ci = reinterpret_cast<int32_t*>(ck + (size_t)a.batch * a.T * p.n_tiles * p.kc);
  const int64_t Emax = (a.t0 + a.T) / a.m;
  if (p.fused) return launch_indexer_fused(a, Emax, s);
  hipError_t err;
  if (p.filter) {
    // workspace after the scores: group maxima, slice counts, candidate keys and indices
    const size_t rows = (size_t)a.batch * a.T;
    char* w = reinterpret_cast<char*>(ws) + p.score_bytes;
    uint32_t* gmax = reinterpret_cast<uint32_t*>(w);
    w += (rows * p.ng_ld * 4 + 255) / 256 * 256;
    int* counts = reinterpret_cast<int*>(w);
    w += (rows * p.n_slices * 4 + 255) / 256 * 256;
    uint32_t* fkey = reinterpret_cast<uint32_t*>(w);
    int32_t* fidx = reinterpret_cast<int32_t*>(fkey + rows * p.n_slices * kFiltSlice);
    err = launch_indexer_scores_mfma(a, scores, p.ld, gmax, p.ng_ld, p.gshift, s, cfuse);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(topk_filter_kernel, dim3((unsigned)p.n_slices, (unsigned)a.T, (unsigned)a.batch),
                       dim3(256), 0, s, a, scores, p.ld, gmax, p.ng_ld, p.gshift, p.n_slices, counts,
                       fkey, fidx);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (!front) {
      hipLaunchKernelGGL(topk_final_kernel<0>, dim3((unsigned)a.T, (unsigned)a.batch), dim3(kFinalThreads),
                         0, s, a, p.n_slices, counts, fkey, fidx, FrontArgs{});
      return hipGetLastError();
    }
    if (a.T != 1) return hipErrorInvalidValue;
    const dim3 fgrid((unsigned)(1 + front->n_comp + front->n_prep), (unsigned)a.batch);
    if (front->gm == 64)
      hipLaunchKernelGGL(topk_final_kernel<64>, fgrid, dim3(kFinalThreads), 0, s, a, p.n_slices, counts,
                         fkey, fidx, *front);
    else if (front->gm == 32)
      hipLaunchKernelGGL(topk_final_kernel<32>, fgrid, dim3(kFinalThreads), 0, s, a, p.n_slices, counts,
                         fkey, fidx, *front);
    else if (front->gm == 16)
      hipLaunchKernelGGL(topk_final_kernel<16>, fgrid, dim3(kFinalThreads), 0, s, a, p.n_slices, counts,
                         fkey, fidx, *front);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (Emax > 0) {
    if (p.mfma_scan) {
      err = launch_indexer_scores_mfma(a, scores, p.ld, nullptr, 0, 0, s, cfuse);
    } else {
      dim3 grid((unsigned)a.T, (unsigned)((Emax + kScoreThreads - 1) / kScoreThreads),
                (unsigned)a.batch);
      const size_t shmem = ((size_t)a.n_hI * a.cI + a.n_hI) * sizeof(float);
      static bool attr_set = false;
      if (!attr_set) {
        hipFuncSetAttribute((const void*)index_scores_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)((16384 + 1024) * sizeof(float)));
        attr_set = true;
      }
      hipLaunchKernelGGL(index_scores_kernel, grid, dim3(kScoreThreads), shmem, s, a, scores, p.ld);
      err = hipGetLastError();
    }
    if (err != hipSuccess) return err;
  }
  const dim3 tgrid((unsigned)a.T, (unsigned)p.n_tiles, (unsigned)a.batch);
  if (p.tile == 4096)
    hipLaunchKernelGGL(topk_tile_reg_kernel<256>, tgrid, dim3(256), 0, s, a, scores, p.ld, p.n_tiles,
                       p.kc, ck, ci);
  else if (p.tile == 16384)
    hipLaunchKernelGGL(topk_tile_reg_kernel<1024>, tgrid, dim3(1024), 0, s, a, scores, p.ld, p.n_tiles,
                       p.kc, ck, ci);
  else
    hipLaunchKernelGGL(topk_tile_kernel, tgrid, dim3(256), 0, s, a, scores, p.ld, p.tile, p.n_tiles,
                       p.kc, ck, ci);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (p.n_tiles > 1) {
    const int64_t N = (int64_t)p.n_tiles * p.kc;
    const dim3 mgrid((unsigned)a.T, (unsigned)a.batch);
    if (N <= 4 * 1024)
      hipLaunchKernelGGL(topk_merge_reg_kernel<4>, mgrid, dim3(1024), 0, s, a, p.n_tiles, p.kc, ck, ci);
    else if (N <= 8 * 1024)
      hipLaunchKernelGGL(topk_merge_reg_kernel<8>, mgrid, dim3(1024), 0, s, a, p.n_tiles, p.kc, ck, ci);
    else if (N <= 16 * 1024)
      hipLaunchKernelGGL(topk_merge_reg_kernel<16>, mgrid, dim3(1024), 0, s, a, p.n_tiles, p.kc, ck, ci);
    else if (N <= 64 * 1024)
      hipLaunchKernelGGL(topk_merge_reg_kernel<64>, mgrid, dim3(1024), 0, s, a, p.n_tiles, p.kc, ck, ci);
    else
      hipLaunchKernelGGL(topk_merge_kernel, mgrid, dim3(1024), 0, s, a, p.n_tiles, p.kc, ck, ci);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace v4a
