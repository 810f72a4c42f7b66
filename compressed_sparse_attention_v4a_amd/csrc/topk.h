// Block-wide exact top-k selection by radix select on order-preserving uint32
// keys, with ties broken towards the lower index, and an order-preserving
// compaction that emits the selected positions in ascending index order.
//
// Used by the indexer ("CSA And HCA: Definition, State, And Cost Model",
// section 3.1: TopK over the completed entries of each query).
#pragma once

#include "device_common.h"

namespace v4a {

struct Selection {
  uint32_t kth;  // key of the K-th largest element
  int need_eq;   // how many elements equal to kth are taken (lowest indices first)
};

// Exclusive prefix count of `flag` over the block in thread order; *total gets
// the block-wide count.  `sh` is LDS scratch of >= 2*nwaves ints.
__device__ __forceinline__ int block_excl_count(bool flag, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  const uint64_t b = __ballot(flag);
  const int in_wave = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) sh[wid] = __popcll(b);
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const int v = sh[i];
    before += (i < wid) ? v : 0;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return before + in_wave;
}

// Radix select of the K-th largest key among get(0..N-1), 1 <= K <= N.
// hist: LDS uint32[256]; sh: LDS int[>= 4].
template <class GetKey>
__device__ Selection block_radix_select(GetKey get, int N, int K, uint32_t* hist, int* sh) {
  uint32_t prefix = 0, pmask = 0;
  int rem = K;
  const int lane = threadIdx.x & 63;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
      const uint32_t key = get(i);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                     c3 = hist[4 * lane + 3];
      const uint32_t mine = c0 + c1 + c2 + c3;
      uint32_t suf = mine;  // inclusive suffix sum over lanes >= lane
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_down(suf, o, 64);
        if (lane + o < 64) suf += v;
      }
      uint32_t above = suf - mine;  // elements in bins >= 4*lane + 4
      const uint32_t cs[4] = {c0, c1, c2, c3};
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < (uint32_t)rem && above + cs[j] >= (uint32_t)rem) {
          sh[0] = 4 * lane + j;
          sh[1] = (int)above;
        }
        above += cs[j];
      }
    }
    __syncthreads();
    const uint32_t d = (uint32_t)sh[0];
    rem -= sh[1];
    prefix |= d << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  return {prefix, rem};
}

// Emit every selected element, in ascending index order: emit(pos, i, key).
// Selection = keys > kth, plus the first need_eq keys equal to kth.  K <= N.
template <class GetKey, class Emit>
__device__ void block_select_emit(GetKey get, int N, int K, Selection sel, int* sh, Emit emit) {
  int base_sel = 0, base_eq = 0;
  for (int i0 = 0; i0 < N && base_sel < K; i0 += blockDim.x) {
    const int i = i0 + threadIdx.x;
    const bool valid = i < N;
    const uint32_t key = valid ? get(i) : 0u;
    const bool gt = valid && key > sel.kth;
    const bool eq = valid && key == sel.kth;
    int eq_tot, sel_tot;
    const int eq_pre = block_excl_count(eq, sh, &eq_tot);
    const bool take = gt || (eq && base_eq + eq_pre < sel.need_eq);
    const int pos = block_excl_count(take, sh, &sel_tot);
    if (take) emit(base_sel + pos, i, key);
    base_eq += eq_tot;
    base_sel += sel_tot;
  }
}

// Emit all N elements in order (the case K >= N).
template <class GetKey, class Emit>
__device__ void block_emit_all(GetKey get, int N, Emit emit) {
  for (int i = threadIdx.x; i < N; i += blockDim.x) emit(i, i, get(i));
}

}  // namespace v4a
