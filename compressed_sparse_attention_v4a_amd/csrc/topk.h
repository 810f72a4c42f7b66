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

// ---- register-resident selection -----------------------------------------------
// Thread t owns the PER contiguous elements [t * PER, t * PER + PER) of a list of N keys
// (elements >= N are absent), loaded into registers once.  The radix passes then read
// registers only, and each thread counts runs of equal digits before touching the LDS
// histogram (keys still in play are concentrated in few bins, where plain per-element
// atomics would serialise on one address).  Emission needs two block-wide prefix counts
// and keeps ascending index order with ties to the lower index.

// Exclusive prefix sum of v over the block in thread order; *total gets the sum.
// sh: LDS int[>= number of waves + 1].
__device__ __forceinline__ int block_excl_sum(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  __syncthreads();
  if (lane == 63) sh[wid] = incl;
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int x = sh[w];
    before += w < wid ? x : 0;
    tot += x;
  }
  *total = tot;
  return before + incl - v;
}

template <int PER>
__device__ Selection reg_radix_select(const uint32_t (&key)[PER], int N, int K, uint32_t* hist,
                                      int* sh) {
  const int lane = threadIdx.x & 63;
  const int base = threadIdx.x * PER;
  uint32_t prefix = 0, pmask = 0;
  int rem = K;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0u;
    __syncthreads();
    uint32_t cur = 0u, run = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (base + j < N && (key[j] & pmask) == prefix) {
        const uint32_t d = (key[j] >> shift) & 255u;
        if (run != 0u && d != cur) {
          atomicAdd(&hist[cur], run);
          run = 0u;
        }
        cur = d;
        ++run;
      }
    }
    if (run != 0u) atomicAdd(&hist[cur], run);
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

// Emit the selection (keys > kth, then the first need_eq keys == kth): emit(pos, i, key)
// with pos ascending in element index.  sh: LDS int[>= number of waves + 1].
template <int PER, class Emit>
__device__ void reg_select_emit(const uint32_t (&key)[PER], int N, Selection sel, int* sh,
                                Emit emit) {
  const int base = threadIdx.x * PER;
  int ngt = 0, neq = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (base + j < N) {
      ngt += key[j] > sel.kth ? 1 : 0;
      neq += key[j] == sel.kth ? 1 : 0;
    }
  }
  int tot;
  const int eq_before = block_excl_sum(neq, sh, &tot);
  const int take_eq = max(0, min(neq, sel.need_eq - eq_before));
  int pos = block_excl_sum(ngt + take_eq, sh, &tot);
  int eq_seen = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (base + j < N) {
      const bool gt = key[j] > sel.kth;
      const bool eq = key[j] == sel.kth && eq_seen < take_eq;
      eq_seen += key[j] == sel.kth ? 1 : 0;
      if (gt || eq) emit(pos++, base + j, key[j]);
    }
  }
}

}  // namespace v4a
