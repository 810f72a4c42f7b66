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
  uint32_t kth;  // key of the K-th largest element (its bits under mask)
  int need_eq;   // how many elements equal to kth are taken (lowest indices first)
  uint32_t mask = 0xFFFFFFFFu;  // key bits the comparisons with kth use
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

// Inclusive prefix sum over the 64 lanes of a wave: shifts within 16-lane rows, then the
// row broadcasts of lanes 15 and 31 (no LDS round trip, unlike a shuffle).
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Bitwise AND and OR of x over the wave (row rotations, then the four row results),
// returned in every lane.
__device__ __forceinline__ void wave_and_or(uint32_t& a, uint32_t& o) {
  a &= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x128, 0xf, 0xf, false);  // row_ror:8
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x128, 0xf, 0xf, false);
  a &= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x124, 0xf, 0xf, false);  // row_ror:4
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x124, 0xf, 0xf, false);
  a &= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x122, 0xf, 0xf, false);  // row_ror:2
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x122, 0xf, 0xf, false);
  a &= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x121, 0xf, 0xf, false);  // row_ror:1
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x121, 0xf, 0xf, false);
  a = (uint32_t)__builtin_amdgcn_readlane((int)a, 0) & (uint32_t)__builtin_amdgcn_readlane((int)a, 16) &
      (uint32_t)__builtin_amdgcn_readlane((int)a, 32) & (uint32_t)__builtin_amdgcn_readlane((int)a, 48);
  o = (uint32_t)__builtin_amdgcn_readlane((int)o, 0) | (uint32_t)__builtin_amdgcn_readlane((int)o, 16) |
      (uint32_t)__builtin_amdgcn_readlane((int)o, 32) | (uint32_t)__builtin_amdgcn_readlane((int)o, 48);
}

// Exclusive prefix sum of v over the block in thread order; *total gets the sum.
// sh: LDS int[>= number of waves + 1].
__device__ __forceinline__ int block_excl_sum(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  const int incl = wave_incl_sum(v);
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

// Per executed pass: run-length atomics into one of three 256-bin histograms, one barrier,
// then every wave scans that histogram itself (no broadcast through LDS) and clears the
// histogram of the pass after next, which is thus cleared one barrier after its last
// readers and one barrier before its next writers: one barrier per pass.  Passes over
// digits that every key shares (common leading bits, found by one block-wide AND/OR) are
// skipped.  hist: LDS uint32[768].  per <= PER: elements per thread (thread t owns
// [t per, t per + per)); a smaller per spreads a short list over more waves.
template <int PER>
__device__ Selection reg_radix_select(const uint32_t (&key)[PER], int N, int K, uint32_t* hist,
                                      int* sh, int last_shift = 0, int per = PER) {
  (void)sh;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  const int base = threadIdx.x * per;
  uint32_t kand = 0xFFFFFFFFu, kor = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (j < per && base + j < N) {
      kand &= key[j];
      kor |= key[j];
    }
  }
  wave_and_or(kand, kor);
  uint32_t* slots = hist + 512;  // third histogram, first cleared by executed pass 0
  if (lane == 0) {
    slots[2 * wid] = kand;
    slots[2 * wid + 1] = kor;
  }
  for (int i = threadIdx.x; i < 512; i += blockDim.x) hist[i] = 0u;
  __syncthreads();
  uint32_t all_and = 0xFFFFFFFFu, all_or = 0u;
  for (int w = 0; w < nw; ++w) {
    all_and &= slots[2 * w];
    all_or |= slots[2 * w + 1];
  }
  const int common = (all_and ^ all_or) ? __builtin_clz(all_and ^ all_or) : 32;
  uint32_t prefix = 0, pmask = 0;
  int rem = K;
  // last_shift > 0 stops early: the result then holds only the key bits above last_shift
  // (kth = those bits of the K-th largest key, low bits zero; need_eq is not meaningful)
  int pass = 0;
  for (int shift = 24; shift >= last_shift; shift -= 8) {
    if (common >= 32 - shift) {
      // every key has this digit: the bucket is all of them
      prefix |= all_and & (255u << shift);
      pmask |= 255u << shift;
      continue;
    }
    uint32_t* h = hist + 256 * (pass % 3);
    uint32_t cur = 0u, run = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (j < per && base + j < N && (key[j] & pmask) == prefix) {
        const uint32_t d = (key[j] >> shift) & 255u;
        if (run != 0u && d != cur) {
          atomicAdd(&h[cur], run);
          run = 0u;
        }
        cur = d;
        ++run;
      }
    }
    if (run != 0u) atomicAdd(&h[cur], run);
    __syncthreads();
    // lane l holds bins 255 - 4 l .. 252 - 4 l (descending), so a prefix sum over the
    // lanes counts the elements in higher bins
    uint32_t cs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cs[j] = h[255 - 4 * lane - j];
    const uint32_t mine = cs[0] + cs[1] + cs[2] + cs[3];
    uint32_t above = (uint32_t)wave_incl_sum((int)mine) - mine;  // elements in bins > 255 - 4 l
    int hit_bin = -1;
    uint32_t hit_above = 0u, hit_count = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (above < (uint32_t)rem && above + cs[j] >= (uint32_t)rem) {
        hit_bin = 255 - 4 * lane - j;
        hit_above = above;
        hit_count = cs[j];
      }
      above += cs[j];
    }
    // exactly one lane holds the bin that contains the rem-th largest remaining key
    const uint64_t m = __ballot(hit_bin >= 0);
    const int src = m ? (int)__builtin_ctzll(m) : 0;  // (no lane only for K > N: misuse)
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane(hit_bin, src);
    rem -= __builtin_amdgcn_readlane((int)hit_above, src);
    prefix |= d << shift;
    pmask |= 255u << shift;
    // a full selection stops once the bin holds exactly the keys still needed: all of them
    // are taken whatever their lower digits (the set the remaining passes would give)
    const bool whole =
        last_shift == 0 && (uint32_t)__builtin_amdgcn_readlane((int)hit_count, src) == (uint32_t)rem;
    uint32_t* h2 = hist + 256 * ((pass + 2) % 3);
    for (int i = threadIdx.x; i < 256; i += blockDim.x) h2[i] = 0u;
    ++pass;
    if (whole) break;
  }
  __syncthreads();  // the last histogram is read before the caller reuses LDS
  return {prefix, rem, pmask};
}

// Selected elements before thread t and their placement: the selection is every key > kth
// plus the first need_eq keys == kth in element order, so the counts of keys > kth and
// == kth before the thread place every element (for PER <= 16 one block-wide scan of the
// two counts packed in 16-bit halves).  emit(pos, j, key) with j the register slot;
// positions ascend in element order.
template <int PER, class Emit>
__device__ void reg_select_emit_slot(const uint32_t (&key)[PER], int N, Selection sel, int* sh,
                                     Emit emit, int per = PER) {
  const int base = threadIdx.x * per;
  int ngt = 0, neq = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (j < per && base + j < N) {
      ngt += (key[j] & sel.mask) > sel.kth ? 1 : 0;
      neq += (key[j] & sel.mask) == sel.kth ? 1 : 0;
    }
  }
  int tot, gt_before, eq_before;
  if constexpr (PER <= 16) {
    // at most 16 x 1024 elements: both counts fit 16 bits (one scan)
    const uint32_t before = (uint32_t)block_excl_sum(ngt | (neq << 16), sh, &tot);
    gt_before = (int)(before & 0xFFFFu);
    eq_before = (int)(before >> 16);
  } else {
    eq_before = block_excl_sum(neq, sh, &tot);
    gt_before = block_excl_sum(ngt, sh, &tot);
  }
  int pos = gt_before + min(eq_before, sel.need_eq);
  int eq_seen = eq_before;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (j < per && base + j < N) {
      const uint32_t kk = key[j] & sel.mask;
      const bool gt = kk > sel.kth;
      const bool eq = kk == sel.kth && eq_seen < sel.need_eq;
      eq_seen += kk == sel.kth ? 1 : 0;
      if (gt || eq) emit(pos++, j, key[j]);
    }
  }
}

// As reg_select_emit_slot with emit(pos, i, key) given the element index i.
template <int PER, class Emit>
__device__ void reg_select_emit(const uint32_t (&key)[PER], int N, Selection sel, int* sh,
                                Emit emit) {
  const int base = threadIdx.x * PER;
  reg_select_emit_slot(key, N, sel, sh, [&](int pos, int j, uint32_t k) { emit(pos, base + j, k); });
}

}  // namespace v4a
