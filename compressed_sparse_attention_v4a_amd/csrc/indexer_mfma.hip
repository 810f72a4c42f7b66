// Matrix-core lightning indexer ("CSA And HCA: Definition, State, And Cost
// Model", section 3.1):  I[t][s] = sum_h wI[t][h] * max(0, qI[t][h] . KI[s]) over
// the completed entries s < floor((t+1)/m), then TopK (ties to the lower index).
//
// Prefill form, bf16 operands, c^I = 128, heads in multiples of 64 (one pass per
// 64 heads is fused here for n_hI = 64):
//   * One workgroup = 4 consecutive queries, one per wave; they share every K^I
//     tile, which streams through LDS 64 entries at a time (double-buffered
//     direct global->LDS loads, 16-byte chunks XOR-swizzled by entry).
//   * S = Q K^T on v_mfma_f32_16x16x32_bf16 with heads as rows: each lane holds 16
//     (head, entry) products of one entry, so the ReLU * w head reduction is 16
//     in-register multiply-adds plus two cross-row shuffles per 16 entries.
//   * Scores never leave LDS: after the scan each wave runs an exact radix select
//     (4 x 8-bit passes, LDS histograms, ballot-based order-preserving compaction)
//     for its query and writes the selected entry indices in ascending order.
// Workgroups are issued longest-first (late queries see the most entries).
#include "compress_rows.h"
#include "device_common.h"
#include "internal.h"
#include "topk.h"

namespace v4a {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((address_space(3))) void* lds_void;

constexpr int kCI = 128;             // indexer key width
constexpr int kRowB = kCI * 2;       // 256 bytes per bf16 key
constexpr int kNE = 64;              // entries per K tile
constexpr int kQ = 4;                // queries per workgroup (one per wave)
constexpr int kHeads = 64;
constexpr int kCutSlack = 64;        // extra candidates a cut inside the stream may keep

// 16-byte chunk (of 16 per key) read by lane group g in k-step s (s < 4); the step
// index sits above the swizzle bits so per-step addresses are immediates.
__device__ __forceinline__ int kchunk(int s, int g) { return 8 * (s >> 1) + 2 * g + (s & 1); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 16x16 score tiles with heads as rows: lane (g, jj) holds heads 16 mt + 4 g + i of entry
// jj.  Returns sum_h w_h ReLU(S_h) over all 64 heads in every lane of column jj: four
// independent partial sums, then the four 16-lane rows are combined with the gfx950
// row-swap instructions (no LDS round trip).  ReLU is an integer maximum of the float bits
// with 0 (one instruction; negative values, -0 included, have negative bit patterns).
__device__ __forceinline__ float relu_weighted_sum(const f32x4 (&S)[4], const float (&w)[4][4]) {
  float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fmaf(w[mt][i], __int_as_float(max(__float_as_int(S[mt][i]), 0)), p[i]);
  float acc = (p[0] + p[1]) + (p[2] + p[3]);
  const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc), __float_as_uint(acc), false, false);
  acc = __uint_as_float(x32[0]) + __uint_as_float(x32[1]);  // rows r and r ^ 2
  const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc), __float_as_uint(acc), false, false);
  return __uint_as_float(x16[0]) + __uint_as_float(x16[1]);  // rows r and r ^ 1
}

// Radix select of the k-th largest of the keys held in registers by one wave: lane l
// holds the contiguous keys [l per, l per + per) of E (per <= PER; slots past per or E
// hold key 0, "absent", below every real key except the one NaN pattern whose key is 0).
// Passes over digits shared by every key (wave AND / OR) are skipped; the others count
// runs of equal digits before touching the histogram (the wave's own, ordered by the
// wave's in-order LDS operations) and find the bin with a DPP prefix sum.  The passes stop
// once the k-th key's bin holds at most slack keys more than are still needed; the whole
// bin is then taken.  On return the selection is: keys whose resolved digits
// (key & pmask) exceed kth, then the first need_eq keys equal to it in position order;
// kept = its size (k when slack = 0, at most k + slack otherwise).  Needs E > k.
template <int PER>
__device__ __forceinline__ void radix_kth(const uint32_t (&key)[PER], int E, int per, int k,
                                          int slack, uint32_t* hist, uint32_t& kth,
                                          uint32_t& pmask_out, int& need_eq, int& kept) {
  const int lane = threadIdx.x & 63;
  const int base = lane * per;
  uint32_t kand = 0xFFFFFFFFu, kor = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool v = j < per && base + j < E;
    kand &= v ? key[j] : 0xFFFFFFFFu;
    kor |= key[j];
  }
  wave_and_or(kand, kor);
  const int common = (kand ^ kor) ? __builtin_clz(kand ^ kor) : 32;
  const uint32_t n_absent = 64u * PER - (uint32_t)E;
  for (int i = lane; i < 256; i += 64) hist[i] = 0u;
  uint32_t prefix = 0, pmask = 0;
  int rem = k, take = -1;  // take >= 0: the whole bin of the k-th key is selected
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (common >= 32 - shift) {
      prefix |= kand & (255u << shift);
      pmask |= 255u << shift;
      continue;
    }
    uint32_t cur = 0u, run = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if ((key[j] & pmask) == prefix) {
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
    if (lane == 0 && prefix == 0u && n_absent) atomicSub(&hist[0], n_absent);
    __builtin_amdgcn_wave_barrier();
    uint32_t cs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cs[j] = hist[255 - 4 * lane - j];
    const uint32_t mine = cs[0] + cs[1] + cs[2] + cs[3];
    uint32_t above = (uint32_t)wave_incl_sum((int)mine) - mine;
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
    const uint64_t m = __ballot(hit_bin >= 0);
    const int src = m ? (int)__builtin_ctzll(m) : 0;
    prefix |= (uint32_t)__builtin_amdgcn_readlane(hit_bin, src) << shift;
    pmask |= 255u << shift;
    rem -= __builtin_amdgcn_readlane((int)hit_above, src);
    const int hc = __builtin_amdgcn_readlane((int)hit_count, src);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 4; ++j) hist[255 - 4 * lane - j] = 0u;  // the bins this lane read
    // the bin holds the keys still needed and at most slack more: all of them are
    // selected, whatever their lower digits (with slack = 0, the same set the remaining
    // passes would find)
    if (hc <= rem + slack) {
      take = hc;
      break;
    }
  }
  kth = prefix;
  pmask_out = pmask;
  need_eq = take >= 0 ? take : rem;
  kept = k - rem + need_eq;
}

// Output slot of each selected key of a lane (position order, ties to the lower
// position): calls emit(j, slot) for every selected register j.
template <int PER, typename F>
__device__ __forceinline__ void radix_emit(const uint32_t (&key)[PER], int E, int per, uint32_t kth,
                                           uint32_t pmask, int need_eq, F&& emit) {
  const int lane = threadIdx.x & 63;
  const int base = lane * per;
  int ngt = 0, neq = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool v = j < per && base + j < E;
    ngt += (v && (key[j] & pmask) > kth) ? 1 : 0;
    neq += (v && (key[j] & pmask) == kth) ? 1 : 0;
  }
  const int packed = ngt | (neq << 16);  // E <= 65535
  const int before = wave_incl_sum(packed) - packed;
  int pos = (before & 0xFFFF) + min(before >> 16, need_eq);
  int eq_seen = before >> 16;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool v = j < per && base + j < E;
    const bool gt = v && (key[j] & pmask) > kth;
    const bool eq = v && (key[j] & pmask) == kth && eq_seen < need_eq;
    eq_seen += (v && (key[j] & pmask) == kth) ? 1 : 0;
    if (gt || eq) {
      emit(j, pos);
      ++pos;
    }
  }
}

// Register form of the one-wave top-k for E <= 64 PER: lane l holds the contiguous keys
// [l per, l per + per), per = ceil(E / 64); radix_kth finds the k-th key and radix_emit
// places each lane's selected keys with one packed prefix sum of (keys > kth, keys ==
// kth).
template <int PER>
__device__ void wave_topk_reg(const float* sc, int E, int k, uint32_t* hist, int32_t* oidx,
                              float* osc, int32_t* ocnt) {
  const int lane = threadIdx.x & 63;
  const int n = E < k ? E : k;
  if (E <= k) {
    for (int i = lane; i < E; i += 64) {
      oidx[i] = i;
      if (osc) osc[i] = sc[i];
    }
  } else {
    const int per = (E + 63) / 64;
    const int base = lane * per;
    uint32_t key[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) key[j] = (j < per && base + j < E) ? score_key(sc[base + j]) : 0u;
    uint32_t kth, pmask;
    int need_eq;
    int kept;
    radix_kth<PER>(key, E, per, k, 0, hist, kth, pmask, need_eq, kept);
    radix_emit<PER>(key, E, per, kth, pmask, need_eq, [&](int j, int pos) {
      oidx[pos] = base + j;
      if (osc) osc[pos] = key_score(key[j]);
    });
  }
  for (int p = n + lane; p < k; p += 64) {
    oidx[p] = -1;
    if (osc) osc[p] = 0.0f;
  }
  if (lane == 0) *ocnt = n;
}

// Candidate buffer of one wave for long key lists: the n > k (key, entry) pairs in
// cp[0..n), in ascending entry order, are cut to the best ones (larger key first,
// ties to the lower entry), kept in ascending entry order in [0, kept).  slack = 0: the k
// best (kept = k).  slack > 0: the k best and at most slack more keys of the k-th key's
// radix bin (the passes stop once that bin is small enough).  Returns the smallest key
// kept: a later entry (higher index) whose key does not exceed it finds at least k kept
// keys as large with lower indices, so it can never be selected.  One wave; n <= 64 PER;
// cp 16-byte aligned.
template <int PER>
__device__ uint32_t wave_shrink_pairs(uint2* cp, int n, int k, int slack, uint32_t* hist, int& kept) {
  static_assert(PER % 2 == 0, "pairs are read two at a time");
  const int lane = threadIdx.x & 63;
  const int base = lane * PER;  // lane l holds pairs [l PER, l PER + PER): 16-byte reads
  uint32_t key[PER];
  int32_t ent[PER];
#pragma unroll
  for (int j = 0; j < PER; j += 2) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(cp + base + j);  // two (key, entry) pairs
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      key[j + i] = base + j + i < n ? q[2 * i] : 0u;
      ent[j + i] = (int32_t)q[2 * i + 1];
    }
  }
  uint32_t kth, pmask;
  int need_eq;
  radix_kth<PER>(key, n, PER, k, slack, hist, kth, pmask, need_eq, kept);
  uint32_t kmin = 0xFFFFFFFFu;
  // every lane has loaded its pairs before any slot is rewritten (slot <= position)
  __builtin_amdgcn_wave_barrier();
  radix_emit<PER>(key, n, PER, kth, pmask, need_eq, [&](int j, int pos) {
    cp[pos] = make_uint2(key[j], (uint32_t)ent[j]);
    kmin = min(kmin, key[j]);
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
  return kmin;
}

// CAPC == 0: every score of a query stays in LDS (CAP of them) and one register top-k
// runs after the scan.  CAPC > 0 (long key lists, any length): each wave keeps only a
// candidate buffer of CAPC (key, entry) pairs: a scored entry enters when its key
// exceeds the k-th key of the last cut (every entry before the first cut), and the
// buffer is cut back to its k best whenever the next chunk could overflow it.  The
// entries arrive in ascending order, so buffer order is entry order and ties keep going
// to the lower entry; the scores never reach HBM.
template <int CAP, int CAPC>
__global__ __launch_bounds__(256, (CAPC > 0 ? CAPC <= 1280 : CAP <= 2048) ? 2 : 1) void indexer_prefill_bf16_kernel(
    IndexerArgs a) {
  __shared__ __attribute__((aligned(1024))) char kbuf[2 * kNE * kRowB];
  __shared__ float sc[kQ][CAPC > 0 ? 1 : CAP];
  // candidate (key, entry) pairs, and one spare slot per lane past CAPC for the lanes
  // that do not enter
  __shared__ __attribute__((aligned(16))) uint2 cpair[kQ][CAPC > 0 ? CAPC + 64 : 1];
  __shared__ uint32_t hist[kQ][256];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, jj = lane & 15;
  const int nblk = (a.T + kQ - 1) / kQ;
  const int blk = nblk - 1 - (int)blockIdx.x;  // longest workgroups first
  const int b = blockIdx.y;
  const int j = blk * kQ + wv;                 // this wave's query row
  const bool qvalid = j < a.T;
  const int jlast = min(blk * kQ + kQ, a.T) - 1;
  const int64_t Ewg = (a.t0 + jlast + 1) / a.m;  // entries any query of the block sees
  const int64_t Eq = qvalid ? (a.t0 + j + 1) / a.m : 0;
  const char* kb = reinterpret_cast<const char*>(a.KI) + (int64_t)b * a.E_cap * kRowB;

  // K tile fill: 16 instructions of 4 entries each; wave wv issues 4 of them (entries
  // 4 (4 wv + r) .. + 3).  The loads are written out (M0 = LDS destination, formed from this
  // wave's part of the tile buffers plus an immediate; the tile's first key as the scalar
  // base and a fixed 32-bit offset per lane, or, on the last tile, the sequence's first key
  // and offsets clamped to the last visible entry) so that the compiler does not wait for
  // them before every later LDS read; the loop waits for them explicitly before the
  // barrier that publishes the tile.  The offsets stay below 2^31: the launcher takes this
  // kernel only for fewer than 2^23 visible entries.  Lanes of a load hold chunk position
  // (lane & 15) ^ (entry & 15) of entry 4 (4 wv + r) + (lane >> 4).
  const int ewg = (int)Ewg;
  const uint32_t lds_wave = (uint32_t)(uintptr_t)(lds_void)kbuf + (uint32_t)wv * 4096u;
  uint32_t lofs[4];  // per-lane offset of load r from the tile's first entry
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = 16 * wv + 4 * r + (lane >> 4);
    lofs[r] = ((uint32_t)e << 8) | ((uint32_t)((lane & 15) ^ (e & 15)) << 4);
  }
  // load r of this wave into buffer NB (M0 = its LDS address), from byte voff past base
  auto load = [lw = lds_wave](auto nb_t, auto r_t, const char* base, uint32_t voff) {
    constexpr int OFF = decltype(nb_t)::value * kNE * kRowB + decltype(r_t)::value * 1024;
    asm volatile("s_add_u32 m0, %0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3"
                 :: "s"(lw), "i"(OFF), "v"(voff), "s"(base) : "memory");
  };
  auto fill = [&](auto nb_t, int s0) {
    using R0 = std::integral_constant<int, 0>;
    using R1 = std::integral_constant<int, 1>;
    using R2 = std::integral_constant<int, 2>;
    using R3 = std::integral_constant<int, 3>;
    if (s0 + kNE <= ewg) {
      // the tile's first key as the scalar base: the lane offsets stay fixed
      const char* tb = kb + (size_t)s0 * kRowB;
      load(nb_t, R0{}, tb, lofs[0]);
      load(nb_t, R1{}, tb, lofs[1]);
      load(nb_t, R2{}, tb, lofs[2]);
      load(nb_t, R3{}, tb, lofs[3]);
    } else {
      // the last tile: rows past the visible entries load entry ewg - 1 (masked later)
      uint32_t v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int se = min(s0 + 16 * wv + 4 * r + (lane >> 4), ewg - 1);
        v[r] = ((uint32_t)se << 8) | (lofs[r] & 0xF0u);
      }
      load(nb_t, R0{}, kb, v[0]);
      load(nb_t, R1{}, kb, v[1]);
      load(nb_t, R2{}, kb, v[2]);
      load(nb_t, R3{}, kb, v[3]);
    }
  };
  const int nchunks = (int)((Ewg + kNE - 1) / kNE);
  if (nchunks > 0) fill(std::integral_constant<int, 0>{}, 0);

  // resident query rows (A operand, heads as rows) and head weights
  bf16x8 qa[4][4];  // [mt][ks]
  float wgt[4][4];  // [mt][i] -> head 16 mt + 4 g + i
  {
    const int jq = qvalid ? j : 0;
    const int64_t qrow = ((int64_t)b * a.T + jq) * a.n_hI;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.qI);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qa[mt][ks] = *reinterpret_cast<const bf16x8*>(qp + (qrow + 16 * mt + jj) * kCI + 8 * kchunk(ks, g));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) wgt[mt][i] = a.wI[qrow + 16 * mt + 4 * g + i];
  }
  // K fragment of k-step ks: chunk kchunk(ks, g) of entry jj, stored at chunk position
  // kchunk ^ jj.  A 16-byte LDS read serves 16 lanes per cycle (64 four-byte banks; lanes
  // grouped by bit 5 and the parity of bits 2-4 of the lane index), and with rows of 256
  // bytes the XOR with the whole entry index gives the 16 lanes of a group 16 different
  // chunk positions.
  int bb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) bb[ks] = jj * kRowB + ((kchunk(ks, g) ^ jj) << 4);
  float* scw = sc[wv];
  uint2* cpw = cpair[wv];
  int ncand = 0;            // candidates in this wave's buffer (CAPC > 0)
  uint32_t tau = 0u;        // a scored entry enters when its key exceeds tau ...
  bool have_tau = false;    // ... once the buffer has been cut at least once

  // The ReLU-weighted head sum of each 16-entry tile runs on the vector unit while the
  // matrix unit multiplies the next tile, so the accumulators of one tile wait in Sp (the
  // first tile's predecessor is a dummy).  A tile's in-lane part is 16 ReLU, 16 FMA and 1
  // add; the four 16-lane rows are then combined for two tiles at once (one row swap
  // exchanges the halves of both: the first tile of the pair ends in lanes 0..31, the
  // second in lanes 32..63), and the pair's 32 scores are stored or compacted by one set
  // of instructions.  At 64 vector instructions per tile the vector unit would take as
  // long as the tile's 16 MFMAs.
  f32x4 Sp[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) Sp[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float acc_a = 0.0f;  // in-lane head sum of the first tile of the pending pair
  // this lane's entry within a pair: lanes 0..15 the first tile, 32..47 the second
  // (lanes 16..31 and 48..63 hold copies and never store)
  const int eoff = jj + 16 * (lane >> 5);
  const uint32_t elim = (lane & 16) ? 0u : (uint32_t)Eq;
  auto inlane = [&]() -> float {
    float p[2] = {0.0f, 0.0f};  // two chains of 8: one add to combine
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p[i & 1] = fmaf(wgt[mt][i], __int_as_float(max(__float_as_int(Sp[mt][i]), 0)), p[i & 1]);
    return p[0] + p[1];
  };
  // the pair whose first entry is e0 (negative for the dummy pair before entry 0, which
  // the unsigned comparison with elim rejects)
  auto flush_pair = [&](float acc_b, int e0) {
    const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc_a), __float_as_uint(acc_b), false, false);
    const float t = __uint_as_float(x32[0]) + __uint_as_float(x32[1]);  // rows r and r ^ 2
    const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    const float u = __uint_as_float(x16[0]) + __uint_as_float(x16[1]);  // rows r and r ^ 1
    const uint32_t e = (uint32_t)(e0 + eoff);
    if constexpr (CAPC == 0) {
      if (e < elim) scw[e] = u;
    } else {
      // the pair's entries lie in ascending order over the ballot's lanes: compaction.
      // The order key of score_key without its fold of -0 into +0: u is never -0 (every
      // head sum starts from +0, and an exact zero sum rounds to +0).
      const uint32_t ub = __float_as_uint(u);
      const uint32_t key = ub ^ ((uint32_t)((int32_t)ub >> 31) | 0x80000000u);
      // (bitwise: both masks come from compares, with no branch between them)
      const bool pass = (e < elim) & (!have_tau | (key > tau));
      const uint64_t bm = __ballot(pass);
      // every lane stores: a lane that does not enter writes its own spare slot past CAPC
      const int pos = pass ? ncand + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u))
                           : CAPC + lane;
      cpw[pos] = make_uint2(key, e);
      ncand += __popcll(bm);
    }
  };
  // cut the buffer back to its best entries: inside the loop (whenever the next two
  // chunks could overflow it) to the k best and at most kCutSlack more, which stops the
  // radix passes early; after the loop to exactly the k best
  auto cut = [&](int slack) {
    if constexpr (CAPC > 0) {
      if (ncand > a.k) {
        int kept;
        tau = wave_shrink_pairs<CAPC / 64>(cpw, ncand, a.k, slack, hist[wv], kept);
        have_tau = true;
        ncand = kept;
      }
    }
  };
  // chunk c lives in buffer c & 1; BUF is a compile-time copy of it, so that buffer
  // offsets are immediates of the LDS instructions
  auto chunk = [&](int c, auto buf_t) {
    constexpr int BUF = decltype(buf_t)::value;
    const char* buf = kbuf + BUF * (kNE * kRowB);
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (c + 1 < nchunks) fill(std::integral_constant<int, 1 - BUF>{}, (c + 1) * kNE);
    __builtin_amdgcn_sched_barrier(0);
    // K fragments of entry tile et + 1 are read while tile et is multiplied; the four head
    // tiles are independent accumulation chains, interleaved k-step by k-step
    auto kread = [&](int et, int ks) {
      return *reinterpret_cast<const bf16x8*>(buf + bb[ks] + et * 16 * kRowB);
    };
    bf16x8 kv[2][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kv[0][ks] = kread(0, ks);
#pragma unroll
    for (int et = 0; et < 4; ++et) {
      if (et + 1 < 4) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kv[(et + 1) & 1][ks] = kread(et + 1, ks);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x4 S[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) S[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          S[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][ks], kv[et & 1][ks], S[mt], 0, 0, 0);
      }
      // tile 4 c + et - 1 waits in Sp: the first of a pair (et odd) keeps its in-lane
      // sum, the second (et even) completes the pair
      if (et & 1) {
        acc_a = inlane();
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two vector ALU instructions
        }
      } else {
        flush_pair(inlane(), kNE * c + 16 * et - 32);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three vector ALU instructions
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) Sp[mt] = S[mt];
    }
  };
  for (int c = 0; c < nchunks; c += 2) {
    // the next two chunks (at most 2 kNE entries) must fit in the candidate buffer
    if constexpr (CAPC > 0) {
      if (ncand > CAPC - 2 * kNE) cut(kCutSlack);
    }
    chunk(c, std::integral_constant<int, 0>{});
    if (c + 1 < nchunks) chunk(c + 1, std::integral_constant<int, 1>{});
  }
  flush_pair(inlane(), kNE * nchunks - 32);  // the last pair (a chunk holds two)

  // per-query top-k by its own wave (no workgroup barrier needed from here on)
  if (qvalid) {
    const int64_t q = (int64_t)b * a.T + j;
    if constexpr (CAPC == 0) {
      wave_topk_reg<CAP / 64>(scw, (int)Eq, a.k, hist[wv], a.topk_idx + q * a.k,
                              a.topk_score ? a.topk_score + q * a.k : nullptr, a.topk_cnt + q);
    } else {
      cut(0);
      // ncand = min(k, Eq): every entry entered before the first cut, k stay after it
      int32_t* oi = a.topk_idx + q * a.k;
      float* os = a.topk_score ? a.topk_score + q * a.k : nullptr;
      for (int p = lane; p < a.k; p += 64) {
        const bool v = p < ncand;
        const uint2 pr = v ? cpw[p] : make_uint2(0u, 0u);
        oi[p] = v ? (int32_t)pr.y : -1;
        if (os) os[p] = v ? key_score(pr.x) : 0.0f;
      }
      if (lane == 0) a.topk_cnt[q] = ncand;
    }
  }
}


// ---------------------------------------------------------------------------
// Scan form for long key lists (decode, or prefill beyond the fused capacity):
// one workgroup scores one query against 1024 consecutive entries, streaming the
// keys from HBM straight into MFMA operand registers (each key byte is used by
// exactly one wave, so no LDS), and writes float32 scores for the two-stage
// top-k kernels.
//   FP8 E4M3 : v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales; the
//              per-row scales are positive, so I = sK_s * sum_h (w_h sQ_h) ReLU(raw).
//   MXFP4    : the same instruction with E2M1 operands and the E8M0 block scales
//              of both operands applied by the hardware, one scale per lane.
//   BF16     : v_mfma_f32_16x16x32_bf16, four k-steps.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int kScanEntries = 1024;  // per workgroup (4 waves x 16 tiles x 16 entries)
constexpr int kScanTiles = kScanEntries / 4 / 16;  // 16-entry tiles per wave

// GS >= 0: also writes gmax, per query the maximum order key (score_key) of every group of
// 16 << GS consecutive entries, for the threshold filter of the decode top-k.
// ci.out set (decode step, bf16 tails, c^I = 128): the index entry that sequence b's new
// token completes, entry E - 1, is compressed here by the wave whose entries include it,
// before that wave's first key load, instead of by a launch the scan would wait for.  The
// layout of 2 channels per lane gives the same bits as the compressor's (see
// compress_rows_body).
template <int DT, int GS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void indexer_scan_kernel(
    IndexerArgs a, float* scores, int64_t ld, uint32_t* gmax, int64_t ng_ld, CompressArgs ci) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, jj = lane & 15;
  const int j = blockIdx.y, b = blockIdx.z;
  const int64_t t = query_pos(a, b, j);
  const int64_t E = (t + 1) / a.m;
  const int64_t e0 = (int64_t)blockIdx.x * kScanEntries + wv * (kScanEntries / 4);
  if (e0 >= E) return;
  if (ci.out) {
    const SlotEntry se = slot_entry(ci, b, 0);
    // no wait for the stores: this wave's later load of the row follows them in program
    // order to the same addresses, which one wave's memory operations keep
    if (se.emit && se.i >= e0 && se.i < e0 + kScanEntries / 4) compress_rows_body<uint16_t, 64, 2>(ci, 0, b, lane);
  }
  const int64_t q = (int64_t)b * a.T + j;
  const int64_t qrow = q * kHeads;
  float wq[4][4];  // w_h (times the FP8 row scale of q): head 16 mt + 4 g + i
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * mt + 4 * g + i;
      float w = a.wI[qrow + h];
      if (DT == kFP8) w *= reinterpret_cast<const float*>(a.qI_scale)[qrow + h];
      wq[mt][i] = w;
    }
  // query operand: lane (g, jj) holds head 16 mt + jj, k-block g (32 elements)
  i32x8 qa[4];
  int qs[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int64_t h = qrow + 16 * mt + jj;
    if (DT == kFP8) {
      const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.qI) + h * kCI + 32 * g);
      const uint4 x0 = p[0], x1 = p[1];
      qa[mt] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      qs[mt] = 127;
    } else if (DT == kMXFP4) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.qI) + h * (kCI / 2) + 16 * g);
      qa[mt] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, 0, 0, 0, 0};
      qs[mt] = reinterpret_cast<const uint8_t*>(a.qI_scale)[h * (kCI / 32) + g];
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.qI) + h * kCI + 32 * g);
      const uint4 x0 = p[0], x1 = p[1];  // channels 32 g .. 32 g + 15 (two k-steps' worth)
      const uint4* p2 = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.qI) + h * kCI + 32 * g + 16);
      const uint4 x2 = p2[0], x3 = p2[1];
      // bf16: k-step s uses channels 32 g + 8 s .. +7 of this lane's 32-channel block
      qa[mt] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      qs[mt] = (int)0;
      (void)x2; (void)x3;
    }
  }
  i32x8 qa_hi[4];  // bf16 only: channels 32 g + 16 .. 32 g + 31
  if (DT == kBF16) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int64_t h = qrow + 16 * mt + jj;
      const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.qI) + h * kCI + 32 * g + 16);
      const uint4 x0 = p[0], x1 = p[1];
      qa_hi[mt] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }
  }
  const uint8_t* kb = reinterpret_cast<const uint8_t*>(a.KI);
  float* srow = scores + q * ld;
  const int64_t qg = q * ng_ld;  // this query's group maxima
  uint32_t gacc = 0u;
  // The wave's 16 tiles go in batches: every key load of a batch is issued before its
  // first MFMA, so a wave waits for four (MXFP4: two) memory round trips instead of one per tile (the
  // compiler, left alone, serialises load -> MFMA per tile).  Four FP8 (eight MXFP4) tiles
  // are 32 key VGPRs, which keeps the kernel within 128 VGPRs, i.e. four waves per SIMD:
  // the whole decode grid is resident at once.  Entries past E read the last valid row (a cache
  // hit) and are not stored.
  constexpr int kB = DT == kBF16 ? 1 : DT == kFP8 ? 4 : 8;  // tiles per batch
  constexpr int kW = DT == kBF16 ? 4 : DT == kFP8 ? 2 : 1;  // 16-byte key loads per lane and tile
#pragma unroll
  for (int b0 = 0; b0 < kScanTiles; b0 += kB) {
    float res[kB];
    uint4 kx[kB][kW];
    float ksf[kB];
    int ksc[kB];
#pragma unroll
    for (int t = 0; t < kB; ++t) {
      int64_t s = e0 + 16 * (b0 + t) + jj;
      if (s >= E) s = E - 1;
      const int64_t row = cache_row(a.seq, a.E_cap, b, s);
      if (DT == kFP8) {
        const uint4* p = reinterpret_cast<const uint4*>(kb + row * kCI + 32 * g);
        kx[t][0] = p[0];
        kx[t][1] = p[1];
        ksf[t] = reinterpret_cast<const float*>(a.KI_scale)[row];
      } else if (DT == kMXFP4) {
        kx[t][0] = *reinterpret_cast<const uint4*>(kb + row * (kCI / 2) + 16 * g);
        ksc[t] = reinterpret_cast<const uint8_t*>(a.KI_scale)[row * (kCI / 32) + g];
      } else {
        const uint16_t* kr = reinterpret_cast<const uint16_t*>(kb) + row * kCI + 32 * g;
        kx[t][0] = reinterpret_cast<const uint4*>(kr)[0];
        kx[t][1] = reinterpret_cast<const uint4*>(kr)[1];
        kx[t][2] = reinterpret_cast<const uint4*>(kr + 16)[0];
        kx[t][3] = reinterpret_cast<const uint4*>(kr + 16)[1];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kB; ++t) {
      f32x4 S[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) S[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      float ks = 1.0f;
      if (DT == kFP8) {
        const uint4 x0 = kx[t][0], x1 = kx[t][1];
        const i32x8 kv = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        ks = ksf[t];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          S[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[mt], kv, S[mt], 0, 0, 0, 127, 0, 127);
      } else if (DT == kMXFP4) {
        const uint4 x0 = kx[t][0];
        const i32x8 kv = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, 0, 0, 0, 0};
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          S[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[mt], kv, S[mt], 4, 4, 0, qs[mt], 0, ksc[t]);
      } else {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const bf16x8 kv = __builtin_bit_cast(bf16x8, kx[t][st]);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            const i32x8 src = st < 2 ? qa[mt] : qa_hi[mt];
            const uint4 qq = (st & 1) ? uint4{(unsigned)src[4], (unsigned)src[5], (unsigned)src[6], (unsigned)src[7]}
                                      : uint4{(unsigned)src[0], (unsigned)src[1], (unsigned)src[2], (unsigned)src[3]};
            S[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qq), kv, S[mt], 0, 0, 0);
          }
        }
      }
      // every lane of column jj holds the full weighted sum after the row reductions
      res[t] = relu_weighted_sum(S, wq) * ks;
    }
    if (kB % 4 == 0) {
      // lane group g stores tiles b0 + g, b0 + g + 4, ...: one instruction writes 64
      // consecutive scores
#pragma unroll
      for (int u = 0; u < kB / 4; ++u) {
        // a bit-mask select: written as a conditional chain, the compiler indexed res[] by g
        // through scratch memory (a store and a dependent load per batch)
        uint32_t v_bits = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) v_bits |= __float_as_uint(res[4 * u + i]) & (0u - (uint32_t)(g == i));
        const float v = __uint_as_float(v_bits);
        const int64_t s = e0 + 16 * (b0 + 4 * u + g) + jj;
        if (s < E) srow[s] = v;
      }
    } else {
#pragma unroll
      for (int t = 0; t < kB; ++t) {
        const int64_t s = e0 + 16 * (b0 + t) + jj;
        if (g == 0 && s < E) srow[s] = res[t];
      }
    }
    if constexpr (GS >= 0) {
      // group maxima of the order keys: a lane keeps the maximum of its column over the
      // group's tiles; at the group's last tile the 16 columns of a row (every row holds the
      // same values) are reduced by row rotations.  Groups never straddle waves.
#pragma unroll
      for (int t = 0; t < kB; ++t) {
        const int tw = b0 + t;
        const int64_t s = e0 + 16 * tw + jj;
        gacc = max(gacc, s < E ? score_key(res[t]) : 0u);
        if (((tw + 1) & ((1 << GS) - 1)) == 0) {
          uint32_t key = gacc;
          key = max(key, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)key, 0x128, 0xf, 0xf, false));
          key = max(key, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)key, 0x124, 0xf, 0xf, false));
          key = max(key, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)key, 0x122, 0xf, 0xf, false));
          key = max(key, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)key, 0x121, 0xf, 0xf, false));
          const int64_t grp = (e0 / 16 + tw) >> GS;  // e0 is a multiple of 256
          if (lane == 0 && (grp << (4 + GS)) < E) gmax[qg + grp] = key;
          gacc = 0u;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace

// The fused prefill kernel covers bf16 keys of 128 channels and 64 heads: with all
// scores in LDS up to 4096 visible entries per query, with the streaming candidate
// buffer beyond that (k <= 1024; multi-query chunks, T > 1), for fewer than 2^23 visible
// entries (32-bit key offsets).
bool indexer_fused_supported(int64_t Emax, int T, int n_hI, int cI, int k, int dt) {
  if (dt != kBF16 || cI != kCI || n_hI != kHeads || Emax >= ((int64_t)1 << 23)) return false;
  return Emax <= 4096 || (T > 1 && k <= 1024);
}

hipError_t launch_indexer_fused(const IndexerArgs& a, int64_t Emax, hipStream_t s) {
  const unsigned nblk = (unsigned)((a.T + kQ - 1) / kQ);
  const dim3 grid(nblk, (unsigned)a.batch);
  // every score in LDS up to 2048 entries; beyond that the streaming buffer (two
  // workgroups per CU) is faster than the 4096-score form (one), which serves only single
  // queries and k > 1024
  if (Emax <= 2048)
    hipLaunchKernelGGL((indexer_prefill_bf16_kernel<2048, 0>), grid, dim3(256), 0, s, a);
  else if (Emax <= 4096 && (a.T == 1 || a.k > 1024))
    hipLaunchKernelGGL((indexer_prefill_bf16_kernel<4096, 0>), grid, dim3(256), 0, s, a);
  else if (a.k <= 512)
    hipLaunchKernelGGL((indexer_prefill_bf16_kernel<0, 1280>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((indexer_prefill_bf16_kernel<0, 2560>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

bool indexer_mfma_supported(int T, int n_hI, int cI, int dt) {
  (void)T;
  return n_hI == kHeads && cI == kCI && (dt == kFP8 || dt == kMXFP4 || dt == kBF16);
}

hipError_t launch_indexer_scores_mfma(const IndexerArgs& a, float* scores, int64_t ld,
                                      uint32_t* gmax, int64_t ng_ld, int gshift, hipStream_t s,
                                      const CompressArgs* ci) {
  CompressArgs cz{};
  if (ci) cz = *ci;  // cz.out == nullptr: no fused compression
  const int64_t Emax = (a.t0 + a.T) / a.m;
  dim3 grid((unsigned)((Emax + kScanEntries - 1) / kScanEntries), (unsigned)a.T, (unsigned)a.batch);
  // GS template: the group size of the optional group maxima (-1: none)
#define V4A_SCAN(gs)                                                                              \
  do {                                                                                           \
    if (a.dt == kFP8)                                                                            \
      hipLaunchKernelGGL((indexer_scan_kernel<kFP8, gs>), grid, dim3(256), 0, s, a, scores, ld,  \
                         gmax, ng_ld, cz);                                                       \
    else if (a.dt == kMXFP4)                                                                     \
      hipLaunchKernelGGL((indexer_scan_kernel<kMXFP4, gs>), grid, dim3(256), 0, s, a, scores, ld, \
                         gmax, ng_ld, cz);                                                       \
    else                                                                                         \
      hipLaunchKernelGGL((indexer_scan_kernel<kBF16, gs>), grid, dim3(256), 0, s, a, scores, ld, \
                         gmax, ng_ld, cz);                                                       \
  } while (0)
  if (!gmax) V4A_SCAN(-1);
  else if (gshift == 0) V4A_SCAN(0);
  else if (gshift == 1) V4A_SCAN(1);
  else if (gshift == 2) V4A_SCAN(2);
  else if (gshift == 3) V4A_SCAN(3);
  else V4A_SCAN(4);
#undef V4A_SCAN
  return hipGetLastError();
}

}  // namespace v4a
