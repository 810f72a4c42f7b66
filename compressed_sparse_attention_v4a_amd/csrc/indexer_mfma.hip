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
#include "device_common.h"
#include "internal.h"
#include "topk.h"

namespace v4a {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((address_space(3))) void* lds_void;

constexpr int kCI = 128;             // indexer key width
constexpr int kRowB = kCI * 2;       // 256 bytes per bf16 key
constexpr int kNE = 64;              // entries per K tile
constexpr int kQ = 4;                // queries per workgroup (one per wave)
constexpr int kHeads = 64;

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

// Register form of the one-wave top-k for E <= 64 PER: lane l holds the contiguous keys
// [l per, l per + per), per = ceil(E / 64).  Passes over digits shared by every key
// (wave AND / OR) are skipped; the others count runs of equal digits before touching the
// histogram (the wave's own, ordered by the wave's in-order LDS operations) and find the
// bin with a DPP prefix sum.  Emission places each lane's run with one packed prefix sum
// of (keys > kth, keys == kth).  The passes stop once the k-th key's bin holds exactly the
// keys still needed.  Same result as wave_topk.
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
    // slots past the lane's range or past E hold key 0 ("absent"): below every real key
    // except the one NaN pattern whose key is 0, so the passes need no per-slot validity;
    // the absent keys land in bin 0 while the prefix is 0 and are subtracted there
    uint32_t key[PER];
    uint32_t kand = 0xFFFFFFFFu, kor = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const bool v = j < per && base + j < E;
      key[j] = v ? score_key(sc[base + j]) : 0u;
      kand &= v ? key[j] : 0xFFFFFFFFu;
      kor |= key[j];
    }
    wave_and_or(kand, kor);
    const int common = (kand ^ kor) ? __builtin_clz(kand ^ kor) : 32;
    const uint32_t n_absent = 64u * PER - (uint32_t)E;
    for (int i = lane; i < 256; i += 64) hist[i] = 0u;
    uint32_t prefix = 0, pmask = 0;
    int rem = k;
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
      const bool whole = (uint32_t)__builtin_amdgcn_readlane((int)hit_count, src) == (uint32_t)rem;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < 4; ++j) hist[255 - 4 * lane - j] = 0u;  // the bins this lane read
      // the bin holds exactly the keys still needed: all of them are selected, whatever
      // their lower digits (the same set the remaining passes would find)
      if (whole) break;
    }
    // selection on the resolved digits: keys above the prefix, then the first rem keys equal
    // to it in index order (all of them when the passes stopped early)
    const uint32_t kth = prefix;
    const int need_eq = rem;
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
        oidx[pos] = base + j;
        if (osc) osc[pos] = key_score(key[j]);
        ++pos;
      }
    }
  }
  for (int p = n + lane; p < k; p += 64) {
    oidx[p] = -1;
    if (osc) osc[p] = 0.0f;
  }
  if (lane == 0) *ocnt = n;
}

// Exact top-k of one query over its scores sc[0..E) by one wave; writes the
// selected indices in ascending order, -1 padding, the count and the scores.
__device__ void wave_topk(const float* sc, int E, int k, uint32_t* hist, int* sh, int32_t* oidx,
                          float* osc, int32_t* ocnt) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = (1ull << lane) - 1ull;
  const int n = E < k ? E : k;
  if (E <= k) {
    for (int i = lane; i < E; i += 64) {
      oidx[i] = i;
      if (osc) osc[i] = sc[i];
    }
  } else {
    uint32_t prefix = 0, pmask = 0;
    int rem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = lane; i < 256; i += 64) hist[i] = 0u;
      __builtin_amdgcn_wave_barrier();
      for (int i = lane; i < E; i += 64) {
        const uint32_t key = score_key(sc[i]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __builtin_amdgcn_wave_barrier();
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                     c3 = hist[4 * lane + 3];
      const uint32_t mine = c0 + c1 + c2 + c3;
      uint32_t suf = mine;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_down(suf, o, 64);
        if (lane + o < 64) suf += v;
      }
      uint32_t above = suf - mine;
      const uint32_t cs[4] = {c0, c1, c2, c3};
      int found_d = -1, found_above = 0;
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        if (above < (uint32_t)rem && above + cs[q] >= (uint32_t)rem) {
          found_d = 4 * lane + q;
          found_above = (int)above;
        }
        above += cs[q];
      }
      const uint64_t who = __ballot(found_d >= 0);
      const int src = __ffsll((unsigned long long)who) - 1;
      const int d = __shfl(found_d, src, 64);
      const int ab = __shfl(found_above, src, 64);
      prefix |= (uint32_t)d << shift;
      pmask |= 255u << shift;
      rem -= ab;
    }
    const uint32_t kth = prefix;
    const int need_eq = rem;
    int base_sel = 0, base_eq = 0;
    for (int i0 = 0; i0 < E && base_sel < k; i0 += 64) {
      const int i = i0 + lane;
      const bool valid = i < E;
      const float s = valid ? sc[i] : 0.0f;
      const uint32_t key = valid ? score_key(s) : 0u;
      const bool gt = valid && key > kth;
      const bool eq = valid && key == kth;
      const uint64_t beq = __ballot(eq);
      const int eq_pre = __popcll(beq & lt);
      const bool take = gt || (eq && base_eq + eq_pre < need_eq);
      const uint64_t bt = __ballot(take);
      if (take) {
        const int pos = base_sel + __popcll(bt & lt);
        oidx[pos] = i;
        if (osc) osc[pos] = s;
      }
      base_eq += __popcll(beq);
      base_sel += __popcll(bt);
    }
  }
  for (int p = n + lane; p < k; p += 64) {
    oidx[p] = -1;
    if (osc) osc[p] = 0.0f;
  }
  if (lane == 0) *ocnt = n;
  (void)sh;
}

template <int CAP>
__global__ __launch_bounds__(256, CAP <= 2048 ? 2 : 1) void indexer_prefill_bf16_kernel(IndexerArgs a) {
  __shared__ __attribute__((aligned(1024))) char kbuf[2 * kNE * kRowB];
  __shared__ float sc[kQ][CAP];
  __shared__ uint32_t hist[kQ][256];
  __shared__ int shw[kQ][4];

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

  // K tile fill: 16 instructions of 4 entries each; wave wv issues 4 of them.  The loads
  // are written out (M0 = LDS destination, per-lane 64-bit source address) so that the
  // compiler does not wait for them before every later LDS read; the loop waits for them
  // explicitly before the barrier that publishes the tile.
  auto fill = [&](char* buf, int64_t s0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ins = 4 * wv + r;          // entries 4 ins .. 4 ins + 3
      const int e = 4 * ins + (lane >> 4);
      int64_t se = s0 + e;
      if (se >= Ewg) se = Ewg - 1;         // padding rows: any visible entry (masked later)
      const int ch = (lane & 15) ^ (e & 7);
      const char* src = kb + se * kRowB + ch * 16;
      const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void)(buf + ins * 1024);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   :: "s"(m0), "v"(src) : "memory");
    }
  };
  const int nchunks = (int)((Ewg + kNE - 1) / kNE);
  if (nchunks > 0) fill(kbuf, 0);

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
  const int bb0 = jj * kRowB + (((2 * g) ^ (jj & 7)) << 4);
  const int bb1 = jj * kRowB + (((2 * g + 1) ^ (jj & 7)) << 4);
  float* scw = sc[wv];

  // The ReLU-weighted head sum of each 16-entry tile runs on the vector unit while the
  // matrix unit multiplies the next tile (three vector instructions per MFMA), so the
  // accumulators of one tile wait in Sp; the first tile's predecessor is a dummy with no
  // entry to store.
  f32x4 Sp[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) Sp[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  int64_t sp = -1;  // entry of this lane's previous tile (-1: none)
  auto reduce_prev = [&]() {
    const float acc = relu_weighted_sum(Sp, wgt);
    if (g == 0 && sp >= 0 && sp < Eq) scw[sp] = acc;
  };
  for (int c = 0; c < nchunks; ++c) {
    const int cur = (c & 1) * (kNE * kRowB);
    const char* buf = kbuf + cur;
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (c + 1 < nchunks) fill(kbuf + (kNE * kRowB - cur), (int64_t)(c + 1) * kNE);
    __builtin_amdgcn_sched_barrier(0);
    // K fragments of entry tile et + 1 are read while tile et is multiplied; the four head
    // tiles are independent accumulation chains, interleaved k-step by k-step
    auto kread = [&](int et, int ks) {
      return *reinterpret_cast<const bf16x8*>(buf + ((ks & 1) ? bb1 : bb0) + et * 16 * kRowB + 128 * (ks >> 1));
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
      reduce_prev();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three vector ALU instructions
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) Sp[mt] = S[mt];
      sp = (int64_t)c * kNE + 16 * et + jj;
    }
  }
  reduce_prev();  // the last tile

  // per-query top-k by its own wave (no workgroup barrier needed from here on)
  if (qvalid) {
    const int64_t q = (int64_t)b * a.T + j;
    wave_topk_reg<CAP / 64>(scw, (int)Eq, a.k, hist[wv], a.topk_idx + q * a.k,
                            a.topk_score ? a.topk_score + q * a.k : nullptr, a.topk_cnt + q);
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
template <int DT, int GS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void indexer_scan_kernel(
    IndexerArgs a, float* scores, int64_t ld, uint32_t* gmax, int64_t ng_ld) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, jj = lane & 15;
  const int j = blockIdx.y, b = blockIdx.z;
  const int64_t t = a.t0 + j;
  const int64_t E = (t + 1) / a.m;
  const int64_t e0 = (int64_t)blockIdx.x * kScanEntries + wv * (kScanEntries / 4);
  if (e0 >= E) return;
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
  const int64_t kbase = (int64_t)b * a.E_cap;
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
      const int64_t row = kbase + s;
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
        const float v = g == 0 ? res[4 * u] : g == 1 ? res[4 * u + 1] : g == 2 ? res[4 * u + 2] : res[4 * u + 3];
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

// The fused prefill kernel covers bf16 keys of 128 channels, 64 heads, and up to
// 4096 visible entries per query.
bool indexer_fused_supported(int64_t Emax, int n_hI, int cI, int dt) {
  return dt == kBF16 && cI == kCI && n_hI == kHeads && Emax <= 4096;
}

hipError_t launch_indexer_fused(const IndexerArgs& a, int64_t Emax, hipStream_t s) {
  const unsigned nblk = (unsigned)((a.T + kQ - 1) / kQ);
  if (Emax <= 2048)
    hipLaunchKernelGGL(indexer_prefill_bf16_kernel<2048>, dim3(nblk, (unsigned)a.batch), dim3(256), 0,
                       s, a);
  else
    hipLaunchKernelGGL(indexer_prefill_bf16_kernel<4096>, dim3(nblk, (unsigned)a.batch), dim3(256), 0,
                       s, a);
  return hipGetLastError();
}

bool indexer_mfma_supported(int T, int n_hI, int cI, int dt) {
  (void)T;
  return n_hI == kHeads && cI == kCI && (dt == kFP8 || dt == kMXFP4 || dt == kBF16);
}

hipError_t launch_indexer_scores_mfma(const IndexerArgs& a, float* scores, int64_t ld,
                                      uint32_t* gmax, int64_t ng_ld, int gshift, hipStream_t s) {
  const int64_t Emax = (a.t0 + a.T) / a.m;
  dim3 grid((unsigned)((Emax + kScanEntries - 1) / kScanEntries), (unsigned)a.T, (unsigned)a.batch);
  // GS template: the group size of the optional group maxima (-1: none)
#define V4A_SCAN(gs)                                                                              \
  do {                                                                                           \
    if (a.dt == kFP8)                                                                            \
      hipLaunchKernelGGL((indexer_scan_kernel<kFP8, gs>), grid, dim3(256), 0, s, a, scores, ld,  \
                         gmax, ng_ld);                                                           \
    else if (a.dt == kMXFP4)                                                                     \
      hipLaunchKernelGGL((indexer_scan_kernel<kMXFP4, gs>), grid, dim3(256), 0, s, a, scores, ld, \
                         gmax, ng_ld);                                                           \
    else                                                                                         \
      hipLaunchKernelGGL((indexer_scan_kernel<kBF16, gs>), grid, dim3(256), 0, s, a, scores, ld, \
                         gmax, ng_ld);                                                           \
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
