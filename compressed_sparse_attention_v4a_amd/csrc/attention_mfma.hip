// Shared-KV MQA attention on the gfx950 matrix cores (bf16, c = 512, heads in
// groups of 64): CSA prefill, CSA and HCA decode (candidate splits) in mqa_mfma_kernel,
// HCA prefill in hca_pair_kernel (two positions per workgroup, further below).
//
// What it computes is the core attention of "CSA And HCA: Definition, State,
// And Cost Model" (sections 3.2, 4, 5.1-5.3): per query position t and head h,
// one softmax over the candidate list (compressed entries || window rows), each
// row serving as key and value of every head, a sink logit in the denominator,
// and inverse RoPE at t on the output.
//
// Work decomposition (one workgroup = one query position x 64 heads, 8 waves, two
// per SIMD, all products on v_mfma_f32_32x32x16_bf16):
//   * Candidate rows (1 KiB each) stream through LDS 64 at a time, double
//     buffered, gathered with direct global->LDS 16-byte loads (one row per
//     instruction, row address in scalar registers), one row at a time between
//     the matrix instructions of the chunk before.  The 16-byte chunks of a row
//     are XOR-swizzled by a function of the row so that both read patterns below
//     are bank-conflict free.  The top-k entries of the rows are loaded into
//     registers a chunk ahead.
//   * Scores S^T = K Q^T: wave w = 4 hh + 2 cc + kx computes head tile hh (32
//     heads) against candidate block cc (32 rows) of the chunk over channel half
//     kx, with its query fragments resident in registers (RMS-normalised scale
//     applied to the float32 scores, rotated at t).  The two halves of a tile
//     trade the partial sums of the elements the other one owns through LDS.
//   * Softmax with a fixed reference maximum per head (the first chunk's
//     maximum): probabilities are exp2(s - m_ref) < 2^64, so O is never rescaled.
//     A chunk maximum past the reference by more than that is noted and acted on
//     after the pass: the item restarts with the pass maximum as reference, which
//     no chunk can exceed (never triggered for normalised queries and rows).  The score accumulator layout of the 32x32 tile is
//     already the A-operand layout of P V (candidate k-slots permuted identically
//     on both sides), so each wave packs its P to bf16 and stores it to LDS as a
//     ready-made fragment.
//   * O += P V: wave w owns output channels 64 w .. 64 w + 63 of all 64 heads (4
//     accumulator tiles), reading P fragments from LDS and V straight from the
//     row-major chunk with the gfx950 transposing LDS read.
//   * Epilogue: normalisation (+ sink), inverse RoPE, bf16 output staged through
//     LDS for coalesced 16-byte stores; the decode form writes float32 partial
//     states (unnormalised O, reference max, sum) for the merge kernel.
// Local window rows are normalised and rotated once by a pre-pass into a bf16
// workspace, so every candidate is a plain row gather.
#include "compress_rows.h"
#include "device_common.h"
#include "internal.h"
#include "window_prep.h"

#include <algorithm>
#include <type_traits>

namespace v4a {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((address_space(3))) void* lds_void;

constexpr int kC = 512;        // channels per row
constexpr int kHG = 64;        // heads per workgroup
constexpr int kNC = 64;        // candidates per chunk
constexpr int kRowBytes = kC * 2;
constexpr int kChunkBytes = kNC * kRowBytes;
constexpr int kWaves = 8;      // two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = kNC / kWaves;  // rows of a chunk gathered by each wave
constexpr int kMaxCand = 2048; // longest candidate list (k + w) served here; longer lists take the general kernel
// Probabilities are exp2(s - m_ref) with m_ref fixed after the first chunk.  They
// stay below 2^kLazy; O (|v| < 2^6, at most 2^11 candidates) stays below 2^81, far
// from float32 overflow.  A chunk maximum that grows further makes the item restart
// with a larger reference, so O is never rescaled.
constexpr float kLazy = 64.0f;

// XOR applied to the low four bits of the 16-byte chunk index of row r.  The LDS has
// 64 four-byte banks: a 16-byte read serves 16 lanes per cycle, which must cover the 16
// chunk positions of a 256-byte span, and a transposing 8-byte read 32 lanes.  Sixteen
// consecutive rows get sixteen different values (score reads: 16 lanes, 16 rows, one
// chunk column), and rows 4h..4h+3 differ in bits 2-3 (transposing V reads: four rows x
// four adjacent chunks per 32 lanes, each row in its own 64-byte quarter).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (N << 8) | (3 << 14));
}

// Workgroup barrier that neither waits for outstanding memory operations (the
// next chunk's gather stays in flight) nor lets the compiler move memory
// accesses across it.  Callers wait for the counters they need first.
__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Values known to be equal in every lane, kept in scalar registers.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Direct global -> LDS loads (16 or 4 bytes per lane; lane i lands at lds + size * i),
// written out so that the compiler does not order every later LDS read behind them:
// each use below is followed by an explicit vmcnt wait and a barrier before the data
// is read.  gbase is wave-uniform (scalar registers), voff a per-lane byte offset.
// No other instruction of these kernels reads M0.
__device__ __forceinline__ void dma_b128(const void* gbase, uint32_t voff, const void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m0), "v"(voff), "s"(gbase) : "memory");
}
__device__ __forceinline__ void dma_b32(const void* gbase, uint32_t voff, const void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(m0), "v"(voff), "s"(gbase) : "memory");
}

// Two floats -> packed bf16 pair (round to nearest even, hardware conversion).
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  const bf16x2 r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

struct MqaArgs {
  const uint16_t* q;      // prefill: [batch][T][n_h][512]; decode: [batch][n_h][512]
  const uint16_t* kvc;    // [batch][E_cap][512], compressed entries as stored
  const uint16_t* kvl;    // [batch][n_lrows][512] normalised+rotated window rows
  const int32_t* idx;     // [batch][T or 1][k]
  const int32_t* cnt;     // [batch][T or 1]
  const float* sink;      // [n_h] or null
  const float* q_gamma;   // [512] or null
  uint16_t* out;          // [batch][T or 1][n_h][512]
  float* part;            // decode partials [batch][splits][n_h][514]
  int64_t t0, E_cap, lrow_base, n_lrows;
  int batch, T, n_h, k, w, m_prime, rope_dims, mode, splits, split_len;
  float eps, rope_base, qscale;
  RopeTab rope;
  // decode serving state: per-sequence positions (tpos) and paged compressed rows.  With
  // pages, kvc is a pool: a CSA list (idx) already holds pool rows, a dense HCA prefix is
  // translated through the block table here.
  const int64_t* tpos;
  const int32_t* pages;
  int64_t max_pages;
  int page_shift;
  int staged;  // dense decode over a staged list: cnt[b] rows per sequence, not (t+1)/m'
};

__device__ __forceinline__ bf16x8 lds_read_b128(const char* base, int off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}

__device__ __forceinline__ u32x2 lds_read_tr(const char* base, int off) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(
      (__attribute__((address_space(3))) char*)(base) + off));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Operand and accumulator layouts of v_mfma_f32_32x32x16_bf16 used below (lane l,
// half hl = l >> 5, l32 = l & 31):
//   A: row l32, k-slots 8 hl .. 8 hl + 7      B: column l32, k-slots 8 hl .. 8 hl + 7
//   C: column l32, element i in row 8 (i >> 2) + 4 hl + (i & 3)
// Candidate <-> k-slot map of one P V step (16 candidates): slot 8 hl + 4 e + r holds
// candidate 8 e + 4 hl + r.  A score tile's elements 8 p' .. 8 p' + 7 are then exactly
// the A fragment of P V step p' of its 32-row block.
//
// Wave roles (8 waves, two per SIMD): wave w = 4 hh + 2 cc + kx scores head tile hh
// against candidate block cc over the channel half kx; the two halves of a tile trade
// the partial sums of the elements the other one owns (elements 8 kx' .. 8 kx' + 7 go to
// the wave with kx = kx'), so each wave ends with the full scores of one P V step of its
// block.  In P V, wave w owns the output channels 64 w .. 64 w + 63 of all 64 heads.
template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void mqa_mfma_kernel(MqaArgs a) {
  __shared__ __attribute__((aligned(1024))) char kvbuf[2 * kChunkBytes];  // chunk buffers / query rows
  __shared__ __attribute__((aligned(16))) char xbuf[kWaves * 2 * 64 * 16]; // partial scores [wave][half][lane]
  __shared__ __attribute__((aligned(16))) char pbuf[2 * 4 * 64 * 16];      // P [head tile][step][lane]
  __shared__ float mx_s[kWaves][32];    // chunk maximum per (wave, head of its tile)
  __shared__ float lsum_s[kWaves][32];  // softmax sums per (wave, head of its tile)
  __shared__ int flag_s[kWaves];
  __shared__ __attribute__((aligned(16))) float den_s[kHG];
  __shared__ float mref_s[kHG];
  __shared__ __attribute__((aligned(16))) float rope_c[kMaxRopeDims / 2], rope_s[kMaxRopeDims / 2];
  __shared__ __attribute__((aligned(16))) float qg_s[kC];  // query RMSNorm weights
  __shared__ float qinv_s[kHG];  // scale * log2 e / rms(q) per head

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int hh = wv >> 2, cc = (wv >> 1) & 1, kx = wv & 1;
  const int hl = lane >> 5, l32 = lane & 31;
  constexpr bool kDec = MODE == kModeDecode || MODE == kModeHCADecode;
  const bool decode = kDec;
  constexpr bool dense = MODE == kModeHCA || MODE == kModeHCADecode;  // every completed entry
  const int nq = decode ? 1 : a.T;
  const int hgroups = a.n_h / kHG;
  const int64_t n_items = decode ? (int64_t)a.batch * hgroups * a.splits : (int64_t)a.batch * hgroups * a.T;

  // ---- work items -----------------------------------------------------------
  // Prefill items run from the latest position (longest candidate list) down; decode
  // items are (sequence, head group, candidate split).
  struct Item {
    int b, hgrp, qi, split;
    int64_t t, ncomp, lo, ub, nrows, nchunks;
  };
  auto describe = [&](int64_t j) {
    Item it;
    if (decode) {
      it.split = (int)(j % a.splits);
      const int64_t r = j / a.splits;
      it.hgrp = (int)(r % hgroups);
      it.b = (int)(r / hgroups);
      it.qi = 0;
      it.t = a.tpos ? a.tpos[it.b] : a.t0;
    } else {
      const int64_t bh = (int64_t)a.batch * hgroups;
      const int64_t u = j / bh, r = j % bh;
      it.b = (int)(r / hgroups);
      it.hgrp = (int)(r % hgroups);
      it.qi = a.T - 1 - (int)u;
      it.split = 0;
      it.t = a.t0 + it.qi;
    }
    if constexpr (dense) {
      it.ncomp = a.staged ? min(max(a.cnt[(int64_t)it.b * nq + it.qi], 0), a.k) : (it.t + 1) / a.m_prime;
    } else {
      it.ncomp = min(max(a.cnt[(int64_t)it.b * nq + it.qi], 0), a.k);
    }
    it.lo = it.t - a.w + 1 > 0 ? it.t - a.w + 1 : 0;
    const int64_t N = it.ncomp + (it.t - it.lo + 1);
    int64_t ub = 0, ue = N;
    if (decode) {
      ub = min((int64_t)it.split * a.split_len, N);
      ue = min(ub + a.split_len, N);
    }
    it.ub = ub;
    it.nrows = ue - ub;
    it.nchunks = (it.nrows + kNC - 1) / kNC;
    it.b = uni(it.b);
    it.hgrp = uni(it.hgrp);
    it.qi = uni(it.qi);
    it.split = uni(it.split);
    it.t = uni(it.t);
    it.ncomp = uni(it.ncomp);
    it.lo = uni(it.lo);
    it.ub = uni(it.ub);
    it.nrows = uni(it.nrows);
    it.nchunks = uni(it.nchunks);
    return it;
  };

  // Query rows (64 heads x 1 KiB) of an item into chunk buffer qbuf, 8 rows per wave,
  // 16-byte chunks swizzled like candidate rows.
  auto issue_query_loads = [&](const Item& it, int qbuf) {
    const char* qrows = reinterpret_cast<const char*>(
        a.q + (((int64_t)it.b * nq + it.qi) * a.n_h + (int64_t)it.hgrp * kHG) * kC);
    char* dst = kvbuf + qbuf * kChunkBytes;
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const int h = kRowsPerWave * wv + r;
      const uint32_t voff = (uint32_t)(lane ^ swz(h)) << 4;
      dma_b128(qrows + (int64_t)h * kRowBytes, voff, dst + h * kRowBytes);
    }
  };

  // Top-k entry of the row that lane j < 8 of wave wv gathers for the chunk starting at
  // candidate r0 (row r0 + 8 wv + j), loaded a chunk ahead into a register.  Clamped to
  // the top-k row; the value is only used for rows inside the compressed part.
  auto load_raw = [&](const Item& it, int64_t r0) -> int {
    if constexpr (dense) {
      // paged: the block-table entry of the row's page (rows inside the compressed prefix)
      if (!a.pages) return 0;
      const int64_t u = it.ub + r0 + kRowsPerWave * wv + (lane & 7);
      const int64_t s = u < it.ncomp ? u : 0;
      return a.pages[(int64_t)it.b * a.max_pages + (s >> a.page_shift)];
    } else {
      if (a.k <= 0) return 0;
      const int32_t* irow = a.idx + ((int64_t)it.b * nq + it.qi) * a.k;
      const int64_t u = it.ub + r0 + kRowsPerWave * wv + (lane & 7);
      return irow[u < a.k ? u : a.k - 1];
    }
  };

  // wave wv gathers rows [8 wv, 8 wv + 8) of the chunk starting at candidate r0; lane i
  // of a row load carries chunk i of the global row into LDS chunk i ^ swz.
  // Address of row r0 + 8 wv + (lane & 7) of the candidate list (lanes j < 8 matter):
  // each row load of gather_row takes it from lane j into scalar registers (the lane
  // offset stays a 32-bit vector operand of the scalar-base form of the load)
  // window rows: prefill workspace row = position - lrow_base; decode row r = position lo + r
  // of the sequence's own window
  const int64_t kv_bstride = a.pages ? 0 : a.E_cap;  // a pool has no per-sequence stride
  const int64_t kv_rows = a.pages ? ((int64_t)1 << 31) - 1 : a.E_cap;
  // Per-lane arithmetic in 32 bits (list positions, entries and window rows are below
  // 2^31); the per-item terms are wave-uniform.
  auto row_addr = [&](const Item& it, int64_t r0, int raw) -> uint64_t {
    const char* kvc_b = reinterpret_cast<const char*>(a.kvc + (int64_t)it.b * kv_bstride * kC);
    const char* kvl_b = reinterpret_cast<const char*>(a.kvl + (int64_t)it.b * a.n_lrows * kC);
    const int64_t wbase = decode ? it.lo : a.lrow_base;
    int myid = -1 - (int)(it.t - wbase);  // past the list end: the query's own window row
    const int rr = (int)r0 + kRowsPerWave * wv + (lane & 7);
    if (rr < (int)it.nrows) {
      const int u = (int)it.ub + rr;
      const int ncomp = (int)it.ncomp;
      if (u < ncomp) {
        if constexpr (dense) {
          myid = a.pages ? ((raw << a.page_shift) | (u & ((1 << a.page_shift) - 1))) : u;
        } else {
          // out-of-range indices must not fault
          myid = min(max(raw, 0), (int)(kv_rows - 1));
        }
      } else {
        myid = -1 - ((int)(it.lo - wbase) + (u - ncomp));
      }
    }
    return myid >= 0 ? (uint64_t)kvc_b + (uint64_t)myid * kRowBytes
                     : (uint64_t)kvl_b + (uint64_t)(-1 - myid) * kRowBytes;
  };
  // row 8 wv + r of a chunk into chunk buffer dst; lane i carries chunk i of the global
  // row into LDS chunk i ^ swz(8 wv + r)
  const uint32_t lane16 = (uint32_t)lane << 4;
  auto gather_row = [&](uint64_t addr, char* dst, int r) {
    // readlane returns int: go through uint32_t so the low half is not sign-extended
    const uint64_t ra = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((uint32_t)(addr >> 32), r) << 32) |
                        (uint64_t)(uint32_t)__builtin_amdgcn_readlane((uint32_t)addr, r);
    // the lane offset is formed at each use by one instruction the compiler cannot hoist
    // (hoisted, the eight per-row offsets would hold eight registers across the loop)
    uint32_t lo;
    asm volatile("v_xor_b32 %0, %1, %2"
                 : "=v"(lo)
                 : "s"((uint32_t)swz(kRowsPerWave * wv + r) << 4), "v"(lane16));
    dma_b128(reinterpret_cast<const char*>(ra), lo, dst + (kRowsPerWave * wv + r) * kRowBytes);
  };
  auto fill = [&](const Item& it, char* dst, int64_t r0, int raw) {
    const uint64_t addr = row_addr(it, r0, raw);
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) gather_row(addr, dst, r);
  };

  // ---- per-lane LDS byte offsets (everything step-dependent is an immediate) --
  // score reads: row 32 cc + (l32 ^ 16 kx), channels 256 kx + 16 s + 8 hl .. + 7, i.e.
  // chunk 32 kx + 16 (s >> 3) + (2 (s & 7) + hl), swizzled within its 256-byte group.
  // The channel-half kx = 1 reads the two 16-row halves of its tile swapped, so that in
  // both halves the rows the wave keeps after the trade (16 kx .. 16 kx + 15 of the tile)
  // land in the first eight accumulator elements.
  const int srow = 32 * cc + (l32 ^ (16 * kx));
  int sb[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) sb[u] = srow * kRowBytes + (((2 * u + hl) ^ swz(srow)) << 4) + 512 * kx;
  // transposing V reads, 16-lane group G = lane >> 4, J = lane & 15 = 4 i + q:
  //   row 16 p + 8 e + 4 (G >> 1) + i, channels 32 T + 16 (G & 1) + 4 q .. +3, T = 2 wv + nt
  //   (wave wv owns the 64 contiguous channels 64 wv ..); chunk 8 wv + 4 nt + x lies at
  //   byte 16 ((8 wv + 4 nt + x) ^ swz(row)) of its row, swz(row) = 4 i + 2 e + (G >> 1)
  int vbase[2][2];  // [nt][e]; step p adds 16 rows (16 KiB)
  {
    const int G = lane >> 4, i = (lane & 15) >> 2, q = lane & 3;
    const int x = 2 * (G & 1) + (q >> 1);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int row = 8 * e + 4 * (G >> 1) + i;
        vbase[nt][e] = row * kRowBytes + (((8 * wv + 4 * nt + x) ^ swz(row)) << 4) + 8 * (q & 1);
      }
  }
  const int pbase = lane * 16;

  const int64_t item = blockIdx.x;
  if (item >= n_items) return;
  constexpr int par = 0;  // chunk c lives in buffer c & 1; the query rows land in buffer 1
  const Item cur = describe(item);
  // every load of the prologue goes out at once: query rows (direct to LDS), the top-k
  // entries of the first two chunks, the query RMSNorm weights
  issue_query_loads(cur, 1);
  __builtin_amdgcn_sched_barrier(0);
  const int raw0 = load_raw(cur, 0);
  const int raw1 = load_raw(cur, kNC);
  const float g = a.q_gamma ? a.q_gamma[tid] : 1.0f;
  const double f = tid < kMaxRopeDims / 2 ? a.rope.inv_freq[tid] : 0.0;
  {
    qg_s[tid] = g;
    // RoPE angles at t for the 32 frequencies (the inverse rotation of the output uses
    // -sin); without RoPE the table is the identity, so the rotations below need no branch
    if (tid < kMaxRopeDims / 2) {
      float cs = 1.0f, sn = 0.0f;
      if (a.rope_dims > 0) rope_cs_fast((double)cur.t, f, cs, sn);
      rope_c[tid] = cs;
      rope_s[tid] = sn;
    }
    wait_vmcnt<0>();
    wait_lgkmcnt<0>();
    block_sync();  // query rows, angles and gamma visible
    // chunk 0 is gathered during the query preparation, four rows before each of its two
    // halves (a burst of eight loads per wave would hold the preparation back)
    const bool first = cur.nchunks > 0;
    const uint64_t addr0 = row_addr(cur, 0, raw0);

    // ---- query rows: q * gamma, rotated at t on the last 64 channels, bf16, in place ----
    // Wave wv prepares heads 8 wv + l8 (l8 = lane & 7); lane group g8 = lane >> 3 takes
    // the 16-byte chunks g8 + 8 u.  The per-head factor scale * log2 e / rms(q) is applied
    // to the float32 scores instead.
    char* qbufp = kvbuf + (par ^ 1) * kChunkBytes;
    {
      const int l8 = lane & 7, g8 = lane >> 3;
      const int hq = kRowsPerWave * wv + l8;
      float ss = 0.0f;
#pragma unroll
      for (int u0 = 0; u0 < 8; u0 += 4) {
        if (first) {
#pragma unroll
          for (int r = u0; r < u0 + 4; ++r) gather_row(addr0, kvbuf + par * kChunkBytes, r);
        }
        u32x4 v[4];
        float4 gm[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = g8 + 8 * (u0 + u);
          v[u] = __builtin_bit_cast(u32x4, lds_read_b128(qbufp, hq * kRowBytes + ((j ^ swz(hq)) << 4)));
          gm[u][0] = *reinterpret_cast<const float4*>(qg_s + 8 * j);
          gm[u][1] = *reinterpret_cast<const float4*>(qg_s + 8 * j + 4);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = g8 + 8 * (u0 + u);
          float x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(v[u][e] << 16);
            x[2 * e + 1] = __uint_as_float(v[u][e] & 0xFFFF0000u);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
          float y[8] = {x[0] * gm[u][0].x, x[1] * gm[u][0].y, x[2] * gm[u][0].z, x[3] * gm[u][0].w,
                        x[4] * gm[u][1].x, x[5] * gm[u][1].y, x[6] * gm[u][1].z, x[7] * gm[u][1].w};
          if (u0 + u == 7) {
            // chunk j = 56 + g8: pairs (8 j + 2 e, +1) use frequency 4 g8 + e (identity
            // angles when RoPE is off)
            const float4 c4 = *reinterpret_cast<const float4*>(rope_c + 4 * g8);
            const float4 s4 = *reinterpret_cast<const float4*>(rope_s + 4 * g8);
            const float cj[4] = {c4.x, c4.y, c4.z, c4.w};
            const float sj[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float y0 = y[2 * e], y1 = y[2 * e + 1];
              y[2 * e] = y0 * cj[e] - y1 * sj[e];
              y[2 * e + 1] = y0 * sj[e] + y1 * cj[e];
            }
          }
          const u32x4 pk = {pk_bf16(y[0], y[1]), pk_bf16(y[2], y[3]), pk_bf16(y[4], y[5]), pk_bf16(y[6], y[7])};
          *reinterpret_cast<u32x4*>(qbufp + hq * kRowBytes + ((j ^ swz(hq)) << 4)) = pk;
        }
      }
      ss += __shfl_xor(ss, 8, 64);
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      if (g8 == 0) qinv_s[hq] = a.q_gamma ? a.qscale / sqrtf(ss / (float)kC + a.eps) : a.qscale;
    }
    wait_lgkmcnt<0>();
    block_sync();  // prepared query rows and factors visible

    // ---- resident query heads: B fragments of S^T = K Q^T ------------------
    // lane (hl, l32): head 32 hh + l32, k-step s covers channels 256 kx + 16 s + 8 hl .. +7
    bf16x8 qb[16];
#pragma unroll
    for (int s = 0; s < 16; ++s)
      qb[s] = lds_read_b128(qbufp, (32 * hh + l32) * kRowBytes + (((32 * kx + 2 * s + hl) ^ swz(l32)) << 4));
    const float qinv = qinv_s[32 * hh + l32];
    // the next chunk's gather overwrites the query rows: every fragment read has returned
    // before the first loop barrier
    wait_lgkmcnt<0>();

    // ---- candidate loop ---------------------------------------------------------
    // Reference maximum from the first chunk; returns false (abandoning the item) when
    // a later chunk maximum exceeds it by more than kLazy.
    float m_ref = -INFINITY;  // head 32 hh + l32 (log2 units)
    const int64_t nchunks = cur.nchunks;
    // largest of the four chunk maxima of this wave's head tile
    auto tile_max = [&]() {
      return fmaxf(fmaxf(mx_s[4 * hh][l32], mx_s[4 * hh + 1][l32]),
                   fmaxf(mx_s[4 * hh + 2][l32], mx_s[4 * hh + 3][l32]));
    };

    // Whether a wave saw a chunk maximum past the reference (read after the barrier that
    // follows the flags, once per pass over the list); the item then takes the largest
    // chunk maximum of the tile as its new reference, so that the next pass cannot
    // overflow.
    auto overflowed = [&]() -> bool {
      if (!uni(flag_s[0] | flag_s[1] | flag_s[2] | flag_s[3] | flag_s[4] | flag_s[5] | flag_s[6] | flag_s[7]))
        return false;
      m_ref = fmaxf(m_ref, tile_max());
      return true;
    };

    auto run = [&](f32x16 (&O)[2][2], float& l_part, int raw_n) -> bool {
      {
        // zero the accumulators with the matrix unit, so that every value reaching the
        // loop-carried accumulators is defined by an MFMA (keeps them in AGPRs)
        const bf16x8 z8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        f32x16 z16;
#pragma unroll
        for (int i = 0; i < 16; ++i) z16[i] = 0.0f;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) O[ht][nt] = mfma32(z8, z8, z16);
      }
      l_part = 0.0f;
      bool ovf = false;          // a chunk maximum past the reference (this lane's head)
      float mx_run = -INFINITY;  // largest chunk maximum so far (the reference of a restart)
      // one chunk; MORE: a next chunk exists (compile time, so that the gathers interleaved
      // below need no branches; the last chunk is a copy without them)
      auto chunk = [&](int64_t c, auto more_t) -> bool {
        constexpr bool more = decltype(more_t)::value;
        const int64_t r0 = c * kNC;
        const int bi = (int)((c + par) & 1);
        const char* buf = kvbuf + bi * kChunkBytes;
        char* nbuf = kvbuf + (bi ^ 1) * kChunkBytes;
        wait_vmcnt<0>();
        block_sync();  // chunk c landed for every wave; chunk c - 1 fully consumed
        // partial scores over this wave's channel half: 16 k-steps, fragment reads two
        // steps ahead
        f32x16 S;
#pragma unroll
        for (int i = 0; i < 16; ++i) S[i] = 0.0f;
        bf16x8 ka[3];
        ka[0] = lds_read_b128(buf, sb[0]);
        ka[1] = lds_read_b128(buf, sb[1]);
        __builtin_amdgcn_sched_barrier(0);
        // the next chunk's rows are gathered one at a time between the matrix
        // instructions (rows 0-3 in the score steps, 4-7 early in the P V steps), so that
        // no wave stalls on a burst of loads while its SIMD's matrix unit idles and the
        // address unit is never saturated; the row addresses are formed while the first
        // fragments are read
        uint64_t naddr = 0;
        if constexpr (more) {
          naddr = row_addr(cur, r0 + kNC, raw_n);
          if (c + 2 < nchunks) raw_n = load_raw(cur, r0 + 2 * kNC);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          if (s + 2 < 16) ka[(s + 2) % 3] = lds_read_b128(buf, sb[(s + 2) & 7] + 256 * ((s + 2) >> 3));
          __builtin_amdgcn_sched_barrier(0);
          S = mfma32(ka[s % 3], qb[s], S);
          if ((s & 3) == 1 && more) gather_row(naddr, nbuf, s >> 2);
          __builtin_amdgcn_sched_barrier(0);
        }
        // trade halves with the other channel half of the tile (wave wv ^ 1): send the
        // elements it owns (elements 8 .. 15, its rows 16 (1 - kx) .. + 15), keep elements
        // 0 .. 7 (rows 16 kx .. 16 kx + 15, by the swapped score reads)
        float own[8], snd[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          own[i] = S[i];
          snd[i] = S[8 + i];
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          *reinterpret_cast<float4*>(xbuf + ((wv * 2 + h2) * 64 + lane) * 16) =
              make_float4(snd[4 * h2], snd[4 * h2 + 1], snd[4 * h2 + 2], snd[4 * h2 + 3]);
        wait_lgkmcnt<0>();
        block_sync();  // partial scores of every wave visible
        float sc[8];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float4 rv = *reinterpret_cast<const float4*>(xbuf + (((wv ^ 1) * 2 + h2) * 64 + lane) * 16);
          sc[4 * h2] = own[4 * h2] + rv.x;
          sc[4 * h2 + 1] = own[4 * h2 + 1] + rv.y;
          sc[4 * h2 + 2] = own[4 * h2 + 2] + rv.z;
          sc[4 * h2 + 3] = own[4 * h2 + 3] + rv.w;
        }
        // candidates past the end of the list (last chunk only): element i is candidate
        // 32 cc + 16 kx + 8 (i >> 2) + 4 hl + (i & 3) of the chunk
        // (32-bit: list lengths are below 2^31, and the scalar unit compares 32-bit values)
        if (__builtin_expect((int)r0 + kNC > (int)cur.nrows, 0)) {
          asm volatile("" ::: "memory");  // keep this a branch: only the last chunk is partial
          const int lim = (int)(cur.nrows - r0) - 32 * cc - 16 * kx - 4 * hl;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (8 * (i >> 2) + (i & 3) >= lim) sc[i] = -INFINITY;
        }
        // the maximum by three-input maxima written out: the scores are sums or -inf, never
        // NaN, so the quieting copies the compiler adds before each fmaxf are not needed
        float lmax;
        asm("v_max3_f32 %0, %1, %2, %3\n\t"
            "v_max3_f32 %0, %0, %4, %5\n\t"
            "v_max3_f32 %0, %0, %6, %7\n\t"
            "v_max_f32 %0, %0, %8"
            : "=&v"(lmax)
            : "v"(sc[0]), "v"(sc[1]), "v"(sc[2]), "v"(sc[3]), "v"(sc[4]), "v"(sc[5]), "v"(sc[6]), "v"(sc[7]));
        {
          // the other half-wave's maximum for the same head (row swap, no LDS round trip)
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lmax), __float_as_uint(lmax), false, false);
          float m2;
          asm("v_max_f32 %0, %1, %2" : "=v"(m2) : "v"(__uint_as_float(sw[0])), "v"(__uint_as_float(sw[1])));
          lmax = m2 * qinv;  // qinv > 0: order kept
        }
        mx_run = fmaxf(mx_run, lmax);
        if (c == 0) {
          // reference maximum: this chunk's maximum over the tile's four waves
          if (hl == 0) mx_s[wv][l32] = lmax;
          wait_lgkmcnt<0>();
          block_sync();
          m_ref = fmaxf(m_ref, tile_max());  // raised by a restart
          if (m_ref == -INFINITY) m_ref = 0.0f;
        } else {
          ovf = ovf || lmax > m_ref + kLazy;
        }
        float pr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], qinv, -m_ref));
        float ls = pr[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) ls += pr[i];
        l_part += ls;
        {
          const u32x4 pk = {pk_bf16(pr[0], pr[1]), pk_bf16(pr[2], pr[3]), pk_bf16(pr[4], pr[5]),
                            pk_bf16(pr[6], pr[7])};
          *reinterpret_cast<u32x4*>(pbuf + ((hh * 4 + 2 * cc + kx) * 64) * 16 + pbase) = pk;
        }
        wait_lgkmcnt<0>();
        block_sync();  // P of every wave visible

        // O^T[channel tiles of wave wv][64 heads] += V^T P^T over 4 steps of 16 candidates:
        // the V fragments are the A operand, the P fragments the B operand, so a lane ends
        // with 4 consecutive channels of one head
        __builtin_amdgcn_sched_barrier(0);
        auto vread = [&](int it) -> bf16x8 {
          // it = 2 p + nt
          const u32x2 v1 = lds_read_tr(buf, vbase[it & 1][0] + 16384 * (it >> 1));
          const u32x2 v2 = lds_read_tr(buf, vbase[it & 1][1] + 16384 * (it >> 1));
          const u32x4 cat = {v1.x, v1.y, v2.x, v2.y};
          return __builtin_bit_cast(bf16x8, cat);
        };
        bf16x8 pa[2][2];
        bf16x8 vb[3];
        pa[0][0] = lds_read_b128(pbuf, pbase);
        pa[0][1] = lds_read_b128(pbuf, pbase + 4 * 1024);
        vb[0] = vread(0);
        vb[1] = vread(1);
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int p = it >> 1, nt = it & 1;
          if (nt == 0 && p + 1 < 4) {
            pa[(p + 1) & 1][0] = lds_read_b128(pbuf, pbase + (p + 1) * 1024);
            pa[(p + 1) & 1][1] = lds_read_b128(pbuf, pbase + 4 * 1024 + (p + 1) * 1024);
          }
          if (it + 2 < 8) vb[(it + 2) % 3] = vread(it + 2);
          __builtin_amdgcn_sched_barrier(0);
          O[0][nt] = mfma32(vb[it % 3], pa[p & 1][0], O[0][nt]);
          if (it < 4 && more) gather_row(naddr, nbuf, 4 + it);
          O[1][nt] = mfma32(vb[it % 3], pa[p & 1][1], O[1][nt]);
          __builtin_amdgcn_sched_barrier(0);
        }
        return true;
      };
      for (int64_t c = 0; c + 1 < nchunks; ++c)
        if (!chunk(c, std::true_type{})) return false;
      if (nchunks > 0 && !chunk(nchunks - 1, std::false_type{})) return false;
      // an overflow is acted on once the pass is over: the pass restarts with a larger
      // reference; the values computed meanwhile are discarded
      {
        const bool any = __ballot(ovf) != 0;
        if (lane == 0) flag_s[wv] = any ? 1 : 0;
        if (hl == 0) mx_s[wv][l32] = mx_run;
      }
      wait_lgkmcnt<0>();
      block_sync();  // flags visible
      return !(nchunks > 0 && overflowed());
    };

    // ---- epilogue -------------------------------------------------------------
    auto finish = [&](f32x16 (&O)[2][2], float l_part) {
      {
        const float l = l_part + __shfl_xor(l_part, 32, 64);
        if (hl == 0) {
          lsum_s[wv][l32] = l;
          if (cc == 0 && kx == 0) mref_s[32 * hh + l32] = m_ref;
        }
      }
      wait_lgkmcnt<0>();
      block_sync();  // sums visible; every wave is done with the chunk buffers
      const bool partial = decode && a.splits > 1;
      if (tid < kHG) {
        const int ht = tid >> 5, h = tid & 31;
        const float l = (lsum_s[4 * ht][h] + lsum_s[4 * ht + 1][h]) + (lsum_s[4 * ht + 2][h] + lsum_s[4 * ht + 3][h]);
        if (partial) {
          den_s[tid] = l;
        } else {
          float den = l;
          if (a.sink) den += __builtin_amdgcn_exp2f(a.sink[cur.hgrp * kHG + tid] * kLog2e - mref_s[tid]);
          den_s[tid] = 1.0f / den;
        }
      }
      wait_lgkmcnt<0>();
      block_sync();  // per-head denominators visible
      // lane (hl, l32) holds, for head tile ht and channel tile T = 2 wv + nt, head
      // 32 ht + l32 at channels 32 T + 8 j + 4 hl + (0..3) in O[ht][nt][4 j .. 4 j + 3]
      if (partial) {
        // partial state: [b][split][h][c + 2] = (O unnormalised, reference max, sum)
        float* pg = a.part + (((int64_t)cur.b * a.splits + cur.split) * a.n_h + (int64_t)cur.hgrp * kHG) * (kC + 2);
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          float* prow = pg + (int64_t)(32 * ht + l32) * (kC + 2);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              // rows are c + 2 floats long, so only 8-byte alignment is guaranteed
              float* d = prow + 64 * wv + 32 * nt + 8 * j + 4 * hl;
              *reinterpret_cast<float2*>(d) = make_float2(O[ht][nt][4 * j], O[ht][nt][4 * j + 1]);
              *reinterpret_cast<float2*>(d + 2) = make_float2(O[ht][nt][4 * j + 2], O[ht][nt][4 * j + 3]);
            }
        }
        if (tid < kHG) {
          float* prow = pg + (int64_t)tid * (kC + 2);
          prow[kC] = mref_s[tid];
          prow[kC + 1] = den_s[tid];
        }
        return;
      }
      // normalise, inverse RoPE on the last 64 channels (wave 7), bf16; the two half-waves
      // swap 4-channel groups so each lane holds 8 consecutive channels, and each wave
      // transposes its 64 heads x 64 channels through its own 8 KiB of the chunk buffers
      // (row = head, 16-byte chunk 4 nt + 2 jp + hl at position chunk ^ (head & 7)), so
      // that every store instruction writes 8 whole 128-byte head segments
      char* tb = kvbuf + wv * 8192;
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const float inv = den_s[32 * ht + l32];
        const int h = 32 * ht + l32;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          uint32_t pk[4][2];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float x[4] = {O[ht][nt][4 * j] * inv, O[ht][nt][4 * j + 1] * inv, O[ht][nt][4 * j + 2] * inv,
                          O[ht][nt][4 * j + 3] * inv};
            if (wv == kWaves - 1) {
              // pairs (ch, ch + 1), ch = 448 + 32 nt + 8 j + 4 hl + 2 e, use frequency
              // (ch - 448) / 2
              const int f = 16 * nt + 4 * j + 2 * hl;
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const float cs = rope_c[f + e], sn = rope_s[f + e];
                const float x0 = x[2 * e], x1 = x[2 * e + 1];
                x[2 * e] = x0 * cs + x1 * sn;
                x[2 * e + 1] = x1 * cs - x0 * sn;
              }
            }
            pk[j][0] = pk_bf16(x[0], x[1]);
            pk[j][1] = pk_bf16(x[2], x[3]);
          }
#pragma unroll
          for (int jp = 0; jp < 2; ++jp) {
            // lower half keeps group 2 jp and takes the upper half's; the upper half keeps
            // group 2 jp + 1 and takes the lower half's: channels 16 jp + 8 hl .. + 7
            const auto w0 = __builtin_amdgcn_permlane32_swap(pk[2 * jp][0], pk[2 * jp + 1][0], false, false);
            const auto w1 = __builtin_amdgcn_permlane32_swap(pk[2 * jp][1], pk[2 * jp + 1][1], false, false);
            const u32x4 v = {w0[0], w1[0], w0[1], w1[1]};
            const int cidx = 4 * nt + 2 * jp + hl;
            *reinterpret_cast<u32x4*>(tb + h * 128 + ((cidx ^ (h & 7)) << 4)) = v;
          }
        }
      }
      asm volatile("" ::: "memory");  // LDS operations of a wave complete in order
      uint16_t* dst = a.out + (((int64_t)cur.b * nq + cur.qi) * a.n_h + (int64_t)cur.hgrp * kHG) * kC;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // lanes 8 k .. 8 k + 7: head 8 i + k, chunk cidx = lane & 7 = channels
        // 64 wv + 8 cidx .. + 7
        const int h = 8 * i + (lane >> 3), cidx = lane & 7;
        const u32x4 v = *reinterpret_cast<const u32x4*>(tb + h * 128 + ((cidx ^ (h & 7)) << 4));
        *reinterpret_cast<u32x4*>(dst + (int64_t)h * kC + 64 * wv + 8 * cidx) = v;
      }
    };

    {
      f32x16 O[2][2];
      float l_part;
      // A chunk maximum past the reference by more than kLazy: run() has raised the
      // reference to the pass maximum; the gather in flight lands, chunk 0 is gathered
      // again and the pass starts over (no rescaling of O inside the loop, and no second
      // launch for such items).  The raised reference is at least every chunk maximum of
      // the list, so the second pass always completes.
      if (__builtin_expect(!run(O, l_part, raw1), 0)) {
        do {
          wait_vmcnt<0>();
          block_sync();
          fill(cur, kvbuf + par * kChunkBytes, 0, raw0);
        } while (!run(O, l_part, raw1));
      }
      finish(O, l_part);
    }
  }
}

// Normalise and rotate the window rows once into a bf16 workspace.
//   prefill/HCA: ws row r <- local position lrow_base + r
//   decode:      ws row r <- position lo + r read from the ring (token t from kv_new),
//                and kv_new is written into ring slot t % w
__global__ __launch_bounds__(256) void local_prep_kernel(LocalPrepArgs a) {
  window_prep_block(a, blockIdx.x, blockIdx.y, threadIdx.x);
}

// Decode front: the independent first steps of a decode step in one launch, so that
// they overlap instead of paying a launch and a memory round trip each (steps whose top-k
// is the threshold filter run them inside the scan and the final top-k launch instead,
// see decode_front_args).  Row b of the
// grid: block v < n_comp runs compressor group v of the main instance in wave 0 and of
// the index instance in wave 1 (first, as they have the longest dependency chain);
// blocks n_comp .. prepare the window rows (kFrontRows per block) and insert the new
// token into the ring.  GM, GI: lanes per entry (c / 8) of the main and index instance
// (bf16 tails).
template <int GM, int GI>
__global__ __launch_bounds__(256) void decode_front_kernel(CompressArgs cm, CompressArgs ci,
                                                           LocalPrepArgs lp, int n_comp) {
  const int b = blockIdx.y;
  if ((int)blockIdx.x >= n_comp) {
    window_prep_block<kFrontRows / 4>(lp, (int)blockIdx.x - n_comp, b, threadIdx.x);
    return;
  }
  const int64_t vb = blockIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wv == 0 && vb * (64 / GM) < cm.n_entries) compress_rows_body<uint16_t, GM>(cm, vb, b, lane);
  if (wv == 1 && vb * (64 / GI) < ci.n_entries) compress_rows_body<uint16_t, GI>(ci, vb, b, lane);
}

// Selected entries of a decode step in the production row format (kKV576), dequantised
// to bf16 into a staging list [batch][k][512] (row u = the u-th selected entry), which
// the attention then reads as a dense prefix of cnt[b] rows.  One wave per row: lane l
// takes channels 8 l .. 8 l + 7 (eight E4M3 codes times the row scale, or eight bf16).
__global__ __launch_bounds__(256) void kv576_gather_kernel(const uint8_t* kv, const float* kv_scale,
                                                           const int32_t* idx, const int32_t* cnt,
                                                           SeqState seq, int64_t E_cap, int k,
                                                           int rope_dims, uint16_t* staged) {
  const int b = blockIdx.y;
  const int u = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (u >= k || u >= cnt[b]) return;
  const int64_t row = cache_row(seq, E_cap, b, idx[(int64_t)b * k + u]);
  const int nq = kC - rope_dims;
  const uint8_t* src = kv + row * kv576_row_bytes(kC, rope_dims);
  const int ch0 = 8 * lane;
  uint4 o;
  if (ch0 < nq) {
    const uint2 v = *reinterpret_cast<const uint2*>(src + ch0);
    const float sc = kv_scale[row];
    const uint32_t w[2] = {v.x, v.y};
    uint32_t p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = (w[e >> 1] >> (16 * (e & 1))) & 255u, hi = (w[e >> 1] >> (16 * (e & 1) + 8)) & 255u;
      p[e] = pk_bf16(e4m3_to_f32(lo) * sc, e4m3_to_f32(hi) * sc);
    }
    o = make_uint4(p[0], p[1], p[2], p[3]);
  } else {
    o = *reinterpret_cast<const uint4*>(src + nq + 2 * (ch0 - nq));
  }
  *reinterpret_cast<uint4*>(staged + ((int64_t)b * k + u) * kC + ch0) = o;
}


// ---- HCA prefill: two consecutive positions per workgroup ---------------------------
// In HCA ("CSA And HCA: Definition, State, And Cost Model", section 4) every position of
// a block sees the same compressed prefix, and positions t and t + 1 share all but one
// window row each, so one workgroup serves both (64 heads each) over the union of their
// candidate lists: every gathered row feeds 128 (position, head) columns of the matrix
// products instead of 64, and the per-chunk chain of landing, barrier and softmax is paid
// once for both.  Candidate u of the union list is compressed entry u for u < n_B, else
// window position lo_A + (u - n_B); position t does not see entry n_A..n_B - 1 (the block
// that t + 1 completes) nor window position t + 1, and t + 1 does not see lo_A when its
// window starts one later.  Those entries get a score of -inf for that position.
//
// Four waves, one per SIMD with the whole register file: wave w = 2 qq + hh owns heads
// 32 hh .. 32 hh + 31 of position qq through both products, so waves share nothing but
// the chunk buffers (one barrier per chunk):
//   * S^T = K Q^T over all 512 channels, one 32-row block of a 64-row chunk at a time:
//     32 k-steps of v_mfma_f32_32x32x16_bf16, query fragments resident (128 registers;
//     the rows land in LDS by whole-row direct loads, each wave reads its fragments and
//     prepares them in registers: q * gamma, rotated at t; the factor
//     scale * log2 e / rms(q) multiplies the float32 scores);
//   * softmax in registers with the fixed reference maximum of the first block (and the
//     in-place restart of the CSA kernel when a later block exceeds it by 2^64);
//   * O^T = V^T P^T for all 512 channels: 16 accumulator tiles (256 accumulation
//     registers); a block's score accumulator is already the P fragment of its two steps.
constexpr int kPairWaves = 4;
constexpr int kPairThreads = 64 * kPairWaves;
constexpr int kPairRows = kNC / kPairWaves;  // rows of a chunk gathered by each wave

// The score products accumulate in vector registers, written as inline assembly: with
// the builtin, every product of a kernel that may use more than 256 registers takes the
// accumulation-register form, and the 16 score registers do not fit beside the 256 of O.
// A chain of products into the same full tile needs no wait states between them; the last
// one waits out the product's latency before its result is read by vector instructions.
__device__ __forceinline__ void mfma_v_first(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_last(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(acc) : "v"(a), "v"(b));
}

__global__ __launch_bounds__(kPairThreads, 1) void hca_pair_kernel(MqaArgs a) {
  __shared__ __attribute__((aligned(1024))) char kvbuf[2 * kChunkBytes];  // chunk buffers / output staging
  __shared__ __attribute__((aligned(16))) float qg_s[kC];                 // query RMSNorm weights
  __shared__ __attribute__((aligned(16))) float rope_c[2][kMaxRopeDims / 2], rope_s[2][kMaxRopeDims / 2];
  __shared__ int flag_s[kPairWaves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qq = wv >> 1, hh = wv & 1;
  const int hl = lane >> 5, l32 = lane & 31;
  const int hgroups = a.n_h / kHG;
  const int npairs = (a.T + 1) / 2;
  const int64_t bh = (int64_t)a.batch * hgroups;
  const int64_t item = blockIdx.x;
  if (item >= bh * npairs) return;
  // pairs run from the latest (longest lists) down
  const int b = uni((int)((item % bh) / hgroups));
  const int hgrp = uni((int)((item % bh) % hgroups));
  const int qi0 = uni(2 * (npairs - 1 - (int)(item / bh)));
  const bool pair = qi0 + 1 < a.T;  // an odd last position runs alone (both halves compute it)
  const int64_t tA = a.t0 + qi0, tB = pair ? tA + 1 : tA;
  const int64_t nA = (tA + 1) / a.m_prime, nB = (tB + 1) / a.m_prime;
  const int64_t loA = tA - a.w + 1 > 0 ? tA - a.w + 1 : 0;
  const int64_t loB = tB - a.w + 1 > 0 ? tB - a.w + 1 : 0;
  // list positions, entries and window rows are below 2^31
  const int nrows = uni((int)(nB + (tB - loA + 1)));
  const int nchunks = uni((nrows + kNC - 1) / kNC);
  const int ncomp = uni((int)nB);
  // candidates this wave's position does not see: u in [xa, xb) and u >= lim
  const int xa = uni(qq == 0 ? (int)nA : (int)nB);
  const int xb = uni(qq == 0 ? (int)nB : (int)(nB + (loB - loA)));
  const int lim = uni(qq == 0 && pair ? nrows - 1 : nrows);
  const int64_t tq = qq ? tB : tA;
  const int qi = pair ? qi0 + qq : qi0;

  // ---- prologue: query rows and weights (direct to LDS), query fragments (to registers),
  // then chunk 0 (direct to LDS) in flight while the fragments are prepared ----
  if (a.q_gamma) {
    // 4-byte pieces (the weights need only float alignment): wave w loads 128 of them
    dma_b32(a.q_gamma + 128 * wv, (uint32_t)lane << 2, qg_s + 128 * wv);
    dma_b32(a.q_gamma + 128 * wv + 64, (uint32_t)lane << 2, qg_s + 128 * wv + 64);
  } else {
    qg_s[tid] = 1.0f;
    qg_s[tid + kPairThreads] = 1.0f;
  }
  const char* kvc_b = reinterpret_cast<const char*>(a.kvc + (int64_t)b * a.E_cap * kC);
  const char* kvl_b = reinterpret_cast<const char*>(a.kvl + (int64_t)b * a.n_lrows * kC);
  const int lwin = (int)(loA - a.lrow_base);  // workspace row of window position lo_A
  // address of list row r0 + 16 wv + (lane & 15) (lanes 0..15 matter); rows past the end
  // of the list repeat its last row (their scores are masked)
  auto row_addr = [&](int r0) __attribute__((always_inline)) -> uint64_t {
    int u = r0 + kPairRows * wv + (lane & 15);
    u = u < nrows ? u : nrows - 1;
    return u < ncomp ? (uint64_t)kvc_b + (uint64_t)(uint32_t)u * kRowBytes
                     : (uint64_t)kvl_b + (uint64_t)(uint32_t)(lwin + u - ncomp) * kRowBytes;
  };
  const uint32_t lane16 = (uint32_t)lane << 4;
  // row 16 wv + r of a chunk: lane i carries chunk i ^ swz(r) of the global row into LDS
  // chunk i (16 wv + r and r have the same low four bits)
  auto gather_row = [&](uint64_t addr, char* dst, int r) __attribute__((always_inline)) {
    const uint64_t ra = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((uint32_t)(addr >> 32), r) << 32) |
                        (uint64_t)(uint32_t)__builtin_amdgcn_readlane((uint32_t)addr, r);
    uint32_t lo;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(lo) : "s"((uint32_t)swz(r) << 4), "v"(lane16));
    // the LDS offset is uniform: keep it in a scalar register for M0
    const int loff = uni((int)(dst - kvbuf) + (kPairRows * wv + r) * kRowBytes);
    dma_b128(reinterpret_cast<const char*>(ra), lo, kvbuf + loff);
  };
  auto fill0 = [&]() __attribute__((always_inline)) {
    const uint64_t addr = row_addr(0);
#pragma unroll
    for (int r = 0; r < kPairRows; ++r) gather_row(addr, kvbuf, r);
  };
  // the 128 query rows (row R = 64 p + h: head h of position p, in chunk buffer p), one
  // whole 1 KiB row per load, 16-byte chunks swizzled like candidate rows
  {
    const int qi1 = pair ? qi0 + 1 : qi0;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const int R = 32 * wv + r;
      const int qsel = R < kHG ? qi0 : qi1;
      const char* src = reinterpret_cast<const char*>(
          a.q + (((int64_t)b * a.T + qsel) * a.n_h + (int64_t)hgrp * kHG + (R & (kHG - 1))) * kC);
      uint32_t lo;
      asm volatile("v_xor_b32 %0, %1, %2" : "=v"(lo) : "s"((uint32_t)swz(r) << 4), "v"(lane16));
      dma_b128(src, lo, kvbuf + R * kRowBytes);
    }
  }
  if (tid < kMaxRopeDims) {
    // angles of position tA (threads 0..31) and tB (32..63); identity without RoPE
    const int p = tid >> 5, f = tid & 31;
    float cs = 1.0f, sn = 0.0f;
    if (a.rope_dims > 0) rope_cs_fast((double)(p ? tB : tA), a.rope.inv_freq[f], cs, sn);
    rope_c[p][f] = cs;
    rope_s[p][f] = sn;
  }
  wait_vmcnt<0>();
  wait_lgkmcnt<0>();
  block_sync();  // query rows, weights and angles visible
  // lane (hl, l32), k-step s: head 32 hh + l32 of position qq, channels 16 s + 8 hl .. + 7
  // (the score reads' pattern on row 32 hh + l32 of chunk buffer qq)
  u32x4 qr[32];
  {
    const char* qbase = kvbuf + qq * kChunkBytes + (32 * hh + l32) * kRowBytes;
#pragma unroll
    for (int s = 0; s < 32; ++s)
      qr[s] = __builtin_bit_cast(u32x4, lds_read_b128(qbase, ((((2 * (s & 7) + hl) ^ swz(l32)) << 4) + 256 * (s >> 3))));
  }
  wait_lgkmcnt<0>();
  block_sync();  // every wave holds its fragments: the buffers take chunk 0
  fill0();

  bf16x8 qb[32];
  float qinv;
  {
    float ssp[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};  // eight short chains
    // The weights of k-step s + kG are read once step s is done: the read address passes
    // through an empty asm statement that takes step s's result, so the compiler cannot
    // hoist all 64 reads (256 registers) to the top.
    constexpr int kG = 2;
    float4 gq[kG + 1][2];
    auto gload = [&](int s, uint32_t dep) __attribute__((always_inline)) {
      uint32_t off = (uint32_t)(16 * s + 8 * hl) * 4u;
      asm volatile("" : "+v"(off) : "v"(dep));
      const char* gp = reinterpret_cast<const char*>(qg_s) + off;
      gq[s % (kG + 1)][0] = *reinterpret_cast<const float4*>(gp);
      gq[s % (kG + 1)][1] = *reinterpret_cast<const float4*>(gp + 16);
    };
#pragma unroll
    for (int s = 0; s < kG; ++s) gload(s, 0u);
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const float4 g0 = gq[s % (kG + 1)][0], g1 = gq[s % (kG + 1)][1];
      const float gm[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      float y[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = __uint_as_float(qr[s][e] << 16), x1 = __uint_as_float(qr[s][e] & 0xFFFF0000u);
        ssp[2 * e] = fmaf(x0, x0, ssp[2 * e]);
        ssp[2 * e + 1] = fmaf(x1, x1, ssp[2 * e + 1]);
        y[2 * e] = x0 * gm[2 * e];
        y[2 * e + 1] = x1 * gm[2 * e + 1];
      }
      if (s >= 28) {
        // pairs (16 s + 8 hl + 2 e, + 1) use frequency 8 (s - 28) + 4 hl + e
        const float4 c4 = *reinterpret_cast<const float4*>(&rope_c[qq][8 * (s - 28) + 4 * hl]);
        const float4 s4 = *reinterpret_cast<const float4*>(&rope_s[qq][8 * (s - 28) + 4 * hl]);
        const float cj[4] = {c4.x, c4.y, c4.z, c4.w};
        const float sj[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float y0 = y[2 * e], y1 = y[2 * e + 1];
          y[2 * e] = y0 * cj[e] - y1 * sj[e];
          y[2 * e + 1] = y0 * sj[e] + y1 * cj[e];
        }
      }
      const u32x4 pk = {pk_bf16(y[0], y[1]), pk_bf16(y[2], y[3]), pk_bf16(y[4], y[5]), pk_bf16(y[6], y[7])};
      qb[s] = __builtin_bit_cast(bf16x8, pk);
      if (s + kG < 32) gload(s + kG, pk[0]);
    }
    float ss = ((ssp[0] + ssp[1]) + (ssp[2] + ssp[3])) + ((ssp[4] + ssp[5]) + (ssp[6] + ssp[7]));
    ss += __shfl_xor(ss, 32, 64);  // the other half of the channels
    qinv = a.q_gamma ? a.qscale / sqrtf(ss / (float)kC + a.eps) : a.qscale;
  }

  // ---- per-lane LDS offsets ---------------------------------------------------------
  // score reads (A operand, row = candidate 32 cb + l32): k-step s reads chunk 2 s + hl,
  // i.e. kb[s & 7] + 256 (s >> 3) + 32 KiB cb
  int kb[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) kb[u] = l32 * kRowBytes + (((2 * u + hl) ^ swz(l32)) << 4);
  // transposing V reads of channel tile T and step p: vb[T & 3][e] + 256 (T >> 2) + 16 KiB p
  // (16-lane group G = lane >> 4, J = lane & 15 = 4 i + q: row 16 p + 8 e + 4 (G >> 1) + i,
  // channels 32 T + 16 (G & 1) + 4 q .. + 3)
  int vb[4][2];
  {
    const int G = lane >> 4, i = (lane & 15) >> 2, q = lane & 3;
    const int x = 2 * (G & 1) + (q >> 1);
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int row = 8 * e + 4 * (G >> 1) + i;
        vb[t4][e] = row * kRowBytes + (((4 * t4 + x) ^ swz(row)) << 4) + 8 * (q & 1);
      }
  }

  float m_ref = -INFINITY;  // head 32 hh + l32 of position qq (log2 units)
  float mx_run = -INFINITY;

  auto run = [&](f32x16 (&O)[16], float& l_part) __attribute__((always_inline)) -> bool {
    {
      const bf16x8 z8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      f32x16 z16;
#pragma unroll
      for (int i = 0; i < 16; ++i) z16[i] = 0.0f;
#pragma unroll
      for (int T = 0; T < 16; ++T) O[T] = mfma32(z8, z8, z16);
    }
    l_part = 0.0f;
    bool ovf = false;
    // one chunk of 64 rows as two blocks of 32 (scores, softmax, P V each), so that one
    // score accumulator tile is live at a time
    auto chunk = [&](int c, auto more_t) __attribute__((always_inline)) {
      constexpr bool more = decltype(more_t)::value;
      const int r0 = c * kNC;
      const char* buf = kvbuf + (c & 1) * kChunkBytes;
      char* nbuf = kvbuf + ((c & 1) ^ 1) * kChunkBytes;
      wait_vmcnt<0>();
      block_sync();  // chunk c landed for every wave; chunk c - 1 fully consumed
      uint64_t naddr = 0;
      if constexpr (more) naddr = row_addr(r0 + kNC);
      constexpr int kAhead = 4;  // fragment reads in flight ahead of the products
      // score fragment s of block cb (rows 32 cb ..)
      auto kread = [&](int cb, int s) __attribute__((always_inline)) -> bf16x8 {
        return lds_read_b128(buf, kb[s & 7] + 256 * (s >> 3) + 32 * kRowBytes * cb);
      };
      bf16x8 ka[kAhead + 1];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) ka[i] = kread(0, i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        // (the first fragments of block 1 were read during block 0's P V)
        f32x16 S;
#pragma unroll
        for (int s2 = 0; s2 < 32; ++s2) {
          if (s2 + kAhead < 32) ka[(s2 + kAhead) % (kAhead + 1)] = kread(cb, s2 + kAhead);
          __builtin_amdgcn_sched_barrier(0);
          if (s2 == 0)
            mfma_v_first(S, ka[0], qb[0]);
          else if (s2 < 31)
            mfma_v(S, ka[s2 % (kAhead + 1)], qb[s2]);
          else
            mfma_v_last(S, ka[s2 % (kAhead + 1)], qb[s2]);
          // the next chunk's 16 rows of this wave go out one per two products of the
          // first block, so that the last of them has three quarters of the chunk to land
          if (more && cb == 0 && (s2 & 1)) gather_row(naddr, nbuf, s2 >> 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        // the first V fragments of the block's P V go out before the softmax, which they do
        // not depend on
        auto vread = [&](int j) __attribute__((always_inline)) -> bf16x8 {  // j = 16 p + T, step 2 cb + p of the chunk
          const int p = j >> 4, T = j & 15;
          const u32x2 v1 = lds_read_tr(buf, vb[T & 3][0] + 256 * (T >> 2) + 16384 * (2 * cb + p));
          const u32x2 v2 = lds_read_tr(buf, vb[T & 3][1] + 256 * (T >> 2) + 16384 * (2 * cb + p));
          const u32x4 cat = {v1.x, v1.y, v2.x, v2.y};
          return __builtin_bit_cast(bf16x8, cat);
        };
        bf16x8 vr[kAhead + 1];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) vr[i] = vread(i);
        __builtin_amdgcn_sched_barrier(0);
        // element i: candidate r0 + 32 cb + 8 (i >> 2) + 4 hl + (i & 3), head l32
        const int rb = r0 + 32 * cb;
        if (__builtin_expect(rb + 32 > lim || (xa < xb && rb < xb && rb + 32 > xa), 0)) {
          asm volatile("" ::: "memory");
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int u = rb + 8 * (i >> 2) + 4 * hl + (i & 3);
            if (u >= lim || (u >= xa && u < xb)) S[i] = -INFINITY;
          }
        }
        float lmax = S[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) lmax = fmaxf(lmax, S[i]);
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lmax), __float_as_uint(lmax), false, false);
          lmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * qinv;  // qinv > 0
        }
        mx_run = fmaxf(mx_run, lmax);
        if (c == 0 && cb == 0) {
          m_ref = fmaxf(m_ref, lmax);  // raised by a restart
          if (m_ref == -INFINITY) m_ref = 0.0f;
        } else {
          ovf = ovf || lmax > m_ref + kLazy;
        }
        bf16x8 pb[2];
        float ls = 0.0f;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          float pr[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) pr[e] = __builtin_amdgcn_exp2f(fmaf(S[8 * p + e], qinv, -m_ref));
#pragma unroll
          for (int e = 0; e < 8; ++e) ls += pr[e];
          const u32x4 pk = {pk_bf16(pr[0], pr[1]), pk_bf16(pr[2], pr[3]), pk_bf16(pr[4], pr[5]), pk_bf16(pr[6], pr[7])};
          pb[p] = __builtin_bit_cast(bf16x8, pk);
        }
        l_part += ls;
        // O^T[channel tile T][32 heads] += V^T P^T over the block's 2 steps of 16 candidates
        // (the first V fragments were read before the softmax)
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          if (j + kAhead < 32) vr[(j + kAhead) % (kAhead + 1)] = vread(j + kAhead);
          __builtin_amdgcn_sched_barrier(0);
          O[j & 15] = mfma32(vr[j % (kAhead + 1)], pb[j >> 4], O[j & 15]);
          if (cb == 0 && j >= 32 - kAhead) ka[j - (32 - kAhead)] = kread(1, j - (32 - kAhead));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    for (int c = 0; c + 1 < nchunks; ++c) chunk(c, std::true_type{});
    chunk(nchunks - 1, std::false_type{});
    // an overflow is acted on once the pass is over (every wave restarts together)
    {
      const bool any = __ballot(ovf) != 0;
      if (lane == 0) flag_s[wv] = any ? 1 : 0;
    }
    wait_lgkmcnt<0>();
    block_sync();  // flags visible
    if (!uni(flag_s[0] | flag_s[1] | flag_s[2] | flag_s[3])) return true;
    m_ref = fmaxf(m_ref, mx_run);
    return false;
  };

  f32x16 O[16];
  float l_part;
  for (;;) {
    if (__builtin_expect(run(O, l_part), 1)) break;
    wait_vmcnt<0>();
    block_sync();  // every wave is done with the chunk buffers
    fill0();
  }

  // ---- epilogue: normalise (+ sink), inverse RoPE, bf16 through LDS, whole-row stores --
  float inv;
  {
    float den = l_part + __shfl_xor(l_part, 32, 64);
    if (a.sink) den += __builtin_amdgcn_exp2f(a.sink[hgrp * kHG + 32 * hh + l32] * kLog2e - m_ref);
    inv = 1.0f / den;
  }
  wait_vmcnt<0>();
  block_sync();  // every wave is done with the chunk buffers
  // wave wv stages its 32 heads x 512 channels in kvbuf[32 KiB wv ..]: row = head, the
  // 16-byte chunk j of a row at position j ^ (head & 15)
  char* tb = kvbuf + wv * 32768;
  // lane (hl, l32) holds head l32 at channels 32 T + 8 j + 4 hl + (0..3) in O[T][4 j .. + 3]
#pragma unroll
  for (int T = 0; T < 16; ++T) {
    uint32_t pk[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x[4] = {O[T][4 * j] * inv, O[T][4 * j + 1] * inv, O[T][4 * j + 2] * inv, O[T][4 * j + 3] * inv};
      if (T >= 14) {
        // pairs (ch, ch + 1), ch = 32 T + 8 j + 4 hl + 2 e, frequency (ch - 448) / 2
        const int f = 16 * (T - 14) + 4 * j + 2 * hl;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float cs = rope_c[qq][f + e], sn = rope_s[qq][f + e];
          const float x0 = x[2 * e], x1 = x[2 * e + 1];
          x[2 * e] = x0 * cs + x1 * sn;
          x[2 * e + 1] = x1 * cs - x0 * sn;
        }
      }
      pk[j][0] = pk_bf16(x[0], x[1]);
      pk[j][1] = pk_bf16(x[2], x[3]);
    }
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      // the lower half keeps group 2 jp and takes the upper half's; the upper half keeps
      // group 2 jp + 1 and takes the lower half's: channels 32 T + 16 jp + 8 hl .. + 7
      const auto w0 = __builtin_amdgcn_permlane32_swap(pk[2 * jp][0], pk[2 * jp + 1][0], false, false);
      const auto w1 = __builtin_amdgcn_permlane32_swap(pk[2 * jp][1], pk[2 * jp + 1][1], false, false);
      const u32x4 v = {w0[0], w1[0], w0[1], w1[1]};
      const int cidx = 4 * T + 2 * jp + hl;
      *reinterpret_cast<u32x4*>(tb + l32 * kRowBytes + ((cidx ^ (l32 & 15)) << 4)) = v;
    }
  }
  asm volatile("" ::: "memory");  // LDS operations of a wave complete in order
  if (qq == 0 || pair) {
    uint16_t* dst = a.out + (((int64_t)b * a.T + qi) * a.n_h + (int64_t)hgrp * kHG + 32 * hh) * kC;
#pragma unroll 4
    for (int h = 0; h < 32; ++h) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(tb + h * kRowBytes + ((lane ^ (h & 15)) << 4));
      *reinterpret_cast<u32x4*>(dst + (int64_t)h * kC + 8 * lane) = v;
    }
  }
}

}  // namespace

// ---------------------------------------------------------------- host side --

hipError_t launch_kv576_gather(const void* kv, const float* kv_scale, const int32_t* idx,
                               const int32_t* cnt, const SeqState& seq, int64_t E_cap, int batch,
                               int k, int rope_dims, void* staged, hipStream_t s) {
  hipLaunchKernelGGL(kv576_gather_kernel, dim3((unsigned)((k + 3) / 4), (unsigned)batch), dim3(256), 0,
                     s, reinterpret_cast<const uint8_t*>(kv), kv_scale, idx, cnt, seq, E_cap, k,
                     rope_dims, reinterpret_cast<uint16_t*>(staged));
  return hipGetLastError();
}

bool attn_mfma_supported(const AttnArgs& a) {
  return a.dt == kBF16 && a.c == kC && a.n_h % kHG == 0 && (a.rope_dims == 0 || a.rope_dims == 64) &&
         (a.mode == kModeHCA || a.mode == kModeHCADecode || (int64_t)a.k + a.w <= kMaxCand);
}

static bool is_decode(const AttnArgs& a) { return a.mode == kModeDecode || a.mode == kModeHCADecode; }

static int64_t local_rows(const AttnArgs& a) {
  if (is_decode(a)) return a.w;
  const int64_t lo = a.t0 - a.w + 1 > 0 ? a.t0 - a.w + 1 : 0;
  return a.t0 + a.T - lo;
}

// longest candidate list of a decode call: k + w (CSA), or every completed entry of the
// latest position plus w (HCA)
int64_t decode_max_list(const AttnArgs& a) {
  if (a.mode == kModeHCADecode && !a.dense_cnt) return (a.t0 + 1) / a.m_prime + a.w;
  return (int64_t)a.k + a.w;
}

static int decode_split_len(const AttnArgs& a) {
  const int64_t N = decode_max_list(a);
  int64_t per = (N + a.num_splits - 1) / a.num_splits;
  return (int)per;
}

// workspace: [window rows bf16][decode partials f32]
size_t attn_mfma_workspace(const AttnArgs& a) {
  size_t loc = ((size_t)a.batch * local_rows(a) * kC * 2 + 255) / 256 * 256;
  size_t part = 0;
  if (is_decode(a) && a.num_splits > 1)
    part = ((size_t)a.batch * a.num_splits * a.n_h * (kC + 2) * sizeof(float) + 255) / 256 * 256;
  return loc + part;
}

hipError_t launch_attention_merge(const AttnArgs& a, const float* part, hipStream_t s);

// workspace pieces: [window rows bf16][decode partials f32]
struct MfmaWs {
  uint16_t* lws;
  float* part;
};
static MfmaWs mfma_ws(const AttnArgs& a, void* ws) {
  const int64_t nl_rows = local_rows(a);
  MfmaWs w;
  w.lws = reinterpret_cast<uint16_t*>(ws);
  const size_t loc_bytes = ((size_t)a.batch * nl_rows * kC * 2 + 255) / 256 * 256;
  w.part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + loc_bytes);
  return w;
}

static LocalPrepArgs prep_args(const AttnArgs& a, const MfmaWs& w) {
  LocalPrepArgs lp{};
  lp.gamma = a.kv_gamma;
  lp.ws = w.lws;
  lp.n_lrows = local_rows(a);
  lp.rope_dims = a.rope_dims;
  lp.eps = a.eps;
  lp.rope_base = a.rope_base;
  lp.rope = a.rope;
  lp.w = a.w;
  lp.tpos = a.seq.tpos;
  if (is_decode(a)) {
    lp.src = reinterpret_cast<const uint16_t*>(a.kv_local);
    lp.ring = reinterpret_cast<uint16_t*>(a.kv_ring);
    lp.kv_new = reinterpret_cast<const uint16_t*>(a.kv_new);
    lp.t = a.t0;
    lp.lrow_base = a.t0 - a.w + 1 > 0 ? a.t0 - a.w + 1 : 0;
    lp.decode = 1;
  } else {
    lp.src = reinterpret_cast<const uint16_t*>(a.kv_local);
    lp.loc_base = a.loc_base;
    lp.n_loc = a.n_loc;
    lp.lrow_base = a.t0 - a.w + 1 > 0 ? a.t0 - a.w + 1 : 0;
    lp.t = a.t0 + a.T - 1;
    lp.decode = 0;
  }
  return lp;
}

static bool tail_rows_ok(const CompressArgs& a) {
  if (a.n_entries <= 0) return true;
  const int npos = a.overlap ? 2 * a.m : a.m;
  return a.in_dt == kBF16 && npos <= 8 && (a.c == 128 || a.c == 256 || a.c == 512);
}

bool decode_front_supported(const CompressArgs& cm, const CompressArgs& ci, const AttnArgs& a,
                            int policy) {
  return is_decode(a) && policy == 0 && attn_mfma_supported(a) && tail_rows_ok(cm) &&
         tail_rows_ok(ci) && cm.batch == a.batch && ci.batch == a.batch;
}

hipError_t decode_front_args(const CompressArgs& cm, const AttnArgs& a, void* attn_ws,
                             FrontArgs& out) {
  out.cm = cm;
  out.lp = prep_args(a, mfma_ws(a, attn_ws));
  out.n_prep = (int)((out.lp.n_lrows + kFrontRows - 1) / kFrontRows);
  out.gm = cm.n_entries > 0 ? cm.c / 8 : 64;
  out.n_comp = cm.n_entries > 0 ? (int)(((int64_t)cm.n_entries + 64 / out.gm - 1) / (64 / out.gm)) : 0;
  if (out.gm != 16 && out.gm != 32 && out.gm != 64) return hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_decode_front(const CompressArgs& cm, const CompressArgs& ci, const AttnArgs& a,
                               void* attn_ws, hipStream_t s) {
  const LocalPrepArgs lp = prep_args(a, mfma_ws(a, attn_ws));
  const int n_prep = (int)((lp.n_lrows + kFrontRows - 1) / kFrontRows);
  auto groups = [](const CompressArgs& x) -> int64_t {
    return x.n_entries > 0 ? ((int64_t)x.n_entries + 64 / (x.c / 8) - 1) / (64 / (x.c / 8)) : 0;
  };
  const int64_t gm = groups(cm), gi = groups(ci);
  const int n_comp = (int)(gm > gi ? gm : gi);
  const int64_t nb = n_prep + n_comp;
  const dim3 grid((unsigned)nb, (unsigned)a.batch);
  // instance widths c / 8 (16, 32 or 64 lanes per entry; checked by tail_rows_ok)
  const int GM = cm.n_entries > 0 ? cm.c / 8 : 64, GI = ci.n_entries > 0 ? ci.c / 8 : 16;
#define V4A_FRONT(gm, gi)                                                                     \
  if (GM == gm && GI == gi) {                                                                  \
    hipLaunchKernelGGL((decode_front_kernel<gm, gi>), grid, dim3(256), 0, s, cm, ci, lp, n_comp); \
    return hipGetLastError();                                                                  \
  }
  V4A_FRONT(64, 16) V4A_FRONT(64, 32) V4A_FRONT(64, 64)
  V4A_FRONT(32, 16) V4A_FRONT(32, 32) V4A_FRONT(32, 64)
  V4A_FRONT(16, 16) V4A_FRONT(16, 32) V4A_FRONT(16, 64)
#undef V4A_FRONT
  return hipErrorInvalidValue;
}

hipError_t launch_attention_mfma(const AttnArgs& a, void* ws, hipStream_t s) {
  const int64_t nl_rows = local_rows(a);
  const MfmaWs wsp = mfma_ws(a, ws);
  uint16_t* lws = wsp.lws;
  float* part = wsp.part;
  const LocalPrepArgs lp = prep_args(a, wsp);
  hipError_t err = hipSuccess;
  if (!a.prep_done) {
    hipLaunchKernelGGL(local_prep_kernel, dim3((unsigned)((nl_rows + 3) / 4), (unsigned)a.batch),
                       dim3(256), 0, s, lp);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }

  MqaArgs m{};
  m.q = reinterpret_cast<const uint16_t*>(a.q);
  m.kvc = reinterpret_cast<const uint16_t*>(a.kv_comp);
  m.kvl = lws;
  m.idx = a.idx;
  m.cnt = a.cnt;
  m.sink = a.sink;
  m.q_gamma = a.q_gamma;
  m.out = reinterpret_cast<uint16_t*>(a.out);
  m.part = part;
  m.t0 = a.t0;
  m.E_cap = a.E_cap;
  m.lrow_base = lp.lrow_base;
  m.n_lrows = nl_rows;
  m.T = a.T;
  m.n_h = a.n_h;
  m.k = a.k;
  m.w = a.w;
  m.m_prime = a.m_prime;
  m.rope_dims = a.rope_dims;
  m.mode = a.mode;
  m.eps = a.eps;
  m.rope_base = a.rope_base;
  m.qscale = a.scale * kLog2e;
  m.rope = a.rope;
  m.batch = a.batch;
  m.tpos = a.seq.tpos;
  m.pages = a.seq.pages;
  m.max_pages = a.seq.max_pages;
  m.page_shift = a.seq.page_shift;
  m.staged = a.dense_cnt != nullptr;
  if (a.dense_cnt) m.cnt = a.dense_cnt;
  // one workgroup per item (64 heads of one query, or of one decode split)
  const int64_t hgroups = a.n_h / kHG;
  if (is_decode(a)) {
    m.splits = a.num_splits > 1 ? a.num_splits : 1;
    m.split_len = m.splits > 1 ? decode_split_len(a) : (int)decode_max_list(a);
    const int64_t items = (int64_t)a.batch * hgroups * m.splits;
    if (a.mode == kModeHCADecode)
      hipLaunchKernelGGL(mqa_mfma_kernel<kModeHCADecode>, dim3((unsigned)items), dim3(kThreads), 0, s, m);
    else
      hipLaunchKernelGGL(mqa_mfma_kernel<kModeDecode>, dim3((unsigned)items), dim3(kThreads), 0, s, m);
    err = hipGetLastError();
    // decode splits restart in place on a reference overflow: no recomputation launch
    if (err != hipSuccess || m.splits <= 1) return err;
    return launch_attention_merge(a, part, s);
  }
  m.splits = 1;
  if (a.mode == kModeHCA) {
    // two consecutive positions per workgroup
    const unsigned grid = (unsigned)((int64_t)a.batch * hgroups * ((a.T + 1) / 2));
    hipLaunchKernelGGL(hca_pair_kernel, dim3(grid), dim3(kPairThreads), 0, s, m);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)((int64_t)a.batch * hgroups * a.T);
  hipLaunchKernelGGL(mqa_mfma_kernel<kModeCSA>, dim3(grid), dim3(kThreads), 0, s, m);
  return hipGetLastError();
}

}  // namespace v4a
