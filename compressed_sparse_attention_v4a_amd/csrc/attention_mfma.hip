// Shared-KV MQA attention on the gfx950 matrix cores (bf16, c = 512, heads in
// groups of 64): CSA prefill, CSA decode (candidate splits) and HCA prefill.
//
// What it computes is the core attention of "CSA And HCA: Definition, State,
// And Cost Model" (sections 3.2, 4, 5.1-5.3): per query position t and head h,
// one softmax over the candidate list (compressed entries || window rows), each
// row serving as key and value of every head, a sink logit in the denominator,
// and inverse RoPE at t on the output.
//
// Work decomposition (one workgroup = one query position x 64 heads, 4 waves):
//   * Candidate rows (1 KiB each) stream through LDS 64 at a time, double
//     buffered, gathered with direct global->LDS 16-byte loads (one row per
//     instruction).  The 16-byte chunks of a row are XOR-swizzled by a function
//     of the row so that both read patterns below are bank-conflict free.
//   * Scores S^T = K Q^T on v_mfma_f32_16x16x32_bf16: wave v computes heads
//     [16v, 16v+16) against all 64 candidates of the chunk with its 16 query heads
//     resident in registers (RMS-normalised, rotated at t, pre-scaled by
//     scale*log2 e), so each wave owns complete softmax rows.
//   * Softmax with a fixed reference maximum per row (the first chunk's maximum):
//     probabilities are exp2(s - m_ref), at most 2^64, so O needs no rescaling;
//     if a later row maximum exceeds the reference by more than that, the
//     workgroup restarts its candidate loop with the larger reference (exact in
//     every case, and never triggered for normalised queries and rows).  The
//     probabilities are rounded to bf16 and written to LDS in the order the PV
//     operands need.
//   * O += P V: wave v owns 128 output channels (16-channel tiles interleaved
//     across the waves) of all 64 heads
//     (fp32 accumulators in registers), reading P from LDS and V straight from
//     the row-major tile with the gfx950 transposing LDS read.
//   * Epilogue: normalisation (+ sink), inverse RoPE, bf16 output staged through
//     LDS for coalesced 16-byte stores; the decode form writes float32 partial
//     states (unnormalised O, running max, running sum) for the merge kernel.
// Local window rows are normalised and rotated once by a pre-pass into a bf16
// workspace, so every candidate is a plain row gather.
#include "device_common.h"
#include "internal.h"

namespace v4a {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((address_space(3))) void* lds_void;

constexpr int kC = 512;        // channels per row
constexpr int kHG = 64;        // heads per workgroup
constexpr int kNC = 64;        // candidates per chunk
constexpr int kRowBytes = kC * 2;
constexpr int kThreads = 256;
constexpr int kMaxCand = 2048; // candidate-list capacity of one workgroup (k + w)
// Probabilities are exp2(s - m_ref) with m_ref fixed after the first chunk.  They
// stay below 2^kLazy; O (|v| < 2^6, at most 2^11 candidates) stays below 2^81, far
// from float32 overflow.  A row max that grows further restarts the candidate loop
// with the larger reference, so O is never rescaled and never leaves the
// accumulation registers.
constexpr float kLazy = 64.0f;

// XOR applied to the 16-byte chunk index of row r (keeps the chunk in its row).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// 16-byte chunk of a row read by lane group g in score k-step s (8 channels).  The
// step's high bits sit above the swizzle bits, so each lane's addresses for all
// steps are two base registers plus immediate offsets.
__device__ __forceinline__ int kchunk(int s, int g) { return 8 * (s >> 1) + 2 * g + (s & 1); }

// First output channel of PV tile nt of wave wv: tiles of 16 channels interleave
// across waves (chunk pair 2wv + 8nt), keeping the tile index above the swizzle bits.
__device__ __forceinline__ int ochan(int wv, int nt) { return 16 * wv + 64 * nt; }

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
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
  int T, n_h, k, w, m_prime, rope_dims, mode, splits, split_len;
  float eps, rope_base, qscale;
  RopeTab rope;
};

__device__ __forceinline__ bf16x8 lds_read_b128(const char* base, int off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}

__device__ __forceinline__ u32x2 lds_read_tr(const char* base, int off) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(
      (__attribute__((address_space(3))) char*)(base) + off));
  return __builtin_bit_cast(u32x2, v);
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void mqa_mfma_kernel(MqaArgs a) {
  __shared__ __attribute__((aligned(1024))) char kvbuf[2 * kNC * kRowBytes];  // double buffer
  __shared__ __attribute__((aligned(16))) char ps[kHG * kNC * 2];  // P, [head][slot] bf16
  __shared__ int rowid_s[MODE == kModeHCA ? 1 : kMaxCand];
  __shared__ int rescale_s[4];
  __shared__ float fin_m[kHG], fin_l[kHG];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 4, j = lane & 15;
  const int b = blockIdx.z;
  const int hgrp = blockIdx.y;
  const bool decode = MODE == kModeDecode;
  const int qi = decode ? 0 : blockIdx.x;            // query row within the chunk
  const int split = decode ? blockIdx.x : 0;
  const int64_t t = decode ? a.t0 : a.t0 + qi;
  const int nq = decode ? 1 : a.T;

  // ---- candidate list of this query --------------------------------------
  int64_t ncomp;
  if (MODE == kModeHCA) {
    ncomp = (t + 1) / a.m_prime;
  } else {
    const int64_t qrow = (int64_t)b * nq + qi;
    ncomp = min(max(a.cnt[qrow], 0), a.k);
  }
  const int64_t lo = t - a.w + 1 > 0 ? t - a.w + 1 : 0;
  const int64_t N = ncomp + (t - lo + 1);
  int64_t ub = 0, ue = N;
  if (decode) {
    ub = min((int64_t)split * a.split_len, N);
    ue = min(ub + a.split_len, N);
  }
  const int64_t nrows = ue - ub;
  const int pad_id = -1 - (int)(t - a.lrow_base);  // the query's own window row
  // row id of candidate u: entry index (>= 0) or -(1 + window workspace row)
  if (MODE != kModeHCA) {
    const int32_t* idx = a.idx + ((int64_t)b * nq + qi) * a.k;
    for (int64_t r = tid; r < nrows; r += kThreads) {
      const int64_t u = ub + r;
      int id;
      if (u < ncomp) {
        int64_t e = idx[u];
        id = (int)min(max(e, (int64_t)0), a.E_cap - 1);  // out-of-range indices must not fault
      } else {
        id = -1 - (int)(lo + (u - ncomp) - a.lrow_base);
      }
      rowid_s[r] = id;
    }
    __syncthreads();
  }
  const char* kvc_b = reinterpret_cast<const char*>(a.kvc + (int64_t)b * a.E_cap * kC);
  const char* kvl_b = reinterpret_cast<const char*>(a.kvl + (int64_t)b * a.n_lrows * kC);
  const int lane_off = lane << 4;

  // wave wv gathers rows [16 wv, 16 wv + 16) of chunk starting at candidate offset r0
  auto fill = [&](char* buf, int64_t r0) {
    int myid = pad_id;
    const int64_t rr = r0 + 16 * wv + j;
    if (MODE == kModeHCA) {
      const int64_t u = ub + rr;
      if (rr < nrows) myid = u < ncomp ? (int)u : -1 - (int)(lo + (u - ncomp) - a.lrow_base);
    } else if (rr < nrows) {
      myid = rowid_s[rr];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int id = __builtin_amdgcn_readlane(myid, r);
      const int R = 16 * wv + r;
      const char* rowp = id >= 0 ? kvc_b + (int64_t)id * kRowBytes : kvl_b + (int64_t)(-1 - id) * kRowBytes;
      __builtin_amdgcn_global_load_lds(rowp + (lane_off ^ (swz(R) << 4)), (lds_void)(buf + R * kRowBytes),
                                       16, 0, 0);
    }
  };

  const int64_t nchunks = (nrows + kNC - 1) / kNC;
  if (nchunks > 0) fill(kvbuf, 0);

  // ---- resident query heads (B operand of S^T = K Q^T) -----------------
  // lane (g, j) holds head 16 wv + j, channels 32 ks + 8 g .. +7
  bf16x8 qb[16];
  {
    const int64_t qrow0 = ((int64_t)b * nq + qi) * a.n_h + (int64_t)hgrp * kHG + wv * 16;
    float cs[8], sn[8];
    const int r0 = kC - a.rope_dims;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      // pairs in k-steps 14, 15 (channels 448..511) when rope_dims == 64
      const int d = 8 * kchunk(14 + p / 4, g) + 2 * (p % 4);
      if (a.rope_dims > 0 && d >= r0) {
        rope_cs((double)t, a.rope.inv_freq[(d - r0) >> 1], cs[p], sn[p]);
      } else {
        cs[p] = 1.0f;
        sn[p] = 0.0f;
      }
    }
    {
      const uint16_t* qr = a.q + (qrow0 + j) * kC;
      // pass 1: sum of squares of the head row (4 lanes share a row)
      float ss = 0.0f;
#pragma unroll 4
      for (int ks = 0; ks < 16; ++ks) {
        const uint4 v = *reinterpret_cast<const uint4*>(qr + 8 * kchunk(ks, g));
        const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = __uint_as_float(wds[e] << 16), x1 = __uint_as_float(wds[e] & 0xFFFF0000u);
          ss = fmaf(x0, x0, ss);
          ss = fmaf(x1, x1, ss);
        }
      }
      float inv = a.qscale;
      if (a.q_gamma) {
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        inv = a.qscale / sqrtf(ss / (float)kC + a.eps);
      }
      // pass 2: normalise, rotate, scale, round to bf16
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const uint4 v = *reinterpret_cast<const uint4*>(qr + 8 * kchunk(ks, g));
        const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
        float y[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[2 * e] = __uint_as_float(wds[e] << 16);
          y[2 * e + 1] = __uint_as_float(wds[e] & 0xFFFF0000u);
        }
        if (a.q_gamma) {
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] *= a.q_gamma[8 * kchunk(ks, g) + e];
        }
        if (ks >= 14) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const int p = (ks - 14) * 4 + e / 2;
            const float y0 = y[e], y1 = y[e + 1];
            y[e] = y0 * cs[p] - y1 * sn[p];
            y[e + 1] = y0 * sn[p] + y1 * cs[p];
          }
        }
        const u32x4 pk = {pk_bf16(y[0] * inv, y[1] * inv), pk_bf16(y[2] * inv, y[3] * inv),
                          pk_bf16(y[4] * inv, y[5] * inv), pk_bf16(y[6] * inv, y[7] * inv)};
        qb[ks] = __builtin_bit_cast(bf16x8, pk);
      }
    }
  }

  // ---- main loop ----------------------------------------------------------
  f32x4 O[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) O[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_ref = -INFINITY;
  float l_run = 0.0f;

  // Per-lane LDS byte offsets; everything step-dependent below is an immediate.
  //   score reads: row 16 ct + j, chunk kchunk(s, g) ^ swz(j) = 8 (s >> 1) + ((2g + (s & 1)) ^ swz(j))
  const int sbase0 = j * kRowBytes + (((2 * g) ^ swz(j)) << 4);
  const int sbase1 = j * kRowBytes + (((2 * g + 1) ^ swz(j)) << 4);
  //   transposed V reads: row 32 kk + 4 g + (j >> 2) (+16), chunk (2 wv + 8 nt + h) ^ swz(row)
  const int trow = 4 * g + (j >> 2);
  const int tbase = trow * kRowBytes + (((2 * wv + ((j & 3) >> 1)) ^ swz(trow)) << 4) + 8 * (j & 1);
  //   P reads: head 16 mt + j, slot chunk (4 kk + g) ^ (j & 7)
  const int pbase0 = j * 128 + (((0 + g) ^ (j & 7)) << 4);
  const int pbase1 = j * 128 + (((4 + g) ^ (j & 7)) << 4);

  for (int64_t c = 0; c < nchunks;) {
    const int64_t r0 = c * kNC;
    const int cur = (int)(c & 1) * (kNC * kRowBytes);
    const char* buf = kvbuf + cur;
    char* nbuf = kvbuf + ((kNC * kRowBytes) - cur);
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // chunk c landed for every wave; chunk c-1 fully consumed
    if (c + 1 < nchunks) fill(nbuf, r0 + kNC);
    __builtin_amdgcn_sched_barrier(0);

    // S^T tiles: [ct] -> lane (g, j): head 16 wv + j, candidates 16 ct + 4 g + i
    f32x4 S[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) S[ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // k-steps are software-pipelined two deep: the reads of step ks + 2 are issued
    // before the MFMAs of step ks (program order pinned by scheduling barriers)
    bf16x8 ka[3][4];
    auto kread = [&](int ks, bf16x8* dst) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        dst[ct] = lds_read_b128(buf, ((ks & 1) ? sbase1 : sbase0) + ct * 16 * kRowBytes + 128 * (ks >> 1));
    };
    kread(0, ka[0]);
    kread(1, ka[1]);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      if (ks + 2 < 16) kread(ks + 2, ka[(ks + 2) % 3]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        S[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks % 3][ct], qb[ks], S[ct], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // mask candidates past the end of the list (last chunk only)
    if (c + 1 == nchunks) {
      const int lim = (int)(nrows - r0);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * ct + 4 * g + i >= lim) S[ct][i] = -INFINITY;
    }
    float cmax = -INFINITY;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, S[ct][i]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    // reference maximum: set by the first chunk, moved only through a restart
    bool restart = false;
    if (c == 0 && m_ref == -INFINITY) {
      m_ref = cmax;
    } else if (cmax > m_ref + kLazy) {
      m_ref = cmax;
      restart = true;
    }
    {
      float ls = 0.0f;
      float pv[16];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float z = S[ct][i];
          const float p = (z == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(z - m_ref);
          ls += p;
          pv[ct * 4 + i] = p;
        }
      l_run += ls;
      const int head = wv * 16 + j;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // slots 32 kk + 8 g .. +7 hold candidates 32 kk + {4g .. 4g+3, 16+4g .. 16+4g+3}
        const float* p0 = pv + 8 * kk;
        const u32x4 pk = {pk_bf16(p0[0], p0[1]), pk_bf16(p0[2], p0[3]), pk_bf16(p0[4], p0[5]),
                          pk_bf16(p0[6], p0[7])};
        *reinterpret_cast<u32x4*>(ps + head * 128 + (((4 * kk + g) ^ (head & 7)) << 4)) = pk;
      }
      const bool any = __ballot(restart) != 0;
      if (lane == 0) rescale_s[wv] = any ? 1 : 0;
    }
    __builtin_amdgcn_s_barrier();

    if (rescale_s[0] | rescale_s[1] | rescale_s[2] | rescale_s[3]) {
      // a reference maximum moved: drop the partial sums and start the list again
      wait_vmcnt<0>();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) O[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      l_run = 0.0f;
      c = 0;
      __builtin_amdgcn_s_barrier();  // every wave is done with both buffers
      fill(kvbuf, 0);
      continue;
    }

    // O[64 heads][channels of wave wv] += P V
    __builtin_amdgcn_sched_barrier(0);
    // PV: P fragments per 32-candidate step, V fragments read two tiles ahead
    bf16x8 pa[2][4];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        pa[kk][mt] = *reinterpret_cast<const bf16x8*>(ps + (kk ? pbase1 : pbase0) + mt * 16 * 128);
    auto vread = [&](int it) -> bf16x8 {
      // it = kk * 8 + nt: rows 32 kk + trow and +16, output channels ochan(wv, nt) .. +15
      const int toff = tbase + (it >> 3) * 32 * kRowBytes + (it & 7) * 128;
      const u32x2 v1 = lds_read_tr(buf, toff);
      const u32x2 v2 = lds_read_tr(buf, toff + 16 * kRowBytes);
      const u32x4 cat = {v1.x, v1.y, v2.x, v2.y};
      return __builtin_bit_cast(bf16x8, cat);
    };
    bf16x8 vb[3];
    vb[0] = vread(0);
    vb[1] = vread(1);
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      if (it + 2 < 16) vb[(it + 2) % 3] = vread(it + 2);
      __builtin_amdgcn_sched_barrier(0);
      const int kk = it >> 3, nt = it & 7;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        O[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[kk][mt], vb[it % 3], O[mt][nt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    ++c;
  }

  // ---- epilogue -------------------------------------------------------------
  {
    float l = l_run;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int head = wv * 16 + j;
    if (g == 0) {
      fin_l[head] = l;
      fin_m[head] = m_ref;
    }
  }
  __syncthreads();

  if (decode && a.splits > 1) {
    // partial state: [b][split][h][c + 2] = (O unnormalised, reference max, sum)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int head = 16 * mt + 4 * g + i;
        const int64_t hglob = (int64_t)hgrp * kHG + head;
        float* pr = a.part + (((int64_t)b * a.splits + split) * a.n_h + hglob) * (kC + 2);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) pr[ochan(wv, nt) + j] = O[mt][nt][i];
        if (wv == 0 && j == 0) {
          pr[kC] = fin_m[head];
          pr[kC + 1] = fin_l[head];
        }
      }
    return;
  }

  // normalise, inverse RoPE, stage bf16 rows in LDS (reusing kv0) and store
  uint16_t* stage = reinterpret_cast<uint16_t*>(kvbuf);  // [64 heads][512]
  const int r0 = kC - a.rope_dims;
  float cs8[8], sn8[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int d = ochan(wv, nt) + j;
    if (a.rope_dims > 0 && d >= r0) {
      rope_cs(-(double)t, a.rope.inv_freq[(d - r0) >> 1], cs8[nt], sn8[nt]);
    } else {
      cs8[nt] = 1.0f;
      sn8[nt] = 0.0f;
    }
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = 16 * mt + 4 * g + i;
      float den = fin_l[head];
      if (a.sink) den += __builtin_amdgcn_exp2f(a.sink[hgrp * kHG + head] * kLog2e - fin_m[head]);
      const float inv = 1.0f / den;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        float x = O[mt][nt][i] * inv;
        const float other = __shfl_xor(x, 1, 64);
        x = (j & 1) ? other * sn8[nt] + x * cs8[nt] : x * cs8[nt] - other * sn8[nt];
        stage[head * kC + ochan(wv, nt) + j] = f32_to_bf16(x);
      }
    }
  __syncthreads();
  uint16_t* dst = a.out + (((int64_t)b * nq + qi) * a.n_h + (int64_t)hgrp * kHG) * kC;
#pragma unroll
  for (int it = 0; it < (kHG * kC) / (8 * kThreads); ++it) {
    const int e = (it * kThreads + tid) * 8;
    *reinterpret_cast<uint4*>(dst + e) = *reinterpret_cast<const uint4*>(stage + e);
  }
}

// Normalise and rotate the window rows once into a bf16 workspace.
//   prefill/HCA: ws row r <- local position lrow_base + r
//   decode:      ws row r <- position lo + r read from the ring (token t from kv_new),
//                and kv_new is written into ring slot t % w
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
};

__global__ __launch_bounds__(256) void local_prep_kernel(LocalPrepArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (r >= a.n_lrows) return;
  const int64_t pos = a.lrow_base + r;
  const uint16_t* src;
  if (a.decode) {
    if (pos > a.t) return;
    src = (pos == a.t && a.kv_new) ? a.kv_new + (int64_t)b * kC
                                   : a.src + ((int64_t)b * a.w + pos % a.w) * kC;
  } else {
    src = a.src + ((int64_t)b * a.n_loc + (pos - a.loc_base)) * kC;
  }
  const uint4 v = *reinterpret_cast<const uint4*>(src + 8 * lane);
  if (a.decode && pos == a.t && a.kv_new)
    *reinterpret_cast<uint4*>(a.ring + ((int64_t)b * a.w + a.t % a.w) * kC + 8 * lane) = v;
  const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
  float x[8];
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(wds[e] << 16);
    x[2 * e + 1] = __uint_as_float(wds[e] & 0xFFFF0000u);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
  if (a.gamma) {
    const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)kC + a.eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] * inv * a.gamma[8 * lane + e];
  }
  const int r0 = kC - a.rope_dims;
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const int d = 8 * lane + e;
    float y0 = x[e], y1 = x[e + 1];
    if (a.rope_dims > 0 && d >= r0) {
      float cs, sn;
      rope_cs((double)pos, a.rope.inv_freq[(d - r0) >> 1], cs, sn);
      const float z0 = y0 * cs - y1 * sn, z1 = y0 * sn + y1 * cs;
      y0 = z0;
      y1 = z1;
    }
    o[e / 2] = (uint32_t)f32_to_bf16(y0) | ((uint32_t)f32_to_bf16(y1) << 16);
  }
  *reinterpret_cast<uint4*>(a.ws + ((int64_t)b * a.n_lrows + r) * kC + 8 * lane) =
      make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

// ---------------------------------------------------------------- host side --

bool attn_mfma_supported(const AttnArgs& a) {
  return a.dt == kBF16 && a.c == kC && a.n_h % kHG == 0 && (a.rope_dims == 0 || a.rope_dims == 64) &&
         (a.mode == kModeHCA || (int64_t)a.k + a.w <= kMaxCand);
}

static int64_t local_rows(const AttnArgs& a) {
  if (a.mode == kModeDecode) return a.w;
  const int64_t lo = a.t0 - a.w + 1 > 0 ? a.t0 - a.w + 1 : 0;
  return a.t0 + a.T - lo;
}

static int decode_split_len(const AttnArgs& a) {
  const int64_t N = (int64_t)a.k + a.w;
  int64_t per = (N + a.num_splits - 1) / a.num_splits;
  return (int)per;
}

size_t attn_mfma_workspace(const AttnArgs& a) {
  size_t loc = ((size_t)a.batch * local_rows(a) * kC * 2 + 255) / 256 * 256;
  size_t part = 0;
  if (a.mode == kModeDecode && a.num_splits > 1)
    part = (size_t)a.batch * a.num_splits * a.n_h * (kC + 2) * sizeof(float);
  return loc + part;
}

hipError_t launch_attention_merge(const AttnArgs& a, const float* part, hipStream_t s);

hipError_t launch_attention_mfma(const AttnArgs& a, void* ws, hipStream_t s) {
  const int64_t nl_rows = local_rows(a);
  uint16_t* lws = reinterpret_cast<uint16_t*>(ws);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                         ((size_t)a.batch * nl_rows * kC * 2 + 255) / 256 * 256);
  LocalPrepArgs lp{};
  lp.gamma = a.kv_gamma;
  lp.ws = lws;
  lp.n_lrows = nl_rows;
  lp.rope_dims = a.rope_dims;
  lp.eps = a.eps;
  lp.rope_base = a.rope_base;
  lp.rope = a.rope;
  lp.w = a.w;
  if (a.mode == kModeDecode) {
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
  hipLaunchKernelGGL(local_prep_kernel, dim3((unsigned)((nl_rows + 3) / 4), (unsigned)a.batch),
                     dim3(256), 0, s, lp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

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
  const unsigned hgroups = (unsigned)(a.n_h / kHG);
  if (a.mode == kModeDecode) {
    m.splits = a.num_splits > 1 ? a.num_splits : 1;
    m.split_len = m.splits > 1 ? decode_split_len(a) : (a.k + a.w);
    hipLaunchKernelGGL(mqa_mfma_kernel<kModeDecode>, dim3((unsigned)m.splits, hgroups, (unsigned)a.batch),
                       dim3(kThreads), 0, s, m);
    err = hipGetLastError();
    if (err != hipSuccess || m.splits <= 1) return err;
    return launch_attention_merge(a, part, s);
  }
  m.splits = 1;
  if (a.mode == kModeHCA)
    hipLaunchKernelGGL(mqa_mfma_kernel<kModeHCA>, dim3((unsigned)a.T, hgroups, (unsigned)a.batch),
                       dim3(kThreads), 0, s, m);
  else
    hipLaunchKernelGGL(mqa_mfma_kernel<kModeCSA>, dim3((unsigned)a.T, hgroups, (unsigned)a.batch),
                       dim3(kThreads), 0, s, m);
  return hipGetLastError();
}

}  // namespace v4a
