// Register-resident compressor body for entries pooling at most 8 positions (CSA tails
// and prefill, m <= 4 with overlap), shared by the compressor kernel and the fused decode
// front kernel.  What it computes: "CSA And HCA: Definition, State, And Cost Model",
// sections 2.1 (overlapping softmax pooling) and 5.2 (RMSNorm and partial RoPE of an
// emitted entry).
#pragma once

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace v4a {
namespace {

template <typename T>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int N = 4;
  using raw = float4;
  __device__ static void load(const void* base, int64_t off, float* dst) {
    float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
  }
};
template <>
struct Vec<uint16_t> {
  static constexpr int N = 8;
  __device__ static void load(const void* base, int64_t off, float* dst) {
    uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dst[2 * i] = __uint_as_float(w[i] << 16);
      dst[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

// N consecutive float32 (N = 2, 4 or 8), in 16-byte loads where N allows
template <int N>
__device__ __forceinline__ void load_f32(const float* p, float* dst) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int v = 0; v < N; v += 4) {
      const float4 x = *reinterpret_cast<const float4*>(p + v);
      dst[v] = x.x; dst[v + 1] = x.y; dst[v + 2] = x.z; dst[v + 3] = x.w;
    }
  } else {
    const float2 x = *reinterpret_cast<const float2*>(p);
    dst[0] = x.x; dst[1] = x.y;
  }
}

// N consecutive elements (N = 2, 4 or 8) of a row, as float
template <typename T, int N>
__device__ __forceinline__ void load_n(const void* base, int64_t off, float* dst) {
  if constexpr (std::is_same<T, float>::value) {
    load_f32<N>(reinterpret_cast<const float*>(base) + off, dst);
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + off;
    uint32_t w[N / 2];
    if constexpr (N == 8) {
      const uint4 x = *reinterpret_cast<const uint4*>(p);
      w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    } else if constexpr (N == 4) {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      w[0] = x.x; w[1] = x.y;
    } else {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      dst[2 * i] = __uint_as_float(w[i] << 16);
      dst[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

// Sum of squares of the c = G VEC channels of an entry whose lane g of the group holds
// channels g VEC .. g VEC + VEC - 1: a perfect binary tree over the channel index (pairs of
// neighbouring channels, then pairs of pairs, ...), so the rounded result is the same for
// every VEC, i.e. for every lane layout of the entry.  No contraction into FMAs.
template <int VEC, int G>
__device__ __forceinline__ float tree_sum_sq(const float (&x)[VEC]) {
  float sq[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) sq[v] = __fmul_rn(x[v], x[v]);
#pragma unroll
  for (int w = 1; w < VEC; w <<= 1)
#pragma unroll
    for (int v = 0; v < VEC; v += 2 * w) sq[v] = __fadd_rn(sq[v], sq[v + w]);
  float ss = sq[0];
#pragma unroll
  for (int o = 1; o < G; o <<= 1) ss = __fadd_rn(ss, __shfl_xor(ss, o, 64));
  return ss;
}

// Entries pooling at most 8 positions (CSA, m <= 4 with overlap): one group of G = c / VEC
// lanes per entry holds every pooled position in registers, so the softmax needs no merge
// across lanes and the RMSNorm / quantisation maxima are shuffle reductions within the
// group.  Each wave covers 64 / G entries; no LDS, no barriers.  VEC (channels per lane)
// changes only the layout: results are bit-identical for every VEC.
// RMSNorm weights of a call without RMSNorm (read, never applied; VEC <= 8)
__device__ __attribute__((aligned(16))) const float kOnes[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};

// Entry `slot` of the call for sequence b: its index, whether it is emitted, and the
// position of row 0 of the sequence's C/Z buffer.  With per-sequence positions each
// sequence emits at most one entry (slot 0), the one its new token completes.
struct SlotEntry {
  int64_t i, tok_base;
  bool emit;
};
__device__ __forceinline__ SlotEntry slot_entry(const CompressArgs& a, int b, int64_t slot) {
  SlotEntry e;
  if (a.seq.tpos) {
    const int64_t t = a.seq.tpos[b];
    e.i = t / a.m;
    e.emit = slot == 0 && (t + 1) % a.m == 0;
    e.tok_base = (int64_t)a.m * e.i - (a.overlap ? a.m : 0);
  } else {
    e.emit = slot < a.n_entries;
    e.i = a.i_begin + (e.emit ? slot : 0);
    e.tok_base = a.tok_base;
  }
  return e;
}

// One wave: entries 64 / G * vblock .. of sequence b; lane = lane of the wave.
template <typename Tin, int G, int VEC = Vec<Tin>::N>
__device__ __forceinline__ void compress_rows_body(const CompressArgs& a, int64_t vblock, int b, int lane) {
  static_assert(VEC == 2 || VEC == 4 || VEC == 8, "2, 4 or 8 channels per lane");
  constexpr int kMaxPos = 8;
  const int c = a.c, m = a.m;
  const int g = lane % G, ch0 = g * VEC;
  const int64_t slot = vblock * (64 / G) + lane / G;
  const SlotEntry se = slot_entry(a, b, slot);
  const bool valid = se.emit;
  const int64_t i = se.i;
  const int width = a.overlap ? 2 * c : c;
  const int npos = (a.overlap && i > 0) ? 2 * m : m;
  const Tin* Cb = reinterpret_cast<const Tin*>(a.C) + (int64_t)b * a.n_buf * width;
  const Tin* Zb = reinterpret_cast<const Tin*>(a.Z) + (int64_t)b * a.n_buf * width;

  // RMSNorm weights go out with the other loads, not after the reduction
  float gw[VEC];
  {
    const float* gp = a.gamma ? a.gamma + ch0 : kOnes;
    load_f32<VEC>(gp, gw);
  }
  // every load first, with no branch between them (a branch per position would make
  // each position's loads wait for the previous ones): logits and values of the pooled
  // positions (u < m: stream a of block i, else stream b of block i - 1) and the
  // positional bias rows.  Positions past npos read a pooled row of the same entry
  // (always inside the buffer) and get logit -inf.
  float lg[kMaxPos][VEC], cv[kMaxPos][VEC];
#pragma unroll
  for (int u = 0; u < kMaxPos; ++u) {
    const bool use = valid && u < npos;
    const int uu = u < npos ? u : 0;
    const bool sa = uu < m;
    const int64_t pos = sa ? (int64_t)m * i + uu : (int64_t)m * (i - 1) + (uu - m);
    const int64_t off = (pos - se.tok_base) * width + (sa ? 0 : c) + ch0;
    load_n<Tin, VEC>(Zb, off, lg[u]);
    load_n<Tin, VEC>(Cb, off, cv[u]);
    const float* brow = a.B + (int64_t)uu * c + ch0;  // B^a rows 0..m-1, B^b rows m..2m-1
    float bv[VEC];
    load_f32<VEC>(brow, bv);
    // arithmetic masking (the loaded values are finite), so no load sits under a branch
    const float lmask = use ? 0.0f : -INFINITY, cmask = use ? 1.0f : 0.0f;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      lg[u][v] = fmaf(lg[u][v] + bv[v], kLog2e, lmask);
      cv[u][v] *= cmask;
    }
  }
  float x[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    float mx = lg[0][v];
#pragma unroll
    for (int u = 1; u < kMaxPos; ++u) mx = fmaxf(mx, lg[u][v]);
    if (mx == -INFINITY) mx = 0.0f;  // lanes of an entry past the end
    float sm = 0.0f, ac = 0.0f;
#pragma unroll
    for (int u = 0; u < kMaxPos; ++u) {
      const float e = __builtin_amdgcn_exp2f(lg[u][v] - mx);
      sm += e;
      ac = fmaf(e, cv[u][v], ac);
    }
    x[v] = valid ? ac / sm : 0.0f;
  }
  if (a.gamma) {
    const float ss = tree_sum_sq<VEC, G>(x);
    const float inv = 1.0f / sqrtf(ss / (float)c + a.eps);
#pragma unroll
    for (int v = 0; v < VEC; ++v) x[v] = x[v] * inv * gw[v];
  }
  if (a.rope_dims > 0 && ch0 + VEC > c - a.rope_dims) {
    const int r0 = c - a.rope_dims;
    const double pos = (double)((int64_t)m * i);
#pragma unroll
    for (int v = 0; v < VEC; v += 2) {
      const int ch = ch0 + v;
      if (ch >= r0) {
        float cs, sn;
        // float32 entries keep the accurate sine; rounded entries take the hardware one
        if (a.out_dt == kF32) rope_cs(pos, a.rope.inv_freq[(ch - r0) >> 1], cs, sn);
        else rope_cs_fast(pos, a.rope.inv_freq[(ch - r0) >> 1], cs, sn);
        const float x0 = x[v], x1 = x[v + 1];
        x[v] = x0 * cs - x1 * sn;
        x[v + 1] = x0 * sn + x1 * cs;
      }
    }
  }

  const int64_t orow = valid ? cache_row(a.seq, a.E_cap, b, i) : 0;
  if (a.out_dt == kF32) {
    if (valid) {
      float* o = reinterpret_cast<float*>(a.out) + orow * c + ch0;
      if constexpr (VEC % 4 == 0) {
#pragma unroll
        for (int v = 0; v < VEC; v += 4) *reinterpret_cast<float4*>(o + v) = make_float4(x[v], x[v + 1], x[v + 2], x[v + 3]);
      } else {
        *reinterpret_cast<float2*>(o) = make_float2(x[0], x[1]);
      }
    }
  } else if (a.out_dt == kBF16) {
    if (valid) {
      uint32_t w[VEC / 2];
#pragma unroll
      for (int v = 0; v < VEC; v += 2) w[v / 2] = (uint32_t)f32_to_bf16(x[v]) | ((uint32_t)f32_to_bf16(x[v + 1]) << 16);
      uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + orow * c + ch0;
      if constexpr (VEC == 8) *reinterpret_cast<uint4*>(o) = make_uint4(w[0], w[1], w[2], w[3]);
      else if constexpr (VEC == 4) *reinterpret_cast<uint2*>(o) = make_uint2(w[0], w[1]);
      else *reinterpret_cast<uint32_t*>(o) = w[0];
    }
  } else if (a.out_dt == kKV576) {
    // E4M3 codes for channels below c - rope_dims (one scale per row), bf16 above
    const int nq = c - a.rope_dims;
    const bool q8 = ch0 < nq;  // VEC divides rope_dims: a lane is all-codes or all-bf16
    float am = 0.0f;
#pragma unroll
    for (int v = 0; v < VEC; ++v) am = fmaxf(am, q8 ? fabsf(x[v]) : 0.0f);
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    float scale = am / 448.0f;
    if (!(scale > 0.0f)) scale = 1.0f;
    if (valid) {
      uint8_t* o = reinterpret_cast<uint8_t*>(a.out) + orow * kv576_row_bytes(c, a.rope_dims);
      if (q8) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float y = x[v] / scale;
          o[ch0 + v] = (uint8_t)(f32_to_e4m3_abs(fabsf(y)) | (y < 0.0f ? 0x80u : 0u));
        }
      } else {
        uint16_t* ob = reinterpret_cast<uint16_t*>(o + nq);
#pragma unroll
        for (int v = 0; v < VEC; ++v) ob[ch0 - nq + v] = f32_to_bf16(x[v]);
      }
      if (g == 0) reinterpret_cast<float*>(a.out_scale)[orow] = scale;
    }
  } else if (a.out_dt == kFP8) {
    float am = 0.0f;
#pragma unroll
    for (int v = 0; v < VEC; ++v) am = fmaxf(am, fabsf(x[v]));
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    float scale = am / 448.0f;
    if (!(scale > 0.0f)) scale = 1.0f;
    if (valid) {
      uint8_t* o = reinterpret_cast<uint8_t*>(a.out) + orow * c + ch0;
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const float y = x[v] / scale;
        o[v] = (uint8_t)(f32_to_e4m3_abs(fabsf(y)) | (y < 0.0f ? 0x80u : 0u));
      }
      if (g == 0) reinterpret_cast<float*>(a.out_scale)[orow] = scale;
    }
  } else {  // MXFP4: blocks of 32 channels = 32 / VEC consecutive lanes of the group
    constexpr int lpb = 32 / VEC;
    float am = 0.0f;
#pragma unroll
    for (int v = 0; v < VEC; ++v) am = fmaxf(am, fabsf(x[v]));
#pragma unroll
    for (int o = 1; o < lpb; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    if (valid) {
      int sexp = 0;
      if (am > 0.0f) sexp = (int)((__float_as_uint(am) >> 23) & 255u) - 127 - 2;
      if (sexp < -127) sexp = -127;
      if (sexp > 127) sexp = 127;
      const float inv = __uint_as_float((uint32_t)(127 - sexp) << 23);  // 2^-sexp (|sexp| <= 127)
      uint8_t* o = reinterpret_cast<uint8_t*>(a.out) + orow * (c / 2) + ch0 / 2;
#pragma unroll
      for (int v = 0; v < VEC; v += 2) {
        const float y0 = x[v] * inv, y1 = x[v + 1] * inv;
        const uint32_t n0 = f32_to_e2m1_abs(fabsf(y0)) | (y0 < 0.0f ? 8u : 0u);
        const uint32_t n1 = f32_to_e2m1_abs(fabsf(y1)) | (y1 < 0.0f ? 8u : 0u);
        o[v / 2] = (uint8_t)(n0 | (n1 << 4));
      }
      if ((g % lpb) == 0)
        reinterpret_cast<uint8_t*>(a.out_scale)[orow * (c / 32) + ch0 / 32] = (uint8_t)(sexp + 127);
    }
  }
}

}  // namespace
}  // namespace v4a
