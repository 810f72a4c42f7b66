// Window-row preparation shared by the attention prep kernel and the fused decode front
// kernel: each local (window) row is RMS-normalised with the key weights and rotated at
// its own position once ("CSA And HCA: Definition, State, And Cost Model", section 5.2),
// then stored as bf16 in the attention workspace, so the attention kernels gather every
// candidate as a plain row.  Decode also inserts the new token's row into the ring.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace v4a {
namespace {

constexpr int kWinC = 512;  // channels of a window row (64 lanes x 8)

// Block blk of sequence b (256 threads, tid = thread index): rows 4 blk .. 4 blk + 3, one per wave.
__device__ __forceinline__ void window_prep_block(const LocalPrepArgs& a, int64_t blk, int b, int tid) {
  if (blk == 0 && b == 0 && tid == 0) a.redo[0] = 0;
  const int lane = tid & 63;
  const int64_t r = blk * 4 + (tid >> 6);
  if (r >= a.n_lrows) return;
  const int64_t pos = a.lrow_base + r;
  const uint16_t* src;
  if (a.decode) {
    if (pos > a.t) return;
    src = (pos == a.t && a.kv_new) ? a.kv_new + (int64_t)b * kWinC
                                   : a.src + ((int64_t)b * a.w + pos % a.w) * kWinC;
  } else {
    src = a.src + ((int64_t)b * a.n_loc + (pos - a.loc_base)) * kWinC;
  }
  const uint4 v = *reinterpret_cast<const uint4*>(src + 8 * lane);
  // RMSNorm weights are loaded with the row, not after the reduction
  float4 g0 = make_float4(1.0f, 1.0f, 1.0f, 1.0f), g1 = g0;
  if (a.gamma) {
    g0 = *reinterpret_cast<const float4*>(a.gamma + 8 * lane);
    g1 = *reinterpret_cast<const float4*>(a.gamma + 8 * lane + 4);
  }
  if (a.decode && pos == a.t && a.kv_new)
    *reinterpret_cast<uint4*>(a.ring + ((int64_t)b * a.w + a.t % a.w) * kWinC + 8 * lane) = v;
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
    const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)kWinC + a.eps);
    const float gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] * inv * gw[e];
  }
  const int r0 = kWinC - a.rope_dims;
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
  *reinterpret_cast<uint4*>(a.ws + ((int64_t)b * a.n_lrows + r) * kWinC + 8 * lane) =
      make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace
}  // namespace v4a
