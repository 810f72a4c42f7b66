// Device helpers shared by the gfx950 kernels: element formats, RoPE angles,
// wave/block reductions.  Wavefronts are 64 lanes wide.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace v4a {

constexpr float kLog2e = 1.4426950408889634f;

// ----------------------------------------------------------------- formats --

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float((uint32_t)u << 16);
}

// float -> bfloat16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// OCP FP8 E4M3: bias 7, exponent field 0 is subnormal (mantissa * 2^-9).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * (1.0f / 512.0f);
  return (b & 0x80u) ? -v : v;
}

// OCP E2M1 (MXFP4 element): {0, .5, 1, 1.5, 2, 3, 4, 6} with a sign bit.
__device__ __forceinline__ float e2m1_to_f32(uint32_t nib) {
  const uint32_t mag = nib & 7u;
  float v = (mag < 2u) ? 0.5f * (float)mag
                       : __uint_as_float(((mag >> 1) + 126u) << 23) * (1.0f + 0.5f * (float)(mag & 1u));
  return (nib & 8u) ? -v : v;
}

// E8M0 scale: 2^(code - 127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t code) {
  return code == 0 ? 5.877471754111438e-39f /* 2^-127 */ : __uint_as_float(code << 23);
}

// |x| <= 448 -> E4M3 magnitude code, round to nearest even on the grid of its binade.
__device__ __forceinline__ uint32_t f32_to_e4m3_abs(float a) {
  a = fminf(a, 448.0f);
  if (!(a > 0.0f)) return 0u;
  int e = (int)((__float_as_uint(a) >> 23) & 255u) - 127;  // floor(log2 a) for normal floats
  if (e < -6) e = -6;
  const float quantum = __uint_as_float((uint32_t)(e - 3 + 127) << 23);
  float q = rintf(a / quantum) * quantum;
  q = fminf(q, 448.0f);
  if (q < 0.015625f) return (uint32_t)rintf(q * 512.0f);  // subnormal codes
  const int e2 = (int)((__float_as_uint(q) >> 23) & 255u) - 127;
  const uint32_t mant = (__float_as_uint(q) >> 20) & 7u;
  return ((uint32_t)(e2 + 7) << 3) | mant;
}

// |x| (already divided by the block scale) -> E2M1 magnitude code, nearest, ties to even.
__device__ __forceinline__ uint32_t f32_to_e2m1_abs(float a) {
  a = fminf(a, 6.0f);
  // midpoints between grid values; at a midpoint the even code wins
  if (a < 0.25f) return 0u;
  if (a == 0.25f) return 0u;
  if (a < 0.75f) return 1u;
  if (a == 0.75f) return 2u;
  if (a < 1.25f) return 2u;
  if (a == 1.25f) return 2u;
  if (a < 1.75f) return 3u;
  if (a == 1.75f) return 4u;
  if (a < 2.5f) return 4u;
  if (a == 2.5f) return 4u;
  if (a < 3.5f) return 5u;
  if (a == 3.5f) return 6u;
  if (a < 5.0f) return 6u;
  if (a == 5.0f) return 6u;
  return 7u;
}

// Order-preserving map of a float score to uint32 (larger score -> larger key).
// -0 is folded into +0 so that equal values compare equal.
__device__ __forceinline__ uint32_t score_key(float f) {
  // negative: all bits flipped; otherwise the sign bit set (an arithmetic shift of the
  // sign gives the mask in two instructions, without a compare and select)
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ------------------------------------------------------------------- RoPE --

// cos/sin of a RoPE rotation by angle pos * inv_freq.  The angle is formed and
// reduced modulo 2 pi in float64 (Cody-Waite, two-part 2 pi) so that positions up
// to 2^31 keep their precision; only the reduced angle goes through float32
// sincos.  inv_freq = base^(-2i/rope_dims) is computed once on the host.
__device__ __forceinline__ void rope_cs(double pos, double inv_freq, float& cs, float& sn) {
  const double ang = pos * inv_freq;
  const double k = rint(ang * 0.15915494309189535);
  double r = fma(-k, 6.283185307179586, ang);
  r = fma(-k, 2.4492935982947064e-16, r);
  sincosf((float)r, &sn, &cs);
}

// Same rotation with the hardware sine/cosine (argument in revolutions, absolute
// error near 1e-6 after the float64 reduction): for operands that are rounded to
// bfloat16 right after the rotation.
__device__ __forceinline__ void rope_cs_fast(double pos, double inv_freq, float& cs, float& sn) {
  const double rev = pos * inv_freq * 0.15915494309189535;
  const float r = (float)(rev - rint(rev));
  sn = __builtin_amdgcn_sinf(r);
  cs = __builtin_amdgcn_cosf(r);
}

// ------------------------------------------------------------- reductions --

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over the whole block; `red` is LDS scratch of >= blockDim/64 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = 0.0f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = red[0];
  for (int i = 1; i < nw; ++i) t = fmaxf(t, red[i]);
  return t;
}

}  // namespace v4a
