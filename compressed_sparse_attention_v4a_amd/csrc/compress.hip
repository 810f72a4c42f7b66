// Learned feature-wise gated compressor and visibility sets.
//
// Compressor: "CSA And HCA: Definition, State, And Cost Model", section 2.1
// (CSA, two streams, overlapping: entry i pools stream a of block i and stream b
// of block i-1 under one per-channel softmax over positions) and section 2.2
// (HCA, one stream, no overlap), followed by the RMSNorm and partial RoPE of
// section 5.2 applied to the emitted entry at its anchor position r*i.
//
// Design (bandwidth-bound): one workgroup of 256 lanes per emitted entry.  Lanes
// own VEC consecutive channels (16-byte loads, so a 64-lane wave reads a full
// 512-channel bf16 row) and the P = 256/(c/VEC) lane groups split the pooled
// positions.  Each lane keeps a per-channel online softmax state (max, sum,
// weighted sum) in float32 with base-2 exponentials, updated four positions at a
// time; the P partial states merge through LDS.  RMSNorm, RoPE and the output
// conversion (f32, bf16, FP8 E4M3 with a row scale, MXFP4 with E8M0 block scales)
// run in the same workgroup, so C and Z are read exactly once and the entry is
// written once.
#include "compress_rows.h"
#include "device_common.h"
#include "internal.h"

namespace v4a {

namespace {

constexpr int kThreads = 256;

template <typename Tin>
__global__ __launch_bounds__(kThreads) void compress_kernel(CompressArgs a) {
  constexpr int VEC = Vec<Tin>::N;
  extern __shared__ float smem[];  // [3][P][c] partial states, then reduction scratch
  const int c = a.c, m = a.m;
  const int G = c / VEC;          // channel groups
  const int P = kThreads / G;     // position splits
  const int tid = threadIdx.x;
  const int g = tid % G, p = tid / G;
  const bool active = p < P;
  const int b = blockIdx.y;
  const SlotEntry se = slot_entry(a, b, blockIdx.x);
  if (!se.emit) return;  // uniform over the workgroup
  const int64_t i = se.i;
  const int width = a.overlap ? 2 * c : c;
  const int npos = (a.overlap && i > 0) ? 2 * m : m;
  const Tin* Cb = reinterpret_cast<const Tin*>(a.C) + (int64_t)b * a.n_buf * width;
  const Tin* Zb = reinterpret_cast<const Tin*>(a.Z) + (int64_t)b * a.n_buf * width;

  float mx[VEC], sm[VEC], acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) { mx[v] = -INFINITY; sm[v] = 0.0f; acc[v] = 0.0f; }

  if (active) {
    const int ch0 = g * VEC;
    // positions u = p, p+P, ... ; u < m: stream a of block i, else stream b of block i-1
    for (int u0 = p; u0 < npos; u0 += 4 * P) {
      float lg[4][VEC], cv[4][VEC];
      int nu = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int u = u0 + r * P;
        if (u < npos) {
          const bool sa = u < m;
          const int64_t pos = sa ? (int64_t)m * i + u : (int64_t)m * (i - 1) + (u - m);
          const int64_t row = pos - se.tok_base;
          const int64_t off = row * width + (sa ? 0 : c) + ch0;
          Vec<Tin>::load(Zb, off, lg[r]);
          Vec<Tin>::load(Cb, off, cv[r]);
          const float* brow = a.B + (int64_t)u * c + ch0;  // B^a rows 0..m-1, B^b rows m..2m-1
#pragma unroll
          for (int v = 0; v < VEC; ++v) lg[r][v] = (lg[r][v] + brow[v]) * kLog2e;
          nu = r + 1;
        }
      }
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        float cm = mx[v];
#pragma unroll
        for (int r = 0; r < 4; ++r) if (r < nu) cm = fmaxf(cm, lg[r][v]);
        const float sc = __builtin_amdgcn_exp2f(mx[v] - cm);
        float s = sm[v] * sc, ac = acc[v] * sc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (r < nu) {
            const float e = __builtin_amdgcn_exp2f(lg[r][v] - cm);
            s += e;
            ac = fmaf(e, cv[r][v], ac);
          }
        }
        mx[v] = cm; sm[v] = s; acc[v] = ac;
      }
    }
  }

  // merge the P partial states of each channel
  float* smx = smem;
  float* ssm = smem + (size_t)P * c;
  float* sac = smem + (size_t)2 * P * c;
  if (active) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const int idx = p * c + g * VEC + v;
      smx[idx] = mx[v]; ssm[idx] = sm[v]; sac[idx] = acc[v];
    }
  }
  __syncthreads();
  float x[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) x[v] = 0.0f;
  const bool owner = tid < G;  // lanes with p == 0 finish the entry
  float ss = 0.0f;
  if (owner) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const int ch = g * VEC + v;
      float M = -INFINITY;
      for (int q = 0; q < P; ++q) M = fmaxf(M, smx[q * c + ch]);
      float S = 0.0f, A = 0.0f;
      for (int q = 0; q < P; ++q) {
        const float f = __builtin_amdgcn_exp2f(smx[q * c + ch] - M);
        S = fmaf(ssm[q * c + ch], f, S);
        A = fmaf(sac[q * c + ch], f, A);
      }
      x[v] = A / S;
      ss = fmaf(x[v], x[v], ss);
    }
  }
  float* red = smem + (size_t)3 * P * c;
  if (a.gamma) {
    const float tot = block_sum(owner ? ss : 0.0f, red);
    const float inv = 1.0f / sqrtf(tot / (float)c + a.eps);
    if (owner) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) x[v] = x[v] * inv * a.gamma[g * VEC + v];
    }
  }
  if (owner && a.rope_dims > 0) {
    const int r0 = c - a.rope_dims;
    const double pos = (double)((int64_t)m * i);
#pragma unroll
    for (int v = 0; v < VEC; v += 2) {
      const int ch = g * VEC + v;
      if (ch >= r0) {
        float cs, sn;
        rope_cs(pos, a.rope.inv_freq[(ch - r0) >> 1], cs, sn);
        const float x0 = x[v], x1 = x[v + 1];
        x[v] = x0 * cs - x1 * sn;
        x[v + 1] = x0 * sn + x1 * cs;
      }
    }
  }

  const int64_t orow = cache_row(a.seq, a.E_cap, b, i);
  if (a.out_dt == kF32) {
    if (owner) {
      float* o = reinterpret_cast<float*>(a.out) + orow * c + g * VEC;
#pragma unroll
      for (int v = 0; v < VEC; ++v) o[v] = x[v];
    }
  } else if (a.out_dt == kBF16) {
    if (owner) {
      uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + orow * c + g * VEC;
#pragma unroll
      for (int v = 0; v < VEC; ++v) o[v] = f32_to_bf16(x[v]);
    }
  } else if (a.out_dt == kKV576) {
    const int nq = c - a.rope_dims;
    float am = 0.0f;
    if (owner) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) am = fmaxf(am, g * VEC + v < nq ? fabsf(x[v]) : 0.0f);
    }
    am = block_max(am, red);
    float scale = am / 448.0f;
    if (!(scale > 0.0f)) scale = 1.0f;
    if (owner) {
      uint8_t* o = reinterpret_cast<uint8_t*>(a.out) + orow * kv576_row_bytes(c, a.rope_dims);
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const int ch = g * VEC + v;
        if (ch < nq) {
          const float y = x[v] / scale;
          o[ch] = (uint8_t)(f32_to_e4m3_abs(fabsf(y)) | (y < 0.0f ? 0x80u : 0u));
        } else {
          reinterpret_cast<uint16_t*>(o + nq)[ch - nq] = f32_to_bf16(x[v]);
        }
      }
      if (g == 0) reinterpret_cast<float*>(a.out_scale)[orow] = scale;
    }
  } else if (a.out_dt == kFP8) {
    float am = 0.0f;
    if (owner) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) am = fmaxf(am, fabsf(x[v]));
    }
    am = block_max(am, red);
    float scale = am / 448.0f;
    if (!(scale > 0.0f)) scale = 1.0f;
    if (owner) {
      uint8_t* o = reinterpret_cast<uint8_t*>(a.out) + orow * c + g * VEC;
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const float y = x[v] / scale;
        o[v] = (uint8_t)(f32_to_e4m3_abs(fabsf(y)) | (y < 0.0f ? 0x80u : 0u));
      }
      if (g == 0) reinterpret_cast<float*>(a.out_scale)[orow] = scale;
    }
  } else {  // MXFP4: blocks of 32 channels = 32/VEC consecutive owner lanes
    const int lpb = 32 / VEC;
    float am = 0.0f;
#pragma unroll
    for (int v = 0; v < VEC; ++v) am = fmaxf(am, fabsf(x[v]));
    for (int o = 1; o < lpb; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    if (owner) {
      int sexp = 0;
      if (am > 0.0f) sexp = (int)((__float_as_uint(am) >> 23) & 255u) - 127 - 2;
      if (sexp < -127) sexp = -127;
      if (sexp > 127) sexp = 127;
      const float inv = __uint_as_float((uint32_t)(127 - sexp) << 23);  // 2^-sexp (|sexp| <= 127)
      uint8_t* o = reinterpret_cast<uint8_t*>(a.out) + orow * (c / 2) + g * VEC / 2;
#pragma unroll
      for (int v = 0; v < VEC; v += 2) {
        const float y0 = x[v] * inv, y1 = x[v + 1] * inv;
        const uint32_t n0 = f32_to_e2m1_abs(fabsf(y0)) | (y0 < 0.0f ? 8u : 0u);
        const uint32_t n1 = f32_to_e2m1_abs(fabsf(y1)) | (y1 < 0.0f ? 8u : 0u);
        o[v / 2] = (uint8_t)(n0 | (n1 << 4));
      }
      if ((g % lpb) == 0)
        reinterpret_cast<uint8_t*>(a.out_scale)[orow * (c / 32) + (g * VEC) / 32] =
            (uint8_t)(sexp + 127);
    }
  }
}

template <typename Tin, int G>
__global__ __launch_bounds__(64) void compress_rows_kernel(CompressArgs a) {
  compress_rows_body<Tin, G>(a, blockIdx.x, blockIdx.y, threadIdx.x);
}

__global__ void visibility_kernel(int64_t t0, int T, int m, int k, int w, int32_t* E, int32_t* cnt,
                                  int32_t* lo, int32_t* len) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= T) return;
  const int64_t t = t0 + j;
  const int64_t e = (t + 1) / m;
  const int64_t a = t - w + 1 > 0 ? t - w + 1 : 0;
  if (E) E[j] = (int32_t)e;
  if (cnt) cnt[j] = (int32_t)((k > 0 && k < e) ? k : e);
  if (lo) lo[j] = (int32_t)a;
  if (len) len[j] = (int32_t)(t - a + 1);
}

}  // namespace

template <typename Tin>
static bool launch_rows(const CompressArgs& a, hipStream_t s) {
  const int VEC = Vec<Tin>::N;
  const int npos = a.overlap ? 2 * a.m : a.m;
  if (npos > 8 || a.c % VEC != 0) return false;
  const int G = a.c / VEC;
  const unsigned waves = (unsigned)((a.n_entries + (64 / G) - 1) / (64 / G));
  const dim3 grid(waves, (unsigned)a.batch);
  switch (G) {
    case 16: hipLaunchKernelGGL((compress_rows_kernel<Tin, 16>), grid, dim3(64), 0, s, a); return true;
    case 32: hipLaunchKernelGGL((compress_rows_kernel<Tin, 32>), grid, dim3(64), 0, s, a); return true;
    case 64: hipLaunchKernelGGL((compress_rows_kernel<Tin, 64>), grid, dim3(64), 0, s, a); return true;
    default: return false;
  }
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  if (a.n_entries <= 0 || a.batch <= 0) return hipSuccess;
  // short pooling windows (CSA): the register-resident kernel; otherwise (HCA, m' = 128)
  // the position-split kernel with its merge through LDS
  if (a.in_dt == kF32 ? launch_rows<float>(a, s) : launch_rows<uint16_t>(a, s)) return hipGetLastError();
  const int VEC = a.in_dt == kF32 ? 4 : 8;
  const int G = a.c / VEC;
  const int P = kThreads / G;
  const size_t shmem = (size_t)3 * P * a.c * sizeof(float) + 16 * sizeof(float);
  dim3 grid((unsigned)a.n_entries, (unsigned)a.batch);
  if (a.in_dt == kF32)
    hipLaunchKernelGGL(compress_kernel<float>, grid, dim3(kThreads), shmem, s, a);
  else
    hipLaunchKernelGGL(compress_kernel<uint16_t>, grid, dim3(kThreads), shmem, s, a);
  return hipGetLastError();
}

hipError_t launch_visibility(int64_t t0, int T, int m, int k, int w, int32_t* E, int32_t* cnt,
                             int32_t* lo, int32_t* len, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(visibility_kernel, dim3((T + 255) / 256), dim3(256), 0, s, t0, T, m, k, w, E,
                     cnt, lo, len);
  return hipGetLastError();
}

}  // namespace v4a
