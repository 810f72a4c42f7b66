// Shared-KV MQA core attention, general kernel (any c <= 1024, f32 or bf16).
//
// "CSA And HCA: Definition, State, And Cost Model": section 3.2 (each selected
// compressed entry is key and value for every head), section 4 (HCA: every
// completed entry), section 5.1 (one candidate list = compressed || window, one
// softmax per head), section 5.2 (RMSNorm, RoPE at the candidate's position,
// inverse RoPE at t on the output), section 5.3 (sink logit in the denominator).
//
// One workgroup handles one query position and a group of 8 heads.  The query
// heads are normalised, rotated and pre-scaled by scale*log2(e) into LDS; the
// candidate rows stream through LDS 16 at a time (local rows normalised and
// rotated on load), and each head keeps an online softmax state (max, sum,
// unnormalised output) in float32.  The decode form splits each sequence's
// candidate list across workgroups and merges the partial states in a second
// kernel (fixed order, so results are reproducible).
#include "device_common.h"
#include "internal.h"

namespace v4a {

namespace {

constexpr int kHG = 8;    // heads per workgroup
constexpr int kCH = 16;   // candidates per chunk
constexpr int kThreads = 256;
constexpr int kMaxC = 1024;
constexpr int kOPT = kMaxC / kThreads;  // output channels per lane per head (max)

__device__ __forceinline__ float ld_elem(const void* p, int64_t i, int dt) {
  return dt == kF32 ? reinterpret_cast<const float*>(p)[i]
                    : bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}

// Load one row of c elements with one wave into dst (LDS), optionally RMS-
// normalising with gamma and rotating the last rope_dims channels at pos.
__device__ void wave_load_row(const void* src, int64_t off, int dt, int c, float* dst,
                              bool norm, const float* gamma, float eps, int rope_dims,
                              const RopeTab& rope, double pos, float mul) {
  const int lane = threadIdx.x & 63;
  float ss = 0.0f;
  // lane owns channel pairs (2*lane + 128*i, +1)
  for (int d = 2 * lane; d < c; d += 128) {
    const float x0 = ld_elem(src, off + d, dt), x1 = ld_elem(src, off + d + 1, dt);
    dst[d] = x0;
    dst[d + 1] = x1;
    ss += x0 * x0 + x1 * x1;
  }
  float inv = 1.0f;
  if (norm) inv = 1.0f / sqrtf(wave_sum(ss) / (float)c + eps);
  const int r0 = c - rope_dims;
  for (int d = 2 * lane; d < c; d += 128) {
    float x0 = dst[d], x1 = dst[d + 1];
    if (norm) {
      x0 *= inv * (gamma ? gamma[d] : 1.0f);
      x1 *= inv * (gamma ? gamma[d + 1] : 1.0f);
    }
    if (rope_dims > 0 && d >= r0) {
      float cs, sn;
      rope_cs(pos, rope.inv_freq[(d - r0) >> 1], cs, sn);
      const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
      x0 = y0;
      x1 = y1;
    }
    dst[d] = x0 * mul;
    dst[d + 1] = x1 * mul;
  }
}

// One query position (prefill/HCA: row j of the chunk; decode: sequence b, candidate
// split `split`) for heads h0 .. h0 + 7, by the whole workgroup.  Decode splits are
// ceil(N / num_splits) candidates long unless split_len > 0 gives the length.
__device__ void attend_item(const AttnArgs& a, float* part, int b, int j, int split, int h0,
                            int64_t split_len, bool insert_new) {
  extern __shared__ float smem[];
  const int c = a.c, cp = c + 1;
  float* qs = smem;                          // [kHG][c]
  float* kvs = qs + kHG * c;                 // [kCH][c+1]
  float* zs = kvs + kCH * cp;                // [kHG][kCH]
  float* st = zs + kHG * kCH;                // [kHG] alpha
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const bool decode = a.mode == kModeDecode;
  const int nsplit = decode ? a.num_splits : 1;
  const int64_t t = decode ? a.t0 : a.t0 + j;
  const int64_t qrow = decode ? (int64_t)b * a.n_h : ((int64_t)b * a.T + j) * a.n_h;

  int64_t ncomp;
  const int32_t* idx = nullptr;
  if (a.mode == kModeHCA) {
    ncomp = (t + 1) / a.m_prime;
  } else {
    const int64_t q = decode ? b : (int64_t)b * a.T + j;
    ncomp = min(max(a.cnt[q], 0), a.k);  // clamp caller data: never read past the index row
    idx = a.idx + q * a.k;
  }
  const int64_t lo = t - a.w + 1 > 0 ? t - a.w + 1 : 0;
  const int64_t nl = t - lo + 1;
  const int64_t N = ncomp + nl;
  const int64_t per = split_len > 0 ? split_len : (N + nsplit - 1) / nsplit;
  const int64_t ub = min((int64_t)split * per, N), ue = min(ub + per, N);

  if (decode && a.kv_new && insert_new) {
    // step 1 of the decode order: the new token's row goes into slot t % w
    const int64_t dst = ((int64_t)b * a.w + t % a.w) * c;
    for (int d = tid; d < c; d += kThreads) {
      if (a.dt == kF32)
        reinterpret_cast<float*>(a.kv_ring)[dst + d] =
            reinterpret_cast<const float*>(a.kv_new)[(int64_t)b * c + d];
      else
        reinterpret_cast<uint16_t*>(a.kv_ring)[dst + d] =
            reinterpret_cast<const uint16_t*>(a.kv_new)[(int64_t)b * c + d];
    }
  }

  const float qmul = a.scale * kLog2e;
  for (int hh = wid; hh < kHG; hh += kThreads / 64) {
    const int h = h0 + hh;
    if (h < a.n_h)
      wave_load_row(a.q, (qrow + h) * c, a.dt, c, qs + hh * c, a.q_gamma != nullptr, a.q_gamma,
                    a.eps, a.rope_dims, a.rope, (double)t, qmul);
    else
      for (int d = lane; d < c; d += 64) qs[hh * c + d] = 0.0f;
  }

  float O[kHG][kOPT];
  float mrun[kHG], lrun[kHG];
#pragma unroll
  for (int hh = 0; hh < kHG; ++hh) {
    mrun[hh] = -INFINITY;
    lrun[hh] = 0.0f;
#pragma unroll
    for (int i = 0; i < kOPT; ++i) O[hh][i] = 0.0f;
  }
  __syncthreads();

  for (int64_t u0 = ub; u0 < ue; u0 += kCH) {
    const int nc = (int)min((int64_t)kCH, ue - u0);
    for (int r = wid; r < nc; r += kThreads / 64) {
      const int64_t u = u0 + r;
      if (u < ncomp) {
        int64_t e = idx ? (int64_t)idx[u] : u;
        e = min(max(e, (int64_t)0), a.E_cap - 1);  // out-of-range indices must not fault
        wave_load_row(a.kv_comp, ((int64_t)b * a.E_cap + e) * c, a.dt, c, kvs + r * cp, false,
                      nullptr, 0.0f, 0, a.rope, 0.0, 1.0f);
      } else {
        const int64_t jj = lo + (u - ncomp);
        const void* src;
        int64_t off;
        if (decode) {
          if (jj == t && a.kv_new) {
            src = a.kv_new;
            off = (int64_t)b * c;
          } else {
            src = a.kv_local;
            off = ((int64_t)b * a.w + jj % a.w) * c;
          }
        } else {
          src = a.kv_local;
          off = ((int64_t)b * a.n_loc + (jj - a.loc_base)) * c;
        }
        wave_load_row(src, off, a.dt, c, kvs + r * cp, a.kv_gamma != nullptr, a.kv_gamma, a.eps,
                      a.rope_dims, a.rope, (double)jj, 1.0f);
      }
    }
    __syncthreads();
    if (tid < kHG * kCH) {
      const int hh = tid / kCH, r = tid % kCH;
      float z = -INFINITY;
      if (r < nc && h0 + hh < a.n_h) {
        z = 0.0f;
        const float* qv = qs + hh * c;
        const float* kv = kvs + r * cp;
        for (int d = 0; d < c; ++d) z = fmaf(qv[d], kv[d], z);
      }
      zs[hh * kCH + r] = z;
    }
    __syncthreads();
    // every lane keeps the same per-head running state (cheap, avoids a barrier)
#pragma unroll
    for (int hh = 0; hh < kHG; ++hh) {
      float cm = mrun[hh];
      for (int r = 0; r < nc; ++r) cm = fmaxf(cm, zs[hh * kCH + r]);
      const float alpha = (cm == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(mrun[hh] - cm);
      float ls = lrun[hh] * alpha;
#pragma unroll
      for (int i = 0; i < kOPT; ++i) O[hh][i] *= alpha;
      for (int r = 0; r < nc; ++r) {
        const float zz = zs[hh * kCH + r];
        const float p = (zz == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(zz - cm);
        ls += p;
#pragma unroll
        for (int i = 0; i < kOPT; ++i) {
          const int d = tid + i * kThreads;
          if (d < c) O[hh][i] = fmaf(p, kvs[r * cp + d], O[hh][i]);
        }
      }
      mrun[hh] = cm;
      lrun[hh] = ls;
    }
    __syncthreads();
  }

  if (decode && nsplit > 1) {
    // partial state: [b][split][h][c + 2] = (O unnormalised, max, sum)
#pragma unroll
    for (int hh = 0; hh < kHG; ++hh) {
      const int h = h0 + hh;
      if (h >= a.n_h) continue;
      float* pr = part + (((int64_t)b * nsplit + split) * a.n_h + h) * (c + 2);
#pragma unroll
      for (int i = 0; i < kOPT; ++i) {
        const int d = tid + i * kThreads;
        if (d < c) pr[d] = O[hh][i];
      }
      if (tid == 0) {
        pr[c] = mrun[hh];
        pr[c + 1] = lrun[hh];
      }
    }
    return;
  }

  const int r0 = c - a.rope_dims;
#pragma unroll
  for (int hh = 0; hh < kHG; ++hh) {
    const int h = h0 + hh;
    float den = lrun[hh];
    if (a.sink) den += __builtin_amdgcn_exp2f(a.sink[h < a.n_h ? h : 0] * kLog2e - mrun[hh]);
    const float inv = 1.0f / den;
#pragma unroll
    for (int i = 0; i < kOPT; ++i) {
      const int d = tid + i * kThreads;
      float x = O[hh][i] * inv;
      const float other = __shfl_xor(x, 1, 64);
      if (a.rope_dims > 0 && d < c && d >= r0) {
        float cs, sn;
        rope_cs(-(double)t, a.rope.inv_freq[(d - r0) >> 1], cs, sn);
        x = (d & 1) ? other * sn + x * cs : x * cs - other * sn;
      }
      if (h < a.n_h && d < c) {
        const int64_t o = (qrow + h) * c + d;
        if (a.dt == kF32)
          reinterpret_cast<float*>(a.out)[o] = x;
        else
          reinterpret_cast<uint16_t*>(a.out)[o] = f32_to_bf16(x);
      }
    }
  }
}

// grid: x = query (prefill/HCA: j < T; decode: sequence b), y = head group,
//       z = batch (prefill/HCA) or split (decode).
__global__ __launch_bounds__(kThreads) void attn_generic_kernel(AttnArgs a, float* part) {
  const bool decode = a.mode == kModeDecode;
  const int b = decode ? blockIdx.x : blockIdx.z;
  const int j = decode ? 0 : blockIdx.x;
  const int split = decode ? blockIdx.z : 0;
  attend_item(a, part, b, j, split, blockIdx.y * kHG, 0, blockIdx.y == 0 && split == 0);
}

// Merge of decode partial states (online-softmax combination over the splits, then the
// sink, normalisation and inverse RoPE at t).  One wave per (head, sequence), four heads
// per block; lane l holds channels 8 l + 512 i .. + 7.  Every split's state is loaded in
// one pass with a running maximum (no separate max / sum / value passes), so the whole
// merge costs one memory round trip per group of splits.
constexpr int kMergeHeads = 4;
__global__ __launch_bounds__(64 * kMergeHeads) void attn_merge_kernel(AttnArgs a, const float* part) {
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * kMergeHeads + (threadIdx.x >> 6), b = blockIdx.y;
  if (h >= a.n_h) return;
  const int c = a.c, ns = a.num_splits;
  const int64_t sstride = (int64_t)a.n_h * (c + 2);
  const float* p0 = part + ((int64_t)b * ns * a.n_h + h) * (c + 2);
  const int r0 = c - a.rope_dims;
  for (int d0 = 8 * lane; d0 < c; d0 += 512) {
    float M = -INFINITY, L = 0.0f, acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int sp = 0; sp < ns; ++sp) {
      const float* ps = p0 + sp * sstride;
      // rows are c + 2 floats long (c even): 8-byte alignment only; channel pairs past c
      // (c not a multiple of 8) are not read
      float2 xp[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        xp[e] = d0 + 2 * e < c ? *reinterpret_cast<const float2*>(ps + d0 + 2 * e) : make_float2(0.0f, 0.0f);
      const float2 ml = *reinterpret_cast<const float2*>(ps + c);  // (reference max, sum)
      if (ml.x == -INFINITY) continue;  // a split without candidates
      const float Mn = fmaxf(M, ml.x);
      const float fo = __builtin_amdgcn_exp2f(M - Mn), fs = __builtin_amdgcn_exp2f(ml.x - Mn);
      const float xs[8] = {xp[0].x, xp[0].y, xp[1].x, xp[1].y, xp[2].x, xp[2].y, xp[3].x, xp[3].y};
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(xs[e], fs, acc[e] * fo);
      L = fmaf(ml.y, fs, L * fo);
      M = Mn;
    }
    if (a.sink) L += __builtin_amdgcn_exp2f(a.sink[h] * kLog2e - M);
    const float inv = 1.0f / L;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int d = d0 + e;
      float x0 = acc[e] * inv, x1 = acc[e + 1] * inv;
      if (a.rope_dims > 0 && d >= r0 && d < c) {
        float cs, sn;
        rope_cs(-(double)(a.seq.tpos ? a.seq.tpos[b] : a.t0), a.rope.inv_freq[(d - r0) >> 1], cs, sn);
        const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
        x0 = y0;
        x1 = y1;
      }
      acc[e] = x0;
      acc[e + 1] = x1;
    }
    const int64_t o = ((int64_t)b * a.n_h + h) * c + d0;
    if ((c & 7) == 0) {
      if (a.dt == kF32) {
        float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + o);
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (uint32_t)f32_to_bf16(acc[2 * e]) | ((uint32_t)f32_to_bf16(acc[2 * e + 1]) << 16);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + o) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        if (d0 + e >= c) break;
        if (a.dt == kF32) {
          reinterpret_cast<float*>(a.out)[o + e] = acc[e];
          reinterpret_cast<float*>(a.out)[o + e + 1] = acc[e + 1];
        } else {
          reinterpret_cast<uint16_t*>(a.out)[o + e] = f32_to_bf16(acc[e]);
          reinterpret_cast<uint16_t*>(a.out)[o + e + 1] = f32_to_bf16(acc[e + 1]);
        }
      }
    }
  }
}

size_t generic_smem(int c) {
  return ((size_t)kHG * c + (size_t)kCH * (c + 1) + kHG * kCH + kHG) * sizeof(float);
}

}  // namespace

hipError_t launch_attention_merge(const AttnArgs& a, const float* part, hipStream_t s);

size_t attn_generic_workspace(const AttnArgs& a) {
  if (a.mode != kModeDecode || a.num_splits <= 1) return 0;
  return (size_t)a.batch * a.num_splits * a.n_h * (a.c + 2) * sizeof(float);
}

hipError_t launch_attention_generic(const AttnArgs& a, void* ws, hipStream_t s) {
  const size_t shmem = generic_smem(a.c);
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)attn_generic_kernel,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)generic_smem(kMaxC));
    attr_set = true;
  }
  const unsigned hg = (unsigned)((a.n_h + kHG - 1) / kHG);
  dim3 grid;
  if (a.mode == kModeDecode)
    grid = dim3((unsigned)a.batch, hg, (unsigned)(a.num_splits > 1 ? a.num_splits : 1));
  else
    grid = dim3((unsigned)a.T, hg, (unsigned)a.batch);
  hipLaunchKernelGGL(attn_generic_kernel, grid, dim3(kThreads), shmem, s, a,
                     reinterpret_cast<float*>(ws));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.mode == kModeDecode && a.num_splits > 1)
    err = launch_attention_merge(a, reinterpret_cast<const float*>(ws), s);
  return err;
}

hipError_t launch_attention_merge(const AttnArgs& a, const float* part, hipStream_t s) {
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((a.n_h + kMergeHeads - 1) / kMergeHeads), (unsigned)a.batch),
                     dim3(64 * kMergeHeads), 0, s, a, part);
  return hipGetLastError();
}

}  // namespace v4a
