// Row-wise transformer pieces: embedding, LayerNorm / RMSNorm (optionally on a
// gathered row list), per-head QK RMSNorm + rotate-half RoPE, and the final
// log-prob combine.  All are HBM-bound: one row per workgroup, the row kept in
// registers between the statistics and the write.
#include "common.h"
#include <math.h>
#include <type_traits>

namespace {

constexpr int NORM_THREADS = 256;
constexpr int NORM_MAXV = 24;      // d <= 256 * 24 = 6144, in 16-byte groups

__device__ __forceinline__ float block_sum(float v, float* sh) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  float t = 0.f;
  const int nw = blockDim.x >> 6;
  for (int i = 0; i < nw; ++i) t += sh[i];
  return t;
}

// merge (count, mean, M2) of two disjoint parts
__device__ __forceinline__ void merge_moments(float& n, float& m, float& m2, float nb, float mb, float m2b) {
  const float nn = n + nb;
  if (nn > 0.f) {
    const float delta = mb - m, f = nb / nn;
    m = m + delta * f;
    m2 = m2 + m2b + delta * delta * n * f;
  }
  n = nn;
}

// every thread ends with the (count, mean, M2) of the whole workgroup
__device__ __forceinline__ void block_merge_moments(float& n, float& m, float& m2, float* sh) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1)
    merge_moments(n, m, m2, __shfl_xor(n, s, 64), __shfl_xor(m, s, 64), __shfl_xor(m2, s, 64));
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  __syncthreads();
  if (l == 0) { sh[3 * w] = n; sh[3 * w + 1] = m; sh[3 * w + 2] = m2; }
  __syncthreads();
  n = sh[0]; m = sh[1]; m2 = sh[2];
  for (int i = 1; i < nw; ++i) merge_moments(n, m, m2, sh[3 * i], sh[3 * i + 1], sh[3 * i + 2]);
}

// Token ids live in device memory, so the kernels that read them validate them: an id
// outside [0, vocab) sets *bad (read back by the host, which then fails the call) and is
// clamped so that every access stays in bounds.
template <typename TW>
__global__ void embed_kernel(const TW* __restrict__ E, const TW* __restrict__ P, const int32_t* __restrict__ tokens,
                             const int32_t* __restrict__ row_src, const int32_t* __restrict__ row_pos, int d,
                             int vocab, float* __restrict__ h, int32_t* __restrict__ bad) {
  const int m = blockIdx.x;
  const int raw = tokens[row_src[m]];
  if ((raw < 0 || raw >= vocab) && threadIdx.x == 0 && bad) *bad = 1;
  const int tok = min(max(raw, 0), vocab - 1);
  const int pos = row_pos[m];
  const TW* e = E + (int64_t)tok * d;
  const TW* pp = P ? P + (int64_t)pos * d : nullptr;
  float* out = h + (int64_t)m * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    float v = to_f32<TW>(e[i]);
    if (pp) v = v + to_f32<TW>(pp[i]);
    out[i] = v;
  }
}

// out[m] = norm(h[rows ? rows[m] : m]); LayerNorm (affine) or RMSNorm (gain only).
// 16-byte loads (d is a multiple of 4); the row stays in registers between the
// statistics and the write.
template <typename T>
__device__ __forceinline__ void store4(T* o, floatx4_t y);
template <>
__device__ __forceinline__ void store4<float>(float* o, floatx4_t y) { *(floatx4_t*)o = y; }
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* o, floatx4_t y) {
  *(uint2*)o = make_uint2(bf16x2_rne(y[0], y[1]), bf16x2_rne(y[2], y[3]));
}
template <>
__device__ __forceinline__ void store4<e4m3_t>(e4m3_t* o, floatx4_t y) {
  *(uint32_t*)o = f32x4_to_e4m3(y[0], y[1], y[2], y[3]);
}
// two-term bf16 expansion: hi at o, lo at o + lo_off
__device__ __forceinline__ void store4_split(bf16_t* o, int lo_off, floatx4_t y) {
  const uint32_t w0 = bf16x2_rne(y[0], y[1]), w1 = bf16x2_rne(y[2], y[3]);
  *(uint2*)o = make_uint2(w0, w1);
  const floatx4_t d = y - floatx4_t{bf16x2_lo(w0), bf16x2_hi(w0), bf16x2_lo(w1), bf16x2_hi(w1)};   // exact
  *(uint2*)(o + lo_off) = make_uint2(bf16x2_rne(d[0], d[1]), bf16x2_rne(d[2], d[3]));
}

template <typename T>
__global__ void __launch_bounds__(NORM_THREADS)
norm_kernel(const float* __restrict__ h, const int32_t* __restrict__ rows, int d, const float* __restrict__ w,
            const float* __restrict__ b, float eps, int rms, T* __restrict__ out, int64_t ld_out, int lo_off) {
  constexpr int NV = NORM_MAXV / 4;
  __shared__ float sh[3 * (NORM_THREADS / 64)];
  const int m = blockIdx.x;
  const int src = rows ? rows[m] : m;
  const float* x = h + (int64_t)src * d;
  floatx4_t v[NV];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int i = 4 * (threadIdx.x + k * NORM_THREADS);
    v[k] = i < d ? *(const floatx4_t*)(x + i) : floatx4_t{0.f, 0.f, 0.f, 0.f};
    s += (v[k][0] + v[k][1]) + (v[k][2] + v[k][3]);
  }
  float mean = 0.f, scale;
  if (!rms) {
    // one reduction: each thread's (count, mean, M2) over its own elements, merged
    // pairwise (Chan et al.'s update for combining partial variances)
    float n = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) n += (4 * (threadIdx.x + k * NORM_THREADS) < d) ? 4.f : 0.f;
    float m = n > 0.f ? s / n : 0.f, m2 = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int i = 4 * (threadIdx.x + k * NORM_THREADS);
      if (i < d) {
        const floatx4_t c = v[k] - m;
        m2 += (c[0] * c[0] + c[1] * c[1]) + (c[2] * c[2] + c[3] * c[3]);
      }
    }
    block_merge_moments(n, m, m2, sh);
    mean = m;
    scale = 1.0f / sqrtf(m2 / (float)d + eps);
  } else {
    float q = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) q += (v[k][0] * v[k][0] + v[k][1] * v[k][1]) + (v[k][2] * v[k][2] + v[k][3] * v[k][3]);
    const float ms = block_sum(q, sh) / (float)d;
    scale = 1.0f / sqrtf(ms + eps);
  }
  T* o = out + (int64_t)m * ld_out;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int i = 4 * (threadIdx.x + k * NORM_THREADS);
    if (i < d) {
      floatx4_t y = (v[k] - mean) * scale * *(const floatx4_t*)(w + i);
      if (b) y += *(const floatx4_t*)(b + i);
      if constexpr (std::is_same<T, bf16_t>::value) {
        if (lo_off) store4_split(o + i, lo_off, y);
        else store4<T>(o + i, y);
      } else {
        store4<T>(o + i, y);
      }
    }
  }
}

// The norm of a layer's input fused with the side input of the projections that read it:
// the same normalisation and store as norm_kernel (bf16, or e4m3 for fp8 models), and then,
// for a row with a candidate, t = y . V for the few used factor columns, with y the stored
// (rounded) values the projection will read and V the bf16 V^T rows of the side operand
// (p.B, row pitch p.ldb).  Column j of the n_used (<= NC) is block j / tp_used, column
// j % tp_used of that block; each thread sums its own elements, the wave's lanes are
// combined by a butterfly and the four waves in order, and t goes through tproj_out like
// the side-input projection's output.  One row per workgroup, no two-term outputs.
// R rows per workgroup (R > 1: the thread's V^T values are loaded once into registers and
// serve the R rows).  Launched with R = 1: at OPT-13B batch 64, R = 4 with q|k|v's six
// columns held in registers halved the occupancy and took the norms from 6.2 to 9.5 ms per
// step, more than the V^T reads through the caches cost.
template <typename T, int NC, int R>
__global__ void __launch_bounds__(NORM_THREADS)
norm_side_kernel(const float* __restrict__ h, int M, int d, const float* __restrict__ w, const float* __restrict__ b,
                 float eps, int rms, T* __restrict__ out, int64_t ld_out, GemmParams p, int n_used) {
  constexpr int NV = NORM_MAXV / 4;
  constexpr bool HOLD = R > 1;
  __shared__ float sh[3 * (NORM_THREADS / 64)];
  __shared__ float red[NORM_THREADS / 64][NC];
  const bf16_t* vt[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int j = min(c, n_used - 1);
    vt[c] = (const bf16_t*)p.B + (int64_t)((j / p.tp_used) * p.tp_ks + j % p.tp_used) * p.ldb;
  }
  uint2 vv[HOLD ? NC : 1][HOLD ? NV : 1];
  if constexpr (HOLD) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int i = 4 * (threadIdx.x + k * NORM_THREADS);
        vv[c][k] = i < d ? *(const uint2*)(vt[c] + i) : make_uint2(0u, 0u);
      }
  }
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int rr = 0; rr < R; ++rr) {
    const int m = blockIdx.x * R + rr;
    if (m >= M) break;                               // workgroup-uniform
    const float* x = h + (int64_t)m * d;
    floatx4_t v[NV];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int i = 4 * (threadIdx.x + k * NORM_THREADS);
      v[k] = i < d ? *(const floatx4_t*)(x + i) : floatx4_t{0.f, 0.f, 0.f, 0.f};
      s += (v[k][0] + v[k][1]) + (v[k][2] + v[k][3]);
    }
    float mean = 0.f, scale;
    if (!rms) {
      float n = 0.f;
#pragma unroll
      for (int k = 0; k < NV; ++k) n += (4 * (threadIdx.x + k * NORM_THREADS) < d) ? 4.f : 0.f;
      float mm = n > 0.f ? s / n : 0.f, m2 = 0.f;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int i = 4 * (threadIdx.x + k * NORM_THREADS);
        if (i < d) {
          const floatx4_t c = v[k] - mm;
          m2 += (c[0] * c[0] + c[1] * c[1]) + (c[2] * c[2] + c[3] * c[3]);
        }
      }
      block_merge_moments(n, mm, m2, sh);
      mean = mm;
      scale = 1.0f / sqrtf(m2 / (float)d + eps);
    } else {
      float q = 0.f;
#pragma unroll
      for (int k = 0; k < NV; ++k) q += (v[k][0] * v[k][0] + v[k][1] * v[k][1]) + (v[k][2] * v[k][2] + v[k][3] * v[k][3]);
      const float ms = block_sum(q, sh) / (float)d;
      scale = 1.0f / sqrtf(ms + eps);
    }
    const int cand = p.row_cand[m];
    T* o = out + (int64_t)m * ld_out;
    float t[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) t[c] = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int i = 4 * (threadIdx.x + k * NORM_THREADS);
      if (i < d) {
        floatx4_t y = (v[k] - mean) * scale * *(const floatx4_t*)(w + i);
        if (b) y += *(const floatx4_t*)(b + i);
        // the values the projection reads: y rounded to the output type
        floatx4_t yr;
        if constexpr (std::is_same<T, e4m3_t>::value) {
          store4<T>(o + i, y);
          if (cand >= 0) {
            const uint32_t code = f32x4_to_e4m3(y[0], y[1], y[2], y[3]);
            const u32x4_t wds = e4m3x8_to_bf16(make_uint2(code, 0u));
            yr = floatx4_t{bf16_to_f32((bf16_t)(wds[0] & 0xFFFFu)), bf16_to_f32((bf16_t)(wds[0] >> 16)),
                           bf16_to_f32((bf16_t)(wds[1] & 0xFFFFu)), bf16_to_f32((bf16_t)(wds[1] >> 16))};
          }
        } else {
          const uint32_t w0 = bf16x2_rne(y[0], y[1]), w1 = bf16x2_rne(y[2], y[3]);
          *(uint2*)(o + i) = make_uint2(w0, w1);
          yr = floatx4_t{bf16x2_lo(w0), bf16x2_hi(w0), bf16x2_lo(w1), bf16x2_hi(w1)};
        }
        if (cand >= 0) {
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            uint2 e;
            if constexpr (HOLD) e = vv[c][k];
            else e = *(const uint2*)(vt[c] + i);
            t[c] = fmaf(yr[0], bf16x2_lo(e.x), t[c]);
            t[c] = fmaf(yr[1], bf16x2_hi(e.x), t[c]);
            t[c] = fmaf(yr[2], bf16x2_lo(e.y), t[c]);
            t[c] = fmaf(yr[3], bf16x2_hi(e.y), t[c]);
          }
        }
      }
    }
    if (cand >= 0) {                                 // workgroup-uniform: one row at a time
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float a = t[c];
#pragma unroll
        for (int sh_ = 32; sh_ >= 1; sh_ >>= 1) a += __shfl_xor(a, sh_, 64);
        if (lane == 0) red[wv][c] = a;
      }
      __syncthreads();
      if ((int)threadIdx.x < n_used) {
        const int c = threadIdx.x;
        float a = red[0][c];
#pragma unroll
        for (int q = 1; q < NORM_THREADS / 64; ++q) a += red[q][c];
        tproj_out<bf16_t>(p, m, (c / p.tp_used) * p.tp_ks + c % p.tp_used, a, cand);
      }
    }
    __syncthreads();                                 // red and sh are reused by the next row
  }
}

// In place on the packed q|k|v row: per-head RMSNorm of q and k, then RoPE
// with pairs (i, i + hd/2) and the position of the row within its sequence.
template <typename T>
__global__ void qknorm_rope_kernel(T* __restrict__ qkv, int ld, int hq, int hkv, int hd,
                                   const float* __restrict__ qw, const float* __restrict__ kw, float eps,
                                   const float2* __restrict__ cs, const int32_t* __restrict__ row_pos) {
  const int m = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int half = hd >> 1;
  const int pos = row_pos[m];
  T* row = qkv + (int64_t)m * ld;
  for (int head = wave; head < hq + hkv; head += nw) {
    T* x = row + head * hd;
    const float* g = head < hq ? qw : kw;
    float a[2], c[2];
    float ss = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i = lane + 64 * t;
      a[t] = i < half ? to_f32<T>(x[i]) : 0.f;
      c[t] = i < half ? to_f32<T>(x[i + half]) : 0.f;
      ss += a[t] * a[t] + c[t] * c[t];
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) ss += __shfl_xor(ss, s, 64);
    const float sc = 1.0f / sqrtf(ss / (float)hd + eps);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i = lane + 64 * t;
      if (i < half) {
        const float x1 = a[t] * sc * g[i], x2 = c[t] * sc * g[i + half];
        const float2 r = cs[(int64_t)pos * half + i];
        x[i] = from_f32<T>(x1 * r.x - x2 * r.y);
        x[i + half] = from_f32<T>(x2 * r.x + x1 * r.y);
      }
    }
  }
}

// Per physical sequence: combine the vocabulary-tile partials of each scored
// row into log p(label) = z_label - (max + log sum exp) in fp64, then sum the
// sequence's rows in order.
__global__ void logp_reduce_kernel(const float2* __restrict__ part, int n_tiles, const float* __restrict__ lab,
                                   const int32_t* __restrict__ seq_first, double* __restrict__ tok64,
                                   float* __restrict__ tok32, double* __restrict__ seq_logp) {
  const int s = blockIdx.x;
  const int r0 = seq_first[s], r1 = seq_first[s + 1];
  for (int r = r0 + threadIdx.x; r < r1; r += blockDim.x) {
    const float2* pr = part + (int64_t)r * n_tiles;
    double M = -INFINITY;
    for (int t = 0; t < n_tiles; ++t) M = fmax(M, (double)pr[t].x);
    double S = 0.0;
    for (int t = 0; t < n_tiles; ++t) S += (double)pr[t].y * exp((double)pr[t].x - M);
    const double lp = (double)lab[r] - (M + log(S));
    tok64[r] = lp;
    if (tok32) tok32[r] = (float)lp;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double acc = 0.0;
    for (int r = r0; r < r1; ++r) acc += tok64[r];
    seq_logp[s] = acc;
  }
}

// labels of the scored rows: dst[i] = src[idx[i]], validated like the embedding's ids
__global__ void gather_label_kernel(const int32_t* __restrict__ src, const int32_t* __restrict__ idx, int n,
                                    int vocab, int32_t* __restrict__ dst, int32_t* __restrict__ bad) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int v = src[idx[i]];
  if ((v < 0 || v >= vocab) && bad) *bad = 1;
  dst[i] = min(max(v, 0), vocab - 1);
}

}  // namespace

hipError_t launch_gather_labels(const int32_t* src, const int32_t* idx, int n, int vocab, int32_t* dst,
                                int32_t* bad, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_label_kernel, dim3((n + 255) / 256), dim3(256), 0, s, src, idx, n, vocab, dst, bad);
  return hipGetLastError();
}

template <typename TW>
hipError_t launch_embed_t(const TW* E, const TW* P, const int32_t* tokens, const int32_t* row_src,
                          const int32_t* row_pos, int M, int d, int vocab, float* h, int32_t* bad, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(embed_kernel<TW>, dim3(M), dim3(256), 0, s, E, P, tokens, row_src, row_pos, d, vocab, h, bad);
  return hipGetLastError();
}
template hipError_t launch_embed_t<float>(const float*, const float*, const int32_t*, const int32_t*,
                                          const int32_t*, int, int, int, float*, int32_t*, hipStream_t);
template hipError_t launch_embed_t<bf16_t>(const bf16_t*, const bf16_t*, const int32_t*, const int32_t*,
                                           const int32_t*, int, int, int, float*, int32_t*, hipStream_t);

template <typename T>
hipError_t launch_norm(const float* h, const int32_t* rows, int M, int d, const float* w, const float* b,
                       float eps, bool rms, T* out, int64_t ld_out, int lo_off, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (d > NORM_THREADS * NORM_MAXV || d % 4 != 0 || ld_out % 4 != 0 || lo_off % 4 != 0) return hipErrorInvalidValue;
  if (lo_off && !std::is_same<T, bf16_t>::value) return hipErrorInvalidValue;
  hipLaunchKernelGGL(norm_kernel<T>, dim3(M), dim3(NORM_THREADS), 0, s, h, rows, d, w, b, eps, rms ? 1 : 0, out,
                     ld_out, lo_off);
  return hipGetLastError();
}
template hipError_t launch_norm<float>(const float*, const int32_t*, int, int, const float*, const float*, float,
                                       bool, float*, int64_t, int, hipStream_t);
template hipError_t launch_norm<bf16_t>(const float*, const int32_t*, int, int, const float*, const float*, float,
                                        bool, bf16_t*, int64_t, int, hipStream_t);
template hipError_t launch_norm<e4m3_t>(const float*, const int32_t*, int, int, const float*, const float*, float,
                                        bool, e4m3_t*, int64_t, int, hipStream_t);

// NC = the used side columns rounded up to 2, 4, 6, 8, 12 or 16
template <typename T>
hipError_t launch_norm_side(const float* h, int M, int d, const float* w, const float* b, float eps, bool rms, T* out,
                            int64_t ld_out, const GemmParams& p, int n_used, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (d > NORM_THREADS * NORM_MAXV || d % 4 != 0 || ld_out % 4 != 0 || p.ldb % 4 != 0 || n_used < 1 || n_used > 16)
    return hipErrorInvalidValue;
  const int iu = rms ? 1 : 0;
#define ZO_NORM_SIDE(NC_)                                                                                    \
  do {                                                                                                       \
    constexpr int R_ = 1;                                                                                    \
    hipLaunchKernelGGL((norm_side_kernel<T, NC_, R_>), dim3((M + R_ - 1) / R_), dim3(NORM_THREADS), 0, s, h, \
                       M, d, w, b, eps, iu, out, ld_out, p, n_used);                                        \
  } while (0)
  if (n_used <= 2) ZO_NORM_SIDE(2);
  else if (n_used <= 4) ZO_NORM_SIDE(4);
  else if (n_used <= 6) ZO_NORM_SIDE(6);
  else if (n_used <= 8) ZO_NORM_SIDE(8);
  else if (n_used <= 12) ZO_NORM_SIDE(12);
  else ZO_NORM_SIDE(16);
#undef ZO_NORM_SIDE
  return hipGetLastError();
}
template hipError_t launch_norm_side<bf16_t>(const float*, int, int, const float*, const float*, float, bool, bf16_t*,
                                             int64_t, const GemmParams&, int, hipStream_t);
template hipError_t launch_norm_side<e4m3_t>(const float*, int, int, const float*, const float*, float, bool, e4m3_t*,
                                             int64_t, const GemmParams&, int, hipStream_t);

template <typename T>
hipError_t launch_qknorm_rope(T* qkv, int M, int ld, int hq, int hkv, int hd, const float* qw, const float* kw,
                              float eps, const float2* rope_cs, const int32_t* row_pos, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (hd > 256 || (hd & 1)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(qknorm_rope_kernel<T>, dim3(M), dim3(256), 0, s, qkv, ld, hq, hkv, hd, qw, kw, eps, rope_cs,
                     row_pos);
  return hipGetLastError();
}
template hipError_t launch_qknorm_rope<float>(float*, int, int, int, int, int, const float*, const float*, float,
                                              const float2*, const int32_t*, hipStream_t);
template hipError_t launch_qknorm_rope<bf16_t>(bf16_t*, int, int, int, int, int, const float*, const float*, float,
                                               const float2*, const int32_t*, hipStream_t);

hipError_t launch_logp_reduce(const float2* part, int n_tiles, const float* lab_logit, int n_scored,
                              const int32_t* seq_first, int n_phys, double* tok_logp64, float* tok_logp32,
                              double* seq_logp, hipStream_t s) {
  (void)n_scored;
  if (n_phys <= 0) return hipSuccess;
  hipLaunchKernelGGL(logp_reduce_kernel, dim3(n_phys), dim3(256), 0, s, part, n_tiles, lab_logit, seq_first,
                     tok_logp64, tok_logp32, seq_logp);
  return hipGetLastError();
}
