// Autoregressive-generation queries: KV cache, single-query attention over the cache,
// and the greedy choice from the vocabulary head's tile partials.
//
// "Inference-Native Zeroth-Order Optimization" (arXiv abstract) has the same candidate-
// state formulation cover autoregressive generation as well as token scoring; a generated
// continuation is produced under each candidate state exactly like a prompt is scored
// (factorized side path on every projection), one new token per physical sequence per
// decode step, with the keys and values of earlier positions kept in a cache instead of
// recomputed.
//
// Cache layout (per layer): K [rows x n_kv_heads x head_dim] and V likewise, in the
// activation type; sequence q owns the rows kv_first[q] .. kv_first[q] + capacity - 1
// (prompt length + generated tokens), position p at row kv_first[q] + p.
#include "common.h"
#include <math.h>
#include <type_traits>

namespace {

template <typename T>
__device__ __forceinline__ float ld_act(const T* p) { return to_f32<T>(*p); }

// Append the k and v parts of each row of the packed q|k|v activations to the cache row
// row_cache[r].  One workgroup per row, 16-byte copies (NKV * head_dim elements each).
template <typename T>
__global__ void kv_append_kernel(const T* __restrict__ qkv, int ld, const int32_t* __restrict__ row_cache,
                                 int nq, int nkv, T* __restrict__ kc, T* __restrict__ vc) {
  const int r = blockIdx.x;
  const int64_t dst = (int64_t)row_cache[r] * nkv;
  const T* src = qkv + (int64_t)r * ld + nq;
  constexpr int V = 16 / sizeof(T);                 // elements per 16-byte chunk
  for (int c = threadIdx.x; c < nkv / V; c += blockDim.x) {
    *(u32x4_t*)(kc + dst + c * V) = *(const u32x4_t*)(src + c * V);
    *(u32x4_t*)(vc + dst + c * V) = *(const u32x4_t*)(src + nkv + c * V);
  }
}

// One query row per (sequence, head): attention of the row at position row_pos[s] over
// the cached keys 0 .. row_pos[s] of sequence s (its own key included: causal).  One wave
// per (sequence, head); keys in chunks of 64, one key a lane for the scores, an online
// softmax across chunks (running max and sum, fp32), and for the weighted sum of values
// every lane owns HD / 64 of the head dimensions and walks the chunk's 64 keys.
template <typename T, int HD>
__global__ void __launch_bounds__(64)
decode_attn_kernel(const T* __restrict__ qkv, int ld, const T* __restrict__ kc, const T* __restrict__ vc,
                   const int32_t* __restrict__ kv_first, const int32_t* __restrict__ row_pos, int hq, int hkv,
                   float scale, T* __restrict__ out, int ld_out) {
  constexpr int DPL = HD / 64 > 0 ? HD / 64 : 1;    // head dimensions per lane in the value sum
  __shared__ float q_s[HD];
  __shared__ float p_s[64];
  const int s = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int kvh = h / (hq / hkv);
  const int nkv = hkv * HD;
  for (int d = lane; d < HD; d += 64) q_s[d] = ld_act<T>(qkv + (int64_t)s * ld + h * HD + d) * scale;
  __syncthreads();
  const int n_keys = row_pos[s] + 1;
  const int64_t base = (int64_t)kv_first[s] * nkv + kvh * HD;
  float run_max = -INFINITY, run_sum = 0.f;
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  for (int k0 = 0; k0 < n_keys; k0 += 64) {
    const int k = k0 + lane;
    float sc = -INFINITY;
    if (k < n_keys) {                             // the lane's key row in 16-byte pieces
      const T* kr = kc + base + (int64_t)k * nkv;
      constexpr int V = 16 / sizeof(T);
      float dot = 0.f;
#pragma unroll 4
      for (int d0 = 0; d0 < HD; d0 += V) {
        const u32x4_t w = *(const u32x4_t*)(kr + d0);
        const T* e = (const T*)&w;
#pragma unroll
        for (int u = 0; u < V; ++u) dot += q_s[d0 + u] * to_f32<T>(e[u]);
      }
      sc = dot;
    }
    float cm = sc;
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) cm = fmaxf(cm, __shfl_xor(cm, sh, 64));
    const float new_max = fmaxf(run_max, cm);
    const float corr = expf(run_max - new_max);   // 0 on the first chunk (run_max = -inf)
    const float pk = k < n_keys ? expf(sc - new_max) : 0.f;
    float ps = pk;
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) ps += __shfl_xor(ps, sh, 64);
    run_sum = run_sum * corr + ps;
    run_max = new_max;
    p_s[lane] = pk;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] *= corr;
    const int kn = min(64, n_keys - k0);
    for (int j = 0; j < kn; ++j) {
      const T* vr = vc + base + (int64_t)(k0 + j) * nkv;
      const float pj = p_s[j];
#pragma unroll
      for (int e = 0; e < DPL; ++e)
        if (lane + 64 * e < HD) acc[e] += pj * ld_act<T>(vr + lane + 64 * e);
    }
    __syncthreads();
  }
  const float inv = 1.0f / run_sum;
#pragma unroll
  for (int e = 0; e < DPL; ++e)
    if (lane + 64 * e < HD) out[(int64_t)s * ld_out + h * HD + lane + 64 * e] = from_f32<T>(acc[e] * inv);
}

// Greedy choice per row from the head's vocabulary-tile partials (max, sum of exp, first
// column of the max): the token is the first column holding the row's maximum logit
// (lowest tile on ties), its log-probability max - logsumexp in fp64.  Writes the token
// (next step's input and tokens_out[row * n_new + step]) and its log-probability.
__global__ void greedy_reduce_kernel(const float2* __restrict__ part, const int32_t* __restrict__ part_idx,
                                     int n_tiles, int n_rows, int32_t* __restrict__ next_tok,
                                     int32_t* __restrict__ tokens_out, float* __restrict__ logp_out, int n_new,
                                     int step) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n_rows) return;
  const float2* pr = part + (int64_t)r * n_tiles;
  int best = 0;
  for (int t = 1; t < n_tiles; ++t)
    if (pr[t].x > pr[best].x) best = t;
  const double M = (double)pr[best].x;
  double S = 0.0;
  for (int t = 0; t < n_tiles; ++t) S += (double)pr[t].y * exp((double)pr[t].x - M);
  const int tok = part_idx[(int64_t)r * n_tiles + best];
  next_tok[r] = tok;
  tokens_out[(int64_t)r * n_new + step] = tok;
  logp_out[(int64_t)r * n_new + step] = (float)(-log(S));
}

}  // namespace

template <typename T>
hipError_t launch_kv_append(const T* qkv, int ld, int M, const int32_t* row_cache, int nq, int nkv, T* kc, T* vc,
                            hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if ((nkv * (int)sizeof(T)) % 16 != 0 || (nq * (int)sizeof(T)) % 16 != 0 || (ld * (int)sizeof(T)) % 16 != 0)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_append_kernel<T>, dim3(M), dim3(128), 0, s, qkv, ld, row_cache, nq, nkv, kc, vc);
  return hipGetLastError();
}
template hipError_t launch_kv_append<float>(const float*, int, int, const int32_t*, int, int, float*, float*,
                                            hipStream_t);
template hipError_t launch_kv_append<bf16_t>(const bf16_t*, int, int, const int32_t*, int, int, bf16_t*, bf16_t*,
                                             hipStream_t);

template <typename T>
hipError_t launch_decode_attention(const T* qkv, int ld, const T* kc, const T* vc, const int32_t* kv_first,
                                   const int32_t* row_pos, int M, int hq, int hkv, int hd, T* out, int ld_out,
                                   hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const float scale = (float)(1.0 / sqrt((double)hd));
  dim3 grid(M, hq);
  switch (hd) {
    case 16: hipLaunchKernelGGL((decode_attn_kernel<T, 16>), grid, dim3(64), 0, s, qkv, ld, kc, vc, kv_first, row_pos, hq, hkv, scale, out, ld_out); break;
    case 32: hipLaunchKernelGGL((decode_attn_kernel<T, 32>), grid, dim3(64), 0, s, qkv, ld, kc, vc, kv_first, row_pos, hq, hkv, scale, out, ld_out); break;
    case 64: hipLaunchKernelGGL((decode_attn_kernel<T, 64>), grid, dim3(64), 0, s, qkv, ld, kc, vc, kv_first, row_pos, hq, hkv, scale, out, ld_out); break;
    case 128: hipLaunchKernelGGL((decode_attn_kernel<T, 128>), grid, dim3(64), 0, s, qkv, ld, kc, vc, kv_first, row_pos, hq, hkv, scale, out, ld_out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template hipError_t launch_decode_attention<float>(const float*, int, const float*, const float*, const int32_t*,
                                                   const int32_t*, int, int, int, int, float*, int, hipStream_t);
template hipError_t launch_decode_attention<bf16_t>(const bf16_t*, int, const bf16_t*, const bf16_t*,
                                                    const int32_t*, const int32_t*, int, int, int, int, bf16_t*, int,
                                                    hipStream_t);

hipError_t launch_greedy_reduce(const float2* part, const int32_t* part_idx, int n_tiles, int n_rows,
                                int32_t* next_tok, int32_t* tokens_out, float* logp_out, int n_new, int step,
                                hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(greedy_reduce_kernel, dim3((n_rows + 127) / 128), dim3(128), 0, s, part, part_idx, n_tiles,
                     n_rows, next_tok, tokens_out, logp_out, n_new, step);
  return hipGetLastError();
}
