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
// the cached keys 0 .. row_pos[s] of sequence s (its own key included: causal).  NW
// waves per (sequence, head), wave w taking the 64-key chunks w, w + NW, ... (one wave
// for short contexts, four beyond 512 keys); inside a
// wave LPK = head_dim / E lanes share a key (E elements = 16 bytes a lane), so every
// cached row is read as whole 16-byte pieces by neighbouring lanes.  Scores: partial dot
// products of the lane's q piece, summed over the key's lanes by shuffles; an online
// softmax across the wave's chunks in fp32; values: the same lane split, then a shuffle
// sum over the keys a lane group covered.  The waves' (max, sum, output) meet in LDS.
template <typename T, int HD, int NW, typename TO>
__global__ void __launch_bounds__(64 * NW)
decode_attn_kernel(const T* __restrict__ qkv, int ld, const T* __restrict__ kc, const T* __restrict__ vc,
                   const int32_t* __restrict__ kv_first, const int32_t* __restrict__ row_pos, int hq, int hkv,
                   float scale, TO* __restrict__ out, int ld_out) {
  constexpr int E = 16 / sizeof(T);                  // elements in a lane's 16-byte piece
  constexpr int LPK = HD / E;                        // lanes per key row
  constexpr int KPI = 64 / LPK;                      // keys per wave-wide step
  static_assert(LPK >= 1 && LPK <= 64 && 64 % LPK == 0, "head_dim");
  __shared__ float sc[NW][64];
  __shared__ float wm[NW], wl[NW];
  __shared__ float wo[NW][HD];
  const int s = blockIdx.x, h = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane % LPK, g = lane / LPK;          // piece of the row, key within the step
  const int kvh = h / (hq / hkv);
  const int nkv = hkv * HD;
  float q[E];
  {
    const u32x4_t w = *(const u32x4_t*)(qkv + (int64_t)s * ld + h * HD + c * E);
    const T* e = (const T*)&w;
#pragma unroll
    for (int u = 0; u < E; ++u) q[u] = to_f32<T>(e[u]) * scale;
  }
  const int n_keys = row_pos[s] + 1;
  const int64_t base = (int64_t)kv_first[s] * nkv + kvh * HD + c * E;
  float run_max = -INFINITY, run_sum = 0.f;
  float acc[E];
#pragma unroll
  for (int u = 0; u < E; ++u) acc[u] = 0.f;
  for (int k0 = wave * 64; k0 < n_keys; k0 += 64 * NW) {
    // scores of the chunk's 64 keys
#pragma unroll 4
    for (int it = 0; it < 64 / KPI; ++it) {
      const int j = it * KPI + g, k = k0 + j;
      float part = 0.f;
      if (k < n_keys) {
        const u32x4_t w = *(const u32x4_t*)(kc + base + (int64_t)k * nkv);
        const T* e = (const T*)&w;
#pragma unroll
        for (int u = 0; u < E; ++u) part += q[u] * to_f32<T>(e[u]);
      }
#pragma unroll
      for (int sh = 1; sh < LPK; sh <<= 1) part += __shfl_xor(part, sh, 64);
      if (c == 0) sc[wave][j] = k < n_keys ? part : -INFINITY;
    }
    __builtin_amdgcn_wave_barrier();
    const float sj = sc[wave][lane];
    float cm = sj;
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) cm = fmaxf(cm, __shfl_xor(cm, sh, 64));
    const float new_max = fmaxf(run_max, cm);
    const float corr = expf(run_max - new_max);      // 0 on the wave's first chunk
    const float pj = sj == -INFINITY ? 0.f : expf(sj - new_max);
    float ps = pj;
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) ps += __shfl_xor(ps, sh, 64);
    run_sum = run_sum * corr + ps;
    run_max = new_max;
    __builtin_amdgcn_wave_barrier();
    sc[wave][lane] = pj;                               // the chunk's probabilities
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < E; ++u) acc[u] *= corr;
#pragma unroll 4
    for (int it = 0; it < 64 / KPI; ++it) {
      const int j = it * KPI + g, k = k0 + j;
      if (k < n_keys) {
        const float p = sc[wave][j];
        const u32x4_t w = *(const u32x4_t*)(vc + base + (int64_t)k * nkv);
        const T* e = (const T*)&w;
#pragma unroll
        for (int u = 0; u < E; ++u) acc[u] += p * to_f32<T>(e[u]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // sum over the key groups of the wave (lanes with the same piece c)
#pragma unroll
  for (int u = 0; u < E; ++u)
#pragma unroll
    for (int sh = LPK; sh < 64; sh <<= 1) acc[u] += __shfl_xor(acc[u], sh, 64);
  if (lane == 0) { wm[wave] = run_max; wl[wave] = run_sum; }
  if (g == 0)
#pragma unroll
    for (int u = 0; u < E; ++u) wo[wave][c * E + u] = acc[u];
  __syncthreads();
  for (int d = threadIdx.x; d < HD; d += 64 * NW) {
    float m = -INFINITY;
    for (int w = 0; w < NW; ++w) m = fmaxf(m, wm[w]);
    float l = 0.f, o = 0.f;
    for (int w = 0; w < NW; ++w) {
      if (wm[w] == -INFINITY) continue;               // a wave without keys
      const float f = expf(wm[w] - m);
      l += wl[w] * f;
      o += wo[w][d] * f;
    }
    if constexpr (std::is_same<TO, e4m3_t>::value)   // the e4m3 input of an fp8 model's o-projection
      out[(int64_t)s * ld_out + h * HD + d] = (e4m3_t)(f32x4_to_e4m3(o / l, 0.f, 0.f, 0.f) & 0xffu);
    else
      out[(int64_t)s * ld_out + h * HD + d] = from_f32<T>(o / l);
  }
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

template <typename T, typename TO>
hipError_t launch_decode_attention(const T* qkv, int ld, const T* kc, const T* vc, const int32_t* kv_first,
                                   const int32_t* row_pos, int M, int hq, int hkv, int hd, TO* out, int ld_out,
                                   int max_keys, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const float scale = (float)(1.0 / sqrt((double)hd));
  const dim3 grid(M, hq);
  const bool wide = max_keys > 512;
#define ZO_DEC(HD)                                                                                          \
  if (wide)                                                                                                 \
    hipLaunchKernelGGL((decode_attn_kernel<T, HD, 4, TO>), grid, dim3(256), 0, s, qkv, ld, kc, vc, kv_first, \
                       row_pos, hq, hkv, scale, out, ld_out);                                               \
  else                                                                                                      \
    hipLaunchKernelGGL((decode_attn_kernel<T, HD, 1, TO>), grid, dim3(64), 0, s, qkv, ld, kc, vc, kv_first,  \
                       row_pos, hq, hkv, scale, out, ld_out);
  switch (hd) {
    case 16: ZO_DEC(16) break;
    case 32: ZO_DEC(32) break;
    case 64: ZO_DEC(64) break;
    case 128: ZO_DEC(128) break;
    default: return hipErrorInvalidValue;
  }
#undef ZO_DEC
  return hipGetLastError();
}
template hipError_t launch_decode_attention<float, float>(const float*, int, const float*, const float*,
                                                          const int32_t*, const int32_t*, int, int, int, int, float*,
                                                          int, int, hipStream_t);
template hipError_t launch_decode_attention<bf16_t, bf16_t>(const bf16_t*, int, const bf16_t*, const bf16_t*,
                                                            const int32_t*, const int32_t*, int, int, int, int,
                                                            bf16_t*, int, int, hipStream_t);
template hipError_t launch_decode_attention<bf16_t, e4m3_t>(const bf16_t*, int, const bf16_t*, const bf16_t*,
                                                            const int32_t*, const int32_t*, int, int, int, int,
                                                            e4m3_t*, int, int, hipStream_t);

hipError_t launch_greedy_reduce(const float2* part, const int32_t* part_idx, int n_tiles, int n_rows,
                                int32_t* next_tok, int32_t* tokens_out, float* logp_out, int n_new, int step,
                                hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(greedy_reduce_kernel, dim3((n_rows + 127) / 128), dim3(128), 0, s, part, part_idx, n_tiles,
                     n_rows, next_tok, tokens_out, logp_out, n_new, step);
  return hipGetLastError();
}
