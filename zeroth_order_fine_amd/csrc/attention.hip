// Varlen causal prefill attention over packed ragged sequences (no padding).
//
// Each workgroup owns one (sequence, 64-query block, query head); a sequence's
// rows attend only to earlier rows of the same sequence, which is what lets the
// batch be packed without padding (arXiv abstract of "Inference-Native
// Zeroth-Order Optimization": padding elimination and variable-length packing).
// GQA: query head h reads key/value head h / (hq / hkv).
//
// bf16 path: the four waves each hold 16 queries.  Scores are computed
// transposed, S^T = K Q^T, so that after the online softmax a lane's
// probabilities (one query, 8 keys) are already the B operand of
// O^T += V^T P^T; the output accumulator then also has one query per lane and
// the rescale needs no cross-lane traffic.  K and V^T tiles are staged in LDS.
#include "common.h"
#include <math.h>
#include <type_traits>

namespace {

// 16-byte chunk swizzle of K tile row kr (CH chunks a row): the fragment reads take one
// logical chunk of 16 consecutive rows, which then touch every 16-byte bank group of the
// 256-byte LDS line once (rows of 256 bytes or more: the low four bits of kr; 128-byte rows:
// row pairs share a line, so (kr / 2) % 8)
template <int CH>
__device__ __forceinline__ int kswz(int kr) { return CH >= 16 ? (kr & 15) : ((kr >> 1) & (CH - 1)); }

constexpr int QB = 64;     // queries per workgroup
#ifndef ATTN_PREFETCH
#define ATTN_PREFETCH 1
#endif
constexpr int KB = 64;     // keys per LDS tile

// Task of workgroup bid in a one-dimensional grid of n_work x hq: workgroups are dispatched
// round-robin over the 8 XCDs, so each XCD is given a contiguous range of the task order
// (key/value head, work item, query head of the group).  The query blocks of one sequence
// and the query heads sharing a key/value head then run on one XCD at about the same time,
// and the K / V rows the later ones read are still in that XCD's L2.
__device__ __forceinline__ void attn_task(int bid, int n_work, int hq, int hkv, int& wi, int& h) {
  const int total = n_work * hq;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = total >> 3, rem = total & 7;
  const int t = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int grp = hq / hkv;
  const int kvh = t / (n_work * grp);
  const int r = t - kvh * n_work * grp;
  wi = r / grp;
  h = kvh * grp + r % grp;
}

// TO: output element type, bf16_t, or e4m3_t for the e4m3 input of an fp8 model's o-projection
#ifndef ATTN_OCC128
#define ATTN_OCC128 3
#endif
template <int HD, typename TO>
__global__ void __launch_bounds__(256, HD == 128 ? ATTN_OCC128 : 4)   // waves per SIMD: the kernel waits on loads
attn_bf16_kernel(const bf16_t* __restrict__ qkv, int ld, TO* __restrict__ out, int ld_out,
                 const int32_t* __restrict__ cu, const int32_t* __restrict__ work, int n_work, int hq, int hkv,
                 float scale_log2) {
  constexpr int KS = HD / 32;        // MFMA k-steps over the head dimension
  constexpr int HB = HD / 16;        // 16-wide blocks of the head dimension
  __shared__ __align__(16) bf16_t sK[KB * HD];        // [key][hd], 16-byte chunks XOR-swizzled
  __shared__ __align__(16) bf16_t sVt[HD * (KB + 8)];  // [hd][key] (+8 pad)
  constexpr int VT_LD = KB + 8;

  int wi, h;
  attn_task(blockIdx.x, n_work, hq, hkv, wi, h);
  const int w = work[wi];
  const int seq = w >> 12, qblk = w & 4095;
  const int kvh = h / (hq / hkv);
  const int base = cu[seq], len = cu[seq + 1] - base;
  const int q0 = qblk * QB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, g = lane >> 4;

  const int kcol = hq * HD + kvh * HD;
  const int vcol = hq * HD + hkv * HD + kvh * HD;

  // this lane's query (as a B-operand column): q = q0 + wave*16 + lr
  const int qi = q0 + wave * 16 + lr;
  const int qrow = base + min(qi, len - 1);
  bf16x8_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = *(const bf16x8_t*)(qkv + (int64_t)qrow * ld + h * HD + ks * 32 + g * 8);

  floatx4_t acc[HB];
#pragma unroll
  for (int i = 0; i < HB; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int q_last = min(q0 + QB, len) - 1;       // last valid query of the block
  const int n_kt = q_last / KB + 1;
  // Staging of a 64-key tile: K [64 x HD] and V^T [HD x 64].  Every global load of the tile
  // is issued before the first LDS write (one wait for all of them); with ATTN_PREFETCH the
  // next tile's loads are issued before the current tile's products and land under them.
  constexpr int CH = HD / 8;                        // 16-byte chunks per row
  constexpr int NKC = KB * CH / 256;                // K chunks per thread
  constexpr int NVG = (KB / 4) * CH;                // V^T groups (4 keys x one chunk)
  static_assert(NKC * 256 == KB * CH && NVG <= 256, "staging shape");
  u32x4_t kreg[NKC], vv[4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int c = tid + i * 256, kr = c / CH, ch = c % CH;
      const int krow = base + min(k0 + kr, len - 1);
      kreg[i] = *(const u32x4_t*)(qkv + (int64_t)krow * ld + kcol + ch * 8);
    }
    if (tid < NVG) {
      const int kg = tid % (KB / 4), ch = tid / (KB / 4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int krow = base + min(k0 + kg * 4 + u, len - 1);
        vv[u] = *(const u32x4_t*)(qkv + (int64_t)krow * ld + vcol + ch * 8);
      }
    }
  };
  // V^T: a thread holds 4 consecutive keys of one 8-wide head-dim chunk, transposes them in
  // registers and writes 8 rows of 4 keys (8 bytes each); the 16 lanes that share a chunk
  // fill one 128-byte stretch of a V^T row
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int c = tid + i * 256, kr = c / CH, ch = c % CH;
      *(u32x4_t*)(sK + kr * HD + ((ch ^ kswz<HD / 8>(kr)) << 3)) = kreg[i];
    }
    if (tid < NVG) {
      const int kg = tid % (KB / 4), ch = tid / (KB / 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wi = e >> 1, sh = (e & 1) * 16;
        const uint32_t lo = ((vv[0][wi] >> sh) & 0xFFFFu) | (((vv[1][wi] >> sh) & 0xFFFFu) << 16);
        const uint32_t hi = ((vv[2][wi] >> sh) & 0xFFFFu) | (((vv[3][wi] >> sh) & 0xFFFFu) << 16);
        *(uint2*)(sVt + (ch * 8 + e) * VT_LD + kg * 4) = make_uint2(lo, hi);
      }
    }
  };
  if (ATTN_PREFETCH) load_tile(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * KB;
    __syncthreads();                                // every wave is done with the previous tile
    if (!ATTN_PREFETCH) load_tile(k0);
    store_tile();
    __syncthreads();
    if (ATTN_PREFETCH && kt + 1 < n_kt) load_tile(k0 + KB);
    // S^T[key][query] for 4 blocks of 16 keys
    floatx4_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      const int kr = kb * 16 + lr;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch = ks * 4 + g;
        bf16x8_t kf = *(const bf16x8_t*)(sK + kr * HD + ((ch ^ kswz<HD / 8>(kr)) << 3));
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], s[kb], 0, 0, 0);
      }
    }
    // scale (log2 domain) and mask; a tile whose keys all precede the block's first query
    // and lie inside the sequence needs no mask (workgroup-uniform)
    float mx = -INFINITY;
    if (k0 + KB <= q0 + 1 && k0 + KB <= len) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[kb][j] *= scale_log2;
          mx = fmaxf(mx, s[kb][j]);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = k0 + kb * 16 + 4 * g + j;
          float v = s[kb][j] * scale_log2;
          if (key > qi || key >= len) v = -INFINITY;
          s[kb][j] = v;
          mx = fmaxf(mx, v);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // Key 0 is unmasked for every query, so m_new is finite from the first tile on; the
    // hardware exp2 then gives exactly 0 for masked scores (-inf) and for alpha on the first
    // tile (m_run = -inf), and flushes results below 2^-126 (negligible probabilities) to 0.
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.f;
    bf16x8_t pf[2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pv = __builtin_amdgcn_exp2f(s[kb][j] - m_new);
        psum += pv;
        pf[kb >> 1][(kb & 1) * 4 + j] = (__bf16)pv;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < HB; ++i) acc[i] *= alpha;
    // O^T[hd][query] += V^T[hd][keys] P^T[keys][query]; lane's 8 keys per 32-key step:
    // 4g..4g+3 of block 2t and of block 2t+1
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const bf16_t* vr = sVt + (hb * 16 + lr) * VT_LD + t * 32 + 4 * g;
        bf16x8_t vf;
        const uint2 lo = *(const uint2*)(vr);
        const uint2 hi = *(const uint2*)(vr + 16);
        u32x4_t packed = u32x4_t{lo.x, lo.y, hi.x, hi.y};
        vf = __builtin_bit_cast(bf16x8_t, packed);
        acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[t], acc[hb], 0, 0, 0);
      }
  }
  // total row sum over the 4 lane groups holding this query's keys
  float lsum = l_run;
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (qi < len) {
    const float inv = 1.0f / lsum;
    TO* orow = out + (int64_t)(base + qi) * ld_out + h * HD;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      if constexpr (std::is_same<TO, e4m3_t>::value) {
        *(uint32_t*)(orow + hb * 16 + 4 * g) =
            f32x4_to_e4m3(acc[hb][0] * inv, acc[hb][1] * inv, acc[hb][2] * inv, acc[hb][3] * inv);
      } else {
        *(uint2*)(orow + hb * 16 + 4 * g) =
            make_uint2(bf16x2_rne(acc[hb][0] * inv, acc[hb][1] * inv), bf16x2_rne(acc[hb][2] * inv, acc[hb][3] * inv));
      }
    }
  }
}

// Two-term path (bf16 weights, ZO_PLAN_ACT_SPLIT): q|k|v arrive in fp32 and every
// MFMA operand is split as x = hi + lo (bf16 each, 16 significant bits); each
// product is formed as hi.hi + lo.hi + hi.lo (the lo.lo term is below 2^-17
// relative), for S^T = K Q^T and for O^T += V^T P^T alike, with the same
// layout as the bf16 kernel.  The output is written as hi | lo for the next
// projection.
__device__ __forceinline__ void split8(const float* v, bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bf16_t h, l;
    split_bf16(v[e], h, l);
    hi[e] = __builtin_bit_cast(__bf16, h);
    lo[e] = __builtin_bit_cast(__bf16, l);
  }
}

__device__ __forceinline__ floatx4_t mfma3(bf16x8_t ah, bf16x8_t al, bf16x8_t bh, bf16x8_t bl, floatx4_t c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
}

template <int HD>
__global__ void __launch_bounds__(256)
attn_split_kernel(const float* __restrict__ qkv, int ld, bf16_t* __restrict__ out, int ld_out, int lo_off,
                  const int32_t* __restrict__ cu, const int32_t* __restrict__ work, int n_work, int hq, int hkv,
                  float scale_log2) {
  constexpr int KS = HD / 32;
  constexpr int HB = HD / 16;
  constexpr int VT_LD = KB + 8;
  __shared__ __align__(16) bf16_t sK[2][KB * HD];        // hi, lo: [key][hd], 16-byte chunks XOR-swizzled
  __shared__ __align__(16) bf16_t sVt[2][HD * VT_LD];    // hi, lo: [hd][key] (+8 pad)

  int wi, h;
  attn_task(blockIdx.x, n_work, hq, hkv, wi, h);
  const int w = work[wi];
  const int seq = w >> 12, qblk = w & 4095;
  const int kvh = h / (hq / hkv);
  const int base = cu[seq], len = cu[seq + 1] - base;
  const int q0 = qblk * QB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, g = lane >> 4;
  const int kcol = hq * HD + kvh * HD;
  const int vcol = hq * HD + hkv * HD + kvh * HD;

  const int qi = q0 + wave * 16 + lr;
  const int qrow = base + min(qi, len - 1);
  bf16x8_t qh[KS], ql[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const float* src = qkv + (int64_t)qrow * ld + h * HD + ks * 32 + g * 8;
    float v[8];
    *(floatx4_t*)v = *(const floatx4_t*)src;
    *(floatx4_t*)(v + 4) = *(const floatx4_t*)(src + 4);
    split8(v, qh[ks], ql[ks]);
  }

  floatx4_t acc[HB];
#pragma unroll
  for (int i = 0; i < HB; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int q_last = min(q0 + QB, len) - 1;
  const int n_kt = q_last / KB + 1;
  // staging as in the bf16 kernel: all global loads of a tile first (fp32), then the
  // hi / lo split and the LDS writes
  constexpr int CH = HD / 8;                        // 8-element chunks per row
  constexpr int NKC = KB * CH / 256;                // K chunks per thread
  constexpr int NVG = (KB / 4) * CH;                // V^T groups (4 keys x one chunk)
  static_assert(NKC * 256 == KB * CH && NVG <= 256, "staging shape");
  floatx4_t kreg[NKC][2], vreg[4][2];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int c = tid + i * 256, kr = c / CH, ch = c % CH;
      const float* src = qkv + (int64_t)(base + min(k0 + kr, len - 1)) * ld + kcol + ch * 8;
      kreg[i][0] = *(const floatx4_t*)src;
      kreg[i][1] = *(const floatx4_t*)(src + 4);
    }
    if (tid < NVG) {
      const int kg = tid % (KB / 4), ch = tid / (KB / 4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float* src = qkv + (int64_t)(base + min(k0 + kg * 4 + u, len - 1)) * ld + vcol + ch * 8;
        vreg[u][0] = *(const floatx4_t*)src;
        vreg[u][1] = *(const floatx4_t*)(src + 4);
      }
    }
  };
  // V^T: 4 consecutive keys of one 8-wide head-dim chunk per thread, transposed in
  // registers, 8-byte writes of 4 keys into 8 rows of each plane
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int c = tid + i * 256, kr = c / CH, ch = c % CH;
      float v[8];
      *(floatx4_t*)v = kreg[i][0];
      *(floatx4_t*)(v + 4) = kreg[i][1];
      bf16x8_t hi, lo;
      split8(v, hi, lo);
      const int o = kr * HD + ((ch ^ kswz<HD / 8>(kr)) << 3);
      *(bf16x8_t*)(sK[0] + o) = hi;
      *(bf16x8_t*)(sK[1] + o) = lo;
    }
    if (tid < NVG) {
      const int kg = tid % (KB / 4), ch = tid / (KB / 4);
      bf16_t vh[4][8], vl[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) split_bf16(vreg[u][e >> 2][e & 3], vh[u][e], vl[u][e]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int o = (ch * 8 + e) * VT_LD + kg * 4;
        *(uint2*)(sVt[0] + o) = make_uint2((uint32_t)vh[0][e] | ((uint32_t)vh[1][e] << 16),
                                          (uint32_t)vh[2][e] | ((uint32_t)vh[3][e] << 16));
        *(uint2*)(sVt[1] + o) = make_uint2((uint32_t)vl[0][e] | ((uint32_t)vl[1][e] << 16),
                                          (uint32_t)vl[2][e] | ((uint32_t)vl[3][e] << 16));
      }
    }
  };
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * KB;
    __syncthreads();
    load_tile(k0);
    store_tile();
    __syncthreads();
    floatx4_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      const int kr = kb * 16 + lr;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int o = kr * HD + (((ks * 4 + g) ^ kswz<HD / 8>(kr)) << 3);
        const bf16x8_t kh = *(const bf16x8_t*)(sK[0] + o), kl = *(const bf16x8_t*)(sK[1] + o);
        s[kb] = mfma3(kh, kl, qh[ks], ql[ks], s[kb]);
      }
    }
    // scale and mask, then the softmax update, as in the bf16 kernel
    float mx = -INFINITY;
    if (k0 + KB <= q0 + 1 && k0 + KB <= len) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[kb][j] *= scale_log2;
          mx = fmaxf(mx, s[kb][j]);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = k0 + kb * 16 + 4 * g + j;
          float v = s[kb][j] * scale_log2;
          if (key > qi || key >= len) v = -INFINITY;
          s[kb][j] = v;
          mx = fmaxf(mx, v);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.f;
    bf16x8_t ph[2], pl[2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pv = __builtin_amdgcn_exp2f(s[kb][j] - m_new);
        psum += pv;
        bf16_t hb, lb;
        split_bf16(pv, hb, lb);
        ph[kb >> 1][(kb & 1) * 4 + j] = __builtin_bit_cast(__bf16, hb);
        pl[kb >> 1][(kb & 1) * 4 + j] = __builtin_bit_cast(__bf16, lb);
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < HB; ++i) acc[i] *= alpha;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        bf16x8_t vf[2];
#pragma unroll
        for (int pl_ = 0; pl_ < 2; ++pl_) {
          const bf16_t* vr = sVt[pl_] + (hb * 16 + lr) * VT_LD + t * 32 + 4 * g;
          const uint2 a = *(const uint2*)(vr);
          const uint2 b = *(const uint2*)(vr + 16);
          vf[pl_] = __builtin_bit_cast(bf16x8_t, u32x4_t{a.x, a.y, b.x, b.y});
        }
        acc[hb] = mfma3(vf[0], vf[1], ph[t], pl[t], acc[hb]);
      }
  }
  float lsum = l_run;
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (qi < len) {
    const float inv = 1.0f / lsum;
    bf16_t* orow = out + (int64_t)(base + qi) * ld_out + h * HD;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      bf16_t hi[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) split_bf16(acc[hb][q] * inv, hi[q], lo[q]);
      *(uint2*)(orow + hb * 16 + 4 * g) =
          make_uint2((uint32_t)hi[0] | ((uint32_t)hi[1] << 16), (uint32_t)hi[2] | ((uint32_t)hi[3] << 16));
      *(uint2*)(orow + lo_off + hb * 16 + 4 * g) =
          make_uint2((uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16));
    }
  }
}

// fp32 path: one thread per query row, online softmax in registers.
template <int HD>
__global__ void attn_f32_kernel(const float* __restrict__ qkv, int ld, float* __restrict__ out, int ld_out,
                                const int32_t* __restrict__ cu, const int32_t* __restrict__ work, int hq, int hkv,
                                float scale) {
  const int w = work[blockIdx.x];
  const int seq = w >> 12, qblk = w & 4095;
  const int h = blockIdx.y;
  const int kvh = h / (hq / hkv);
  const int base = cu[seq], len = cu[seq + 1] - base;
  const int qi = qblk * QB + threadIdx.x;
  if (threadIdx.x >= QB || qi >= len) return;
  const float* q = qkv + (int64_t)(base + qi) * ld + h * HD;
  float o[HD];
#pragma unroll
  for (int i = 0; i < HD; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int k = 0; k <= qi; ++k) {
    const float* kr = qkv + (int64_t)(base + k) * ld + hq * HD + kvh * HD;
    const float* vr = qkv + (int64_t)(base + k) * ld + hq * HD + hkv * HD + kvh * HD;
    float sdot = 0.f;
#pragma unroll
    for (int i = 0; i < HD; ++i) sdot += q[i] * kr[i];
    sdot *= scale;
    const float mn = fmaxf(m, sdot);
    const float a = expf(m - mn), p = expf(sdot - mn);
    l = l * a + p;
#pragma unroll
    for (int i = 0; i < HD; ++i) o[i] = o[i] * a + p * vr[i];
    m = mn;
  }
  float* orow = out + (int64_t)(base + qi) * ld_out + h * HD;
#pragma unroll
  for (int i = 0; i < HD; ++i) orow[i] = o[i] / l;
}

}  // namespace

template <typename TO>
hipError_t launch_attention_bf16_to(const bf16_t* qkv, int ld_qkv, TO* out, int ld_out, const int32_t* cu,
                                    const int32_t* work, int n_work, int hq, int hkv, int hd, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
  if ((int64_t)n_work * hq > 0x7fffffff || hq % hkv != 0) return hipErrorInvalidValue;
  dim3 grid(n_work * hq);
  switch (hd) {
    case 32: hipLaunchKernelGGL((attn_bf16_kernel<32, TO>), grid, dim3(256), 0, s, qkv, ld_qkv, out, ld_out, cu, work, n_work, hq, hkv, scale_log2); break;
    case 64: hipLaunchKernelGGL((attn_bf16_kernel<64, TO>), grid, dim3(256), 0, s, qkv, ld_qkv, out, ld_out, cu, work, n_work, hq, hkv, scale_log2); break;
    case 128: hipLaunchKernelGGL((attn_bf16_kernel<128, TO>), grid, dim3(256), 0, s, qkv, ld_qkv, out, ld_out, cu, work, n_work, hq, hkv, scale_log2); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <>
hipError_t launch_attention<bf16_t>(const bf16_t* qkv, int ld_qkv, bf16_t* out, int ld_out, const int32_t* cu,
                                    int n_seq, const int32_t* work, int n_work, int hq, int hkv, int hd,
                                    hipStream_t s) {
  (void)n_seq;
  return launch_attention_bf16_to<bf16_t>(qkv, ld_qkv, out, ld_out, cu, work, n_work, hq, hkv, hd, s);
}

hipError_t launch_attention_e4m3(const bf16_t* qkv, int ld_qkv, e4m3_t* out, int ld_out, const int32_t* cu,
                                 const int32_t* work, int n_work, int hq, int hkv, int hd, hipStream_t s) {
  return launch_attention_bf16_to<e4m3_t>(qkv, ld_qkv, out, ld_out, cu, work, n_work, hq, hkv, hd, s);
}

template <>
hipError_t launch_attention<float>(const float* qkv, int ld_qkv, float* out, int ld_out, const int32_t* cu,
                                   int n_seq, const int32_t* work, int n_work, int hq, int hkv, int hd,
                                   hipStream_t s) {
  (void)n_seq;
  if (n_work <= 0) return hipSuccess;
  const float scale = (float)(1.0 / sqrt((double)hd));
  dim3 grid(n_work, hq);
  switch (hd) {
    case 16: hipLaunchKernelGGL(attn_f32_kernel<16>, grid, dim3(QB), 0, s, qkv, ld_qkv, out, ld_out, cu, work, hq, hkv, scale); break;
    case 32: hipLaunchKernelGGL(attn_f32_kernel<32>, grid, dim3(QB), 0, s, qkv, ld_qkv, out, ld_out, cu, work, hq, hkv, scale); break;
    case 64: hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(QB), 0, s, qkv, ld_qkv, out, ld_out, cu, work, hq, hkv, scale); break;
    case 128: hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(QB), 0, s, qkv, ld_qkv, out, ld_out, cu, work, hq, hkv, scale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention_split(const float* qkv, int ld_qkv, bf16_t* out, int ld_out, int lo_off,
                                  const int32_t* cu, const int32_t* work, int n_work, int hq, int hkv, int hd,
                                  hipStream_t s) {
  if (lo_off <= 0 || lo_off % 4 != 0 || ld_out % 4 != 0 || ld_qkv % 4 != 0) return hipErrorInvalidValue;
  if (n_work <= 0) return hipSuccess;
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
  if ((int64_t)n_work * hq > 0x7fffffff || hq % hkv != 0) return hipErrorInvalidValue;
  dim3 grid(n_work * hq);
  switch (hd) {
    case 32: hipLaunchKernelGGL(attn_split_kernel<32>, grid, dim3(256), 0, s, qkv, ld_qkv, out, ld_out, lo_off, cu, work, n_work, hq, hkv, scale_log2); break;
    case 64: hipLaunchKernelGGL(attn_split_kernel<64>, grid, dim3(256), 0, s, qkv, ld_qkv, out, ld_out, lo_off, cu, work, n_work, hq, hkv, scale_log2); break;
    case 128: hipLaunchKernelGGL(attn_split_kernel<128>, grid, dim3(256), 0, s, qkv, ld_qkv, out, ld_out, lo_off, cu, work, n_work, hq, hkv, scale_log2); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
