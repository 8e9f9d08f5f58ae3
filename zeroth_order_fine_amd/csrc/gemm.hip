// Shared-weight projection GEMM with the factorized side path and fused epilogues.
//
// C = A . B^T with A [M x K] activations and B [N x K] the frozen weight
// (row-major, K contiguous, i.e. exactly the nn.Linear layout).  The per-row
// side path of a candidate state theta + s*eps*G V^T + sum_j U_j V_j^T
// ("Inference-Native Zeroth-Order Optimization", arXiv abstract: factorized
// side states, LoRA banks; "Zeroth-Order Fine-Tuning Was an Inference Workload
// All Along", section "The System Reorganization") is folded into the same
// accumulation as an extended K: the tile's last K-steps read
// As [M x ks] = per-row [t_j | s*eps*t_d] and Bs [N x ks] = [U_j | G_d], so W
// is never written and rows without a candidate carry zeros.
//
// bf16 path: v_mfma_f32_16x16x32_bf16, 64-wide wavefronts, LDS double buffer
// with an XOR swizzle on 16-byte chunks, one barrier per K-step, XCD-aware
// mapping of workgroups to tiles.  fp32 path: VALU FMA with the same
// accumulator layout (lane l holds rows 4*(l/16)+j, column l%16 of every
// 16x16 block), so both share the epilogues.
//
// A row's result never depends on what else is in the batch: the register-staged
// tiles depend only on the call site (N and K), and the projection kernel's tile
// choices (which may follow M) all form each output element by the same MFMA
// sequence (same 128x64 wave tile, same K loop, no split-K).
#include "common.h"
#include <math.h>
#include <stdlib.h>
#include <type_traits>

namespace {

// compile-time loop: f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>)
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

constexpr int BK_BF16 = 64;
constexpr int BK_F32 = 16;

__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// Epilogue forms for the bf16 projection kernel, whose outputs are rounded to bf16 (or
// to a 16-bit two-term expansion): a few VALU operations per element instead of the
// library erf/exp/divide, which made the fc1 epilogue a tenth of that launch.
// erf from Abramowitz & Stegun 7.1.26 (rational approximation times exp(-z^2), absolute
// error <= 1.5e-7; <= 5e-7 with the hardware reciprocal and exp2 in fp32), so the
// GELU differs from the exact one by at most 5e-7 absolute.
__device__ __forceinline__ float gelu_fast(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f), -0.284496736f), 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(-(z * z) * 1.4426950408889634f);
  const float erf_abs = fmaf(-poly, e, 1.0f);
  return x * fmaf(0.5f, copysignf(erf_abs, x), 0.5f);
}
// x * sigmoid(x) with the hardware exp2 and reciprocal (a few fp32 ulp)
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

__device__ __forceinline__ int tile_swizzle(int bid, int total, int& logical) {
  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous range of logical tiles so neighbouring tiles share its L2.
  int xcd = bid & 7, local = bid >> 3;
  int per = total >> 3, rem = total & 7;
  logical = (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  return logical;
}

// one activation output at element offset o of C: fp32 models store fp32; bf16
// models store bf16 (plus the lo term at + c_lo when set), or fp32 for a STORE
// with c_f32
template <typename TAct>
__device__ __forceinline__ void store_act(const GemmParams& p, int64_t o, float v, bool store_epi) {
  if constexpr (std::is_same<TAct, float>::value) {
    ((float*)p.C)[o] = v;
  } else {
    if (store_epi && p.c_f32) {
      ((float*)p.C)[o] = v;
      return;
    }
    bf16_t hi, lo;
    split_bf16(v, hi, lo);
    ((bf16_t*)p.C)[o] = hi;
    if (p.c_lo) ((bf16_t*)p.C)[o + p.c_lo] = lo;
  }
}

// ------------------------------------------------------------------------------
// epilogue, shared by both paths.  acc[i][j][q]: row r0 + i*16 + 4*(lane>>4) + q,
// column c0 + j*16 + (lane&15).
template <int EPI, int TM, int TN, int BM, int BN, int WM, int WN, typename TAct>
__device__ __forceinline__ void epilogue(const GemmParams& p, floatx4_t (&acc)[TM][TN], int m0, int n0, int nt,
                                         int wm, int wn, int lane, float* red) {
  const int rbase = m0 + wm * WM + 4 * (lane >> 4);
  const int cbase = n0 + wn * WN + (lane & 15);
  constexpr int epi = EPI;
  if constexpr (epi == EPI_STORE || epi == EPI_GELU || epi == EPI_RESID || epi == EPI_TPROJ) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = rbase + i * 16 + q;
        if (r >= p.M) continue;
        int cand = -1;
        if constexpr (epi == EPI_TPROJ) cand = p.row_cand[r];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int c = cbase + j * 16;
          if (c >= p.N) continue;
          float v = acc[i][j][q];
          if constexpr (epi == EPI_TPROJ) {
            tproj_out<TAct>(p, r, c, v, cand);
          } else {
            if (p.bias) v += p.bias[c];
            if constexpr (epi == EPI_RESID) {
              float* hp = p.H + (int64_t)r * p.ldh + c;
              *hp = *hp + v;
            } else {
              if constexpr (epi == EPI_GELU) v = gelu_erf(v);
              store_act<TAct>(p, (int64_t)r * p.ldc + c, v, epi == EPI_STORE);
            }
          }
        }
      }
    return;
  }
  if constexpr (epi == EPI_PARTIAL) {
    float* out = p.partial + (int64_t)blockIdx.z * p.M * p.N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = rbase + i * 16 + q;
        if (r >= p.M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int c = cbase + j * 16;
          if (c < p.N) out[(int64_t)r * p.N + c] = acc[i][j][q];
        }
      }
    return;
  }
  if constexpr (epi == EPI_SWIGLU) {
    // packed rows: 16 gate rows then 16 up rows; output column = gate index
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = rbase + i * 16 + q;
        if (r >= p.M) continue;
#pragma unroll
        for (int jp = 0; jp < TN / 2; ++jp) {
          const int cg = cbase + (2 * jp) * 16;
          if (cg >= p.N) continue;
          const int oc = (n0 + wn * WN) / 2 + jp * 16 + (lane & 15);
          float g = acc[i][2 * jp][q], u = acc[i][2 * jp + 1][q];
          store_act<TAct>(p, (int64_t)r * p.ldc + oc, silu(g) * u, false);
        }
      }
    return;
  }
  if constexpr (epi == EPI_LMHEAD) {
    constexpr int NWN = BN / WN;
    // red: [2][NWN][BM] floats
    float* rmax = red;
    float* rsum = red + NWN * BM;
    int* ridx = (int*)(red + 2 * NWN * BM);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < TN; ++j)
          if (cbase + j * 16 < p.N) m = fmaxf(m, acc[i][j][q]);
#pragma unroll
        for (int s = 1; s < 16; s <<= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
        if ((lane & 15) == 0) rmax[wn * BM + wm * WM + i * 16 + 4 * (lane >> 4) + q] = m;
      }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rl = wm * WM + i * 16 + 4 * (lane >> 4) + q;
        float m = rmax[rl];
#pragma unroll
        for (int w = 1; w < NWN; ++w) m = fmaxf(m, rmax[w * BM + rl]);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < TN; ++j)
          if (cbase + j * 16 < p.N) s += expf(acc[i][j][q] - m);
#pragma unroll
        for (int sh = 1; sh < 16; sh <<= 1) s += __shfl_xor(s, sh, 64);
        if ((lane & 15) == 0) rsum[wn * BM + rl] = s;
        if (p.part_idx) {              // first column holding the row maximum
          int ix = 0x7fffffff;
#pragma unroll
          for (int j = TN - 1; j >= 0; --j)
            if (cbase + j * 16 < p.N && acc[i][j][q] == m) ix = cbase + j * 16;
#pragma unroll
          for (int sh = 1; sh < 16; sh <<= 1) ix = min(ix, __shfl_xor(ix, sh, 64));
          if ((lane & 15) == 0) ridx[wn * BM + rl] = ix;
        }
        const int r = m0 + rl;
        if (r < p.M) {
          const int lab = p.labels[r];
#pragma unroll
          for (int j = 0; j < TN; ++j)
            if (cbase + j * 16 == lab) p.lab_logit[r] = acc[i][j][q];
        }
      }
    __syncthreads();
    const int tid = threadIdx.x;
    for (int rl = tid; rl < BM; rl += blockDim.x) {
      const int r = m0 + rl;
      if (r >= p.M) continue;
      float m = rmax[rl], s = 0.f;
      for (int w = 1; w < NWN; ++w) m = fmaxf(m, rmax[w * BM + rl]);
      for (int w = 0; w < NWN; ++w) s += rsum[w * BM + rl];
      p.part[(int64_t)r * p.n_ntiles + nt] = make_float2(m, s);
      if (p.part_idx) {
        int ix = ridx[rl];
        for (int w = 1; w < NWN; ++w) ix = min(ix, ridx[w * BM + rl]);
        p.part_idx[(int64_t)r * p.n_ntiles + nt] = ix;
      }
    }
  }
}

// ------------------------------------------------------------------------------
// bf16 MFMA kernel.  A8: the main segment's A holds e4m3 codes, widened to bf16 (exactly)
// between the global load and the LDS store.
template <int BM, int BN, int WM, int WN, int EPI, bool A8>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_bf16_kernel(GemmParams p) {
  constexpr int NWM = BM / WM, NWN = BN / WN, NT = NWM * NWN * 64;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int BK = BK_BF16;
  constexpr int CA = BM * BK / 8 / NT, CB = BN * BK / 8 / NT;
  static_assert(CA * NT * 8 == BM * BK && CB * NT * 8 == BN * BK, "tile/threads mismatch");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16_t* sm = (bf16_t*)smem_raw;
  constexpr int STAGE = (BM + BN) * BK;

  const int n_mt = (p.M + BM - 1) / BM, n_nt = (p.N + BN - 1) / BN;
  int logical;
  tile_swizzle(blockIdx.x, n_mt * n_nt, logical);
  const int mt = logical % n_mt, nt = logical / n_mt;
  const int m0 = mt * BM, n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;

  const int grp = (p.n_bounds > 0 && n0 >= p.bounds[0]) + (p.n_bounds > 1 && n0 >= p.bounds[1]) +
                  (p.n_bounds > 2 && n0 >= p.bounds[2]);
  const int a_side_off = grp * (p.as_stride ? p.as_stride : p.ks_tile);
  int nkb = p.K / BK, nk = nkb + p.ks_tile / BK;
  const int nkwa = p.kwa ? p.kwa / BK : (1 << 30), nkwb = p.kwb ? p.kwb / BK : (1 << 30);
  const int nkwas = p.kwas ? p.kwas / BK : (1 << 30);
  int kt_off = 0;                           // first base K-step of this workgroup
  const bf16_t* Ab = (const bf16_t*)p.A;
  const bf16_t* Bb = (const bf16_t*)p.B;
  if constexpr (EPI == EPI_PARTIAL) {       // K-slice of this workgroup (no side path)
    const int per = nkb / p.ksplit;
    kt_off = blockIdx.z * per;
    nkb = per;
    nk = per;
  }
  const bf16_t* Asb = (const bf16_t*)p.As;
  const bf16_t* Bsb = (const bf16_t*)p.Bs;

  // Thread t loads 16-byte chunk (t & 7) of tile rows (t >> 3) + i * NT/8.
  // Offsets are 32-bit element offsets (the host checks every operand fits).
  constexpr int RSTEP = NT / 8;
  const int ch = tid & 7, r0 = tid >> 3;
  int arow[CA], brow[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) arow[i] = min(m0 + r0 + i * RSTEP, p.M - 1);
#pragma unroll
  for (int i = 0; i < CB; ++i) brow[i] = min(n0 + r0 + i * RSTEP, p.N - 1);
  const int lda = (int)p.lda, ldb = (int)p.ldb, ldas = (int)p.ldas, ldbs = (int)p.ldbs;

  u32x4_t ra[CA], rb[CB];
#define ZO_GLOAD(kt_)                                                              \
  do {                                                                            \
    const int kt__ = (kt_);                                                       \
    const bool side__ = kt__ >= nkb;                                              \
    const bf16_t* ga__ = side__ ? Asb : Ab;                                       \
    const bf16_t* gb__ = side__ ? Bsb : Bb;                                       \
    const int la__ = side__ ? ldas : lda, lb__ = side__ ? ldbs : ldb;             \
    const int kk__ = side__ ? (kt__ - nkb) : kt__ + kt_off;                       \
    const int wa__ = side__ ? nkwas : nkwa, wb__ = side__ ? (1 << 30) : nkwb;     \
    const int ka__ = (kk__ >= wa__ ? kk__ - wa__ : kk__) * BK + ch * 8 + (side__ ? a_side_off : 0); \
    const int kb__ = (kk__ >= wb__ ? kk__ - wb__ : kk__) * BK + ch * 8;           \
    if (A8 && !side__)                                                            \
      static_for<0, CA>([&](auto i) {                                             \
        ra[i] = e4m3x8_to_bf16(*(const uint2*)((const e4m3_t*)p.A + (arow[i] * la__ + ka__))); \
      });                                                                         \
    else                                                                          \
      static_for<0, CA>([&](auto i) { ra[i] = *(const u32x4_t*)(ga__ + (arow[i] * la__ + ka__)); }); \
    static_for<0, CB>([&](auto i) { rb[i] = *(const u32x4_t*)(gb__ + (brow[i] * lb__ + kb__)); }); \
  } while (0)
#define ZO_SSTORE(buf_)                                                           \
  do {                                                                            \
    bf16_t* sA_ = sm + (buf_) * STAGE;                                            \
    bf16_t* sB_ = sA_ + BM * BK;                                                  \
    static_for<0, CA>([&](auto i) {                                               \
      const int rr = r0 + i * RSTEP;                                              \
      *(u32x4_t*)(sA_ + rr * BK + ((ch ^ ((rr >> 1) & 7)) << 3)) = ra[i];           \
    });                                                                           \
    static_for<0, CB>([&](auto i) {                                               \
      const int rr = r0 + i * RSTEP;                                              \
      *(u32x4_t*)(sB_ + rr * BK + ((ch ^ ((rr >> 1) & 7)) << 3)) = rb[i];           \
    });                                                                           \
  } while (0)

  floatx4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    ZO_GLOAD(0);
    ZO_SSTORE(0);
    __syncthreads();
  }
  const int lr = lane & 15, lk = lane >> 4;
  const int sw = (lr >> 1) & 7;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) ZO_GLOAD(kt + 1);
    const bf16_t* sA = sm + cur * STAGE;
    const bf16_t* sB = sA + BM * BK;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = ((kk * 4 + lk) ^ sw) << 3;
      bf16x8_t a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = *(const bf16x8_t*)(sA + (wm * WM + i * 16 + lr) * BK + ch);
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = *(const bf16x8_t*)(sB + (wn * WN + j * 16 + lr) * BK + ch);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) ZO_SSTORE(cur ^ 1);
    __syncthreads();
  }
  epilogue<EPI, TM, TN, BM, BN, WM, WN, bf16_t>(p, acc, m0, n0, nt, wm, wn, lane, (float*)smem_raw);
#undef ZO_GLOAD
#undef ZO_SSTORE
}

// ------------------------------------------------------------------------------
// Epilogue of the projection kernel, whose MFMAs take the weight fragment as the
// first operand: acc[i][j][q] is C[m][n] with m = i*16 + (lane & 15) and
// n = j*16 + 4*(lane >> 4) + q inside the wave tile, so every lane owns four
// consecutive output columns and writes them with one 8-byte (bf16) or 16-byte
// (fp32 residual) access.
// four consecutive bf16 outputs (8 bytes), plus their lo terms at + c_lo when set; returns
// the values written (the hi terms), as the next projection reads them
__device__ __forceinline__ floatx4_t store_bf16x4(const GemmParams& p, bf16_t* o, floatx4_t v) {
  const uint32_t w0 = bf16x2_rne(v[0], v[1]), w1 = bf16x2_rne(v[2], v[3]);
  *(uint2*)o = make_uint2(w0, w1);
  const floatx4_t hi = floatx4_t{bf16x2_lo(w0), bf16x2_hi(w0), bf16x2_lo(w1), bf16x2_hi(w1)};
  if (p.c_lo) {
    const floatx4_t d = v - hi;                        // exact in fp32
    *(uint2*)(o + p.c_lo) = make_uint2(bf16x2_rne(d[0], d[1]), bf16x2_rne(d[2], d[3]));
  }
  return hi;
}

// four consecutive outputs as e4m3 codes (4 bytes)
__device__ __forceinline__ void store_e4m3x4(e4m3_t* o, floatx4_t v) {
  *(uint32_t*)o = f32x4_to_e4m3(v[0], v[1], v[2], v[3]);
}

// The values a four-column store wrote, as the next projection reads them (bf16 or e4m3).
template <bool F8>
__device__ __forceinline__ floatx4_t stored4(floatx4_t v) {
  floatx4_t r;
  if constexpr (F8) {
    const u32x4_t w = e4m3x8_to_bf16(make_uint2(f32x4_to_e4m3(v[0], v[1], v[2], v[3]), 0u));
    r = floatx4_t{bf16_to_f32((bf16_t)(w[0] & 0xFFFFu)), bf16_to_f32((bf16_t)(w[0] >> 16)),
                  bf16_to_f32((bf16_t)(w[1] & 0xFFFFu)), bf16_to_f32((bf16_t)(w[1] >> 16))};
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = bf16_to_f32(f32_to_bf16(v[q]));
  }
  return r;
}

// The used V^T values of four consecutive output columns (from col), loaded once per column
// group and used for every row of the wave tile
__device__ __forceinline__ void side_v4(const GemmParams& p, int col, uint2 (&e)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (c < p.sf_n)
      e[c] = *(const uint2*)((const bf16_t*)p.sf_vt +
                             (int64_t)((c / p.sf_used) * p.sf_ks + c % p.sf_used) * p.sf_ldv + col);
}

// Adds y . V over four consecutive output columns to the lane's partial sums
__device__ __forceinline__ void side_partial4(const GemmParams& p, floatx4_t y, const uint2 (&e)[4], float (&t)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (c < p.sf_n) {
      t[c] = fmaf(y[0], bf16x2_lo(e[c].x), t[c]);
      t[c] = fmaf(y[1], bf16x2_hi(e[c].x), t[c]);
      t[c] = fmaf(y[2], bf16x2_lo(e[c].y), t[c]);
      t[c] = fmaf(y[3], bf16x2_hi(e[c].y), t[c]);
    }
}

// The side input's partial sums of a workgroup tile, per row and unit of two adjacent wave
// tiles (128 packed output columns): the four lanes holding one row's columns of a wave tile
// (lane, +16, +32, +48) combine, the wave tiles meet in LDS (red: [BM][NWN][4]), and each
// unit's two wave tiles are added in order; unit u of the N extent goes to group u.  The
// units do not depend on the workgroup tile shape (both shapes are pairs of 64-column wave
// tiles), so a row's partials do not depend on the batch.
template <int TM, int BM, int BN, int WM, int WN>
__device__ __forceinline__ void side_partials_wg(const GemmParams& p, float (&t)[TM][4], int m0, int n0, int wm,
                                                 int wn, int lane, float* red) {
  constexpr int NWN = BN / WN, NU = NWN / 2;
  static_assert(NWN % 2 == 0 && WN == 64, "pairs of 64-column wave tiles");
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      t[i][c] += __shfl_xor(t[i][c], 16, 64);
      t[i][c] += __shfl_xor(t[i][c], 32, 64);
    }
  __syncthreads();                                   // every wave is past its last LDS read of the stages
  if (lane < 16)
#pragma unroll
    for (int i = 0; i < TM; ++i)
      *(floatx4_t*)(red + ((wm * WM + i * 16 + lane) * NWN + wn) * 4) = floatx4_t{t[i][0], t[i][1], t[i][2], t[i][3]};
  __syncthreads();
  for (int it = threadIdx.x; it < BM * NU; it += blockDim.x) {
    const int row = it / NU, u = it - row * NU, r = m0 + row;
    if (r >= p.M || n0 + 2 * u * WN >= p.N) continue;
    const float* a = red + (row * NWN + 2 * u) * 4;
    const int unit = (n0 + 2 * u * WN) / (2 * WN);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (c < p.sf_n) p.sf_part[((int64_t)r * p.sf_groups + unit) * p.sf_n + c] = a[c] + a[4 + c];
  }
}

template <int EPI, int TM, int TN, int BM, int BN, int WM, int WN, bool F8>
__device__ __forceinline__ void epilogue_rows(const GemmParams& p, floatx4_t (&acc)[TM][TN], int m0, int n0, int wm,
                                              int wn, int lane, float* red) {
  const int rb = m0 + wm * WM + (lane & 15);
  const int cb = n0 + wn * WN + 4 * (lane >> 4);
  if constexpr (EPI == EPI_PARTIAL) {
    // fp32 sums of this workgroup's K-slice (blockIdx.z), [M x N] per slice; N is a
    // multiple of 16, so each lane's four columns are one aligned 16-byte store
    float* out = p.partial + (int64_t)blockIdx.z * p.M * p.N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = rb + i * 16;
      if (r >= p.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j)
        if (cb + j * 16 < p.N) *(floatx4_t*)(out + (int64_t)r * p.N + cb + j * 16) = acc[i][j];
    }
    return;
  } else if constexpr (EPI == EPI_LMHEAD) {
    // per row and 256-column tile: max and sum of exp of the logits, and the label's
    // logit; logits never leave registers.  A row's 64 columns of a wave sit in the
    // four lanes l, l + 16, l + 32, l + 48; the NWN waves along N meet in LDS.
    constexpr int NWN = BN / WN;
    float* rmax = red;                 // [NWN][BM]
    float* rsum = red + NWN * BM;      // [NWN][BM]
    int* ridx = (int*)(red + 2 * NWN * BM);   // [NWN][BM] (greedy decoding)
    __syncthreads();                   // every wave is past its last LDS read of the stages
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (cb + j * 16 + q < p.N) m = fmaxf(m, acc[i][j][q]);
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (lane < 16) rmax[wn * BM + wm * WM + i * 16 + lane] = m;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int rl = wm * WM + i * 16 + (lane & 15);
      float m = rmax[rl];
#pragma unroll
      for (int w = 1; w < NWN; ++w) m = fmaxf(m, rmax[w * BM + rl]);
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (cb + j * 16 + q < p.N) sum += expf(acc[i][j][q] - m);
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      if (lane < 16) rsum[wn * BM + rl] = sum;
      if (p.part_idx) {                // first column holding the row maximum
        int ix = 0x7fffffff;
#pragma unroll
        for (int j = TN - 1; j >= 0; --j)
#pragma unroll
          for (int q = 3; q >= 0; --q)
            if (cb + j * 16 + q < p.N && acc[i][j][q] == m) ix = cb + j * 16 + q;
        ix = min(ix, __shfl_xor(ix, 16, 64));
        ix = min(ix, __shfl_xor(ix, 32, 64));
        if (lane < 16) ridx[wn * BM + rl] = ix;
      }
      const int r = m0 + rl;
      if (r < p.M) {
        const int lab = p.labels[r];
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (cb + j * 16 + q == lab) p.lab_logit[r] = acc[i][j][q];
      }
    }
    __syncthreads();
    const int nt = n0 / BN;
    for (int rl = threadIdx.x; rl < BM; rl += blockDim.x) {
      const int r = m0 + rl;
      if (r >= p.M) continue;
      float m = rmax[rl], sum = 0.f;
      for (int w = 1; w < NWN; ++w) m = fmaxf(m, rmax[w * BM + rl]);
      for (int w = 0; w < NWN; ++w) sum += rsum[w * BM + rl];
      p.part[(int64_t)r * p.n_ntiles + nt] = make_float2(m, sum);
      if (p.part_idx) {
        int ix = ridx[rl];
        for (int w = 1; w < NWN; ++w) ix = min(ix, ridx[w * BM + rl]);
        p.part_idx[(int64_t)r * p.n_ntiles + nt] = ix;
      }
    }
    return;
  } else if constexpr (EPI == EPI_TPROJ) {
    // side input t: columns of x.[V...] kept for the bank entries, scaled by s * eps~
    // for the row's own direction, zero elsewhere (as in the register-staged epilogue)
    static_for<0, TM>([&](auto i) {
      const int r = rb + i * 16;
      const int cand = r < p.M ? p.row_cand[r] : -1;
      if (cand >= 0) {
        static_for<0, TN>([&](auto j) {
          if (cb + j * 16 < p.N) {
            static_for<0, 4>([&](auto q) {
              tproj_out<bf16_t>(p, r, cb + j * 16 + q, acc[i][j][decltype(q)::value], cand);
            });
          }
        });
      }
    });
    return;
  } else if constexpr (EPI == EPI_SWIGLU) {
    // packed rows: blocks of 16 gate rows then 16 up rows; output column = gate index
    const int ob = (n0 + wn * WN) / 2 + 4 * (lane >> 4);
    float t[TM][4];
#pragma unroll
    for (int i = 0; i < TM; ++i) t[i][0] = t[i][1] = t[i][2] = t[i][3] = 0.f;
    // V values of the wave tile's output columns loaded once; rows outer (as in the GELU
    // epilogue, so that a row's stores follow one another)
    uint2 e[TN / 2][4];
    if (p.sf_n)
#pragma unroll
      for (int jp = 0; jp < TN / 2; ++jp)
        if (cb + 2 * jp * 16 < p.N) side_v4(p, ob + jp * 16, e[jp]);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = rb + i * 16;
      if (r >= p.M) continue;
#pragma unroll
      for (int jp = 0; jp < TN / 2; ++jp) {
        if (cb + 2 * jp * 16 >= p.N) continue;                  // N is a multiple of 32 here
        // (e4m3 main segments sum in units of 2^-11 of the result)
        constexpr float unit = F8 ? 1.0f / (float)(1 << ZO_FP8_WEIGHT_EXP) : 1.0f;
        const floatx4_t g = acc[i][2 * jp] * unit, u = acc[i][2 * jp + 1] * unit;
        floatx4_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = silu_fast(g[q]) * u[q];
        if constexpr (F8) {            // the e4m3 input of the down projection
          store_e4m3x4((e4m3_t*)p.C + (int64_t)r * p.ldc + ob + jp * 16, v);
          if (p.sf_n) side_partial4(p, stored4<true>(v), e[jp], t[i]);
        } else {
          const floatx4_t y = store_bf16x4(p, (bf16_t*)p.C + (int64_t)r * p.ldc + ob + jp * 16, v);
          if (p.sf_n) side_partial4(p, y, e[jp], t[i]);
        }
      }
    }
    if (p.sf_n) side_partials_wg<TM, BM, BN, WM, WN>(p, t, m0, n0, wm, wn, lane, red);   // every thread takes part
    return;
  } else {
    // a lane's four columns are all inside N or all outside (N is a multiple of 16)
    floatx4_t bias[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bias[j] = (p.bias && cb + j * 16 < p.N) ? *(const floatx4_t*)(p.bias + cb + j * 16)
                                              : floatx4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (EPI == EPI_GELU) {
      // the side input's V values of all the wave tile's columns are loaded once, before the
      // rows; rows outer, so that the stores of one row's 64 columns follow one another (with
      // the column blocks outer, the L2 wrote each output line back twice)
      float t[TM][4];
#pragma unroll
      for (int i = 0; i < TM; ++i) t[i][0] = t[i][1] = t[i][2] = t[i][3] = 0.f;
      if constexpr (F8) {
        // e4m3: column blocks outer, one block's V values live at a time (holding all of
        // them took this variant past 256 registers a lane, one wave a SIMD instead of
        // two); a row's partial sums still take its columns in ascending order
        constexpr float unit = 1.0f / (float)(1 << ZO_FP8_WEIGHT_EXP);   // main segments in units of 2^-11
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if (cb + j * 16 >= p.N) continue;
          uint2 ej[4];
          if (p.sf_n) side_v4(p, cb + j * 16, ej);
          const floatx4_t bj = p.bias ? *(const floatx4_t*)(p.bias + cb + j * 16) : floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const int r = rb + i * 16;
            if (r >= p.M) continue;
            floatx4_t v = acc[i][j] * unit + bj;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = gelu_fast(v[q]);
            store_e4m3x4((e4m3_t*)p.C + (int64_t)r * p.ldc + cb + j * 16, v);   // the next e4m3 projection's input
            if (p.sf_n) side_partial4(p, stored4<true>(v), ej, t[i]);
          }
        }
      } else {
        uint2 e[TN][4];
        if (p.sf_n)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            if (cb + j * 16 < p.N) side_v4(p, cb + j * 16, e[j]);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int r = rb + i * 16;
          if (r >= p.M) continue;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if (cb + j * 16 >= p.N) continue;
            floatx4_t v = acc[i][j] + bias[j];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = gelu_fast(v[q]);
            const floatx4_t y = store_bf16x4(p, (bf16_t*)p.C + (int64_t)r * p.ldc + cb + j * 16, v);
            if (p.sf_n) side_partial4(p, y, e[j], t[i]);
          }
        }
      }
      if (p.sf_n) side_partials_wg<TM, BM, BN, WM, WN>(p, t, m0, n0, wm, wn, lane, red);   // every thread takes part
      return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = rb + i * 16;
      if (r >= p.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if (cb + j * 16 >= p.N) continue;
        // e4m3 main segments sum in units of 2^-11 of the result (the weights hold w * 2^11)
        constexpr float unit = F8 ? 1.0f / (float)(1 << ZO_FP8_WEIGHT_EXP) : 1.0f;
        floatx4_t v = F8 ? acc[i][j] * unit + bias[j] : acc[i][j] + bias[j];
        if constexpr (EPI == EPI_RESID) {
          floatx4_t* hp = (floatx4_t*)(p.H + (int64_t)r * p.ldh + cb + j * 16);
          *hp = *hp + v;
        } else {
          if (EPI == EPI_STORE && p.c_f32)
            *(floatx4_t*)((float*)p.C + (int64_t)r * p.ldc + cb + j * 16) = v;
          else
            store_bf16x4(p, (bf16_t*)p.C + (int64_t)r * p.ldc + cb + j * 16, v);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------
// bf16 MFMA kernel for the shared-weight projections.
//
// Workgroup tiles of WM x WN wave tiles (256 x 256 of 128 x 64: eight waves, two per
// SIMD; 128 x 128 of 64 x 64 for small batches), K steps of 64 held in two LDS stages
// of (BM + BN) x 64 bf16; with EPI_PARTIAL, blockIdx.z selects one of ksplit K-slices.  Tiles are streamed
// global -> LDS by buffer loads straight into LDS (no register staging; a fixed
// per-lane byte offset in a VGPR, the K position in the scalar offset): the loads of
// stage k + 1 are issued right after the barrier that opens step k, so they run under
// the step's 2 x TM x TN MFMAs; one barrier per 64-deep step.  LDS holds
// [A0 | A1 | B0 | B1], so the stage switch is an immediate offset of the LDS reads.
// Within a 1 KB block (8 rows x 64 k, 128-byte rows) lane L of a load writes row L/8,
// 16-byte chunk L%8, which holds logical chunk (L%8) ^ swz8(row), swz8(row) = (row / 2) % 8:
// a fragment read (16 consecutive rows, one logical chunk) then touches each 16-byte bank
// group of the 256-byte LDS line once.  Measured with eight waves streaming the fragment
// pattern: 209 bytes per clock per CU, against 118 for (row ^ row / 8) % 8 (which spreads
// only 8-row phases) and 176 for plain contiguous 1 KB reads.  Each output element is
// accumulated by the same MFMA sequence (k ascending, 32 per instruction) for every
// workgroup and wave tile shape.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// buffer resource over `bytes` bytes at `base` (raw addressing: offsets past the end read 0)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes > (int64_t)0xffffffff ? 0xffffffffu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)n, 0x00020000);
}

template <int BM, int BN, int WM, int WN, int EPI, bool F8, bool SK = false>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_bf16_pipe_kernel(GemmParams p) {
  constexpr int BK = 64;                               // bf16 elements of a K-step (128 bytes a row)
  constexpr int BKM = F8 ? 128 : 64;                   // main-segment elements of a K-step (128 bytes a row)
  constexpr int NWM = BM / WM, NWN = BN / WN, NW = NWM * NWN;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int ASZ = BM * BK, BSZ = BN * BK;          // elements of one stage of A / of B
  constexpr int ABLK = BM / 8, BBLK = BN / 8;          // 1 KB blocks per stage
  constexpr int IA = ABLK / NW, IB = BBLK / NW;        // loads per wave per stage
  static_assert(IA * NW == ABLK && IB * NW == BBLK, "blocks per wave");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16_t* sm = (bf16_t*)smem_raw;                      // [A stage 0 | A stage 1 | B stage 0 | B stage 1]

  const int n_mt = (p.M + BM - 1) / BM, n_nt = (p.N + BN - 1) / BN;
  // logical tile -> origin (m0, n0): groups of GM m-tiles, column-major inside a group:
  // the ~32 tiles an XCD runs at once share a few A and B panels, so each K-step's chunks
  // are fetched into its L2 once and reused.  a_side_off: the side-segment As columns of
  // the kind group the column tile lies in.
  constexpr int GM = 4;
  int m0 = 0, n0 = 0, a_side_off = 0;
  auto set_tile = [&](int logical) {
    const int per_group = GM * n_nt;
    const int g = logical / per_group, gm0 = g * GM;
    const int gsize = min(GM, n_mt - gm0);
    const int in_g = logical - g * per_group;
    m0 = (gm0 + in_g % gsize) * BM;
    n0 = (in_g / gsize) * BN;
    const int grp = (p.n_bounds > 0 && n0 >= p.bounds[0]) + (p.n_bounds > 1 && n0 >= p.bounds[1]) +
                    (p.n_bounds > 2 && n0 >= p.bounds[2]);
    a_side_off = grp * (p.as_stride ? p.as_stride : p.ks_tile);
  };
  if constexpr (!SK) {
    int logical;
    tile_swizzle(blockIdx.x, n_mt * n_nt, logical);
    set_tile(logical);
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave / NWN, wn = wave % NWN;
  int nkb = p.K / BKM, nk = nkb + p.ks_tile / BK;
  int kt_off = 0;                      // first K-step of this workgroup's K-slice
  if constexpr (EPI == EPI_PARTIAL) {  // split-K: the last K-slice also runs the side segment
    const int nks_all = nk - nkb;
    nkb = nkb / p.ksplit;
    kt_off = blockIdx.z * nkb;
    nk = nkb + ((int)blockIdx.z == p.ksplit - 1 ? nks_all : 0);
  }
  const int nkwa = p.kwa ? p.kwa / BKM : (1 << 30), nkwb = p.kwb ? p.kwb / BKM : (1 << 30);
  const int nkwas = p.kwas ? p.kwas / BK : (1 << 30);
  constexpr int ESZ = F8 ? 1 : 2;                      // main-segment bytes per element
  // The split-tail kernel keeps the per-lane offsets tile-independent (rows of the tile, no clamp) and
  // moves the tile origin into the buffer resources, which end at the last row (rows past
  // it read as zero and feed only outputs that are never stored); otherwise the resources
  // cover the whole operands and rows are clamped to the last one.
  __amdgpu_buffer_rsrc_t rA = raw_rsrc(p.A, (int64_t)p.M * p.lda * ESZ);
  __amdgpu_buffer_rsrc_t rB = raw_rsrc(p.B, (int64_t)p.N * p.ldb * ESZ);
  auto set_rsrc = [&]() {
    rA = raw_rsrc((const unsigned char*)p.A + (int64_t)m0 * p.lda * ESZ, (int64_t)(p.M - m0) * p.lda * ESZ);
    rB = raw_rsrc((const unsigned char*)p.B + (int64_t)n0 * p.ldb * ESZ, (int64_t)(p.N - n0) * p.ldb * ESZ);
  };

  // load i of this wave fills 1 KB block wave * I + i: tile row blk * 8 + lane / 8, the
  // lane's 16 bytes holding logical chunk (lane % 8) ^ swz8(row).  Byte offsets of the
  // row and chunk stay in VGPRs; the K position goes in the scalar offset.
  const int lrow = lane >> 3;
  // tile row and physical 16-byte chunk of load i; its element offset (row * ld +
  // 8 * chunk for bf16) is recomputed where needed rather than kept
  auto a_row = [&](int i) { return min(m0 + (wave * IA + i) * 8 + lrow, p.M - 1); };
  auto b_row = [&](int i) { return min(n0 + (wave * IB + i) * 8 + lrow, p.N - 1); };
  auto a_chk = [&](int i) { return (lane & 7) ^ swz8((wave * IA + i) * 8 + lrow); };
  auto b_chk = [&](int i) { return (lane & 7) ^ swz8((wave * IB + i) * 8 + lrow); };
  auto a_elem = [&](int i, int ld) { return a_row(i) * ld + (a_chk(i) << 3); };
  auto b_elem = [&](int i, int ld) { return b_row(i) * ld + (b_chk(i) << 3); };
  // byte offsets: the host keeps every operand under 2^31 elements, so they fit 32 unsigned
  // bits (e4m3 operands: one byte an element, 16 elements a chunk)
  uint32_t aoff[IA], boff[IB];
  auto set_offsets = [&]() {
    if constexpr (SK) {
      static_for<0, IA>([&](auto i) { aoff[i] = (uint32_t)(((wave * IA + i) * 8 + lrow) * (int)p.lda + (a_chk(i) << 3)) * 2u; });
      static_for<0, IB>([&](auto i) { boff[i] = (uint32_t)(((wave * IB + i) * 8 + lrow) * (int)p.ldb + (b_chk(i) << 3)) * 2u; });
    } else if constexpr (F8) {
      static_for<0, IA>([&](auto i) { aoff[i] = (uint32_t)(a_row(i) * (int)p.lda) + (uint32_t)(a_chk(i) << 4); });
      static_for<0, IB>([&](auto i) { boff[i] = (uint32_t)(b_row(i) * (int)p.ldb) + (uint32_t)(b_chk(i) << 4); });
    } else {
      static_for<0, IA>([&](auto i) { aoff[i] = (uint32_t)a_elem(i, (int)p.lda) * 2u; });
      static_for<0, IB>([&](auto i) { boff[i] = (uint32_t)b_elem(i, (int)p.ldb) * 2u; });
    }
  };
  if constexpr (!SK) set_offsets();
  // K-step order: bf16 kernels run the main segment, then the side segment; the e4m3
  // kernel runs its (bf16) side segment first, so that the side operands' offsets are dead
  // before the main loop, which needs every register it has
  const int nks = nk - nkb;                            // side-segment steps
  auto issue = [&](int s, auto slot) {
    bf16_t* sA = sm + slot * ASZ;
    bf16_t* sB = sm + 2 * ASZ + slot * BSZ;
    if (F8 ? s >= nks : s < nkb) {
      const int sk = (F8 ? s - nks : s) + kt_off;
      const int ka = (sk >= nkwa ? sk - nkwa : sk) * BKM * ESZ;
      const int kb = (sk >= nkwb ? sk - nkwb : sk) * BKM * ESZ;
      static_for<0, IA>([&](auto i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rA, (__attribute__((address_space(3))) void*)(sA + (wave * IA + i) * 8 * BK), 16, aoff[i], ka, 0, 0);
      });
      static_for<0, IB>([&](auto i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rB, (__attribute__((address_space(3))) void*)(sB + (wave * IB + i) * 8 * BK), 16, boff[i], kb, 0, 0);
      });
    } else if constexpr (SK) {                // side segment, split-tail form
      const __amdgpu_buffer_rsrc_t rAs =
          raw_rsrc((const unsigned char*)p.As + (int64_t)m0 * p.ldas * 2, (int64_t)(p.M - m0) * p.ldas * 2);
      const __amdgpu_buffer_rsrc_t rBs =
          raw_rsrc((const unsigned char*)p.Bs + (int64_t)n0 * p.ldbs * 2, (int64_t)(p.N - n0) * p.ldbs * 2);
      const int kk = s - nkb;
      const int ka = ((kk >= nkwas ? kk - nkwas : kk) * BK + a_side_off) * 2;
      const int kb = kk * BK * 2;
      static_for<0, IA>([&](auto i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rAs, (__attribute__((address_space(3))) void*)(sA + (wave * IA + i) * 8 * BK), 16,
            (uint32_t)(((wave * IA + i) * 8 + lrow) * (int)p.ldas + (a_chk(i) << 3)) * 2u, ka, 0, 0);
      });
      static_for<0, IB>([&](auto i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rBs, (__attribute__((address_space(3))) void*)(sB + (wave * IB + i) * 8 * BK), 16,
            (uint32_t)(((wave * IB + i) * 8 + lrow) * (int)p.ldbs + (b_chk(i) << 3)) * 2u, kb, 0, 0);
      });
    } else {                                  // side segment
      const __amdgpu_buffer_rsrc_t rAs = raw_rsrc(p.As, (int64_t)p.M * p.ldas * 2);
      const __amdgpu_buffer_rsrc_t rBs = raw_rsrc(p.Bs, (int64_t)p.N * p.ldbs * 2);
      const int kk = F8 ? s : s - nkb;
      const int ka = ((kk >= nkwas ? kk - nkwas : kk) * BK + a_side_off) * 2;
      const int kb = kk * BK * 2;
      static_for<0, IA>([&](auto i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rAs, (__attribute__((address_space(3))) void*)(sA + (wave * IA + i) * 8 * BK), 16,
            (uint32_t)a_elem(i, (int)p.ldas) * 2u, ka, 0, 0);
      });
      static_for<0, IB>([&](auto i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rBs, (__attribute__((address_space(3))) void*)(sB + (wave * IB + i) * 8 * BK), 16,
            (uint32_t)b_elem(i, (int)p.ldbs) * 2u, kb, 0, 0);
      });
    }
  };
  // fragment offsets of the two 32-deep halves u of a stage (stage 0; stage 1 adds an
  // immediate)
  const int lr = lane & 15, lk = lane >> 4;
  int aro[2][TM], bro[2][TN];
  static_for<0, 2>([&](auto u) {
    static_for<0, TM>([&](auto i) {
      const int row = wm * WM + i * 16 + lr;
      aro[u][i] = row * BK + (((4 * u + lk) ^ swz8(row)) << 3);
    });
    static_for<0, TN>([&](auto j) {
      const int row = wn * WN + j * 16 + lr;
      bro[u][j] = 2 * ASZ + row * BK + (((4 * u + lk) ^ swz8(row)) << 3);
    });
  });
  bf16x8_t fa[2][TM], fb[2][TN];
  auto rd = [&](auto slot, auto u) {
    static_for<0, TM>([&](auto i) { fa[u][i] = *(const bf16x8_t*)(sm + slot * ASZ + aro[u][i]); });
    static_for<0, TN>([&](auto j) { fb[u][j] = *(const bf16x8_t*)(sm + slot * BSZ + bro[u][j]); });
  };
  floatx4_t acc[TM][TN];
  auto zero_acc = [&]() {
    static_for<0, TM>([&](auto i) {
      static_for<0, TN>([&](auto j) { acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f}; });
    });
  };
  if constexpr (!SK) zero_acc();
  int kend = nk;                                       // the current K range ends before step kend
  auto mm = [&](auto u) {
    static_for<0, TM>([&](auto i) {
      static_for<0, TN>([&](auto j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[u][j], fa[u][i], acc[i][j], 0, 0, 0);
      });
    });
  };
  constexpr int MPR = (TM * TN) / (TM + TN);           // MFMAs per interleaved LDS read
  auto step_bf16 = [&](int kt, auto slot) {
    if (kt + 1 < kend) issue(kt + 1, std::integral_constant<int, 1 - slot>{});
    rd(slot, std::integral_constant<int, 0>{});
    rd(slot, std::integral_constant<int, 1>{});
    mm(std::integral_constant<int, 0>{});
    mm(std::integral_constant<int, 1>{});
    __builtin_amdgcn_sched_group_barrier(0x020, IA + IB, 0);                 // the loads
    __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);                 // first half's fragments
    static_for<0, TM + TN>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);                   // MFMAs on ready fragments
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                     // one read of the second half
    });
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * TM * TN - MPR * (TM + TN), 0);
  };
  // Steps of the e4m3 kernel.  Every fragment is 32 bytes a lane: row lr, logical 16-byte
  // chunks lk and lk + 4 of the 128-byte row.  Main steps (128 e4m3 k): one
  // v_mfma_f32_16x16x128_f8f6f4 per 16x16 block; A and B bytes at the same lane group and
  // position meet in one product and the four lane groups cover the row's 128 elements
  // once, so the instruction sums all 128 products.  Side steps (64 bf16 k): the two
  // 16-byte halves are the two 32-deep bf16 fragments of the bf16 kernel (k ascending).
  // Both read the same LDS addresses into the same registers.
  typedef __attribute__((ext_vector_type(8))) int i32x8_t;
  typedef __attribute__((ext_vector_type(4))) int i32x4_t;
  auto step8 = [&](int kt, auto slot, auto side) {
    if (kt + 1 < kend) issue(kt + 1, std::integral_constant<int, 1 - slot>{});
    // chunk lk + 4 = chunk lk ^ 4, so its offset is the first one's with bit 5 flipped (row
    // starts are multiples of 64 elements); only the first offsets stay in registers
    i32x8_t ga[TM], gb[TN];
    static_for<0, TN>([&](auto j) {
      const i32x4_t x0 = *(const i32x4_t*)(sm + slot * BSZ + bro[0][j]);
      const i32x4_t x1 = *(const i32x4_t*)(sm + slot * BSZ + (bro[0][j] ^ 32));
      gb[j] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    });
    static_for<0, TM>([&](auto i) {
      const i32x4_t x0 = *(const i32x4_t*)(sm + slot * ASZ + aro[0][i]);
      const i32x4_t x1 = *(const i32x4_t*)(sm + slot * ASZ + (aro[0][i] ^ 32));
      ga[i] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    });
    static_for<0, TM>([&](auto i) {
      static_for<0, TN>([&](auto j) {
        if constexpr (decltype(side)::value) {
          const i32x4_t bl = __builtin_shufflevector(gb[j], gb[j], 0, 1, 2, 3);
          const i32x4_t bh = __builtin_shufflevector(gb[j], gb[j], 4, 5, 6, 7);
          const i32x4_t al = __builtin_shufflevector(ga[i], ga[i], 0, 1, 2, 3);
          const i32x4_t ah = __builtin_shufflevector(ga[i], ga[i], 4, 5, 6, 7);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bl),
                                                              __builtin_bit_cast(bf16x8_t, al), acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bh),
                                                              __builtin_bit_cast(bf16x8_t, ah), acc[i][j], 0, 0, 0);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(gb[j], ga[i], acc[i][j], 0, 0, 0, 0, 0, 0);
        }
      });
    });
    // A fragments ping-pong: the read of fragment i + 2 follows row i's MFMAs (whose
    // registers it reuses), so fragment i + 1 is in flight while row i runs
    constexpr int PER = decltype(side)::value ? 2 : 1;                       // MFMAs per block
    __builtin_amdgcn_sched_group_barrier(0x020, IA + IB, 0);                 // the loads
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * TN + 4, 0);              // B fragments, A fragments 0 and 1
    static_for<0, TM - 2>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x008, PER * TN, 0);              // one row of blocks
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                     // A fragment two rows on
    });
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * PER * TN, 0);
  };
  // this wave's loads of stage kt have landed; after the barrier so have every wave's,
  // and every read of the other stage (kt - 1) is retired
  auto wait_stage = [&]() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // bf16 K-steps [kb, ke) of the current tile, stage kt in slot (kt - kb) & 1
  auto kloop_bf16 = [&](int kb, int ke) {
    kend = ke;
    if (kb < ke) issue(kb, S0{});
    for (int kt = kb; kt < ke; kt += 2) {
      wait_stage(); step_bf16(kt, S0{});
      if (kt + 1 < ke) { wait_stage(); step_bf16(kt + 1, S1{}); }
    }
  };
  // the epilogue's coordinates come from the wave index in a scalar register and the lane
  // index counted afresh, so no vector register is kept live across the K loop (where every
  // one is taken) for them
  auto finish = [&]() {
    const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    epilogue_rows<EPI, TM, TN, BM, BN, WM, WN, F8>(p, acc, m0, n0, wave_s / NWN, wave_s % NWN, lane_e,
                                                  (float*)smem_raw);
  };
  if constexpr (!SK) {
    if constexpr (F8) {
      // the bf16 side segment, then the e4m3 main segment, in separate loops (stage kt in
      // slot kt & 1)
      if (nk > 0) issue(0, S0{});
      int kt = 0;
      using SIDE = std::true_type;
      using MAIN = std::false_type;
      for (; kt < nks; ++kt) {
        wait_stage();
        if (kt & 1) step8(kt, S1{}, SIDE{});
        else step8(kt, S0{}, SIDE{});
      }
      if ((kt & 1) && kt < nk) { wait_stage(); step8(kt, S1{}, MAIN{}); ++kt; }
      for (; kt + 1 < nk; kt += 2) {
        wait_stage(); step8(kt, S0{}, MAIN{});
        wait_stage(); step8(kt + 1, S1{}, MAIN{});
      }
      if (kt < nk) { wait_stage(); step8(kt, S0{}, MAIN{}); }
    } else {
      kloop_bf16(0, nk);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no LDS write outlives the workgroup
    finish();
  } else {
    // Split tail: gridDim.x persistent workgroups, dispatched round-robin over the 8 XCDs
    // (workgroup b on XCD b % 8, slot b / 8 of Px there).  Each XCD owns the contiguous
    // logical tiles tile_swizzle gives it.  All but the last one to two rounds of them run
    // as whole tiles (round r: tile r * Px + slot, as the data-parallel launch orders them).
    // The last Tsk tiles (Px <= Tsk < 2 Px) are cut along K into S equal slices (S from 1 to
    // 4: the fewest rounds of slices, in tiles), and the Tsk * S pieces are dealt round-robin:
    // piece q, slice q / Tsk of tile q % Tsk, goes to slot q % Px.  A round's pieces are then
    // mostly one slice of Px consecutive tiles, all at the same K-steps, so the XCD's L2
    // serves them from shared panel chunks as in a whole-tile round.  Slice j > 0 of a tile
    // starts from the fp32 accumulators slice j - 1 left in the tile's sk_part buffer (its
    // flag then reads j) and continues the same MFMA sequence, so every element gets the bits
    // of the whole-tile kernel; the last slice runs the epilogue and clears the flag.  A slice
    // waits only for the previous slice of its tile, dealt to an earlier round; the wait is
    // bounded all the same.
    static_assert(!F8 && EPI != EPI_PARTIAL && EPI != EPI_LMHEAD && EPI != EPI_TPROJ, "split tail: projections");
    const int Px = (int)(gridDim.x >> 3), xcd = (int)(blockIdx.x & 7), sl = (int)(blockIdx.x >> 3);
    const int T = n_mt * n_nt, per = T >> 3, rem = T & 7;
    const int Tx = per + (xcd < rem ? 1 : 0);
    const int t0 = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
    const int R = Tx / Px > 0 ? Tx / Px - 1 : 0;       // whole-tile rounds
    const int tb = t0 + R * Px;                        // first shared tile
    const int Tsk = Tx - R * Px;                       // shared tiles
    // S: the fewest rounds of slices, in tiles (ceil(Tsk S / Px) / S), among the S for which
    // no slot runs two slices j and j + k (k >= 2) of one tile: a slot reads a tile's buffer
    // at most once, so its L1 never holds a stale copy of it
    int S = 1, best = (Tsk + Px - 1) / Px;
    for (int c = 2; c <= 4 && nk / c >= 2; ++c) {
      bool ok = true;
      for (int k = 2; k < c; ++k) ok = ok && (k * Tsk) % Px != 0;
      const int rounds = (Tsk * c + Px - 1) / Px;
      if (ok && rounds * S < best * c) { S = c; best = rounds; }
    }
    const int nq = Tsk * S;
    const int npc = R + (nq > sl ? (nq - sl + Px - 1) / Px : 0);
    constexpr int NACC = TM * TN;
    // accumulator image of shared tile t: [wave][block i * TN + j][lane] of 16-byte quads,
    // coalesced 1 KB rows (the lane index counted afresh, as in the epilogue)
    auto part_at = [&](int buf) {
      const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      return (float*)((floatx4_t*)(p.sk_part + (int64_t)buf * (BM * BN)) + (int64_t)wave_s * NACC * 64 + ln);
    };
    auto first_thread = [&]() {
      return wave_s == 0 && __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) == 0;
    };
    // The handover goes through the XCD's L2 (plain stores, loads that miss the L1: the buffer
    // was never read on this CU), which holds only if producer and consumer share an XCD.
    // Workgroups whose indices agree modulo 8 do under the round-robin dispatch (a tile's
    // slices stay within one such class); each workgroup records the XCD it runs on, and a
    // consumer that finds its producer on another XCD reports it (sk_err = 2) instead of
    // trusting the data.
    int32_t* const xcc_of = p.sk_flag + 2 * ZO_SK_MAX_WG;
    const int my_xcc = __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11));   // HW_REG_XCC_ID[3:0]
    if (first_thread()) __hip_atomic_store(xcc_of + blockIdx.x, my_xcc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    set_offsets();                                     // tile-independent (the origin is in rA / rB)
    for (int pc = 0; pc < npc; ++pc) {
      int logical, kb = 0, ke = nk, j = 0, t = 0;
      if (pc < R) {
        logical = t0 + pc * Px + sl;
      } else {
        const int q = (pc - R) * Px + sl;
        j = q / Tsk;
        t = q - j * Tsk;
        logical = tb + t;
        kb = nk * j / S;
        ke = nk * (j + 1) / S;
      }
      const int buf = xcd * 2 * Px + t;                // 2 Px buffers per XCD
      set_tile(logical);
      set_rsrc();
      __syncthreads();                                 // the previous piece's LDS reads are done
      if (j > 0) {
        if (first_thread()) {
          int n = 0;
          while (__hip_atomic_load(p.sk_flag + buf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != j) {
            if (++n > (1 << 20)) { __hip_atomic_store(p.sk_err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); break; }
            __builtin_amdgcn_s_sleep(2);
          }
          // producer of slice j - 1: piece q - Tsk, slot (q - Tsk) % Px of this XCD class
          const int prod = (((pc - R) * Px + sl - Tsk) % Px) * 8 + xcd;
          if (__hip_atomic_load(xcc_of + prod, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != my_xcc)
            __hip_atomic_store(p.sk_err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        float* src = part_at(buf);
        static_for<0, TM>([&](auto i) {
          static_for<0, TN>([&](auto jj) { acc[i][jj] = *(const floatx4_t*)(src + (i * TN + jj) * 256); });
        });
      } else {
        zero_acc();
      }
      kloop_bf16(kb, ke);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (pc >= R && j < S - 1) {
        // plain stores into the XCD's L2 (no agent-scope release: it would write back the
        // whole L2), complete before the barrier; the flag moves on after it
        float* dst = part_at(buf);
        static_for<0, TM>([&](auto i) {
          static_for<0, TN>([&](auto jj) { *(floatx4_t*)(dst + (i * TN + jj) * 256) = acc[i][jj]; });
        });
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __syncthreads();
        if (first_thread()) __hip_atomic_store(p.sk_flag + buf, j + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        if (j > 0 && first_thread()) __hip_atomic_store(p.sk_flag + buf, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        finish();
      }
    }
  }
}

// ------------------------------------------------------------------------------
// fp32 VALU kernel (fp32 models); same accumulator layout as the MFMA path.
template <int BM, int BN, int WM, int WN, int EPI>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_f32_kernel(GemmParams p) {
  constexpr int NWM = BM / WM, NWN = BN / WN, NT = NWM * NWN * 64;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int BK = BK_F32;
  __shared__ float sA[BM][BK + 1];
  __shared__ float sB[BN][BK + 1];
  __shared__ float red[3 * NWN * BM];
  const int n_mt = (p.M + BM - 1) / BM, n_nt = (p.N + BN - 1) / BN;
  int logical;
  tile_swizzle(blockIdx.x, n_mt * n_nt, logical);
  const int mt = logical % n_mt, nt = logical / n_mt;
  const int m0 = mt * BM, n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int grp = (p.n_bounds > 0 && n0 >= p.bounds[0]) + (p.n_bounds > 1 && n0 >= p.bounds[1]) +
                  (p.n_bounds > 2 && n0 >= p.bounds[2]);
  const int a_side_off = grp * p.ks_tile;
  const int nkb = p.K / BK, nk = nkb + p.ks_tile / BK;
  const float* Af = (const float*)p.A;
  const float* Bf = (const float*)p.B;
  const float* Asf = (const float*)p.As;
  const float* Bsf = (const float*)p.Bs;

  floatx4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  for (int kt = 0; kt < nk; ++kt) {
    for (int e = tid; e < BM * BK; e += NT) {
      int r = e / BK, k = e % BK;
      int gr = min(m0 + r, p.M - 1);
      sA[r][k] = kt < nkb ? Af[(int64_t)gr * p.lda + kt * BK + k]
                          : Asf[(int64_t)gr * p.ldas + a_side_off + (kt - nkb) * BK + k];
    }
    for (int e = tid; e < BN * BK; e += NT) {
      int r = e / BK, k = e % BK;
      int gr = min(n0 + r, p.N - 1);
      sB[r][k] = kt < nkb ? Bf[(int64_t)gr * p.ldb + kt * BK + k]
                          : Bsf[(int64_t)gr * p.ldbs + (kt - nkb) * BK + k];
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < BK; ++k) {
      float bv[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) bv[j] = sB[wn * WN + j * 16 + (lane & 15)][k];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float av = sA[wm * WM + i * 16 + 4 * (lane >> 4) + q][k];
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j][q] += av * bv[j];
        }
    }
    __syncthreads();
  }
  epilogue<EPI, TM, TN, BM, BN, WM, WN, float>(p, acc, m0, n0, nt, wm, wn, lane, red);
}

template <int BM, int BN, int WM, int WN, int EPI, bool A8 = false>
hipError_t launch_bf16(const GemmParams& p, hipStream_t s) {
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  const size_t stage = (size_t)(BM + BN) * BK_BF16 * sizeof(bf16_t);
  size_t smem = 2 * stage;
  const size_t red = (size_t)3 * (BN / WN) * BM * sizeof(float);
  if (smem < red) smem = red;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_kernel<BM, BN, WM, WN, EPI, A8>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const int z = EPI == EPI_PARTIAL ? p.ksplit : 1;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, EPI, A8>), dim3(tiles, 1, z), dim3(NT), smem, s, p);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int EPI, bool F8 = false>
hipError_t launch_bf16_pipe(const GemmParams& p, hipStream_t s) {
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  const size_t smem = (size_t)2 * (BM + BN) * 64 * sizeof(bf16_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_pipe_kernel<BM, BN, WM, WN, EPI, F8>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const int z = EPI == EPI_PARTIAL ? p.ksplit : 1;
  hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, EPI, F8>), dim3(tiles, 1, z), dim3(NT), smem, s, p);
  return hipGetLastError();
}

// Split-tail launch of the 256x256 projection kernel: p.sk_ncu persistent workgroups
template <int EPI>
hipError_t launch_bf16_pipe_sk(const GemmParams& p, hipStream_t s) {
  constexpr int BM = 256, BN = 256, WM = 128, WN = 64;
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  const size_t smem = (size_t)2 * (BM + BN) * 64 * sizeof(bf16_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_pipe_kernel<BM, BN, WM, WN, EPI, false, true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, EPI, false, true>), dim3(p.sk_ncu), dim3(NT), smem, s, p);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int EPI>
hipError_t launch_f32(const GemmParams& p, hipStream_t s) {
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, WM, WN, EPI>), dim3(tiles), dim3(NT), 0, s, p);
  return hipGetLastError();
}

// Sum the K-slices in order and apply the side-input epilogue (see EPI_TPROJ).
template <typename TAct>
__global__ void tproj_reduce_kernel(GemmParams p) {
  const int64_t n = (int64_t)p.M * p.N;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(e / p.N), c = (int)(e - (int64_t)r * p.N);
    float v = 0.f;
#pragma unroll 8
    for (int z = 0; z < p.ksplit; ++z) v += p.partial[(int64_t)z * n + e];   // loads in flight together, sums in order
    tproj_out<TAct>(p, r, c, v, p.row_cand[r]);
  }
}

// Sum the K-slices of a projection in order and apply its epilogue (bias, then the bf16
// store, GELU, SwiGLU pairing or the fp32 residual update), the same forms as the
// projection kernel's epilogue.
__global__ void proj_reduce_kernel(GemmParams p) {
  const int NO = p.epi == EPI_SWIGLU ? p.N / 2 : p.N;      // output columns
  const int64_t n = (int64_t)p.M * NO, mn = (int64_t)p.M * p.N;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(e / NO), c = (int)(e - (int64_t)r * NO);
    // e4m3 main segments sum in units of 2^-11 of the result (the weights hold w * 2^11)
    const float unit = p.b_e4m3 ? 1.0f / (float)(1 << ZO_FP8_WEIGHT_EXP) : 1.0f;
    auto sum = [&](int col) {
      float v = 0.f;
#pragma unroll 8
      for (int z = 0; z < p.ksplit; ++z) v += p.partial[(int64_t)z * mn + (int64_t)r * p.N + col];
      return v * unit + (p.bias ? p.bias[col] : 0.f);
    };
    if (p.epi == EPI_SWIGLU) {       // packed rows: 16 gate rows, then the 16 matching up rows
      const int g = (c / 16) * 32 + c % 16;
      const float v = silu_fast(sum(g)) * sum(g + 16);
      if (p.a_e4m3)                  // the e4m3 input of the down projection
        ((e4m3_t*)p.C)[(int64_t)r * p.ldc + c] = (e4m3_t)(f32x4_to_e4m3(v, 0.f, 0.f, 0.f) & 0xffu);
      else
        ((bf16_t*)p.C)[(int64_t)r * p.ldc + c] = f32_to_bf16(v);
    } else if (p.epi == EPI_RESID) {
      p.H[(int64_t)r * p.ldh + c] += sum(c);
    } else if (p.epi == EPI_GELU) {
      const float v = gelu_fast(sum(c));
      if (p.a_e4m3)                  // the e4m3 input of the next projection
        ((e4m3_t*)p.C)[(int64_t)r * p.ldc + c] = (e4m3_t)(f32x4_to_e4m3(v, 0.f, 0.f, 0.f) & 0xffu);
      else
        ((bf16_t*)p.C)[(int64_t)r * p.ldc + c] = f32_to_bf16(v);
    } else {
      ((bf16_t*)p.C)[(int64_t)r * p.ldc + c] = f32_to_bf16(sum(c));
    }
  }
}

// ------------------------------------------------------------------------------
// Side-input projection for few factor columns (rank <= 8, a few t slots): a streaming
// kernel on the vector units instead of an MFMA tile that is mostly padding.  A workgroup
// takes R rows; its 256 lanes split each row into 8-element chunks (lane l of wave w takes
// chunks l + 64 w + 256 i), multiply them with the same chunks of NC used V^T rows
// (bf16, read through the caches, shared by every row) and sum in fp32; the partial sums
// are reduced across a wave's lanes (butterfly) and then across the four waves in wave
// order, so each (row, column) value is formed by the same operations whatever the batch.
// Column c_j = (j / tp_used) * tp_ks + j % tp_used (kind block, used column of the block);
// the result goes through tproj_out like the tiled kernel's.  A8: e4m3 activations.
template <int R, int NC, bool A8>
__global__ void __launch_bounds__(256)
side_dot_kernel(GemmParams p, int j0, int n_used) {
  __shared__ float red[4][R][NC];
  const int m0 = blockIdx.x * R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncols = min(NC, n_used - j0);            // used columns of this pass
  const int nch = p.K / 8;
  int rows[R];
  bool live = false;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    rows[i] = min(m0 + i, p.M - 1);
    live |= (m0 + i < p.M) && p.row_cand[rows[i]] >= 0;
  }
  if (!live) return;                                   // foreground rows only: nothing to write
  const bf16_t* vrow[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int j = j0 + min(c, ncols - 1);
    const int col = (j / p.tp_used) * p.tp_ks + j % p.tp_used;
    vrow[c] = (const bf16_t*)p.B + (int64_t)col * p.ldb;
  }
  float acc[R][NC];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[i][c] = 0.f;
  for (int ch = tid; ch < nch; ch += 256) {
    float v[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const u32x4_t w = *(const u32x4_t*)(vrow[c] + ch * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[c][2 * e] = bf16_to_f32((bf16_t)(w[e] & 0xFFFFu));
        v[c][2 * e + 1] = bf16_to_f32((bf16_t)(w[e] >> 16));
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float x[8];
      if constexpr (A8) {
        const uint2 b = *(const uint2*)((const e4m3_t*)p.A + (int64_t)rows[i] * p.lda + ch * 8);
        const u32x4_t w = e4m3x8_to_bf16(b);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = bf16_to_f32((bf16_t)(w[e] & 0xFFFFu));
          x[2 * e + 1] = bf16_to_f32((bf16_t)(w[e] >> 16));
        }
      } else {
        const u32x4_t w = *(const u32x4_t*)((const bf16_t*)p.A + (int64_t)rows[i] * p.lda + ch * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = bf16_to_f32((bf16_t)(w[e] & 0xFFFFu));
          x[2 * e + 1] = bf16_to_f32((bf16_t)(w[e] >> 16));
        }
      }
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][c] = fmaf(x[e], v[c][e], acc[i][c]);
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float a = acc[i][c];
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) a += __shfl_xor(a, sh, 64);
      if (lane == 0) red[wave][i][c] = a;
    }
  __syncthreads();
  if (tid < R * NC) {
    const int i = tid / NC, c = tid % NC;
    const int r = m0 + i;
    if (r < p.M && c < ncols) {
      const float t = ((red[0][i][c] + red[1][i][c]) + red[2][i][c]) + red[3][i][c];
      const int j = j0 + c;
      tproj_out<bf16_t>(p, r, (j / p.tp_used) * p.tp_ks + j % p.tp_used, t, p.row_cand[r]);
    }
  }
}

// t of the projection that reads an epilogue's output: one wave per row sums the row's group
// partials ([M][groups][sf_n], a row's contiguous): lane l takes groups l, l + 64, ... in order,
// then a fixed butterfly over the lanes, so each (row, column) value is formed by the same
// operations whatever the batch
__global__ void __launch_bounds__(256) side_part_reduce_kernel(GemmParams p) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= p.M) return;                               // wave-uniform
  const int cand = p.row_cand[r];
  if (cand < 0) return;
  const float* pr = p.sf_part + (int64_t)r * p.sf_groups * p.sf_n;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int g = lane; g < p.sf_groups; g += 64)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (c < p.sf_n) v[c] += pr[g * p.sf_n + c];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) v[c] += __shfl_xor(v[c], sh, 64);
  if (lane == 0)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (c < p.sf_n) tproj_out<bf16_t>(p, r, (c / p.tp_used) * p.tp_ks + c % p.tp_used, v[c], cand);
}

}  // namespace

hipError_t launch_side_part_reduce(const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.sf_n <= 0) return hipSuccess;
  if (p.sf_n > 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(side_part_reduce_kernel, dim3((unsigned)((p.M + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Used factor columns of a side-input projection (the kind blocks times the used columns
// of each block) when the streaming kernel serves it, else 0.
static int side_dot_columns(const GemmParams& p) {
  if (p.epi != EPI_TPROJ || p.kwa || p.tp_unit || p.b_e4m3 || p.tp_used <= 0 || p.tp_ks <= 0) return 0;
  if (p.K % 8 != 0 || p.lda % 8 != 0 || p.ldb % 8 != 0 || p.N % p.tp_ks != 0) return 0;
  // measured at OPT-13B batch 64: two columns (one kind block at r = 2) stream at about the
  // rate of the tiled kernel without its K-slice reduction; six columns (q|k|v) ran at a
  // third of it (the per-row reduction of 64 partial sums dominates), so wider sets keep
  // the tiled kernel
  const int n = (p.N / p.tp_ks) * p.tp_used;
  return n <= 2 ? n : 0;
}

// R rows per workgroup: 8 for large batches, 2 for small ones (more workgroups in flight).
// A lane's chunks and the reduction order do not depend on R, so neither does any result.
template <int R, int NC>
static hipError_t launch_side_dot_rnc(const GemmParams& p, int j0, int ncols, hipStream_t s) {
  const int blocks = (p.M + R - 1) / R;
  if (p.a_e4m3)
    hipLaunchKernelGGL((side_dot_kernel<R, NC, true>), dim3(blocks), dim3(256), 0, s, p, j0, ncols);
  else
    hipLaunchKernelGGL((side_dot_kernel<R, NC, false>), dim3(blocks), dim3(256), 0, s, p, j0, ncols);
  return hipGetLastError();
}
template <int NC>
static hipError_t launch_side_dot_nc(const GemmParams& p, int j0, int ncols, hipStream_t s) {
  return p.M >= 4096 ? launch_side_dot_rnc<8, NC>(p, j0, ncols, s) : launch_side_dot_rnc<2, NC>(p, j0, ncols, s);
}

static hipError_t launch_side_dot(const GemmParams& p, int ncols, hipStream_t s) {
  return launch_side_dot_nc<2>(p, 0, ncols, s);
}

hipError_t launch_proj_reduce(const GemmParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.M * (p.epi == EPI_SWIGLU ? p.N / 2 : p.N);
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(proj_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_tproj_reduce(const GemmParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.M * p.N;
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(tproj_reduce_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Tile shapes per call site.  BIG: the shared-weight projections; NARROW: the
// side-input projection (N = a few kind blocks); HEAD: the vocabulary head (the
// projection kernel with 256-column tiles).
int gemm_cfg_bm(int cfg, bool bf16) {
  if (!bf16) return 64;
  return cfg == GEMM_CFG_NARROW ? 64 : 256;
}
int gemm_cfg_bn(int cfg, bool bf16) {
  if (!bf16) return 64;
  return cfg == GEMM_CFG_NARROW ? 128 : 256;
}
// K granularity of each call site: every bf16 kernel steps K by 64.
int gemm_cfg_bk(int cfg, bool bf16) {
  (void)cfg;
  return bf16 ? BK_BF16 : BK_F32;
}
// side-input column granularity (a multiple of every consumer's K-step)
int gemm_bk(bool bf16) { return bf16 ? BK_BF16 : BK_F32; }

template <int BM, int BN, int WM, int WN>
hipError_t launch_pipe_epi(const GemmParams& p, hipStream_t s) {
  if (p.a_e4m3 || p.b_e4m3) {
    // e4m3 x e4m3 main segment (fp8 models: no two-term operands)
    if constexpr (BM == 128 && BN == 128) {
      if (!(p.a_e4m3 && p.b_e4m3) || p.kwa || p.kwb || p.kwas || p.c_lo || p.c_f32 || p.K % 128 != 0)
        return hipErrorInvalidValue;
      switch (p.epi) {
        case EPI_STORE: return launch_bf16_pipe<BM, BN, WM, WN, EPI_STORE, true>(p, s);
        case EPI_GELU: return launch_bf16_pipe<BM, BN, WM, WN, EPI_GELU, true>(p, s);
        case EPI_SWIGLU: return launch_bf16_pipe<BM, BN, WM, WN, EPI_SWIGLU, true>(p, s);
        case EPI_RESID: return launch_bf16_pipe<BM, BN, WM, WN, EPI_RESID, true>(p, s);
        default: break;
      }
    }
    return hipErrorInvalidValue;
  }
  switch (p.epi) {
    case EPI_STORE: return launch_bf16_pipe<BM, BN, WM, WN, EPI_STORE>(p, s);
    case EPI_GELU: return launch_bf16_pipe<BM, BN, WM, WN, EPI_GELU>(p, s);
    case EPI_SWIGLU: return launch_bf16_pipe<BM, BN, WM, WN, EPI_SWIGLU>(p, s);
    case EPI_RESID: return launch_bf16_pipe<BM, BN, WM, WN, EPI_RESID>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// Workgroup tile of the projection kernel: 256x256 (eight 128x64 wave tiles) or 128x128
// (four 64x64 wave tiles).  Every wave tile is a grid of 16x16 MFMA blocks fed with the
// same operands in the same K order (32 per instruction, ascending), so every output
// element is formed by the same MFMA sequence whichever tile holds it; the choice can
// follow the batch without changing a row's result (checked bit for bit).  The 256x256
// tile is the most efficient per CU; measured on the projections of small batches, the
// 128x128 tile pays off when 256x256 tiles would occupy fewer than half of the 256 CUs.
int pipe_tile(const GemmParams& p) {
  const int64_t t256 = (int64_t)((p.M + 255) / 256) * ((p.N + 255) / 256);
  return t256 >= 128 ? 0 : 1;
}

// Split tail for a 256x256-tile projection: when the workspace provides for it, every CU can
// hold a workgroup, there is at least one whole round of tiles, and the last round of the
// data-parallel launch would leave more than 2 % of the CU time idle.  ZO_GEMM_SPLIT_TAIL=0
// turns it off (the outputs are the same bits either way).
bool use_split_tail(const GemmParams& p) {
  if (!p.sk_part || !p.sk_flag || !p.sk_err || p.sk_ncu < 8 || p.sk_ncu % 8 != 0 || p.sk_ncu > ZO_SK_MAX_WG)
    return false;
  if (p.a_e4m3 || p.b_e4m3 || p.ksplit > 1) return false;
  // (the GELU / SwiGLU epilogues with their side-input partials would spill in the K loop
  // beside the piece state)
  if (p.epi != EPI_STORE && p.epi != EPI_RESID) return false;
  // the slices' handovers pay for themselves on long K only (measured at OPT-13B batch 64:
  // fc2, 320 K-steps, 1590 -> 1487 us; o, 80 K-steps, 431 -> 476 us)
  if (p.K / 64 + p.ks_tile / 64 < 160) return false;
  const char* env = getenv("ZO_GEMM_SPLIT_TAIL");
  if (env && env[0] == '0') return false;
  const int64_t t = (int64_t)((p.M + 255) / 256) * ((p.N + 255) / 256), P = p.sk_ncu;
  if (t < P) return false;
  const int64_t rounds = (t + P - 1) / P;
  return (double)(rounds * P - t) > 0.02 * (double)t;
}

hipError_t gemm_launch_bf16(const GemmParams& p, int cfg, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (cfg == GEMM_CFG_BIG) {
    // K-slices (decode steps of generation: a few rows, so the weights are streamed by
    // ksplit x more workgroups): fp32 partial sums of the 128x128-tile kernel, the side
    // segment in the last slice, then an ordered reduction that applies the epilogue
    if (p.ksplit > 1) {
      const bool f8 = p.a_e4m3 && p.b_e4m3;
      if (p.a_e4m3 != p.b_e4m3 || p.kwa || p.kwb || p.kwas || p.c_lo || p.c_f32 || !p.partial ||
          (p.K / (f8 ? 128 : 64)) % p.ksplit != 0)
        return hipErrorInvalidValue;
      GemmParams q = p;
      q.epi = EPI_PARTIAL;
      hipError_t e = f8 ? launch_bf16_pipe<128, 128, 64, 64, EPI_PARTIAL, true>(q, s)
                        : launch_bf16_pipe<128, 128, 64, 64, EPI_PARTIAL>(q, s);
      if (e != hipSuccess) return e;
      return launch_proj_reduce(p, s);
    }
    // e4m3 projections: always 128x128 tiles of four 64x64 wave tiles.  The 128x64 wave
    // tile needs 128 accumulator registers next to 32-byte fragments, more than the 256 a
    // lane has at two waves a SIMD (spills); the 128x128 tile streams the same bytes per
    // product from L2 as the bf16 256x256 tile (half-size elements)
    if (p.a_e4m3 || p.b_e4m3) return launch_pipe_epi<128, 128, 64, 64>(p, s);
    // (measured at OPT-13B batch 64: finishing the last partial round of 256x256 tiles in
    // 128x128 tiles of a second launch made the projections 6 % slower, not faster)
    if (pipe_tile(p) == 0) {
      if (use_split_tail(p)) {
        if (p.epi == EPI_STORE) return launch_bf16_pipe_sk<EPI_STORE>(p, s);
        return launch_bf16_pipe_sk<EPI_RESID>(p, s);
      }
      return launch_pipe_epi<256, 256, 128, 64>(p, s);
    }
    return launch_pipe_epi<128, 128, 64, 64>(p, s);
  }
  if (cfg == GEMM_CFG_NARROW) {
    if (p.b_e4m3 || (p.a_e4m3 && (p.epi != EPI_TPROJ || p.N > 128 || p.kwa))) return hipErrorInvalidValue;
    // rank <= 8 with a few t slots: the streaming kernel over the used columns only
    if (const int nc = side_dot_columns(p)) return launch_side_dot(p, nc, s);
    if (p.a_e4m3) {
      // e4m3 activations against the bf16 factor rows: the register-staged tiles, which
      // widen A to bf16 (exactly) on its way to LDS
      const bool thin = p.N <= 32;
      if (p.ksplit <= 1)
        return thin ? launch_bf16<128, 32, 32, 32, EPI_TPROJ, true>(p, s)
                    : launch_bf16<64, 128, 32, 64, EPI_TPROJ, true>(p, s);
      GemmParams q = p;
      q.epi = EPI_PARTIAL;
      hipError_t e = thin ? launch_bf16<128, 32, 32, 32, EPI_PARTIAL, true>(q, s)
                          : launch_bf16<64, 128, 32, 64, EPI_PARTIAL, true>(q, s);
      if (e != hipSuccess) return e;
      return launch_tproj_reduce(p, s);
    }
    // more than one 128-column tile of factor columns (high rank, several entries): the
    // pipelined projection kernel; with K-slices, fp32 partial sums and the fixed-order
    // reduction that applies the epilogue
    if (p.epi == EPI_TPROJ && p.N > 128 && p.N % 16 == 0 && p.K % 64 == 0) {
      if (p.ksplit <= 1) return launch_bf16_pipe<256, 256, 128, 64, EPI_TPROJ>(p, s);
      if ((p.K / 64) % p.ksplit != 0) return hipErrorInvalidValue;
      GemmParams q = p;
      q.epi = EPI_PARTIAL;
      hipError_t e = launch_bf16_pipe<256, 256, 128, 64, EPI_PARTIAL>(q, s);
      if (e != hipSuccess) return e;
      return launch_tproj_reduce(p, s);
    }
    if (p.epi == EPI_TPROJ) {
      // N <= 32 (one kind block at rank <= 8 and few entries): a 128 x 32 tile, so the
      // factor rows are not re-read for absent columns
      const bool thin = p.N <= 32;
      if (p.ksplit <= 1)
        return thin ? launch_bf16<128, 32, 32, 32, EPI_TPROJ>(p, s) : launch_bf16<64, 128, 32, 64, EPI_TPROJ>(p, s);
      // split-K partial sums, then a fixed-order reduction that applies the epilogue
      GemmParams q = p;
      q.epi = EPI_PARTIAL;
      hipError_t e = thin ? launch_bf16<128, 32, 32, 32, EPI_PARTIAL>(q, s) : launch_bf16<64, 128, 32, 64, EPI_PARTIAL>(q, s);
      if (e != hipSuccess) return e;
      return launch_tproj_reduce(p, s);
    }
    if (p.epi == EPI_STORE) return launch_bf16<64, 128, 32, 64, EPI_STORE>(p, s);
    return hipErrorInvalidValue;
  }
  // the vocabulary head: always 256-column tiles (the log-sum-exp partials, and so each
  // row's result, then do not depend on the batch); 128 or 256 rows per tile
  if (p.epi == EPI_LMHEAD) {
    if (p.a_e4m3 || p.b_e4m3) return hipErrorInvalidValue;
    auto tiles = [&](int bm) { return (int64_t)((p.M + bm - 1) / bm) * ((p.N + 255) / 256); };
    if (tiles(256) >= 128) return launch_bf16_pipe<256, 256, 128, 64, EPI_LMHEAD>(p, s);
    return launch_bf16_pipe<128, 256, 128, 64, EPI_LMHEAD>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t gemm_launch_f32(const GemmParams& p, int cfg, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  (void)cfg;
  switch (p.epi) {
    case EPI_STORE: return launch_f32<64, 64, 32, 32, EPI_STORE>(p, s);
    case EPI_GELU: return launch_f32<64, 64, 32, 32, EPI_GELU>(p, s);
    case EPI_SWIGLU: return launch_f32<64, 64, 32, 32, EPI_SWIGLU>(p, s);
    case EPI_RESID: return launch_f32<64, 64, 32, 32, EPI_RESID>(p, s);
    case EPI_TPROJ: return launch_f32<64, 64, 32, 32, EPI_TPROJ>(p, s);
    case EPI_LMHEAD: return launch_f32<64, 64, 32, 32, EPI_LMHEAD>(p, s);
    default: return hipErrorInvalidValue;
  }
}
