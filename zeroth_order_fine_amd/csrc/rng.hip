// Counter-based random streams on the GPU: Philox4x32-10 and an exact-operation
// Box-Muller transform.
//
// Philox4x32-10 is written from its published definition (Salmon et al.,
// "Parallel random numbers: as easy as 1, 2, 3", SC'11).  The Gaussian
// transform uses only correctly rounded binary64 +, -, *, / and sqrt, in a
// fixed order with contraction disabled, so that any implementation of the
// same specification produces the same bits:
//   u = (w + 1/2) 2^-32,  R = sqrt(-2 ln u)
//   ln u: frexp split u = m 2^e, m in [sqrt(1/2), sqrt 2); s = (m-1)/(m+1);
//         ln m = 2 s sum_{k<=11} s^(2k)/(2k+1) (Horner); ln u = e*ln2_hi + (e*ln2_lo + ln m)
//   angle word: quadrant = bits 31..30, half bit = bit 29, f = (bits 28..0 + 1/2) 2^-29,
//         phi = f*pi/4, (cos, sin) by nested Taylor forms, swapped when the half bit
//         is set (psi = pi/2 - phi), then rotated by the quadrant (sign flips / swaps).
// Stream element e of (seed, tag, tau) is lane e%4 of the block with counter
// (e/4, tag, lo32 tau, hi32 tau) and key (lo32 seed, hi32 seed); lanes (0,1) and
// (2,3) are the two Box-Muller pairs (radius word first).
//
// The method draws its random directions from seed, step and layer
// ("Zeroth-Order Fine-Tuning Was an Inference Workload All Along", section
// "The System Reorganization": the random-direction stream is unchanged, V is
// held for a window, the other factor is resampled each step), so the factors
// are regenerated here rather than stored.
#include "common.h"

namespace {

struct u4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                           uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  return u4{c0, c1, c2, c3};
}

__device__ __forceinline__ double ln_exact(double u) {
#pragma clang fp contract(off)
  int e;
  double m = frexp(u, &e);
  const int below = m < 0x1.6a09e667f3bcdp-1;
  m = below ? m * 2.0 : m;
  e = e - below;
  double s = (m - 1.0) / (m + 1.0);
  double s2 = s * s;
  double p = 1.0 / 23.0;
#pragma unroll
  for (int k = 10; k >= 0; --k) {
    double t = p * s2;
    p = t + 1.0 / (double)(2 * k + 1);
  }
  double sp = s * p;
  double lnm = sp + sp;
  double ed = (double)e;
  double lo = ed * 0x1.a39ef35793c76p-33;
  double hi = ed * 0x1.62e42fee00000p-1;
  return hi + (lo + lnm);
}

__device__ __forceinline__ double sin_q(double x) {
#pragma clang fp contract(off)
  double x2 = x * x;
  double p = 1.0;
#pragma unroll
  for (int k = 10; k >= 1; --k) {
    double r = 1.0 / (double)((2 * k) * (2 * k + 1));
    double t = x2 * r;
    double tp = t * p;
    p = 1.0 - tp;
  }
  return x * p;
}

__device__ __forceinline__ double cos_q(double x) {
#pragma clang fp contract(off)
  double x2 = x * x;
  double p = 1.0;
#pragma unroll
  for (int k = 11; k >= 1; --k) {
    double r = 1.0 / (double)((2 * k - 1) * (2 * k));
    double t = x2 * r;
    double tp = t * p;
    p = 1.0 - tp;
  }
  return p;
}

__device__ __forceinline__ double flip_sign(double x, uint32_t neg) {
  return __builtin_bit_cast(double, __builtin_bit_cast(uint64_t, x) ^ ((uint64_t)neg << 63));
}

// Branch-free selection: every case computes the same operations, then picks
// bits, so the rotation by the quadrant is exact sign flips and swaps.
__device__ __forceinline__ double pick(uint32_t cond, double a, double b) {   // cond ? a : b
  const uint64_t m = 0ull - (uint64_t)(cond & 1u);
  return __builtin_bit_cast(double, (__builtin_bit_cast(uint64_t, a) & m) | (__builtin_bit_cast(uint64_t, b) & ~m));
}

__device__ __forceinline__ void box_muller(uint32_t wa, uint32_t wb, double& za, double& zb) {
#pragma clang fp contract(off)
  double u = ((double)wa + 0.5) * 0x1p-32;
  double l = ln_exact(u);
  double m2 = -2.0 * l;
  double R = __builtin_sqrt(m2);
  const uint32_t quad = wb >> 30;
  const uint32_t h = (wb >> 29) & 1u;
  double f = ((double)(wb & 0x1FFFFFFFu) + 0.5) * 0x1p-29;
  double phi = f * 0x1.921fb54442d18p-1;
  double c = cos_q(phi), s = sin_q(phi);
  const double cp = pick(h, s, c), sp = pick(h, c, s);          // psi = pi/2 - phi when h
  const double x = pick(quad, sp, cp), y = pick(quad, cp, sp);  // odd quadrant: swap
  const double ct = flip_sign(x, ((quad + 1) >> 1) & 1u);       // negative in quadrants 1, 2
  const double st = flip_sign(y, quad >> 1);                    // negative in quadrants 2, 3
  za = R * ct;
  zb = R * st;
}

// The 4 Gaussians of Philox block j of stream (seed, tag, tau).
__device__ __forceinline__ void normal4(uint64_t seed, uint32_t tag, uint64_t tau, uint64_t j, double z[4]) {
  u4 w = philox4x32_10((uint32_t)j, tag, (uint32_t)tau, (uint32_t)(tau >> 32), (uint32_t)seed,
                       (uint32_t)(seed >> 32));
  box_muller(w.x, w.y, z[0], z[1]);
  box_muller(w.z, w.w, z[2], z[3]);
}

__device__ __forceinline__ int64_t interleave16_row(int64_t row, int which) {
  // packed [gate 16 rows | up 16 rows] groups: which = 1 gate, 2 up
  return (row >> 4) * 32 + (which == 2 ? 16 : 0) + (row & 15);
}

__global__ void normal_jobs_kernel(const NormalJob* __restrict__ jobs, int64_t max_blocks) {
#pragma clang fp contract(off)
  const NormalJob jb = jobs[blockIdx.y];
  const int64_t n = jb.rows * jb.cols;
  const int64_t nblk = (n + 3) / 4;
  const int init = jb.mode & 15;      // 0: 0.02 z, 1: 1 + 0.02 z
  const int layout = (int)jb.aux;     // 0 plain, 1 gate, 2 up (16-row interleave)
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < nblk;
       j += (int64_t)gridDim.x * blockDim.x) {
    double z[4];
    normal4(jb.seed, jb.tag, jb.tau, (uint64_t)j, z);
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      int64_t e = 4 * j + l;
      if (e >= n) break;
      double v = 0.02 * z[l];
      if (init == 1) v = 1.0 + v;
      float f = (float)v;
      int64_t row = e / jb.cols, col = e - row * jb.cols;
      int64_t prow = layout ? interleave16_row(row, layout) : row;
      int64_t off = prow * jb.ld + col;
      if (jb.dtype == 1) {
        ((bf16_t*)jb.dst)[off] = f32_to_bf16(f);
      } else if (jb.dtype == 2) {         // e4m3 code of f * 2^11 (exact scaling, then one rounding)
        const float x = f * (float)(1 << ZO_FP8_WEIGHT_EXP);
        ((e4m3_t*)jb.dst)[off] = (e4m3_t)(f32x4_to_e4m3(x, 0.f, 0.f, 0.f) & 0xffu);
      } else {
        ((float*)jb.dst)[off] = f;
      }
    }
  }
}

__global__ void normal_fill_f64_kernel(uint64_t seed, uint32_t tag, uint64_t tau, int64_t first, int64_t n,
                                       double* out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    int64_t e = first + i;
    double z[4];
    normal4(seed, tag, tau, (uint64_t)(e >> 2), z);
    out[i] = z[e & 3];
  }
}

__global__ void words_fill_kernel(uint64_t seed, uint32_t tag, uint64_t tau, int64_t first_block, int64_t n_blocks,
                                  uint32_t* out) {
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < n_blocks;
       b += (int64_t)gridDim.x * blockDim.x) {
    uint64_t j = (uint64_t)(first_block + b);
    u4 w = philox4x32_10((uint32_t)j, tag, (uint32_t)tau, (uint32_t)(tau >> 32), (uint32_t)seed,
                         (uint32_t)(seed >> 32));
    out[4 * b + 0] = w.x; out[4 * b + 1] = w.y; out[4 * b + 2] = w.z; out[4 * b + 3] = w.w;
  }
}

// fp32, bf16, or (split > 0, bf16) the copies hi | hi | lo at off, off + split, off + 2 split;
// dtype 2: bf16 of v * 2^11 (exact scaling), the side factors of fp8 models' projections
__device__ __forceinline__ void store_as(void* dst, int64_t off, float v, int dtype, int64_t split) {
  if (dtype == 2) {
    ((bf16_t*)dst)[off] = f32_to_bf16(v * (float)(1 << ZO_FP8_WEIGHT_EXP));
  } else if (dtype == 1) {
    bf16_t* o = (bf16_t*)dst + off;
    if (split > 0) {
      bf16_t hi, lo;
      split_bf16(v, hi, lo);
      o[0] = hi;
      o[split] = hi;
      o[2 * split] = lo;
    } else {
      *o = f32_to_bf16(v);
    }
  } else {
    ((float*)dst)[off] = v;
  }
}

__global__ void side_jobs_kernel(const SideJob* __restrict__ jobs) {
  const SideJob jb = jobs[blockIdx.y];
  const int64_t n_el = jb.n * jb.r;
  if (jb.src == 0 || jb.src == 1) {            // V (transposed rows) or G stream
    const int64_t nblk = (n_el + 3) / 4;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < nblk;
         j += (int64_t)gridDim.x * blockDim.x) {
      double z[4];
      normal4(jb.seed, jb.tag, jb.tau, (uint64_t)j, z);
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        int64_t e = 4 * j + l;
        if (e >= n_el) break;
        int64_t i = e / jb.r, k = e - i * jb.r;
        float f = (float)z[l];                  // factors are fp32 N(0,1)
        int64_t off;
        if (jb.src == 0) off = k * jb.ld + i;   // Vt[k][i] = V[i][k]
        else {
          int64_t prow = jb.row_map ? interleave16_row(i, jb.row_map) : i;
          off = prow * jb.ld + jb.col0 + k;
        }
        store_as(jb.dst, off, f, jb.dtype, jb.split);
      }
    }
  } else if (jb.src == 2) {                     // bank U -> Bs columns
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n_el;
         e += (int64_t)gridDim.x * blockDim.x) {
      int64_t i = e / jb.r, k = e - i * jb.r;
      int64_t prow = jb.row_map ? interleave16_row(i, jb.row_map) : i;
      store_as(jb.dst, prow * jb.ld + jb.col0 + k, jb.u_src[e], jb.dtype, jb.split);
    }
  }
}

__global__ void update_kernel(UpdateArgs a) {
#pragma clang fp contract(off)
  const int layer = blockIdx.y / a.n_kinds, kk = blockIdx.y % a.n_kinds;
  const int d = blockIdx.z;
  const int64_t n = a.kind_n[kk];
  float* U = a.u_base + a.slot_off[d] + (int64_t)layer * a.layer_stride + a.kind_off[kk];
  const uint32_t tag = ((uint32_t)layer << 8) | ((uint32_t)a.kind_id[kk] << 1);   // factor G
  const int64_t nblk = (n + 3) / 4;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < nblk;
       j += (int64_t)gridDim.x * blockDim.x) {
    double z[4];
    normal4(a.seed[d], tag, a.t, (uint64_t)j, z);
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      int64_t e = 4 * j + l;
      if (e >= n) break;
      double g = (double)(float)z[l];          // G entries are fp32 values
      double u = a.fresh[d] ? 0.0 : (double)U[e];
      double t = a.coef[d] * g;
      U[e] = (float)(u - t);
    }
  }
}

// W <- round(W + sum_k U[:, k] V[:, k]^T) for one target linear: fp64 sum in k order
// (no contraction), then fp64 -> fp32 -> (bf16) by round to nearest even.
// value of an OCP e4m3 code (exact: subnormals mant * 2^-9, normals (8 + mant) * 2^(exp - 10))
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, mant = c & 7u;
  const float mag = e == 0 ? (float)mant * 0x1p-9f : ldexpf((float)(8u + mant), (int)e - 10);
  return (c & 0x80u) ? -mag : mag;
}

__global__ void fold_kernel(FoldArgs a) {
#pragma clang fp contract(off)
  const int64_t n = a.n_out * a.n_in;
  constexpr float kUnit = 1.0f / (float)(1 << ZO_FP8_WEIGHT_EXP);
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / a.n_in, j = e - i * a.n_in;
    const int64_t prow = a.layout ? interleave16_row(i, a.layout) : i;
    const int64_t off = prow * a.ld + j;
    double acc = a.dtype == 1   ? (double)bf16_to_f32(((const bf16_t*)a.w)[off])
                 : a.dtype == 2 ? (double)(e4m3_value(((const e4m3_t*)a.w)[off]) * kUnit)
                                : (double)((const float*)a.w)[off];
    for (int k = 0; k < a.r; ++k) acc = acc + (double)a.u[i * a.r + k] * (double)a.v[j * a.r + k];
    const float f = (float)acc;
    if (a.dtype == 1) ((bf16_t*)a.w)[off] = f32_to_bf16(f);
    else if (a.dtype == 2)   // requantize: the e4m3 code of f * 2^11 (nearest even, saturating)
      ((e4m3_t*)a.w)[off] = (e4m3_t)(f32x4_to_e4m3(f * (float)(1 << ZO_FP8_WEIGHT_EXP), 0.f, 0.f, 0.f) & 0xFFu);
    else ((float*)a.w)[off] = f;
  }
}

__global__ void side_job_single_kernel(SideJob jb) {
  const int64_t n_el = jb.n * jb.r;
  const int64_t nblk = (n_el + 3) / 4;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < nblk;
       j += (int64_t)gridDim.x * blockDim.x) {
    double z[4];
    normal4(jb.seed, jb.tag, jb.tau, (uint64_t)j, z);
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      int64_t e = 4 * j + l;
      if (e >= n_el) break;
      ((float*)jb.dst)[e] = (float)z[l];
    }
  }
}

inline unsigned grid_for(int64_t items, int threads, int64_t cap = 65535) {
  int64_t g = (items + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_normal_jobs(const NormalJob* jobs_dev, int n_jobs, int64_t max_blocks, hipStream_t s) {
  if (n_jobs <= 0) return hipSuccess;
  dim3 grid(grid_for(max_blocks, 256, 4096), n_jobs);
  hipLaunchKernelGGL(normal_jobs_kernel, grid, dim3(256), 0, s, jobs_dev, max_blocks);
  return hipGetLastError();
}

hipError_t launch_normal_fill_f64(uint64_t seed, uint32_t tag, uint64_t tau, int64_t first, int64_t n,
                                  double* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(normal_fill_f64_kernel, dim3(grid_for(n, 256, 8192)), dim3(256), 0, s, seed, tag, tau,
                     first, n, out);
  return hipGetLastError();
}

hipError_t launch_words_fill(uint64_t seed, uint32_t tag, uint64_t tau, int64_t first_block, int64_t n_blocks,
                             uint32_t* out, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(words_fill_kernel, dim3(grid_for(n_blocks, 256, 8192)), dim3(256), 0, s, seed, tag, tau,
                     first_block, n_blocks, out);
  return hipGetLastError();
}

hipError_t launch_side_jobs(const SideJob* jobs_dev, int n_jobs, int64_t max_items, hipStream_t s) {
  for (int j0 = 0; j0 < n_jobs; j0 += 65535) {
    const int nj = n_jobs - j0 < 65535 ? n_jobs - j0 : 65535;
    dim3 grid(grid_for(max_items, 256, 1024), nj);
    hipLaunchKernelGGL(side_jobs_kernel, grid, dim3(256), 0, s, jobs_dev + j0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_update(const UpdateArgs& a, int n_layers, int64_t max_n, hipStream_t s) {
  if (a.n_dirs <= 0 || a.n_kinds <= 0 || n_layers <= 0) return hipSuccess;
  dim3 grid(grid_for((max_n + 3) / 4, 256, 256), n_layers * a.n_kinds, a.n_dirs);
  hipLaunchKernelGGL(update_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fold(const FoldArgs& a, hipStream_t s) {
  const int64_t n = a.n_out * a.n_in;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fold_kernel, dim3(grid_for(n, 256, 16384)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stream_rowmajor(const SideJob& jb, hipStream_t s) {
  hipLaunchKernelGGL(side_job_single_kernel, dim3(grid_for((jb.n * jb.r + 3) / 4, 256, 1024)), dim3(256), 0, s, jb);
  return hipGetLastError();
}
