// Microbenchmarks for the measured ceilings bench.py reports beside the published
// peaks: a dense bf16 MFMA loop (16 independent accumulators per wave, four waves per
// SIMD), once on constant operands and once on random ones (the matrix cores draw more
// power, and the clock drops, when the operand bits toggle as they do in a real product),
// and a streaming copy / read over a buffer much larger than the caches.  Not
// part of the method; built into a separate library that only bench.py loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float floatx4_t;

namespace {

__global__ void __launch_bounds__(256) mfma_loop(float* out, int iters) {
  bf16x8_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 0.001f + i);
    b[i] = (__bf16)(i * 0.5f);
  }
  floatx4_t acc[16];
  for (int i = 0; i < 16; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
  return x;
}

// The same loop on random operands: per lane two A fragments uniform in [-1, 1) and two B
// fragments uniform in [-0.05, 0.05) (the ranges of normalised activations and of the
// weights), alternated so that consecutive MFMAs see different operand bits.
__global__ void __launch_bounds__(256) mfma_loop_random(float* out, int iters) {
  bf16x8_t a[2], b[2];
  for (int v = 0; v < 2; ++v)
    for (int i = 0; i < 8; ++i) {
      const uint32_t h = mix32((blockIdx.x * 256u + threadIdx.x) * 977u + i * 31u + v * 7u);
      a[v][i] = (__bf16)((float)(h & 0xffffu) / 32768.0f - 1.0f);
      b[v][i] = (__bf16)((float)(h >> 16) / 655360.0f - 0.05f);
    }
  floatx4_t acc[16];
  for (int i = 0; i < 16; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i & 1], b[(i >> 1) & 1], acc[i], 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) copy_kernel(const floatx4_t* __restrict__ src, floatx4_t* __restrict__ dst,
                                                   int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__global__ void __launch_bounds__(256) read_kernel(const floatx4_t* __restrict__ src, float* __restrict__ out,
                                                   int64_t n) {
  floatx4_t s = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    s += src[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

// R reads per write: dst[i] = src[i] + src[i + n] (+ src[i + 2n]), the read:write byte mix
// of the norms (R = 2: fp32 in, bf16 out) and of attention (R = 3: q, k, v in, output out)
template <int R>
__global__ void __launch_bounds__(256) mix_kernel(const floatx4_t* __restrict__ src, floatx4_t* __restrict__ dst,
                                                  int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    floatx4_t v = src[i];
#pragma unroll
    for (int r = 1; r < R; ++r) v += src[i + r * n];
    dst[i] = v;
  }
}

float time_ms(void (*launch)(void*), void* arg, int reps) {
  hipEvent_t a, b;
  hipEventCreate(&a);
  hipEventCreate(&b);
  launch(arg);                       // warm-up
  hipEventRecord(a, 0);
  for (int r = 0; r < reps; ++r) launch(arg);
  hipEventRecord(b, 0);
  hipEventSynchronize(b);
  float ms = 0.f;
  hipEventElapsedTime(&ms, a, b);
  hipEventDestroy(a);
  hipEventDestroy(b);
  return ms / reps;
}

struct Buf { void* src; void* dst; int64_t n16; int blocks; int iters; };

void launch_mfma(void* p) {
  Buf* b = (Buf*)p;
  hipLaunchKernelGGL(mfma_loop, dim3(b->blocks), dim3(256), 0, 0, (float*)b->dst, b->iters);
}
void launch_mfma_random(void* p) {
  Buf* b = (Buf*)p;
  hipLaunchKernelGGL(mfma_loop_random, dim3(b->blocks), dim3(256), 0, 0, (float*)b->dst, b->iters);
}
void launch_copy(void* p) {
  Buf* b = (Buf*)p;
  hipLaunchKernelGGL(copy_kernel, dim3(b->blocks), dim3(256), 0, 0, (const floatx4_t*)b->src, (floatx4_t*)b->dst,
                     b->n16);
}
void launch_mix2(void* p) {
  Buf* b = (Buf*)p;
  hipLaunchKernelGGL(mix_kernel<2>, dim3(b->blocks), dim3(256), 0, 0, (const floatx4_t*)b->src, (floatx4_t*)b->dst,
                     b->n16);
}
void launch_mix3(void* p) {
  Buf* b = (Buf*)p;
  hipLaunchKernelGGL(mix_kernel<3>, dim3(b->blocks), dim3(256), 0, 0, (const floatx4_t*)b->src, (floatx4_t*)b->dst,
                     b->n16);
}
void launch_read(void* p) {
  Buf* b = (Buf*)p;
  hipLaunchKernelGGL(read_kernel, dim3(b->blocks), dim3(256), 0, 0, (const floatx4_t*)b->src, (float*)b->dst,
                     b->n16);
}

}  // namespace

extern "C" {

// Dense bf16 MFMA rate in TFLOP/s; `scratch` holds blocks * 256 floats.
double zo_peak_mfma_bf16(void* scratch, int blocks, int iters) {
  Buf b = {nullptr, scratch, 0, blocks, iters};
  const float ms = time_ms(launch_mfma, &b, 3);
  const double flop = (double)blocks * 4 * iters * 16 * (2.0 * 16 * 16 * 32);
  return flop / (ms * 1e-3) / 1e12;
}

// The same on random operands (see mfma_loop_random).
double zo_peak_mfma_bf16_random(void* scratch, int blocks, int iters) {
  Buf b = {nullptr, scratch, 0, blocks, iters};
  const float ms = time_ms(launch_mfma_random, &b, 3);
  const double flop = (double)blocks * 4 * iters * 16 * (2.0 * 16 * 16 * 32);
  return flop / (ms * 1e-3) / 1e12;
}

// Streaming copy of `bytes` (multiple of 16) from src to dst: GB/s of bytes read + written.
double zo_peak_copy(const void* src, void* dst, int64_t bytes, int blocks) {
  Buf b = {(void*)src, dst, bytes / 16, blocks, 0};
  const float ms = time_ms(launch_copy, &b, 5);
  return 2.0 * (double)bytes / (ms * 1e-3) / 1e9;
}

// Streaming with `reads` (2 or 3) reads per write of `write_bytes` (multiple of 16): GB/s of
// bytes read + written; src holds reads * write_bytes.
double zo_peak_mix(const void* src, void* dst, int64_t write_bytes, int reads, int blocks) {
  if (reads != 2 && reads != 3) return 0.0;
  Buf b = {(void*)src, dst, write_bytes / 16, blocks, 0};
  const float ms = time_ms(reads == 2 ? launch_mix2 : launch_mix3, &b, 5);
  return (double)(reads + 1) * (double)write_bytes / (ms * 1e-3) / 1e9;
}

// Streaming read of `bytes`: GB/s; `out` holds blocks * 256 floats.
double zo_peak_read(const void* src, void* out, int64_t bytes, int blocks) {
  Buf b = {(void*)src, out, bytes / 16, blocks, 0};
  const float ms = time_ms(launch_read, &b, 5);
  return (double)bytes / (ms * 1e-3) / 1e9;
}

}  // extern "C"
