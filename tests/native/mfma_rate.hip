// Matrix-core throughput on register operands, as a function of the operand
// values: the rate the GPU's products reach under its power limit when
// nothing else runs.  A measurement aid for the benchmark (bench.py
// --mfma-ceiling), kept out of the attention library.
//
// 8 waves per CU (2 per SIMD), each looping over 16 v_mfma 32x32x16 products
// per iteration on 4 independent accumulator chains; the operands are loaded
// once from a device buffer filled with one of: N(0,1) samples rounded to the
// product's type, a constant (0.7), or zeros.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kBlocks = 1024;          // four per CU over the run
constexpr int kChunksPerThread = 8;    // 16-byte operand chunks: 4 for A, 4 for B

// 32-bit integer hash (an xorshift-multiply finaliser) of a counter
__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// bf16 bits of x, rounded to nearest even (finite x)
__device__ __forceinline__ uint16_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__global__ void fill_kernel(uint16_t* dst, int64_t n, int f16, int kind, uint32_t seed) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    float x = 0.f;
    if (kind == 0) {
      // Box-Muller on two hashed uniforms in (0, 1]
      const uint32_t h1 = hash32((uint32_t)(2 * i) ^ seed), h2 = hash32((uint32_t)(2 * i + 1) ^ (seed * 0x9e3779b9u));
      const float u1 = ((float)(h1 >> 8) + 1.0f) * (1.0f / 16777216.0f);
      const float u2 = (float)(h2 >> 8) * (1.0f / 16777216.0f);
      x = sqrtf(-2.0f * logf(u1)) * cosf(6.28318530718f * u2);
    } else if (kind == 1) {
      x = 0.7f;
    }
    if (f16) {
      const _Float16 h = (_Float16)x;
      dst[i] = __builtin_bit_cast(uint16_t, h);
    } else {
      dst[i] = bf16_bits(x);
    }
  }
}

template <bool F16>
__global__ __launch_bounds__(kThreads, 1) void rate_kernel(const u32x4* __restrict__ src, int iters, float* out) {
  const int64_t base = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kChunksPerThread;
  u32x4 a[4], b[4];
  for (int i = 0; i < 4; ++i) {
    a[i] = src[base + i];
    b[i] = src[base + 4 + i];
  }
  f32x16 c[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (F16)
          c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[(j + k) & 3]),
                                                        __builtin_bit_cast(f16x8, b[k]), c[j], 0, 0, 0);
        else
          c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[(j + k) & 3]),
                                                         __builtin_bit_cast(bf16x8, b[k]), c[j], 0, 0, 0);
      }
  }
  // keep the products: one sum per thread
  float r = 0.f;
  for (int j = 0; j < 4; ++j)
    for (int e = 0; e < 16; ++e) r += c[j][e];
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = r;
}

}  // namespace

// TFLOP/s of 32x32x16 products (f16 != 0: fp16 operands, else bf16) on
// operands of `kind` (0 N(0,1), 1 the constant 0.7, 2 zeros), best of three
// timed launches of `iters` iterations after one untimed launch, on the
// current device and the null stream.  Allocates and frees its own 66 MiB.
// Returns 0, or -3 on a HIP error.
extern "C" int ffa_probe_mfma_rate(int f16, int kind, int iters, double* tflops) {
  const int64_t n16 = (int64_t)kBlocks * kThreads * kChunksPerThread * 8;  // 16-bit operands
  uint16_t* buf = nullptr;
  float* out = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = 0;
  if (hipMalloc(&buf, n16 * 2) != hipSuccess || hipMalloc(&out, sizeof(float) * kBlocks * kThreads) != hipSuccess ||
      hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    rc = -3;
  } else {
    hipLaunchKernelGGL(fill_kernel, dim3(2048), dim3(256), 0, 0, buf, n16, f16, kind, 12345u);
    float best = 1e30f;
    for (int rep = 0; rep < 4 && rc == 0; ++rep) {
      (void)hipEventRecord(e0, 0);
      if (f16)
        hipLaunchKernelGGL(rate_kernel<true>, dim3(kBlocks), dim3(kThreads), 0, 0,
                           reinterpret_cast<const u32x4*>(buf), iters, out);
      else
        hipLaunchKernelGGL(rate_kernel<false>, dim3(kBlocks), dim3(kThreads), 0, 0,
                           reinterpret_cast<const u32x4*>(buf), iters, out);
      (void)hipEventRecord(e1, 0);
      if (hipEventSynchronize(e1) != hipSuccess) rc = -3;
      float ms = 0.f;
      if (rc == 0 && hipEventElapsedTime(&ms, e0, e1) != hipSuccess) rc = -3;
      if (rep > 0 && ms < best) best = ms;
    }
    if (rc == 0 && hipGetLastError() != hipSuccess) rc = -3;
    // products per launch: 16 per wave and iteration, 8 waves per block
    const double flop = 2.0 * 32 * 32 * 16 * 16.0 * iters * (double)kBlocks * (kThreads / 64);
    if (rc == 0) *tflops = flop / (best * 1e-3) / 1e12;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (buf) (void)hipFree(buf);
  if (out) (void)hipFree(out);
  return rc;
}
