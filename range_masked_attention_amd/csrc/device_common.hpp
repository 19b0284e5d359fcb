// Device-side helpers shared by the gfx950 kernels: vector types for the
// bf16 MFMA operands, buffer resources, and the plan records the kernels read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A slice as the kernels see it: rows [qs, qe), keys [ks, ke), causal flag.
// 32 bytes so a record is one aligned scalar load.
struct DevSlice {
  int32_t qs, qe, ks, ke, causal, pad0, pad1, pad2;
};

// One plan entry: the other axis' tile and (slice << 1 | partial).
struct DevEntry {
  int32_t tile;
  int32_t meta;
};

// D = A(32x16) * B(16x32) + C on the matrix cores, bf16 in, fp32 accumulate.
// Lane l holds A row (l % 32) and B column (l % 32), eight k values each
// (which eight is the instruction's business: A and B agree).  C/D: lane l
// holds column (l % 32), rows 8 * (v / 4) + 4 * (l / 32) + (v % 4), v = 0..15.
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Buffer resource over [base, base + bytes): loads past the end return 0,
// stores past the end are dropped.  bytes is clamped to [0, 2^32 - 1].
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  if (bytes > 0xFFFFFFFFll) bytes = 0xFFFFFFFFll;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(uint32_t)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  i32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return __builtin_bit_cast(u32x4, x);
}

// The plan (offsets, entries, slices, order) stays unchanged while a kernel
// runs.  Reading it through the constant address space lets the compiler use
// scalar loads for wave-uniform indices: those count on lgkmcnt, so waiting
// for an entry never also waits for the tile fetches in flight on vmcnt.
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
template <typename V>
__device__ __forceinline__ V const_load(const void* p, int64_t i) {
  return ((const __attribute__((address_space(4))) V*)(p))[i];
}
__device__ __forceinline__ int32_t plan_i32(const int32_t* p, int64_t i) { return const_load<int32_t>(p, i); }
__device__ __forceinline__ DevEntry plan_entry(const DevEntry* p, int64_t i) {
  return __builtin_bit_cast(DevEntry, const_load<u32x2>(p, i));
}
__device__ __forceinline__ DevSlice plan_slice(const DevSlice* p, int64_t i) {
  return __builtin_bit_cast(DevSlice, const_load<i32x8>(p, i));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// tanh(x) for x given as y = 2 * x * log2(e): 1 - 2 / (2^y + 1).
// Saturates cleanly: 2^y -> inf gives 1, 2^y -> 0 gives -1.
__device__ __forceinline__ float tanh_from_2xlog2e(float y) {
  return 1.0f - 2.0f * fast_rcp(fast_exp2(y) + 1.0f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

}  // namespace ffa
