// Device-side helpers shared by the gfx950 kernels: vector types for the
// bf16 MFMA operands, buffer resources, and the plan records the kernels read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
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

// The same product with fp16 operands (same rate, 11 significant bits
// instead of 8).  Operands are passed as raw 16-bit lanes.
__device__ __forceinline__ f32x16 mfma_32x32x16_f16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                0, 0, 0);
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

// Two fp32 values to fp16, round to nearest even, packed low | high << 16.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 p;
  p[0] = (_Float16)lo;
  p[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

// bf16 bits of x rounded to nearest even, and the bf16 bits of what that
// rounding left out (x - hi, rounded again): together 16 significant bits.
// x is the fp32 value as given: the subtraction is never fused with a
// product that formed x, so every kernel gets the same residual.
__device__ __forceinline__ void split_bf16(float x, uint16_t* hi, uint16_t* lo) {
#pragma clang fp contract(off)
  const __bf16 h = (__bf16)x;
  const float r = x - (float)h;
  *hi = __builtin_bit_cast(uint16_t, h);
  *lo = __builtin_bit_cast(uint16_t, (__bf16)r);
}

// Power of two s with max_abs * s in [2^(L-1), 2^L) (s = 1 for 0), from the
// fp32 bits of a non-negative finite max_abs: it maps a tensor's range onto
// fp16's (exact scaling; clamped to 2^-100 .. 2^100).
__device__ __forceinline__ float range_scale(uint32_t max_bits, int L) {
  if (max_bits == 0) return 1.0f;
  int e = (int)(max_bits >> 23);  // biased exponent; subnormals count as 2^-126
  if (e == 0) e = 1;
  // max < 2^(e - 126), so s = 2^(L - (e - 126)) gives max * s < 2^L
  int se = L - (e - 126);
  se = se < -100 ? -100 : (se > 100 ? 100 : se);
  return __uint_as_float((uint32_t)(se + 127) << 23);
}

// Scale of the fp16 copies of v and k: 1 when max |x| already lies in
// [2^-3, 2^L) (the copy at scale 1 is then exact for every value from 2^-17
// up, and what lies below rounds at 2^-25, under 2^-22 of max |x|), else
// range_scale.  The copy is made at scale 1 in the same pass that finds
// max |x| and redone only outside that window.
__device__ __forceinline__ float copy_scale(uint32_t max_bits, int L) {
  const uint32_t lo = (uint32_t)(127 - 3) << 23, hi = (uint32_t)(127 + L) << 23;
  return (max_bits >= lo && max_bits < hi) ? 1.0f : range_scale(max_bits, L);
}

// Range bounds L (largest |x| mapped into [2^(L-1), 2^L)) of the fp16
// operand copies: 15 for q and k, 4 for v (bounding it; copy_scale may leave
// it lower).  dO's bound is kRangeDOV - (v's): max |dO| max |v| after
// scaling lies in [2^5, 2^7) whatever v's scale, which keeps |dS| =
// P |dP - D| below 2^15 in the backward (|dP| <= d max|dO| max|v| <
// 128 * 2^7, and |D| <= max |dP| since D is a convex combination of a row's
// dP) and as far above fp16's subnormal range as that allows.  Word slots
// of the ranges in a range-word array.
constexpr int kRangeQ = 15, kRangeK = 15, kRangeV = 4, kRangeDOV = 7;
enum { kRgQ = 0, kRgK = 1, kRgV = 2, kRgDO = 3 };

// L with max_abs * s in [2^(L-1), 2^L), for the fp32 bits of a non-negative
// finite max_abs and a power of two s (L = kRangeV for 0).
__device__ __forceinline__ int range_top(uint32_t max_bits, float s) {
  if (max_bits == 0) return kRangeV;
  int e = (int)(max_bits >> 23);  // max in [2^(e-127), 2^(e-126)) for e > 0
  if (e == 0) e = 1;
  return e - 126 + (int)((__float_as_uint(s) >> 23) & 0xFF) - 127;
}

// 8 bf16 values times s (a power of two) to fp16, round to nearest even.
__device__ __forceinline__ u32x4 to_f16x8(u32x4 w, float s) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r[j] = pack_f16x2(__uint_as_float(w[j] << 16) * s, __uint_as_float(w[j] & 0xFFFF0000u) * s);
  return r;
}

// ---------------------------------------------------------------- LDS tiles
// A 64-row x D tile in LDS, fetched by direct-to-LDS loads.  One load
// instruction fills 64 consecutive 16-byte slots (lane L -> slot L); the
// slots of instruction i start at byte 1088 * i (1024 + 64 bytes padding).
//   D = 128: instruction i holds rows 4i .. 4i + 3, slot L = row 4i + L % 4,
//            chunk L / 4, so one instruction reads 4 whole rows from HBM;
//   D = 64:  instruction i holds chunk i of all 64 rows (slot L = row L).
// Either way the byte offset of (row, chunk) is linear in row and chunk as
// long as the row offsets added are multiples of 4 (D = 128) -- see off() --
// so every read address is a per-lane base plus a compile-time immediate.
// Row operands (16 lanes, 16 consecutive rows, one chunk) and transposed
// operands (4 rows x 4 chunks per 32 lanes) both land on 16 distinct
// 16-byte bank groups: no LDS bank conflicts on the 64 banks.
template <int D>
struct ColTile {
  static constexpr int kChunks = D / 8;
  static constexpr int kRG = (D == 128) ? 4 : 64;       // rows per instruction group
  static constexpr int kCS = (D == 128) ? 64 : 1088;    // bytes between chunks
  static constexpr int kGS = 1088;                      // bytes between row groups
  static constexpr int kBytes = kChunks * 1088;
  static_assert(D == 64 || D == 128, "head dim");

  __device__ __forceinline__ static constexpr int off(int row, int chunk) {
    return (row / kRG) * kGS + chunk * kCS + (row % kRG) * 16;
  }

  // Fetch rows [0, 64) of a tile whose row r starts at byte r * row_bytes
  // of resource `r` (rows past the resource read as zeros), shared by NW
  // waves: wave w issues instructions w * kChunks / NW .. +kChunks / NW.
  template <int NW = 4>
  __device__ __forceinline__ static void load(__amdgpu_buffer_rsrc_t r, uint32_t row_bytes, char* dst,
                                              int w, int lane) {
    constexpr int kPer = kChunks / NW;
    static_assert(kPer * NW == kChunks, "waves must split the tile evenly");
    uint32_t lane_off, step;
    if constexpr (D == 128) {
      lane_off = (uint32_t)(lane & 3) * row_bytes + (uint32_t)(lane >> 2) * 16;
      step = 4 * row_bytes;
    } else {
      lane_off = (uint32_t)lane * row_bytes;
      step = 16;
    }
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int i = w * kPer + c;  // wave-uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(dst + i * 1088), 16, lane_off + (uint32_t)i * step, 0, 0, 0);
    }
  }
  // Row operand: 8 elements (16 bytes) of row r0 + n, chunk c0 + hh, with
  // lane_row = off(n, hh) and r0 a multiple of 32, c0 even.
  __device__ __forceinline__ static bf16x8 row8(const char* t, int lane_row, int r0, int c0) {
    return *reinterpret_cast<const bf16x8*>(t + lane_row + off(r0, c0));
  }
};

// Byte offset of this lane's transpose-read source inside a ColTile: the
// 16-lane group g16 / index sl of lane `lane` points at row 4*hh + sl/4 and
// 4 dims at 16*(g16 & 1) + 4*(sl & 3).  Adding the block offsets below
// gives, in each lane, 4 consecutive rows (of the 8 the MFMA k index needs)
// of one dim: the order of a 32x32 accumulator's rows, so the accumulator's
// registers can be the other operand directly.
template <int D>
__device__ __forceinline__ int tr_lane_offset(int lane) {
  const int hh = lane >> 5, g16 = lane >> 4, sl = lane & 15;
  const int col = 16 * (g16 & 1) + 4 * (sl & 3);
  return ColTile<D>::off(4 * hh + (sl >> 2), col >> 3) + (col & 7) * 2;
}

// A operand of C[dims x 32] += T^T[dims 32db.. x rows] X[rows x 32]: the
// transposed tile T, rows 32*(t >> 1) + 16*(t & 1) + {0..3, 8..11} + 4*hh.
template <int D>
__device__ __forceinline__ bf16x8 tr8(const char* t, int lane_off, int db, int t4) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const int r0 = 32 * (t4 >> 1) + 16 * (t4 & 1);
  const char* p = t + lane_off + ColTile<D>::off(r0, 4 * db);
  const char* p8 = t + lane_off + ColTile<D>::off(r0 + 8, 4 * db);
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(const_cast<char*>(p)));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(const_cast<char*>(p8)));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  u32x4 x;
  x[0] = l2[0]; x[1] = l2[1]; x[2] = h2[0]; x[3] = h2[1];
  return __builtin_bit_cast(bf16x8, x);
}

// LDS address of tile `t` plus a per-lane offset, as a value the compiler
// cannot see through.  A read of such a base plus a compile-time offset then
// takes the offset as the instruction's immediate, also for tiles that sit
// above the 64 KiB an immediate reaches from address 0; otherwise the
// compiler keeps a separate address register per read of those tiles.
__device__ __forceinline__ const char* lane_base(const char* t, int lane_off) {
  const uint32_t t32 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)t;
  uint32_t a = t32 + (uint32_t)lane_off;
  asm volatile("" : "+v"(a));
  // still an offset from t, so the compiler knows which buffer is read
  return t + (int)(a - t32);
}

// Wait for this wave's direct-to-LDS loads, then for the whole workgroup.
__device__ __forceinline__ void dma_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

}  // namespace ffa
