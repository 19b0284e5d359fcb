// fp16 operand copies for the products that need more than bf16's 8
// significant bits (the forward's P V, every backward product).
//
// A tensor is copied to fp16 times s = 2^e, the power of two that maps its
// largest |x| into [2^(L-1), 2^L) (range_scale): exact, since a bf16 value
// has 8 significant bits and fp16 keeps 11, for every value down to 2^-14 of
// 2^L; below that fp16 rounds at 2^-25 of 2^L.  The largest |x| comes from a
// grid-stride pass (one atomic per workgroup and tensor) before the copy.
// The copies of v (forward) and k (backward) instead take scale 1 whenever
// their range allows (copy_scale), are made in the pass that finds the range
// (partial maxima per workgroup, no atomics), and are redone only when it
// does not.
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace ffa {

namespace {

constexpr int kThreads = 256;

// The largest bf16 magnitude bits among 8 values (finite values order like
// their bit patterns).
__device__ __forceinline__ uint32_t max_mag16(u32x4 w) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
  return m;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t m) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  return m;
}

__global__ void range_clear_kernel(uint32_t* words, int n) {
  if ((int)threadIdx.x < n) words[threadIdx.x] = 0u;
}

// words[t.word] = fp32 bits of max |x| over tensor t, for each of n tensors:
// four loads in flight per thread, a workgroup-wide maximum in LDS, then one
// atomic per workgroup and tensor (one per wave made the atomics on a single
// word the slowest part).
__global__ __launch_bounds__(kThreads) void range_max_kernel(RangeJob job) {
  __shared__ uint32_t wmax[kThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int t = 0; t < job.n; ++t) {
    const u32x4* src = static_cast<const u32x4*>(job.src[t]);
    const int64_t n = job.chunks[t];
    uint32_t m = 0;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
      const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
      m = max(max(m, max(max_mag16(a), max_mag16(b))), max(max_mag16(c), max_mag16(d)));
    }
    for (; i < n; i += stride) m = max(m, max_mag16(src[i]));
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t b = 0;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) b = max(b, wmax[w]);
      if (b) atomicMax(&job.words[job.word[t]], b << 16);
    }
    __syncthreads();
  }
}

// The largest of m over a workgroup's threads, in every thread.
__device__ __forceinline__ uint32_t block_max(uint32_t m) {
  __shared__ uint32_t wmax[kThreads / 64];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t b = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) b = max(b, wmax[w]);
  return b;
}

// Tracked copy (v's in the forward, k's in the backward), first pass: dst =
// fp16(src) at scale 1, two chunks in flight per thread, and
// parts[workgroup] = fp32 bits of the largest |src| it saw.
__global__ __launch_bounds__(kThreads) void convert_track_kernel(const u32x4* __restrict__ src,
                                                                u32x4* __restrict__ dst, int64_t n,
                                                                uint32_t* __restrict__ parts) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t m = 0;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + stride < n; i += 2 * stride) {
    const u32x4 a = src[i], b = src[i + stride];
    m = max(m, max(max_mag16(a), max_mag16(b)));
    dst[i] = to_f16x8(a, 1.0f);
    dst[i + stride] = to_f16x8(b, 1.0f);
  }
  if (i < n) {
    const u32x4 a = src[i];
    m = max(m, max_mag16(a));
    dst[i] = to_f16x8(a, 1.0f);
  }
  m = block_max(m);
  if (threadIdx.x == 0) parts[blockIdx.x] = m << 16;
}

// Second pass: max |src| from the first pass's n_parts partial maxima
// (every workgroup reduces them; workgroup 0 writes words[word], and with
// clear_others sets words[0..3] but that one to 0), then the copy redone at
// copy_scale where that is not 1 (a range outside [2^-3, 2^L)); otherwise
// every workgroup returns there.
__global__ __launch_bounds__(kThreads) void convert_fix_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                              int64_t n, const uint32_t* __restrict__ parts,
                                                              int n_parts, uint32_t* __restrict__ words, int word,
                                                              int L, int clear_others) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n_parts; i += kThreads) m = max(m, parts[i]);
  m = block_max(m);
  if (blockIdx.x == 0 && threadIdx.x < 4 && (clear_others || (int)threadIdx.x == word))
    words[threadIdx.x] = (int)threadIdx.x == word ? m : 0u;
  const float s = copy_scale(m, L);
  if (s == 1.0f) return;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) dst[i] = to_f16x8(src[i], s);
}

int64_t grid_for(int64_t n, int64_t cap) {
  const int64_t b = (n + kThreads - 1) / kThreads;
  return b < 1 ? 1 : (b > cap ? cap : b);
}

}  // namespace

void launch_range_clear(uint32_t* words, int n, hipStream_t stream) {
  hipLaunchKernelGGL(range_clear_kernel, dim3(1), dim3(64), 0, stream, words, n);
}

void launch_range_max(const RangeJob& job, hipStream_t stream) {
  int64_t most = 0;
  for (int t = 0; t < job.n; ++t) most = job.chunks[t] > most ? job.chunks[t] : most;
  if (most == 0) return;
  // about 8 chunks per thread of the largest tensor, at most 1024 workgroups
  hipLaunchKernelGGL(range_max_kernel, dim3((unsigned)grid_for((most + 7) / 8, 1024)), dim3(kThreads), 0, stream,
                     job);
}

void launch_convert_tracked(const void* src, void* dst, int64_t chunks, uint32_t* parts, uint32_t* words, int word,
                            int L, bool clear_others, hipStream_t stream) {
  // two chunks per thread and step: about 4 steps per thread at the largest
  // sizes, and at least a few workgroups per CU on small tensors; the
  // second pass, which copies again only for a range outside its window,
  // takes one workgroup per CU
  const unsigned g = (unsigned)grid_for((chunks + 1) / 2, kVRangeParts);
  if (chunks > 0)
    hipLaunchKernelGGL(convert_track_kernel, dim3(g), dim3(kThreads), 0, stream, static_cast<const u32x4*>(src),
                       static_cast<u32x4*>(dst), chunks, parts);
  hipLaunchKernelGGL(convert_fix_kernel, dim3(chunks > 0 ? std::min(g, 256u) : 1u), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), chunks,
                     static_cast<const uint32_t*>(parts), chunks > 0 ? (int)g : 0, words, word, L,
                     clear_others ? 1 : 0);
}

SavedLayout saved_layout(int64_t Tq, int64_t Tk, int hq, int hkv, int d) {
  auto r256 = [](size_t x) { return (x + 255) & ~size_t(255); };
  SavedLayout L{};
  const size_t nq = (size_t)(Tq > 0 ? Tq : 0) * (size_t)(hq > 0 ? hq : 0) * (size_t)(d > 0 ? d : 0);
  const size_t nk = (size_t)(Tk > 0 ? Tk : 0) * (size_t)(hkv > 0 ? hkv : 0) * (size_t)(d > 0 ? d : 0);
  size_t off = 0;
  L.words = off;
  off += 256;
  L.out_lo = off;
  off += r256(nq * 2);
  L.v16 = off;
  off += r256(nk * 2);
  L.parts = off;
  off += r256((size_t)kVRangeParts * 4);
  L.total = off;
  return L;
}

}  // namespace ffa
