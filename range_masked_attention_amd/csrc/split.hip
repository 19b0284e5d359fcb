// Work-list split shared by the kernels that walk one tile's plan list per
// workgroup (forward: per q tile; dK/dV: per key tile).
//
// Such a list is one serial chain, so a tile whose list is far longer than
// the average (a global "sink" that every q block attends, a short query
// block against a long context) sets the kernel's duration by itself.  The
// split kernel cuts every list longer than `ec` entries into runs of at most
// ec entries, with ec chosen so that the runs of all tiles, times the
// workgroups that walk each tile (`units`: q heads or kv heads), number
// about `balance`.  No run is then longer than (units * work) / balance,
// which for balance = twice the resident workgroup slots is half of one
// slot's share.  Runs never go below `min_steps` steps (an entry costs
// `steps_per_entry` steps).  Runs of a split tile write partial results that
// a second pass combines in run order, so results do not depend on timing.
//
// Output, in the plan's tile order (runs of one tile consecutive):
//   items[i]  = {tile, first entry, end entry, partial slot or -1}
//   splits[s] = {tile, first slot, runs, 0} for each tile cut into >= 2 runs
//   counts    = {items, splits}
// With E the entries of all tiles, items <= n_tiles + E / ec and splits <
// E / ec, so both are bounded by split_caps(); partial slots times units
// stay <= max_slot_units (ec doubles until they fit).  The kernel runs in one
// workgroup on the device, so it works on plans built on the device and
// under graph capture.
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace ffa {

namespace {

constexpr int kSplitThreads = 1024;

// Inclusive prefix sums of three values over the 1024 threads.
__device__ __forceinline__ void block_scan3(int v[3], int (*s_wave)[16]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1)
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int y = __shfl_up(v[j], d, 64);
      if (lane >= d) v[j] += y;
    }
  if (lane == 63)
    for (int j = 0; j < 3; ++j) s_wave[j][w] = v[j];
  __syncthreads();
  for (int j = 0; j < 3; ++j) {
    int off = 0;
    for (int i = 0; i < w; ++i) off += s_wave[j][i];
    v[j] += off;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kSplitThreads) void split_kernel(const int32_t* __restrict__ row_ptr,
                                                              const int32_t* __restrict__ order, int n_tiles,
                                                              int steps_per_entry, int units, int min_steps,
                                                              int balance, int max_slot_units, i32x4* items,
                                                              int items_cap, i32x4* splits, int splits_cap,
                                                              int32_t* counts) {
  __shared__ int s_wave[3][16];
  __shared__ int s_tot[3];
  __shared__ long long s_slots;
  const int tid = threadIdx.x;
  const long long E = (long long)row_ptr[n_tiles] - row_ptr[0];
  long long ec = max((long long)((min_steps + steps_per_entry - 1) / steps_per_entry),
                     (E * units + balance - 1) / balance);
  if (ec < 1) ec = 1;
  // runs of split tiles (one partial buffer each per unit) for this ec
  for (;;) {
    if (tid == 0) s_slots = 0;
    __syncthreads();
    long long part = 0;
    for (int u = tid; u < n_tiles; u += kSplitThreads) {
      const int t = order[u];
      const long long len = (long long)row_ptr[t + 1] - row_ptr[t];
      if (len > ec) part += (len + ec - 1) / ec;
    }
    if (part) atomicAdd(reinterpret_cast<unsigned long long*>(&s_slots), (unsigned long long)part);
    __syncthreads();
    const long long slots = s_slots;
    __syncthreads();
    if (slots * units <= max_slot_units) break;
    ec *= 2;
  }

  int base_item = 0, base_slot = 0, base_split = 0;
  for (int u0 = 0; u0 < n_tiles; u0 += kSplitThreads) {
    const int u = u0 + tid;
    int t = 0, lo = 0, len = 0, ns = 0;
    if (u < n_tiles) {
      t = order[u];
      lo = row_ptr[t];
      len = row_ptr[t + 1] - lo;
      ns = len > ec ? (int)((len + ec - 1) / ec) : 1;
    }
    const bool sp = ns > 1;
    int v[3] = {ns, sp ? ns : 0, sp ? 1 : 0};
    block_scan3(v, s_wave);
    if (u < n_tiles) {
      const int item0 = base_item + v[0] - ns;
      const int slot0 = base_slot + v[1] - (sp ? ns : 0);
      const int ce = (len + ns - 1) / ns;
      for (int c = 0; c < ns; ++c) {
        const int e_lo = lo + min(len, c * ce), e_hi = lo + min(len, (c + 1) * ce);
        if (item0 + c < items_cap) items[item0 + c] = i32x4{t, e_lo, e_hi, sp ? slot0 + c : -1};
      }
      const int si = base_split + v[2] - 1;
      if (sp && si < splits_cap) splits[si] = i32x4{t, slot0, ns, 0};
    }
    if (tid == kSplitThreads - 1)
      for (int j = 0; j < 3; ++j) s_tot[j] = v[j];
    __syncthreads();
    base_item += s_tot[0];
    base_slot += s_tot[1];
    base_split += s_tot[2];
    __syncthreads();
  }
  if (tid == 0) {
    counts[0] = min(base_item, items_cap);
    counts[1] = min(base_split, splits_cap);
  }
}

}  // namespace

SplitCaps split_caps(int64_t n_tiles, int units, int balance) {
  SplitCaps c;
  const int64_t per_unit = units > 0 ? balance / units : balance;
  c.items = n_tiles + per_unit;
  c.splits = per_unit > 0 ? per_unit : 1;
  return c;
}

bool split_possible(int64_t n_entries, int64_t max_len, int steps_per_entry, int units, int min_steps,
                    int balance) {
  if (n_entries < 0 || max_len < 0) return true;
  // the kernel's first run length; it only grows from there
  int64_t ec = std::max<int64_t>((min_steps + steps_per_entry - 1) / steps_per_entry,
                                 (n_entries * units + balance - 1) / balance);
  if (ec < 1) ec = 1;
  return max_len > ec;
}

void launch_split(const SplitLaunch& s, hipStream_t stream) {
  hipLaunchKernelGGL(split_kernel, dim3(1), dim3(kSplitThreads), 0, stream, s.row_ptr, s.order, (int)s.n_tiles,
                     s.steps_per_entry, s.units, s.min_steps, s.balance, s.max_slot_units,
                     static_cast<i32x4*>(s.items), (int)s.items_cap, static_cast<i32x4*>(s.splits),
                     (int)s.splits_cap, s.counts);
}

}  // namespace ffa
