// Device-side planner: the block-sparse plan of the host planner, built by
// kernels from slice arrays that already sit in device memory.
//
// The plan is the BlockMask of the FlexAttention paper summary, section 4
// (per tile of rows, the non-masked column tiles, FULL ones needing no mask),
// built from the slice list of flex_flash_attn_func.  In the MagiAttention
// issue on dummy/padded slices the ranges are device tensors padded with
// empty [x, x] slices for torch.compile; planning on the device avoids the
// host copy (a synchronisation) and makes the planned call capturable in a
// HIP graph: re-running these kernels on new range contents rebuilds the plan.
//
// The result equals the host planner's entry for entry, and the same tile
// order:
//  * a slice meets a tile in one contiguous interval of other-axis tiles, so
//    the entries of a tile sorted by (other tile, slice bounds) can be
//    placed directly: the position of (o, r) is the number of entries of
//    the tile with a smaller other tile plus the number of slices ordered
//    before r whose interval holds o;
//  * tiles are ordered by (longest list of the tile's group, the group's
//    slice start row, own length, index), a rank computed by counting.
// No sort, no atomics in the ordering: the plan is the same on every run.
// Status (invalid slice, capacity exceeded) goes to a device word; the plan
// is then left empty, so the attention kernels write zeros and -inf lse.
#include <climits>

#include "device_common.hpp"
#include "launch.hpp"

namespace ffa {

namespace {

constexpr int kBlock = 256;

struct PlanSlice {  // a slice as the planner reads it
  int64_t qs, qe, ks, ke;
  bool causal, live;
};

__device__ __forceinline__ PlanSlice read_slice(const DevSlice* s, int r) {
  const DevSlice v = s[r];
  PlanSlice p;
  p.qs = v.qs; p.qe = v.qe; p.ks = v.ks; p.ke = v.ke;
  p.causal = v.causal != 0;
  p.live = v.pad0 != 0;
  return p;
}

// Key tiles reached by row tile qt of slice s (rows of bm, keys of bn):
// [kt0, kt1], or false if none.  Same arithmetic as the host planner.
__device__ __forceinline__ bool row_tile_keys(const PlanSlice& s, int64_t qt, int bm, int bn, int64_t* kt0,
                                              int64_t* kt1) {
  if (qt < s.qs / bm || qt > (s.qe - 1) / bm) return false;
  const int64_t r0 = qt * bm, r1 = r0 + bm;
  int64_t a = max(r0, s.qs);
  const int64_t b = min(r1, s.qe);
  int64_t col_end = s.ke;
  if (s.causal) {
    const int64_t diag = s.ke - s.qe;  // row i sees keys j <= i + diag
    a = max(a, s.ks - diag);
    col_end = min(s.ke, b + diag);
  }
  if (a >= b || col_end <= s.ks) return false;
  *kt0 = s.ks / bn;
  *kt1 = (col_end - 1) / bn;
  return true;
}

// FULL (0) or PARTIAL (1) for the cells of tile (qt, kt) under slice s.
__device__ __forceinline__ int32_t tile_kind(const PlanSlice& s, int64_t qt, int64_t kt, int bm, int bn) {
  const int64_t r0 = qt * bm, r1 = r0 + bm, c0 = kt * bn, c1 = c0 + bn;
  bool full = r0 >= s.qs && r1 <= s.qe && c0 >= s.ks && c1 <= s.ke;
  if (full && s.causal) full = (c1 - 1) <= (r0 + (s.ke - s.qe));
  return full ? 0 : 1;
}

// The other-axis tiles of slice s in tile t: [lo, lo + len).  For the
// key-side list (transpose) t is a key tile and the other tiles are row
// tiles: those that reach key tile t form a suffix of the slice's row tiles
// (the rows that see any key are a suffix, and the last key tile a row tile
// reaches does not decrease along the rows), found by binary search.
__device__ __forceinline__ void tile_interval(const PlanSlice& s, int64_t t, int bm, int bn, bool transpose,
                                              int64_t* lo, int64_t* len) {
  *lo = 0;
  *len = 0;
  if (!s.live) return;
  int64_t kt0, kt1;
  if (!transpose) {
    if (row_tile_keys(s, t, bm, bn, &kt0, &kt1)) {
      *lo = kt0;
      *len = kt1 - kt0 + 1;
    }
    return;
  }
  const int64_t q_first = s.qs / bm, q_last = (s.qe - 1) / bm;
  if (t < s.ks / bn || !row_tile_keys(s, q_last, bm, bn, &kt0, &kt1) || kt1 < t) return;
  // first row tile that reaches key tile t (the predicate holds on a suffix)
  int64_t lo_q = q_first, hi_q = q_last;
  while (lo_q < hi_q) {
    const int64_t mid = lo_q + (hi_q - lo_q) / 2;
    if (row_tile_keys(s, mid, bm, bn, &kt0, &kt1) && kt1 >= t) hi_q = mid;
    else lo_q = mid + 1;
  }
  *lo = lo_q;
  *len = q_last - lo_q + 1;
}

// ---------------------------------------------------------------- kernels
__global__ void reset_kernel(int32_t* status) { *status = 0; }

// Validate and copy the slices; invalid ones set the status and are dropped.
__global__ __launch_bounds__(kBlock) void slices_kernel(const int32_t* qr, const int32_t* kr, const int32_t* ty,
                                                        int R, int64_t Tq, int64_t Tk, DevSlice* out,
                                                        int32_t* status) {
  const int r = blockIdx.x * kBlock + threadIdx.x;
  if (r >= R) return;
  const int32_t qs = qr[2 * r], qe = qr[2 * r + 1], ks = kr[2 * r], ke = kr[2 * r + 1], t = ty[r];
  const bool valid = qs >= 0 && qs <= qe && qe <= Tq && ks >= 0 && ks <= ke && ke <= Tk && (t == 0 || t == 1);
  if (!valid) atomicOr(status, kPlanBadSlice);
  DevSlice s;
  s.qs = qs; s.qe = qe; s.ks = ks; s.ke = ke;
  s.causal = (t == 1) ? 1 : 0;
  s.pad0 = (valid && qs < qe && ks < ke) ? 1 : 0;  // live: takes part in the plan
  s.pad1 = 0;
  s.pad2 = 0;
  out[r] = s;
}

// Rank of each live slice in the order (qs, qe, ks, ke, type, index).
__global__ __launch_bounds__(kBlock) void rank_kernel(const DevSlice* sl, int R, int32_t* rank) {
  const int r = blockIdx.x * kBlock + threadIdx.x;
  if (r >= R) return;
  const DevSlice a = sl[r];
  if (!a.pad0) {
    rank[r] = -1;
    return;
  }
  int n = 0;
  for (int i = 0; i < R; ++i) {
    const DevSlice b = sl[i];
    if (!b.pad0) continue;
    bool less;
    if (b.qs != a.qs) less = b.qs < a.qs;
    else if (b.qe != a.qe) less = b.qe < a.qe;
    else if (b.ks != a.ks) less = b.ks < a.ks;
    else if (b.ke != a.ke) less = b.ke < a.ke;
    else if (b.causal != a.causal) less = b.causal < a.causal;
    else less = i < r;
    n += less;
  }
  rank[r] = n;
}

struct PartArgs {
  const DevSlice* slices;
  const int32_t* rank;
  int32_t* status;
  int R;
  int64_t n_tiles;
  int bm, bn;
  bool transpose;
  int64_t cap;       // entry capacity
  int32_t* count;    // [n_tiles]
  int32_t* key;      // [n_tiles] smallest slice start row in the list (INT_MAX if empty)
  int32_t* glen;     // [n_tiles] longest list among tiles with the same key
  int32_t* row_ptr;  // [n_tiles + 1]
  DevEntry* entries; // [cap]
  int32_t* order;    // [n_tiles]
};

// Per tile: number of entries and the group key.
__global__ __launch_bounds__(kBlock) void count_kernel(PartArgs a) {
  const int64_t t = blockIdx.x;
  __shared__ int64_t s_sum[kBlock];
  __shared__ int32_t s_min[kBlock];
  int64_t sum = 0;
  int32_t mn = INT_MAX;
  for (int r = threadIdx.x; r < a.R; r += kBlock) {
    const PlanSlice s = read_slice(a.slices, r);
    int64_t lo, len;
    tile_interval(s, t, a.bm, a.bn, a.transpose, &lo, &len);
    if (len > 0) {
      sum += len;
      mn = min(mn, (int32_t)s.qs);
    }
  }
  s_sum[threadIdx.x] = sum;
  s_min[threadIdx.x] = mn;
  __syncthreads();
  for (int w = kBlock / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      s_sum[threadIdx.x] += s_sum[threadIdx.x + w];
      s_min[threadIdx.x] = min(s_min[threadIdx.x], s_min[threadIdx.x + w]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    // a tile list longer than 2^30 entries cannot be stored: count it as overflow
    a.count[t] = (int32_t)min<int64_t>(s_sum[0], int64_t(1) << 30);
    a.key[t] = s_min[0];
  }
}

// row_ptr = exclusive scan of count (one workgroup).  With a bad slice or a
// total above the capacity the plan is left empty and the status says why.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void scan_kernel(PartArgs a) {
  __shared__ int64_t s[kScanThreads];
  const int tid = threadIdx.x;
  const int64_t per = (a.n_tiles + kScanThreads - 1) / kScanThreads;
  const int64_t b = min<int64_t>(a.n_tiles, tid * per), e = min<int64_t>(a.n_tiles, b + per);
  int64_t local = 0;
  for (int64_t i = b; i < e; ++i) local += a.count[i];
  s[tid] = local;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {  // inclusive Hillis-Steele scan
    const int64_t v = tid >= off ? s[tid - off] : 0;
    __syncthreads();
    s[tid] += v;
    __syncthreads();
  }
  const int64_t total = s[kScanThreads - 1];
  const bool too_many = total > a.cap || total >= (int64_t(1) << 30);
  if (tid == 0 && too_many) atomicOr(a.status, kPlanCapacity);
  __syncthreads();
  const bool empty = too_many || (__atomic_load_n(a.status, __ATOMIC_RELAXED) & kPlanBadSlice);
  int64_t run = s[tid] - local;
  for (int64_t i = b; i < e; ++i) {
    a.row_ptr[i] = empty ? 0 : (int32_t)run;
    run += a.count[i];
  }
  if (tid == kScanThreads - 1) a.row_ptr[a.n_tiles] = empty ? 0 : (int32_t)total;
}

// Entries of one tile, each written at its place in the canonical order.
constexpr int kMaxPlanSlices = 4096;
__global__ __launch_bounds__(kBlock) void fill_kernel(PartArgs a) {
  const int64_t t = blockIdx.x;
  const int32_t base = a.row_ptr[t], n = a.row_ptr[t + 1] - base;
  if (n <= 0) return;
  __shared__ int32_t s_lo[kMaxPlanSlices], s_len[kMaxPlanSlices], s_rank[kMaxPlanSlices];
  __shared__ int32_t s_cum[kMaxPlanSlices + 1];
  __shared__ int32_t s_part[kBlock];
  for (int r = threadIdx.x; r < a.R; r += kBlock) {
    const PlanSlice s = read_slice(a.slices, r);
    int64_t lo, len;
    tile_interval(s, t, a.bm, a.bn, a.transpose, &lo, &len);
    s_lo[r] = (int32_t)lo;
    s_len[r] = (int32_t)len;
    s_rank[r] = a.rank[r];
  }
  __syncthreads();
  // s_cum = exclusive scan of s_len over the slices (chunk per thread)
  const int per = (a.R + kBlock - 1) / kBlock;
  const int rb = min(a.R, (int)threadIdx.x * per), re = min(a.R, rb + per);
  int32_t local = 0;
  for (int r = rb; r < re; ++r) local += s_len[r];
  s_part[threadIdx.x] = local;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t run = 0;
    for (int i = 0; i < kBlock; ++i) {
      const int32_t v = s_part[i];
      s_part[i] = run;
      run += v;
    }
  }
  __syncthreads();
  int32_t run = s_part[threadIdx.x];
  for (int r = rb; r < re; ++r) {
    s_cum[r] = run;
    run += s_len[r];
  }
  if (threadIdx.x == 0) s_cum[a.R] = n;
  __syncthreads();
  for (int32_t j = threadIdx.x; j < n; j += kBlock) {
    // slice r whose run of entries holds j: last r with s_cum[r] <= j and s_len[r] > 0
    int lo_r = 0, hi_r = a.R - 1;
    while (lo_r < hi_r) {
      const int mid = (lo_r + hi_r + 1) / 2;
      if (s_cum[mid] <= j) lo_r = mid;
      else hi_r = mid - 1;
    }
    // the last slice whose run starts at or before j is the owner: a slice
    // with no entries shares its start with the next slice, so it is never last
    const int r = lo_r;
    const int32_t o = s_lo[r] + (j - s_cum[r]);
    const int32_t rk = s_rank[r];
    int32_t pos = 0;
    for (int i = 0; i < a.R; ++i) {
      const int32_t l = s_lo[i], c = s_len[i];
      if (c == 0) continue;
      pos += min(max(o - l, 0), c);                     // entries of slice i with a smaller other tile
      pos += (s_rank[i] < rk && o >= l && o < l + c);   // slice i before r on the same other tile
    }
    const PlanSlice s = read_slice(a.slices, r);
    const int64_t qt = a.transpose ? o : t, kt = a.transpose ? t : o;
    // the row tiles here are bm rows and the key tiles bn keys in both lists
    DevEntry en;
    en.tile = o;
    en.meta = (r << 1) | tile_kind(s, qt, kt, a.bm, a.bn);
    a.entries[base + pos] = en;
  }
}

// The all-pairs passes below stream the per-tile arrays through LDS in
// chunks; every thread of a block then reads the same element (a broadcast).
constexpr int kChunk = 1024;

// Longest list in each tile's group (tiles with the same key).
__global__ __launch_bounds__(kBlock) void group_kernel(PartArgs a) {
  __shared__ int32_t c_key[kChunk], c_len[kChunk];
  const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const bool mine = t < a.n_tiles;
  const int32_t k = mine ? a.key[t] : 0;
  int32_t m = 0;
  for (int64_t base = 0; base < a.n_tiles; base += kChunk) {
    const int cnt = (int)min<int64_t>(kChunk, a.n_tiles - base);
    __syncthreads();
    for (int i = threadIdx.x; i < cnt; i += kBlock) {
      c_key[i] = a.key[base + i];
      c_len[i] = a.row_ptr[base + i + 1] - a.row_ptr[base + i];
    }
    __syncthreads();
    if (mine)
      for (int i = 0; i < cnt; ++i)
        if (c_key[i] == k) m = max(m, c_len[i]);
  }
  if (mine) a.glen[t] = m;
}

// Position of each tile in the order (-group length, key, -length, index).
__global__ __launch_bounds__(kBlock) void order_kernel(PartArgs a) {
  __shared__ int32_t c_g[kChunk], c_key[kChunk], c_len[kChunk];
  const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const bool mine = t < a.n_tiles;
  const int32_t g = mine ? a.glen[t] : 0, k = mine ? a.key[t] : 0;
  const int32_t l = mine ? a.row_ptr[t + 1] - a.row_ptr[t] : 0;
  int64_t pos = 0;
  for (int64_t base = 0; base < a.n_tiles; base += kChunk) {
    const int cnt = (int)min<int64_t>(kChunk, a.n_tiles - base);
    __syncthreads();
    for (int i = threadIdx.x; i < cnt; i += kBlock) {
      c_g[i] = a.glen[base + i];
      c_key[i] = a.key[base + i];
      c_len[i] = a.row_ptr[base + i + 1] - a.row_ptr[base + i];
    }
    __syncthreads();
    if (mine)
      for (int i = 0; i < cnt; ++i) {
        const int32_t gi = c_g[i], ki = c_key[i], li = c_len[i];
        bool before;
        if (gi != g) before = gi > g;
        else if (ki != k) before = ki < k;
        else if (li != l) before = li > l;
        else before = base + i < t;
        pos += before;
      }
  }
  if (mine) a.order[pos] = (int32_t)t;
}

hipError_t build_part(const PlanDeviceLaunch& L, const PlanDevicePart& P, hipStream_t stream) {
  if (P.n_tiles == 0) return hipSuccess;
  PartArgs a;
  a.slices = reinterpret_cast<const DevSlice*>(L.slices);
  a.rank = L.rank;
  a.status = L.status;
  a.R = L.R;
  a.n_tiles = P.n_tiles;
  a.bm = P.bm;
  a.bn = P.bn;
  a.transpose = P.transpose;
  a.cap = P.cap;
  a.count = P.count;
  a.key = P.key;
  a.glen = P.glen;
  a.row_ptr = P.row_ptr;
  a.entries = reinterpret_cast<DevEntry*>(P.entries);
  a.order = P.order;
  const unsigned tiles = (unsigned)P.n_tiles;
  const unsigned blocks = (unsigned)((P.n_tiles + kBlock - 1) / kBlock);
  hipLaunchKernelGGL(count_kernel, dim3(tiles), dim3(kBlock), 0, stream, a);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, a);
  hipLaunchKernelGGL(fill_kernel, dim3(tiles), dim3(kBlock), 0, stream, a);
  hipLaunchKernelGGL(group_kernel, dim3(blocks), dim3(kBlock), 0, stream, a);
  hipLaunchKernelGGL(order_kernel, dim3(blocks), dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int plan_device_max_slices() { return kMaxPlanSlices; }

hipError_t launch_plan_device(const PlanDeviceLaunch& L, hipStream_t stream) {
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(1), 0, stream, L.status);
  if (L.R > 0) {
    const unsigned blocks = (unsigned)((L.R + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(slices_kernel, dim3(blocks), dim3(kBlock), 0, stream, L.q_ranges, L.k_ranges,
                       L.types, L.R, L.Tq, L.Tk, reinterpret_cast<DevSlice*>(L.slices), L.status);
    hipLaunchKernelGGL(rank_kernel, dim3(blocks), dim3(kBlock), 0, stream,
                       reinterpret_cast<const DevSlice*>(L.slices), L.R, L.rank);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int i = 0; i < L.n_parts; ++i) {
    e = build_part(L, L.part[i], stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ffa
