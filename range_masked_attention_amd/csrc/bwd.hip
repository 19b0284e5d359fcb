// Backward kernels of range-masked flash attention for gfx950 (CDNA4).
//
// Gradients of sum(dO * out) through the forward (the usual flash-attention
// backward, recomputing probabilities from the saved lse):
//   P = exp(s - lse),  dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * out),
//   dS = P (dP - D) [* (1 - tanh^2) with softcap],  dQ = scale dS K,
//   dK = scale dS^T Q.
// The pages show this pass only through autograd (MagiAttention issue on
// dummy slices: out.backward(do) gives q.grad, k.grad, v.grad) and leave the
// varlen backward design open (CUTLASS issue #2192); this one is built for
// the slice plan:
//
//  bwd_pre   D for every (row, q head).
//  bwd_dkdv  one workgroup per (128-key tile, kv head); its 4 waves own 32
//            keys each and walk the key-side plan (64-row q tiles) for every
//            q head of the group, accumulating dK^T and dV^T in registers.
//  bwd_dq    one workgroup per (128-row q tile, q head), walking the same
//            per-q-tile list as the forward and accumulating dQ^T.
// dQ is recomputed in its own pass instead of being scattered with atomics:
// no fp32 accumulator buffer, no contention, and the result does not depend
// on the order in which workgroups finish.
#include "device_common.hpp"
#include "launch.hpp"

namespace ffa {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- bwd_pre
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(const __bf16* __restrict__ out,
                                                          const __bf16* __restrict__ dout,
                                                          float* __restrict__ dvec, int64_t n_rows) {
  const int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (r >= n_rows) return;
  const u32x4* po = reinterpret_cast<const u32x4*>(out + r * D);
  const u32x4* pd = reinterpret_cast<const u32x4*>(dout + r * D);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const u32x4 a = po[c], b = pd[c];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc += __uint_as_float(a[j] << 16) * __uint_as_float(b[j] << 16);
      acc += __uint_as_float(a[j] & 0xFFFF0000u) * __uint_as_float(b[j] & 0xFFFF0000u);
    }
  }
  dvec[r] = acc;
}

// ---------------------------------------------------------------- staging
// A ROWS x D bf16 tile read from global in units of 4 rows x 8 columns (one
// 16-byte load per row), written to LDS row-major (stride D + 8) and/or
// transposed (stride ROWS + 4, i.e. [column][row]).
template <int ROWS, int D>
struct Stage {
  static constexpr int kRmStr = D + 8;
  static constexpr int kTStr = ROWS + 4;
  static constexpr int kRm = ROWS * kRmStr;  // elements
  static constexpr int kT = D * kTStr;
  static constexpr int kUnits = (ROWS / 4) * (D / 8);
  static constexpr int kPerThread = (kUnits + kThreads - 1) / kThreads;

  u32x4 reg[kPerThread][4];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int64_t row_bytes, int tid) {
#pragma unroll
    for (int c = 0; c < kPerThread; ++c) {
      const int u = tid + kThreads * c;
      if (kUnits % kThreads == 0 || u < kUnits) {
        const int cc = u / (ROWS / 4), rg = u % (ROWS / 4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          reg[c][i] = buf_load16(r, (uint32_t)((4 * rg + i) * row_bytes + cc * 16));
      }
    }
  }

  __device__ __forceinline__ void store(__bf16* rm, __bf16* tr, int tid) const {
#pragma unroll
    for (int c = 0; c < kPerThread; ++c) {
      const int u = tid + kThreads * c;
      if (kUnits % kThreads == 0 || u < kUnits) {
        const int cc = u / (ROWS / 4), rg = u % (ROWS / 4);
        if (rm) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4*>(rm + (4 * rg + i) * kRmStr + 8 * cc) = reg[c][i];
        }
        if (tr) {
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            const int sh = (p & 1) * 16;
            u32x2 w;
            w[0] = ((reg[c][0][p >> 1] >> sh) & 0xFFFFu) | (((reg[c][1][p >> 1] >> sh) & 0xFFFFu) << 16);
            w[1] = ((reg[c][2][p >> 1] >> sh) & 0xFFFFu) | (((reg[c][3][p >> 1] >> sh) & 0xFFFFu) << 16);
            *reinterpret_cast<u32x2*>(tr + (8 * cc + p) * kTStr + 4 * rg) = w;
          }
        }
      }
    }
  }
};

// Reads 8 bf16 of a transposed tile: positions base..base+3 and base+8..base+11
// of row `row` -- the key (or query) order that matches a 32x32 accumulator's
// rows when it is reused as an MFMA operand.
__device__ __forceinline__ bf16x8 read_t8(const __bf16* t, int row, int stride, int base) {
  const __bf16* p = t + row * stride + base;
  const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 8);
  u32x4 x;
  x[0] = lo[0]; x[1] = lo[1]; x[2] = hi[0]; x[3] = hi[1];
  return __builtin_bit_cast(bf16x8, x);
}

// Row range of slice `sl` that key j sees: [lo, hi) (empty if hi <= lo).
__device__ __forceinline__ void key_rows(const DevSlice& sl, int j, int* lo, int* hi) {
  *lo = sl.qs;
  *hi = sl.qe;
  if (j < sl.ks || j >= sl.ke) *hi = *lo;
  else if (sl.causal) *lo = max(sl.qs, j - (sl.ke - sl.qe));
}

// Key range of slice `sl` that row i sees: [lo, hi).
__device__ __forceinline__ void row_keys(const DevSlice& sl, int i, int* lo, int* hi) {
  *lo = sl.ks;
  *hi = sl.ke;
  if (sl.causal) *hi = min(*hi, i + 1 + (sl.ke - sl.qe));
  if (i < sl.qs || i >= sl.qe) *hi = *lo;
}

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const float* lse;
  const float* dvec;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  const int32_t* row_ptr;   // plan walked by this kernel
  const DevEntry* entries;
  const int32_t* order;
  const DevSlice* slices;
  int32_t Tq, Tk, hq, hkv, grp;
  int32_t n_units;
  float scale;
  float score_mult;  // scale*log2(e), or 1 with softcap
  float cap_in;      // softcap: 2*scale*log2(e)/softcap
  float cap_out;     // softcap: softcap*log2(e)
};

// Scores to exponent units (base 2) and, with softcap, the tanh value the
// derivative needs.
template <bool SOFTCAP>
__device__ __forceinline__ float score_to_t(const BwdArgs& a, float s, float* th) {
  if constexpr (SOFTCAP) {
    *th = tanh_from_2xlog2e(s * a.cap_in);
    return a.cap_out * *th;
  } else {
    *th = 0.f;
    return s * a.score_mult;
  }
}

// ---------------------------------------------------------------- bwd_dkdv
constexpr int kDkvKeys = 128;  // keys per workgroup (32 per wave)
constexpr int kDkvRows = 64;   // q rows per step

template <int D>
struct DkvSmem {
  using St = Stage<kDkvRows, D>;
  static constexpr int kElems = 2 * (St::kRm + St::kT);  // Q and dO, row-major + transposed
};

template <int D, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using St = Stage<kDkvRows, D>;
  constexpr int KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 smem[DkvSmem<D>::kElems];
  __shared__ float s_lse[kDkvRows], s_dv[kDkvRows];
  __bf16* q_rm = smem;
  __bf16* q_t = q_rm + St::kRm;
  __bf16* o_rm = q_t + St::kT;
  __bf16* o_t = o_rm + St::kRm;

  const int u = blockIdx.x;
  if (u >= a.n_units) return;
  const int kt = a.order[u / a.hkv], g = u % a.hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 31, hh = lane >> 5;
  const int k0 = kt * kDkvKeys;
  const int key = k0 + 32 * w + n;  // this lane's key (accumulator column)
  const int64_t kv_row_bytes = (int64_t)a.hkv * D * 2;
  const int64_t q_row_bytes = (int64_t)a.hq * D * 2;

  // K and V fragments of this wave's 32 keys (B operands: key n, dims 16ks + 8hh ..)
  bf16x8 kf[KS], vf[KS];
  {
    const int64_t r0 = k0 + 32 * w;
    const int64_t off = (r0 * a.hkv + g) * D;
    const int64_t valid = ((int64_t)a.Tk - r0) * kv_row_bytes - (int64_t)g * D * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + off, valid);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + off, valid);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t o = (uint32_t)(n * kv_row_bytes + (16 * ks + 8 * hh) * 2);
      kf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rk, o));
      vf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rv, o));
    }
  }

  f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dk_acc[i] = dv_acc[i] = f32x16{};

  const int e_begin = a.row_ptr[kt], e_end = a.row_ptr[kt + 1];
  const int n_steps = (e_end - e_begin) * a.grp;

  St sq, so;
  auto issue = [&](int step) {
    const int e = e_begin + step / a.grp;
    const int head = g * a.grp + step % a.grp;
    const int64_t q0 = (int64_t)a.entries[e].tile * kDkvRows;
    const int64_t off = (q0 * a.hq + head) * D;
    const int64_t valid = ((int64_t)a.Tq - q0) * q_row_bytes - (int64_t)head * D * 2;
    sq.load(make_rsrc(a.q + off, valid), q_row_bytes, tid);
    so.load(make_rsrc(a.dout + off, valid), q_row_bytes, tid);
  };
  if (n_steps > 0) issue(0);

  for (int step = 0; step < n_steps; ++step) {
    const int e = e_begin + step / a.grp;
    const int head = g * a.grp + step % a.grp;
    const DevEntry ent = a.entries[e];
    const int q0 = ent.tile * kDkvRows;

    __syncthreads();  // previous step's LDS reads are done
    sq.store(q_rm, q_t, tid);
    so.store(o_rm, o_t, tid);
    if (tid < kDkvRows) {
      const int r = q0 + tid;
      const bool ok = r < a.Tq;
      const float l = ok ? a.lse[(int64_t)r * a.hq + head] : INFINITY;
      // rows nothing sees have lse = -inf: their P must be 0, not exp(+inf)
      s_lse[tid] = (l == -INFINITY) ? INFINITY : l * 1.4426950408889634f;
      s_dv[tid] = ok ? a.dvec[(int64_t)r * a.hq + head] : 0.f;
    }
    __syncthreads();
    if (step + 1 < n_steps) issue(step + 1);

    // ---- S = Q K^T and dP = dO V^T : [64 q x 32 keys] as two 32-row blocks
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = f32x16{};
      dp[qb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int o = (32 * qb + n) * St::kRmStr + 16 * ks + 8 * hh;
        s[qb] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(q_rm + o), kf[ks], s[qb]);
        dp[qb] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(o_rm + o), vf[ks], dp[qb]);
      }
    }

    // ---- P and dS, element (qb, v) is row 32qb + 8(v/4) + 4hh + v%4, key `key`
    int lo = 0, hi = kDkvRows;
    if (ent.meta & 1) {
      const DevSlice sl = a.slices[ent.meta >> 1];
      key_rows(sl, key, &lo, &hi);
      lo -= q0;
      hi -= q0;
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int rbase = 32 * qb + 8 * v4 + 4 * hh;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(s_lse + rbase);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(s_dv + rbase);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = 4 * v4 + i;
          float th;
          const float t = score_to_t<SOFTCAP>(a, s[qb][v], &th);
          float p = fast_exp2(t - l4[i]);
          if (rbase + i < lo || rbase + i >= hi) p = 0.f;
          float ds = p * (dp[qb][v] - d4[i]);
          if constexpr (SOFTCAP) ds *= 1.0f - th * th;
          s[qb][v] = p;
          dp[qb][v] = ds;
        }
      }

    // ---- dV^T += dO^T P and dK^T += Q^T dS : contraction over the 64 rows
    bf16x8 pf[4], df[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int qb = t >> 1, h8 = (t & 1) * 8;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        pf[t][e8] = (__bf16)s[qb][h8 + e8];
        df[t][e8] = (__bf16)dp[qb][h8 + e8];
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int base = 32 * (t >> 1) + 16 * (t & 1) + 4 * hh;
        dv_acc[db] = mfma_32x32x16(read_t8(o_t, 32 * db + n, St::kTStr, base), pf[t], dv_acc[db]);
        dk_acc[db] = mfma_32x32x16(read_t8(q_t, 32 * db + n, St::kTStr, base), df[t], dk_acc[db]);
      }
  }

  // ---- epilogue: accumulator column n is key `key`, rows are head dims
  if (key < a.Tk) {
    const int64_t off = ((int64_t)key * a.hkv + g) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * db + 8 * j + 4 * hh;
        u32x2 wv, wk;
        wv[0] = pack_bf16x2(dv_acc[db][4 * j + 0], dv_acc[db][4 * j + 1]);
        wv[1] = pack_bf16x2(dv_acc[db][4 * j + 2], dv_acc[db][4 * j + 3]);
        wk[0] = pack_bf16x2(a.scale * dk_acc[db][4 * j + 0], a.scale * dk_acc[db][4 * j + 1]);
        wk[1] = pack_bf16x2(a.scale * dk_acc[db][4 * j + 2], a.scale * dk_acc[db][4 * j + 3]);
        *reinterpret_cast<u32x2*>(a.dv + off + d0) = wv;
        *reinterpret_cast<u32x2*>(a.dk + off + d0) = wk;
      }
  }
}

// ---------------------------------------------------------------- bwd_dq
constexpr int kDqRows = 128;  // q rows per workgroup (32 per wave)
constexpr int kDqKeys = 64;   // keys per k tile

template <int D>
struct DqSmem {
  using St = Stage<kDqKeys, D>;
  static constexpr int kElems = 2 * St::kRm + St::kT;  // K row-major + transposed, V row-major
};

template <int D, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  using St = Stage<kDqKeys, D>;
  constexpr int KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 smem[DqSmem<D>::kElems];
  __bf16* k_rm = smem;
  __bf16* k_t = k_rm + St::kRm;
  __bf16* v_rm = k_t + St::kT;

  // work item: (q tile, head), q heads of one kv head on one XCD
  const int wg = blockIdx.x;
  const int xcd = wg & 7, slot = wg >> 3;
  const int r = slot % a.grp;
  const int u = (slot / a.grp) * 8 + xcd;
  if (u >= a.n_units) return;
  const int qt = a.order[u / a.hkv], g = u % a.hkv, head = g * a.grp + r;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 31, hh = lane >> 5;
  const int q0 = qt * kDqRows;
  const int row = q0 + 32 * w + n;
  const int64_t q_row_bytes = (int64_t)a.hq * D * 2;
  const int64_t kv_row_bytes = (int64_t)a.hkv * D * 2;

  bf16x8 qf[KS], of[KS];
  {
    const int64_t r0 = q0 + 32 * w;
    const int64_t off = (r0 * a.hq + head) * D;
    const int64_t valid = ((int64_t)a.Tq - r0) * q_row_bytes - (int64_t)head * D * 2;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + off, valid);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.dout + off, valid);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t o = (uint32_t)(n * q_row_bytes + (16 * ks + 8 * hh) * 2);
      qf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rq, o));
      of[ks] = __builtin_bit_cast(bf16x8, buf_load16(ro, o));
    }
  }
  float lse2 = INFINITY, dval = 0.f;
  if (row < a.Tq) {
    const float l = a.lse[(int64_t)row * a.hq + head];
    lse2 = (l == -INFINITY) ? INFINITY : l * 1.4426950408889634f;
    dval = a.dvec[(int64_t)row * a.hq + head];
  }

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  const int e_begin = a.row_ptr[qt], e_end = a.row_ptr[qt + 1];
  St sk, sv;
  auto issue = [&](int e) {
    const int64_t k0 = (int64_t)a.entries[e].tile * kDqKeys;
    const int64_t off = (k0 * a.hkv + g) * D;
    const int64_t valid = ((int64_t)a.Tk - k0) * kv_row_bytes - (int64_t)g * D * 2;
    sk.load(make_rsrc(a.k + off, valid), kv_row_bytes, tid);
    sv.load(make_rsrc(a.v + off, valid), kv_row_bytes, tid);
  };
  if (e_begin < e_end) issue(e_begin);

  for (int e = e_begin; e < e_end; ++e) {
    const DevEntry ent = a.entries[e];
    __syncthreads();
    sk.store(k_rm, k_t, tid);
    sv.store(v_rm, nullptr, tid);
    __syncthreads();
    if (e + 1 < e_end) issue(e + 1);

    // ---- S^T = K Q^T and dP^T = V dO^T : [64 keys x 32 q]
    f32x16 s[2], dp[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = f32x16{};
      dp[b] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int o = (32 * b + n) * St::kRmStr + 16 * ks + 8 * hh;
        s[b] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(k_rm + o), qf[ks], s[b]);
        dp[b] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(v_rm + o), of[ks], dp[b]);
      }
    }

    int lo = 0, hi = kDqKeys;
    if (ent.meta & 1) {
      const DevSlice sl = a.slices[ent.meta >> 1];
      row_keys(sl, row, &lo, &hi);
      lo -= ent.tile * kDqKeys + 4 * hh;
      hi -= ent.tile * kDqKeys + 4 * hh;
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int off = 32 * b + 8 * (v >> 2) + (v & 3);
        float th;
        const float t = score_to_t<SOFTCAP>(a, s[b][v], &th);
        float p = fast_exp2(t - lse2);
        if (off < lo || off >= hi) p = 0.f;
        float ds = p * (dp[b][v] - dval);
        if constexpr (SOFTCAP) ds *= 1.0f - th * th;
        s[b][v] = ds;
      }

    // ---- dQ^T += K^T dS^T : contraction over the 64 keys
    bf16x8 df[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int b = t >> 1, h8 = (t & 1) * 8;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) df[t][e8] = (__bf16)s[b][h8 + e8];
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int base = 32 * (t >> 1) + 16 * (t & 1) + 4 * hh;
        acc[db] = mfma_32x32x16(read_t8(k_t, 32 * db + n, St::kTStr, base), df[t], acc[db]);
      }
  }

  if (row < a.Tq) {
    __bf16* drow = a.dq + ((int64_t)row * a.hq + head) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w2;
        w2[0] = pack_bf16x2(a.scale * acc[db][4 * j + 0], a.scale * acc[db][4 * j + 1]);
        w2[1] = pack_bf16x2(a.scale * acc[db][4 * j + 2], a.scale * acc[db][4 * j + 3]);
        *reinterpret_cast<u32x2*>(drow + 32 * db + 8 * j + 4 * hh) = w2;
      }
  }
}

void fill_args(const BwdLaunch& p, BwdArgs* a) {
  a->q = static_cast<const __bf16*>(p.q);
  a->k = static_cast<const __bf16*>(p.k);
  a->v = static_cast<const __bf16*>(p.v);
  a->dout = static_cast<const __bf16*>(p.dout);
  a->lse = p.lse;
  a->dvec = p.dvec;
  a->dq = static_cast<__bf16*>(p.dq);
  a->dk = static_cast<__bf16*>(p.dk);
  a->dv = static_cast<__bf16*>(p.dv);
  a->slices = reinterpret_cast<const DevSlice*>(p.slices);
  a->Tq = (int32_t)p.Tq;
  a->Tk = (int32_t)p.Tk;
  a->hq = p.hq;
  a->hkv = p.hkv;
  a->grp = p.hq / p.hkv;
  a->scale = p.scale;
  const float log2e = 1.4426950408889634f;
  if (p.softcap > 0.f) {
    a->score_mult = 1.0f;
    a->cap_in = 2.0f * p.scale * log2e / p.softcap;
    a->cap_out = p.softcap * log2e;
  } else {
    a->score_mult = p.scale * log2e;
    a->cap_in = a->cap_out = 0.f;
  }
}

template <int D, bool SC>
hipError_t launch_bwd_t(const BwdLaunch& p, hipStream_t stream) {
  const int64_t rows = p.Tq * p.hq;
  if (rows > 0)
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, static_cast<const __bf16*>(p.out),
                       static_cast<const __bf16*>(p.dout), p.dvec, rows);
  BwdArgs a;
  fill_args(p, &a);
  // dK, dV: one workgroup per (key tile, kv head), every key tile listed
  a.row_ptr = p.kv_row_ptr;
  a.entries = reinterpret_cast<const DevEntry*>(p.kv_entries);
  a.order = p.kv_order;
  const int64_t n_kt = (p.Tk + kDkvKeys - 1) / kDkvKeys;
  a.n_units = (int32_t)(n_kt * p.hkv);
  if (a.n_units > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, SC>), dim3((unsigned)a.n_units), dim3(kThreads), 0, stream, a);
  // dQ: one workgroup per (q tile, head)
  a.row_ptr = p.q_row_ptr;
  a.entries = reinterpret_cast<const DevEntry*>(p.q_entries);
  a.order = p.q_order;
  const int64_t n_qt = (p.Tq + kDqRows - 1) / kDqRows;
  a.n_units = (int32_t)(n_qt * p.hkv);
  const int64_t n_wg = ((a.n_units + 7) / 8) * 8 * (int64_t)a.grp;
  if (n_wg > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<D, SC>), dim3((unsigned)n_wg), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int bwd_kv_tile_rows() { return kDkvRows; }
int bwd_kv_tile_cols() { return kDkvKeys; }
int bwd_q_tile_rows() { return kDqRows; }
int bwd_q_tile_cols() { return kDqKeys; }

hipError_t launch_bwd(const BwdLaunch& p, hipStream_t stream) {
  const bool sc = p.softcap > 0.f;
  if (p.d == 64) return sc ? launch_bwd_t<64, true>(p, stream) : launch_bwd_t<64, false>(p, stream);
  return sc ? launch_bwd_t<128, true>(p, stream) : launch_bwd_t<128, false>(p, stream);
}

}  // namespace ffa
