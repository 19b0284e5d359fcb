// Backward kernels of range-masked flash attention for gfx950 (CDNA4).
//
// Gradients of sum(dO * out) through the forward (the usual flash-attention
// backward, recomputing probabilities from the saved lse):
//   P = exp(s - lse),  dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * out),
//   dS = P (dP - D) [* (1 - tanh^2) with softcap],  dQ = scale dS K,
//   dK = scale dS^T Q.
// With the optional distance bias (ALiBi: FlexAttention paper summary,
// sections 2 and 3.1) the scores gain slope[head] * (j - i) after the
// softcap; it only changes P, recomputed here exactly as in the forward.
// The pages show this pass only through autograd (MagiAttention issue on
// dummy slices: out.backward(do) gives q.grad, k.grad, v.grad) and leave the
// varlen backward design open (CUTLASS issue #2192); this one is built for
// the slice plan:
//
//  bwd_prep  (after the range pass of convert.hip over dO and k's tracked
//            fp16 copy; q's range comes with the forward's record)
//            fp16 copies of q and dO, each times the power of two that maps
//            its range onto fp16's (k's comes from convert.hip, v's with the
//            record the training forward saved); D for every (row, q head)
//            from dO and the forward's output with its rounding residual,
//            and lse in exp2 units, both stored head-major ([hq][Tq]) so
//            that a step's 64 rows are contiguous.
//  bwd_dkdv  one workgroup per (128-key tile, kv head); its 4 wave pairs own
//            32 keys each and walk the key-side plan (64-row q tiles) for
//            every q head of the group, accumulating dK^T and dV^T in
//            registers.
//  bwd_dq    one workgroup per (128-row q tile, q head), walking the per-q-
//            tile list of 64-key tiles and accumulating dQ^T.
// A list much longer than the average is cut into runs (split.hip), one
// workgroup each; runs write fp32 partial sums that bwd_dkdv_reduce and
// bwd_dq_reduce add in run order.  dQ is recomputed in its own pass instead
// of being scattered with atomics: no contention, and the result does not
// depend on the order in which workgroups finish.
//
// Precision: the products run on fp16 operands (11 significant bits; bf16
// has 8) at the same matrix-core rate, so P and dS enter them with 2^-11
// relative rounding instead of 2^-8.  The fp16 copies of q, k, v and dO are
// exact (bf16 values times a power of two, inside fp16's normal range up to
// values far below the largest, which round at 2^-25 after scaling; v's copy
// comes from the forward, at scale 1 when its range allows), and the powers
// of two come back out exactly in the score multiplier and the final scaling
// of dq, dk and dv.  D is formed from out plus its rounding
// residual, from a forward whose P V product also ran in fp16, so it carries
// neither out's bf16 rounding nor a bf16 rounding of P.
//
// Tiles of 64 rows are fetched straight into LDS (buffer_load ... lds), one
// load instruction per 16-byte chunk column: LDS holds a tile column-major by
// chunk, 64 rows x 16 bytes per column plus 64 bytes of padding.  Row-wise
// MFMA operands are then 16 lanes x 16 contiguous bytes, and transposed
// operands come from transpose reads (ds_read_b64_tr_b16) hitting 4 columns
// 16 banks apart: neither conflicts on the 64 LDS banks.  Tiles are double
// buffered, with one barrier per step.
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace ffa {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- bwd_prep
// D * sdo * sv for every (row, head), lse in exp2 units, and the fp16 copies
// of q and dO (convert.hip's scaling).  D / 8 lanes per (row, head), one
// 16-byte chunk each, so a wave reads whole rows; lse2 turns -inf (a row that
// sees nothing) into +inf, so that exp2(s - lse2) is 0 there rather than NaN.
// D = rowsum(dO * (out + out_lo)) in fp32, out_lo being the rounding
// residual the training forward saved.  Thread 0 also writes the four scales
// [q, k, v, dO] for the kernels after it.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(const u32x4* __restrict__ q, const u32x4* __restrict__ out,
                                                          const u32x4* __restrict__ out_lo,
                                                          const u32x4* __restrict__ dout, const float* __restrict__ lse,
                                                          const uint32_t* __restrict__ range,
                                                          const uint32_t* __restrict__ vwords, u32x4* __restrict__ q16,
                                                          u32x4* __restrict__ do16, float* __restrict__ dvec,
                                                          float* __restrict__ lse2, float* __restrict__ scales,
                                                          int64_t Tq, int hq) {
  constexpr int kL = D / 8;  // lanes per (row, head)
  const float sq = range_scale(vwords[kRgQ], kRangeQ), sk = copy_scale(range[kRgK], kRangeK);
  const float sv = copy_scale(vwords[kRgV], kRangeV);
  const float sdo = range_scale(range[kRgDO], kRangeDOV - range_top(vwords[kRgV], sv));
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i == 0) {
    scales[kRgQ] = sq;
    scales[kRgK] = sk;
    scales[kRgV] = sv;
    scales[kRgDO] = sdo;
  }
  const int64_t r = i / kL;  // (row, head) = (r / hq, r % hq)
  const bool live = r < Tq * hq;
  float acc = 0.f;
  if (live) {
    const u32x4 a = out[i], b = out_lo[i], g = dout[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float d0 = __uint_as_float(g[j] << 16), d1 = __uint_as_float(g[j] & 0xFFFF0000u);
      acc += d0 * (__uint_as_float(a[j] << 16) + __uint_as_float(b[j] << 16));
      acc += d1 * (__uint_as_float(a[j] & 0xFFFF0000u) + __uint_as_float(b[j] & 0xFFFF0000u));
    }
    q16[i] = to_f16x8(q[i], sq);
    do16[i] = to_f16x8(g, sdo);
  }
#pragma unroll
  for (int o = 1; o < kL; o <<= 1) acc += __shfl_xor(acc, o);
  if (live && (i % kL) == 0) {
    const int64_t row = r / hq, head = r - row * hq;
    const int64_t t = head * Tq + row;
    dvec[t] = acc * sdo * sv;
    const float l = lse[r];
    lse2[t] = (l == -INFINITY) ? INFINITY : l * 1.4426950408889634f;
  }
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

// q, k, v and dout point at the fp16 copies (16-bit lanes carried in bf16
// vector types; the fp16 products read them as fp16); `scales` holds their
// powers of two, [q, k, v, dO].
struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const float* scales;
  const float* lse;
  const float* dvec;        // D, head-major [hq][Tq]
  const float* lse2;        // lse in exp2 units (+inf: nothing visible), head-major
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  const int32_t* row_ptr;   // plan walked by this kernel
  const DevEntry* entries;
  const int32_t* order;
  const DevSlice* slices;
  const i32x4* items;       // dK/dV work items (key tile, entries, slot)
  const i32x4* splits;      // key tiles split over several items
  const int32_t* counts;    // [0] items, [1] split tiles
  float* partial;           // fp32 dK^T / dV^T of the items of split tiles (dQ: fp32 dQ)
  const float* slopes;      // [hq] distance-bias slopes (biased kernels only)
  int32_t Tq, Tk, hq, hkv, grp;
  int32_t n_units;
  int32_t direct;           // dK/dV: 1 = one item per key tile, from the plan itself
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

__device__ __forceinline__ u32x4 pack8(const float* p) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_f16x2(p[2 * i], p[2 * i + 1]);
  return w;
}

// The operand scales folded into the score multipliers: s' = sq sk s, so
// the multipliers that turn raw scores into exponent (or tanh) units take
// 1 / (sq sk).  Powers of two: exact.
__device__ __forceinline__ void fold_scales(BwdArgs* a, float* sq, float* sk, float* sv, float* sdo) {
  *sq = const_load<float>(a->scales, 0);
  *sk = const_load<float>(a->scales, 1);
  *sv = const_load<float>(a->scales, 2);
  *sdo = const_load<float>(a->scales, 3);
  const float inv = 1.0f / (*sq * *sk);
  a->score_mult *= inv;
  a->cap_in *= inv;
}

// ---------------------------------------------------------------- bwd_dkdv
// 8 waves in 4 pairs; pair p owns keys 32p .. 32p + 31 of the 128-key tile.
// In a pair the producer wave (w < 4) computes S = Q K^T, P and dV^T += dO^T P
// and hands P (times 1 - tanh^2 with softcap) to its consumer wave through
// LDS; the consumer (w >= 4) computes dP = dO V^T and, one step behind,
// dS = P (dP - D) and dK^T += Q^T dS.  Each wave keeps one K or V fragment
// and one accumulator (half of what one wave doing both would need), so two
// waves fit on each SIMD and one's exponentials overlap the other's matrix
// work.  Q tiles are triple buffered (the consumer reads tile j - 1 while
// the producer reads tile j and tile j + 1 is in flight), dO tiles double
// buffered; one barrier per step.  Each buffer is its own LDS object and the
// step loops are unrolled six times so that every access names its buffer
// at compile time: the compiler then knows a read of one buffer does not
// depend on a fetch into another and does not wait for it.
constexpr int kDkvKeys = 128;    // keys per workgroup (32 per wave pair)
constexpr int kDkvRows = 64;     // q rows per step
constexpr int kDkvThreads = 512;

template <int R>
using IC = std::integral_constant<int, R>;

template <int D, bool SOFTCAP, bool BIAS>
__global__ __launch_bounds__(kDkvThreads, 1) void bwd_dkdv_kernel(BwdArgs a0) {
  using T = ColTile<D>;
  BwdArgs a = a0;
  float sq, sk, sv, sdo;
  fold_scales(&a, &sq, &sk, &sv, &sdo);
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int kXchg = kDkvRows * 32;  // fp32 P of one pair and step (floats)
  // softcap without the bias: the producer works from r = 1 / (2^y + 1)
  // (tanh = 1 - 2r, 1 - tanh^2 = 4r(1 - r)) and forms 4P, its rows' lse
  // term holding cap_out + 2 - lse; dV then accumulates 4 dV
  constexpr bool RCAP = SOFTCAP && !BIAS;
  const float cap_m2 = -2.0f * a.cap_out;
  __shared__ __attribute__((aligned(1024))) char q_s0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char q_s1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char q_s2[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char o_s0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char o_s1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) float xchg[2][4][kXchg];
  __shared__ float s_lse[3][kDkvRows], s_dv[3][kDkvRows];
  auto qbuf = [&](auto r) -> char* {
    if constexpr (decltype(r)::value % 3 == 0) return q_s0;
    else if constexpr (decltype(r)::value % 3 == 1) return q_s1;
    else return q_s2;
  };
  auto obuf = [&](auto r) -> char* {
    if constexpr (decltype(r)::value % 2 == 0) return o_s0;
    else return o_s1;
  };

  // work item: a run of one key tile's entries (or, with a.direct, the
  // whole list of the key tile at that place in the plan order), kv head g
  const int u = blockIdx.x;
  const int item = u / a.hkv, g = u % a.hkv;
  int kt, e_begin, e_end, slot;
  if (a.direct) {
    if (item >= a.n_units) return;
    kt = plan_i32(a.order, item);
    e_begin = plan_i32(a.row_ptr, kt);
    e_end = plan_i32(a.row_ptr, kt + 1);
    slot = -1;
  } else {
    if (item >= plan_i32(a.counts, 0)) return;
    const i32x4 it = const_load<i32x4>(a.items, item);
    kt = it[0];
    e_begin = it[1];
    e_end = it[2];
    slot = it[3];
  }
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = w & 3;
  const bool producer = w < 4;
  const int k0 = kt * kDkvKeys;
  const int key = k0 + 32 * pair + n;  // this lane's key (accumulator column)
  const int64_t kv_row_bytes = (int64_t)a.hkv * D * 2;
  const int64_t q_row_bytes = (int64_t)a.hq * D * 2;

  // K (producer) or V (consumer) fragment of the pair's 32 keys
  // (B operand: key n, dims 16ks + 8hh ..)
  bf16x8 frag[KS];
  {
    const int64_t r0 = k0 + 32 * pair;
    const int64_t off = (r0 * a.hkv + g) * D;
    const int64_t valid = ((int64_t)a.Tk - r0) * kv_row_bytes - (int64_t)g * D * 2;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc((producer ? a.k : a.v) + off, valid);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 f = buf_load16(rs, (uint32_t)(n * kv_row_bytes + (16 * ks + 8 * hh) * 2));
      // the consumer holds -V (fp16 sign bits): its products give -dP
      if (!producer) f ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      frag[ks] = __builtin_bit_cast(bf16x8, f);
    }
  }

  f32x16 acc[DB];  // dV^T (producer) or dK^T (consumer): rows dims, column key
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  const int n_steps = (e_end - e_begin) * a.grp;
  const int tro = tr_lane_offset<D>(lane);
  const int lrow = T::off(n, hh);
  // read bases of the tile buffers: producers read Q rows and dO transposed,
  // consumers Q transposed and dO rows
  const char* qb3[3];
  const char* ob2[2];

  // step st = (entry e, q head): producers fetch the Q tile, consumers the
  // dO tile; wave 0 also fetches the step's lse and D (first, so that a
  // wait for them never waits for the tile fetches behind them).  Entries
  // are walked last to first: key tiles of one causal sequence then all
  // start at the sequence's last q tile and move down together, so the
  // workgroups resident at the same time read the same Q/dO tiles from L2.
  float lse_raw = 0.f, d_raw = 0.f, bias_row = 0.f;
  // Steps go head-minor: step st is entry e_end - 1 - st / grp, head
  // g * grp + st % grp.  Counters advanced once per step stand in for the
  // divisions: (f_e, f_h) for the next step to fetch, (p_e, p_h) for the
  // producer's current step.
  int f_e = e_end - 1, f_h = 0, p_e = e_end - 1, p_h = 0;
  auto advance = [&](int& e_, int& h_) {
    if (++h_ == a.grp) {
      h_ = 0;
      --e_;
    }
  };
  auto issue = [&](char* dst) {
    const int e = f_e;
    const int head = g * a.grp + f_h;
    advance(f_e, f_h);
    const int64_t q0 = (int64_t)plan_entry(a.entries, e).tile * kDkvRows;
    if (tid < kDkvRows) {
      const int64_t r = q0 + tid;
      lse_raw = INFINITY;
      d_raw = 0.f;
      if (r < a.Tq) {
        lse_raw = a.lse2[(int64_t)head * a.Tq + r];
        d_raw = a.dvec[(int64_t)head * a.Tq + r];
      }
      // the row's part of the bias, -slope (i - q0), moves into its lse:
      // exp2(t + slope (j - i) - lse) = exp2(t + slope (j - q0) - (lse + slope (i - q0)))
      if constexpr (BIAS) bias_row = const_load<float>(a.slopes, head) * 1.4426950408889634f * (float)tid;
    }
    const int64_t off = (q0 * a.hq + head) * D;
    const int64_t valid = ((int64_t)a.Tq - q0) * q_row_bytes - (int64_t)head * D * 2;
    T::load(make_rsrc((producer ? a.q : a.dout) + off, valid), (uint32_t)q_row_bytes, dst, pair, lane);
  };
  // the step loops run six steps per turn from st = 0, so a step's slot in
  // the 3- and 2-deep buffers is fixed by its position R in the turn
  auto publish = [&](int slot) {
    if (tid < kDkvRows) {
      // lse in exp2 units (+inf for rows nothing sees, so their P is 0)
      s_lse[slot][tid] = RCAP ? (a.cap_out + 2.0f) - lse_raw : lse_raw + bias_row;
      s_dv[slot][tid] = d_raw;
    }
  };

  // producer step st (st == n_steps: nothing left but the barrier)
  auto pstep = [&](int st, auto r) {
    if (st < n_steps) {
      constexpr int R = decltype(r)::value;
      if (st + 1 < n_steps) issue(qbuf(IC<R + 1>{}));
      const DevEntry ent = plan_entry(a.entries, p_e);
      // the key's part of the bias, slope (j - q0), in exp2 units
      float bias_key = 0.f;
      if constexpr (BIAS)
        bias_key = const_load<float>(a.slopes, g * a.grp + p_h) * 1.4426950408889634f *
                   (float)(key - ent.tile * kDkvRows);
      advance(p_e, p_h);
      const char* qt = qb3[R % 3];  // rows of Q
      const char* ot = ob2[R % 2];  // transposed dO
      float* xch = xchg[st & 1][pair];

      // S = Q K^T : [64 q x 32 keys] as two 32-row blocks
      f32x16 s[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        s[qb] = f32x16{};
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) s[qb] = mfma_32x32x16_f16(T::row8(qt, 0, 32 * qb, 2 * ks), frag[ks], s[qb]);
      // P; element (qb, v) is row 32qb + 8(v/4) + 4hh + v%4, key `key`
      // the per-cell mask only on PARTIAL entries (a FULL entry has every
      // cell visible, tails included), chosen once per step
      u32x4 pw[4];
      auto p_tile = [&](auto partial) {
        constexpr bool PARTIAL = decltype(partial)::value;
        int lo = 0, hi = kDkvRows;
        if constexpr (PARTIAL) {
          const DevSlice sl = plan_slice(a.slices, ent.meta >> 1);
          key_rows(sl, key, &lo, &hi);
          lo -= ent.tile * kDkvRows;
          hi -= ent.tile * kDkvRows;
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int rbase = 32 * qb + 8 * v4 + 4 * hh;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(&s_lse[st % 3][rbase]);
            f32x4 px;
            float p4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if constexpr (RCAP) {
                const float rc = fast_rcp(fast_exp2(s[qb][4 * v4 + i] * a.cap_in) + 1.0f);
                float p = fast_exp2(__builtin_fmaf(rc, cap_m2, l4[i]));  // 4P
                if constexpr (PARTIAL)
                  if (rbase + i < lo || rbase + i >= hi) p = 0.f;
                p4[i] = p;
                px[i] = p * __builtin_fmaf(-rc, rc, rc);  // P (1 - tanh^2)
              } else {
                float th;
                const float t = score_to_t<SOFTCAP>(a, s[qb][4 * v4 + i], &th);
                float p = BIAS ? fast_exp2(t + (bias_key - l4[i])) : fast_exp2(t - l4[i]);
                if constexpr (PARTIAL)
                  if (rbase + i < lo || rbase + i >= hi) p = 0.f;
                p4[i] = p;
                px[i] = SOFTCAP ? p * (1.0f - th * th) : p;
              }
            }
            *reinterpret_cast<f32x4*>(xch + ((qb * 4 + v4) * 64 + lane) * 4) = px;
            pw[2 * qb + (v4 >> 1)][2 * (v4 & 1)] = pack_f16x2(p4[0], p4[1]);
            pw[2 * qb + (v4 >> 1)][2 * (v4 & 1) + 1] = pack_f16x2(p4[2], p4[3]);
          }
      };
      if (ent.meta & 1)
        p_tile(std::true_type{});
      else
        p_tile(std::false_type{});
      // dV^T += dO^T P : contraction over the 64 rows
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[db] = mfma_32x32x16_f16(tr8<D>(ot, 0, db, t4), __builtin_bit_cast(bf16x8, pw[t4]), acc[db]);
      if (st + 1 < n_steps) publish((st + 1) % 3);
    }
    dma_barrier();
  };

  // consumer step st: D - dP of step st on the matrix cores (accumulators
  // start from the rows' D, and the consumer's V fragment is held negated),
  // then -dS = P (D - dP) of step st - 1 from what the previous step left,
  // whose arithmetic runs in the shadow of those products, and dK of step
  // st - 1 (accumulating -dK^T; the final scaling flips the sign back).
  // D - dP alternates between two register sets by step parity.
  f32x16 dp0[2], dp1[2];
  auto cstep = [&](int st, auto r) {
    constexpr int R = decltype(r)::value;
    f32x16* dcur = R % 2 == 0 ? dp0 : dp1;   // D - dP of step st
    f32x16* dprev = R % 2 == 0 ? dp1 : dp0;  // D - dP of step st - 1
    const char* ot = ob2[R % 2];             // rows of dO, step st
    const char* qt = qb3[(R + 5) % 3];       // transposed Q of step st - 1
    const float* xch = xchg[(st - 1) & 1][pair];
    if (st + 1 < n_steps) issue(obuf(IC<R + 1>{}));
    auto dp_products = [&]() {
      // element (qb, 4 v4 + i) is row 32 qb + 8 v4 + 4 hh + i
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&s_dv[st % 3][32 * qb + 8 * v4 + 4 * hh]);
#pragma unroll
          for (int i = 0; i < 4; ++i) dcur[qb][4 * v4 + i] = d4[i];
        }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          dcur[qb] = mfma_32x32x16_f16(T::row8(ot, 0, 32 * qb, 2 * ks), frag[ks], dcur[qb]);
    };
    auto ds_dk = [&]() {
      u32x4 dw[4];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int qb = x >> 2, v4 = x & 3;
        const f32x4 px = *reinterpret_cast<const f32x4*>(xch + (x * 64 + lane) * 4);
        float ds[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ds[i] = px[i] * dprev[qb][4 * v4 + i];
        dw[2 * qb + (v4 >> 1)][2 * (v4 & 1)] = pack_f16x2(ds[0], ds[1]);
        dw[2 * qb + (v4 >> 1)][2 * (v4 & 1) + 1] = pack_f16x2(ds[2], ds[3]);
      }
      // -dK^T += Q^T (-dS)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[db] = mfma_32x32x16_f16(tr8<D>(qt, 0, db, t4), __builtin_bit_cast(bf16x8, dw[t4]), acc[db]);
    };
    if (st < n_steps) dp_products();
    if (st > 0) ds_dk();
    dma_barrier();
  };

  if (n_steps > 0) {
    issue(producer ? qbuf(IC<0>{}) : obuf(IC<0>{}));
    publish(0);
    dma_barrier();
    // n_steps + 1 steps in both roles, so both pass the same barriers
    if (producer) {
      qb3[0] = lane_base(q_s0, lrow);
      qb3[1] = lane_base(q_s1, lrow);
      qb3[2] = lane_base(q_s2, lrow);
      ob2[0] = lane_base(o_s0, tro);
      ob2[1] = lane_base(o_s1, tro);
      for (int st = 0; st <= n_steps; st += 6) {
        pstep(st, IC<0>{});
        if (st + 1 > n_steps) break;
        pstep(st + 1, IC<1>{});
        if (st + 2 > n_steps) break;
        pstep(st + 2, IC<2>{});
        if (st + 3 > n_steps) break;
        pstep(st + 3, IC<3>{});
        if (st + 4 > n_steps) break;
        pstep(st + 4, IC<4>{});
        if (st + 5 > n_steps) break;
        pstep(st + 5, IC<5>{});
      }
    } else {
      qb3[0] = lane_base(q_s0, tro);
      qb3[1] = lane_base(q_s1, tro);
      qb3[2] = lane_base(q_s2, tro);
      ob2[0] = lane_base(o_s0, lrow);
      ob2[1] = lane_base(o_s1, lrow);
      for (int st = 0; st <= n_steps; st += 6) {
        cstep(st, IC<0>{});
        if (st + 1 > n_steps) break;
        cstep(st + 1, IC<1>{});
        if (st + 2 > n_steps) break;
        cstep(st + 2, IC<2>{});
        if (st + 3 > n_steps) break;
        cstep(st + 3, IC<3>{});
        if (st + 4 > n_steps) break;
        cstep(st + 4, IC<4>{});
        if (st + 5 > n_steps) break;
        cstep(st + 5, IC<5>{});
      }
    }
  }

  // accumulator column n is key `key`, rows are head dims
  if (slot >= 0) {
    // one run of a split key tile: fp32 partial sums, [-dK^T | dV^T][key][dim]
    float* dst = a.partial + ((int64_t)slot * a.hkv + g) * (2 * kDkvKeys * D) +
                 (producer ? kDkvKeys * D : 0) + (32 * pair + n) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 x;
        x[0] = acc[db][4 * j + 0];
        x[1] = acc[db][4 * j + 1];
        x[2] = acc[db][4 * j + 2];
        x[3] = acc[db][4 * j + 3];
        *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * j + 4 * hh) = x;
      }
  } else if (key < a.Tk) {
    const int64_t off = ((int64_t)key * a.hkv + g) * D;
    __bf16* dst = producer ? a.dv : a.dk;
    // dV^T accumulated sdo dV (4 sdo dV in the reciprocal form); the consumer
    // accumulated -sdo sv sq dK^T / scale
    const float mul = producer ? (RCAP ? 0.25f : 1.0f) / sdo : -a.scale / (sdo * sv * sq);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 wv;
        wv[0] = pack_bf16x2(mul * acc[db][4 * j + 0], mul * acc[db][4 * j + 1]);
        wv[1] = pack_bf16x2(mul * acc[db][4 * j + 2], mul * acc[db][4 * j + 3]);
        *reinterpret_cast<u32x2*>(dst + off + 32 * db + 8 * j + 4 * hh) = wv;
      }
  }
}

// ---------------------------------------------------------------- split
// A key tile's list is one serial chain in the dK/dV kernel, so a tile that
// many q tiles see (a global "sink" that every block attends, a long causal
// sequence shared by few heads) would set the kernel's duration by itself.
// The split pass (split.hip) cuts long lists into runs so that the runs of
// all tiles over all kv heads number about kDkvBalance (twice the 256 CUs);
// runs of a split tile write fp32 partial sums and bwd_dkdv_reduce adds them
// in run order, so the result does not depend on timing.
constexpr int kDkvBalance = 512;
constexpr int kDkvMinSteps = 32;   // (entry, q head) steps: never split below this
constexpr int kDkvMaxSlots = 512;  // partial buffers: runs of split tiles x kv heads

// Sum of the partial dK^T / dV^T of a split tile's runs, in run order, to
// bf16 dK (times the softmax scale) and dV: one 16-byte chunk per thread,
// kDkvReduceParts workgroups per (split tile, kv head).
template <int D>
constexpr int kDkvReduceParts = 2 * kDkvKeys * D / 4 / kThreads;

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_reduce_kernel(BwdArgs a0) {
  BwdArgs a = a0;
  float sq, sk, sv, sdo;
  fold_scales(&a, &sq, &sk, &sv, &sdo);
  constexpr int kSlot = 2 * kDkvKeys * D;  // floats per (run, kv head)
  const int u = blockIdx.x / kDkvReduceParts<D>, part = blockIdx.x % kDkvReduceParts<D>;
  const int s = u / a.hkv, g = u % a.hkv;
  if (s >= plan_i32(a.counts, 1)) return;
  const i32x4 sp = const_load<i32x4>(a.splits, s);
  const int kt = sp[0], slot0 = sp[1], ns = sp[2];
  {
    const int i = 4 * (part * kThreads + (int)threadIdx.x);
    f32x4 sum = f32x4{};
#pragma unroll 4
    for (int c = 0; c < ns; ++c)
      sum += *reinterpret_cast<const f32x4*>(a.partial + ((int64_t)(slot0 + c) * a.hkv + g) * kSlot + i);
    const bool is_v = i >= kDkvKeys * D;
    const int r = is_v ? i - kDkvKeys * D : i;
    const int key = kt * kDkvKeys + r / D, dim = r % D;
    if (key < a.Tk) {
      // dK^T partials carry -dK; dV partials 4 dV with softcap and no bias
      const float vmul = (a.cap_out > 0.f && a.slopes == nullptr) ? 0.25f : 1.0f;
      const float mul = is_v ? vmul / sdo : -a.scale / (sdo * sv * sq);
      u32x2 w;
      w[0] = pack_bf16x2(mul * sum[0], mul * sum[1]);
      w[1] = pack_bf16x2(mul * sum[2], mul * sum[3]);
      *reinterpret_cast<u32x2*>((is_v ? a.dv : a.dk) + ((int64_t)key * a.hkv + g) * D + dim) = w;
    }
  }
}

// ---------------------------------------------------------------- bwd_dq
// K and V tiles double buffered in four LDS objects, loop unrolled twice so
// each access names its buffer at compile time (see the dK/dV kernel).
constexpr int kDqRows = 128;  // q rows per workgroup (32 per wave)
constexpr int kDqKeys = 64;   // keys per k tile
// Long q-tile lists are cut into runs as in the forward (split.hip): lists
// longer than one workgroup slot's share (512 slots: two per CU) become runs
// of at least kDqMinSteps key tiles, whose fp32 dQ bwd_dq_reduce adds in run
// order.
constexpr int kDqBalance = 512;
constexpr int kDqMinSteps = 64;
constexpr int kDqMaxSlots = 512;  // partial buffers: runs of split tiles x q heads

template <int D, bool SOFTCAP, bool BIAS>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs a0) {
  using T = ColTile<D>;
  BwdArgs a = a0;
  float sq, sk, sv, sdo;
  fold_scales(&a, &sq, &sk, &sv, &sdo);
  // dQ^T accumulates sdo sv sk dQ / scale
  const float out_mul = a.scale / (sdo * sv * sk);
  constexpr int KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(1024))) char k_s0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char k_s1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char v_s0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char v_s1[T::kBytes];

  // work item: (run of a q tile's list, head), q heads of one kv head on
  // one XCD; with a.direct the whole list of the q tile at that place in the
  // plan order
  const int wg = blockIdx.x;
  const int xcd = wg & 7, wslot = wg >> 3;
  const int r = wslot % a.grp;
  const int u = (wslot / a.grp) * 8 + xcd;
  const int item = u / a.hkv, g = u % a.hkv, head = g * a.grp + r;
  int qt, e_begin, e_end, pslot;
  if (a.direct) {
    if (u >= a.n_units) return;
    qt = plan_i32(a.order, item);
    e_begin = plan_i32(a.row_ptr, qt);
    e_end = plan_i32(a.row_ptr, qt + 1);
    pslot = -1;
  } else {
    if (item >= plan_i32(a.counts, 0)) return;
    const i32x4 it = const_load<i32x4>(a.items, item);
    qt = it[0];
    e_begin = it[1];
    e_end = it[2];
    pslot = it[3];
  }

  const int tid = threadIdx.x, lane = tid & 63, n = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    lse2 = a.lse2[(int64_t)head * a.Tq + row];
    dval = a.dvec[(int64_t)head * a.Tq + row];
  }

  // distance bias in exp2 units: slope * (j - i) for key j
  const float slope2 = BIAS ? const_load<float>(a.slopes, head) * 1.4426950408889634f : 0.f;

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  const int tro = tr_lane_offset<D>(lane);
  const int lrow = T::off(n, hh);
  auto issue = [&](int e, char* kd, char* vd) {
    const int64_t k0 = (int64_t)plan_entry(a.entries, e).tile * kDqKeys;
    const int64_t off = (k0 * a.hkv + g) * D;
    const int64_t valid = ((int64_t)a.Tk - k0) * kv_row_bytes - (int64_t)g * D * 2;
    T::load(make_rsrc(a.k + off, valid), (uint32_t)kv_row_bytes, kd, w, lane);
    T::load(make_rsrc(a.v + off, valid), (uint32_t)kv_row_bytes, vd, w, lane);
  };

  auto step = [&](int e, const char* kt, const char* vt, char* kn, char* vn) {
    const DevEntry ent = plan_entry(a.entries, e);
    if (e + 1 < e_end) issue(e + 1, kn, vn);

    // ---- S^T = K Q^T and dP^T = V dO^T : [64 keys x 32 q]
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s[kb] = mfma_32x32x16_f16(T::row8(kt, lrow, 32 * kb, 2 * ks), qf[ks], s[kb]);
        dp[kb] = mfma_32x32x16_f16(T::row8(vt, lrow, 32 * kb, 2 * ks), of[ks], dp[kb]);
      }
    }

    // exp2 argument offset of the tile: slope (j0 - i) - lse, j0 = first key + 4 hh;
    // register v adds slope * off
    const float base = BIAS ? slope2 * (float)(ent.tile * kDqKeys + 4 * hh - row) - lse2 : 0.f;
    // dS^T of the tile; the per-cell mask only on PARTIAL entries (a FULL
    // entry has every cell visible, tails included), chosen once per tile
    u32x4 dw[4];
    auto ds_tile = [&](auto partial) {
      constexpr bool PARTIAL = decltype(partial)::value;
      int lo = 0, hi = kDqKeys;
      if constexpr (PARTIAL) {
        const DevSlice sl = plan_slice(a.slices, ent.meta >> 1);
        row_keys(sl, row, &lo, &hi);
        lo -= ent.tile * kDqKeys + 4 * hh;
        hi -= ent.tile * kDqKeys + 4 * hh;
      }
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int kb = t4 >> 1, h8 = (t4 & 1) * 8;
        float d8[8];
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          const int v = h8 + e8;
          const int off = 32 * kb + 8 * (v >> 2) + (v & 3);
          float th;
          const float t = score_to_t<SOFTCAP>(a, s[kb][v], &th);
          float p = BIAS ? fast_exp2(t + __builtin_fmaf(slope2, (float)off, base)) : fast_exp2(t - lse2);
          if constexpr (PARTIAL)
            if (off < lo || off >= hi) p = 0.f;
          float ds = p * (dp[kb][v] - dval);
          if constexpr (SOFTCAP) ds *= 1.0f - th * th;
          d8[e8] = ds;
        }
        dw[t4] = pack8(d8);
      }
    };
    if (ent.meta & 1)
      ds_tile(std::true_type{});
    else
      ds_tile(std::false_type{});

    // ---- dQ^T += K^T dS^T : contraction over the 64 keys
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
        acc[db] = mfma_32x32x16_f16(tr8<D>(kt, tro, db, t4), __builtin_bit_cast(bf16x8, dw[t4]), acc[db]);

    dma_barrier();
  };

  if (e_begin < e_end) {
    issue(e_begin, k_s0, v_s0);
    dma_barrier();
    // whole pairs, then the odd last step: a loop with one exit keeps the
    // accumulators in place (an exit between the two steps made the
    // compiler copy them every turn)
    int e = e_begin;
    for (; e + 1 < e_end; e += 2) {
      step(e, k_s0, v_s0, k_s1, v_s1);
      step(e + 1, k_s1, v_s1, k_s0, v_s0);
    }
    if (e < e_end) step(e, k_s0, v_s0, k_s1, v_s1);
  }

  if (pslot >= 0) {
    // one run of a split q tile: fp32 dQ for bwd_dq_reduce
    float* prow = a.partial + (((int64_t)pslot * a.hq + head) * kDqRows + (row - q0)) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 x;
        x[0] = out_mul * acc[db][4 * j + 0];
        x[1] = out_mul * acc[db][4 * j + 1];
        x[2] = out_mul * acc[db][4 * j + 2];
        x[3] = out_mul * acc[db][4 * j + 3];
        *reinterpret_cast<f32x4*>(prow + 32 * db + 8 * j + 4 * hh) = x;
      }
  } else if (row < a.Tq) {
    __bf16* drow = a.dq + ((int64_t)row * a.hq + head) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w2;
        w2[0] = pack_bf16x2(out_mul * acc[db][4 * j + 0], out_mul * acc[db][4 * j + 1]);
        w2[1] = pack_bf16x2(out_mul * acc[db][4 * j + 2], out_mul * acc[db][4 * j + 3]);
        *reinterpret_cast<u32x2*>(drow + 32 * db + 8 * j + 4 * hh) = w2;
      }
  }
}

// Sum of the fp32 dQ of a split q tile's runs, in run order, to bf16 dQ: one
// 16-byte chunk per thread, kDqReduceParts workgroups per (split tile, head).
template <int D>
constexpr int kDqReduceParts = kDqRows * D / 4 / kThreads;

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_reduce_kernel(BwdArgs a) {
  const int u = blockIdx.x / kDqReduceParts<D>, part = blockIdx.x % kDqReduceParts<D>;
  const int s = u / a.hq, head = u % a.hq;
  if (s >= plan_i32(a.counts, 1)) return;
  const i32x4 sp = const_load<i32x4>(a.splits, s);
  const int qt = sp[0], slot0 = sp[1], ns = sp[2];
  {
    const int i = 4 * (part * kThreads + (int)threadIdx.x);
    const int64_t row = (int64_t)qt * kDqRows + i / D;
    if (row >= a.Tq) return;
    f32x4 sum = f32x4{};
#pragma unroll 4
    for (int c = 0; c < ns; ++c)
      sum += *reinterpret_cast<const f32x4*>(a.partial + ((int64_t)(slot0 + c) * a.hq + head) * kDqRows * D + i);
    u32x2 w;
    w[0] = pack_bf16x2(sum[0], sum[1]);
    w[1] = pack_bf16x2(sum[2], sum[3]);
    *reinterpret_cast<u32x2*>(a.dq + (row * a.hq + head) * D + i % D) = w;
  }
}

void fill_args(const BwdLaunch& p, const BwdWorkspaceLayout& L, BwdArgs* a) {
  unsigned char* ws = static_cast<unsigned char*>(p.workspace);
  a->q = reinterpret_cast<const __bf16*>(ws + L.q16);
  a->k = reinterpret_cast<const __bf16*>(ws + L.k16);
  a->v = nullptr;  // the saved record's fp16 copy of v, set by the launch
  a->dout = reinterpret_cast<const __bf16*>(ws + L.do16);
  a->scales = reinterpret_cast<const float*>(ws + L.range + 16);
  a->lse = p.lse;
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

template <int D, bool SC, bool BIAS>
hipError_t launch_bwd_t(const BwdLaunch& p, hipStream_t stream) {
  const BwdWorkspaceLayout L = bwd_workspace_layout(p.Tq, p.Tk, p.hq, p.hkv, p.d);
  unsigned char* ws = static_cast<unsigned char*>(p.workspace);
  const int64_t rows = p.Tq * p.hq;
  BwdArgs a;
  fill_args(p, L, &a);
  float* dvec = reinterpret_cast<float*>(ws + L.dvec);
  float* lse2 = reinterpret_cast<float*>(ws + L.lse2);
  a.dvec = dvec;
  a.lse2 = lse2;
  a.counts = reinterpret_cast<const int32_t*>(ws + L.counts);
  a.items = reinterpret_cast<const i32x4*>(ws + L.items);
  a.splits = reinterpret_cast<const i32x4*>(ws + L.splits);
  a.partial = reinterpret_cast<float*>(ws + L.partial);
  a.slopes = p.alibi_slopes;
  // ranges: dO's from a pass over it; q's and v's (with v's fp16 copy) come
  // with the saved record; k's from its tracked copy.  Then the fp16 copies
  // of q and dO, D and lse in exp2 units
  const SavedLayout S = saved_layout(p.Tq, p.Tk, p.hq, p.hkv, D);
  const unsigned char* saved = static_cast<const unsigned char*>(p.saved);
  uint32_t* range = reinterpret_cast<uint32_t*>(ws + L.range);
  const int64_t nq = rows * D / 8, nk = p.Tk * p.hkv * D / 8;  // 16-byte chunks
  launch_range_clear(range, 8, stream);
  RangeJob job{};
  job.n = 1;
  job.src[0] = p.dout;
  job.chunks[0] = nq;
  job.word[0] = kRgDO;
  job.words = range;
  launch_range_max(job, stream);
  launch_convert_tracked(p.k, ws + L.k16, nk, reinterpret_cast<uint32_t*>(ws + L.parts), range, kRgK, kRangeK, false,
                         stream);
  {
    // also writes the scales (thread 0), so it runs even without rows
    const int64_t blocks = std::max<int64_t>((nq + kThreads - 1) / kThreads, 1);
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(p.q), static_cast<const u32x4*>(p.out),
                       reinterpret_cast<const u32x4*>(saved + S.out_lo), static_cast<const u32x4*>(p.dout), p.lse,
                       range, reinterpret_cast<const uint32_t*>(saved + S.words),
                       reinterpret_cast<u32x4*>(ws + L.q16), reinterpret_cast<u32x4*>(ws + L.do16), dvec, lse2,
                       reinterpret_cast<float*>(ws + L.range + 16), p.Tq, p.hq);
  }
  a.v = reinterpret_cast<const __bf16*>(saved + S.v16);
  // dK, dV: key tiles cut into runs, one workgroup per (run, kv head), then
  // the sums over the runs of split tiles
  a.row_ptr = p.kv_row_ptr;
  a.entries = reinterpret_cast<const DevEntry*>(p.kv_entries);
  a.order = p.kv_order;
  const int64_t n_kt = (p.Tk + kDkvKeys - 1) / kDkvKeys;
  a.direct = 0;
  if (n_kt > 0 && !split_possible(p.kv_n_entries, p.kv_max_len, a.grp, a.hkv, kDkvMinSteps, kDkvBalance)) {
    // no list can be cut: one workgroup per (key tile, kv head), no reduce
    a.direct = 1;
    a.n_units = (int32_t)n_kt;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, SC, BIAS>), dim3((unsigned)(n_kt * p.hkv)), dim3(kDkvThreads), 0,
                       stream, a);
  } else if (n_kt > 0) {
    SplitLaunch sp;
    sp.row_ptr = p.kv_row_ptr;
    sp.order = p.kv_order;
    sp.n_tiles = n_kt;
    sp.steps_per_entry = a.grp;
    sp.units = a.hkv;
    sp.min_steps = kDkvMinSteps;
    sp.balance = kDkvBalance;
    sp.max_slot_units = kDkvMaxSlots;
    sp.items = ws + L.items;
    sp.items_cap = L.items_cap;
    sp.splits = ws + L.splits;
    sp.splits_cap = L.splits_cap;
    sp.counts = reinterpret_cast<int32_t*>(ws + L.counts);
    launch_split(sp, stream);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, SC, BIAS>), dim3((unsigned)(L.items_cap * p.hkv)), dim3(kDkvThreads), 0,
                       stream, a);
    hipLaunchKernelGGL((bwd_dkdv_reduce_kernel<D>), dim3((unsigned)(L.splits_cap * p.hkv * kDkvReduceParts<D>)),
                       dim3(kThreads), 0,
                       stream, a);
  }
  // dQ: one workgroup per (q tile or run of its list, q head), then the
  // sums over the runs of split q tiles
  a.row_ptr = p.q_row_ptr;
  a.entries = reinterpret_cast<const DevEntry*>(p.q_entries);
  a.order = p.q_order;
  a.counts = reinterpret_cast<const int32_t*>(ws + L.dq_counts);
  a.items = reinterpret_cast<const i32x4*>(ws + L.dq_items);
  a.splits = reinterpret_cast<const i32x4*>(ws + L.dq_splits);
  a.partial = reinterpret_cast<float*>(ws + L.dq_partial);
  const int64_t n_qt = (p.Tq + kDqRows - 1) / kDqRows;
  if (n_qt > 0 && !split_possible(p.q_n_entries, p.q_max_len, 1, p.hq, kDqMinSteps, kDqBalance)) {
    a.direct = 1;
    a.n_units = (int32_t)(n_qt * p.hkv);
    const int64_t n_wg = ((a.n_units + 7) / 8) * 8 * (int64_t)a.grp;
    hipLaunchKernelGGL((bwd_dq_kernel<D, SC, BIAS>), dim3((unsigned)n_wg), dim3(kThreads), 0, stream, a);
  } else if (n_qt > 0) {
    a.direct = 0;
    const SplitCaps caps = split_caps(n_qt, p.hq, kDqBalance);
    SplitLaunch sp;
    sp.row_ptr = p.q_row_ptr;
    sp.order = p.q_order;
    sp.n_tiles = n_qt;
    sp.steps_per_entry = 1;
    sp.units = p.hq;
    sp.min_steps = kDqMinSteps;
    sp.balance = kDqBalance;
    sp.max_slot_units = kDqMaxSlots;
    sp.items = ws + L.dq_items;
    sp.items_cap = caps.items;
    sp.splits = ws + L.dq_splits;
    sp.splits_cap = caps.splits;
    sp.counts = reinterpret_cast<int32_t*>(ws + L.dq_counts);
    launch_split(sp, stream);
    const int64_t n_units = caps.items * p.hkv;
    const int64_t n_wg = ((n_units + 7) / 8) * 8 * (int64_t)a.grp;
    hipLaunchKernelGGL((bwd_dq_kernel<D, SC, BIAS>), dim3((unsigned)n_wg), dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL((bwd_dq_reduce_kernel<D>), dim3((unsigned)(caps.splits * p.hq * kDqReduceParts<D>)),
                       dim3(kThreads), 0,
                       stream, a);
  }
  return hipGetLastError();
}

}  // namespace

int bwd_kv_tile_rows() { return kDkvRows; }
int bwd_kv_tile_cols() { return kDkvKeys; }
int bwd_q_tile_rows() { return kDqRows; }
int bwd_q_tile_cols() { return kDqKeys; }

static size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

BwdWorkspaceLayout bwd_workspace_layout(int64_t Tq, int64_t Tk, int hq, int hkv, int d) {
  BwdWorkspaceLayout L{};
  const int64_t n_kt = Tk > 0 ? (Tk + kDkvKeys - 1) / kDkvKeys : 0;
  const SplitCaps caps = split_caps(n_kt, hkv > 0 ? hkv : 1, kDkvBalance);
  L.items_cap = caps.items;
  L.splits_cap = caps.splits;
  const int64_t slot_heads = kDkvMaxSlots;
  size_t off = 0;
  L.dvec = off;
  off += round256((size_t)(Tq > 0 ? Tq : 0) * (size_t)(hq > 0 ? hq : 0) * sizeof(float));
  L.lse2 = off;
  off += round256((size_t)(Tq > 0 ? Tq : 0) * (size_t)(hq > 0 ? hq : 0) * sizeof(float));
  L.counts = off;
  off += 256;
  L.items = off;
  off += round256((size_t)L.items_cap * 16);
  L.splits = off;
  off += round256((size_t)L.splits_cap * 16);
  L.partial = off;
  if (n_kt > 0) off += (size_t)slot_heads * 2 * kDkvKeys * (size_t)d * sizeof(float);
  // dQ runs: counters, items and split records for the largest caps (one
  // head), fp32 partial dQ for kDqMaxSlots (run, q head) pairs
  const int64_t n_qt = Tq > 0 ? (Tq + kDqRows - 1) / kDqRows : 0;
  const SplitCaps qc = split_caps(n_qt, 1, kDqBalance);
  off = round256(off);
  L.dq_counts = off;
  off += 256;
  L.dq_items = off;
  off += round256((size_t)qc.items * 16);
  L.dq_splits = off;
  off += round256((size_t)qc.splits * 16);
  L.dq_partial = off;
  if (n_qt > 0) off += (size_t)kDqMaxSlots * kDqRows * (size_t)d * sizeof(float);
  // range words and scales of the fp16 copies, the copies of q, dO and k,
  // and the forward re-run's saved record, out and lse
  const size_t nq = (size_t)(Tq > 0 ? Tq : 0) * (size_t)(hq > 0 ? hq : 0) * (size_t)d;
  const size_t nk = (size_t)(Tk > 0 ? Tk : 0) * (size_t)(hkv > 0 ? hkv : 0) * (size_t)d;
  off = round256(off);
  L.range = off;
  off += 256;
  L.parts = off;
  off += round256((size_t)kVRangeParts * 4);
  L.q16 = off;
  off += round256(nq * 2);
  L.do16 = off;
  off += round256(nq * 2);
  L.k16 = off;
  off += round256(nk * 2);
  L.re_saved = off;
  off += round256(saved_layout(Tq, Tk, hq, hkv, d).total);
  L.re_out = off;
  off += round256(nq * 2);
  L.re_lse = off;
  off += round256((size_t)(Tq > 0 ? Tq : 0) * (size_t)(hq > 0 ? hq : 0) * sizeof(float));
  L.total = off;
  return L;
}

template <int D>
hipError_t launch_bwd_d(const BwdLaunch& p, hipStream_t stream) {
  const bool sc = p.softcap > 0.f, bias = p.alibi_slopes != nullptr;
  if (bias) return sc ? launch_bwd_t<D, true, true>(p, stream) : launch_bwd_t<D, false, true>(p, stream);
  return sc ? launch_bwd_t<D, true, false>(p, stream) : launch_bwd_t<D, false, false>(p, stream);
}

hipError_t launch_bwd(const BwdLaunch& p, hipStream_t stream) {
  return p.d == 64 ? launch_bwd_d<64>(p, stream) : launch_bwd_d<128>(p, stream);
}

}  // namespace ffa
