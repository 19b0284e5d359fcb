// Forward kernel of range-masked flash attention for gfx950 (CDNA4).
//
// One workgroup = one (128-row q tile, q head) work item; 4 waves of 64
// lanes, each wave owning 32 query rows.  The workgroup walks the plan's list
// of 64-key tiles for its q tile (the BlockMask-style list of non-masked
// blocks: FlexAttention paper summary, section 4, block sparsity), merging
// every slice that reaches the q tile into one online softmax.
//
// Per k tile, on the matrix cores (bf16 in, fp32 accumulate):
//   S^T = K * Q^T     keys x queries, so each lane holds one query's scores
//   O^T += V^T * P^T  head_dim x queries, P^T taken straight from S^T's registers
// Working with transposed tiles keeps a query row inside one lane (16 keys
// per 32x32 block), so the row max and row sum are in-lane work plus one
// exchange between the two half-waves, and the rescale of O is a per-lane
// scalar.  K and V are staged row-major in LDS, double-buffered so the next
// tile's global loads are in flight while the current tile computes
// (prefetching later KV tiles: same section, data prefetching pipeline); the
// PV contraction runs over keys, so V^T fragments are read with the gfx950
// LDS transpose load (ds_read_b64_tr_b16) instead of transposing in
// registers.  The running max moves only when a row's tile max exceeds it by
// more than 2^8 (in exp2 units), so the O rescale is skipped for most tiles.
// The per-cell mask is evaluated
// only on PARTIAL tiles (full-block optimisation); invisible cells become
// -inf before the softmax (masking P in softmax, as recommended in CUTLASS
// issue #2192 on ex77 varlen handling), and rows past the end of a tensor
// are read as zeros through range-checked buffer loads and never stored.
#include "device_common.hpp"
#include "launch.hpp"

namespace ffa {

namespace {

constexpr int kBM = 128;  // q rows per work item
constexpr int kBN = 64;   // keys per k tile
constexpr int kThreads = 256;

struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* out;
  float* lse;
  const int32_t* row_ptr;   // [n_qtiles + 1]
  const DevEntry* entries;  // grouped by q tile
  const int32_t* order;     // q tiles, longest list first
  const DevSlice* slices;
  int32_t Tq, Tk, hq, hkv, grp;
  int32_t n_units;          // n_qtiles * hkv
  float score_mult;         // exponent multiplier: scale*log2(e), or 1 with softcap
  float cap_in;             // softcap: 2*scale*log2(e)/softcap (tanh argument, see tanh_from_2xlog2e)
  float cap_out;            // softcap: softcap*log2(e)
  float rescale_thr;        // 8 exp2 units in the units of the running max
};

template <int D>
struct FwdSmem {
  static constexpr int kStr = D + 8;      // K row stride (bf16): 16 B pad
  static constexpr int vStr = D + 32;     // V row stride (bf16): 64 B pad, so a transpose read's four rows x 64 B fill the 64 LDS banks
  static constexpr int kBuf = kBN * kStr;
  static constexpr int vBuf = kBN * vStr;
  static constexpr int kElems = 2 * (kBuf + vBuf);
};

// Work-item decode.  Workgroups are handed to the 8 XCDs round-robin
// (wg % 8); all q heads that share a kv head for one q tile go to the same
// XCD on consecutive slots, so the K/V tiles they read are shared in that
// XCD's L2.  Units (q tile, kv head) are spread over XCDs in plan order,
// longest list first.
__device__ __forceinline__ bool decode_item(const FwdArgs& a, int* qt, int* head, int* g) {
  const int wg = blockIdx.x;
  const int xcd = wg & 7, slot = wg >> 3;
  const int r = slot % a.grp;
  const int u = (slot / a.grp) * 8 + xcd;
  if (u >= a.n_units) return false;
  *qt = a.order[u / a.hkv];
  *g = u % a.hkv;
  *head = *g * a.grp + r;
  return true;
}

template <int D>
struct TileLoader {
  // K and V tiles: kBN rows x D, 16-byte chunks spread over the workgroup
  static constexpr int kChunksPerRow = D / 8;
  static constexpr int kLoads = kBN * kChunksPerRow / kThreads;
  static_assert(kLoads * kThreads == kBN * kChunksPerRow, "tile must split evenly");

  u32x4 kreg[kLoads];
  u32x4 vreg[kLoads];

  __device__ __forceinline__ void load(const FwdArgs& a, int ktile, int g, int tid) {
    const int64_t row_bytes = (int64_t)a.hkv * D * 2;
    const int64_t k0 = (int64_t)ktile * kBN;
    const int64_t base_off = (k0 * a.hkv + g) * D;
    const int64_t valid = ((int64_t)a.Tk - k0) * row_bytes - (int64_t)g * D * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + base_off, valid);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + base_off, valid);
#pragma unroll
    for (int c = 0; c < kLoads; ++c) {
      const int idx = tid + kThreads * c;
      const int row = idx / kChunksPerRow, col = idx % kChunksPerRow;
      const uint32_t off = (uint32_t)(row * row_bytes + col * 16);
      kreg[c] = buf_load16(rk, off);
      vreg[c] = buf_load16(rv, off);
    }
  }

  __device__ __forceinline__ void store(__bf16* kl, __bf16* vl, int tid) {
#pragma unroll
    for (int c = 0; c < kLoads; ++c) {
      const int idx = tid + kThreads * c;
      const int row = idx / kChunksPerRow, col = idx % kChunksPerRow;
      *reinterpret_cast<u32x4*>(kl + row * FwdSmem<D>::kStr + col * 8) = kreg[c];
      *reinterpret_cast<u32x4*>(vl + row * FwdSmem<D>::vStr + col * 8) = vreg[c];
    }
  }
};

// Transpose read of a row-major tile: in each 16-lane group, lane i receives
// element i % 4 of the 8-byte chunks addressed by lanes 4r + i / 4, r = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const __bf16* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(const_cast<__bf16*>(p)));
  return __builtin_bit_cast(u32x2, r);
}

template <int D, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(FwdArgs a) {
  using Smem = FwdSmem<D>;
  constexpr int KS = D / 16;  // k steps of the QK^T contraction
  constexpr int DB = D / 32;  // 32-wide blocks of the head dim in O^T
  __shared__ __attribute__((aligned(16))) __bf16 smem[Smem::kElems];

  int qt, head, g;
  if (!decode_item(a, &qt, &head, &g)) return;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, n = lane & 31, hh = lane >> 5;
  const int q0 = qt * kBM;
  const int row = q0 + w * 32 + n;  // the query row this lane's column holds
  const int64_t q_row_bytes = (int64_t)a.hq * D * 2;

  // Q fragments (B operand of S^T = K Q^T): lane (n, hh) holds row `row`,
  // dims 16*ks + 8*hh .. +8
  bf16x8 qf[KS];
  {
    const int64_t wrow0 = q0 + w * 32;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(
        a.q + (wrow0 * a.hq + head) * D, ((int64_t)a.Tq - wrow0) * q_row_bytes - (int64_t)head * D * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(n * q_row_bytes + (16 * ks + 8 * hh) * 2)));
  }

  const int e_begin = a.row_ptr[qt], e_end = a.row_ptr[qt + 1];

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};
  float m_run = -INFINITY;  // running row max, in the units fed to score_mult
  float l_part = 0.f;       // this half-wave's share of the row sum

  TileLoader<D> ld;
  if (e_begin < e_end) {
    ld.load(a, a.entries[e_begin].tile, g, tid);
    ld.store(smem, smem + Smem::kBuf, tid);
  }
  __syncthreads();

  for (int e = e_begin; e < e_end; ++e) {
    const int buf = (e - e_begin) & 1;
    const __bf16* kl = smem + buf * (Smem::kBuf + Smem::vBuf);
    const __bf16* vl = kl + Smem::kBuf;
    const DevEntry ent = a.entries[e];
    const bool has_next = e + 1 < e_end;
    if (has_next) ld.load(a, a.entries[e + 1].tile, g, tid);

    // ---- S^T = K Q^T : two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + (32 * b + n) * Smem::kStr + 16 * ks + 8 * hh);
        s[b] = mfma_32x32x16(kf, qf[ks], s[b]);
      }
    }

    // ---- softcap, then mask (a capped -inf would come back finite)
    if constexpr (SOFTCAP) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[b][v] = a.cap_out * tanh_from_2xlog2e(s[b][v] * a.cap_in);
    }
    if (ent.meta & 1) {
      const DevSlice sl = a.slices[ent.meta >> 1];
      const int k0 = ent.tile * kBN;
      int lo = sl.ks, hi = sl.ke;
      if (sl.causal) hi = min(hi, row + 1 + (sl.ke - sl.qe));
      if (row < sl.qs || row >= sl.qe) hi = lo;  // row outside the slice: nothing visible
      lo -= k0 + 4 * hh;
      hi -= k0 + 4 * hh;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int off = 32 * b + 8 * (v >> 2) + (v & 3);
          if (off < lo || off >= hi) s[b][v] = -INFINITY;
        }
    }

    // ---- online softmax (row = this lane's column; other half-wave holds the rest)
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[b][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // move the running max only when this tile's max exceeds it by more than
    // 2^8 in exp2 units (all lanes together, so the branch is uniform); until
    // then exp2 values stay <= 2^8 and O, l need no rescale
    if (__builtin_amdgcn_ballot_w64(mx > m_run + a.rescale_thr) != 0) {
      const float m_new = fmaxf(m_run, mx);
      // rows whose max does not move keep their scale (this also covers rows
      // that have seen nothing yet: -inf - -inf would be NaN); a row whose
      // first visible key arrives gets exp2(-inf) = 0
      const float alpha = (m_new == m_run) ? 1.0f : fast_exp2((m_run - m_new) * a.score_mult);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    const float neg = (m_run == -INFINITY) ? 0.f : -m_run * a.score_mult;
    // exp2 weights; the row sum is taken in fp32 on the unrounded values (the
    // lse must hold to 1e-3 even for rows with a handful of keys), in four
    // independent chains
    bf16x8 pf[4];
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int b = t >> 1, h8 = (t & 1) * 8;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const float p = fast_exp2(__builtin_fmaf(s[b][h8 + e8], a.score_mult, neg));
        rs[e8 & 3] += p;
        pf[t][e8] = (__bf16)p;
      }
    }
    l_part += (rs[0] + rs[1]) + (rs[2] + rs[3]);

    // ---- O^T += V^T P^T : four k-steps of 16 keys; A = V^T by transpose reads
    {
      const int g16 = lane >> 4, sl = lane & 15;
      const int col = 16 * (g16 & 1) + 4 * (sl & 3);
      const int krow = 4 * hh + (sl >> 2);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int kb = 32 * (t >> 1) + 16 * (t & 1) + krow;
          const __bf16* vp = vl + kb * Smem::vStr + 32 * db + col;
          const u32x2 lo4 = lds_read_tr16(vp);
          const u32x2 hi4 = lds_read_tr16(vp + 8 * Smem::vStr);
          u32x4 av;
          av[0] = lo4[0]; av[1] = lo4[1]; av[2] = hi4[0]; av[3] = hi4[1];
          o[db] = mfma_32x32x16(__builtin_bit_cast(bf16x8, av), pf[t], o[db]);
        }
    }

    if (has_next) {
      __bf16* nk = smem + (buf ^ 1) * (Smem::kBuf + Smem::vBuf);
      ld.store(nk, nk + Smem::kBuf, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: normalise once in fp32, round to bf16 once
  const float l = l_part + __shfl_xor(l_part, 32);
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  if (row < a.Tq) {
    __bf16* orow = a.out + ((int64_t)row * a.hq + head) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w2;
        w2[0] = pack_bf16x2(o[db][4 * j + 0] * inv, o[db][4 * j + 1] * inv);
        w2[1] = pack_bf16x2(o[db][4 * j + 2] * inv, o[db][4 * j + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * j + 4 * hh) = w2;
      }
    if (hh == 0) {
      const float lse = l > 0.f ? (m_run * a.score_mult + fast_log2(l)) * 0.69314718055994531f : -INFINITY;
      a.lse[(int64_t)row * a.hq + head] = lse;
    }
  }
}

template <int D, bool SC>
hipError_t launch_fwd_t(const FwdLaunch& p, hipStream_t stream) {
  FwdArgs a;
  a.q = static_cast<const __bf16*>(p.q);
  a.k = static_cast<const __bf16*>(p.k);
  a.v = static_cast<const __bf16*>(p.v);
  a.out = static_cast<__bf16*>(p.out);
  a.lse = p.lse;
  a.row_ptr = p.row_ptr;
  a.entries = reinterpret_cast<const DevEntry*>(p.entries);
  a.order = p.order;
  a.slices = reinterpret_cast<const DevSlice*>(p.slices);
  a.Tq = (int32_t)p.Tq;
  a.Tk = (int32_t)p.Tk;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.grp = p.hq / p.hkv;
  const int64_t n_qt = (p.Tq + kBM - 1) / kBM;
  a.n_units = (int32_t)(n_qt * p.hkv);
  const float log2e = 1.4426950408889634f;
  if (SC) {
    a.score_mult = 1.0f;
    a.cap_in = 2.0f * p.scale * log2e / p.softcap;
    a.cap_out = p.softcap * log2e;
  } else {
    a.score_mult = p.scale * log2e;
    a.cap_in = a.cap_out = 0.f;
  }
  a.rescale_thr = 8.0f / a.score_mult;
  const int64_t n_wg = ((a.n_units + 7) / 8) * 8 * (int64_t)a.grp;
  if (n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_kernel<D, SC>), dim3((unsigned)n_wg), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int fwd_tile_rows() { return kBM; }
int fwd_tile_cols() { return kBN; }

hipError_t launch_fwd(const FwdLaunch& p, hipStream_t stream) {
  const bool sc = p.softcap > 0.f;
  if (p.d == 64) return sc ? launch_fwd_t<64, true>(p, stream) : launch_fwd_t<64, false>(p, stream);
  return sc ? launch_fwd_t<128, true>(p, stream) : launch_fwd_t<128, false>(p, stream);
}

}  // namespace ffa
