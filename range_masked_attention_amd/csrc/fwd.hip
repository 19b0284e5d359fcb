// Forward kernel of range-masked flash attention for gfx950 (CDNA4).
//
// One workgroup = one (128-row q tile, q head) work item; 4 waves of 64
// lanes, each wave owning 32 query rows.  The workgroup walks the plan's list
// of 64-key tiles for its q tile (the BlockMask-style list of non-masked
// blocks: FlexAttention paper summary, section 4, block sparsity), merging
// every slice that reaches the q tile into one online softmax.  A list much
// longer than the average is cut into runs (split.hip), each walked by its
// own workgroup, and fwd_combine merges the runs' outputs by their lse.
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
//
// Optional distance bias (ALiBi: a bias that depends on the distance between
// query and key positions, FlexAttention paper summary, section 2 and
// section 3.1): score += slope[head] * (j - i) after the softcap.  Without
// softcap the bias, in raw score units, is the initial value of the S^T
// accumulator, so everything after the QK product is unchanged; with softcap
// it is folded into the cap's final multiply.  j - i is formed in integers
// (a per-lane base per tile plus a compile-time offset per register), so
// the only rounding is that of slope * (j - i).
#include <type_traits>

#include <cstdlib>
#include <cstring>

#include "device_common.hpp"
#include "launch.hpp"

namespace ffa {

namespace {

constexpr int kBM = 128;  // q rows per work item
constexpr int kBN = 64;   // keys per k tile
constexpr int kThreads = 256;

// Long q-tile lists (a short query block against a long context, global
// query rows) are cut into runs by the split pass (split.hip): lists longer
// than one resident workgroup slot's share of the work (kFwdBalance = the
// 512 slots of two workgroups per CU) are cut into runs of at most that
// share, each of at least kFwdMinSteps key tiles; balanced lists (the
// longest-first order already spreads them) stay whole.  Runs of a split tile write their own
// normalised output and lse in fp32, and fwd_combine merges them by their
// lse in run order.  The plan holds the scratch (fwd_scratch_layout), sized
// for kFwdMaxSlots (run, q head) pairs.
constexpr int kFwdBalance = 512;
constexpr int kFwdMinSteps = 64;
constexpr int kFwdMaxSlots = 512;
constexpr int kFwdMaxD = 128;
// Two q heads per workgroup only with at least this many such workgroups
// (two per CU): with fewer the chip is better filled one head each.
constexpr int64_t kFwdPairMinWorkgroups = 512;

struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* out;
  float* lse;
  __bf16* out_lo;           // rounding residual of out (training forward), or null
  const uint32_t* v_words;  // range words of v (v is its fp16 copy times the scale they give)
  uint32_t* q_range;        // training forward: the record's word for max |q| (kRgQ), or null
  const DevEntry* entries;  // grouped by q tile
  const DevSlice* slices;
  const int32_t* row_ptr;   // [n_qtiles + 1]
  const int32_t* order;     // q tiles, longest list first
  int32_t direct;           // 1: one item per q tile, taken from the plan itself
  int32_t n_units;          // direct: n_qtiles * hkv
  const i32x4* items;       // runs of q-tile lists, in plan order (split.hip)
  const i32x4* splits;      // q tiles cut into several runs
  const int32_t* counts;    // [0] items, [1] split tiles
  float* partial_o;         // [slot][hq][kBM][D] normalised output of one run
  float* partial_lse;       // [slot][hq][kBM] its lse (natural log)
  int32_t Tq, Tk, hq, hkv, grp;
  float score_mult;         // exponent multiplier: scale*log2(e), or 1 with softcap
  float cap_in;             // softcap: 2*scale*log2(e)/softcap (tanh argument, see tanh_from_2xlog2e)
  float cap_out;            // softcap: softcap*log2(e)
  float rescale_thr;        // 8 exp2 units in the units of the running max
  const float* slopes;      // [hq] distance-bias slopes (biased kernels only)
  float bias_mult;          // slope to running-max units: 1/scale, or log2(e) with softcap
};

// LDS tiles are unpadded kBN x D bf16, filled by direct-to-LDS loads; 16-byte
// chunks are XOR-swizzled within each row so the reads below hit all 64
// banks: K (row-major reads of one chunk by 16 rows) uses slot = chunk ^
// (row & 15) (d = 128) or ^ ((row >> 1) & 7) (d = 64); V (transpose reads of
// 4 rows x 64 bytes per half-wave) uses slot = chunk ^ 4 (row & 3) (d = 128)
// or ^ 4 ((row >> 1) & 1) (d = 64).
template <int D>
struct FwdSmem {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                 // 16-byte chunks per row
  static constexpr int kTileBytes = kBN * kRowBytes;
  static constexpr int kElems = 4 * kTileBytes / 2;     // K[2], V[2]
  __device__ __forceinline__ static int k_swz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  __device__ __forceinline__ static int v_swz(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
};

// Work-item decode.  Workgroups are handed to the 8 XCDs round-robin
// (wg % 8); all q heads that share a kv head for one run go to the same XCD
// on consecutive slots, so the K/V tiles they read are shared in that XCD's
// L2.  Units (run, kv head) are spread over XCDs in plan order, longest list
// first.  A workgroup takes hpw consecutive q heads; `head` is the first.
struct FwdItem {
  int qt, head, g, e_begin, e_end, slot;
};
__device__ __forceinline__ bool decode_item(const FwdArgs& a, int hpw, FwdItem* it) {
  const int wg = blockIdx.x;
  const int xcd = wg & 7, slot = wg >> 3;
  const int wgs = a.grp / hpw;  // workgroups per (run, kv head): hpw q heads each
  const int r = slot % wgs;
  const int u = (slot / wgs) * 8 + xcd;
  const int item = u / a.hkv;
  if (a.direct) {
    if (u >= a.n_units) return false;
    it->qt = plan_i32(a.order, item);
    it->e_begin = plan_i32(a.row_ptr, it->qt);
    it->e_end = plan_i32(a.row_ptr, it->qt + 1);
    it->slot = -1;
  } else {
    if (item >= plan_i32(a.counts, 0)) return false;
    const i32x4 run = const_load<i32x4>(a.items, item);
    it->qt = run[0];
    it->e_begin = run[1];
    it->e_end = run[2];
    it->slot = run[3];
  }
  it->g = u % a.hkv;
  it->head = it->g * a.grp + hpw * r;
  return true;
}

// Direct-to-LDS tile loads: lane L of a load instruction writes 16 bytes at
// the instruction's LDS base + 16 L; each lane fetches the global chunk that
// belongs at that slot under the swizzle.  Rows past the end of the tensor
// read as zeros (buffer range check).
template <int D, int NT>
struct TileDma {
  using Smem = FwdSmem<D>;
  static constexpr int kPerThread = kBN * Smem::kChunks / NT;  // 16-byte loads per thread
  static constexpr int kRowsPerLoad = 64 / Smem::kChunks;      // rows one wave load covers
  static_assert(kPerThread * NT == kBN * Smem::kChunks, "tile must split evenly");

  // Load c of wave w: lane L fills chunk slot P = (w * kPerThread + c) * 64 + L,
  // i.e. row (w * kPerThread + c) * kRowsPerLoad + L / kChunks, slot L % kChunks.
  // The swizzle of that row depends on L and c only through row bits that
  // L / kChunks and c set without carries, so the global offset splits into a
  // per-lane part and a wave-uniform part.
  uint32_t lane_row_bytes;  // (L / kChunks) * row_bytes
  int lane_slot, lane_row;  // L % kChunks, L / kChunks
  uint32_t row_bytes, tile_bytes;
  // this workgroup's kv head: first row of K and V, and the bytes from there
  // to the end of the tensor; a tile's resource starts at its first row
  const char* kbase;
  const char* vbase;
  int64_t bytes;

  __device__ __forceinline__ void init(const FwdArgs& a, int g, int lane) {
    lane_slot = lane % Smem::kChunks;
    lane_row = lane / Smem::kChunks;
    row_bytes = (uint32_t)a.hkv * D * 2;
    tile_bytes = kBN * row_bytes;
    lane_row_bytes = (uint32_t)lane_row * row_bytes;
    kbase = reinterpret_cast<const char*>(a.k + (int64_t)g * D);
    vbase = reinterpret_cast<const char*>(a.v + (int64_t)g * D);
    bytes = (int64_t)a.Tk * row_bytes - (int64_t)g * D * 2;
  }
  template <bool IS_K>
  __device__ __forceinline__ void load(int ktile, __bf16* dst, int w) const {
    const int64_t t0 = (int64_t)(uint32_t)ktile * tile_bytes;
    const __amdgpu_buffer_rsrc_t r = make_rsrc((IS_K ? kbase : vbase) + t0, bytes - t0);
#pragma unroll
    for (int c = 0; c < kPerThread; ++c) {
      const int row0 = (w * kPerThread + c) * kRowsPerLoad;  // wave-uniform
      const int row = row0 + lane_row;
      const int swz = IS_K ? Smem::k_swz(row) : Smem::v_swz(row);
      const uint32_t off = (uint32_t)row0 * row_bytes + lane_row_bytes + (uint32_t)((lane_slot ^ swz) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(dst + (w * kPerThread + c) * 512), 16, off, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void load_k(int ktile, __bf16* dst, int w) const { load<true>(ktile, dst, w); }
  __device__ __forceinline__ void load_v(int ktile, __bf16* dst, int w) const { load<false>(ktile, dst, w); }
};

// Transpose read of a row-major tile: in each 16-lane group, lane i receives
// element i % 4 of the 8-byte chunks addressed by lanes 4r + i / 4, r = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const __bf16* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(const_cast<__bf16*>(p)));
  return __builtin_bit_cast(u32x2, r);
}

// Key offset (from the tile's first key + 4 hh) of register v of block b
// in the S^T layout: 32 b + 8 (v / 4) + v % 4.
__device__ __forceinline__ constexpr int key_off(int b, int v) { return 32 * b + 8 * (v >> 2) + (v & 3); }

// sigma * (j - i) for this lane's 32 cells of tile `ktile`: d0 = 4 hh - row.
__device__ __forceinline__ void bias_tile(float sigma, int ktile, int d0, f32x16* s) {
  const float base = sigma * (float)(ktile * kBN + d0);
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) s[b][v] = __builtin_fmaf(sigma, (float)key_off(b, v), base);
}

// S^T = K Q^T for one 64-key tile: two 32-key blocks.  Lane (n, hh) reads
// row 32b + n, logical chunk 2ks + hh.  With INIT the accumulators start
// from s (the distance bias), else from zero.
template <int D, bool INIT = false>
__device__ __forceinline__ void qk_tile(const __bf16* kl, const bf16x8* qf, int n, int hh, f32x16* s) {
  using Smem = FwdSmem<D>;
  const int swz = Smem::k_swz(n);  // rows n and 32 + n share it
  if constexpr (!INIT) {
    s[0] = f32x16{};
    s[1] = f32x16{};
  }
  // the two blocks' accumulator chains take turns
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int byte = (32 * b + n) * Smem::kRowBytes + (((2 * ks + hh) ^ swz) * 16);
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(kl) + byte);
      s[b] = mfma_32x32x16(kf, qf[ks], s[b]);
    }
}

// Softcap in exp2 units: cap*log2(e) * tanh(scale * s / cap), plus with BIAS
// sigma * (j - i) (sigma in exp2 units; see bias_tile).
// cap_out tanh(x) = cap_out - 2 cap_out r with r = 1 / (2^y + 1).  With the
// bias, the capped score is formed here (the bias joins the constant term).
// Without it the tile keeps r itself: the capped score falls as r grows, so
// the row max comes from the row min of r (capped_max), invisible cells hold
// r = +inf, and the exp2 weight takes one multiply-add of r, which also
// subtracts the running max.
template <bool BIAS>
__device__ __forceinline__ void softcap_tile(const FwdArgs& a, f32x16* s, float sigma, int ktile, int d0) {
  const float base = (BIAS ? sigma * (float)(ktile * kBN + d0) : 0.f) + a.cap_out;
  const float m2 = -2.0f * a.cap_out;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float r = fast_rcp(fast_exp2(s[b][v] * a.cap_in) + 1.0f);
      if constexpr (BIAS)
        s[b][v] = __builtin_fmaf(m2, r, __builtin_fmaf(sigma, (float)key_off(b, v), base));
      else
        s[b][v] = r;
    }
}

// Row max over this lane's 32 scores and the other half-wave's 32 (the
// halves trade their partial maxima by a lane swap, not through LDS).
__device__ __forceinline__ float tile_max(const f32x16* s) {
  float mx = -INFINITY;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[b][v]);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// The same row max for a tile that holds softcap's r (no bias): the capped
// score cap_out - 2 cap_out r of the smallest r (a row with no visible cell
// has r = +inf everywhere and gets -inf).
__device__ __forceinline__ float capped_max(const f32x16* s, float cap_out) {
  float mn = INFINITY;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) mn = fminf(mn, s[b][v]);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
  mn = fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  return __builtin_fmaf(-2.0f * cap_out, mn, cap_out);
}

// Invisible cells of a PARTIAL tile become `hidden` (cell (row, key) of
// slice sl): -inf for scores, +inf for softcap's r.
__device__ __forceinline__ void mask_tile(const DevSlice& sl, int ktile, int row, int hh, f32x16* s,
                                          float hidden) {
  int lo = sl.ks, hi = sl.ke;
  if (sl.causal) hi = min(hi, row + 1 + (sl.ke - sl.qe));
  if (row < sl.qs || row >= sl.qe) hi = lo;  // row outside the slice: nothing visible
  const int base = ktile * kBN + 4 * hh;
  lo -= base;
  hi -= base;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int off = 32 * b + 8 * (v >> 2) + (v & 3);
      if (off < lo || off >= hi) s[b][v] = hidden;
    }
}

// P V on fp16 operands: v is the fp16 copy of v times its scale s_v (made
// before the kernel, see launch_fwd_t), P enters the product in fp16 (11
// significant bits instead of bf16's 8), and the epilogue divides by s_v as
// well.  Each weight enters P V rounded (relative error up to half an ulp)
// while the row sum that divides out is of the unrounded weights, so out can
// be off by up to that half ulp times max |v|: 2^-12 with fp16 P, where
// bf16's 2^-9 would, with out's own rounding, come near 2e-2 for |v| around 6.
//
// HPW q heads of one kv head per workgroup (four waves each, on the same q
// tile): the heads share every K and V tile fetched into LDS, which halves
// the fetches per product when two heads share a kv head.
template <int D, bool SOFTCAP, bool BIAS, int HPW>
__global__ __launch_bounds__(kThreads * HPW, 2) void fwd_kernel(FwdArgs a) {
  using Smem = FwdSmem<D>;
  constexpr int KS = D / 16;  // k steps of the QK^T contraction
  constexpr int DB = D / 32;  // 32-wide blocks of the head dim in O^T
  constexpr int kTileElems = Smem::kTileBytes / 2;
  // score tiles hold softcap's r in place of the capped score
  constexpr bool RCAP = SOFTCAP && !BIAS;
  // K and V double buffers as separate LDS objects: the compiler can then
  // tell a direct-to-LDS fetch into one buffer from reads of another and
  // does not make those reads wait for the fetch
  __shared__ __attribute__((aligned(1024))) __bf16 kb0[kTileElems];
  __shared__ __attribute__((aligned(1024))) __bf16 kb1[kTileElems];
  __shared__ __attribute__((aligned(1024))) __bf16 vb0[kTileElems];
  __shared__ __attribute__((aligned(1024))) __bf16 vb1[kTileElems];

  FwdItem item;
  if (!decode_item(a, HPW, &item)) return;
  const int tid = threadIdx.x;
  // w: wave of the workgroup (its share of each tile fetch); wq: its 32
  // rows of the q tile, for head item.head + w / 4
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, n = lane & 31, hh = lane >> 5;
  const int wq = w & 3;
  const int qt = item.qt, head = item.head + (w >> 2), g = item.g;
  const int q0 = qt * kBM;
  const int row = q0 + wq * 32 + n;  // the query row this lane's column holds
  const int64_t q_row_bytes = (int64_t)a.hq * D * 2;

  // Q fragments (B operand of S^T = K Q^T): lane (n, hh) holds row `row`,
  // dims 16*ks + 8*hh .. +8
  bf16x8 qf[KS];
  {
    const int64_t wrow0 = q0 + wq * 32;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(
        a.q + (wrow0 * a.hq + head) * D, ((int64_t)a.Tq - wrow0) * q_row_bytes - (int64_t)head * D * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(n * q_row_bytes + (16 * ks + 8 * hh) * 2)));
  }
  // the training forward also leaves max |q| in its record for the
  // backward's fp16 copy of q (every q row is loaded by some wave; rows past
  // the end load as 0): the largest bf16 magnitude bits, one atomic per wave
  if (a.q_range) {
    uint32_t m = 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 w4 = __builtin_bit_cast(u32x4, qf[ks]);
#pragma unroll
      for (int j = 0; j < 4; ++j) m = max(m, max(w4[j] & 0x7FFFu, (w4[j] >> 16) & 0x7FFFu));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    if (lane == 0 && m) atomicMax(&a.q_range[kRgQ], m << 16);
  }

  const int e_begin = item.e_begin, e_end = item.e_end;
  const int n_tiles = e_end - e_begin;
  // distance bias: slope of this head in running-max units, and j - i of
  // this lane's first cell minus the tile's first key
  const float sigma = BIAS ? const_load<float>(a.slopes, head) * a.bias_mult : 0.f;
  const int d0 = 4 * hh - row;
  // tile j of the walk.  With a positive slope the bias grows with the key,
  // so the list is walked from its last key tile down: the first tiles then
  // set the running max and later ones rarely move it (walked upwards, every
  // tile would raise the max by slope * 64 and force a rescale of O)
  // (one direction for the workgroup: that of its first head)
  const bool down = BIAS && (HPW == 1 ? sigma > 0.f : const_load<float>(a.slopes, item.head) > 0.f);
  auto entry = [&](int j) { return plan_entry(a.entries, down ? e_end - 1 - j : e_begin + j); };
  // S^T of a tile: accumulators start from the bias (no softcap), or the
  // bias joins the softcap
  auto scores = [&](const __bf16* kl, int ktile, f32x16* s) {
    if constexpr (BIAS && !SOFTCAP) {
      bias_tile(sigma, ktile, d0, s);
      qk_tile<D, true>(kl, qf, n, hh, s);
    } else {
      qk_tile<D>(kl, qf, n, hh, s);
    }
    if constexpr (SOFTCAP) softcap_tile<BIAS>(a, s, sigma, ktile, d0);
  };
  auto row_max = [&](const f32x16* s) {
    if constexpr (RCAP)
      return capped_max(s, a.cap_out);
    else
      return tile_max(s);
  };

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};
  float m_run = -INFINITY;  // running row max, in the units fed to score_mult
  float l4[4] = {0.f, 0.f, 0.f, 0.f};  // this half-wave's share of the row sum, four chains

  // V^T fragments by transpose reads: lane (group g16, index sl) points at
  // key row v_krow (+ block offsets), 4 dims at v_col
  const int g16 = lane >> 4, sl16 = lane & 15;
  const int v_col = 16 * (g16 & 1) + 4 * (sl16 & 3);
  const int v_krow = 4 * hh + (sl16 >> 2);
  const int v_sw = Smem::v_swz(v_krow);  // every key row read by this lane shares it

  if (n_tiles > 0) {
    TileDma<D, kThreads * HPW> dma;
    dma.init(a, g, lane);
    // ---- prologue: K0, V0 and K1 in LDS; S0 and its row max
    dma.load_k(entry(0).tile, kb0, w);
    dma.load_v(entry(0).tile, vb0, w);
    if (n_tiles > 1) dma.load_k(entry(1).tile, kb1, w);
    dma_barrier();
    f32x16 sa[2], sb[2];
    scores(kb0, entry(0).tile, sa);
    float mx_cur = row_max(sa);
    // entries of walk positions j, j + 1 and j + 2 for step j (positions
    // past the end of the list repeat its last entry).  Later entries arrive
    // by vector loads issued with a step's fetches, so the step's closing
    // wait for those fetches covers them; a scalar load of the plan would be
    // waited for inside the step, which also drains the LDS reads in flight,
    // and it misses the scalar cache every few steps.
    DevEntry e0 = entry(0);
    DevEntry e1 = entry(min(1, n_tiles - 1));
    DevEntry e2 = entry(min(2, n_tiles - 1));
    const __amdgpu_buffer_rsrc_t ers = make_rsrc(a.entries, (int64_t)e_end * 8);
    __syncthreads();  // K0's buffer is refilled in the first step

    // One pipeline step on tile j whose scores are in s_cur.  K_j sits in
    // kcur (already consumed), K_{j+1} in knext, V_j in vcur; V_{j-1}'s
    // buffer is vnext.  With MORE, tile j+1 exists: its scores go to s_next.
    auto step = [&](int j, f32x16* s_cur, f32x16* s_next, __bf16* kcur, const __bf16* knext,
                    const __bf16* vcur, __bf16* vnext, auto more_tag) {
      constexpr bool MORE = decltype(more_tag)::value;
      // ---- tile j: mask (PARTIAL only) and the running max
      const DevEntry ent = e0;
      if (ent.meta & 1) {
        mask_tile(plan_slice(a.slices, ent.meta >> 1), ent.tile, row, hh, s_cur, RCAP ? INFINITY : -INFINITY);
        mx_cur = row_max(s_cur);
      }
      // move the running max only when this tile's max exceeds it by more
      // than 2^8 in exp2 units (all lanes together, so the branch is
      // uniform); until then exp2 values stay <= 2^8 and O, l keep their scale
      if (__builtin_amdgcn_ballot_w64(mx_cur > m_run + a.rescale_thr) != 0) {
        const float m_new = fmaxf(m_run, mx_cur);
        // rows whose max does not move keep their scale (this also covers
        // rows that have seen nothing yet: -inf - -inf would be NaN); a row
        // whose first visible key arrives gets exp2(-inf) = 0
        const float alpha = (m_new == m_run) ? 1.0f : fast_exp2((m_run - m_new) * a.score_mult);
#pragma unroll
        for (int i = 0; i < 4; ++i) l4[i] *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) o[i] *= alpha;
        m_run = m_new;
      }
      const float neg = (m_run == -INFINITY) ? 0.f : -m_run * a.score_mult;
      // exp2 argument: score * score_mult - m_run * score_mult, or with r,
      // cap_out - 2 cap_out r - m_run (score_mult is 1 with softcap)
      const float p_mult = RCAP ? -2.0f * a.cap_out : a.score_mult;
      const float p_add = RCAP ? a.cap_out + neg : neg;

      // ---- A: S_{j+1} = K_{j+1} Q^T on the matrix cores, while
      //      B: the VALU turns tile j into exp2 weights
      // (raised wave priority: the other workgroup's wave on this SIMD gets
      // the issue slots this phase leaves)
      i32x2 ev;
      if constexpr (MORE) {
        __builtin_amdgcn_s_setprio(1);
        // entry of walk position j + 3, then direct loads for later tiles,
        // K two ahead and V one ahead, issued among the QK products (the
        // schedule below spreads them); past the last tile the K fetch
        // reloads the last tile into a buffer nobody reads again, so every
        // step issues the same loads
        const int x3 = min(j + 3, n_tiles - 1);
        ev = __builtin_amdgcn_raw_buffer_load_b64(ers, 0, (down ? e_end - 1 - x3 : e_begin + x3) * 8, 0);
        dma.load_k(e2.tile, kcur, w);
        const int next_tile = e1.tile;
        dma.load_v(next_tile, vnext, w);
        if constexpr (BIAS && !SOFTCAP) {
          bias_tile(sigma, next_tile, d0, s_next);
          qk_tile<D, true>(knext, qf, n, hh, s_next);
        } else {
          qk_tile<D>(knext, qf, n, hh, s_next);
        }
      }
      // fp32 sum of the unrounded weights (the lse must hold to 1e-3 even
      // for rows with a handful of keys), four independent chains.  (Summing
      // the fp16-rounded weights two at a time with v_dot2_f32_f16 would do
      // for the lse, but measured slower than these adds.)
      u32x4 pw[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int b = t >> 1, h8 = (t & 1) * 8;
        float p[8];
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          p[e8] = fast_exp2(__builtin_fmaf(s_cur[b][h8 + e8], p_mult, p_add));
          l4[e8 & 3] += p[e8];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[t][i] = pack_f16x2(p[2 * i], p[2 * i + 1]);
      }

      if constexpr (MORE) {
        // Instruction order for the block above: the K reads run 4 ahead of
        // the QK products, and the softmax VALU fills the shadow of each MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          if (i < 2 * TileDma<D, kThreads * HPW>::kPerThread + 1)
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // entry load, direct-to-LDS fetches
          if (i < 12) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, SOFTCAP ? 5 : 7, 0);  // VALU
        }
        __builtin_amdgcn_s_setprio(0);
      }
      // ---- C: O^T += V_j^T P_j^T (V^T fragments by transpose reads), while
      //      B': softcap and the unmasked row max of tile j+1
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int kb = 32 * (t >> 1) + 16 * (t & 1) + v_krow;
          const int col_byte = 2 * (32 * db + v_col);
          const int byte = kb * Smem::kRowBytes + (((col_byte >> 4) ^ v_sw) << 4) + (col_byte & 15);
          const __bf16* vp = reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(vcur) + byte);
          const u32x2 lo4 = lds_read_tr16(vp);
          const u32x2 hi4 = lds_read_tr16(vp + 8 * D);
          u32x4 av;
          av[0] = lo4[0]; av[1] = lo4[1]; av[2] = hi4[0]; av[3] = hi4[1];
          o[db] = mfma_32x32x16_f16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, pw[t]), o[db]);
        }
      if constexpr (MORE) {
        if constexpr (SOFTCAP) softcap_tile<BIAS>(a, s_next, sigma, e1.tile, d0);
        mx_cur = row_max(s_next);
        // Instruction order for the block above: the V transpose reads run 8
        // ahead of the PV products, with the row max of the next tile in
        // their shadows.
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // DS read
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < 12) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, SOFTCAP ? 8 : 2, 0);
        }
        // K_{j+2}, V_{j+1} and the entry have landed, and every wave is done
        // reading K_{j+1} and V_j, whose buffers the next steps refill
        dma_barrier();
        e0 = e1;
        e1 = e2;
        e2.tile = __builtin_amdgcn_readfirstlane(ev[0]);
        e2.meta = __builtin_amdgcn_readfirstlane(ev[1]);
      }
    };
    using More = std::integral_constant<bool, true>;
    using Last = std::integral_constant<bool, false>;

    // steady state in pairs, so the two score arrays and the buffer roles
    // alternate without copies
    int j = 0;
    for (; j + 2 < n_tiles; j += 2) {
      step(j, sa, sb, kb0, kb1, vb0, vb1, More{});
      step(j + 1, sb, sa, kb1, kb0, vb1, vb0, More{});
    }
    if (j + 1 < n_tiles) {
      step(j, sa, sb, kb0, kb1, vb0, vb1, More{});
      step(j + 1, sb, sa, kb1, kb0, vb1, vb0, Last{});
    } else {
      step(j, sa, sb, kb0, kb1, vb0, vb1, Last{});
    }
  }

  // ---- epilogue: normalise once in fp32, round to bf16 once
  const float l_part = (l4[0] + l4[1]) + (l4[2] + l4[3]);
  const float l = l_part + __shfl_xor(l_part, 32);
  float inv = l > 0.f ? 1.0f / l : 0.f;
  inv *= 1.0f / copy_scale(const_load<uint32_t>(a.v_words, kRgV), kRangeV);
  if (item.slot >= 0) {
    // one run of a split q tile: fp32 output and lse for fwd_combine
    const int64_t pr = ((int64_t)item.slot * a.hq + head) * kBM + (row - q0);
    float* po = a.partial_o + pr * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 x;
        x[0] = o[db][4 * j + 0] * inv;
        x[1] = o[db][4 * j + 1] * inv;
        x[2] = o[db][4 * j + 2] * inv;
        x[3] = o[db][4 * j + 3] * inv;
        *reinterpret_cast<f32x4*>(po + 32 * db + 8 * j + 4 * hh) = x;
      }
    if (hh == 0)
      a.partial_lse[pr] = l > 0.f ? (m_run * a.score_mult + fast_log2(l)) * 0.69314718055994531f : -INFINITY;
  } else {
    // out (and with the saved record, what rounding it to bf16 left out,
    // from which the backward forms rowsum(dO * out)) through LDS: each wave
    // writes its 32 rows into the K and V buffers, now free, and reads them
    // back a row at a time, so every global store writes whole 256-byte rows
    // instead of 16 bytes of 32 rows.  16-byte chunks are XOR-swizzled with
    // the row so that both the writes and the read-back spread over the banks.
    constexpr int kRowB = 2 * D, kCh = D / 8, kRowsPer = 64 / kCh;
    __syncthreads();  // every wave is done with the K and V tiles
    // this wave's 32 rows: one of the eight 8 KB halves of the four buffers
    __bf16* const buf = (w >> 1) == 0 ? kb0 : (w >> 1) == 1 ? kb1 : (w >> 1) == 2 ? vb0 : vb1;
    char* so = reinterpret_cast<char*>(buf) + (w & 1) * 32 * kRowB;
    const bool lo = a.out_lo != nullptr;
    u32x2 hw[DB * 4], lw[DB * 4];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint16_t h[4], lr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (lo) {
            split_bf16(o[db][4 * j + i] * inv, &h[i], &lr[i]);
          } else {
            h[i] = __builtin_bit_cast(uint16_t, (__bf16)(o[db][4 * j + i] * inv));
            lr[i] = 0;
          }
        }
        hw[4 * db + j][0] = h[0] | (uint32_t)h[1] << 16;
        hw[4 * db + j][1] = h[2] | (uint32_t)h[3] << 16;
        lw[4 * db + j][0] = lr[0] | (uint32_t)lr[1] << 16;
        lw[4 * db + j][1] = lr[2] | (uint32_t)lr[3] << 16;
      }
    // one output through the region: this lane's pieces in, whole rows out
    // (LDS carries out a wave's accesses in order, so the residual can follow
    // out through the same region)
    auto emit = [&](const u32x2* x, __bf16* dst) {
#pragma unroll
      for (int c = 0; c < 4 * DB; ++c)  // chunk c: dims 8 c .. + 8
        *reinterpret_cast<u32x2*>(so + n * kRowB + ((c ^ (n % kCh)) << 4) + 8 * hh) = x[c];
#pragma unroll
      for (int i = 0; i < kCh / 2; ++i) {
        const int r = i * kRowsPer + lane / kCh, c = lane % kCh;
        const int64_t grow = (int64_t)q0 + wq * 32 + r;
        const u32x4 y = *reinterpret_cast<const u32x4*>(so + r * kRowB + ((c ^ (r % kCh)) << 4));
        if (grow < a.Tq) *reinterpret_cast<u32x4*>(dst + (grow * a.hq + head) * D + c * 8) = y;
      }
    };
    emit(hw, a.out);
    if (lo) emit(lw, a.out_lo);
    if (hh == 0 && row < a.Tq) {
      const float lse = l > 0.f ? (m_run * a.score_mult + fast_log2(l)) * 0.69314718055994531f : -INFINITY;
      a.lse[(int64_t)row * a.hq + head] = lse;
    }
  }
}

// Merge of the runs of a split q tile, per (row, head): lse = log sum_r
// exp(lse_r), out = sum_r exp(lse_r - lse) out_r, runs taken in order.  One
// (row, 4-dim chunk) per thread, kCombineParts workgroups per (split tile,
// head): each thread's loads are a few dependent rounds, not a loop of them.
template <int D>
constexpr int kCombineParts = kBM * (D / 4) / kThreads;

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_combine_kernel(FwdArgs a) {
  constexpr int kChunks = D / 4;
  const int u = blockIdx.x / kCombineParts<D>, part = blockIdx.x % kCombineParts<D>;
  const int s = u / a.hq, head = u % a.hq;
  if (s >= plan_i32(a.counts, 1)) return;
  const i32x4 sp = const_load<i32x4>(a.splits, s);
  const int qt = sp[0], slot0 = sp[1], ns = sp[2];
  const float log2e = 1.4426950408889634f;
  const int i = part * kThreads + threadIdx.x;
  const int rl = i / kChunks, c = i % kChunks;
  const int64_t row = (int64_t)qt * kBM + rl;
  if (row >= a.Tq) return;
  auto at = [&](int r) { return ((int64_t)(slot0 + r) * a.hq + head) * kBM + rl; };
  float m = -INFINITY;
#pragma unroll 4
  for (int r = 0; r < ns; ++r) m = fmaxf(m, a.partial_lse[at(r)]);
  f32x4 acc = f32x4{};
  float sum = 0.f;
  if (m != -INFINITY) {
#pragma unroll 4
    for (int r = 0; r < ns; ++r) {
      const float lr = a.partial_lse[at(r)];
      const f32x4 o = *reinterpret_cast<const f32x4*>(a.partial_o + at(r) * D + 4 * c);
      if (lr == -INFINITY) continue;
      const float wr = fast_exp2((lr - m) * log2e);
      sum += wr;
      acc += wr * o;
    }
  }
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  uint16_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) split_bf16(acc[j] * inv, &h[j], &l[j]);
  u32x2 w2;
  w2[0] = h[0] | (uint32_t)h[1] << 16;
  w2[1] = h[2] | (uint32_t)h[3] << 16;
  *reinterpret_cast<u32x2*>(a.out + (row * a.hq + head) * D + 4 * c) = w2;
  if (a.out_lo) {
    u32x2 r2;
    r2[0] = l[0] | (uint32_t)l[1] << 16;
    r2[1] = l[2] | (uint32_t)l[3] << 16;
    *reinterpret_cast<u32x2*>(a.out_lo + (row * a.hq + head) * D + 4 * c) = r2;
  }
  if (c == 0) a.lse[row * a.hq + head] = sum > 0.f ? m + fast_log2(sum) * 0.69314718055994531f : -INFINITY;
}

// FFA_FWD_PAIRED=1 makes the forward take two q heads per workgroup
// wherever q heads pair up within a kv head, =0 never (for tests and
// measurements); unset, the grid size decides.
int paired_mode() {
  const char* s = std::getenv("FFA_FWD_PAIRED");
  if (!s || !*s) return -1;
  return std::strcmp(s, "0") != 0 ? 1 : 0;
}

// Launch of fwd_kernel over n_units (work item, kv head) units: two q heads
// per workgroup (eight waves, one workgroup per CU) when heads pair up and
// the pairs still fill the chip twice over, else one.
template <int D, bool SC, bool BIAS>
void launch_fwd_kernel(const FwdArgs& a, int64_t n_units, hipStream_t stream) {
  const int64_t n8 = ((n_units + 7) / 8) * 8;
  const int mode = paired_mode();
  const bool pairs = a.grp % 2 == 0;
  if (pairs && (mode == 1 || (mode < 0 && n_units * (a.grp / 2) >= kFwdPairMinWorkgroups)))
    hipLaunchKernelGGL((fwd_kernel<D, SC, BIAS, 2>), dim3((unsigned)(n8 * (a.grp / 2))), dim3(2 * kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((fwd_kernel<D, SC, BIAS, 1>), dim3((unsigned)(n8 * a.grp)), dim3(kThreads), 0, stream, a);
}

template <int D, bool SC, bool BIAS>
hipError_t launch_fwd_t(const FwdLaunch& p, hipStream_t stream) {
  FwdArgs a;
  a.q = static_cast<const __bf16*>(p.q);
  a.k = static_cast<const __bf16*>(p.k);
  a.v = static_cast<const __bf16*>(p.v);
  a.out = static_cast<__bf16*>(p.out);
  a.lse = p.lse;
  a.out_lo = nullptr;
  a.q_range = nullptr;
  {
    // v's range and fp16 copy (read below as v): in the record for the
    // backward, with out's rounding residual, or in the caller's room for
    // them (fwd_v16_bytes), without a residual
    unsigned char* v16 = nullptr;
    uint32_t* words = nullptr;
    uint32_t* parts = nullptr;
    if (p.saved) {
      const SavedLayout S = saved_layout(p.Tq, p.Tk, p.hq, p.hkv, D);
      unsigned char* sv = static_cast<unsigned char*>(p.saved);
      words = reinterpret_cast<uint32_t*>(sv + S.words);
      v16 = sv + S.v16;
      parts = reinterpret_cast<uint32_t*>(sv + S.parts);
      a.out_lo = reinterpret_cast<__bf16*>(sv + S.out_lo);
      a.q_range = words;  // cleared by the copy's second pass below, before the kernel
    } else {
      if (!p.v16) return hipErrorInvalidValue;
      unsigned char* room = static_cast<unsigned char*>(p.v16);
      words = reinterpret_cast<uint32_t*>(room);
      v16 = room + 256;
      parts = reinterpret_cast<uint32_t*>(room + fwd_v16_parts(p.Tk, p.hkv, D));
    }
    const int64_t nk = p.Tk * p.hkv * D / 8;
    launch_convert_tracked(p.v, v16, nk, parts, words, kRgV, kRangeV, true, stream);
    a.v = reinterpret_cast<const __bf16*>(v16);
    a.v_words = words;
  }
  a.entries = reinterpret_cast<const DevEntry*>(p.entries);
  a.slices = reinterpret_cast<const DevSlice*>(p.slices);
  a.row_ptr = p.row_ptr;
  a.order = p.order;
  a.Tq = (int32_t)p.Tq;
  a.Tk = (int32_t)p.Tk;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.grp = p.hq / p.hkv;
  const int64_t n_qt = (p.Tq + kBM - 1) / kBM;
  const FwdScratchLayout S = fwd_scratch_layout(p.Tq);
  unsigned char* ws = static_cast<unsigned char*>(p.scratch);
  a.items = reinterpret_cast<const i32x4*>(ws + S.items);
  a.splits = reinterpret_cast<const i32x4*>(ws + S.splits);
  a.counts = reinterpret_cast<const int32_t*>(ws + S.counts);
  a.partial_o = reinterpret_cast<float*>(ws + S.partial_o);
  a.partial_lse = reinterpret_cast<float*>(ws + S.partial_lse);
  // runs for this head count: the caps below are within the scratch's, which
  // hold for a single head
  const SplitCaps caps = split_caps(n_qt, p.hq, kFwdBalance);
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
  a.slopes = p.alibi_slopes;
  a.bias_mult = SC ? log2e : 1.0f / p.scale;
  if (n_qt == 0) return hipSuccess;
  if (!split_possible(p.n_entries, p.max_len, 1, p.hq, kFwdMinSteps, kFwdBalance)) {
    // no list can be cut: one work item per q tile, straight from the plan
    a.direct = 1;
    a.n_units = (int32_t)(n_qt * p.hkv);
    launch_fwd_kernel<D, SC, BIAS>(a, a.n_units, stream);
    return hipGetLastError();
  }
  a.direct = 0;
  a.n_units = 0;
  SplitLaunch sp;
  sp.row_ptr = p.row_ptr;
  sp.order = p.order;
  sp.n_tiles = n_qt;
  sp.steps_per_entry = 1;
  sp.units = p.hq;
  sp.min_steps = kFwdMinSteps;
  sp.balance = kFwdBalance;
  sp.max_slot_units = kFwdMaxSlots;
  sp.items = ws + S.items;
  sp.items_cap = caps.items;
  sp.splits = ws + S.splits;
  sp.splits_cap = caps.splits;
  sp.counts = reinterpret_cast<int32_t*>(ws + S.counts);
  launch_split(sp, stream);
  launch_fwd_kernel<D, SC, BIAS>(a, caps.items * p.hkv, stream);
  hipLaunchKernelGGL((fwd_combine_kernel<D>), dim3((unsigned)(caps.splits * p.hq * kCombineParts<D>)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

static size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

FwdScratchLayout fwd_scratch_layout(int64_t Tq) {
  FwdScratchLayout L{};
  const int64_t n_qt = Tq > 0 ? (Tq + kBM - 1) / kBM : 0;
  const SplitCaps caps = split_caps(n_qt, 1, kFwdBalance);  // one head: the largest caps
  L.items_cap = caps.items;
  L.splits_cap = caps.splits;
  size_t off = 0;
  L.counts = off;
  off += 256;
  L.items = off;
  off += round256((size_t)L.items_cap * 16);
  L.splits = off;
  off += round256((size_t)L.splits_cap * 16);
  L.partial_lse = off;
  off += round256((size_t)kFwdMaxSlots * kBM * sizeof(float));
  L.partial_o = off;
  off += (size_t)kFwdMaxSlots * kBM * kFwdMaxD * sizeof(float);
  L.total = off;
  return L;
}

size_t fwd_scratch_bytes(int64_t Tq, int64_t max_len) {
  const FwdScratchLayout L = fwd_scratch_layout(Tq);
  // split_possible() needs a list longer than the minimum run of
  // kFwdMinSteps entries, whatever the head count
  return max_len <= kFwdMinSteps ? L.partial_lse : L.total;
}

size_t fwd_v16_parts(int64_t Tk, int hkv, int d) {
  const size_t nk = (size_t)(Tk > 0 ? Tk : 0) * (size_t)(hkv > 0 ? hkv : 0) * (size_t)(d > 0 ? d : 0);
  return 256 + round256(nk * 2);
}

size_t fwd_v16_bytes(int64_t Tk, int hkv, int d) {
  return fwd_v16_parts(Tk, hkv, d) + round256((size_t)kVRangeParts * 4);
}

int fwd_tile_rows() { return kBM; }
int fwd_tile_cols() { return kBN; }

template <int D>
hipError_t launch_fwd_d(const FwdLaunch& p, hipStream_t stream) {
  const bool sc = p.softcap > 0.f, bias = p.alibi_slopes != nullptr;
  if (bias) return sc ? launch_fwd_t<D, true, true>(p, stream) : launch_fwd_t<D, false, true>(p, stream);
  return sc ? launch_fwd_t<D, true, false>(p, stream) : launch_fwd_t<D, false, false>(p, stream);
}

hipError_t launch_fwd(const FwdLaunch& p, hipStream_t stream) {
  return p.d == 64 ? launch_fwd_d<64>(p, stream) : launch_fwd_d<128>(p, stream);
}

}  // namespace ffa
