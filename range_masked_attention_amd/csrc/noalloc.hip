// ffa_fwd_noalloc: the forward of ffa_fwd with every piece of device memory
// beyond the caller's inputs and outputs taken from one file-scope device
// array, for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The array holds a copy of the slice arrays, the block-sparse plan built
// from them on the device (the device planner of plan_device.hip, forward
// list only), the forward's run scratch and the fp16 copy of v that its
// P V product reads.  Each GPU has its own copy of
// the array; its address comes from hipGetSymbolAddress once per device.
// Calls on one GPU share it, so calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "ffa.h"
#include "launch.hpp"

namespace ffa {

constexpr size_t kNoAllocScratchBytes = size_t(256) << 20;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

size_t r256(size_t x) { return (x + 255) & ~size_t(255); }

// Device address of this device's array, looked up once per device.
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

// Layout of the array for one call (byte offsets, 256-byte aligned).
struct NoAllocLayout {
  size_t status, qr, kr, ty, slices, rank, row_ptr, order, count, key, glen, entries, fwd, v16, total;
  int64_t cap;  // entries the rest of the array holds
};

NoAllocLayout layout(int64_t Tq, int64_t Tk, int hkv, int d, int R) {
  NoAllocLayout L{};
  const size_t r = (size_t)(R > 0 ? R : 1);
  const size_t nt = (size_t)((Tq + fwd_tile_rows() - 1) / fwd_tile_rows());
  size_t off = 0;
  L.status = off; off += 256;
  L.qr = off; off += r256(r * 8);
  L.kr = off; off += r256(r * 8);
  L.ty = off; off += r256(r * 4);
  L.slices = off; off += r256(r * sizeof(HostDevSlice));
  L.rank = off; off += r256(r * 4);
  L.row_ptr = off; off += r256((nt + 1) * 4);
  L.order = off; off += r256((nt > 0 ? nt : 1) * 4);
  L.count = off; off += r256((nt > 0 ? nt : 1) * 4);
  L.key = off; off += r256((nt > 0 ? nt : 1) * 4);
  L.glen = off; off += r256((nt > 0 ? nt : 1) * 4);
  L.fwd = off; off += r256(fwd_scratch_layout(Tq).total);
  L.v16 = off; off += r256(fwd_v16_bytes(Tk, hkv, d));
  L.entries = off;
  L.cap = off < kNoAllocScratchBytes ? (int64_t)((kNoAllocScratchBytes - off) / sizeof(HostDevEntry)) : -1;
  L.total = kNoAllocScratchBytes;
  return L;
}

// Entries of the forward list (q tiles of fwd_tile_rows rows, key tiles of
// fwd_tile_cols keys): one per (q tile, key tile, slice) with a visible
// cell.  A CAUSAL slice's rows see a key prefix that grows with the row, so
// a q tile's keys are those of its last row.  No allocation.
int64_t forward_entries(const int32_t* qr, const int32_t* kr, const int32_t* ty, int R) {
  const int64_t BM = fwd_tile_rows(), BN = fwd_tile_cols();
  int64_t n = 0;
  for (int r = 0; r < R; ++r) {
    const int64_t qs = qr[2 * r], qe = qr[2 * r + 1], ks = kr[2 * r], ke = kr[2 * r + 1];
    if (qs == qe || ks == ke) continue;
    for (int64_t t = qs / BM; t <= (qe - 1) / BM; ++t) {
      const int64_t last = std::min(qe, (t + 1) * BM) - 1;  // last row of the slice in tile t
      const int64_t hi = ty[r] == FFA_CAUSAL ? std::min(ke, last + 1 + ke - qe) : ke;
      if (hi > ks) n += (hi - 1) / BN - ks / BN + 1;
    }
  }
  return n;
}

}  // namespace

}  // namespace ffa

// error reporting of the C ABI layer (ffa_api.cpp)
namespace ffa_abi {
int fail(int code, const std::string& msg);
int check_forward_args(const void* q, const void* k, const void* v, int64_t Tq, int64_t Tk, int hq, int hkv,
                       int d, const int32_t* q_ranges, const int32_t* k_ranges, const int32_t* attn_type_map,
                       int R, float scale, float softcap, const void* out, const float* lse);
}

extern "C" int ffa_fwd_noalloc(const void* q, const void* k, const void* v, int64_t Tq, int64_t Tk, int hq,
                               int hkv, int d, const int32_t* q_ranges, const int32_t* k_ranges,
                               const int32_t* attn_type_map, int R, float scale, float softcap, void* out,
                               float* lse, void* stream) {
  using namespace ffa;
  int rc = ffa_abi::check_forward_args(q, k, v, Tq, Tk, hq, hkv, d, q_ranges, k_ranges, attn_type_map, R, scale,
                                       softcap, out, lse);
  if (rc != FFA_OK) return rc;
  if (R > plan_device_max_slices())
    return ffa_abi::fail(FFA_ERR_INVALID_ARG, "ffa_fwd_noalloc takes at most " +
                                                  std::to_string(plan_device_max_slices()) + " slices");
  const NoAllocLayout L = layout(Tq, Tk, hkv, d, R);
  if (L.cap < 0)
    return ffa_abi::fail(FFA_ERR_INVALID_ARG,
                         "ffa_fwd_noalloc: the fp16 copy of v and the run scratch need " + std::to_string(L.entries) +
                             " bytes; its " + std::to_string(kNoAllocScratchBytes >> 20) + " MiB device array holds " +
                             std::to_string(kNoAllocScratchBytes));
  const int64_t need = forward_entries(q_ranges, k_ranges, attn_type_map, R);
  if (L.cap < 0 || need > L.cap)
    return ffa_abi::fail(FFA_ERR_INVALID_ARG,
                         "ffa_fwd_noalloc: the plan needs " + std::to_string(need) + " entries at Tq " +
                             std::to_string(Tq) + "; its " + std::to_string(kNoAllocScratchBytes >> 20) +
                             " MiB device array holds " + std::to_string(L.cap < 0 ? 0 : L.cap));
  if (Tq == 0) return FFA_OK;
  void* base = nullptr;
  hipError_t e = scratch_ptr(&base);
  if (e != hipSuccess) return ffa_abi::fail(FFA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                                             hipGetErrorString(e));
  unsigned char* b = static_cast<unsigned char*>(base);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the slice arrays, then the plan, both built on the device
  if (R > 0) {
    e = hipMemcpyAsync(b + L.qr, q_ranges, (size_t)R * 8, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(b + L.kr, k_ranges, (size_t)R * 8, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(b + L.ty, attn_type_map, (size_t)R * 4, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return ffa_abi::fail(FFA_ERR_HIP, std::string("copying the slices: ") + hipGetErrorString(e));
  }
  PlanDeviceLaunch P{};
  P.q_ranges = reinterpret_cast<const int32_t*>(b + L.qr);
  P.k_ranges = reinterpret_cast<const int32_t*>(b + L.kr);
  P.types = reinterpret_cast<const int32_t*>(b + L.ty);
  P.R = R;
  P.Tq = Tq;
  P.Tk = Tk;
  P.slices = b + L.slices;
  P.rank = reinterpret_cast<int32_t*>(b + L.rank);
  P.status = reinterpret_cast<int32_t*>(b + L.status);
  P.n_parts = 1;
  PlanDevicePart& pp = P.part[0];
  pp.n_tiles = (Tq + fwd_tile_rows() - 1) / fwd_tile_rows();
  pp.bm = fwd_tile_rows();
  pp.bn = fwd_tile_cols();
  pp.transpose = false;
  pp.cap = L.cap;
  pp.count = reinterpret_cast<int32_t*>(b + L.count);
  pp.key = reinterpret_cast<int32_t*>(b + L.key);
  pp.glen = reinterpret_cast<int32_t*>(b + L.glen);
  pp.row_ptr = reinterpret_cast<int32_t*>(b + L.row_ptr);
  pp.entries = b + L.entries;
  pp.order = reinterpret_cast<int32_t*>(b + L.order);
  e = launch_plan_device(P, st);
  if (e != hipSuccess) return ffa_abi::fail(FFA_ERR_HIP, std::string("device planner launch: ") + hipGetErrorString(e));
  FwdLaunch F;
  F.q = q; F.k = k; F.v = v; F.out = out; F.lse = lse;
  F.Tq = Tq; F.Tk = Tk; F.hq = hq; F.hkv = hkv; F.d = d;
  F.scale = scale; F.softcap = softcap;
  F.row_ptr = pp.row_ptr;
  F.entries = pp.entries;
  F.order = pp.order;
  F.slices = P.slices;
  F.scratch = b + L.fwd;
  F.v16 = b + L.v16;
  e = launch_fwd(F, st);
  if (e != hipSuccess) return ffa_abi::fail(FFA_ERR_HIP, std::string("forward kernel launch: ") + hipGetErrorString(e));
  return FFA_OK;
}
