// C ABI of the range-masked attention library: argument validation, host
// planning, plan upload and kernel launches.  See include/ffa.h.
#include "ffa.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "launch.hpp"
#include "planner.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(FFA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool debug_checks() {
  const char* s = std::getenv("FFA_DEBUG");
  return s && *s && std::strcmp(s, "0") != 0;
}

// ---------------------------------------------------------------- validation
struct Shape {
  int64_t Tq, Tk;
  int hq, hkv, d;
};

std::string check_shape(const Shape& s, float scale, float softcap) {
  if (s.Tq < 0 || s.Tk < 0) return "Tq and Tk must be >= 0";
  if (s.hq <= 0 || s.hkv <= 0) return "hq and hkv must be positive";
  if (s.hq % s.hkv != 0) return "hq must be a multiple of hkv";
  if (s.d <= 0) return "d must be positive";
  const int64_t lim = int64_t(1) << 31;
  if (s.Tq * s.hq * int64_t(s.d) >= lim || s.Tk * s.hkv * int64_t(s.d) >= lim)
    return "tensors must have fewer than 2^31 elements";
  if (!(std::isfinite(scale) && scale > 0.f)) return "scale must be finite and > 0";
  if (!(std::isfinite(softcap) && softcap >= 0.f)) return "softcap must be finite and >= 0";
  return "";
}

int check_common(const Shape& sh, float scale, float softcap, const int32_t* qr, const int32_t* kr,
                 const int32_t* ty, int R, std::vector<ffa::Slice>* slices) {
  std::string m = check_shape(sh, scale, softcap);
  if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  if (sh.d != 64 && sh.d != 128)
    return fail(FFA_ERR_UNSUPPORTED, "head size " + std::to_string(sh.d) + " is not built (64, 128)");
  m = ffa::validate_slices(sh.Tq, sh.Tk, qr, kr, ty, R, slices);
  if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  if (debug_checks()) {
    m = ffa::check_disjoint(*slices);
    if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  }
  return FFA_OK;
}

// ---------------------------------------------------------------- plan upload
// A plan is packed into one host image, copied through a pinned staging
// slot, and read by the kernels from one stream-ordered device allocation.
struct PlanImage {
  std::vector<unsigned char> bytes;
  size_t off_row_ptr = 0, off_entries = 0, off_order = 0, off_slices = 0;
};

size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

std::string pack_plan(const ffa::Plan& plan, const std::vector<ffa::Slice>& slices, PlanImage* img) {
  if (plan.entries.size() >= (size_t(1) << 31)) return "plan has too many entries";
  const size_t n_rp = plan.row_ptr.size(), n_e = plan.entries.size(), n_o = plan.order.size();
  img->off_row_ptr = 0;
  img->off_entries = align16(n_rp * 4);
  img->off_order = img->off_entries + align16(n_e * sizeof(ffa::HostDevEntry));
  img->off_slices = img->off_order + align16(n_o * 4);
  const size_t total = img->off_slices + align16((slices.size() + 1) * sizeof(ffa::HostDevSlice));
  img->bytes.assign(total, 0);
  auto* rp = reinterpret_cast<int32_t*>(img->bytes.data() + img->off_row_ptr);
  for (size_t i = 0; i < n_rp; ++i) rp[i] = static_cast<int32_t>(plan.row_ptr[i]);
  auto* en = reinterpret_cast<ffa::HostDevEntry*>(img->bytes.data() + img->off_entries);
  for (size_t i = 0; i < n_e; ++i)
    en[i] = ffa::HostDevEntry{plan.entries[i].other, (plan.entries[i].slice << 1) | plan.entries[i].kind};
  auto* od = reinterpret_cast<int32_t*>(img->bytes.data() + img->off_order);
  for (size_t i = 0; i < n_o; ++i) od[i] = plan.order[i];
  auto* sl = reinterpret_cast<ffa::HostDevSlice*>(img->bytes.data() + img->off_slices);
  for (size_t i = 0; i < slices.size(); ++i)
    sl[i] = ffa::HostDevSlice{slices[i].qs, slices[i].qe, slices[i].ks, slices[i].ke,
                              slices[i].type == ffa::kCausal ? 1 : 0, 0, 0, 0};
  return "";
}

struct StageSlot {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t done = nullptr;
  bool pending = false;
};

constexpr int kMaxDevices = 64;
constexpr int kSlots = 4;

struct DeviceStaging {
  std::mutex mu;
  StageSlot slot[kSlots];
  int next = 0;
};

DeviceStaging g_staging[kMaxDevices];

// Copies `src` to device memory `dst` on `stream` through a pinned slot; the
// slot is reused only after its previous copy has completed.
int upload(const void* src, size_t bytes, void* dst, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FFA_ERR_UNSUPPORTED, "device index too large");
  DeviceStaging& ds = g_staging[dev];
  std::lock_guard<std::mutex> lock(ds.mu);
  StageSlot& s = ds.slot[ds.next];
  ds.next = (ds.next + 1) % kSlots;
  if (s.pending) {
    e = hipEventSynchronize(s.done);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(staging)");
    s.pending = false;
  }
  if (!s.done) {
    e = hipEventCreateWithFlags(&s.done, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  }
  if (s.cap < bytes) {
    if (s.host) (void)hipHostFree(s.host);
    s.host = nullptr;
    s.cap = 0;
    const size_t want = std::max<size_t>(bytes * 2, 64 * 1024);
    e = hipHostMalloc(&s.host, want, hipHostMallocDefault);
    if (e != hipSuccess) return fail(FFA_ERR_NOMEM, "hipHostMalloc of plan staging failed");
    s.cap = want;
  }
  std::memcpy(s.host, src, bytes);
  e = hipMemcpyAsync(dst, s.host, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(plan)");
  e = hipEventRecord(s.done, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(staging)");
  s.pending = true;
  return FFA_OK;
}

// Device copy of a plan image; freed on the stream after the kernels.
struct DevicePlan {
  unsigned char* base = nullptr;
  hipStream_t stream = nullptr;
  ~DevicePlan() {
    if (base) (void)hipFreeAsync(base, stream);
  }
};

int stage_plan(const PlanImage& img, hipStream_t stream, DevicePlan* dp) {
  dp->stream = stream;
  hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&dp->base), img.bytes.size(), stream);
  if (e != hipSuccess) {
    dp->base = nullptr;
    return fail(FFA_ERR_NOMEM, std::string("hipMallocAsync(plan): ") + hipGetErrorString(e));
  }
  return upload(img.bytes.data(), img.bytes.size(), dp->base, stream);
}

}  // namespace

extern "C" {

const char* ffa_last_error(void) { return g_err.c_str(); }

const char* ffa_build_info(void) {
  static std::string info = [] {
    std::string s = "arch=gfx950 fwd_tile=" + std::to_string(ffa::fwd_tile_rows()) + "x" +
                    std::to_string(ffa::fwd_tile_cols()) + " head_dims=64,128 softcap=tanh" +
                    " compiler=" + __VERSION__;
    return s;
  }();
  return info.c_str();
}

int64_t ffa_plan_host(int64_t Tq, int64_t Tk, const int32_t* q_ranges, const int32_t* k_ranges,
                      const int32_t* attn_type_map, int R, int bm, int bn, int transpose,
                      int64_t* row_ptr, int32_t* entries, int64_t cap, int32_t* order) {
  if (Tq < 0 || Tk < 0) return fail(FFA_ERR_INVALID_ARG, "Tq and Tk must be >= 0");
  if (bm <= 0 || bn <= 0) return fail(FFA_ERR_INVALID_ARG, "tile sizes must be positive");
  if (Tq >= (int64_t(1) << 31) || Tk >= (int64_t(1) << 31))
    return fail(FFA_ERR_INVALID_ARG, "token counts must be below 2^31");
  std::vector<ffa::Slice> slices;
  std::string m = ffa::validate_slices(Tq, Tk, q_ranges, k_ranges, attn_type_map, R, &slices);
  if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  ffa::Plan plan;
  try {
    ffa::build_plan(slices, Tq, Tk, bm, bn, transpose != 0, &plan);
  } catch (const std::bad_alloc&) {
    return fail(FFA_ERR_NOMEM, "out of host memory while planning");
  }
  const int64_t n = static_cast<int64_t>(plan.entries.size());
  if (row_ptr)
    for (size_t i = 0; i < plan.row_ptr.size(); ++i) row_ptr[i] = plan.row_ptr[i];
  if (order)
    for (size_t i = 0; i < plan.order.size(); ++i) order[i] = plan.order[i];
  if (entries)
    for (int64_t i = 0; i < std::min(n, cap); ++i) {
      entries[3 * i + 0] = plan.entries[i].other;
      entries[3 * i + 1] = slices[plan.entries[i].slice].r;
      entries[3 * i + 2] = plan.entries[i].kind;
    }
  return n;
}

int ffa_fwd(const void* q, const void* k, const void* v, int64_t Tq, int64_t Tk, int hq, int hkv,
            int d, const int32_t* q_ranges, const int32_t* k_ranges, const int32_t* attn_type_map,
            int R, float scale, float softcap, void* out, float* lse, void* stream) {
  g_err.clear();
  std::vector<ffa::Slice> slices;
  const Shape sh{Tq, Tk, hq, hkv, d};
  int rc = check_common(sh, scale, softcap, q_ranges, k_ranges, attn_type_map, R, &slices);
  if (rc != FFA_OK) return rc;
  if (Tq > 0 && (!q || !out || !lse)) return fail(FFA_ERR_INVALID_ARG, "q, out and lse must not be NULL");
  if (Tk > 0 && (!k || !v)) return fail(FFA_ERR_INVALID_ARG, "k and v must not be NULL");
  if (Tq == 0) return FFA_OK;

  ffa::Plan plan;
  PlanImage img;
  try {
    ffa::build_plan(slices, Tq, Tk, ffa::fwd_tile_rows(), ffa::fwd_tile_cols(), false, &plan);
    std::string m = pack_plan(plan, slices, &img);
    if (!m.empty()) return fail(FFA_ERR_UNSUPPORTED, m);
  } catch (const std::bad_alloc&) {
    return fail(FFA_ERR_NOMEM, "out of host memory while planning");
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  DevicePlan dp;
  rc = stage_plan(img, st, &dp);
  if (rc != FFA_OK) return rc;

  ffa::FwdLaunch p;
  p.q = q; p.k = k; p.v = v; p.out = out; p.lse = lse;
  p.Tq = Tq; p.Tk = Tk; p.hq = hq; p.hkv = hkv; p.d = d;
  p.scale = scale; p.softcap = softcap;
  p.row_ptr = reinterpret_cast<const int32_t*>(dp.base + img.off_row_ptr);
  p.entries = dp.base + img.off_entries;
  p.order = reinterpret_cast<const int32_t*>(dp.base + img.off_order);
  p.slices = dp.base + img.off_slices;
  hipError_t e = ffa::launch_fwd(p, st);
  if (e != hipSuccess) return hip_fail(e, "forward kernel launch");
  return FFA_OK;
}

size_t ffa_bwd_workspace_size(int64_t Tq, int hq) {
  if (Tq <= 0 || hq <= 0) return 0;
  return static_cast<size_t>(Tq) * static_cast<size_t>(hq) * sizeof(float);
}

int ffa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
            const void* dout, int64_t Tq, int64_t Tk, int hq, int hkv, int d,
            const int32_t* q_ranges, const int32_t* k_ranges, const int32_t* attn_type_map, int R,
            float scale, float softcap, void* dq, void* dk, void* dv, void* workspace,
            size_t workspace_bytes, void* stream) {
  g_err.clear();
  (void)q; (void)k; (void)v; (void)out; (void)lse; (void)dout; (void)dq; (void)dk; (void)dv;
  (void)workspace; (void)workspace_bytes; (void)stream;
  std::vector<ffa::Slice> slices;
  const Shape sh{Tq, Tk, hq, hkv, d};
  int rc = check_common(sh, scale, softcap, q_ranges, k_ranges, attn_type_map, R, &slices);
  if (rc != FFA_OK) return rc;
  return fail(FFA_ERR_UNSUPPORTED, "backward pass not built yet");
}

}  // extern "C"
