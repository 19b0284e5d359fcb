// C ABI of the range-masked attention library: argument validation, host
// planning, plan upload and kernel launches.  See include/ffa.h.
#include "ffa.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
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

// Fault injection for the error path: with FFA_INJECT_NOMEM set (to anything
// but "0"), every host-side planning step fails as if the host allocator had
// run out, so callers can test their FFA_ERR_NOMEM handling.
void maybe_inject_nomem() {
  const char* s = std::getenv("FFA_INJECT_NOMEM");
  if (s && *s && std::strcmp(s, "0") != 0) throw std::bad_alloc();
}

// ---------------------------------------------------------------- validation
std::string check_sizes(int64_t Tq, int64_t Tk) {
  if (Tq < 0 || Tk < 0) return "Tq and Tk must be >= 0";
  if (Tq >= (int64_t(1) << 31) || Tk >= (int64_t(1) << 31)) return "token counts must be below 2^31";
  return "";
}

int check_heads(int64_t Tq, int64_t Tk, int hq, int hkv, int d, float scale, float softcap) {
  if (hq <= 0 || hkv <= 0) return fail(FFA_ERR_INVALID_ARG, "hq and hkv must be positive");
  if (hq % hkv != 0) return fail(FFA_ERR_INVALID_ARG, "hq must be a multiple of hkv");
  if (d <= 0) return fail(FFA_ERR_INVALID_ARG, "d must be positive");
  const int64_t lim = int64_t(1) << 31;
  if (Tq * hq * int64_t(d) >= lim || Tk * hkv * int64_t(d) >= lim)
    return fail(FFA_ERR_INVALID_ARG, "tensors must have fewer than 2^31 elements");
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(FFA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!(std::isfinite(softcap) && softcap >= 0.f))
    return fail(FFA_ERR_INVALID_ARG, "softcap must be finite and >= 0");
  if (d != 64 && d != 128)
    return fail(FFA_ERR_UNSUPPORTED, "head size " + std::to_string(d) + " is not built (64, 128)");
  return FFA_OK;
}

// Device pointers must be non-NULL when their tensor is non-empty and
// 16-byte aligned (the kernels move 16-byte vectors).
int check_ptr(const void* p, bool needed, const char* name) {
  if (!needed) return FFA_OK;
  if (!p) return fail(FFA_ERR_INVALID_ARG, std::string(name) + " must not be NULL");
  if (reinterpret_cast<uintptr_t>(p) & 15)
    return fail(FFA_ERR_INVALID_ARG, std::string(name) + " must be 16-byte aligned");
  return FFA_OK;
}

// Slice list checks (plus the overlap scan when FFA_DEBUG is set).
int check_slices(int64_t Tq, int64_t Tk, const int32_t* qr, const int32_t* kr, const int32_t* ty, int R) {
  std::vector<ffa::Slice> slices;
  std::string m = ffa::validate_slices(Tq, Tk, qr, kr, ty, R, &slices);
  if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  if (debug_checks()) {
    m = ffa::check_disjoint(slices);
    if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  }
  return FFA_OK;
}

// ---------------------------------------------------------------- plan upload
struct PlanPart {
  size_t off_row_ptr = 0, off_entries = 0, off_order = 0;
  int64_t n_tiles = 0;
  // host-built lists: entry count and longest list, which let the launch
  // skip the run split when no list can be cut (-1: built on the device)
  int64_t n_entries = -1, max_len = -1;
};

size_t align16(size_t x) { return (x + 15) & ~size_t(15); }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

void append_part(const ffa::Plan& plan, std::vector<unsigned char>* img, PlanPart* part) {
  const size_t n_rp = plan.row_ptr.size(), n_e = plan.entries.size(), n_o = plan.order.size();
  part->n_tiles = plan.n_tiles;
  part->n_entries = static_cast<int64_t>(plan.entries.size());
  part->max_len = 0;
  for (size_t i = 0; i + 1 < plan.row_ptr.size(); ++i)
    part->max_len = std::max<int64_t>(part->max_len, plan.row_ptr[i + 1] - plan.row_ptr[i]);
  part->off_row_ptr = img->size();
  part->off_entries = part->off_row_ptr + align16(n_rp * 4);
  part->off_order = part->off_entries + align16(n_e * sizeof(ffa::HostDevEntry));
  img->resize(part->off_order + align16(std::max<size_t>(n_o, 1) * 4), 0);
  auto* rp = reinterpret_cast<int32_t*>(img->data() + part->off_row_ptr);
  for (size_t i = 0; i < n_rp; ++i) rp[i] = static_cast<int32_t>(plan.row_ptr[i]);
  auto* en = reinterpret_cast<ffa::HostDevEntry*>(img->data() + part->off_entries);
  for (size_t i = 0; i < n_e; ++i)
    en[i] = ffa::HostDevEntry{plan.entries[i].other, (plan.entries[i].slice << 1) | plan.entries[i].kind};
  auto* od = reinterpret_cast<int32_t*>(img->data() + part->off_order);
  for (size_t i = 0; i < n_o; ++i) od[i] = plan.order[i];
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

enum : int { kWantFwd = 1, kWantBwd = 2 };

}  // namespace

// For ffa_fwd_noalloc (noalloc.hip): the forward's argument checks with no
// allocation on success.  Overlapping slices are not looked for (the check
// under FFA_DEBUG keeps a list of the slices).
namespace ffa_abi {
int fail(int code, const std::string& msg) { return ::fail(code, msg); }
int check_forward_args(const void* q, const void* k, const void* v, int64_t Tq, int64_t Tk, int hq, int hkv,
                       int d, const int32_t* q_ranges, const int32_t* k_ranges, const int32_t* attn_type_map,
                       int R, float scale, float softcap, const void* out, const float* lse) {
  g_err.clear();
  std::string m = check_sizes(Tq, Tk);
  if (!m.empty()) return ::fail(FFA_ERR_INVALID_ARG, m);
  int rc = check_heads(Tq, Tk, hq, hkv, d, scale, softcap);
  if (rc != FFA_OK) return rc;
  if (R < 0) return ::fail(FFA_ERR_INVALID_ARG, "R must be >= 0");
  if (R > 0 && (!q_ranges || !k_ranges || !attn_type_map))
    return ::fail(FFA_ERR_INVALID_ARG, "slice arrays must not be NULL when R > 0");
  for (int r = 0; r < R; ++r) {
    m = ffa::check_slice(Tq, Tk, q_ranges, k_ranges, attn_type_map, r);
    if (!m.empty()) return ::fail(FFA_ERR_INVALID_ARG, m);
  }
  const bool has_q = Tq > 0, has_k = Tk > 0;
  if ((rc = check_ptr(q, has_q, "q")) || (rc = check_ptr(out, has_q, "out")) ||
      (rc = check_ptr(lse, has_q, "lse")) || (rc = check_ptr(k, has_k, "k")) || (rc = check_ptr(v, has_k, "v")))
    return rc;
  return FFA_OK;
}
}  // namespace ffa_abi

// The plan handle: sizes, the non-empty slices and the device copy of the
// block-sparse lists.
struct ffa_plan_s {
  int64_t Tq = 0, Tk = 0;
  int want = 0;
  size_t n_slices = 0;
  size_t off_slices = 0;
  PlanPart fwd, kv, dq;  // forward q tiles; per key tile (dK/dV); dQ q tiles
  unsigned char* dev = nullptr;
  size_t bytes = 0;
  size_t off_fwd_scratch = 0;  // the forward's scratch (fwd_scratch_layout), after the lists
  // room for v's fp16 copy for forwards without a saved record: allocated by
  // the first that needs it (or more room), freed with the plan
  mutable unsigned char* v16 = nullptr;
  mutable size_t v16_bytes = 0;
  // host-built plans: the caller's index of each slice in the device table
  std::vector<int32_t> slice_index;
  // plans built on the device: the planner's arguments (re-run by
  // ffa_plan_refresh) and its status word; `dev` is the caller's workspace
  bool on_device = false;
  ffa::PlanDeviceLaunch dl{};
};

namespace {

int plan_create(int64_t Tq, int64_t Tk, const int32_t* qr, const int32_t* kr, const int32_t* ty,
                int R, int want, hipStream_t stream, ffa_plan_s** out) {
  *out = nullptr;
  std::string m = check_sizes(Tq, Tk);
  if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  std::vector<ffa::Slice> slices;
  m = ffa::validate_slices(Tq, Tk, qr, kr, ty, R, &slices);
  if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  if (debug_checks()) {
    m = ffa::check_disjoint(slices);
    if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  }
  ffa_plan_s* p = new (std::nothrow) ffa_plan_s;
  if (!p) return fail(FFA_ERR_NOMEM, "out of host memory");
  p->Tq = Tq;
  p->Tk = Tk;
  p->want = want;
  p->n_slices = slices.size();
  try {
    p->slice_index.resize(slices.size());
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(FFA_ERR_NOMEM, "out of host memory");
  }
  for (size_t i = 0; i < slices.size(); ++i) p->slice_index[i] = slices[i].r;
  std::vector<unsigned char> img;
  try {
    maybe_inject_nomem();
    img.resize(align16((slices.size() + 1) * sizeof(ffa::HostDevSlice)), 0);
    auto* sl = reinterpret_cast<ffa::HostDevSlice*>(img.data());
    for (size_t i = 0; i < slices.size(); ++i)
      sl[i] = ffa::HostDevSlice{slices[i].qs, slices[i].qe, slices[i].ks, slices[i].ke,
                                slices[i].type == ffa::kCausal ? 1 : 0, 0, 0, 0};
    ffa::Plan plan;
    if (want & kWantFwd) {
      ffa::build_plan(slices, Tq, Tk, ffa::fwd_tile_rows(), ffa::fwd_tile_cols(), false, &plan);
      if (plan.entries.size() >= (size_t(1) << 30)) {
        delete p;
        return fail(FFA_ERR_UNSUPPORTED, "plan has too many entries");
      }
      append_part(plan, &img, &p->fwd);
    }
    if (want & kWantBwd) {
      ffa::build_plan(slices, Tq, Tk, ffa::bwd_kv_tile_rows(), ffa::bwd_kv_tile_cols(), true, &plan);
      if (plan.entries.size() >= (size_t(1) << 30)) {
        delete p;
        return fail(FFA_ERR_UNSUPPORTED, "plan has too many entries");
      }
      append_part(plan, &img, &p->kv);
      if ((want & kWantFwd) && ffa::bwd_q_tile_rows() == ffa::fwd_tile_rows() &&
          ffa::bwd_q_tile_cols() == ffa::fwd_tile_cols()) {
        p->dq = p->fwd;  // same tiles: the dQ pass walks the forward lists
      } else {
        ffa::build_plan(slices, Tq, Tk, ffa::bwd_q_tile_rows(), ffa::bwd_q_tile_cols(), false, &plan);
        append_part(plan, &img, &p->dq);
      }
    }
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(FFA_ERR_NOMEM, "out of host memory while planning");
  }
  p->bytes = img.size();
  if (want & kWantFwd) {
    p->off_fwd_scratch = align256(img.size());
    p->bytes = p->off_fwd_scratch + ffa::fwd_scratch_bytes(Tq, p->fwd.max_len);
  }
  hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&p->dev), p->bytes, stream);
  if (e != hipSuccess) {
    delete p;
    return fail(FFA_ERR_NOMEM, std::string("hipMallocAsync(plan): ") + hipGetErrorString(e));
  }
  int rc = upload(img.data(), img.size(), p->dev, stream);
  if (rc != FFA_OK) {
    (void)hipFreeAsync(p->dev, stream);
    delete p;
    return rc;
  }
  *out = p;
  return FFA_OK;
}

int plan_destroy(ffa_plan_s* p, hipStream_t stream) {
  if (!p) return FFA_OK;
  hipError_t e = hipSuccess;
  if (p->v16) e = hipFreeAsync(p->v16, stream);
  if (p->dev && !p->on_device) {
    const hipError_t ef = hipFreeAsync(p->dev, stream);
    if (e == hipSuccess) e = ef;
  }
  delete p;
  if (e != hipSuccess) return hip_fail(e, "hipFreeAsync(plan)");
  return FFA_OK;
}

int check_slopes(const float* slopes) {
  if (slopes && (reinterpret_cast<uintptr_t>(slopes) & 3))
    return fail(FFA_ERR_INVALID_ARG, "alibi_slopes must be 4-byte aligned");
  return FFA_OK;
}

int fwd_planned(const ffa_plan_s* p, const void* q, const void* k, const void* v, int hq, int hkv,
                int d, float scale, float softcap, const float* slopes, void* out, float* lse,
                void* saved, hipStream_t stream) {
  if (!(p->want & kWantFwd)) return fail(FFA_ERR_INVALID_ARG, "plan was built without the forward lists");
  int rc = check_heads(p->Tq, p->Tk, hq, hkv, d, scale, softcap);
  if (rc != FFA_OK) return rc;
  const bool has_q = p->Tq > 0, has_k = p->Tk > 0;
  if ((rc = check_ptr(q, has_q, "q")) || (rc = check_ptr(out, has_q, "out")) ||
      (rc = check_ptr(lse, has_q, "lse")) || (rc = check_ptr(k, has_k, "k")) ||
      (rc = check_ptr(v, has_k, "v")) || (rc = check_slopes(slopes)) ||
      (saved && (rc = check_ptr(saved, true, "saved"))))
    return rc;
  if (p->Tq == 0) return FFA_OK;
  ffa::FwdLaunch L;
  L.q = q; L.k = k; L.v = v; L.out = out; L.lse = lse; L.saved = saved;
  L.Tq = p->Tq; L.Tk = p->Tk; L.hq = hq; L.hkv = hkv; L.d = d;
  L.scale = scale; L.softcap = softcap;
  L.row_ptr = reinterpret_cast<const int32_t*>(p->dev + p->fwd.off_row_ptr);
  L.entries = p->dev + p->fwd.off_entries;
  L.order = reinterpret_cast<const int32_t*>(p->dev + p->fwd.off_order);
  L.slices = p->dev + p->off_slices;
  L.alibi_slopes = slopes;
  L.scratch = p->dev + p->off_fwd_scratch;
  L.n_entries = p->fwd.n_entries;
  L.max_len = p->fwd.max_len;
  // without a record, the fp16 copy of v goes to the plan's room for it
  if (!saved) {
    const size_t need = ffa::fwd_v16_bytes(p->Tk, hkv, d);
    if (p->v16_bytes < need) {
      if (p->v16) {
        const hipError_t ef = hipFreeAsync(p->v16, stream);
        p->v16 = nullptr;
        p->v16_bytes = 0;
        if (ef != hipSuccess) return hip_fail(ef, "hipFreeAsync(v16)");
      }
      const hipError_t ea = hipMallocAsync(reinterpret_cast<void**>(&p->v16), need, stream);
      if (ea != hipSuccess) {
        p->v16 = nullptr;
        return fail(FFA_ERR_NOMEM, std::string("hipMallocAsync(v16): ") + hipGetErrorString(ea));
      }
      p->v16_bytes = need;
    }
    L.v16 = p->v16;
  }
  hipError_t e = ffa::launch_fwd(L, stream);
  if (e != hipSuccess) return hip_fail(e, "forward kernel launch");
  return FFA_OK;
}

int bwd_planned(const ffa_plan_s* p, const void* q, const void* k, const void* v, const void* out,
                const float* lse, const void* saved, const void* dout, int hq, int hkv, int d, float scale,
                float softcap, const float* slopes, void* dq, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  if (!(p->want & kWantBwd)) return fail(FFA_ERR_INVALID_ARG, "plan was built without the backward lists");
  if (!saved && !(p->want & kWantFwd))
    return fail(FFA_ERR_INVALID_ARG, "without a saved record the plan needs the forward lists (to re-run the forward)");
  int rc = check_heads(p->Tq, p->Tk, hq, hkv, d, scale, softcap);
  if (rc != FFA_OK) return rc;
  const bool has_q = p->Tq > 0, has_k = p->Tk > 0;
  if ((rc = check_ptr(q, has_q, "q")) || (rc = check_ptr(out, has_q, "out")) ||
      (rc = check_ptr(lse, has_q, "lse")) || (rc = check_ptr(dout, has_q, "dout")) ||
      (rc = check_ptr(dq, has_q, "dq")) || (rc = check_ptr(k, has_k, "k")) ||
      (rc = check_ptr(v, has_k, "v")) || (rc = check_ptr(dk, has_k, "dk")) ||
      (rc = check_ptr(dv, has_k, "dv")) || (rc = check_slopes(slopes)) ||
      (saved && (rc = check_ptr(saved, true, "saved"))))
    return rc;
  const size_t need = ffa_bwd_workspace_size(p->Tq, p->Tk, hq, hkv, d);
  if (workspace && workspace_bytes < need)
    return fail(FFA_ERR_INVALID_ARG, "workspace is smaller than ffa_bwd_workspace_size()");
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 15))
    return fail(FFA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (p->Tq == 0 && p->Tk == 0) return FFA_OK;
  void* ws = workspace;
  if (!ws && need) {
    hipError_t e = hipMallocAsync(&ws, need, stream);
    if (e != hipSuccess) return fail(FFA_ERR_NOMEM, std::string("hipMallocAsync(workspace): ") + hipGetErrorString(e));
  }
  const ffa::BwdWorkspaceLayout WL = ffa::bwd_workspace_layout(p->Tq, p->Tk, hq, hkv, d);
  if (!saved) {
    // no record from the caller: re-run the training forward into the
    // workspace to get one (its out and lse are the caller's bits again)
    unsigned char* b = static_cast<unsigned char*>(ws);
    void* re_saved = b + WL.re_saved;
    if (p->Tq > 0) {
      rc = fwd_planned(p, q, k, v, hq, hkv, d, scale, softcap, slopes, b + WL.re_out,
                       reinterpret_cast<float*>(b + WL.re_lse), re_saved, stream);
      if (rc != FFA_OK) {
        if (ws != workspace) (void)hipFreeAsync(ws, stream);
        return rc;
      }
      out = b + WL.re_out;
    } else if (p->Tk > 0) {
      // no rows: the record is only read for v's copy, which nothing uses;
      // give its range word a defined value
      const ffa::SavedLayout S = ffa::saved_layout(p->Tq, p->Tk, hq, hkv, d);
      ffa::launch_range_clear(reinterpret_cast<uint32_t*>(b + WL.re_saved + S.words), 4, stream);
    }
    saved = re_saved;
  }
  ffa::BwdLaunch L;
  L.q = q; L.k = k; L.v = v; L.out = out; L.saved = saved; L.lse = lse; L.dout = dout;
  L.dq = dq; L.dk = dk; L.dv = dv; L.workspace = ws;
  L.Tq = p->Tq; L.Tk = p->Tk; L.hq = hq; L.hkv = hkv; L.d = d;
  L.scale = scale; L.softcap = softcap;
  L.kv_row_ptr = reinterpret_cast<const int32_t*>(p->dev + p->kv.off_row_ptr);
  L.kv_entries = p->dev + p->kv.off_entries;
  L.kv_order = reinterpret_cast<const int32_t*>(p->dev + p->kv.off_order);
  L.q_row_ptr = reinterpret_cast<const int32_t*>(p->dev + p->dq.off_row_ptr);
  L.q_entries = p->dev + p->dq.off_entries;
  L.q_order = reinterpret_cast<const int32_t*>(p->dev + p->dq.off_order);
  L.slices = p->dev + p->off_slices;
  L.alibi_slopes = slopes;
  L.kv_n_entries = p->kv.n_entries;
  L.kv_max_len = p->kv.max_len;
  L.q_n_entries = p->dq.n_entries;
  L.q_max_len = p->dq.max_len;
  hipError_t e = ffa::launch_bwd(L, stream);
  if (ws != workspace) (void)hipFreeAsync(ws, stream);
  if (e != hipSuccess) return hip_fail(e, "backward kernel launch");
  return FFA_OK;
}

// Layout of a device-built plan inside the caller's workspace (256-byte
// aligned pieces): slice table, slice ranks, status word, then per list
// row_ptr, entries, order and three scratch arrays.

struct DeviceLayout {
  size_t slices, rank, status, fwd_scratch, total;
  struct Part {
    int64_t n_tiles;
    size_t row_ptr, entries, order, count, key, glen;
  } part[2];
};

DeviceLayout device_layout(int64_t Tq, int64_t Tk, int R, int64_t cap) {
  DeviceLayout L{};
  size_t off = 0;
  L.slices = off;
  off += align256(size_t(std::max(R, 1)) * sizeof(ffa::HostDevSlice));
  L.rank = off;
  off += align256(size_t(std::max(R, 1)) * 4);
  L.status = off;
  off += 256;
  const int64_t n_tiles[2] = {(Tq + ffa::fwd_tile_rows() - 1) / ffa::fwd_tile_rows(),
                              (Tk + ffa::bwd_kv_tile_cols() - 1) / ffa::bwd_kv_tile_cols()};
  for (int i = 0; i < 2; ++i) {
    const size_t n = size_t(n_tiles[i]);
    DeviceLayout::Part& P = L.part[i];
    P.n_tiles = n_tiles[i];
    P.row_ptr = off; off += align256((n + 1) * 4);
    P.entries = off; off += align256(size_t(std::max<int64_t>(cap, 1)) * sizeof(ffa::HostDevEntry));
    P.order = off;   off += align256(std::max<size_t>(n, 1) * 4);
    P.count = off;   off += align256(std::max<size_t>(n, 1) * 4);
    P.key = off;     off += align256(std::max<size_t>(n, 1) * 4);
    P.glen = off;    off += align256(std::max<size_t>(n, 1) * 4);
  }
  L.fwd_scratch = off;
  off += align256(ffa::fwd_scratch_layout(Tq).total);
  L.total = off;
  return L;
}

std::string check_device_plan_args(int64_t Tq, int64_t Tk, int R, int64_t max_entries) {
  std::string m = check_sizes(Tq, Tk);
  if (!m.empty()) return m;
  if (R < 0) return "R must be >= 0";
  if (R > ffa::plan_device_max_slices())
    return "the device planner takes at most " + std::to_string(ffa::plan_device_max_slices()) + " slices";
  if (max_entries < 0 || max_entries >= (int64_t(1) << 30)) return "max_entries must be in [0, 2^30)";
  if (ffa::bwd_q_tile_rows() != ffa::fwd_tile_rows() || ffa::bwd_q_tile_cols() != ffa::fwd_tile_cols())
    return "device planner expects the dQ pass to share the forward tiles";
  return "";
}

}  // namespace

extern "C" {

const char* ffa_last_error(void) { return g_err.c_str(); }

// hash of the sources the library was built from (the build passes it;
// see range_masked_attention_amd/_build.py source_hash)
#ifndef FFA_SOURCE_HASH
#define FFA_SOURCE_HASH "unknown"
#endif

const char* ffa_build_info(void) {
  static std::string info = [] {
    std::string s = "arch=gfx950 fwd_tile=" + std::to_string(ffa::fwd_tile_rows()) + "x" +
                    std::to_string(ffa::fwd_tile_cols()) + " bwd_kv_tile=" +
                    std::to_string(ffa::bwd_kv_tile_rows()) + "x" + std::to_string(ffa::bwd_kv_tile_cols()) +
                    " bwd_q_tile=" + std::to_string(ffa::bwd_q_tile_rows()) + "x" +
                    std::to_string(ffa::bwd_q_tile_cols()) + " head_dims=64,128 softcap=tanh source=" +
                    FFA_SOURCE_HASH + " compiler=" + __VERSION__;
    return s;
  }();
  return info.c_str();
}

int64_t ffa_plan_host(int64_t Tq, int64_t Tk, const int32_t* q_ranges, const int32_t* k_ranges,
                      const int32_t* attn_type_map, int R, int bm, int bn, int transpose,
                      int64_t* row_ptr, int32_t* entries, int64_t cap, int32_t* order) {
  g_err.clear();
  std::string m = check_sizes(Tq, Tk);
  if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  if (bm <= 0 || bn <= 0) return fail(FFA_ERR_INVALID_ARG, "tile sizes must be positive");
  std::vector<ffa::Slice> slices;
  m = ffa::validate_slices(Tq, Tk, q_ranges, k_ranges, attn_type_map, R, &slices);
  if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  ffa::Plan plan;
  try {
    maybe_inject_nomem();
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

int64_t ffa_block_slices(int64_t Tq, int64_t Tk, int block_q, int block_k, const int32_t* kv_num_blocks,
                         const int32_t* kv_indices, int max_blocks, int32_t* q_ranges, int32_t* k_ranges,
                         int32_t* attn_type_map, int64_t cap) {
  g_err.clear();
  std::string m = check_sizes(Tq, Tk);
  if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  std::vector<ffa::RangePair> sl;
  try {
    maybe_inject_nomem();
    m = ffa::block_slices(Tq, Tk, block_q, block_k, kv_num_blocks, kv_indices, max_blocks, &sl);
  } catch (const std::bad_alloc&) {
    return fail(FFA_ERR_NOMEM, "out of host memory while converting blocks");
  }
  if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  const int64_t n = static_cast<int64_t>(sl.size());
  for (int64_t i = 0; i < std::min(n, cap); ++i) {
    if (q_ranges) { q_ranges[2 * i] = sl[i].qs; q_ranges[2 * i + 1] = sl[i].qe; }
    if (k_ranges) { k_ranges[2 * i] = sl[i].ks; k_ranges[2 * i + 1] = sl[i].ke; }
    if (attn_type_map) attn_type_map[i] = FFA_FULL;
  }
  return n;
}

int ffa_plan_create(int64_t Tq, int64_t Tk, const int32_t* q_ranges, const int32_t* k_ranges,
                    const int32_t* attn_type_map, int R, void* stream, ffa_plan_t* plan) {
  g_err.clear();
  if (!plan) return fail(FFA_ERR_INVALID_ARG, "plan must not be NULL");
  return plan_create(Tq, Tk, q_ranges, k_ranges, attn_type_map, R, kWantFwd | kWantBwd,
                     static_cast<hipStream_t>(stream), plan);
}

int ffa_plan_destroy(ffa_plan_t plan, void* stream) {
  g_err.clear();
  return plan_destroy(plan, static_cast<hipStream_t>(stream));
}

int ffa_fwd_planned_ex(ffa_plan_t plan, const void* q, const void* k, const void* v, int hq, int hkv,
                       int d, float scale, float softcap, const float* alibi_slopes, void* out,
                       float* lse, void* saved, void* stream) {
  g_err.clear();
  if (!plan) return fail(FFA_ERR_INVALID_ARG, "plan must not be NULL");
  return fwd_planned(plan, q, k, v, hq, hkv, d, scale, softcap, alibi_slopes, out, lse, saved,
                     static_cast<hipStream_t>(stream));
}

int ffa_fwd_planned(ffa_plan_t plan, const void* q, const void* k, const void* v, int hq, int hkv,
                    int d, float scale, float softcap, void* out, float* lse, void* stream) {
  return ffa_fwd_planned_ex(plan, q, k, v, hq, hkv, d, scale, softcap, nullptr, out, lse, nullptr, stream);
}

int ffa_bwd_planned_ex(ffa_plan_t plan, const void* q, const void* k, const void* v, const void* out,
                       const float* lse, const void* saved, const void* dout, int hq, int hkv, int d,
                       float scale, float softcap, const float* alibi_slopes, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!plan) return fail(FFA_ERR_INVALID_ARG, "plan must not be NULL");
  return bwd_planned(plan, q, k, v, out, lse, saved, dout, hq, hkv, d, scale, softcap, alibi_slopes, dq,
                     dk, dv, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int ffa_bwd_planned(ffa_plan_t plan, const void* q, const void* k, const void* v, const void* out,
                    const float* lse, const void* dout, int hq, int hkv, int d, float scale,
                    float softcap, void* dq, void* dk, void* dv, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return ffa_bwd_planned_ex(plan, q, k, v, out, lse, nullptr, dout, hq, hkv, d, scale, softcap, nullptr, dq,
                            dk, dv, workspace, workspace_bytes, stream);
}

int ffa_fwd(const void* q, const void* k, const void* v, int64_t Tq, int64_t Tk, int hq, int hkv,
            int d, const int32_t* q_ranges, const int32_t* k_ranges, const int32_t* attn_type_map,
            int R, float scale, float softcap, void* out, float* lse, void* stream) {
  return ffa_fwd_ex(q, k, v, Tq, Tk, hq, hkv, d, q_ranges, k_ranges, attn_type_map, R, scale, softcap,
                    nullptr, out, lse, nullptr, stream);
}

int ffa_fwd_ex(const void* q, const void* k, const void* v, int64_t Tq, int64_t Tk, int hq, int hkv,
               int d, const int32_t* q_ranges, const int32_t* k_ranges, const int32_t* attn_type_map,
               int R, float scale, float softcap, const float* alibi_slopes, void* out, float* lse,
               void* saved, void* stream) {
  g_err.clear();
  std::string m = check_sizes(Tq, Tk);
  if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  int rc = check_heads(Tq, Tk, hq, hkv, d, scale, softcap);
  if (rc != FFA_OK) return rc;
  if ((rc = check_slices(Tq, Tk, q_ranges, k_ranges, attn_type_map, R)) != FFA_OK) return rc;
  const bool has_q = Tq > 0, has_k = Tk > 0;
  if ((rc = check_ptr(q, has_q, "q")) || (rc = check_ptr(out, has_q, "out")) ||
      (rc = check_ptr(lse, has_q, "lse")) || (rc = check_ptr(k, has_k, "k")) ||
      (rc = check_ptr(v, has_k, "v")) || (rc = check_slopes(alibi_slopes)) ||
      (saved && (rc = check_ptr(saved, true, "saved"))))
    return rc;
  if (Tq == 0) return FFA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  ffa_plan_s* p = nullptr;
  rc = plan_create(Tq, Tk, q_ranges, k_ranges, attn_type_map, R, kWantFwd, st, &p);
  if (rc != FFA_OK) return rc;
  rc = fwd_planned(p, q, k, v, hq, hkv, d, scale, softcap, alibi_slopes, out, lse, saved, st);
  const std::string err = g_err;
  const int rc2 = plan_destroy(p, st);
  if (rc != FFA_OK) return fail(rc, err);
  return rc2;
}

size_t ffa_saved_size(int64_t Tq, int64_t Tk, int hq, int hkv, int d) {
  if (Tq < 0 || Tk < 0 || hq <= 0 || hkv <= 0 || (d != 64 && d != 128)) return 0;
  return ffa::saved_layout(Tq, Tk, hq, hkv, d).total;
}

size_t ffa_bwd_workspace_size(int64_t Tq, int64_t Tk, int hq, int hkv, int d) {
  if (Tq < 0 || Tk < 0 || hq <= 0 || hkv <= 0 || (d != 64 && d != 128)) return 0;
  if (Tq == 0 && Tk == 0) return 0;
  return ffa::bwd_workspace_layout(Tq, Tk, hq, hkv, d).total;
}

int ffa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
            const void* dout, int64_t Tq, int64_t Tk, int hq, int hkv, int d,
            const int32_t* q_ranges, const int32_t* k_ranges, const int32_t* attn_type_map, int R,
            float scale, float softcap, void* dq, void* dk, void* dv, void* workspace,
            size_t workspace_bytes, void* stream) {
  return ffa_bwd_ex(q, k, v, out, lse, nullptr, dout, Tq, Tk, hq, hkv, d, q_ranges, k_ranges, attn_type_map,
                    R, scale, softcap, nullptr, dq, dk, dv, workspace, workspace_bytes, stream);
}

int ffa_bwd_ex(const void* q, const void* k, const void* v, const void* out, const float* lse,
               const void* saved, const void* dout, int64_t Tq, int64_t Tk, int hq, int hkv, int d,
               const int32_t* q_ranges, const int32_t* k_ranges, const int32_t* attn_type_map, int R,
               float scale, float softcap, const float* alibi_slopes, void* dq, void* dk, void* dv,
               void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  std::string m = check_sizes(Tq, Tk);
  if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  int rc = check_heads(Tq, Tk, hq, hkv, d, scale, softcap);
  if (rc != FFA_OK) return rc;
  if ((rc = check_slices(Tq, Tk, q_ranges, k_ranges, attn_type_map, R)) != FFA_OK) return rc;
  const bool has_q = Tq > 0, has_k = Tk > 0;
  if ((rc = check_ptr(q, has_q, "q")) || (rc = check_ptr(out, has_q, "out")) ||
      (rc = check_ptr(lse, has_q, "lse")) || (rc = check_ptr(dout, has_q, "dout")) ||
      (rc = check_ptr(dq, has_q, "dq")) || (rc = check_ptr(k, has_k, "k")) ||
      (rc = check_ptr(v, has_k, "v")) || (rc = check_ptr(dk, has_k, "dk")) ||
      (rc = check_ptr(dv, has_k, "dv")) || (rc = check_slopes(alibi_slopes)) ||
      (saved && (rc = check_ptr(saved, true, "saved"))))
    return rc;
  if (workspace && workspace_bytes < ffa_bwd_workspace_size(Tq, Tk, hq, hkv, d))
    return fail(FFA_ERR_INVALID_ARG, "workspace is smaller than ffa_bwd_workspace_size()");
  if (Tq == 0 && Tk == 0) return FFA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  ffa_plan_s* p = nullptr;
  // without a saved record the forward is re-run, which needs its lists too
  rc = plan_create(Tq, Tk, q_ranges, k_ranges, attn_type_map, R, saved ? kWantBwd : (kWantFwd | kWantBwd), st,
                   &p);
  if (rc != FFA_OK) return rc;
  rc = bwd_planned(p, q, k, v, out, lse, saved, dout, hq, hkv, d, scale, softcap, alibi_slopes, dq, dk, dv,
                   workspace, workspace_bytes, st);
  const std::string err = g_err;
  const int rc2 = plan_destroy(p, st);
  if (rc != FFA_OK) return fail(rc, err);
  return rc2;
}

int ffa_plan_device_workspace_size(int64_t Tq, int64_t Tk, int R, int64_t max_entries, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(FFA_ERR_INVALID_ARG, "bytes must not be NULL");
  const std::string m = check_device_plan_args(Tq, Tk, R, max_entries);
  if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  *bytes = device_layout(Tq, Tk, R, max_entries).total;
  return FFA_OK;
}

int ffa_plan_create_device(int64_t Tq, int64_t Tk, const int32_t* q_ranges, const int32_t* k_ranges,
                           const int32_t* attn_type_map, int R, int64_t max_entries, void* workspace,
                           size_t workspace_bytes, void* stream, ffa_plan_t* plan) {
  g_err.clear();
  if (!plan) return fail(FFA_ERR_INVALID_ARG, "plan must not be NULL");
  *plan = nullptr;
  const std::string m = check_device_plan_args(Tq, Tk, R, max_entries);
  if (!m.empty()) return fail(FFA_ERR_INVALID_ARG, m);
  if (R > 0 && (!q_ranges || !k_ranges || !attn_type_map))
    return fail(FFA_ERR_INVALID_ARG, "slice arrays must not be NULL");
  if ((reinterpret_cast<uintptr_t>(q_ranges) | reinterpret_cast<uintptr_t>(k_ranges) |
       reinterpret_cast<uintptr_t>(attn_type_map)) & 3)
    return fail(FFA_ERR_INVALID_ARG, "slice arrays must be 4-byte aligned");
  const DeviceLayout L = device_layout(Tq, Tk, R, max_entries);
  if (!workspace) return fail(FFA_ERR_INVALID_ARG, "workspace must not be NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(FFA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(FFA_ERR_INVALID_ARG, "workspace is smaller than ffa_plan_device_workspace_size()");
  ffa_plan_s* p = new (std::nothrow) ffa_plan_s;
  if (!p) return fail(FFA_ERR_NOMEM, "out of host memory");
  auto* base = static_cast<unsigned char*>(workspace);
  p->Tq = Tq;
  p->Tk = Tk;
  p->want = kWantFwd | kWantBwd;
  p->n_slices = size_t(R);
  p->off_slices = L.slices;
  p->dev = base;
  p->bytes = L.total;
  p->off_fwd_scratch = L.fwd_scratch;
  p->on_device = true;
  PlanPart* parts[2] = {&p->fwd, &p->kv};
  ffa::PlanDeviceLaunch& D = p->dl;
  D.q_ranges = q_ranges;
  D.k_ranges = k_ranges;
  D.types = attn_type_map;
  D.R = R;
  D.Tq = Tq;
  D.Tk = Tk;
  D.slices = base + L.slices;
  D.rank = reinterpret_cast<int32_t*>(base + L.rank);
  D.status = reinterpret_cast<int32_t*>(base + L.status);
  D.n_parts = 2;
  for (int i = 0; i < 2; ++i) {
    const DeviceLayout::Part& LP = L.part[i];
    parts[i]->n_tiles = LP.n_tiles;
    parts[i]->off_row_ptr = LP.row_ptr;
    parts[i]->off_entries = LP.entries;
    parts[i]->off_order = LP.order;
    ffa::PlanDevicePart& P = D.part[i];
    P.n_tiles = LP.n_tiles;
    P.bm = i == 0 ? ffa::fwd_tile_rows() : ffa::bwd_kv_tile_rows();
    P.bn = i == 0 ? ffa::fwd_tile_cols() : ffa::bwd_kv_tile_cols();
    P.transpose = i == 1;
    P.cap = max_entries;
    P.count = reinterpret_cast<int32_t*>(base + LP.count);
    P.key = reinterpret_cast<int32_t*>(base + LP.key);
    P.glen = reinterpret_cast<int32_t*>(base + LP.glen);
    P.row_ptr = reinterpret_cast<int32_t*>(base + LP.row_ptr);
    P.entries = base + LP.entries;
    P.order = reinterpret_cast<int32_t*>(base + LP.order);
  }
  p->dq = p->fwd;  // the dQ pass walks the forward lists
  hipError_t e = ffa::launch_plan_device(D, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "device planner launch");
  }
  *plan = p;
  return FFA_OK;
}

int ffa_plan_refresh(ffa_plan_t plan, void* stream) {
  g_err.clear();
  if (!plan) return fail(FFA_ERR_INVALID_ARG, "plan must not be NULL");
  if (!plan->on_device) return fail(FFA_ERR_INVALID_ARG, "plan was not built by ffa_plan_create_device");
  hipError_t e = ffa::launch_plan_device(plan->dl, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "device planner launch");
  return FFA_OK;
}

int ffa_plan_status(ffa_plan_t plan, void* stream, int* status) {
  g_err.clear();
  if (!plan || !status) return fail(FFA_ERR_INVALID_ARG, "plan and status must not be NULL");
  *status = 0;
  if (!plan->on_device) return FFA_OK;
  int32_t word = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&word, plan->dl.status, sizeof(word), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the planner status");
  *status = word;
  return FFA_OK;
}

int64_t ffa_plan_export(ffa_plan_t plan, int which, int64_t* n_tiles, int64_t* row_ptr, int32_t* entries,
                        int64_t cap, int32_t* order, void* stream) {
  g_err.clear();
  if (!plan) return fail(FFA_ERR_INVALID_ARG, "plan must not be NULL");
  if (which < 0 || which > 2) return fail(FFA_ERR_INVALID_ARG, "which must be 0, 1 or 2");
  const int need = which == 0 ? kWantFwd : kWantBwd;
  if (!(plan->want & need)) return fail(FFA_ERR_INVALID_ARG, "the plan has no such list");
  const PlanPart& P = which == 0 ? plan->fwd : which == 1 ? plan->kv : plan->dq;
  if (n_tiles) *n_tiles = P.n_tiles;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<int32_t> rp, od;
  std::vector<ffa::HostDevEntry> en;
  try {
    rp.resize(size_t(P.n_tiles) + 1);
    od.resize(size_t(std::max<int64_t>(P.n_tiles, 1)));
  } catch (const std::bad_alloc&) {
    return fail(FFA_ERR_NOMEM, "out of host memory");
  }
  hipError_t e = hipMemcpyAsync(rp.data(), plan->dev + P.off_row_ptr, rp.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && P.n_tiles > 0)
    e = hipMemcpyAsync(od.data(), plan->dev + P.off_order, size_t(P.n_tiles) * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the plan");
  const int64_t n = rp.back();
  try {
    en.resize(size_t(std::max<int64_t>(n, 1)));
  } catch (const std::bad_alloc&) {
    return fail(FFA_ERR_NOMEM, "out of host memory");
  }
  if (n > 0) {
    e = hipMemcpyAsync(en.data(), plan->dev + P.off_entries, size_t(n) * sizeof(ffa::HostDevEntry),
                       hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "reading the plan");
  }
  if (row_ptr)
    for (size_t i = 0; i < rp.size(); ++i) row_ptr[i] = rp[i];
  if (order)
    for (int64_t i = 0; i < P.n_tiles; ++i) order[i] = od[size_t(i)];
  if (entries)
    for (int64_t i = 0; i < std::min(n, cap); ++i) {
      const int32_t slice = en[size_t(i)].meta >> 1;
      entries[3 * i + 0] = en[size_t(i)].tile;
      entries[3 * i + 1] = plan->on_device ? slice : plan->slice_index[size_t(slice)];
      entries[3 * i + 2] = en[size_t(i)].meta & 1;
    }
  return n;
}

}  // extern "C"
