// Host-side launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace ffa {

// Device plan records, mirrored on the host for the upload.
struct HostDevSlice {
  int32_t qs, qe, ks, ke, causal, pad0, pad1, pad2;
};
struct HostDevEntry {
  int32_t tile;
  int32_t meta;  // slice << 1 | partial
};

struct FwdLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int64_t Tq, Tk;
  int hq, hkv, d;
  float scale, softcap;
  const int32_t* row_ptr;  // device: [n_qtiles + 1]
  const void* entries;     // device: HostDevEntry[]
  const int32_t* order;    // device: [n_qtiles]
  const void* slices;      // device: HostDevSlice[]
};

int fwd_tile_rows();
int fwd_tile_cols();
hipError_t launch_fwd(const FwdLaunch& p, hipStream_t stream);

}  // namespace ffa
