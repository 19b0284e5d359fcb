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

// Workgroups of the pass that copies v to fp16: each leaves the largest |v|
// it saw in a slot of its own (kVRangeParts words after the copy).
constexpr int kVRangeParts = 2048;

// What the training forward saves for the backward (device memory of
// saved_layout(...).total bytes): range words (fp32 bits of max |v| in word
// kRgV, of max |q| in word kRgQ), out's bf16 rounding residual [Tq][hq][d], the fp16 copy of v
// [Tk][hkv][d] that the forward's P V product read (times its scale), and
// the copy pass's partial maxima.
struct SavedLayout {
  size_t words, out_lo, v16, parts, total;
};
SavedLayout saved_layout(int64_t Tq, int64_t Tk, int hq, int hkv, int d);

// Room for the forward's fp16 copy of v (P V runs in fp16) when it saves no
// record: v's range words (256 bytes), the copy [Tk][hkv][d], then the copy
// pass's partial maxima (fwd_v16_parts: the byte offset of those).
size_t fwd_v16_bytes(int64_t Tk, int hkv, int d);
size_t fwd_v16_parts(int64_t Tk, int hkv, int d);

// fp16 operand copies (convert.hip): largest |x| of up to four bf16 tensors
// into range words (range_max), and the tracked copies below.
struct RangeJob {
  int n;
  const void* src[4];
  int64_t chunks[4];  // 16-byte chunks of each tensor
  int word[4];        // its word slot
  uint32_t* words;
};
void launch_range_clear(uint32_t* words, int n, hipStream_t stream);
void launch_range_max(const RangeJob& job, hipStream_t stream);
// v's copy (and k's in the backward): dst = fp16(src * copy_scale) in one
// pass where that scale is 1, two otherwise; words[word] = fp32 bits of
// max |src|, and with clear_others the other three of words[0..3] = 0.
// parts: kVRangeParts words of scratch.
void launch_convert_tracked(const void* src, void* dst, int64_t chunks, uint32_t* parts, uint32_t* words, int word,
                            int L, bool clear_others, hipStream_t stream);

struct FwdLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  void* saved = nullptr;  // device, saved_layout(): filled for the backward, or null
  void* v16 = nullptr;    // device, fwd_v16_bytes(): room for v's fp16 copy when saved is null
  int64_t Tq, Tk;
  int hq, hkv, d;
  float scale, softcap;
  const int32_t* row_ptr;  // device: [n_qtiles + 1]
  const void* entries;     // device: HostDevEntry[]
  const int32_t* order;    // device: [n_qtiles]
  const void* slices;      // device: HostDevSlice[]
  const float* alibi_slopes = nullptr;  // device: [hq], or null for no distance bias
  void* scratch = nullptr;  // device: fwd_scratch_layout(Tq).total bytes (held by the plan)
  // entries and longest list of the q-tile lists when the host knows them
  // (host-built plans), else -1: with them the launch skips the run split
  // when no list can be cut
  int64_t n_entries = -1, max_len = -1;
};

// The forward's scratch (held by the plan): work items and the partial
// results of q tiles cut into several runs.  Independent of the head count
// and head size (sized for the largest).
struct FwdScratchLayout {
  size_t counts, items, splits, partial_lse, partial_o, total;
  int64_t items_cap, splits_cap;
};
FwdScratchLayout fwd_scratch_layout(int64_t Tq);
// Bytes of that scratch a plan whose longest forward list has max_len
// entries needs: no list that short is ever cut into runs, so such a plan
// needs none of the partial-output buffers.
size_t fwd_scratch_bytes(int64_t Tq, int64_t max_len);

struct BwdLaunch {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* saved;  // device, saved_layout(): the training forward's record (never null here)
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  void* workspace;  // device memory laid out by bwd_workspace_layout()
  int64_t Tq, Tk;
  int hq, hkv, d;
  float scale, softcap;
  // key-side plan (dK, dV): per key tile, the q tiles
  const int32_t* kv_row_ptr;
  const void* kv_entries;
  const int32_t* kv_order;
  // query-side plan (dQ): per q tile, the key tiles
  const int32_t* q_row_ptr;
  const void* q_entries;
  const int32_t* q_order;
  const void* slices;
  const float* alibi_slopes = nullptr;  // device: [hq], or null for no distance bias
  int64_t kv_n_entries = -1, kv_max_len = -1;  // key-side lists, as in FwdLaunch
  int64_t q_n_entries = -1, q_max_len = -1;    // dQ lists, as in FwdLaunch
};

int fwd_tile_rows();
int fwd_tile_cols();
hipError_t launch_fwd(const FwdLaunch& p, hipStream_t stream);

// Device-side planner (plan_device.hip).  Status bits in the device word.
enum : int32_t { kPlanBadSlice = 1, kPlanCapacity = 2 };  // FFA_PLAN_* in ffa.h

struct PlanDevicePart {
  int64_t n_tiles;
  int bm, bn;      // row-tile rows, key-tile keys
  bool transpose;  // tiles are key tiles, entries name row tiles
  int64_t cap;     // entry capacity
  int32_t* count;  // scratch [n_tiles]
  int32_t* key;    // scratch [n_tiles]
  int32_t* glen;   // scratch [n_tiles]
  int32_t* row_ptr;  // [n_tiles + 1]
  void* entries;     // HostDevEntry[cap]
  int32_t* order;    // [n_tiles]
};

struct PlanDeviceLaunch {
  const int32_t* q_ranges;  // device [R][2]
  const int32_t* k_ranges;  // device [R][2]
  const int32_t* types;     // device [R]
  int R;
  int64_t Tq, Tk;
  void* slices;     // HostDevSlice[R], indexed by the caller's slice index
  int32_t* rank;    // scratch [R]
  int32_t* status;  // device word: kPlan* bits of the last build
  int n_parts;
  PlanDevicePart part[2];
};

int plan_device_max_slices();
hipError_t launch_plan_device(const PlanDeviceLaunch& L, hipStream_t stream);

int bwd_kv_tile_rows();  // q rows per step of the dK/dV kernel
int bwd_kv_tile_cols();  // keys per dK/dV workgroup
int bwd_q_tile_rows();   // q rows per dQ workgroup
int bwd_q_tile_cols();   // keys per dQ step
hipError_t launch_bwd(const BwdLaunch& p, hipStream_t stream);

// Run split of plan lists (split.hip): the work items of the kernels that
// walk one tile's list per workgroup.  See split.hip for the rule.
struct SplitLaunch {
  const int32_t* row_ptr;  // device: [n_tiles + 1]
  const int32_t* order;    // device: [n_tiles]
  int64_t n_tiles;
  int steps_per_entry, units, min_steps, balance, max_slot_units;
  void* items;             // device: int32x4 [items_cap]
  int64_t items_cap;
  void* splits;            // device: int32x4 [splits_cap]
  int64_t splits_cap;
  int32_t* counts;         // device: [2]
};
struct SplitCaps {
  int64_t items, splits;
};
SplitCaps split_caps(int64_t n_tiles, int units, int balance);
// false when lists of n_entries entries in all, none longer than max_len,
// certainly stay whole under the split rule (n_entries < 0: unknown).
bool split_possible(int64_t n_entries, int64_t max_len, int steps_per_entry, int units, int min_steps,
                    int balance);
void launch_split(const SplitLaunch& s, hipStream_t stream);

// Byte offsets of the backward workspace pieces (each 256-byte aligned):
// the row term D and lse in exp2 units, both [hq][Tq] fp32, two counters, the dK/dV work items and the
// split-tile records (capacities in records), and the fp32 partial sums;
// the range words and scales of the fp16 operand copies, the copies
// themselves (q16, do16 [Tq][hq][d], k16 [Tk][hkv][d]; v's comes with the
// saved record), and room for a forward re-run (its saved record, out and
// lse) when the caller has no saved record.
struct BwdWorkspaceLayout {
  size_t dvec, lse2, counts, items, splits, partial;
  size_t dq_counts, dq_items, dq_splits, dq_partial;
  size_t range, parts, q16, k16, do16, re_saved, re_out, re_lse, total;
  int64_t items_cap, splits_cap;
};
BwdWorkspaceLayout bwd_workspace_layout(int64_t Tq, int64_t Tk, int hq, int hkv, int d);

}  // namespace ffa
