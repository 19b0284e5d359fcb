/*
 * ffa.h -- C ABI of the MI355X (gfx950) range-masked ("flex") flash attention library.
 *
 * The operation: attention over packed, variable-length tokens whose mask is
 * a list of slices.  Slice r covers query rows [q_ranges[r][0], q_ranges[r][1])
 * and key columns [k_ranges[r][0], k_ranges[r][1]); attn_type_map[r] is
 * FFA_FULL (every cell of that rectangle is visible) or FFA_CAUSAL (cell
 * (i, j) is visible iff j - ke <= i - qe: the causal diagonal runs through
 * the rectangle's bottom-right corner).  A slice whose q range or k range is
 * empty (start == end) covers nothing and costs nothing, so callers may pad
 * the slice list to a fixed length with such rows.  These are the
 * q_ranges / k_ranges / attn_type_map arguments of flex_flash_attn_func in the
 * MagiAttention issue "Using dummy/padded attention slices with
 * flex_flash_attn_func for torch.compile static shapes" (repro script: int32
 * [R,2] ranges, 0 = FULL, 1 = CAUSAL; maintainer reply: zero-area slices are
 * skipped).
 *
 * Per q head h (kv head g = h / (hq / hkv)) and query row i:
 *   u_ij  = scale * <q_i, k_j>
 *   s_ij  = softcap > 0 ? softcap * tanh(u_ij / softcap) : u_ij   (masked cells: -inf)
 *   lse_i = log(sum_j exp(s_ij))                                  (natural log)
 *   out_i = sum_j exp(s_ij - lse_i) v_j
 * A row with no visible key gets out = 0 and lse = -inf.
 *
 * Conventions shared by every entry point:
 *  - Tensors are packed token-major ("THD"): q, out, dq, do are [Tq][hq][d],
 *    k, v, dk, dv are [Tk][hkv][d], all bf16 and densely contiguous; lse is
 *    fp32 [Tq][hq].  Device pointers, allocated and owned by the caller; the
 *    library keeps none of them after the call returns.  Inputs are never
 *    written.  Inputs must be finite.
 *  - q_ranges, k_ranges (int32 [R][2]) and attn_type_map (int32 [R]) are HOST
 *    arrays, read before the call returns.  Slices may come in any order; no
 *    (i, j) cell may be covered by two slices.
 *  - d is 64 or 128; hq is a positive multiple of hkv; scale > 0 and finite;
 *    softcap >= 0 and finite (0 = off).  Tq, Tk >= 0 and every tensor must be
 *    below 2^31 elements.
 *  - Device pointers must be 16-byte aligned.
 *  - Environment: FFA_DEBUG=1 makes planning reject slice lists in which two
 *    slices cover one cell (FFA_ERR_INVALID_ARG); FFA_INJECT_NOMEM=1 makes
 *    every host-side planning step fail with FFA_ERR_NOMEM, for testing a
 *    caller's handling of that error; FFA_FWD_PAIRED=1 / =0 makes the
 *    forward take two q heads per workgroup wherever q heads pair up within
 *    a kv head, or never, instead of choosing by grid size (the results are
 *    the same bits either way).
 *  - stream is a hipStream_t (NULL = the default stream).  Calls enqueue work
 *    and return; argument errors are reported synchronously before any GPU
 *    work is enqueued.  The return value is FFA_OK or a negative FFA_ERR_*;
 *    ffa_last_error() then describes the failure (thread-local).
 */
#ifndef FFA_H
#define FFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* attn_type_map values (repro script: 0 = FULL, 1 = CAUSAL) */
enum { FFA_FULL = 0, FFA_CAUSAL = 1 };

/* status codes */
enum {
  FFA_OK = 0,
  FFA_ERR_INVALID_ARG = -1, /* bad shape, range, type, scale or softcap */
  FFA_ERR_UNSUPPORTED = -2, /* valid but not built (e.g. head size 96) */
  FFA_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed */
  FFA_ERR_NOMEM = -4        /* host or device allocation failed */
};

/*
 * ffa_fwd -- forward pass: out and lse.
 *
 * Plans the block-sparse work on the host (drops empty slices, lists for each
 * 128-row q tile the 64-column k tiles any slice makes visible, FULL or
 * PARTIAL; FlexAttention paper summary, section 4, block sparsity and the
 * full-block optimisation), uploads the plan on `stream`, and runs one fused
 * kernel.  out: bf16 [Tq][hq][d], lse: fp32 [Tq][hq], both written in full
 * (rows nothing sees included).  Deterministic: the same inputs give the
 * same bits, also when empty slices are added anywhere or the slices are
 * permuted.
 *
 * Precision.  QK^T runs on bf16 operands, P V on fp16 ones, both with fp32
 * accumulation.  fp16 gives the probabilities 11 significant bits instead of
 * bf16's 8: each enters P V rounded while out is divided by the sum of the
 * unrounded ones, which with bf16 can move out by up to 2^-9 max |v|.  v is
 * copied to fp16 first (exact: at scale 1 when max |v| lies in [2^-3, 16),
 * else times the power of two that maps max |v| into [8, 16)), into
 * stream-ordered device memory (2 Tk hkv d bytes) allocated on `stream` and
 * released after the kernel.
 */
int ffa_fwd(const void* q, const void* k, const void* v,
            int64_t Tq, int64_t Tk, int hq, int hkv, int d,
            const int32_t* q_ranges, const int32_t* k_ranges,
            const int32_t* attn_type_map, int R,
            float scale, float softcap,
            void* out, float* lse,
            void* stream);

/*
 * ffa_bwd_workspace_size -- bytes of device workspace ffa_bwd and
 * ffa_bwd_planned need for these sizes (0 for invalid sizes or Tq == Tk == 0):
 * the fp32 row term D = rowsum(dO * out) and a copy of lse, [hq][Tq] each, the work lists of the
 * dK/dV and dQ passes, and fp32 partial sums for tiles whose list is cut
 * into several runs (a list much longer than the average, e.g. a key block
 * every query sees or a short query block against a long context): at most
 * 512 runs x kv heads of 128 keys x d x 2 (present when Tk > 0) plus 512
 * runs x q heads of 128 rows x d (present when Tq > 0), 96 MiB in all at
 * d = 128; fp16 copies of q, k and dO (2 bytes per element each); and
 * room for re-running the forward when no saved record is given (a record of
 * ffa_saved_size bytes, out and lse).  At the 64K-token, 32/8-head, d = 128
 * size that is about 2.3 GB.  The contents need no initialisation and are
 * scratch after the call.
 */
size_t ffa_bwd_workspace_size(int64_t Tq, int64_t Tk, int hq, int hkv, int d);

/*
 * ffa_bwd -- backward pass of ffa_fwd for upstream gradient `dout`.
 *
 * Inputs q, k, v, out (bf16) and lse (fp32) are those of the forward call
 * with the same slices, scale and softcap.  Writes dq [Tq][hq][d] and dk, dv
 * [Tk][hkv][d] (bf16) in full, zeros where a row or key takes part in no
 * visible cell.  dk and dv of a kv head sum over the q heads that read it.
 * `workspace` is 16-byte aligned device memory of
 * ffa_bwd_workspace_size(Tq, Tk, hq, hkv, d) bytes (or NULL: then the
 * library allocates it on `stream`).  Deterministic: the same inputs give
 * the same bits, whatever the order in which workgroups run.
 *
 * Precision.  The products run on the matrix cores with fp16 operands
 * (11 significant bits) and fp32 accumulation: q, k, v and dout are copied
 * to fp16, each times a power of two that fits its largest |x| into fp16's
 * range (exact; v's copy is the forward's), and P and dS are rounded to
 * fp16 for the second products.  The row term D = rowsum(dout * out) needs out more precisely
 * than bf16 holds it: ffa_bwd (no saved record) re-runs the forward into the
 * workspace in its training form (see ffa_fwd_ex, `saved`), which costs one
 * forward pass; ffa_bwd_ex takes the record a training forward saved and
 * skips that.
 */
int ffa_bwd(const void* q, const void* k, const void* v,
            const void* out, const float* lse, const void* dout,
            int64_t Tq, int64_t Tk, int hq, int hkv, int d,
            const int32_t* q_ranges, const int32_t* k_ranges,
            const int32_t* attn_type_map, int R,
            float scale, float softcap,
            void* dq, void* dk, void* dv,
            void* workspace, size_t workspace_bytes,
            void* stream);

/*
 * ffa_fwd_noalloc -- ffa_fwd for callers that cannot allocate: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, results (bitwise) and errors as ffa_fwd, and it allocates
 * nothing: the slice arrays' device copy, the block-sparse plan (built on
 * the device from that copy), the forward's run scratch and the fp16 copy of
 * v live in one 256 MiB device array of the library's (each GPU holds its
 * own copy from the first call on it until the process ends).  The slice
 * arrays are copied to it with hipMemcpyAsync on `stream`.  Limits, checked
 * on the host before any GPU work (FFA_ERR_INVALID_ARG): at most 4096
 * slices, v's fp16 copy (2 Tk hkv d bytes) and the run scratch (about
 * 32 MiB) must fit the array, and the plan must fit what is left: about
 * 10 million (q tile, key tile, slice) entries at Tk hkv d = 64M (the
 * 64K-token, 8-kv-head, d = 128 size), more for smaller v (the message gives
 * the counts).  Overlapping
 * slices are not looked for under FFA_DEBUG.  All calls on one GPU share the
 * array: calls that overlap in time on one GPU (different streams, or
 * different host threads) race and must not be made.
 */
int ffa_fwd_noalloc(const void* q, const void* k, const void* v,
                    int64_t Tq, int64_t Tk, int hq, int hkv, int d,
                    const int32_t* q_ranges, const int32_t* k_ranges,
                    const int32_t* attn_type_map, int R,
                    float scale, float softcap,
                    void* out, float* lse,
                    void* stream);

/*
 * Distance bias (ALiBi).  The FlexAttention paper summary lists ALiBi among
 * the attention variants as a bias that depends on the distance between the
 * query and key positions (section 2; section 3.1, a position-dependent score
 * bias).  The _ex entry points take it as one fp32 slope per q head:
 *   s_ij += alibi_slopes[h] * (j - i)      (after the softcap, before the mask)
 * with i and j the token indices along the q and k axes.  With slope > 0 on a
 * causal mask (j <= i) this is ALiBi's linear penalty on distance.
 *   alibi_slopes  DEVICE pointer to hq finite fp32 values, 4-byte aligned,
 *                 read by the kernels (left alone); NULL = no bias, which is
 *                 exactly the entry point without _ex.
 * lse includes the bias.  The bias is formed as slope * (j - i) in fp32 from
 * the exact integer j - i; where every visible key of a row is far from it
 * (|slope * (j - i)| in the thousands), lse itself is large and carries fp32
 * rounding of that size.
 *
 * Training forward (saved record).  A forward whose backward will follow
 * can save what that backward needs:
 *   saved         DEVICE memory of ffa_saved_size(Tq, Tk, hq, hkv, d) bytes,
 *                 16-byte aligned, or NULL (the plain forward).  With it the
 *                 forward puts v's fp16 copy (see Precision under ffa_fwd)
 *                 into the record instead of temporary memory, and stores
 *                 out's bf16 rounding residual bf16(x - out) for each fp32
 *                 result x; out and lse are the plain forward's bits.
 * The _ex backward takes the record (NULL: re-run the training forward to
 * get one, see ffa_bwd) and forms D = rowsum(dout * (out + residual)) from
 * it, reusing the fp16 v.  A record belongs to the q, k, v, slices, scale,
 * softcap and slopes of its forward.  Errors as for the entry points without
 * _ex.
 */
int ffa_fwd_ex(const void* q, const void* k, const void* v,
               int64_t Tq, int64_t Tk, int hq, int hkv, int d,
               const int32_t* q_ranges, const int32_t* k_ranges,
               const int32_t* attn_type_map, int R,
               float scale, float softcap, const float* alibi_slopes,
               void* out, float* lse, void* saved, void* stream);

/* Bytes of the training forward's saved record (0 for invalid sizes): a
 * 256-byte header, out's residual (2 bytes per element of q), the fp16 copy
 * of v (2 bytes per element of v), each 256-byte aligned, and 8 KiB of
 * scratch for the pass that makes the copy. */
size_t ffa_saved_size(int64_t Tq, int64_t Tk, int hq, int hkv, int d);

int ffa_bwd_ex(const void* q, const void* k, const void* v,
               const void* out, const float* lse, const void* saved,
               const void* dout,
               int64_t Tq, int64_t Tk, int hq, int hkv, int d,
               const int32_t* q_ranges, const int32_t* k_ranges,
               const int32_t* attn_type_map, int R,
               float scale, float softcap, const float* alibi_slopes,
               void* dq, void* dk, void* dv,
               void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * ffa_plan_host -- the block-sparse plan, on the host only (no GPU call).
 *
 * For tiles of bm query rows by bn key columns, lists every (tile, other
 * tile, slice) triple where slice r makes at least one cell visible.  With
 * transpose == 0 the tiles are q tiles and the other tiles k tiles (the
 * forward's list); with transpose == 1 it is the reverse (the key-side list
 * the backward walks).  Kind 0 (FULL) means slice r makes every cell of the
 * whole bm x bn tile visible, kind 1 (PARTIAL) means the kernel must mask.
 * Empty slices are dropped; r indexes the caller's slice list.
 *
 * row_ptr    [n_tiles + 1] CSR offsets (may be NULL)
 * entries    [cap][3] int32 (other_tile, r, kind), sorted within each tile
 *            by other_tile and then by the slice's bounds (may be NULL)
 * order      [n_tiles] the order the kernels take tiles in (may be NULL):
 *            tiles are grouped by the smallest slice start row (qs) among
 *            the slices in their list, groups by descending longest list,
 *            tiles within a group by descending entry count, then by index
 * Returns the number of entries (>= 0, even when cap is too small: call with
 * cap = 0 to size the buffers) or a negative FFA_ERR_*.
 */
int64_t ffa_plan_host(int64_t Tq, int64_t Tk,
                      const int32_t* q_ranges, const int32_t* k_ranges,
                      const int32_t* attn_type_map, int R,
                      int bm, int bn, int transpose,
                      int64_t* row_ptr, int32_t* entries, int64_t cap,
                      int32_t* order);

/*
 * ffa_block_slices -- slices for a BlockMask-style block list (host only).
 *
 * The FlexAttention paper summary (section 4, block sparsity) describes the
 * BlockMask: per query block, the number of key blocks that are not masked
 * and their indices, which need not be contiguous.  Here query block b
 * (rows [b*block_q, (b+1)*block_q), clipped to Tq) sees every cell of the
 * key blocks kv_indices[b*max_blocks .. b*max_blocks + kv_num_blocks[b])
 * (keys [kb*block_k, (kb+1)*block_k), clipped to Tk); listed blocks are fully
 * visible.  The result is a list of disjoint FULL slices covering exactly
 * those cells, for ffa_fwd / ffa_bwd / ffa_plan_create: adjacent key blocks
 * merge into one key range and a key range repeated over consecutive query
 * blocks into one slice.  Slices are sorted by (q start, k start).
 *
 * kv_num_blocks  [ceil(Tq / block_q)] int32, each in [0, max_blocks]
 * kv_indices     [ceil(Tq / block_q)][max_blocks] int32; the first
 *                kv_num_blocks[b] of row b are distinct key block indices in
 *                [0, ceil(Tk / block_k)), any order; the rest is ignored
 * q_ranges, k_ranges [cap][2], attn_type_map [cap] int32 outputs (any may
 *                be NULL); the first min(R, cap) slices are written
 * Returns R >= 0, the number of slices (call with cap = 0 to size the
 * outputs), or FFA_ERR_INVALID_ARG for a bad count, index or repeat.
 */
int64_t ffa_block_slices(int64_t Tq, int64_t Tk, int block_q, int block_k,
                         const int32_t* kv_num_blocks, const int32_t* kv_indices,
                         int max_blocks, int32_t* q_ranges, int32_t* k_ranges,
                         int32_t* attn_type_map, int64_t cap);

/*
 * Plans that outlive one call.  A plan depends only on Tq, Tk and the slice
 * list (not on heads, head size, scale or data), so callers whose layers
 * share one mask plan once and launch many times.
 */
typedef struct ffa_plan_s* ffa_plan_t;

/*
 * ffa_plan_create -- validate the slices, build the forward (per q tile) and
 * backward (per key tile) block lists on the host and copy them to device
 * memory on `stream`.  *plan receives the handle.  Use the plan on `stream`
 * (or after synchronising with it).  Errors as for ffa_fwd.
 *
 * The plan also holds the forward's scratch (about 32 MiB, reserved only
 * when some q tile's list is longer than 64 key tiles): a q tile whose list
 * is longer than one workgroup slot's share of the work (a short query
 * block against a long context) is walked by several workgroups whose
 * partial outputs are merged by their lse, in a fixed order.  Forward calls
 * on one plan therefore must not run concurrently on different streams;
 * backward calls keep their own workspace.
 */
int ffa_plan_create(int64_t Tq, int64_t Tk,
                    const int32_t* q_ranges, const int32_t* k_ranges,
                    const int32_t* attn_type_map, int R,
                    void* stream, ffa_plan_t* plan);

/* ffa_fwd with a plan from ffa_plan_create: launches the forward kernels
 * only (no host planning, no host copy).  Tensors as for ffa_fwd.  The fp16
 * copy of v that the kernel reads goes to room the plan keeps for it
 * (2 Tk hkv d bytes and 8.25 KiB): allocated stream-ordered on `stream` by the
 * first call that needs it (or needs more), and freed by ffa_plan_destroy.
 * With a saved record (ffa_fwd_planned_ex) the copy goes to the record
 * instead and nothing is allocated; ffa_fwd_noalloc allocates nothing
 * either. */
int ffa_fwd_planned(ffa_plan_t plan,
                    const void* q, const void* k, const void* v,
                    int hq, int hkv, int d, float scale, float softcap,
                    void* out, float* lse, void* stream);

/* ffa_bwd with a plan from ffa_plan_create: launches the backward kernels
 * only.  With workspace == NULL it allocates one on `stream`. */
int ffa_bwd_planned(ffa_plan_t plan,
                    const void* q, const void* k, const void* v,
                    const void* out, const float* lse, const void* dout,
                    int hq, int hkv, int d, float scale, float softcap,
                    void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ffa_fwd_planned / ffa_bwd_planned with the distance bias and the saved
 * record of ffa_fwd_ex / ffa_bwd_ex (alibi_slopes: device, hq fp32 slopes,
 * or NULL; saved: device, ffa_saved_size bytes, or NULL).  Without a record
 * the backward re-runs the forward on the plan (so it uses the plan's
 * forward scratch: see ffa_plan_create). */
int ffa_fwd_planned_ex(ffa_plan_t plan,
                       const void* q, const void* k, const void* v,
                       int hq, int hkv, int d, float scale, float softcap,
                       const float* alibi_slopes,
                       void* out, float* lse, void* saved, void* stream);

int ffa_bwd_planned_ex(ffa_plan_t plan,
                       const void* q, const void* k, const void* v,
                       const void* out, const float* lse, const void* saved,
                       const void* dout,
                       int hq, int hkv, int d, float scale, float softcap,
                       const float* alibi_slopes,
                       void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Release a plan: its device memory is freed in order on `stream`, after the
 * work already enqueued there (a plan from ffa_plan_create_device lives in
 * the caller's workspace, which is left alone; its room for v's fp16 copy,
 * if a forward allocated one, is freed).  NULL is a no-op. */
int ffa_plan_destroy(ffa_plan_t plan, void* stream);

/*
 * Plans built on the device.  The slice arrays of flex_flash_attn_func are
 * device tensors in the MagiAttention issue on dummy/padded slices (padded
 * to a fixed count for torch.compile).  ffa_plan_create_device builds the
 * same plan as ffa_plan_create (the same entries in the same order, and the
 * same tile order) with kernels that read those arrays in device memory: no
 * host copy, no synchronisation, no allocation.  ffa_plan_refresh re-runs
 * the build on the current contents of the same arrays, so a sequence
 * "refresh, forward into a saved record, backward on that record" (calls
 * that allocate nothing when given the record and a workspace) can be
 * captured once in a HIP graph and replayed for every new slice list of the
 * same length.
 *
 * q_ranges [R][2], k_ranges [R][2], attn_type_map [R]: DEVICE int32 arrays,
 *            4-byte aligned, read by every build; they must stay valid
 *            (and keep their address) until the plan is destroyed.
 * R          0 .. 4096 slices (FFA_ERR_INVALID_ARG above).
 * max_entries  capacity of each of the plan's two block lists, in entries
 *            (0 .. 2^30 - 1).  A list needs one entry per (tile, other tile,
 *            slice) triple with a visible cell; ffa_plan_host gives the
 *            exact count for a slice list.  A build that needs more leaves
 *            the plan empty and sets FFA_PLAN_CAPACITY in its status.
 * workspace  device memory of at least ffa_plan_device_workspace_size()
 *            bytes, 256-byte aligned, owned by the caller, holding the plan
 *            and the forward's scratch (about 32 MiB, as for ffa_plan_create:
 *            forward calls on one plan must not overlap across streams); it
 *            must outlive the plan and not be shared with another plan.
 * Validation of Tq, Tk, R, max_entries and the pointers is synchronous (the
 * usual FFA_ERR_* codes).  The slice values are only seen by the kernels: a
 * slice with start > end, a range outside [0, T) or a type other than 0/1
 * leaves the plan empty and sets FFA_PLAN_BAD_SLICE.  An empty plan makes
 * the attention calls write out = 0, lse = -inf, zero gradients.  Slices
 * must not overlap, as for ffa_fwd (not checked on the device).
 * The build is enqueued on `stream`; use the plan on that stream.
 */
enum {
  FFA_PLAN_BAD_SLICE = 1, /* a slice failed validation */
  FFA_PLAN_CAPACITY = 2   /* a block list needed more than max_entries */
};

int ffa_plan_device_workspace_size(int64_t Tq, int64_t Tk, int R, int64_t max_entries,
                                   size_t* bytes);

int ffa_plan_create_device(int64_t Tq, int64_t Tk,
                           const int32_t* q_ranges, const int32_t* k_ranges,
                           const int32_t* attn_type_map, int R, int64_t max_entries,
                           void* workspace, size_t workspace_bytes,
                           void* stream, ffa_plan_t* plan);

/* Re-run the device build of a plan from ffa_plan_create_device on the
 * current contents of its slice arrays (enqueue only; capturable).
 * FFA_ERR_INVALID_ARG for a plan built on the host. */
int ffa_plan_refresh(ffa_plan_t plan, void* stream);

/* Status bits (FFA_PLAN_*) of the last device build; 0 if it succeeded or
 * if the plan was built on the host.  Synchronises with `stream`. */
int ffa_plan_status(ffa_plan_t plan, void* stream, int* status);

/*
 * ffa_plan_export -- copy one block list of a plan back to the host, in the
 * format of ffa_plan_host: which = 0 the forward list (per q tile), 1 the
 * key-side list of dK/dV, 2 the q-tile list of the dQ pass.  *n_tiles
 * receives the number of tiles; row_ptr [n_tiles + 1], entries [cap][3]
 * (other_tile, caller's slice index, kind), order [n_tiles]; any pointer may
 * be NULL (call once with NULLs to size the buffers).  Returns the number of
 * entries or a negative FFA_ERR_*.  Synchronises with `stream`.
 */
int64_t ffa_plan_export(ffa_plan_t plan, int which, int64_t* n_tiles, int64_t* row_ptr,
                        int32_t* entries, int64_t cap, int32_t* order, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* ffa_last_error(void);

/* Build facts: target architecture, tile sizes, a hash of the sources the
 * library was built from (source=, 16 hex digits) and the compiler (cf. the
 * build-flag file exposed at run time in flash-attention PR "Add
 * torch.compile support to flash attention 3").  A static string owned by
 * the library. */
const char* ffa_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* FFA_H */
