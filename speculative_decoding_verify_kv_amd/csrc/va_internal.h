// Internal declarations shared by the host entry points and the kernel
// launchers of libverify_attn.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "verify_attn.h"

namespace va {

constexpr int kPage = 16;
constexpr int kMaxSplits = 256;
constexpr int kMaxRows = 64;         // B limit of a uniform plan (ancestry bitmask width)
constexpr int kMaxRowsRagged = 4096; // per-sequence row limit of a ragged plan (chains past 64)
constexpr size_t kHeaderBytes = 256; // workspace flag header
// Device memory verify_attn_run_noalloc keeps its split partials in (per GPU)
constexpr size_t kScratchBytes = (size_t)64 << 20;
// Ragged calls: fewest pages a split of a sequence takes (eight 64-token
// tiles).  A sequence shorter than S such splits uses fewer splits, and the
// rest of its workgroups exit at once.  Longer minimum splits cost a short
// sequence's rows some parallelism but save each split's fixed cost (Q
// staging, partial write-back, a workgroup slot) and its partials.
constexpr int kMinSplitPages = 32;
// Ragged plans: most sequences one call may hold (the work-list pass keeps
// a few words per sequence in LDS).
constexpr int kMaxSchedSeqs = 2048;
// Ragged calls: rows whose sequence has at most this many splits are merged
// one wave per (row, head) rather than one workgroup.
constexpr int kMergeLightSplits = 8;

// Ragged work-list entries: (sequence | flags, row group << 16 | split << 8 |
// KV head).  kItemThin marks a sequence of at most kThinRows (row, head)
// pairs, which the partial kernel runs with its 32-row body.
constexpr int kItemSeqMask = 0x3fffffff;
constexpr int kItemThin = 0x40000000;
constexpr int kThinRows = 32;
// The merge's row list of a ragged call: each entry is a packed row with its
// sequence's split count, row | (splits - 1) << kMergeSplitShift (rows stay
// below 2^23: one split's partials are capped at 2^31 bytes at plan time).
constexpr int kMergeSplitShift = 23;
constexpr int kMergeRowMask = (1 << kMergeSplitShift) - 1;
static_assert(((int64_t)(kMaxSplits - 1) << kMergeSplitShift) <= 0x7fffffff, "split count bits overflow");

// Kernel-side dtype codes (same values as va_dtype).
enum : int { kF32 = 0, kF16 = 1, kBF16 = 2, kQ8 = 3 };

// Everything a launch needs; passed to the kernels by value.
struct PartialParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const void* k_scale;
  const void* v_scale;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const int32_t* parent;  // NULL => chain
  const int32_t* cu_rows; // NULL => B rows per sequence; else [num_seqs + 1] packed row offsets
  void* out;              // direct mode output
  float* lse;             // direct mode lse (may be NULL)
  float* part_o;          // [S][nrows][D]
  uint64_t* part_ml;      // [S][nrows] (m, l) pairs: m (log2 units) in the low word, l in the high word
  const int2* items;      // ragged calls: the work list (sequence, row group << 16 | split << 8 | KV head)
  const int32_t* item_count;  // ragged calls: entries of `items` in use
  uint32_t* flags;
  int32_t num_seqs, B, H, KVH, G, D;  // B: rows per sequence (ragged: the largest count)
  int32_t total_rows;     // ragged: capacity of the packed rows
  int32_t num_pages, max_pages, max_ctx;
  int32_t S;              // splits in this launch
  int32_t row_groups;     // workgroups along the B*G rows of one KV head
  int32_t rows_per_group; // 16 * NT
  int32_t q_dtype, out_dtype;
  int32_t direct;         // 1: write out/lse, 0: write partials
  float scale_log2;       // softmax scale * log2(e)
  int64_t nrows;          // num_seqs * B * H
  int32_t item_cap;       // ragged calls: workgroups launched (entries `items` can hold)
};

struct MergeParams {
  const float* part_o;
  const uint64_t* part_ml;
  void* out;
  float* lse;
  const int32_t* merge_rows;  // ragged: packed rows to merge, in order; NULL: row = block / heads
  const int32_t* merge_count; // ragged: [0] entries of merge_rows in use, [1] the leading ones merged by workgroup
  int32_t heads;
  int32_t S, D, out_dtype;
  int64_t nrows;
};

struct AppendParams {
  const void* k_new;      // [num_seqs*B, KVH, D] new_dtype
  const void* v_new;
  void* k_pool;
  void* v_pool;
  void* k_scale;          // 8-bit pools only
  void* v_scale;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  uint32_t* flags;
  int32_t num_seqs, B, KVH, D;
  int32_t num_pages, max_pages, max_ctx;
  int32_t new_dtype, kv_dtype;
};

// Cache-policy operand of the buffer load / store builtins for the bits a
// relaxed system-scope atomic access gets on gfx950 (sc0 sc1), and the
// descriptor flags of a raw buffer (no swizzle, 32-bit format).
constexpr int kSystemScopeBits = 17;
constexpr int kRawBufferFlags = 0x00020000;

struct PromoteParams {
  const int32_t* accepted;   // [num_seqs, B] root-first path rows
  const int32_t* n_accepted; // [num_seqs]
  const int32_t* parent;     // [num_seqs, B] or NULL (chain)
  void* k_pool;
  void* v_pool;
  void* k_scale;             // 8-bit pools only
  void* v_scale;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  int32_t* new_ctx;          // [num_seqs] or NULL
  uint32_t* flags;           // cumulative workspace flag word
  uint32_t* status;          // this call's check word
  char* staging;             // num_seqs * B * KVH * 2 rows of row_bytes
  int64_t row_bytes;
  int32_t num_seqs, B, KVH, D;
  int32_t num_pages, max_pages, max_ctx;
  int32_t esz, kv_is_q8;
};

// The work-list pass of a ragged call (one workgroup, ahead of the partial
// kernel): the partial kernel's items and the merge's row order.
struct ScheduleParams {
  const int32_t* cu_rows;
  const int32_t* ctx_lens;
  int32_t* count;         // [0] items listed, [1] rows listed, [2] of them with more than kMergeLightSplits splits
  int2* items;            // [cap]
  int32_t* merge_rows;    // [total_rows]
  uint32_t* flags;
  int32_t num_seqs, B, total_rows, G, qrows, S, KVH, max_ctx, max_pages, cap;
};

// Tiling the plan picks for the partial kernel.
struct Tiling {
  int nt;          // 16-row MFMA tiles per workgroup (2, 4 or 6)
  int row_groups;  // ceil(B*G / (16*nt))
};

Tiling choose_tiling(int B, int G, int D);
bool partial_supported(int D, int kv_dtype, int nt);

hipError_t launch_partial(const PartialParams& p, int kv_dtype, int nt, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);
hipError_t launch_schedule(const ScheduleParams& p, hipStream_t stream);
hipError_t launch_append(const AppendParams& p, hipStream_t stream);
size_t promote_row_bytes(int D, int kv_dtype);
hipError_t launch_promote(const PromoteParams& p, hipStream_t stream);
// True when the call runs as one launch (the batch's staging fits in LDS).
bool promote_one_launch(const PromoteParams& p);

}  // namespace va

struct va_plan {
  va_problem prob;
  int32_t num_splits;       // heuristic (or requested) S
  int32_t max_splits;       // workspace sized for this many
  int32_t num_cus;
  va::Tiling tiling;
  float scale;              // resolved softmax scale
  size_t workspace_bytes;
};
