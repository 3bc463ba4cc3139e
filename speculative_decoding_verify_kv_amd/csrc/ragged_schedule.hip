// Work list of a ragged verify call, gfx950.
//
// A ragged call splits each sequence by its own context (at least
// kMinSplitPages pages per split), so the (sequence, row group, split, KV
// head) items of one call differ in size and number from call to call, and
// only the device knows them (cu_rows and ctx_lens live there).  This pass
// runs ahead of the partial kernel, as one wave for calls of up to 64
// sequences and as one workgroup of 1,024 threads for more, and lists:
//   * the items, densely from item 0: workgroups are dealt to the 8 XCDs
//     round-robin by block id, so a dense list spreads the work evenly over
//     them, where a grid holding every possible item would leave the empty
//     ones (which exit at once) between the real ones and pile more than 32
//     real workgroups on some XCDs;
//   * longest first: sequences in decreasing order of split count (then of
//     pages per split, then by index), each sequence's items by split, row
//     group and KV head, so a call that takes more than one wave of
//     workgroups starts its long items first (a sequence with more than the
//     minimum pages per split has about S splits, the most there are);
//   * a sequence of at most kThinRows (row, head) pairs has its items marked
//     thin (when the plan's row groups are larger), and the partial kernel
//     runs them with its 32-row body;
//   * the packed rows for the merge in the same sequence order, each with its
//     sequence's split count (the merge weighs no later split): rows of
//     sequences with many splits, whose merge reads the most, first, then
//     the rows with at most kMergeLightSplits splits, which the merge takes
//     one wave per (row, head) instead of a workgroup.
// Sequences are taken in index order while their rows fit the packed
// capacity and their items the grid (only overlapping bad cu_rows entries
// can exceed either).  Which items a sequence has, and what each computes,
// follow from that sequence's context, the plan and the call's split count
// alone, so its outputs do not depend on the other sequences of the call
// (page "perf(qwen35): retain speculation during paged prefill", Correctness
// failure found during qualification); the order only decides when each
// item runs.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "va_internal.h"

namespace va {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kSortSeqs = 256;  // sequences ordered by size up to this count; beyond it, by index

struct SeqInfo {
  int rows, a, groups, splits, items, pp;
};

// The first word of a sequence's items: its index, and kItemThin for a
// sequence the partial kernel runs with its 32-row body.
__device__ __forceinline__ int item_seq_word(const ScheduleParams& p, int s, int rows) {
  return s | (p.qrows > kThinRows && rows * p.G <= kThinRows ? kItemThin : 0);
}

// cu: the call's cu_rows and ctx: its ctx_lens, staged in LDS
__device__ __forceinline__ SeqInfo seq_info(const ScheduleParams& p, const int* cu, const int* ctxs, int s) {
  SeqInfo q;
  const int a = cu[s], e = cu[s + 1];
  const bool bad = a < 0 || e < a || e > p.total_rows || e - a > p.B;
  q.rows = bad ? 0 : e - a;
  q.a = a;
  q.groups = (q.rows * p.G + p.qrows - 1) / p.qrows;
  // the partial kernel's split rule for this sequence (a bad context keeps
  // split 0 alone, which reports it)
  const int ctx = ctxs[s];
  const bool ctx_bad = ctx < q.rows || ctx > p.max_ctx || ctx > p.max_pages * kPage;
  const int np = ctx_bad ? 0 : (ctx + kPage - 1) / kPage;
  q.pp = max((np + p.S - 1) / p.S, kMinSplitPages);
  q.splits = max(1, (np + q.pp - 1) / q.pp);
  q.items = q.groups * q.splits * p.KVH;
  return q;
}

// first r in [0, n) with pre[r] > x (pre inclusive, non-decreasing; x < pre[n-1])
__device__ __forceinline__ int upper_rank(const int* pre, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] > x) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// Block-wide inclusive scan of one value per thread (kSchedThreads threads).
__device__ __forceinline__ int64_t block_scan(int64_t v, int64_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  __syncthreads();
  return before + inc;
}

__global__ __launch_bounds__(kSchedThreads) void ragged_schedule_kernel(const ScheduleParams p) {
  __shared__ int cu[kMaxSchedSeqs + 1];
  __shared__ int ctxs[kMaxSchedSeqs];
  __shared__ int key[kMaxSchedSeqs];
  __shared__ int order[kMaxSchedSeqs];
  __shared__ int pre_items[kMaxSchedSeqs];
  __shared__ int pre_rows[kMaxSchedSeqs];
  __shared__ int64_t wsum[kSchedThreads / 64];
  const int tid = threadIdx.x;
  const int n = p.num_seqs;
  for (int s = tid; s <= n; s += kSchedThreads) {
    cu[s] = p.cu_rows[s];
    if (s < n) ctxs[s] = p.ctx_lens[s];
  }
  __syncthreads();

  // Which sequences the list takes: in sequence order, as long as their rows
  // fit the packed capacity and their entries the grid (cu_rows entries that
  // are each valid but overlap can claim more; the sequences past that point
  // are left out, unwritten).  Then the sort keys: pages per split, then
  // split count (0: no entries).  Each thread takes a run of consecutive
  // sequences.
  const int per = (n + kSchedThreads - 1) / kSchedThreads;
  const int r0 = min(n, tid * per), r1 = min(n, r0 + per);
  int bad = 0;
  {
    int64_t my_items = 0, my_rows = 0;
    for (int s = r0; s < r1; ++s) {
      const SeqInfo q = seq_info(p, cu, ctxs, s);
      const int a = cu[s], e = cu[s + 1];
      bad |= (a < 0 || e < a || e > p.total_rows || e - a > p.B);
      my_items += q.items;
      my_rows += q.rows;
    }
    int64_t ib = block_scan(my_items, wsum) - my_items;
    int64_t rb = block_scan(my_rows, wsum) - my_rows;
    for (int s = r0; s < r1; ++s) {
      const SeqInfo q = seq_info(p, cu, ctxs, s);
      ib += q.items;
      rb += q.rows;
      const bool fits = ib <= (int64_t)p.cap && rb <= (int64_t)p.total_rows;
      key[s] = (fits && q.items > 0) ? (q.splits << 21) + min(q.pp, (1 << 21) - 1) : 0;
    }
  }
  if (__syncthreads_or(bad) && tid == 0) atomicOr(p.flags, (uint32_t)VA_FLAG_BAD_ROWS);

  // rank of each sequence: larger key first, ties by index
  for (int s = tid; s < n; s += kSchedThreads) {
    int r = s;
    if (n <= kSortSeqs) {
      const int k = key[s];
      r = 0;
      for (int j = 0; j < n; ++j) {
        const int kj = key[j];
        r += (kj > k) || (kj == k && j < s);
      }
    }
    order[r] = s;
  }
  __syncthreads();

  // entries and rows up to each rank (the sequences taken fit both
  // capacities, so these stay within them), and the rows of sequences with
  // more than kMergeLightSplits splits (they lead the order)
  {
    int my_items = 0, my_rows = 0, my_heavy = 0;
    for (int r = r0; r < r1; ++r) {
      const int s = order[r];
      const SeqInfo q = seq_info(p, cu, ctxs, s);
      my_items += key[s] ? q.items : 0;
      my_rows += key[s] ? q.rows : 0;
      my_heavy += (key[s] && q.splits > kMergeLightSplits) ? q.rows : 0;
    }
    int ib = (int)(block_scan(my_items, wsum) - my_items);
    int rb = (int)(block_scan(my_rows, wsum) - my_rows);
    const int heavy = (int)block_scan(my_heavy, wsum);
    for (int r = r0; r < r1; ++r) {
      const int s = order[r];
      const SeqInfo q = seq_info(p, cu, ctxs, s);
      ib += key[s] ? q.items : 0;
      rb += key[s] ? q.rows : 0;
      pre_items[r] = ib;
      pre_rows[r] = rb;
    }
    if (tid == kSchedThreads - 1) p.count[2] = heavy;
  }
  __syncthreads();
  const int total_items = n > 0 ? pre_items[n - 1] : 0;
  const int total_rows = n > 0 ? pre_rows[n - 1] : 0;
  if (tid == 0) {
    p.count[0] = total_items;
    p.count[1] = total_rows;
  }

  // the items, longest sequences first
  for (int i = tid; i < total_items; i += kSchedThreads) {
    const int r = upper_rank(pre_items, n, i);
    const int s = order[r];
    const SeqInfo q = seq_info(p, cu, ctxs, s);
    const int t = i - (r > 0 ? pre_items[r - 1] : 0);
    const int per_split = q.groups * p.KVH;
    const int split = t / per_split, rem = t - split * per_split;
    const int g = rem / p.KVH, kvh = rem - g * p.KVH;
    p.items[i] = make_int2(item_seq_word(p, s, q.rows), (g << 16) | (split << 8) | kvh);
  }
  // the packed rows to merge, in the same sequence order
  for (int k = tid; k < total_rows; k += kSchedThreads) {
    const int r = upper_rank(pre_rows, n, k);
    const int s = order[r];
    const SeqInfo q = seq_info(p, cu, ctxs, s);
    p.merge_rows[k] = (q.a + (k - (r > 0 ? pre_rows[r - 1] : 0))) | ((q.splits - 1) << kMergeSplitShift);
  }
}

// The same list for calls of at most 64 sequences, by one wave: a lane per
// sequence, the sort and the sums across lanes, no barriers.  (The block
// form spends several microseconds on its passes and barriers; a ragged
// call usually holds a few sequences.)
__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

__global__ __launch_bounds__(64) void ragged_schedule_wave_kernel(const ScheduleParams p) {
  const int lane = threadIdx.x;
  const int n = p.num_seqs;
  const bool live = lane < n;
  int a = 0, e = 0, ctx = 0;
  if (live) {
    a = p.cu_rows[lane];
    e = p.cu_rows[lane + 1];
    ctx = p.ctx_lens[lane];
  }
  const bool bad = live && (a < 0 || e < a || e > p.total_rows || e - a > p.B);
  const int rows = (live && !bad) ? e - a : 0;
  const int groups = (rows * p.G + p.qrows - 1) / p.qrows;
  const bool ctx_bad = ctx < rows || ctx > p.max_ctx || ctx > p.max_pages * kPage;
  const int np = ctx_bad ? 0 : (ctx + kPage - 1) / kPage;
  const int pp = max((np + p.S - 1) / p.S, kMinSplitPages);
  const int splits = max(1, (np + pp - 1) / pp);
  const int items = groups * splits * p.KVH;
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) atomicOr(p.flags, (uint32_t)VA_FLAG_BAD_ROWS);
  // taken while the rows and entries so far (sequence order) fit
  const int64_t ib = wave_incl_scan(items, lane), rb = wave_incl_scan(rows, lane);
  const bool fits = ib <= (int64_t)p.cap && rb <= (int64_t)p.total_rows;
  const int key = (fits && items > 0) ? (splits << 21) + min(pp, (1 << 21) - 1) : 0;
  // rank: larger key first, ties by index; then lane r holds the rank-r sequence
  int rank = 0;
  for (int j = 0; j < n; ++j) {
    const int kj = __builtin_amdgcn_readlane(key, j);
    rank += (kj > key) || (kj == key && j < lane);
  }
  if (!live) rank = lane;  // lanes past the sequences keep their place
  const int s = __builtin_amdgcn_ds_permute(4 * rank, lane);  // order[rank] = lane
  // (every lane takes part in each exchange: a lane left out of one
  // supplies no value to the lanes that read from it)
  const int key_r = __shfl(key, s);
  const int items_s = __shfl(items, s);
  const int rows_s = __shfl(rows, s);
  const int items_r = key_r ? items_s : 0;
  const int rows_r = key_r ? rows_s : 0;
  const int groups_r = __shfl(groups, s);
  const int splits_r = __shfl(splits, s);
  const int a_r = __shfl(a, s);
  const int pre_i = (int)wave_incl_scan(items_r, lane) - items_r;  // exclusive
  const int pre_r = (int)wave_incl_scan(rows_r, lane) - rows_r;
  const int heavy = (int)wave_incl_scan((live && splits_r > kMergeLightSplits) ? rows_r : 0, lane);
  if (lane == 63) {
    p.count[0] = pre_i + items_r;
    p.count[1] = pre_r + rows_r;
    p.count[2] = heavy;
  }
  for (int r = 0; r < n; ++r) {
    const int cnt = __builtin_amdgcn_readlane(items_r, r);
    const int base = __builtin_amdgcn_readlane(pre_i, r);
    const int sq = item_seq_word(p, __builtin_amdgcn_readlane(s, r), __builtin_amdgcn_readlane(rows_r, r));
    const int groups_q = __builtin_amdgcn_readlane(groups_r, r);
    // entry t of the sequence is (split, group, KV head) = t in the mixed
    // radix (groups, KVH), counted incrementally: lane t starts at its own
    // digits, then each step of 64 entries adds the digits of 64
    const int per_split = groups_q * p.KVH;
    int split = lane / per_split, rem = lane - split * per_split;
    int g = rem / p.KVH, kvh = rem - g * p.KVH;
    const int d_split = 64 / per_split, d_rem = 64 - d_split * per_split;
    const int d_g = d_rem / p.KVH, d_kvh = d_rem - d_g * p.KVH;
    for (int t = lane; t < cnt; t += 64) {
      p.items[base + t] = make_int2(sq, (g << 16) | (split << 8) | kvh);
      kvh += d_kvh;
      g += d_g;
      if (kvh >= p.KVH) { kvh -= p.KVH; ++g; }
      split += d_split;
      if (g >= groups_q) { g -= groups_q; ++split; }
    }
    const int nr = __builtin_amdgcn_readlane(rows_r, r);
    const int rbase = __builtin_amdgcn_readlane(pre_r, r);
    const int ar = __builtin_amdgcn_readlane(a_r, r);
    const int sr = __builtin_amdgcn_readlane(splits_r, r);
    for (int t = lane; t < nr; t += 64) p.merge_rows[rbase + t] = (ar + t) | ((sr - 1) << kMergeSplitShift);
  }
}

}  // namespace

hipError_t launch_schedule(const ScheduleParams& p, hipStream_t stream) {
  if (p.num_seqs <= 64)
    hipLaunchKernelGGL(ragged_schedule_wave_kernel, dim3(1), dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL(ragged_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace va
