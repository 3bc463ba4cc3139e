// Accepted-path KV promotion for tree verification, gfx950.
//
// After verification the caller names, per sequence, the accepted path
// r_0, ..., r_{n-1} of drafted rows (root first, parent[r_k] == r_{k-1}).
// Their K / V vectors (and 8-bit scales) move to the consecutive slots right
// after the first node's parent, dst = ctx - B + parent[r_0] + 1, so the
// durable prefix reads as the accepted tokens in order; new_ctx = dst + n.
// Only the accepted prefix is promoted and every sequence is checked before
// any pool byte changes (page "perf(qwen35): retain speculation during paged
// prefill", State and commit invariants).
//
// Every accepted row is read before any is written (sources and destinations
// may overlap), and nothing is written unless every check passed.  Two forms
// with that order:
//  * one launch when the batch has at most 256 (sequence, path slot) pairs:
//    a workgroup per (sequence, KV head) checks every pair of the batch,
//    stages its own accepted rows in LDS, then writes them and new_ctx;
//  * otherwise three stream-ordered launches: (1) clear this call's status
//    word, (2) check every (sequence, path node) and gather the accepted rows
//    into workspace staging, (3) if no check failed, scatter the staging rows
//    to their destination slots and write new_ctx.
// The three-launch form runs one wave per (sequence, path slot, KV head, K or
// V): lane l moves head_dim entries 4l .. 4l + 3 and lane b < D/32 the scale
// of block b (the one-launch form's lanes are described at its kernel).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "va_internal.h"

namespace va {
namespace {

struct Item {
  int s, k, g, which;
};

// Limits of the one-launch form: (sequence, path slot) pairs of a batch (one
// thread each), rows per sequence and staged row bytes (fp16 at D 256).
constexpr int kPromoteMaxPairs = 256;
constexpr int kMaxRowsPerSeq = 64;
constexpr int kPromoteMaxRowBytes = 512;

__device__ __forceinline__ int64_t total_rows(const PromoteParams& p) {
  return (int64_t)p.num_seqs * p.B * p.KVH * 2;
}

// Row idx of the staging order ((s * B + k) * KVH + g) * 2 + which.
__device__ __forceinline__ void decode_idx(const PromoteParams& p, int64_t idx, Item& it) {
  it.which = (int)(idx % 2);
  idx /= 2;
  it.g = (int)(idx % p.KVH);
  idx /= p.KVH;
  it.k = (int)(idx % p.B);
  it.s = (int)(idx / p.B);
}

__device__ __forceinline__ bool decode(const PromoteParams& p, Item& it) {
  const int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= total_rows(p)) return false;
  decode_idx(p, idx, it);
  return true;
}

// Element offset of (page, KV head g, slot, dim d): K token-major, V dim-major.
__device__ __forceinline__ int64_t elem(const PromoteParams& p, int which, int64_t page, int g, int slot, int d) {
  const int64_t head = (page * p.KVH + g) * kPage * p.D;
  return which ? head + (int64_t)d * kPage + slot : head + (int64_t)slot * p.D + d;
}

__device__ __forceinline__ int64_t scale_idx(const PromoteParams& p, int which, int64_t page, int g, int slot,
                                             int blk) {
  const int NB = p.D / 32;
  return which ? ((page * p.KVH + g) * NB + blk) * kPage + slot : ((page * p.KVH + g) * kPage + slot) * NB + blk;
}

__device__ __forceinline__ int parent_of(const PromoteParams& p, int s, int r) {
  return p.parent ? p.parent[(int64_t)s * p.B + r] : r - 1;
}

__device__ __forceinline__ char* staging_row(const PromoteParams& p, const Item& it) {
  return p.staging + ((((int64_t)it.s * p.B + it.k) * p.KVH + it.g) * 2 + it.which) * p.row_bytes;
}

// Lane l's head_dim entries 4l .. 4l + 3 and lane b's block scale between a
// pool slot and a staging row (dims contiguous, then the D/32 scales):
// pool -> row when `gather`, else row -> pool.
__device__ __forceinline__ void copy_row(const PromoteParams& p, const Item& it, int64_t page, int slot, char* row,
                                         bool gather) {
  const int lane = threadIdx.x & 63;
  const int d0 = 4 * lane;
  char* pool = reinterpret_cast<char*>(it.which ? p.v_pool : p.k_pool);
  if (!it.which) {  // token-major K: the 4 entries are contiguous
    if (d0 < p.D) {
      char* pe = pool + elem(p, 0, page, it.g, slot, d0) * p.esz;
      char* re = row + (int64_t)d0 * p.esz;
      if (p.esz == 1) {
        if (gather) *reinterpret_cast<uint32_t*>(re) = *reinterpret_cast<const uint32_t*>(pe);
        else *reinterpret_cast<uint32_t*>(pe) = *reinterpret_cast<const uint32_t*>(re);
      } else {
        if (gather) *reinterpret_cast<uint2*>(re) = *reinterpret_cast<const uint2*>(pe);
        else *reinterpret_cast<uint2*>(pe) = *reinterpret_cast<const uint2*>(re);
      }
    }
  } else if (d0 < p.D) {  // dim-major V: 16 slots apart
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = d0 + e;
      {
        char* pe = pool + elem(p, 1, page, it.g, slot, d) * p.esz;
        char* re = row + (int64_t)d * p.esz;
        if (p.esz == 1) {
          if (gather) *re = *pe;
          else *pe = *re;
        } else {
          if (gather) *reinterpret_cast<uint16_t*>(re) = *reinterpret_cast<const uint16_t*>(pe);
          else *reinterpret_cast<uint16_t*>(pe) = *reinterpret_cast<const uint16_t*>(re);
        }
      }
    }
  }
  if (p.kv_is_q8 && lane < p.D / 32) {
    uint16_t* sc = reinterpret_cast<uint16_t*>(it.which ? p.v_scale : p.k_scale) +
                   scale_idx(p, it.which, page, it.g, slot, lane);
    uint16_t* rs = reinterpret_cast<uint16_t*>(row + (int64_t)p.D * p.esz) + lane;
    if (gather) *rs = *sc;
    else *sc = *rs;
  }
}

__global__ void promote_clear_kernel(uint32_t* status) { *status = 0u; }

// Source and destination (page, slot) of one accepted row; ps < 0 when the
// (sequence, path slot) moves nothing.
struct Move {
  int ps, ts, pd, td;
};

// Checks of path slot k of sequence s.  Returns the failed checks' flag bits;
// m says what moves when they pass.
__device__ __forceinline__ uint32_t check_pair(const PromoteParams& p, int s, int k, Move& m) {
  m.ps = -1;
  m.ts = m.pd = m.td = 0;
  uint32_t bad = 0;
  const int ctx = p.ctx_lens[s];
  const int n = p.n_accepted[s];
  if (ctx < p.B || ctx > p.max_ctx || ctx > p.max_pages * kPage) bad |= VA_FLAG_BAD_CTX;
  if (n < 0 || n > p.B) bad |= VA_FLAG_BAD_PATH;
  if (!bad && k < n) {
    const int r = p.accepted[(int64_t)s * p.B + k];
    if (r < 0 || r >= p.B) {
      bad |= VA_FLAG_BAD_PATH;
    } else {
      const int par = parent_of(p, s, r);
      if (par < -1 || par >= r) bad |= VA_FLAG_BAD_PARENT;
      else if (k > 0 && par != p.accepted[(int64_t)s * p.B + k - 1]) bad |= VA_FLAG_BAD_PATH;
    }
    if (!bad) {
      const int base = ctx - p.B;
      const int r0 = p.accepted[(int64_t)s * p.B];
      const int par0 = (r0 >= 0 && r0 < p.B) ? parent_of(p, s, r0) : -2;
      if (par0 < -1 || par0 >= r0) bad |= VA_FLAG_BAD_PATH;
      const int t_src = base + r;
      const int t_dst = base + par0 + 1 + k;
      if (!bad && (t_dst < 0 || t_dst > t_src)) bad |= VA_FLAG_BAD_PATH;  // a valid path never moves forward
      if (!bad) {
        const int32_t* bt = p.block_table + (int64_t)s * p.max_pages;
        const int ps = bt[t_src / kPage], pd = bt[t_dst / kPage];
        if (ps < 0 || ps >= p.num_pages || pd < 0 || pd >= p.num_pages) {
          bad |= VA_FLAG_BAD_PAGE;
        } else {
          m.ps = ps;
          m.ts = t_src % kPage;
          m.pd = pd;
          m.td = t_dst % kPage;
        }
      }
    }
  }
  return bad;
}

// Checks of one (sequence, path slot) and, when they pass and the slot is on
// the path, the gather of its row (K or V of KV head g) into `row`.  Returns
// the failed checks' flag bits.
__device__ uint32_t check_gather(const PromoteParams& p, const Item& it, char* row) {
  Move m;
  const uint32_t bad = check_pair(p, it.s, it.k, m);
  if (m.ps >= 0) copy_row(p, it, m.ps, m.ts, row, true);  // the source row (and its scales) into staging
  return bad;
}

// Row `row` to its destination slot when every check passed (`ok`), and
// new_ctx of the sequence (from its first item).
__device__ void scatter_one(const PromoteParams& p, const Item& it, bool ok, char* row) {
  const int ctx = p.ctx_lens[it.s];
  const int n = p.n_accepted[it.s];
  if (it.k == 0 && it.g == 0 && it.which == 0 && (threadIdx.x & 63) == 0 && p.new_ctx) {
    int nc = ctx;
    if (ok && n > 0) nc = ctx - p.B + parent_of(p, it.s, p.accepted[(int64_t)it.s * p.B]) + 1 + n;
    else if (ok) nc = ctx - p.B;
    p.new_ctx[it.s] = nc;
  }
  if (!ok || it.k >= n) return;
  const int r0 = p.accepted[(int64_t)it.s * p.B];
  const int t_dst = ctx - p.B + parent_of(p, it.s, r0) + 1 + it.k;
  const int pd = p.block_table[(int64_t)it.s * p.max_pages + t_dst / kPage];
  copy_row(p, it, pd, t_dst % kPage, row, false);
}

__global__ __launch_bounds__(256) void promote_gather_kernel(const PromoteParams p) {
  Item it;
  if (!decode(p, it)) return;
  const uint32_t bad = check_gather(p, it, staging_row(p, it));
  if (bad && (threadIdx.x & 63) == 0) {
    atomicOr(p.status, bad);
    atomicOr(p.flags, bad);
  }
}

__global__ __launch_bounds__(256) void promote_scatter_kernel(const PromoteParams p) {
  Item it;
  if (!decode(p, it)) return;
  scatter_one(p, it, *p.status == 0u, staging_row(p, it));
}

// One row's share of a lane in registers: K (token-major) entries
// 4l .. 4l + 3 packed in e[0] (8-bit) or e[0..1] (fp16); V (dim-major)
// entries l + 64 j in e[j], so one access covers 64 consecutive dims; and
// the scale of block l.
struct Frag {
  uint32_t e[4];
  uint32_t sc;
};

template <int ESZ>
using Elem = typename std::conditional<ESZ == 1, uint8_t, uint16_t>::type;

// Loads of one row (ESZ-byte entries, 8-bit scales when Q8; V when V_ROW).
// Every lane loads from an in-bounds address (entries past head_dim re-read
// the last one and are dropped), so no load sits behind a branch and a
// wave's loads of several rows are all in flight before the first wait.
template <int ESZ, bool Q8, bool V_ROW>
__device__ __forceinline__ Frag load_frag(const PromoteParams& p, int g, int64_t page, int slot) {
  const int lane = threadIdx.x & 63;
  Frag f;
  if constexpr (!V_ROW) {
    const char* pe = reinterpret_cast<const char*>(p.k_pool) + elem(p, 0, page, g, slot, min(4 * lane, p.D - 4)) * ESZ;
    if constexpr (ESZ == 1) {
      f.e[0] = *reinterpret_cast<const uint32_t*>(pe);
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(pe);
      f.e[0] = x.x;
      f.e[1] = x.y;
    }
  } else {
    const Elem<ESZ>* pool = reinterpret_cast<const Elem<ESZ>*>(p.v_pool);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.e[j] = pool[elem(p, 1, page, g, slot, min(lane + 64 * j, p.D - 1))];
  }
  if constexpr (Q8)
    f.sc = reinterpret_cast<const uint16_t*>(V_ROW ? p.v_scale : p.k_scale)[scale_idx(p, V_ROW, page, g, slot,
                                                                                      min(lane, p.D / 32 - 1))];
  return f;
}

template <int ESZ, bool Q8, bool V_ROW>
__device__ __forceinline__ void store_frag(const PromoteParams& p, int g, int64_t page, int slot, const Frag& f) {
  const int lane = threadIdx.x & 63;
  if constexpr (!V_ROW) {
    if (4 * lane < p.D) {
      char* pe = reinterpret_cast<char*>(p.k_pool) + elem(p, 0, page, g, slot, 4 * lane) * ESZ;
      if constexpr (ESZ == 1) *reinterpret_cast<uint32_t*>(pe) = f.e[0];
      else *reinterpret_cast<uint2*>(pe) = make_uint2(f.e[0], f.e[1]);
    }
  } else {
    Elem<ESZ>* pool = reinterpret_cast<Elem<ESZ>*>(p.v_pool);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j < p.D) pool[elem(p, 1, page, g, slot, lane + 64 * j)] = (Elem<ESZ>)f.e[j];
  }
  if constexpr (Q8) {
    if (lane < p.D / 32)
      reinterpret_cast<uint16_t*>(V_ROW ? p.v_scale : p.k_scale)[scale_idx(p, V_ROW, page, g, slot, lane)] =
          (uint16_t)f.sc;
  }
}

// A lane's share of a staging row (dims in order, then the scales) to and
// from LDS, in the lane mapping of load_frag.
template <int ESZ, bool Q8, bool V_ROW>
__device__ __forceinline__ void put_row(const PromoteParams& p, char* row, const Frag& f) {
  const int lane = threadIdx.x & 63;
  if constexpr (!V_ROW) {
    if (4 * lane < p.D) {
      if constexpr (ESZ == 1) *reinterpret_cast<uint32_t*>(row + 4 * lane) = f.e[0];
      else *reinterpret_cast<uint2*>(row + 8 * lane) = make_uint2(f.e[0], f.e[1]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j < p.D) reinterpret_cast<Elem<ESZ>*>(row)[lane + 64 * j] = (Elem<ESZ>)f.e[j];
  }
  if constexpr (Q8) {
    if (lane < p.D / 32) reinterpret_cast<uint16_t*>(row + p.D * ESZ)[lane] = (uint16_t)f.sc;
  }
}

template <int ESZ, bool Q8, bool V_ROW>
__device__ __forceinline__ Frag get_row(const PromoteParams& p, const char* row) {
  const int lane = threadIdx.x & 63;
  Frag f;
  if constexpr (!V_ROW) {
    const int d0 = min(4 * lane, p.D - 4);
    if constexpr (ESZ == 1) {
      f.e[0] = *reinterpret_cast<const uint32_t*>(row + d0);
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(row + 2 * d0);
      f.e[0] = x.x;
      f.e[1] = x.y;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) f.e[j] = reinterpret_cast<const Elem<ESZ>*>(row)[min(lane + 64 * j, p.D - 1)];
  }
  if constexpr (Q8) f.sc = reinterpret_cast<const uint16_t*>(row + p.D * ESZ)[min(lane, p.D / 32 - 1)];
  return f;
}

// The one-launch form, for batches of at most kPromoteMaxPairs (sequence,
// path slot) pairs (the host checks): one workgroup per (sequence s, KV head
// g).
//  1. Every workgroup runs the checks of every pair of the batch, one thread
//     each, so each knows on its own whether the batch may be written; the
//     threads of sequence s keep their slot's source and destination.
//  2. If every check passed, the workgroup stages the K and V rows of head g
//     of s's accepted slots in LDS, kGatherRows rows per wave in flight
//     (loads first, then the LDS writes).  Overlapping sources and
//     destinations of one (sequence, KV head) are all in this workgroup;
//     different sequences' drafted slots lie in pages of their own.
//  3. After the barrier: new_ctx (the g = 0 workgroup), and the rows to
//     their destinations.
// Row r = 2 k + (V ? 1 : 0) of accepted slot k is staged at r * row_bytes.  A
// wave's rows r = wave + 4 m keep the wave's parity, so even waves move K
// rows and odd waves V rows.
constexpr int kGatherRows = 8;
constexpr int kPromoteWaves = 4;

template <int ESZ, bool Q8, bool V_ROW>
__device__ __forceinline__ void gather_rows(const PromoteParams& p, int g, char* stage, const int* pages,
                                            const uint8_t* slots, int rows) {
  const int wave = threadIdx.x >> 6;
  for (int r0 = wave; r0 < rows; r0 += kPromoteWaves * kGatherRows) {
    Frag f[kGatherRows];
#pragma unroll
    for (int u = 0; u < kGatherRows; ++u) {
      // past the end: reload the wave's first row of the batch (not written)
      const int r = r0 + kPromoteWaves * u < rows ? r0 + kPromoteWaves * u : r0;
      f[u] = load_frag<ESZ, Q8, V_ROW>(p, g, pages[r >> 1], slots[r >> 1]);
    }
#pragma unroll
    for (int u = 0; u < kGatherRows; ++u) {
      const int r = r0 + kPromoteWaves * u;
      if (r < rows) put_row<ESZ, Q8, V_ROW>(p, stage + (int64_t)r * p.row_bytes, f[u]);
    }
  }
}

template <int ESZ, bool Q8, bool V_ROW>
__device__ __forceinline__ void scatter_rows(const PromoteParams& p, int g, const char* stage, const int* pages,
                                             const uint8_t* slots, int rows) {
  const int wave = threadIdx.x >> 6;
  for (int r0 = wave; r0 < rows; r0 += kPromoteWaves * kGatherRows) {
    Frag f[kGatherRows];
#pragma unroll
    for (int u = 0; u < kGatherRows; ++u) {
      const int r = r0 + kPromoteWaves * u < rows ? r0 + kPromoteWaves * u : r0;
      f[u] = get_row<ESZ, Q8, V_ROW>(p, stage + (int64_t)r * p.row_bytes);
    }
#pragma unroll
    for (int u = 0; u < kGatherRows; ++u) {
      const int r = r0 + kPromoteWaves * u;
      if (r < rows) store_frag<ESZ, Q8, V_ROW>(p, g, pages[r >> 1], slots[r >> 1], f[u]);
    }
  }
}

template <int ESZ, bool Q8>
__global__ __launch_bounds__(256) void promote_onepass_kernel(const PromoteParams p) {
  __shared__ __align__(16) char stage[2 * kMaxRowsPerSeq * kPromoteMaxRowBytes];
  __shared__ int src_page[kMaxRowsPerSeq], dst_page[kMaxRowsPerSeq];
  __shared__ uint8_t src_slot[kMaxRowsPerSeq], dst_slot[kMaxRowsPerSeq];
  __shared__ uint32_t bad_all;
  const int tid = threadIdx.x;
  const int s = blockIdx.x / p.KVH, g = blockIdx.x - s * p.KVH;
  if (tid == 0) bad_all = 0u;
  __syncthreads();
  const int npairs = p.num_seqs * p.B;
  if (tid < npairs) {
    Move m;
    const uint32_t bad = check_pair(p, tid / p.B, tid % p.B, m);
    if (bad) atomicOr(&bad_all, bad);
    if (tid / p.B == s) {
      const int k = tid - s * p.B;
      src_page[k] = m.ps;
      src_slot[k] = (uint8_t)m.ts;
      dst_page[k] = m.pd;
      dst_slot[k] = (uint8_t)m.td;
    }
  }
  __syncthreads();
  const uint32_t bad = bad_all;
  // with every check passed, sequence s moves exactly its slots k < n
  const int rows = bad ? 0 : 2 * p.n_accepted[s];
  const bool v_wave = (tid >> 6) & 1;
  if (v_wave) gather_rows<ESZ, Q8, true>(p, g, stage, src_page, src_slot, rows);
  else gather_rows<ESZ, Q8, false>(p, g, stage, src_page, src_slot, rows);
  __syncthreads();  // every row of (s, g) read before any is written
  if (g == 0 && tid == 0) {
    if (p.new_ctx) {
      const int ctx = p.ctx_lens[s];
      const int n = p.n_accepted[s];
      int nc = ctx;
      if (!bad && n > 0) nc = ctx - p.B + parent_of(p, s, p.accepted[(int64_t)s * p.B]) + 1 + n;
      else if (!bad) nc = ctx - p.B;
      p.new_ctx[s] = nc;
    }
    if (s == 0 && bad) atomicOr(p.flags, bad);
  }
  if (v_wave) scatter_rows<ESZ, Q8, true>(p, g, stage, dst_page, dst_slot, rows);
  else scatter_rows<ESZ, Q8, false>(p, g, stage, dst_page, dst_slot, rows);
}

}  // namespace

size_t promote_row_bytes(int D, int kv_dtype) {
  const size_t esz = kv_dtype == kQ8 ? 1 : 2;
  const size_t raw = (size_t)D * esz + (kv_dtype == kQ8 ? (size_t)(D / 32) * 2 : 0);
  return (raw + 15) & ~(size_t)15;
}

bool promote_one_launch(const PromoteParams& p) {
  const int64_t pairs = (int64_t)p.num_seqs * p.B;
  return pairs > 0 && pairs <= kPromoteMaxPairs && p.B <= kMaxRowsPerSeq && p.row_bytes <= kPromoteMaxRowBytes;
}

hipError_t launch_promote(const PromoteParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.num_seqs * p.B * p.KVH * 2;  // waves, 4 per workgroup
  if (promote_one_launch(p)) {
    const dim3 grid((unsigned)(p.num_seqs * p.KVH));
    if (p.kv_is_q8) hipLaunchKernelGGL((promote_onepass_kernel<1, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((promote_onepass_kernel<2, false>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(promote_clear_kernel, dim3(1), dim3(1), 0, stream, p.status);
  if (total > 0) {
    const unsigned blocks = (unsigned)((total + 3) / 4);
    hipLaunchKernelGGL(promote_gather_kernel, dim3(blocks), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(promote_scatter_kernel, dim3(blocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace va
