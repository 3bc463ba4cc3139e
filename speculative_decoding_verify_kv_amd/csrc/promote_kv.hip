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
// Three stream-ordered launches: (1) clear this call's status word, (2) check
// every (sequence, path node) and gather the accepted rows into workspace
// staging (sources and destinations may overlap), (3) if no check failed,
// scatter the staging rows to their destination slots and write new_ctx.
// One wave per (sequence, path slot, KV head, K or V): lane l moves head_dim
// entries 4l .. 4l + 3 and lane b < D/32 the scale of block b.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "va_internal.h"

namespace va {
namespace {

struct Item {
  int s, k, g, which;
};

__device__ __forceinline__ bool decode(const PromoteParams& p, Item& it) {
  int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t total = (int64_t)p.num_seqs * p.B * p.KVH * 2;
  if (idx >= total) return false;
  it.which = (int)(idx % 2);
  idx /= 2;
  it.g = (int)(idx % p.KVH);
  idx /= p.KVH;
  it.k = (int)(idx % p.B);
  it.s = (int)(idx / p.B);
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
  if (d0 < p.D) {
    if (!it.which) {  // token-major K: the 4 entries are contiguous
      char* pe = pool + elem(p, 0, page, it.g, slot, d0) * p.esz;
      char* re = row + (int64_t)d0 * p.esz;
      if (p.esz == 1) {
        if (gather) *reinterpret_cast<uint32_t*>(re) = *reinterpret_cast<const uint32_t*>(pe);
        else *reinterpret_cast<uint32_t*>(pe) = *reinterpret_cast<const uint32_t*>(re);
      } else {
        if (gather) *reinterpret_cast<uint2*>(re) = *reinterpret_cast<const uint2*>(pe);
        else *reinterpret_cast<uint2*>(pe) = *reinterpret_cast<const uint2*>(re);
      }
    } else {  // dim-major V: 16 slots apart
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        char* pe = pool + elem(p, 1, page, it.g, slot, d0 + e) * p.esz;
        char* re = row + (int64_t)(d0 + e) * p.esz;
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

__global__ __launch_bounds__(256) void promote_gather_kernel(const PromoteParams p) {
  Item it;
  if (!decode(p, it)) return;
  uint32_t bad = 0;
  const int ctx = p.ctx_lens[it.s];
  const int n = p.n_accepted[it.s];
  if (ctx < p.B || ctx > p.max_ctx || ctx > p.max_pages * kPage) bad |= VA_FLAG_BAD_CTX;
  if (n < 0 || n > p.B) bad |= VA_FLAG_BAD_PATH;
  if (!bad && it.k < n) {
    const int r = p.accepted[(int64_t)it.s * p.B + it.k];
    if (r < 0 || r >= p.B) {
      bad |= VA_FLAG_BAD_PATH;
    } else {
      const int par = parent_of(p, it.s, r);
      if (par < -1 || par >= r) bad |= VA_FLAG_BAD_PARENT;
      else if (it.k > 0 && par != p.accepted[(int64_t)it.s * p.B + it.k - 1]) bad |= VA_FLAG_BAD_PATH;
    }
    if (!bad) {
      const int base = ctx - p.B;
      const int r0 = p.accepted[(int64_t)it.s * p.B];
      const int par0 = (r0 >= 0 && r0 < p.B) ? parent_of(p, it.s, r0) : -2;
      if (par0 < -1 || par0 >= r0) bad |= VA_FLAG_BAD_PATH;
      const int t_src = base + r;
      const int t_dst = base + par0 + 1 + it.k;
      if (!bad && (t_dst < 0 || t_dst > t_src)) bad |= VA_FLAG_BAD_PATH;  // a valid path never moves forward
      if (!bad) {
        const int32_t* bt = p.block_table + (int64_t)it.s * p.max_pages;
        const int ps = bt[t_src / kPage], pd = bt[t_dst / kPage];
        if (ps < 0 || ps >= p.num_pages || pd < 0 || pd >= p.num_pages) {
          bad |= VA_FLAG_BAD_PAGE;
        } else {
          // gather the source row (and its scales) into staging
          copy_row(p, it, ps, t_src % kPage, staging_row(p, it), true);
        }
      }
    }
  }
  if (bad && (threadIdx.x & 63) == 0) {
    atomicOr(p.status, bad);
    atomicOr(p.flags, bad);
  }
}

__global__ __launch_bounds__(256) void promote_scatter_kernel(const PromoteParams p) {
  Item it;
  if (!decode(p, it)) return;
  const bool ok = (*p.status == 0u);
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
  copy_row(p, it, pd, t_dst % kPage, staging_row(p, it), false);
}

}  // namespace

size_t promote_row_bytes(int D, int kv_dtype) {
  const size_t esz = kv_dtype == kQ8 ? 1 : 2;
  const size_t raw = (size_t)D * esz + (kv_dtype == kQ8 ? (size_t)(D / 32) * 2 : 0);
  return (raw + 15) & ~(size_t)15;
}

hipError_t launch_promote(const PromoteParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.num_seqs * p.B * p.KVH * 2;  // waves, 4 per workgroup
  hipLaunchKernelGGL(promote_clear_kernel, dim3(1), dim3(1), 0, stream, p.status);
  if (total > 0) {
    const unsigned blocks = (unsigned)((total + 3) / 4);
    hipLaunchKernelGGL(promote_gather_kernel, dim3(blocks), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(promote_scatter_kernel, dim3(blocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace va
