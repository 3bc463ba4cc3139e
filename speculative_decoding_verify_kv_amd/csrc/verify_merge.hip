// Log-sum-exp merge of split partials for verify attention, gfx950.
//
// Each split k left, per (row, head) R: m_k (running max of the scaled scores,
// log2 units), l_k (sum of 2^(t - m_k)) and O_k (sum of 2^(t - m_k) v, fp32).
// The merge takes M = max over non-empty splits, w_k = 2^(m_k - M),
// O = sum w_k O_k / sum w_k l_k and lse = ln2 * (M + log2 sum w_k l_k): the
// merge step of the split-KV schedule on the page "perf(gfx1100): speed up
// long-context DFlash verify 13.4% with FA2 split-KV and retain HipGraph/Redline
// PM4" (Performance, batch-16 kernel screen).  Empty splits (l == 0) get weight
// 0 and their O is never used; a NaN l (a split that saw bad metadata) makes
// the row NaN.
//
// One wave per (row, head).  Lane k first loads (m_k, l_k) of split k, so all
// split headers arrive in one round trip; the weights are reduced across the
// wave and kept in LDS.  Then each lane owns D/64 consecutive outputs and
// streams the S partial rows in batches of 8 independent loads.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "va_internal.h"

namespace va {
namespace {

typedef _Float16 h16;

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int E> struct VecT { typedef float type __attribute__((ext_vector_type(E))); };
template <> struct VecT<1> { typedef float type; };

template <int D>
__global__ __launch_bounds__(64) void verify_merge_kernel(const MergeParams p) {
  constexpr int E = D / 64;  // outputs per lane
  constexpr int BATCH = 8;
  __shared__ float wts[kMaxSplits];
  const int64_t R = blockIdx.x;
  const int lane = threadIdx.x;
  const int S = p.S;

  // split headers: lane k holds split k, k + 64, ...
  float M = -INFINITY;
  bool nan_row = false;
  for (int k = lane; k < S; k += 64) {
    const float l = p.part_l[(int64_t)k * p.nrows + R];
    const float m = p.part_m[(int64_t)k * p.nrows + R];
    nan_row |= (l != l);
    if (l > 0.f) M = fmaxf(M, m);
  }
  M = wave_max(M);
  nan_row = __builtin_amdgcn_ballot_w64(nan_row) != 0;
  float Lpart = 0.f;
  for (int k = lane; k < S; k += 64) {
    const float l = p.part_l[(int64_t)k * p.nrows + R];
    const float w = (l > 0.f) ? __builtin_amdgcn_exp2f(p.part_m[(int64_t)k * p.nrows + R] - M) : 0.f;
    wts[k] = w;
    Lpart += w * l;
  }
  const float L = wave_sum(Lpart);
  __syncthreads();

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  const float* base = p.part_o + R * D + E * lane;
  const int64_t kstride = p.nrows * D;
  typedef typename VecT<E>::type vec;
  for (int k0 = 0; k0 < S; k0 += BATCH) {
    vec v[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int k = k0 + b < S ? k0 + b : S - 1;  // clamped: in bounds, weight 0 below
      v[b] = *reinterpret_cast<const vec*>(base + (int64_t)k * kstride);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int k = k0 + b;
      const float w = (k < S) ? wts[k] : 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float x;
        if constexpr (E == 1) x = v[b];
        else x = v[b][e];
        acc[e] += (w > 0.f) ? w * x : 0.f;
      }
    }
  }

  const float inv = nan_row ? __builtin_nanf("") : 1.0f / L;
  const int64_t o = R * D + E * lane;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float x = acc[e] * inv;
    if (p.out_dtype == kF32) reinterpret_cast<float*>(p.out)[o + e] = x;
    else if (p.out_dtype == kF16) reinterpret_cast<h16*>(p.out)[o + e] = (h16)x;
    else reinterpret_cast<uint16_t*>(p.out)[o + e] = (uint16_t)f32_to_bf16_bits(x);
  }
  if (lane == 0 && p.lse)
    p.lse[R] = nan_row ? __builtin_nanf("") : 0.6931471805599453f * (M + __builtin_log2f(L));
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.nrows);
  switch (p.D) {
    case 256: hipLaunchKernelGGL(verify_merge_kernel<256>, grid, dim3(64), 0, stream, p); break;
    case 128: hipLaunchKernelGGL(verify_merge_kernel<128>, grid, dim3(64), 0, stream, p); break;
    case 64: hipLaunchKernelGGL(verify_merge_kernel<64>, grid, dim3(64), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace va
