// Log-sum-exp merge of split partials for verify attention, gfx950.
//
// Each split k left, per (row, head) R: m_k (running max of the scaled scores,
// log2 units), l_k (sum of 2^(t - m_k)) and O_k (sum of 2^(t - m_k) v, fp32).
// The merge takes M = max over non-empty splits, w_k = 2^(m_k - M),
// O = sum w_k O_k / sum w_k l_k and lse = ln2 * (M + log2 sum w_k l_k): the
// merge step of the split-KV schedule on the page "perf(gfx1100): speed up
// long-context DFlash verify 13.4% with FA2 split-KV and retain HipGraph/Redline
// PM4" (Performance, batch-16 kernel screen).  Empty splits (l == 0) are
// skipped without reading their O; a NaN l (a split that saw bad metadata)
// makes the row NaN.
//
// One wave per (row, head); each lane owns D/64 consecutive output elements,
// so every split's O row is one coalesced read of D fp32.

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

template <int D>
__global__ __launch_bounds__(64) void verify_merge_kernel(const MergeParams p) {
  constexpr int E = D / 64;  // elements per lane
  const int64_t R = blockIdx.x;
  const int lane = threadIdx.x;
  const int S = p.S;

  float M = -INFINITY;
  bool nan_row = false;
  for (int k = 0; k < S; ++k) {
    const float l = p.part_l[(int64_t)k * p.nrows + R];
    const float m = p.part_m[(int64_t)k * p.nrows + R];
    if (l != l) nan_row = true;
    if (l > 0.f) M = fmaxf(M, m);
  }
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float L = 0.f;
  for (int k = 0; k < S; ++k) {
    const float l = p.part_l[(int64_t)k * p.nrows + R];
    if (!(l > 0.f)) continue;
    const float w = __builtin_amdgcn_exp2f(p.part_m[(int64_t)k * p.nrows + R] - M);
    L += w * l;
    const float* o = p.part_o + ((int64_t)k * p.nrows + R) * D + E * lane;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += w * o[e];
  }
  const float inv = nan_row ? __builtin_nanf("") : 1.0f / L;
  const int64_t base = R * D + E * lane;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float v = acc[e] * inv;
    if (p.out_dtype == kF32) reinterpret_cast<float*>(p.out)[base + e] = v;
    else if (p.out_dtype == kF16) reinterpret_cast<h16*>(p.out)[base + e] = (h16)v;
    else reinterpret_cast<uint16_t*>(p.out)[base + e] = (uint16_t)f32_to_bf16_bits(v);
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
