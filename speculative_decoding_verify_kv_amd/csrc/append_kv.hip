// KV append for verify attention, gfx950: the B drafted rows' K and V vectors
// are converted (fp16 pools) or block-quantised (8-bit pools) and written into
// their page slots ctx - B + i, the step that precedes the verify attention
// (page "perf(qwen35): retain speculation during paged prefill", State and
// commit invariants: the drafted rows' KV writes are shared by every row kind).
//
// 8-bit format: per (token, KV head) one fp16 scale per 32 consecutive
// head_dim entries, scale = max|x| / 127 computed in fp32 and rounded to fp16
// (nearest even); codes = clamp(round half away from zero (x / scale),
// -127, 127) in fp32 with the stored fp16 scale; an all-zero block stores
// scale 0 and codes 0, a NaN entry stores code 0.
//
// One thread per (sequence, row, KV head, K or V, 32-entry block).  The work
// is tiny (B * KVH * 2 * D elements per sequence), so the kernel favours
// plain per-thread code over coalescing.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "va_internal.h"

namespace va {
namespace {

typedef _Float16 h16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float load_elem(const void* src, int dtype, int64_t idx) {
  if (dtype == kF32) return reinterpret_cast<const float*>(src)[idx];
  const uint16_t b = reinterpret_cast<const uint16_t*>(src)[idx];
  if (dtype == kF16) return (float)__builtin_bit_cast(h16, b);
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

__global__ __launch_bounds__(256) void append_kv_kernel(const AppendParams p) {
  const int NB = p.D / 32;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.num_seqs * p.B * p.KVH * 2 * NB;
  if (idx >= total) return;
  const int blk = (int)(idx % NB);
  idx /= NB;
  const int which = (int)(idx % 2);  // 0: K, 1: V
  idx /= 2;
  const int g = (int)(idx % p.KVH);
  idx /= p.KVH;
  const int i = (int)(idx % p.B);
  const int s = (int)(idx / p.B);

  const int ctx = p.ctx_lens[s];
  if (ctx < p.B || ctx > p.max_ctx || ctx > p.max_pages * kPage) {
    if (i == 0 && g == 0 && which == 0 && blk == 0) atomicOr(p.flags, (uint32_t)VA_FLAG_BAD_CTX);
    return;
  }
  const int t = ctx - p.B + i;
  const int id = p.block_table[(int64_t)s * p.max_pages + t / kPage];
  if (id < 0 || id >= p.num_pages) {
    if (g == 0 && which == 0 && blk == 0) atomicOr(p.flags, (uint32_t)VA_FLAG_BAD_PAGE);
    return;
  }
  const int slot = t % kPage;
  const int D = p.D;
  const void* src = which ? p.v_new : p.k_new;
  const int64_t e0 = ((int64_t)(s * p.B + i) * p.KVH + g) * D + 32 * blk;
  float x[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) x[e] = load_elem(src, p.new_dtype, e0 + e);

  const int64_t head = (int64_t)id * p.KVH + g;  // (page, KV head) index
  if (p.kv_dtype == kF16) {
    h16* pool = reinterpret_cast<h16*>(which ? p.v_pool : p.k_pool) + head * kPage * D;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int d = 32 * blk + e;
      if (which) pool[(int64_t)d * kPage + slot] = (h16)x[e];
      else pool[(int64_t)slot * D + d] = (h16)x[e];
    }
    return;
  }

  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const float a = __builtin_fabsf(x[e]);
    amax = a > amax ? a : amax;  // a NaN entry never raises the max
  }
  const h16 dh = (h16)__fdiv_rn(amax, 127.0f);
  const float d16 = (float)dh;
  int8_t* pool = reinterpret_cast<int8_t*>(which ? p.v_pool : p.k_pool) + head * kPage * D;
  int8_t q[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    float r = d16 != 0.f ? __fdiv_rn(x[e], d16) : 0.f;
    if (r != r) r = 0.f;
    r = roundf(r);
    r = fminf(fmaxf(r, -127.f), 127.f);
    q[e] = (int8_t)(int)r;
  }
  if (which) {
#pragma unroll
    for (int e = 0; e < 32; ++e) pool[(int64_t)(32 * blk + e) * kPage + slot] = q[e];
    reinterpret_cast<h16*>(p.v_scale)[(head * NB + blk) * kPage + slot] = dh;
  } else {
    u32x4 w0, w1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w0[k] = (uint32_t)(uint8_t)q[4 * k] | ((uint32_t)(uint8_t)q[4 * k + 1] << 8) |
              ((uint32_t)(uint8_t)q[4 * k + 2] << 16) | ((uint32_t)(uint8_t)q[4 * k + 3] << 24);
      w1[k] = (uint32_t)(uint8_t)q[16 + 4 * k] | ((uint32_t)(uint8_t)q[16 + 4 * k + 1] << 8) |
              ((uint32_t)(uint8_t)q[16 + 4 * k + 2] << 16) | ((uint32_t)(uint8_t)q[16 + 4 * k + 3] << 24);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(pool + (int64_t)slot * D + 32 * blk);
    dst[0] = w0;
    dst[1] = w1;
    reinterpret_cast<h16*>(p.k_scale)[(head * kPage + slot) * NB + blk] = dh;
  }
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.num_seqs * p.B * p.KVH * 2 * (p.D / 32);
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(append_kv_kernel, dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace va
