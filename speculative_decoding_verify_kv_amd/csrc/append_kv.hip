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
// One wave per (sequence, row, KV head, K or V); see the kernel.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "va_internal.h"

namespace va {
namespace {

typedef _Float16 h16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef h16 h16x4 __attribute__((ext_vector_type(4)));

// One wave per (sequence, row, KV head, K or V): lane l holds head_dim
// entries 4l .. 4l + 3, so a 32-entry block spans 8 lanes and its maximum is
// taken across them; the per-entry arithmetic is that of the format above.
__global__ __launch_bounds__(256) void append_kv_kernel(const AppendParams p) {
  const int lane = threadIdx.x & 63;
  int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t total = (int64_t)p.num_seqs * p.B * p.KVH * 2;
  if (idx >= total) return;
  const int which = (int)(idx % 2);  // 0: K, 1: V
  idx /= 2;
  const int g = (int)(idx % p.KVH);
  idx /= p.KVH;
  const int i = (int)(idx % p.B);
  const int s = (int)(idx / p.B);

  const int ctx = p.ctx_lens[s];
  if (ctx < p.B || ctx > p.max_ctx || ctx > p.max_pages * kPage) {
    if (i == 0 && g == 0 && which == 0 && lane == 0) atomicOr(p.flags, (uint32_t)VA_FLAG_BAD_CTX);
    return;
  }
  const int t = ctx - p.B + i;
  const int id = p.block_table[(int64_t)s * p.max_pages + t / kPage];
  if (id < 0 || id >= p.num_pages) {
    if (g == 0 && which == 0 && lane == 0) atomicOr(p.flags, (uint32_t)VA_FLAG_BAD_PAGE);
    return;
  }
  const int slot = t % kPage;
  const int D = p.D;
  const int NB = D / 32;
  const bool act = 4 * lane < D;  // whole 8-lane blocks: D / 4 is a multiple of 8
  const int d0 = 4 * lane;
  const void* src = which ? p.v_new : p.k_new;
  const int64_t e0 = ((int64_t)(s * p.B + i) * p.KVH + g) * D + d0;
  float x[4] = {0.f, 0.f, 0.f, 0.f};
  if (act) {
    if (p.new_dtype == kF32) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(src) + e0);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = v[e];
    } else {
      const u32x2 w = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(src) + e0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t b = (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        x[e] = p.new_dtype == kF16 ? (float)__builtin_bit_cast(h16, (uint16_t)b) : __builtin_bit_cast(float, b << 16);
      }
    }
  }

  const int64_t head = (int64_t)id * p.KVH + g;  // (page, KV head) index
  if (p.kv_dtype == kF16) {
    if (!act) return;
    h16* pool = reinterpret_cast<h16*>(which ? p.v_pool : p.k_pool) + head * kPage * D;
    if (which) {
#pragma unroll
      for (int e = 0; e < 4; ++e) pool[(int64_t)(d0 + e) * kPage + slot] = (h16)x[e];
    } else {
      h16x4 h;
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = (h16)x[e];
      *reinterpret_cast<h16x4*>(pool + (int64_t)slot * D + d0) = h;
    }
    return;
  }

  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = __builtin_fabsf(x[e]);
    amax = a > amax ? a : amax;  // a NaN entry never raises the max
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    const float a = __shfl_xor(amax, o);
    amax = a > amax ? a : amax;
  }
  const h16 dh = (h16)__fdiv_rn(amax, 127.0f);
  const float d16 = (float)dh;
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float r = d16 != 0.f ? __fdiv_rn(x[e], d16) : 0.f;
    if (r != r) r = 0.f;
    r = roundf(r);
    r = fminf(fmaxf(r, -127.f), 127.f);
    packed |= (uint32_t)(uint8_t)(int8_t)(int)r << (8 * e);
  }
  if (!act) return;
  int8_t* pool = reinterpret_cast<int8_t*>(which ? p.v_pool : p.k_pool) + head * kPage * D;
  const int blk = lane >> 3;
  if (which) {
#pragma unroll
    for (int e = 0; e < 4; ++e) pool[(int64_t)(d0 + e) * kPage + slot] = (int8_t)(packed >> (8 * e));
    if ((lane & 7) == 0) reinterpret_cast<h16*>(p.v_scale)[(head * NB + blk) * kPage + slot] = dh;
  } else {
    *reinterpret_cast<uint32_t*>(pool + (int64_t)slot * D + d0) = packed;
    if ((lane & 7) == 0) reinterpret_cast<h16*>(p.k_scale)[(head * kPage + slot) * NB + blk] = dh;
  }
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.num_seqs * p.B * p.KVH * 2;  // waves, 4 per workgroup
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 3) / 4);
  hipLaunchKernelGGL(append_kv_kernel, dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace va
