// Log-sum-exp merge of split partials for verify attention, gfx950.
//
// Each split k left, per (row, head) R: m_k (running max of the scaled scores,
// log2 units), l_k (sum of 2^(t - m_k)) and O_k (sum of 2^(t - m_k) v, fp32).
// The merge takes M = max over non-empty splits, w_k = 2^(m_k - M),
// O = sum w_k O_k / sum w_k l_k and lse = ln2 * (M + log2 sum w_k l_k): the
// merge step of the split-KV schedule on the page "perf(gfx1100): speed up
// long-context DFlash verify 13.4% with FA2 split-KV and retain HipGraph/Redline
// PM4" (Performance, batch-16 kernel screen).  In a ragged call only the
// first n splits of a row hold keys (n, carried in the row's entry of the
// work list, is below S for a sequence too short to fill S splits of the
// minimum size); empty splits (l == 0) get weight 0 and their O is never used; a NaN l (a split that saw
// bad metadata) makes the row NaN.
//
// One workgroup of 8 waves per (row, head).  Wave w owns splits w, w + 8,
// ...; it issues the loads of up to 4 of its split rows at once (16 bytes
// per lane each at D = 256) right away, so the partial rows are in flight
// while the weights are formed.  Wave 0 alone loads the split headers, just
// before its rows (lane: splits lane, lane + 64, ...; each split's (m, l)
// is one 8-byte pair, a lone read from its own cache line, so one wave's
// worth is cheaper than eight), and hands the weights to the other waves
// through LDS.  The 8 waves' sums meet in LDS.

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

constexpr int kMergeWaves = 8;
constexpr int kMergeBatch = 4;   // split rows in flight per wave

template <int E>
__device__ __forceinline__ void store_row(const MergeParams& p, int64_t R, int lane, const float* sum, float inv,
                                          bool nan_row, float M, float L) {
  constexpr int D = 64 * E;
  const int64_t o = R * D + E * lane;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float x = sum[e] * inv;
    if (p.out_dtype == kF32) reinterpret_cast<float*>(p.out)[o + e] = x;
    else if (p.out_dtype == kF16) reinterpret_cast<h16*>(p.out)[o + e] = (h16)x;
    else reinterpret_cast<uint16_t*>(p.out)[o + e] = (uint16_t)f32_to_bf16_bits(x);
  }
  if (lane == 0 && p.lse)
    p.lse[R] = nan_row ? __builtin_nanf("") : 0.6931471805599453f * (M + __builtin_log2f(L));
}

// Partials are read with system-scope loads (sc0 sc1, the bits of a relaxed
// system-scope atomic load), as the partial kernel writes them: no L2 line
// left from an earlier use of the workspace is read in their place.  A
// split's row of one (row, head) is D floats; lane l reads entries E l ..
// E l + E - 1.
template <typename V>
__device__ __forceinline__ V load_partial(const float* row, int lane) {
  constexpr int E = sizeof(V) / sizeof(float);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), 0, 64 * E * (int)sizeof(float), kRawBufferFlags);
  if constexpr (E == 4) return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane, 0, kSystemScopeBits));
  else if constexpr (E == 2) return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(rs, 8 * lane, 0, kSystemScopeBits));
  else return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * lane, 0, kSystemScopeBits));
}

// A split's (m, l) pair of one (row, head): one 8-byte system-scope load.
__device__ __forceinline__ void load_header(const uint64_t* x, float& m, float& l) {
  const uint64_t ml = __hip_atomic_load(x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  m = __builtin_bit_cast(float, (uint32_t)ml);
  l = __builtin_bit_cast(float, (uint32_t)(ml >> 32));
}

// One wave merges (row, head) R alone: for ragged rows whose sequence has at
// most kMergeLightSplits splits.  Same arithmetic, in the same order, as the
// workgroup form below gives such a row (each of its waves then holds at
// most one split, and their sums are added in wave order), so the two agree
// bit for bit.
template <int D>
__device__ __forceinline__ void merge_one_wave(const MergeParams& p, int64_t R, int Sr, int lane) {
  constexpr int E = D / 64;
  constexpr int HJ = kMaxSplits / 64;
  typedef typename VecT<E>::type vec;
  const int S = p.S;
  const int64_t kstride = p.nrows * D;
  float mh[HJ], lh[HJ];
#pragma unroll
  for (int j = 0; j < HJ; ++j) {
    const int k = lane + 64 * j;
    mh[j] = -INFINITY;
    lh[j] = 0.f;
    if (k < Sr) {
      load_header(p.part_ml + (int64_t)k * p.nrows + R, mh[j], lh[j]);
    }
  }
  float M = -INFINITY;
  bool nan_row = false;
#pragma unroll
  for (int j = 0; j < HJ; ++j) {
    nan_row |= (lh[j] != lh[j]);
    if (lh[j] > 0.f) M = fmaxf(M, mh[j]);
  }
  M = wave_max(M);
  nan_row = __builtin_amdgcn_ballot_w64(nan_row) != 0;
  float wk[HJ];
  float Lpart = 0.f;
#pragma unroll
  for (int j = 0; j < HJ; ++j) {
    wk[j] = (lh[j] > 0.f) ? __builtin_amdgcn_exp2f(mh[j] - M) : 0.f;
    Lpart = __builtin_fmaf(wk[j], lh[j], Lpart);
  }
  const float L = wave_sum(Lpart);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int k0 = 0; k0 < Sr; k0 += kMergeBatch) {
    vec v[kMergeBatch];
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b)
      v[b] = load_partial<vec>(p.part_o + (int64_t)min(k0 + b, S - 1) * kstride + R * D, lane);
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) {
      const int k = k0 + b;  // wave-uniform
      const int j = k >> 6;
      float wsel = wk[0];
#pragma unroll
      for (int jj = 1; jj < HJ; ++jj) wsel = (j == jj) ? wk[jj] : wsel;
      const float w = (k < Sr) ? __shfl(wsel, k & 63) : 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float x;
        if constexpr (E == 1) x = v[b];
        else x = v[b][e];
        // the workgroup form: this split's wave sum (the rounded product, a
        // negative zero made positive), added to the running sum in order
        const float t = ((w > 0.f) ? __fmul_rn(w, x) : 0.f) + 0.f;
        if (k < Sr) acc[e] += t;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] += 0.f;
  const float inv = nan_row ? __builtin_nanf("") : 1.0f / L;
  store_row<E>(p, R, lane, acc, inv, nan_row, M, L);
}

// RAGGED: the rows come from the work list (merge_rows, merge_count).
template <int D, bool RAGGED>
__device__ __forceinline__ void merge_body(const MergeParams& p) {
  constexpr int E = D / 64;  // outputs per lane
  constexpr int HJ = kMaxSplits / 64;
  typedef typename VecT<E>::type vec;
  __shared__ float red[kMergeWaves][D];
  // (row, head) of this workgroup: block / heads and block % heads, or in a
  // ragged call the row at that place of the work list's row order (rows
  // with the most splits first; blocks past the rows in use leave)
  // Ragged calls: the rows with more than kMergeLightSplits splits lead the
  // list, one workgroup per (row, head); the rest follow, one wave per
  // (row, head), 8 to a workgroup.
  int64_t R = blockIdx.x;
  int Sr = p.S;  // splits that hold keys of the row's sequence (fewer for a short one in a ragged call)
  if constexpr (RAGGED) {
    // each row entry carries its sequence's split count; the entry a heavy
    // row would take is loaded beside the counts (it lies inside the list:
    // the grid is the row capacity times the heads) and used only if it is one
    const auto* mc = reinterpret_cast<const __attribute__((address_space(4))) int*>((uintptr_t)p.merge_count);
    const int64_t kh = R / p.heads;
    const int eh = *reinterpret_cast<const __attribute__((address_space(4))) int*>((uintptr_t)(p.merge_rows + kh));
    const int64_t heavy = (int64_t)mc[1] * p.heads;
    if (R >= heavy) {
      const int64_t pr = heavy + (R - heavy) * kMergeWaves + (threadIdx.x >> 6);
      if (pr >= (int64_t)mc[0] * p.heads) return;
      const int64_t k = pr / p.heads;
      const int e = *reinterpret_cast<const __attribute__((address_space(4))) int*>((uintptr_t)(p.merge_rows + k));
      merge_one_wave<D>(p, (int64_t)(e & kMergeRowMask) * p.heads + (pr - k * p.heads),
                        max(1, min(p.S, (e >> kMergeSplitShift) + 1)), threadIdx.x & 63);
      return;
    }
    R = (int64_t)(eh & kMergeRowMask) * p.heads + (R - kh * p.heads);
    Sr = max(1, min(p.S, (eh >> kMergeSplitShift) + 1));
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = p.S;
  // splits past Sr hold stale data and are never weighed
  const int64_t kstride = p.nrows * D;

  auto load = [&](int k) __attribute__((always_inline)) -> vec {
    return load_partial<vec>(p.part_o + (int64_t)min(k, S - 1) * kstride + R * D, lane);  // clamped: weight 0 below
  };
  // Split headers, read by wave 0 alone (lane: splits lane + 64 j) ahead of
  // its partial rows, so the weights are ready first; they reach the other
  // waves through LDS.  M, L and the NaN state stay in wave 0, which writes
  // the row.
  float mh[HJ], lh[HJ];
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < HJ; ++j) {
      const int k = lane + 64 * j;
      mh[j] = -INFINITY;
      lh[j] = 0.f;
      if (k < Sr) {
        load_header(p.part_ml + (int64_t)k * p.nrows + R, mh[j], lh[j]);
      }
    }
  }
  vec v[kMergeBatch];
#pragma unroll
  for (int b = 0; b < kMergeBatch; ++b) v[b] = load(wave + kMergeWaves * b);

  __shared__ float wsh[kMaxSplits];
  float M = -INFINITY, L = 0.f;
  bool nan_row = false;
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < HJ; ++j) {
      nan_row |= (lh[j] != lh[j]);
      if (lh[j] > 0.f) M = fmaxf(M, mh[j]);
    }
    M = wave_max(M);
    nan_row = __builtin_amdgcn_ballot_w64(nan_row) != 0;
    float Lpart = 0.f;
#pragma unroll
    for (int j = 0; j < HJ; ++j) {
      const float wk = (lh[j] > 0.f) ? __builtin_amdgcn_exp2f(mh[j] - M) : 0.f;
      Lpart = __builtin_fmaf(wk, lh[j], Lpart);
      wsh[lane + 64 * j] = wk;
    }
    L = wave_sum(Lpart);
  }
  __syncthreads();

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int k0 = wave; k0 < Sr; k0 += kMergeWaves * kMergeBatch) {
    if (k0 != wave) {
#pragma unroll
      for (int b = 0; b < kMergeBatch; ++b) v[b] = load(k0 + kMergeWaves * b);
    }
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) {
      const int k = k0 + kMergeWaves * b;  // wave-uniform
      const float w = (k < Sr) ? wsh[min(k, Sr - 1)] : 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float x;
        if constexpr (E == 1) x = v[b];
        else x = v[b][e];
        acc[e] += (w > 0.f) ? w * x : 0.f;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[wave][E * lane + e] = acc[e];
  __syncthreads();
  if (wave != 0) return;

  const float inv = nan_row ? __builtin_nanf("") : 1.0f / L;
  float sum[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    sum[e] = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) sum[e] += red[w][E * lane + e];
  }
  store_row<E>(p, R, lane, sum, inv, nan_row, M, L);
}

// Uniform calls: the leading arguments repeat the fields of the parameter
// block that the first loads need (the partials' addresses, the split count,
// the heads); the build preloads them into SGPRs at wave launch
// (-amdgpu-kernarg-preload-count), so the header and partial loads wait for
// no read of the argument block.
template <int D>
__global__ __launch_bounds__(64 * kMergeWaves) void verify_merge_kernel(const float* part_o, const uint64_t* part_ml,
                                                                      int64_t nrows, int32_t S, int32_t heads,
                                                                      const MergeParams p0) {
  MergeParams p = p0;
  p.part_o = part_o;
  p.part_ml = part_ml;
  p.nrows = nrows;
  p.S = S;
  p.heads = heads;
  merge_body<D, false>(p);
}

// Ragged calls read the work list first, which needs the parameter block
// anyway: no preloaded arguments, which would only add to the launch.
template <int D>
__global__ __launch_bounds__(64 * kMergeWaves) void verify_merge_ragged_kernel(const MergeParams p) {
  merge_body<D, true>(p);
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.nrows);
  const dim3 block(64 * kMergeWaves);
#define VA_MERGE_LAUNCH(DD)                                                                                       \
  do {                                                                                                             \
    if (p.merge_rows)                                                                                              \
      hipLaunchKernelGGL((verify_merge_ragged_kernel<DD>), grid, block, 0, stream, p);                             \
    else                                                                                                           \
      hipLaunchKernelGGL((verify_merge_kernel<DD>), grid, block, 0, stream, p.part_o, p.part_ml, p.nrows, p.S,     \
                         p.heads, p);                                                                              \
  } while (0)
  switch (p.D) {
    case 256: VA_MERGE_LAUNCH(256); break;
    case 128: VA_MERGE_LAUNCH(128); break;
    case 64: VA_MERGE_LAUNCH(64); break;
    default: return hipErrorInvalidValue;
  }
#undef VA_MERGE_LAUNCH
  return hipGetLastError();
}

}  // namespace va
