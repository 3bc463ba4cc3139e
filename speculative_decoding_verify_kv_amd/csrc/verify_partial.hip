// Split-KV partial kernel for speculative-decoding verify attention, gfx950.
//
// One workgroup = (sequence s, KV head, split k, row group).  Its rows are
// 16*NT (drafted row, query head) pairs of one KV group: because every query
// head of a GQA group reads the same KV head, the group's B*G rows form the M
// side of a real matrix product with the streamed keys, so each fetched KV
// byte feeds many rows (the multi-row verifier idea of the page "perf(gfx11):
// optimize Qwen DFlash speculative verify", alpineQ's notes, taken to the whole
// group).  The split's pages are dealt to the 4 waves in pairs; each wave runs
// an independent online softmax over its pages and the waves are merged
// through LDS at the end, so the hot loop has no barrier.
//
// Per wave iteration (Q8: two 16-token pages = 32 keys; fp16: one page):
//   1. LDS-DMA (global_load_lds_dwordx4) of the NEXT iteration's K page(s), V
//      page(s) and scales into the wave's other ring stage (no VGPRs hold
//      in-flight data; the wave only waits on its own vmcnt).
//   2. K fragments from LDS -> int8 to fp16 dequant in registers -> S^T = K Q^T
//      on v_mfma_f32_16x16x32_f16 (keys on M, rows on N, fp32 accumulate).
//   3. Causal / tree / page-tail masking by select (only on iterations that
//      reach the drafted suffix or the split end), online softmax in the log2
//      domain with lazily rescaled running max, P packed to fp16.
//   4. V^T fragments (dim-major pages: 8 tokens of one dim are contiguous) ->
//      dequant -> O^T += V^T P^T on MFMA.  The S^T accumulator layout is
//      already the P^T operand layout, so P never leaves registers.
// Epilogue: (m, l) exchange, O rescale, reduce-scatter of O across waves
// through LDS, then either fp32 partials (split) or the final output (direct).
//
// Split partials + log-sum-exp merge and "S1 is the direct path" follow the
// page "perf(gfx1100): speed up long-context DFlash verify 13.4% with FA2
// split-KV and retain HipGraph/Redline PM4" (Performance, batch-16 kernel
// screen).  Splits are equal page-aligned ranges computed from the sequence's
// own ctx and S only, and partials are fp32, so rows never change with what
// else is in the launch (page "perf(qwen35): retain speculation during paged
// prefill", Correctness failure found during qualification).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "va_internal.h"

namespace va {
namespace {

typedef _Float16 h16;
typedef h16 h16x8 __attribute__((ext_vector_type(8)));
typedef h16 h16x4 __attribute__((ext_vector_type(4)));
typedef h16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, off) (reinterpret_cast<__attribute__((address_space(3))) T*>(off))

constexpr float kLazyRescale = 15.0f;  // 2^15 < 65504: the largest P value fp16 holds safely
constexpr float kLn2 = 0.6931471805599453f;

// ---- LDS-DMA helpers -------------------------------------------------------
// global_load_lds_dwordx4: each active lane copies 16 bytes from its global
// address to LDS at M0 + 16 * lane.  M0 is saved and restored around it.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// sbase and lds must be wave-uniform; readfirstlane makes that explicit.
__device__ __forceinline__ void dma_saddr(const void* sbase_in, uint32_t voff, uint32_t lds_in) {
  const void* sbase = uniform_ptr(sbase_in);
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_in);
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

__device__ __forceinline__ void dma_vaddr(const void* vaddr, uint32_t lds_in) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_in);
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(vaddr), "s"(lds)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---- geometry of one wave's ring stage --------------------------------------
template <int D, int KVT>
struct Geo {
  static constexpr bool Q8 = (KVT == kQ8);
  static constexpr int PPI = Q8 ? 2 : 1;         // pages per wave iteration
  static constexpr int ESZ = Q8 ? 1 : 2;         // bytes per K/V element
  static constexpr int KROW = D * ESZ;            // bytes of one token's K
  static constexpr int KPAGE = 16 * KROW;         // K bytes of one page (one KV head)
  static constexpr int VPAGE = D * 16 * ESZ;      // V bytes of one page
  static constexpr int SPAGE = Q8 ? D : 0;       // bytes of one page's K (or V) scales
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = PPI * KPAGE;
  static constexpr int KS_OFF = V_OFF + PPI * VPAGE;
  static constexpr int VS_OFF = KS_OFF + PPI * SPAGE;
  static constexpr int STAGE = VS_OFF + PPI * SPAGE;
  static constexpr int KCH = KROW / 16;           // 16-byte chunks per K token row
  static constexpr int K_DMA = KPAGE / 1024;      // 1 KB DMA instructions per K page
  static constexpr int V_DMA = VPAGE / 1024;
  static constexpr int S_LANES = Q8 ? (4 * SPAGE) / 16 : 0;
  static constexpr int NDMA = PPI * (K_DMA + V_DMA) + (Q8 ? 1 : 0);
  static constexpr int MT = D / 16;               // 16-dim tiles of O
  static_assert(KPAGE % 1024 == 0 && VPAGE % 1024 == 0, "page must be whole KB");
  static_assert(S_LANES <= 64, "scale DMA fits one instruction");
};

// XOR swizzle of the 16-byte chunk position inside a K token row in LDS, so
// the lanes that read one fragment hit distinct banks.
template <int D, int KVT>
__device__ __forceinline__ int kswz(int t, int slot) {
  constexpr int KCH = Geo<D, KVT>::KCH;
  if constexpr (KVT == kQ8) {
    int v = (t & 3) | (((t >> 3) & 1) << 2) | (((t >> 2) & 1) << 3);
    return (v ^ (slot << 3)) & (KCH - 1);
  } else {
    return t & (KCH - 1);
  }
}

// ---- numeric helpers ---------------------------------------------------------
__device__ __forceinline__ h16x2 as_h2(uint32_t u) { return __builtin_bit_cast(h16x2, u); }

// 4 int8 (one dword) -> two fp16 pairs holding the exact integers.
// (b ^ 0x80) placed under exponent byte 0x64 is 1024 + 128 + b; subtracting
// 1152 leaves b exactly.
__device__ __forceinline__ void i8x4_to_h(uint32_t w, h16x2& lo, h16x2& hi) {
  const uint32_t x = w ^ 0x80808080u;
  const h16x2 bias = {(h16)1152.0f, (h16)1152.0f};
  lo = as_h2(__builtin_amdgcn_perm(0x64646464u, x, 0x04010400u)) - bias;
  hi = as_h2(__builtin_amdgcn_perm(0x64646464u, x, 0x04030402u)) - bias;
}

__device__ __forceinline__ h16x8 cat(h16x2 a, h16x2 b, h16x2 c, h16x2 d) {
  h16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ h16x8 load_q8(const void* q, int dtype, int64_t elem) {
  if (dtype == kBF16) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(q) + elem);
    h16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[2 * i] = (h16)__builtin_bit_cast(float, raw[i] << 16);
      r[2 * i + 1] = (h16)__builtin_bit_cast(float, raw[i] & 0xffff0000u);
    }
    return r;
  } else if (dtype == kF16) {
    return *reinterpret_cast<const h16x8*>(reinterpret_cast<const h16*>(q) + elem);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(q) + elem);
    const f32x4 b = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(q) + elem + 4);
    h16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = (h16)a[i];
      r[4 + i] = (h16)b[i];
    }
    return r;
  }
}

__device__ __forceinline__ float wave_max16(float x) {  // max over lanes l, l^16, l^32, l^48
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum16(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---- the kernel -------------------------------------------------------------
template <int D, int KVT, int NT>
struct Smem {
  using G = Geo<D, KVT>;
  static constexpr int RING = kWaves * 2 * G::STAGE;
  static constexpr int QUARTER = (G::MT / 4) * NT * 1024;  // one wave's O slice for one dim quarter
  static constexpr int EPI = 12 * QUARTER;                   // 4 destinations x 3 sources
  static constexpr int BIG = RING > EPI ? RING : EPI;
  static constexpr int ML_OFF = BIG;                         // float2 (m, l) per (wave, row)
  static constexpr int POISON_OFF = ML_OFF + kWaves * 16 * NT * 8;
  static constexpr int ANC_OFF = POISON_OFF + 16;               // uint64 ancestry mask per drafted row
  static constexpr int BYTES = ANC_OFF + kMaxRows * 8;
};

template <int D, int KVT, int NT>
__global__ __launch_bounds__(256, 1) void verify_partial_kernel(const PartialParams p) {
  using G = Geo<D, KVT>;
  using SM = Smem<D, KVT, NT>;
  static_assert(SM::BYTES <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[SM::BYTES];

  constexpr int KSTEPS = D / 32;  // k-steps of 32 dims in Q K^T
  constexpr int MT = G::MT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m16 = lane & 15;  // M index (key / dim) or N index (row) within a 16x16 tile
  const int g4 = lane >> 4;   // lane group

  const int s = blockIdx.z;
  const int kvh = blockIdx.y;
  const int split = blockIdx.x % p.S;
  const int rg = blockIdx.x / p.S;
  const int B = p.B;
  const int M = B * p.G;
  const int rowbase = rg * p.rows_per_group;

  // ---- validate sequence metadata (device-resident) ----
  int ctx = p.ctx_lens[s];
  bool poison = false;
  if (ctx < B || ctx > p.max_ctx || ctx > p.max_pages * kPage) {
    poison = true;
    ctx = 0;
  }
  uint32_t flagbits = poison ? VA_FLAG_BAD_CTX : 0u;
  if (p.parent) {
    bool bad = false;
    if (lane < B) {
      const int par = p.parent[(int64_t)s * B + lane];
      bad = (par < -1 || par >= lane);
    }
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
      poison = true;
      flagbits |= VA_FLAG_BAD_PARENT;
    }
  }
  const int base = ctx - B;  // slot of drafted row 0

  // ---- prologue through LDS: Q rows as fp16 and per-row ancestry masks ----
  // The ring is not in use yet, so its first bytes stage the workgroup's Q
  // tile [16*NT rows][D] (fp16, row-major) and the B ancestry bitmasks.
  constexpr int QROWS = 16 * NT;
  h16* q_lds = reinterpret_cast<h16*>(smem);
  uint64_t* anc_lds = reinterpret_cast<uint64_t*>(smem + SM::ANC_OFF);
  static_assert(QROWS * D * 2 <= SM::RING, "prologue staging fits the ring");
  {
    // 8 consecutive elements per thread per step
    constexpr int CH = D / 8;
    for (int idx = tid; idx < QROWS * CH; idx += kThreads) {
      const int rr = idx / CH, c8 = idx % CH;
      const int r = rowbase + rr;
      h16x8 v = h16x8{};
      if (r < M) {
        const int hl = r / B, b = r % B;
        const int64_t qrow = ((int64_t)(s * B + b) * p.H + kvh * p.G + hl) * D;
        v = load_q8(p.q, p.q_dtype, qrow + 8 * c8);
      }
      *reinterpret_cast<h16x8*>(q_lds + rr * D + 8 * c8) = v;
    }
    if (tid < B) {
      uint64_t a = 0;
      int i = tid;
      for (int guard = 0; guard < kMaxRows && i >= 0; ++guard) {
        a |= (uint64_t)1 << i;
        const int par = p.parent ? p.parent[(int64_t)s * B + i] : i - 1;
        i = (par < i) ? par : -1;  // a malformed parent is flagged above; stop the walk
      }
      anc_lds[tid] = poison ? 0 : a;
    }
  }
  __syncthreads();
  h16x8 qf[NT][KSTEPS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int rr = 16 * nt + m16;
    const int r = rowbase + rr;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      int dim0;
      if constexpr (KVT == kQ8) dim0 = 64 * (ks >> 1) + 16 * g4 + 8 * (ks & 1);
      else dim0 = 32 * ks + 8 * g4;
      qf[nt][ks] = *reinterpret_cast<const h16x8*>(q_lds + rr * D + dim0);
    }
  }
  __syncthreads();  // the ring may now overwrite the staging area

  // ---- this split's pages ----
  const int npages = (ctx + kPage - 1) / kPage;
  const int pps = (npages + p.S - 1) / p.S;
  const int p_begin = min(split * pps, npages);
  const int p_end = min(p_begin + pps, npages);
  const int split_end = min(ctx, p_end * kPage);
  const int mask_from = min(base, split_end);  // first token that needs a per-key test
  const int npairs = (p_end - p_begin + G::PPI - 1) / G::PPI;
  const int n_my = npairs > wave ? (npairs - wave + kWaves - 1) / kWaves : 0;
  const int32_t* bt_row = p.block_table + (int64_t)s * p.max_pages;

  const char* kbase = reinterpret_cast<const char*>(p.k_pool) + (int64_t)kvh * G::KPAGE;
  const char* vbase = reinterpret_cast<const char*>(p.v_pool) + (int64_t)kvh * G::VPAGE;
  const char* ksbase = reinterpret_cast<const char*>(p.k_scale) + (int64_t)kvh * G::SPAGE;
  const char* vsbase = reinterpret_cast<const char*>(p.v_scale) + (int64_t)kvh * G::SPAGE;
  const int64_t kstride = (int64_t)p.KVH * G::KPAGE;  // bytes between pages
  const int64_t vstride = (int64_t)p.KVH * G::VPAGE;
  const int64_t sstride = (int64_t)p.KVH * G::SPAGE;

  const uint32_t lds_ring = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)smem);
  const uint32_t my_ring = __builtin_amdgcn_readfirstlane(lds_ring + wave * 2 * G::STAGE);

  // K DMA: instruction c of a page fills LDS bytes [1024c, 1024c + 1024) of
  // the page slot; the lane's destination chunk (token t, position pos) takes
  // global chunk pos ^ swizzle(t).
  auto kdma_off = [&](int sl, int c) __attribute__((always_inline)) -> uint32_t {
    const int byte = 1024 * c + 16 * lane;
    const int t = byte / G::KROW;
    const int pos = (byte % G::KROW) / 16;
    return (uint32_t)(t * G::KROW + 16 * (pos ^ kswz<D, KVT>(t, sl)));
  };

  // Page ids: one per lane for the next 64 pages this wave will stream (lane
  // l <-> wave iteration x = chunk*IPC + l/PPI, slot l%PPI), read back with a
  // uniform readlane.  Reloading happens once per 64 pages; it is a plain
  // vector load, so the compiler drains the in-flight DMA there (rare).
  constexpr int IPC = 64 / G::PPI;  // wave iterations per id chunk
  bool bad_page = false;
  int idreg = 0;
  auto load_ids = [&](int chunk) {
    const int x = chunk * IPC + lane / G::PPI;
    const int sl = lane % G::PPI;
    int pidx = p_begin + G::PPI * (wave + kWaves * x) + sl;
    if (pidx >= p_end) pidx = p_begin;  // padding slot: any valid page, never unmasked
    int id = (p_begin < p_end) ? p.block_table[(int64_t)s * p.max_pages + pidx] : 0;
    const bool bad = (id < 0 || id >= p.num_pages);
    if (__builtin_amdgcn_ballot_w64(bad) != 0) bad_page = true;
    idreg = bad ? 0 : id;
  };

  auto issue = [&](int x, int stage) {
    if (x % IPC == 0) load_ids(x / IPC);
    int ids[G::PPI];
#pragma unroll
    for (int sl = 0; sl < G::PPI; ++sl) ids[sl] = __builtin_amdgcn_readlane(idreg, G::PPI * (x % IPC) + sl);
    const uint32_t st = my_ring + stage * G::STAGE;
#pragma unroll
    for (int sl = 0; sl < G::PPI; ++sl) {
      const char* kp = kbase + (int64_t)ids[sl] * kstride;
#pragma unroll
      for (int c = 0; c < G::K_DMA; ++c) dma_saddr(kp, kdma_off(sl, c), st + G::K_OFF + sl * G::KPAGE + 1024 * c);
      const char* vp = vbase + (int64_t)ids[sl] * vstride;
#pragma unroll
      for (int c = 0; c < G::V_DMA; ++c) dma_saddr(vp + 1024 * c, 16 * lane, st + G::V_OFF + sl * G::VPAGE + 1024 * c);
    }
    if constexpr (G::Q8) {
      // [KS slot0 | KS slot1 | VS slot0 | VS slot1], SPAGE bytes each; lane 0
      // is always active, so the instruction counts once in vmcnt.
      if (lane < G::S_LANES) {
        const int byte = 16 * lane;
        const int region = byte / G::SPAGE;
        const int off = byte % G::SPAGE;
        const int sl = region & 1;
        const int id = sl ? ids[G::PPI - 1] : ids[0];
        const char* src = (region < 2 ? ksbase : vsbase) + (int64_t)id * sstride + off;
        dma_vaddr(src, st + G::KS_OFF);
      }
    }
  };

  // ---- online softmax state ----
  f32x4 oacc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) oacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
  }
  const float c2 = p.scale_log2;

  constexpr int UT = G::PPI;   // 16-key tiles per wave iteration
  constexpr int KPL = 4 * UT;  // keys per lane per row tile

  // Iteration state shared by the phases below.
  uint32_t st = 0;
  int tok0 = 0;
  bool masked = false;
  float sv[NT][KPL];  // raw scores (masked ones -inf) of the current iteration
  float tmax[NT];     // their per-row max, log2 units

  // Phase 1: wait for this iteration's pages, S^T = K Q^T, mask, row max.
  // Returns true when some row's max passed the lazy-rescale threshold.
  auto begin_iter = [&](int it) __attribute__((always_inline)) {
    const int pair = wave + kWaves * it;
    st = my_ring + (it & 1) * G::STAGE;
    tok0 = (p_begin + G::PPI * pair) * kPage;
    masked = (tok0 + G::PPI * kPage) > mask_from;
  };

  auto phase_scores = [&]() __attribute__((always_inline)) -> bool {

    f32x4 sacc[UT][NT];
#pragma unroll
    for (int u = 0; u < UT; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[u][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int u = 0; u < UT; ++u) {
      if constexpr (KVT == kQ8) {
        // M row m16 of tile u is key (slot m16/8, token 8*((m16/4)&1) + 4u + m16%4)
        const int sl = m16 >> 3;
        const int t = 8 * ((m16 >> 2) & 1) + 4 * u + (m16 & 3);
        const uint32_t krow = st + G::K_OFF + sl * G::KPAGE + t * G::KROW;
        const uint32_t srow = st + G::KS_OFF + sl * G::SPAGE + t * (D / 32) * 2;
        h16 kscale[D / 64];
#pragma unroll
        for (int j = 0; j < D / 64; ++j) kscale[j] = *LDS_PTR(h16, srow + 2 * (2 * j + (g4 >> 1)));
#pragma unroll
        for (int j = 0; j < D / 64; ++j) {
          const int c = 4 * j + g4;
          const u32x4 raw = *LDS_PTR(u32x4, krow + 16 * (c ^ kswz<D, KVT>(t, sl)));
          const h16x2 d2 = {kscale[j], kscale[j]};
          h16x2 a0, a1, a2, a3, b0, b1, b2, b3;
          i8x4_to_h(raw[0], a0, a1);
          i8x4_to_h(raw[1], a2, a3);
          i8x4_to_h(raw[2], b0, b1);
          i8x4_to_h(raw[3], b2, b3);
          const h16x8 k0 = cat(a0 * d2, a1 * d2, a2 * d2, a3 * d2);
          const h16x8 k1 = cat(b0 * d2, b1 * d2, b2 * d2, b3 * d2);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            sacc[u][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qf[nt][2 * j], sacc[u][nt], 0, 0, 0);
            sacc[u][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, qf[nt][2 * j + 1], sacc[u][nt], 0, 0, 0);
          }
        }
      } else {
        const int t = m16;
        const uint32_t krow = st + G::K_OFF + t * G::KROW;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const int c = 4 * ks + g4;
          const h16x8 k0 = *LDS_PTR(h16x8, krow + 16 * (c ^ kswz<D, KVT>(t, 0)));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            sacc[u][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qf[nt][ks], sacc[u][nt], 0, 0, 0);
        }
      }
    }

    // Lane (row m16, group g4) holds, per tile u, accumulator element i = key
    // (slot g4/2, token 8*(g4&1) + 4u + i) for Q8, or token 4*g4 + i for fp16.
    bool need = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int u = 0; u < UT; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[nt][4 * u + i] = sacc[u][nt][i];
      if (masked) {
        const int r = rowbase + 16 * nt + m16;
        const uint64_t anc = (r < M) ? anc_lds[r % B] : 0;
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          int j;
          if constexpr (KVT == kQ8) j = tok0 + 16 * (g4 >> 1) + 8 * (g4 & 1) + e;
          else j = tok0 + 4 * g4 + e;
          // visible iff j < split_end and (j < base or bit (j - base) of anc);
          // branch-free: 0 <= j - base < 64 always holds when j >= base here.
          const uint32_t rel = (uint32_t)(j - base) & 63u;
          const uint32_t bit = (uint32_t)(anc >> rel) & 1u;
          const uint32_t vis = (uint32_t)(j < split_end) & ((uint32_t)(j < base) | bit);
          sv[nt][e] = vis ? sv[nt][e] : -INFINITY;
        }
      }
      float mx = sv[nt][0];
#pragma unroll
      for (int e = 1; e < KPL; ++e) mx = fmaxf(mx, sv[nt][e]);
      tmax[nt] = mx * c2;
      need |= tmax[nt] > m_run[nt] + kLazyRescale;
    }
    return __builtin_amdgcn_ballot_w64(need) != 0;
  };

  // Raise every row's reference max to the largest scaled score seen so far.
  auto raise_reference = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) m_run[nt] = fmaxf(m_run[nt], wave_max16(tmax[nt]));
  };

  // Phase 2: P = 2^(t - m_ref) in fp16 (registers only), O^T += V^T P^T.
  auto phase_pv = [&]() __attribute__((always_inline)) {
    h16x8 pf[NT];   // Q8: 8 keys per lane (one 32-key k-step)
    h16x4 pf4[NT];  // fp16: 4 keys per lane (one 16-key k-step)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mref = (m_run[nt] == -INFINITY) ? 0.f : m_run[nt];
      float lsum = 0.f;
      float pv[KPL];
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        pv[e] = fast_exp2(__builtin_fmaf(sv[nt][e], c2, -mref));
        lsum += pv[e];
      }
      l_run[nt] += lsum;
      if constexpr (KVT == kQ8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[nt][e] = (h16)pv[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) pf4[nt][e] = (h16)pv[e];
      }
    }

    if constexpr (KVT == kQ8) {
      const int sl = g4 >> 1;
      const uint32_t vrow = st + G::V_OFF + sl * G::VPAGE + 8 * (g4 & 1);
      const uint32_t vsrow = st + G::VS_OFF + sl * G::SPAGE + 16 * (g4 & 1);
      // This lane's 8 tokens that lie past the split end carry no data (stale
      // LDS, NaN-poisoned tails): zero their scales so their V reads as 0.
      u32x4 smask;
      {
        const int jt0 = tok0 + 16 * sl + 8 * (g4 & 1);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          smask[e2] = (jt0 + 2 * e2 < split_end ? 0x0000ffffu : 0u) | (jt0 + 2 * e2 + 1 < split_end ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int b = 0; b < D / 32; ++b) {
        h16x8 vs = *LDS_PTR(h16x8, vsrow + 32 * b);
        vs = __builtin_bit_cast(h16x8, __builtin_bit_cast(u32x4, vs) & smask);
        const h16x2 s01 = {vs[0], vs[1]}, s23 = {vs[2], vs[3]}, s45 = {vs[4], vs[5]}, s67 = {vs[6], vs[7]};
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int mt = 2 * b + half;
          const u32x2 raw = *LDS_PTR(u32x2, vrow + (16 * mt + m16) * 16);
          h16x2 v01, v23, v45, v67;
          i8x4_to_h(raw[0], v01, v23);
          i8x4_to_h(raw[1], v45, v67);
          const h16x8 vf = cat(v01 * s01, v23 * s23, v45 * s45, v67 * s67);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            oacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[nt], oacc[mt][nt], 0, 0, 0);
        }
      }
    } else {
      const uint32_t vrow = st + G::V_OFF + 8 * g4;
      u32x2 vmask;
      {
        const int jt0 = tok0 + 4 * g4;
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2)
          vmask[e2] = (jt0 + 2 * e2 < split_end ? 0x0000ffffu : 0u) | (jt0 + 2 * e2 + 1 < split_end ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        h16x4 vf = *LDS_PTR(h16x4, vrow + (16 * mt + m16) * 32);
        vf = __builtin_bit_cast(h16x4, __builtin_bit_cast(u32x2, vf) & vmask);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          oacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, pf4[nt], oacc[mt][nt], 0, 0, 0);
      }
    }
  };

  auto prefetch = [&](int it) __attribute__((always_inline)) {
    if (it + 1 < n_my) {
      issue(it + 1, (it + 1) & 1);
      wait_vmcnt<G::NDMA>();
    } else {
      wait_vmcnt<0>();
    }
  };

  // P is stored as fp16, so a score may exceed its row's reference max by at
  // most kLazyRescale (log2 units) before 2^(t - m_ref) leaves the fp16 range.
  // The reference is fixed while accumulating; if a later page carries a
  // score beyond that margin (rare: the first page usually sets a max that
  // holds), the wave raises every row's reference to the largest score seen
  // so far, clears its accumulators and streams its pages again.  Each such
  // restart raises some reference by more than the margin, so the number of
  // restarts is bounded by the score range.
  if (n_my > 0) issue(0, 0);
  int it = 0;
  for (;;) {
    bool restart = false;
    for (; it < n_my; ++it) {  // hot loop: nothing here rewrites the accumulators
      prefetch(it);
      begin_iter(it);
      if (phase_scores()) {
        if (it > 0) {
          restart = true;
          break;
        }
        raise_reference();  // first page of a pass: nothing accumulated yet
      }
      phase_pv();
    }
    if (!restart) break;
    // Rare path: raise the references, clear and stream this wave's pages again.
    raise_reference();
    wait_vmcnt<0>();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) oacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) l_run[nt] = 0.f;
    it = 0;
    issue(0, 0);
  }

  if (bad_page) {
    poison = true;
    flagbits |= VA_FLAG_BAD_PAGE;
  }
  if (flagbits && lane == 0) atomicOr(p.flags, flagbits);

  // ---- epilogue: merge the 4 waves' states ----
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) l_run[nt] = wave_sum16(l_run[nt]);

  float2* ml = reinterpret_cast<float2*>(smem + SM::ML_OFF);
  int* poison_w = reinterpret_cast<int*>(smem + SM::POISON_OFF);
  __syncthreads();  // every wave is past its ring; LDS may be reused
  if (g4 == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) ml[wave * 16 * NT + 16 * nt + m16] = make_float2(m_run[nt], l_run[nt]);
  }
  if (lane == 0) poison_w[wave] = poison ? 1 : 0;
  __syncthreads();
  bool any_poison = false;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) any_poison |= (poison_w[w] != 0);

  float Mrow[NT], Lrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) Mx = fmaxf(Mx, ml[w * 16 * NT + 16 * nt + m16].x);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float2 v = ml[w * 16 * NT + 16 * nt + m16];
      L += (v.x == -INFINITY) ? 0.f : v.y * fast_exp2(v.x - Mx);
    }
    Mrow[nt] = Mx;
    Lrow[nt] = L;
    const float wown = (m_run[nt] == -INFINITY) ? 0.f : fast_exp2(m_run[nt] - Mx);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[mt][nt] *= wown;
  }

  // Reduce-scatter over dim quarters: wave w finalises dim tiles [w*MT/4, (w+1)*MT/4).
  constexpr int QMT = MT / 4;
  auto epi_slot = [&](int dst, int src) -> int {  // 12 slots: (dst, src != dst)
    return dst * 3 + (src < dst ? src : src - 1);
  };
#pragma unroll
  for (int dst = 0; dst < kWaves; ++dst) {
    if (dst == wave) continue;
    char* region = smem + epi_slot(dst, wave) * SM::QUARTER;
#pragma unroll
    for (int qm = 0; qm < QMT; ++qm)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<f32x4*>(region + (qm * NT + nt) * 1024 + 16 * lane) = oacc[dst * QMT + qm][nt];
  }
  __syncthreads();
  f32x4 fin[QMT][NT];
#pragma unroll
  for (int qm = 0; qm < QMT; ++qm)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      // own contribution: pick the static slice with a uniform switch
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (w == wave) acc = oacc[w * QMT + qm][nt];
#pragma unroll
      for (int src = 0; src < kWaves; ++src) {
        if (src == wave) continue;
        const char* region = smem + epi_slot(wave, src) * SM::QUARTER;
        acc += *reinterpret_cast<const f32x4*>(region + (qm * NT + nt) * 1024 + 16 * lane);
      }
      fin[qm][nt] = acc;
    }

  // ---- write ----
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = rowbase + 16 * nt + m16;
    if (r >= M) continue;
    const int hl = r / B, b = r % B;
    const int64_t R = (int64_t)(s * B + b) * p.H + kvh * p.G + hl;
    const float Mx = Mrow[nt], L = Lrow[nt];
    if (p.direct) {
      const float inv = any_poison ? __builtin_nanf("") : 1.0f / L;
#pragma unroll
      for (int qm = 0; qm < QMT; ++qm) {
        const int dim = 16 * (wave * QMT + qm) + 4 * g4;
        const f32x4 o = fin[qm][nt] * inv;
        if (p.out_dtype == kF32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + R * D + dim) = o;
        } else if (p.out_dtype == kF16) {
          h16x4 h = {(h16)o[0], (h16)o[1], (h16)o[2], (h16)o[3]};
          *reinterpret_cast<h16x4*>(reinterpret_cast<h16*>(p.out) + R * D + dim) = h;
        } else {
          u32x2 w;
#pragma unroll
          for (int i = 0; i < 2; ++i) w[i] = f32_to_bf16_bits(o[2 * i]) | (f32_to_bf16_bits(o[2 * i + 1]) << 16);
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + R * D + dim) = w;
        }
      }
      if (wave == 0 && g4 == 0 && p.lse)
        p.lse[R] = any_poison ? __builtin_nanf("") : kLn2 * (Mx + __builtin_log2f(L));
    } else {
      float* po = p.part_o + ((int64_t)split * p.nrows + R) * D;
#pragma unroll
      for (int qm = 0; qm < QMT; ++qm) {
        const int dim = 16 * (wave * QMT + qm) + 4 * g4;
        *reinterpret_cast<f32x4*>(po + dim) = any_poison ? f32x4{__builtin_nanf(""), 0.f, 0.f, 0.f} : fin[qm][nt];
      }
      if (wave == 0 && g4 == 0) {
        p.part_m[(int64_t)split * p.nrows + R] = any_poison ? 0.f : Mx;
        p.part_l[(int64_t)split * p.nrows + R] = any_poison ? __builtin_nanf("") : L;
      }
    }
  }
}

}  // namespace

// ---- dispatch -----------------------------------------------------------------

Tiling choose_tiling(int B, int G, int D) {
  const int M = B * G;
  const int nt_max = (D >= 256) ? 3 : 6;
  const int tiles = (M + 15) / 16;
  Tiling t;
  t.row_groups = (tiles + nt_max - 1) / nt_max;
  int nt = (tiles + t.row_groups - 1) / t.row_groups;
  if (nt == 5) nt = 6;
  t.nt = nt;
  return t;
}

bool partial_supported(int D, int kv_dtype, int nt) {
  if (kv_dtype != kQ8 && kv_dtype != kF16) return false;
  if (D != 64 && D != 128 && D != 256) return false;
  if (D == 256) return nt >= 1 && nt <= 3;
  return nt == 1 || nt == 2 || nt == 3 || nt == 4 || nt == 6;
}

template <int D, int KVT, int NT>
static hipError_t launch_t(const PartialParams& p, hipStream_t stream) {
  dim3 grid((unsigned)(p.S * p.row_groups), (unsigned)p.KVH, (unsigned)p.num_seqs);
  hipLaunchKernelGGL((verify_partial_kernel<D, KVT, NT>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, int KVT>
static hipError_t launch_nt(const PartialParams& p, int nt, hipStream_t stream) {
  switch (nt) {
    case 1: return launch_t<D, KVT, 1>(p, stream);
    case 2: return launch_t<D, KVT, 2>(p, stream);
    case 3: return launch_t<D, KVT, 3>(p, stream);
    default: break;
  }
  if constexpr (D <= 128) {
    if (nt == 4) return launch_t<D, KVT, 4>(p, stream);
    if (nt == 6) return launch_t<D, KVT, 6>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_partial(const PartialParams& p, int kv_dtype, int nt, hipStream_t stream) {
  if (kv_dtype == kQ8) {
    if (p.D == 256) return launch_nt<256, kQ8>(p, nt, stream);
    if (p.D == 128) return launch_nt<128, kQ8>(p, nt, stream);
    if (p.D == 64) return launch_nt<64, kQ8>(p, nt, stream);
  } else if (kv_dtype == kF16) {
    if (p.D == 256) return launch_nt<256, kF16>(p, nt, stream);
    if (p.D == 128) return launch_nt<128, kF16>(p, nt, stream);
    if (p.D == 64) return launch_nt<64, kF16>(p, nt, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace va
