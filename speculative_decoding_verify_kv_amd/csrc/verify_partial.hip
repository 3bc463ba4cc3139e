// Split-KV partial kernel for speculative-decoding verify attention, gfx950.
//
// One workgroup = (sequence s, KV head, split k, row group).  Its rows are
// 16*NT (query head, drafted row) pairs of one KV group: every query head of
// a GQA group reads the same KV head, so the group's B*G rows form the N side
// of a real matrix product with the streamed keys and each fetched KV byte
// feeds all of them (the multi-row verifier idea of the page "perf(gfx11):
// optimize Qwen DFlash speculative verify", alpineQ's notes, taken to the
// whole group).
//
// The workgroup has 8 waves in two roles, one of each role per SIMD, so that
// one wave's matrix-core work overlaps the other's vector work:
//   score waves (rh, kh)   rows half rh, pages 2kh and 2kh + 1 of every
//                          64-key tile: S^T = K Q^T on v_mfma_f32_16x16x32_f16
//                          (keys on M, rows on N, Q resident in registers);
//                          8-bit K enters as its exact int8 codes, one MFMA
//                          per 32-dim scale block, and the block scale is
//                          applied to each fp32 block product; causal / tree /
//                          page-tail mask, P = 2^(t - m_ref) in fp16 -> LDS.
//   output waves q = 0..3  each owns head_dim quarter q: dequant of that
//                          quarter of the tile's V, O^T += V^T P^T on the same
//                          MFMA, with P of the previous tile read from LDS.
//                          They also issue every LDS-DMA: page q of K (and its
//                          scales), that quarter of V (and page q's scales).
// Every V element is therefore dequantised once per workgroup (K codes are
// converted once per row half), and O lives in exactly one wave, so the
// epilogue needs no cross-wave O reduction.
//
// Pipeline: separate K and V rings of R stages, filled by
// global_load_lds_dwordx4 (no VGPR holds data in flight).  Iteration i: score
// waves compute tile i while output waves accumulate tile i-1; one barrier per
// iteration.  K of tile i + R_K - 1 and V of tile i + R_V - 2 are issued at the
// start of iteration i by the output waves, which wait on their own vmcnt
// before the barrier; the score waves, whose work bounds the loop, issue no
// DMA and wait on nothing but the barrier.
//
// Softmax: log2 domain with a reference max per row held by every wave.  A
// score may exceed its row's reference by at most 15 (P stays within fp16);
// when one does (always on the first tile), all waves take a short rare path
// after the barrier: the score waves publish the tile's row maxima, every wave
// raises the reference, the output waves rescale O, the score waves rescale l
// and rewrite the tile's P.
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

constexpr int kRoleWaves = 4;                      // score waves; as many output waves
constexpr int kBlockThreads = 64 * 2 * kRoleWaves;  // 512
// A lane's partial row sum over its P values of a tile bounds each of them, so
// sums at or below 2^15 keep every P value well inside fp16 (max 65504).
constexpr float kLazyRescale = 32768.0f;
constexpr float kFiniteFloor = -1e30f;  // stands for an unset (-inf) reference in differences
constexpr float kLn2 = 0.6931471805599453f;

// ---- LDS-DMA helpers -------------------------------------------------------
// global_load_lds_dword[x4]: each active lane copies 4 (16) bytes from its
// global address to LDS at M0 + 4 (16) * lane.  M0 is saved and restored.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

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

__device__ __forceinline__ void dma_saddr_b32(const void* sbase_in, uint32_t voff, uint32_t lds_in) {
  const void* sbase = uniform_ptr(sbase_in);
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_in);
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most n * PER of this wave's vector-memory loads are in flight
// (n is clamped to [0, 4]).
template <int PER>
__device__ __forceinline__ void wait_vmcnt_n(int n) {
  if (n <= 0) wait_vmcnt<0>();
  else if (n == 1) wait_vmcnt<PER>();
  else if (n == 2) wait_vmcnt<2 * PER>();
  else if (n == 3) wait_vmcnt<3 * PER>();
  else wait_vmcnt<4 * PER>();
}

// Workgroup barrier that makes this wave's LDS writes visible; it does not
// wait for in-flight global loads (the ring waits on vmcnt itself).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---- geometry ------------------------------------------------------------------
template <int D, int KVT>
struct Geo {
  static constexpr bool Q8 = (KVT == kQ8);
  static constexpr int ESZ = Q8 ? 1 : 2;          // bytes per K/V element
  static constexpr int KROW = D * ESZ;            // bytes of one token's K row
  static constexpr int KPAGE = 16 * KROW;         // K bytes of one page (one KV head)
  static constexpr int KCH = KPAGE / 1024;        // 1 KB chunks of a K page
  static constexpr int SPB = Q8 ? D : 0;          // bytes of one page's K (or V) scales
  static constexpr int VROW = 16 * ESZ;           // bytes of one dim row (16 tokens) of a V page
  static constexpr int VPAGE = D * VROW;
  static constexpr int DO = D / 4;                // head_dim entries per output wave
  static constexpr int MTO = DO / 16;             // 16-dim tiles per output wave
  static constexpr int VCH = MTO * (VROW / 16);   // 1 KB V chunks per output wave per tile
  static constexpr int NDMA = KCH + (Q8 ? 1 : 0); // DMA instructions of one K page or V quarter of a tile
  static constexpr int K_STAGE = 4 * KPAGE + 4 * SPB;
  static constexpr int V_STAGE = 4 * VPAGE + 4 * SPB;
  static constexpr int KSTEPS = D / 32;
  static_assert(KCH == VCH, "a tile's K page and V quarter take the same number of DMAs");
  static_assert(KPAGE % 1024 == 0, "page must be whole KB");
};

template <int D, int KVT, int NT>
struct Lay {
  using G = Geo<D, KVT>;
  static constexpr int P_BUF = 2 * NT * 1024;  // one tile's P: [h][nt][lane] x 16 B
  static constexpr int EX_BYTES = 2 * 16 * NT * 4;
  static constexpr int MISC = 512 + 512 + EX_BYTES + 64;
  static constexpr int BUDGET = 160 * 1024;
  static constexpr int AVAIL = BUDGET - 2 * P_BUF - MISC;
  // deepest K / V rings that fit (V is consumed one iteration after K)
  static constexpr int pick() {
    constexpr int c[5][2] = {{4, 4}, {3, 4}, {3, 3}, {2, 3}, {2, 2}};
    for (int i = 0; i < 5; ++i)
      if (c[i][0] * G::K_STAGE + c[i][1] * G::V_STAGE <= AVAIL) return i;
    return 4;
  }
  static constexpr int RK = pick() == 0 ? 4 : pick() <= 2 ? 3 : 2;
  static constexpr int RV = pick() <= 1 ? 4 : pick() <= 3 ? 3 : 2;
  static constexpr int KR_OFF = 0;
  static constexpr int VR_OFF = RK * G::K_STAGE;
  static constexpr int P_OFF = VR_OFF + RV * G::V_STAGE;
  static constexpr int IDS_OFF = P_OFF + 2 * P_BUF;  // int32 [2][64] page ids
  static constexpr int ANC_OFF = IDS_OFF + 512;      // uint64 [64] ancestry masks
  static constexpr int EX_OFF = ANC_OFF + 512;       // float [2][16 NT] row exchange
  static constexpr int FLAG_OFF = EX_OFF + EX_BYTES; // int flags [16]: [0..3] shared, [8..15] one per wave
  static constexpr int BYTES = FLAG_OFF + 64;
  // Q staging (fp16 [16 NT][D]) during the prologue: the V ring receives
  // nothing before the first iteration.
  static constexpr int QST_BYTES = 16 * NT * D * 2;
  // when the V ring's stages 1.. hold it, stage 0 takes V of tile 0 before
  // the staging is read (EV)
  static constexpr bool EV = RV >= 2 && (RV - 1) * G::V_STAGE >= QST_BYTES;
  static constexpr int QST_OFF = EV ? VR_OFF + G::V_STAGE : VR_OFF;
  static_assert(BYTES <= BUDGET, "LDS budget");
  static_assert(QST_OFF + QST_BYTES <= VR_OFF + RV * G::V_STAGE, "Q staging fits the V ring");
  static_assert(RK >= 2 && RV >= 2, "ring depth");
};

// ---- numeric helpers ---------------------------------------------------------
__device__ __forceinline__ h16x2 as_h2(uint32_t u) { return __builtin_bit_cast(h16x2, u); }

// 4 int8 (one dword) -> two fp16 pairs holding the exact integers: each
// byte is sign-extended and converted by a byte-selecting v_cvt_f16_i16 into
// one half of a packed register (4 instructions per dword).
__device__ __forceinline__ void i8x4_to_h(uint32_t w, h16x2& lo, h16x2& hi) {
  uint32_t a, c;
  asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(a) : "v"(w));
  asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1" : "+v"(a) : "v"(w));
  asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(c) : "v"(w));
  asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3" : "+v"(c) : "v"(w));
  lo = as_h2(a);
  hi = as_h2(c);
}

__device__ __forceinline__ h16x8 cat(h16x2 a, h16x2 b, h16x2 c, h16x2 d) {
  h16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Two dwords of int8 (8 values) times per-pair scales -> one MFMA fragment.
__device__ __forceinline__ h16x8 deq8(uint32_t w0, uint32_t w1, h16x2 s0, h16x2 s1, h16x2 s2, h16x2 s3) {
  h16x2 a, b, c, d;
  i8x4_to_h(w0, a, b);
  i8x4_to_h(w1, c, d);
  return cat(a * s0, b * s1, c * s2, d * s3);
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

// Keep-mask for 8 consecutive tokens starting at `first`: fp16 lanes of
// tokens at or past `end` are cleared (their pages may hold anything).
__device__ __forceinline__ u32x4 tail_mask(int first, int end) {
  u32x4 m;
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2)
    m[e2] = (first + 2 * e2 < end ? 0x0000ffffu : 0u) | (first + 2 * e2 + 1 < end ? 0xffff0000u : 0u);
  return m;
}

// ---- the kernel -------------------------------------------------------------
// SQ: split each sequence by its own context with at least kMinSplitPages
// pages per split (ragged calls, whose sequences differ widely in length);
// otherwise every sequence takes S equal splits.
// One workgroup's work in the LDS block `smem` (16 NT rows of the group list
// per workgroup).
template <int D, int KVT, int NT, bool SQ>
__device__ __forceinline__ void partial_body(const PartialParams p, char* smem) {
  using G = Geo<D, KVT>;
  using L = Lay<D, KVT, NT>;
  static_assert(NT % 2 == 0, "the score waves take half the rows each");
  constexpr int RK = L::RK, RV = L::RV;
  constexpr int NS = NT / 2;  // row tiles per score wave
  constexpr int KSTEPS = G::KSTEPS;
  constexpr int NDMA = G::NDMA;
  constexpr int QROWS = 16 * NT;
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)smem);

  // The kernel arguments span four 64-byte scalar-cache lines.  Reading one
  // field of each at once puts all four in one round trip; the compiler
  // would otherwise fetch them in dependent batches as branches need them,
  // a memory latency each when every workgroup starts at once.  Uniform
  // calls get the arguments their Q copies need in SGPRs at wave launch (the
  // leading kernel arguments, preloaded) and touch the lines after issuing
  // the copies, below.
  if constexpr (SQ) asm volatile("" ::"s"(p.q), "s"(p.cu_rows), "s"(p.num_seqs), "s"(p.S));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool is_score = wave < kRoleWaves;
  const int role = is_score ? wave : wave - kRoleWaves;  // page (score) or dim quarter (output)
  const int n16 = lane & 15;  // M or N index within a 16x16 tile
  const int g4 = lane >> 4;   // lane group

  // Workgroup -> (split, row group).  When every split has several row
  // groups, the row groups of one split get block ids 8 apart: blocks are
  // dealt round-robin to the 8 XCDs, so they share one L2 and run together.
  // Ragged calls (SQ) take their (sequence, row group, split, KV head) from
  // the work list the schedule pass wrote: entry blockIdx.x, while entries
  // are in use (the grid holds as many workgroups as the list can).  The list
  // is dense and longest first, so the workgroups that do work are dealt
  // evenly to the 8 XCDs (round-robin by block id) and the long ones start
  // first; the pass also reports bad cu_rows entries (their sequences have
  // no entries).
  int s, kvh, split, rg;
  if constexpr (SQ) {
    const auto* cnt = reinterpret_cast<const __attribute__((address_space(4))) int*>((uintptr_t)p.item_count);
    if ((int)blockIdx.x >= cnt[0]) return;
    const auto* it =
        reinterpret_cast<const __attribute__((address_space(4))) int*>((uintptr_t)(p.items + blockIdx.x));
    s = it[0] & kItemSeqMask;
    const int packed = it[1];
    rg = packed >> 16;
    split = (packed >> 8) & 255;
    kvh = packed & 255;
  } else {
    s = blockIdx.z;
    kvh = blockIdx.y;
    if (p.row_groups > 1 && (p.S & 7) == 0) {
      const int x = blockIdx.x, hi = x >> 3;
      rg = hi % p.row_groups;
      split = (hi / p.row_groups) * 8 + (x & 7);
    } else {
      split = blockIdx.x % p.S;
      rg = blockIdx.x / p.S;
    }
  }
  // Rows of this sequence: B each, or (ragged) cu_rows[s] .. cu_rows[s+1]
  // of the packed q / out rows.  Row r of the group list is (head hl, row b)
  // with r = hl * B + b.
  int B = p.B;
  int64_t r0 = (int64_t)s * p.B;
  bool bad_rows = false;
  if (SQ && p.cu_rows) {
    const auto* cu = reinterpret_cast<const __attribute__((address_space(4))) int*>((uintptr_t)(p.cu_rows + s));
    const int a = cu[0], e = cu[1];
    bad_rows = a < 0 || e < a || e > p.total_rows || e - a > p.B;
    B = bad_rows ? 0 : e - a;
    r0 = a;
  }
  const int M = B * p.G;
  const int rowbase = rg * QROWS;
  if (rowbase >= M) {
    // no rows of this sequence in this group (nothing is written)
    if (bad_rows && tid == 0 && (SQ ? split == 0 && rg == 0 : blockIdx.x == 0) && kvh == 0)
      atomicOr(p.flags, (uint32_t)VA_FLAG_BAD_ROWS);
    return;
  }

  const int32_t* bt_row;
  int npg_max, pps_spec, pb_spec, pe_spec;
  // The split's place at ctx = max_ctx and its row of the block table (z is
  // 0: in uniform calls it comes from an asm statement after the Q copies,
  // which keeps these reads of the argument block behind them).
  auto split_meta = [&](int z) __attribute__((always_inline)) {
    bt_row = p.block_table + (int64_t)s * p.max_pages + z;
    npg_max = (p.max_ctx + z + kPage - 1) / kPage;
    pps_spec = SQ ? max((npg_max + p.S - 1) / p.S, kMinSplitPages) : (npg_max + p.S - 1) / p.S;
    pb_spec = min(split * pps_spec, npg_max);
    pe_spec = min(pb_spec + pps_spec, npg_max);
  };
  int id_spec = 0;
  if constexpr (SQ) {
    split_meta(0);
    if (tid < 128 && pb_spec + tid < pe_spec) id_spec = bt_row[pb_spec + tid];
  }

  // ---- prologue loads, all in flight together ----
  // (1) ctx; (2) the block-table entries of this split as placed for
  // ctx = max_ctx (the usual case; checked below, reloaded otherwise);
  // (3) the group's Q rows as raw 16-byte units; (4) the parent array.
  // Uniform metadata is read through the scalar cache (it is never written
  // while the kernel runs), so no vector wait sits in front of the loads below.
  // Scalar loads return out of order, so a use of any of them waits for all:
  // in uniform calls ctx and the page ids are read after the Q copies are
  // issued, which then need not wait for those memory round trips.  (Ragged
  // calls read ctx first: a workgroup past its sequence's splits leaves
  // before copying anything.)
  int ctx = 0;
  if constexpr (SQ) ctx = *reinterpret_cast<const __attribute__((address_space(4))) int*>((uintptr_t)(p.ctx_lens + s));

  const bool qf32 = p.q_dtype == kF32;
  h16* q_lds = reinterpret_cast<h16*>(smem + L::QST_OFF);
  // 16-byte unit u of staged row rr sits at unit u ^ (rr & QSW): the fragment
  // reads below take one unit from each of 16 consecutive rows, which would
  // otherwise all fall in the same LDS banks (rows are 2 D bytes apart)
  constexpr int QSW = (D / 8 >= 16) ? 15 : 7;
  auto q_unit = [&](int rr, int u) __attribute__((always_inline)) { return q_lds + rr * D + 8 * (u ^ (rr & QSW)); };

  // 16-bit Q: the waves copy the group's Q rows into the staging area with
  // LDS-DMA (slot s of the swizzled layout = its own 16-byte source unit),
  // so the output waves hold no vector load of their own and can send the
  // first K tiles right away; the page ids of those tiles (split page
  // 4j + q) come through the scalar cache.  fp32 Q is loaded below by all
  // threads.
  int kid[L::RK - 1];
  auto load_kid = [&](int z) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < L::RK - 1; ++j) {
      const int off = pb_spec + 4 * j + (wave - kRoleWaves);
      kid[j] = 0;
      if (!is_score && off < pe_spec)
        kid[j] = *reinterpret_cast<const __attribute__((address_space(4))) int*>((uintptr_t)(bt_row + off + z));
    }
  };
  if constexpr (SQ) load_kid(0);
  if constexpr (SQ) {
    // Splits of a sequence take at least kMinSplitPages pages each, so a
    // short sequence fills fewer than S of them.  A workgroup past those has
    // no keys: it leaves before copying anything (the merge reads only the
    // splits that hold keys; each row's entry in its list carries the count).
    // ctx is already waited for here, ahead of the Q copies.
    const bool ctx_bad = ctx < B || ctx > p.max_ctx || ctx > p.max_pages * kPage;
    const int np = ctx_bad ? 0 : (ctx + kPage - 1) / kPage;
    const int pp = max((np + p.S - 1) / p.S, kMinSplitPages);
    if (__builtin_expect(split > 0 && split * pp >= np, 0)) {
      wait_vmcnt<0>();
      return;
    }
  }
  constexpr int QUPR = D / 8;                          // 16-byte units of a 16-bit Q row
  // All 8 waves copy Q when the rows split into whole instructions per wave
  // (half the copy instructions per wave: the copies are issued sooner)
  constexpr bool Q8W = (QROWS * QUPR / 8) % 64 == 0;
  constexpr int QSPW = QROWS * QUPR / (Q8W ? 8 : kRoleWaves);  // staging units per copying wave
  constexpr int QDMA = QSPW / 64;                      // LDS-DMA instructions per copying wave
  static_assert(QSPW % 64 == 0, "whole Q DMA instructions");
  if (!qf32 && (Q8W || !is_score)) {
    const int q4 = Q8W ? wave : wave - kRoleWaves;
    constexpr int RPI = 64 / QUPR;  // staged rows per instruction
    int rr = (q4 * QSPW + lane) / QUPR;
    const int phys = lane & (QUPR - 1);
    const int r_first = min(rowbase + rr, M - 1);
    int hl = r_first / B;
    int b = r_first - hl * B;
    const int dh = RPI / B, db = RPI - dh * B;
    const int64_t rowb = (int64_t)D * 2;
    const char* qb = reinterpret_cast<const char*>(p.q);
    const int64_t off0 = ((r0 + b) * p.H + kvh * p.G + hl) * rowb;  // a valid row for clamped slots
#pragma unroll
    for (int k = 0; k < QDMA; ++k) {
      const bool valid = rowbase + rr < M;  // rows past the group's last are copies of a valid one
      const int64_t off = valid ? ((r0 + b) * p.H + kvh * p.G + hl) * rowb : off0;
      dma_vaddr(qb + off + 16 * (phys ^ (rr & QSW)), lds0 + L::QST_OFF + (q4 * QSPW + 64 * k) * 16);
      rr += RPI;
      b += db;
      hl += dh;
      if (b >= B) {
        b -= B;
        ++hl;
      }
    }
  }

  if constexpr (!SQ) {
    // z is 0; taking it from an asm statement placed after the Q copies keeps
    // the compiler from moving these loads (of invariant memory) ahead of
    // them.  Its inputs, one field of each line of the argument block that
    // is not preloaded, bring those lines in one round trip.
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z) : "s"(p.k_pool), "s"(p.cu_rows), "s"(p.num_seqs), "s"(p.scale_log2));
    split_meta(z);
    ctx = *reinterpret_cast<const __attribute__((address_space(4))) int*>((uintptr_t)(p.ctx_lens + s + z));
    load_kid(0);
    if (tid < 128 && pb_spec + tid < pe_spec) id_spec = bt_row[pb_spec + tid];
  }
  const int upr = qf32 ? D / 4 : D / 8;  // 16-byte Q units per row (a power of two)
  constexpr int QU_MAX = (QROWS * (D / 4) + kBlockThreads - 1) / kBlockThreads;
  u32x4 qraw[QU_MAX];
  if (qf32) {
    // unit u of this thread is 16-byte column c of group row rr + u * step;
    // row r = hl * B + b is stepped without a division per unit
    const int step = kBlockThreads / upr;
    const int c = tid & (upr - 1);
    int rr = tid / upr;
    int hl = (rowbase + rr) / B;
    int b = rowbase + rr - hl * B;
    const int dh = step / B, db = step - dh * B;
#pragma unroll
    for (int u = 0; u < QU_MAX; ++u) {
      qraw[u] = u32x4{0u, 0u, 0u, 0u};
      if (rr < QROWS && rowbase + rr < M) {
        const int64_t qrow = ((r0 + b) * p.H + kvh * p.G + hl) * D;
        const char* src = reinterpret_cast<const char*>(p.q) + (qrow + (int64_t)c * (qf32 ? 4 : 8)) * (qf32 ? 4 : 2);
        qraw[u] = *reinterpret_cast<const u32x4*>(src);
      }
      rr += step;
      hl += dh;
      b += db;
      if (b >= B) {
        b -= B;
        ++hl;
      }
    }
  }
  int par = 0;
  if (p.parent && is_score && lane < B) par = p.parent[r0 + lane];
  // The ancestry bitmask covers 64 rows: a longer sequence (a ragged prefill
  // segment) is a positioned causal chain, and a supplied parent array must
  // say so (parent[i] == i - 1 for every row).
  const bool long_rows = B > 64;
  bool chain_bad = false;
  if (long_rows && p.parent && is_score)
    for (int i = tid; i < B; i += 64 * kRoleWaves) chain_bad |= p.parent[r0 + i] != i - 1;

  // ---- validate sequence metadata (device-resident) ----
  bool poison = false;
  if (ctx < B || ctx > p.max_ctx || ctx > p.max_pages * kPage) {
    poison = true;
    ctx = 0;
  }
  uint32_t flagbits = poison ? VA_FLAG_BAD_CTX : 0u;
  // (the score waves check the parent array; wave 0 publishes the result in
  // flag 3 for the output waves, which read it after the first barrier)
  bool parent_bad = false;
  if (p.parent) {
    const bool bad = is_score && lane < B && (par < -1 || par >= lane);
    parent_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (parent_bad) {
      poison = true;
      flagbits |= VA_FLAG_BAD_PARENT;
    }
  } else {
    par = lane - 1;
  }
  const int base = ctx - B;  // slot of drafted row 0


  // Last key any row of this group can see: row b sees no slot past base + b.
  const int rend = min(rowbase + QROWS, M);
  int bmax = B - 1;
  if (rend - rowbase < B) {
    const int b0 = rowbase % B, b1 = (rend - 1) % B;
    if (b1 >= b0) bmax = b1;
  }
  const int vis_pages = (base + bmax + 1 + kPage - 1) / kPage;

  // ---- this split's pages (cut at the group's last visible key) and tiles of 4 pages ----
  const int npages = (ctx + kPage - 1) / kPage;
  const int pps = SQ ? max((npages + p.S - 1) / p.S, kMinSplitPages) : (npages + p.S - 1) / p.S;
  const int p_begin = min(split * pps, npages);
  const int p_end = max(p_begin, min(min(p_begin + pps, npages), vis_pages));
  const int npg = p_end - p_begin;
  const int T = (npg + 3) >> 2;
  const int split_end = min(ctx, p_end * kPage);
  const int mask_from = min(base, split_end);  // first token that needs a per-key test

  int* ids_lds = reinterpret_cast<int*>(smem + L::IDS_OFF);
  uint64_t* anc_lds = reinterpret_cast<uint64_t*>(smem + L::ANC_OFF);
  float* ex_lds = reinterpret_cast<float*>(smem + L::EX_OFF);
  // [0], [1]: overflow flag of even / odd iterations (double-buffered so a
  // score wave that runs ahead cannot set the flag a slow reader is reading);
  // [2]: some wave saw an out-of-range page id.
  auto flag_ref = [&](int idx) __attribute__((always_inline)) -> volatile __attribute__((address_space(3))) int& {
    return *LDS_PTR(volatile int, lds0 + L::FLAG_OFF + 4 * idx);
  };
  // wave-uniform read of a flag after a barrier
  auto flag_set = [&](int idx) __attribute__((always_inline)) -> bool {
    return __builtin_amdgcn_readfirstlane(flag_ref(idx)) != 0;
  };

  // ---- DMA issue ----
  const char* kbase = reinterpret_cast<const char*>(p.k_pool) + (int64_t)kvh * G::KPAGE;
  const char* vbase = reinterpret_cast<const char*>(p.v_pool) + (int64_t)kvh * G::VPAGE;
  const char* ksbase = reinterpret_cast<const char*>(p.k_scale) + (int64_t)kvh * G::SPB;
  const char* vsbase = reinterpret_cast<const char*>(p.v_scale) + (int64_t)kvh * G::SPB;
  const int64_t kstride = (int64_t)p.KVH * G::KPAGE;  // bytes between pages
  const int64_t vstride = (int64_t)p.KVH * G::VPAGE;
  const int64_t sstride = (int64_t)p.KVH * G::SPB;
  bool bad_page = false;

  // Physical id of split page `off` (per lane).  Padding pages past the split
  // end read page 0 and are masked; an out-of-range id is flagged and replaced.
  auto page_id = [&](int off) __attribute__((always_inline)) -> int {
    if (off >= npg) return 0;
    int id = ids_lds[((off >> 6) & 1) * 64 + (off & 63)];
    if (id < 0 || id >= p.num_pages) {
      bad_page = true;
      id = 0;
    }
    return id;
  };

  // Score wave w: K page w of tile j (1 KB chunks; lane (g, m) of chunk c
  // carries token m, bytes [64c + 16g, 64c + 16g + 16)), plus its scales.
  auto issue_k_id = [&](int j, int id) __attribute__((always_inline)) {
    const uint32_t st = lds0 + L::KR_OFF + (j % RK) * G::K_STAGE;
    const char* src = kbase + (int64_t)id * kstride;
    const uint32_t voff = n16 * G::KROW + 16 * g4;
#pragma unroll
    for (int c = 0; c < G::KCH; ++c) dma_saddr(src + 64 * c, voff, st + role * G::KPAGE + 1024 * c);
    if constexpr (G::Q8) {
      if (lane < D / 16) dma_saddr(ksbase + (int64_t)id * sstride, 16 * lane, st + 4 * G::KPAGE + role * D);
    }
  };
  auto issue_k = [&](int j) __attribute__((always_inline)) {
    issue_k_id(j, __builtin_amdgcn_readfirstlane(page_id(4 * j + role)));
  };

  // Output wave q: dims [q*DO, q*DO + DO) of all 4 pages of tile j (lane
  // (g, m) of chunk (mt, hh) carries page g, dim q*DO + 16mt + m, bytes
  // [16hh, 16hh + 16) of its 16-token row), plus page q's V scales.
  auto issue_v = [&](int j) __attribute__((always_inline)) {
    const int id = page_id(4 * j + g4);
    const uint32_t st = lds0 + L::VR_OFF + (j % RV) * G::V_STAGE;
    const char* src = vbase + (int64_t)id * vstride + (int64_t)(role * G::DO + n16) * G::VROW;
#pragma unroll
    for (int mt = 0; mt < G::MTO; ++mt)
#pragma unroll
      for (int hh = 0; hh < G::VROW / 16; ++hh)
        dma_vaddr(src + 16 * mt * G::VROW + 16 * hh, st + (role * G::VCH + mt * (G::VROW / 16) + hh) * 1024);
    if constexpr (G::Q8) {
      const int idq = __builtin_amdgcn_readlane(id, 16 * role);
      if (lane < D / 16) dma_saddr(vsbase + (int64_t)idq * sstride, 16 * lane, st + 4 * G::VPAGE + role * D);
    }
  };

  // ---- prologue stores: page ids of the first 128 pages, ancestry, Q ----
  if (tid < 128) {
    const bool spec_ok = (p_begin == pb_spec) && (npg <= pe_spec - pb_spec);
    ids_lds[tid] = (tid < npg) ? (spec_ok ? id_spec : bt_row[p_begin + tid]) : 0;
  }
  if (wave == 0 && !p.parent) {
    // chain: the positional limit alone decides
    anc_lds[lane] = poison ? 0 : ~(uint64_t)0;
  } else if (wave == 0) {
    // anc(i) = {i} + anc(parent[i]) by pointer jumping: after k rounds, a
    // holds the ancestors within distance 2^k and pr the one at distance 2^k.
    int pr = (lane < B && par < lane) ? par : -1;
    uint64_t a = (lane < B) ? (uint64_t)1 << lane : 0;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int src = pr < 0 ? lane : pr;
      const uint64_t pa = __shfl(a, src);
      const int pp = __shfl(pr, src);
      if (pr >= 0) {
        a |= pa;
        pr = pp;
      }
    }
    // (a sequence past 64 rows is a chain: its rows are limited by position alone)
    if (lane < B) anc_lds[lane] = poison ? 0 : long_rows ? ~(uint64_t)0 : a;
  }
  if (tid == 0) {
    flag_ref(0) = 0;
    flag_ref(1) = 0;
    flag_ref(2) = 0;
    flag_ref(3) = parent_bad ? 1 : 0;
  }
  if (long_rows && p.parent) {
    const bool wbad = __builtin_amdgcn_ballot_w64(chain_bad) != 0;
    if (lane == 0) flag_ref(8 + wave) = wbad ? 1 : 0;
  }
  bool early_k = false;
  if (qf32) {
#pragma unroll
    for (int u = 0; u < QU_MAX; ++u) {
      const int idx = tid + u * kBlockThreads;
      const int rr = idx / upr, c = idx % upr;
      if (rr < QROWS) {
        const f32x4 x = __builtin_bit_cast(f32x4, qraw[u]);
        h16x4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (h16)x[e];
        *reinterpret_cast<h16x4*>(q_unit(rr, c >> 1) + 4 * (c & 1)) = h;
      }
    }
  } else if (!is_score) {
    // the first K tiles, when this split starts where it would for
    // ctx = max_ctx (otherwise after the barrier, from the LDS page ids)
    early_k = T > 0 && p_begin == pb_spec && npg <= pe_spec - pb_spec;
    if (early_k) {
#pragma unroll
      for (int j = 0; j < RK - 1; ++j) {
        if (j < T) {
          const int off = 4 * j + role;
          int id = kid[j];
          if (off >= npg) {
            id = 0;
          } else if (id < 0 || id >= p.num_pages) {
            bad_page = true;
            id = 0;
          }
          issue_k_id(j, id);
        }
      }
      // the Q rows have landed once only those K groups are in flight
      wait_vmcnt_n<NDMA>(min(T, RK - 1));
    } else {
      wait_vmcnt<0>();
    }
  } else if (Q8W) {
    wait_vmcnt<0>();  // this score wave's Q copies
  }
  __syncthreads();
  if (!qf32) {
    if (p.q_dtype == kBF16) {
      // bf16 -> fp16 in place, one staged 16-byte unit per thread and step
      for (int su = tid; su < QROWS * QUPR; su += kBlockThreads) {
        const u32x4 w = *LDS_PTR(u32x4, lds0 + L::QST_OFF + 16 * su);
        h16x8 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[2 * e] = (h16)__builtin_bit_cast(float, w[e] << 16);
          h[2 * e + 1] = (h16)__builtin_bit_cast(float, w[e] & 0xffff0000u);
        }
        *LDS_PTR(h16x8, lds0 + L::QST_OFF + 16 * su) = h;
      }
      __syncthreads();
    }
  }
  if (flag_set(3)) {  // the score waves found a bad parent array
    poison = true;
    flagbits |= VA_FLAG_BAD_PARENT;
  }
  if (long_rows && p.parent) {
    bool bad = false;
#pragma unroll
    for (int w = 0; w < kBlockThreads / 64; ++w) bad |= flag_set(8 + w);
    if (bad) {
      poison = true;
      flagbits |= VA_FLAG_BAD_PARENT;
    }
  }

  const float c2 = p.scale_log2;
  constexpr int fbuf = L::P_BUF;  // bytes of one P buffer

  if (is_score) {
    // ========================= score waves =========================
    // wave (rh, kh): rows [16 NS rh, 16 NS (rh + 1)) of the group, pages
    // 2kh and 2kh + 1 of every tile.
    const int rh = role & 1, kh = role >> 1;

    // Q fragments: k-step ks covers dims dim0(ks, g) + [0, 8) for lane group g.
    h16x8 qf[KSTEPS][NS];
    int brow[NS];  // drafted-row index of each of this lane's rows (ancestry mask)
#pragma unroll
    for (int nt = 0; nt < NS; ++nt) {
      const int rr = 16 * (NS * rh + nt) + n16;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        // k-step ks covers dims [32 ks, 32 ks + 32): one 8-bit scale block
        const int dim0 = 32 * ks + 8 * g4;
        qf[ks][nt] = *reinterpret_cast<const h16x8*>(q_unit(rr, dim0 >> 3));
      }
      const int r = rowbase + rr;
      brow[nt] = (r < M) ? r % B : 0;
    }
    __syncthreads();  // tile 0's K has landed (the output waves waited for it)

    float mref[NS], lacc[NS], lt[NS];
    f32x4 sacc[2][NS];
#pragma unroll
    for (int nt = 0; nt < NS; ++nt) {
      mref[nt] = -INFINITY;
      lacc[nt] = 0.f;
      lt[nt] = 0.f;
      sacc[0][nt] = sacc[1][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Scaled score of accumulator element (u, nt, i) of the current tile;
    // with MK, -inf where the key is not visible to the row.
    int tile_tok0 = 0;
    bool masked = false;
    auto zval = [&](int u, int nt, int i, auto mk) __attribute__((always_inline)) -> float {
      const float z = sacc[u][nt][i] * c2;
      if constexpr (!decltype(mk)::value) {
        return z;
      } else {
        // the prefix plus the row's ancestors (all earlier rows of a chain),
        // never a slot past the row's own
        const int j = tile_tok0 + 16 * (2 * kh + u) + 4 * g4 + i;
        const uint64_t anc = anc_lds[brow[nt] & 63];
        const uint32_t rel = (uint32_t)(j - base) & 63u;
        const uint32_t bit = (uint32_t)(anc >> rel) & 1u;
        const uint32_t vis = (uint32_t)(j < split_end) & (uint32_t)(j - base <= brow[nt]) & ((uint32_t)(j < base) | bit);
        return vis ? z : -INFINITY;
      }
    };

    // P = 2^(z - m_ref) -> fp16 into the tile's P buffer; leaves the lane's
    // row sums in lt and returns the largest of them (the overflow test).
    auto write_p_t = [&](int j, auto mk) __attribute__((always_inline)) -> float {
      float lmx = 0.f;
      const uint32_t pb = lds0 + L::P_OFF + (j & 1) * fbuf + (g4 >> 1) * NT * 1024 + 8 * (g4 & 1);
#pragma unroll
      for (int nt = 0; nt < NS; ++nt) {
        const float mre = fmaxf(mref[nt], kFiniteFloor);
        float ls = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float pv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float t;
            if constexpr (decltype(mk)::value) t = zval(u, nt, i, mk) - mre;
            else t = __builtin_fmaf(sacc[u][nt][i], c2, -mre);
            pv[i] = fast_exp2(t);
          }
          const h16x4 ph = {(h16)pv[0], (h16)pv[1], (h16)pv[2], (h16)pv[3]};
          *LDS_PTR(h16x4, pb + (NS * rh + nt) * 1024 + (n16 + 16 * (2 * kh + u)) * 16) = ph;
          // the row sum adds the fp16 weights P.V uses, so a row that one key
          // dominates returns that key's V unscaled by P's rounding
          const h16x2 one2 = {(h16)1.0f, (h16)1.0f};
          ls = __builtin_amdgcn_fdot2(h16x2{ph[0], ph[1]}, one2, ls, false);
          ls = __builtin_amdgcn_fdot2(h16x2{ph[2], ph[3]}, one2, ls, false);
        }
        lt[nt] = ls;
        lmx = fmaxf(lmx, ls);
      }
      return lmx;
    };
    auto write_p = [&](int j) __attribute__((always_inline)) -> float {
      return masked ? write_p_t(j, std::true_type{}) : write_p_t(j, std::false_type{});
    };
    // Row maxima of the tile's visible scaled scores over this wave's pages.
    auto row_max = [&](int nt) __attribute__((always_inline)) -> float {
      float rm = -INFINITY;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) rm = fmaxf(rm, zval(u, nt, e, std::true_type{}));
      return wave_max16(rm);
    };

    for (int i = 0; i <= T; ++i) {
      if (i < T) {
        const int j = i;
        tile_tok0 = (p_begin + 4 * j) * kPage;
        masked = tile_tok0 + 64 > mask_from;
        const uint32_t st = lds0 + L::KR_OFF + (j % RK) * G::K_STAGE;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int nt = 0; nt < NS; ++nt) sacc[u][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (G::Q8) {
          // K stays exact: the int8 codes become fp16 integers (exact), and
          // each k-step of 32 dims, one scale block, is its own MFMA from a
          // zero accumulator; its fp32 result is multiplied by the block
          // scale of each key and added to the score.  (Scaling the codes in
          // fp16 first would round every K element to 11 bits, an error that
          // grows with the score.)  Lane (g, m) of a k-step holds dims
          // 8g .. 8g + 7 of the block for key m: 8 bytes of the 16-byte DMA
          // slot (g', m) of chunk ks / 2 with g' = 2 (ks & 1) + g / 2.
          constexpr int SW = D / 64;  // scale dwords of one token (D/32 fp16)
          // this lane's output keys 4g .. 4g + 3 (MFMA rows) of each page: all
          // their block scales
          uint32_t ksc[2][4][SW];
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t sp = st + 4 * G::KPAGE + (2 * kh + u) * D + (4 * g4 + e) * (D / 16);
              if constexpr (SW == 4) {
                const u32x4 t = *LDS_PTR(u32x4, sp);
                ksc[u][e][0] = t[0]; ksc[u][e][1] = t[1]; ksc[u][e][2] = t[2]; ksc[u][e][3] = t[3];
              } else if constexpr (SW == 2) {
                const u32x2 t = *LDS_PTR(u32x2, sp);
                ksc[u][e][0] = t[0]; ksc[u][e][1] = t[1];
              } else {
                ksc[u][e][0] = *LDS_PTR(uint32_t, sp);
              }
            }
          // the whole tile's K bytes for this wave in one burst of LDS reads,
          // so one read latency is paid per tile rather than one per k-step
          u32x2 raw_k[2][KSTEPS];
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
              raw_k[u][ks] = *LDS_PTR(u32x2, st + (2 * kh + u) * G::KPAGE + 1024 * (ks >> 1) +
                                                 16 * (16 * (2 * (ks & 1) + (g4 >> 1)) + n16) + 8 * (g4 & 1));
          // keep the burst together (the scheduler would otherwise sink each
          // read next to its use and wait for it there)
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) asm volatile("" : "+v"(raw_k[u][ks]));
          const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
          // per k-step: both pages' fragments, the 2 NS block products, then
          // their scaled adds (the products are in flight while the next
          // k-step's fragments are converted)
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks) {
            h16x8 kf[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              h16x2 a, b, c, d;
              i8x4_to_h(raw_k[u][ks][0], a, b);
              i8x4_to_h(raw_k[u][ks][1], c, d);
              kf[u] = cat(a, b, c, d);
            }
            f32x4 r[2][NS];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int nt = 0; nt < NS; ++nt)
                r[u][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[u], qf[ks][nt], zero4, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int nt = 0; nt < NS; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const h16x2 sc = as_h2(ksc[u][e][ks >> 1]);
                  sacc[u][nt][e] = __builtin_fmaf((float)sc[ks & 1], r[u][nt][e], sacc[u][nt][e]);
                }
          }
        } else {
#pragma unroll
          for (int c = 0; c < G::KCH; ++c) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const h16x8 k0 = *LDS_PTR(h16x8, st + (2 * kh + u) * G::KPAGE + 1024 * c + 16 * lane);
#pragma unroll
              for (int nt = 0; nt < NS; ++nt)
                sacc[u][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qf[c][nt], sacc[u][nt], 0, 0, 0);
            }
          }
        }
        if (write_p(j) > kLazyRescale) flag_ref(i & 1) = 1;  // an unset reference gives +inf sums
      }
      lds_barrier();
      if (flag_set(i & 1)) {
        // ---- rare path: raise the references (score side) ----
#pragma unroll
        for (int nt = 0; nt < NS; ++nt) {
          const float rm = row_max(nt);
          if (g4 == 0) ex_lds[kh * QROWS + 16 * (NS * rh + nt) + n16] = rm;
        }
        lds_barrier();
        if (wave == 0 && lane == 0) flag_ref(i & 1) = 0;
#pragma unroll
        for (int nt = 0; nt < NS; ++nt) {
          const int row = 16 * (NS * rh + nt) + n16;
          const float nr = fmaxf(mref[nt], fmaxf(ex_lds[row], ex_lds[QROWS + row]));
          lacc[nt] *= fast_exp2(fmaxf(mref[nt], kFiniteFloor) - fmaxf(nr, kFiniteFloor));
          mref[nt] = nr;
        }
        write_p(i);
#pragma unroll
        for (int nt = 0; nt < NS; ++nt) lacc[nt] += lt[nt];
        lds_barrier();
      } else if (i < T) {
#pragma unroll
        for (int nt = 0; nt < NS; ++nt) lacc[nt] += lt[nt];
      }
    }
    wait_vmcnt<0>();
    if (__builtin_amdgcn_ballot_w64(bad_page) != 0 && lane == 0) flag_ref(2) = 1;

    // ---- epilogue (score side): publish the row sums over this wave's keys ----
#pragma unroll
    for (int nt = 0; nt < NS; ++nt) {
      const float l = wave_sum16(lacc[nt]);
      if (g4 == 0) ex_lds[kh * QROWS + 16 * (NS * rh + nt) + n16] = l;
    }
    __syncthreads();
  } else {
    // ========================= output waves =========================
    // Output wave q issues every DMA of the loop: page q of each tile's K
    // (and its scales) besides its quarter of V, so the score waves, which
    // bound the loop, issue none.  The K ring is free from the start.
    if (!early_k) {
#pragma unroll
      for (int j = 0; j < RK - 1; ++j)
        if (j < T) issue_k(j);
    }
    constexpr int EV0 = L::EV ? 1 : 0;  // V of tile 0 goes out here too
    if (EV0 && T > 0) issue_v(0);
    // tile 0's K must have landed before the score waves' first iteration
    if (T > 0) wait_vmcnt_n<NDMA>(min(T, RK - 1) - 1 + EV0);
    __syncthreads();  // matches the score waves' Q-fragment barrier

    // DMA groups (one tile's K page or V quarter, NDMA instructions each) in
    // issue order: K 0 .. RK-2 (and, with EV, V 0) before the loop; at
    // iteration t, K t+RK-1, then V EV0 .. RV-2 (t = 0) or V t+RV-2 (t > 0),
    // each while below T.  ck(t) / cv(t): K / V groups issued through
    // iteration t.
    auto ck = [&](int t) __attribute__((always_inline)) { return min(T, RK + t); };
    auto cv = [&](int t) __attribute__((always_inline)) { return t < 0 ? min(T, EV0) : min(T, RV - 1 + t); };
    // 1-based issue position of K j and of V j
    auto pos_k = [&](int j) __attribute__((always_inline)) { return j <= RK - 2 ? j + 1 : ck(j - RK) + cv(j - RK) + 1; };
    auto pos_v = [&](int j) __attribute__((always_inline)) {
      if (EV0 && j == 0) return ck(-1) + 1;
      if (j <= RV - 2) return ck(0) + cv(-1) + j + 1 - EV0;
      const int t = j - RV + 2;
      return ck(t) + cv(t - 1) + 1;
    };

    f32x4 oacc[G::MTO][NT];
#pragma unroll
    for (int mt = 0; mt < G::MTO; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) oacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mref[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) mref[nt] = -INFINITY;

    for (int i = 0; i <= T; ++i) {
      if (i + RK - 1 < T) issue_k(i + RK - 1);
      if (i == 0) {
        // the V ring's later stages held the Q staging until the barrier above
#pragma unroll
        for (int j = EV0; j < RV - 1; ++j)
          if (j < T) issue_v(j);
      } else if (i + RV - 2 < T) {
        issue_v(i + RV - 2);
      }
      if (wave == kRoleWaves && (i & 15) == 1 && i > 16) {
        // page ids of chunk (i/16 + 1) into the buffer chunk i/16 - 1 used
        const int chunk = (i >> 4) + 1;
        const int off = 64 * chunk + lane;
        if (off < npg) dma_saddr_b32(bt_row + p_begin + 64 * chunk, 4 * lane, lds0 + L::IDS_OFF + (chunk & 1) * 256);
      }
      if (i >= 1) {
        const int j = i - 1;
        const int tile_tok0 = (p_begin + 4 * j) * kPage;
        const bool vtail = tile_tok0 + 64 > split_end;  // only a split's last tile
        const uint32_t st = lds0 + L::VR_OFF + (j % RV) * G::V_STAGE;
        const uint32_t pb = lds0 + L::P_OFF + (j & 1) * fbuf;
        h16x8 pf[2][NT];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) pf[h][nt] = *LDS_PTR(h16x8, pb + (h * NT + nt) * 1024 + 16 * lane);
        const int tok_lane = tile_tok0 + 16 * g4;  // this lane's page starts here
        if constexpr (G::Q8) {
          constexpr int NB = (G::DO >= 32) ? G::DO / 32 : 1;  // scale blocks per output wave
          const int bb0 = (role * G::DO) / 32;
          if (vtail) {
            // Slots at or past split_end may hold anything (NaN included):
            // clear this wave's scales of them in the stage, so their V reads
            // as 0.  Lane (g, m) owns slot m of page g; the wave reads only
            // its own blocks, after these writes (LDS keeps one wave's order).
            if (tile_tok0 + lane >= split_end)
#pragma unroll
              for (int b = 0; b < NB; ++b)
                *LDS_PTR(uint16_t, st + 4 * G::VPAGE + g4 * D + (bb0 + b) * 32 + 2 * n16) = 0;
          }
          // scales of block bb, tokens 8h..8h+7 of page g: one 16-byte read
          h16x2 vs[NB][2][4];
#pragma unroll
          for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const u32x4 w = *LDS_PTR(u32x4, st + 4 * G::VPAGE + g4 * D + (bb0 + b) * 32 + 16 * h);
#pragma unroll
              for (int e = 0; e < 4; ++e) vs[b][h][e] = as_h2(w[e]);
            }
          }
#pragma unroll
          for (int mt = 0; mt < G::MTO; ++mt) {
            const int b = (G::DO >= 32) ? (16 * mt) / 32 : 0;
            const u32x4 raw = *LDS_PTR(u32x4, st + (role * G::VCH + mt) * 1024 + 16 * lane);
            const h16x8 v0 = deq8(raw[0], raw[1], vs[b][0][0], vs[b][0][1], vs[b][0][2], vs[b][0][3]);
            const h16x8 v1 = deq8(raw[2], raw[3], vs[b][1][0], vs[b][1][1], vs[b][1][2], vs[b][1][3]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              oacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v0, pf[0][nt], oacc[mt][nt], 0, 0, 0);
              oacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v1, pf[1][nt], oacc[mt][nt], 0, 0, 0);
            }
          }
        } else {
          u32x4 tm[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) tm[h] = vtail ? tail_mask(tok_lane + 8 * h, split_end) : u32x4{~0u, ~0u, ~0u, ~0u};
#pragma unroll
          for (int mt = 0; mt < G::MTO; ++mt)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              u32x4 raw = *LDS_PTR(u32x4, st + (role * G::VCH + 2 * mt + h) * 1024 + 16 * lane);
              raw &= tm[h];
              const h16x8 vf = __builtin_bit_cast(h16x8, raw);
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
                oacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[h][nt], oacc[mt][nt], 0, 0, 0);
            }
        }
      }
      // K of tile i + 1 and V of tile i must have landed before the barrier:
      // wait until only the groups issued after both are in flight
      if (i < T) {
        const int need = max(i + 1 < T ? pos_k(i + 1) : 0, pos_v(i));
        wait_vmcnt_n<NDMA>(ck(i) + cv(i) - need);
      }
      lds_barrier();
      if (flag_set(i & 1)) {
        // ---- rare path: raise the references (output side) ----
        lds_barrier();
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int row = 16 * nt + n16;
          const float nr = fmaxf(mref[nt], fmaxf(ex_lds[row], ex_lds[QROWS + row]));
          const float alpha = fast_exp2(fmaxf(mref[nt], kFiniteFloor) - fmaxf(nr, kFiniteFloor));
#pragma unroll
          for (int mt = 0; mt < G::MTO; ++mt) oacc[mt][nt] *= alpha;
          mref[nt] = nr;
        }
        lds_barrier();
      }
    }
    wait_vmcnt<0>();
    if (__builtin_amdgcn_ballot_w64(bad_page) != 0 && lane == 0) flag_ref(2) = 1;
    __syncthreads();  // the score waves' row sums are in ex_lds

    // ---- epilogue (output side): normalise or write partials ----
    const bool any_poison = poison || flag_set(2);
    const int dq = role;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = rowbase + 16 * nt + n16;
      if (r >= M) continue;
      const float Lrow = ex_lds[16 * nt + n16] + ex_lds[QROWS + 16 * nt + n16];
      const int hl = r / B, b = r % B;
      const int64_t Rg = (r0 + b) * p.H + kvh * p.G + hl;
      if (p.direct) {
        const float inv = any_poison ? __builtin_nanf("") : 1.0f / Lrow;
#pragma unroll
        for (int mt = 0; mt < G::MTO; ++mt) {
          const int dim = dq * G::DO + 16 * mt + 4 * g4;
          const f32x4 o = oacc[mt][nt] * inv;
          if (p.out_dtype == kF32) {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + Rg * D + dim) = o;
          } else if (p.out_dtype == kF16) {
            h16x4 h;
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = (h16)o[e];
            *reinterpret_cast<h16x4*>(reinterpret_cast<h16*>(p.out) + Rg * D + dim) = h;
          } else {
            u32x2 w;
#pragma unroll
            for (int e = 0; e < 2; ++e) w[e] = f32_to_bf16_bits(o[2 * e]) | (f32_to_bf16_bits(o[2 * e + 1]) << 16);
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + Rg * D + dim) = w;
          }
        }
        if (dq == 0 && g4 == 0 && p.lse)
          p.lse[Rg] = any_poison ? __builtin_nanf("") : kLn2 * (mref[nt] + __builtin_log2f(Lrow));
      } else {
        // System-scope stores (the cache bits, sc0 sc1, of a relaxed
        // system-scope atomic store), matched by the merge's system-scope
        // loads: the partials reach memory without waiting in an XCD's L2
        // for the end-of-kernel write-back, and no L2 line left from an
        // earlier use of the workspace can be read in their place.  One
        // split's block (nrows * D floats, below 2^31 bytes: checked at plan
        // time) is the descriptor's range; lanes address it by byte offset.
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            p.part_o + (int64_t)split * p.nrows * D, 0, p.nrows * D * (int)sizeof(float), kRawBufferFlags);
#pragma unroll
        for (int mt = 0; mt < G::MTO; ++mt) {
          const int dim = dq * G::DO + 16 * mt + 4 * g4;
          const f32x4 val = any_poison ? f32x4{__builtin_nanf(""), 0.f, 0.f, 0.f} : oacc[mt][nt];
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, val), rs, (Rg * D + dim) * 4, 0,
                                                 kSystemScopeBits);
        }
        if (dq == 0 && g4 == 0) {
          // the row's (m, l) as one 8-byte pair
          const float mv = any_poison ? 0.f : mref[nt], lv = any_poison ? __builtin_nanf("") : Lrow;
          const uint64_t ml = (uint64_t)__builtin_bit_cast(uint32_t, mv) | (uint64_t)__builtin_bit_cast(uint32_t, lv) << 32;
          __hip_atomic_store(p.part_ml + (int64_t)split * p.nrows + Rg, ml, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
      }
    }
    if (wave == kRoleWaves && lane == 0) {
      const uint32_t bits = flagbits | (flag_set(2) ? (uint32_t)VA_FLAG_BAD_PAGE : 0u);
      if (bits) atomicOr(p.flags, bits);
    }
  }
}

// The kernel.  A ragged entry the work-list pass marked thin (a sequence of
// at most 32 (row, head) pairs) runs the 32-row body, as a uniform call with
// so few rows would: a larger body would carry 64 or more copied rows through
// every MFMA and softmax.  Rows do not depend on the body that computes them
// (each row's scores, softmax and P.V are its own; the rare rescale is taken
// for the group's distinct rows, the same in either body), so the choice
// changes no value.
template <int D, int KVT, int NT, bool SQ>
//
// The leading arguments repeat the fields of the parameter block that a
// workgroup of a uniform call needs to issue its Q copies; the build preloads
// them into SGPRs at wave launch (-amdgpu-kernarg-preload-count), so the
// copies wait for no read of the argument block.  (A ragged call's first
// reads are the work list and cu_rows, which need the block anyway.)
__global__ __launch_bounds__(kBlockThreads, 1) void verify_partial_kernel(const void* q, int32_t B, int32_t H, int32_t G,
                                                                           int32_t S, int32_t row_groups, int32_t q_dtype,
                                                                           const PartialParams p0) {
  PartialParams p = p0;
  if constexpr (!SQ) {
    p.q = q;
    p.B = B;
    p.H = H;
    p.G = G;
    p.S = S;
    p.row_groups = row_groups;
    p.q_dtype = q_dtype;
  }
  constexpr bool kThinBody = SQ && NT > 2;
  constexpr int kBytes = kThinBody && Lay<D, KVT, 2>::BYTES > Lay<D, KVT, NT>::BYTES ? Lay<D, KVT, 2>::BYTES
                                                                                     : Lay<D, KVT, NT>::BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[kBytes];
  if constexpr (kThinBody) {
    const auto* cnt = reinterpret_cast<const __attribute__((address_space(4))) int*>((uintptr_t)p.item_count);
    const auto* it =
        reinterpret_cast<const __attribute__((address_space(4))) int*>((uintptr_t)(p.items + blockIdx.x));
    if ((int)blockIdx.x < cnt[0] && (it[0] & kItemThin) != 0) {
      partial_body<D, KVT, 2, true>(p, smem);
      return;
    }
  }
  partial_body<D, KVT, NT, SQ>(p, smem);
}

}  // namespace

// ---- dispatch -----------------------------------------------------------------

Tiling choose_tiling(int B, int G, int D) {
  (void)D;
  const int M = B * G;
  const int tiles = (M + 15) / 16;
  Tiling t;
  t.row_groups = (tiles + 5) / 6;
  const int per = (tiles + t.row_groups - 1) / t.row_groups;
  t.nt = (per + 1) & ~1;  // even: the score waves take half the rows each
  return t;
}

bool partial_supported(int D, int kv_dtype, int nt) {
  if (kv_dtype != kQ8 && kv_dtype != kF16) return false;
  if (D != 64 && D != 128 && D != 256) return false;
  return nt == 2 || nt == 4 || nt == 6;
}

template <int D, int KVT, int NT>
static hipError_t launch_t(const PartialParams& p, hipStream_t stream) {
  dim3 grid((unsigned)(p.S * p.row_groups), (unsigned)p.KVH, (unsigned)p.num_seqs);
  if (p.items) {
    // ragged: one workgroup per entry the work list can hold
    hipLaunchKernelGGL((verify_partial_kernel<D, KVT, NT, true>), dim3((unsigned)p.item_cap),
                       dim3(kBlockThreads), 0, stream, p.q, p.B, p.H, p.G, p.S, p.row_groups, p.q_dtype, p);
  }
  else
    hipLaunchKernelGGL((verify_partial_kernel<D, KVT, NT, false>), grid, dim3(kBlockThreads), 0, stream, p.q, p.B, p.H,
                       p.G, p.S, p.row_groups, p.q_dtype, p);
  return hipGetLastError();
}

template <int D, int KVT>
static hipError_t launch_nt(const PartialParams& p, int nt, hipStream_t stream) {
  switch (nt) {
    case 2: return launch_t<D, KVT, 2>(p, stream);
    case 4: return launch_t<D, KVT, 4>(p, stream);
    case 6: return launch_t<D, KVT, 6>(p, stream);
    default: break;
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
