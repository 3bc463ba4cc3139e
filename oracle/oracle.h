/*
 * fp64 CPU oracle for speculative-decoding verify attention.
 *
 * TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library.  The product
 * path (the HIP library) never links, imports or falls back to it, and the
 * two share no code: this header and oracle.c are self-contained.
 *
 * What is computed: split-KV verify attention.  Sources: the page "perf(gfx1100):
 * speed up long-context DFlash verify 13.4% with FA2 split-KV and retain
 * HipGraph/Redline PM4" (Summary; Performance, batch-16 kernel screen: split
 * partials plus a merge, S1 identical to direct) and the page "perf(qwen35):
 * retain speculation during paged prefill" (Mechanism; State and commit
 * invariants: parent metadata covers only the tree suffix, other rows are
 * positioned causal reads; Correctness failure: 16-token paged blocks).
 * Where the pages are silent (row positions, the GQA head map, the 8-bit
 * block format) the plainest reading is taken:
 *
 *   For sequence s with ctx_s valid tokens (the B drafted rows included, row i
 *   sits at slot base + i with base = ctx_s - B), row i, query head h, KV head
 *   g = h / (H / KVH):
 *     anc(i)  = {i} plus anc(parent[i]) when parent[i] >= 0; parent == NULL
 *               means parent[i] = i - 1 (a chain, i.e. causal)
 *     Vis(i)  = {j : 0 <= j < base} plus {base + a : a in anc(i)}
 *     z_j     = scale * sum_d Q[s*B+i, h, d] * K_j[d]        (fp64, d ascending)
 *     M = max z_j,  L = sum e^(z_j - M),  O = sum e^(z_j - M) V_j / L,
 *     lse = M + ln L                                           (natural log)
 *
 *   Ragged rows (cu_rows != NULL; the page "perf(qwen35): retain speculation
 *   during paged prefill", Mechanism: one step lowers paged ragged prefill
 *   segments, ordinary direct rows and fixed-width tree rows together):
 *   sequence s owns the packed rows cu_rows[s] .. cu_rows[s+1] - 1 of q / out,
 *   n_s = cu_rows[s+1] - cu_rows[s] >= 0 of them, row i at slot ctx_s - n_s + i,
 *   and B above reads n_s, s*B + i reads cu_rows[s] + i.  parent is then
 *   packed the same way ([total_rows], sequence-local indices).  A prefill
 *   segment or a direct row is a chain; a tree is a parent array.
 *
 *   Split form (partials then log-sum-exp merge), any token partition
 *   0 = b_0 <= b_1 <= ... <= b_S = ctx_s:
 *     m_k = max z over Vis within [b_{k-1}, b_k)   (-inf if empty)
 *     l_k = sum e^(z - m_k),  O_k = sum e^(z - m_k) V_j  (unnormalised)
 *     merge over non-empty k: M = max m_k, w_k = e^(m_k - M), L = sum w_k l_k,
 *     O = sum w_k O_k / L, lse = M + ln L.
 *
 * Memory layouts (C-contiguous, the same documented contract the HIP library
 * accepts, re-implemented here from that description):
 *   q        [num_seqs*B, H, D]          f32 | f16 | bf16  ([total_rows, H, D] ragged)
 *   parent   [num_seqs, B] int32 or NULL ([total_rows] ragged)
 *   cu_rows  [num_seqs + 1] int32 or NULL (cu_rows[0] = 0, non-decreasing)
 *   k_pool   [num_pages, KVH, 16, D]     token-major        (f32 | f16 | int8)
 *   v_pool   [num_pages, KVH, D, 16]     dim-major          (f32 | f16 | int8)
 *   k_scale  [num_pages, KVH, 16, D/32]  f16 bits (8-bit pools only)
 *   v_scale  [num_pages, KVH, D/32, 16]  f16 bits (8-bit pools only)
 *   8-bit decode: x_d = double(scale[d/32]) * double(q_d)   (exact in fp64)
 *   block_table [num_seqs, max_pages] int32; token j of seq s lives in page
 *   block_table[s][j/16], slot j%16.
 *
 * Errors: every function returns ORC_OK or ORC_EINVAL (ctx_s < n_s or beyond
 * the block table, parent outside [-1, i), page id outside [0, num_pages),
 * D not a multiple of 32 for 8-bit pools, H not a multiple of KVH).
 */
#ifndef VERIFY_ORACLE_H
#define VERIFY_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_Q8 = 3 };
enum { ORC_OK = 0, ORC_EINVAL = -1 };

typedef struct {
  int32_t num_seqs;
  int32_t B;
  int32_t H;
  int32_t KVH;
  int32_t D;
  int32_t num_pages;
  int32_t max_pages;
  int32_t q_dtype;   /* ORC_F32 | ORC_F16 | ORC_BF16 */
  int32_t kv_dtype;  /* ORC_F32 | ORC_F16 | ORC_Q8 */
  double scale;      /* softmax scale (an fp32 value widened to fp64) */
} orc_shape;

/* Direct (definition) evaluation for every (row, head).
 * out [rows, H, D], lse [rows, H]; rows = num_seqs*B, or cu_rows[num_seqs]. */
int orc_attention(const orc_shape* p, const void* q, const void* k_pool, const void* v_pool,
                  const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* block_table,
                  const int32_t* ctx_lens, const int32_t* parent, const int32_t* cu_rows,
                  double* out, double* lse, int nthreads);

/* Same definition for a chosen set of (seq, row, head) triples only (row is
 * sequence-local).  items [n_items*3]; out [n_items, D]; lse [n_items]. */
int orc_attention_items(const orc_shape* p, const void* q, const void* k_pool, const void* v_pool,
                        const uint16_t* k_scale, const uint16_t* v_scale,
                        const int32_t* block_table, const int32_t* ctx_lens,
                        const int32_t* parent, const int32_t* cu_rows, int32_t n_items,
                        const int32_t* items, double* out, double* lse, int nthreads);

/* Split partials over a caller-chosen token partition.
 * bounds [num_seqs, nsplit+1] (b_0 = 0, b_nsplit = ctx_s, non-decreasing).
 * m, l [nsplit, rows, H]; o [nsplit, rows, H, D] (rows as for orc_attention). */
int orc_split_partials(const orc_shape* p, const void* q, const void* k_pool,
                       const void* v_pool, const uint16_t* k_scale, const uint16_t* v_scale,
                       const int32_t* block_table, const int32_t* ctx_lens,
                       const int32_t* parent, const int32_t* cu_rows, int32_t nsplit,
                       const int32_t* bounds, double* m, double* l, double* o, int nthreads);

/* Log-sum-exp merge of split partials (empty splits have l == 0 and are skipped).
 * m, l [nsplit, nrows]; o [nsplit, nrows, D]; out [nrows, D]; lse [nrows]. */
int orc_merge(int32_t nsplit, int64_t nrows, int32_t D, const double* m, const double* l,
              const double* o, double* out, double* lse);

/* The oracle's own decoders of 16-bit inputs, exposed so that they can be
 * checked bit pattern by bit pattern: IEEE binary16 (normal, subnormal, zero,
 * inf, NaN) and bfloat16 bit patterns -> double (n values). */
int orc_decode_f16(int64_t n, const uint16_t* h, double* out);
int orc_decode_bf16(int64_t n, const uint16_t* b, double* out);

/* fp32 -> IEEE binary16 bits, round to nearest even (n values). */
int orc_f32_to_f16(int64_t n, const float* x, uint16_t* out);

/* 8-bit block quantisation of nblocks blocks of 32 fp32 values:
 * d = fp16(max|x| / 127) (fp32 arithmetic, fp16 RNE), q = clamp(round half
 * away from zero (x / d), -127, 127) in fp32; all-zero block -> d = 0, q = 0;
 * NaN -> code 0.  q [nblocks*32] int8, d [nblocks] fp16 bits. */
int orc_quantize_blocks(int64_t nblocks, const float* x, int8_t* q, uint16_t* d);

/* KV append: write the B drafted rows' K and V (k_new, v_new
 * [num_seqs*B, KVH, D] in new_dtype: ORC_F32 | ORC_F16 | ORC_BF16) into slots
 * ctx_s - B + i of the pools (kv_dtype ORC_Q8: int8 codes + fp16 scales as
 * above; ORC_F16: fp16 RNE).  Returns ORC_EINVAL (nothing written) on bad
 * metadata. */
int orc_append_kv(const orc_shape* p, int32_t new_dtype, const void* k_new, const void* v_new,
                  void* k_pool, void* v_pool, uint16_t* k_scale, uint16_t* v_scale,
                  const int32_t* block_table, const int32_t* ctx_lens);

/* Accepted-path KV promotion: for each sequence copy the K / V (and scales)
 * of drafted rows accepted[s][0..n_accepted[s]) -- a root-first path,
 * parent[r_k] == r_{k-1} -- to the consecutive slots starting right after the
 * first node's parent slot (dst = ctx - B + parent[r_0] + 1); new_ctx[s] =
 * dst + n (optional).  All sequences are validated before any write;
 * ORC_EINVAL and nothing written on failure.  accepted [num_seqs, B],
 * n_accepted [num_seqs], parent [num_seqs, B] or NULL (chain). */
int orc_promote_kv(const orc_shape* p, const int32_t* accepted, const int32_t* n_accepted,
                   const int32_t* parent, void* k_pool, void* v_pool, uint16_t* k_scale,
                   uint16_t* v_scale, const int32_t* block_table, const int32_t* ctx_lens,
                   int32_t* new_ctx);

#ifdef __cplusplus
}
#endif
#endif
