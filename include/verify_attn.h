/*
 * verify_attn.h -- C ABI of the MI355X (gfx950) speculative-decoding verify
 * attention library (libverify_attn.so).
 *
 * WHAT IT COMPUTES
 *   B drafted query rows per sequence attend over that sequence's paged KV
 *   cache with a causal or draft-tree mask, grouped-query heads, and fp16 or
 *   8-bit KV, evaluated as a split-KV (flash-decoding) schedule: one partial
 *   kernel writes per-split (running max m, sum l, unnormalised O) and a
 *   log-sum-exp merge kernel combines them.  Sources:
 *     - page "perf(gfx1100): speed up long-context DFlash verify 13.4% with FA2
 *       split-KV and retain HipGraph/Redline PM4": Summary (split-KV S8 for
 *       B=16 verify, caller-owned partial workspace); Default and admission
 *       policy (dense H24/KV4/D256, B 4..32, fail-closed admission); Performance,
 *       batch-16 kernel screen (separate partial / merge / direct entries, S1 is
 *       the direct path);
 *     - page "perf(gfx11): optimize Qwen DFlash speculative verify": alpineQ's
 *       notes (one KV fetch shared by many query rows, q8_0 KV);
 *     - page "perf(qwen35): retain speculation during paged prefill": Mechanism
 *       and State and commit invariants (tree rows use ancestry metadata over
 *       the fixed suffix; other rows are positioned causal reads), Correctness
 *       failure found during qualification (16-token paged blocks; direct rows
 *       must not change when other rows join the launch).
 *
 *   For sequence s (ctx = ctx_lens[s] valid tokens, the B drafted rows
 *   included), drafted row i (0 <= i < B) sits at token slot base + i with
 *   base = ctx - B.  Its ancestor set anc(i) = {i} + anc(parent[i]) when
 *   parent[i] >= 0 (parent == NULL means parent[i] = i - 1, i.e. causal).  Row
 *   i sees tokens [0, base) plus {base + a : a in anc(i)}.  Query head h reads
 *   KV head h / (H / KVH).  out = softmax(scale * q k^T) v over the visible
 *   tokens; lse = natural log of the softmax denominator (with the max folded
 *   back in).
 *
 * MEMORY LAYOUTS (all C-contiguous, device memory unless marked host)
 *   q           [num_seqs*B, H, D]            q_dtype (F32 | F16 | BF16)
 *   k_pool      [num_pages, KVH, 16, D]       token-major: one D-vector per slot
 *   v_pool      [num_pages, KVH, D, 16]       dim-major: the 16 slots of a page
 *                                             are contiguous for each dimension
 *   k_scale     [num_pages, KVH, 16, D/32]    f16, Q8_0 only (else NULL)
 *   v_scale     [num_pages, KVH, D/32, 16]    f16, Q8_0 only (else NULL)
 *   block_table [num_seqs, max_pages_per_seq] int32 physical page ids
 *   ctx_lens    [num_seqs]                    int32
 *   parent      [num_seqs, B]                 int32, or NULL for causal
 *   out         [num_seqs*B, H, D]            out_dtype (F16 | BF16 | F32)
 *   lse         [num_seqs*B, H]               f32, optional (NULL = not written)
 *   Q8_0: each KV element is int8 q with value scale * q, one f16 scale per
 *   32 consecutive head_dim indices of one (token, KV head).  Token j of
 *   sequence s lives in page block_table[s][j / 16], slot j % 16.  K enters
 *   the score product exactly (codes as fp16 integers, the block scale
 *   applied to the fp32 product of each 32-dim block).  V is formed as
 *   scale * q in fp16 for the P.V product, so every V value must lie within
 *   fp16's range, |scale * q| <= 65504: a V block scale of 516 or more (or of
 *   512 or more with a code of -128) overflows there and makes the rows that
 *   see it NaN.  The library's own quantiser (verify_attn_append_kv) gives
 *   such scales only for values beyond fp16's range (max|x| > 65,500).
 *   The V page is stored dim-major because the P.V contraction reduces over
 *   tokens: that way a matrix-core operand (8 consecutive tokens of one
 *   dimension) is one contiguous load.  This departs from a token-major V
 *   cache (V laid out like K): a caller holding one transposes each 16-slot
 *   V page and its scales once when writing it; verify_attn_append_kv writes
 *   drafted rows in this layout.
 *
 * OWNERSHIP AND STREAMS
 *   The caller owns every device buffer and the stream.  The library never
 *   allocates device memory per call (its one device allocation is the
 *   64 MiB file-scope array behind verify_attn_run_noalloc, created with the
 *   code object on each device), never synchronises inside verify_attn_run, and
 *   enqueues its kernels asynchronously on `stream` (a hipStream_t; NULL is the
 *   null stream).  A plan is immutable host memory owned by the library until
 *   verify_attn_plan_destroy; it may be shared across threads and streams.
 *   Concurrent runs need distinct workspaces.
 *
 * WORKSPACE
 *   verify_attn_plan reports workspace_bytes.  The first 256 bytes hold a
 *   uint32 flag word (kernels OR error bits into it); then the fp32 split
 *   partials; a ragged plan's workspace ends with the call's work list
 *   (what verify_attn_run_ragged's first kernel writes for the other two).
 *   Zero the workspace once after allocating it; the flags stay set until
 *   verify_attn_read_flags clears them.
 *
 * ERRORS (fail closed: nothing is launched on any error; page "perf(gfx1100):
 * speed up long-context DFlash verify 13.4% with FA2 split-KV and retain
 * HipGraph/Redline PM4", Default and admission policy: unsupported shapes and
 * resources that are not ready fail closed instead of running; Maintainer-
 * review follow-up: the caller-owned partial workspace is part of admission,
 * here VA_EWORKSPACE)
 *   VA_EUNSUPPORTED  shape or dtype outside what the kernels implement
 *   VA_EINVAL        NULL or misaligned (16 B) required pointer, bad argument
 *   VA_EWORKSPACE    workspace smaller than the plan needs, or num_splits
 *                    above the plan's maximum
 *   VA_EHIP          a HIP call or kernel launch failed
 *   Device-resident metadata (ctx_lens, block_table, parent) is validated on
 *   the device: a bad value sets a bit in the flag word (VA_FLAG_*) and the
 *   affected sequence's outputs become NaN; no out-of-range memory is read.
 */
#ifndef VERIFY_ATTN_H
#define VERIFY_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status and dtype codes are plain 32-bit integers across the ABI (the enums
 * only name their values), so a caller may pass any value: an unknown dtype
 * is refused (VA_EUNSUPPORTED in a va_problem, VA_EINVAL as the new_dtype of
 * verify_attn_append_kv) and an unknown status reads "unknown status". */
typedef int32_t va_status;
enum { VA_OK = 0, VA_EINVAL = -1, VA_EUNSUPPORTED = -2, VA_EWORKSPACE = -3, VA_EHIP = -4 };

typedef int32_t va_dtype;
enum { VA_F32 = 0, VA_F16 = 1, VA_BF16 = 2, VA_Q8_0 = 3 };

/* Device flag bits (workspace header, read with verify_attn_read_flags). */
#define VA_FLAG_BAD_CTX 0x1u    /* ctx_lens[s] < B, > max_ctx, or beyond the block table */
#define VA_FLAG_BAD_PAGE 0x2u   /* block_table entry outside [0, num_pages) */
#define VA_FLAG_BAD_PARENT 0x4u /* parent[s][i] outside [-1, i) */
#define VA_FLAG_BAD_PATH 0x8u   /* promotion: accepted rows not a root-first parent chain, or n outside [0, B] */
#define VA_FLAG_BAD_ROWS 0x10u  /* ragged: cu_rows not non-decreasing from >= 0, a count above rows_per_seq, or past max_total_rows */

typedef struct {
  int32_t num_seqs;          /* >= 1 */
  int32_t rows_per_seq;      /* B, 1..64 */
  int32_t num_q_heads;       /* H */
  int32_t num_kv_heads;      /* KVH, H % KVH == 0 */
  int32_t head_dim;          /* D in {64, 128, 256} */
  int32_t page_size;         /* must be 16 */
  int32_t num_pages;         /* pool capacity in pages */
  int32_t max_pages_per_seq; /* block_table row stride */
  int32_t max_ctx;           /* upper bound of every ctx_lens[s]; sizes the split grid */
  va_dtype q_dtype;          /* VA_F32 | VA_F16 | VA_BF16 */
  va_dtype kv_dtype;         /* VA_F16 | VA_Q8_0 */
  va_dtype out_dtype;        /* VA_F16 | VA_BF16 | VA_F32 */
  float scale;               /* softmax scale; 0 => 1/sqrt(D) in fp32 */
  int32_t has_parent;        /* 0: causal rows (parent must be NULL); 1: parent array required */
  int32_t max_total_rows;    /* 0: B rows per sequence (verify_attn_run).  > 0: ragged rows
                                (verify_attn_run_ragged): rows_per_seq is then the largest
                                per-sequence count (1..4096) and this the packed row capacity,
                                at most num_seqs * rows_per_seq */
} va_problem;

typedef struct va_plan va_plan; /* opaque, host-only, immutable */

/* Read-only summary of a plan (host). */
typedef struct {
  int32_t num_splits;        /* S used when verify_attn_run gets num_splits = 0 */
  int32_t max_splits;        /* largest num_splits the workspace is sized for */
  int32_t row_groups;        /* workgroups per (sequence, KV head, split) along the rows */
  int32_t rows_per_group;    /* query rows (drafted row x head of one KV group) per workgroup */
  int32_t num_cus;           /* compute units the heuristic assumed */
  int32_t pages_per_split;   /* pages per split at max_ctx with num_splits */
  size_t workspace_bytes;    /* bytes the caller must provide */
} va_plan_info;

/*
 * Validate `problem`, choose the split count and size the workspace: the
 * admission step (page "perf(gfx1100): speed up long-context DFlash verify
 * 13.4% with FA2 split-KV and retain HipGraph/Redline PM4", Default and
 * admission policy: shape, dtype and context admission at the boundary;
 * Maintainer-review follow-up: the partial workspace is sized and checked as
 * part of admission).  The pages fix S = 8 for their part; here S follows the
 * device's CU count and max_ctx.
 *   problem          (host) copied into the plan
 *   num_splits       0 = choose from the device's CU count and max_ctx; else the
 *                    split count to size for (1..256)
 *   device_ordinal   HIP device whose CU count drives the heuristic
 *   out_plan         (host) receives the plan; NULL on error
 *   workspace_bytes  (host, may be NULL) receives the workspace size
 * Returns VA_OK, VA_EINVAL or VA_EUNSUPPORTED (or VA_EHIP if the device query fails).
 * VA_EUNSUPPORTED besides shapes and dtypes the kernels do not implement: one
 * split's partials (row capacity x num_q_heads x head_dim fp32 values) of
 * 2^31 bytes or more (their stores and loads take 32-bit offsets), and
 * ragged plans of more than 2,048 sequences or 256 KV heads.
 */
va_status verify_attn_plan(const va_problem* problem, int32_t num_splits, int32_t device_ordinal,
                           va_plan** out_plan, size_t* workspace_bytes);

/* Same as verify_attn_plan but with an explicit CU count instead of a device
 * query (num_cus >= 1).  Host-only; used to test the heuristic without a GPU. */
va_status verify_attn_plan_for_cus(const va_problem* problem, int32_t num_splits, int32_t num_cus,
                                   va_plan** out_plan, size_t* workspace_bytes);

/* Fill `info` (host) from a plan: the split count, row grouping and
 * workspace size admission chose.  VA_EINVAL if either pointer is NULL. */
va_status verify_attn_plan_get_info(const va_plan* plan, va_plan_info* info);

/* Free a plan (host memory only; NULL is a no-op).  The caller must not
 * destroy a plan while another thread is using it. */
void verify_attn_plan_destroy(va_plan* plan);

/*
 * Run the whole verify attention: the partial kernel, then (num_splits > 1)
 * the merge kernel; with one split the partial kernel writes out / lse
 * directly (the "direct" path).  Page "perf(gfx1100): speed up long-context
 * DFlash verify 13.4% with FA2 split-KV and retain HipGraph/Redline PM4":
 * Summary (split-KV verify of the drafted rows over the Q8 cache, partials
 * in a caller-owned workspace); Performance, batch-16 kernel screen (partial
 * and merge launches; one split is the direct path).
 *   num_splits  0 = the plan's choice; else 1..max_splits
 *   workspace   device buffer of at least the plan's workspace_bytes
 * Pointers as in MEMORY LAYOUTS; k_scale / v_scale must be NULL unless
 * kv_dtype is VA_Q8_0; parent must be NULL iff has_parent == 0.  Plans with
 * max_total_rows > 0 are refused (VA_EINVAL): they run through
 * verify_attn_run_ragged.  So are they by the partial / merge pair, the KV
 * append and the promotion below.
 */
va_status verify_attn_run(const va_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                          const void* k_scale, const void* v_scale, const int32_t* block_table,
                          const int32_t* ctx_lens, const int32_t* parent, int32_t num_splits,
                          void* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * verify_attn_run without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The split partials live in a device array the
 * library holds, one per GPU, for the life of the process (the first plan
 * made for a device, or the first call on it, looks its address up);
 * nothing is allocated, freed or cleared per call.
 *   flags   device uint32, caller-owned, 4-byte aligned: the VA_FLAG_* bits of
 *           the device-side metadata checks are ORed into it (zero it once;
 *           it is never cleared by the library)
 * Every other argument as for verify_attn_run.  Uniform plans only (ragged
 * plans: VA_EINVAL).  Limit: S * num_seqs * B * H * (head_dim + 2) * 4 bytes
 * of partials must fit the array's 64 MiB (16 sequences of the B = 16,
 * H = 24, D = 256 shape at S = 64, for instance), else VA_EWORKSPACE and
 * nothing is launched.  All calls on one GPU share the array: two calls that
 * overlap in time on one GPU (different streams without ordering between
 * them) race on it and may corrupt each other's outputs.
 */
va_status verify_attn_run_noalloc(const va_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                                  const void* k_scale, const void* v_scale, const int32_t* block_table,
                                  const int32_t* ctx_lens, const int32_t* parent, int32_t num_splits, void* out,
                                  float* lse, uint32_t* flags, void* stream);

/*
 * Ragged rows: one call that mixes paged prefill segments, ordinary direct
 * rows and draft trees (page "perf(qwen35): retain speculation during paged
 * prefill", Mechanism: a step lowers [prefill segments][direct rows][tree
 * rows] together, prefill and direct rows being positioned causal reads and
 * parent metadata covering only the tree; Correctness failure found during
 * qualification: the rows of one sequence must not change when other rows
 * join the call).  Needs a plan with max_total_rows > 0.
 *   cu_rows  [num_seqs + 1] int32, device: sequence s owns the packed rows
 *            cu_rows[s] .. cu_rows[s+1] - 1 of q / out / lse (cu_rows[0] = 0,
 *            non-decreasing, counts <= rows_per_seq, cu_rows[num_seqs] <=
 *            max_total_rows; a count of 0 is allowed).  Its n_s rows are the
 *            last n_s tokens of its context: row i at slot ctx_s - n_s + i.
 *   q, out   [cu_rows[num_seqs], H, D] packed rows; lse [cu_rows[num_seqs], H]
 *   parent   NULL (every row causal) or [cu_rows[num_seqs]] int32 packed the
 *            same way with sequence-local values in [-1, i).  A sequence with
 *            more than 64 rows must be a chain (parent[i] == i - 1).
 * Every other argument as for verify_attn_run.  A sequence's outputs depend
 * only on its own rows, context and pages and on the plan and num_splits.
 * The call runs three kernels: a one-workgroup pass that lists the call's
 * work from cu_rows and ctx_lens (each sequence split by its own context,
 * longest work first, packed densely so the workgroups spread evenly over
 * the device), the partial kernel over that list, and the merge.  A plan
 * with num_splits = 0 sizes S for one sequence at max_ctx plus num_seqs - 1
 * sequences of up to 64 pages running as one wave of workgroups; batches of
 * B rows per sequence whose contexts differ widely (a long decode beside
 * short ones) therefore run faster here with cu_rows = [0, B, 2B, ...] than
 * through verify_attn_run, whose plan sizes S for every sequence at max_ctx
 * (and suits batches of similar contexts better).
 * Limits: num_seqs <= 2048 and num_kv_heads <= 256 (VA_EUNSUPPORTED).
 * A bad cu_rows entry sets VA_FLAG_BAD_ROWS; that sequence writes nothing
 * (outputs of rows it would own are unspecified).  Sequences are taken in
 * order while their rows fit max_total_rows and their work fits the grid;
 * where bad entries make sequences' rows overlap, the sequences past that
 * point are left unwritten (their rows unspecified).  The grid is fixed by
 * the plan, so the call can be captured in a graph with live cu_rows.
 */
va_status verify_attn_run_ragged(const va_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                                 const void* k_scale, const void* v_scale, const int32_t* block_table,
                                 const int32_t* ctx_lens, const int32_t* cu_rows, const int32_t* parent,
                                 int32_t num_splits, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * The two launches of verify_attn_run, callable separately (same arguments
 * and checks).  verify_attn_run_partial enqueues only the partial kernel
 * (with num_splits == 1 it writes out / lse, otherwise the workspace
 * partials); verify_attn_run_merge enqueues only the merge kernel, reading
 * the partials a preceding verify_attn_run_partial with the same num_splits
 * wrote into `workspace` (VA_EINVAL when num_splits == 1).
 */
va_status verify_attn_run_partial(const va_plan* plan, const void* q, const void* k_pool,
                                  const void* v_pool, const void* k_scale, const void* v_scale,
                                  const int32_t* block_table, const int32_t* ctx_lens,
                                  const int32_t* parent, int32_t num_splits, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream);
va_status verify_attn_run_merge(const va_plan* plan, int32_t num_splits, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * KV append: the step before verify_attn_run.  Writes the B drafted rows' K
 * and V vectors of every sequence into their token slots ctx_lens[s] - B + i
 * of the pools, converting them to the pool format (the drafted rows' KV
 * writes precede the verify read: page "perf(qwen35): retain speculation
 * during paged prefill", State and commit invariants).
 *   k_new, v_new  [num_seqs*B, KVH, D] in new_dtype (VA_F32 | VA_F16 | VA_BF16),
 *                 16-byte aligned, device memory, read only
 *   k_pool ... v_scale, block_table, ctx_lens   as for verify_attn_run; the
 *                 pools (and scales) are written at the drafted slots only
 *   workspace     device buffer of at least 256 bytes (its flag word is used)
 * VA_F16 pools receive the values rounded to nearest even.  VA_Q8_0 pools
 * receive, per (token, KV head) and 32 consecutive head_dim entries, the fp16
 * scale d = max|x| / 127 (fp32 arithmetic, rounded to nearest even) and the
 * codes clamp(round half away from zero (x / d), -127, 127) computed in fp32
 * with the stored d; an all-zero block stores d = 0 and zero codes, a NaN
 * entry stores code 0.  A bad ctx_lens[s] or page id sets VA_FLAG_BAD_CTX /
 * VA_FLAG_BAD_PAGE and that sequence's (or row's) writes are skipped; nothing
 * outside the drafted slots is written.  Sequences must not share the pages
 * that hold their drafted slots.
 */
va_status verify_attn_append_kv(const va_plan* plan, const void* k_new, const void* v_new, va_dtype new_dtype,
                                void* k_pool, void* v_pool, void* k_scale, void* v_scale,
                                const int32_t* block_table, const int32_t* ctx_lens, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Accepted-path KV promotion: the step after verification in tree mode.  For
 * each sequence s the caller names the accepted path
 *   accepted[s][0 .. n_accepted[s])   drafted-row indices, root first, each
 *                                     the child of the previous one
 *                                     (parent[s][r_k] == r_{k-1})
 * The K / V vectors (and 8-bit scales) of those rows move, in path order, to
 * the consecutive slots right after the first row's parent:
 *   dst = ctx_lens[s] - B + parent[s][r_0] + 1   (ctx_lens[s] - B when -1)
 * and new_ctx[s] = dst + n_accepted[s], the length of the durable prefix now
 * holding the accepted tokens (n_accepted[s] == 0 gives ctx_lens[s] - B).
 * Only the accepted rows move (page "perf(qwen35): retain speculation during
 * paged prefill", State and commit invariants: promotion moves the accepted
 * prefix and preflights all state before mutating).  Every sequence is
 * checked on the device before any pool byte changes: a bad path, ctx, parent
 * or page id sets VA_FLAG_BAD_PATH / _CTX / _PARENT / _PAGE, nothing is
 * written to any pool, and new_ctx[s] = ctx_lens[s] for every s.
 *   accepted, n_accepted     [num_seqs, B] / [num_seqs] int32, device
 *   parent                   [num_seqs, B] or NULL (chain), device
 *   new_ctx                  [num_seqs] int32 output, device, optional (NULL);
 *                            not ctx_lens itself (VA_EINVAL)
 *   workspace                device, 256-byte aligned, at least
 *                            verify_attn_promote_workspace_bytes(plan) bytes:
 *                            flag word at byte 0, this call's check word at
 *                            byte 4, staging of the accepted rows after 256
 * Sources and destinations may overlap (the rows are staged first).
 * Sequences must not share the pages that hold their drafted slots (as for
 * verify_attn_append_kv).  A batch of at most 256 (sequence, path slot)
 * pairs is one launch (a workgroup per sequence and KV head, each repeating
 * the batch's checks and staging its rows in LDS); a larger one is three
 * launches that stage the rows in the workspace.
 */
va_status verify_attn_promote_kv(const va_plan* plan, const int32_t* accepted, const int32_t* n_accepted,
                                 const int32_t* parent, void* k_pool, void* v_pool, void* k_scale, void* v_scale,
                                 const int32_t* block_table, const int32_t* ctx_lens, int32_t* new_ctx,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes verify_attn_promote_kv needs for this plan (0 if plan is NULL). */
size_t verify_attn_promote_workspace_bytes(const va_plan* plan);

/* Copy the workspace flag word to *flags (host) after synchronising `stream`,
 * then clear it on the device.  For tests and debugging; it blocks.  The
 * flag word is this library's device-side counterpart of fail-closed
 * admission (page "perf(gfx1100): speed up long-context DFlash verify 13.4%
 * with FA2 split-KV and retain HipGraph/Redline PM4", Default and admission
 * policy): metadata that only the device sees (ctx_lens, block_table,
 * parent) cannot be checked before launch, so a bad value is reported here
 * and its rows are NaN.  VA_EINVAL on a NULL argument, VA_EHIP if a copy
 * fails. */
va_status verify_attn_read_flags(const va_plan* plan, void* workspace, void* stream, uint32_t* flags);

/* Static description of a status code (any int32; unknown codes read
 * "unknown status").  The string is owned by the library. */
const char* verify_attn_status_string(va_status status);

#ifdef __cplusplus
}
#endif
#endif /* VERIFY_ATTN_H */
