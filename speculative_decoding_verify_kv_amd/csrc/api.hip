// Host entry points of libverify_attn.so (the C ABI in include/verify_attn.h).
//
// Admission is fail-closed, as the page "perf(gfx1100): speed up long-context
// DFlash verify 13.4% with FA2 split-KV and retain HipGraph/Redline PM4"
// describes for its split verifier (Default and admission policy; Maintainer
// review follow-up: the caller-owned partial workspace is checked, an
// undersized one is refused): every check here returns an error before anything
// is enqueued, and there is no fallback to another algorithm.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "va_internal.h"

// Device memory of verify_attn_run_noalloc: the split partials of a call live
// here instead of in a caller workspace.  Each GPU the library runs on holds
// its own copy for the life of the process; host code reaches it only through
// the per-device address hipGetSymbolAddress returns (scratch_on_device).
static __device__ __align__(256) char scratch[va::kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of `scratch` on the current device, looked up once per device.
va_status scratch_on_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VA_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return VA_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return VA_OK;
}

// The same at plan time, with `device` made current for the lookup.
va_status scratch_setup(int device) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return VA_EHIP;
  if (cur != device && hipSetDevice(device) != hipSuccess) return VA_EHIP;
  void* ptr = nullptr;
  const va_status st = scratch_on_device(&ptr);
  if (cur != device && hipSetDevice(cur) != hipSuccess) return VA_EHIP;
  return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool ragged(const va_problem& p) { return p.max_total_rows > 0; }

// Packed query rows the plan holds: num_seqs * B, or max_total_rows (ragged).
int64_t rows_capacity(const va_problem& p) {
  return ragged(p) ? (int64_t)p.max_total_rows : (int64_t)p.num_seqs * p.rows_per_seq;
}

va_status check_problem(const va_problem* p) {
  if (!p) return VA_EINVAL;
  if (p->num_seqs < 1 || p->rows_per_seq < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 ||
      p->num_pages < 1 || p->max_pages_per_seq < 1 || p->max_ctx < 1 || p->max_total_rows < 0)
    return VA_EINVAL;
  if (p->num_q_heads % p->num_kv_heads) return VA_EINVAL;
  if (p->rows_per_seq > (ragged(*p) ? va::kMaxRowsRagged : va::kMaxRows)) return VA_EUNSUPPORTED;
  if (ragged(*p) && (int64_t)p->max_total_rows > (int64_t)p->num_seqs * p->rows_per_seq) return VA_EINVAL;
  if (p->page_size != va::kPage) return VA_EUNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256) return VA_EUNSUPPORTED;
  if (p->q_dtype != VA_F32 && p->q_dtype != VA_F16 && p->q_dtype != VA_BF16) return VA_EUNSUPPORTED;
  if (p->kv_dtype != VA_F16 && p->kv_dtype != VA_Q8_0) return VA_EUNSUPPORTED;
  if (p->out_dtype != VA_F32 && p->out_dtype != VA_F16 && p->out_dtype != VA_BF16) return VA_EUNSUPPORTED;
  if (p->has_parent != 0 && p->has_parent != 1) return VA_EINVAL;
  if (!(p->scale >= 0.f) || isinf(p->scale)) return VA_EINVAL;  // negative or NaN
  if (p->max_ctx < p->rows_per_seq) return VA_EINVAL;
  if ((int64_t)p->max_ctx > (int64_t)p->max_pages_per_seq * va::kPage) return VA_EINVAL;
  if (rows_capacity(*p) * p->num_q_heads > INT32_MAX) return VA_EUNSUPPORTED;
  // one split's partials (rows x heads x head_dim floats) are addressed by
  // 32-bit byte offsets
  if (rows_capacity(*p) * p->num_q_heads * p->head_dim * (int64_t)sizeof(float) > INT32_MAX) return VA_EUNSUPPORTED;
  // ragged calls list their work per sequence (sequence, KV head and split
  // packed with the row group in 8-byte entries)
  if (ragged(*p) && (p->num_seqs > va::kMaxSchedSeqs || p->num_kv_heads > 256)) return VA_EUNSUPPORTED;
  return VA_OK;
}

// Split-count model.  Work units are (sequence, KV head, row group, split);
// the partial kernel runs one workgroup per CU, and a split's time is a fixed
// part plus one step per 64-token tile.  So: size the splits such that
// num_seqs sequences at max_ctx fill the CUs once (never a straggler second
// round), give every split whole tiles, at least two of them, and take the
// fewest splits with that many tiles, since each split also writes fp32
// partials that the merge reads back.  A ragged plan mixes prefill segments,
// short decoders and long ones in one call: it is sized for one long decode
// sequence (one row group) filling the CUs left after two minimum-size
// splits (kMinSplitPages) per KV head for each of the other num_seqs - 1
// sequences (at most half the CUs are kept back), so a long sequence and
// short ones of up to 64 pages each run as one wave of workgroups.  Each
// sequence's splits still follow from its own context, the plan and the
// call's split count only.
int32_t heuristic_splits(const va_problem& p, const va::Tiling& t, int cus) {
  const int64_t units = ragged(p) ? (int64_t)p.num_kv_heads
                                  : (int64_t)p.num_seqs * p.num_kv_heads * t.row_groups;
  int64_t room = cus;
  if (ragged(p))
    room -= std::min<int64_t>((int64_t)cus / 2,
                              (int64_t)(p.num_seqs - 1) * p.num_kv_heads * 2 /* two minimum splits each */);
  const int64_t s0 = std::max<int64_t>(1, room / units);
  const int64_t npages = ceil_div(p.max_ctx, va::kPage);
  const int64_t tiles = std::max<int64_t>(2, ceil_div(npages, 4 * s0));
  int64_t S = ceil_div(npages, 4 * tiles);
  if (S > va::kMaxSplits) S = va::kMaxSplits;
  if (S < 1) S = 1;
  return (int32_t)S;
}

// Ragged calls: entries of the work list a call with S splits can have,
// S * groups * KVH, where groups bounds sum_s ceil(rows_s * G / QROWS) over
// sequences whose rows sum to at most the packed capacity.
int64_t ragged_item_cap(const va_problem& p, const va::Tiling& t, int S) {
  const int64_t QR = 16 * t.nt;
  const int64_t all = (int64_t)p.num_seqs * t.row_groups;
  const int64_t bound =
      ((int64_t)p.max_total_rows * (p.num_q_heads / p.num_kv_heads) + (int64_t)p.num_seqs * (QR - 1)) / QR;
  const int64_t groups = std::max<int64_t>(1, std::min(bound, all));
  return (int64_t)S * groups * p.num_kv_heads;
}

// Workspace: the flag header; with S > 1 the fp32 partials (O, then the
// (m, l) pairs) of S splits for every (row, head); for a ragged plan then,
// 256-byte aligned, the work list: the int32 counts (16 bytes), the packed
// rows to merge (one int32 each, with the row's split count, padded to 16
// bytes) and the entries (8 bytes each).
size_t sched_offset(const va_problem& p, int S) {
  const size_t nrows = (size_t)rows_capacity(p) * p.num_q_heads;
  if (S <= 1) return va::kHeaderBytes;
  const size_t end = va::kHeaderBytes + (size_t)S * nrows * ((size_t)p.head_dim + 2) * sizeof(float);
  return (end + 255) & ~(size_t)255;
}

size_t merge_rows_bytes(const va_problem& p) { return ((size_t)rows_capacity(p) * sizeof(int32_t) + 15) & ~(size_t)15; }

size_t workspace_for(const va_problem& p, const va::Tiling& t, int S) {
  const size_t nrows = (size_t)rows_capacity(p) * p.num_q_heads;
  if (ragged(p))
    return sched_offset(p, S) + 16 + merge_rows_bytes(p) + (size_t)ragged_item_cap(p, t, S) * sizeof(int2);
  if (S <= 1) return va::kHeaderBytes;
  return va::kHeaderBytes + (size_t)S * nrows * ((size_t)p.head_dim + 2) * sizeof(float);
}

va_status make_plan(const va_problem* problem, int32_t num_splits, int32_t cus, va_plan** out_plan,
                    size_t* workspace_bytes) {
  if (out_plan) *out_plan = nullptr;
  if (!out_plan) return VA_EINVAL;
  va_status st = check_problem(problem);
  if (st != VA_OK) return st;
  if (num_splits < 0 || num_splits > va::kMaxSplits || cus < 1) return VA_EINVAL;
  const va_problem& p = *problem;
  const int G = p.num_q_heads / p.num_kv_heads;
  const va::Tiling t = va::choose_tiling(p.rows_per_seq, G, p.head_dim);
  if (!va::partial_supported(p.head_dim, p.kv_dtype, t.nt)) return VA_EUNSUPPORTED;
  va_plan* plan = new (std::nothrow) va_plan;
  if (!plan) return VA_EINVAL;
  plan->prob = p;
  plan->tiling = t;
  plan->num_cus = cus;
  plan->num_splits = num_splits ? num_splits : heuristic_splits(p, t, cus);
  plan->max_splits = plan->num_splits;
  if (ragged(p) && (t.row_groups >= 65536 || ragged_item_cap(p, t, plan->max_splits) > INT32_MAX)) {
    delete plan;
    return VA_EUNSUPPORTED;
  }
  plan->scale = p.scale > 0.f ? p.scale : 1.0f / sqrtf((float)p.head_dim);
  plan->workspace_bytes = workspace_for(p, t, plan->max_splits);
  *out_plan = plan;
  if (workspace_bytes) *workspace_bytes = plan->workspace_bytes;
  return VA_OK;
}

struct RunArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const void* k_scale;
  const void* v_scale;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const int32_t* parent;
  const int32_t* cu_rows;  // ragged plans only
};

va_status check_run(const va_plan* plan, const RunArgs& a, int32_t num_splits, void* out, float* lse,
                    void* workspace, size_t workspace_bytes, int32_t* S_out) {
  if (!plan) return VA_EINVAL;
  const va_problem& p = plan->prob;
  if (!a.q || !a.k_pool || !a.v_pool || !a.block_table || !a.ctx_lens || !out || !workspace) return VA_EINVAL;
  if (!aligned(a.q, 16) || !aligned(a.k_pool, 16) || !aligned(a.v_pool, 16) || !aligned(out, 16) ||
      !aligned(workspace, 256))
    return VA_EINVAL;
  if (!aligned(a.block_table, 4) || !aligned(a.ctx_lens, 4) || (lse && !aligned(lse, 4))) return VA_EINVAL;
  if (p.kv_dtype == VA_Q8_0) {
    if (!a.k_scale || !a.v_scale || !aligned(a.k_scale, 16) || !aligned(a.v_scale, 16)) return VA_EINVAL;
  } else if (a.k_scale || a.v_scale) {
    return VA_EINVAL;
  }
  if ((p.has_parent != 0) != (a.parent != nullptr)) return VA_EINVAL;
  if (a.parent && !aligned(a.parent, 4)) return VA_EINVAL;
  if (ragged(p) != (a.cu_rows != nullptr)) return VA_EINVAL;  // ragged plans run through verify_attn_run_ragged
  if (a.cu_rows && !aligned(a.cu_rows, 4)) return VA_EINVAL;
  const int32_t S = num_splits ? num_splits : plan->num_splits;
  if (S < 1) return VA_EINVAL;
  if (S > plan->max_splits) return VA_EWORKSPACE;
  if (workspace_bytes < plan->workspace_bytes) return VA_EWORKSPACE;
  *S_out = S;
  return VA_OK;
}

va::PartialParams partial_params(const va_plan* plan, const RunArgs& a, int32_t S, void* out, float* lse,
                                 void* workspace) {
  const va_problem& p = plan->prob;
  va::PartialParams pp;
  memset(&pp, 0, sizeof pp);
  pp.q = a.q;
  pp.k_pool = a.k_pool;
  pp.v_pool = a.v_pool;
  pp.k_scale = a.k_scale;
  pp.v_scale = a.v_scale;
  pp.block_table = a.block_table;
  pp.ctx_lens = a.ctx_lens;
  pp.parent = a.parent;
  pp.cu_rows = a.cu_rows;
  pp.out = out;
  pp.lse = lse;
  const int64_t nrows = rows_capacity(p) * p.num_q_heads;
  char* ws = static_cast<char*>(workspace);
  pp.flags = reinterpret_cast<uint32_t*>(ws);
  float* part = reinterpret_cast<float*>(ws + va::kHeaderBytes);
  pp.part_o = part;
  pp.part_ml = reinterpret_cast<uint64_t*>(part + (int64_t)plan->max_splits * nrows * p.head_dim);
  // ragged calls split each sequence by its own context (see kMinSplitPages)
  if (ragged(p)) {
    char* sched = ws + sched_offset(p, plan->max_splits);
    pp.item_count = reinterpret_cast<const int32_t*>(sched);
    pp.items = reinterpret_cast<const int2*>(sched + 16 + merge_rows_bytes(p));
    pp.item_cap = (int32_t)ragged_item_cap(p, plan->tiling, S);
  }
  pp.num_seqs = p.num_seqs;
  pp.B = p.rows_per_seq;
  pp.total_rows = (int32_t)rows_capacity(p);
  pp.H = p.num_q_heads;
  pp.KVH = p.num_kv_heads;
  pp.G = p.num_q_heads / p.num_kv_heads;
  pp.D = p.head_dim;
  pp.num_pages = p.num_pages;
  pp.max_pages = p.max_pages_per_seq;
  pp.max_ctx = p.max_ctx;
  pp.S = S;
  pp.row_groups = plan->tiling.row_groups;
  pp.rows_per_group = 16 * plan->tiling.nt;
  pp.q_dtype = p.q_dtype;
  pp.out_dtype = p.out_dtype;
  pp.direct = (S == 1) ? 1 : 0;
  pp.scale_log2 = plan->scale * 1.4426950408889634f;
  pp.nrows = nrows;
  return pp;
}

va::MergeParams merge_params(const va::PartialParams& pp, void* out, float* lse) {
  va::MergeParams mp;
  mp.part_o = pp.part_o;
  mp.part_ml = pp.part_ml;
  mp.out = out;
  mp.lse = lse;
  if (pp.items) {
    mp.merge_count = pp.item_count + 1;
    mp.merge_rows = pp.item_count + 4;
  } else {
    mp.merge_rows = nullptr;
    mp.merge_count = nullptr;
  }
  mp.heads = pp.H;
  mp.S = pp.S;
  mp.D = pp.D;
  mp.out_dtype = pp.out_dtype;
  mp.nrows = pp.nrows;
  return mp;
}

}  // namespace

extern "C" {

va_status verify_attn_plan(const va_problem* problem, int32_t num_splits, int32_t device_ordinal,
                           va_plan** out_plan, size_t* workspace_bytes) {
  if (out_plan) *out_plan = nullptr;
  va_status st = check_problem(problem);
  if (st != VA_OK) return st;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device_ordinal) != hipSuccess) return VA_EHIP;
  // set-up of verify_attn_run_noalloc's device memory on this device
  if (scratch_setup(device_ordinal) != VA_OK) return VA_EHIP;
  return make_plan(problem, num_splits, prop.multiProcessorCount, out_plan, workspace_bytes);
}

va_status verify_attn_plan_for_cus(const va_problem* problem, int32_t num_splits, int32_t num_cus,
                                   va_plan** out_plan, size_t* workspace_bytes) {
  return make_plan(problem, num_splits, num_cus, out_plan, workspace_bytes);
}

va_status verify_attn_plan_get_info(const va_plan* plan, va_plan_info* info) {
  if (!plan || !info) return VA_EINVAL;
  info->num_splits = plan->num_splits;
  info->max_splits = plan->max_splits;
  info->row_groups = plan->tiling.row_groups;
  info->rows_per_group = 16 * plan->tiling.nt;
  info->num_cus = plan->num_cus;
  const int64_t npages = ceil_div(plan->prob.max_ctx, va::kPage);
  info->pages_per_split = (int32_t)ceil_div(npages, plan->num_splits);
  info->workspace_bytes = plan->workspace_bytes;
  return VA_OK;
}

void verify_attn_plan_destroy(va_plan* plan) { delete plan; }

va_status verify_attn_run_partial(const va_plan* plan, const void* q, const void* k_pool,
                                  const void* v_pool, const void* k_scale, const void* v_scale,
                                  const int32_t* block_table, const int32_t* ctx_lens,
                                  const int32_t* parent, int32_t num_splits, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  const RunArgs a{q, k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, parent, nullptr};
  int32_t S = 0;
  va_status st = check_run(plan, a, num_splits, out, lse, workspace, workspace_bytes, &S);
  if (st != VA_OK) return st;
  const va::PartialParams pp = partial_params(plan, a, S, out, lse, workspace);
  if (va::launch_partial(pp, plan->prob.kv_dtype, plan->tiling.nt, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return VA_EHIP;
  return VA_OK;
}

va_status verify_attn_run_merge(const va_plan* plan, int32_t num_splits, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan || !out || !workspace) return VA_EINVAL;
  if (ragged(plan->prob)) return VA_EINVAL;  // the live row count comes with verify_attn_run_ragged
  if (!aligned(out, 16) || !aligned(workspace, 256) || (lse && !aligned(lse, 4))) return VA_EINVAL;
  const int32_t S = num_splits ? num_splits : plan->num_splits;
  if (S < 2) return VA_EINVAL;
  if (S > plan->max_splits || workspace_bytes < plan->workspace_bytes) return VA_EWORKSPACE;
  // Only the workspace layout and the output are needed.
  const RunArgs none{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  const va::PartialParams pp = partial_params(plan, none, S, out, lse, workspace);
  if (va::launch_merge(merge_params(pp, out, lse), static_cast<hipStream_t>(stream)) != hipSuccess)
    return VA_EHIP;
  return VA_OK;
}

va_status verify_attn_run(const va_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                          const void* k_scale, const void* v_scale, const int32_t* block_table,
                          const int32_t* ctx_lens, const int32_t* parent, int32_t num_splits,
                          void* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream) {
  const RunArgs a{q, k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, parent, nullptr};
  int32_t S = 0;
  va_status st = check_run(plan, a, num_splits, out, lse, workspace, workspace_bytes, &S);
  if (st != VA_OK) return st;
  const va::PartialParams pp = partial_params(plan, a, S, out, lse, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (va::launch_partial(pp, plan->prob.kv_dtype, plan->tiling.nt, s) != hipSuccess) return VA_EHIP;
  if (S > 1 && va::launch_merge(merge_params(pp, out, lse), s) != hipSuccess) return VA_EHIP;
  return VA_OK;
}

va_status verify_attn_run_noalloc(const va_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                                  const void* k_scale, const void* v_scale, const int32_t* block_table,
                                  const int32_t* ctx_lens, const int32_t* parent, int32_t num_splits, void* out,
                                  float* lse, uint32_t* flags, void* stream) {
  if (!plan || !flags || !aligned(flags, 4)) return VA_EINVAL;
  if (ragged(plan->prob)) return VA_EINVAL;  // uniform plans only
  const va_problem& p = plan->prob;
  const int32_t S = num_splits ? num_splits : plan->num_splits;
  if (S < 1 || S > va::kMaxSplits) return VA_EINVAL;
  // split partials: fp32 O, m and l of S splits for every (row, head)
  const size_t need = S > 1 ? (size_t)S * (size_t)rows_capacity(p) * p.num_q_heads * ((size_t)p.head_dim + 2) *
                                  sizeof(float)
                            : 0;
  if (need > va::kScratchBytes) return VA_EWORKSPACE;
  void* base = nullptr;
  if (scratch_on_device(&base) != VA_OK) return VA_EHIP;
  // check_run with a workspace stand-in: the scratch partials sized for S
  va_plan local = *plan;
  local.max_splits = S;
  local.workspace_bytes = 0;
  const RunArgs a{q, k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, parent, nullptr};
  int32_t S_run = 0;
  va_status st = check_run(&local, a, S, out, lse, base, 0, &S_run);
  if (st != VA_OK) return st;
  va::PartialParams pp = partial_params(&local, a, S, out, lse, base);
  // partials start at the array's base (the header of a workspace is not
  // needed: flag bits go to the caller's word)
  const int64_t nrows = pp.nrows;
  float* part = static_cast<float*>(base);
  pp.part_o = part;
  pp.part_ml = reinterpret_cast<uint64_t*>(part + (int64_t)S * nrows * p.head_dim);
  pp.flags = flags;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (va::launch_partial(pp, p.kv_dtype, plan->tiling.nt, s) != hipSuccess) return VA_EHIP;
  if (S > 1 && va::launch_merge(merge_params(pp, out, lse), s) != hipSuccess) return VA_EHIP;
  return VA_OK;
}

va_status verify_attn_run_ragged(const va_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                                 const void* k_scale, const void* v_scale, const int32_t* block_table,
                                 const int32_t* ctx_lens, const int32_t* cu_rows, const int32_t* parent,
                                 int32_t num_splits, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!plan || !cu_rows) return VA_EINVAL;
  const RunArgs a{q, k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, parent, cu_rows};
  int32_t S = 0;
  va_status st = check_run(plan, a, num_splits, out, lse, workspace, workspace_bytes, &S);
  if (st != VA_OK) return st;
  const va::PartialParams pp = partial_params(plan, a, S, out, lse, workspace);
  // the work list first: the partial kernel's entries and the merge's rows
  va::ScheduleParams sp;
  sp.cu_rows = cu_rows;
  sp.ctx_lens = ctx_lens;
  sp.count = const_cast<int32_t*>(pp.item_count);
  sp.items = const_cast<int2*>(pp.items);
  sp.merge_rows = const_cast<int32_t*>(pp.item_count) + 4;
  sp.flags = pp.flags;
  sp.num_seqs = pp.num_seqs;
  sp.B = pp.B;
  sp.total_rows = pp.total_rows;
  sp.G = pp.G;
  sp.qrows = pp.rows_per_group;
  sp.S = S;
  sp.KVH = pp.KVH;
  sp.max_ctx = pp.max_ctx;
  sp.max_pages = pp.max_pages;
  sp.cap = pp.item_cap;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (va::launch_schedule(sp, s) != hipSuccess) return VA_EHIP;
  if (va::launch_partial(pp, plan->prob.kv_dtype, plan->tiling.nt, s) != hipSuccess) return VA_EHIP;
  if (S > 1 && va::launch_merge(merge_params(pp, out, lse), s) != hipSuccess) return VA_EHIP;
  return VA_OK;
}

va_status verify_attn_append_kv(const va_plan* plan, const void* k_new, const void* v_new, va_dtype new_dtype,
                                void* k_pool, void* v_pool, void* k_scale, void* v_scale,
                                const int32_t* block_table, const int32_t* ctx_lens, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!plan || ragged(plan->prob)) return VA_EINVAL;  // B drafted rows per sequence only
  const va_problem& p = plan->prob;
  if (new_dtype != VA_F32 && new_dtype != VA_F16 && new_dtype != VA_BF16) return VA_EINVAL;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_table || !ctx_lens || !workspace) return VA_EINVAL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(workspace, 256) || !aligned(block_table, 4) || !aligned(ctx_lens, 4))
    return VA_EINVAL;
  if (p.kv_dtype == VA_Q8_0) {
    if (!k_scale || !v_scale || !aligned(k_scale, 16) || !aligned(v_scale, 16)) return VA_EINVAL;
  } else if (k_scale || v_scale) {
    return VA_EINVAL;
  }
  if (workspace_bytes < va::kHeaderBytes) return VA_EWORKSPACE;
  va::AppendParams ap;
  memset(&ap, 0, sizeof ap);
  ap.k_new = k_new;
  ap.v_new = v_new;
  ap.k_pool = k_pool;
  ap.v_pool = v_pool;
  ap.k_scale = k_scale;
  ap.v_scale = v_scale;
  ap.block_table = block_table;
  ap.ctx_lens = ctx_lens;
  ap.flags = static_cast<uint32_t*>(workspace);
  ap.num_seqs = p.num_seqs;
  ap.B = p.rows_per_seq;
  ap.KVH = p.num_kv_heads;
  ap.D = p.head_dim;
  ap.num_pages = p.num_pages;
  ap.max_pages = p.max_pages_per_seq;
  ap.max_ctx = p.max_ctx;
  ap.new_dtype = new_dtype;
  ap.kv_dtype = p.kv_dtype;
  if (va::launch_append(ap, static_cast<hipStream_t>(stream)) != hipSuccess) return VA_EHIP;
  return VA_OK;
}

size_t verify_attn_promote_workspace_bytes(const va_plan* plan) {
  if (!plan) return 0;
  const va_problem& p = plan->prob;
  return va::kHeaderBytes + (size_t)p.num_seqs * p.rows_per_seq * p.num_kv_heads * 2 *
                                va::promote_row_bytes(p.head_dim, p.kv_dtype);
}

va_status verify_attn_promote_kv(const va_plan* plan, const int32_t* accepted, const int32_t* n_accepted,
                                 const int32_t* parent, void* k_pool, void* v_pool, void* k_scale, void* v_scale,
                                 const int32_t* block_table, const int32_t* ctx_lens, int32_t* new_ctx,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan || ragged(plan->prob)) return VA_EINVAL;  // B drafted rows per sequence only
  const va_problem& p = plan->prob;
  if (!accepted || !n_accepted || !k_pool || !v_pool || !block_table || !ctx_lens || !workspace) return VA_EINVAL;
  if (!aligned(accepted, 4) || !aligned(n_accepted, 4) || (parent && !aligned(parent, 4)) ||
      (new_ctx && !aligned(new_ctx, 4)) || !aligned(block_table, 4) || !aligned(ctx_lens, 4) ||
      !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(workspace, 256))
    return VA_EINVAL;
  if (p.kv_dtype == VA_Q8_0) {
    if (!k_scale || !v_scale || !aligned(k_scale, 16) || !aligned(v_scale, 16)) return VA_EINVAL;
  } else if (k_scale || v_scale) {
    return VA_EINVAL;
  }
  if ((p.has_parent != 0) != (parent != nullptr)) return VA_EINVAL;
  if (new_ctx && new_ctx == ctx_lens) return VA_EINVAL;  // rows still read ctx_lens while new_ctx is written
  if (workspace_bytes < verify_attn_promote_workspace_bytes(plan)) return VA_EWORKSPACE;
  va::PromoteParams pp;
  memset(&pp, 0, sizeof pp);
  pp.accepted = accepted;
  pp.n_accepted = n_accepted;
  pp.parent = parent;
  pp.k_pool = k_pool;
  pp.v_pool = v_pool;
  pp.k_scale = k_scale;
  pp.v_scale = v_scale;
  pp.block_table = block_table;
  pp.ctx_lens = ctx_lens;
  pp.new_ctx = new_ctx;
  char* ws = static_cast<char*>(workspace);
  pp.flags = reinterpret_cast<uint32_t*>(ws);
  pp.status = reinterpret_cast<uint32_t*>(ws + 4);
  pp.staging = ws + va::kHeaderBytes;
  pp.row_bytes = (int64_t)va::promote_row_bytes(p.head_dim, p.kv_dtype);
  pp.num_seqs = p.num_seqs;
  pp.B = p.rows_per_seq;
  pp.KVH = p.num_kv_heads;
  pp.D = p.head_dim;
  pp.num_pages = p.num_pages;
  pp.max_pages = p.max_pages_per_seq;
  pp.max_ctx = p.max_ctx;
  pp.esz = p.kv_dtype == VA_Q8_0 ? 1 : 2;
  pp.kv_is_q8 = p.kv_dtype == VA_Q8_0 ? 1 : 0;
  if (va::launch_promote(pp, static_cast<hipStream_t>(stream)) != hipSuccess) return VA_EHIP;
  return VA_OK;
}

va_status verify_attn_read_flags(const va_plan* plan, void* workspace, void* stream, uint32_t* flags) {
  if (!plan || !workspace || !flags) return VA_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(flags, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess) return VA_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return VA_EHIP;
  if (hipMemsetAsync(workspace, 0, sizeof(uint32_t), s) != hipSuccess) return VA_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return VA_EHIP;
  return VA_OK;
}

const char* verify_attn_status_string(va_status status) {
  switch (status) {
    case VA_OK: return "ok";
    case VA_EINVAL: return "invalid argument";
    case VA_EUNSUPPORTED: return "unsupported shape or dtype";
    case VA_EWORKSPACE: return "workspace too small or too many splits";
    case VA_EHIP: return "HIP error";
  }
  return "unknown status";
}

}  // extern "C"
