/*
 * A plain-C caller of libverify_attn.so: the C ABI of include/verify_attn.h
 * used without Python.  It plans, sizes and allocates the workspace itself,
 * runs verify_attn_run (and, for a split plan, verify_attn_run_partial +
 * verify_attn_run_merge into a second output), reads the flag word and
 * checks the admission errors a caller can hit, with device memory from the
 * HIP runtime's C API.
 *
 *   verify_c_client <input file> <output file>
 *
 * Input (little-endian, written by tests/test_gpu_c_client.py): the 8 bytes
 * "VACLIENT", the va_problem struct as the library declares it, int32
 * num_splits, then 8 arrays, each an int64 byte count followed by the bytes:
 * q, k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, parent (a
 * count of 0 passes NULL).
 * Output: int32 values (status of every call made, flag words, the plan's
 * split count, the admission checks), then the out bytes and lse bytes of
 * verify_attn_run, then those of the partial + merge pair.
 * Exit status 0 when every call behaved as documented, 1 otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "verify_attn.h"

#define NARR 8

static int fail(const char* what) {
  fprintf(stderr, "verify_c_client: %s\n", what);
  return 1;
}

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "verify_c_client: %s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

static size_t elem_bytes(va_dtype t) { return t == VA_F32 ? 4 : 2; }

int main(int argc, char** argv) {
  if (argc != 3) return fail("usage: verify_c_client <input> <output>");
  FILE* in = fopen(argv[1], "rb");
  if (!in) return fail("cannot open the input file");
  char magic[8];
  va_problem prob;
  int32_t num_splits;
  if (fread(magic, 1, 8, in) != 8 || memcmp(magic, "VACLIENT", 8) != 0) return fail("bad magic");
  if (fread(&prob, sizeof prob, 1, in) != 1 || fread(&num_splits, 4, 1, in) != 1) return fail("short header");
  void* host[NARR];
  int64_t bytes[NARR];
  void* dev[NARR];
  for (int i = 0; i < NARR; ++i) {
    if (fread(&bytes[i], 8, 1, in) != 1 || bytes[i] < 0) return fail("bad array size");
    host[i] = NULL;
    dev[i] = NULL;
    if (bytes[i] == 0) continue;
    host[i] = malloc((size_t)bytes[i]);
    if (!host[i] || fread(host[i], 1, (size_t)bytes[i], in) != (size_t)bytes[i]) return fail("short array");
    if (!hip_ok(hipMalloc(&dev[i], (size_t)bytes[i]), "hipMalloc input")) return 1;
    if (!hip_ok(hipMemcpy(dev[i], host[i], (size_t)bytes[i], hipMemcpyHostToDevice), "copy input")) return 1;
  }
  fclose(in);

  int32_t rec[32];
  int nrec = 0;
  int bad = 0;

  va_plan* plan = NULL;
  size_t ws_bytes = 0;
  const va_status st_plan = verify_attn_plan(&prob, num_splits, 0, &plan, &ws_bytes);
  rec[nrec++] = st_plan;
  if (st_plan != VA_OK) return fail(verify_attn_status_string(st_plan));
  va_plan_info info;
  rec[nrec++] = verify_attn_plan_get_info(plan, &info);
  rec[nrec++] = info.num_splits;
  const int S = num_splits ? num_splits : info.num_splits;

  const size_t rows = (size_t)prob.num_seqs * (size_t)prob.rows_per_seq;
  const size_t out_bytes = rows * (size_t)prob.num_q_heads * (size_t)prob.head_dim * elem_bytes(prob.out_dtype);
  const size_t lse_bytes = rows * (size_t)prob.num_q_heads * sizeof(float);
  void *ws = NULL, *out = NULL, *out2 = NULL;
  float *lse = NULL, *lse2 = NULL;
  if (!hip_ok(hipMalloc(&ws, ws_bytes), "hipMalloc workspace") || !hip_ok(hipMalloc(&out, out_bytes), "out") ||
      !hip_ok(hipMalloc(&out2, out_bytes), "out2") || !hip_ok(hipMalloc((void**)&lse, lse_bytes), "lse") ||
      !hip_ok(hipMalloc((void**)&lse2, lse_bytes), "lse2"))
    return 1;
  if (!hip_ok(hipMemset(ws, 0, ws_bytes), "zero workspace")) return 1;

  /* admission: a workspace one byte short, and a NULL pool, launch nothing */
  rec[nrec++] = verify_attn_run(plan, dev[0], dev[1], dev[2], dev[3], dev[4], (const int32_t*)dev[5],
                                (const int32_t*)dev[6], (const int32_t*)dev[7], num_splits, out, lse, ws,
                                ws_bytes - 1, NULL);
  rec[nrec++] = verify_attn_run(plan, dev[0], NULL, dev[2], dev[3], dev[4], (const int32_t*)dev[5],
                                (const int32_t*)dev[6], (const int32_t*)dev[7], num_splits, out, lse, ws, ws_bytes,
                                NULL);
  bad |= rec[nrec - 2] != VA_EWORKSPACE || rec[nrec - 1] != VA_EINVAL;

  /* the call itself, on the null stream */
  rec[nrec++] = verify_attn_run(plan, dev[0], dev[1], dev[2], dev[3], dev[4], (const int32_t*)dev[5],
                                (const int32_t*)dev[6], (const int32_t*)dev[7], num_splits, out, lse, ws, ws_bytes,
                                NULL);
  bad |= rec[nrec - 1] != VA_OK;
  uint32_t flags = 0xffffffffu;
  rec[nrec++] = verify_attn_read_flags(plan, ws, NULL, &flags);
  rec[nrec++] = (int32_t)flags;

  /* the same work as two launches: partials, then the merge */
  rec[nrec++] = verify_attn_run_partial(plan, dev[0], dev[1], dev[2], dev[3], dev[4], (const int32_t*)dev[5],
                                        (const int32_t*)dev[6], (const int32_t*)dev[7], num_splits, out2, lse2, ws,
                                        ws_bytes, NULL);
  rec[nrec++] = S > 1 ? verify_attn_run_merge(plan, num_splits, out2, lse2, ws, ws_bytes, NULL) : VA_OK;
  bad |= rec[nrec - 2] != VA_OK || rec[nrec - 1] != VA_OK;
  uint32_t flags2 = 0xffffffffu;
  rec[nrec++] = verify_attn_read_flags(plan, ws, NULL, &flags2);
  rec[nrec++] = (int32_t)flags2;
  rec[nrec++] = (int32_t)strlen(verify_attn_status_string(VA_EWORKSPACE));
  if (!hip_ok(hipDeviceSynchronize(), "synchronize")) return 1;

  char* o1 = malloc(out_bytes);
  char* o2 = malloc(out_bytes);
  char* l1 = malloc(lse_bytes);
  char* l2 = malloc(lse_bytes);
  if (!o1 || !o2 || !l1 || !l2) return fail("host allocation");
  if (!hip_ok(hipMemcpy(o1, out, out_bytes, hipMemcpyDeviceToHost), "copy out") ||
      !hip_ok(hipMemcpy(o2, out2, out_bytes, hipMemcpyDeviceToHost), "copy out2") ||
      !hip_ok(hipMemcpy(l1, lse, lse_bytes, hipMemcpyDeviceToHost), "copy lse") ||
      !hip_ok(hipMemcpy(l2, lse2, lse_bytes, hipMemcpyDeviceToHost), "copy lse2"))
    return 1;

  FILE* o = fopen(argv[2], "wb");
  if (!o) return fail("cannot open the output file");
  const int32_t n = nrec;
  if (fwrite(&n, 4, 1, o) != 1 || fwrite(rec, 4, (size_t)nrec, o) != (size_t)nrec ||
      fwrite(o1, 1, out_bytes, o) != out_bytes || fwrite(l1, 1, lse_bytes, o) != lse_bytes ||
      fwrite(o2, 1, out_bytes, o) != out_bytes || fwrite(l2, 1, lse_bytes, o) != lse_bytes)
    return fail("short write");
  fclose(o);

  verify_attn_plan_destroy(plan);
  verify_attn_plan_destroy(NULL);
  for (int i = 0; i < NARR; ++i) {
    if (dev[i]) hipFree(dev[i]);
    free(host[i]);
  }
  hipFree(ws);
  hipFree(out);
  hipFree(out2);
  hipFree(lse);
  hipFree(lse2);
  free(o1);
  free(o2);
  free(l1);
  free(l2);
  return bad ? 1 : 0;
}
