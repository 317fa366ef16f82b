/*
 * Host-side driver for the sanitizer lane (tests/test_sanitize.py): built
 * with -fsanitize=address,undefined and linked either against the fp64
 * oracle (ORACLE_DRIVER) or against a build of the C-ABI library whose host
 * code carries the same sanitizers (ABI_DRIVER).  It exercises the host
 * paths only: the oracle's loops on tiny inputs in every stored format, and
 * the library's argument checks, error text, provenance and workspace
 * arithmetic, none of which launches GPU work.  Exit status 0 = every check
 * held and the sanitizers reported nothing.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                               \
    }                                                         \
  } while (0)

#ifdef ORACLE_DRIVER
int oracle_prefill(const void* q, int qdtype, const void* k, const void* v, int kvdtype,
                   double* o, double* lse, const int32_t* cu_seqlens, int32_t batch, int32_t hq,
                   int32_t hkv, int32_t d, int32_t window, double scale, const int32_t* spans,
                   int32_t num_spans, const int64_t* rows, int64_t n_rows, int32_t threads);
int oracle_decode(const void* q, int qdtype, const void* k_cache, const void* v_cache,
                  int kvdtype, const int32_t* block_table, int32_t max_blocks,
                  const int32_t* seq_lens, int32_t batch, int32_t hq, int32_t hkv, int32_t d,
                  int32_t block_size, int32_t window, double scale, double* o, double* lse,
                  int32_t threads);
int oracle_prefill_backward(const void* q, int qdtype, const void* k, const void* v,
                            int kvdtype, const void* dout, int dodtype, double* dq, double* dk,
                            double* dv, const int32_t* cu_seqlens, int32_t batch, int32_t hq,
                            int32_t hkv, int32_t d, int32_t window, double scale,
                            const int32_t* spans, int32_t num_spans, int32_t threads);
int oracle_prefill_backward_units(const void* q, int qdtype, const void* k, const void* v,
                                  int kvdtype, const void* dout, int dodtype, double* dq,
                                  double* dk, double* dv, const int32_t* cu_seqlens,
                                  int32_t batch, int32_t hq, int32_t hkv, int32_t d,
                                  int32_t window, double scale, const int32_t* spans,
                                  int32_t num_spans, const int64_t* dq_units, int64_t n_dq,
                                  const int64_t* kv_units, int64_t n_kv, int32_t threads);

static double frand(unsigned* s) {
  *s = *s * 1103515245u + 12345u;
  return ((*s >> 8) & 0xffff) / 32768.0 - 1.0;
}

int main(void) {
  enum { T = 23, HQ = 4, HKV = 2, D = 8 };
  const int32_t cu[4] = {0, 1, 9, 23};
  const int32_t spans[2][2] = {{2, 6}, {12, 20}};
  unsigned seed = 7;
  double q[T * HQ * D], k[T * HKV * D], v[T * HKV * D], dout[T * HQ * D];
  float qf[T * HQ * D], kf[T * HKV * D], vf[T * HKV * D];
  uint16_t qb[T * HQ * D], kb[T * HKV * D], vb[T * HKV * D];
  for (int i = 0; i < T * HQ * D; ++i) {
    q[i] = frand(&seed);
    dout[i] = frand(&seed);
    qf[i] = (float)q[i];
    memcpy(&qb[i], (const char*)&qf[i] + 2, 2);
  }
  for (int i = 0; i < T * HKV * D; ++i) {
    k[i] = frand(&seed);
    v[i] = frand(&seed);
    kf[i] = (float)k[i];
    vf[i] = (float)v[i];
    memcpy(&kb[i], (const char*)&kf[i] + 2, 2);
    memcpy(&vb[i], (const char*)&vf[i] + 2, 2);
  }
  double o[T * HQ * D], lse[T * HQ], o2[T * HQ * D];
  const int windows[3] = {-1, 1, 5};
  for (int w = 0; w < 3; ++w) {
    CHECK(oracle_prefill(q, 2, k, v, 2, o, lse, cu, 3, HQ, HKV, D, windows[w], 0.35,
                         &spans[0][0], 2, NULL, 0, 2) == 0);
    CHECK(oracle_prefill(qf, 1, kf, vf, 1, o2, NULL, cu, 3, HQ, HKV, D, windows[w], 0.35,
                         &spans[0][0], 2, NULL, 0, 1) == 0);
    CHECK(oracle_prefill(qb, 0, kb, vb, 0, o2, NULL, cu, 3, HQ, HKV, D, windows[w], 0.35,
                         &spans[0][0], 2, NULL, 0, 1) == 0);
    for (int i = 0; i < T * HQ * D; ++i) CHECK(isfinite(o[i]) && isfinite(o2[i]));
  }
  const int64_t rows[3][2] = {{0, 0}, {22, 3}, {10, 1}};
  double orow[3 * D], lrow[3];
  CHECK(oracle_prefill(q, 2, k, v, 2, orow, lrow, cu, 3, HQ, HKV, D, 4, 0.35, NULL, 0,
                       &rows[0][0], 3, 1) == 0);
  const int64_t bad[1][2] = {{T, 0}};
  CHECK(oracle_prefill(q, 2, k, v, 2, orow, NULL, cu, 3, HQ, HKV, D, 4, 0.35, NULL, 0,
                       &bad[0][0], 1, 1) == -1);
  /* decode: 2 sequences over a 4-block cache of 4-token blocks */
  enum { NB = 4, BS = 4 };
  double kc[NB * BS * HKV * D], vc[NB * BS * HKV * D], qd[2 * HQ * D], od[2 * HQ * D], ld[2 * HQ];
  for (int i = 0; i < NB * BS * HKV * D; ++i) {
    kc[i] = frand(&seed);
    vc[i] = frand(&seed);
  }
  for (int i = 0; i < 2 * HQ * D; ++i) qd[i] = frand(&seed);
  const int32_t bt[2][2] = {{3, 1}, {0, 2}};
  const int32_t sl[2] = {7, 2};
  CHECK(oracle_decode(qd, 2, kc, vc, 2, &bt[0][0], 2, sl, 2, HQ, HKV, D, BS, -1, 0.35, od, ld,
                      2) == 0);
  CHECK(oracle_decode(qd, 2, kc, vc, 2, &bt[0][0], 2, sl, 2, HQ, HKV, D, BS, 3, 0.35, od, NULL,
                      1) == 0);
  const int32_t sl_bad[2] = {9, 2};
  CHECK(oracle_decode(qd, 2, kc, vc, 2, &bt[0][0], 2, sl_bad, 2, HQ, HKV, D, BS, -1, 0.35, od,
                      NULL, 1) == -1);
  double dq[T * HQ * D], dk[T * HKV * D], dv[T * HKV * D];
  CHECK(oracle_prefill_backward(q, 2, k, v, 2, dout, 2, dq, dk, dv, cu, 3, HQ, HKV, D, 5, 0.35,
                                &spans[0][0], 2, 2) == 0);
  for (int i = 0; i < T * HKV * D; ++i) CHECK(isfinite(dk[i]) && isfinite(dv[i]));
  /* a few listed units: the same values as the full call */
  const int64_t dq_units[3] = {0, 7 * HQ + 1, (T - 1) * HQ + HQ - 1};
  const int64_t kv_units[2] = {HKV - 1, (T - 1) * HKV};
  double uq[3 * D], uk[2 * D], uv[2 * D];
  CHECK(oracle_prefill_backward_units(q, 2, k, v, 2, dout, 2, uq, uk, uv, cu, 3, HQ, HKV, D, 5,
                                      0.35, &spans[0][0], 2, dq_units, 3, kv_units, 2, 2) == 0);
  for (int u = 0; u < 3; ++u)
    for (int c = 0; c < D; ++c) CHECK(uq[u * D + c] == dq[dq_units[u] * D + c]);
  for (int u = 0; u < 2; ++u)
    for (int c = 0; c < D; ++c)
      CHECK(uk[u * D + c] == dk[kv_units[u] * D + c] && uv[u * D + c] == dv[kv_units[u] * D + c]);
  const int64_t bad_unit[1] = {(int64_t)T * HQ};
  CHECK(oracle_prefill_backward_units(q, 2, k, v, 2, dout, 2, uq, uk, uv, cu, 3, HQ, HKV, D, 5,
                                      0.35, &spans[0][0], 2, bad_unit, 1, NULL, 0, 2) == -1);
  printf("oracle driver ok\n");
  return 0;
}
#endif

#ifdef ABI_DRIVER
#include "invattn.h"

int main(void) {
  char buf[2048];
  void* p = (void*)(uintptr_t)(1u << 20); /* never dereferenced: every call fails its checks */
  void* odd = (void*)(uintptr_t)((1u << 20) + 2);
  const int32_t* ip = (const int32_t*)p;
  CHECK(strncmp(attn_version(), "invattn", 7) == 0);
  CHECK(attn_last_provenance(buf, sizeof buf) == -1);
  /* prefill argument checks */
  CHECK(attn_prefill_varlen(p, p, p, p, NULL, ip, -1, 16, 4, 2, 64, -1, 0.125f, NULL, 0, NULL) == ATTN_E_SHAPE);
  CHECK(strlen(attn_last_error()) > 0);
  CHECK(attn_prefill_varlen(p, p, p, p, NULL, ip, 2, 16, 4, 3, 64, -1, 0.125f, NULL, 0, NULL) == ATTN_E_SHAPE);
  CHECK(attn_prefill_varlen(p, p, p, p, NULL, ip, 2, 16, 48, 3, 64, -1, 0.125f, NULL, 0, NULL) == ATTN_E_UNSUPPORTED);
  CHECK(attn_prefill_varlen(p, p, p, p, NULL, ip, 2, 16, 4, 2, 128, -1, 0.125f, NULL, 0, NULL) == ATTN_E_UNSUPPORTED);
  CHECK(attn_prefill_varlen(p, p, p, p, NULL, ip, 2, 16, 4, 2, 64, 0, 0.125f, NULL, 0, NULL) == ATTN_E_UNSUPPORTED);
  CHECK(attn_prefill_varlen(p, p, p, p, NULL, ip, 2, 16, 4, 2, 64, -1, NAN, NULL, 0, NULL) == ATTN_E_UNSUPPORTED);
  CHECK(attn_prefill_varlen(NULL, p, p, p, NULL, ip, 2, 16, 4, 2, 64, -1, 0.125f, NULL, 0, NULL) == ATTN_E_NULL);
  CHECK(attn_prefill_varlen(odd, p, p, p, NULL, ip, 2, 16, 4, 2, 64, -1, 0.125f, NULL, 0, NULL) == ATTN_E_ALIGN);
  CHECK(attn_prefill_varlen(p, p, p, p, NULL, ip, 2, 16, 4, 2, 64, -1, 0.125f, NULL, 3, NULL) == ATTN_E_NULL);
  CHECK(attn_prefill_varlen(p, p, p, p, NULL, ip, 2, 1 << 30, 4, 2, 512, -1, 0.125f, NULL, 0, NULL) == ATTN_E_UNSUPPORTED);
  /* paged prefill */
  CHECK(attn_prefill_paged(p, p, p, p, NULL, ip, ip, ip, 4, 2, 16, 64, 8, 32, 4, 2, 64, -1, 0.125f, NULL) == ATTN_E_UNSUPPORTED);
  CHECK(attn_prefill_paged(p, p, p, p, NULL, ip, ip, ip, 4, 2, 16, 8, 8, 16, 4, 2, 64, -1, 0.125f, NULL) == ATTN_E_SHAPE);
  CHECK(attn_prefill_paged(p, p, p, p, NULL, ip, ip, NULL, 4, 2, 16, 64, 8, 16, 4, 2, 64, -1, 0.125f, NULL) == ATTN_E_NULL);
  /* backward */
  CHECK(attn_prefill_varlen_backward(p, p, p, p, (float*)p, p, (float*)p, (float*)p, (float*)p,
                                     (float*)p, -1, ip, 2, 16, 4, 2, 64, -1, 0.125f, NULL, 0, NULL) == ATTN_E_SHAPE);
  CHECK(attn_prefill_varlen_backward(p, p, p, p, (float*)p, p, (float*)p, (float*)p, (float*)odd,
                                     (float*)p, 64, ip, 2, 16, 4, 2, 64, -1, 0.125f, NULL, 0, NULL) == ATTN_E_ALIGN);
  /* decode */
  CHECK(attn_decode_workspace_size(64, 32768, 32, 512) == (size_t)64 * 32 * 64 * 516 * 4);
  CHECK(attn_decode_workspace_size(0, 10, 8, 64) == 0);
  CHECK(attn_decode_paged(p, p, p, ip, 8, ip, 2, 100, 16, 16, 32, 4, 512, -1, 0.044f, p, 16, p, NULL) == ATTN_E_WORKSPACE);
  CHECK(attn_decode_paged(p, p, p, ip, 8, ip, 2, 100, 16, 8, 32, 4, 512, -1, 0.044f, p, 1 << 20, p, NULL) == ATTN_E_UNSUPPORTED);
  CHECK(attn_decode_paged(p, p, p, ip, 4, ip, 2, 100, 16, 16, 32, 4, 512, -1, 0.044f, p, 1 << 20, p, NULL) == ATTN_E_SHAPE);
  CHECK(attn_decode_paged_noalloc(p, p, p, ip, 2048, ip, 64, 32768, 100, 16, 32, 4, 512, -1, 0.044f, p, NULL) == ATTN_E_WORKSPACE);
  CHECK(strstr(attn_last_error(), "scratch") != NULL);
  /* the prologue's argument checks (no launch), then its empty-input record */
  const float* fp = (const float*)p;
  CHECK(attn_qk_prologue(p, p, ip, 8, 4, 2, 128, fp, fp, 1e-6f, 0.f, 128, 128, 1e4, NULL) == ATTN_E_UNSUPPORTED);
  CHECK(attn_qk_prologue(p, p, ip, 8, 4, 2, 256, fp, fp, 1e-6f, 0.f, 4, 256, 1e4, NULL) == ATTN_E_UNSUPPORTED);
  CHECK(attn_qk_prologue(p, p, ip, 8, 4, 2, 256, fp, fp, -1.f, 0.f, 256, 256, 1e4, NULL) == ATTN_E_UNSUPPORTED);
  CHECK(attn_qk_prologue(p, p, ip, 8, 4, 2, 256, fp, fp, 1e-6f, 0.f, 256, 256, 0.0, NULL) == ATTN_E_UNSUPPORTED);
  CHECK(attn_qk_prologue(NULL, p, ip, 8, 4, 2, 256, fp, fp, 1e-6f, 0.f, 256, 256, 1e4, NULL) == ATTN_E_NULL);
  CHECK(attn_qk_prologue(odd, p, ip, 8, 4, 2, 256, fp, fp, 1e-6f, 0.f, 256, 256, 1e4, NULL) == ATTN_E_ALIGN);
  CHECK(attn_qk_prologue(p, p, ip, -1, 4, 2, 256, fp, fp, 1e-6f, 0.f, 256, 256, 1e4, NULL) == ATTN_E_SHAPE);
  CHECK(attn_qk_prologue(NULL, NULL, NULL, 0, 4, 2, 256, NULL, NULL, 1e-6f, 0.f, 256, 256, 1e4, NULL) == ATTN_OK);
  CHECK(attn_last_provenance(buf, sizeof buf) > 0);
  CHECK(strstr(buf, "attn_qk_prologue") != NULL);
  printf("abi driver ok\n");
  return 0;
}
#endif
