/*
 * Plain-C client of the LeapQuant C ABI (include/leapquant.h): the library
 * as a C program sees it, with no Python or torch in between.
 *
 *   lq_c_driver --check    argument validation, status strings and the ABI
 *                          version (no GPU work: every call made here fails
 *                          its checks before anything is launched)
 *   lq_c_driver IN OUT     quantize the initial states, decode T tokens (the
 *                          last token of every window fused with its close,
 *                          leapquant_decode_close), dequantize the final
 *                          boundary state; all on the current HIP device
 *
 * IN  (little-endian): int32 {magic 0x3143514c, n, p, r, gate, flags, T};
 *     fp32 S0 [n][128][128]; q, k, v [T][n][128]; beta [T][n];
 *     alpha [T][n] (LQ_GATE_GDN) or [T][n][128] (LQ_GATE_KDA).
 * OUT: fp32 o [T][n][128]; int8 codes [n][16384] (stored layout); fp32
 *     row_scale [n][128], col_scale [n][128]; int32 comp_idx [n][r]; fp32
 *     comp_val [n][r][128]; fp32 dequantized boundary state [n][128][128].
 * Exit status 0 on success; a message on stderr otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "leapquant.h"

#define D 128
#define MAGIC 0x3143514c

static int fail(const char *what) {
  fprintf(stderr, "lq_c_driver: %s\n", what);
  return 1;
}

#define HIPCHECK(x)                                                        \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "lq_c_driver: %s: %s\n", #x, hipGetErrorString(e_)); \
      return 1;                                                            \
    }                                                                      \
  } while (0)

#define LQCHECK(x)                                                                    \
  do {                                                                                \
    int rc_ = (x);                                                                    \
    if (rc_ != LQ_OK) {                                                               \
      fprintf(stderr, "lq_c_driver: %s: %s\n", #x, leapquant_status_string(rc_));     \
      return 1;                                                                       \
    }                                                                                 \
  } while (0)

#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    int rc_ = (call);                                                                   \
    if (rc_ != (want)) {                                                                \
      fprintf(stderr, "lq_c_driver: %s returned %d, expected %d\n", #call, rc_, (want)); \
      return 1;                                                                         \
    }                                                                                   \
  } while (0)

/* Argument checks only.  The pointers below are host addresses that are
 * never dereferenced: each call is rejected by validation first. */
static int check_mode(void) {
  if (leapquant_abi_version() != LEAPQUANT_ABI_VERSION) return fail("ABI version mismatch");
  const int codes[] = {LQ_OK, LQ_ERR_NULL, LQ_ERR_SHAPE, LQ_ERR_UNSUPPORTED, LQ_ERR_ALIGN, LQ_ERR_ALIAS, LQ_ERR_HIP};
  for (size_t i = 0; i < sizeof codes / sizeof codes[0]; ++i) {
    const char *s = leapquant_status_string(codes[i]);
    if (!s || !*s || strcmp(s, "unknown status") == 0) return fail("missing status string");
  }
  if (strcmp(leapquant_status_string(12345), "unknown status") != 0) return fail("unknown status text");

  static float arena[1 << 16] __attribute__((aligned(64)));
  char *base = (char *)arena;
  lq_params prm = {4, D, D, 16, 4, LQ_GATE_GDN, 0u, 0};
  lq_state st;
  st.codes = (int8_t *)(base);
  st.row_scale = (float *)(base + 65536);
  st.col_scale = (float *)(base + 65536 + 2048);
  st.comp_idx = (int32_t *)(base + 65536 + 4096);
  st.comp_val = (float *)(base + 65536 + 4096 + 64);
  st.buf_gate = (float *)(base + 65536 + 16384);
  st.buf_k = (float *)(base + 65536 + 16384 + 256);
  st.buf_u = (float *)(base + 65536 + 16384 + 256 + 32768);
  st.comp_key = NULL;
  float *tok = (float *)(base + 196608);
  float *o = (float *)(base + 229376);

  EXPECT(leapquant_decode_step(NULL, &st, 0, tok, tok, tok, tok, tok, o, NULL), LQ_ERR_NULL);
  EXPECT(leapquant_decode_step(&prm, NULL, 0, tok, tok, tok, tok, tok, o, NULL), LQ_ERR_NULL);
  lq_params bad = prm;
  bad.n = 0;
  EXPECT(leapquant_decode_step(&bad, &st, 0, tok, tok, tok, tok, tok, o, NULL), LQ_ERR_SHAPE);
  bad = prm;
  bad.dk = 64;
  EXPECT(leapquant_window_close(&bad, &st, 16, NULL), LQ_ERR_UNSUPPORTED);
  bad = prm;
  bad.p = 65;
  EXPECT(leapquant_window_close(&bad, &st, 16, NULL), LQ_ERR_SHAPE);
  bad = prm;
  bad.flags = 1u << 7;
  EXPECT(leapquant_window_close(&bad, &st, 16, NULL), LQ_ERR_SHAPE);
  EXPECT(leapquant_decode_step(&prm, &st, 16, tok, tok, tok, tok, tok, o, NULL), LQ_ERR_SHAPE);
  EXPECT(leapquant_decode_step(&prm, &st, -1, tok, tok, tok, tok, tok, o, NULL), LQ_ERR_SHAPE);
  EXPECT(leapquant_window_close(&prm, &st, 0, NULL), LQ_ERR_SHAPE);
  EXPECT(leapquant_decode_step(&prm, &st, 0, NULL, tok, tok, tok, tok, o, NULL), LQ_ERR_NULL);
  lq_state mis = st;
  mis.codes = (int8_t *)(base + 8);
  EXPECT(leapquant_decode_step(&prm, &mis, 0, tok, tok, tok, tok, tok, o, NULL), LQ_ERR_ALIGN);
  /* the fp32 source of a quantize overlapping the codes it writes */
  EXPECT(leapquant_quantize_state(&prm, (const float *)st.codes, &st, NULL), LQ_ERR_ALIAS);
  /* two arrays of the state overlapping each other */
  lq_state ovl = st;
  ovl.buf_u = ovl.buf_k;
  EXPECT(leapquant_window_close(&prm, &ovl, 16, NULL), LQ_ERR_ALIAS);
  /* o overlapping a token input */
  EXPECT(leapquant_decode_step(&prm, &st, 0, tok, tok, tok, tok, tok, tok, NULL), LQ_ERR_ALIAS);
  /* dense compensators need comp_key */
  lq_params dense = prm;
  dense.flags = LQ_DENSE_COMP;
  EXPECT(leapquant_window_close(&dense, &st, 16, NULL), LQ_ERR_NULL);
  printf("lq_c_driver: argument checks passed (ABI version %d)\n", leapquant_abi_version());
  return 0;
}

static int read_all(FILE *f, void *dst, size_t bytes) { return fread(dst, 1, bytes, f) == bytes; }
static int write_all(FILE *f, const void *src, size_t bytes) { return fwrite(src, 1, bytes, f) == bytes; }

static int run_mode(const char *in_path, const char *out_path) {
  FILE *fi = fopen(in_path, "rb");
  if (!fi) return fail("cannot open input");
  int32_t hdr[7];
  if (!read_all(fi, hdr, sizeof hdr) || hdr[0] != MAGIC) return fail("bad input header");
  const int n = hdr[1], p = hdr[2], r = hdr[3], gate = hdr[4], T = hdr[6];
  const uint32_t flags = (uint32_t)hdr[5];
  if (n < 1 || p < 1 || r < 0 || T < 1 || (gate != LQ_GATE_GDN && gate != LQ_GATE_KDA))
    return fail("bad sizes in header");
  const size_t ns = (size_t)n, nt = (size_t)T;
  const size_t s_elems = ns * D * D, v_elems = nt * ns * D;
  const size_t a_elems = gate == LQ_GATE_KDA ? nt * ns * D : nt * ns;
  const size_t a_row = gate == LQ_GATE_KDA ? ns * D : ns;
  float *h_S = malloc(s_elems * 4), *h_q = malloc(v_elems * 4), *h_k = malloc(v_elems * 4);
  float *h_v = malloc(v_elems * 4), *h_b = malloc(nt * ns * 4), *h_a = malloc(a_elems * 4);
  float *h_o = malloc(v_elems * 4);
  if (!h_S || !h_q || !h_k || !h_v || !h_b || !h_a || !h_o) return fail("out of host memory");
  if (!read_all(fi, h_S, s_elems * 4) || !read_all(fi, h_q, v_elems * 4) || !read_all(fi, h_k, v_elems * 4) ||
      !read_all(fi, h_v, v_elems * 4) || !read_all(fi, h_b, nt * ns * 4) || !read_all(fi, h_a, a_elems * 4))
    return fail("short input file");
  fclose(fi);

  lq_params prm = {n, D, D, p, r, gate, flags, 0};
  lq_state st;
  memset(&st, 0, sizeof st);
  const size_t gate_elems = gate == LQ_GATE_KDA ? ns * p * D : ns * p;
  HIPCHECK(hipMalloc((void **)&st.codes, ns * D * D));
  HIPCHECK(hipMalloc((void **)&st.row_scale, ns * D * 4));
  HIPCHECK(hipMalloc((void **)&st.col_scale, ns * D * 4));
  if (r > 0) {
    HIPCHECK(hipMalloc((void **)&st.comp_idx, ns * r * 4));
    HIPCHECK(hipMalloc((void **)&st.comp_val, ns * r * D * 4));
  }
  HIPCHECK(hipMalloc((void **)&st.buf_gate, gate_elems * 4));
  HIPCHECK(hipMalloc((void **)&st.buf_k, ns * p * D * 4));
  HIPCHECK(hipMalloc((void **)&st.buf_u, ns * p * D * 4));
  float *d_S, *d_q, *d_k, *d_v, *d_b, *d_a, *d_o;
  HIPCHECK(hipMalloc((void **)&d_S, s_elems * 4));
  HIPCHECK(hipMalloc((void **)&d_q, v_elems * 4));
  HIPCHECK(hipMalloc((void **)&d_k, v_elems * 4));
  HIPCHECK(hipMalloc((void **)&d_v, v_elems * 4));
  HIPCHECK(hipMalloc((void **)&d_b, nt * ns * 4));
  HIPCHECK(hipMalloc((void **)&d_a, a_elems * 4));
  HIPCHECK(hipMalloc((void **)&d_o, v_elems * 4));
  HIPCHECK(hipMemcpy(d_S, h_S, s_elems * 4, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(d_q, h_q, v_elems * 4, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(d_k, h_k, v_elems * 4, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(d_v, h_v, v_elems * 4, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(d_b, h_b, nt * ns * 4, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(d_a, h_a, a_elems * 4, hipMemcpyHostToDevice));
  hipStream_t stream;
  HIPCHECK(hipStreamCreate(&stream));

  LQCHECK(leapquant_quantize_state(&prm, d_S, &st, stream));
  for (int t = 0; t < T; ++t) {
    const int j = t % p;
    const size_t vo = (size_t)t * ns * D;
    const float *q = d_q + vo, *k = d_k + vo, *v = d_v + vo;
    const float *b = d_b + (size_t)t * ns, *a = d_a + (size_t)t * a_row;
    float *o = d_o + vo;
    if (j == p - 1)
      LQCHECK(leapquant_decode_close(&prm, &st, j, q, k, v, b, a, o, stream));
    else
      LQCHECK(leapquant_decode_step(&prm, &st, j, q, k, v, b, a, o, stream));
  }
  LQCHECK(leapquant_dequantize_state(&prm, &st, d_S, stream));
  HIPCHECK(hipStreamSynchronize(stream));

  int8_t *h_codes = malloc(ns * D * D);
  float *h_rs = malloc(ns * D * 4), *h_cs = malloc(ns * D * 4);
  int32_t *h_ci = malloc(ns * (size_t)(r ? r : 1) * 4);
  float *h_cv = malloc(ns * (size_t)(r ? r : 1) * D * 4);
  if (!h_codes || !h_rs || !h_cs || !h_ci || !h_cv) return fail("out of host memory");
  HIPCHECK(hipMemcpy(h_o, d_o, v_elems * 4, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(h_codes, st.codes, ns * D * D, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(h_rs, st.row_scale, ns * D * 4, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(h_cs, st.col_scale, ns * D * 4, hipMemcpyDeviceToHost));
  if (r > 0) {
    HIPCHECK(hipMemcpy(h_ci, st.comp_idx, ns * r * 4, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(h_cv, st.comp_val, ns * r * D * 4, hipMemcpyDeviceToHost));
  }
  HIPCHECK(hipMemcpy(h_S, d_S, s_elems * 4, hipMemcpyDeviceToHost));

  FILE *fo = fopen(out_path, "wb");
  if (!fo) return fail("cannot open output");
  if (!write_all(fo, h_o, v_elems * 4) || !write_all(fo, h_codes, ns * D * D) ||
      !write_all(fo, h_rs, ns * D * 4) || !write_all(fo, h_cs, ns * D * 4) ||
      (r > 0 && (!write_all(fo, h_ci, ns * r * 4) || !write_all(fo, h_cv, ns * r * D * 4))) ||
      !write_all(fo, h_S, s_elems * 4))
    return fail("short write");
  if (fclose(fo) != 0) return fail("cannot close output");

  HIPCHECK(hipStreamDestroy(stream));
  void *dev[] = {st.codes, st.row_scale, st.col_scale, st.comp_idx, st.comp_val, st.buf_gate,
                 st.buf_k, st.buf_u, d_S, d_q, d_k, d_v, d_b, d_a, d_o};
  for (size_t i = 0; i < sizeof dev / sizeof dev[0]; ++i)
    if (dev[i]) HIPCHECK(hipFree(dev[i]));
  free(h_S); free(h_q); free(h_k); free(h_v); free(h_b); free(h_a); free(h_o);
  free(h_codes); free(h_rs); free(h_cs); free(h_ci); free(h_cv);
  printf("lq_c_driver: %d states, %d tokens, window %d, r %d, gate %d: done\n", n, T, p, r, gate);
  return 0;
}

int main(int argc, char **argv) {
  if (argc == 2 && strcmp(argv[1], "--check") == 0) return check_mode();
  if (argc == 3) return run_mode(argv[1], argv[2]);
  fprintf(stderr, "usage: lq_c_driver --check | lq_c_driver IN OUT\n");
  return 2;
}
