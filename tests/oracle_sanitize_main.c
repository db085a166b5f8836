/*
 * oracle_sanitize_main.c -- a driver that runs the fp64 oracle (oracle/spec_verify_ref.c)
 * under AddressSanitizer and UndefinedBehaviorSanitizer on the CPU (test infrastructure;
 * built and run by tests/test_oracle_sanitize.py).
 *
 * Usage: oracle_sanitize <case file> <output file>.  A case file holds a header of int32
 * and double fields followed by the arrays of one call; the driver makes that call and
 * writes every output array, so the test can compare them with the regular build.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int ref_spec_verify(const void *target, const void *draft, int dtype, const int32_t *tokens,
                    const float *u_accept, const float *u_sample, int B, int G, int V,
                    double temperature, int top_k, int32_t *accepted_len, int32_t *out_tokens,
                    double *row_logz, double *accept_margin, double *sample_margin, int nthreads);
int ref_tree_verify(const void *target, const void *draft, int dtype, const int32_t *tokens,
                    const int32_t *parent, const float *u_accept, const float *u_sample, int B,
                    int N, int V, double T, int top_k, int32_t *accepted_len,
                    int32_t *out_tokens, int32_t *path_nodes, double *accept_margin,
                    double *sample_margin, int nthreads);
int ref_typical_verify(const void *target, int dtype, const int32_t *tokens, int B, int G, int V,
                       double T, int top_k, double eps, double delta, int32_t *accepted_len,
                       int32_t *out_tokens, double *margin, double *entropy_out, int nthreads);
int ref_overlap(const void *target, const void *draft, int dtype, int B, int G, int V,
                int target_rows, double temperature, int top_k, double *beta, double *tv,
                int32_t *status, int nthreads);
int ref_sample_rows(const void *logits, int dtype, int R, int V, double temperature, int top_k,
                    const float *u, int32_t *tokens, int32_t *status, double *margin, int nthreads);

static void *readn(FILE *f, size_t n) {
  void *p = malloc(n ? n : 1);
  if (n && fread(p, 1, n, f) != n) {
    fprintf(stderr, "short case file\n");
    exit(2);
  }
  return p;
}

static void writen(FILE *f, const void *p, size_t n) {
  if (n && fwrite(p, 1, n, f) != n) exit(3);
}

int main(int argc, char **argv) {
  if (argc != 3) return 2;
  FILE *f = fopen(argv[1], "rb");
  if (!f) return 2;
  int32_t h[8];
  double d[3];
  if (fread(h, sizeof h, 1, f) != 1 || fread(d, sizeof d, 1, f) != 1) return 2;
  const int fn = h[0], dtype = h[1], B = h[2], G = h[3], V = h[4], k = h[5], x = h[6];
  const double T = d[0];
  const size_t esz = dtype ? 2 : 4;
  FILE *o = fopen(argv[2], "wb");
  if (!o) return 2;
  int rc = 0;
  if (fn == 0) { /* chain verification: target [B,G+1,V], draft [B,G,V], tokens, u_accept, u_sample */
    void *t = readn(f, (size_t)B * (G + 1) * V * esz), *dr = readn(f, (size_t)B * G * V * esz);
    int32_t *tok = readn(f, (size_t)B * G * 4);
    float *ua = readn(f, (size_t)B * G * 4), *us = readn(f, (size_t)B * 4);
    int32_t *acc = malloc((size_t)B * 4), *out = malloc((size_t)B * (G + 1) * 4);
    double *lz = malloc((size_t)B * (2 * G + 1) * 8 + 8), *am = malloc((size_t)B * G * 8 + 8), *sm = malloc((size_t)B * 8);
    rc = ref_spec_verify(t, dr, dtype, tok, ua, us, B, G, V, T, k, acc, out, lz, am, sm, 2);
    writen(o, acc, (size_t)B * 4);
    writen(o, out, (size_t)B * (G + 1) * 4);
    writen(o, sm, (size_t)B * 8);
    free(t); free(dr); free(tok); free(ua); free(us); free(acc); free(out); free(lz); free(am); free(sm);
  } else if (fn == 1) { /* tree verification: N = G nodes */
    const int N = G;
    void *t = readn(f, (size_t)B * N * V * esz), *dr = readn(f, (size_t)B * N * V * esz);
    int32_t *tok = readn(f, (size_t)B * N * 4), *par = readn(f, (size_t)B * N * 4);
    float *ua = readn(f, (size_t)B * N * 4), *us = readn(f, (size_t)B * 4);
    int32_t *acc = malloc((size_t)B * 4), *out = malloc((size_t)B * N * 4), *path = malloc((size_t)B * N * 4);
    double *am = malloc((size_t)B * N * 8), *sm = malloc((size_t)B * 8);
    rc = ref_tree_verify(t, dr, dtype, tok, par, ua, us, B, N, V, T, k, acc, out, path, am, sm, 2);
    writen(o, acc, (size_t)B * 4);
    writen(o, out, (size_t)B * N * 4);
    writen(o, path, (size_t)B * N * 4);
    free(t); free(dr); free(tok); free(par); free(ua); free(us); free(acc); free(out); free(path); free(am); free(sm);
  } else if (fn == 2) { /* typical acceptance: eps = d[1], delta = d[2] */
    void *t = readn(f, (size_t)B * (G + 1) * V * esz);
    int32_t *tok = readn(f, (size_t)B * G * 4);
    int32_t *acc = malloc((size_t)B * 4), *out = malloc((size_t)B * (G + 1) * 4);
    double *mg = malloc((size_t)B * G * 8 + 8), *en = malloc((size_t)B * (G + 1) * 8);
    rc = ref_typical_verify(t, dtype, tok, B, G, V, T, k, d[1], d[2], acc, out, mg, en, 2);
    writen(o, acc, (size_t)B * 4);
    writen(o, out, (size_t)B * (G + 1) * 4);
    writen(o, en, (size_t)B * (G + 1) * 8);
    free(t); free(tok); free(acc); free(out); free(mg); free(en);
  } else if (fn == 3) { /* overlap: target rows x = G or G + 1 */
    void *t = readn(f, (size_t)B * x * V * esz), *dr = readn(f, (size_t)B * G * V * esz);
    double *be = malloc((size_t)B * G * 8 + 8), *tv = malloc((size_t)B * G * 8 + 8);
    int32_t *s = malloc((size_t)B * G * 4 + 4);
    rc = ref_overlap(t, dr, dtype, B, G, V, x, T, k, be, tv, s, 2);
    writen(o, be, (size_t)B * G * 8);
    writen(o, tv, (size_t)B * G * 8);
    writen(o, s, (size_t)B * G * 4);
    free(t); free(dr); free(be); free(tv); free(s);
  } else { /* batched sampler: B rows of V */
    void *z = readn(f, (size_t)B * V * esz);
    float *u = readn(f, (size_t)B * 4);
    int32_t *tok = malloc((size_t)B * 4), *s = malloc((size_t)B * 4);
    double *mg = malloc((size_t)B * 8);
    rc = ref_sample_rows(z, dtype, B, V, T, k, u, tok, s, mg, 2);
    writen(o, tok, (size_t)B * 4);
    writen(o, s, (size_t)B * 4);
    free(z); free(u); free(tok); free(s); free(mg);
  }
  fclose(o);
  fclose(f);
  return rc == 0 ? 0 : 4;
}
