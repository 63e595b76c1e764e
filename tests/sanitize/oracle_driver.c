/* Runs the recurrent oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer on inputs read from a file and writes its
 * outputs, so that a test can compare them with the regular build.
 *
 * Input file (native endianness): int32 header {U, L, d, G, W, C, m, t_max,
 * merge, route, partials, n_threads}, float64 {eps, scale}, then float32
 * q [U,G,L,d], k, v [U,L,d], F [U,d,d], gate [U,G], ext [U,L].
 * Output file: int32 rc, then float64 y [U,G,L,d], score [U,L], S [U,d,d],
 * z [U,d], pending [U,C], int32 sel [U,n_dec,lam], n_pool [U], and with
 * partials float64 y_sa, y_la [U,G,L,d], lse_sa, lse_la [U,G,L]. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int still_oracle_run(int n_units, int L, int d, int G, int W, int C, int m, int t_max,
                     double eps, double scale, const float* q, const float* k,
                     const float* v, const float* F, const float* gate, int n_threads,
                     double* y, double* score, int32_t* sel, double* S, double* z,
                     double* pending, int32_t* n_pool, int merge, double* y_sa,
                     double* lse_sa, double* y_la, double* lse_la, int route,
                     const float* ext, const double* decay, int fp8_from);

static void* rd(FILE* f, size_t n, size_t sz) {
  void* p = malloc(n * sz > 0 ? n * sz : 1);
  if (!p || fread(p, sz, n, f) != n) {
    fprintf(stderr, "short input\n");
    exit(2);
  }
  return p;
}

int main(int argc, char** argv) {
  if (argc != 3) return 2;
  FILE* fi = fopen(argv[1], "rb");
  if (!fi) return 2;
  int32_t* h = rd(fi, 12, 4);
  const int U = h[0], L = h[1], d = h[2], G = h[3], W = h[4], C = h[5], m = h[6], tm = h[7];
  const int merge = h[8], route = h[9], part = h[10], nt = h[11];
  double* es = rd(fi, 2, 8);
  const size_t nq = (size_t)U * G * L * d, nk = (size_t)U * L * d;
  float* q = rd(fi, nq, 4);
  float* k = rd(fi, nk, 4);
  float* v = rd(fi, nk, 4);
  float* F = rd(fi, (size_t)U * d * d, 4);
  float* g = rd(fi, (size_t)U * G, 4);
  float* ext = rd(fi, (size_t)U * L, 4);
  fclose(fi);
  int lam = m >= W ? (m - W) / tm : 0;
  if (lam > C) lam = C;
  const int n_dec = L > 0 ? (L - 1) / C : 0;
  double* y = calloc(nq + 1, 8);
  double* sc = calloc((size_t)U * L + 1, 8);
  double* S = calloc((size_t)U * d * d + 1, 8);
  double* z = calloc((size_t)U * d + 1, 8);
  double* pend = calloc((size_t)U * C + 1, 8);
  int32_t* sel = calloc((size_t)U * n_dec * lam + 1, 4);
  int32_t* np = calloc((size_t)U + 1, 4);
  double *ysa = NULL, *yla = NULL, *lsa = NULL, *lla = NULL;
  if (part) {
    ysa = calloc(nq + 1, 8);
    yla = calloc(nq + 1, 8);
    lsa = calloc((size_t)U * G * L + 1, 8);
    lla = calloc((size_t)U * G * L + 1, 8);
  }
  const int32_t rc = still_oracle_run(U, L, d, G, W, C, m, tm, es[0], es[1], q, k, v, F, g, nt, y, sc, sel,
                                      S, z, pend, np, merge, ysa, lsa, yla, lla, route, ext, NULL, -1);
  FILE* fo = fopen(argv[2], "wb");
  if (!fo) return 2;
  fwrite(&rc, 4, 1, fo);
  fwrite(y, 8, nq, fo);
  fwrite(sc, 8, (size_t)U * L, fo);
  fwrite(S, 8, (size_t)U * d * d, fo);
  fwrite(z, 8, (size_t)U * d, fo);
  fwrite(pend, 8, (size_t)U * C, fo);
  fwrite(sel, 4, (size_t)U * n_dec * lam, fo);
  fwrite(np, 4, (size_t)U, fo);
  if (part) {
    fwrite(ysa, 8, nq, fo);
    fwrite(yla, 8, nq, fo);
    fwrite(lsa, 8, (size_t)U * G * L, fo);
    fwrite(lla, 8, (size_t)U * G * L, fo);
  }
  fclose(fo);
  free(h); free(es); free(q); free(k); free(v); free(F); free(g); free(ext);
  free(y); free(sc); free(S); free(z); free(pend); free(sel); free(np);
  free(ysa); free(yla); free(lsa); free(lla);
  return 0;
}
