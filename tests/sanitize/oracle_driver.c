/*
 * oracle_driver.c -- runs the fp64 oracle (oracle/lstm_oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer on the CPU: forward and
 * backward at small shapes, both directions of time, every optional tensor
 * present and absent, and the empty cases (T = 0, B = 0, I = 0).  Every
 * buffer is allocated at exactly its documented size, so a read or write
 * past any of them is reported.  Exit status 0 when every call returned 0
 * and every output is finite.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_lstm_fwd(long T, long B, long I, long H, int reverse, const double* x, const double* W,
                    const double* b, const double* h0, const double* c0, const double* mask, double* y,
                    double* hT, double* cT, double* gates, double* cell);
int oracle_lstm_bwd(long T, long B, long I, long H, int reverse, const double* x, const double* W,
                    const double* h0, const double* c0, const double* mask, const double* y, const double* gates,
                    const double* cell, const double* dy, const double* dhT, const double* dcT, double* dx,
                    double* dW, double* db, double* dh0, double* dc0, double* dgates, double* dcell);

static unsigned long long rng_state = 88172645463325252ull;
static double uniform(void) { /* xorshift64, values in [-0.5, 0.5) */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (double)(rng_state >> 11) / 9007199254740992.0 - 0.5;
}

/* n doubles (at least one byte is requested, so that n = 0 is still a valid
 * allocation whose every access is out of bounds) */
static double* alloc(long n, int fill) {
  double* p = (double*)malloc(n > 0 ? (size_t)n * sizeof(double) : 1);
  if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
  if (fill) for (long i = 0; i < n; ++i) p[i] = uniform();
  return p;
}

static int finite_all(const double* p, long n) {
  for (long i = 0; i < n; ++i) if (!isfinite(p[i])) return 0;
  return 1;
}

static int run(long T, long B, long I, long H, int reverse, int opt) {
  const long Z = H + I, G4 = 4 * H;
  double *x = alloc(T * B * I, 1), *W = alloc(G4 * Z, 1), *b = alloc(G4, 1), *h0 = alloc(B * H, 1),
         *c0 = alloc(B * H, 1), *mask = alloc(T * B * H, 1);
  double *y = alloc(T * B * H, 0), *hT = alloc(B * H, 0), *cT = alloc(B * H, 0);
  double *gates = alloc(T * B * G4, 0), *cell = alloc(T * B * H, 0);
  double *dy = alloc(T * B * H, 1), *dhT = alloc(B * H, 1), *dcT = alloc(B * H, 1);
  double *dx = alloc(T * B * I, 0), *dW = alloc(G4 * Z, 0), *db = alloc(G4, 0), *dh0 = alloc(B * H, 0),
         *dc0 = alloc(B * H, 0), *dgates = alloc(T * B * G4, 0), *dcell = alloc(T * B * H, 0);
  /* opt: 1 = every optional tensor present, 0 = every one absent (NULL) */
  int rc = oracle_lstm_fwd(T, B, I, H, reverse, x, W, opt ? b : NULL, opt ? h0 : NULL, opt ? c0 : NULL,
                           opt ? mask : NULL, y, hT, cT, gates, cell);
  if (rc == 0)
    rc = oracle_lstm_bwd(T, B, I, H, reverse, x, W, opt ? h0 : NULL, opt ? c0 : NULL, opt ? mask : NULL, y, gates,
                         cell, dy,
                         opt ? dhT : NULL, opt ? dcT : NULL, dx, dW, opt ? db : NULL, dh0, dc0,
                         opt ? dgates : NULL, opt ? dcell : NULL);
  int ok = rc == 0 && finite_all(y, T * B * H) && finite_all(hT, B * H) && finite_all(cT, B * H) &&
           finite_all(dx, T * B * I) && finite_all(dW, G4 * Z) && finite_all(dh0, B * H) && finite_all(dc0, B * H) &&
           (!opt || finite_all(db, G4));
  if (!ok) fprintf(stderr, "FAILED T=%ld B=%ld I=%ld H=%ld reverse=%d optional=%d rc=%d\n", T, B, I, H, reverse, opt, rc);
  free(x); free(W); free(b); free(h0); free(c0); free(mask); free(y); free(hT); free(cT); free(gates); free(cell);
  free(dy); free(dhT); free(dcT); free(dx); free(dW); free(db); free(dh0); free(dc0); free(dgates); free(dcell);
  return ok;
}

int main(void) {
  static const long shapes[][4] = {{1, 1, 1, 1}, {3, 2, 5, 4}, {4, 3, 0, 6}, {0, 3, 2, 5}, {2, 0, 3, 4}, {5, 7, 9, 11}};
  int ok = 1, n = 0;
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
    for (int reverse = 0; reverse < 2; ++reverse)
      for (int opt = 0; opt < 2; ++opt) {
        ok &= run(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], reverse, opt);
        ++n;
      }
  /* an invalid size is rejected, nothing is touched */
  ok &= oracle_lstm_fwd(1, 1, 1, 0, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == -1;
  printf("%d oracle runs under the sanitizers: %s\n", n, ok ? "ok" : "FAILED");
  return ok ? 0 : 1;
}
