/* Drives the oracle's C functions on small inputs for a build with address
 * and undefined-behaviour sanitizers (tests/test_sanitize_host.py).  Checks a
 * few closed forms so that the run also fails on wrong results. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void orc_m2_decays(int T, int batch, int H, const double* A, const double* dt, double* a);
void orc_m2_recur(int T, int batch, int H, int G, int P, int N, const double* a,
                  const double* dt, const double* x, const double* Bm, const double* Cm,
                  const double* D, double* hs, double* y);
void orc_gdn_recur(int T, int batch, int H, int DK, int DV, const double* q, const double* k,
                   const double* v, const double* alpha, const double* beta, double* S,
                   double* o);
void orc_bf16_encode(long n, const float* in, uint16_t* out);
void orc_bf16_decode(long n, const uint16_t* in, double* out);
void orc_e4m3_encode(long n, const float* in, uint8_t* out);
void orc_e4m3_decode(long n, const uint8_t* in, double* out);
long orc_e4m3_quant_heads(long nheads, long per_head, const float* s, float* scale,
                          uint8_t* out);

static double frand(unsigned* s) {
  *s = *s * 1664525u + 1013904223u;
  return ((*s >> 8) / 16777216.0) - 0.5;
}

static int fail(const char* what) {
  fprintf(stderr, "FAILED: %s\n", what);
  return 1;
}

int main(void) {
  unsigned seed = 1;
  enum { T = 5, B = 2, H = 4, G = 2, P = 3, N = 6, DK = 4, DV = 5 };
  /* Mamba-2 with dt = 0: the state stays, y = h C + D x */
  double A[H], D[H], dt[T * B * H], a[T * B * H], x[T * B * H * P], Bm[T * B * G * N],
      Cm[T * B * G * N], hs[B * H * P * N], h0[B * H * P * N], y[T * B * H * P];
  for (int i = 0; i < H; ++i) { A[i] = -1.0 - i; D[i] = frand(&seed); }
  for (int i = 0; i < T * B * H; ++i) dt[i] = 0.0;
  for (int i = 0; i < T * B * H * P; ++i) x[i] = frand(&seed);
  for (int i = 0; i < T * B * G * N; ++i) { Bm[i] = frand(&seed); Cm[i] = frand(&seed); }
  for (int i = 0; i < B * H * P * N; ++i) hs[i] = h0[i] = frand(&seed);
  orc_m2_decays(T, B, H, A, dt, a);
  orc_m2_recur(T, B, H, G, P, N, a, dt, x, Bm, Cm, D, hs, y);
  for (int i = 0; i < B * H * P * N; ++i)
    if (hs[i] != h0[i]) return fail("m2 dt = 0 keeps the state");
  for (int t = 0; t < T; ++t)
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < H; ++h) {
        const int g = h * G / H;
        for (int p = 0; p < P; ++p) {
          double want = D[h] * x[((t * B + b) * H + h) * P + p];
          for (int n = 0; n < N; ++n)
            want += h0[((b * H + h) * P + p) * N + n] * Cm[((t * B + b) * G + g) * N + n];
          if (fabs(y[((t * B + b) * H + h) * P + p] - want) > 1e-12) return fail("m2 y");
        }
      }
  /* GDN with beta = 0: only decay */
  double q[T * B * H * DK], k[T * B * H * DK], v[T * B * H * DV], al[T * B * H], be[T * B * H],
      S[B * H * DV * DK], S0[B * H * DV * DK], o[T * B * H * DV];
  for (int i = 0; i < T * B * H * DK; ++i) { q[i] = frand(&seed); k[i] = frand(&seed); }
  for (int i = 0; i < T * B * H * DV; ++i) v[i] = frand(&seed);
  for (int i = 0; i < T * B * H; ++i) { al[i] = 0.5; be[i] = 0.0; }
  for (int i = 0; i < B * H * DV * DK; ++i) S[i] = S0[i] = frand(&seed);
  orc_gdn_recur(T, B, H, DK, DV, q, k, v, al, be, S, o);
  for (int i = 0; i < B * H * DV * DK; ++i)
    if (fabs(S[i] - S0[i] / 32.0) > 1e-15) return fail("gdn beta = 0 decays by 2^-5");
  /* codecs over every bit pattern class */
  enum { M = 4096 };
  float f[M];
  uint16_t c16[M];
  uint8_t c8[M];
  double back[M];
  for (int i = 0; i < M; ++i) f[i] = (float)(ldexp(frand(&seed), (i % 40) - 20));
  f[0] = 0.0f; f[1] = -0.0f; f[2] = INFINITY; f[3] = NAN; f[4] = 1e30f; f[5] = -448.0f;
  orc_bf16_encode(M, f, c16);
  orc_bf16_decode(M, c16, back);
  orc_e4m3_encode(M, f, c8);
  orc_e4m3_decode(M, c8, back);
  float sc[4];
  uint8_t codes[M];
  if (orc_e4m3_quant_heads(4, M / 4, f, sc, codes) != 1) return fail("one non-finite tile");
  printf("oracle under sanitizers: ok\n");
  return 0;
}
