/*
 * oracle.c -- plain, slow, fp64 CPU reference for the ReplaySSM decode-time
 * state engine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP path, and the HIP path never calls it.
 *
 * What it computes is the plain *eager* definition of each recurrence: read the
 * whole state, update it with the step's input, produce the output.  The
 * ReplaySSM pages ("ReplaySSM: Cache SSM Inputs, Not State", Abstract (arXiv);
 * frontier.agentik-os.com explainer, "What ReplaySSM is solving") describe the
 * method as an execution-order change of exactly this recurrence (checkpoint +
 * buffer of recent inputs, replayed), so the eager result *is* the answer the
 * replay path must reach, up to rounding order.  The pages do not print the
 * update equations (explainer, "What is not documented"); they are the textbook
 * ones of the two layer types the pages name, Mamba-2 (SSD) and Gated DeltaNet,
 * both listed under "Builds on" on the mlsanity index page.
 *
 * Every floating-point operation is in double precision on inputs that the
 * caller has widened exactly from fp32.  Independent (sequence, head) units are
 * distributed over OpenMP threads; inside a unit the time loop is sequential.
 *
 * The low-precision codecs at the end (bf16, OCP FP8 E4M3) are written from
 * the number formats' definitions (IEEE-754 round-to-nearest-even on the
 * binary16-style bfloat16 layout; OCP 8-bit Floating Point Specification v1.0,
 * E4M3: bias 7, no infinities, S.1111.111 = NaN, max normal 448).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <fenv.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* Mamba-2 (SSD) decode recurrence, per head h with group g = h*G/H:         */
/*   a_t = exp(dt_t * A_h)                       (scalar decay per head)     */
/*   h_t = a_t * h_{t-1} + dt_t * x_t B_t^T      (P x N state)               */
/*   y_t = h_t C_t + D_h * x_t                                               */
/* ------------------------------------------------------------------------ */

/* Decays a[t][b][h] = exp(dt[t][b][h] * A[h]).  Kept separate from the
 * recurrence so that exact-arithmetic tests can feed dyadic decays directly. */
void orc_m2_decays(int T, int batch, int H, const double* A, const double* dt,
                   double* a) {
  for (long t = 0; t < T; ++t)
    for (long b = 0; b < batch; ++b)
      for (long h = 0; h < H; ++h) {
        long i = (t * batch + b) * H + h;
        a[i] = exp(dt[i] * A[h]);
      }
}

/* T eager steps from the state held in hs, which is updated in place.
 *   a, dt : [T][batch][H]        x : [T][batch][H][P]
 *   Bm, Cm: [T][batch][G][N]     D : [H]
 *   hs    : [batch][H][P][N]     y : [T][batch][H][P] (output)              */
void orc_m2_recur(int T, int batch, int H, int G, int P, int N,
                  const double* a, const double* dt, const double* x,
                  const double* Bm, const double* Cm, const double* D,
                  double* hs, double* y) {
  long units = (long)batch * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (long u = 0; u < units; ++u) {
    long b = u / H, h = u % H;
    long g = h * G / H;
    double* st = hs + u * (long)P * N;
    for (long t = 0; t < T; ++t) {
      double at = a[(t * batch + b) * H + h];
      double dtt = dt[(t * batch + b) * H + h];
      const double* xt = x + ((t * batch + b) * H + h) * (long)P;
      const double* Bt = Bm + ((t * batch + b) * G + g) * (long)N;
      const double* Ct = Cm + ((t * batch + b) * G + g) * (long)N;
      double* yt = y + ((t * batch + b) * H + h) * (long)P;
      for (long p = 0; p < P; ++p) {
        double acc = 0.0;
        for (long n = 0; n < N; ++n) {
          double v = at * st[p * N + n] + dtt * xt[p] * Bt[n];
          st[p * N + n] = v;
          acc += v * Ct[n];
        }
        yt[p] = acc + D[h] * xt[p];
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Gated DeltaNet decode recurrence, per head (state S is dv x dk):          */
/*   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T          */
/*   o_t = S_t q_t                                                           */
/* S (I - beta k k^T) is expanded as S - beta (S k) k^T, which is the same    */
/* matrix product written out for a rank-one term.                           */
/*   q, k : [T][batch][H][DK]   v : [T][batch][H][DV]                        */
/*   alpha, beta : [T][batch][H]                                              */
/*   S : [batch][H][DV][DK] in/out      o : [T][batch][H][DV]                 */
/* ------------------------------------------------------------------------ */
void orc_gdn_recur(int T, int batch, int H, int DK, int DV,
                   const double* q, const double* k, const double* v,
                   const double* alpha, const double* beta,
                   double* S, double* o) {
  long units = (long)batch * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (long u = 0; u < units; ++u) {
    long b = u / H, h = u % H;
    double* st = S + u * (long)DV * DK;
    for (long t = 0; t < T; ++t) {
      long ui = (t * batch + b) * H + h;
      double al = alpha[ui], be = beta[ui];
      const double* qt = q + ui * (long)DK;
      const double* kt = k + ui * (long)DK;
      const double* vt = v + ui * (long)DV;
      double* ot = o + ui * (long)DV;
      for (long r = 0; r < DV; ++r) {
        double* row = st + r * DK;
        double sk = 0.0;
        for (long c = 0; c < DK; ++c) sk += row[c] * kt[c];
        double acc = 0.0;
        for (long c = 0; c < DK; ++c) {
          double nv = al * (row[c] - be * sk * kt[c]) + be * vt[r] * kt[c];
          row[c] = nv;
          acc += nv * qt[c];
        }
        ot[r] = acc;
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Number formats.                                                           */
/* ------------------------------------------------------------------------ */

/* Round-to-nearest, ties-to-even of m to an integer (default FP environment
 * rounding mode is to-nearest-even; nearbyint honours it). */
static double rne(double m) { return nearbyint(m); }

/* fp32 -> bfloat16 (1 sign, 8 exponent, 7 fraction bits; same exponent range
 * as binary32), round to nearest even.  A bf16 value with exponent e has
 * spacing 2^(e-7) between neighbours (normals, e >= -126) and 2^(-133) in the
 * subnormal range.  Values that round beyond the largest finite bf16 become
 * infinity, NaN stays NaN (quiet, sign kept). */
static uint16_t bf16_encode_one(float f) {
  uint32_t bits;
  memcpy(&bits, &f, 4);
  uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  if (isnan(f)) return (uint16_t)(sign | 0x7FC0u);
  double a = fabs((double)f);
  if (isinf(f)) return (uint16_t)(sign | 0x7F80u);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);          /* a = m * 2^e, m in [0.5, 1): leading bit 2^(e-1) */
  int lead = e - 1;      /* floor(log2 a) */
  if (lead < -126) lead = -126;          /* subnormal range: fixed spacing */
  double step = ldexp(1.0, lead - 7);
  double q = rne(a / step) * step;       /* exact: a/step has <= 24 bits */
  if (q == 0.0) return sign;             /* rounded to (signed) zero */
  if (q >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
  /* pack: q is an exact bf16 value */
  int qe;
  double qm = frexp(q, &qe);             /* q = qm * 2^qe */
  int ql = qe - 1;
  uint32_t expo, frac;
  if (ql < -126) {                       /* subnormal */
    expo = 0;
    frac = (uint32_t)(q / ldexp(1.0, -133));
  } else {
    expo = (uint32_t)(ql + 127);
    frac = (uint32_t)((qm * 2.0 - 1.0) * 128.0);
  }
  return (uint16_t)(sign | (expo << 7) | frac);
}

static double bf16_decode_one(uint16_t c) {
  uint32_t expo = (c >> 7) & 0xFFu, frac = c & 0x7Fu;
  double s = (c & 0x8000u) ? -1.0 : 1.0;
  if (expo == 0xFF) return frac ? NAN : s * INFINITY;
  if (expo == 0) return s * ldexp((double)frac, -133);
  return s * ldexp(1.0 + frac / 128.0, (int)expo - 127);
}

void orc_bf16_encode(long n, const float* in, uint16_t* out) {
  for (long i = 0; i < n; ++i) out[i] = bf16_encode_one(in[i]);
}

void orc_bf16_decode(long n, const uint16_t* in, double* out) {
  for (long i = 0; i < n; ++i) out[i] = bf16_decode_one(in[i]);
}

/* OCP E4M3: value = (-1)^s * 2^(E-7) * (1 + M/8) for E in 1..15 (except
 * E=15,M=7 which is NaN), and (-1)^s * 2^-6 * (M/8) for E = 0.  Encoding of a
 * finite value: round to nearest representable, ties to even mantissa, and
 * saturate to +-448 (the largest finite magnitude) when the rounded magnitude
 * would exceed it.  NaN input encodes as S.1111.111. */
static uint8_t e4m3_encode_one(float f) {
  uint32_t bits;
  memcpy(&bits, &f, 4);
  uint8_t sign = (uint8_t)((bits >> 24) & 0x80u);
  if (isnan(f)) return (uint8_t)(sign | 0x7Fu);
  if (isinf(f)) return (uint8_t)(sign | 0x7Eu);  /* no infinity: saturates to 448 */
  double a = fabs((double)f);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int lead = e - 1;                       /* floor(log2 a) */
  if (lead < -6) lead = -6;               /* subnormals share 2^-6's spacing */
  double step = ldexp(1.0, lead - 3);     /* 3 fraction bits */
  double q = rne(a / step) * step;
  if (q > 448.0) q = 448.0;               /* saturating */
  /* pack */
  int qe;
  frexp(q, &qe);
  int ql = qe - 1;
  uint8_t expo, frac;
  if (q < ldexp(1.0, -6)) {               /* subnormal (or zero) */
    expo = 0;
    frac = (uint8_t)(q / ldexp(1.0, -9));
  } else {
    expo = (uint8_t)(ql + 7);
    frac = (uint8_t)((q / ldexp(1.0, ql) - 1.0) * 8.0);
  }
  return (uint8_t)(sign | (expo << 3) | frac);
}

static double e4m3_decode_one(uint8_t c) {
  uint32_t expo = (c >> 3) & 0xFu, frac = c & 0x7u;
  double s = (c & 0x80u) ? -1.0 : 1.0;
  if (expo == 0xF && frac == 0x7) return NAN;
  if (expo == 0) return s * ldexp((double)frac, -9);
  return s * ldexp(1.0 + frac / 8.0, (int)expo - 7);
}

void orc_e4m3_encode(long n, const float* in, uint8_t* out) {
  for (long i = 0; i < n; ++i) out[i] = e4m3_encode_one(in[i]);
}

void orc_e4m3_decode(long n, const uint8_t* in, double* out) {
  for (long i = 0; i < n; ++i) out[i] = e4m3_decode_one(in[i]);
}

/* Per-head scaled E4M3 quantisation of fp32 state tiles (one tile per head):
 *   amax  = max |s| over the tile (fp32)
 *   scale = amax / 448 in fp32 arithmetic, or 1 when that is 0 (amax 0, or
 *           amax so small that the fp32 quotient underflows to 0)
 *   code  = E4M3(s / scale) with the fp32 quotient rounded once (IEEE)
 * A tile holding a NaN or an infinity has no meaningful amax: its scale is 1
 * and its values are encoded as they are (saturating, NaN kept).
 * The decisions are taken in fp32, the precision in which a kernel holds its
 * state, so that identical fp32 tiles give identical codes.
 * Returns the number of tiles that held a non-finite value.                 */
long orc_e4m3_quant_heads(long nheads, long per_head, const float* s,
                          float* scale, uint8_t* out) {
  long nonfinite = 0;
  for (long h = 0; h < nheads; ++h) {
    const float* tile = s + h * per_head;
    float amax = 0.0f;
    int finite = 1;
    for (long i = 0; i < per_head; ++i) {
      float v = fabsf(tile[i]);
      if (!isfinite(v)) finite = 0;
      if (v > amax) amax = v;
    }
    nonfinite += !finite;
    volatile float sc = (finite && amax > 0.0f) ? amax / 448.0f : 1.0f;
    if (sc == 0.0f) sc = 1.0f;   /* amax / 448 below the smallest subnormal: as for amax 0 */
    scale[h] = sc;
    for (long i = 0; i < per_head; ++i) {
      volatile float qv = tile[i] / sc;
      out[h * per_head + i] = e4m3_encode_one(qv);
    }
  }
  return nonfinite;
}
