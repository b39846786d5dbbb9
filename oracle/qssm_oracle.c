/*
 * qssm_oracle.c — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, sequential fp64 CPU reference for the quantized state-space hot path. Only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark may load it; the product
 * library never calls it and shares no source with it.
 *
 * Every function follows the definition it cites, in the order the definition states it, with no
 * blocking, fusion or reordering. Loops over time are sequential; OpenMP is used only across
 * independent chains, so results do not depend on the thread count.
 *
 * Sources (page title, section):
 *  [Q2]  "Quamba2: A Robust and Scalable Post-training Quantization Framework for Selective State
 *        Space Models" — abstract and method steps 1-4: per-group x scales over sorted/clustered
 *        channels, per-state-group B/C scales, offline rearrangement (compute invariance).
 *  [S4D] "Quantizing Small-Scale State-Space Models for Edge AI" — abstract: S4D layer under
 *        quantization, A and the state are sensitive, heterogeneous precision.
 *  [SSD] SSDi8 page — abstract: structured state-space duality (recurrent and attention modes),
 *        persistent INT8 path, quantization at cost-effective points.
 *  [SE]  Quamba-SE soft-edge blog — 2.1 three scales, 2.2 classifier and byte layout, 4.1 thresholds.
 *
 * Numbers are double unless a definition fixes fp32 (scales are fp32 values; codes are decided
 * from the exact quotient of fp32 operands).
 */
#include <complex.h>
#include <omp.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------------------------ */
/* Quantizer. q = clamp(RNE(v / s), lo, hi) with v / s the exact rational quotient.
 * For fp32 v and s the fp64 quotient never crosses or lands on a half-integer unless the exact
 * quotient is one (its distance to the nearest half-integer is at least 2^-48 relative, far above
 * the 2^-53 rounding of the fp64 division), so rint() of the fp64 quotient is the exact RNE.
 * A scale outside [2^-100, 2^100] (or NaN) is invalid: the caller writes 0 for the whole group. */
static int scale_valid(double s) { return s >= 0x1p-100 && s <= 0x1p100; }

static int32_t round_sat(float v, double s, int32_t lo, int32_t hi) {
  if (isnan(v)) return 0;
  double r = rint((double)v / s);
  if (r < (double)lo) return lo;
  if (r > (double)hi) return hi;
  return (int32_t)r;
}

EXPORT int32_t orc_quant_code(float v, float s) {
  if (!scale_valid((double)s)) return 0;
  return round_sat(v, (double)s, -128, 127);
}

/* [Q2] x grouped quantization: q[o,c,i] = quant(x[o, perm[c], i], scales[group_of[c]]). */
EXPORT void orc_quant_group_x(const float* x, int64_t outer, int64_t C, int64_t inner,
                              const int32_t* perm, const uint8_t* group_of, const float* scales,
                              int8_t* q) {
  for (int64_t o = 0; o < outer; ++o)
    for (int64_t c = 0; c < C; ++c) {
      int64_t src = perm ? perm[c] : c;
      float s = scales[group_of[c]];
      for (int64_t i = 0; i < inner; ++i)
        q[(o * C + c) * inner + i] = (int8_t)orc_quant_code(x[(o * C + src) * inner + i], s);
    }
}

/* [Q2] per-state-group quantization of B or C viewed as [outer, Gbc, N, inner]. */
EXPORT void orc_quant_state_group(const float* bc, int64_t outer, int64_t Gbc, int64_t N,
                                  int64_t inner, int64_t gs, const float* scales, int8_t* q) {
  int64_t ngs = N / gs;
  for (int64_t o = 0; o < outer; ++o)
    for (int64_t g = 0; g < Gbc; ++g)
      for (int64_t n = 0; n < N; ++n) {
        float s = scales[g * ngs + n / gs];
        for (int64_t i = 0; i < inner; ++i) {
          int64_t k = ((o * Gbc + g) * N + n) * inner + i;
          q[k] = (int8_t)orc_quant_code(bc[k], s);
        }
      }
}

/* Calibration scale from an absmax: fl32(absmax / 127) (fp32 division, correctly rounded);
 * absmax 0 -> 1; clamped into the valid range. */
EXPORT float orc_scale_from_absmax(float absmax) {
  if (absmax == 0.0f) return 1.0f;
  float s = absmax / 127.0f;
  if (s < 0x1p-100f) s = 0x1p-100f;
  if (s > 0x1p100f) s = 0x1p100f;
  return s;
}

/* ------------------------------------------------------------------------------------------ */
/* [SE] 2.1-2.2 soft-edge code of one value. Classification on |v| with strict comparisons;
 * the {small, large} case table: (1,0) -> scale/ratio, (0,1) -> scale*ratio, otherwise the base
 * scale. ratio is 4 for the form of sections 2.1-2.2 and 2 for the shift-only form that section 4.1
 * suggests for small hardware (one shift instead of a multiplier); nothing else changes. */
static int ratio_ok(int32_t ratio) { return ratio == 2 || ratio == 4; }

EXPORT uint8_t orc_softedge_code(float v, float s, float L, float H, int32_t ratio) {
  if (!ratio_ok(ratio) || !scale_valid((double)s) || isnan(v)) return 0x00;
  float a = fabsf(v);
  int is_small = a < L;
  int is_large = a > H;
  if (is_small && !is_large) {
    int32_t q = round_sat(v, (double)s / (double)ratio, -32, 31);
    return (uint8_t)(0x80 | (q & 0x3F));
  }
  if (is_large && !is_small) {
    int32_t q = round_sat(v, (double)s * (double)ratio, -32, 31);
    return (uint8_t)(0xC0 | (q & 0x3F));
  }
  int32_t q = round_sat(v, (double)s, -64, 63);
  return (uint8_t)(q & 0x7F);
}

/* Value of a soft-edge byte in fp64 (exact: a small integer times a power-of-two multiple of s). */
EXPORT double orc_softedge_value(uint8_t b, float s, int32_t ratio) {
  if (!ratio_ok(ratio) || !scale_valid((double)s)) return 0.0;
  if ((b & 0x80) == 0) {
    int32_t q = (b & 0x40) ? (int32_t)(b & 0x7F) - 128 : (int32_t)(b & 0x7F); /* sign-extend 7 bits */
    return (double)q * (double)s;
  }
  int32_t q = (b & 0x20) ? (int32_t)(b & 0x3F) - 64 : (int32_t)(b & 0x3F); /* sign-extend 6 bits */
  if ((b & 0x40) == 0) return (double)q * ((double)s / (double)ratio);
  return (double)q * ((double)s * (double)ratio);
}

/* The fp32 decode defined by the library contract: the fp64 value rounded once to fp32
 * (the product of a <= 7-bit integer and an fp32 scale is exact in fp64). */
EXPORT float orc_softedge_decode_f32(uint8_t b, float s, int32_t ratio) {
  return (float)orc_softedge_value(b, s, ratio);
}

EXPORT void orc_softedge_encode(const float* x, int64_t outer, int64_t C, int64_t inner,
                                const int32_t* perm, const uint8_t* group_of, const float* s,
                                const float* L, const float* H, int32_t ratio, uint8_t* code) {
  for (int64_t o = 0; o < outer; ++o)
    for (int64_t c = 0; c < C; ++c) {
      int64_t src = perm ? perm[c] : c;
      int g = group_of[c];
      for (int64_t i = 0; i < inner; ++i)
        code[(o * C + c) * inner + i] =
            orc_softedge_code(x[(o * C + src) * inner + i], s[g], L[g], H[g], ratio);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* [Q2] step 2, clustering of the sorted channel absmax values into G contiguous groups.
 * Exact 1-D k-means: minimize the sum over groups of sum (v - mean)^2 by dynamic programming
 * over split points. Segment cost from prefix sums in fp64, accumulated in sorted order:
 *   cost(j, i) = (S2[i] - S2[j]) - (S1[i] - S1[j])^2 / (i - j)   for sorted positions j..i-1.
 * Ties between split points go to the smallest split index. `sorted` is ascending. */
EXPORT void orc_cluster_sorted(const double* sorted, int32_t C, int32_t G, uint8_t* group_of) {
  double* S1 = calloc((size_t)C + 1, sizeof(double));
  double* S2 = calloc((size_t)C + 1, sizeof(double));
  double* dp = malloc(sizeof(double) * (size_t)(G + 1) * (size_t)(C + 1));
  int32_t* arg = malloc(sizeof(int32_t) * (size_t)(G + 1) * (size_t)(C + 1));
  for (int32_t i = 0; i < C; ++i) {
    S1[i + 1] = S1[i] + sorted[i];
    S2[i + 1] = S2[i] + sorted[i] * sorted[i];
  }
#define DP(k, i) dp[(size_t)(k) * (size_t)(C + 1) + (size_t)(i)]
#define ARG(k, i) arg[(size_t)(k) * (size_t)(C + 1) + (size_t)(i)]
  for (int32_t i = 0; i <= C; ++i) { DP(0, i) = INFINITY; ARG(0, i) = 0; }
  DP(0, 0) = 0.0;
  for (int32_t k = 1; k <= G; ++k)
    for (int32_t i = 0; i <= C; ++i) {
      DP(k, i) = INFINITY;
      ARG(k, i) = 0;
      /* the k-th group covers sorted positions j .. i-1, with at least one element */
      for (int32_t j = k - 1; j < i; ++j) {
        if (DP(k - 1, j) == INFINITY) continue;
        double s1 = S1[i] - S1[j], s2 = S2[i] - S2[j];
        double cost = s2 - s1 * s1 / (double)(i - j);
        double tot = DP(k - 1, j) + cost;
        if (tot < DP(k, i)) { DP(k, i) = tot; ARG(k, i) = j; }
      }
    }
  int32_t end = C;
  for (int32_t k = G; k >= 1; --k) {
    int32_t start = ARG(k, end);
    for (int32_t c = start; c < end; ++c) group_of[c] = (uint8_t)(k - 1);
    end = start;
  }
#undef DP
#undef ARG
  free(S1); free(S2); free(dp); free(arg);
}

/* ------------------------------------------------------------------------------------------ */
/* [Q2] selective scan, sequential in time, all fp64. Layouts as in the library:
 *   xh, delta, y [B, D, L]; A [D, N]; Bh, Ch [B, Gbc, N, L]; Dskip [D]; h0, h_last [B, D, N].
 * Per (b, d, n): h = exp(delta_t * A[d,n]) * h + delta_t * Bh[n,t] * xh_t,
 *                y_t = sum_n Ch[n,t] * h_t + Dskip[d] * xh_t. */
EXPORT void orc_selective_scan(int64_t B, int64_t L, int64_t D, int64_t N, int64_t Gbc,
                               const double* xh, const double* delta, const double* A,
                               const double* Bh, const double* Ch, const double* Dskip,
                               const double* h0, double* y, double* h_last) {
  int64_t dpg = D / Gbc;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t d = 0; d < D; ++d) {
      int64_t g = d / dpg;
      double* h = malloc(sizeof(double) * (size_t)N);
      for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        double dt = delta[(b * D + d) * L + t];
        double xv = xh[(b * D + d) * L + t];
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          double bn = Bh[((b * Gbc + g) * N + n) * L + t];
          double cn = Ch[((b * Gbc + g) * N + n) * L + t];
          h[n] = exp(dt * A[d * N + n]) * h[n] + dt * bn * xv;
          acc += cn * h[n];
        }
        y[(b * D + d) * L + t] = acc + (Dskip ? Dskip[d] : 0.0) * xv;
      }
      if (h_last)
        for (int64_t n = 0; n < N; ++n) h_last[(b * D + d) * N + n] = h[n];
      free(h);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* [S4D] diagonal LTI scan with zero-order hold, complex fp64.
 *   u [B, H, L] (dequantized input), Ah, Bh, Ch [H, N] complex (re, im interleaved),
 *   dt [H] (= exp(log_dt)), Dskip [H].
 *   Abar = exp(dt*Ah); Bbar = (Abar - 1) / Ah * Bh (dt * Bh when Ah == 0);
 *   h_t = Abar h_{t-1} + Bbar u_t; y_t = Re(sum_n Ch h_t) + Dskip u_t.
 * state_scale == NULL: fp64 state. Otherwise each part is replaced after every step by
 *   state_scale[h] * clamp(RNE(part / state_scale[h]), -32768, 32767)  (int16 state).
 * h0 / h_last: [B, H, N] complex or NULL. */
EXPORT void orc_s4d_zoh(const double* Ah, const double* Bh, double dt, int64_t n,
                        double* Abar, double* Bbar) {
  for (int64_t k = 0; k < n; ++k) {
    double complex a = Ah[2 * k] + I * Ah[2 * k + 1];
    double complex bb = Bh[2 * k] + I * Bh[2 * k + 1];
    double complex ab = cexp(dt * a);
    double complex bbar = (a == 0.0) ? dt * bb : (ab - 1.0) / a * bb;
    Abar[2 * k] = creal(ab); Abar[2 * k + 1] = cimag(ab);
    Bbar[2 * k] = creal(bbar); Bbar[2 * k + 1] = cimag(bbar);
  }
}

static double q16(double v, double s) {
  double r = rint(v / s);
  if (r < -32768.0) r = -32768.0;
  if (r > 32767.0) r = 32767.0;
  return s * r;
}

EXPORT void orc_s4d_scan(int64_t B, int64_t L, int64_t H, int64_t N, const double* u,
                         const double* Ah, const double* Bh, const double* Ch, const double* dt,
                         const double* Dskip, const double* state_scale, const double* h0,
                         double* y, double* h_last) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t hh = 0; hh < H; ++hh) {
      double* Abar = malloc(sizeof(double) * 2 * (size_t)N);
      double* Bbar = malloc(sizeof(double) * 2 * (size_t)N);
      double complex* st = malloc(sizeof(double complex) * (size_t)N);
      orc_s4d_zoh(Ah + 2 * hh * N, Bh + 2 * hh * N, dt[hh], N, Abar, Bbar);
      for (int64_t k = 0; k < N; ++k) {
        const double* p = h0 ? h0 + 2 * ((b * H + hh) * N + k) : NULL;
        st[k] = p ? p[0] + I * p[1] : 0.0;
      }
      for (int64_t t = 0; t < L; ++t) {
        double ut = u[(b * H + hh) * L + t];
        double acc = 0.0;
        for (int64_t k = 0; k < N; ++k) {
          double complex ab = Abar[2 * k] + I * Abar[2 * k + 1];
          double complex bb = Bbar[2 * k] + I * Bbar[2 * k + 1];
          double complex c = Ch[2 * (hh * N + k)] + I * Ch[2 * (hh * N + k) + 1];
          st[k] = ab * st[k] + bb * ut;
          if (state_scale)
            st[k] = q16(creal(st[k]), state_scale[hh]) + I * q16(cimag(st[k]), state_scale[hh]);
          acc += creal(c * st[k]);
        }
        y[(b * H + hh) * L + t] = acc + (Dskip ? Dskip[hh] : 0.0) * ut;
      }
      if (h_last)
        for (int64_t k = 0; k < N; ++k) {
          h_last[2 * ((b * H + hh) * N + k)] = creal(st[k]);
          h_last[2 * ((b * H + hh) * N + k) + 1] = cimag(st[k]);
        }
      free(Abar); free(Bbar); free(st);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* [SSD] Mamba2 chunked form (structured state-space duality), fp64.
 * Layouts: xh, y [B, L, nh, P]; delta [B, L, nh]; A, Dskip [nh]; Bh, Ch [B, L, Gbc, N];
 * h0, h_last [B, nh, P, N]. Chunks of Q steps from t = 0, the last may be partial.
 * Per (b, h), state H (P x N) starting at h0, and per chunk with local steps i, j:
 *   cum_i     = sum_{k <= i} delta_k * A_h
 *   Y_intra   = sum_{j <= i} (Ch_i . Bh_j) * exp(cum_i - cum_j) * delta_j * xh_j
 *   Y_inter   = exp(cum_i) * Ch_i . H^T
 *   y_i       = Y_intra + Y_inter + Dskip_h * xh_i
 *   S[p, n]   = sum_j exp(cum_last - cum_j) * delta_j * xh_j[p] * Bh_j[n]          (mode 0)
 *   H         = exp(cum_last) * H + S
 * Mode 1 (int8 chunk state, requantization at a cost-effective point): with
 *   w_j = delta_j * exp(cum_last - cum_j), w_max = max_j w_j,
 *   r[j,p] = clamp(RNE(qx[j,p] * w_j / w_max), -128, 127)  (decided in fp64),
 *   S[p, n] = w_max * sx[p] * sum_j r[j,p] * Bh_j[n].
 * Mode 2 (int8 intra-chunk output, the SSDi8 persistent int8 path through Y_intra; combinable with
 * mode 1): row i of the intra-chunk weights W[i, j] = (Ch_i . Bh_j) exp(cum_i - cum_j) delta_j
 * (j <= i) is requantized with its own scale: m_i = max_j |W[i, j]|,
 *   r[i, j] = clamp(RNE(W[i, j] * 127 / m_i), -127, 127)  (0 when m_i = 0; decided in fp64),
 *   Y_intra[i, p] = (m_i / 127) * sx[p] * sum_j r[i, j] * qx[j, p].
 * Modes 1 and 2 need the x codes (qx [B, L, nh, P]) and per-channel x scales (sx [nh * P]). */
EXPORT void orc_ssd_chunked(int64_t B, int64_t L, int64_t nh, int64_t P, int64_t N, int64_t Gbc,
                            int64_t Q, const double* xh, const double* delta, const double* A,
                            const double* Bh, const double* Ch, const double* Dskip,
                            const double* h0, int32_t mode, const int8_t* qx, const double* sx,
                            double* y, double* h_last) {
  int64_t hpg = nh / Gbc;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < nh; ++h) {
      int64_t g = h / hpg;
      double* Hs = malloc(sizeof(double) * (size_t)(P * N));
      double* S = malloc(sizeof(double) * (size_t)(P * N));
      double* cum = malloc(sizeof(double) * (size_t)Q);
      double* w = malloc(sizeof(double) * (size_t)Q);
      double* G = malloc(sizeof(double) * (size_t)(Q * Q));
      double* wrow = malloc(sizeof(double) * (size_t)Q);
      double* rrow = malloc(sizeof(double) * (size_t)Q);
      for (int64_t k = 0; k < P * N; ++k) Hs[k] = h0 ? h0[(b * nh + h) * P * N + k] : 0.0;
#define XH(t, p) xh[((b * L + (t)) * nh + h) * P + (p)]
#define QX(t, p) qx[((b * L + (t)) * nh + h) * P + (p)]
#define DT(t) delta[(b * L + (t)) * nh + h]
#define BH(t, n) Bh[((b * L + (t)) * Gbc + g) * N + (n)]
#define CH(t, n) Ch[((b * L + (t)) * Gbc + g) * N + (n)]
      for (int64_t t0 = 0; t0 < L; t0 += Q) {
        int64_t q = (L - t0 < Q) ? L - t0 : Q;
        double run = 0.0;
        for (int64_t i = 0; i < q; ++i) { run += DT(t0 + i) * A[h]; cum[i] = run; }
        /* G = Ch Bh^T of this chunk (lower triangle) */
        for (int64_t i = 0; i < q; ++i)
          for (int64_t j = 0; j <= i; ++j) {
            double cb = 0.0;
            for (int64_t n = 0; n < N; ++n) cb += CH(t0 + i, n) * BH(t0 + j, n);
            G[i * Q + j] = cb;
          }
        /* outputs of this chunk use the state entering it */
        for (int64_t i = 0; i < q; ++i) {
          /* mode & 2: the intra-chunk weights W[i, j] = G exp(cum_i - cum_j) delta_j of row i are
           * requantized to int8 with the row's own scale m_i / 127 (m_i = max_j |W[i, j]|), and
           * multiply the x codes: intra = (m_i / 127) sx[p] sum_j r[i, j] qx[j, p] */
          double mi = 0.0;
          if (mode & 2) {
            for (int64_t j = 0; j <= i; ++j) {
              wrow[j] = G[i * Q + j] * exp(cum[i] - cum[j]) * DT(t0 + j);
              if (fabs(wrow[j]) > mi) mi = fabs(wrow[j]);
            }
            for (int64_t j = 0; j <= i; ++j) {
              double r = (mi > 0.0) ? rint(wrow[j] * 127.0 / mi) : 0.0;
              if (r < -127.0) r = -127.0;
              if (r > 127.0) r = 127.0;
              rrow[j] = r;
            }
          }
          for (int64_t p = 0; p < P; ++p) {
            double intra = 0.0;
            if (mode & 2) {
              for (int64_t j = 0; j <= i; ++j) intra += rrow[j] * (double)QX(t0 + j, p);
              intra *= (mi / 127.0) * sx[h * P + p];
            } else {
              for (int64_t j = 0; j <= i; ++j)
                intra += G[i * Q + j] * exp(cum[i] - cum[j]) * DT(t0 + j) * XH(t0 + j, p);
            }
            double inter = 0.0;
            for (int64_t n = 0; n < N; ++n) inter += CH(t0 + i, n) * Hs[p * N + n];
            inter *= exp(cum[i]);
            y[((b * L + t0 + i) * nh + h) * P + p] =
                intra + inter + (Dskip ? Dskip[h] : 0.0) * XH(t0 + i, p);
          }
        }
        /* chunk state and state passing */
        for (int64_t j = 0; j < q; ++j) w[j] = DT(t0 + j) * exp(cum[q - 1] - cum[j]);
        if (!(mode & 1)) {
          for (int64_t p = 0; p < P; ++p)
            for (int64_t n = 0; n < N; ++n) {
              double acc = 0.0;
              for (int64_t j = 0; j < q; ++j) acc += w[j] * XH(t0 + j, p) * BH(t0 + j, n);
              S[p * N + n] = acc;
            }
        } else if (mode & 1) {
          double wmax = 0.0;
          for (int64_t j = 0; j < q; ++j) if (w[j] > wmax) wmax = w[j];
          for (int64_t p = 0; p < P; ++p)
            for (int64_t n = 0; n < N; ++n) {
              double acc = 0.0;
              if (wmax > 0.0)
                for (int64_t j = 0; j < q; ++j) {
                  double r = rint((double)QX(t0 + j, p) * w[j] / wmax);
                  if (r < -128.0) r = -128.0;
                  if (r > 127.0) r = 127.0;
                  acc += r * BH(t0 + j, n);
                }
              S[p * N + n] = wmax * sx[h * P + p] * acc;
            }
        }
        for (int64_t k = 0; k < P * N; ++k) Hs[k] = exp(cum[q - 1]) * Hs[k] + S[k];
      }
      if (h_last)
        for (int64_t k = 0; k < P * N; ++k) h_last[(b * nh + h) * P * N + k] = Hs[k];
#undef XH
#undef QX
#undef DT
#undef BH
#undef CH
      free(Hs); free(S); free(cum); free(w); free(G); free(wrow); free(rrow);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* [Q2] generation stage: one recurrence step per sequence for Mamba2-shaped state, fp64 state.
 *   xh [B, nh, P], Bh, Ch [B, Gbc, N], delta [B, nh], A, Dskip [nh], state [B, nh, P, N] in/out.
 *   state = exp(delta*A_h) * state + delta * xh[p] * Bh[n];  y[p] = sum_n Ch[n] state + D xh[p]. */
EXPORT void orc_decode_step(int64_t B, int64_t nh, int64_t P, int64_t N, int64_t Gbc,
                            const double* xh, const double* Bh, const double* Ch,
                            const double* delta, const double* A, const double* Dskip,
                            double* state, double* y) {
  int64_t hpg = nh / Gbc;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < nh; ++h) {
      int64_t g = h / hpg;
      double dt = delta[b * nh + h];
      double dA = exp(dt * A[h]);
      for (int64_t p = 0; p < P; ++p) {
        double xv = xh[(b * nh + h) * P + p];
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          double* s = &state[((b * nh + h) * P + p) * N + n];
          *s = dA * *s + dt * xv * Bh[(b * Gbc + g) * N + n];
          acc += Ch[(b * Gbc + g) * N + n] * *s;
        }
        y[(b * nh + h) * P + p] = acc + (Dskip ? Dskip[h] : 0.0) * xv;
      }
    }
}

/* Number of OpenMP threads the parallel loops above use (for reporting the baseline's cores). */
/* ------------------------------------------------------------------------------------------ */
/* [Q2] W4A8 linear layer (abstract: W4A8 for large-batch decoding). Reading taken (the page gives
 * only the bit widths): symmetric 4-bit weights with one scale per output channel n and group of
 * `group` consecutive input channels, s = fl32(absmax / 7) (absmax 0 -> 1, clamped into the valid
 * range), codes clamp(RNE(w / s), -8, 7) by the exact quotient; int8 activations with one scale;
 *   y[m, n] = bias[n] + sum_g (sa * sw[n, g]) * sum_{k in g} qa[m, k] * qw[n, k]
 * in fp64 (each inner sum is an exact integer). */
EXPORT float orc_w4_scale_from_absmax(float absmax) {
  if (absmax == 0.0f) return 1.0f;
  float s = absmax / 7.0f;
  if (s < 0x1p-100f) s = 0x1p-100f;
  if (s > 0x1p100f) s = 0x1p100f;
  return s;
}

EXPORT void orc_quant_w4(const float* w, int64_t N, int64_t K, int64_t group, const float* scales,
                         int8_t* q) {
  const int64_t ng = K / group;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      const float s = scales[n * ng + k / group];
      q[n * K + k] = scale_valid((double)s) ? (int8_t)round_sat(w[n * K + k], (double)s, -8, 7) : 0;
    }
}

EXPORT void orc_gemm_w4a8(int64_t M, int64_t N, int64_t K, int64_t group, const int8_t* qa,
                          float sa, const int8_t* qw, const float* sw, const double* bias,
                          double* y) {
  const int64_t ng = K / group;
  const double a_s = scale_valid((double)sa) ? (double)sa : 0.0;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double acc = bias ? bias[n] : 0.0;
      for (int64_t g = 0; g < ng; ++g) {
        int64_t dot = 0;
        for (int64_t k = g * group; k < (g + 1) * group; ++k)
          dot += (int64_t)qa[m * K + k] * (int64_t)qw[n * K + k];
        const double s = scale_valid((double)sw[n * ng + g]) ? (double)sw[n * ng + g] : 0.0;
        acc += (a_s * s) * (double)dot;
      }
      y[m * N + n] = acc;
    }
}

EXPORT int orc_max_threads(void) { return omp_get_max_threads(); }
