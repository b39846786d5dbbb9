// Host-side offline calibration of libqssm (CPU only, no device calls).
//
// Quamba2, method steps 1-2: activation statistics of x collected offline, channels sorted by
// magnitude and clustered into groups that share one scale. Quamba-SE blog, section 4.1: soft-edge
// thresholds L = 5th and H = 99.9th percentile, smoothed by an exponential moving average
// (alpha = 0.1). Built with -ffp-contract=off: the arithmetic below is evaluated exactly as written.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>
#include <numeric>
#include <vector>

#include "common.hpp"

using qssm::fail;

namespace {

float calib_scale(float absmax) {
  if (absmax == 0.0f) return 1.0f;
  float s = absmax / 127.0f;
  if (s < 0x1p-100f) s = 0x1p-100f;
  if (s > 0x1p100f) s = 0x1p100f;
  return s;
}

// Percentile with linear interpolation between order statistics (the "linear" rule:
// virtual index (n-1) q), on ascending values.
double percentile_linear(const std::vector<double>& sorted, double pct) {
  const int64_t n = (int64_t)sorted.size();
  const double q = pct / 100.0;
  const double vi = (double)(n - 1) * q;
  if (vi >= (double)(n - 1)) return sorted[n - 1];
  if (vi < 0.0) return sorted[0];
  const double lo = std::floor(vi);
  const double t = vi - lo;
  const double a = sorted[(int64_t)lo], b = sorted[(int64_t)lo + 1];
  const double diff = b - a;
  if (t >= 0.5) return b - diff * (1.0 - t);
  return a + diff * t;
}

}  // namespace

extern "C" {

qssm_status qssm_calib_channel_absmax(const float* x, int64_t outer, int64_t C, int64_t inner,
                                      float* absmax_out) {
  qssm::clear_error();
  if (outer < 0 || C < 0 || inner < 0) return fail(QSSM_ERR_INVALID_ARG, "negative extent");
  if (!absmax_out || (!x && outer * C * inner > 0))
    return fail(QSSM_ERR_INVALID_ARG, "null pointer");
  for (int64_t c = 0; c < C; ++c) absmax_out[c] = 0.0f;
  for (int64_t o = 0; o < outer; ++o)
    for (int64_t c = 0; c < C; ++c) {
      const float* row = x + (o * C + c) * inner;
      float m = absmax_out[c];
      for (int64_t i = 0; i < inner; ++i) {
        float a = std::fabs(row[i]);
        if (std::isfinite(a) && a > m) m = a;
      }
      absmax_out[c] = m;
    }
  return QSSM_OK;
}

qssm_status qssm_calib_scales(const float* absmax, int64_t n, float* scales) {
  qssm::clear_error();
  if (n < 0) return fail(QSSM_ERR_INVALID_ARG, "negative count");
  if (n > 0 && (!absmax || !scales)) return fail(QSSM_ERR_INVALID_ARG, "null pointer");
  for (int64_t i = 0; i < n; ++i)
    if (!(absmax[i] >= 0.0f) || !std::isfinite(absmax[i]))
      return fail(QSSM_ERR_INVALID_ARG, "absmax[%lld] is negative or not finite", (long long)i);
  for (int64_t i = 0; i < n; ++i) scales[i] = calib_scale(absmax[i]);
  return QSSM_OK;
}

qssm_status qssm_calib_cluster_channels(const float* absmax, int32_t C, int32_t G,
                                        int32_t* perm_out, uint8_t* group_of_out) {
  qssm::clear_error();
  if (C < 1 || G < 1 || G > C || G > 256)
    return fail(QSSM_ERR_INVALID_ARG, "need 1 <= G <= min(C, 256), got C=%d G=%d", C, G);
  if (!absmax || !perm_out || !group_of_out) return fail(QSSM_ERR_INVALID_ARG, "null pointer");
  for (int32_t c = 0; c < C; ++c)
    if (!(absmax[c] >= 0.0f) || !std::isfinite(absmax[c]))
      return fail(QSSM_ERR_INVALID_ARG, "absmax[%d] is negative or not finite", c);

  std::vector<int32_t> order(C);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return absmax[a] < absmax[b]; });

  // Prefix sums of the sorted values and squares (fp64, in sorted order).
  std::vector<double> p1(C + 1, 0.0), p2(C + 1, 0.0);
  for (int32_t k = 0; k < C; ++k) {
    const double v = (double)absmax[order[k]];
    p1[k + 1] = p1[k] + v;
    p2[k + 1] = p2[k] + v * v;
  }
  // best[g][e]: least cost of splitting sorted positions [0, e) into g groups;
  // from[g][e]: start of the last of those groups (first minimum wins).
  const double inf = std::numeric_limits<double>::infinity();
  std::vector<double> best((size_t)(G + 1) * (C + 1), inf);
  std::vector<int32_t> from((size_t)(G + 1) * (C + 1), 0);
  auto B = [&](int g, int e) -> double& { return best[(size_t)g * (C + 1) + e]; };
  auto F = [&](int g, int e) -> int32_t& { return from[(size_t)g * (C + 1) + e]; };
  B(0, 0) = 0.0;
  for (int32_t g = 1; g <= G; ++g)
    for (int32_t e = g; e <= C; ++e)
      for (int32_t s = g - 1; s < e; ++s) {
        if (B(g - 1, s) == inf) continue;
        const double s1 = p1[e] - p1[s], s2 = p2[e] - p2[s];
        const double seg = s2 - s1 * s1 / (double)(e - s);
        const double total = B(g - 1, s) + seg;
        if (total < B(g, e)) { B(g, e) = total; F(g, e) = s; }
      }
  int32_t e = C;
  for (int32_t g = G; g >= 1; --g) {
    const int32_t s = F(g, e);
    for (int32_t k = s; k < e; ++k) group_of_out[k] = (uint8_t)(g - 1);
    e = s;
  }
  for (int32_t k = 0; k < C; ++k) perm_out[k] = order[k];
  return QSSM_OK;
}

qssm_status qssm_calib_softedge(const float* v, int64_t n, double alpha, int32_t ema_valid,
                                double* ema_state, float* s_out, float* L_out, float* H_out) {
  qssm::clear_error();
  if (n < 1) return fail(QSSM_ERR_INVALID_ARG, "need at least one sample");
  if (!v || !ema_state || !s_out || !L_out || !H_out)
    return fail(QSSM_ERR_INVALID_ARG, "null pointer");
  if (!(alpha >= 0.0 && alpha <= 1.0)) return fail(QSSM_ERR_INVALID_ARG, "alpha outside [0, 1]");
  std::vector<double> a(n);
  for (int64_t i = 0; i < n; ++i) {
    if (!std::isfinite(v[i])) return fail(QSSM_ERR_INVALID_ARG, "sample %lld not finite", (long long)i);
    a[i] = std::fabs((double)v[i]);
  }
  std::sort(a.begin(), a.end());
  double l = percentile_linear(a, 5.0);
  double h = percentile_linear(a, 99.9);
  if (ema_valid) {
    l = alpha * l + (1.0 - alpha) * ema_state[0];
    h = alpha * h + (1.0 - alpha) * ema_state[1];
  }
  ema_state[0] = l;
  ema_state[1] = h;
  const float L32 = (float)l, H32 = (float)h;
  *L_out = L32;
  *H_out = H32;
  *s_out = (H32 == 0.0f) ? 1.0f : H32 / 63.0f;
  return QSSM_OK;
}

qssm_status qssm_calib_channel_error_mean(const float* ref, const float* approx, int64_t outer,
                                          int64_t C, int64_t inner, float* mean_out) {
  qssm::clear_error();
  if (outer < 1 || C < 1 || inner < 1) return fail(QSSM_ERR_INVALID_ARG, "bad shape");
  if (!ref || !approx || !mean_out) return fail(QSSM_ERR_INVALID_ARG, "null pointer");
  std::vector<double> sum(C, 0.0);
  for (int64_t o = 0; o < outer; ++o)
    for (int64_t c = 0; c < C; ++c) {
      const int64_t base = (o * C + c) * inner;
      for (int64_t i = 0; i < inner; ++i) {
        const float r = ref[base + i], q = approx[base + i];
        if (!std::isfinite(r) || !std::isfinite(q))
          return fail(QSSM_ERR_INVALID_ARG, "value %lld not finite", (long long)(base + i));
        sum[c] += (double)r - (double)q;
      }
    }
  const double n = (double)outer * (double)inner;
  for (int64_t c = 0; c < C; ++c) mean_out[c] = (float)(sum[c] / n);
  return QSSM_OK;
}

qssm_status qssm_calib_group_absmax(const float* absmax, const uint8_t* group_of, int64_t C,
                                    int32_t G, float* out) {
  qssm::clear_error();
  if (C < 0 || G < 1 || G > 256) return fail(QSSM_ERR_INVALID_ARG, "bad C or G");
  if (!out || (C > 0 && (!absmax || !group_of))) return fail(QSSM_ERR_INVALID_ARG, "null pointer");
  for (int32_t g = 0; g < G; ++g) out[g] = 0.0f;
  for (int64_t c = 0; c < C; ++c) {
    const int g = group_of[c];
    if (g >= G) return fail(QSSM_ERR_INVALID_ARG, "group_of[%lld] = %d is not below G", (long long)c, g);
    if (!(absmax[c] >= 0.0f) || std::isinf(absmax[c]))
      return fail(QSSM_ERR_INVALID_ARG, "absmax[%lld] is not finite and >= 0", (long long)c);
    if (absmax[c] > out[g]) out[g] = absmax[c];
  }
  return QSSM_OK;
}

qssm_status qssm_calib_block_absmax(const float* absmax, int64_t n, int32_t block, float* out) {
  qssm::clear_error();
  if (n < 0 || block < 1 || n % block != 0)
    return fail(QSSM_ERR_INVALID_ARG, "block must divide n");
  if (!out || (n > 0 && !absmax)) return fail(QSSM_ERR_INVALID_ARG, "null pointer");
  for (int64_t k = 0; k < n / block; ++k) {
    float m = 0.0f;
    for (int32_t i = 0; i < block; ++i) {
      const float a = absmax[k * block + i];
      if (!(a >= 0.0f) || std::isinf(a))
        return fail(QSSM_ERR_INVALID_ARG, "absmax[%lld] is not finite and >= 0",
                    (long long)(k * block + i));
      if (a > m) m = a;
    }
    out[k] = m;
  }
  return QSSM_OK;
}

qssm_status qssm_calib_s4d_state_scale(int64_t H, int64_t N, int64_t L, const int8_t* A_re,
                                       const float* A_re_s, const int8_t* B_re,
                                       const float* B_re_s, const int8_t* B_im,
                                       const float* B_im_s, const float* log_dt,
                                       const float* umax, double headroom, float* out) {
  qssm::clear_error();
  if (H < 1 || N < 1 || L < 0) return fail(QSSM_ERR_INVALID_ARG, "bad shape");
  if (!A_re || !A_re_s || !B_re || !B_re_s || !B_im || !B_im_s || !log_dt || !umax || !out)
    return fail(QSSM_ERR_INVALID_ARG, "null pointer");
  if (!(headroom >= 1.0)) return fail(QSSM_ERR_INVALID_ARG, "headroom must be >= 1");
  const double steps = (double)(L > 0 ? L : 1);
  for (int64_t h = 0; h < H; ++h) {
    const double dt = std::exp((double)log_dt[h]);
    double m = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const int64_t i = h * N + n;
      const double are = (double)A_re_s[h] * (double)A_re[i];
      const double bre = (double)B_re_s[h] * (double)B_re[i];
      const double bim = (double)B_im_s[h] * (double)B_im[i];
      // |Bbar| = |exp(dt A) - 1| / |A| |B| <= dt |B| exp(max(0, dt Re A)); |Abar| = exp(dt Re A)
      const double ab = std::exp(dt * are);
      const double bbar = dt * std::sqrt(bre * bre + bim * bim) * (ab > 1.0 ? ab : 1.0);
      // sum over at most L steps of |Abar|^k
      double geo;
      if (ab < 1.0) {
        geo = 1.0 / (1.0 - ab);
        if (geo > steps) geo = steps;
      } else {
        geo = steps * std::pow(ab, steps - 1.0);
      }
      const double bound = bbar * (double)umax[h] * geo;
      if (bound > m) m = bound;
    }
    double s = headroom * m / 32767.0;
    if (!(s >= 0x1p-100)) s = 0x1p-100;
    if (s > 0x1p100) s = 0x1p100;
    out[h] = (float)s;
  }
  return QSSM_OK;
}

qssm_status qssm_quant_w4(const float* w, int64_t N, int64_t K, int32_t group, float* scales,
                          uint8_t* packed) {
  qssm::clear_error();
  if (N < 0 || K < 0 || group < 8 || group % 8 != 0 || K % group != 0)
    return fail(QSSM_ERR_INVALID_ARG, "group must be a multiple of 8 that divides K");
  if ((N * K > 0) && (!w || !scales || !packed)) return fail(QSSM_ERR_INVALID_ARG, "null pointer");
  const int64_t ng = K / group;
  std::vector<int8_t> q((size_t)K);
  for (int64_t n = 0; n < N; ++n) {
    const float* row = w + n * K;
    for (int64_t g = 0; g < ng; ++g) {
      float m = 0.0f;
      for (int64_t k = g * group; k < (g + 1) * group; ++k) {
        const float a = std::fabs(row[k]);
        if (a <= std::numeric_limits<float>::max() && a > m) m = a;
      }
      float s = (m == 0.0f) ? 1.0f : m / 7.0f;
      if (s < 0x1p-100f) s = 0x1p-100f;
      if (s > 0x1p100f) s = 0x1p100f;
      scales[n * ng + g] = s;
      for (int64_t k = g * group; k < (g + 1) * group; ++k)
        q[(size_t)k] = (int8_t)qssm::rne_sat(row[k], s, -8.0f, 7.0f);
    }
    // eight consecutive codes per 4 bytes: byte b = code k0 + b (low nibble), k0 + 4 + b (high)
    uint8_t* out = packed + n * (K / 2);
    for (int64_t k0 = 0; k0 < K; k0 += 8)
      for (int b = 0; b < 4; ++b)
        out[k0 / 2 + b] = (uint8_t)(((uint8_t)q[(size_t)(k0 + b)] & 0x0Fu) |
                                    (((uint8_t)q[(size_t)(k0 + 4 + b)] & 0x0Fu) << 4));
  }
  return QSSM_OK;
}

}  // extern "C"
