// Shared device helpers and host-side error handling of libqssm (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "qssm.h"

namespace qssm {

// ---------------------------------------------------------------------------------------------
// Host: error reporting (thread-local message, never an exception across the ABI).
qssm_status fail(qssm_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
// Maps a pending launch error to QSSM_ERR_DEVICE (with the runtime's message).
qssm_status launch_status(const char* what);

// Ceil division for launch geometry.
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------------------------
// Device: the quantization rule.
//
// q = clamp(RNE(v / s), lo, hi) with v / s the exact rational quotient (Quamba2's 8-bit codes,
// rounding half to even, saturating). The fp32 division is correctly rounded, and rounding is
// monotone, so rint() of the fp32 quotient f differs from the exact RNE only when f itself is a
// half-integer k + 1/2 while the exact quotient is not: then the sign of the exact remainder
// v - f*s, which one fused multiply-add yields without intermediate rounding, decides the side.
// Valid scales lie in [2^-100, 2^100]; there every non-zero remainder is at least 2^-149 in
// magnitude, so its sign survives the final rounding of the fma.
__host__ __device__ __forceinline__ bool scale_ok(float s) { return s >= 0x1p-100f && s <= 0x1p100f; }

__host__ __device__ __forceinline__ int rne_sat(float v, float s, float lo, float hi) {
  float f = v / s;
  float r = rintf(f);
  if (fabsf(f - r) == 0.5f) {
    float rem = fmaf(-f, s, v);
    if (rem > 0.0f) r = f + 0.5f;
    else if (rem < 0.0f) r = f - 0.5f;
  }
  r = fminf(fmaxf(r, lo), hi);
  return (v != v) ? 0 : (int)r;  // NaN encodes as 0
}

__host__ __device__ __forceinline__ int8_t quant8(float v, float s) {
  return scale_ok(s) ? (int8_t)rne_sat(v, s, -128.0f, 127.0f) : (int8_t)0;
}

// The same rule from a reciprocal r = fl32(1/s), for which |v*r - v/s| <= 2^-23 |v/s| + 2^-48 |v/s|
// <= 3.1e-5 when |v/s| <= 256. Let f = v*r clamped to [-256, 256] (beyond that the code saturates
// anyway) and c = rint(f). If |f - c| <= 1/2 - 2^-14, the exact quotient d lies within
// 1/2 - 2^-14 + 3.1e-5 < 1/2 of c and RNE(d) = c. Otherwise d may sit on or beyond the
// half-integer b = c +- 1/2 on f's side of c (d is within 1/2 of f). The exact v - b*s is a multiple of 2^-149 (b is a multiple of 1/2 and s >= 2^-102 in
// every use), so the single rounding of fmaf(-b, s, v) keeps its sign and its zero-ness:
// beyond b moves to the neighbour c +- 1, exactly on b is a tie resolved to the even neighbour.
// The rare near-boundary branch is skipped by a whole wave when none of its lanes needs it.
// Returns the unsaturated code as a float; the caller clamps and handles NaN and invalid scales.
__host__ __device__ __forceinline__ float rne_recip(float v, float s, float r) {
  const float f = fminf(fmaxf(v * r, -256.0f), 256.0f);
  float c = rintf(f);
  const float t = f - c;
  if (fabsf(t) > 0.5f - 0x1p-14f) {
    const float h = copysignf(0.5f, t);
    const float e = fmaf(-(c + h), s, v);
    const float eh = (h > 0.0f) ? e : -e;        // > 0: beyond the boundary on f's side
    const bool odd = (c * 0.5f) != rintf(c * 0.5f);
    if (eh > 0.0f || (eh == 0.0f && odd)) c += h + h;
  }
  return c;
}

__host__ __device__ __forceinline__ int rne_sat_recip(float v, float s, float r, int lo, int hi) {
  const float c = fminf(fmaxf(rne_recip(v, s, r), (float)lo), (float)hi);
  return (v == v) ? (int)c : 0;  // NaN encodes as 0
}

// Reciprocal used with rne_sat_recip; 0 marks a scale outside the valid range (codes 0).
__host__ __device__ __forceinline__ float recip_or_zero(float s) { return scale_ok(s) ? 1.0f / s : 0.0f; }

__host__ __device__ __forceinline__ int8_t quant8_r(float v, float s, float r) {
  return (r != 0.0f) ? (int8_t)rne_sat_recip(v, s, r, -128, 127) : (int8_t)0;
}

// Soft-edge byte (Quamba-SE blog, 2.1 and 2.2): strict |v| < L selects scale/m with a 6-bit
// payload (tag 10), |v| > H selects scale*m (tag 11), anything else (including both tests true)
// the base scale with a 7-bit payload (tag 0). Payloads are two's complement. The mode ratio m is 4
// (sections 2.1-2.2) or 2 (the shift-only form of section 4.1); im = 1/m. r = recip_or_zero(s):
// the small and large modes scale s and r by exact powers of two.
__host__ __device__ __forceinline__ uint8_t softedge_code_r(float v, float s, float r, float L, float H,
                                                            float m, float im) {
  if (r == 0.0f) return 0;
  const float a = fabsf(v);
  const bool small = a < L, large = a > H;
  const bool sm = small && !large, lg = large && !small;
  const float ss = sm ? im * s : (lg ? m * s : s);
  const float rr = sm ? m * r : (lg ? im * r : r);
  const int lim = (sm || lg) ? 32 : 64;
  const int q = rne_sat_recip(v, ss, rr, -lim, lim - 1);
  const uint32_t code = sm ? (0x80u | ((uint32_t)q & 0x3Fu))
                           : (lg ? (0xC0u | ((uint32_t)q & 0x3Fu)) : ((uint32_t)q & 0x7Fu));
  return (uint8_t)code;  // NaN: neither small nor large, payload 0
}

// Value of a soft-edge byte in units of the base scale: the payload times 1, 1/m or m (exact).
__host__ __device__ __forceinline__ float softedge_unit(uint32_t b, float m, float im) {
  if ((b & 0x80u) == 0) return (float)((b & 0x40u) ? (int)(b & 0x7Fu) - 128 : (int)(b & 0x7Fu));
  const int q = (b & 0x20u) ? (int)(b & 0x3Fu) - 64 : (int)(b & 0x3Fu);
  return (float)q * ((b & 0x40u) ? m : im);
}

// Value of a soft-edge byte as one correctly rounded fp32 product (0 for an invalid scale):
// the exact unit times s (m * s and im * s are exact for a valid s, so unit * s rounds once).
__host__ __device__ __forceinline__ float softedge_value(uint32_t b, float s, float m, float im) {
  if (!scale_ok(s)) return 0.0f;
  if ((b & 0x80u) == 0) return softedge_unit(b, m, im) * s;
  const int q = (b & 0x20u) ? (int)(b & 0x3Fu) - 64 : (int)(b & 0x3Fu);
  return (float)q * ((b & 0x40u) ? s * m : s * im);
}

// Mode ratio of a soft-edge code type (QSSM_X_SOFTEDGE: 4, QSSM_X_SOFTEDGE2: 2).
__host__ __device__ __forceinline__ float softedge_ratio(int code_type) {
  return code_type == QSSM_X_SOFTEDGE2 ? 2.0f : 4.0f;
}

// Scale from a group absmax (device side of compute_scales): fl32(absmax / 127), 0 -> 1,
// clamped to the valid range.
__device__ __forceinline__ float scale_from_absmax(float a) {
  if (a == 0.0f) return 1.0f;
  float s = a / 127.0f;
  return fminf(fmaxf(s, 0x1p-100f), 0x1p100f);
}

// |v| if finite, else 0 (absmax ignores NaN and infinities).
__device__ __forceinline__ float finite_abs(float v) {
  float a = fabsf(v);
  return (a <= 3.402823466e38f) ? a : 0.0f;
}

// Wave-uniform value in an SGPR (so loads indexed by it can go through the scalar cache).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace qssm
