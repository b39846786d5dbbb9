// a1-a3: group quantization of x, per-state-group quantization of B/C, soft-edge encode/decode.
//
// Quamba2 (abstract, method steps 1-3): x quantized to int8 with one scale per cluster of sorted
// channels; B and C with one scale per state group. Quamba-SE blog (2.1, 2.2): three-scale byte.
//
// These are HBM-bound elementwise passes (4 bytes in, 1 byte out per element). Each thread handles
// 16 consecutive output elements: one 16-byte store and, whenever the source run is contiguous,
// four 16-byte loads. The per-group scales (and soft-edge thresholds) of a launch are staged in LDS.
#include <hip/hip_runtime.h>

#include "common.hpp"

using namespace qssm;

namespace {

constexpr int kThreads = 256;
constexpr int kVec = 16;          // elements per thread
constexpr int kMaxLdsGroups = 1024;

enum Op { OP_QUANT = 0, OP_ABSMAX = 1, OP_SOFTEDGE = 2 };
enum Map { MAP_GROUP = 0, MAP_STATE = 1 };

struct Geometry {
  int64_t total, C, inner;
  const int32_t* perm;      // MAP_GROUP only, may be null
  const uint8_t* group_of;  // MAP_GROUP
  int32_t N, gs, ngs;       // MAP_STATE: channel c = g*N + n -> scale g*ngs + n/gs
  int32_t nscales;
};

template <int MAP>
__device__ __forceinline__ int scale_index(const Geometry& g, int64_t c) {
  if (MAP == MAP_GROUP) return g.group_of[c];
  int64_t grp = c / g.N, n = c - grp * g.N;
  return (int)(grp * g.ngs + n / g.gs);
}

// Visits the kVec elements of one thread: calls f(k, value, scale_index) for each valid one.
template <int MAP, typename F>
__device__ __forceinline__ int visit(const Geometry& g, const float* __restrict__ x, int64_t e0,
                                     F&& f) {
  const int64_t row = e0 / g.inner;
  int64_t i = e0 - row * g.inner;
  int64_t c = row % g.C, o = row / g.C;
  const int nvalid = (int)((g.total - e0) < kVec ? (g.total - e0) : kVec);
  if (g.inner % kVec == 0) {
    // all elements share one channel row
    const int64_t src = (MAP == MAP_GROUP && g.perm) ? g.perm[c] : c;
    const int si = scale_index<MAP>(g, c);
    const float4* p = reinterpret_cast<const float4*>(x + (o * g.C + src) * g.inner + i);
#pragma unroll
    for (int k = 0; k < kVec / 4; ++k) {
      float4 v = p[k];
      f(4 * k + 0, v.x, si);
      f(4 * k + 1, v.y, si);
      f(4 * k + 2, v.z, si);
      f(4 * k + 3, v.w, si);
    }
    return kVec;
  }
  const bool contiguous = !(MAP == MAP_GROUP && g.perm) && nvalid == kVec;
  float v[kVec];
  if (contiguous) {
    const float4* p = reinterpret_cast<const float4*>(x + e0);
#pragma unroll
    for (int k = 0; k < kVec / 4; ++k) {
      float4 t = p[k];
      v[4 * k] = t.x; v[4 * k + 1] = t.y; v[4 * k + 2] = t.z; v[4 * k + 3] = t.w;
    }
  }
#pragma unroll
  for (int k = 0; k < kVec; ++k) {
    if (k < nvalid) {
      float val;
      if (contiguous) {
        val = v[k];
      } else {
        const int64_t src = (MAP == MAP_GROUP && g.perm) ? g.perm[c] : c;
        val = x[(o * g.C + src) * g.inner + i];
      }
      f(k, val, scale_index<MAP>(g, c));
      if (++i == g.inner) { i = 0; if (++c == g.C) { c = 0; ++o; } }
    }
  }
  return nvalid;
}

template <int OP, int MAP>
__global__ __launch_bounds__(kThreads) void k_elementwise(
    const float* __restrict__ x, Geometry g, const float* __restrict__ scales,
    const float* __restrict__ Lth, const float* __restrict__ Hth, void* __restrict__ out) {
  __shared__ float s_scale[kMaxLdsGroups];
  __shared__ float s_L[OP == OP_SOFTEDGE ? kMaxLdsGroups : 1];
  __shared__ float s_H[OP == OP_SOFTEDGE ? kMaxLdsGroups : 1];
  __shared__ unsigned s_max[OP == OP_ABSMAX ? kMaxLdsGroups : 1];
  const bool lds = g.nscales <= kMaxLdsGroups;
  if (lds) {
    for (int k = threadIdx.x; k < g.nscales; k += kThreads) {
      if (OP == OP_ABSMAX) s_max[k] = 0u;
      else s_scale[k] = scales[k];
      if (OP == OP_SOFTEDGE) { s_L[k] = Lth[k]; s_H[k] = Hth[k]; }
    }
    __syncthreads();
  }
  const int64_t e0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kVec;
  if (e0 < g.total) {
    if (OP == OP_ABSMAX) {
      // running max per scale index; consecutive elements usually share it
      int cur = -1;
      float m = 0.0f;
      auto flush = [&]() {
        if (cur >= 0 && m > 0.0f) {
          if (lds) atomicMax(&s_max[cur], __float_as_uint(m));
          else atomicMax(reinterpret_cast<unsigned*>(out) + cur, __float_as_uint(m));
        }
      };
      visit<MAP>(g, x, e0, [&](int, float v, int si) {
        if (si != cur) { flush(); cur = si; m = 0.0f; }
        m = fmaxf(m, finite_abs(v));
      });
      flush();
    } else {
      alignas(16) uint8_t res[kVec];
      const int n = visit<MAP>(g, x, e0, [&](int k, float v, int si) {
        const float s = lds ? s_scale[si] : scales[si];
        if (OP == OP_QUANT) {
          res[k] = (uint8_t)quant8(v, s);
        } else {
          const float L = lds ? s_L[si] : Lth[si];
          const float H = lds ? s_H[si] : Hth[si];
          res[k] = softedge_code(v, s, L, H);
        }
      });
      uint8_t* o8 = reinterpret_cast<uint8_t*>(out) + e0;
      if (n == kVec) {
        *reinterpret_cast<uint4*>(o8) = *reinterpret_cast<const uint4*>(res);
      } else {
        for (int k = 0; k < n; ++k) o8[k] = res[k];
      }
    }
  }
  if (OP == OP_ABSMAX && lds) {
    __syncthreads();
    unsigned* gmax = reinterpret_cast<unsigned*>(out);
    for (int k = threadIdx.x; k < g.nscales; k += kThreads)
      if (s_max[k]) atomicMax(gmax + k, s_max[k]);
  }
}

__global__ void k_fill_u32(unsigned* p, int n, unsigned v) {
  int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n) p[k] = v;
}

// scales hold absmax bit patterns on entry (non-negative floats order like their bits).
__global__ void k_finalize_scales(float* scales, int n) {
  int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n) scales[k] = scale_from_absmax(scales[k]);
}

__global__ __launch_bounds__(kThreads) void k_softedge_decode(
    const uint8_t* __restrict__ code, int64_t total, int64_t C, int64_t inner,
    const uint8_t* __restrict__ group_of, int nscales, const float* __restrict__ s,
    float* __restrict__ out) {
  __shared__ float s_scale[256];
  for (int k = threadIdx.x; k < nscales; k += kThreads) s_scale[k] = s[k];
  __syncthreads();
  const int64_t e0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kVec;
  if (e0 >= total) return;
  const int64_t row = e0 / inner;
  int64_t i = e0 - row * inner, c = row % C;
  const int n = (int)((total - e0) < kVec ? (total - e0) : kVec);
  alignas(16) uint8_t b[kVec];
  if (n == kVec) *reinterpret_cast<uint4*>(b) = *reinterpret_cast<const uint4*>(code + e0);
  else for (int k = 0; k < n; ++k) b[k] = code[e0 + k];
  alignas(16) float v[kVec];
#pragma unroll
  for (int k = 0; k < kVec; ++k) {
    if (k < n) {
      v[k] = softedge_value(b[k], s_scale[group_of[c]]);
      if (++i == inner) { i = 0; if (++c == C) c = 0; }
    }
  }
  if (n == kVec) {
#pragma unroll
    for (int k = 0; k < kVec / 4; ++k)
      reinterpret_cast<float4*>(out + e0)[k] = reinterpret_cast<const float4*>(v)[k];
  } else {
    for (int k = 0; k < n; ++k) out[e0 + k] = v[k];
  }
}

qssm_status check_extents(int64_t outer, int64_t C, int64_t inner) {
  if (outer < 0 || C < 0 || inner < 0) return fail(QSSM_ERR_INVALID_ARG, "negative extent");
  if (outer > 0 && inner > 0 && C > 0 && outer > INT64_MAX / C / inner)
    return fail(QSSM_ERR_INVALID_ARG, "tensor too large");
  return QSSM_OK;
}

template <int OP, int MAP>
qssm_status launch(const float* x, const Geometry& g, float* scales, int compute_scales,
                   const float* L, const float* H, void* out, hipStream_t st) {
  if (compute_scales) {
    k_fill_u32<<<(unsigned)cdiv(g.nscales, 256), 256, 0, st>>>(
        reinterpret_cast<unsigned*>(scales), g.nscales, 0u);
    if (g.total > 0)
      k_elementwise<OP_ABSMAX, MAP><<<(unsigned)cdiv(g.total, (int64_t)kThreads * kVec), kThreads,
                                      0, st>>>(x, g, nullptr, nullptr, nullptr, scales);
    k_finalize_scales<<<(unsigned)cdiv(g.nscales, 256), 256, 0, st>>>(scales, g.nscales);
  }
  if (g.total > 0)
    k_elementwise<OP, MAP><<<(unsigned)cdiv(g.total, (int64_t)kThreads * kVec), kThreads, 0,
                             st>>>(x, g, scales, L, H, out);
  return launch_status("quantize");
}

}  // namespace

extern "C" {

qssm_status qssm_quant_group_x(const float* x, int64_t outer, int64_t C, int64_t inner,
                               const int32_t* perm, const uint8_t* group_of, int32_t G,
                               float* scales, int32_t compute_scales, int8_t* q,
                               hipStream_t stream) {
  clear_error();
  if (qssm_status s = check_extents(outer, C, inner)) return s;
  if (G < 1 || G > 256) return fail(QSSM_ERR_INVALID_ARG, "G must be in 1..256, got %d", G);
  const int64_t total = outer * C * inner;
  if (!scales) return fail(QSSM_ERR_INVALID_ARG, "scales is null");
  if (total > 0 && (!x || !q || !group_of)) return fail(QSSM_ERR_INVALID_ARG, "null tensor pointer");
  if (total / (outer ? outer : 1) / (inner ? inner : 1) > (int64_t)1 << 31)
    return fail(QSSM_ERR_INVALID_ARG, "too many channels");
  Geometry g{total, C, inner, perm, group_of, 1, 1, 1, G};
  return launch<OP_QUANT, MAP_GROUP>(x, g, scales, compute_scales, nullptr, nullptr, q, stream);
}

qssm_status qssm_quant_state_group_BC(const float* bc, int64_t outer, int32_t Gbc, int32_t N,
                                      int64_t inner, int32_t gs, float* scales,
                                      int32_t compute_scales, int8_t* q, hipStream_t stream) {
  clear_error();
  if (Gbc < 1 || N < 1) return fail(QSSM_ERR_INVALID_ARG, "Gbc and N must be positive");
  if (qssm_status s = check_extents(outer, (int64_t)Gbc * N, inner)) return s;
  if (gs < 1 || N % gs != 0)
    return fail(QSSM_ERR_INVALID_ARG, "state group size %d must divide N=%d", gs, N);
  const int64_t total = outer * Gbc * N * inner;
  if (!scales) return fail(QSSM_ERR_INVALID_ARG, "scales is null");
  if (total > 0 && (!bc || !q)) return fail(QSSM_ERR_INVALID_ARG, "null tensor pointer");
  const int64_t nscales = (int64_t)Gbc * (N / gs);
  if (nscales > (1 << 24)) return fail(QSSM_ERR_INVALID_ARG, "too many state groups");
  Geometry g{total, (int64_t)Gbc * N, inner, nullptr, nullptr, N, gs, N / gs, (int32_t)nscales};
  return launch<OP_QUANT, MAP_STATE>(bc, g, scales, compute_scales, nullptr, nullptr, q, stream);
}

qssm_status qssm_softedge_encode(const float* x, int64_t outer, int64_t C, int64_t inner,
                                 const int32_t* perm, const uint8_t* group_of, int32_t G,
                                 const float* s, const float* L, const float* H, uint8_t* code,
                                 hipStream_t stream) {
  clear_error();
  if (qssm_status st = check_extents(outer, C, inner)) return st;
  if (G < 1 || G > 256) return fail(QSSM_ERR_INVALID_ARG, "G must be in 1..256, got %d", G);
  const int64_t total = outer * C * inner;
  if (!s || !L || !H) return fail(QSSM_ERR_INVALID_ARG, "null scale or threshold pointer");
  if (total > 0 && (!x || !code || !group_of))
    return fail(QSSM_ERR_INVALID_ARG, "null tensor pointer");
  Geometry g{total, C, inner, perm, group_of, 1, 1, 1, G};
  return launch<OP_SOFTEDGE, MAP_GROUP>(x, g, const_cast<float*>(s), 0, L, H, code, stream);
}

qssm_status qssm_softedge_decode(const uint8_t* code, int64_t outer, int64_t C, int64_t inner,
                                 const uint8_t* group_of, int32_t G, const float* s, float* out,
                                 hipStream_t stream) {
  clear_error();
  if (qssm_status st = check_extents(outer, C, inner)) return st;
  if (G < 1 || G > 256) return fail(QSSM_ERR_INVALID_ARG, "G must be in 1..256, got %d", G);
  const int64_t total = outer * C * inner;
  if (!s) return fail(QSSM_ERR_INVALID_ARG, "null scale pointer");
  if (total > 0 && (!code || !out || !group_of))
    return fail(QSSM_ERR_INVALID_ARG, "null tensor pointer");
  if (total > 0)
    k_softedge_decode<<<(unsigned)cdiv(total, (int64_t)kThreads * kVec), kThreads, 0, stream>>>(
        code, total, C, inner, group_of, G, s, out);
  return launch_status("softedge_decode");
}

}  // extern "C"
