// a1-a3: group quantization of x, per-state-group quantization of B/C, soft-edge encode/decode.
//
// Quamba2 (abstract, method steps 1-3): x quantized to int8 with one scale per cluster of sorted
// channels; B and C with one scale per state group. Quamba-SE blog (2.1, 2.2): three-scale byte.
//
// These are HBM-bound elementwise passes (4 bytes in, 1 byte out per element). Each thread handles
// two chunks of 4 consecutive elements a block-width apart (16-byte loads, 4-byte stores, every
// wave instruction one contiguous run). The per-group scales (and soft-edge thresholds) of a launch
// are staged in LDS when they fit.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.hpp"

using namespace qssm;

namespace {

constexpr int kThreads = 256;
constexpr int kMaxLdsGroups = 1024;
constexpr int kDecVec = 16;       // elements per thread of the soft-edge decoder

typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Op { OP_QUANT = 0, OP_ABSMAX = 1, OP_SOFTEDGE = 2 };
// Chunks of 4 elements per thread: two for the int8 quantizer and the absmax pass, four for the
// soft-edge encoder, whose longer per-value arithmetic needs more values in flight per thread
// (measured on the Mamba1-130M x: int8 fastest with two, soft-edge with four).
template <int OP>
constexpr int chunks_of() { return OP == OP_SOFTEDGE ? 4 : 2; }
enum Map { MAP_GROUP = 0, MAP_STATE = 1 };
// Work split: thread t of block x handles chunks k = 0..kChunks-1 of 4 consecutive elements at
// e = x * kBlockElems + (k * kThreads + t) * 4, so that every load and store instruction of a
// wave covers one contiguous run (64 lanes x 16 bytes in, x 4 bytes out).
// ROWS: inner % 4 == 0, a chunk lies in one channel row (one scale).
// CHANNELS: inner == 1, C % 4 == 0, no permutation, the group map 4-byte aligned; a chunk is 4
//           consecutive channels (4 group ids from one 4-byte load; for STATE, gs % 4 == 0 gives
//           one scale per chunk).
// GENERIC: any other shape, element by element.
enum Layout { L_ROWS = 0, L_CHANNELS = 1, L_GENERIC = 2 };

struct Geometry {
  int64_t total, C, inner;
  const int32_t* perm;      // MAP_GROUP only, may be null
  const uint8_t* group_of;  // MAP_GROUP
  int32_t N, gs, ngs;       // MAP_STATE: channel c = g*N + n -> scale g*ngs + n/gs
  int32_t nscales;
  // Advance of (position in row, channel, outer index) between a thread's consecutive chunks,
  // kStride = kThreads * 4 elements apart (set on the host): stride % inner, (stride / inner) % C,
  // stride / inner / C.
  int64_t step_i, step_c, step_o;
  float se_m = 4.0f, se_im = 0.25f;  // soft-edge mode ratio and its reciprocal (exact)
};

constexpr int64_t kStride = (int64_t)kThreads * 4;

// a / b, in 32-bit arithmetic when both fit (the common case), else 64-bit.
__device__ __forceinline__ int64_t div_fast(int64_t a, int64_t b) {
  if (((uint64_t)a | (uint64_t)b) >> 32 == 0) return (int64_t)((uint32_t)a / (uint32_t)b);
  return a / b;
}

template <int MAP>
__device__ __forceinline__ int scale_index(const Geometry& g, int64_t c) {
  if (MAP == MAP_GROUP) return min((int)g.group_of[c], g.nscales - 1);
  const int64_t grp = div_fast(c, g.N), n = c - grp * g.N;
  return (int)(grp * g.ngs + div_fast(n, g.gs));
}

// One chunk: up to 4 values, their scale indices (one when uniform), how many are valid.
template <int MAP, int LAYOUT>
struct Chunk {
  static constexpr bool kUniform = LAYOUT == L_ROWS || (LAYOUT == L_CHANNELS && MAP == MAP_STATE);
  f32x4 v;
  int si[kUniform ? 1 : 4];
  int n;
};

// ROWS and CHANNELS are loaded in phases, so that a thread's loads of all its chunks are in
// flight together instead of one chunk's index load, wait, value load, and so on: first the index
// loads of every chunk (permutation entry, group map entry or word; the channel c of a chunk is
// always in range, so they need no guard), then the value loads, then the group ids are unpacked.

// GENERIC: element by element from e.
template <int MAP, int LAYOUT>
__device__ __forceinline__ void load_chunk(const Geometry& g, const float* __restrict__ x,
                                           int64_t e, Chunk<MAP, LAYOUT>& ch) {
  const int64_t row = div_fast(e, g.inner);
  int64_t i = e - row * g.inner;
  int64_t o = div_fast(row, g.C), c = row - o * g.C;
  ch.n = (int)((g.total - e) < 4 ? (g.total - e) : 4);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    ch.v[k] = 0.0f;
    if (k < ch.n) {
      const int64_t src = (MAP == MAP_GROUP && g.perm) ? g.perm[c] : c;
      ch.v[k] = x[(o * g.C + src) * g.inner + i];
      ch.si[Chunk<MAP, LAYOUT>::kUniform ? 0 : k] = scale_index<MAP>(g, c);
      if (++i == g.inner) { i = 0; if (++c == g.C) { c = 0; ++o; } }
    }
  }
}

template <int OP>
__device__ __forceinline__ uint32_t encode(float v, float2 sr, float2 lh, float m, float im) {
  if (OP == OP_QUANT) return (uint32_t)(uint8_t)quant8_r(v, sr.x, sr.y);
  return softedge_code_r(v, sr.x, sr.y, lh.x, lh.y, m, im);
}

// Four int8 codes (quant8_r of each value, packed little-endian) with one wave-level branch for
// the rare near-boundary correction instead of one per value. Per value the arithmetic is that of
// rne_recip / rne_sat_recip: the clamp of v*r to [-256, 256] is a med3 (the same for non-NaN
// values; a NaN value, or r = 0 for an invalid scale, yields code 0 whatever it computes).
__device__ __forceinline__ uint32_t quant4(f32x4 v, const float (&s)[4], const float (&r)[4]) {
  float c[4], f[4];
  bool any = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = __builtin_amdgcn_fmed3f(v[i] * r[i], -256.0f, 256.0f);
    c[i] = rintf(f[i]);
    any |= fabsf(f[i] - c[i]) > 0.5f - 0x1p-14f;
  }
  if (any) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float t = f[i] - c[i];
      if (fabsf(t) > 0.5f - 0x1p-14f) {
        const float h = copysignf(0.5f, t);
        const float e = fmaf(-(c[i] + h), s[i], v[i]);
        const float eh = (h > 0.0f) ? e : -e;
        const bool odd = (c[i] * 0.5f) != rintf(c[i] * 0.5f);
        if (eh > 0.0f || (eh == 0.0f && odd)) c[i] += h + h;
      }
    }
  }
  int q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qi = (int)__builtin_amdgcn_fmed3f(c[i], -128.0f, 127.0f);
    q[i] = (r[i] != 0.0f && v[i] == v[i]) ? qi : 0;
  }
  // bytes: [q0, q1, 0, 0] and [q2, q3, 0, 0], then the low halves side by side
  const uint32_t lo = __builtin_amdgcn_perm((uint32_t)q[1], (uint32_t)q[0], 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm((uint32_t)q[3], (uint32_t)q[2], 0x0c0c0400u);
  return lo | (hi << 16);
}

// Four soft-edge bytes (softedge_code_r of each value, packed little-endian), with the mode
// classification done first and then the arithmetic of quant4 on the mode's scale and reciprocal
// (exact power-of-two multiples of s and r): one wave-level branch for the rare near-boundary
// correction instead of one per value.
__device__ __forceinline__ uint32_t softedge4(f32x4 v, const float (&s)[4], const float (&r)[4],
                                              const float (&Lt)[4], const float (&Ht)[4], float m,
                                              float im) {
  float f[4], c[4];
  bool sm[4], lg[4];
  bool any = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = fabsf(v[i]);
    const bool small = a < Lt[i], large = a > Ht[i];
    sm[i] = small && !large;
    lg[i] = large && !small;
    // the mode's reciprocal unit; the unit itself is only needed near a rounding boundary
    const float rr = sm[i] ? m * r[i] : (lg[i] ? im * r[i] : r[i]);
    f[i] = __builtin_amdgcn_fmed3f(v[i] * rr, -256.0f, 256.0f);
    c[i] = rintf(f[i]);
    any |= fabsf(f[i] - c[i]) > 0.5f - 0x1p-14f;
  }
  if (any) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float t = f[i] - c[i];
      if (fabsf(t) > 0.5f - 0x1p-14f) {
        const float ss = sm[i] ? im * s[i] : (lg[i] ? m * s[i] : s[i]);
        const float h = copysignf(0.5f, t);
        const float e = fmaf(-(c[i] + h), ss, v[i]);
        const float eh = (h > 0.0f) ? e : -e;
        const bool odd = (c[i] * 0.5f) != rintf(c[i] * 0.5f);
        if (eh > 0.0f || (eh == 0.0f && odd)) c[i] += h + h;
      }
    }
  }
  uint32_t word = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // payload: 7-bit two's complement in [-64, 63] (standard), 6-bit in [-32, 31] under the mode
    // bits 10 (small) or 11 (large); the integer clamp is one med3
    const bool md = sm[i] || lg[i];
    const int lim = md ? 31 : 63;
    const int q = min(max((int)c[i], ~lim), lim);
    const uint32_t b = ((uint32_t)q & (uint32_t)(2 * lim + 1)) | (md ? (lg[i] ? 0xC0u : 0x80u) : 0u);
    word |= ((r[i] != 0.0f && v[i] == v[i]) ? b : 0u) << (8 * i);
  }
  return word;
}

template <int OP, int MAP, int LAYOUT, bool LDS>
__global__ __launch_bounds__(kThreads) void k_elementwise(
    const float* __restrict__ x, Geometry g, const float* __restrict__ scales,
    const float* __restrict__ Lth, const float* __restrict__ Hth, void* __restrict__ out) {
  __shared__ float2 s_sr[OP == OP_ABSMAX || !LDS ? 1 : kMaxLdsGroups];  // (s, 1/s or 0 if invalid)
  __shared__ float2 s_LH[OP == OP_SOFTEDGE && LDS ? kMaxLdsGroups : 1];
  __shared__ unsigned s_max[OP == OP_ABSMAX && LDS ? kMaxLdsGroups : 1];
  constexpr bool lds = LDS;  // the launch picks LDS when g.nscales <= kMaxLdsGroups
  auto scale_of = [&](int si) -> float2 {
    if (lds) return s_sr[si];
    const float sc = scales[si];
    return make_float2(sc, recip_or_zero(sc));
  };
  auto thresholds_of = [&](int si) -> float2 {
    if (OP != OP_SOFTEDGE) return make_float2(0.0f, 0.0f);
    return lds ? s_LH[si] : make_float2(Lth[si], Hth[si]);
  };
  constexpr bool kUniform = Chunk<MAP, LAYOUT>::kUniform;
  constexpr bool kStepped = LAYOUT != L_GENERIC;
  constexpr int kChunks = chunks_of<OP>();
  constexpr int64_t kBlockElems = (int64_t)kThreads * kChunks * 4;
  Chunk<MAP, LAYOUT> ch[kChunks];
  int64_t e[kChunks];
  // position of the thread's first chunk; later chunks step by kStride elements
  int64_t pi = 0, pc = 0, po = 0;
  if (kStepped) {
    const int64_t e0 = (int64_t)blockIdx.x * kBlockElems + (int64_t)threadIdx.x * 4;
    const int64_t row = div_fast(e0, g.inner);
    pi = e0 - row * g.inner;
    po = div_fast(row, g.C);
    pc = row - po * g.C;
  }
  int64_t off[kChunks];    // element offset of each chunk's values
  int64_t src[kChunks];    // ROWS: source channel of each chunk
  uint32_t gidw[kChunks];  // CHANNELS with a group map: the 4 group ids of each chunk
  // index phase, branch-free (the permutation test is hoisted: one copy of the loop per case)
  auto index_phase = [&](auto use_perm) {
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      e[k] = (int64_t)blockIdx.x * kBlockElems + ((int64_t)k * kThreads + threadIdx.x) * 4;
      ch[k].n = 4;
      if (LAYOUT == L_ROWS) {
        src[k] = decltype(use_perm)::value ? (int64_t)g.perm[pc] : pc;
        ch[k].si[0] = scale_index<MAP>(g, pc);
        off[k] = po * g.C * g.inner + pi;  // plus src * inner once the index has arrived
      } else {
        if (MAP == MAP_GROUP) gidw[k] = *reinterpret_cast<const uint32_t*>(g.group_of + pc);
        else ch[k].si[0] = scale_index<MAP>(g, pc);
        off[k] = e[k];
      }
      pi += g.step_i;
      const bool wrap_i = pi >= g.inner;
      pi = wrap_i ? pi - g.inner : pi;
      const int64_t cc = pc + g.step_c + (wrap_i ? 1 : 0);
      const bool wrap_c = cc >= g.C;
      pc = wrap_c ? cc - g.C : cc;
      po += g.step_o + (wrap_c ? 1 : 0);
    }
  };
  if (kStepped) {
    if (LAYOUT == L_ROWS && MAP == MAP_GROUP && g.perm) index_phase(std::true_type{});
    else index_phase(std::false_type{});
  } else {
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      e[k] = (int64_t)blockIdx.x * kBlockElems + ((int64_t)k * kThreads + threadIdx.x) * 4;
      if (e[k] < g.total) load_chunk<MAP, LAYOUT>(g, x, e[k], ch[k]);
    }
  }
  if (kStepped) {
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      if (LAYOUT == L_ROWS) off[k] += src[k] * g.inner;
      if (e[k] < g.total) ch[k].v = *reinterpret_cast<const f32x4*>(x + off[k]);
    }
    if (LAYOUT == L_CHANNELS && MAP == MAP_GROUP) {
#pragma unroll
      for (int k = 0; k < kChunks; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          ch[k].si[j % (Chunk<MAP, LAYOUT>::kUniform ? 1 : 4)] =
              min((int)((gidw[k] >> (8 * j)) & 0xFFu), g.nscales - 1);
    }
  }
  // The per-group scales are staged after the chunk loads are issued, so that the two memory
  // latencies overlap instead of adding up.
  if (lds) {
    for (int k = threadIdx.x; k < g.nscales; k += kThreads) {
      if (OP == OP_ABSMAX) {
        s_max[k] = 0u;
      } else {
        const float sc = scales[k];
        s_sr[k] = make_float2(sc, recip_or_zero(sc));
      }
      if (OP == OP_SOFTEDGE) s_LH[k] = make_float2(Lth[k], Hth[k]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    if (e[k] >= g.total) continue;
    const Chunk<MAP, LAYOUT>& c = ch[k];
    if (OP == OP_ABSMAX) {
      unsigned* gmax = reinterpret_cast<unsigned*>(out);
      auto push = [&](int si, float m) {
        if (m > 0.0f) {
          if (lds) atomicMax(&s_max[si], __float_as_uint(m));
          else atomicMax(gmax + si, __float_as_uint(m));
        }
      };
      if (kUniform) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, finite_abs(c.v[i]));
        push(c.si[0], m);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < c.n) push(c.si[kUniform ? 0 : i], finite_abs(c.v[i]));
      }
    } else if (OP == OP_QUANT && kStepped) {
      float sv[4], rv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 sr = scale_of(c.si[kUniform ? 0 : i]);
        sv[i] = sr.x;
        rv[i] = sr.y;
      }
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(out) + e[k]) = quant4(c.v, sv, rv);
    } else if (OP == OP_SOFTEDGE && kStepped) {
      float sv[4], rv[4], lv[4], hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 sr = scale_of(c.si[kUniform ? 0 : i]);
        const float2 lh = thresholds_of(c.si[kUniform ? 0 : i]);
        sv[i] = sr.x;
        rv[i] = sr.y;
        lv[i] = lh.x;
        hv[i] = lh.y;
      }
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(out) + e[k]) =
          softedge4(c.v, sv, rv, lv, hv, g.se_m, g.se_im);
    } else {
      uint32_t word = 0u;
      if (kUniform) {
        const float2 sr = scale_of(c.si[0]);
        const float2 lh = thresholds_of(c.si[0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) word |= encode<OP>(c.v[i], sr, lh, g.se_m, g.se_im) << (8 * i);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < c.n) {
            const int si = c.si[kUniform ? 0 : i];
            word |= encode<OP>(c.v[i], scale_of(si), thresholds_of(si), g.se_m, g.se_im) << (8 * i);
          }
        }
      }
      uint8_t* o8 = reinterpret_cast<uint8_t*>(out) + e[k];
      if (c.n == 4) {
        *reinterpret_cast<uint32_t*>(o8) = word;
      } else {
        for (int i = 0; i < c.n; ++i) o8[i] = (uint8_t)(word >> (8 * i));
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
    const uint8_t* __restrict__ group_of, int nscales, const float* __restrict__ s, float m,
    float im, float* __restrict__ out) {
  __shared__ float s_scale[256];
  for (int k = threadIdx.x; k < nscales; k += kThreads) s_scale[k] = s[k];
  __syncthreads();
  const int64_t e0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kDecVec;
  if (e0 >= total) return;
  const int64_t row = e0 / inner;
  int64_t i = e0 - row * inner, c = row % C;
  const int n = (int)((total - e0) < kDecVec ? (total - e0) : kDecVec);
  alignas(16) uint8_t b[kDecVec];
  if (n == kDecVec) *reinterpret_cast<uint4*>(b) = *reinterpret_cast<const uint4*>(code + e0);
  else for (int k = 0; k < n; ++k) b[k] = code[e0 + k];
  alignas(16) float v[kDecVec];
#pragma unroll
  for (int k = 0; k < kDecVec; ++k) {
    if (k < n) {
      v[k] = softedge_value(b[k], s_scale[min((int)group_of[c], nscales - 1)], m, im);
      if (++i == inner) { i = 0; if (++c == C) c = 0; }
    }
  }
  if (n == kDecVec) {
#pragma unroll
    for (int k = 0; k < kDecVec / 4; ++k)
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
int choose_layout(const Geometry& g) {
  if (g.inner % 4 == 0) return L_ROWS;
  if (g.inner == 1 && g.C % 4 == 0) {
    if (MAP == MAP_GROUP && !g.perm && (reinterpret_cast<uintptr_t>(g.group_of) % 4) == 0)
      return L_CHANNELS;
    if (MAP == MAP_STATE && g.N % 4 == 0 && g.gs % 4 == 0) return L_CHANNELS;
  }
  return L_GENERIC;
}

template <int OP, int MAP, int LAYOUT>
void launch_elementwise(const float* x, const Geometry& g, const float* scales, const float* L,
                        const float* H, void* out, hipStream_t st) {
  const unsigned blocks = (unsigned)cdiv(g.total, (int64_t)kThreads * chunks_of<OP>() * 4);
  if (g.nscales <= kMaxLdsGroups)
    k_elementwise<OP, MAP, LAYOUT, true><<<blocks, kThreads, 0, st>>>(x, g, scales, L, H, out);
  else
    k_elementwise<OP, MAP, LAYOUT, false><<<blocks, kThreads, 0, st>>>(x, g, scales, L, H, out);
}

template <int OP, int MAP>
void launch_any(int layout, const float* x, const Geometry& g, const float* scales, const float* L,
                const float* H, void* out, hipStream_t st) {
  if (layout == L_ROWS) launch_elementwise<OP, MAP, L_ROWS>(x, g, scales, L, H, out, st);
  else if (layout == L_CHANNELS) launch_elementwise<OP, MAP, L_CHANNELS>(x, g, scales, L, H, out, st);
  else launch_elementwise<OP, MAP, L_GENERIC>(x, g, scales, L, H, out, st);
}

template <int OP, int MAP>
qssm_status launch(const float* x, Geometry g, float* scales, int compute_scales,
                   const float* L, const float* H, void* out, hipStream_t st) {
  const int layout = choose_layout<OP, MAP>(g);
  if (g.inner > 0 && g.C > 0) {
    g.step_i = kStride % g.inner;
    g.step_c = (kStride / g.inner) % g.C;
    g.step_o = kStride / g.inner / g.C;
  }
  if (compute_scales) {
    k_fill_u32<<<(unsigned)cdiv(g.nscales, 256), 256, 0, st>>>(
        reinterpret_cast<unsigned*>(scales), g.nscales, 0u);
    if (g.total > 0) launch_any<OP_ABSMAX, MAP>(layout, x, g, nullptr, nullptr, nullptr, scales, st);
    k_finalize_scales<<<(unsigned)cdiv(g.nscales, 256), 256, 0, st>>>(scales, g.nscales);
  }
  if (g.total > 0) launch_any<OP, MAP>(layout, x, g, scales, L, H, out, st);
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
                                 const float* s, const float* L, const float* H, int32_t form,
                                 uint8_t* code, hipStream_t stream) {
  clear_error();
  if (form != QSSM_X_SOFTEDGE && form != QSSM_X_SOFTEDGE2)
    return fail(QSSM_ERR_INVALID_ARG, "form must be QSSM_X_SOFTEDGE or QSSM_X_SOFTEDGE2");
  if (qssm_status st = check_extents(outer, C, inner)) return st;
  if (G < 1 || G > 256) return fail(QSSM_ERR_INVALID_ARG, "G must be in 1..256, got %d", G);
  const int64_t total = outer * C * inner;
  if (!s || !L || !H) return fail(QSSM_ERR_INVALID_ARG, "null scale or threshold pointer");
  if (total > 0 && (!x || !code || !group_of))
    return fail(QSSM_ERR_INVALID_ARG, "null tensor pointer");
  Geometry g{total, C, inner, perm, group_of, 1, 1, 1, G};
  g.se_m = softedge_ratio(form);
  g.se_im = 1.0f / g.se_m;
  return launch<OP_SOFTEDGE, MAP_GROUP>(x, g, const_cast<float*>(s), 0, L, H, code, stream);
}

qssm_status qssm_softedge_decode(const uint8_t* code, int64_t outer, int64_t C, int64_t inner,
                                 const uint8_t* group_of, int32_t G, const float* s, int32_t form,
                                 float* out, hipStream_t stream) {
  clear_error();
  if (form != QSSM_X_SOFTEDGE && form != QSSM_X_SOFTEDGE2)
    return fail(QSSM_ERR_INVALID_ARG, "form must be QSSM_X_SOFTEDGE or QSSM_X_SOFTEDGE2");
  if (qssm_status st = check_extents(outer, C, inner)) return st;
  if (G < 1 || G > 256) return fail(QSSM_ERR_INVALID_ARG, "G must be in 1..256, got %d", G);
  const int64_t total = outer * C * inner;
  if (!s) return fail(QSSM_ERR_INVALID_ARG, "null scale pointer");
  if (total > 0 && (!code || !out || !group_of))
    return fail(QSSM_ERR_INVALID_ARG, "null tensor pointer");
  if (total > 0)
    k_softedge_decode<<<(unsigned)cdiv(total, (int64_t)kThreads * kDecVec), kThreads, 0, stream>>>(
        code, total, C, inner, group_of, G, s, softedge_ratio(form), 1.0f / softedge_ratio(form),
        out);
  return launch_status("softedge_decode");
}

}  // extern "C"
