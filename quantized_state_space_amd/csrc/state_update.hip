// a14: fused decode state update (generation stage), Mamba2-shaped.
//
// Quamba2, abstract: W8A8 generation for the Mamba2 backbone. One token per sequence: x, B and C
// are quantized with static scales (the a1/a2 rule), then for every state element of head h
//     state = exp(delta A_h) state + delta xh[p] Bh[n],    y[p] = sum_n Ch[n] state + D_h xh[p]
//
// The state (P x N per (b, h), fp32 or fp16) is the only large operand: the kernel is one
// streaming read-modify-write pass over it. A workgroup owns one (b, h) state tile: it quantizes
// and dequantizes the P x values and the N B/C values of its group into LDS once, then each thread
// updates 4 (fp32) or 8 (fp16) consecutive states per 16-byte access with fully coalesced wave
// accesses, and the readout sum over n is a shuffle reduction among the lanes sharing a row.
#include <hip/hip_runtime.h>

#include "common.hpp"

using namespace qssm;

namespace {

constexpr int kThreads = 256;

struct UpdParams {
  int64_t B, nh, P, N;
  int32_t Gbc, hpg, gs, G;
  const float* x;
  const uint8_t* x_group_of;
  const float* x_scales;
  const float* Bm;
  const float* Cm;
  const float* B_scales;
  const float* C_scales;
  const float* delta;
  const float* A;
  const float* Dskip;
  void* state;
  void* y;
  int8_t* xq_out;
  int8_t* Bq_out;
  int8_t* Cq_out;
  int32_t yi8, Gy;            // int8 output, number of output groups
  const uint8_t* y_group_of;  // int8 output: [nh * P]
  const float* y_scales;      // int8 output: [Gy]
  const float* y_bias;        // int8 output: [nh * P] or NULL
};

// CH consecutive states per thread access: 4 for fp32 (16 bytes), 8 for fp16 (16 bytes).
// R = N / CH lanes share one state row.
template <int F16, int R>
__global__ __launch_bounds__(kThreads) void k_state_update(UpdParams p) {
  constexpr int CH = F16 ? 8 : 4;
  extern __shared__ float smem[];
  float* xs = smem;                    // [P], padded to a multiple of 4
  float* bs = xs + ((p.P + 3) & ~3);   // [N], 16-byte aligned (N % 4 == 0)
  float* cs = bs + p.N;                // [N]

  const int64_t bh = blockIdx.x;  // b * nh + h
  const int64_t b = bh / p.nh, h = bh % p.nh;
  const int64_t g = h / p.hpg;
  const int ngs = (int)(p.N / p.gs);
  const bool write_bc = (h % p.hpg) == 0;  // one head per group publishes the B/C codes

  for (int64_t k = threadIdx.x; k < p.P; k += kThreads) {
    const int64_t i = bh * p.P + k;
    const float s = p.x_scales[min((int)p.x_group_of[h * p.P + k], p.G - 1)];
    const int8_t q = quant8(p.x[i], s);
    if (p.xq_out) p.xq_out[i] = q;
    xs[k] = scale_ok(s) ? (float)q * s : 0.0f;
  }
  for (int64_t n = threadIdx.x; n < p.N; n += kThreads) {
    const int64_t i = (b * p.Gbc + g) * p.N + n;
    const float sb = p.B_scales[g * ngs + n / p.gs];
    const float sc = p.C_scales[g * ngs + n / p.gs];
    const int8_t qb = quant8(p.Bm[i], sb), qc = quant8(p.Cm[i], sc);
    if (write_bc) {
      if (p.Bq_out) p.Bq_out[i] = qb;
      if (p.Cq_out) p.Cq_out[i] = qc;
    }
    bs[n] = scale_ok(sb) ? (float)qb * sb : 0.0f;
    cs[n] = scale_ok(sc) ? (float)qc * sc : 0.0f;
  }
  __syncthreads();

  const float dt = p.delta[bh];
  const float dA = expf(dt * p.A[h]);
  const float Dh = p.Dskip ? p.Dskip[h] : 0.0f;
  const int64_t nch = p.N / CH;
  const int64_t total = p.P * nch;  // CH-element chunks of the tile
  const int lane = threadIdx.x & 63;

  for (int64_t base = 0; base < total; base += kThreads) {
    const int64_t f = base + threadIdx.x;
    const bool on = f < total;
    const int64_t row = on ? f / nch : 0;
    const int64_t n0 = on ? (f - row * nch) * CH : 0;
    float s[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) s[k] = 0.0f;
    uint4 raw = make_uint4(0u, 0u, 0u, 0u);
    if (on) raw = reinterpret_cast<const uint4*>(p.state)[bh * total + f];
    if (F16) {
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const __half2 v = *reinterpret_cast<const __half2*>(&w[k]);
        s[2 * k] = __low2float(v);
        s[2 * k + 1] = __high2float(v);
      }
    } else {
      s[0] = __uint_as_float(raw.x); s[1] = __uint_as_float(raw.y);
      s[2] = __uint_as_float(raw.z); s[3] = __uint_as_float(raw.w);
    }
    const float dtx = dt * xs[row];
    // B and C of the CH states in 16-byte LDS reads (n0 and the N-float arrays are 4-aligned)
    float bv[CH], cv[CH];
#pragma unroll
    for (int k4 = 0; k4 < CH / 4; ++k4) {
      const float4 b4 = *reinterpret_cast<const float4*>(bs + n0 + 4 * k4);
      const float4 c4 = *reinterpret_cast<const float4*>(cs + n0 + 4 * k4);
      bv[4 * k4] = b4.x; bv[4 * k4 + 1] = b4.y; bv[4 * k4 + 2] = b4.z; bv[4 * k4 + 3] = b4.w;
      cv[4 * k4] = c4.x; cv[4 * k4 + 1] = c4.y; cv[4 * k4 + 2] = c4.z; cv[4 * k4 + 3] = c4.w;
    }
    float yp = 0.0f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      s[k] = fmaf(dA, s[k], dtx * bv[k]);
      yp = fmaf(cv[k], s[k], yp);
    }
    if (on) {
      uint4 out;
      if (F16) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const __half2 v = __floats2half2_rn(s[2 * k], s[2 * k + 1]);
          w[k] = *reinterpret_cast<const uint32_t*>(&v);
        }
        out = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        out = make_uint4(__float_as_uint(s[0]), __float_as_uint(s[1]), __float_as_uint(s[2]),
                         __float_as_uint(s[3]));
      }
      reinterpret_cast<uint4*>(p.state)[bh * total + f] = out;
    }
    // rows occupy R consecutive lanes (R divides 64 and kThreads): reduce within them
#pragma unroll
    for (int off = R / 2; off > 0; off >>= 1) yp += __shfl_xor(yp, off, 64);
    if (on && (lane % R) == 0) {
      const float yv = fmaf(Dh, xs[row], yp);
      if (p.yi8) {
        // persistent int8 output: fl32(y + correction term), the exact rule with the channel's
        // static output scale
        const int64_t ch = h * p.P + row;
        const float sy = p.y_scales[min((int)p.y_group_of[ch], p.Gy - 1)];
        const float yb = p.y_bias ? p.y_bias[ch] : 0.0f;
        reinterpret_cast<int8_t*>(p.y)[bh * p.P + row] = quant8_r(yv + yb, sy, recip_or_zero(sy));
      } else {
        reinterpret_cast<float*>(p.y)[bh * p.P + row] = yv;
      }
    }
  }
}

template <int R>
qssm_status launch_r(const UpdParams& p, int f16, hipStream_t st) {
  const size_t smem = (size_t)(((p.P + 3) & ~3) + 2 * p.N) * sizeof(float);
  const unsigned grid = (unsigned)(p.B * p.nh);
  if (f16) {
    if constexpr (R % 2 == 0) k_state_update<1, R / 2><<<grid, kThreads, smem, st>>>(p);
  } else {
    k_state_update<0, R><<<grid, kThreads, smem, st>>>(p);
  }
  return launch_status("state_update");
}

}  // namespace

extern "C" qssm_status qssm_state_update(const qssm_update_args* a, hipStream_t stream) {
  clear_error();
  if (!a) return fail(QSSM_ERR_INVALID_ARG, "args is null");
  const int64_t B = a->batch, nh = a->nheads, P = a->headdim, N = a->dstate;
  if (B < 0 || nh < 1 || P < 1 || N < 1) return fail(QSSM_ERR_INVALID_ARG, "bad shape");
  if (a->ngroups < 1 || nh % a->ngroups != 0)
    return fail(QSSM_ERR_INVALID_ARG, "ngroups must divide nheads");
  if (a->bc_group_size < 1 || N % a->bc_group_size != 0)
    return fail(QSSM_ERR_INVALID_ARG, "bc_group_size must divide dstate");
  if (a->x_groups < 1 || a->x_groups > 256) return fail(QSSM_ERR_INVALID_ARG, "x_groups not in 1..256");
  if (a->state_dtype != QSSM_F32 && a->state_dtype != QSSM_F16)
    return fail(QSSM_ERR_INVALID_ARG, "state_dtype must be QSSM_F32 or QSSM_F16");
  if (a->y_dtype != QSSM_F32 && a->y_dtype != QSSM_I8)
    return fail(QSSM_ERR_INVALID_ARG, "y_dtype must be QSSM_F32 or QSSM_I8");
  if (a->y_dtype == QSSM_I8) {
    if (a->y_groups < 1 || a->y_groups > 256)
      return fail(QSSM_ERR_INVALID_ARG, "y_groups not in 1..256");
    if (!a->y_group_of || !a->y_scales)
      return fail(QSSM_ERR_INVALID_ARG, "QSSM_I8 output needs y_group_of and y_scales");
  }
  const int64_t R = N / 4;
  if (N % 4 != 0 || !(R == 1 || R == 2 || R == 4 || R == 8 || R == 16 || R == 32 || R == 64))
    return fail(QSSM_ERR_UNSUPPORTED, "dstate must be 4 * 2^k with 4 <= dstate <= 256");
  if (a->state_dtype == QSSM_F16 && N < 8)
    return fail(QSSM_ERR_UNSUPPORTED, "an fp16 state needs dstate >= 8");
  if ((((P + 3) & ~3) + 2 * N) * 4 > 64 * 1024) return fail(QSSM_ERR_UNSUPPORTED, "headdim too large");
  if (B == 0) return QSSM_OK;
  if (!a->x || !a->x_group_of || !a->x_scales || !a->B || !a->C || !a->B_scales || !a->C_scales ||
      !a->delta || !a->A || !a->state || !a->y)
    return fail(QSSM_ERR_INVALID_ARG, "null required pointer");
  if ((uintptr_t)a->state % 16 != 0) return fail(QSSM_ERR_INVALID_ARG, "state must be 16-byte aligned");
  if (B * nh > 0x7fffffffLL) return fail(QSSM_ERR_INVALID_ARG, "batch * nheads too large");
  UpdParams p{B, nh, P, N, a->ngroups, (int32_t)(nh / a->ngroups), a->bc_group_size, a->x_groups, a->x,
              a->x_group_of, a->x_scales, a->B, a->C, a->B_scales, a->C_scales, a->delta, a->A,
              a->Dskip, a->state, a->y, a->xq_out, a->Bq_out, a->Cq_out,
              a->y_dtype == QSSM_I8, a->y_dtype == QSSM_I8 ? a->y_groups : 1, a->y_group_of,
              a->y_scales, a->y_bias};
  const int f16 = a->state_dtype == QSSM_F16;
  switch (R) {
    case 1: return launch_r<1>(p, f16, stream);
    case 2: return launch_r<2>(p, f16, stream);
    case 4: return launch_r<4>(p, f16, stream);
    case 8: return launch_r<8>(p, f16, stream);
    case 16: return launch_r<16>(p, f16, stream);
    case 32: return launch_r<32>(p, f16, stream);
    default: return launch_r<64>(p, f16, stream);
  }
}
