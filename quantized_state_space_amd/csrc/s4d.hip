// a5-a7, S4D form: diagonal LTI scan with int8 parameters and input, fp32 or int16 state.
//
// "Quantizing Small-Scale State-Space Models for Edge AI", abstract: an S4D layer with quantized
// parameters and activations, where A and the internal state are the sensitive parts and components
// may use different precisions. Per channel h and complex state n:
//   Abar = exp(dt Ah), Bbar = (Abar - 1)/Ah Bh (zero-order hold), h_t = Abar h_{t-1} + Bbar u_t,
//   y_t = Re(sum_n Ch h_t) + D u_t.
//
// Mapping: one wave per (batch, channel) chain set, lane = state n (N <= 64 * NPL). The input code
// of each step is the same for every lane: per block of 64 steps, lane t converts code t once and
// the step loop reads it from LDS. Each lane keeps its complex state, Abar, Bbar, C in registers
// (computed once in the prologue, with expm1 for Abar - 1 to keep small dt accurate); the input
// scale is folded into Bbar. With an fp32 state the chain runs on g = h / Bbar' (one complex
// multiply-add per step, no input product), converted back for h_last. The readout sum over states
// is a transpose through LDS: lane n writes its term for 64 steps, then lane t sums row t.
#include <hip/hip_runtime.h>

#include "common.hpp"

using namespace qssm;

namespace {

constexpr int kBlk = 64;  // time steps per readout block
constexpr int kRed = kBlk + 4;  // padded row of the readout transpose (16-byte rows, no conflicts)

struct S4dParams {
  int64_t B, L, H, N;
  const int8_t* uq;
  const float* u_scale;
  const int8_t* wq;
  const float* w_scale;
  const int8_t *Are, *Aim, *Bre, *Bim, *Cre, *Cim;
  const float *sAre, *sAim, *sBre, *sBim, *sCre, *sCim;
  const float* log_dt;
  const float* Dskip;
  const float* state_scale;
  const void* h0;
  float* y;
  void* h_last;
};

__device__ __forceinline__ float deq(int8_t q, float s) { return scale_ok(s) ? (float)q * s : 0.0f; }

__device__ __forceinline__ float q16(float v, float s, float inv) {
  return s * fminf(fmaxf(rintf(v * inv), -32768.0f), 32767.0f);
}

// Runs the steps [tb, tb + nt) of one readout block. G = true: the lane's chain is kept as
// g = h / Bbar' (Bbar' = Bbar times the input scale), so an update is g = Abar g + q_t (two fmas
// and a multiply-add for the complex product, no input multiply) and the readout uses
// C' = C Bbar'. G = false: the state h itself (needed for the int16 grid). q_t, the raw input
// code of step t, is read from LDS (the same address for every lane).
template <int NPL, int I16, bool G, bool FULL>
__device__ __forceinline__ void s4d_block(int nt, const float* __restrict__ ub, float (&ar)[NPL],
                                          float (&ai)[NPL], float (&br)[NPL], float (&bi)[NPL],
                                          float (&cr)[NPL], float (&ci)[NPL], float (&hr)[NPL],
                                          float (&hi)[NPL], float ss, float sinv,
                                          float (*red)[kRed], int lane) {
  auto step = [&](int t) {
    const float q = ub[t];
    float yp = 0.0f;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      float nr, ni;
      if (G) {
        nr = fmaf(ar[k], hr[k], fmaf(-ai[k], hi[k], q));
        ni = fmaf(ar[k], hi[k], ai[k] * hr[k]);
      } else {
        nr = fmaf(ar[k], hr[k], fmaf(-ai[k], hi[k], br[k] * q));
        ni = fmaf(ar[k], hi[k], fmaf(ai[k], hr[k], bi[k] * q));
      }
      if (I16) {
        hr[k] = q16(nr, ss, sinv);
        hi[k] = q16(ni, ss, sinv);
      } else {
        hr[k] = nr;
        hi[k] = ni;
      }
      yp = fmaf(cr[k], hr[k], fmaf(-ci[k], hi[k], yp));
    }
    red[t][lane] = yp;
  };
  if (FULL) {
#pragma unroll
    for (int t = 0; t < kBlk; ++t) step(t);
  } else {
    for (int t = 0; t < nt; ++t) step(t);
  }
}

template <int NPL, int I16>
__global__ __launch_bounds__(256) void k_s4d(S4dParams p) {
  __shared__ __align__(16) float red[4][kBlk][kRed];
  __shared__ __align__(16) float ubuf[4][kBlk];
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int64_t chain = (int64_t)blockIdx.x * 4 + w;
  const bool active = chain < p.B * p.H;
  const int64_t cc = active ? chain : 0;
  const int64_t b = cc / p.H, hh = cc % p.H;
  const int64_t L = p.L;

  // input scale: lifted scalar input (u = su sw qw_h q_t), or per-channel input (u = su_h q_t)
  const bool lifted = p.wq != nullptr;
  float us;
  const int8_t* urow;
  if (lifted) {
    us = p.u_scale[0] * p.w_scale[0];
    us = (scale_ok(p.u_scale[0]) && scale_ok(p.w_scale[0])) ? us * (float)p.wq[hh] : 0.0f;
    urow = p.uq + b * L;
  } else {
    us = scale_ok(p.u_scale[hh]) ? p.u_scale[hh] : 0.0f;
    urow = p.uq + (b * p.H + hh) * L;
  }
  const float Dd = p.Dskip ? p.Dskip[hh] : 0.0f;

  float ar[NPL], ai[NPL], br[NPL], bi[NPL], cr[NPL], ci[NPL], hr[NPL], hi[NPL];
  const float dt = expf(p.log_dt[hh]);
  const float ss = I16 ? p.state_scale[hh] : 1.0f;
  const float sinv = I16 ? 1.0f / ss : 1.0f;
  bool zero_b = false;  // some state of this lane has Bbar' = 0
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int64_t n = lane + 64 * k;
    const bool on = n < p.N;
    const int64_t pi = hh * p.N + (on ? n : 0);
    const float Ar = on ? deq(p.Are[pi], p.sAre[hh]) : 0.0f;
    const float Ai = on ? deq(p.Aim[pi], p.sAim[hh]) : 0.0f;
    const float Br = on ? deq(p.Bre[pi], p.sBre[hh]) : 0.0f;
    const float Bi = on ? deq(p.Bim[pi], p.sBim[hh]) : 0.0f;
    cr[k] = on ? deq(p.Cre[pi], p.sCre[hh]) : 0.0f;
    ci[k] = on ? deq(p.Cim[pi], p.sCim[hh]) : 0.0f;
    // zero-order hold
    const float re = dt * Ar, im = dt * Ai;
    float sn, cs, sh, ch;
    sincosf(im, &sn, &cs);
    sincosf(0.5f * im, &sh, &ch);
    const float er = expf(re);
    ar[k] = er * cs;
    ai[k] = er * sn;
    const float em1_re = fmaf(expm1f(re), cs, -2.0f * sh * sh);  // Re(Abar - 1)
    const float em1_im = er * sn;                                 // Im(Abar - 1)
    const float den = Ar * Ar + Ai * Ai;
    if (den == 0.0f) {
      br[k] = dt * Br;
      bi[k] = dt * Bi;
    } else {
      // (Abar - 1) / Ah
      const float qr = (em1_re * Ar + em1_im * Ai) / den;
      const float qi = (em1_im * Ar - em1_re * Ai) / den;
      br[k] = qr * Br - qi * Bi;
      bi[k] = qr * Bi + qi * Br;
    }
    // the input scale moves into Bbar: the loop feeds the raw code
    br[k] *= us;
    bi[k] *= us;
    if (on && br[k] == 0.0f && bi[k] == 0.0f) zero_b = true;
    hr[k] = 0.0f;
    hi[k] = 0.0f;
    if (p.h0 && on) {
      const int64_t si = (b * p.H + hh) * p.N + n;
      if (I16) {
        const short2 v = reinterpret_cast<const short2*>(p.h0)[si];
        hr[k] = ss * (float)v.x;
        hi[k] = ss * (float)v.y;
      } else {
        const float2 v = reinterpret_cast<const float2*>(p.h0)[si];
        hr[k] = v.x;
        hi[k] = v.y;
      }
    }
  }
  // fp32 state: run g = h / Bbar' unless a state of the wave has Bbar' = 0 (a uniform choice)
  const bool gform = !I16 && !__builtin_amdgcn_ballot_w64(zero_b);
  if (gform) {
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const float m = br[k] * br[k] + bi[k] * bi[k];
      const bool on = lane + 64 * k < p.N;
      // g0 = h0 / Bbar' ; C' = C Bbar'
      const float gr = on ? (hr[k] * br[k] + hi[k] * bi[k]) / m : 0.0f;
      const float gi = on ? (hi[k] * br[k] - hr[k] * bi[k]) / m : 0.0f;
      const float c2r = cr[k] * br[k] - ci[k] * bi[k];
      const float c2i = cr[k] * bi[k] + ci[k] * br[k];
      hr[k] = gr;
      hi[k] = gi;
      cr[k] = c2r;
      ci[k] = c2i;
    }
  }

  for (int64_t tb = 0; tb < L; tb += kBlk) {
    const int nt = (int)((L - tb) < kBlk ? (L - tb) : kBlk);
    // lane t converts the code of step tb + t once; the loop reads it back from LDS
    const float q_lane = (lane < nt) ? (float)urow[tb + lane] : 0.0f;
    ubuf[w][lane] = q_lane;
    __syncthreads();
    if (gform) {
      if (nt == kBlk) s4d_block<NPL, 0, true, true>(nt, ubuf[w], ar, ai, br, bi, cr, ci, hr, hi, ss, sinv, red[w], lane);
      else s4d_block<NPL, 0, true, false>(nt, ubuf[w], ar, ai, br, bi, cr, ci, hr, hi, ss, sinv, red[w], lane);
    } else {
      if (nt == kBlk) s4d_block<NPL, I16, false, true>(nt, ubuf[w], ar, ai, br, bi, cr, ci, hr, hi, ss, sinv, red[w], lane);
      else s4d_block<NPL, I16, false, false>(nt, ubuf[w], ar, ai, br, bi, cr, ci, hr, hi, ss, sinv, red[w], lane);
    }
    __syncthreads();
    if (lane < nt) {
      // row `lane` holds the 64 lanes' partials of step tb + lane: 16-byte reads, four sums
      const float4* row = reinterpret_cast<const float4*>(&red[w][lane][0]);
      float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
      for (int j4 = 0; j4 < kBlk / 4; ++j4) {
        const float4 v = row[j4];
        s0 += v.x;
        s1 += v.y;
        s2 += v.z;
        s3 += v.w;
      }
      const float sum = (s0 + s1) + (s2 + s3);
      if (active) p.y[(b * p.H + hh) * L + tb + lane] = fmaf(Dd * us, q_lane, sum);
    }
    __syncthreads();
  }

  if (active && p.h_last) {
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const int64_t n = lane + 64 * k;
      if (n < p.N) {
        float fr = hr[k], fi = hi[k];
        if (gform) {  // h = Bbar' g
          fr = br[k] * hr[k] - bi[k] * hi[k];
          fi = br[k] * hi[k] + bi[k] * hr[k];
        }
        const int64_t si = (b * p.H + hh) * p.N + n;
        if (I16) {
          reinterpret_cast<short2*>(p.h_last)[si] =
              make_short2((short)rintf(fr * sinv), (short)rintf(fi * sinv));
        } else {
          reinterpret_cast<float2*>(p.h_last)[si] = make_float2(fr, fi);
        }
      }
    }
  }
}

template <int NPL>
qssm_status launch_s4d(const S4dParams& p, int i16, hipStream_t st) {
  const unsigned grid = (unsigned)cdiv(p.B * p.H, 4);
  if (i16) k_s4d<NPL, 1><<<grid, 256, 0, st>>>(p);
  else k_s4d<NPL, 0><<<grid, 256, 0, st>>>(p);
  return launch_status("s4d_scan");
}

}  // namespace

extern "C" qssm_status qssm_s4d_scan(const qssm_s4d_args* a, hipStream_t stream) {
  clear_error();
  if (!a) return fail(QSSM_ERR_INVALID_ARG, "args is null");
  if (a->batch < 0 || a->seqlen < 0 || a->channels < 1 || a->dstate < 1)
    return fail(QSSM_ERR_INVALID_ARG, "bad shape");
  if (a->dstate > 256) return fail(QSSM_ERR_UNSUPPORTED, "dstate above 256");
  if (a->state_dtype != QSSM_F32 && a->state_dtype != QSSM_I16)
    return fail(QSSM_ERR_INVALID_ARG, "state_dtype must be QSSM_F32 or QSSM_I16");
  if (a->state_dtype == QSSM_I16 && !a->state_scale)
    return fail(QSSM_ERR_INVALID_ARG, "QSSM_I16 needs state_scale");
  if (a->batch == 0) return QSSM_OK;
  // the input and output sequences are not touched when seqlen == 0 and may then be null
  if ((a->seqlen > 0 && !a->uq) || !a->u_scale || (a->wq && !a->w_scale) || !a->A_re || !a->A_im || !a->B_re ||
      !a->B_im || !a->C_re || !a->C_im || !a->A_re_s || !a->A_im_s || !a->B_re_s || !a->B_im_s ||
      !a->C_re_s || !a->C_im_s || !a->log_dt || (a->seqlen > 0 && !a->y))
    return fail(QSSM_ERR_INVALID_ARG, "null required pointer");
  S4dParams p{a->batch, a->seqlen, a->channels, a->dstate, a->uq, a->u_scale, a->wq, a->w_scale,
              a->A_re, a->A_im, a->B_re, a->B_im, a->C_re, a->C_im, a->A_re_s, a->A_im_s,
              a->B_re_s, a->B_im_s, a->C_re_s, a->C_im_s, a->log_dt, a->Dskip, a->state_scale,
              a->h0, a->y, a->h_last};
  const int i16 = a->state_dtype == QSSM_I16;
  if (a->dstate <= 64) return launch_s4d<1>(p, i16, stream);
  if (a->dstate <= 128) return launch_s4d<2>(p, i16, stream);
  return launch_s4d<4>(p, i16, stream);
}
