// a4-a7: Mamba1 selective scan with int8 (or soft-edge) x and int8 B, C.
//
// Quamba2, abstract: the 8-bit linear recurrence of the Mamba1 backbone, with x in clustered
// per-group int8 and B, C in per-state-group int8. Per channel d and state n:
//     h = exp(delta_t A[d,n]) h + delta_t Bh[n,t] xh_t,    y_t = sum_n Ch[n,t] h + D[d] xh_t
//
// Mapping on CDNA4 (wave64):
//  * A workgroup owns 64 channels of one batch row; lane = channel, so every lane runs its own
//    chains sequentially in time and the sum over states stays in registers.
//  * The N states are split across the W = N / NS waves of the workgroup (NS states per lane).
//    B and C do not depend on the channel, so for a given (b, t) they are the same for every lane
//    of a wave: a staging pass dequantizes them to fp32 once, and the scan reads them with scalar
//    (SMEM) loads straight into SGPR operands of the VALU instructions.
//  * delta and the x codes stream per lane in blocks of T steps (16-byte loads, next block
//    prefetched into registers while the current one is computed).
//  * Each wave writes its partial y (its NS states) for the block to LDS; after a barrier the
//    W partials are summed with the D-skip term and stored (double-buffered LDS, one barrier per
//    block).
//  * exp(delta A) is evaluated as exp2(delta * A log2(e)) with the hardware v_exp_f32.
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.hpp"

using namespace qssm;

namespace {

constexpr int kT = 16;          // time steps per block
constexpr int kPadRows = 64;    // zero rows after L in every staged plane (>= kT + largest batch)
constexpr int kLanes = 64;      // channels per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxWindows = 16;  // time windows of the scan's window form, at most

typedef const uint32_t __attribute__((address_space(4))) cu32;  // constant (scalar-loadable) memory

struct ScanParams {
  int64_t B, L, D, N;
  int32_t G, Gbc, gs, dpg;  // dpg = D / Gbc channels per B/C group
  int32_t Gy;               // int8 output: number of output groups
  const void* x;
  const uint8_t* x_group_of;
  const float* x_scales;
  const float* delta;
  const float* A;
  const void* stage;  // [B, Gbc, N/NS, L + pad, 2*NS]: (B[NS], C[NS]) per wave plane and step
  const float* B_scales;  // [Gbc, N / gs]
  const float* C_scales;
  const float* Dskip;
  const float* h0;
  void* y;
  float* h_last;
  const uint8_t* y_group_of;  // int8 output: [D] output group of each channel
  const float* y_scales;      // int8 output: [Gy] static output scales
  const float* y_bias;        // int8 output: [D] correction term, or NULL
  float se_m, se_im;          // soft-edge x: mode ratio (4 or 2) and its reciprocal
  // Time windows (blockIdx.z = window k covers steps [k Lw, min(L, (k + 1) Lw))):
  //   phase 1: each window from h = 0, no y; writes its end state and its delta sum;
  //   phase 2: each window from its entering state, folded from h0 and the earlier windows' end
  //            states, with y; the last window writes h_last.
  int64_t Lw;
  int32_t phase;
  float* carry;  // [K, B, D, N] window end states from zero (real units)
  float* dsum;   // [K, B, D] sum of delta over each window
};

enum { kYF32 = 0, kYF16 = 1, kYI8 = 2 };  // output forms of the scan

// Stage B and C once into the layout read by the scan: for every (b, g), the states are cut into
// planes of `ns` consecutive states (the states one wave owns), and each plane stores per step the
// ns B values followed by the ns C values.
//  * CODE16 = false: dequantized fp32 values, [B, Gbc, N/ns, L + pad, 2*ns] floats.
//  * CODE16 = true: the code units as fp16 (exact), [B, Gbc, N/ns, L + pad, 2*ns] halves; used
//    when every plane lies inside one state group, so that its scales factor out of the plane's
//    chains (the scan applies them once per output). Codes of a group whose scale is not valid
//    are staged as 0.
// The unit of a code is the int8 value, or for soft-edge bytes (se != 0) the payload times 1, 1/m
// or m (at most 128 in magnitude and a multiple of 1/4: exact in fp16); the value is unit * scale,
// one rounding (m * scale is exact), as the soft-edge decoder defines it.
template <bool CODE16>
__global__ __launch_bounds__(256) void k_stage_bc(const int8_t* __restrict__ Bq,
                                                  const int8_t* __restrict__ Cq,
                                                  const float* __restrict__ Bs,
                                                  const float* __restrict__ Cs, int64_t B,
                                                  int Gbc, int N, int64_t L, int gs, int ns,
                                                  int se, float m, float im,
                                                  void* __restrict__ stage) {
  const int64_t Lp = L + kPadRows;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // over (b, g, n, t < Lp)
  const int64_t total = B * Gbc * N * Lp;
  if (idx >= total) return;
  const int64_t t = idx % Lp;
  const int64_t r = idx / Lp;  // (b, g, n)
  const int n = (int)(r % N);
  const int64_t bg = r / N;
  const int g = (int)(bg % Gbc);
  const int ngs = N / gs;
  const float sb = Bs[g * ngs + n / gs], sc = Cs[g * ngs + n / gs];
  const int plane = n / ns, k = n % ns;
  const int64_t row = ((bg * (N / ns) + plane) * Lp + t) * (2 * ns);
  // rows past L are zero (read by the last batches, times delta = 0)
  const uint32_t bb = t < L ? (uint32_t)(uint8_t)Bq[r * L + t] : 0u;
  const uint32_t cb = t < L ? (uint32_t)(uint8_t)Cq[r * L + t] : 0u;
  const float ub = se ? softedge_unit(bb, m, im) : (float)(int8_t)bb;
  const float uc = se ? softedge_unit(cb, m, im) : (float)(int8_t)cb;
  const float qb = scale_ok(sb) ? ub : 0.0f;
  const float qc = scale_ok(sc) ? uc : 0.0f;
  if (CODE16) {
    _Float16* dst = reinterpret_cast<_Float16*>(stage) + row;
    dst[k] = (_Float16)qb;
    dst[ns + k] = (_Float16)qc;
  } else {
    float* dst = reinterpret_cast<float*>(stage) + row;
    dst[k] = qb * sb;
    dst[ns + k] = qc * sc;
  }
}

// Unscaled x value of a code byte: the int8 code, or the soft-edge code times its mode factor
// (1, 1/m or m; exact), so that the dequantized value is sx * xunit.
// Branch-free soft-edge decode for base scale 1: tag 0 -> 7-bit payload, tag 10 -> 6-bit payload
// times 1/m, tag 11 -> 6-bit payload times m (the layout of softedge_value).
template <int XCODE>
__device__ __forceinline__ float xunit(uint32_t byte, float m, float im) {
  if (XCODE == QSSM_X_SOFTEDGE) {
    const int q7 = __builtin_amdgcn_sbfe((int)byte, 0, 7);
    const int q6 = __builtin_amdgcn_sbfe((int)byte, 0, 6);
    const bool tagged = (byte & 0x80u) != 0;
    const float f = tagged ? ((byte & 0x40u) ? m : im) : 1.0f;
    return (float)(tagged ? q6 : q7) * f;
  }
  return (float)(int8_t)(byte & 0xFFu);
}

template <int NS, int W, int XCODE, int YOUT, int kBatch, int PFD, bool CODE16, bool WIN>
__global__ __launch_bounds__(64 * W) void k_scan_m1(ScanParams p) {
  __shared__ float ybuf[2][W][kT][kLanes];
  constexpr int kS = CODE16 ? NS : 2 * NS;  // staged 32-bit words per step
  // Soft-edge codes: instead of every wave decoding every step, wave w decodes steps
  // [w kT/W, (w+1) kT/W) of the next block and shares them through LDS (per lane 16 values in a
  // row padded to 20 floats: conflict-free 16-byte accesses); the per-block barrier orders it.
  constexpr bool kShareX = XCODE == QSSM_X_SOFTEDGE;
  constexpr int kXdRow = 20;
  constexpr int kPerX = kT / W;
  __shared__ __align__(16) float xd[kShareX ? 2 : 1][kShareX ? kLanes : 1][kShareX ? kXdRow : 1];
  // int8 output: the codes of eight blocks (128 steps) gather per channel in LDS (rows padded to
  // 132 bytes) and leave as whole 128-byte lines, two groups of blocks in turn
  constexpr bool kGather = YOUT == kYI8;
  constexpr int kGrpBlocks = 8;
  constexpr int kRowB = kGrpBlocks * kT + 4;
  __shared__ __align__(16) uint8_t ycode[kGather ? 2 : 1][kGather ? kLanes : 1][kGather ? kRowB : 4];

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int64_t b = blockIdx.y;
  const int64_t d0 = (int64_t)blockIdx.x * kLanes;
  const int64_t d = d0 + lane;
  const bool valid = d < p.D;
  const int64_t dc = valid ? d : p.D - 1;  // clamped channel for loads
  const int64_t L = p.L;
  const int g = uniform((int)(d0 / p.dpg));

  // Scales. x: per channel (lane); a channel whose scale is not valid has every x value 0, so its
  // codes are masked to 0 and its scale taken as 0. The chains run in input units: a wave's chain
  // holds h / su, with su the scale of its per-step input (sx, times the B scale of the wave's
  // state group when fp16 codes are staged), so each step adds dt * x_code * B; su and the C scale
  // multiply the wave's partial output once, in the combine. An invalid B or C scale is 0 (its
  // codes are staged as 0 as well); a zero su (no input reaches the chain) is replaced by 1.
  // su is kept as m * 2^e (m = the product of the two scales' significands): two valid scales can
  // have a product outside the normal fp32 range (2^-80 * 2^-80), and then the factors below are
  // formed from the exponent sum with ldexp, so an output that fp32 can represent stays exact.
  // Group indices at or above the group count are clamped to the last group.
  float sx = p.x_scales[min((int)p.x_group_of[dc], p.G - 1)];
  const bool sx_ok = scale_ok(sx);
  const uint32_t xmask = sx_ok ? 0xFFFFFFFFu : 0u;
  if (!sx_ok) sx = 0.0f;
  const int ngs = (int)(p.N / p.gs);
  float cf[W];        // factor of each wave's partial output (C scale x that wave's su)
  float sum_ = 1.0f;  // this wave's su as m * 2^se
  int se = 0;
#pragma unroll
  for (int ww = 0; ww < W; ++ww) {
    float sb = 1.0f, sc = 1.0f;
    if (CODE16) {
      sb = p.B_scales[g * ngs + (ww * NS) / p.gs];
      sb = scale_ok(sb) ? sb : 0.0f;
      sc = p.C_scales[g * ngs + (ww * NS) / p.gs];
      sc = scale_ok(sc) ? sc : 0.0f;
    }
    int ex = 0, eb = 0;
    float m = frexpf(sx, &ex) * frexpf(sb, &eb);
    int e = ex + eb;
    if (m == 0.0f) {
      m = 1.0f;
      e = 0;
    }
    cf[ww] = ldexpf(sc * m, e);
    if (ww == w) {
      sum_ = m;
      se = e;
    }
  }
  const float Dsx = (p.Dskip ? p.Dskip[dc] : 0.0f) * sx;
  // int8 output: this channel's output scale (its reciprocal, 0 for an invalid scale) and
  // correction term
  float sy = 1.0f, ry = 0.0f, yb = 0.0f;
  if (YOUT == kYI8) {
    sy = p.y_scales[min((int)p.y_group_of[dc], p.Gy - 1)];
    ry = recip_or_zero(sy);
    yb = p.y_bias ? p.y_bias[dc] : 0.0f;
  }

  // WIN = false: the chain form (phase 0, steps [0, L)); true: phases 1 and 2 on window
  // blockIdx.z
  const int64_t kw = WIN ? (int64_t)blockIdx.z : 0;
  const int64_t tbeg = WIN ? kw * p.Lw : 0;
  const int64_t tend = WIN ? ((tbeg + p.Lw < L) ? tbeg + p.Lw : L) : L;
  const bool local = WIN && p.phase == 1;  // window end states only
  float a2[NS], h[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int n = w * NS + k;
    a2[k] = p.A[dc * p.N + n] * kLog2e;
    if (!WIN) {
      h[k] = p.h0 ? ldexpf(p.h0[(b * p.D + dc) * p.N + n] / sum_, -se) : 0.0f;
    } else if (local) {
      h[k] = 0.0f;
    } else {
      // entering state of window kw: h0 carried through the earlier windows, window k2 scaling
      // it by exp(A * its delta sum) and adding its end state from zero
      // (at most kMaxWindows terms, all loads issued before the dependent chain)
      float hv = p.h0 ? p.h0[(b * p.D + dc) * p.N + n] : 0.0f;
      float ds[kMaxWindows], ce[kMaxWindows];
#pragma unroll
      for (int k2 = 0; k2 < kMaxWindows; ++k2) {
        const int64_t kk = k2 < kw ? k2 : 0;
        ds[k2] = p.dsum[(kk * p.B + b) * p.D + dc];
        ce[k2] = p.carry[((kk * p.B + b) * p.D + dc) * p.N + n];
      }
#pragma unroll
      for (int k2 = 0; k2 < kMaxWindows; ++k2)
        if (k2 < kw) hv = fmaf(__builtin_amdgcn_exp2f(a2[k] * ds[k2]), hv, ce[k2]);
      h[k] = ldexpf(hv / sum_, -se);
    }
  }
  float dacc = 0.0f;  // phase 1: sum of delta over the window

  const float* __restrict__ drow = p.delta + (b * p.D + dc) * L;
  const uint8_t* __restrict__ xrow = reinterpret_cast<const uint8_t*>(p.x) + (b * p.D + dc) * L;
  // this wave's plane of staged (B, C): kS words per step, read through the constant address
  // space (wave-uniform addresses -> scalar loads into SGPRs)
  const uint32_t* stg = reinterpret_cast<const uint32_t*>(p.stage) +
                        ((b * p.Gbc + g) * (p.N / NS) + w) * (L + kPadRows) * kS;
  const cu32* st = (const cu32*)stg;
  const bool vec_ok = (L % 16) == 0;

  auto load_block = [&](int64_t tb, float* dv, uint32_t* xv) {
    if (vec_ok && tb + kT <= L) {
#pragma unroll
      for (int k = 0; k < kT / 4; ++k) {
        float4 t4 = reinterpret_cast<const float4*>(drow + tb)[k];
        dv[4 * k] = t4.x; dv[4 * k + 1] = t4.y; dv[4 * k + 2] = t4.z; dv[4 * k + 3] = t4.w;
      }
#pragma unroll
      for (int k = 0; k < kT / 16; ++k) {
        uint4 u = reinterpret_cast<const uint4*>(xrow + tb)[k];
        xv[4 * k] = u.x; xv[4 * k + 1] = u.y; xv[4 * k + 2] = u.z; xv[4 * k + 3] = u.w;
      }
    } else {
      // ragged tail: steps past L get delta = 0 and x = 0, which leave h exactly unchanged
#pragma unroll
      for (int k = 0; k < kT; ++k) dv[k] = (tb + k < L) ? drow[tb + k] : 0.0f;
#pragma unroll
      for (int k = 0; k < kT / 4; ++k) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t t = tb + 4 * k + j;
          const uint32_t byte = (t < L) ? xrow[t] : 0u;
          word |= byte << (8 * j);
        }
        xv[k] = word;
      }
    }
  };

  // Scalar loads return out of order, so waiting for one means waiting for all: the staged values
  // are fetched one batch of steps ahead and the loop drains the scalar queue (lgkmcnt 0) once per
  // batch, right before issuing the next batch, so each batch's latency hides behind the previous
  // batch's arithmetic. Steps past L read the zero pad rows (times delta = 0).
  uint32_t bcur[kBatch][kS], bnxt[kBatch][kS];
  auto sload = [&](int64_t t0, uint32_t (&dst)[kBatch][kS]) {
    const cu32* src = st + t0 * kS;
#pragma unroll
    for (int s2 = 0; s2 < kBatch; ++s2)
#pragma unroll
      for (int j = 0; j < kS; ++j) dst[s2][j] = src[s2 * kS + j];
  };
  // B and C operand k of a staged step
  auto opB = [&](const uint32_t (&row)[kS], int k) -> float {
    if (CODE16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(row[k / 2] >> (16 * (k % 2))));
    return __uint_as_float(row[k]);
  };
  auto opC = [&](const uint32_t (&row)[kS], int k) -> float {
    if (CODE16)
      return (float)__builtin_bit_cast(_Float16, (uint16_t)(row[NS / 2 + k / 2] >> (16 * (k % 2))));
    return __uint_as_float(row[NS + k]);
  };

  float dlA[kT], dlB[kT];
  uint32_t xqA[kT / 4], xqB[kT / 4];
#pragma unroll
  for (int k = 0; k < kT; ++k) dlB[k] = 0.0f;
#pragma unroll
  for (int k = 0; k < kT / 4; ++k) xqB[k] = 0u;
  load_block(tbeg, dlA, xqA);
  sload(tbeg, bcur);
  // decoded x units of the next block, this wave's share, into LDS buffer nb
  auto share_x = [&](const uint32_t (&codes)[kT / 4], int nb) {
    if (kShareX) {
      float v[kPerX];
#pragma unroll
      for (int j = 0; j < kPerX; ++j) {
        const int t = w * kPerX + j;  // w is wave-uniform: a runtime register index is avoided
        uint32_t word = 0u;            // by selecting the word with uniform compares
#pragma unroll
        for (int k = 0; k < kT / 4; ++k) word = (t / 4 == k) ? codes[k] : word;
        v[j] = xunit<XCODE>((word & xmask) >> (8 * (t % 4)), p.se_m, p.se_im);
      }
#pragma unroll
      for (int j = 0; j < kPerX; ++j) xd[nb][lane][w * kPerX + j] = v[j];
    }
  };
  if (kShareX) {
    share_x(xqA, 0);
    __syncthreads();
  }
  // exp(delta A) of the next two steps, by step parity
  float dAr[2][NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    dAr[0][k] = __builtin_amdgcn_exp2f(dlA[0] * a2[k]);
    dAr[1][k] = __builtin_amdgcn_exp2f(dlA[1] * a2[k]);
  }
  // Store the gathered codes of block group grp (steps [grp*128, grp*128 + 128) of the 64
  // channels): 16-byte pieces, eight per channel row, spread over the workgroup's threads.
  auto flush_codes = [&](int64_t grp) {
    const int gb = (int)(grp & 1);
    const int64_t tg = grp * (kGrpBlocks * kT);
    for (int idx = threadIdx.x; idx < kLanes * 8; idx += 64 * W) {
      const int row = idx >> 3, piece = idx & 7;
      const int64_t dd = d0 + row;
      const int64_t t = tg + piece * 16;
      if (dd >= p.D || t >= L) continue;
      const uint32_t* src = reinterpret_cast<const uint32_t*>(&ycode[gb][row][piece * 16]);
      int8_t* dst = reinterpret_cast<int8_t*>(p.y) + (b * p.D + dd) * L + t;
      if (vec_ok && t + 16 <= L) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(src[0], src[1], src[2], src[3]);
      } else {
        for (int j = 0; j < 16 && t + j < L; ++j) dst[j] = (int8_t)ycode[gb][row][piece * 16 + j];
      }
    }
  };
  // One block of kT steps: dl/xq hold this block's delta and x codes, dn/xn receive the next
  // block's; buf selects the LDS buffers. The block loop is unrolled twice with the two register
  // sets swapping roles, so that no copy of the next block's values is needed between blocks.
  auto block = [&](int64_t tb, float (&dl)[kT], float (&dn)[kT], uint32_t (&xq)[kT / 4],
                   uint32_t (&xn)[kT / 4], const int buf) {
    // (masking the codes of the current block here, not at load time, keeps the next block's
    // loads in flight during this block's arithmetic)
#pragma unroll
    for (int k = 0; k < kT / 4; ++k) xq[k] &= xmask;
    if (tb + kT < tend) load_block(tb + kT, dn, xn);
    if (local) {
#pragma unroll
      for (int k = 0; k < kT; ++k) dacc += dl[k];
    }
    // Pull the staged rows of the block PFD blocks ahead into L2 with one vector load per
    // 128-byte line, so that the scalar loads of that block hit L2 instead of going to memory.
    // The loaded value is only consumed (without use) after this block's arithmetic.
    uint32_t pf = 0u;
    if (PFD > 0) {
      const int64_t tp = tb + (int64_t)PFD * kT;
      constexpr int kLines = (kT * kS * 4 + 127) / 128;
      if (tp < L && lane < kLines) pf = stg[tp * kS + lane * 32];
    }
    float xcur[kShareX ? kT : 1];  // this block's decoded x units (soft-edge)
    if (kShareX) {
#pragma unroll
      for (int k = 0; k < kT / 4; ++k) {
        const float4 v4 = *reinterpret_cast<const float4*>(&xd[buf][lane][4 * k]);
        xcur[4 * k] = v4.x; xcur[4 * k + 1] = v4.y; xcur[4 * k + 2] = v4.z; xcur[4 * k + 3] = v4.w;
      }
    }

#pragma unroll
    for (int bt = 0; bt < kT; bt += kBatch) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the current batch has landed
      sload(tb + bt + kBatch, bnxt);
#pragma unroll
      for (int s2 = 0; s2 < kBatch; ++s2) {
        const int t = bt + s2;
        const float dt = dl[t];
        const float u = dt * (kShareX ? xcur[kShareX ? t : 0]
                                      : xunit<XCODE>(xq[t / 4] >> (8 * (t % 4)), p.se_m, p.se_im));
        float dA[NS];
#pragma unroll
        for (int k = 0; k < NS; ++k) dA[k] = dAr[t % 2][k];
        // exp of the step two ahead (this block's, or the next block's first two), so that its
        // latency is covered by two steps of arithmetic
        const float dt2 = (t + 2 < kT) ? dl[t + 2] : dn[t + 2 - kT];
#pragma unroll
        for (int k = 0; k < NS; ++k) dAr[t % 2][k] = __builtin_amdgcn_exp2f(dt2 * a2[k]);
        float yp;
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          // fma with a zero addend keeps the fp16 operand in a mixed-precision fma
          const float in = CODE16 ? fmaf(u, opB(bcur[s2], k), 0.0f) : u * opB(bcur[s2], k);
          h[k] = fmaf(dA[k], h[k], in);
          yp = fmaf(opC(bcur[s2], k), h[k], k == 0 ? 0.0f : yp);
        }
        ybuf[buf][w][t][lane] = yp;
      }
#pragma unroll
      for (int s2 = 0; s2 < kBatch; ++s2)
#pragma unroll
        for (int j = 0; j < kS; ++j) bcur[s2][j] = bnxt[s2][j];
    }
    if (PFD > 0) asm volatile("" ::"v"(pf));
    if (kShareX && tb + kT < tend) share_x(xn, buf ^ 1);
    __syncthreads();
    if (local) return;

    // combine: wave w finalizes steps [w*kT/W, (w+1)*kT/W) of every channel of the block
    constexpr int kPer = kT / W;
    float yo[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int t = w * kPer + j;
      float sum = 0.0f;
#pragma unroll
      for (int ww = 0; ww < W; ++ww)
        sum = fmaf(cf[ww], ybuf[buf][ww][t][lane], sum);
      const float xu = kShareX ? xd[buf][lane][kShareX ? t : 0]
                               : xunit<XCODE>(xq[t / 4] >> (8 * (t % 4)), p.se_m, p.se_im);
      yo[j] = fmaf(Dsx, xu, sum);
    }
    const int64_t t0 = tb + w * kPer;
    if (kGather) {
      // the previous group's codes, complete since this block's barrier, leave first; this
      // block's codes go to the other buffer
      const int64_t blk = tb / kT;
      if (blk % kGrpBlocks == 0 && blk > 0) flush_codes(blk / kGrpBlocks - 1);
      uint32_t code[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) code[j] = (uint8_t)quant8_r(yo[j] + yb, sy, ry);
      uint8_t* crow = &ycode[(blk / kGrpBlocks) & 1][lane][(blk % kGrpBlocks) * kT + w * kPer];
      if (kPer % 4 == 0) {
#pragma unroll
        for (int j = 0; j < kPer / 4; ++j)
          reinterpret_cast<uint32_t*>(crow)[j] = code[4 * j] | (code[4 * j + 1] << 8) |
                                                 (code[4 * j + 2] << 16) | (code[4 * j + 3] << 24);
      } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) crow[j] = (uint8_t)code[j];
      }
    } else if (valid) {
      if (YOUT == kYF16) {
        __half* yr = reinterpret_cast<__half*>(p.y) + (b * p.D + d) * L;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          if (t0 + j < L) yr[t0 + j] = __float2half_rn(yo[j]);
      } else {
        float* yr = reinterpret_cast<float*>(p.y) + (b * p.D + d) * L;
        if (vec_ok && t0 + kPer <= L && kPer % 4 == 0) {
#pragma unroll
          for (int j = 0; j < kPer / 4; ++j)
            reinterpret_cast<float4*>(yr + t0)[j] =
                make_float4(yo[4 * j], yo[4 * j + 1], yo[4 * j + 2], yo[4 * j + 3]);
        } else {
#pragma unroll
          for (int j = 0; j < kPer; ++j)
            if (t0 + j < L) yr[t0 + j] = yo[j];
        }
      }
    }
  };
  for (int64_t tb = tbeg; tb < tend; tb += 2 * kT) {
    block(tb, dlA, dlB, xqA, xqB, 0);
    if (tb + kT < tend) block(tb + kT, dlB, dlA, xqB, xqA, 1);
  }
  if (kGather && L > 0) {
    // the last (possibly partial) group
    __syncthreads();
    flush_codes((L - 1) / (kGrpBlocks * kT));
  }

  if (valid && p.h_last && (!WIN || (!local && kw == (int64_t)gridDim.z - 1))) {
#pragma unroll
    for (int k = 0; k < NS; ++k) p.h_last[(b * p.D + d) * p.N + w * NS + k] = ldexpf(h[k] * sum_, se);
  }
  if (valid && local) {
#pragma unroll
    for (int k = 0; k < NS; ++k)
      p.carry[((kw * p.B + b) * p.D + d) * p.N + w * NS + k] = ldexpf(h[k] * sum_, se);
    if (w == 0) p.dsum[(kw * p.B + b) * p.D + d] = dacc;
  }
}

template <int NS, int W, int BATCH, bool CODE16, int XCODE>
void launch_scan_x(const ScanParams& p, int yout, dim3 grid, dim3 block, hipStream_t st) {
  if (grid.z > 1) {  // time windows (never with the int8 output)
    if (yout == kYF16) k_scan_m1<NS, W, XCODE, kYF16, BATCH, 1, CODE16, true><<<grid, block, 0, st>>>(p);
    else k_scan_m1<NS, W, XCODE, kYF32, BATCH, 1, CODE16, true><<<grid, block, 0, st>>>(p);
    return;
  }
  if (yout == kYF16) k_scan_m1<NS, W, XCODE, kYF16, BATCH, 1, CODE16, false><<<grid, block, 0, st>>>(p);
  else if (yout == kYI8) k_scan_m1<NS, W, XCODE, kYI8, BATCH, 1, CODE16, false><<<grid, block, 0, st>>>(p);
  else k_scan_m1<NS, W, XCODE, kYF32, BATCH, 1, CODE16, false><<<grid, block, 0, st>>>(p);
}

template <int NS, int W, int BATCH, bool CODE16>
void launch_scan_t(const ScanParams& p, int xcode, int yout, dim3 grid, dim3 block, hipStream_t st) {
  if (xcode == QSSM_X_INT8) launch_scan_x<NS, W, BATCH, CODE16, QSSM_X_INT8>(p, yout, grid, block, st);
  else launch_scan_x<NS, W, BATCH, CODE16, QSSM_X_SOFTEDGE>(p, yout, grid, block, st);
}

// BATCH16 / BATCH32: steps per scalar-load batch with fp16 codes / fp32 values staged (two
// batches of kS words per step must fit the SGPR budget next to the kernel's other scalars)
template <int NS, int W, int BATCH16, int BATCH32>
qssm_status launch_scan(const ScanParams& p, int xcode, int yout, bool code16, int nwin,
                        hipStream_t st) {
  dim3 grid((unsigned)cdiv(p.D, kLanes), (unsigned)p.B, (unsigned)nwin);
  dim3 block(64 * W);
  if (code16) launch_scan_t<NS, W, BATCH16, true>(p, xcode, yout, grid, block, st);
  else launch_scan_t<NS, W, BATCH32, false>(p, xcode, yout, grid, block, st);
  return launch_status("scan_w8a8");
}

// states per wave for a state size N (the workgroup has N / NS waves)
int states_per_wave(int64_t N) { return N == 8 ? 2 : (N == 64 ? 8 : 4); }

size_t stage_bytes(const qssm_scan_args* a) {
  return (size_t)a->batch * (size_t)a->bc_groups * (size_t)a->dstate *
         (size_t)(a->seqlen + kPadRows) * 2 * sizeof(float);
}

// Time windows of the scan: (count, length). One window is the chain form. More windows cut each
// chain into pieces that run in parallel (each piece's end state from zero; then each piece again
// from its entering state, which it folds from h0 and the earlier pieces' end states): twice the
// recurrence arithmetic, for parallelism when batch x channel blocks leave the GPU mostly idle. time_blocks = 0 chooses:
// windows when fewer than kWindowWgs channel blocks exist, enough for about 2 x kWindowWgs
// workgroups; time_blocks = 1 forces the chain form, K >= 2 asks for K windows (at most
// kMaxWindows; fewer when the sequence has fewer 16-step blocks). The int8 output
// always uses the chain form (its codes are gathered over 128-step groups of the chain).
constexpr int64_t kWindowWgs = 128;

struct Windows {
  int64_t count, len;
};

Windows scan_windows(const qssm_scan_args* a) {
  const int64_t L = a->seqlen;
  const int64_t blocks = (L + kT - 1) / kT;
  int64_t K = 1;
  if (a->y_dtype != QSSM_I8 && blocks >= 2) {
    if (a->time_blocks >= 2) {
      K = a->time_blocks;
    } else if (a->time_blocks == 0) {
      const int64_t wgs = (a->dim + kLanes - 1) / kLanes * a->batch;
      if (wgs < kWindowWgs) K = (2 * kWindowWgs + wgs - 1) / (wgs > 0 ? wgs : 1);
    }
  }
  if (K > blocks) K = blocks;
  if (K > kMaxWindows) K = kMaxWindows;
  if (K < 2) return Windows{1, L};
  const int64_t len = ((L + K - 1) / K + kT - 1) / kT * kT;
  return Windows{(L + len - 1) / len, len};
}

// Workspace: the B/C staging, then (with windows) the carries [K, B, D, N] and the window delta
// sums [K, B, D], each 256-byte aligned.
struct ScanWs {
  size_t carry_off, dsum_off, total;
};

ScanWs scan_ws(const qssm_scan_args* a) {
  const Windows win = scan_windows(a);
  ScanWs w;
  w.carry_off = (stage_bytes(a) + 255) & ~(size_t)255;
  w.dsum_off = w.carry_off;
  w.total = stage_bytes(a);
  if (win.count > 1) {
    const size_t nc = (size_t)win.count * a->batch * a->dim;
    w.dsum_off = (w.carry_off + nc * a->dstate * sizeof(float) + 255) & ~(size_t)255;
    w.total = w.dsum_off + nc * sizeof(float);
  }
  return w;
}

constexpr size_t kScanScratchBytes = (size_t)QSSM_SCAN_SCRATCH_BYTES;

// Validation, B/C staging and the scan launch; `ws` is 256-byte aligned and holds
// scan_ws(a).total bytes (it may be null when that is 0).
qssm_status scan_impl(const qssm_scan_args* a, void* ws, hipStream_t stream) {
  const int64_t B = a->batch, L = a->seqlen, D = a->dim, N = a->dstate;
  const int64_t dpg = D / a->bc_groups;
  float* stage = reinterpret_cast<float*>(ws);
  const int ns = states_per_wave(N);
  // fp16 codes when every wave's states lie inside one B/C state group
  const bool code16 = (a->bc_group_size % ns) == 0;
  const int64_t nstage = B * a->bc_groups * N * (L + kPadRows);
  const int bse = a->bc_code != QSSM_X_INT8;
  const float bm = softedge_ratio(a->bc_code), bim = 1.0f / bm;
  if (nstage > 0) {
    if (code16)
      k_stage_bc<true><<<(unsigned)cdiv(nstage, 256), 256, 0, stream>>>(
          a->Bq, a->Cq, a->B_scales, a->C_scales, B, a->bc_groups, (int)N, L, a->bc_group_size,
          ns, bse, bm, bim, stage);
    else
      k_stage_bc<false><<<(unsigned)cdiv(nstage, 256), 256, 0, stream>>>(
          a->Bq, a->Cq, a->B_scales, a->C_scales, B, a->bc_groups, (int)N, L, a->bc_group_size,
          ns, bse, bm, bim, stage);
    if (qssm_status s = launch_status("scan_w8a8 staging")) return s;
  }
  const Windows win = scan_windows(a);
  const ScanWs wl = scan_ws(a);
  char* wsb = reinterpret_cast<char*>(ws);
  ScanParams p{B, L, D, N, a->x_groups, a->bc_groups, a->bc_group_size, (int32_t)dpg,
               a->y_dtype == QSSM_I8 ? a->y_groups : 1,
               a->x, a->x_group_of, a->x_scales, a->delta, a->A, stage, a->B_scales,
               a->C_scales, a->Dskip, a->h0, a->y, a->h_last, a->y_group_of, a->y_scales,
               a->y_bias, softedge_ratio(a->x_code), 1.0f / softedge_ratio(a->x_code),
               win.len, 0, win.count > 1 ? reinterpret_cast<float*>(wsb + wl.carry_off) : nullptr,
               win.count > 1 ? reinterpret_cast<float*>(wsb + wl.dsum_off) : nullptr};
  const int yout = a->y_dtype == QSSM_F16 ? kYF16 : (a->y_dtype == QSSM_I8 ? kYI8 : kYF32);
  auto run = [&](const ScanParams& q, int nwin) -> qssm_status {
    switch (N) {
      case 4: return launch_scan<4, 1, 8, 8>(q, a->x_code, yout, code16, nwin, stream);
      case 8: return launch_scan<2, 4, 16, 16>(q, a->x_code, yout, code16, nwin, stream);
      case 16: return launch_scan<4, 4, 8, 8>(q, a->x_code, yout, code16, nwin, stream);
      case 32: return launch_scan<4, 8, 8, 8>(q, a->x_code, yout, code16, nwin, stream);
      default: return launch_scan<8, 8, 4, 4>(q, a->x_code, yout, code16, nwin, stream);
    }
  };
  if (win.count == 1) return run(p, 1);
  const int K = (int)win.count;
  p.phase = 1;
  if (qssm_status s = run(p, K)) return s;
  p.phase = 2;
  return run(p, K);
}

// Argument checks shared by both entry points; QSSM_OK means "launch", and *done is set when the
// call has nothing to do (B == 0).
qssm_status validate(const qssm_scan_args* a, bool* done) {
  *done = false;
  if (!a) return fail(QSSM_ERR_INVALID_ARG, "args is null");
  const int64_t B = a->batch, L = a->seqlen, D = a->dim, N = a->dstate;
  if (B < 0 || L < 0 || D < 1 || N < 1) return fail(QSSM_ERR_INVALID_ARG, "bad shape");
  if (L > 0x7fffff00LL) return fail(QSSM_ERR_UNSUPPORTED, "seqlen must be below 2^31 - 256");
  if (a->x_code != QSSM_X_INT8 && a->x_code != QSSM_X_SOFTEDGE && a->x_code != QSSM_X_SOFTEDGE2)
    return fail(QSSM_ERR_INVALID_ARG, "x_code must be QSSM_X_INT8, QSSM_X_SOFTEDGE or QSSM_X_SOFTEDGE2");
  if (a->bc_code != QSSM_X_INT8 && a->bc_code != QSSM_X_SOFTEDGE && a->bc_code != QSSM_X_SOFTEDGE2)
    return fail(QSSM_ERR_INVALID_ARG, "bc_code must be QSSM_X_INT8, QSSM_X_SOFTEDGE or QSSM_X_SOFTEDGE2");
  if (a->y_dtype != QSSM_F32 && a->y_dtype != QSSM_F16 && a->y_dtype != QSSM_I8)
    return fail(QSSM_ERR_INVALID_ARG, "y_dtype must be QSSM_F32, QSSM_F16 or QSSM_I8");
  if (a->y_dtype == QSSM_I8) {
    if (a->y_groups < 1 || a->y_groups > 256)
      return fail(QSSM_ERR_INVALID_ARG, "y_groups not in 1..256");
    if (!a->y_group_of || !a->y_scales)
      return fail(QSSM_ERR_INVALID_ARG, "QSSM_I8 output needs y_group_of and y_scales");
  }
  if (a->x_groups < 1 || a->x_groups > 256) return fail(QSSM_ERR_INVALID_ARG, "x_groups not in 1..256");
  if (a->bc_groups < 1 || D % a->bc_groups != 0)
    return fail(QSSM_ERR_INVALID_ARG, "bc_groups must divide D");
  if (a->bc_group_size < 1 || N % a->bc_group_size != 0)
    return fail(QSSM_ERR_INVALID_ARG, "bc_group_size must divide N");
  const int64_t dpg = D / a->bc_groups;
  if (a->bc_groups > 1 && dpg % kLanes != 0)
    return fail(QSSM_ERR_UNSUPPORTED, "with bc_groups > 1, D / bc_groups must be a multiple of 64");
  if (N != 4 && N != 8 && N != 16 && N != 32 && N != 64)
    return fail(QSSM_ERR_UNSUPPORTED, "dstate must be 4, 8, 16, 32 or 64");
  if (B == 0) {
    *done = true;
    return QSSM_OK;
  }
  // the per-step buffers are not touched when L == 0 and may then be null
  if (!a->x_group_of || !a->x_scales || !a->A || !a->B_scales || !a->C_scales ||
      (L > 0 && (!a->x || !a->delta || !a->Bq || !a->Cq || !a->y)))
    return fail(QSSM_ERR_INVALID_ARG, "null required pointer");
  if (((uintptr_t)a->x | (uintptr_t)a->delta | (uintptr_t)a->y) % 16 != 0)
    return fail(QSSM_ERR_INVALID_ARG, "x, delta and y must be 16-byte aligned");
  return QSSM_OK;
}

}  // namespace

// Allocation-free variant: the staging buffer lives in a library-owned device array of fixed size,
// one copy per GPU. Host code reaches it only through the address hipGetSymbolAddress returns for
// the current device (the array's own name is a host-side stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[kScanScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];  // per device, set once under the mutex

// Device address of the scratch array on the current device (looked up once per device, with that
// device current).
qssm_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(QSSM_ERR_DEVICE, "cannot query the current device");
  if (dev >= kMaxScratchDevices)
    return fail(QSSM_ERR_UNSUPPORTED, "device index %d above %d", dev, kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(QSSM_ERR_DEVICE, "hipGetSymbolAddress of the scan scratch array: %s",
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QSSM_OK;
}

}  // namespace

extern "C" {

size_t qssm_scan_workspace_size(const qssm_scan_args* a) {
  if (!a || a->batch < 0 || a->seqlen < 0 || a->dim < 1 || a->bc_groups < 1 || a->dstate < 1)
    return 0;
  return scan_ws(a).total + 256;
}

qssm_status qssm_scan_w8a8(const qssm_scan_args* a, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  clear_error();
  bool done = false;
  if (qssm_status s = validate(a, &done)) return s;
  if (done) return QSSM_OK;
  const size_t need = scan_ws(a).total;
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(QSSM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  void* stage = reinterpret_cast<void*>(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  if ((size_t)((char*)stage - (char*)ws) + need > ws_bytes)
    return fail(QSSM_ERR_WORKSPACE, "workspace too small after 256-byte alignment");
  return scan_impl(a, stage, stream);
}

qssm_status qssm_scan_w8a8_noalloc(const qssm_scan_args* a, hipStream_t stream) {
  clear_error();
  bool done = false;
  if (qssm_status s = validate(a, &done)) return s;
  if (done) return QSSM_OK;
  const size_t need = scan_ws(a).total;
  if (need > kScanScratchBytes)
    return fail(QSSM_ERR_UNSUPPORTED,
                "the scan needs %zu bytes of scratch (B/C staging and window carries), above the "
                "%zu-byte array of the allocation-free entry point", need, kScanScratchBytes);
  void* stage = nullptr;
  if (qssm_status s = scratch_address(&stage)) return s;
  return scan_impl(a, stage, stream);
}

}  // extern "C"
