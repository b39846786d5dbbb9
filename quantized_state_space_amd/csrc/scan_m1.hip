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

#include "common.hpp"

using namespace qssm;

namespace {

constexpr int kT = 32;          // time steps per block
constexpr int kPadRows = 64;    // zero rows after L in every staged plane (>= kT + largest batch)
constexpr int kLanes = 64;      // channels per workgroup
constexpr float kLog2e = 1.4426950408889634f;

typedef const float __attribute__((address_space(4))) cfloat;  // constant (scalar-loadable) memory

struct ScanParams {
  int64_t B, L, D, N;
  int32_t G, Gbc, gs, dpg;  // dpg = D / Gbc channels per B/C group
  const void* x;
  const uint8_t* x_group_of;
  const float* x_scales;
  const float* delta;
  const float* A;
  const float* stage;  // [B, Gbc, N/NS, L, 2*NS]: (Bh[NS], Ch[NS]) per wave plane and step
  const float* Dskip;
  const float* h0;
  void* y;
  float* h_last;
};

// Dequantize B and C once into the staging layout read by the scan: for every (b, g), the states
// are cut into planes of `ns` consecutive states (the states one wave owns), and each plane stores
// per step the ns B values followed by the ns C values: [B, Gbc, N/ns, L, 2*ns] fp32.
__global__ __launch_bounds__(256) void k_stage_bc(const int8_t* __restrict__ Bq,
                                                  const int8_t* __restrict__ Cq,
                                                  const float* __restrict__ Bs,
                                                  const float* __restrict__ Cs, int64_t B,
                                                  int Gbc, int N, int64_t L, int gs, int ns,
                                                  float* __restrict__ stage) {
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
  float vb = 0.0f, vc = 0.0f;  // rows past L are zero (read by the last batches, times delta = 0)
  if (t < L) {
    vb = scale_ok(sb) ? (float)Bq[r * L + t] * sb : 0.0f;
    vc = scale_ok(sc) ? (float)Cq[r * L + t] * sc : 0.0f;
  }
  const int plane = n / ns, k = n % ns;
  float* dst = stage + (((bg * (N / ns) + plane) * Lp + t) * (2 * ns));
  dst[k] = vb;
  dst[ns + k] = vc;
}

template <int XCODE>
__device__ __forceinline__ float xval(uint32_t byte, float s) {
  if (XCODE == QSSM_X_SOFTEDGE) return softedge_value(byte, s);
  return (float)(int8_t)(byte & 0xFFu) * s;
}

template <int NS, int W, int XCODE, int YF16, int kBatch>
__global__ __launch_bounds__(64 * W) void k_scan_m1(ScanParams p) {
  __shared__ float ybuf[2][W][kT][kLanes];
  constexpr int kS = 2 * NS;  // staged floats per step

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int64_t b = blockIdx.y;
  const int64_t d0 = (int64_t)blockIdx.x * kLanes;
  const int64_t d = d0 + lane;
  const bool valid = d < p.D;
  const int64_t dc = valid ? d : p.D - 1;  // clamped channel for loads
  const int64_t L = p.L;
  const int g = uniform((int)(d0 / p.dpg));

  // x scale (int8 value = s * q; soft-edge base scale), a valid scale is required, else 0
  float sx = p.x_scales[p.x_group_of[dc]];
  if (XCODE == QSSM_X_INT8 && !scale_ok(sx)) sx = 0.0f;
  const float Dd = p.Dskip ? p.Dskip[dc] : 0.0f;

  float a2[NS], h[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int n = w * NS + k;
    a2[k] = p.A[dc * p.N + n] * kLog2e;
    h[k] = p.h0 ? p.h0[(b * p.D + dc) * p.N + n] : 0.0f;
  }

  const float* __restrict__ drow = p.delta + (b * p.D + dc) * L;
  const uint8_t* __restrict__ xrow = reinterpret_cast<const uint8_t*>(p.x) + (b * p.D + dc) * L;
  // this wave's plane of staged (Bh, Ch): kS floats per step, read through the constant address
  // space (wave-uniform addresses -> scalar loads into SGPRs)
  const cfloat* st =
      (const cfloat*)(p.stage + ((b * p.Gbc + g) * (p.N / NS) + w) * (L + kPadRows) * kS);
  const bool vec_ok = (L % 16) == 0;

  float dl[kT];
  uint32_t xq[kT / 4];
  float dn[kT] = {};
  uint32_t xn[kT / 4] = {};

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
  float bcur[kBatch][kS], bnxt[kBatch][kS];
  auto sload = [&](int t0, float (&dst)[kBatch][kS]) {
    const cfloat* src = st + (int64_t)t0 * kS;
#pragma unroll
    for (int s2 = 0; s2 < kBatch; ++s2)
#pragma unroll
      for (int j = 0; j < kS; ++j) dst[s2][j] = src[s2 * kS + j];
  };

  load_block(0, dl, xq);
  sload(0, bcur);
  int buf = 0;
  for (int64_t tb = 0; tb < L; tb += kT) {
    if (tb + kT < L) load_block(tb + kT, dn, xn);

#pragma unroll
    for (int bt = 0; bt < kT; bt += kBatch) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the current batch has landed
      sload((int)tb + bt + kBatch, bnxt);
#pragma unroll
      for (int s2 = 0; s2 < kBatch; ++s2) {
        const int t = bt + s2;
        const float xh = xval<XCODE>((xq[t / 4] >> (8 * (t % 4))) & 0xFFu, sx);
        const float dt = dl[t];
        const float dtx = dt * xh;
        float yp;
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          const float dA = __builtin_amdgcn_exp2f(dt * a2[k]);
          h[k] = fmaf(dA, h[k], dtx * bcur[s2][k]);
          yp = (k == 0) ? bcur[s2][NS] * h[0] : fmaf(bcur[s2][NS + k], h[k], yp);
        }
        ybuf[buf][w][t][lane] = yp;
      }
#pragma unroll
      for (int s2 = 0; s2 < kBatch; ++s2)
#pragma unroll
        for (int j = 0; j < kS; ++j) bcur[s2][j] = bnxt[s2][j];
    }
    __syncthreads();

    // combine: wave w finalizes steps [w*kT/W, (w+1)*kT/W) of every channel of the block
    constexpr int kPer = kT / W;
    float yo[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int t = w * kPer + j;
      float sum = 0.0f;
#pragma unroll
      for (int ww = 0; ww < W; ++ww) sum += ybuf[buf][ww][t][lane];
      const float xh = xval<XCODE>((xq[t / 4] >> (8 * (t % 4))) & 0xFFu, sx);
      yo[j] = fmaf(Dd, xh, sum);
    }
    const int64_t t0 = tb + w * kPer;
    if (valid) {
      if (YF16) {
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
    buf ^= 1;
#pragma unroll
    for (int k = 0; k < kT; ++k) dl[k] = dn[k];
#pragma unroll
    for (int k = 0; k < kT / 4; ++k) xq[k] = xn[k];
  }

  if (valid && p.h_last) {
#pragma unroll
    for (int k = 0; k < NS; ++k) p.h_last[(b * p.D + d) * p.N + w * NS + k] = h[k];
  }
}

template <int NS, int W, int BATCH>
qssm_status launch_scan(const ScanParams& p, int xcode, int yf16, hipStream_t st) {
  dim3 grid((unsigned)cdiv(p.D, kLanes), (unsigned)p.B);
  dim3 block(64 * W);
  if (xcode == QSSM_X_INT8) {
    if (yf16) k_scan_m1<NS, W, QSSM_X_INT8, 1, BATCH><<<grid, block, 0, st>>>(p);
    else k_scan_m1<NS, W, QSSM_X_INT8, 0, BATCH><<<grid, block, 0, st>>>(p);
  } else {
    if (yf16) k_scan_m1<NS, W, QSSM_X_SOFTEDGE, 1, BATCH><<<grid, block, 0, st>>>(p);
    else k_scan_m1<NS, W, QSSM_X_SOFTEDGE, 0, BATCH><<<grid, block, 0, st>>>(p);
  }
  return launch_status("scan_w8a8");
}

// states per wave for a state size N (the workgroup has N / NS waves)
int states_per_wave(int64_t N) { return N == 8 ? 2 : (N == 64 ? 8 : 4); }

size_t stage_bytes(const qssm_scan_args* a) {
  return (size_t)a->batch * (size_t)a->bc_groups * (size_t)a->dstate *
         (size_t)(a->seqlen + kPadRows) * 2 * sizeof(float);
}

}  // namespace

extern "C" {

size_t qssm_scan_workspace_size(const qssm_scan_args* a) {
  if (!a || a->batch < 0 || a->seqlen < 0 || a->bc_groups < 1 || a->dstate < 1) return 0;
  return stage_bytes(a) + 256;
}

qssm_status qssm_scan_w8a8(const qssm_scan_args* a, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  clear_error();
  if (!a) return fail(QSSM_ERR_INVALID_ARG, "args is null");
  const int64_t B = a->batch, L = a->seqlen, D = a->dim, N = a->dstate;
  if (B < 0 || L < 0 || D < 1 || N < 1) return fail(QSSM_ERR_INVALID_ARG, "bad shape");
  if (L > 0x7fffff00LL) return fail(QSSM_ERR_UNSUPPORTED, "seqlen must be below 2^31 - 256");
  if (a->x_code != QSSM_X_INT8 && a->x_code != QSSM_X_SOFTEDGE)
    return fail(QSSM_ERR_INVALID_ARG, "x_code must be QSSM_X_INT8 or QSSM_X_SOFTEDGE");
  if (a->y_dtype != QSSM_F32 && a->y_dtype != QSSM_F16)
    return fail(QSSM_ERR_INVALID_ARG, "y_dtype must be QSSM_F32 or QSSM_F16");
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
  if (B == 0) return QSSM_OK;
  if (!a->x || !a->x_group_of || !a->x_scales || !a->delta || !a->A || !a->Bq || !a->Cq ||
      !a->B_scales || !a->C_scales || !a->y)
    return fail(QSSM_ERR_INVALID_ARG, "null required pointer");
  if (((uintptr_t)a->x | (uintptr_t)a->delta | (uintptr_t)a->y) % 16 != 0)
    return fail(QSSM_ERR_INVALID_ARG, "x, delta and y must be 16-byte aligned");
  const size_t need = stage_bytes(a);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(QSSM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  float* stage = reinterpret_cast<float*>(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  if ((size_t)((char*)stage - (char*)ws) + need > ws_bytes)
    return fail(QSSM_ERR_WORKSPACE, "workspace too small after 256-byte alignment");

  const int ns = states_per_wave(N);
  const int64_t nstage = B * a->bc_groups * N * (L + kPadRows);
  if (nstage > 0) {
    k_stage_bc<<<(unsigned)cdiv(nstage, 256), 256, 0, stream>>>(
        a->Bq, a->Cq, a->B_scales, a->C_scales, B, a->bc_groups, (int)N, L, a->bc_group_size, ns,
        stage);
    if (qssm_status s = launch_status("scan_w8a8 staging")) return s;
  }

  ScanParams p{B, L, D, N, a->x_groups, a->bc_groups, a->bc_group_size, (int32_t)dpg,
               a->x, a->x_group_of, a->x_scales, a->delta, a->A, stage, a->Dskip, a->h0,
               a->y, a->h_last};
  const int yf16 = a->y_dtype == QSSM_F16;
  switch (N) {
    case 4: return launch_scan<4, 1, 8>(p, a->x_code, yf16, stream);
    case 8: return launch_scan<2, 4, 16>(p, a->x_code, yf16, stream);
    case 16: return launch_scan<4, 4, 8>(p, a->x_code, yf16, stream);
    case 32: return launch_scan<4, 8, 8>(p, a->x_code, yf16, stream);
    default: return launch_scan<8, 8, 4>(p, a->x_code, yf16, stream);
  }
}

}  // extern "C"
