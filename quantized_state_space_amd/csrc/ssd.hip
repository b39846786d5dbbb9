// a8-a13: Mamba2 SSD chunked form with an int8 path.
//
// SSDi8 (abstract): a persistent INT8 path through the structured state-space duality, with
// activations quantized at cost-effective points; Quamba2 (abstract): W8A8 for the Mamba2 backbone.
// Per batch b, head h (B/C group g), chunk of Q = 256 steps with local indices i, j:
//   cum_i   = sum_{k<=i} delta_k A_h
//   G       = Ch Bh^T                               int8 MFMA, int32 per state group, fp32 scales
//   Y_intra = (G o exp(cum_i - cum_j) [j<=i] o delta_j) . xh           fp16 MFMA, fp32 accumulate
//   S       = sum_j w_j xh_j Bh_j^T,  w_j = delta_j e^{cum_Q - cum_j}
//             fp16 MFMA over time on fp16(w_j qx) and the B codes (default), or int8 MFMA on the
//             requantized r = sat8(RNE(qx * w_j / w_max)) (option); kept as F sx sB S16, S16 in
//             fp16, code units over a per-head bound that rules out overflow
//   H_c     = exp(cum_Q) H_{c-1} + S                  fp32 state passing
//   Y_inter = exp(cum_i) Ch . H_{c-1}^T               fp16 MFMA
//   y       = Y_intra + Y_inter + D_h xh
//
// Three kernels (the chunk states make one round trip through the workspace):
//   K1 k_ssd_chunk_state  one workgroup per (b, chunk, B/C group): B chunk transposed once into
//                         fp16 operands held in registers, then per head the chunk's cumsum
//                         (also written out for K3), the weighted x tile and a 64x128x256 MFMA.
//   K2 k_ssd_state_pass   per (b, h) state element: sequential over chunks, writes the state
//                         entering each chunk (fp16, C-scaled) and the final state.
//   K3 k_ssd_output       one workgroup per (b, chunk, B/C group): G^T is built once with int8 MFMA
//                         and kept in registers (8 waves, one query block of causal 32x32 tiles
//                         each, two waves per SIMD); per head the inter-chunk product, the
//                         intra-chunk product and the D term, with the next head's inputs
//                         arriving in LDS by direct loads meanwhile.
// The chunk states (K1) and y (K3) are written with nontemporal stores: they stream past the
// caches instead of evicting staged inputs or leaving dirty lines for the next kernel.
// MFMA lane layouts (verified on gfx950): operand lane l holds row/column l%32 and a run of
// consecutive k at offset (K/2)*(l/32); the 32x32 accumulator register r of lane l is element
// (8*(r/4) + 4*(l/32) + r%4, l%32).
#include <hip/hip_runtime.h>

#include <atomic>

#include "common.hpp"

using namespace qssm;

namespace {

constexpr int kQ = 256;   // chunk length
constexpr int kP = 64;    // head dim
constexpr int kN = 128;   // state size
constexpr int kGS = 16;   // state-group size (one int8 MFMA K step)
constexpr int kNSG = kN / kGS;
constexpr int kRow256 = 272;  // padded bytes of a [*][256] int8 LDS row
constexpr int kRow128 = 136;  // padded bytes of a [*][128] int8 LDS row
constexpr int kXtRow = 260;   // padded halves of a [*][256] fp16 LDS row (520 bytes)
constexpr int kHsRow = 136;   // padded halves of a [*][128] fp16 LDS row (272 bytes)
constexpr int kBufferWord3 = 0x00020000;  // buffer resource word 3 for raw 32-bit access (gfx9)
constexpr int kYPolicy = 2;  // cache policy of the y stores: nontemporal (streaming)
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima). Issued through the builtin, not
// inline asm, so that the compiler's wait insertion sees the direct LDS loads completed and does not
// add a vmcnt(0) of its own at the next LDS barrier (which would also wait for the y stores).
constexpr int kVmcnt0 = 0x0F70;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

struct SsdParams {
  int64_t B, L, nh, nc;
  int32_t Gbc, hpg, yf16, G;
  const int8_t* xq;
  const uint8_t* x_group_of;
  const float* x_scales;
  const float* delta;
  const float* A;
  const float* Dskip;
  const int8_t* Bq;
  const int8_t* Cq;
  const float* B_scales;
  const float* C_scales;
  const float* h0;
  void* y;
  float* h_last;
  _Float16* S;    // [B, nc, nh, P, N]: chunk states in code units over F, fp16 (see K1)
  float* F;       // [B, nc, nh]: chunk state factor, S = F * sx[p] * sB[n] * S16
  float* dec;     // [B, nc, nh]: exp(cum at the last step of the chunk)
  _Float16* Hh;   // [B, nc, nh, P, N]: sC(n) * state entering the chunk, fp16 (K3's operand)
  float* sxt;     // [nh, P]: x scale of each channel, 0 where invalid (written by K1, read by K3)
  float* cumw;    // [B, nc, nh, Q]: cumulative sum of delta * A within the chunk (K1 -> K3)
};

__device__ __forceinline__ float valid_or_zero(float s) { return scale_ok(s) ? s : 0.0f; }

// Inclusive prefix sum over the 256 threads of the block (one value each, in thread order).
__device__ __forceinline__ float block_scan(float v, float* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  float pre = 0.0f;
  for (int k = 0; k < w; ++k) pre += sh[k];
  __syncthreads();
  return v + pre;
}

__device__ __forceinline__ float block_max(float v, float* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if (lane == 0) sh[w] = v;
  __syncthreads();
  const float m = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
  __syncthreads();
  return m;
}

__device__ __forceinline__ uint32_t byte_of(uint32_t d, int e) { return (d >> (8 * e)) & 0xFFu; }

__device__ __forceinline__ v8h i8x8_to_h(int64_t v) {
  v8h o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (_Float16)(float)(int8_t)((v >> (8 * e)) & 0xFF);
  return o;
}


// 16 dwords (row r holds 4 bytes, columns 0..3) -> column e as 16 bytes (rows 0..15).
__device__ __forceinline__ uint4 column16(const uint32_t (&d)[16], int e) {
  uint4 o;
  o.x = byte_of(d[0], e) | byte_of(d[1], e) << 8 | byte_of(d[2], e) << 16 | byte_of(d[3], e) << 24;
  o.y = byte_of(d[4], e) | byte_of(d[5], e) << 8 | byte_of(d[6], e) << 16 | byte_of(d[7], e) << 24;
  o.z = byte_of(d[8], e) | byte_of(d[9], e) << 8 | byte_of(d[10], e) << 16 | byte_of(d[11], e) << 24;
  o.w = byte_of(d[12], e) | byte_of(d[13], e) << 8 | byte_of(d[14], e) << 16 | byte_of(d[15], e) << 24;
  return o;
}

// Loads of one head's delta (step tid) and x codes (rows 16 (tid / 16) .. + 15, codes
// 4 (tid % 16) .. + 3) into registers, issued one head ahead of their use in K1.
__device__ __forceinline__ void fetch_head(const SsdParams& p, int64_t b, int64_t c, int64_t t0,
                                              int q, int64_t h, int tid, float& dt,
                                              uint32_t (&x)[16], float& sx) {
  const int jb = tid / 16, p4 = tid % 16;
  dt = (tid < q) ? p.delta[(b * p.L + t0 + tid) * p.nh + h] : 0.0f;
  sx = valid_or_zero(p.x_scales[min((int)p.x_group_of[h * kP + (tid & (kP - 1))], p.G - 1)]);
  // rows advance by one time step; the opaque stride keeps the 16 row addresses from being
  // precomputed once for all heads (they would stay live across the caller's head loop)
  int64_t step = p.nh * kP;
  __asm__ volatile("" : "+s"(step));
  const int8_t* row = p.xq + ((b * p.L + t0 + jb * 16) * p.nh + h) * kP + p4 * 4;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int jj = jb * 16 + r;
    x[r] = (jj < q) ? *reinterpret_cast<const uint32_t*>(row + r * step) : 0u;
  }
}

// ---------------------------------------------------------------------------------------------
// K1: chunk states, S[p][n] = sum_j w_j xh_j[p] Bh_j[n], w_j = delta_j exp(cum_last - cum_j).
// I8 = false: fp16 operands fp16(w_j * qx[j][p]) and the exact B codes, fp32 accumulate. The
//             accumulator is at most 127^2 sum_j w_j (times 1 + 2^-11 for the fp16 operand) in
//             magnitude, so acc / sum_j w_j fits fp16 (|.| < 16200); it is stored so, with
//             F = sum_j w_j.
// I8 = true:  the weighted x is requantized per (b, chunk, head), r = sat8(RNE(qx * w_j / w_max)),
//             int8 MFMA with int32 accumulate (|acc| <= 127^2 * 256); stored as fp16(acc / 256)
//             with F = 256 w_max.
// Either way S = F * sx[p] * sB[n] * S16 (fp16 keeps a relative precision of 2^-11; the factors
// are applied in fp32 by K2).
constexpr int kXwRow = 264;  // padded halves of a [*][256] fp16 LDS row (528 bytes)

template <bool I8>
struct K1Smem {
  int8_t qBT[kN * kRow256];  // B chunk transposed, [n][j]
  int8_t rT[I8 ? kP * kRow256 : 16];                  // requantized x, [p][j] (I8)
  _Float16 xw[I8 ? 8 : kP * kXwRow];                  // weighted x, [p][j] (fp16)
  float wv[kQ];                                       // w_j (fp16 path) or w_j / w_max (I8)
  float sh[12];
};

template <bool I8>
__global__ __launch_bounds__(256) void k_ssd_chunk_state(SsdParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  K1Smem<I8>& s = *reinterpret_cast<K1Smem<I8>*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t c = blockIdx.x;
  const int64_t b = blockIdx.y / p.Gbc;
  const int g = (int)(blockIdx.y % p.Gbc);
  const int64_t t0 = c * kQ;
  const int q = (int)((p.L - t0) < kQ ? (p.L - t0) : kQ);

  // B chunk of group g, transposed to [n][j]; rows past the sequence are zero
  for (int u = tid; u < 16 * (kN / 4); u += 256) {
    const int jb = u / (kN / 4), n4 = u % (kN / 4);
    uint32_t d[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = jb * 16 + r;
      d[r] = (j < q) ? *reinterpret_cast<const uint32_t*>(
                           p.Bq + ((b * p.L + t0 + j) * p.Gbc + g) * kN + n4 * 4)
                     : 0u;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      *reinterpret_cast<uint4*>(s.qBT + (n4 * 4 + e) * kRow256 + jb * 16) = column16(d, e);
  }

  const int n = w * 32 + (lane & 31);  // this lane's output column (state)
  const int kh = lane >> 5;
  // fp16 path: the B codes of this lane's column as fp16 B operands, converted once for all heads
  v8h BB[I8 ? 1 : kQ / 16];
  if (!I8) {
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kQ / 16; ++ks)
      BB[ks] = i8x8_to_h(*reinterpret_cast<const int64_t*>(s.qBT + n * kRow256 + ks * 16 + 8 * kh));
  }

  float pf_dt, pf_sx;
  uint32_t pf_x[16];
  fetch_head(p, b, c, t0, q, (int64_t)g * p.hpg, tid, pf_dt, pf_x, pf_sx);
  for (int hh = 0; hh < p.hpg; ++hh) {
    const int64_t h = (int64_t)g * p.hpg + hh;
    const float Ah = p.A[h];
    const int j = tid;
    const float dt = pf_dt;
    const float cum = block_scan(dt * Ah, s.sh);
    p.cumw[((b * p.nc + c) * p.nh + h) * kQ + j] = cum;
    if (j == q - 1) s.sh[4] = cum;
    __syncthreads();
    const float cum_last = s.sh[4];
    const float wj = (j < q) ? dt * expf(cum_last - cum) : 0.0f;
    float wmax = 1.0f;
    if (I8) {
      wmax = block_max(wj, s.sh);
      s.wv[j] = (wmax > 0.0f) ? wj / wmax : 0.0f;
    } else {
      s.wv[j] = wj;
      // per-wave partial sums of w_j, combined after the barrier below
      float ws = wj;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) ws += __shfl_xor(ws, off, 64);
      if (lane == 0) s.sh[8 + w] = ws;
    }
    if (tid == 0) p.dec[(b * p.nc + c) * p.nh + h] = expf(cum_last);
    if (b == 0 && c == 0 && tid < kP) p.sxt[h * kP + tid] = pf_sx;
    __syncthreads();

    // weighted x tile, transposed [p][j]
    {
      const int jb = tid / 16, p4 = tid % 16;
      const uint32_t (&raw)[16] = pf_x;
      if (I8) {
        uint32_t d[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float rt = s.wv[jb * 16 + r];
          uint32_t word = 0u;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = (float)(int8_t)byte_of(raw[r], e) * rt;
            const int rq = (int)fminf(fmaxf(rintf(v), -128.0f), 127.0f);
            word |= ((uint32_t)rq & 0xFFu) << (8 * e);
          }
          d[r] = word;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<uint4*>(s.rT + (p4 * 4 + e) * kRow256 + jb * 16) = column16(d, e);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v8h lo, hi;
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            lo[r] = (_Float16)((float)(int8_t)byte_of(raw[r], e) * s.wv[jb * 16 + r]);
            hi[r] = (_Float16)((float)(int8_t)byte_of(raw[8 + r], e) * s.wv[jb * 16 + 8 + r]);
          }
          _Float16* dst = s.xw + (p4 * 4 + e) * kXwRow + jb * 16;
          *reinterpret_cast<v8h*>(dst) = lo;
          *reinterpret_cast<v8h*>(dst + 8) = hi;
        }
      }
    }
    __syncthreads();
    if (hh + 1 < p.hpg) fetch_head(p, b, c, t0, q, h + 1, tid, pf_dt, pf_x, pf_sx);

    // S16[p][n] for p in two 32-row tiles; wave w owns state columns [32w, 32w + 32)
    _Float16* Sout = p.S + ((b * p.nc + c) * p.nh + h) * (int64_t)(kP * kN);
    if (I8) {
      v16i acc0 = {}, acc1 = {};
#pragma unroll
      for (int ks = 0; ks < kQ / 32; ++ks) {
        const int ko = ks * 32 + 16 * kh;
        const v4i bv = *reinterpret_cast<const v4i*>(s.qBT + n * kRow256 + ko);
        const v4i a0 = *reinterpret_cast<const v4i*>(s.rT + (lane & 31) * kRow256 + ko);
        const v4i a1 = *reinterpret_cast<const v4i*>(s.rT + (32 + (lane & 31)) * kRow256 + ko);
        acc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bv, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bv, acc1, 0, 0, 0);
      }
      if (tid == 0) p.F[(b * p.nc + c) * p.nh + h] = 256.0f * wmax;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int prow = 8 * (r / 4) + 4 * kh + (r % 4);
        __builtin_nontemporal_store((_Float16)((float)acc0[r] * (1.0f / 256.0f)), &Sout[prow * kN + n]);
        __builtin_nontemporal_store((_Float16)((float)acc1[r] * (1.0f / 256.0f)),
                                    &Sout[(32 + prow) * kN + n]);
      }
    } else {
      v16f acc0 = {}, acc1 = {};
#pragma unroll
      for (int ks = 0; ks < kQ / 16; ++ks) {
        const int ko = ks * 16 + 8 * kh;
        const v8h bv = BB[ks];
        const v8h a0 = *reinterpret_cast<const v8h*>(s.xw + (lane & 31) * kXwRow + ko);
        const v8h a1 = *reinterpret_cast<const v8h*>(s.xw + (32 + (lane & 31)) * kXwRow + ko);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, bv, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, bv, acc1, 0, 0, 0);
      }
      const float wsum = s.sh[8] + s.sh[9] + s.sh[10] + s.sh[11];
      const float inv = (wsum > 0.0f) ? 1.0f / wsum : 0.0f;
      if (tid == 0) p.F[(b * p.nc + c) * p.nh + h] = wsum;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int prow = 8 * (r / 4) + 4 * kh + (r % 4);
        __builtin_nontemporal_store((_Float16)(acc0[r] * inv), &Sout[prow * kN + n]);
        __builtin_nontemporal_store((_Float16)(acc1[r] * inv), &Sout[(32 + prow) * kN + n]);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// K2: inter-chunk state passing, H_c = dec_c H_{c-1} + S_c in fp32, S_c = F sx[p] sB[n] S16. The
// state entering chunk c, scaled by the C scale of its state group, goes to slot c of Hh in fp16:
// exactly the operand of the inter-chunk product in K3 (which rounds it to fp16 anyway), at half
// the bytes.
__global__ __launch_bounds__(256) void k_ssd_state_pass(SsdParams p) {
  constexpr int kE4 = kP * kN / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= p.B * p.nh * kE4) return;
  const int64_t e4 = idx % kE4, bh = idx / kE4;
  const int64_t b = bh / p.nh, h = bh % p.nh;
  const int g = (int)(h / p.hpg);
  const int sgi = g * kNSG + (int)((4 * e4) % kN) / kGS;  // the 4 states share one state group
  const float sc = valid_or_zero(p.C_scales[sgi]);
  const float sxb = p.sxt[h * kP + (4 * e4) / kN] * valid_or_zero(p.B_scales[sgi]);
  float4 H = p.h0 ? reinterpret_cast<const float4*>(p.h0)[bh * kE4 + e4]
                  : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t c = 0; c < p.nc; ++c) {
    const int64_t slot = ((b * p.nc + c) * p.nh + h) * (int64_t)kE4 + e4;
    const v4h s16 = reinterpret_cast<const v4h*>(p.S)[slot];
    const float f = p.F[(b * p.nc + c) * p.nh + h] * sxb;
    const float4 s = make_float4(f * (float)s16[0], f * (float)s16[1], f * (float)s16[2],
                                 f * (float)s16[3]);
    const v4h hv = {(_Float16)(sc * H.x), (_Float16)(sc * H.y), (_Float16)(sc * H.z),
                    (_Float16)(sc * H.w)};
    reinterpret_cast<v4h*>(p.Hh)[slot] = hv;
    const float d = p.dec[(b * p.nc + c) * p.nh + h];
    H = make_float4(fmaf(d, H.x, s.x), fmaf(d, H.y, s.y), fmaf(d, H.z, s.z), fmaf(d, H.w, s.w));
  }
  if (p.h_last) reinterpret_cast<float4*>(p.h_last)[bh * kE4 + e4] = H;
}

// ---------------------------------------------------------------------------------------------
// K3: chunk outputs.
struct K3Smem {
  int8_t qB[kQ * kRow128];  // B chunk rows [j][n]
  int8_t qC[kQ * kRow128];  // C chunk rows [i][n]
  _Float16 xT[kP * kXtRow];  // x codes of the head, [p][j] (exact in fp16)
  _Float16 Hs[kP * kHsRow];  // sC(n) * H_prev[p][n]
  // The next head's inputs, written by direct global-to-LDS loads while the current head computes:
  // x codes in 1 KB blocks of 16 rows (row r of block jb at slot (r + jb) % 16, so that the
  // transposing reads below hit distinct banks), the entering state as stored in Hh, delta, sx.
  int8_t stx[kQ * kP];
  _Float16 sth[kP * kN];
  float stdt[kQ];
  float stcum[kQ];
  float stsx[kP];
  float cum[kQ];
  float dtv[kQ];
  float ecum[kQ];   // exp(cum_i)
  float cjv[kQ];    // exp(cum at the end of j's 32-block - cum_j) * delta_j
  float sxs[kP];
  float stad;  // staged D_h
  float dh;    // D_h of the current head
};
static_assert(offsetof(K3Smem, stcum) % 16 == 0 && offsetof(K3Smem, cum) % 16 == 0 &&
                  offsetof(K3Smem, dtv) % 16 == 0 &&
                  offsetof(K3Smem, ecum) % 16 == 0 && offsetof(K3Smem, cjv) % 16 == 0,
              "16-byte vector reads of the decay terms");


// Compiler-only fence: keeps one tile's work from being interleaved with the next tile's.
__device__ __forceinline__ void tile_fence() { __asm__ volatile("" ::: "memory"); }

__device__ __forceinline__ void build_g_tile(v16f& G, const K3Smem& s, const float* sBC, int I,
                                             int J, int lane) {
  const int kofs = 8 * (lane >> 5);
  G = v16f{};
#pragma unroll
  for (int sg = 0; sg < kNSG; ++sg) {
    int64_t a = *reinterpret_cast<const int64_t*>(s.qB + (J * 32 + (lane & 31)) * kRow128 + sg * kGS + kofs);
    int64_t bq = *reinterpret_cast<const int64_t*>(s.qC + (I * 32 + (lane & 31)) * kRow128 + sg * kGS + kofs);
    // empty asm that reads G and "rewrites" this group's operands: the MFMA of state group sg
    // cannot issue before the epilogue of group sg - 1, so one int32 accumulator is live at a time
    __asm__ volatile("" : "+v"(a), "+v"(bq) : "v"(G));
    const v16i acc = __builtin_amdgcn_mfma_i32_32x32x16_i8(a, bq, v16i{}, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) G[r] = fmaf(sBC[sg], (float)acc[r], G[r]);
  }
}

// G tile kept as fp16 (accumulator order): the M tile below is rounded to fp16 anyway.
struct GTile {
  v8h lo, hi;
};

__device__ __forceinline__ GTile pack_g(const v16f& G) {
  GTile t;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    t.lo[e] = (_Float16)G[e];
    t.hi[e] = (_Float16)G[8 + e];
  }
  return t;
}

// M tile = G o exp(cum_i - cum_j) [j <= i] o delta_j as two fp16 A operands (k-slots follow the
// accumulator rows of G, see the B operand gather below). Register r of lane l holds column
// j = 32 J + 4 (l / 32) + 8 (r / 4) + r % 4, so the column terms come in runs of four (16-byte
// reads, the same address for each half-wave). Each element is one mixed-precision fma from the
// fp16 G value, rounded once to fp16.
__device__ __forceinline__ void m_tile(const GTile& Gt, const K3Smem& s, int I, int J, int lane,
                                       v8h& a0, v8h& a1) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const int i = I * 32 + (lane & 31);  // this lane's query row
  const int jb = J * 32 + 4 * (lane >> 5);
  const float ci = s.cum[i];
  float f[16];
  if (J < I) {
    // both factors are at most 1 (cum does not increase): no overflow for long decays
    const float ri = __expf(ci - s.cum[J * 32 + 31]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4f c4 = *reinterpret_cast<const v4f*>(s.cjv + jb + 8 * q);
#pragma unroll
      for (int k = 0; k < 4; ++k) f[4 * q + k] = ri * c4[k];
    }
  } else {
    // diagonal tile, branch-free: past the diagonal cum_j <= cum_i, the clamped exponent is 0
    // and the select discards the value
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4f c4 = *reinterpret_cast<const v4f*>(s.cum + jb + 8 * q);
      const v4f d4 = *reinterpret_cast<const v4f*>(s.dtv + jb + 8 * q);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float e = __expf(fminf(ci - c4[k], 0.0f)) * d4[k];
        f[4 * q + k] = (jb + 8 * q + k <= i) ? e : 0.0f;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a0[e] = (_Float16)fmaf((float)Gt.lo[e], f[e], 0.0f);
    a1[e] = (_Float16)fmaf((float)Gt.hi[e], f[8 + e], 0.0f);
  }
}

// x B operand for MFMA mm of tile column block J: lane l supplies column p and the 8 j's whose G
// accumulator rows sit in registers 8 mm .. 8 mm + 7 of the same lane half
__device__ __forceinline__ v8h x_operand(const K3Smem& s, int J, int mm, int pt, int lane) {
  const int j0 = J * 32 + 16 * mm + 4 * (lane >> 5);
  const _Float16* row = s.xT + (pt * 32 + (lane & 31)) * kXtRow;
  const v4h lo = *reinterpret_cast<const v4h*>(row + j0);
  const v4h hi = *reinterpret_cast<const v4h*>(row + j0 + 8);
  return v8h{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Workgroup barrier that orders LDS only: outstanding global stores (and the direct LDS loads,
// which every wave waits for itself with vmcnt before it arrives) are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Row r (0..15) of a 16-row x block jb sits at slot ((r ^ ((r >> 3) << 1)) + jb) & 15 of its 1 KB
// staging block (a bijection). With eight rows per thread in the transposing reads, the four row
// blocks a wave reads at one step land in four distinct 64-byte bank groups. stx_row inverts it.
__device__ __forceinline__ int stx_slot(int r, int jb) { return ((r ^ ((r >> 3) << 1)) + jb) & 15; }
__device__ __forceinline__ int stx_row(int slot, int jb) {
  const int t = (slot - jb) & 15;
  return t ^ ((t >> 3) << 1);
}

// Issues the direct global-to-LDS loads of head h's inputs into the staging area (no registers
// are held: the loads complete in the background and are waited for with vmcnt before use). Rows
// past the sequence are clamped to the last valid row here and masked by the consumer.
__device__ __forceinline__ void stage_head(const SsdParams& p, K3Smem& s, int64_t b, int64_t c,
                                           int64_t t0, int q, int64_t h, int wave, int lane) {
  // LDS destinations are wave-uniform (they go to M0): byte offsets from the staging base, made
  // uniform explicitly
  unsigned char* const base = reinterpret_cast<unsigned char*>(&s);
  // an opaque lane id: the per-lane source addresses are recomputed at each call instead of being
  // hoisted out of the caller's head loop, where they would stay live across the products
  __asm__ volatile("" : "+v"(lane));
  // x codes: wave w fills blocks 2w and 2w + 1 (16 rows of 64 bytes each, 4 lanes per row);
  // lane l writes slot l / 4 of its block, which holds row stx_row(l / 4, block)
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int jb = 2 * wave + k;
    const int r = stx_row(lane >> 2, jb);
    const int j = min(jb * 16 + r, q - 1);
    const int8_t* src = p.xq + ((b * p.L + t0 + j) * p.nh + h) * kP + (lane & 3) * 16;
    const int dst = uniform((int)offsetof(K3Smem, stx) + jb * 1024);
    __builtin_amdgcn_global_load_lds(src, base + dst, 16, 0, 0);
  }
  // entering state: 16 KB contiguous, 1 KB per instruction
  const _Float16* hsrc = p.Hh + ((b * p.nc + c) * p.nh + h) * (int64_t)(kP * kN);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int blk = 2 * wave + k;
    const int dst = uniform((int)offsetof(K3Smem, sth) + blk * 1024);
    __builtin_amdgcn_global_load_lds(hsrc + blk * 512 + lane * 8, base + dst, 16, 0, 0);
  }
  if (wave < 4) {  // delta of steps 64 w .. 64 w + 63
    const int j = min(wave * 64 + lane, q - 1);
    const int dst = uniform((int)offsetof(K3Smem, stdt) + wave * 256);
    __builtin_amdgcn_global_load_lds(p.delta + (b * p.L + t0 + j) * p.nh + h, base + dst, 4, 0, 0);
  } else if (wave == 4) {
    const int dst = uniform((int)offsetof(K3Smem, stsx));
    __builtin_amdgcn_global_load_lds(p.sxt + h * kP + lane, base + dst, 4, 0, 0);
  } else if (wave == 5) {  // the chunk's cumulative decay exponents, 1 KB contiguous
    const int dst = uniform((int)offsetof(K3Smem, stcum));
    __builtin_amdgcn_global_load_lds(p.cumw + ((b * p.nc + c) * p.nh + h) * kQ + lane * 4, base + dst,
                                     16, 0, 0);
  } else if (wave == 6 && lane == 0 && p.Dskip) {
    const int dst = uniform((int)offsetof(K3Smem, stad));
    __builtin_amdgcn_global_load_lds(p.Dskip + h, base + dst, 4, 0, 0);
  }
}

// Eight waves; wave v owns query block I = v (v < 4) or 11 - v (v >= 4), so that the two waves
// on one SIMD (v and v + 4) hold blocks s and 7 - s: 9 causal tiles per SIMD. A wave keeps the
// G tiles (I, J <= I) of its block in registers and produces all 64 output columns of it. Each
// head's inputs arrive in LDS by direct loads issued during the previous head's products.
__global__ __launch_bounds__(512) void k_ssd_output(SsdParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  K3Smem& s = *reinterpret_cast<K3Smem*>(smem_raw);
  const int tid = threadIdx.x;
  const int64_t c = blockIdx.x;
  const int64_t b = blockIdx.y / p.Gbc;
  const int g = (int)(blockIdx.y % p.Gbc);
  const int64_t t0 = c * kQ;
  const int q = (int)((p.L - t0) < kQ ? (p.L - t0) : kQ);

  // B and C chunk rows of group g (zero past the sequence), 8-byte LDS stores
  if (tid < kQ) {
    const int j = tid;
    const int64_t* bsrc = reinterpret_cast<const int64_t*>(p.Bq + ((b * p.L + t0 + j) * p.Gbc + g) * kN);
    const int64_t* csrc = reinterpret_cast<const int64_t*>(p.Cq + ((b * p.L + t0 + j) * p.Gbc + g) * kN);
#pragma unroll
    for (int k = 0; k < kN / 8; ++k) {
      *reinterpret_cast<int64_t*>(s.qB + j * kRow128 + 8 * k) = (j < q) ? bsrc[k] : 0;
      *reinterpret_cast<int64_t*>(s.qC + j * kRow128 + 8 * k) = (j < q) ? csrc[k] : 0;
    }
  }
  float sBC[kNSG];  // sB * sC per state group (wave-uniform)
#pragma unroll
  for (int sg = 0; sg < kNSG; ++sg)
    sBC[sg] = valid_or_zero(p.B_scales[g * kNSG + sg]) * valid_or_zero(p.C_scales[g * kNSG + sg]);
  lds_barrier();
  // the first head's inputs load while G is built
  stage_head(p, s, b, c, t0, q, (int64_t)g * p.hpg, uniform(tid >> 6), tid & 63);

  GTile G[8];
  {
    const int lane = tid & 63;
    const int v = uniform(tid >> 6);
    const int I = v < 4 ? v : 11 - v;
#pragma unroll
    for (int J = 0; J < 8; ++J) {
      if (J <= I) {
        v16f Gf;
        build_g_tile(Gf, s, sBC, I, J, lane);
        G[J] = pack_g(Gf);
      }
      tile_fence();
    }
  }
  // the C codes of this wave's query block as fp16 A operands of the inter-chunk product (the
  // same for every head)
  v8h QC[kN / 16];
  {
    const int lane = tid & 63;
    const int I = uniform(uniform(tid >> 6) < 4 ? uniform(tid >> 6) : 11 - uniform(tid >> 6));
#pragma unroll
    for (int ks = 0; ks < kN / 16; ++ks)
      QC[ks] = i8x8_to_h(*reinterpret_cast<const int64_t*>(s.qC + (I * 32 + (lane & 31)) * kRow128 +
                                                           ks * 16 + 8 * (lane >> 5)));
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);

  const int rs = (int)(p.nh * kP);  // row stride of y in elements
  const bool full = q == kQ;
  for (int hh = 0; hh < p.hpg; ++hh) {
    const int64_t h = (int64_t)g * p.hpg + hh;
    // every wave has waited for its own staging loads of head h and is done with head h - 1
    lds_barrier();
    // decay terms of head h
    if (tid < kQ) {
      const int j = tid;
      const float dt = (tid < q) ? s.stdt[j] : 0.0f;
      const float cum = s.stcum[j];
      s.cum[j] = cum;
      s.dtv[j] = dt;
      s.ecum[j] = expf(cum);
      // exp(cum at the end of j's 32-block - cum_j) * delta_j; that step sits in this wave
      const float cl = __shfl(cum, (tid & 63) | 31, 64);
      s.cjv[j] = expf(cl - cum) * dt;
    }
    if (tid < kP) s.sxs[tid] = s.stsx[tid];
    if (tid == 0) s.dh = p.Dskip ? s.stad : 0.0f;
    // state entering the chunk (sC-scaled fp16 rows [p][n] of 128 halves), into padded rows
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int u = tid + 512 * k;
      *reinterpret_cast<uint4*>(s.Hs + (u / 16) * kHsRow + (u % 16) * 8) =
          *reinterpret_cast<const uint4*>(s.sth + u * 8);
    }
    {
      // x codes of head h, transposed [p][j] in fp16 (zero for an invalid x scale and past the
      // sequence): thread (jh, p4) takes rows 8 jh .. 8 jh + 7, channels 4 p4 .. 4 p4 + 3
      const int jh = tid / 16, p4 = tid % 16;
      const int jb = jh >> 1, r0 = 8 * (jh & 1);
      uint32_t raw[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint32_t d = *reinterpret_cast<const uint32_t*>(s.stx + jb * 1024 + stx_slot(r0 + r, jb) * 64 + p4 * 4);
        raw[r] = (jh * 8 + r < q) ? d : 0u;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pc = p4 * 4 + e;
        const bool on = s.stsx[pc] > 0.0f;
        _Float16* dst = s.xT + pc * kXtRow + jh * 8;
#pragma unroll
        for (int r4 = 0; r4 < 2; ++r4) {
          v4h vv;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            vv[k] = on ? (_Float16)(float)(int8_t)byte_of(raw[4 * r4 + k], e) : (_Float16)0.0f;
          *reinterpret_cast<v4h*>(dst + 4 * r4) = vv;
        }
      }
    }
    lds_barrier();
    // the staging area is free: the next head's inputs load during this head's products
    if (hh + 1 < p.hpg) stage_head(p, s, b, c, t0, q, h + 1, uniform(tid >> 6), tid & 63);

    // Opaque copies of the lane and wave ids: the tile addresses below do not depend on the head,
    // and hoisting all of them out of the head loop would keep them live across it (spills).
    int lane = tid & 63;
    __asm__ volatile("" : "+v"(lane));
    int v = uniform(tid >> 6);
    __asm__ volatile("" : "+s"(v));
    const int I = uniform(v < 4 ? v : 11 - v);  // (the asm output is not known to be uniform)
    const int kofs = 8 * (lane >> 5);
    v16f Y[2] = {};
    // Y_inter = exp(cum_i) * qC[i, :] . Hs[:, p]
#pragma unroll
    for (int ks = 0; ks < kN / 16; ++ks) {
      const v8h a = QC[ks];
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const v8h bv = *reinterpret_cast<const v8h*>(s.Hs + (pt * 32 + (lane & 31)) * kHsRow + ks * 16 + kofs);
        Y[pt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bv, Y[pt], 0, 0, 0);
      }
    }
    // row scale exp(cum_i), column scale 1 / sx[p] (the intra part accumulates raw x codes);
    // register r holds row i = 32 I + 4 (lane / 32) + 8 (r / 4) + r % 4
    {
      typedef float v4f __attribute__((ext_vector_type(4)));
      float er[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f e4 = *reinterpret_cast<const v4f*>(s.ecum + I * 32 + 4 * (lane >> 5) + 8 * q);
#pragma unroll
        for (int k = 0; k < 4; ++k) er[4 * q + k] = e4[k];
      }
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const float sx = s.sxs[pt * 32 + (lane & 31)];
        const float inv = (sx > 0.0f) ? 1.0f / sx : 1.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) Y[pt][r] *= er[r] * inv;
      }
    }
    // Y_intra on top, tile by tile
#pragma unroll
    for (int J = 0; J < 8; ++J) {
      tile_fence();
      if (J <= I) {
        // opaque per head: keeps the fp32 widening of the G tile inside the head loop (hoisted,
        // the widened copies of all tiles would stay live and spill)
        __asm__ volatile("" : "+v"(G[J].lo), "+v"(G[J].hi));
        v8h a0, a1;
        m_tile(G[J], s, I, J, lane, a0, a1);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          const v8h b0 = x_operand(s, J, 0, pt, lane);
          const v8h b1 = x_operand(s, J, 1, pt, lane);
          Y[pt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, Y[pt], 0, 0, 0);
          Y[pt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, Y[pt], 0, 0, 0);
        }
      }
    }
    tile_fence();
    // the staging loads were issued long before; waiting here keeps the y stores below out of
    // the count waited for at the next head's start
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    // y = sx * acc + D * xh; rows past the sequence (ragged last chunk) are not stored
    const float Dh = s.dh;
    const int64_t base = ((b * p.L + t0) * p.nh + h) * kP;  // y[b, t0, h, 0]
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const int pc = pt * 32 + (lane & 31);
      const float sx = s.sxs[pc];
      const float mult = (sx > 0.0f) ? sx : 1.0f;
      const float Dsx = Dh * sx;
      float yv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4h x4 = *reinterpret_cast<const v4h*>(s.xT + pc * kXtRow + I * 32 + 4 * (lane >> 5) + 8 * q);
#pragma unroll
        for (int k = 0; k < 4; ++k) yv[4 * q + k] = fmaf(Dsx, (float)x4[k], mult * Y[pt][4 * q + k]);
      }
      // register r holds row 32 I + 8 (r / 4) + r % 4 + 4 (lane / 32): buffer stores with the
      // head's y block as the resource, a per-register wave-uniform row offset (soffset) and one
      // per-lane offset, so the stores need no per-lane 64-bit address arithmetic (all offsets fit
      // 32 bits: nheads <= 2^14 is checked on the host)
      const int ilane = 4 * (lane >> 5);
      const int esz = p.yf16 ? 2 : 4;
      const uint64_t ya = reinterpret_cast<uint64_t>(static_cast<char*>(p.y) + base * esz);
      void* const yblk = reinterpret_cast<void*>(
          ((uint64_t)(uint32_t)uniform((int)(ya >> 32)) << 32) | (uint32_t)uniform((int)ya));
      const __amdgpu_buffer_rsrc_t yrs =
          __builtin_amdgcn_make_buffer_rsrc(yblk, (short)0, 0x7FFFFFFF, kBufferWord3);
      const int voff = (ilane * rs + pc) * esz;
      // the full-chunk path stores unconditionally; the ragged last chunk masks rows past q
      if (p.yf16) {
        if (full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ir = I * 32 + 8 * (r / 4) + (r % 4);
            __builtin_amdgcn_raw_buffer_store_b16(
                __builtin_bit_cast(unsigned short, __float2half_rn(yv[r])), yrs, voff, uniform(ir * rs * 2), kYPolicy);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ir = I * 32 + 8 * (r / 4) + (r % 4);
            if (ir + ilane < q)
              __builtin_amdgcn_raw_buffer_store_b16(
                  __builtin_bit_cast(unsigned short, __float2half_rn(yv[r])), yrs, voff, uniform(ir * rs * 2), kYPolicy);
          }
        }
      } else {
        if (full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ir = I * 32 + 8 * (r / 4) + (r % 4);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, yv[r]), yrs, voff,
                                                  uniform(ir * rs * 4), kYPolicy);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ir = I * 32 + 8 * (r / 4) + (r % 4);
            if (ir + ilane < q)
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, yv[r]), yrs, voff,
                                                    uniform(ir * rs * 4), kYPolicy);
          }
        }
      }
    }
  }
}

// The dynamic-LDS limit of a kernel is raised once per device (hipFuncSetAttribute applies on the
// current device; two threads racing both make the same idempotent call).
constexpr int kMaxDevices = 64;
enum { kAttrK1F16 = 0, kAttrK1I8 = 1, kAttrK3 = 2 };
std::atomic<bool> g_lds_raised[3][kMaxDevices];

bool raise_lds_limit(int which, const void* fn, size_t bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached && g_lds_raised[which][dev].load(std::memory_order_acquire)) return true;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess)
    return false;
  if (cached) g_lds_raised[which][dev].store(true, std::memory_order_release);
  return true;
}

struct WsLayout {
  size_t s_bytes, f_off, dec_off, hh_off, sx_off, cum_off, total;
};

// workspace: S16 (fp16 chunk states), F, dec, Hh (fp16 entering states), sxt, cumw, each
// 256-byte aligned
WsLayout ws_layout(const qssm_ssd_args* a) {
  const int64_t nc = (a->seqlen + kQ - 1) / kQ;
  const size_t elems = (size_t)a->batch * nc * a->nheads * kP * kN;
  WsLayout w;
  w.s_bytes = elems * sizeof(_Float16);
  w.f_off = (w.s_bytes + 255) & ~(size_t)255;
  w.dec_off = (w.f_off + (size_t)a->batch * nc * a->nheads * sizeof(float) + 255) & ~(size_t)255;
  w.hh_off = (w.dec_off + (size_t)a->batch * nc * a->nheads * sizeof(float) + 255) & ~(size_t)255;
  w.sx_off = (w.hh_off + elems * sizeof(_Float16) + 255) & ~(size_t)255;
  w.cum_off = (w.sx_off + (size_t)a->nheads * kP * sizeof(float) + 255) & ~(size_t)255;
  w.total = w.cum_off + (size_t)a->batch * nc * a->nheads * kQ * sizeof(float) + 256;
  return w;
}

}  // namespace

extern "C" {

size_t qssm_ssd_workspace_size(const qssm_ssd_args* a) {
  if (!a || a->batch < 0 || a->seqlen < 0 || a->nheads < 1) return 0;
  return ws_layout(a).total + 256;
}

qssm_status qssm_ssd_chunk_int8(const qssm_ssd_args* a, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  clear_error();
  if (!a) return fail(QSSM_ERR_INVALID_ARG, "args is null");
  const int64_t B = a->batch, L = a->seqlen, nh = a->nheads;
  if (B < 0 || L < 0 || nh < 1 || a->headdim < 1 || a->dstate < 1)
    return fail(QSSM_ERR_INVALID_ARG, "bad shape");
  if (a->ngroups < 1 || nh % a->ngroups != 0)
    return fail(QSSM_ERR_INVALID_ARG, "ngroups must divide nheads");
  if (a->x_groups < 1 || a->x_groups > 256) return fail(QSSM_ERR_INVALID_ARG, "x_groups not in 1..256");
  if (a->bc_group_size < 1 || a->dstate % a->bc_group_size != 0)
    return fail(QSSM_ERR_INVALID_ARG, "bc_group_size must divide dstate");
  if (a->y_dtype != QSSM_F32 && a->y_dtype != QSSM_F16)
    return fail(QSSM_ERR_INVALID_ARG, "y_dtype must be QSSM_F32 or QSSM_F16");
  if (a->fused != 0) return fail(QSSM_ERR_UNSUPPORTED, "fused must be 0");
  if (a->state_mma != QSSM_MMA_F16 && a->state_mma != QSSM_MMA_I8)
    return fail(QSSM_ERR_INVALID_ARG, "state_mma must be QSSM_MMA_F16 or QSSM_MMA_I8");
  if (a->chunk != kQ || a->headdim != kP || a->dstate != kN || a->bc_group_size != kGS)
    return fail(QSSM_ERR_UNSUPPORTED,
                "the library implements chunk=256, headdim=64, dstate=128, bc_group_size=16");
  if (L > ((int64_t)1 << 40)) return fail(QSSM_ERR_UNSUPPORTED, "seqlen too large");
  if (nh > (1 << 14)) return fail(QSSM_ERR_UNSUPPORTED, "nheads too large");
  if (B == 0) return QSSM_OK;
  // the per-step buffers are not touched when L == 0 and may then be null
  if (!a->x_group_of || !a->x_scales || !a->A || !a->B_scales || !a->C_scales ||
      (L > 0 && (!a->xq || !a->delta || !a->Bq || !a->Cq || !a->y)))
    return fail(QSSM_ERR_INVALID_ARG, "null required pointer");
  if (((uintptr_t)a->xq | (uintptr_t)a->Bq | (uintptr_t)a->Cq) % 16 != 0 ||
      (a->h0 && (uintptr_t)a->h0 % 16 != 0) || (a->h_last && (uintptr_t)a->h_last % 16 != 0))
    return fail(QSSM_ERR_INVALID_ARG, "xq, Bq, Cq, h0 and h_last must be 16-byte aligned");
  const WsLayout wl = ws_layout(a);
  if (!ws || ws_bytes < wl.total + 256)
    return fail(QSSM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", wl.total + 256,
                ws_bytes);
  char* base = reinterpret_cast<char*>(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  const int64_t nc = (L + kQ - 1) / kQ;
  SsdParams p{B, L, nh, nc, a->ngroups, (int32_t)(nh / a->ngroups), a->y_dtype == QSSM_F16,
              a->x_groups,
              a->xq, a->x_group_of, a->x_scales, a->delta, a->A, a->Dskip, a->Bq, a->Cq,
              a->B_scales, a->C_scales, a->h0, a->y, a->h_last,
              reinterpret_cast<_Float16*>(base), reinterpret_cast<float*>(base + wl.f_off),
              reinterpret_cast<float*>(base + wl.dec_off),
              reinterpret_cast<_Float16*>(base + wl.hh_off),
              reinterpret_cast<float*>(base + wl.sx_off),
              reinterpret_cast<float*>(base + wl.cum_off)};
  if ((int64_t)B * a->ngroups > 65535 || nc > 0x7fffffff)
    return fail(QSSM_ERR_UNSUPPORTED, "grid too large");
  const dim3 grid((unsigned)nc, (unsigned)(B * a->ngroups));
  if (nc > 0) {
    const int i8 = a->state_mma == QSSM_MMA_I8;
    const void* k1 = i8 ? reinterpret_cast<const void*>(&k_ssd_chunk_state<true>)
                        : reinterpret_cast<const void*>(&k_ssd_chunk_state<false>);
    const size_t k1_lds = i8 ? sizeof(K1Smem<true>) : sizeof(K1Smem<false>);
    if (!raise_lds_limit(i8 ? kAttrK1I8 : kAttrK1F16, k1, k1_lds))
      return fail(QSSM_ERR_DEVICE, "cannot raise the LDS limit of the SSD chunk-state kernel");
    if (i8) k_ssd_chunk_state<true><<<grid, 256, k1_lds, stream>>>(p);
    else k_ssd_chunk_state<false><<<grid, 256, k1_lds, stream>>>(p);
    if (qssm_status s = launch_status("ssd chunk state")) return s;
  }
  k_ssd_state_pass<<<(unsigned)cdiv(B * nh * (kP * kN / 4), 256), 256, 0, stream>>>(p);
  if (qssm_status s = launch_status("ssd state passing")) return s;
  if (nc > 0) {
    if (!raise_lds_limit(kAttrK3, reinterpret_cast<const void*>(&k_ssd_output), sizeof(K3Smem)))
      return fail(QSSM_ERR_DEVICE, "cannot raise the LDS limit of the SSD output kernel");
    k_ssd_output<<<grid, 512, sizeof(K3Smem), stream>>>(p);
    if (qssm_status s = launch_status("ssd output")) return s;
  }
  return QSSM_OK;
}

}  // extern "C"
