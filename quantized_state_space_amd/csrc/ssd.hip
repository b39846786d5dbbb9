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
//             requantized r = sat8(RNE(qx * w_j / w_max)) with int32 accumulate (option; the
//             weights and the rounding decisions in fp64)
//   H_c     = exp(cum_Q) H_{c-1} + S                  fp32 state passing
//   Y_inter = exp(cum_i) Ch . H_{c-1}^T               fp16 MFMA
//   y       = Y_intra + Y_inter + D_h xh
//
// Two kernels:
//   K1 k_ssd_state   one workgroup per (b, head), chunks in order: per chunk the cumsum (written
//                    out for K2), the weights, the transposed B chunk and weighted x tile in LDS, the
//                    chunk state S^T (rows n, columns p) on MFMA, then the state entering the chunk
//                    is written out for K2 (fp16, C-scaled, in the exact register order of K2's MFMA
//                    operand) and H is updated in fp32 registers. The final H is h_last.
//   K2 k_ssd_output  one workgroup per (b, chunk, B/C group): G^T is built once with int8 MFMA
//                    and kept in registers (8 waves, one query block of causal 32x32 tiles
//                    each, two waves per SIMD); per head the inter-chunk product, the
//                    intra-chunk product and the D term, with the next head's inputs
//                    arriving in LDS by direct loads meanwhile.
// y is written with nontemporal stores: it streams past the caches instead of evicting staged
// inputs or leaving dirty lines for the next kernel.
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
constexpr int kSlotsA = 5;    // causal tiles of the waves of the first half (fp16 intra product)
constexpr int kSlotsB = 4;    // causal tiles of the waves of the second half
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
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

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
  _Float16* Hh;   // [B, nc, nh, 16 KB]: sC(n) * state entering the chunk, fp16, K2's operand order
  float* sxt;     // [nh, P]: x scale of each channel, 0 where invalid (written by K1, read by K2)
  float* cumw;    // [B, nc, nh, Q]: cumulative sum of delta * A within the chunk (K1 -> K2)
  int32_t yi8, Gy;            // int8 output, number of output groups
  const uint8_t* y_group_of;  // int8 output: [nh * P]
  const float* y_scales;      // int8 output: [Gy]
  const float* y_bias;        // int8 output: [nh * P] or NULL
  float* syt;                 // [nh, P]: output scale of each channel (written by K1, read by K2)
  int32_t intra8;             // int8 intra-chunk output (row-requantized weights, int8 MFMA)
};

__device__ __forceinline__ float valid_or_zero(float s) { return scale_ok(s) ? s : 0.0f; }

// Workgroup barrier that orders LDS only: outstanding global loads and stores are not waited for
// (direct LDS loads are waited for with vmcnt by every wave before it arrives, where needed).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t byte_of(uint32_t d, int e) { return (d >> (8 * e)) & 0xFFu; }

__device__ __forceinline__ v8h i8x8_to_h(int64_t v) {
  v8h o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (_Float16)(float)(int8_t)((v >> (8 * e)) & 0xFF);
  return o;
}


// 8 rows of 8 bytes (d[r] holds row r) -> column e (0..7) as 8 bytes (rows 0..7).
__device__ __forceinline__ uint2 column8(const v2u (&d)[8], int e) {
  const int k = e >> 2, b = e & 3;
  uint2 o;
  o.x = byte_of(d[0][k], b) | byte_of(d[1][k], b) << 8 | byte_of(d[2][k], b) << 16 |
        byte_of(d[3][k], b) << 24;
  o.y = byte_of(d[4][k], b) | byte_of(d[5][k], b) << 8 | byte_of(d[6][k], b) << 16 |
        byte_of(d[7][k], b) << 24;
  return o;
}

// ---------------------------------------------------------------------------------------------
// K1: chunk states and their passing. One workgroup (8 waves) per pair of heads of one (b, B/C
// group): waves 0-3 run head 2k, waves 4-7 head 2k + 1 (a half with no head, when the group has an
// odd number of heads, repeats head 2k), chunks in order. The two heads share
// the transposed B chunk. In a half, wave w owns states n in [32w, 32w + 32) and the state H^T
// lives in two 32x32 fp32 accumulator tiles per wave (columns p in [0, 32) and [32, 64)): register
// r of lane l holds H[p = 32 pt + l % 32][n = 32 w + 8 (r / 4) + 4 (l / 32) + r % 4]. Per chunk:
//   S^T[n][p] = sum_j qB_j[n] * v_j[p], on MFMA with K = time:
//     I8 = false: v = fp16(w_j qx_j[p]) and the B codes in fp16, fp32 accumulate; S^T = sB sx acc.
//     I8 = true:  v = r_j[p] = sat8(RNE(qx_j[p] w_j / w_max)), w_j, w_max and the decision in
//                 fp64 (cum in fp64 from the exact products delta * A); int8 MFMA with int32
//                 accumulate; S^T = w_max sB sx acc.
//   The state entering the chunk goes out first: registers 8 kb .. 8 kb + 7 of tile pt hold, for
//   ks = 2 w + kb, the states n = 16 ks + 4 (l / 32) + {0..3, 8..11} of column p: exactly the fp16
//   B operand K2's lane l needs for its inter-chunk product (column p, K block ks, in that
//   within-block order), so each (pt, ks) pair is stored as 1 KB, 16 bytes per lane.
//   Then H = exp(cum_last) H + S (fp32, sB and sx applied as two products: their own product
//   can leave the fp32 range while H does not).
// Loads run one chunk ahead, into registers (B and x codes as 8 rows of 8 bytes per thread, one
// delta per thread), with no wait before their first use; the barriers order LDS only. They go
// through buffer resources that end with the batch's sequence, so that rows past it read as zero
// with no clamp or mask. Each step's delta is loaded once per workgroup and shared through LDS
// (written at the end of the chunk before, read after its closing barrier): a delta load touches
// one cache line per lane, so loading the whole chunk's deltas in every wave cost more cache
// lookups than the B and x codes together.
constexpr int kXwRow = 264;  // padded halves of a [*][256] fp16 LDS row (528 bytes)

template <bool I8>
struct K1Smem {
  _Float16 qBh[I8 ? 8 : kN * kXwRow];        // B chunk transposed, [n][j], fp16 (fp16 path)
  int8_t qBT[I8 ? kN * kRow256 : 16];        // B chunk transposed, [n][j], int8 (I8)
  int8_t rT[I8 ? 2 * kP * kRow256 : 16];    // requantized x per head, [p][j] (I8)
  _Float16 xw[I8 ? 8 : 2 * kP * kXwRow];    // weighted x per head, [p][j] (fp16)
  double ratio[I8 ? 2 * kQ : 1];            // w_j / w_max per head (I8)
  float wv[I8 ? 1 : 2 * kQ];                // w_j per head (fp16 path)
  float dts[2 * kQ];                        // delta of the chunk per head
  float sxp[2 * kP];                        // x scale of each channel of each head (0: invalid)
  float sh[16];
  double shd[16];
};

// Raw buffer resource over n bytes at ptr (offsets are 32-bit: the host checks that one
// sequence's codes, steps and deltas stay below 2^31 bytes); loads past n bytes return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t seq_rsrc(const void* ptr, int64_t n) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  void* const u = reinterpret_cast<void*>(((uint64_t)(uint32_t)uniform((int)(a >> 32)) << 32) |
                                          (uint32_t)uniform((int)a));
  return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, (int)uniform((int)n), kBufferWord3);
}

// Register loads of the B chunk c of group g for the transposition: thread tid takes rows
// 8 (tid / 16) .. + 7, bytes 8 (tid % 16) .. + 7. rs covers the batch's [L, Gbc, N] codes.
__device__ __forceinline__ void fetch_b(const SsdParams& p, __amdgpu_buffer_rsrc_t rs, int g,
                                        int64_t c, int tid, v2u (&bq)[8]) {
  const int ub = tid / (kN / 8), n8 = tid % (kN / 8);
  const int bstep = p.Gbc * kN;
  int voff = ((ub * 8) * p.Gbc + g) * kN + n8 * 8;
  // opaque per call: the per-row offsets are formed here, one add each, instead of being hoisted
  // out of the chunk loop (8 registers held across it)
  __asm__ volatile("" : "+v"(voff));
  voff += (int)c * kQ * bstep;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    bq[r] = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, 0, 0);
    voff += bstep;
  }
}

// Register load of one head's delta at step lt of chunk c (lt = thread index within the half).
// rd covers the batch's [L, nh] deltas.
__device__ __forceinline__ float fetch_dt(const SsdParams& p, __amdgpu_buffer_rsrc_t rd, int64_t h,
                                          int64_t c, int lt) {
  const int nh = (int)p.nh;
  int doff = (lt * nh + (int)h) * 4;
  __asm__ volatile("" : "+v"(doff));  // as in fetch_b
  doff += (int)c * kQ * nh * 4;
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, doff, 0, 0));
}

// Register loads of one head's x codes of chunk c: rows 8 (lt / 8) .. + 7, bytes 8 (lt % 8) .. + 7.
// rx covers the batch's [L, nh, P] codes.
__device__ __forceinline__ void fetch_x(const SsdParams& p, __amdgpu_buffer_rsrc_t rx, int64_t h,
                                        int64_t c, int lt, v2u (&x)[8]) {
  const int jb = lt / 8, p8 = lt % 8;
  const int xstep = (int)p.nh * kP;
  int voff = (jb * 8 * (int)p.nh + (int)h) * kP + p8 * 8;
  __asm__ volatile("" : "+v"(voff));  // as in fetch_b
  voff += (int)c * kQ * xstep;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    x[r] = __builtin_amdgcn_raw_buffer_load_b64(rx, voff, 0, 0);
    voff += xstep;
  }
}

template <bool I8>
__global__ __launch_bounds__(512) void k_ssd_state(SsdParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  K1Smem<I8>& s = *reinterpret_cast<K1Smem<I8>*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int hs = uniform(wave >> 2);   // half: which head of the pair
  const int w = uniform(wave & 3);     // wave within the half
  const int lt = tid & 255;            // thread within the half
  // the pairs of one (b, group) run on one XCD (blocks are dealt to the 8 XCDs in turn), so that
  // the group's B chunks are read from memory once and then from that XCD's L2
  const int pairs = (p.hpg + 1) / 2;
  const int64_t nblk = p.B * p.Gbc * pairs;
  int64_t id = blockIdx.x;
  if (nblk % 8 == 0) id = (id % 8) * (nblk / 8) + id / 8;
  const int64_t bg = id / pairs;
  const int64_t b = bg / p.Gbc;
  const int g = (int)(bg % p.Gbc);
  const int hl = 2 * (int)(id % pairs) + hs;
  // a half with no head computes head 2k again; its per-chunk stores write the same values to the
  // same places as the other half's (unconditional stores keep the waits for the loads exact)
  const bool active = hl < p.hpg;
  const int64_t h = (int64_t)g * p.hpg + (active ? hl : hl - 1);
  const int kh = lane >> 5;
  const float Ah = p.A[h];
  float* const sxp = s.sxp + hs * kP;

  if (lt < kP) {
    const float sx = valid_or_zero(p.x_scales[min((int)p.x_group_of[h * kP + lt], p.G - 1)]);
    sxp[lt] = sx;
    if (b == 0 && active) {
      p.sxt[h * kP + lt] = sx;
      if (p.yi8) p.syt[h * kP + lt] = p.y_scales[min((int)p.y_group_of[h * kP + lt], p.Gy - 1)];
    }
  }
  // B and C scales of this wave's two state groups (ks = 2 w + kb), wave-uniform
  float sB[2], sC[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    sB[kb] = valid_or_zero(p.B_scales[g * kNSG + 2 * w + kb]);
    sC[kb] = valid_or_zero(p.C_scales[g * kNSG + 2 * w + kb]);
  }

  // H^T tiles from h0 (rows n = 32 w + 8 q + 4 kh + 0..3 of column p in one 16-byte read)
  v16f H[2];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt) {
    const int pc = pt * 32 + (lane & 31);
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (p.h0)
        v = *reinterpret_cast<const float4*>(p.h0 + ((b * p.nh + h) * kP + pc) * kN + 32 * w +
                                             8 * qd + 4 * kh);
      H[pt][4 * qd] = v.x; H[pt][4 * qd + 1] = v.y; H[pt][4 * qd + 2] = v.z; H[pt][4 * qd + 3] = v.w;
    }
  }

  // Two register sets for the loads, swapping roles from one chunk to the next (the chunk loop is
  // unrolled twice), so that the loaded registers are never copied: a copy would wait for the
  // loads at the end of every chunk instead of at their use one chunk later.
  float dtA = 0.0f, dtB = 0.0f;
  v2u xA[8], xB[8], bA[8], bB[8];
  const __amdgpu_buffer_rsrc_t rsb = seq_rsrc(p.Bq + b * p.L * p.Gbc * kN, p.L * p.Gbc * kN);
  const __amdgpu_buffer_rsrc_t rsx = seq_rsrc(p.xq + b * p.L * p.nh * kP, p.L * p.nh * kP);
  const __amdgpu_buffer_rsrc_t rsd = seq_rsrc(p.delta + b * p.L * p.nh, p.L * p.nh * 4);

  if (p.nc > 0) {
    dtA = fetch_dt(p, rsd, h, 0, lt);
    fetch_b(p, rsb, g, 0, tid, bA);
    fetch_x(p, rsx, h, 0, lt, xA);
  }
  s.dts[hs * kQ + lt] = dtA;
  lds_barrier();  // s.sxp, s.dts
  auto chunk = [&](const int64_t c, const v2u (&pf_x)[8], const v2u (&pf_b)[8], float& nx_dt,
                   v2u (&nx_x)[8], v2u (&nx_b)[8]) {
    // B chunk, transposed to [n][j] (rows past the sequence were loaded as zero): unit tid takes
    // rows 8 (tid / 16) .. + 7, bytes 8 (tid % 16) .. + 7. The fp16 path stores it as fp16 (the
    // codes are exact), converted once for both heads.
    {
      const int ub = tid / (kN / 8), n8 = tid % (kN / 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (I8) {
          *reinterpret_cast<uint2*>(s.qBT + (n8 * 8 + e) * kRow256 + ub * 8) = column8(pf_b, e);
        } else {
          v8h col;
#pragma unroll
          for (int r = 0; r < 8; ++r) col[r] = (_Float16)(float)(int8_t)byte_of(pf_b[r][e >> 2], e & 3);
          *reinterpret_cast<v8h*>(s.qBh + (n8 * 8 + e) * kXwRow + ub * 8) = col;
        }
      }
    }
    // this chunk's delta of steps 4 lane .. 4 lane + 3 (steps past the sequence were loaded as zero)
    float dt[4];
    {
      const v4f d4 = *reinterpret_cast<const v4f*>(s.dts + hs * kQ + 4 * lane);
      dt[0] = d4[0]; dt[1] = d4[1]; dt[2] = d4[2]; dt[3] = d4[3];
    }
    // the next chunk's loads, also after the last chunk (rows past the sequence read as zero): a
    // branch around them would leave the compiler's waits for this chunk's x codes counted for the
    // path without them, i.e. waiting for most of these loads as well
    nx_dt = fetch_dt(p, rsd, h, c + 1, lt);
    fetch_b(p, rsb, g, c + 1, tid, nx_b);
    fetch_x(p, rsx, h, c + 1, lt, nx_x);
    // the state entering chunk c, C-scaled fp16, in K2's operand order (after the next chunk's
    // loads, so that waiting for those does not wait for these stores)
    {
      // a wave-uniform base and 32-bit lane offsets (no 64-bit addresses held in registers)
      char* const dst = reinterpret_cast<char*>(p.Hh) + ((b * p.nc + c) * p.nh + h) * (int64_t)(kP * kN * 2);
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          v8h o;
#pragma unroll
          for (int m = 0; m < 8; ++m) o[m] = (_Float16)(sC[kb] * H[pt][8 * kb + m]);
          const int ks = 2 * w + kb;
          __builtin_nontemporal_store(
              o, reinterpret_cast<v8h*>(dst + (uint32_t)(((pt * 8 + ks) * 64 + lane) * 16)));
        }
    }


    // Cumulative decay over the chunk, computed whole by every wave (lane l holds steps 4 l .. 4 l + 3:
    // a serial prefix of four, then a wave scan of the lane totals), so no barrier is needed; each
    // wave then publishes the weights of its own 64 steps (the rows of its part of the x tile) in
    // its own LDS slice and writes their cumulative sums for K2.
    const bool own = (lane >> 4) == w;  // lanes 16 w .. 16 w + 15 hold this wave's steps
    char* const cw = reinterpret_cast<char*>(p.cumw) + ((b * p.nc + c) * p.nh + h) * (int64_t)(kQ * 4);
    float dec, wmax_f = 1.0f;
    if (I8) {
      // weights and requantization ratios in fp64 (delta * A is exact there)
      double cs[4];
      cs[0] = (double)dt[0] * (double)Ah;
#pragma unroll
      for (int k = 1; k < 4; ++k) cs[k] = cs[k - 1] + (double)dt[k] * (double)Ah;
      double incl = cs[3];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      const double excl = incl - cs[3];
      const double tot = __shfl(incl, 63, 64);
      double wj[4];
      double wmax = 0.0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        cs[k] += excl;
        wj[k] = (double)dt[k] * exp(tot - cs[k]);
        wmax = fmax(wmax, wj[k]);
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) wmax = fmax(wmax, __shfl_xor(wmax, off, 64));
      if (own) {
        double* rt = s.ratio + hs * kQ + 4 * lane;
#pragma unroll
        for (int k = 0; k < 4; ++k) rt[k] = (wmax > 0.0) ? wj[k] / wmax : 0.0;
        __builtin_nontemporal_store(v4f{(float)cs[0], (float)cs[1], (float)cs[2], (float)cs[3]},
                                    reinterpret_cast<v4f*>(cw + (uint32_t)(lane * 16)));
      }
      dec = (float)exp(tot);
      wmax_f = (float)wmax;
    } else {
      float cs[4];
      cs[0] = dt[0] * Ah;
#pragma unroll
      for (int k = 1; k < 4; ++k) cs[k] = fmaf(dt[k], Ah, cs[k - 1]);
      float incl = cs[3];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      const float excl = incl - cs[3];
      const float tot = __shfl(incl, 63, 64);
      if (own) {
        float* wv = s.wv + hs * kQ + 4 * lane;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          cs[k] += excl;
          wv[k] = dt[k] * expf(tot - cs[k]);
        }
        __builtin_nontemporal_store(v4f{cs[0], cs[1], cs[2], cs[3]},
                                    reinterpret_cast<v4f*>(cw + (uint32_t)(lane * 16)));
      }
      dec = expf(tot);
    }
    // weighted (or requantized) x tile of this half's head, transposed [p][j] (a channel with an
    // invalid scale has sx = 0 and contributes nothing): unit lt takes rows 8 (lt / 8) .. + 7,
    // channels 8 (lt % 8) .. + 7
    {
      const int jb = lt / 8, p8 = lt % 8;
      if (I8) {
        const double* rt = s.ratio + hs * kQ + jb * 8;
        v2u d[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            uint32_t word = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const double v = (double)(int8_t)byte_of(pf_x[r][k], e) * rt[r];
              const int rq = (int)fmin(fmax(rint(v), -128.0), 127.0);
              word |= ((uint32_t)rq & 0xFFu) << (8 * e);
            }
            d[r][k] = word;
          }
        }
        int8_t* rT = s.rT + hs * (kP * kRow256);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<uint2*>(rT + (p8 * 8 + e) * kRow256 + jb * 8) = column8(d, e);
      } else {
        const v4f wlo = *reinterpret_cast<const v4f*>(s.wv + hs * kQ + jb * 8);
        const v4f whi = *reinterpret_cast<const v4f*>(s.wv + hs * kQ + jb * 8 + 4);
        const float wr[8] = {wlo[0], wlo[1], wlo[2], wlo[3], whi[0], whi[1], whi[2], whi[3]};
        _Float16* xw = s.xw + hs * (kP * kXwRow);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v8h col;
#pragma unroll
          for (int r = 0; r < 8; ++r)
            col[r] = (_Float16)((float)(int8_t)byte_of(pf_x[r][e >> 2], e & 3) * wr[r]);
          *reinterpret_cast<v8h*>(xw + (p8 * 8 + e) * kXwRow + jb * 8) = col;
        }
      }
    }
    lds_barrier();

    // S^T tiles on MFMA
    v16f acc[2];
    const int nrow = 32 * w + (lane & 31);
    if (I8) {
      const int8_t* rT = s.rT + hs * (kP * kRow256);
      v16i ai[2] = {};
#pragma unroll
      for (int ks = 0; ks < kQ / 32; ++ks) {
        const int ko = ks * 32 + 16 * kh;
        const v4i av = *reinterpret_cast<const v4i*>(s.qBT + nrow * kRow256 + ko);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          const v4i bv = *reinterpret_cast<const v4i*>(rT + (pt * 32 + (lane & 31)) * kRow256 + ko);
          ai[pt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, ai[pt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[pt][r] = (float)ai[pt][r] * wmax_f;
    } else {
      const _Float16* xw = s.xw + hs * (kP * kXwRow);
      acc[0] = v16f{};
      acc[1] = v16f{};
#pragma unroll
      for (int ks = 0; ks < kQ / 16; ++ks) {
        const int ko = ks * 16 + 8 * kh;
        const v8h av = *reinterpret_cast<const v8h*>(s.qBh + nrow * kXwRow + ko);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          const v8h bv = *reinterpret_cast<const v8h*>(xw + (pt * 32 + (lane & 31)) * kXwRow + ko);
          acc[pt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc[pt], 0, 0, 0);
        }
      }
    }
    // H = dec H + (S sB) sx
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const float sx = sxp[pt * 32 + (lane & 31)];
#pragma unroll
      for (int r = 0; r < 16; ++r) H[pt][r] = fmaf(dec, H[pt][r], (acc[pt][r] * sB[r / 8]) * sx);
    }
    // the next chunk's deltas (every wave has read this chunk's before the barrier above)
    s.dts[hs * kQ + lt] = nx_dt;
    lds_barrier();  // qBT and the x tiles are rewritten by the next chunk
  };
  for (int64_t c = 0; c < p.nc; c += 2) {
    chunk(c, xA, bA, dtB, xB, bB);
    if (c + 1 < p.nc) chunk(c + 1, xB, bB, dtA, xA, bA);
  }

  if (p.h_last && active) {
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const int pc = pt * 32 + (lane & 31);
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<float4*>(p.h_last + ((b * p.nh + h) * kP + pc) * kN + 32 * w + 8 * qd +
                                   4 * kh) =
            make_float4(H[pt][4 * qd], H[pt][4 * qd + 1], H[pt][4 * qd + 2], H[pt][4 * qd + 3]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// K2: chunk outputs.
struct K2Smem {
  union {
    int8_t qB[kQ * kRow128];  // B chunk rows [j][n] (prologue only)
    // fp16 intra-chunk product: the partial outputs that wave s (s < 4) computes for query block
    // 7 - s, handed to wave s + 4 (after the prologue)
    float part[4][2 * 16 * 64];
  };
  int8_t qC[kQ * kRow128];  // C chunk rows [i][n]
  // x codes of the head, [p][j]: fp16 (exact) for the fp16 intra-chunk product, int8 rows of
  // kRow256 bytes for the int8 one
  union {
    _Float16 xT[kP * kXtRow];
    int8_t xT8[kP * kRow256];
  };
  // The entering state of heads hh (buffer hh % 2) as stored by K1: the inter-chunk product's B
  // operands, 1 KB per (column tile, K block); the next head's arrives by direct loads while the
  // current head's is read.
  _Float16 sth[2][kP * kN];
  // The next head's other inputs, written by direct global-to-LDS loads while the current head
  // computes: x codes in 1 KB blocks of 16 rows (row r of block jb at slot (r + jb) % 16, so that
  // the transposing reads below hit distinct banks), delta, the cumulative decay exponents, sx.
  int8_t stx[kQ * kP];
  float stdt[kQ];
  float stcum[kQ];
  float stsx[kP];
  float stsy[kP];   // int8 output: staged output scale and correction term of each channel
  float styb[kP];
  float cum[kQ];
  float dtv[kQ];
  float ecum[kQ];   // exp(cum_i)
  float cjv[kQ];    // exp(cum at the end of j's 32-block - cum_j) * delta_j
  float sxs[kP];
  float sys[kP];
  float syb[kP];
  float stad;  // staged D_h
  float dh;    // D_h of the current head
  float sig[8][32];  // int8 intra-chunk output: row scales of each wave's query block
};
static_assert(offsetof(K2Smem, stcum) % 16 == 0 && offsetof(K2Smem, cum) % 16 == 0 &&
                  offsetof(K2Smem, dtv) % 16 == 0 &&
                  offsetof(K2Smem, ecum) % 16 == 0 && offsetof(K2Smem, cjv) % 16 == 0,
              "16-byte vector reads of the decay terms");


// Compiler-only fence: keeps one tile's work from being interleaved with the next tile's.
__device__ __forceinline__ void tile_fence() { __asm__ volatile("" ::: "memory"); }

__device__ __forceinline__ void build_g_tile(v16f& G, const K2Smem& s, const float* sBC, int I,
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

// Decay factors of tile (I, J): f[r] = exp(cum_i - cum_j) delta_j [j <= i] in the order of the G
// accumulator: register r of lane l holds row i = 32 I + l % 32 and column
// j = 32 J + 4 (l / 32) + 8 (r / 4) + r % 4, so the column terms come in runs of four (16-byte
// reads, the same address for each half-wave).
__device__ __forceinline__ void tile_factors(const K2Smem& s, int I, int J, int lane,
                                             float (&f)[16]) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const int i = I * 32 + (lane & 31);  // this lane's query row
  const int jb = J * 32 + 4 * (lane >> 5);
  const float ci = s.cum[i];
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
}

// M tile = G o exp(cum_i - cum_j) [j <= i] o delta_j as two fp16 A operands (k-slots follow the
// accumulator rows of G, see the B operand gather below). Each element is one mixed-precision fma
// from the fp16 G value, rounded once to fp16.
__device__ __forceinline__ void m_tile(const GTile& Gt, const K2Smem& s, int I, int J, int lane,
                                       v8h& a0, v8h& a1) {
  float f[16];
  tile_factors(s, I, J, lane, f);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a0[e] = (_Float16)fmaf((float)Gt.lo[e], f[e], 0.0f);
    a1[e] = (_Float16)fmaf((float)Gt.hi[e], f[8 + e], 0.0f);
  }
}

// int8 B operand of the int8 intra-chunk product (K = 32, the whole tile column block J): lane l
// supplies column p and, as bytes 4 q + k, the x codes of j = 32 J + 4 (l / 32) + 8 q + k, the
// column order of the A operand (the G accumulator order, byte r for register r).
__device__ __forceinline__ v4i x8_operand(const K2Smem& s, int J, int pt, int lane) {
  const int8_t* row = s.xT8 + (pt * 32 + (lane & 31)) * kRow256 + J * 32 + 4 * (lane >> 5);
  v4i o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = *reinterpret_cast<const int*>(row + 8 * q);
  return o;
}

// x B operand for MFMA mm of tile column block J: lane l supplies column p and the 8 j's whose G
// accumulator rows sit in registers 8 mm .. 8 mm + 7 of the same lane half
__device__ __forceinline__ v8h x_operand(const K2Smem& s, int J, int mm, int pt, int lane) {
  const int j0 = J * 32 + 16 * mm + 4 * (lane >> 5);
  const _Float16* row = s.xT + (pt * 32 + (lane & 31)) * kXtRow;
  const v4h lo = *reinterpret_cast<const v4h*>(row + j0);
  const v4h hi = *reinterpret_cast<const v4h*>(row + j0 + 8);
  return v8h{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
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
__device__ __forceinline__ void stage_head(const SsdParams& p, K2Smem& s, int64_t b, int64_t c,
                                           int64_t t0, int q, int64_t h, int hbuf, int wave,
                                           int lane) {
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
    const int dst = uniform((int)offsetof(K2Smem, stx) + jb * 1024);
    __builtin_amdgcn_global_load_lds(src, base + dst, 16, 0, 0);
  }
  // entering state: 16 KB contiguous, 1 KB per instruction, into buffer hbuf
  const _Float16* hsrc = p.Hh + ((b * p.nc + c) * p.nh + h) * (int64_t)(kP * kN);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int blk = 2 * wave + k;
    const int dst = uniform((int)offsetof(K2Smem, sth) + hbuf * (kP * kN * 2) + blk * 1024);
    __builtin_amdgcn_global_load_lds(hsrc + blk * 512 + lane * 8, base + dst, 16, 0, 0);
  }
  if (wave < 4) {  // delta of steps 64 w .. 64 w + 63
    const int j = min(wave * 64 + lane, q - 1);
    const int dst = uniform((int)offsetof(K2Smem, stdt) + wave * 256);
    __builtin_amdgcn_global_load_lds(p.delta + (b * p.L + t0 + j) * p.nh + h, base + dst, 4, 0, 0);
  } else if (wave == 4) {
    const int dst = uniform((int)offsetof(K2Smem, stsx));
    __builtin_amdgcn_global_load_lds(p.sxt + h * kP + lane, base + dst, 4, 0, 0);
  } else if (wave == 5) {  // the chunk's cumulative decay exponents, 1 KB contiguous
    const int dst = uniform((int)offsetof(K2Smem, stcum));
    __builtin_amdgcn_global_load_lds(p.cumw + ((b * p.nc + c) * p.nh + h) * kQ + lane * 4, base + dst,
                                     16, 0, 0);
  } else if (wave == 6) {
    if (lane == 0 && p.Dskip) {
      const int dst = uniform((int)offsetof(K2Smem, stad));
      __builtin_amdgcn_global_load_lds(p.Dskip + h, base + dst, 4, 0, 0);
    }
    if (p.yi8) {
      const int dst = uniform((int)offsetof(K2Smem, stsy));
      __builtin_amdgcn_global_load_lds(p.syt + h * kP + lane, base + dst, 4, 0, 0);
    }
  } else if (wave == 7 && p.yi8 && p.y_bias) {
    const int dst = uniform((int)offsetof(K2Smem, styb));
    __builtin_amdgcn_global_load_lds(p.y_bias + h * kP + lane, base + dst, 4, 0, 0);
  }
}

// Eight waves; wave v owns query block I = v (v < 4) or 11 - v (v >= 4), so that the two waves
// on one SIMD (v and v + 4) hold blocks s and 7 - s: 9 causal tiles per SIMD. A wave keeps the
// G tiles (I, J <= I) of its block in registers and produces all 64 output columns of it. Each
// head's inputs arrive in LDS by direct loads issued during the previous head's products.
// I8I: the intra-chunk product on int8 MFMA. Each query row's weights W[i, j] = G exp(cum_i -
// cum_j) delta_j are requantized with the row's own scale (m_i = max_j |W[i, j]|, codes
// rint(W * 127 / m_i) in [-127, 127]); int8 MFMA against the x codes with int32 accumulate over
// the whole row, then m_i / 127 per row. W is formed from the fp16 G tiles kept in registers (as
// for the fp16 product), and the row maximum takes a first pass over the row's tiles.
template <bool I8I>
__global__ __launch_bounds__(512) void k_ssd_output(SsdParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  K2Smem& s = *reinterpret_cast<K2Smem*>(smem_raw);
  const int tid = threadIdx.x;
  const int64_t c = blockIdx.x;
  const int64_t b = blockIdx.y / p.Gbc;
  const int g = (int)(blockIdx.y % p.Gbc);
  const int64_t t0 = c * kQ;
  const int q = (int)((p.L - t0) < kQ ? (p.L - t0) : kQ);

  // B and C chunk rows of group g (zero past the sequence): all eight waves, eight 16-byte loads
  // per thread issued together (rows clamped into the sequence), then masked and stored to LDS
  {
    uint4 v[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int row = (tid >> 3) + 64 * (m & 3), c16 = tid & 7;
      const int8_t* src = (m < 4 ? p.Bq : p.Cq) +
                          ((b * p.L + t0 + min(row, q - 1)) * p.Gbc + g) * kN + c16 * 16;
      v[m] = *reinterpret_cast<const uint4*>(src);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int row = (tid >> 3) + 64 * (m & 3), c16 = tid & 7;
      const bool on = row < q;
      int8_t* dst = (m < 4 ? s.qB : s.qC) + row * kRow128 + c16 * 16;
      *reinterpret_cast<uint2*>(dst) = on ? make_uint2(v[m].x, v[m].y) : make_uint2(0u, 0u);
      *reinterpret_cast<uint2*>(dst + 8) = on ? make_uint2(v[m].z, v[m].w) : make_uint2(0u, 0u);
    }
  }
  float sBC[kNSG];  // sB * sC per state group (wave-uniform)
#pragma unroll
  for (int sg = 0; sg < kNSG; ++sg)
    sBC[sg] = valid_or_zero(p.B_scales[g * kNSG + sg]) * valid_or_zero(p.C_scales[g * kNSG + sg]);
  lds_barrier();
  // the first head's inputs load while G is built
  stage_head(p, s, b, c, t0, q, (int64_t)g * p.hpg, 0, uniform(tid >> 6), tid & 63);

  // G tiles held by this wave. int8 intra-chunk product: the tiles (I, J <= I) of the wave's own
  // query block I. fp16 product: the 9 causal tiles of the two blocks s and 7 - s on one SIMD
  // (waves s and s + 4) are split 5 + 4, so that both waves carry the same work: wave s takes
  // tile slots k = 0..4 = (s, 0..s) then (7 - s, 0..3 - s); wave s + 4 takes (7 - s, 4 - s + k)
  // for k = 0..3, and adds wave s's partial sums for block 7 - s before its output.
  GTile G[8];
  {
    const int lane = tid & 63;
    const int v = uniform(tid >> 6);
    const int I = v < 4 ? v : 11 - v;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (I8I) {
        if (k <= I) {
          v16f Gf;
          build_g_tile(Gf, s, sBC, I, k, lane);
          G[k] = pack_g(Gf);
        }
      } else if (k < kSlotsA) {
        const int sw = v & 3;
        if (k < (v < 4 ? kSlotsA : kSlotsB)) {
          const int Ik = v < 4 ? (k <= sw ? sw : 7 - sw) : 7 - sw;
          const int Jk = v < 4 ? (k <= sw ? k : k - sw - 1) : 4 - sw + k;
          v16f Gf;
          build_g_tile(Gf, s, sBC, Ik, Jk, lane);
          G[k] = pack_g(Gf);
        }
      }
      tile_fence();
    }
  }
  // the C codes of this wave's query block as fp16 A operands of the inter-chunk product (the
  // same for every head), in the K order of the stored entering state: slot m of lane half kh in
  // K block ks is state n = 16 ks + 4 kh + (m < 4 ? m : m + 4)
  // (the int8 intra-chunk variant reads them from LDS at each head instead: registers are short)
  v8h QC[I8I ? 1 : kN / 16];
  if constexpr (!I8I) {
    const int lane = tid & 63;
    const int I = uniform(uniform(tid >> 6) < 4 ? uniform(tid >> 6) : 11 - uniform(tid >> 6));
    const int8_t* crow = s.qC + (I * 32 + (lane & 31)) * kRow128 + 4 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < kN / 16; ++ks) {
      const uint32_t lo = *reinterpret_cast<const uint32_t*>(crow + ks * 16);
      const uint32_t hi = *reinterpret_cast<const uint32_t*>(crow + ks * 16 + 8);
      QC[ks] = i8x8_to_h((int64_t)(((uint64_t)hi << 32) | lo));
    }
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);

  const int rs = (int)(p.nh * kP);  // row stride of y in elements
  const bool full = q == kQ;
  // a head's output values, computed at its end and stored after the next head's first barrier
  float yv[2][16], ep_mult[2], ep_sy[2] = {}, ep_yb[2] = {};
  auto finish = [&](int hprev) {
    const int lane = tid & 63;
    const int v = uniform(tid >> 6);
    const int I = v < 4 ? v : 11 - v;
    if constexpr (!I8I) {
      if (v >= 4) {
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            yv[pt][r] = fmaf(ep_mult[pt], s.part[v & 3][(pt * 16 + r) * 64 + lane], yv[pt][r]);
      }
    }
    const int64_t base = ((b * p.L + t0) * p.nh + (int64_t)g * p.hpg + hprev) * kP;  // y[b, t0, h, 0]
    // register r holds row 32 I + 8 (r / 4) + r % 4 + 4 (lane / 32): buffer stores with the head's
    // y block as the resource, a per-register wave-uniform row offset (soffset) and one per-lane
    // offset, so the stores need no per-lane 64-bit address arithmetic (all offsets fit 32 bits:
    // nheads <= 2^14 is checked on the host)
    const int ilane = 4 * (lane >> 5);
    const int esz = p.yi8 ? 1 : (p.yf16 ? 2 : 4);
    const uint64_t ya = reinterpret_cast<uint64_t>(static_cast<char*>(p.y) + base * esz);
    void* const yblk = reinterpret_cast<void*>(
        ((uint64_t)(uint32_t)uniform((int)(ya >> 32)) << 32) | (uint32_t)uniform((int)ya));
    const __amdgpu_buffer_rsrc_t yrs =
        __builtin_amdgcn_make_buffer_rsrc(yblk, (short)0, 0x7FFFFFFF, kBufferWord3);
    if (!p.yf16 && !p.yi8) {
      // fp32: each store of a wave writes two full 128-byte lines (rows i and i + 4, 32 channels)
      // (a whole chunk stores with no per-row test: one branch per head instead of one per store)
      if (full) {
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          const int voff = (ilane * rs + pt * 32 + (lane & 31)) * 4;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ir = I * 32 + 8 * (r / 4) + (r % 4);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, yv[pt][r]), yrs,
                                                  voff, uniform(ir * rs * 4), kYPolicy);
          }
        }
      } else {
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          const int voff = (ilane * rs + pt * 32 + (lane & 31)) * 4;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ir = I * 32 + 8 * (r / 4) + (r % 4);
            if (ir + ilane < q)
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, yv[pt][r]),
                                                    yrs, voff, uniform(ir * rs * 4), kYPolicy);
          }
        }
      }
    } else {
      // fp16 or int8: neighbouring lanes trade one value so that each holds two adjacent channels
      // of one row: an even lane channels (c, c + 1) of the first 32, an odd lane (32 + c - 1,
      // 32 + c); one store of a wave then writes rows i and i + 4 whole (64 channels each)
      const bool odd = lane & 1;
      const int c0 = lane & 31;
      const int col = odd ? 32 + c0 - 1 : c0;
      const int voff = (ilane * rs + col) * esz;
      uint32_t v0[16], v1[16];  // the element of each tile as bits (fp16 or int8 code)
      if (p.yi8) {
        // persistent int8 output: fl32(y + correction term) quantized with the channel's static
        // output scale by the exact rule (an invalid scale gives 0)
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          const float sy = ep_sy[pt];
          const float ry = recip_or_zero(sy);
          const float yb = ep_yb[pt];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t cd = (uint8_t)quant8_r(yv[pt][r] + yb, sy, ry);
            if (pt == 0) v0[r] = cd; else v1[r] = cd;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          v0[r] = __builtin_bit_cast(unsigned short, __float2half_rn(yv[0][r]));
          v1[r] = __builtin_bit_cast(unsigned short, __float2half_rn(yv[1][r]));
        }
      }
      const int shift = p.yi8 ? 8 : 16;
      uint32_t pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // DPP quad permutation [1, 0, 3, 2]: the value of the neighbouring lane
        const uint32_t send = odd ? v0[r] : v1[r];
        const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
        pr[r] = odd ? (recv | (v1[r] << shift)) : (v0[r] | (recv << shift));
      }
      // (a whole chunk stores with no per-row test, as above)
      if (full && p.yi8) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)pr[r], yrs, voff,
                                                uniform((I * 32 + 8 * (r / 4) + (r % 4)) * rs),
                                                kYPolicy);
      } else if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(pr[r], yrs, voff,
                                                uniform((I * 32 + 8 * (r / 4) + (r % 4)) * rs * 2),
                                                kYPolicy);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ir = I * 32 + 8 * (r / 4) + (r % 4);
          if (ir + ilane < q) {
            if (p.yi8)
              __builtin_amdgcn_raw_buffer_store_b16((unsigned short)pr[r], yrs, voff,
                                                    uniform(ir * rs), kYPolicy);
            else
              __builtin_amdgcn_raw_buffer_store_b32(pr[r], yrs, voff, uniform(ir * rs * 2),
                                                    kYPolicy);
          }
        }
      }
    }
  };
  for (int hh = 0; hh < p.hpg; ++hh) {
    const int64_t h = (int64_t)g * p.hpg + hh;
    // every wave has waited for its own staging loads of head h and is done with head h - 1
    lds_barrier();
    if (hh > 0) finish(hh - 1);
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
    if (tid < kP) {
      s.sxs[tid] = s.stsx[tid];
      if (p.yi8) {
        s.sys[tid] = s.stsy[tid];
        s.syb[tid] = p.y_bias ? s.styb[tid] : 0.0f;
      }
    }
    if (tid == 0) s.dh = p.Dskip ? s.stad : 0.0f;
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
        if constexpr (I8I) {
          // bytes e of the 8 rows, as two words
          uint32_t w[2];
#pragma unroll
          for (int r4 = 0; r4 < 2; ++r4) {
            const uint32_t lo = __builtin_amdgcn_perm(raw[4 * r4 + 1], raw[4 * r4], 0x0c0c0400u + 0x00000101u * e);
            const uint32_t hi = __builtin_amdgcn_perm(raw[4 * r4 + 3], raw[4 * r4 + 2], 0x0c0c0400u + 0x00000101u * e);
            w[r4] = on ? (lo | (hi << 16)) : 0u;
          }
          *reinterpret_cast<uint2*>(s.xT8 + pc * kRow256 + jh * 8) = make_uint2(w[0], w[1]);
        } else {
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
    }
    lds_barrier();
    // the staging area is free: the next head's inputs load during this head's products
    if (hh + 1 < p.hpg) stage_head(p, s, b, c, t0, q, h + 1, (hh + 1) & 1, uniform(tid >> 6), tid & 63);

    // Opaque copies of the lane and wave ids: the tile addresses below do not depend on the head,
    // and hoisting all of them out of the head loop would keep them live across it (spills).
    int lane = tid & 63;
    __asm__ volatile("" : "+v"(lane));
    int v = uniform(tid >> 6);
    __asm__ volatile("" : "+s"(v));
    const int I = uniform(v < 4 ? v : 11 - v);  // (the asm output is not known to be uniform)
    v16f Y[2] = {};
    // Y_inter = exp(cum_i) * qC[i, :] . (sC H)[:, p], operands straight from the staged state
    const _Float16* hs = s.sth[hh & 1];
#pragma unroll
    for (int ks = 0; ks < kN / 16; ++ks) {
      v8h a;
      if constexpr (I8I) {
        const int8_t* crow = s.qC + (I * 32 + (lane & 31)) * kRow128 + 4 * (lane >> 5);
        const uint32_t lo = *reinterpret_cast<const uint32_t*>(crow + ks * 16);
        const uint32_t hi = *reinterpret_cast<const uint32_t*>(crow + ks * 16 + 8);
        a = i8x8_to_h((int64_t)(((uint64_t)hi << 32) | lo));
      } else {
        a = QC[ks];
      }
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const v8h bv = *reinterpret_cast<const v8h*>(hs + ((pt * 8 + ks) * 64 + lane) * 8);
        Y[pt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bv, Y[pt], 0, 0, 0);
      }
    }
    // row scale exp(cum_i), column scale 1 / sx[p] (the intra part accumulates raw x codes);
    // register r holds row i = 32 I + 4 (lane / 32) + 8 (r / 4) + r % 4
    {
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
    if constexpr (!I8I) {
      // Y_intra on top, tile slot by tile slot (see the prologue for the assignment); wave s < 4
      // accumulates its slots past s, the tiles of block 7 - s, into Yp
      const int sw = v & 3;
      const bool wa = v < 4;
      v16f Yp[2] = {};
#pragma unroll
      for (int k = 0; k < kSlotsA; ++k) {
        tile_fence();
        if (k < (wa ? kSlotsA : kSlotsB)) {
          const bool own = !wa || k <= sw;
          const int Ik = wa ? (k <= sw ? sw : 7 - sw) : 7 - sw;
          const int Jk = wa ? (k <= sw ? k : k - sw - 1) : 4 - sw + k;
          // opaque per head: keeps the fp32 widening of the G tile inside the head loop
          // (hoisted, the widened copies of all tiles would stay live and spill)
          __asm__ volatile("" : "+v"(G[k].lo), "+v"(G[k].hi));
          v8h a0, a1;
          m_tile(G[k], s, Ik, Jk, lane, a0, a1);
#pragma unroll
          for (int pt = 0; pt < 2; ++pt) {
            const v8h b0 = x_operand(s, Jk, 0, pt, lane);
            const v8h b1 = x_operand(s, Jk, 1, pt, lane);
            if (own) {
              Y[pt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, Y[pt], 0, 0, 0);
              Y[pt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, Y[pt], 0, 0, 0);
            } else {
              Yp[pt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, Yp[pt], 0, 0, 0);
              Yp[pt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, Yp[pt], 0, 0, 0);
            }
          }
        }
      }
      tile_fence();
      // hand wave s's partial sums for block 7 - s to wave s + 4, which adds them after the next
      // barrier (the area is free: wave s + 4 read the previous head's before this head's second
      // barrier)
      if (wa) {
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
          for (int r = 0; r < 16; ++r) s.part[sw][(pt * 16 + r) * 64 + lane] = Yp[pt][r];
      }
    } else {
      // opaque per head, as above
#pragma unroll
      for (int J = 0; J < 8; ++J)
        if (J <= I) __asm__ volatile("" : "+v"(G[J].lo), "+v"(G[J].hi));
      // row maximum of |W| over the row's tiles (lane l and l + 32 hold the two column halves)
      float mx = 0.0f;
#pragma unroll
      for (int J = 0; J < 8; ++J) {
        tile_fence();
        if (J <= I) {
          float f[16];
          tile_factors(s, I, J, lane, f);
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            mx = fmaxf(mx, fabsf(fmaf((float)G[J].lo[r], f[r], 0.0f)));
            mx = fmaxf(mx, fabsf(fmaf((float)G[J].hi[r], f[8 + r], 0.0f)));
          }
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float inv = mx > 0.0f ? 127.0f / mx : 0.0f;
      if (lane < 32) s.sig[v][lane] = mx / 127.0f;
      v16i acc8[2] = {};
#pragma unroll
      for (int J = 0; J < 8; ++J) {
        tile_fence();
        if (J <= I) {
          float f[16];
          tile_factors(s, I, J, lane, f);
          // |W * inv| <= 127 (1 + 2^-22): the rounded code is in [-127, 127] without a clamp; it
          // is packed as the unsigned byte code + 128 and the bias removed from all four bytes
          v4i a;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t w = 0u;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int r = 4 * q + k;
              const float wv = fmaf(r < 8 ? (float)G[J].lo[r] : (float)G[J].hi[r - 8], f[r], 0.0f);
              w = __builtin_amdgcn_cvt_pk_u8_f32(rintf(wv * inv) + 128.0f, k, w);
            }
            a[q] = (int)(w ^ 0x80808080u);
          }
#pragma unroll
          for (int pt = 0; pt < 2; ++pt)
            acc8[pt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, x8_operand(s, J, pt, lane), acc8[pt],
                                                            0, 0, 0);
        }
      }
      // register r holds row 32 I + 4 (lane / 32) + 8 (r / 4) + r % 4: its scale from the wave's
      // row scales (written by the lanes that own the rows)
      typedef float v4f __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f g4 = *reinterpret_cast<const v4f*>(&s.sig[v][4 * (lane >> 5) + 8 * q]);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
          for (int k = 0; k < 4; ++k)
            Y[pt][4 * q + k] = fmaf(g4[k], (float)acc8[pt][4 * q + k], Y[pt][4 * q + k]);
      }
    }
    tile_fence();
    // y = sx * acc + D * xh, from this head's LDS values (the next head rewrites them); wave
    // s + 4 of the fp16 path adds wave s's partial sums (times sx) after the next barrier, and
    // every wave stores its rows there
    {
      const float Dh = s.dh;
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const int pc = pt * 32 + (lane & 31);
        const float sx = s.sxs[pc];
        const float mult = (sx > 0.0f) ? sx : 1.0f;
        const float Dsx = Dh * sx;
        ep_mult[pt] = mult;
        if (p.yi8) {
          ep_sy[pt] = s.sys[pc];
          ep_yb[pt] = s.syb[pc];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float xc[4];
          if constexpr (I8I) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(s.xT8 + pc * kRow256 + I * 32 + 4 * (lane >> 5) + 8 * q);
#pragma unroll
            for (int k = 0; k < 4; ++k) xc[k] = (float)(int8_t)byte_of(w, k);
          } else {
            const v4h x4 = *reinterpret_cast<const v4h*>(s.xT + pc * kXtRow + I * 32 + 4 * (lane >> 5) + 8 * q);
#pragma unroll
            for (int k = 0; k < 4; ++k) xc[k] = (float)x4[k];
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) yv[pt][4 * q + k] = fmaf(Dsx, xc[k], mult * Y[pt][4 * q + k]);
        }
      }
    }
    // the staging loads were issued long before; waiting here keeps the y stores out of the count
    // waited for at the next head's start
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
  }
  // the last head's output
  if (p.hpg > 0) {
    lds_barrier();
    finish(p.hpg - 1);
  }
}

// The dynamic-LDS limit of a kernel is raised once per device (hipFuncSetAttribute applies on the
// current device; two threads racing both make the same idempotent call).
constexpr int kMaxDevices = 64;
enum { kAttrK1F16 = 0, kAttrK1I8 = 1, kAttrK2 = 2, kAttrK2I8 = 3 };
std::atomic<bool> g_lds_raised[4][kMaxDevices];

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
  size_t sx_off, sy_off, cum_off, total;  // Hh at offset 0
};

// workspace: Hh (fp16 entering states), sxt, syt, cumw, each 256-byte aligned
WsLayout ws_layout(const qssm_ssd_args* a) {
  const int64_t nc = (a->seqlen + kQ - 1) / kQ;
  const size_t elems = (size_t)a->batch * nc * a->nheads * kP * kN;
  WsLayout w;
  w.sx_off = (elems * sizeof(_Float16) + 255) & ~(size_t)255;
  w.sy_off = (w.sx_off + (size_t)a->nheads * kP * sizeof(float) + 255) & ~(size_t)255;
  w.cum_off = (w.sy_off + (size_t)a->nheads * kP * sizeof(float) + 255) & ~(size_t)255;
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
  if (a->y_dtype != QSSM_F32 && a->y_dtype != QSSM_F16 && a->y_dtype != QSSM_I8)
    return fail(QSSM_ERR_INVALID_ARG, "y_dtype must be QSSM_F32, QSSM_F16 or QSSM_I8");
  if (a->y_dtype == QSSM_I8) {
    if (a->y_groups < 1 || a->y_groups > 256)
      return fail(QSSM_ERR_INVALID_ARG, "y_groups not in 1..256");
    if (!a->y_group_of || !a->y_scales)
      return fail(QSSM_ERR_INVALID_ARG, "QSSM_I8 output needs y_group_of and y_scales");
  }
  if (a->fused != 0) return fail(QSSM_ERR_UNSUPPORTED, "fused must be 0");
  if (a->state_mma != QSSM_MMA_F16 && a->state_mma != QSSM_MMA_I8)
    return fail(QSSM_ERR_INVALID_ARG, "state_mma must be QSSM_MMA_F16 or QSSM_MMA_I8");
  if (a->intra_mma != QSSM_MMA_F16 && a->intra_mma != QSSM_MMA_I8)
    return fail(QSSM_ERR_INVALID_ARG, "intra_mma must be QSSM_MMA_F16 or QSSM_MMA_I8");
  if (a->chunk != kQ || a->headdim != kP || a->dstate != kN || a->bc_group_size != kGS)
    return fail(QSSM_ERR_UNSUPPORTED,
                "the library implements chunk=256, headdim=64, dstate=128, bc_group_size=16");
  if (L > ((int64_t)1 << 40)) return fail(QSSM_ERR_UNSUPPORTED, "seqlen too large");
  if (nh > (1 << 14)) return fail(QSSM_ERR_UNSUPPORTED, "nheads too large");
  // the state kernel addresses one sequence's x and B codes and deltas with 32-bit offsets, over
  // whole chunks and one chunk past the last (its loads run one chunk ahead)
  const int64_t Lc = (L + kQ - 1) / kQ * kQ + kQ;
  if (Lc * nh * kP >= ((int64_t)1 << 31) || Lc * a->ngroups * kN >= ((int64_t)1 << 31))
    return fail(QSSM_ERR_UNSUPPORTED, "one sequence's x or B codes exceed 2^31 bytes");
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
              reinterpret_cast<_Float16*>(base), reinterpret_cast<float*>(base + wl.sx_off),
              reinterpret_cast<float*>(base + wl.cum_off), a->y_dtype == QSSM_I8,
              a->y_dtype == QSSM_I8 ? a->y_groups : 1, a->y_group_of, a->y_scales, a->y_bias,
              reinterpret_cast<float*>(base + wl.sy_off), a->intra_mma == QSSM_MMA_I8};
  if ((int64_t)B * a->ngroups > 65535 || nc > 0x7fffffff || B * nh > 0x7fffffff)
    return fail(QSSM_ERR_UNSUPPORTED, "grid too large");
  // K1 runs even for an empty sequence: it writes h_last = h0 (or zeros)
  {
    const int i8 = a->state_mma == QSSM_MMA_I8;
    const void* k1 = i8 ? reinterpret_cast<const void*>(&k_ssd_state<true>)
                        : reinterpret_cast<const void*>(&k_ssd_state<false>);
    const size_t k1_lds = i8 ? sizeof(K1Smem<true>) : sizeof(K1Smem<false>);
    if (!raise_lds_limit(i8 ? kAttrK1I8 : kAttrK1F16, k1, k1_lds))
      return fail(QSSM_ERR_DEVICE, "cannot raise the LDS limit of the SSD state kernel");
    const unsigned k1_grid = (unsigned)(B * a->ngroups * ((nh / a->ngroups + 1) / 2));
    if (i8) k_ssd_state<true><<<k1_grid, 512, k1_lds, stream>>>(p);
    else k_ssd_state<false><<<k1_grid, 512, k1_lds, stream>>>(p);
    if (qssm_status s = launch_status("ssd chunk states")) return s;
  }
  if (nc > 0) {
    const bool i8 = p.intra8 != 0;
    const void* k2 = i8 ? reinterpret_cast<const void*>(&k_ssd_output<true>)
                        : reinterpret_cast<const void*>(&k_ssd_output<false>);
    if (!raise_lds_limit(i8 ? kAttrK2I8 : kAttrK2, k2, sizeof(K2Smem)))
      return fail(QSSM_ERR_DEVICE, "cannot raise the LDS limit of the SSD output kernel");
    const dim3 grid((unsigned)nc, (unsigned)(B * a->ngroups));
    if (i8) k_ssd_output<true><<<grid, 512, sizeof(K2Smem), stream>>>(p);
    else k_ssd_output<false><<<grid, 512, sizeof(K2Smem), stream>>>(p);
    if (qssm_status s = launch_status("ssd output")) return s;
  }
  return QSSM_OK;
}

}  // extern "C"
