// W4A8 linear layer: 4-bit weights x int8 activations on int8 MFMA with int32 accumulation.
//
// Quamba2, abstract: W4A8 for large-batch decoding (the in and out projections around the
// recurrence). Per output channel n and group g of `group` consecutive input channels:
//     y[m, n] = bias[n] + sum_g (sa * sw[n, g]) * sum_{k in g} qa[m, k] * qw[n, k]
// with qa int8 activation codes (one scale sa) and qw in [-8, 7] packed two per byte.
//
// Packed weight layout (per output channel, K / 2 bytes): each run of 8 consecutive input channels
// k0 .. k0 + 7 takes 4 bytes, byte b holding k0 + b in its low nibble and k0 + 4 + b in its high
// nibble (two's complement nibbles). Masking a 32-bit word with 0xF0F0F0F0 after a left shift by 4
// (low nibbles) or without it (high nibbles) then yields the 8 codes times 16 as int8 bytes, in k
// order: the unpacking costs two instructions per 8 codes and no sign extension. The factor 16 is
// exact and divided out of the scale.
//
// Tiling (CDNA4, wave64): a workgroup of 4 waves computes a 128 x 128 tile of y, K in steps of 64
// staged through LDS (double-buffered, the next step's global loads in registers during the
// current step's products); wave (wm, wn) owns a 64 x 64 block = 2 x 2 tiles of
// v_mfma_i32_32x32x32_i8 (operand lane l: row or column l % 32, 16 consecutive k at 16 (l / 32)).
// The int32 sums of a weight group are scaled into fp32 at the group's end.
#include <hip/hip_runtime.h>

#include "common.hpp"

using namespace qssm;

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int64_t kWideMinM = 1024;  // tokens from which the wide-tile form is used
constexpr int kARow = 80;  // padded bytes of an activation row in LDS (64 + 16): no bank conflicts
constexpr int kWRow = 40;  // padded bytes of a packed weight row in LDS (32 + 8)

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

struct GemmParams {
  int64_t M, N, K;
  int32_t group, yf16;
  const int8_t* a;
  const float* a_scale;
  const uint8_t* w;
  const float* w_scales;
  const float* bias;
  void* y;
};

struct GemmSmem {
  int8_t a[2][kBM * kARow];
  uint8_t w[2][kBN * kWRow];
};

// Global loads of K step kt: thread t takes activation row t / 2 (32 bytes at (t % 2) * 32) and
// weight row t / 2 (16 bytes at (t % 2) * 16). Branch-free: rows past M or N load a valid row and
// are zeroed by the store.
__device__ __forceinline__ void load_step(const GemmParams& p, int64_t m0, int64_t n0, int64_t kt,
                                          int tid, uint4 (&ra)[2], uint4& rw) {
  const int row = tid >> 1, half = tid & 1;
  const int64_t m = min(m0 + row, p.M - 1), n = min(n0 + row, p.N - 1);
  const uint4* src = reinterpret_cast<const uint4*>(p.a + m * p.K + kt * kBK + half * 32);
  ra[0] = src[0];
  ra[1] = src[1];
  rw = *reinterpret_cast<const uint4*>(p.w + n * (p.K / 2) + kt * (kBK / 2) + half * 16);
}

__device__ __forceinline__ uint4 masked(uint4 v, bool on) {
  return on ? v : make_uint4(0u, 0u, 0u, 0u);
}

__device__ __forceinline__ void store_step(GemmSmem& s, int buf, int tid, bool a_on, bool w_on,
                                           const uint4 (&ra)[2], const uint4& rw) {
  const int row = tid >> 1, half = tid & 1;
  uint4* da = reinterpret_cast<uint4*>(s.a[buf] + row * kARow + half * 32);
  da[0] = masked(ra[0], a_on);
  da[1] = masked(ra[1], a_on);
  *reinterpret_cast<uint4*>(s.w[buf] + row * kWRow + half * 16) = masked(rw, w_on);
}

// 16 codes (times 16) of 16 consecutive input channels from their 8 packed bytes
__device__ __forceinline__ v4i unpack16(uint2 d) {
  v4i o;
  o[0] = (int)((d.x << 4) & 0xF0F0F0F0u);
  o[1] = (int)(d.x & 0xF0F0F0F0u);
  o[2] = (int)((d.y << 4) & 0xF0F0F0F0u);
  o[3] = (int)(d.y & 0xF0F0F0F0u);
  return o;
}

// (sa / 16) * sw[n, g], 0 for a column past N or an invalid weight scale
__device__ __forceinline__ float group_scale(const GemmParams& p, int64_t n, int64_t ngroups,
                                             int64_t g, float sa16) {
  if (n >= p.N) return 0.0f;
  const float sw = p.w_scales[n * ngroups + g];
  return scale_ok(sw) ? sa16 * sw : 0.0f;
}

template <bool GROUPED>
__global__ __launch_bounds__(256) void k_gemm_w4a8(GemmParams p) {
  __shared__ __align__(16) GemmSmem s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
  const int64_t nk = p.K / kBK;
  const int64_t steps_per_group = p.group / kBK;
  const int kh = lane >> 5;
  // activation scale over 16 (the unpacked weight codes carry a factor 16); an invalid scale
  // gives 0 as the activations are then all 0
  const float sa = p.a_scale[0];
  const float sa16 = scale_ok(sa) ? sa * 0.0625f : 0.0f;

  v16i acc[2][2];
  float out[GROUPED ? 2 : 1][GROUPED ? 2 : 1][GROUPED ? 16 : 1];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      acc[mt][nt] = v16i{};
      if (GROUPED)
#pragma unroll
        for (int r = 0; r < 16; ++r) out[GROUPED ? mt : 0][GROUPED ? nt : 0][GROUPED ? r : 0] = 0.0f;
    }

  // this lane's output column of column tile nt is ncol0 + 32 nt
  const int64_t ncol0 = n0 + wn * 64 + (lane & 31);
  const int64_t ngroups = p.K / p.group;

  // rows of this thread's loads inside M and N
  const bool a_on = m0 + (tid >> 1) < p.M, w_on = n0 + (tid >> 1) < p.N;
  uint4 ra[2], rw;
  load_step(p, m0, n0, 0, tid, ra, rw);
  store_step(s, 0, tid, a_on, w_on, ra, rw);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < nk) load_step(p, m0, n0, kt + 1, tid, ra, rw);
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      v4i av[2], bv[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        av[mt] = *reinterpret_cast<const v4i*>(s.a[buf] + (wm * 64 + mt * 32 + (lane & 31)) * kARow +
                                               ks * 32 + 16 * kh);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        bv[nt] = unpack16(*reinterpret_cast<const uint2*>(
            s.w[buf] + (wn * 64 + nt * 32 + (lane & 31)) * kWRow + ks * 16 + 8 * kh));
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[mt], bv[nt], acc[mt][nt], 0, 0, 0);
    }
    if (GROUPED && (kt + 1) % steps_per_group == 0) {
      // end of a weight group: scale its exact int32 sums into fp32
      const int64_t g = kt / steps_per_group;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float f = group_scale(p, ncol0 + 32 * nt, ngroups, g, sa16);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            out[GROUPED ? mt : 0][GROUPED ? nt : 0][GROUPED ? r : 0] =
                fmaf(f, (float)acc[mt][nt][r], out[GROUPED ? mt : 0][GROUPED ? nt : 0][GROUPED ? r : 0]);
          acc[mt][nt] = v16i{};
        }
      }
    }
    if (kt + 1 < nk) {
      store_step(s, buf ^ 1, tid, a_on, w_on, ra, rw);
      __syncthreads();
    }
  }

  // y = bias + out; register r of a tile holds row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int64_t n = ncol0 + 32 * nt;
    if (n >= p.N) continue;
    const float bn = p.bias ? p.bias[n] : 0.0f;
    const float f = GROUPED ? 0.0f : group_scale(p, n, ngroups, 0, sa16);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + mt * 32 + 8 * (r / 4) + 4 * kh + (r % 4);
        if (m >= p.M) continue;
        const float v = GROUPED ? out[GROUPED ? mt : 0][GROUPED ? nt : 0][GROUPED ? r : 0] + bn
                                : fmaf(f, (float)acc[mt][nt][r], bn);
        if (p.yf16) reinterpret_cast<__half*>(p.y)[m * p.N + n] = __float2half_rn(v);
        else reinterpret_cast<float*>(p.y)[m * p.N + n] = v;
      }
  }
}

// Few-token form (one weight scale per output channel): BM x BN tiles of y (BM = 64 or 128, BN =
// 64 or 128; four waves, wave (wm, wn) owning a BM / 2 x BN / 2 block), K in steps of 128 through
// double-buffered LDS (rows padded to 144 and 72 bytes), with the global loads of each step issued
// kDeep steps ahead (kDeep register sets, named statically by unrolling the K loop kDeep times).
// With few tokens a tile's K loop is a chain of short steps and a load issued one step ahead is
// not back in time: the loop waits out a memory latency per step. The loads are unconditional
// (the steps past the end reload the last one), so that the compiler's waits for each register
// set stay exact, and they go through buffer resources that end at the tensors' ends: rows past M
// or N read as zero, and the stores to LDS need no mask (a mask is a select on the loaded
// registers, which the scheduler may hoist into earlier steps together with a wait for those
// loads). The row tiles that share weight columns run on one XCD: the tiles, row tile fastest,
// are cut into 8 contiguous ranges, one per XCD (workgroups are dealt to the XCDs in turn; the grid
// is padded to a multiple of 8 and the padding exits at once).
constexpr int kBKd = 128;   // K step
constexpr int kARowD = 144;  // padded bytes of an activation row in LDS (128 + 16)
constexpr int kWRowD = 72;   // padded bytes of a packed weight row in LDS (64 + 8)
constexpr int kDeep = 4;     // steps the loads run ahead
constexpr int kBufferWord3 = 0x00020000;  // buffer resource word 3 for raw 32-bit access (gfx9)

// Raw buffer resource over the n bytes at ptr (a kernel argument: wave-uniform); loads past n
// bytes return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tensor_rsrc(const void* ptr, int64_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(ptr), (short)0, (int)n, kBufferWord3);
}

template <int BM, int BN>
struct GemmSmemD {
  int8_t a[2][BM * kARowD];
  uint8_t w[2][BN * kWRowD];
};

// One K step in registers: activation chunks c = tid + 256 i (row c / 8, 16 bytes at 16 (c % 8))
// and weight chunks c = tid + 256 i (row c / 4, 16 packed bytes at 16 (c % 4)).
template <int BM, int BN>
struct StageD {
  uint4 a[BM / 32];
  uint4 w[BN / 64];
};

// Buffer loads of K step kt, at the byte offsets aoff and woff of step 0.
template <int BM, int BN>
__device__ __forceinline__ void load_deep(__amdgpu_buffer_rsrc_t rsa, __amdgpu_buffer_rsrc_t rsw,
                                          const int (&aoff)[BM / 32], const int (&woff)[BN / 64],
                                          int kt, StageD<BM, BN>& st) {
#pragma unroll
  for (int i = 0; i < BM / 32; ++i)
    st.a[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsa, aoff[i] + kt * kBKd, 0, 0));
#pragma unroll
  for (int i = 0; i < BN / 64; ++i)
    st.w[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsw, woff[i] + kt * (kBKd / 2), 0, 0));
}

template <int BM, int BN>
__device__ __forceinline__ void store_deep(GemmSmemD<BM, BN>& s, int buf, int tid,
                                           const StageD<BM, BN>& st) {
#pragma unroll
  for (int i = 0; i < BM / 32; ++i) {
    const int c = tid + 256 * i;
    *reinterpret_cast<uint4*>(s.a[buf] + (c >> 3) * kARowD + (c & 7) * 16) = st.a[i];
  }
#pragma unroll
  for (int i = 0; i < BN / 64; ++i) {
    const int c = tid + 256 * i;
    *reinterpret_cast<uint4*>(s.w[buf] + (c >> 2) * kWRowD + (c & 3) * 16) = st.w[i];
  }
}

template <int BM, int BN>
__global__ __launch_bounds__(256) void k_gemm_w4a8_deep(GemmParams p) {
  constexpr int MT = BM / 64, NT = BN / 64;  // 32 x 32 MFMA tiles of a wave's block
  __shared__ __align__(16) GemmSmemD<BM, BN> s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int kh = lane >> 5;
  const int64_t nm = (p.M + BM - 1) / BM, T = nm * ((p.N + BN - 1) / BN);
  const int64_t id = (int64_t)(blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  if (id >= T) return;  // grid padding (the whole workgroup)
  const int64_t m0 = (id % nm) * BM, n0 = (id / nm) * BN;
  const int nk1 = (int)(p.K / kBKd) - 1;  // K / kBKd is a multiple of kDeep (host)
  const float sa = p.a_scale[0];
  const float sa16 = scale_ok(sa) ? sa * 0.0625f : 0.0f;

  v16i acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v16i{};

  // 32-bit offsets: the host checks M * K < 2^31 and N * K / 2 < 2^31 for this form
  const __amdgpu_buffer_rsrc_t rsa = tensor_rsrc(p.a, p.M * p.K);
  const __amdgpu_buffer_rsrc_t rsw = tensor_rsrc(p.w, p.N * (p.K / 2));
  int aoff[BM / 32], woff[BN / 64];
#pragma unroll
  for (int i = 0; i < BM / 32; ++i) {
    const int c = tid + 256 * i;
    aoff[i] = (int)((m0 + (c >> 3)) * p.K) + (c & 7) * 16;
  }
#pragma unroll
  for (int i = 0; i < BN / 64; ++i) {
    const int c = tid + 256 * i;
    woff[i] = (int)((n0 + (c >> 2)) * (p.K / 2)) + (c & 3) * 16;
  }
  // register set d holds K step kt with kt % kDeep == d, until it is stored to LDS
  StageD<BM, BN> st[kDeep];
#pragma unroll
  for (int d = 0; d < kDeep; ++d) load_deep<BM, BN>(rsa, rsw, aoff, woff, min(d, nk1), st[d]);
  store_deep<BM, BN>(s, 0, tid, st[0]);
  load_deep<BM, BN>(rsa, rsw, aoff, woff, min(kDeep, nk1), st[0]);
  __syncthreads();
  for (int k0 = 0; k0 <= nk1; k0 += kDeep) {
#pragma unroll
    for (int d = 0; d < kDeep; ++d) {
      const int kt = k0 + d;
      const int buf = d & 1;  // kt & 1: k0 is even
#pragma unroll
      for (int ks = 0; ks < kBKd / 32; ++ks) {
        v4i av[MT], bv[NT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          av[mt] = *reinterpret_cast<const v4i*>(
              s.a[buf] + (wm * (BM / 2) + mt * 32 + (lane & 31)) * kARowD + ks * 32 + 16 * kh);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          bv[nt] = unpack16(*reinterpret_cast<const uint2*>(
              s.w[buf] + (wn * (BN / 2) + nt * 32 + (lane & 31)) * kWRowD + ks * 16 + 8 * kh));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[mt], bv[nt], acc[mt][nt], 0, 0, 0);
      }
      // step kt + 1 (loaded kDeep steps ago) into the other stage, then step kt + 1 + kDeep into
      // the registers it leaves free (after the last step: an unused stage and the last step again)
      const int nx = (d + 1) % kDeep;
      store_deep<BM, BN>(s, buf ^ 1, tid, st[nx]);
      load_deep<BM, BN>(rsa, rsw, aoff, woff, min(kt + 1 + kDeep, nk1), st[nx]);
      __syncthreads();
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the reloads of the last steps have landed

  // y = bias + (sa / 16) sw[n] acc; register r of a tile holds row 8 (r / 4) + 4 (l / 32) + r % 4,
  // column l % 32
  const int64_t ncol0 = n0 + wn * (BN / 2) + (lane & 31);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t n = ncol0 + 32 * nt;
    if (n >= p.N) continue;
    const float bn = p.bias ? p.bias[n] : 0.0f;
    const float f = group_scale(p, n, 1, 0, sa16);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * (BM / 2) + mt * 32 + 8 * (r / 4) + 4 * kh + (r % 4);
        if (m >= p.M) continue;
        const float v = fmaf(f, (float)acc[mt][nt][r], bn);
        if (p.yf16) reinterpret_cast<__half*>(p.y)[m * p.N + n] = __float2half_rn(v);
        else reinterpret_cast<float*>(p.y)[m * p.N + n] = v;
      }
  }
}

// Launches the few-token form with BM-row tiles: 128-column tiles when they all fit one per CU,
// else 64-column tiles when they fit three per CU (their registers and LDS allow three), else
// 128-column tiles when they fit two per CU (128 x 128: two per CU). Returns false when none fits.
template <int BM>
bool launch_deep(const GemmParams& p, hipStream_t stream) {
  const int64_t nm = (p.M + BM - 1) / BM;
  const int64_t t128 = nm * ((p.N + 127) / 128), t64 = nm * ((p.N + 63) / 64);
  const auto grid = [](int64_t t) { return (unsigned)((t + 7) / 8 * 8); };
  if (t128 <= 256) k_gemm_w4a8_deep<BM, 128><<<grid(t128), 256, 0, stream>>>(p);
  else if (t64 <= 768) k_gemm_w4a8_deep<BM, 64><<<grid(t64), 256, 0, stream>>>(p);
  else if (t128 <= 512) k_gemm_w4a8_deep<BM, 128><<<grid(t128), 256, 0, stream>>>(p);
  else return false;
  return true;
}

// Large-M form (one weight scale per output channel): 128 x 256 tiles of y, four waves each
// owning a 64 x 128 block (2 x 4 tiles of v_mfma_i32_32x32x32_i8, 16 MFMAs per K step of 64), and
// the global loads run two K steps ahead of the products (two register sets; the LDS stages are
// double-buffered), so that a load's latency is covered by two steps of products. The tiles are
// ordered in groups of 8 row tiles (row tile fastest) and the order is cut into 8 contiguous
// ranges, one per XCD (workgroups are dealt to the XCDs in turn), so that the workgroups that run
// together on one XCD share their A rows and weight columns in that XCD's L2.
constexpr int kBN2 = 256;

struct GemmSmem2 {
  int8_t a[2][kBM * kARow];
  int8_t w[2][kBN2 * kARow];  // weight codes times 16, unpacked once per step: rows of 64 + 16 bytes
};

struct Stage2 {
  uint4 a[2], w[2];
};

// K step kt: thread t takes A chunks c = t, t + 256 (row c / 4, 16 bytes at 16 (c % 4)) and
// weight chunks c = t, t + 256 (row c / 2, 16 packed bytes at 16 (c % 2)); rows past M or N load
// a valid row and are zeroed by the store.
__device__ __forceinline__ void load2(const GemmParams& p, int64_t m0, int64_t n0, int64_t kt,
                                      int tid, Stage2& st) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    const int64_t m = min(m0 + (c >> 2), p.M - 1);
    st.a[i] = *reinterpret_cast<const uint4*>(p.a + m * p.K + kt * kBK + (c & 3) * 16);
    const int64_t n = min(n0 + (c >> 1), p.N - 1);
    st.w[i] = *reinterpret_cast<const uint4*>(p.w + n * (p.K / 2) + kt * (kBK / 2) + (c & 1) * 16);
  }
}

// Stores a K step into LDS stage buf: the A chunks as they are, the weight chunks unpacked (16
// packed bytes -> 32 code bytes, 32 k in order); an interior tile stores without masks.
__device__ __forceinline__ void store2(const GemmParams& p, GemmSmem2& s, int buf, int64_t m0,
                                       int64_t n0, bool interior, int tid, const Stage2& st) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    uint4 av = st.a[i], wv = st.w[i];
    if (!interior) {
      av = masked(av, m0 + (c >> 2) < p.M);
      wv = masked(wv, n0 + (c >> 1) < p.N);
    }
    *reinterpret_cast<uint4*>(s.a[buf] + (c >> 2) * kARow + (c & 3) * 16) = av;
    const v4i lo = unpack16(make_uint2(wv.x, wv.y)), hi = unpack16(make_uint2(wv.z, wv.w));
    int8_t* wd = s.w[buf] + (c >> 1) * kARow + (c & 1) * 32;
    *reinterpret_cast<v4i*>(wd) = lo;
    *reinterpret_cast<v4i*>(wd + 16) = hi;
  }
}

__global__ __launch_bounds__(256, 2) void k_gemm_w4a8_wide(GemmParams p) {
  __shared__ __align__(16) GemmSmem2 s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int kh = lane >> 5;
  // tile of this workgroup
  const int64_t nm = (p.M + kBM - 1) / kBM, nn = (p.N + kBN2 - 1) / kBN2, T = nm * nn;
  int64_t id = blockIdx.x;
  if (T % 8 == 0) id = (id % 8) * (T / 8) + id / 8;
  constexpr int64_t kGM = 8;
  const int64_t grp = id / (kGM * nn), fm = grp * kGM;
  const int64_t gsz = min(nm - fm, kGM), within = id - grp * kGM * nn;
  const int64_t m0 = (fm + within % gsz) * kBM, n0 = (within / gsz) * kBN2;
  const int64_t nk = p.K / kBK;
  const bool interior = m0 + kBM <= p.M && n0 + kBN2 <= p.N;
  const float sa = p.a_scale[0];
  const float sa16 = scale_ok(sa) ? sa * 0.0625f : 0.0f;

  v16i acc[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = v16i{};

  Stage2 st[2];
  load2(p, m0, n0, 0, tid, st[0]);
  load2(p, m0, n0, min((int64_t)1, nk - 1), tid, st[1]);
  store2(p, s, 0, m0, n0, interior, tid, st[0]);
  load2(p, m0, n0, min((int64_t)2, nk - 1), tid, st[0]);
  __syncthreads();
  // one K step: the products from LDS stage kt % 2, then step kt + 1 (loaded two steps ago, held
  // in nx) into the other stage and step kt + 3 into the registers it leaves free
  auto step = [&](int64_t kt, Stage2& nx) {
    const int buf = (int)(kt & 1);
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      v4i av[2], bv[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        av[mt] = *reinterpret_cast<const v4i*>(s.a[buf] + (wm * 64 + mt * 32 + (lane & 31)) * kARow +
                                               ks * 32 + 16 * kh);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        bv[nt] = *reinterpret_cast<const v4i*>(s.w[buf] + (wn * 128 + nt * 32 + (lane & 31)) * kARow +
                                               ks * 32 + 16 * kh);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[mt], bv[nt], acc[mt][nt], 0, 0, 0);
    }
    // unconditional, so that the compiler's wait for these registers stays exact (the last steps
    // store into the unused stage and reload the last step)
    store2(p, s, buf ^ 1, m0, n0, interior, tid, nx);
    load2(p, m0, n0, min(kt + 3, nk - 1), tid, nx);
    __syncthreads();
  };
  // the loop is unrolled twice so that the register sets are named statically (step kt + 1 lives
  // in st[1] when kt is even, in st[0] when it is odd)
  // (nk is even here: the host takes this form only for K % 128 == 0)
  for (int64_t kt = 0; kt < nk; kt += 2) {
    step(kt, st[1]);
    step(kt + 1, st[0]);
  }
  __builtin_amdgcn_s_waitcnt(0);  // the reloads of the last steps have landed

  // y = bias + (sa / 16) sw[n] acc; register r of a tile holds row 8 (r / 4) + 4 (l / 32) + r % 4,
  // column l % 32
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t n = n0 + wn * 128 + nt * 32 + (lane & 31);
    if (n >= p.N) continue;
    const float bn = p.bias ? p.bias[n] : 0.0f;
    const float f = group_scale(p, n, 1, 0, sa16);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + mt * 32 + 8 * (r / 4) + 4 * kh + (r % 4);
        if (m >= p.M) continue;
        const float v = fmaf(f, (float)acc[mt][nt][r], bn);
        if (p.yf16) reinterpret_cast<__half*>(p.y)[m * p.N + n] = __float2half_rn(v);
        else reinterpret_cast<float*>(p.y)[m * p.N + n] = v;
      }
  }
}

}  // namespace

extern "C" qssm_status qssm_gemm_w4a8(const qssm_gemm_args* a, hipStream_t stream) {
  clear_error();
  if (!a) return fail(QSSM_ERR_INVALID_ARG, "args is null");
  const int64_t M = a->M, N = a->N, K = a->K;
  if (M < 0 || N < 0 || K < 0) return fail(QSSM_ERR_INVALID_ARG, "negative extent");
  if (a->y_dtype != QSSM_F32 && a->y_dtype != QSSM_F16)
    return fail(QSSM_ERR_INVALID_ARG, "y_dtype must be QSSM_F32 or QSSM_F16");
  if (K <= 0 || K % kBK != 0) return fail(QSSM_ERR_UNSUPPORTED, "K must be a positive multiple of 64");
  if (a->group < kBK || a->group % kBK != 0 || K % a->group != 0)
    return fail(QSSM_ERR_UNSUPPORTED, "group must be a multiple of 64 that divides K");
  if (a->group > 131072) return fail(QSSM_ERR_UNSUPPORTED, "group above 131072 (int32 sums)");
  if (M == 0 || N == 0) return QSSM_OK;
  if (!a->a_scale || !a->w_scales || !a->a || !a->w || !a->y)
    return fail(QSSM_ERR_INVALID_ARG, "null required pointer");
  if (((uintptr_t)a->a | (uintptr_t)a->w) % 16 != 0)
    return fail(QSSM_ERR_INVALID_ARG, "a and w must be 16-byte aligned");
  const int64_t gx = (N + kBN - 1) / kBN, gy = (M + kBM - 1) / kBM;
  if (gx > 0x7fffffff || gy > 65535) return fail(QSSM_ERR_UNSUPPORTED, "grid too large");
  GemmParams p{M, N, K, a->group, a->y_dtype == QSSM_F16, a->a, a->a_scale, a->w, a->w_scales,
               a->bias, a->y};
  const dim3 grid((unsigned)gx, (unsigned)gy);
  // one scale per output channel: the wide-tile form for many tokens (enough tiles to fill the
  // GPU); for few tokens the form with loads kDeep steps ahead when K allows it and its tiles all
  // run at once (64-row tiles up to 64 tokens: no MFMA work on rows past M); the 128 x 128 form
  // with one step ahead otherwise and for weight groups
  const int64_t wide_tiles = gy * ((N + kBN2 - 1) / kBN2);
  const bool deep = a->group == K && M < kWideMinM && K % (kBKd * kDeep) == 0 &&
                    M * K < ((int64_t)1 << 31) && N * (K / 2) < ((int64_t)1 << 31);
  if (a->group == K && M >= kWideMinM && K % (2 * kBK) == 0 && wide_tiles <= 0x7fffffff) {
    k_gemm_w4a8_wide<<<(unsigned)wide_tiles, 256, 0, stream>>>(p);
  } else if (!deep || !(M <= 64 ? launch_deep<64>(p, stream) : launch_deep<128>(p, stream))) {
    if (a->group == K) k_gemm_w4a8<false><<<grid, 256, 0, stream>>>(p);
    else k_gemm_w4a8<true><<<grid, 256, 0, stream>>>(p);
  }
  return launch_status("gemm_w4a8");
}
