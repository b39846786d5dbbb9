// f3: on-device soft-edge threshold tracking.
//
// Quamba-SE blog, section 4.1: the low threshold L sits at the 5th and the high threshold H at the
// 99.9th percentile of |activation|, followed over mini-batches by an exponential moving average.
// Here both percentiles of every group are found exactly on the device by radix selection over
// the bit patterns of |x| (non-negative floats order like their bits), so that the thresholds
// equal what the host computes from a full sort, and no host round trip sits between a batch and
// its encode.
//
// Per group, four order statistics are selected: ranks k and k+1 of each percentile's
// interpolation. The 31 magnitude bits are resolved in four digits from the top (8, 8, 8, 7 bits):
//  * k_track_count<P>: one pass over x. Every value whose already-resolved high bits equal a
//    target's prefix is counted in that target's 256-bin histogram of the next digit. Histograms
//    live in LDS per workgroup (32-bit counts) and are added to a global 64-bit histogram at the
//    end. Pass 0 has a single histogram per group (every target starts with an empty prefix).
//  * k_track_select<P>: one workgroup per group, one wave per target. A wave prefix sum over the
//    256 bins finds the bin holding the target's rank; the bin extends the prefix and the rank
//    becomes the rank inside the bin. The wave then clears the bins it read for the next pass.
//    After pass 0 it also counts the group's values and places the targets; after pass 3 the
//    prefixes are the selected values and the last select applies the interpolation and the EMA
//    in fp64, in the order the host helper uses.
// Traffic: four reads of x; everything else is a few KB per group.
#include <hip/hip_runtime.h>

#include "common.hpp"

using namespace qssm;

namespace {

constexpr int kThreads = 1024;   // counting workgroup
constexpr int kIters = 8;        // chunks of 4 values per thread
constexpr int64_t kPerBlock = (int64_t)kThreads * 4 * kIters;
constexpr int kBins = 256;
constexpr int kTargets = 4;      // ranks k_lo, k_lo + 1, k_hi, k_hi + 1
constexpr int kMaxGroups = 32;
constexpr double kPLow = 5.0, kPHigh = 99.9;

// low bit of the digit resolved by pass P, and the digit width
__host__ __device__ constexpr int digit_low(int pass) { return pass == 0 ? 23 : (pass == 1 ? 15 : (pass == 2 ? 7 : 0)); }
__host__ __device__ constexpr uint32_t digit_mask(int pass) { return pass == 3 ? 0x7Fu : 0xFFu; }

struct Target {
  uint32_t prefix;  // magnitude bits resolved so far (lower bits zero)
  uint32_t active;  // 0 for the targets of an empty group
  uint64_t rank;    // rank among the values that carry the prefix
};

struct GroupMeta {
  uint64_t n;     // values in the group
  double vi[2];   // interpolation positions of the two percentiles
};

struct Workspace {
  uint64_t* hist;   // [G][kTargets][kBins]
  Target* tgt;      // [G][kTargets]
  GroupMeta* meta;  // [G]
};

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t hist_bytes(int G) { return align256((size_t)G * kTargets * kBins * sizeof(uint64_t)); }
size_t tgt_bytes(int G) { return align256((size_t)G * kTargets * sizeof(Target)); }
size_t meta_bytes(int G) { return align256((size_t)G * sizeof(GroupMeta)); }

Workspace carve(void* base, int G) {
  char* p = reinterpret_cast<char*>(base);
  Workspace w;
  w.hist = reinterpret_cast<uint64_t*>(p);
  w.tgt = reinterpret_cast<Target*>(p + hist_bytes(G));
  w.meta = reinterpret_cast<GroupMeta*>(p + hist_bytes(G) + tgt_bytes(G));
  return w;
}

struct Geometry {
  int64_t total, C, inner;
  const int32_t* perm;
  const uint8_t* group_of;
  int G;
};

__global__ void k_track_clear(uint64_t* __restrict__ hist, int n) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n) hist[k] = 0;
}

// a / b in 32-bit arithmetic when both fit
__device__ __forceinline__ int64_t div_fast(int64_t a, int64_t b) {
  if (((uint64_t)a | (uint64_t)b) >> 32 == 0) return (int64_t)((uint32_t)a / (uint32_t)b);
  return a / b;
}

template <int PASS, int GMAX>
__global__ __launch_bounds__(kThreads) void k_track_count(const float* __restrict__ x, Geometry g,
                                                          const Target* __restrict__ tgt,
                                                          uint64_t* __restrict__ hist) {
  constexpr int kSlots = PASS == 0 ? 1 : kTargets;
  constexpr int kCells = GMAX * kSlots * kBins;
  __shared__ uint32_t h[kCells];
  __shared__ uint32_t pref[PASS == 0 ? 1 : GMAX * kTargets];
  __shared__ uint32_t act[PASS == 0 ? 1 : GMAX * kTargets];
  for (int k = threadIdx.x; k < kCells; k += kThreads) h[k] = 0u;
  if (PASS > 0) {
    for (int k = threadIdx.x; k < g.G * kTargets; k += kThreads) {
      pref[k] = tgt[k].prefix;
      act[k] = tgt[k].active;
    }
  }
  __syncthreads();
  constexpr int lowp = PASS == 0 ? 31 : digit_low(PASS - 1);  // resolved bits: [lowp, 31)
  constexpr int low = digit_low(PASS);
  constexpr uint32_t dmask = digit_mask(PASS);
  auto count = [&](float v, int grp) {
    const uint32_t u = __float_as_uint(v) & 0x7FFFFFFFu;
    const uint32_t d = (u >> low) & dmask;
    if (PASS == 0) {
      atomicAdd(&h[grp * kBins + d], 1u);
    } else {
#pragma unroll
      for (int t = 0; t < kTargets; ++t) {
        const int k = grp * kTargets + t;
        if (act[k] && (u >> lowp) == (pref[k] >> lowp)) atomicAdd(&h[k * kBins + d], 1u);
      }
    }
  };
  const int64_t base = (int64_t)blockIdx.x * kPerBlock;
  const bool rows4 = g.inner % 4 == 0;
#pragma unroll 2
  for (int it = 0; it < kIters; ++it) {
    const int64_t e = base + ((int64_t)it * kThreads + threadIdx.x) * 4;
    if (e >= g.total) break;
    if (rows4) {
      // 4 values in one row: one group, one 16-byte load
      const int64_t row = div_fast(e, g.inner), i = e - row * g.inner;
      const int64_t o = div_fast(row, g.C), c = row - o * g.C;
      const int64_t src = g.perm ? (int64_t)g.perm[c] : c;
      const int grp = min((int)g.group_of[c], g.G - 1);
      const float4 v = *reinterpret_cast<const float4*>(x + (o * g.C + src) * g.inner + i);
      count(v.x, grp);
      count(v.y, grp);
      count(v.z, grp);
      count(v.w, grp);
    } else {
      for (int j = 0; j < 4 && e + j < g.total; ++j) {
        const int64_t row = div_fast(e + j, g.inner), i = e + j - row * g.inner;
        const int64_t o = div_fast(row, g.C), c = row - o * g.C;
        const int64_t src = g.perm ? (int64_t)g.perm[c] : c;
        count(x[(o * g.C + src) * g.inner + i], min((int)g.group_of[c], g.G - 1));
      }
    }
  }
  __syncthreads();
  for (int k = threadIdx.x; k < g.G * kSlots * kBins; k += kThreads) {
    const uint32_t n = h[k];
    if (n) {
      // global layout [G][kTargets][kBins]; pass 0 uses slot 0 of each group
      const int gi = PASS == 0 ? (k / kBins) * kTargets * kBins + (k % kBins) : k;
      atomicAdd(reinterpret_cast<unsigned long long*>(hist + gi), (unsigned long long)n);
    }
  }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint64_t wave_inclusive_sum(uint64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// Percentile positions, interpolation and EMA in fp64, every operation rounded as written (the
// host helper's order; no contraction into fused multiply-adds).
__device__ double position(uint64_t n, double pct) {
#pragma clang fp contract(off)
  const double q = pct / 100.0;
  return (double)(n - 1) * q;
}

__device__ double interpolate(double vi, double a, double b, uint64_t n) {
#pragma clang fp contract(off)
  if (vi >= (double)(n - 1) || vi < 0.0) return a;  // a is then the selected end value
  const double t = vi - floor(vi);
  const double diff = b - a;
  if (t >= 0.5) return b - diff * (1.0 - t);
  return a + diff * t;
}

__device__ double ema(double alpha, double now, double prev) {
#pragma clang fp contract(off)
  return alpha * now + (1.0 - alpha) * prev;
}

template <int PASS>
__global__ __launch_bounds__(256) void k_track_select(Workspace ws, int G, double alpha,
                                                      int ema_valid, double* __restrict__ state,
                                                      float* __restrict__ s_out,
                                                      float* __restrict__ L_out,
                                                      float* __restrict__ H_out) {
  const int grp = blockIdx.x;
  const int t = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __shared__ Target s_tg[kTargets];  // the group's targets as this kernel leaves them
  Target* tg = ws.tgt + grp * kTargets;
  const int slot = PASS == 0 ? 0 : t;
  uint64_t* hb = ws.hist + ((size_t)grp * kTargets + slot) * kBins;
  uint64_t c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = hb[lane * 4 + j];
  const uint64_t mine = c[0] + c[1] + c[2] + c[3];
  const uint64_t incl = wave_inclusive_sum(mine);
  if (PASS == 0) {
    // the group's size, then the targets: ranks k and k + 1 of each percentile's interpolation
    const uint64_t n = __shfl(incl, 63, 64);
    if (threadIdx.x == 0) {
      GroupMeta m;
      m.n = n;
      m.vi[0] = n > 0 ? position(n, kPLow) : 0.0;
      m.vi[1] = n > 0 ? position(n, kPHigh) : 0.0;
      ws.meta[grp] = m;
      for (int j = 0; j < 2; ++j) {
        uint64_t k0 = 0, k1 = 0;
        if (n > 0) {
          const double vi = m.vi[j];
          if (vi >= (double)(n - 1)) k0 = k1 = n - 1;
          else if (vi < 0.0) k0 = k1 = 0;
          else { k0 = (uint64_t)floor(vi); k1 = k0 + 1; }
        }
        s_tg[2 * j] = Target{0u, n > 0 ? 1u : 0u, k0};
        s_tg[2 * j + 1] = Target{0u, n > 0 ? 1u : 0u, k1};
      }
    }
  } else if (lane == 0) {
    s_tg[t] = tg[t];
  }
  __syncthreads();
  const Target me = s_tg[t];
  __syncthreads();
  if (me.active) {
    // the bin holding rank `me.rank`: lanes own bins 4*lane .. 4*lane + 3 (exactly one matches)
    uint64_t before = incl - mine;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (me.rank >= before && me.rank < before + c[j]) {
        const uint32_t bin = (uint32_t)(lane * 4 + j);
        s_tg[t] = Target{me.prefix | (bin << digit_low(PASS)), 1u, me.rank - before};
      }
      before += c[j];
    }
  }
  __syncthreads();  // the new targets are in LDS; every wave has read the shared pass-0 histogram
  if (PASS > 0 || t == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) hb[lane * 4 + j] = 0;
  }
  if (lane == 0) tg[t] = s_tg[t];
  if (PASS == 3 && threadIdx.x == 0) {
    const GroupMeta m = ws.meta[grp];
    double lh[2];
    const bool empty = m.n == 0;
    for (int j = 0; j < 2; ++j) {
      const double a = (double)__uint_as_float(s_tg[2 * j].prefix);
      const double b = (double)__uint_as_float(s_tg[2 * j + 1].prefix);
      lh[j] = empty ? 0.0 : interpolate(m.vi[j], a, b, m.n);
    }
    double l, h;
    if (empty) {
      l = ema_valid ? state[2 * grp] : 0.0;
      h = ema_valid ? state[2 * grp + 1] : 0.0;
    } else if (ema_valid) {
      l = ema(alpha, lh[0], state[2 * grp]);
      h = ema(alpha, lh[1], state[2 * grp + 1]);
    } else {
      l = lh[0];
      h = lh[1];
    }
    state[2 * grp] = l;
    state[2 * grp + 1] = h;
    const float L32 = (float)l, H32 = (float)h;
    L_out[grp] = L32;
    H_out[grp] = H32;
    s_out[grp] = (H32 == 0.0f) ? 1.0f : H32 / 63.0f;
  }
}

template <int GMAX>
void launch_counts(int pass, const float* x, const Geometry& g, const Workspace& ws,
                   unsigned blocks, hipStream_t st) {
  switch (pass) {
    case 0: k_track_count<0, GMAX><<<blocks, kThreads, 0, st>>>(x, g, ws.tgt, ws.hist); break;
    case 1: k_track_count<1, GMAX><<<blocks, kThreads, 0, st>>>(x, g, ws.tgt, ws.hist); break;
    case 2: k_track_count<2, GMAX><<<blocks, kThreads, 0, st>>>(x, g, ws.tgt, ws.hist); break;
    default: k_track_count<3, GMAX><<<blocks, kThreads, 0, st>>>(x, g, ws.tgt, ws.hist); break;
  }
}

}  // namespace

extern "C" {

size_t qssm_softedge_track_workspace_size(int32_t G) {
  if (G < 1 || G > kMaxGroups) return 0;
  return hist_bytes(G) + tgt_bytes(G) + meta_bytes(G) + 256;
}

qssm_status qssm_softedge_track(const float* x, int64_t outer, int64_t C, int64_t inner,
                                const int32_t* perm, const uint8_t* group_of, int32_t G,
                                double alpha, int32_t ema_valid, double* ema_state, float* s,
                                float* L, float* H, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  clear_error();
  if (outer < 0 || C < 0 || inner < 0) return fail(QSSM_ERR_INVALID_ARG, "negative extent");
  if (outer > 0 && inner > 0 && C > 0 && outer > INT64_MAX / C / inner)
    return fail(QSSM_ERR_INVALID_ARG, "tensor too large");
  if (G < 1 || G > kMaxGroups)
    return fail(QSSM_ERR_INVALID_ARG, "G must be in 1..%d, got %d", kMaxGroups, G);
  if (!(alpha >= 0.0 && alpha <= 1.0)) return fail(QSSM_ERR_INVALID_ARG, "alpha outside [0, 1]");
  if (!ema_state || !s || !L || !H) return fail(QSSM_ERR_INVALID_ARG, "null output pointer");
  const int64_t total = outer * C * inner;
  if (total > 0 && (!x || !group_of)) return fail(QSSM_ERR_INVALID_ARG, "null tensor pointer");
  if (total > 0 && inner % 4 == 0 && reinterpret_cast<uintptr_t>(x) % 16 != 0)
    return fail(QSSM_ERR_INVALID_ARG, "x must be 16-byte aligned");
  const size_t need = qssm_softedge_track_workspace_size(G);
  if (!workspace || workspace_bytes < need)
    return fail(QSSM_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  void* base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~(uintptr_t)255);
  const Workspace ws = carve(base, G);
  const Geometry g{total, C, inner, perm, group_of, G};
  const int ncells = G * kTargets * kBins;
  k_track_clear<<<(unsigned)cdiv(ncells, 256), 256, 0, stream>>>(ws.hist, ncells);
  const unsigned blocks = (unsigned)cdiv(total, kPerBlock);
  for (int pass = 0; pass < 4; ++pass) {
    if (total > 0) {
      if (G <= 8) launch_counts<8>(pass, x, g, ws, blocks, stream);
      else launch_counts<kMaxGroups>(pass, x, g, ws, blocks, stream);
    }
    switch (pass) {
      case 0: k_track_select<0><<<G, 256, 0, stream>>>(ws, G, alpha, ema_valid, ema_state, s, L, H); break;
      case 1: k_track_select<1><<<G, 256, 0, stream>>>(ws, G, alpha, ema_valid, ema_state, s, L, H); break;
      case 2: k_track_select<2><<<G, 256, 0, stream>>>(ws, G, alpha, ema_valid, ema_state, s, L, H); break;
      default: k_track_select<3><<<G, 256, 0, stream>>>(ws, G, alpha, ema_valid, ema_state, s, L, H); break;
    }
  }
  return launch_status("softedge_track");
}

}  // extern "C"
