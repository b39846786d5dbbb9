// Measurement support: instruction-rate loops behind the roofline figures of the scans and the
// SSD contractions (how fast v_exp_f32 issues, alone and mixed with FMA, and the dense MFMA rates
// of the two operand types the SSD kernels use). Each thread (or wave, for MFMA) runs independent
// chains so that the loop measures issue rate, not latency; the results go to a sink so that
// nothing is optimized away.
#include <hip/hip_runtime.h>

#include "common.hpp"

using namespace qssm;

namespace {

constexpr int kThreads = 256;
constexpr int kChains = 8;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

template <int KIND>
__global__ __launch_bounds__(kThreads) void k_probe(int64_t iters, float* __restrict__ sink) {
  const int tid = blockIdx.x * kThreads + threadIdx.x;
  if (KIND <= QSSM_PROBE_EXP_FMA) {
    float e[kChains], f[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      e[c] = -1e-3f * (float)(c + 1 + (tid & 7));
      f[c] = 1.0f + 1e-7f * (float)c;
    }
    const float m = 0.999999f, a = 1e-9f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) {
        // one v_exp_f32 per chain step (the value runs up to +inf, where it stays; the issue
        // rate does not depend on it), one v_fma_f32 per fma chain step
        if (KIND != QSSM_PROBE_FMA) e[c] = __builtin_amdgcn_exp2f(e[c]);
        if (KIND != QSSM_PROBE_EXP) f[c] = fmaf(f[c], m, a);
      }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += e[c] + f[c];
    sink[tid] = s;
  } else if (KIND == QSSM_PROBE_MFMA_I8) {
    const v4i a = {tid, tid + 1, tid + 2, tid + 3};
    v16i acc0 = {}, acc1 = {};
    for (int64_t it = 0; it < iters; ++it) {
      acc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, acc1, 0, 0, 0);
    }
    sink[tid] = (float)(acc0[0] + acc1[15]);
  } else {
    const v8h a = {(_Float16)1, (_Float16)2, (_Float16)3, (_Float16)4,
                   (_Float16)5, (_Float16)6, (_Float16)7, (_Float16)(tid & 7)};
    v16f acc0 = {}, acc1 = {};
    for (int64_t it = 0; it < iters; ++it) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, acc1, 0, 0, 0);
    }
    sink[tid] = acc0[0] + acc1[15];
  }
}

}  // namespace

extern "C" {

qssm_status qssm_probe_rate(int32_t kind, int64_t iters, int32_t blocks, float* sink,
                            hipStream_t stream) {
  clear_error();
  if (kind < QSSM_PROBE_EXP || kind > QSSM_PROBE_MFMA_F16)
    return fail(QSSM_ERR_INVALID_ARG, "unknown probe kind %d", kind);
  if (iters < 1 || blocks < 1) return fail(QSSM_ERR_INVALID_ARG, "iters and blocks must be positive");
  if (!sink) return fail(QSSM_ERR_INVALID_ARG, "sink is null");
  switch (kind) {
    case QSSM_PROBE_EXP: k_probe<QSSM_PROBE_EXP><<<blocks, kThreads, 0, stream>>>(iters, sink); break;
    case QSSM_PROBE_FMA: k_probe<QSSM_PROBE_FMA><<<blocks, kThreads, 0, stream>>>(iters, sink); break;
    case QSSM_PROBE_EXP_FMA:
      k_probe<QSSM_PROBE_EXP_FMA><<<blocks, kThreads, 0, stream>>>(iters, sink);
      break;
    case QSSM_PROBE_MFMA_I8:
      k_probe<QSSM_PROBE_MFMA_I8><<<blocks, kThreads, 0, stream>>>(iters, sink);
      break;
    default: k_probe<QSSM_PROBE_MFMA_F16><<<blocks, kThreads, 0, stream>>>(iters, sink); break;
  }
  return launch_status("probe");
}

}  // extern "C"
