// Host build of the library's device rounding helpers (common.hpp), so that CPU tests can check
// the exact round-half-to-even rule the kernels use against the oracle on many inputs.
#include "../quantized_state_space_amd/csrc/common.hpp"

extern "C" {

void host_quant8(const float* v, int64_t n, float s, int8_t* out) {
  const float r = qssm::recip_or_zero(s);
  for (int64_t i = 0; i < n; ++i) out[i] = qssm::quant8_r(v[i], s, r);
}

void host_quant8_div(const float* v, int64_t n, float s, int8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = qssm::quant8(v[i], s);
}

void host_softedge(const float* v, int64_t n, float s, float L, float H, int32_t ratio,
                   uint8_t* out) {
  const float r = qssm::recip_or_zero(s);
  const float m = (float)ratio, im = 1.0f / (float)ratio;
  for (int64_t i = 0; i < n; ++i) out[i] = qssm::softedge_code_r(v[i], s, r, L, H, m, im);
}

}  // extern "C"
