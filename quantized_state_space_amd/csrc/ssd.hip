// a8-a13: Mamba2 SSD chunked form with an int8 path (work in progress: entry points validate and
// report QSSM_ERR_UNSUPPORTED until the kernels land).
#include <hip/hip_runtime.h>

#include "common.hpp"

using namespace qssm;

extern "C" {

size_t qssm_ssd_workspace_size(const qssm_ssd_args* a) { return a ? 0 : 0; }

qssm_status qssm_ssd_chunk_int8(const qssm_ssd_args* a, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  (void)ws; (void)ws_bytes; (void)stream;
  clear_error();
  if (!a) return fail(QSSM_ERR_INVALID_ARG, "args is null");
  return fail(QSSM_ERR_UNSUPPORTED, "SSD chunked kernels are not built yet");
}

}  // extern "C"
