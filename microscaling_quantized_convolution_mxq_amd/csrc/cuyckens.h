// cuyckens.h -- launchers of the square-block comparator (cuyckens.hip), for
// the C ABI layer. Host-side only; arguments are already validated.
#pragma once
#include "mqconv_internal.h"

namespace mq {

size_t cuyckens_col_codes_bytes(const Conv& cv, int fx);
size_t cuyckens_col_scales_bytes(const Conv& cv);
size_t cuyckens_workspace_bytes(const Conv& cv, int op, int fa, int fb);
hipError_t launch_cuyckens_im2col_quantize(const Conv& cv, const float* x, int fx, uint8_t* col_codes,
                                           uint8_t* col_scales, hipStream_t st);
hipError_t launch_cuyckens_forward(const Conv& cv, const uint8_t* col_codes, const uint8_t* col_scales, int fx,
                                   const float* w, int fw, float* y, void* ws, hipStream_t st);
hipError_t launch_cuyckens_backward_data(const Conv& cv, const float* dy, const float* w, int fdy, int fw, float* dx,
                                         void* ws, hipStream_t st);
hipError_t launch_cuyckens_backward_weight(const Conv& cv, const float* dy, const uint8_t* col_codes,
                                           const uint8_t* col_scales, int fdy, int fx, float* dw, void* ws,
                                           hipStream_t st);

}  // namespace mq
