// nvfp.h -- launcher of the two-level (NVFP-style) quantization (nvfp.hip),
// for the C ABI layer. Host-side only; arguments are already validated.
#pragma once
#include "mqconv_internal.h"

namespace mq {

// partial maxima of the tensor-maximum pass (fp32 bit patterns)
constexpr int kNvfpParts = 1024;
inline size_t nvfp_workspace_bytes() { return kNvfpParts * sizeof(uint32_t); }
// [A][P][B] x C view as launch_quantize; block scales [A][B][ceil(P/8)][ceil(C/8)]
hipError_t launch_nvfp_quantize(const float* src, uint8_t* codes, uint8_t* bscales, float* tscale, int fmt, int A,
                                int P, int B, int C, void* ws, hipStream_t st);

}  // namespace mq
