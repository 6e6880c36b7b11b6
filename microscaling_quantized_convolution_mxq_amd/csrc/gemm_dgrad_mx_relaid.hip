// gemm_dgrad_mx_relaid.hip -- backward-data GEMM with MX-quantized dX for
// 6/4-bit weight codes, which are first re-laid with runs along Cout.
#include "dgrad_mx.h"

namespace mq {

hipError_t launch_dgrad_mx_relaid(const Conv& cv, int fa, int fb, const DgradProb& p, MxOutView yq, hipStream_t st) {
  return launch_dgrad_mx(cv, fa, fb, p, yq, st);
}

}  // namespace mq
