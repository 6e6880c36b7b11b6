// gemm_wgrad_sub.hip -- backward-weight GEMM reading 8-bit gradient codes and
// 6/4-bit activation codes where quantization left them (WgradNatSubProb).
#include "gemm_kernel.h"

namespace mq {

hipError_t launch_wgrad_nat_sub(int fa, int fb, const WgradNatSubProb& q, int Ma, int Nb, int S, hipStream_t st) {
  return launch_tiled(fa, fb, q, Ma, Nb, S, st);
}

}  // namespace mq
