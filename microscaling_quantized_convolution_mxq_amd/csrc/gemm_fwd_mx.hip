// gemm_fwd_mx.hip -- forward GEMM launcher whose epilogue writes Y as MX codes
// and scales (the activation of the next layer) instead of fp32.
#include "gemm_kernel.h"

namespace mq {

hipError_t launch_forward(const Conv& cv, MxView x, MxView w, float* y, void* ws, size_t ws_bytes, hipStream_t st,
                          FwdProb* out);

hipError_t launch_forward_mx(const Conv& cv, MxView x, MxView w, MxOutView yq, hipStream_t st) {
  FwdMxProb q;
  // the forward problem itself, set up exactly as for fp32 output
  const hipError_t e = launch_forward(cv, x, w, nullptr, nullptr, 0, st, &q);
  if (e != hipSuccess) return e;
  q.y = nullptr;
  q.yc = yq.codes; q.ys = yq.scales; q.yfmt = yq.fmt;
  q.ynCB = ceil_div(cv.cout, 32);
  q.yrb = (int)row_bytes(yq.fmt, cv.cout);
  q.ynPB = ceil_div(cv.n, yq.bp);
  if (yq.bp == 1) q.ymode = 0;
  else if (cv.n % 32 == 0) q.ymode = 1;
  else if (32 % cv.n == 0) q.ymode = 2;
  else return hipErrorInvalidValue;  // blocks would straddle tile strips (rejected by the caller)
  return launch_tiled(x.fmt, w.fmt, q, q.M, cv.cout, 1, st);
}

}  // namespace mq
