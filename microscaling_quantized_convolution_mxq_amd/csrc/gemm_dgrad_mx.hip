// gemm_dgrad_mx.hip -- backward-data GEMM launcher whose epilogue writes dX as
// MX codes and scales (the gradient the previous layer consumes) instead of
// fp32.
#include "gemm_kernel.h"

namespace mq {

hipError_t prepare_backward_data(const Conv& cv, MxView dy, MxView w, float* dx, void* ws, hipStream_t st,
                                 DgradNatProb* nat, DgradProb* gen, bool* natural_out);
int dgrad_rows(const Conv& cv);

template <class Q>
static hipError_t launch_mx(const Conv& cv, int fa, int fb, const Q& q, MxOutView yq, hipStream_t st) {
  MxOutProb<Q> o;
  static_cast<Q&>(o) = q;
  o.dx = nullptr;
  o.yc = yq.codes; o.ys = yq.scales; o.yfmt = yq.fmt;
  o.ynCB = ceil_div(cv.cin, 32);
  o.yrb = (int)row_bytes(yq.fmt, cv.cin);
  o.ynPB = ceil_div(cv.n, yq.bp);
  if (yq.bp == 1) o.ymode = 0;
  else if (cv.n % 32 == 0) o.ymode = 1;
  else if (32 % cv.n == 0) o.ymode = 2;
  else return hipErrorInvalidValue;  // blocks would straddle tile strips (rejected by the caller)
  return launch_tiled(fa, fb, o, dgrad_rows(cv), cv.cin, cv.sh * cv.sw, st);
}

hipError_t launch_backward_data_mx(const Conv& cv, MxView dy, MxView w, MxOutView dxq, void* ws, size_t,
                                   hipStream_t st) {
  // validate the block mode before anything is enqueued
  if (dxq.bp != 1 && cv.n % 32 != 0 && 32 % cv.n != 0) return hipErrorInvalidValue;
  DgradNatProb q;
  DgradProb p;
  bool natural = false;
  const hipError_t e = prepare_backward_data(cv, dy, w, nullptr, ws, st, &q, &p, &natural);
  if (e != hipSuccess) return e;
  if (natural) return launch_mx(cv, dy.fmt, w.fmt, q, dxq, st);
  return launch_mx(cv, dy.fmt, w.fmt, p, dxq, st);
}

}  // namespace mq
