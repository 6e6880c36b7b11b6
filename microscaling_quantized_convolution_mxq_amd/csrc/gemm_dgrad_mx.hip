// gemm_dgrad_mx.hip -- backward-data GEMM whose epilogue writes dX as MX codes
// and scales (the gradient the previous layer consumes) instead of fp32: the
// entry launcher and the path that reads 8-bit weight codes in place.
#include "dgrad_mx.h"

namespace mq {

hipError_t launch_backward_data_mx(const Conv& cv, MxView dy, MxView w, MxOutView dxq, void* ws, size_t,
                                   hipStream_t st) {
  // validate the block mode before anything is enqueued
  if (dxq.bp != 1 && cv.n % 32 != 0 && 32 % cv.n != 0) return hipErrorInvalidValue;
  DgradNatProb q;
  DgradProb p;
  bool natural = false;
  const hipError_t e = prepare_backward_data(cv, dy, w, nullptr, ws, st, &q, &p, &natural);
  if (e != hipSuccess) return e;
  if (natural) return launch_dgrad_mx(cv, dy.fmt, w.fmt, q, dxq, st);
  return launch_dgrad_mx_relaid(cv, dy.fmt, w.fmt, p, dxq, st);
}

}  // namespace mq
