// dgrad_mx.h -- shared set-up of the backward-data problem whose epilogue
// writes dX as MX codes and scales (one translation unit per weight path, so
// that the two sets of GEMM instantiations compile in parallel).
#pragma once
#include "gemm_kernel.h"

namespace mq {

hipError_t prepare_backward_data(const Conv& cv, MxView dy, MxView w, float* dx, void* ws, hipStream_t st,
                                 DgradNatProb* nat, DgradProb* gen, bool* natural_out);
int dgrad_rows(const Conv& cv);
int dgrad_ksteps(const Conv& cv);
// the GEMM launch of the re-laid weight path (6/4-bit weight codes)
hipError_t launch_dgrad_mx_relaid(const Conv& cv, int fa, int fb, const DgradProb& p, MxOutView yq, hipStream_t st);

template <class Q>
static hipError_t launch_dgrad_mx(const Conv& cv, int fa, int fb, const Q& q, MxOutView yq, hipStream_t st) {
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
  return launch_tiled(fa, fb, o, dgrad_rows(cv), cv.cin, cv.sh * cv.sw, st, dgrad_ksteps(cv));
}

}  // namespace mq
