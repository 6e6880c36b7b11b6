// gemm_fwd.hip -- forward GEMM launcher (implicit CBF im2col).
#include "gemm_kernel.h"

namespace mq {

// out != nullptr: only fill *out with the problem (no launch)
hipError_t launch_forward(const Conv& cv, MxView x, MxView w, float* y, void*, size_t, hipStream_t st,
                          FwdProb* out) {
  FwdProb p;
  p.xc = x.codes; p.xs = x.scales; p.wc = w.codes; p.ws = w.scales; p.y = y;
  p.N = cv.n; p.H = cv.h; p.W = cv.w; p.Cin = cv.cin; p.Cout = cv.cout; p.KW = cv.kw;
  p.T = cv.kh * cv.kw; p.sh = cv.sh; p.sw = cv.sw; p.ph = cv.ph; p.pw = cv.pw; p.Wo = cv.wo();
  p.M = cv.ho() * cv.wo() * cv.n;
  p.ncb = ceil_div(cv.cin, 32);
  p.npair = (p.ncb + 1) / 2;
  p.xRB = (int)run_bytes(x.fmt); p.xrb = p.ncb * p.xRB; p.xbp = x.bp; p.xnPB = ceil_div(cv.n, x.bp);
  p.wRB = (int)run_bytes(w.fmt); p.wrb = p.ncb * p.wRB; p.wbp = w.bp; p.wnCoB = ceil_div(cv.cout, w.bp);
  p.xc_bytes = (long long)cv.h * cv.w * cv.n * p.xrb; p.xs_bytes = (long long)cv.h * cv.w * p.xnPB * p.ncb;
  p.wc_bytes = (long long)cv.cout * p.T * p.wrb; p.ws_bytes = (long long)p.T * p.wnCoB * p.ncb;
  // padding moves the first tap of border rows before the buffer
  const long long lead = (long long)cv.ph * cv.w + cv.pw;
  p.xcb = (int)(lead * cv.n * p.xrb); p.xsb = (int)(lead * p.xnPB * p.ncb);
  if (!offsets_fit(p.xc_bytes, p.xcb) || !offsets_fit(p.xs_bytes, p.xsb)) return hipErrorInvalidValue;
  // rows of A are (pixel, n): a block is 32 (or all N < 32) of them; rows of B are Cout
  p.xbps = x.bp == 32 ? 5 : 0; p.wbps = w.bp == 32 ? 5 : 0;
  p.dN = make_fastdiv(cv.n); p.dWo = make_fastdiv(p.Wo); p.dKW = make_fastdiv(cv.kw); p.dnp = make_fastdiv(p.npair);
  p.khalf = cv.cin <= 16;
  p.ga = scale_group_rows(x.bp, cv.n);
  p.gb = w.bp == 32 ? 32 : 0;
  if (out) {
    *out = p;
    return hipSuccess;
  }
  return launch_tiled(x.fmt, w.fmt, p, p.M, cv.cout, 1, st);
}

hipError_t launch_forward(const Conv& cv, MxView x, MxView w, float* y, void* ws, size_t ws_bytes, hipStream_t st) {
  return launch_forward(cv, x, w, y, ws, ws_bytes, st, nullptr);
}


}  // namespace mq
