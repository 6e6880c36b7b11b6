// gemm_dgrad.hip -- backward-data GEMM launcher (stride parity classes).
#include "gemm_kernel.h"

namespace mq {

// Fills the problem (in *nat when the weight codes are read in place, else
// in *gen, *natural telling which) and launches the re-laying of 6/4-bit
// weight codes into the workspace; the caller launches the GEMM.
hipError_t prepare_backward_data(const Conv& cv, MxView dy, MxView w, float* dx, void* ws, hipStream_t st,
                                 DgradNatProb* nat, DgradProb* gen, bool* natural_out) {
  uint8_t* wt = static_cast<uint8_t*>(ws);
  DgradProb p;
  // rows of A are (pixel, n); rows of B are Cin, 32 to a block
  p.khalf = cv.cout <= 16;
  p.ga = scale_group_rows(dy.bp, cv.n);
  p.gb = 32;
  // 8-bit weight codes are read where quantization left them (K-major
  // staging); other formats are first re-laid with runs along Cout
  const bool natural = w.fmt <= 1;
  const bool half = !natural && half_k_blocks(p.ga, p.gb, p.khalf, dy.fmt, w.fmt);
  p.dyc = dy.codes; p.dys = dy.scales; p.wtc = wt; p.ws = w.scales; p.dx = dx;
  p.N = cv.n; p.H = cv.h; p.W = cv.w; p.Cin = cv.cin; p.Cout = cv.cout; p.KH = cv.kh; p.KW = cv.kw;
  p.sh = cv.sh; p.sw = cv.sw; p.ph = cv.ph; p.pw = cv.pw; p.Ho = cv.ho(); p.Wo = cv.wo();
  p.ncob = ceil_div(cv.cout, 32);
  p.npair = (p.ncob + 1) / 2;
  p.dyRB = (int)run_bytes(dy.fmt); p.dyrb = p.ncob * p.dyRB; p.dybp = dy.bp; p.dynPB = ceil_div(cv.n, dy.bp);
  p.wRB = half ? 16 : (int)run_bytes(w.fmt); p.ncbi = ceil_div(cv.cin, 32);
  const long long T = (long long)cv.kh * cv.kw;
  p.dyc_bytes = (long long)p.Ho * p.Wo * cv.n * p.dyrb; p.dys_bytes = (long long)p.Ho * p.Wo * p.dynPB * p.ncob;
  p.wtc_bytes = T * cv.cin * p.ncob * p.wRB; p.ws_bytes = T * p.ncob * p.ncbi;
  // the taps step backwards from a row's first output pixel by up to dmax pixels
  const long long dmax = (long long)(ceil_div(cv.kh, cv.sh) - 1) * p.Wo + (ceil_div(cv.kw, cv.sw) - 1);
  p.dycb = (int)(dmax * cv.n * p.dyrb); p.dysb = (int)(dmax * p.dynPB * p.ncob);
  if (!offsets_fit(p.dyc_bytes, p.dycb) || !offsets_fit(p.dys_bytes, p.dysb)) return hipErrorInvalidValue;
  p.dybps = dy.bp == 32 ? 5 : 0;
  p.dN = make_fastdiv(cv.n); p.dnp = make_fastdiv(p.npair);
  for (int c = 0; c < 8; c++) {  // parity class with column offset c (c < sw): width, tap columns
    const int wc = c < cv.sw && cv.w > c ? (cv.w - c + cv.sw - 1) / cv.sw : 1;
    p.dWc[c] = make_fastdiv((unsigned)(wc > 0 ? wc : 1));
    const int kw0 = c < cv.sw ? (c + cv.pw) % cv.sw : 0;
    const int nkw = kw0 < cv.kw ? (cv.kw - kw0 + cv.sw - 1) / cv.sw : 0;
    p.dNkw[c] = make_fastdiv((unsigned)(nkw > 0 ? nkw : 1));
  }
  // every check has passed: only now is anything enqueued
  if (!natural) {
    const hipError_t e = launch_transpose_codes(w.codes, wt, w.fmt, half, 1, cv.cout, cv.kh * cv.kw, cv.cin, st);
    if (e != hipSuccess) return e;
  }
  *natural_out = natural;
  if (natural) {
    static_cast<DgradProb&>(*nat) = p;
    nat->T = (int)T; nat->wrb = (int)row_bytes(w.fmt, cv.cin);
    nat->wtc = w.codes; nat->wtc_bytes = (long long)cv.cout * T * nat->wrb;
  } else {
    *gen = p;
  }
  return hipSuccess;
}

// rows of the problem: every parity class spans at most maxHc x maxWc pixels
int dgrad_rows(const Conv& cv) { return ceil_div(cv.h, cv.sh) * ceil_div(cv.w, cv.sw) * cv.n; }
// K-steps of a tile on average over the parity classes: taps per class times
// the pairs of Cout blocks
int dgrad_ksteps(const Conv& cv) {
  return (cv.kh * cv.kw + cv.sh * cv.sw - 1) / (cv.sh * cv.sw) * ((ceil_div(cv.cout, 32) + 1) / 2);
}

hipError_t launch_backward_data(const Conv& cv, MxView dy, MxView w, float* dx, void* ws, size_t,
                                hipStream_t st) {
  DgradNatProb q;
  DgradProb p;
  bool natural = false;
  const hipError_t e = prepare_backward_data(cv, dy, w, dx, ws, st, &q, &p, &natural);
  if (e != hipSuccess) return e;
  if (natural) return launch_tiled(dy.fmt, w.fmt, q, dgrad_rows(cv), cv.cin, cv.sh * cv.sw, st, dgrad_ksteps(cv));
  return launch_tiled(dy.fmt, w.fmt, p, dgrad_rows(cv), cv.cin, cv.sh * cv.sw, st, dgrad_ksteps(cv));
}


}  // namespace mq
