// naive.hip -- the comparison path that MicroQonv improves on (§II-C classic
// im2col, §III-C quantizing the im2col-expanded tensor along each GEMM
// direction; Table I "Dacapo" column). Kept only to measure bytes moved.
//
// Every tensor stays fp32 in memory. The activation is expanded with the
// classic im2col (rows m = (ho, wo, n), columns k = (ci, kh, kw), the
// channel-major patch flattening of §II-C1/§II-C2) before it is quantized,
// and X', W and G_Y are each quantized twice, in 1-D blocks of 32 along the
// contraction of each GEMM that uses them:
//   forward:          Y    = Q_k(X')  . Q_k(W_f)^T
//   backward-data:    G_X' = Q_co(G_Y) . Q_co(W_f), then col2im -> G_X
//   backward-weight:  G_W  = Q_m(G_Y)^T . Q_m(X')
// The operands that are quantized along co or m (W_f^T for backward-data,
// X'^T for backward-weight) keep their rows in tap-major order k' = (kh, kw,
// ci): a block runs along one row, so the row order leaves every block, and
// every product, as in the channel-major order, but the products' columns
// then come out in (kh, kw, ci) order. col2im then reads whole channel runs,
// W_f^T is a plain transpose of W, and the backward-weight GEMM writes dW in
// its own [Cout][Kh][Kw][Cin] layout.
#include "comparator_kernels.h"

namespace mq {

static inline size_t al(size_t x) { return (x + 255) & ~(size_t)255; }
static inline unsigned nblk(long long n) { return (unsigned)((n + 255) / 256); }

// Quantizes the rows of an R x L fp32 matrix in 1-D blocks of 32 along L.
static hipError_t quantize_rows(const float* src, uint8_t* codes, uint8_t* scales, int fmt, long long R, int L,
                                hipStream_t st) {
  return launch_quantize(src, codes, scales, fmt, 1, 1, (int)R, 1, L, st);
}

struct NaiveSizes {
  long long M, K;
};
static NaiveSizes nsz(const Conv& cv) {
  NaiveSizes s;
  s.M = (long long)cv.ho() * cv.wo() * cv.n;
  s.K = (long long)cv.cin * cv.kh * cv.kw;
  return s;
}

size_t naive_workspace_bytes(const Conv& cv, int op, int fa, int fb) {
  const NaiveSizes s = nsz(cv);
  if (op == 0) {  // fa = X format, fb = W format
    return al(s.M * s.K * 4) + al(s.M * row_bytes(fa, s.K)) + al(s.M * ceil_div(s.K, 32)) +
           al(cv.cout * s.K * 4) + al(cv.cout * row_bytes(fb, s.K)) + al(cv.cout * ceil_div(s.K, 32));
  }
  if (op == 1) {  // fa = dY format, fb = W format
    return al(s.M * row_bytes(fa, cv.cout)) + al(s.M * ceil_div(cv.cout, 32)) + al(s.K * cv.cout * 4) +
           al(s.K * row_bytes(fb, cv.cout)) + al(s.K * ceil_div(cv.cout, 32)) + al(s.M * s.K * 4);
  }
  // op 2: fa = dY format, fb = X format
  const int S = plain_gemm_splits(cv.cout, s.K, ceil_div(s.M, 32));
  return al(cv.cout * s.M * 4) + al(cv.cout * row_bytes(fa, s.M)) + al(cv.cout * ceil_div(s.M, 32)) +
         al(s.K * s.M * 4) + al(s.K * row_bytes(fb, s.M)) + al(s.K * ceil_div(s.M, 32)) +
         al((size_t)S * cv.cout * s.K * 4);
}

hipError_t launch_naive_forward(const Conv& cv, const float* x, const float* w, int fx, int fw, float* y, void* ws,
                                hipStream_t st) {
  const NaiveSizes s = nsz(cv);
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* xcol = reinterpret_cast<float*>(p); p += al(s.M * s.K * 4);
  uint8_t* xc = p; p += al(s.M * row_bytes(fx, s.K));
  uint8_t* xs = p; p += al(s.M * ceil_div(s.K, 32));
  float* wf = reinterpret_cast<float*>(p); p += al(cv.cout * s.K * 4);
  uint8_t* wc = p; p += al(cv.cout * row_bytes(fw, s.K));
  uint8_t* wsc = p;
  hipLaunchKernelGGL(classic_im2col_kernel, dim3(nblk(s.M * s.K)), dim3(256), 0, st, x, xcol, cv.n, cv.cin,
                     cv.h, cv.w, cv.kh, cv.kw, cv.sh, cv.sw, cv.ph, cv.pw, cv.wo(), s.M, (int)s.K);
  hipError_t e = launch_check();
  if (e != hipSuccess) return e;
  if ((e = quantize_rows(xcol, xc, xs, fx, s.M, (int)s.K, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(flatten_w_kernel, dim3(nblk(cv.cout * s.K)), dim3(256), 0, st, w, wf, cv.cout, cv.cin, cv.kh,
                     cv.kw);
  if ((e = launch_check()) != hipSuccess) return e;
  if ((e = quantize_rows(wf, wc, wsc, fw, cv.cout, (int)s.K, st)) != hipSuccess) return e;
  return launch_plain_gemm(fx, fw, xc, xs, wc, wsc, (int)s.M, cv.cout, ceil_div(s.K, 32), y, 1, st);
}

hipError_t launch_naive_backward_data(const Conv& cv, const float* dy, const float* w, int fdy, int fw, float* dx,
                                      void* ws, hipStream_t st) {
  const NaiveSizes s = nsz(cv);
  uint8_t* p = static_cast<uint8_t*>(ws);
  uint8_t* gc = p; p += al(s.M * row_bytes(fdy, cv.cout));
  uint8_t* gs = p; p += al(s.M * ceil_div(cv.cout, 32));
  float* wft = reinterpret_cast<float*>(p); p += al(s.K * cv.cout * 4);
  uint8_t* wc = p; p += al(s.K * row_bytes(fw, cv.cout));
  uint8_t* wsc = p; p += al(s.K * ceil_div(cv.cout, 32));
  float* gcol = reinterpret_cast<float*>(p);
  hipError_t e;
  if ((e = quantize_rows(dy, gc, gs, fdy, s.M, cv.cout, st)) != hipSuccess) return e;
  // W_f^T with tap-major rows: W viewed as [Cout][(kh, kw, ci)], transposed
  hipLaunchKernelGGL(transpose_f32_kernel, dim3((unsigned)ceil_div(cv.cout, 32), (unsigned)ceil_div(s.K, 32)),
                     dim3(256), 0, st, w, wft, (long long)cv.cout, (int)s.K);
  if ((e = launch_check()) != hipSuccess) return e;
  if ((e = quantize_rows(wft, wc, wsc, fw, s.K, cv.cout, st)) != hipSuccess) return e;
  if ((e = launch_plain_gemm(fdy, fw, gc, gs, wc, wsc, (int)s.M, (int)s.K, ceil_div(cv.cout, 32), gcol, 1, st)) !=
      hipSuccess)
    return e;
  hipLaunchKernelGGL(col2im_kernel<true>, dim3(nblk((long long)cv.h * cv.w * cv.n * cv.cin)), dim3(256), 0, st, gcol, dx,
                     cv.n, cv.cin, cv.h, cv.w, cv.kh, cv.kw, cv.sh, cv.sw, cv.ph, cv.pw, cv.ho(), cv.wo());
  return launch_check();
}

hipError_t launch_naive_backward_weight(const Conv& cv, const float* dy, const float* x, int fdy, int fx, float* dw,
                                        void* ws, hipStream_t st) {
  const NaiveSizes s = nsz(cv);
  const int nmb = ceil_div(s.M, 32);
  const int S = plain_gemm_splits(cv.cout, s.K, nmb);
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* gt = reinterpret_cast<float*>(p); p += al(cv.cout * s.M * 4);
  uint8_t* gc = p; p += al(cv.cout * row_bytes(fdy, s.M));
  uint8_t* gs = p; p += al((size_t)cv.cout * nmb);
  float* xt = reinterpret_cast<float*>(p); p += al(s.K * s.M * 4);
  uint8_t* xc = p; p += al(s.K * row_bytes(fx, s.M));
  uint8_t* xs = p; p += al((size_t)s.K * nmb);
  float* part = reinterpret_cast<float*>(p);
  hipLaunchKernelGGL(transpose_f32_kernel, dim3((unsigned)ceil_div(s.M, 32), (unsigned)ceil_div(cv.cout, 32)), dim3(256),
                     0, st, dy, gt, s.M, cv.cout);
  hipError_t e = launch_check();
  if (e != hipSuccess) return e;
  if ((e = quantize_rows(gt, gc, gs, fdy, cv.cout, (int)s.M, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(classic_im2col_t_kernel,
                     dim3((unsigned)ceil_div(s.M, 32), (unsigned)ceil_div(cv.cin, 32), (unsigned)(cv.kh * cv.kw)),
                     dim3(256), 0, st, x, xt, cv.n, cv.cin, cv.h, cv.w, cv.kw, cv.sh, cv.sw, cv.ph, cv.pw, cv.wo(), s.M);
  if ((e = launch_check()) != hipSuccess) return e;
  if ((e = quantize_rows(xt, xc, xs, fx, s.K, (int)s.M, st)) != hipSuccess) return e;
  // the GEMM's columns are tap-major: its output is dW's own layout
  if (S == 1) return launch_plain_gemm(fdy, fx, gc, gs, xc, xs, cv.cout, (int)s.K, nmb, dw, 1, st);
  if ((e = launch_plain_gemm(fdy, fx, gc, gs, xc, xs, cv.cout, (int)s.K, nmb, part, S, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(sum_slices_kernel, dim3(nblk(cv.cout * s.K)), dim3(256), 0, st, part, dw, cv.cout * s.K, S);
  return launch_check();
}

}  // namespace mq
