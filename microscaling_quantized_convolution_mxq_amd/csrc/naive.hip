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
#include "mx_common.h"
#include "mqconv_internal.h"

namespace mq {

// X'[m][k] (transposed = false) or X'^T[k][m] (transposed = true).
template <bool TR>
__global__ __launch_bounds__(256) void classic_im2col_kernel(const float* __restrict__ x, float* __restrict__ out,
                                                            int N, int C, int H, int W, int KH, int KW, int sh,
                                                            int sw, int ph, int pw, int Wo, long long M, int K) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * K) return;
  long long m;
  int k;
  if (TR) { k = (int)(idx / M); m = idx - (long long)k * M; }
  else { m = idx / K; k = (int)(idx - m * K); }
  const int n = (int)(m % N);
  const int o = (int)(m / N);
  const int ho = o / Wo, wo = o - ho * Wo;
  const int ci = k / (KH * KW);
  const int r = k - ci * KH * KW;
  const int kh = r / KW, kw = r - kh * KW;
  const int hi = ho * sh + kh - ph, wi = wo * sw + kw - pw;
  float v = 0.0f;
  if (hi >= 0 && hi < H && wi >= 0 && wi < W) v = x[(((long long)hi * W + wi) * N + n) * C + ci];
  out[idx] = v;
}

// W_f[co][k] (TR = false) or W_f^T[k][co] (TR = true), k = (ci, kh, kw); w is [Cout][Kh][Kw][Cin].
template <bool TR>
__global__ __launch_bounds__(256) void flatten_w_kernel(const float* __restrict__ w, float* __restrict__ out, int Cout,
                                                       int Cin, int KH, int KW) {
  const long long K = (long long)Cin * KH * KW;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= K * Cout) return;
  int co, k;
  if (TR) { k = (int)(idx / Cout); co = (int)(idx - (long long)k * Cout); }
  else { co = (int)(idx / K); k = (int)(idx - (long long)co * K); }
  const int ci = k / (KH * KW);
  const int r = k - ci * KH * KW;
  const int kh = r / KW, kw = r - kh * KW;
  out[idx] = w[(((long long)co * KH + kh) * KW + kw) * Cin + ci];
}

// out[c][r] = in[r][c] for an R x C fp32 matrix, through a 32 x 33 LDS tile.
__global__ __launch_bounds__(256) void transpose_f32_kernel(const float* __restrict__ in, float* __restrict__ out,
                                                           long long R, int C) {
  __shared__ float t[32][33];
  const long long r0 = (long long)blockIdx.x * 32;
  const int c0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    long long r = r0 + i;
    int c = c0 + tx;
    t[i][tx] = (r < R && c < C) ? in[r * C + c] : 0.0f;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    int c = c0 + i;
    long long r = r0 + tx;
    if (c < C && r < R) out[(long long)c * R + r] = t[tx][i];
  }
}

// col2im (the adjoint of classic im2col) in gather form: every G_X element
// sums the G_X' entries copied from it. gcol is [M][K] with K = (ci, kh, kw).
__global__ __launch_bounds__(256) void col2im_kernel(const float* __restrict__ gcol, float* __restrict__ dx, int N,
                                                     int C, int H, int W, int KH, int KW, int sh, int sw, int ph,
                                                     int pw, int Ho, int Wo) {
  const long long total = (long long)H * W * N * C;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int ci = (int)(idx % C);
  const long long hwn = idx / C;
  const int n = (int)(hwn % N);
  const int hw = (int)(hwn / N);
  const int h = hw / W, w = hw - h * W;
  const int K = C * KH * KW;
  float s = 0.0f;
  for (int kh = 0; kh < KH; kh++) {
    const int th = h + ph - kh;
    if (th < 0 || th % sh) continue;
    const int ho = th / sh;
    if (ho >= Ho) continue;
    for (int kw = 0; kw < KW; kw++) {
      const int tw = w + pw - kw;
      if (tw < 0 || tw % sw) continue;
      const int wo = tw / sw;
      if (wo >= Wo) continue;
      const long long m = ((long long)ho * Wo + wo) * N + n;
      s += gcol[m * K + (ci * KH + kh) * KW + kw];
    }
  }
  dx[idx] = s;
}

// dW[co][kh][kw][ci] = sum_z part[z][co][k], k = (ci, kh, kw), fixed order.
__global__ __launch_bounds__(256) void wgrad_reduce_permute_kernel(const float* __restrict__ part, float* __restrict__ dw,
                                                                  int Cout, int Cin, int KH, int KW, int splits) {
  const long long K = (long long)Cin * KH * KW;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= K * Cout) return;
  const int ci = (int)(idx % Cin);
  const long long r = idx / Cin;
  const int kw = (int)(r % KW);
  const long long r2 = r / KW;
  const int kh = (int)(r2 % KH);
  const int co = (int)(r2 / KH);
  const long long k = ((long long)ci * KH + kh) * KW + kw;
  float s = 0.0f;
  for (int z = 0; z < splits; z++) s += part[((long long)z * Cout + co) * K + k];
  dw[idx] = s;
}

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
  hipLaunchKernelGGL(classic_im2col_kernel<false>, dim3(nblk(s.M * s.K)), dim3(256), 0, st, x, xcol, cv.n, cv.cin,
                     cv.h, cv.w, cv.kh, cv.kw, cv.sh, cv.sw, cv.ph, cv.pw, cv.wo(), s.M, (int)s.K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = quantize_rows(xcol, xc, xs, fx, s.M, (int)s.K, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(flatten_w_kernel<false>, dim3(nblk(cv.cout * s.K)), dim3(256), 0, st, w, wf, cv.cout, cv.cin,
                     cv.kh, cv.kw);
  if ((e = hipGetLastError()) != hipSuccess) return e;
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
  hipLaunchKernelGGL(flatten_w_kernel<true>, dim3(nblk(cv.cout * s.K)), dim3(256), 0, st, w, wft, cv.cout, cv.cin,
                     cv.kh, cv.kw);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = quantize_rows(wft, wc, wsc, fw, s.K, cv.cout, st)) != hipSuccess) return e;
  if ((e = launch_plain_gemm(fdy, fw, gc, gs, wc, wsc, (int)s.M, (int)s.K, ceil_div(cv.cout, 32), gcol, 1, st)) !=
      hipSuccess)
    return e;
  hipLaunchKernelGGL(col2im_kernel, dim3(nblk((long long)cv.h * cv.w * cv.n * cv.cin)), dim3(256), 0, st, gcol, dx,
                     cv.n, cv.cin, cv.h, cv.w, cv.kh, cv.kw, cv.sh, cv.sw, cv.ph, cv.pw, cv.ho(), cv.wo());
  return hipGetLastError();
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
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = quantize_rows(gt, gc, gs, fdy, cv.cout, (int)s.M, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(classic_im2col_kernel<true>, dim3(nblk(s.M * s.K)), dim3(256), 0, st, x, xt, cv.n, cv.cin, cv.h,
                     cv.w, cv.kh, cv.kw, cv.sh, cv.sw, cv.ph, cv.pw, cv.wo(), s.M, (int)s.K);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = quantize_rows(xt, xc, xs, fx, s.K, (int)s.M, st)) != hipSuccess) return e;
  if ((e = launch_plain_gemm(fdy, fx, gc, gs, xc, xs, cv.cout, (int)s.K, nmb, part, S, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(wgrad_reduce_permute_kernel, dim3(nblk(cv.cout * s.K)), dim3(256), 0, st, part, dw, cv.cout,
                     cv.cin, cv.kh, cv.kw, S);
  return hipGetLastError();
}

}  // namespace mq
