// comparator_kernels.h -- element-wise kernels of the two comparison paths
// (the naive quantize-twice path and the square-block comparator), both of
// which expand the activation with the classic im2col of §II-C1 (rows
// m = (ho, wo, n), columns k = (ci, kh, kw), channel-major as in §II-C2) and
// fold the input gradient back with col2im.
#pragma once
#include "mx_common.h"
#include "mqconv_internal.h"

namespace mq {

// X'[m][k] (transposed = false) or X'^T[k][m] (transposed = true).
template <bool TR>
static __global__ __launch_bounds__(256) void classic_im2col_kernel(const float* __restrict__ x, float* __restrict__ out,
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
static __global__ __launch_bounds__(256) void flatten_w_kernel(const float* __restrict__ w, float* __restrict__ out, int Cout,
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
static __global__ __launch_bounds__(256) void transpose_f32_kernel(const float* __restrict__ in, float* __restrict__ out,
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
static __global__ __launch_bounds__(256) void col2im_kernel(const float* __restrict__ gcol, float* __restrict__ dx, int N,
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
static __global__ __launch_bounds__(256) void wgrad_reduce_permute_kernel(const float* __restrict__ part, float* __restrict__ dw,
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

}  // namespace mq
