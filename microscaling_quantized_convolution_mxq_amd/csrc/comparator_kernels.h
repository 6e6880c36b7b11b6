// comparator_kernels.h -- element-wise kernels of the two comparison paths
// (the naive quantize-twice path and the square-block comparator), both of
// which expand the activation with the classic im2col of §II-C1 (rows
// m = (ho, wo, n), columns k = (ci, kh, kw), channel-major as in §II-C2) and
// fold the input gradient back with col2im.
#pragma once
#include "mx_common.h"
#include "mqconv_internal.h"

namespace mq {

// X'[m][k], k = (ci, kh, kw): one thread per element, in row order.
static __global__ __launch_bounds__(256) void classic_im2col_kernel(const float* __restrict__ x, float* __restrict__ out,
                                                                    int N, int C, int H, int W, int KH, int KW, int sh,
                                                                    int sw, int ph, int pw, int Wo, long long M, int K) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * K) return;
  const long long m = idx / K;
  const int k = (int)(idx - m * K);
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

// X'^T with its rows in tap-major order, out[(kh*KW + kw)*C + ci][m] =
// X'[m][(ci, kh, kw)] (the same rows as the channel-major X'^T, permuted):
// one 32 x 32 tile of (m, ci) of one tap per workgroup, through LDS, so the
// reads run along ci (contiguous in X) and the writes along m.
// Grid: (ceil(M/32), ceil(C/32), KH*KW).
static __global__ __launch_bounds__(256) void classic_im2col_t_kernel(const float* __restrict__ x,
                                                                      float* __restrict__ out, int N, int C, int H,
                                                                      int W, int KW, int sh, int sw, int ph, int pw,
                                                                      int Wo, long long M) {
  __shared__ float t[32][33];
  const long long m0 = (long long)blockIdx.x * 32;
  const int c0 = blockIdx.y * 32;
  const int tap = blockIdx.z, kh = tap / KW, kw = tap - kh * KW;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const long long m = m0 + i;
    const int ci = c0 + tx;
    float v = 0.0f;
    if (m < M && ci < C) {
      const long long o = m / N;
      const int n = (int)(m - o * N);
      const int ho = (int)(o / Wo), wo = (int)(o - (long long)ho * Wo);
      const int hi = ho * sh + kh - ph, wi = wo * sw + kw - pw;
      if (hi >= 0 && hi < H && wi >= 0 && wi < W) v = x[(((long long)hi * W + wi) * N + n) * C + ci];
    }
    t[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int ci = c0 + i;
    const long long m = m0 + tx;
    if (ci < C && m < M) out[((long long)tap * C + ci) * M + m] = t[tx][i];
  }
}

// W_f[co][k], k = (ci, kh, kw); w is [Cout][Kh][Kw][Cin].
static __global__ __launch_bounds__(256) void flatten_w_kernel(const float* __restrict__ w, float* __restrict__ out,
                                                               int Cout, int Cin, int KH, int KW) {
  const long long K = (long long)Cin * KH * KW;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= K * Cout) return;
  const int co = (int)(idx / K);
  const int k = (int)(idx - (long long)co * K);
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
// sums the G_X' entries copied from it, taps in (kh, kw) order. gcol is
// [M][K] with columns k = (ci, kh, kw) (TAPS = false) or (kh, kw, ci) (TAPS =
// true: neighbouring threads, neighbouring channels, read neighbouring
// words).
template <bool TAPS>
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
      s += gcol[m * K + (TAPS ? (kh * KW + kw) * C + ci : (ci * KH + kh) * KW + kw)];
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

// dw[i] = sum_z part[z][i] over the split-K slices, in slice order (the
// slices already hold dW's own [Cout][Kh][Kw][Cin] order).
static __global__ __launch_bounds__(256) void sum_slices_kernel(const float* __restrict__ part, float* __restrict__ dw,
                                                                long long total, int splits) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  float s = 0.0f;
  for (int z = 0; z < splits; z++) s += part[(long long)z * total + idx];
  dw[idx] = s;
}

}  // namespace mq
