// layout.hip -- data movement on packed MX tensors; no code is requantized.
//
// cbf_im2col: channel-batch-first im2col of an already-quantized activation
//   (MicroQonv §IV-A, Fig. 3): X'[ho][wo][n][kh][kw][:] = X[ho*s+kh-p][wo*s+kw-p][n][:]
//   Every output row is a verbatim copy of one input row (all channel runs of
//   one sample at one pixel) or zeros outside the image, and each block of X'
//   takes the scale byte of its source block (0 outside the image).
//
// transpose_codes: re-lays packed codes so that runs of 32 codes go along the
//   partner dimension (N for activations and gradients, Cout for weights)
//   instead of along the channel. The square blocks (§IV-B) make the scale of
//   such a run the scale of the block it lies in, so only codes move.
#include "mx_common.h"
#include "mqconv_internal.h"

namespace mq {

// ----------------------------------------------------------------------------
// CBF im2col. Codes: one thread per CH-byte chunk of output (CH = 16 when rows
// are 16-byte multiples, else 8). Scales: one thread per output scale byte,
// in the trailing blocks of the same grid.
// ----------------------------------------------------------------------------
template <int CH>
__global__ __launch_bounds__(256) void cbf_im2col_kernel(
    const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs, uint8_t* __restrict__ oc,
    uint8_t* __restrict__ os, int N, int H, int W, int KH, int KW, int sh, int sw, int ph, int pw,
    int Wo, int cpr /*chunks per row*/, long long nchunks, int nsb /*scale bytes per pixel*/,
    long long nscales, long long code_blocks) {
  if ((long long)blockIdx.x < code_blocks) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= nchunks) return;
    const int T = KH * KW;
    const int ch = (int)(idx % cpr);
    const long long row = idx / cpr;  // ((o*N + n)*T + t)
    const int t = (int)(row % T);
    const long long on = row / T;
    const int n = (int)(on % N);
    const int o = (int)(on / N);
    const int ho = o / Wo, wo = o - ho * Wo;
    const int kh = t / KW, kw = t - kh * KW;
    const int hi = ho * sh + kh - ph, wi = wo * sw + kw - pw;
    typedef typename std::conditional<CH == 16, uint4, uint2>::type V;
    V v = {};
    if (hi >= 0 && hi < H && wi >= 0 && wi < W)
      v = reinterpret_cast<const V*>(xc)[((long long)(hi * W + wi) * N + n) * cpr + ch];
    reinterpret_cast<V*>(oc)[idx] = v;
  } else {
    const long long idx = ((long long)blockIdx.x - code_blocks) * 256 + threadIdx.x;
    if (idx >= nscales) return;
    const int T = KH * KW;
    const int k = (int)(idx % nsb);
    const long long ot = idx / nsb;  // o*T + t
    const int t = (int)(ot % T);
    const int o = (int)(ot / T);
    const int ho = o / Wo, wo = o - ho * Wo;
    const int kh = t / KW, kw = t - kh * KW;
    const int hi = ho * sh + kh - ph, wi = wo * sw + kw - pw;
    uint8_t s = 0;
    if (hi >= 0 && hi < H && wi >= 0 && wi < W) s = xs[(long long)(hi * W + wi) * nsb + k];
    os[idx] = s;
  }
}

hipError_t launch_cbf_im2col(const Conv& cv, MxView x, uint8_t* col_codes, uint8_t* col_scales,
                             hipStream_t st) {
  const long long rb = row_bytes(x.fmt, cv.cin);
  const int CH = (rb % 16 == 0) ? 16 : 8;
  const int cpr = (int)(rb / CH);
  const long long Ho = cv.ho(), Wo = cv.wo(), T = (long long)cv.kh * cv.kw;
  const long long nchunks = Ho * Wo * cv.n * T * cpr;
  const int nsb = ceil_div(cv.n, x.bp) * ceil_div(cv.cin, 32);
  const long long nscales = Ho * Wo * T * nsb;
  const long long cblocks = (nchunks + 255) / 256, sblocks = (nscales + 255) / 256;
  if (CH == 16)
    hipLaunchKernelGGL(cbf_im2col_kernel<16>, dim3((unsigned)(cblocks + sblocks)), dim3(256), 0, st,
                       x.codes, x.scales, col_codes, col_scales, cv.n, cv.h, cv.w, cv.kh, cv.kw,
                       cv.sh, cv.sw, cv.ph, cv.pw, (int)Wo, cpr, nchunks, nsb, nscales, cblocks);
  else
    hipLaunchKernelGGL(cbf_im2col_kernel<8>, dim3((unsigned)(cblocks + sblocks)), dim3(256), 0, st,
                       x.codes, x.scales, col_codes, col_scales, cv.n, cv.h, cv.w, cv.kh, cv.kw,
                       cv.sh, cv.sw, cv.ph, cv.pw, (int)Wo, cpr, nchunks, nsb, nscales, cblocks);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Code transpose. One workgroup per (a*B + b, 32-row partner block). For each
// chunk of 64 channels: 32 rows x 64 codes are unpacked to bytes in LDS, then
// written back as 64 runs of 32 codes along the partner dimension.
// ----------------------------------------------------------------------------
template <int F>
__device__ __forceinline__ void unpack8(const uint8_t* p, uint8_t* out) {
  constexpr int bits = Fmt<F>::bits;
  if constexpr (bits == 8) {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    for (int i = 0; i < 4; i++) { out[i] = (v.x >> (8 * i)) & 0xff; out[4 + i] = (v.y >> (8 * i)) & 0xff; }
  } else if constexpr (bits == 6) {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);  // 6 bytes, 2-byte aligned
    unsigned long long v = (unsigned long long)q[0] | ((unsigned long long)q[1] << 16) | ((unsigned long long)q[2] << 32);
    for (int i = 0; i < 8; i++) out[i] = (v >> (6 * i)) & 0x3f;
  } else {
    uint32_t v = *reinterpret_cast<const uint32_t*>(p);
    for (int i = 0; i < 8; i++) out[i] = (v >> (4 * i)) & 0xf;
  }
}

template <int F>
__device__ __forceinline__ void pack8_store(uint8_t* dst, const uint8_t* c) {
  constexpr int bits = Fmt<F>::bits;
  if constexpr (bits == 8) {
    uint2 v;
    v.x = c[0] | (c[1] << 8) | (c[2] << 16) | ((uint32_t)c[3] << 24);
    v.y = c[4] | (c[5] << 8) | (c[6] << 16) | ((uint32_t)c[7] << 24);
    *reinterpret_cast<uint2*>(dst) = v;
  } else if constexpr (bits == 6) {
    unsigned long long v = 0;
    for (int i = 0; i < 8; i++) v |= (unsigned long long)c[i] << (6 * i);
    uint16_t* q = reinterpret_cast<uint16_t*>(dst);
    q[0] = v & 0xffff; q[1] = (v >> 16) & 0xffff; q[2] = (v >> 32) & 0xffff;
  } else {
    uint32_t v = 0;
    for (int i = 0; i < 8; i++) v |= (uint32_t)c[i] << (4 * i);
    *reinterpret_cast<uint32_t*>(dst) = v;
  }
}

template <int F>
__global__ __launch_bounds__(256) void transpose_codes_kernel(const uint8_t* __restrict__ in,
                                                             uint8_t* __restrict__ out, int P, int B,
                                                             int C, int nPB) {
  __shared__ uint8_t tile[32][64 + 4];
  constexpr int RB = run_bytes_of(F);
  constexpr int B8 = Fmt<F>::bits;  // bytes per 8 codes
  const int pb = blockIdx.x % nPB;
  const long long ab = blockIdx.x / nPB;
  const long long a = ab / B;
  const int b = (int)(ab % B);
  const int nCB = (C + 31) / 32;
  const long long rb = (long long)nCB * RB;
  const int Cpad = nCB * 32;
  const int t = threadIdx.x;
  for (int c0 = 0; c0 < C; c0 += 64) {
    {  // gather: row r, 8 codes starting at channel c0 + part*8
      const int r = t >> 3, part = t & 7;
      const int p = pb * 32 + r;
      const int cc = c0 + part * 8;
      uint8_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (p < P && cc < Cpad) {
        const long long row = (a * P + p) * B + b;
        unpack8<F>(in + row * rb + (long long)cc * B8 / 8, v);
      }
      for (int i = 0; i < 8; i++) tile[r][part * 8 + i] = v[i];
    }
    __syncthreads();
    {  // scatter: channel c0 + cl, partner rows quarter*8 .. +8
      const int cl = t >> 2, quarter = t & 3;
      const int c = c0 + cl;
      if (c < C) {
        uint8_t v[8];
        for (int i = 0; i < 8; i++) v[i] = tile[quarter * 8 + i][cl];
        pack8_store<F>(out + ((ab * C + c) * nPB + pb) * RB + quarter * B8, v);
      }
    }
    __syncthreads();
  }
}

hipError_t launch_transpose_codes(const uint8_t* in, uint8_t* out, int fmt, int A, int P, int B,
                                  int C, hipStream_t st) {
  const int nPB = ceil_div(P, 32);
  const long long blocks = (long long)A * B * nPB;
  switch (fmt) {
    case 0: case 1:
      hipLaunchKernelGGL(transpose_codes_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, in, out, P, B, C, nPB);
      break;
    case 2: case 3:
      hipLaunchKernelGGL(transpose_codes_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, st, in, out, P, B, C, nPB);
      break;
    default:
      hipLaunchKernelGGL(transpose_codes_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, st, in, out, P, B, C, nPB);
  }
  return hipGetLastError();
}

}  // namespace mq
