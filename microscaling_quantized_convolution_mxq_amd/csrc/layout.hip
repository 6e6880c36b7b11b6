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

#include <algorithm>

namespace mq {

// ----------------------------------------------------------------------------
// CBF im2col. One workgroup per output pixel o = (ho, wo): its output is one
// contiguous stretch of N * T * row_bytes code bytes ([n][kh][kw][row]) and
// T * nsb scale bytes ([kh][kw][nsb]), written with consecutive 16-byte
// (8-byte when rows are not 16-byte multiples) stores; every chunk copies the
// matching chunk of the source row (n at pixel (ho*s+kh-p, wo*s+kw-p)) or
// zeros outside the image. Divisions by the launch's runtime extents use
// precomputed multiply-shift reciprocals.
// ----------------------------------------------------------------------------
template <int CH>
__global__ __launch_bounds__(256) void cbf_im2col_kernel(
    const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs, uint8_t* __restrict__ oc,
    uint8_t* __restrict__ os, int N, int H, int W, int sh, int sw, int ph, int pw, int T, int cpr,
    int nsb, FastDiv div_tc /* T*cpr */, FastDiv div_c /* cpr */, FastDiv div_kw /* KW */,
    FastDiv div_nsb /* nsb */, FastDiv div_wo /* Wo */) {
  typedef typename std::conditional<CH == 16, uint4, uint2>::type V;
  const unsigned o = blockIdx.x;
  const unsigned ho = fdiv(o, div_wo), wo = o - ho * div_wo.d;
  const int hb = (int)ho * sh - ph, wb = (int)wo * sw - pw;
  const unsigned per_n = T * cpr;
  const unsigned nch = N * per_n;
  const V* src = reinterpret_cast<const V*>(xc);
  V* dst = reinterpret_cast<V*>(oc) + (unsigned long long)o * nch;
  // blockIdx.y splits a pixel's chunks when there are few pixels
  const unsigned per = (nch + gridDim.y - 1) / gridDim.y;
  const unsigned c_lo = blockIdx.y * per, c_hi = min(nch, c_lo + per);
  // U chunks per thread in flight: all loads first, then the stores
  constexpr int U = 4;
  for (unsigned c0 = c_lo + threadIdx.x; c0 < c_hi; c0 += U * 256) {
    V v[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const unsigned c = c0 + u * 256;
      const unsigned n = fdiv(c, div_tc);
      const unsigned r = c - n * per_n;
      const unsigned t = fdiv(r, div_c);
      const unsigned ch = r - t * cpr;
      const unsigned kh = fdiv(t, div_kw), kw = t - kh * div_kw.d;
      const int hi = hb + (int)kh, wi = wb + (int)kw;
      v[u] = V{};
      if (c < c_hi && (unsigned)hi < (unsigned)H && (unsigned)wi < (unsigned)W)
        v[u] = src[((unsigned long long)(hi * W + wi) * N + n) * cpr + ch];
    }
    // streaming stores: the expanded tensor is not read back by this step,
    // and keeping it out of the caches leaves them to the source rows
    typedef unsigned NV __attribute__((ext_vector_type(CH / 4)));
#pragma unroll
    for (int u = 0; u < U; u++)
      if (c0 + u * 256 < c_hi)
        __builtin_nontemporal_store(*reinterpret_cast<const NV*>(&v[u]), reinterpret_cast<NV*>(&dst[c0 + u * 256]));
  }
  const unsigned ns = T * nsb;
  for (unsigned c = threadIdx.x; blockIdx.y == 0 && c < ns; c += 256) {
    const unsigned t = fdiv(c, div_nsb), k = c - t * nsb;
    const unsigned kh = fdiv(t, div_kw), kw = t - kh * div_kw.d;
    const int hi = hb + (int)kh, wi = wb + (int)kw;
    uint8_t v = 0;
    if ((unsigned)hi < (unsigned)H && (unsigned)wi < (unsigned)W) v = xs[(unsigned long long)(hi * W + wi) * nsb + k];
    os[(unsigned long long)o * ns + c] = v;
  }
}

hipError_t launch_cbf_im2col(const Conv& cv, MxView x, uint8_t* col_codes, uint8_t* col_scales,
                             hipStream_t st) {
  const long long rb = row_bytes(x.fmt, cv.cin);
  const int CH = (rb % 16 == 0) ? 16 : 8;
  const int cpr = (int)(rb / CH);
  const int Ho = cv.ho(), Wo = cv.wo(), T = cv.kh * cv.kw;
  const int nsb = ceil_div(cv.n, x.bp) * ceil_div(cv.cin, 32);
  // per-pixel chunk indices stay below 2^31 (tensor sizes are capped at 2^30 elements)
  const FastDiv dtc = make_fastdiv((unsigned)(T * cpr)), dc = make_fastdiv((unsigned)cpr),
                dkw = make_fastdiv((unsigned)cv.kw), dnsb = make_fastdiv((unsigned)nsb),
                dwo = make_fastdiv((unsigned)Wo);
  const unsigned blocks = (unsigned)Ho * (unsigned)Wo;
  // at least ~2048 workgroups, but no split below 1024 chunks per workgroup
  const unsigned nch = (unsigned)cv.n * T * cpr;
  unsigned split = blocks >= 2048 ? 1u : (2048u + blocks - 1) / blocks;
  split = std::max(1u, std::min(split, nch / 1024u));
  const dim3 grid(blocks, split);
  if (CH == 16)
    hipLaunchKernelGGL(cbf_im2col_kernel<16>, grid, dim3(256), 0, st, x.codes, x.scales, col_codes,
                       col_scales, cv.n, cv.h, cv.w, cv.sh, cv.sw, cv.ph, cv.pw, T, cpr, nsb, dtc, dc, dkw,
                       dnsb, dwo);
  else
    hipLaunchKernelGGL(cbf_im2col_kernel<8>, grid, dim3(256), 0, st, x.codes, x.scales, col_codes,
                       col_scales, cv.n, cv.h, cv.w, cv.sh, cv.sw, cv.ph, cv.pw, T, cpr, nsb, dtc, dc, dkw,
                       dnsb, dwo);
  return launch_check();
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

// 8-bit codes: one wave per tile of 32 partner rows x 64 channels. The wave
// stages the tile in LDS (row pitch 72 bytes: the transposing reads of 8 rows
// then hit distinct banks) and reads it back with ds_read_b64_tr_b8: in each
// group of 16 lanes, lanes 2i and 2i+1 address the two 8-byte halves of row
// r0+i, and lane t receives rows r0..r0+7 of column t of the group. Four such
// reads give every lane the 32 partner codes of one channel: one output run,
// stored as RS contiguous bytes (consecutive lanes, consecutive channels):
// 32, or 16 when P <= 16 (only the first 16 codes can be nonzero).
__global__ __launch_bounds__(256) void transpose_codes8_kernel(const uint8_t* __restrict__ in,
                                                              uint8_t* __restrict__ out, int P, int B,
                                                              int C, int nPB, int nCC, long long ntiles,
                                                              int RS) {
  constexpr int PITCH = 72;
  __shared__ __attribute__((aligned(16))) uint8_t lds[4][32 * PITCH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long tile = (long long)blockIdx.x * 4 + wave;
  if (tile >= ntiles) return;  // whole wave (no workgroup barrier below)
  const int cc = (int)(tile % nCC);
  const long long rest = tile / nCC;
  const int pb = (int)(rest % nPB);
  const long long ab = rest / nPB;
  const long long a = ab / B;
  const int b = (int)(ab % B);
  const int nCB = (C + 31) / 32;
  const long long rb = (long long)nCB * 32;
  const int c0 = cc * 64;
  uint8_t* t = lds[wave];
  {  // load: lane -> row lane/2, 32 bytes at column c0 + 32*(lane%2)
    const int r = lane >> 1, hc = (lane & 1) * 32;
    const int p = pb * 32 + r;
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
    if (p < P && c0 + hc < rb) {
      const uint4* src = reinterpret_cast<const uint4*>(in + ((a * P + p) * B + b) * rb + c0 + hc);
      v0 = src[0];
      v1 = src[1];
    }
    uint2* d = reinterpret_cast<uint2*>(t + r * PITCH + hc);
    d[0] = make_uint2(v0.x, v0.y); d[1] = make_uint2(v0.z, v0.w);
    d[2] = make_uint2(v1.x, v1.y); d[3] = make_uint2(v1.z, v1.w);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's tile is in LDS
  __builtin_amdgcn_wave_barrier();
  typedef v2i __attribute__((address_space(3)))* lds_v2i_ptr;
  const int g = lane >> 4, j = lane & 15;
  uint32_t run[8];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int row = 8 * q + (j >> 1), col = 16 * g + 8 * (j & 1);
    const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_ptr)(t + row * PITCH + col));
    run[2 * q] = r.x; run[2 * q + 1] = r.y;
  }
  const int c = c0 + lane;
  if (c < C) {
    uint4* dst = reinterpret_cast<uint4*>(out + ((ab * C + c) * nPB + pb) * RS);
    dst[0] = make_uint4(run[0], run[1], run[2], run[3]);
    if (RS == 32) dst[1] = make_uint4(run[4], run[5], run[6], run[7]);
  }
}

hipError_t launch_transpose_codes(const uint8_t* in, uint8_t* out, int fmt, bool half, int A, int P, int B,
                                  int C, hipStream_t st) {
  if (half && (fmt > 1 || P > 16)) return hipErrorInvalidValue;
  if (fmt <= 1) {  // 8-bit codes
    const int nPB = ceil_div(P, 32), nCC = ceil_div(ceil_div(C, 32) * 32, 64);
    const long long ntiles = (long long)A * B * nPB * nCC;
    hipLaunchKernelGGL(transpose_codes8_kernel, dim3((unsigned)((ntiles + 3) / 4)), dim3(256), 0, st, in, out,
                       P, B, C, nPB, nCC, ntiles, half ? 16 : 32);
    return launch_check();
  }
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
  return launch_check();
}

}  // namespace mq
