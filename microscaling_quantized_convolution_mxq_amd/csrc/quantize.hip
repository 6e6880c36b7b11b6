// quantize.hip -- mxq_quantize: fp32 tensor -> packed MX codes + E8M0 scales,
// performed once per tensor (MicroQonv §III-A microscaling quantization,
// §IV-B square blocks along both GEMM directions).
//
// Tensor view [A][P][B][C] (C = channel, contiguous; P = partner dimension):
//   activations / gradients [H][W][N][C]: A = H*W, P = N, B = 1
//   weights [Cout][Kh][Kw][Cin]:          A = 1,   P = Cout, B = Kh*Kw
// memory row of (a, p, b) = (a*P + p)*B + b; a block is 32 channels x bp
// partner rows of one (a, b); its scale byte sits at
// ((a*B + b)*nPB + p/bp)*nCB + c/32.
//
// Mapping: one wave per tile of 32 partner rows x 32 channels; lane l takes
// row l/2 and the channel half l%2 (16 consecutive fp32 = 64 contiguous
// bytes, so each row's 128-byte segment is read by two neighbouring lanes).
// The wave walks all channel blocks of its 32 rows, so every row's packed
// codes are written by one wave in consecutive iterations. The block maximum
// is a max over the lane pair (bp = 1) or over the whole wave (bp = 32).
#include "mx_common.h"
#include "mqconv_internal.h"

namespace mq {

template <int F>
__device__ __forceinline__ void store_half_run(uint8_t* dst, const uint32_t (&c)[16]) {
  constexpr int bits = Fmt<F>::bits;
  if constexpr (bits == 8) {
    uint4 w;
    w.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    w.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    w.z = c[8] | (c[9] << 8) | (c[10] << 16) | (c[11] << 24);
    w.w = c[12] | (c[13] << 8) | (c[14] << 16) | (c[15] << 24);
    *reinterpret_cast<uint4*>(dst) = w;
  } else if constexpr (bits == 6) {
    // 16 codes x 6 bits = 96 bits, code j at bits [6j, 6j+6)
    uint32_t w0 = c[0] | (c[1] << 6) | (c[2] << 12) | (c[3] << 18) | (c[4] << 24) | (c[5] << 30);
    uint32_t w1 = (c[5] >> 2) | (c[6] << 4) | (c[7] << 10) | (c[8] << 16) | (c[9] << 22) | (c[10] << 28);
    uint32_t w2 = (c[10] >> 4) | (c[11] << 2) | (c[12] << 8) | (c[13] << 14) | (c[14] << 20) | (c[15] << 26);
    uint32_t* d = reinterpret_cast<uint32_t*>(dst);  // 4-byte aligned: offsets are multiples of 12
    d[0] = w0; d[1] = w1; d[2] = w2;
  } else {
    uint2 w;
    w.x = c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12) | (c[4] << 16) | (c[5] << 20) | (c[6] << 24) | (c[7] << 28);
    w.y = c[8] | (c[9] << 4) | (c[10] << 8) | (c[11] << 12) | (c[12] << 16) | (c[13] << 20) | (c[14] << 24) | (c[15] << 28);
    *reinterpret_cast<uint2*>(dst) = w;
  }
}

template <int F, bool SQUARE>
__global__ __launch_bounds__(256) void mxq_quantize_kernel(const float* __restrict__ src,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, int A, int P,
                                                          int B, int C, int bp, long long ntiles) {
  const int lane = threadIdx.x & 63;
  const long long tile = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= ntiles) return;
  const int nPT = (P + 31) / 32;  // 32-row tiles along the partner dimension
  const int pt = (int)(tile % nPT);
  const long long ab = tile / nPT;  // = a*B + b
  const int b = (int)(ab % B);
  const long long a = ab / B;
  const int r = lane >> 1, half = lane & 1;
  const int p = pt * 32 + r;
  const bool row_ok = p < P;
  const long long row = (a * P + p) * B + b;
  const int nCB = (C + 31) / 32;
  const int nPB = (P + bp - 1) / bp;
  constexpr int RB = run_bytes_of(F);
  const long long row_bytes = (long long)nCB * RB;
  const float* srow = src + row * (long long)C;
  const bool vec = (C & 3) == 0;

  for (int cb = 0; cb < nCB; cb++) {
    const int c0 = cb * 32 + half * 16;
    float x[16];
    if (row_ok && vec && c0 + 16 <= C) {
      const float4* s4 = reinterpret_cast<const float4*>(srow + c0);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        float4 t = s4[i];
        x[4 * i] = t.x; x[4 * i + 1] = t.y; x[4 * i + 2] = t.z; x[4 * i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; i++) x[i] = (row_ok && c0 + i < C) ? srow[c0 + i] : 0.0f;
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) m = max(m, __float_as_uint(x[i]) & 0x7fffffffu);
    // block max: lane pair (a line of 32 channels) or the whole wave (square)
    m = max(m, (uint32_t)__shfl_xor((int)m, 1));
    if constexpr (SQUARE) {
#pragma unroll
      for (int o = 2; o < 64; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    }
    const uint32_t S = scale_byte_from_amax<F>(m);
    uint32_t c[16];
    if (S == 255u) {
#pragma unroll
      for (int i = 0; i < 16; i++) c[i] = 0;
    } else {
      const float inv = inv_scale_from_byte(S);
#pragma unroll
      for (int i = 0; i < 16; i++) c[i] = encode_scaled<F>(x[i] * inv);
    }
    if (row_ok) {
      store_half_run<F>(codes + row * row_bytes + (long long)cb * RB + half * (RB / 2), c);
      if (SQUARE) {
        if (lane == 0) scales[(ab * nPB + (long long)pt * 32 / bp) * nCB + cb] = (uint8_t)S;
      } else {
        if (half == 0) scales[(ab * nPB + p) * nCB + cb] = (uint8_t)S;
      }
    }
  }
}

template <int F, bool SQ>
static hipError_t launch_q(const float* src, uint8_t* codes, uint8_t* scales, int A, int P, int B,
                           int C, int bp, hipStream_t st) {
  const long long ntiles = (long long)A * B * ((P + 31) / 32);
  const long long blocks = (ntiles + 3) / 4;
  hipLaunchKernelGGL((mxq_quantize_kernel<F, SQ>), dim3((unsigned)blocks), dim3(256), 0, st, src,
                     codes, scales, A, P, B, C, bp, ntiles);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* src, uint8_t* codes, uint8_t* scales, int fmt, int bp, int A,
                           int P, int B, int C, hipStream_t st) {
  const bool sq = bp == 32;
  switch (fmt) {
    case 0: return sq ? launch_q<0, true>(src, codes, scales, A, P, B, C, bp, st) : launch_q<0, false>(src, codes, scales, A, P, B, C, bp, st);
    case 1: return sq ? launch_q<1, true>(src, codes, scales, A, P, B, C, bp, st) : launch_q<1, false>(src, codes, scales, A, P, B, C, bp, st);
    case 2: return sq ? launch_q<2, true>(src, codes, scales, A, P, B, C, bp, st) : launch_q<2, false>(src, codes, scales, A, P, B, C, bp, st);
    case 3: return sq ? launch_q<3, true>(src, codes, scales, A, P, B, C, bp, st) : launch_q<3, false>(src, codes, scales, A, P, B, C, bp, st);
    default: return sq ? launch_q<4, true>(src, codes, scales, A, P, B, C, bp, st) : launch_q<4, false>(src, codes, scales, A, P, B, C, bp, st);
  }
}

}  // namespace mq
