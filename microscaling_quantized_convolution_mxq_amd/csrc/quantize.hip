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
// Mapping: one wave per tile of 32 rows x 32 channels; lane l takes row l/2
// and the channel half l%2 (16 consecutive fp32 = 64 contiguous bytes, so
// each row's 128-byte segment is read by two neighbouring lanes). The wave
// walks all channel blocks of its 32 rows, so every row's packed codes are
// written by one wave in consecutive iterations. The block maximum is a
// cross-lane max; the scaled values are clamped to the format's largest
// finite value and rounded by the hardware conversion instructions.
#include "mx_common.h"
#include "mqconv_internal.h"

namespace mq {

// Converts 16 scaled values (|v| <= max normal already) to codes and stores
// them as half a packed run, with gfx950's conversion instructions: FP8 two
// codes per instruction, FP4 two codes per byte, FP6 sixteen codes per
// instruction (its output interleaves the two 16-value operands, so the even
// values go in the first operand and the odd ones in the second). These
// instructions round to nearest even, keep the sign of zero and produce the
// element formats' subnormals.
template <int F>
__device__ __forceinline__ void convert_store_half_run(uint8_t* dst, const float (&v)[16]) {
  constexpr int bits = Fmt<F>::bits;
  if constexpr (bits == 8) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      uint32_t r;
      if constexpr (F == 0) {
        r = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * i], v[4 * i + 1], 0, false);
        r = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * i + 2], v[4 * i + 3], r, true);
      } else {
        r = __builtin_amdgcn_cvt_pk_bf8_f32(v[4 * i], v[4 * i + 1], 0, false);
        r = __builtin_amdgcn_cvt_pk_bf8_f32(v[4 * i + 2], v[4 * i + 3], r, true);
      }
      w[i] = r;
    }
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  } else if constexpr (bits == 6) {
    v16f even, odd;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      even[i] = v[2 * i]; odd[i] = v[2 * i + 1];
      even[8 + i] = 0.0f; odd[8 + i] = 0.0f;
    }
    typedef int v6i __attribute__((ext_vector_type(6)));
    v6i p;
    if constexpr (F == 2) p = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(even, odd, 1.0f);
    else p = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(even, odd, 1.0f);
    uint32_t* d = reinterpret_cast<uint32_t*>(dst);  // 4-byte aligned: offsets are multiples of 12
    d[0] = p[0]; d[1] = p[1]; d[2] = p[2];
  } else {
    uint32_t w[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      uint32_t r = 0;
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i], v[8 * i + 1], 1.0f, 0);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i + 2], v[8 * i + 3], 1.0f, 1);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i + 4], v[8 * i + 5], 1.0f, 2);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i + 6], v[8 * i + 7], 1.0f, 3);
      w[i] = r;
    }
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  }
}

// MODE 0: line blocks (bp = 1), one block per row and channel block.
// MODE 1: square blocks (bp = 32): a tile is 32 partner rows of one (a, b).
// MODE 2: square blocks over a partner extent P in {1, 2, 4, 8, 16} with
//         B = 1: a tile is 32 consecutive memory rows = 32/P whole pixels,
//         and each pixel's P rows form one block (no idle lanes for small N).
// ST: the tile's 32 rows are consecutive in memory (B = 1) and short
// (at most 8 channel blocks): the wave packs them in LDS and writes the
// tile's bytes as one contiguous stretch, so every store covers whole
// cache lines (6-bit runs are 24 bytes, which direct stores would split).
constexpr int kStageCB = 8;
template <int F, int MODE, bool ST>
__global__ __launch_bounds__(256) void mxq_quantize_kernel(const float* __restrict__ src,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, int A, int P,
                                                          int B, int C, int bp, long long ntiles) {
  __shared__ __attribute__((aligned(16))) uint8_t stage_buf[ST ? 4 : 1][ST ? 32 * kStageCB * 32 : 16];
  const int lane = threadIdx.x & 63;
  const long long tile = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= ntiles) return;
  const int r = lane >> 1, half = lane & 1;
  const int nCB = (C + 31) / 32;
  const int nPB = (P + bp - 1) / bp;
  long long row, sidx;  // memory row; scale byte index of channel block 0
  bool row_ok, writes_scale;
  if constexpr (MODE == 2) {
    row = tile * 32 + r;
    row_ok = row < (long long)A * P;
    const long long a = row / P;
    sidx = a * nCB;                                     // one partner block per pixel (P <= bp)
    writes_scale = (lane & (2 * P - 1)) == 0;           // first lane of the pixel's group
  } else {
    const int nPT = (P + 31) / 32;  // 32-row tiles along the partner dimension
    const int pt = (int)(tile % nPT);
    const long long ab = tile / nPT;  // = a*B + b
    const int b = (int)(ab % B);
    const long long a = ab / B;
    const int p = pt * 32 + r;
    row_ok = p < P;
    row = (a * P + p) * B + b;
    if constexpr (MODE == 1) {
      sidx = (ab * nPB + (long long)pt * 32 / bp) * nCB;
      writes_scale = lane == 0;
    } else {
      sidx = (ab * nPB + p) * nCB;
      writes_scale = half == 0;
    }
  }
  constexpr int RB = run_bytes_of(F);
  const long long row_bytes = (long long)nCB * RB;
  const float* srow = src + row * (long long)C;
  const bool vec = (C & 3) == 0;
  constexpr float maxv = Fmt<F>::maxv;

  // blockIdx.y splits the channel blocks of small tensors over workgroups
  // (gridDim.y is 1 with LDS staging, which needs a tile's whole rows)
  for (int cb = blockIdx.y; cb < nCB; cb += gridDim.y) {
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
    // block max: the lane pair (a line of 32 channels), the whole wave
    // (32 partner rows) or the 2P lanes of one pixel
    m = max(m, (uint32_t)__shfl_xor((int)m, 1));
    if constexpr (MODE == 1) {
#pragma unroll
      for (int o = 2; o < 64; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    } else if constexpr (MODE == 2) {
#pragma unroll
      for (int o = 2; o < 32; o <<= 1)
        if (o < 2 * P) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    }
    const uint32_t S = scale_byte_from_amax<F>(m);
    // scaled values, clamped to the largest finite code (saturation); a block
    // holding a NaN or an infinity gets all-zero codes
    const float inv = inv_scale_from_byte(S == 255u ? 127u : S);
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] = S == 255u ? 0.0f : fminf(fmaxf(x[i] * inv, -maxv), maxv);
    if constexpr (ST) {
      convert_store_half_run<F>(&stage_buf[threadIdx.x >> 6][r * row_bytes + cb * RB + half * (RB / 2)], v);
      if (row_ok && writes_scale) scales[sidx + cb] = (uint8_t)S;
    } else if (row_ok) {
      convert_store_half_run<F>(codes + row * row_bytes + (long long)cb * RB + half * (RB / 2), v);
      if (writes_scale) scales[sidx + cb] = (uint8_t)S;
    }
  }
  if constexpr (ST) {
    // rows row0 .. row0 + nvalid - 1 of this tile are valid and consecutive
    const long long row0 = __shfl(row, 0);
    const int nvalid = __popcll(__ballot(row_ok && half == 0));
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's packed rows are in LDS
    __builtin_amdgcn_wave_barrier();
    const int words = (int)(nvalid * row_bytes / 4);
    const uint32_t* from = reinterpret_cast<const uint32_t*>(stage_buf[threadIdx.x >> 6]);
    uint32_t* to = reinterpret_cast<uint32_t*>(codes + row0 * row_bytes);
    for (int i = lane; i < words; i += 64) to[i] = from[i];
  }
}

template <int F, int MODE>
static hipError_t launch_q(const float* src, uint8_t* codes, uint8_t* scales, int A, int P, int B,
                           int C, int bp, hipStream_t st) {
  const long long ntiles = MODE == 2 ? ((long long)A * P + 31) / 32 : (long long)A * B * ((P + 31) / 32);
  const long long blocks = (ntiles + 3) / 4;
  if (B == 1 && (C + 31) / 32 <= kStageCB)
    hipLaunchKernelGGL((mxq_quantize_kernel<F, MODE, true>), dim3((unsigned)blocks), dim3(256), 0, st, src,
                       codes, scales, A, P, B, C, bp, ntiles);
  else  // small tensors: one workgroup per channel block as well (one memory round trip)
    hipLaunchKernelGGL((mxq_quantize_kernel<F, MODE, false>),
                       dim3((unsigned)blocks, blocks < 512 ? (unsigned)((C + 31) / 32) : 1u), dim3(256), 0, st, src,
                       codes, scales, A, P, B, C, bp, ntiles);
  return hipGetLastError();
}

template <int F>
static hipError_t launch_f(const float* src, uint8_t* codes, uint8_t* scales, int A, int P, int B,
                           int C, int bp, hipStream_t st) {
  if (bp != 32) return launch_q<F, 0>(src, codes, scales, A, P, B, C, bp, st);
  if (B == 1 && P < 32 && (32 % P) == 0) return launch_q<F, 2>(src, codes, scales, A, P, B, C, bp, st);
  return launch_q<F, 1>(src, codes, scales, A, P, B, C, bp, st);
}

hipError_t launch_quantize(const float* src, uint8_t* codes, uint8_t* scales, int fmt, int bp, int A,
                           int P, int B, int C, hipStream_t st) {
  switch (fmt) {
    case 0: return launch_f<0>(src, codes, scales, A, P, B, C, bp, st);
    case 1: return launch_f<1>(src, codes, scales, A, P, B, C, bp, st);
    case 2: return launch_f<2>(src, codes, scales, A, P, B, C, bp, st);
    case 3: return launch_f<3>(src, codes, scales, A, P, B, C, bp, st);
    default: return launch_f<4>(src, codes, scales, A, P, B, C, bp, st);
  }
}

}  // namespace mq
