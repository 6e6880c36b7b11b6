// nvfp.hip -- two-level (NVFP-style) microscaling, Eqs. (4)-(6) of MicroQonv
// §II-D / §III-A, with the pages' square blocks of B = 64 (8 channels x 8
// partner indices, §IV-B):
//   T   = max|X| / (448 m)                  FP32 tensor scale (m: largest element)
//   B_i = E4M3(max|X_i| / (T m))            block scale, rounded to nearest
//   q   = code of X_i / (B_i T)             element, rounded to nearest even
// in fp32 arithmetic (IEEE division and products), as the FP32 tensor scale
// implies. A zero tensor gets T = 0 and zero codes; a block whose scale rounds
// to 0 gets zero codes; non-finite values are left out of T and their block
// gets the E4M3 NaN scale 0x7F and zero codes.
// Two launches: partial maxima of |X| over slices of the tensor, then the
// block quantization, in which every workgroup first reduces the partials
// (a fixed set: the result is the same in every workgroup).
#include <algorithm>

#include "mx_common.h"
#include "nvfp.h"

namespace mq {

__global__ __launch_bounds__(256) void nvfp_amax_kernel(const float* __restrict__ src, long long n,
                                                        uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[4];
  uint32_t m = 0;
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const uint32_t a = __float_as_uint(src[i]) & 0x7fffffffu;
    if (a < 0x7f800000u) m = max(m, a);  // finite values only
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// E4M3 code of a non-negative fp32 value, nearest even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_code(float s) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(fminf(s, 448.0f), 0.0f, 0, false) & 0xffu;
}

// One wave per tile of 32 partner rows x all channels of one (a, b); lane l
// takes row l/2 and 16 channels (l%2)*16.. of each 32-channel run, i.e. two
// 8-channel groups; a block's maximum is a maximum over the 8 lanes of its
// rows (lane bits 1..3) for each group.
template <int F>
__global__ __launch_bounds__(256) void nvfp_quantize_kernel(const float* __restrict__ src, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ bscales, float* __restrict__ tscale,
                                                            const uint32_t* __restrict__ partial, int nparts, int A,
                                                            int P, int B, int C, long long ntiles) {
  __shared__ uint32_t red[4];
  uint32_t am = 0;
  for (int i = threadIdx.x; i < nparts; i += 256) am = max(am, partial[i]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __syncthreads();
  am = max(max(red[0], red[1]), max(red[2], red[3]));
  constexpr float m = Fmt<F>::maxv;
  const float T = __uint_as_float(am) / (448.0f * m);
  const float Tm = T * m;
  if (blockIdx.x == 0 && threadIdx.x == 0) *tscale = T;

  const long long tile = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= ntiles) return;  // whole wave
  const int lane = threadIdx.x & 63, r = lane >> 1, half = lane & 1;
  const int nPT = (P + 31) / 32;
  const int pt = (int)(tile % nPT);
  const long long ab = tile / nPT;
  const int b = (int)(ab % B);
  const long long a = ab / B;
  const int p = pt * 32 + r;
  const bool row_ok = p < P;
  const long long row = (a * P + (row_ok ? p : 0)) * B + b;
  const int nCB = (C + 31) / 32, nPB8 = (P + 7) / 8, nCB8 = (C + 7) / 8;
  constexpr int RB = run_bytes_of(F);
  const long long rbytes = (long long)nCB * RB;
  const float* srow = src + row * (long long)C;
  for (int cb = 0; cb < nCB; cb++) {
    const int c0 = cb * 32 + half * 16;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; i++) x[i] = (row_ok && c0 + i < C) ? srow[c0 + i] : 0.0f;
    float v[16];
#pragma unroll
    for (int g = 0; g < 2; g++) {
      uint32_t bm = 0, nf = 0;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t ab_ = __float_as_uint(x[8 * g + i]) & 0x7fffffffu;
        if (ab_ >= 0x7f800000u) nf = 1;
        else bm = max(bm, ab_);
      }
#pragma unroll
      for (int off = 2; off <= 8; off <<= 1) {
        bm = max(bm, (uint32_t)__shfl_xor((int)bm, off));
        nf |= (uint32_t)__shfl_xor((int)nf, off);
      }
      const uint32_t sc = nf ? 0x7Fu : (T == 0.0f ? 0u : e4m3_code(__uint_as_float(bm) / Tm));
      const float d = __builtin_amdgcn_cvt_f32_fp8((int)sc, 0) * T;
      const bool zero = nf || sc == 0u;
#pragma unroll
      for (int i = 0; i < 8; i++) v[8 * g + i] = zero ? 0.0f : fminf(fmaxf(x[8 * g + i] / d, -m), m);
      const int c = c0 + 8 * g;
      if (row_ok && (r & 7) == 0 && c < C) bscales[((ab * nPB8) + p / 8) * nCB8 + c / 8] = (uint8_t)sc;
    }
    if (row_ok) convert_store_half_run<F>(codes + row * rbytes + (long long)cb * RB + half * (RB / 2), v);
  }
}

hipError_t launch_nvfp_quantize(const float* src, uint8_t* codes, uint8_t* bscales, float* tscale, int fmt, int A,
                                int P, int B, int C, void* ws, hipStream_t st) {
  uint32_t* partial = static_cast<uint32_t*>(ws);
  const long long n = (long long)A * P * B * C;
  const int nparts = (int)std::min<long long>(kNvfpParts, std::max<long long>(1, (n + 4095) / 4096));
  hipLaunchKernelGGL(nvfp_amax_kernel, dim3(nparts), dim3(256), 0, st, src, n, partial);
  hipError_t e = launch_check();
  if (e != hipSuccess) return e;
  const long long ntiles = (long long)A * B * ((P + 31) / 32);
  const dim3 grid((unsigned)((ntiles + 3) / 4));
#define MQ_NV(F)                                                                                               \
  hipLaunchKernelGGL(nvfp_quantize_kernel<F>, grid, dim3(256), 0, st, src, codes, bscales, tscale, partial, nparts, \
                     A, P, B, C, ntiles)
  switch (fmt) {
    case 0: MQ_NV(0); break;
    case 1: MQ_NV(1); break;
    case 2: MQ_NV(2); break;
    case 3: MQ_NV(3); break;
    default: MQ_NV(4); break;
  }
#undef MQ_NV
  return launch_check();
}

}  // namespace mq
