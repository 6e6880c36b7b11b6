// mx_common.h -- device-side building blocks shared by the gfx950 kernels:
// MX element-format traits, the block-scaled MFMA wrapper and operand
// register images.
//
// Element formats are the OCP MX ones the MicroQonv paper names (FP8 E4M3 /
// E5M2, FP6 E2M3 / E3M2, FP4 E2M1; §II-D, §III-A, §IV-D) with one E8M0 scale
// per block (§II-D "power of two encoded in E8M0"). The enumeration values
// equal the gfx950 MFMA format selectors (cbsz/blgp): 0 fp8 E4M3,
// 1 bf8 E5M2, 2 fp6 E2M3, 3 bf6 E3M2, 4 fp4 E2M1.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));

template <int F> struct Fmt;
// bits: code width; M: mantissa bits; E: exponent bits; bias; emax: exponent of
// the largest binade; emin: exponent of the smallest normal; maxbits: fp32 bit
// pattern of the largest finite value.
template <> struct Fmt<0> { static constexpr int bits = 8, E = 4, M = 3, bias = 7,  emax = 8,  emin = -6;  static constexpr float maxv = 448.0f; };
template <> struct Fmt<1> { static constexpr int bits = 8, E = 5, M = 2, bias = 15, emax = 15, emin = -14; static constexpr float maxv = 57344.0f; };
template <> struct Fmt<2> { static constexpr int bits = 6, E = 2, M = 3, bias = 1,  emax = 2,  emin = 0;   static constexpr float maxv = 7.5f; };
template <> struct Fmt<3> { static constexpr int bits = 6, E = 3, M = 2, bias = 3,  emax = 4,  emin = -2;  static constexpr float maxv = 28.0f; };
template <> struct Fmt<4> { static constexpr int bits = 4, E = 2, M = 1, bias = 1,  emax = 2,  emin = 0;   static constexpr float maxv = 6.0f; };

__host__ __device__ constexpr int run_bytes_of(int fmt) { return fmt <= 1 ? 32 : (fmt <= 3 ? 24 : 16); }
__host__ __device__ constexpr int bits_of(int fmt) { return fmt <= 1 ? 8 : (fmt <= 3 ? 6 : 4); }

// Round an fp32 value that has already been multiplied by 2^-e onto the
// element grid: nearest, ties to even mantissa, saturating at the largest
// finite value, sign of zero kept. Returns the sign-magnitude code.
template <int F>
__device__ __forceinline__ uint32_t encode_scaled(float v) {
  using T = Fmt<F>;
  const uint32_t ub = __float_as_uint(v);
  const uint32_t sign = ub >> 31;
  float a = fminf(__uint_as_float(ub & 0x7fffffffu), T::maxv);
  const uint32_t ab = __float_as_uint(a);
  // normal range of the element format: round the fp32 mantissa to M bits
  constexpr int sh = 23 - T::M;
  uint32_t r = ab + ((1u << (sh - 1)) - 1u) + ((ab >> sh) & 1u);
  uint32_t mag_norm = (r >> sh) - (uint32_t)((127 - T::bias) << T::M);
  // subnormal range: adding 2^(emin - M + 23) makes the fp32 adder round
  // |v| to a multiple of the element's subnormal spacing 2^(emin - M)
  constexpr uint32_t Kbits = (uint32_t)(T::emin - T::M + 23 + 127) << 23;
  uint32_t mag_sub = __float_as_uint(a + __uint_as_float(Kbits)) - Kbits;
  constexpr uint32_t min_normal_bits = (uint32_t)(T::emin + 127) << 23;
  uint32_t mag = (ab < min_normal_bits) ? mag_sub : mag_norm;
  return mag | (sign << (T::bits - 1));
}

// E8M0 scale byte of a block from the fp32 bit pattern of its |max|
// (sign bit cleared): S = max(exponent field - emax, 0); 0xFF if the block
// holds a NaN or an infinity.
template <int F>
__device__ __forceinline__ uint32_t scale_byte_from_amax(uint32_t amax_bits) {
  if (amax_bits >= 0x7f800000u) return 255u;
  int ef = (int)(amax_bits >> 23);
  int s = ef - Fmt<F>::emax;
  return (uint32_t)(s < 0 ? 0 : s);
}

// 2^(127 - S) as fp32 for S in [0, 253].
__device__ __forceinline__ float inv_scale_from_byte(uint32_t S) {
  return __uint_as_float((254u - S) << 23);
}

// The 16 values of half a block run divided by the block's scale 2^(S-127)
// and clamped to the format's largest finite value (saturation). A block
// holding a NaN or an infinity (S = 0xFF) is divided by 1 here and its codes
// are zeroed at conversion (code_keep(S) as the keep mask): a mask after the
// conversion instead of a select per value, so no value takes a branch.
template <int F>
__device__ __forceinline__ void scale_clamp16(const float (&x)[16], uint32_t S, float (&v)[16]) {
  constexpr float maxv = Fmt<F>::maxv;
  const float inv = inv_scale_from_byte(S == 255u ? 127u : S);
#pragma unroll
  for (int i = 0; i < 16; i++) v[i] = fminf(fmaxf(x[i] * inv, -maxv), maxv);
}

// Mask of the code words of a block with scale byte S: all-zero codes for a
// block that holds a NaN or an infinity.
__device__ __forceinline__ uint32_t code_keep(uint32_t S) { return S == 255u ? 0u : ~0u; }

typedef int v6i __attribute__((ext_vector_type(6)));
// The 2 x 16 FP6 conversion (output code 2i from a[i], 2i+1 from b[i]). The
// instruction writes its six result registers while it still reads its
// operands, so a result register placed on an operand register that is read
// later corrupts that operand; the compiler does not keep them apart by
// itself. The empty statement after it takes the result and both operands,
// so all three are live together and no result register can share an
// operand register.
template <int F>
__device__ __forceinline__ v6i cvt_2xpk16_fp6(const v16f& a, const v16f& b) {
  v6i p;
  if constexpr (F == 2) p = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, 1.0f);
  else p = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(a, b, 1.0f);
  asm volatile("" : "+v"(p) : "v"(a), "v"(b));
  return p;
}

// Converts 16 scaled values (|v| <= max normal already) to codes and stores
// them as half a packed run, each code word ANDed with keep, with gfx950's
// conversion instructions: FP8 two codes per instruction, FP4 two codes per
// byte, FP6 sixteen codes per instruction (its output interleaves the two
// 16-value operands, so the even values go in the first operand and the odd
// ones in the second). These instructions round to nearest even, keep the
// sign of zero and produce the element formats' subnormals.
template <int F>
__device__ __forceinline__ void convert_store_half_run(uint8_t* dst, const float (&v)[16], uint32_t keep = ~0u) {
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
      w[i] = r & keep;
    }
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  } else if constexpr (bits == 6) {
    v16f even, odd;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      even[i] = v[2 * i]; odd[i] = v[2 * i + 1];
      even[8 + i] = 0.0f; odd[8 + i] = 0.0f;
    }
    const v6i p = cvt_2xpk16_fp6<F>(even, odd);
    uint32_t* d = reinterpret_cast<uint32_t*>(dst);  // 4-byte aligned: offsets are multiples of 12
    d[0] = p[0] & keep; d[1] = p[1] & keep; d[2] = p[2] & keep;
  } else {
    uint32_t w[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      uint32_t r = 0;
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i], v[8 * i + 1], 1.0f, 0);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i + 2], v[8 * i + 3], 1.0f, 1);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i + 4], v[8 * i + 5], 1.0f, 2);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i + 6], v[8 * i + 7], 1.0f, 3);
      w[i] = r & keep;
    }
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  }
}

// FP6 only: two half runs (v0 to dst0, v1 to dst1) from one conversion
// instruction, whose 32 outputs are v0's 16 codes then v1's.
template <int F>
__device__ __forceinline__ void convert_store_two_half_runs6(uint8_t* dst0, uint8_t* dst1, const float (&v0)[16],
                                                             const float (&v1)[16], uint32_t keep0, uint32_t keep1) {
  static_assert(Fmt<F>::bits == 6, "FP6 formats");
  v16f even, odd;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    even[i] = v0[2 * i]; odd[i] = v0[2 * i + 1];
    even[8 + i] = v1[2 * i]; odd[8 + i] = v1[2 * i + 1];
  }
  const v6i p = cvt_2xpk16_fp6<F>(even, odd);
  uint32_t* d0 = reinterpret_cast<uint32_t*>(dst0);
  uint32_t* d1 = reinterpret_cast<uint32_t*>(dst1);
  d0[0] = p[0] & keep0; d0[1] = p[1] & keep0; d0[2] = p[2] & keep0;
  d1[0] = p[3] & keep1; d1[1] = p[4] & keep1; d1[2] = p[5] & keep1;
}

// Maximum over aligned groups of g lanes (g = 2, 4, ..., 64, uniform), every
// lane of a group receiving it: swaps within quads, mirrors within 8 and 16
// lanes (DPP), a swizzle across the two 16-lane rows of 32 lanes, and the two
// wave halves.
template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp(uint32_t a) {
  return max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t group_max(uint32_t a, int g) {
  a = max_dpp<0xB1>(a);                // quad_perm [1,0,3,2]: lane ^ 1
  if (g >= 4) a = max_dpp<0x4E>(a);    // quad_perm [2,3,0,1]: lane ^ 2
  if (g >= 8) a = max_dpp<0x141>(a);   // row_half_mirror: 7 - lane within 8
  if (g >= 16) a = max_dpp<0x140>(a);  // row_mirror: 15 - lane within 16
  if (g >= 32) a = max(a, (uint32_t)__builtin_amdgcn_ds_swizzle((int)a, 0x401F));  // lane ^ 16 within 32
  if (g >= 64) a = max((uint32_t)__builtin_amdgcn_readlane((int)a, 0), (uint32_t)__builtin_amdgcn_readlane((int)a, 32));
  return a;
}

// Block-scaled MFMA 32x32x64 with E8M0 scales (gfx950 v_mfma_scale_f32_32x32x64_f8f6f4).
// Register images (lane l = row r + 32 q, rows of A and of B^T are "rows"):
//   8-bit formats: bytes 0..15 = codes [16q, 16q+16) of K-block 0 of the pair,
//                  bytes 16..31 = codes [16q, 16q+16) of K-block 1;
//   6/4-bit formats: the whole packed 32-code run of K-block q.
//   scale operand: the E8M0 byte of K-block q of this lane's row.
template <int FA, int FB>
__device__ __forceinline__ v16f mfma_scaled_32x32x64(const v8i& a, const v8i& b, int sa, int sb, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, sa, 0, sb);
}

}  // namespace mq
