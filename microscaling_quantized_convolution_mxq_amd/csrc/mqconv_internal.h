// mqconv_internal.h -- launchers shared between the C ABI layer and the
// kernel translation units. Host-side only; arguments are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace mq {

// Geometry of one convolution (copied from the ABI descriptor).
struct Conv {
  int n, cin, h, w, cout, kh, kw, sh, sw, ph, pw;
  int ho() const { return (h + 2 * ph - kh) / sh + 1; }
  int wo() const { return (w + 2 * pw - kw) / sw + 1; }
};

// A packed MX operand as the kernels see it.
struct MxView {
  const uint8_t* codes;
  const uint8_t* scales;
  int fmt;
  int bp;
};
// an MX tensor a kernel writes
struct MxOutView {
  uint8_t* codes;
  uint8_t* scales;
  int fmt;
  int bp;
};

inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// x / d for 0 <= x < 2^31 as (x * m) >> (32 + s), m = ceil(2^(31+l) / d),
// l = ceil(log2 d), s = l - 1: m * d exceeds 2^(31+l) by less than d <= 2^l,
// so the error stays below 1/d and the floor is exact; m < 2^32.
struct FastDiv {
  unsigned m, s, d;
};
inline FastDiv make_fastdiv(unsigned d) {
  FastDiv f; f.d = d;
  if (d == 1) { f.m = 0; f.s = 0; return f; }
  unsigned l = 0;
  while ((1ull << l) < d) l++;
  f.m = (unsigned)(((1ull << (31 + l)) + d - 1) / d);
  f.s = l - 1;
  return f;
}
__device__ __forceinline__ unsigned fdiv(unsigned x, const FastDiv& f) {
  return f.d == 1 ? x : (__umulhi(x, f.m) >> f.s);
}

inline long long run_bytes(int fmt) { return fmt <= 1 ? 32 : (fmt <= 3 ? 24 : 16); }
inline long long row_bytes(int fmt, long long C) { return ((C + 31) / 32) * run_bytes(fmt); }

hipError_t launch_quantize(const float* src, uint8_t* codes, uint8_t* scales, int fmt, int bp, int A,
                           int P, int B, int C, hipStream_t st);
// the same with the elements rounded stochastically (random words from seed)
hipError_t launch_quantize_sr(const float* src, uint8_t* codes, uint8_t* scales, int fmt, int bp, int A,
                              int P, int B, int C, uint64_t seed, hipStream_t st);
// one tensor of a grouped quantization: [A][P][B] x C view as launch_quantize
struct QReq {
  const float* src;
  uint8_t *codes, *scales;
  int fmt, bp, A, P, B, C;
};
hipError_t launch_quantize_group(const QReq* reqs, int count, hipStream_t st);

// Status of the kernel launches enqueued so far (hipGetLastError), or a
// launch failure when a failure injected for the tests of the error paths
// (mqconv_inject_launch_failure) falls due at this check.
hipError_t launch_check();

hipError_t launch_cbf_im2col(const Conv& cv, MxView x, uint8_t* col_codes, uint8_t* col_scales,
                             hipStream_t st);

// Codes of a [A][P][B] x C tensor re-laid out so that runs of 32 codes run
// along P: out[((a*B + b)*C + c)*nPB*RB + pb*RB ...] (zeros for p >= P).
// half: 8-bit codes with P <= 16 stored as 16-byte runs (the upper 16 codes
// of a 32-code run would all be zero)
hipError_t launch_transpose_codes(const uint8_t* in, uint8_t* out, int fmt, bool half, int A, int P, int B,
                                  int C, hipStream_t st);
// Workspace bytes of a re-laid tensor (runs along the partner index P). The
// 16-byte runs of the half-block case fit in the same space.
inline size_t transposed_bytes(int fmt, long long A, long long P, long long B, long long C) {
  return (size_t)(A * B * C * ((P + 31) / 32) * run_bytes(fmt));
}

size_t gemm_workspace_bytes(const Conv& cv, int op, int fa, int fb);
// whether the 32-bit buffer offsets of a GEMM's operands fit (op 0 forward:
// fa = X format, bpa = X bp; op 1 backward-data: fa = dY format, bpa = dY bp;
// op 2 backward-weight: fa = dY format, fb = X format)
bool gemm_offsets_ok(const Conv& cv, int op, int fa, int fb, int bpa);
hipError_t launch_forward(const Conv& cv, MxView x, MxView w, float* y, void* ws, size_t ws_bytes,
                          hipStream_t st);
// forward with Y MX-quantized in the epilogue (bp 1, or bp 32 with N % 32 == 0 or 32 % N == 0)
hipError_t launch_forward_mx(const Conv& cv, MxView x, MxView w, MxOutView yq, hipStream_t st);
hipError_t launch_backward_data(const Conv& cv, MxView dy, MxView w, float* dx, void* ws,
                                size_t ws_bytes, hipStream_t st);
// backward-data with dX MX-quantized in the epilogue (same block rules as the forward's Y)
hipError_t launch_backward_data_mx(const Conv& cv, MxView dy, MxView w, MxOutView dxq, void* ws,
                                   size_t ws_bytes, hipStream_t st);
hipError_t launch_backward_weight(const Conv& cv, MxView dy, MxView x, float* dw, void* ws,
                                  size_t ws_bytes, hipStream_t st);

// Plain packed GEMM (runs already along the contraction); splits > 1 writes
// partial products [splits][Ma][Nb] to `out`.
int plain_gemm_splits(long long Ma, long long Nb, long long nkb);
hipError_t launch_plain_gemm(int fa, int fb, const uint8_t* ac, const uint8_t* as, const uint8_t* bc,
                             const uint8_t* bs, int Ma, int Nb, int nkb, float* out, int splits,
                             hipStream_t st);

size_t naive_workspace_bytes(const Conv& cv, int op, int fa, int fb);
hipError_t launch_naive_forward(const Conv& cv, const float* x, const float* w, int fx, int fw,
                                float* y, void* ws, hipStream_t st);
hipError_t launch_naive_backward_data(const Conv& cv, const float* dy, const float* w, int fdy,
                                      int fw, float* dx, void* ws, hipStream_t st);
hipError_t launch_naive_backward_weight(const Conv& cv, const float* dy, const float* x, int fdy,
                                        int fx, float* dw, void* ws, hipStream_t st);

}  // namespace mq
