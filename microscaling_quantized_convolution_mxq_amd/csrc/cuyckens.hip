// cuyckens.hip -- the square-block comparator of §III-C: the method of [25]
// (square blocks on the im2col-expanded activation of a fully connected
// layer) extended to convolution. X' (classic im2col, §II-C1/§II-C2: rows
// m = (ho, wo, n), columns k = (ci, kh, kw)) is quantized ONCE in 32 x 32
// squares and saved for the backward pass; W_f [Cout][k] and G_Y [m][Cout]
// are quantized once in squares too. A square serves the GEMM along either
// of its directions, so nothing is quantized twice (Table I: x9 / x1 / x1
// quantizations, the 9 being X''s copies of each activation for a 3x3
// kernel), but X' is stored expanded (Table I: x9 backward memory).
// A GEMM whose contraction runs across the codes' runs reads a re-laid copy
// of the codes (runs along the other direction): codes move, values do not.
//   forward:          Y    = X'q . W_fq^T
//   backward-data:    G_X' = G_Yq . W_fq, then col2im -> G_X
//   backward-weight:  G_W  = G_Yq^T . X'q
#include "comparator_kernels.h"
#include "cuyckens.h"
#include "gemm_kernel.h"

namespace mq {

// X' quantized in squares straight from the CBF activation (no fp32 X' in
// memory): one wave per 32 x 32 square (rows m0.., columns k0..); lane l
// takes row l/2 and the 16 columns (l%2)*16.. of the square, gathers them from
// x (0 outside the image), and the square's maximum is a maximum over the
// whole wave. Codes [M][ceil(K/32) runs], scales [ceil(M/32)][ceil(K/32)].
template <int F>
__global__ __launch_bounds__(256) void square_im2col_quantize_kernel(const float* __restrict__ x,
                                                                    uint8_t* __restrict__ codes,
                                                                    uint8_t* __restrict__ scales, int N, int C,
                                                                    int H, int W, int KH, int KW, int sh, int sw,
                                                                    int ph, int pw, int Wo, long long M, int K,
                                                                    long long nsq) {
  const long long sq = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (sq >= nsq) return;  // uniform per wave
  const int nKB = (K + 31) / 32;
  const long long mb = sq / nKB;
  const int kb = (int)(sq - mb * nKB);
  const int lane = threadIdx.x & 63, r = lane >> 1, half = lane & 1;
  const long long m = mb * 32 + r;
  const bool row_ok = m < M;
  float xv[16];
  const int n = row_ok ? (int)(m % N) : 0;
  const long long o = row_ok ? m / N : 0;
  const int ho = (int)(o / Wo), wo = (int)(o - (long long)ho * Wo);
  const int T = KH * KW;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int k = kb * 32 + half * 16 + i;
    float v = 0.0f;
    if (row_ok && k < K) {
      const int ci = k / T, t = k - ci * T;
      const int kh = t / KW, kw = t - kh * KW;
      const int hi = ho * sh + kh - ph, wi = wo * sw + kw - pw;
      if (hi >= 0 && hi < H && wi >= 0 && wi < W) v = x[(((long long)hi * W + wi) * N + n) * C + ci];
    }
    xv[i] = v;
  }
  uint32_t a = 0;
#pragma unroll
  for (int i = 0; i < 16; i++) a = max(a, __float_as_uint(xv[i]) & 0x7fffffffu);
  a = group_max(a, 64);
  const uint32_t S = scale_byte_from_amax<F>(a);
  float v[16];
  scale_clamp16<F>(xv, S, v);
  constexpr int RB = run_bytes_of(F);
  if (row_ok)
    convert_store_half_run<F>(codes + m * ((long long)nKB * RB) + (long long)kb * RB + half * (RB / 2), v, code_keep(S));
  if (lane == 0) scales[mb * nKB + kb] = (uint8_t)S;
}

// The plain GEMM over square-quantized operands: a row's scale is the one of
// its 32-row group, either in a [row group][K-block] array (runs along K,
// as quantized) or in a [K-block][row group] array (codes re-laid with runs
// along the square's other direction). Scale of (row r, K-block kb):
// (r >> sh) * rs + kb * ks.
struct SquareProb : PlainProb {
  int ash, ars, aks, bsh, brs, bks;
  __device__ PairDelta pd_a() const { return PairDelta{aRB, aks, 0, 0}; }
  __device__ PairDelta pd_b() const { return PairDelta{bRB, bks, 0, 0}; }
  __device__ RowInfo row_a(const Ctx&, int m) const {
    RowInfo r; r.ok = m < Ma; const int mm = r.ok ? m : 0;
    r.code = mm * arb; r.scale = (mm >> ash) * ars; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_a(const Ctx&, const KS& k) const { return KInfo{k.u * aRB, k.u * aks, 0, 0}; }
  __device__ RowInfo row_b(const Ctx&, int c) const {
    RowInfo r; r.ok = c < Nb; const int cc = r.ok ? c : 0;
    r.code = cc * brb; r.scale = (cc >> bsh) * brs; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_b(const Ctx&, const KS& k) const { return KInfo{k.u * bRB, k.u * bks, 0, 0}; }
};

// Square-quantized operand as a GEMM sees it: rows of packed runs along the
// contraction, and the square scales addressed as above.
struct SqOperand {
  const uint8_t *codes, *scales;
  int rows, fmt, sh, rs, ks;
  long long scale_bytes;
};

static hipError_t square_gemm(const SqOperand& a, const SqOperand& b, int nkb, float* out, int splits,
                              hipStream_t st) {
  SquareProb p;
  p.ac = a.codes; p.as = a.scales; p.bc = b.codes; p.bs = b.scales; p.out = out;
  p.Ma = a.rows; p.Nb = b.rows; p.nkb = nkb;
  p.aRB = (int)run_bytes(a.fmt); p.bRB = (int)run_bytes(b.fmt);
  p.arb = nkb * p.aRB; p.brb = nkb * p.bRB;
  p.ac_bytes = (long long)a.rows * p.arb; p.as_bytes = a.scale_bytes;
  p.bc_bytes = (long long)b.rows * p.brb; p.bs_bytes = b.scale_bytes;
  p.ash = a.sh; p.ars = a.rs; p.aks = a.ks; p.bsh = b.sh; p.brs = b.rs; p.bks = b.ks;
  p.pairs_per_split = ceil_div((nkb + 1) / 2, splits);
  return launch_tiled(a.fmt, b.fmt, p, a.rows, b.rows, splits, st);
}

static inline size_t al(size_t x) { return (x + 255) & ~(size_t)255; }
static inline unsigned nblk(long long n) { return (unsigned)((n + 255) / 256); }

struct SqSizes {
  long long M, K;
  int nMB, nKB, nCoB;
};
static SqSizes sq_sizes(const Conv& cv) {
  SqSizes s;
  s.M = (long long)cv.ho() * cv.wo() * cv.n;
  s.K = (long long)cv.cin * cv.kh * cv.kw;
  s.nMB = ceil_div(s.M, 32); s.nKB = ceil_div(s.K, 32); s.nCoB = ceil_div(cv.cout, 32);
  return s;
}

size_t cuyckens_col_codes_bytes(const Conv& cv, int fx) {
  const SqSizes s = sq_sizes(cv);
  return (size_t)(s.M * row_bytes(fx, s.K));
}
size_t cuyckens_col_scales_bytes(const Conv& cv) {
  const SqSizes s = sq_sizes(cv);
  return (size_t)s.nMB * s.nKB;
}

static int cuyckens_wgrad_splits(const Conv& cv) {
  const SqSizes s = sq_sizes(cv);
  return plain_gemm_splits(cv.cout, s.K, s.nMB);
}

size_t cuyckens_workspace_bytes(const Conv& cv, int op, int fa, int fb) {
  const SqSizes s = sq_sizes(cv);
  if (op == 0) {  // fa = X format (of the saved X'q), fb = W format: W_f fp32, its codes and scales
    return al(cv.cout * s.K * 4) + al(cv.cout * row_bytes(fb, s.K)) + al((size_t)s.nCoB * s.nKB);
  }
  if (op == 1) {  // fa = dY format, fb = W format
    return al(s.M * row_bytes(fa, cv.cout)) + al((size_t)s.nMB * s.nCoB) + al(cv.cout * s.K * 4) +
           al(cv.cout * row_bytes(fb, s.K)) + al((size_t)s.nCoB * s.nKB) + al(s.K * row_bytes(fb, cv.cout)) +
           al(s.M * s.K * 4);
  }
  // op 2: fa = dY format, fb = X format: dY codes and scales, both re-laid operands, partial sums
  const int S = cuyckens_wgrad_splits(cv);
  return al(s.M * row_bytes(fa, cv.cout)) + al((size_t)s.nMB * s.nCoB) + al(cv.cout * row_bytes(fa, s.M)) +
         al(s.K * row_bytes(fb, s.M)) + al((size_t)S * cv.cout * s.K * 4);
}

hipError_t launch_cuyckens_im2col_quantize(const Conv& cv, const float* x, int fx, uint8_t* col_codes,
                                           uint8_t* col_scales, hipStream_t st) {
  const SqSizes s = sq_sizes(cv);
  const long long nsq = (long long)s.nMB * s.nKB;
  const dim3 grid((unsigned)((nsq + 3) / 4));
#define MQ_SQ(F)                                                                                            \
  hipLaunchKernelGGL(square_im2col_quantize_kernel<F>, grid, dim3(256), 0, st, x, col_codes, col_scales, cv.n, \
                     cv.cin, cv.h, cv.w, cv.kh, cv.kw, cv.sh, cv.sw, cv.ph, cv.pw, cv.wo(), s.M, (int)s.K, nsq)
  switch (fx) {
    case 0: MQ_SQ(0); break;
    case 1: MQ_SQ(1); break;
    case 2: MQ_SQ(2); break;
    case 3: MQ_SQ(3); break;
    default: MQ_SQ(4); break;
  }
#undef MQ_SQ
  return launch_check();
}

// W_f [Cout][K] quantized in squares into (codes, scales) of the workspace.
static hipError_t square_weight(const Conv& cv, const float* w, int fw, float* wf, uint8_t* wc, uint8_t* wsc,
                                hipStream_t st) {
  const SqSizes s = sq_sizes(cv);
  hipLaunchKernelGGL(flatten_w_kernel, dim3(nblk(cv.cout * s.K)), dim3(256), 0, st, w, wf, cv.cout, cv.cin,
                     cv.kh, cv.kw);
  const hipError_t e = launch_check();
  if (e != hipSuccess) return e;
  return launch_quantize(wf, wc, wsc, fw, 32, 1, cv.cout, 1, (int)s.K, st);
}

hipError_t launch_cuyckens_forward(const Conv& cv, const uint8_t* col_codes, const uint8_t* col_scales, int fx,
                                   const float* w, int fw, float* y, void* ws, hipStream_t st) {
  const SqSizes s = sq_sizes(cv);
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* wf = reinterpret_cast<float*>(p); p += al(cv.cout * s.K * 4);
  uint8_t* wc = p; p += al(cv.cout * row_bytes(fw, s.K));
  uint8_t* wsc = p;
  hipError_t e = square_weight(cv, w, fw, wf, wc, wsc, st);
  if (e != hipSuccess) return e;
  // A: X'q rows m, runs along k; B: W_fq rows co, runs along k
  const SqOperand a{col_codes, col_scales, (int)s.M, fx, 5, s.nKB, 1, (long long)s.nMB * s.nKB};
  const SqOperand b{wc, wsc, cv.cout, fw, 5, s.nKB, 1, (long long)s.nCoB * s.nKB};
  return square_gemm(a, b, s.nKB, y, 1, st);
}

hipError_t launch_cuyckens_backward_data(const Conv& cv, const float* dy, const float* w, int fdy, int fw, float* dx,
                                         void* ws, hipStream_t st) {
  const SqSizes s = sq_sizes(cv);
  uint8_t* p = static_cast<uint8_t*>(ws);
  uint8_t* gc = p; p += al(s.M * row_bytes(fdy, cv.cout));
  uint8_t* gs = p; p += al((size_t)s.nMB * s.nCoB);
  float* wf = reinterpret_cast<float*>(p); p += al(cv.cout * s.K * 4);
  uint8_t* wc = p; p += al(cv.cout * row_bytes(fw, s.K));
  uint8_t* wsc = p; p += al((size_t)s.nCoB * s.nKB);
  uint8_t* wct = p; p += al(s.K * row_bytes(fw, cv.cout));
  float* gcol = reinterpret_cast<float*>(p);
  hipError_t e = launch_quantize(dy, gc, gs, fdy, 32, 1, (int)s.M, 1, cv.cout, st);  // G_Y [m][co] in squares
  if (e != hipSuccess) return e;
  if ((e = square_weight(cv, w, fw, wf, wc, wsc, st)) != hipSuccess) return e;
  // W_fq codes re-laid with runs along Cout (rows k)
  if ((e = launch_transpose_codes(wc, wct, fw, false, 1, cv.cout, 1, (int)s.K, st)) != hipSuccess) return e;
  // A: G_Yq rows m, runs along co; B: re-laid W_fq rows k, runs along co
  const SqOperand a{gc, gs, (int)s.M, fdy, 5, s.nCoB, 1, (long long)s.nMB * s.nCoB};
  const SqOperand b{wct, wsc, (int)s.K, fw, 5, 1, s.nKB, (long long)s.nCoB * s.nKB};
  if ((e = square_gemm(a, b, s.nCoB, gcol, 1, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(col2im_kernel<false>, dim3(nblk((long long)cv.h * cv.w * cv.n * cv.cin)), dim3(256), 0, st, gcol, dx,
                     cv.n, cv.cin, cv.h, cv.w, cv.kh, cv.kw, cv.sh, cv.sw, cv.ph, cv.pw, cv.ho(), cv.wo());
  return launch_check();
}

hipError_t launch_cuyckens_backward_weight(const Conv& cv, const float* dy, const uint8_t* col_codes,
                                           const uint8_t* col_scales, int fdy, int fx, float* dw, void* ws,
                                           hipStream_t st) {
  const SqSizes s = sq_sizes(cv);
  const int S = cuyckens_wgrad_splits(cv);
  uint8_t* p = static_cast<uint8_t*>(ws);
  uint8_t* gc = p; p += al(s.M * row_bytes(fdy, cv.cout));
  uint8_t* gs = p; p += al((size_t)s.nMB * s.nCoB);
  uint8_t* gct = p; p += al(cv.cout * row_bytes(fdy, s.M));
  uint8_t* xct = p; p += al(s.K * row_bytes(fx, s.M));
  float* part = reinterpret_cast<float*>(p);
  hipError_t e = launch_quantize(dy, gc, gs, fdy, 32, 1, (int)s.M, 1, cv.cout, st);
  if (e != hipSuccess) return e;
  // both operands re-laid with runs along m (rows co, and rows k of the saved X'q)
  if ((e = launch_transpose_codes(gc, gct, fdy, false, 1, (int)s.M, 1, cv.cout, st)) != hipSuccess) return e;
  if ((e = launch_transpose_codes(col_codes, xct, fx, false, 1, (int)s.M, 1, (int)s.K, st)) != hipSuccess) return e;
  const SqOperand a{gct, gs, cv.cout, fdy, 5, 1, s.nCoB, (long long)s.nMB * s.nCoB};
  const SqOperand b{xct, col_scales, (int)s.K, fx, 5, 1, s.nKB, (long long)s.nMB * s.nKB};
  if ((e = square_gemm(a, b, s.nMB, part, S, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(wgrad_reduce_permute_kernel, dim3(nblk(cv.cout * s.K)), dim3(256), 0, st, part, dw, cv.cout,
                     cv.cin, cv.kh, cv.kw, S);
  return launch_check();
}

}  // namespace mq
