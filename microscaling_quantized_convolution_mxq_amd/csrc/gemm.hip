// gemm.hip -- the three block-scaled convolution GEMMs of MicroQonv §IV-B on
// gfx950 block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4):
//   forward          Y_f   = W_f . X'      (K = (kh, kw, ci), X' gathered on the
//                                           fly from the CBF activation: implicit
//                                           channel-batch-first im2col, §IV-A)
//   backward-data    G_X   = W^T * G_Y     (Eq. 2; K = (kh, kw, co); output rows
//                                           grouped by stride parity class so every
//                                           row of a tile has the same valid taps)
//   backward-weight  G_W_f = G_Y_f . X'^T  (Eq. 3; K = (ho, wo, n); split over K
//                                           with a deterministic reduction)
// Each 32-wide K-block of an operand row is one run of 32 packed codes with
// one E8M0 scale, which is exactly the block-scaled dot product of Eq. (7):
// the MFMA multiplies the codes and applies both block scales per K-block.
//
// Tiling: 256 threads = 4 waves in a WM x WN grid; each wave owns a 64 x 64
// output tile = 2 x 2 MFMA tiles of 32 x 32; one K-step covers two K-blocks.
// Operands are loaded straight from global memory into the MFMA register
// images (see mx_common.h), one K-step ahead of the MFMAs that use them.
#include "mx_common.h"
#include "mqconv_internal.h"

namespace mq {

// Loads one 32x32x64 operand register image for a row from up to two runs.
// p0/p1: runs of K-blocks kb0 and kb0+1 (nullptr = zero block).
template <int F>
__device__ __forceinline__ v8i load_operand(const uint8_t* p0, const uint8_t* p1, int q) {
  v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (F <= 1) {
    if (p0) { v4i t = *reinterpret_cast<const v4i*>(p0 + 16 * q); r[0] = t[0]; r[1] = t[1]; r[2] = t[2]; r[3] = t[3]; }
    if (p1) { v4i t = *reinterpret_cast<const v4i*>(p1 + 16 * q); r[4] = t[0]; r[5] = t[1]; r[6] = t[2]; r[7] = t[3]; }
  } else if constexpr (F <= 3) {
    const uint8_t* p = q ? p1 : p0;
    if (p) {
      const uint2* s = reinterpret_cast<const uint2*>(p);
      uint2 a = s[0], b = s[1], c = s[2];
      r[0] = a.x; r[1] = a.y; r[2] = b.x; r[3] = b.y; r[4] = c.x; r[5] = c.y;
    }
  } else {
    const uint8_t* p = q ? p1 : p0;
    if (p) { v4i t = *reinterpret_cast<const v4i*>(p); r[0] = t[0]; r[1] = t[1]; r[2] = t[2]; r[3] = t[3]; }
  }
  return r;
}

// ---------------------------------------------------------------------------
// Problem descriptors. K-block kb is addressed as (u, v) = (kb / nin, kb % nin).
// run_X(row, u, v, &scale) returns the run's address or nullptr for a zero
// block, and sets `scale` to its E8M0 byte.
// ---------------------------------------------------------------------------
struct FwdProb {
  const uint8_t *xc, *xs, *wc, *ws;
  float* y;
  int N, H, W, Cin, Cout, KW, T, sh, sw, ph, pw, Wo, M;
  int xrb, xRB, xbp, xnPB, ncb;   // activation row bytes, run bytes, bp, partner blocks, channel blocks
  int wrb, wRB, wnCoB, wbp;        // weight row bytes, run bytes, Cout blocks, bp
  struct RA { int ho, wo, n; bool ok; };
  struct RB { int co; bool ok; };
  __device__ int rows_a(int) const { return M; }
  __device__ int nin() const { return ncb; }
  __device__ void krange(int, int& lo, int& hi) const { lo = 0; hi = T * ncb; }
  __device__ RA setup_a(int, int m) const {
    RA r; r.ok = m < M; int mm = r.ok ? m : 0;
    int pix = mm / N; r.n = mm - pix * N; r.ho = pix / Wo; r.wo = pix - r.ho * Wo; return r;
  }
  __device__ RB setup_b(int, int c) const { RB r; r.ok = c < Cout; r.co = r.ok ? c : 0; return r; }
  __device__ const uint8_t* run_a(const RA& r, int u, int v, int kh, int kw, uint8_t& s) const {
    const int hi = r.ho * sh + kh - ph, wi = r.wo * sw + kw - pw;
    if (!r.ok || hi < 0 || hi >= H || wi < 0 || wi >= W) { s = 0; return nullptr; }
    const long long pix = (long long)hi * W + wi;
    s = xs[(pix * xnPB + r.n / xbp) * ncb + v];
    return xc + (pix * N + r.n) * xrb + (long long)v * xRB;
  }
  __device__ const uint8_t* run_b(const RB& r, int u, int v, uint8_t& s) const {
    if (!r.ok) { s = 0; return nullptr; }
    s = ws[((long long)u * wnCoB + r.co / wbp) * ncb + v];
    return wc + ((long long)r.co * T + u) * wrb + (long long)v * wRB;
  }
  // tap coordinates of outer index u (uniform)
  __device__ void tap_of(int, int u, int& kh, int& kw) const { kh = u / KW; kw = u - kh * KW; }
  __device__ void store(int, int m, int c, float val) const {
    if (m < M && c < Cout) y[(long long)m * Cout + c] = val;
  }
};

struct DgradProb {
  const uint8_t *dyc, *dys, *wtc, *ws;
  float* dx;
  int N, H, W, Cin, Cout, KH, KW, sh, sw, ph, pw, Ho, Wo;
  int dyrb, dyRB, dybp, dynPB, ncob;  // gradient row bytes, run bytes, bp, partner blocks, Cout blocks
  int wRB, ncbi;                      // weight run bytes, Cin blocks
  struct Cls { int ph_c, pw_c, Hc, Wc, kh0, kw0, nkh, nkw; };
  __device__ Cls cls(int z) const {
    Cls c; c.ph_c = z / sw; c.pw_c = z - c.ph_c * sw;
    c.Hc = (H - c.ph_c + sh - 1) / sh; c.Wc = (W - c.pw_c + sw - 1) / sw;
    if (c.Hc < 0) c.Hc = 0;
    if (c.Wc < 0) c.Wc = 0;
    c.kh0 = (c.ph_c + ph) % sh; c.kw0 = (c.pw_c + pw) % sw;
    c.nkh = c.kh0 < KH ? (KH - c.kh0 + sh - 1) / sh : 0;
    c.nkw = c.kw0 < KW ? (KW - c.kw0 + sw - 1) / sw : 0;
    return c;
  }
  struct RA { int h, w, n; bool ok; };
  struct RB { int ci; bool ok; };
  __device__ int rows_a(int z) const { Cls c = cls(z); return c.Hc * c.Wc * N; }
  __device__ int nin() const { return ncob; }
  __device__ void krange(int z, int& lo, int& hi) const { Cls c = cls(z); lo = 0; hi = c.nkh * c.nkw * ncob; }
  __device__ RA setup_a(int z, int m) const {
    Cls c = cls(z); RA r; r.ok = m < c.Hc * c.Wc * N; int mm = r.ok ? m : 0;
    int pix = mm / N; r.n = mm - pix * N; int hq = pix / c.Wc, wq = pix - hq * c.Wc;
    r.h = hq * sh + c.ph_c; r.w = wq * sw + c.pw_c; return r;
  }
  __device__ RB setup_b(int, int c) const { RB r; r.ok = c < Cin; r.ci = r.ok ? c : 0; return r; }
  __device__ void tap_of(int z, int u, int& kh, int& kw) const {
    Cls c = cls(z); int i = u / c.nkw; kh = c.kh0 + sh * i; kw = c.kw0 + sw * (u - i * c.nkw);
  }
  __device__ const uint8_t* run_a(const RA& r, int u, int v, int kh, int kw, uint8_t& s) const {
    const int th = r.h + ph - kh, tw = r.w + pw - kw;  // divisible by the stride by class choice
    const int ho = th / sh, wo = tw / sw;
    if (!r.ok || th < 0 || tw < 0 || ho >= Ho || wo >= Wo) { s = 0; return nullptr; }
    const long long pix = (long long)ho * Wo + wo;
    s = dys[(pix * dynPB + r.n / dybp) * ncob + v];
    return dyc + (pix * N + r.n) * dyrb + (long long)v * dyRB;
  }
  __device__ const uint8_t* run_b_tap(const RB& r, int tap, int v, uint8_t& s) const {
    if (!r.ok) { s = 0; return nullptr; }
    s = ws[((long long)tap * ncob + v) * ncbi + r.ci / 32];
    return wtc + (((long long)tap * Cin + r.ci) * ncob + v) * wRB;
  }
  __device__ void store(int z, int m, int c, float val) const {
    Cls k = cls(z);
    if (m >= k.Hc * k.Wc * N || c >= Cin) return;
    int pix = m / N, n = m - pix * N; int hq = pix / k.Wc, wq = pix - hq * k.Wc;
    int h = hq * sh + k.ph_c, w = wq * sw + k.pw_c;
    dx[(((long long)h * W + w) * N + n) * Cin + c] = val;
  }
};

struct WgradProb {
  const uint8_t *dytc, *dys, *xtc, *xs;
  float* part;
  int N, H, W, Cin, Cout, KW, T, sh, sw, ph, pw, Wo, nNB, ncob, ncbi;
  int dyRB, xRB;
  int npix;        // Ho*Wo
  int pix_per_split;
  struct RA { int co; bool ok; };
  struct RB { int kh, kw, ci; bool ok; };
  __device__ int rows_a(int) const { return Cout; }
  __device__ int nin() const { return nNB; }
  __device__ void krange(int z, int& lo, int& hi) const {
    int p0 = z * pix_per_split, p1 = min(npix, p0 + pix_per_split);
    lo = p0 * nNB; hi = max(p0, p1) * nNB;
  }
  __device__ RA setup_a(int, int m) const { RA r; r.ok = m < Cout; r.co = r.ok ? m : 0; return r; }
  __device__ RB setup_b(int, int j) const {
    RB r; r.ok = j < T * Cin; int jj = r.ok ? j : 0; int tap = jj / Cin; r.ci = jj - tap * Cin;
    r.kh = tap / KW; r.kw = tap - r.kh * KW; return r;
  }
  __device__ const uint8_t* run_a(const RA& r, int u, int v, uint8_t& s) const {
    if (!r.ok) { s = 0; return nullptr; }
    s = dys[((long long)u * nNB + v) * ncob + r.co / 32];
    return dytc + (((long long)u * Cout + r.co) * nNB + v) * dyRB;
  }
  __device__ const uint8_t* run_b(const RB& r, int ho, int wo, int v, uint8_t& s) const {
    const int hi = ho * sh + r.kh - ph, wi = wo * sw + r.kw - pw;
    if (!r.ok || hi < 0 || hi >= H || wi < 0 || wi >= W) { s = 0; return nullptr; }
    const long long pix = (long long)hi * W + wi;
    s = xs[(pix * nNB + v) * ncbi + r.ci / 32];
    return xtc + ((pix * Cin + r.ci) * nNB + v) * xRB;
  }
  __device__ void store(int z, int m, int c, float val) const {
    if (m < Cout && c < T * Cin) part[((long long)z * Cout + m) * ((long long)T * Cin) + c] = val;
  }
};

// Plain GEMM out[m][c] = sum_kb A[m][kb] . B[c][kb] over packed rows whose
// runs already follow the contraction (used by the naive comparison path).
// Split over K-blocks: slice z covers [z*kb_per_split, (z+1)*kb_per_split)
// and writes its partial product to out + z*Ma*Nb.
struct PlainProb {
  const uint8_t *ac, *as, *bc, *bs;
  float* out;
  int Ma, Nb, nkb, aRB, bRB, kb_per_split;
  long long arb, brb;
  struct RA { int m; bool ok; };
  struct RB { int n; bool ok; };
  __device__ int rows_a(int) const { return Ma; }
  __device__ int nin() const { return 1; }
  __device__ void krange(int z, int& lo, int& hi) const {
    lo = z * kb_per_split; hi = min(nkb, lo + kb_per_split); if (hi < lo) hi = lo;
  }
  __device__ RA setup_a(int, int m) const { RA r; r.ok = m < Ma; r.m = r.ok ? m : 0; return r; }
  __device__ RB setup_b(int, int c) const { RB r; r.ok = c < Nb; r.n = r.ok ? c : 0; return r; }
  __device__ void store(int z, int m, int c, float val) const {
    if (m < Ma && c < Nb) out[((long long)z * Ma + m) * Nb + c] = val;
  }
};

// Per-problem dispatch of one operand row's run pointer for K-block (u, v).
template <class P> struct Access;
template <> struct Access<FwdProb> {
  static __device__ const uint8_t* a(const FwdProb& p, int z, const FwdProb::RA& r, int u, int v, uint8_t& s) {
    int kh, kw; p.tap_of(z, u, kh, kw); return p.run_a(r, u, v, kh, kw, s);
  }
  static __device__ const uint8_t* b(const FwdProb& p, int, const FwdProb::RB& r, int u, int v, uint8_t& s) {
    return p.run_b(r, u, v, s);
  }
};
template <> struct Access<DgradProb> {
  static __device__ const uint8_t* a(const DgradProb& p, int z, const DgradProb::RA& r, int u, int v, uint8_t& s) {
    int kh, kw; p.tap_of(z, u, kh, kw); return p.run_a(r, u, v, kh, kw, s);
  }
  static __device__ const uint8_t* b(const DgradProb& p, int z, const DgradProb::RB& r, int u, int v, uint8_t& s) {
    int kh, kw; p.tap_of(z, u, kh, kw); return p.run_b_tap(r, kh * p.KW + kw, v, s);
  }
};
template <> struct Access<WgradProb> {
  static __device__ const uint8_t* a(const WgradProb& p, int, const WgradProb::RA& r, int u, int v, uint8_t& s) {
    return p.run_a(r, u, v, s);
  }
  static __device__ const uint8_t* b(const WgradProb& p, int, const WgradProb::RB& r, int u, int v, uint8_t& s) {
    int ho = u / p.Wo, wo = u - ho * p.Wo; return p.run_b(r, ho, wo, v, s);
  }
};

template <> struct Access<PlainProb> {
  static __device__ const uint8_t* a(const PlainProb& p, int, const PlainProb::RA& r, int u, int, uint8_t& s) {
    if (!r.ok) { s = 0; return nullptr; }
    s = p.as[(long long)r.m * p.nkb + u];
    return p.ac + (long long)r.m * p.arb + (long long)u * p.aRB;
  }
  static __device__ const uint8_t* b(const PlainProb& p, int, const PlainProb::RB& r, int u, int, uint8_t& s) {
    if (!r.ok) { s = 0; return nullptr; }
    s = p.bs[(long long)r.n * p.nkb + u];
    return p.bc + (long long)r.n * p.brb + (long long)u * p.bRB;
  }
};

template <int FA, int FB, class P, int WM, int WN>
__global__ __launch_bounds__(256) void mx_gemm_kernel(P prob) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int z = blockIdx.z;
  const int m_base = blockIdx.x * (WM * 64) + wm * 64;
  const int n_base = blockIdx.y * (WN * 64) + wn * 64;
  if (blockIdx.x * (WM * 64) >= prob.rows_a(z)) return;  // whole tile beyond this class's rows
  const int r32 = lane & 31, q = lane >> 5;
  typename P::RA ra[2];
  typename P::RB rb[2];
#pragma unroll
  for (int i = 0; i < 2; i++) ra[i] = prob.setup_a(z, m_base + i * 32 + r32);
#pragma unroll
  for (int j = 0; j < 2; j++) rb[j] = prob.setup_b(z, n_base + j * 32 + r32);

  int kb_lo, kb_hi;
  prob.krange(z, kb_lo, kb_hi);
  const int nin = prob.nin();
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  // K-block coordinates of the current pair (kb, kb+1)
  int u0 = kb_lo / nin, v0 = kb_lo - (kb_lo / nin) * nin;
  v8i a_cur[2], b_cur[2];
  int sa_cur[2], sb_cur[2];
  auto load_step = [&](int kb, int uu0, int vv0, v8i (&av)[2], v8i (&bv)[2], int (&sa)[2], int (&sb)[2]) {
    int uu1 = uu0, vv1 = vv0 + 1;
    if (vv1 == nin) { vv1 = 0; uu1++; }
    const bool ok0 = kb < kb_hi, ok1 = kb + 1 < kb_hi;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      uint8_t s0 = 0, s1 = 0;
      const uint8_t* p0 = ok0 ? Access<P>::a(prob, z, ra[i], uu0, vv0, s0) : nullptr;
      const uint8_t* p1 = ok1 ? Access<P>::a(prob, z, ra[i], uu1, vv1, s1) : nullptr;
      av[i] = load_operand<FA>(p0, p1, q);
      sa[i] = q ? s1 : s0;
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
      uint8_t s0 = 0, s1 = 0;
      const uint8_t* p0 = ok0 ? Access<P>::b(prob, z, rb[j], uu0, vv0, s0) : nullptr;
      const uint8_t* p1 = ok1 ? Access<P>::b(prob, z, rb[j], uu1, vv1, s1) : nullptr;
      bv[j] = load_operand<FB>(p0, p1, q);
      sb[j] = q ? s1 : s0;
    }
  };
  auto advance = [&](int& uu, int& vv) {
    vv += 2;
    while (vv >= nin) { vv -= nin; uu++; }
  };

  if (kb_lo < kb_hi) {
    load_step(kb_lo, u0, v0, a_cur, b_cur, sa_cur, sb_cur);
    for (int kb = kb_lo; kb < kb_hi; kb += 2) {
      v8i a_nxt[2], b_nxt[2];
      int sa_nxt[2], sb_nxt[2];
      int u1 = u0, v1 = v0;
      advance(u1, v1);
      const bool more = kb + 2 < kb_hi;
      if (more) load_step(kb + 2, u1, v1, a_nxt, b_nxt, sa_nxt, sb_nxt);
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
          acc[i][j] = mfma_scaled_32x32x64<FA, FB>(a_cur[i], b_cur[j], sa_cur[i], sb_cur[j], acc[i][j]);
      if (more) {
#pragma unroll
        for (int i = 0; i < 2; i++) { a_cur[i] = a_nxt[i]; sa_cur[i] = sa_nxt[i]; b_cur[i] = b_nxt[i]; sb_cur[i] = sb_nxt[i]; }
      }
      u0 = u1; v0 = v1;
    }
  }
  // epilogue: lane holds column r32 of rows 8*(e/4) + 4*q + e%4 of each 32x32 tile
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int e = 0; e < 16; e++)
        prob.store(z, m_base + i * 32 + 8 * (e >> 2) + 4 * q + (e & 3), n_base + j * 32 + r32, acc[i][j][e]);
}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            float* __restrict__ out, long long n,
                                                            int splits) {
  long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int z = 0; z < splits; z++) s += part[(long long)z * n + i];  // fixed order: deterministic
  out[i] = s;
}

// ---------------------------------------------------------------------------
// Format dispatch
// ---------------------------------------------------------------------------
template <class P, int WM, int WN>
static hipError_t launch_gemm(int fa, int fb, const P& prob, dim3 grid, hipStream_t st) {
#define MQ_CASE(A, B)                                                                        \
  if (fa == A && fb == B) {                                                                  \
    hipLaunchKernelGGL((mx_gemm_kernel<A, B, P, WM, WN>), grid, dim3(256), 0, st, prob);     \
    return hipGetLastError();                                                                \
  }
  MQ_CASE(0, 0) MQ_CASE(0, 1) MQ_CASE(0, 2) MQ_CASE(0, 3) MQ_CASE(0, 4)
  MQ_CASE(1, 0) MQ_CASE(1, 1) MQ_CASE(1, 2) MQ_CASE(1, 3) MQ_CASE(1, 4)
  MQ_CASE(2, 0) MQ_CASE(2, 1) MQ_CASE(2, 2) MQ_CASE(2, 3) MQ_CASE(2, 4)
  MQ_CASE(3, 0) MQ_CASE(3, 1) MQ_CASE(3, 2) MQ_CASE(3, 3) MQ_CASE(3, 4)
  MQ_CASE(4, 0) MQ_CASE(4, 1) MQ_CASE(4, 2) MQ_CASE(4, 3) MQ_CASE(4, 4)
#undef MQ_CASE
  return hipErrorInvalidValue;
}

template <class P>
static hipError_t launch_tiled(int fa, int fb, const P& prob, int M, int Ncols, int Z, hipStream_t st) {
  if (Ncols <= 64) {
    dim3 grid(ceil_div(M, 256), ceil_div(Ncols, 64), Z);
    return launch_gemm<P, 4, 1>(fa, fb, prob, grid, st);
  }
  if (M <= 64) {
    dim3 grid(ceil_div(M, 64), ceil_div(Ncols, 256), Z);
    return launch_gemm<P, 1, 4>(fa, fb, prob, grid, st);
  }
  dim3 grid(ceil_div(M, 128), ceil_div(Ncols, 128), Z);
  return launch_gemm<P, 2, 2>(fa, fb, prob, grid, st);
}

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// wgrad split over output pixels: enough workgroups to cover the GPU twice.
static int wgrad_splits(const Conv& cv) {
  const long long tiles_m = ceil_div(cv.cout, cv.cout <= 64 ? 64 : 128);
  const long long nj = (long long)cv.kh * cv.kw * cv.cin;
  const long long tiles_n = cv.cout <= 64 ? ceil_div(nj, 256) : ceil_div(nj, 128);
  const long long tiles = tiles_m * tiles_n;
  const long long npix = (long long)cv.ho() * cv.wo();
  long long s = (512 + tiles - 1) / tiles;
  if (s > npix) s = npix;
  if (s < 1) s = 1;
  return (int)s;
}

size_t gemm_workspace_bytes(const Conv& cv, int op, int fa, int fb) {
  if (op == 0) return 0;
  if (op == 1) {  // W re-laid with runs along Cout
    return align256(transposed_bytes(fb, 1, cv.cout, (long long)cv.kh * cv.kw, cv.cin));
  }
  // op 2: fa = gradient format, fb = activation format
  const size_t dyt = align256(transposed_bytes(fa, (long long)cv.ho() * cv.wo(), cv.n, 1, cv.cout));
  const size_t xt = align256(transposed_bytes(fb, (long long)cv.h * cv.w, cv.n, 1, cv.cin));
  const int S = wgrad_splits(cv);
  const size_t part = S > 1 ? align256((size_t)S * cv.cout * cv.kh * cv.kw * cv.cin * 4) : 0;
  return dyt + xt + part;
}

int plain_gemm_splits(long long Ma, long long Nb, long long nkb) {
  const long long tiles = Nb <= 64 ? ceil_div(Ma, 256) : (Ma <= 64 ? ceil_div(Nb, 256) : ceil_div(Ma, 128) * ceil_div(Nb, 128));
  long long s = (512 + tiles - 1) / tiles;
  if (s > nkb / 8) s = nkb / 8;  // keep at least 8 K-blocks per slice
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_plain_gemm(int fa, int fb, const uint8_t* ac, const uint8_t* as, const uint8_t* bc,
                             const uint8_t* bs, int Ma, int Nb, int nkb, float* out, int splits,
                             hipStream_t st) {
  PlainProb p;
  p.ac = ac; p.as = as; p.bc = bc; p.bs = bs; p.out = out; p.Ma = Ma; p.Nb = Nb; p.nkb = nkb;
  p.aRB = (int)run_bytes(fa); p.bRB = (int)run_bytes(fb);
  p.arb = (long long)nkb * p.aRB; p.brb = (long long)nkb * p.bRB;
  p.kb_per_split = ceil_div(nkb, splits);
  return launch_tiled(fa, fb, p, Ma, Nb, splits, st);
}

hipError_t launch_forward(const Conv& cv, MxView x, MxView w, float* y, void*, size_t, hipStream_t st) {
  FwdProb p;
  p.xc = x.codes; p.xs = x.scales; p.wc = w.codes; p.ws = w.scales; p.y = y;
  p.N = cv.n; p.H = cv.h; p.W = cv.w; p.Cin = cv.cin; p.Cout = cv.cout; p.KW = cv.kw;
  p.T = cv.kh * cv.kw; p.sh = cv.sh; p.sw = cv.sw; p.ph = cv.ph; p.pw = cv.pw; p.Wo = cv.wo();
  p.M = cv.ho() * cv.wo() * cv.n;
  p.ncb = ceil_div(cv.cin, 32);
  p.xRB = (int)run_bytes(x.fmt); p.xrb = p.ncb * p.xRB; p.xbp = x.bp; p.xnPB = ceil_div(cv.n, x.bp);
  p.wRB = (int)run_bytes(w.fmt); p.wrb = p.ncb * p.wRB; p.wbp = w.bp; p.wnCoB = ceil_div(cv.cout, w.bp);
  return launch_tiled(x.fmt, w.fmt, p, p.M, cv.cout, 1, st);
}

hipError_t launch_backward_data(const Conv& cv, MxView dy, MxView w, float* dx, void* ws, size_t,
                                hipStream_t st) {
  uint8_t* wt = static_cast<uint8_t*>(ws);
  hipError_t e = launch_transpose_codes(w.codes, wt, w.fmt, 1, cv.cout, cv.kh * cv.kw, cv.cin, st);
  if (e != hipSuccess) return e;
  DgradProb p;
  p.dyc = dy.codes; p.dys = dy.scales; p.wtc = wt; p.ws = w.scales; p.dx = dx;
  p.N = cv.n; p.H = cv.h; p.W = cv.w; p.Cin = cv.cin; p.Cout = cv.cout; p.KH = cv.kh; p.KW = cv.kw;
  p.sh = cv.sh; p.sw = cv.sw; p.ph = cv.ph; p.pw = cv.pw; p.Ho = cv.ho(); p.Wo = cv.wo();
  p.ncob = ceil_div(cv.cout, 32);
  p.dyRB = (int)run_bytes(dy.fmt); p.dyrb = p.ncob * p.dyRB; p.dybp = dy.bp; p.dynPB = ceil_div(cv.n, dy.bp);
  p.wRB = (int)run_bytes(w.fmt); p.ncbi = ceil_div(cv.cin, 32);
  const int maxHc = ceil_div(cv.h, cv.sh), maxWc = ceil_div(cv.w, cv.sw);
  return launch_tiled(dy.fmt, w.fmt, p, maxHc * maxWc * cv.n, cv.cin, cv.sh * cv.sw, st);
}

hipError_t launch_backward_weight(const Conv& cv, MxView dy, MxView x, float* dw, void* ws, size_t,
                                  hipStream_t st) {
  uint8_t* base = static_cast<uint8_t*>(ws);
  const long long npix_o = (long long)cv.ho() * cv.wo();
  uint8_t* dyt = base;
  const size_t dyt_b = align256(transposed_bytes(dy.fmt, npix_o, cv.n, 1, cv.cout));
  uint8_t* xt = base + dyt_b;
  const size_t xt_b = align256(transposed_bytes(x.fmt, (long long)cv.h * cv.w, cv.n, 1, cv.cin));
  float* part = reinterpret_cast<float*>(base + dyt_b + xt_b);
  hipError_t e = launch_transpose_codes(dy.codes, dyt, dy.fmt, (int)npix_o, cv.n, 1, cv.cout, st);
  if (e != hipSuccess) return e;
  e = launch_transpose_codes(x.codes, xt, x.fmt, cv.h * cv.w, cv.n, 1, cv.cin, st);
  if (e != hipSuccess) return e;
  const int S = wgrad_splits(cv);
  WgradProb p;
  p.dytc = dyt; p.dys = dy.scales; p.xtc = xt; p.xs = x.scales; p.part = S > 1 ? part : dw;
  p.N = cv.n; p.H = cv.h; p.W = cv.w; p.Cin = cv.cin; p.Cout = cv.cout; p.KW = cv.kw;
  p.T = cv.kh * cv.kw; p.sh = cv.sh; p.sw = cv.sw; p.ph = cv.ph; p.pw = cv.pw; p.Wo = cv.wo();
  p.nNB = ceil_div(cv.n, 32); p.ncob = ceil_div(cv.cout, 32); p.ncbi = ceil_div(cv.cin, 32);
  p.dyRB = (int)run_bytes(dy.fmt); p.xRB = (int)run_bytes(x.fmt);
  p.npix = (int)npix_o; p.pix_per_split = ceil_div(npix_o, S);
  const int Sx = ceil_div(npix_o, p.pix_per_split);
  const long long nj = (long long)p.T * cv.cin;
  e = launch_tiled(dy.fmt, x.fmt, p, cv.cout, (int)nj, S, st);
  if (e != hipSuccess) return e;
  if (S > 1) {
    const long long n = (long long)cv.cout * nj;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       part, dw, n, S);
    e = hipGetLastError();
  }
  (void)Sx;
  return e;
}

}  // namespace mq
