// gemm_kernel.h -- the three block-scaled convolution GEMMs of MicroQonv §IV-B on
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
// one E8M0 scale, which is the block-scaled dot product of Eq. (7): the MFMA
// multiplies the codes and applies both block scales per K-block.
//
// Kernel: 256 threads = 4 waves in a WM x WN grid (512 = two such groups
// splitting the K range, for the weight gradient); each wave owns TM x TN
// MFMA tiles of 32 x 32. A K-step is a pair of K-blocks (64 codes per row),
// or two pairs. Operands go from HBM straight into LDS with buffer loads
// that write LDS (no register staging): an NS-deep ring of LDS stages, so
// the loads of step s+NS-1 are in flight while the MFMAs of step s run, with
// one workgroup barrier per step. 8-bit operands whose contraction runs
// across their rows are staged K-major and transposed by the LDS reads.
#pragma once
#include <type_traits>

#include "mx_common.h"
#include "mqconv_internal.h"

namespace mq {

// Byte offsets into a problem's code and scale buffers are the sum of a
// per-row part (fixed per lane, the buffer load's vector offset) and a
// per-step part (uniform across the workgroup, the load's scalar offset; the
// kernel computes it for 64 steps at a time, one step per lane, from
// kstart/k_a/k_b, and reads each step's into scalar registers):
//   code  = row.code + k.code,   scale = row.scale + k.scale
// Both parts are kept non-negative: where a row or a step moves backwards
// (padding, backward taps) the problem adds a bias to one part and the
// buffer descriptor starts that many bytes before the buffer.
// A block is valid iff row.ok && (row.p0 + k.g0) in [0, lim0) && (row.p1 +
// k.g1) in [0, lim1); the geometric test covers the image borders of the
// implicit im2col. Invalid (zero) blocks read from past the end of the
// buffer, where raw buffer loads return 0 (the range check covers the sum of
// both offsets, per dword). K-block j of a step is the first one moved j
// times by a problem-wide PairDelta; a step with fewer K-blocks (odd counts,
// row ends) says how many are valid with nvalid().
constexpr int kOOB = 0x7fffff00;
constexpr int kFar = 0x40000000;  // row coordinate that fails every border test
struct RowInfo { int code, scale, p0, p1; bool ok; };
struct KInfo { int code, scale, g0, g1; };
struct PairDelta { int code, scale, g0, g1; };
struct GRange { int min0, max0, min1, max1; };
// Reciprocals of the grid's x extent and x*y extent (workgroup re-ordering).
// The logical tile grid (tx x ty x tz tiles) and, for a persistent launch,
// the workgroups per XCD (gx; 0: one workgroup per tile).
struct GridDivs { FastDiv nx, nxy; int tx, ty, tz, gx; };

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, long long bytes) {
  const int n = bytes < (long long)kOOB ? (int)bytes : kOOB;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}

// ---------------------------------------------------------------------------
// Problem descriptors
// ---------------------------------------------------------------------------
// Forward: rows m = (ho, wo, n); a step is channel blocks (v, v+1) of tap (kh, kw).
struct FwdProb {
  const uint8_t *xc, *xs, *wc, *ws;
  float* y;
  long long xc_bytes, xs_bytes, wc_bytes, ws_bytes;
  int N, H, W, Cin, Cout, KW, T, sh, sw, ph, pw, Wo, M;
  int xrb, xRB, xbp, xnPB, ncb, npair;  // activation row bytes, run bytes, bp, partner blocks, channel blocks, pairs
  int wrb, wRB, wnCoB, wbp;              // weight row bytes, run bytes, Cout blocks, bp
  int xcb, xsb;                          // bias of the activation row offsets (padding)
  int ga, gb;                            // rows sharing one scale (A, B); 0: per-row scales
  int xbps, wbps;                        // log2 of the activation and weight bp
  int khalf;                             // every K-block holds at most 16 valid codes
  FastDiv dN, dWo, dKW, dnp;             // reciprocals of N, Wo, KW, npair
  GridDivs grid;
  static constexpr bool kGeoA = true, kGeoB = false, kCanGroup = true;
  static constexpr bool kKMajA = false, kKMajB = false;
  static constexpr bool kQuad = false;
  struct Ctx {};
  struct KS { int kh, kw, v; };
  __device__ Ctx ctx(int) const { return Ctx{}; }
  __device__ int rows_a(const Ctx&) const { return M; }
  __device__ int ncols() const { return Cout; }
  __device__ void steps(const Ctx&, int, int& lo, int& hi) const { lo = 0; hi = T * npair; }
  __device__ KS kstart(const Ctx&, int s) const {
    const int u = (int)fdiv((unsigned)s, dnp); KS k; k.v = 2 * (s - u * npair);
    k.kh = (int)fdiv((unsigned)u, dKW); k.kw = u - k.kh * KW; return k;
  }
  __device__ int nvalid(const Ctx&, const KS& k) const { return k.v + 1 >= ncb ? 1 : 2; }
  __device__ PairDelta pd_a() const { return PairDelta{xRB, 1, 0, 0}; }
  __device__ PairDelta pd_b() const { return PairDelta{wRB, 1, 0, 0}; }
  __device__ RowInfo row_a(const Ctx&, int m) const {
    RowInfo r; r.ok = m < M; const int mm = r.ok ? m : 0;
    const int pix = (int)fdiv((unsigned)mm, dN), n = mm - pix * N;
    const int ho = (int)fdiv((unsigned)pix, dWo), wo = pix - ho * Wo;
    r.p0 = ho * sh - ph; r.p1 = wo * sw - pw;
    const int p = r.p0 * W + r.p1;
    r.code = (p * N + n) * xrb + xcb; r.scale = (p * xnPB + (n >> xbps)) * ncb + xsb; return r;
  }
  __device__ KInfo k_a(const Ctx&, const KS& k) const {
    const int d = k.kh * W + k.kw;
    return KInfo{d * N * xrb + k.v * xRB, d * xnPB * ncb + k.v, k.kh, k.kw};
  }
  __device__ RowInfo row_b(const Ctx&, int c) const {
    RowInfo r; r.ok = c < Cout; const int cc = r.ok ? c : 0;
    r.code = cc * T * wrb; r.scale = (cc >> wbps) * ncb; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_b(const Ctx&, const KS& k) const {
    const int tap = k.kh * KW + k.kw;
    return KInfo{tap * wrb + k.v * wRB, tap * wnCoB * ncb + k.v, 0, 0};
  }
  __device__ int lim_a0() const { return H; }
  __device__ int lim_a1() const { return W; }
  __device__ int lim_b0() const { return 1; }
  __device__ int lim_b1() const { return 1; }
  // range of (k.g0, k.g1) over all steps, and steps valid for every row
  __device__ GRange g_range_a(const Ctx&) const { return GRange{0, T / KW - 1, 0, KW - 1}; }
  __device__ GRange g_range_b(const Ctx&) const { return GRange{0, 0, 0, 0}; }
  __device__ bool step_interior_a(const Ctx&, const KS&) const { return false; }
  __device__ bool step_interior_b(const Ctx&, const KS&) const { return true; }
  __device__ float* out_row(const Ctx&, int, int m) const { return m < M ? y + (long long)m * Cout : nullptr; }
  // rows m .. m + run - 1 lie at out_row(m) + j * ncols()
  __device__ int row_run(const Ctx&, int) const { return 1 << 30; }
  // row of the [pixel][N] output that row m of the problem is
  __device__ long long out_index(const Ctx&, int m) const { return m; }
};

// A problem whose epilogue MX-quantizes its output (an activation or a
// gradient [pixel][N][C], quantized as a separate quantization of the fp32
// output would do it) instead of writing fp32: blocks of 32 channels x (1
// row: ymode 0; the 32 rows of a 32-row group within one pixel: ymode 1,
// N % 32 == 0; each pixel's N rows: ymode 2, N dividing 32), so every block
// lies inside one 32-row strip of a tile and one 32-column block of it.
template <class Base>
struct MxOutProb : Base {
  uint8_t *yc, *ys;
  int yfmt, ymode, yrb, ynPB, ynCB;
  static constexpr bool kMxOut = true;
};
using FwdMxProb = MxOutProb<FwdProb>;
template <class P, class = void>
struct MxOut : std::false_type {};
template <class P>
struct MxOut<P, std::void_t<decltype(P::kMxOut)>> : std::bool_constant<P::kMxOut> {};
// problems whose K-major B operand holds 6- or 4-bit codes (kSubB)
template <class P, class = void>
struct SubB : std::false_type {};
template <class P>
struct SubB<P, std::void_t<decltype(P::kSubB)>> : std::bool_constant<P::kSubB> {};

// Backward-data: rows of parity class z are h = hq*sh + ph_c, w = wq*sw + pw_c
// (and all n); the taps reaching them are kh = kh0 + sh*ih, kw = kw0 + sw*iw,
// from output pixel (ho0 - ih, wo0 - iw). A step is Cout blocks (v, v+1) of
// tap (ih, iw).
struct DgradProb {
  const uint8_t *dyc, *dys, *wtc, *ws;
  float* dx;
  long long dyc_bytes, dys_bytes, wtc_bytes, ws_bytes;
  int N, H, W, Cin, Cout, KH, KW, sh, sw, ph, pw, Ho, Wo;
  int dyrb, dyRB, dybp, dynPB, ncob, npair;  // gradient row bytes, run bytes, bp, partner blocks, Cout blocks, pairs
  int wRB, ncbi;                             // weight run bytes, Cin blocks
  int dycb, dysb;                            // bias of the step offsets (backward taps)
  int ga, gb;                                // rows sharing one scale (A, B); 0: per-row scales
  int dybps;                                 // log2 of the gradient bp
  int khalf;                                 // every K-block holds at most 16 valid codes
  FastDiv dN, dnp;                           // reciprocals of N and npair
  FastDiv dWc[8], dNkw[8];                   // reciprocals of each class's width and tap columns (by pw_c)
  GridDivs grid;
  static constexpr bool kGeoA = true, kGeoB = false, kCanGroup = true;
  static constexpr bool kKMajA = false, kKMajB = false;
  static constexpr bool kQuad = false;
  // the class's divisors and output-pixel offsets are taken out of the
  // argument arrays once per workgroup (a dynamic index into them would
  // reload them from memory at every use)
  struct Ctx { int ph_c, pw_c, Hc, Wc, kh0, kw0, nkh, nkw, M, hoff, woff; FastDiv dwc, dnkw; };
  struct KS { int ih, iw, v; };
  __device__ Ctx ctx(int z) const {
    Ctx c; c.ph_c = z / sw; c.pw_c = z - c.ph_c * sw;
    c.Hc = H > c.ph_c ? (H - c.ph_c + sh - 1) / sh : 0;
    c.Wc = W > c.pw_c ? (W - c.pw_c + sw - 1) / sw : 0;
    c.kh0 = (c.ph_c + ph) % sh; c.kw0 = (c.pw_c + pw) % sw;
    c.nkh = c.kh0 < KH ? (KH - c.kh0 + sh - 1) / sh : 0;
    c.nkw = c.kw0 < KW ? (KW - c.kw0 + sw - 1) / sw : 0;
    c.M = c.Hc * c.Wc * N;
    c.hoff = (c.ph_c + ph - c.kh0) / sh; c.woff = (c.pw_c + pw - c.kw0) / sw;
    // (selected, not indexed: an indexed kernel-argument array inside the
    // persistent tile loop became a private-memory copy)
    c.dwc = dWc[0]; c.dnkw = dNkw[0];
#pragma unroll
    for (int k = 1; k < 8; k++)
      if (c.pw_c == k) { c.dwc = dWc[k]; c.dnkw = dNkw[k]; }
    return c;
  }
  __device__ int rows_a(const Ctx& c) const { return c.M; }
  __device__ int ncols() const { return Cin; }
  __device__ void steps(const Ctx& c, int, int& lo, int& hi) const { lo = 0; hi = c.nkh * c.nkw * npair; }
  __device__ KS kstart(const Ctx& c, int s) const {
    const int u = (int)fdiv((unsigned)s, dnp); KS k; k.v = 2 * (s - u * npair);
    k.ih = (int)fdiv((unsigned)u, c.dnkw); k.iw = u - k.ih * c.nkw; return k;
  }
  __device__ int nvalid(const Ctx&, const KS& k) const { return k.v + 1 >= ncob ? 1 : 2; }
  __device__ PairDelta pd_a() const { return PairDelta{dyRB, 1, 0, 0}; }
  __device__ PairDelta pd_b() const { return PairDelta{wRB, ncbi, 0, 0}; }
  __device__ RowInfo row_a(const Ctx& c, int m) const {
    RowInfo r; r.ok = m < c.M; const int mm = r.ok ? m : 0;
    const int wc = c.Wc > 0 ? c.Wc : 1;
    const int pix = (int)fdiv((unsigned)mm, dN), n = mm - pix * N;
    const int hq = (int)fdiv((unsigned)pix, c.dwc), wq = pix - hq * wc;
    // output pixel of tap (kh0, kw0); exact division by the class choice
    r.p0 = hq + c.hoff;
    r.p1 = wq + c.woff;
    const int p = r.p0 * Wo + r.p1;
    r.code = (p * N + n) * dyrb; r.scale = (p * dynPB + (n >> dybps)) * ncob; return r;
  }
  __device__ KInfo k_a(const Ctx&, const KS& k) const {
    const int d = k.ih * Wo + k.iw;
    return KInfo{-d * N * dyrb + k.v * dyRB + dycb, -d * dynPB * ncob + k.v + dysb, -k.ih, -k.iw};
  }
  __device__ RowInfo row_b(const Ctx&, int c) const {
    RowInfo r; r.ok = c < Cin; const int cc = r.ok ? c : 0;
    r.code = cc * ncob * wRB; r.scale = cc / 32; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_b(const Ctx& c, const KS& k) const {
    const int tap = (c.kh0 + sh * k.ih) * KW + (c.kw0 + sw * k.iw);
    return KInfo{(tap * Cin * ncob + k.v) * wRB, (tap * ncob + k.v) * ncbi, 0, 0};
  }
  __device__ int lim_a0() const { return Ho; }
  __device__ int lim_a1() const { return Wo; }
  __device__ int lim_b0() const { return 1; }
  __device__ int lim_b1() const { return 1; }
  __device__ GRange g_range_a(const Ctx& c) const { return GRange{1 - c.nkh, 0, 1 - c.nkw, 0}; }
  __device__ GRange g_range_b(const Ctx&) const { return GRange{0, 0, 0, 0}; }
  __device__ bool step_interior_a(const Ctx&, const KS&) const { return false; }
  __device__ bool step_interior_b(const Ctx&, const KS&) const { return true; }
  // rows m .. m + run - 1 lie at out_row(m) + j * ncols(): the rest of the
  // pixel (all rows with stride 1)
  __device__ int row_run(const Ctx&, int m) const {
    if (sh == 1 && sw == 1) return 1 << 30;
    return N - (m - (int)fdiv((unsigned)m, dN) * N);
  }
  __device__ float* out_row(const Ctx& c, int, int m) const {
    if (m >= c.M) return nullptr;
    return dx + out_index(c, m) * Cin;
  }
  // row of dX [H][W][N] that row m of class c is
  __device__ long long out_index(const Ctx& c, int m) const {
    if (sh == 1 && sw == 1) return m;  // one class: rows in dX order
    const int pix = (int)fdiv((unsigned)m, dN), n = m - pix * N;
    const int hq = (int)fdiv((unsigned)pix, c.dwc), wq = pix - hq * c.Wc;
    const int h = hq * sh + c.ph_c, w = wq * sw + c.pw_c;
    return ((long long)h * W + w) * N + n;
  }
};

// Backward-weight on codes re-laid with runs along N: rows co (A) and
// j = (kh, kw, ci) (B); K-block (ho, wo, nb). A step takes kps N blocks
// (nb .. nb+kps-1) of one output pixel, or, when N fits one block, the
// output pixels (ho, wo) .. (ho, wo+kps-1); the last step of a pixel or row
// takes fewer. Slice z covers steps [z*steps_per_split, ...).
struct WgradProb {
  const uint8_t *dytc, *dys, *xtc, *xs;
  float* part;
  long long dytc_bytes, dys_bytes, xtc_bytes, xs_bytes;
  int N, H, W, Cin, Cout, KW, T, sh, sw, ph, pw, Ho, Wo, nNB, ncob, ncbi;
  int dyRB, xRB;
  int pair_w;          // 1: steps along wo (nNB == 1), 0: steps along nb
  int nsub;            // steps per pixel (pair_w 0) or per output row (pair_w 1)
  int total_steps, steps_per_split;
  int kps;             // K-blocks per step: 4 with half K-blocks, else 2
  int xtcb, xsb;       // bias of the activation row offsets (padding)
  int ga, gb;          // rows sharing one scale (A, B); 0: per-row scales
  FastDiv dCin, dKW;   // reciprocals of Cin and KW
  FastDiv dnsub, dWo;  // reciprocals of nsub and Wo
  int khalf;           // every K-block holds at most 16 valid codes (N <= 16)
  GridDivs grid;
  static constexpr bool kGeoA = false, kGeoB = true, kCanGroup = true;
  static constexpr bool kKMajA = false, kKMajB = false;
  static constexpr bool kQuad = true;  // four K-blocks per step with half K-blocks
  struct Ctx {};
  struct KS { int ho, wo, v; };
  __device__ Ctx ctx(int) const { return Ctx{}; }
  __device__ int rows_a(const Ctx&) const { return Cout; }
  __device__ int ncols() const { return T * Cin; }
  __device__ void steps(const Ctx&, int z, int& lo, int& hi) const {
    lo = min(total_steps, z * steps_per_split); hi = min(total_steps, lo + steps_per_split);
  }
  __device__ KS kstart(const Ctx&, int s) const {
    KS k;
    const int u = (int)fdiv((unsigned)s, dnsub);
    if (pair_w) { k.ho = u; k.wo = kps * (s - u * nsub); k.v = 0; }
    else { k.v = kps * (s - u * nsub); k.ho = (int)fdiv((unsigned)u, dWo); k.wo = u - k.ho * Wo; }
    return k;
  }
  __device__ int nvalid(const Ctx&, const KS& k) const { return min(kps, pair_w ? Wo - k.wo : nNB - k.v); }
  __device__ PairDelta pd_a() const {
    return pair_w ? PairDelta{Cout * nNB * dyRB, nNB * ncob, 0, 0} : PairDelta{dyRB, ncob, 0, 0};
  }
  __device__ PairDelta pd_b() const {
    return pair_w ? PairDelta{sw * Cin * nNB * xRB, sw * nNB * ncbi, 0, sw} : PairDelta{xRB, ncbi, 0, 0};
  }
  __device__ RowInfo row_a(const Ctx&, int m) const {
    RowInfo r; r.ok = m < Cout; const int co = r.ok ? m : 0;
    r.code = co * nNB * dyRB; r.scale = co / 32; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_a(const Ctx&, const KS& k) const {
    const int pix = k.ho * Wo + k.wo;
    return KInfo{(pix * Cout * nNB + k.v) * dyRB, (pix * nNB + k.v) * ncob, 0, 0};
  }
  __device__ RowInfo row_b(const Ctx&, int j) const {
    RowInfo r; r.ok = j < T * Cin; const int jj = r.ok ? j : 0;
    const int tap = (int)fdiv((unsigned)jj, dCin), ci = jj - tap * Cin;
    const int kh = (int)fdiv((unsigned)tap, dKW), kw = tap - kh * KW;
    r.p0 = kh - ph; r.p1 = kw - pw;
    const int p = r.p0 * W + r.p1;
    r.code = (p * Cin + ci) * nNB * xRB + xtcb; r.scale = p * nNB * ncbi + ci / 32 + xsb; return r;
  }
  __device__ KInfo k_b(const Ctx&, const KS& k) const {
    const int g0 = k.ho * sh, g1 = k.wo * sw, d = g0 * W + g1;
    return KInfo{(d * Cin * nNB + k.v) * xRB, (d * nNB + k.v) * ncbi, g0, g1};
  }
  __device__ int lim_a0() const { return 1; }
  __device__ int lim_a1() const { return 1; }
  __device__ int lim_b0() const { return H; }
  __device__ int lim_b1() const { return W; }
  __device__ GRange g_range_a(const Ctx&) const { return GRange{0, 0, 0, 0}; }
  __device__ GRange g_range_b(const Ctx&) const { return GRange{0, (Ho - 1) * sh, 0, (Wo - 1) * sw}; }
  __device__ bool step_interior_a(const Ctx&, const KS&) const { return true; }
  // every tap of every row in range for this step (all its pixels along wo)
  __device__ bool step_interior_b(const Ctx&, const KS& k) const {
    const int h0 = k.ho * sh - ph, w0 = k.wo * sw - pw, w1 = w0 + (pair_w ? (kps - 1) * sw : 0);
    return (h0 >= 0) & (h0 + T / KW - 1 < H) & (w0 >= 0) & (w1 + KW - 1 < W);
  }
  __device__ int row_run(const Ctx&, int) const { return 1 << 30; }
  __device__ float* out_row(const Ctx&, int z, int m) const {
    return m < Cout ? part + ((long long)z * Cout + m) * ((long long)T * Cin) : nullptr;
  }
};

// Plain GEMM out[m][c] = sum_kb A[m][kb] . B[c][kb] over packed rows whose
// runs already follow the contraction (used by the naive comparison path).
// Slice z covers K-block pairs [z*pairs_per_split, (z+1)*pairs_per_split)
// and writes its partial product to out + z*Ma*Nb.
struct PlainProb {
  const uint8_t *ac, *as, *bc, *bs;
  float* out;
  long long ac_bytes, as_bytes, bc_bytes, bs_bytes;
  int Ma, Nb, nkb, aRB, bRB, pairs_per_split, arb, brb;
  int ga = 0, gb = 0;
  GridDivs grid;
  static constexpr bool kGeoA = false, kGeoB = false, kCanGroup = false;
  static constexpr bool kKMajA = false, kKMajB = false;
  static constexpr bool kQuad = false;
  struct Ctx {};
  struct KS { int u; };
  __device__ Ctx ctx(int) const { return Ctx{}; }
  __device__ int rows_a(const Ctx&) const { return Ma; }
  __device__ int ncols() const { return Nb; }
  __device__ void steps(const Ctx&, int z, int& lo, int& hi) const {
    const int np = (nkb + 1) / 2;
    lo = min(np, z * pairs_per_split); hi = min(np, lo + pairs_per_split);
  }
  __device__ KS kstart(const Ctx&, int s) const { return KS{2 * s}; }
  __device__ int nvalid(const Ctx&, const KS& k) const { return k.u + 1 >= nkb ? 1 : 2; }
  __device__ PairDelta pd_a() const { return PairDelta{aRB, 1, 0, 0}; }
  __device__ PairDelta pd_b() const { return PairDelta{bRB, 1, 0, 0}; }
  __device__ RowInfo row_a(const Ctx&, int m) const {
    RowInfo r; r.ok = m < Ma; const int mm = r.ok ? m : 0;
    r.code = mm * arb; r.scale = mm * nkb; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_a(const Ctx&, const KS& k) const { return KInfo{k.u * aRB, k.u, 0, 0}; }
  __device__ RowInfo row_b(const Ctx&, int c) const {
    RowInfo r; r.ok = c < Nb; const int cc = r.ok ? c : 0;
    r.code = cc * brb; r.scale = cc * nkb; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_b(const Ctx&, const KS& k) const { return KInfo{k.u * bRB, k.u, 0, 0}; }
  __device__ int lim_a0() const { return 1; }
  __device__ int lim_a1() const { return 1; }
  __device__ int lim_b0() const { return 1; }
  __device__ int lim_b1() const { return 1; }
  __device__ GRange g_range_a(const Ctx&) const { return GRange{0, 0, 0, 0}; }
  __device__ GRange g_range_b(const Ctx&) const { return GRange{0, 0, 0, 0}; }
  __device__ bool step_interior_a(const Ctx&, const KS&) const { return true; }
  __device__ bool step_interior_b(const Ctx&, const KS&) const { return true; }
  __device__ int row_run(const Ctx&, int) const { return 1 << 30; }
  __device__ float* out_row(const Ctx&, int z, int m) const {
    return m < Ma ? out + ((long long)z * Ma + m) * Nb : nullptr;
  }
};

// Backward-data reading the weight codes where quantization left them
// ([Cout][Kh][Kw][Cin], runs along Cin): the B operand (rows ci, K = co of
// one tap) is staged K-major, one line of Cin codes per co. wtc, wtc_bytes
// and wRB are unused; wrb is the weight row bytes (Cin padded to 32).
// Lines past Cout lie past the end of the buffer and read zeros.
struct DgradNatProb : DgradProb {
  int T, wrb;
  static constexpr bool kKMajA = false, kKMajB = true;
  __device__ int kext_b() const { return 32; }
  __device__ int kstride_b() const { return T * wrb; }
  __device__ PairDelta pd_b() const { return PairDelta{32 * T * wrb, ncbi, 0, 0}; }
  __device__ RowInfo row_b(const Ctx&, int c) const {
    RowInfo r; r.ok = c < Cin; const int cc = r.ok ? c : 0;
    r.code = cc; r.scale = cc / 32; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_b(const Ctx& c, const KS& k) const {
    const int tap = (c.kh0 + sh * k.ih) * KW + (c.kw0 + sw * k.iw);
    return KInfo{(32 * k.v * T + tap) * wrb, (tap * ncob + k.v) * ncbi, 0, 0};
  }
};

// Backward-weight reading the gradient and activation codes where
// quantization left them ([H][W][N][C], runs along C): both operands (rows
// co, and j = (kh, kw, ci)) are staged K-major, one line of channel codes
// per n. dytc / xtc point at the natural codes with dyrb / xrb row bytes;
// dyRB and xRB are unused. Needs Cin % 16 == 0 (a 16-row chunk of B stays in
// one tap) and N <= 32 or N % 32 == 0 (a K-block's lines are N values of one
// pixel; lines past N, when N < 32, read zeros).
struct WgradNatProb : WgradProb {
  int dyrb, xrb;
  int xbits;  // bits per activation code (8; 6 or 4 in WgradNatSubProb)
  static constexpr bool kKMajA = true, kKMajB = true;
  __device__ int kext_a() const { return N < 32 ? N : 32; }
  __device__ int kext_b() const { return N < 32 ? N : 32; }
  __device__ int kstride_a() const { return dyrb; }
  __device__ int kstride_b() const { return xrb; }
  __device__ PairDelta pd_a() const {
    return pair_w ? PairDelta{N * dyrb, nNB * ncob, 0, 0} : PairDelta{32 * dyrb, ncob, 0, 0};
  }
  __device__ PairDelta pd_b() const {
    return pair_w ? PairDelta{sw * N * xrb, sw * nNB * ncbi, 0, sw} : PairDelta{32 * xrb, ncbi, 0, 0};
  }
  __device__ RowInfo row_a(const Ctx&, int m) const {
    RowInfo r; r.ok = m < Cout; const int co = r.ok ? m : 0;
    r.code = co; r.scale = co / 32; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_a(const Ctx&, const KS& k) const {
    const int pix = k.ho * Wo + k.wo;
    return KInfo{(pix * N + 32 * k.v) * dyrb, (pix * nNB + k.v) * ncob, 0, 0};
  }
  __device__ RowInfo row_b(const Ctx&, int j) const {
    RowInfo r; r.ok = j < T * Cin; const int jj = r.ok ? j : 0;
    const int tap = (int)fdiv((unsigned)jj, dCin), ci = jj - tap * Cin;
    const int kh = (int)fdiv((unsigned)tap, dKW), kw = tap - kh * KW;
    r.p0 = kh - ph; r.p1 = kw - pw;
    const int p = r.p0 * W + r.p1;
    r.code = p * N * xrb + ((ci * xbits) >> 3) + xtcb; r.scale = p * nNB * ncbi + ci / 32 + xsb; return r;
  }
  __device__ KInfo k_b(const Ctx&, const KS& k) const {
    const int g0 = k.ho * sh, g1 = k.wo * sw, d = g0 * W + g1;
    return KInfo{(d * N + 32 * k.v) * xrb, (d * nNB + k.v) * ncbi, g0, g1};
  }
};

// Backward-weight reading the 8-bit gradient codes and 6- or 4-bit
// activation codes both where quantization left them: as WgradNatProb, with
// the activation's 16-channel chunks (12 or 8 code bytes) staged one per
// 16-byte LDS slot and read with the 6/4-bit transposing LDS reads
// (lds_operand_k_sub). Needs Cin % 16 == 0 (chunk offsets ci * bits / 8 stay
// whole bytes and a chunk stays in one tap); never half K-blocks.
struct WgradNatSubProb : WgradNatProb {
  static constexpr bool kSubB = true;
};

// Backward-weight with the 8-bit gradient codes read where quantization
// left them (A staged K-major, as in WgradNatProb) and 6- or 4-bit
// activation codes re-laid with runs along N (B as in WgradProb). dytc
// points at the natural gradient codes with dyrb row bytes.
struct WgradMixProb : WgradProb {
  int dyrb;
  static constexpr bool kKMajA = true, kKMajB = false;
  __device__ int kext_a() const { return N < 32 ? N : 32; }
  __device__ int kstride_a() const { return dyrb; }
  __device__ PairDelta pd_a() const {
    return pair_w ? PairDelta{N * dyrb, nNB * ncob, 0, 0} : PairDelta{32 * dyrb, ncob, 0, 0};
  }
  __device__ RowInfo row_a(const Ctx&, int m) const {
    RowInfo r; r.ok = m < Cout; const int co = r.ok ? m : 0;
    r.code = co; r.scale = co / 32; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_a(const Ctx&, const KS& k) const {
    const int pix = k.ho * Wo + k.wo;
    return KInfo{(pix * N + 32 * k.v) * dyrb, (pix * nNB + k.v) * ncob, 0, 0};
  }
};

// Buffers of each problem: (A codes, A scales, B codes, B scales).
__device__ inline void rsrcs(const FwdProb& p, __amdgpu_buffer_rsrc_t (&r)[4]) {
  r[0] = make_rsrc(p.xc - p.xcb, p.xc_bytes + p.xcb); r[1] = make_rsrc(p.xs - p.xsb, p.xs_bytes + p.xsb);
  r[2] = make_rsrc(p.wc, p.wc_bytes); r[3] = make_rsrc(p.ws, p.ws_bytes);
}
__device__ inline void rsrcs(const DgradProb& p, __amdgpu_buffer_rsrc_t (&r)[4]) {
  r[0] = make_rsrc(p.dyc - p.dycb, p.dyc_bytes + p.dycb); r[1] = make_rsrc(p.dys - p.dysb, p.dys_bytes + p.dysb);
  r[2] = make_rsrc(p.wtc, p.wtc_bytes); r[3] = make_rsrc(p.ws, p.ws_bytes);
}
__device__ inline void rsrcs(const WgradProb& p, __amdgpu_buffer_rsrc_t (&r)[4]) {
  r[0] = make_rsrc(p.dytc, p.dytc_bytes); r[1] = make_rsrc(p.dys, p.dys_bytes);
  r[2] = make_rsrc(p.xtc - p.xtcb, p.xtc_bytes + p.xtcb); r[3] = make_rsrc(p.xs - p.xsb, p.xs_bytes + p.xsb);
}
__device__ inline void rsrcs(const PlainProb& p, __amdgpu_buffer_rsrc_t (&r)[4]) {
  r[0] = make_rsrc(p.ac, p.ac_bytes); r[1] = make_rsrc(p.as, p.as_bytes);
  r[2] = make_rsrc(p.bc, p.bc_bytes); r[3] = make_rsrc(p.bs, p.bs_bytes);
}

// ---------------------------------------------------------------------------
// LDS image of one operand stage
// ---------------------------------------------------------------------------
// Stage layout of a row-major operand: [row][SPR] 16-byte slots, SPR = the
// step's K-blocks x NPK slots per run (8-bit and 6-bit codes: NPK = 2, the
// 6-bit ones carrying 12 code bytes each; 4-bit codes and half K-blocks: 1).
// A 64-lane load that writes LDS fills 64 consecutive slots, so it covers
// 64 / SPR whole rows, and each row's part of the step (all its K-blocks)
// comes from one stretch of memory: 64 bytes per row (8-bit, two K-blocks)
// instead of 32 per lane pair. The L1 serves loads of 64-byte pieces at
// about twice the rate of loads of 32-byte pieces (measured on MI355X: 18.7
// against 8.7 TB/s of L2-to-LDS traffic over the whole chip). Slot u of row
// r holds the row's logical slot u ^ row_swz(r) (logical slot kb * NPK +
// piece), so that the 16-byte reads of one logical slot by 8 or 16
// consecutive rows hit distinct LDS banks. Scales: one dword per (kb, row),
// [kb][row].
template <int F>
struct Op {
  static constexpr int RB = run_bytes_of(F);
  static constexpr int NPK = RB == 16 ? 1 : 2;   // slots per run
  static constexpr int CH = RB == 24 ? 12 : 16;  // code bytes per slot
};
template <int SPR>
__device__ __forceinline__ int row_swz(int r) {
  static_assert(SPR == 2 || SPR == 4, "slots per row");
  if constexpr (SPR == 2) return ((r >> 2) ^ (r >> 3)) & 1;
  else return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1);
}
// LDS code reads per 32x32x64 operand image
template <int F>
constexpr int F_READS() { return F <= 3 ? 2 : 1; }

// Reads one 32x32x64 operand register image (see mx_common.h) of row `row`,
// pair p of the step (K-blocks 2p and 2p+1), from a row-major stage with SPR
// slots per row; h = row_swz(row).
template <int F, int SPR>
__device__ __forceinline__ v8i lds_operand(const uint8_t* op, int row, int h, int p, int q) {
  const uint8_t* const base = op + row * SPR * 16;
  auto slot = [&](int L) { return *reinterpret_cast<const v4i*>(base + 16 * (L ^ h)); };
  v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (F <= 1) {
    // bytes 0..15: K-block 2p, piece q; bytes 16..31: K-block 2p+1, piece q
    const v4i lo = slot(4 * p + q), hi = slot(4 * p + 2 + q);
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3]; r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  } else if constexpr (F <= 3) {
    // the 24-byte run of K-block 2p+q: 12 bytes from each of its two slots
    const int kb = 2 * p + q;
    const v4i lo = slot(2 * kb), hi = slot(2 * kb + 1);
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = hi[0]; r[4] = hi[1]; r[5] = hi[2];
  } else {
    // the 16-byte run of K-block 2p+q
    const v4i x = slot(2 * p + q);
    r[0] = x[0]; r[1] = x[1]; r[2] = x[2]; r[3] = x[3];
  }
  return r;
}

// Operand image of an 8-bit row from a stage that holds only the first 16
// codes of each run (one slot per K-block), for K-blocks with at most 16
// valid codes: lanes of the upper half (q = 1) read a 16-byte zero slot.
template <int SPR>
__device__ __forceinline__ v8i lds_operand_half(const uint8_t* op, const uint8_t* zero, int row, int h, int p, int q) {
  const uint8_t* const base = op + row * SPR * 16;
  const v4i lo = *reinterpret_cast<const v4i*>(q ? zero : base + 16 * ((2 * p) ^ h));
  const v4i hi = *reinterpret_cast<const v4i*>(q ? zero : base + 16 * ((2 * p + 1) ^ h));
  v8i r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return r;
}

// K-major stage of an 8-bit operand with BR rows: [kb][k][BR] bytes, one
// line of BR codes per K index k (the operand's rows side by side, as they
// lie in memory when the contraction runs along the partner or the tap
// dimension). Its 16-byte chunks (CPR = BR / 16 per line) are permuted
// within aligned groups by kswz, so that the transposing reads below hit
// distinct LDS banks (a 16-byte slot covers 4 of the 64 banks; two lines
// of 128 bytes cover all of them):
//   8-bit codes, CPR a multiple of 8: 2 * ((k >> 1) & 3) in groups of 8 --
//     the 32 lanes of a ds_read_b64_tr_b8 read 8 lines of two neighbouring
//     chunks, which then sit in 16 different bank groups;
//   6/4-bit codes, CPR a multiple of 8: (k >> 1) & 7 -- a 16-lane group of
//     ds_read_b96_tr_b6 / ds_read_b64_tr_b4 reads 16 lines of one chunk;
//   otherwise (k >> 1) & 3 in groups of 4.
template <bool SUB, int CPR>
__device__ __forceinline__ int kswz(int k) {
  if constexpr (CPR % 8 != 0) return (k >> 1) & 3;
  else if constexpr (SUB) return (k >> 1) & 7;
  else return ((k >> 1) & 3) << 1;
}
// Operand image of rows r0..r0+31 from a K-major stage with ds_read_b64_tr_b8:
// in each 16-lane group, lanes 2i and 2i+1 address the two halves of the
// 16-byte chunk of line k0+i that holds the group's 16 rows, and lane t
// receives lines k0..k0+7 of row t. Lane (r, q) gets K indices 16q..16q+15
// of both K-blocks: four such reads. HALF: the stage holds 16 lines per
// K-block (K-blocks of at most 16 values); the upper lanes (q = 1) repeat the
// lower lanes' reads, and with ZQ1 their image is then zeroed. A product of
// the upper K halves vanishes when one of the two operands is zero there
// (codes are always finite), so only one operand needs ZQ1.
template <int BR, bool HALF, bool ZQ1>
__device__ __forceinline__ v8i lds_operand_k(const uint8_t* stage, int r0, int lane) {
  typedef v2i __attribute__((address_space(3)))* lds_v2i_ptr;
  constexpr int KL = HALF ? 16 : 32;  // lines per K-block
  const int g = lane >> 4, t = lane & 15, q = HALF ? 0 : g >> 1;
  const int chunk = (r0 >> 4) + (g & 1);
  // k = 16q + 8h + t/2, so kswz(k) = kswz(t/2) for every read
  const uint8_t* base = stage + (16 * q + (t >> 1)) * BR + 16 * (chunk ^ kswz<false, BR / 16>(t >> 1)) + 8 * (t & 1);
  v8i r;
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_ptr)(base + (kb * KL + 8 * h) * BR));
      r[4 * kb + 2 * h] = x[0];
      r[4 * kb + 2 * h + 1] = x[1];
    }
  if constexpr (HALF && ZQ1) {
    const bool upper = lane >= 32;
#pragma unroll
    for (int e = 0; e < 8; e++) r[e] = upper ? 0 : r[e];
  }
  return r;
}

// Operand image of rows r0..r0+31 from a K-major stage of 6- or 4-bit codes:
// the stage is laid out as for 8-bit codes ([kb][k][BR / 16 slots of 16
// bytes], slots permuted by kswz(k)), but slot c of line k holds the 12
// (6-bit) or 8 (4-bit) code bytes of the line's 16-row chunk c, copied with
// the bytes after them. The image is the packed 32-code run of K-block q
// (dwords 0-5 for 6-bit, 0-3 for 4-bit): lane t of each 16-lane group
// addresses line 16h + t of K-block q in the slot of the group's rows
// (16-byte aligned, as ds_read_b96_tr_b6 needs), and
// ds_read_b96_tr_b6 / ds_read_b64_tr_b4 hand lane t its row's 16 values on
// those lines, line j at bits [bits*j, bits*(j+1)).
template <int F, int BR>
__device__ __forceinline__ v8i lds_operand_k_sub(const uint8_t* stage, int r0, int lane) {
  static_assert(Fmt<F>::bits == 6 || Fmt<F>::bits == 4, "6- or 4-bit codes");
  typedef v2i __attribute__((address_space(3)))* lds_v2i_ptr;
  typedef int v3i_t __attribute__((ext_vector_type(3)));
  typedef v3i_t __attribute__((address_space(3)))* lds_v3i_ptr;
  const int g = lane >> 4, t = lane & 15, q = g >> 1;
  const int chunk = (r0 >> 4) + (g & 1);
  v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int k = 16 * h + t;  // line within K-block q
    const uint8_t* src = stage + (32 * q + k) * BR + 16 * (chunk ^ kswz<true, BR / 16>(k));
    if constexpr (Fmt<F>::bits == 6) {
      const v3i_t x = __builtin_amdgcn_ds_read_tr6_b96_v3i32((lds_v3i_ptr)src);
      r[3 * h] = x[0]; r[3 * h + 1] = x[1]; r[3 * h + 2] = x[2];
    } else {
      const v2i x = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_v2i_ptr)src);
      r[2 * h] = x[0]; r[2 * h + 1] = x[1];
    }
  }
  return r;
}

// Per-lane part of one LDS-writing load: byte offset of the lane's piece
// relative to the step's uniform offset (kOOB when the row is outside the
// problem or the load only keeps the count uniform), the row's border
// coordinates for the piece's K-block, and that K-block within the step
// (row-major code loads; 0 for the others).
struct LaneLd { int off, p0, p1, kb; };

typedef __attribute__((address_space(3))) void* lds_ptr_t;
// 16 bytes per lane into LDS at lds + 16*lane, from voff + soff
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}
// one byte per lane, zero-extended into the dword at lds + 4*lane
__device__ __forceinline__ void dma1(__amdgpu_buffer_rsrc_t r, uint8_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 1, voff, soff, 0, 0);
}
// s_waitcnt with vmcnt(N) and lgkmcnt(0) (expcnt not waited)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// Workgroup barrier without a memory fence: the waits that complete an LDS
// stage are explicit (wait_vm_lgkm0), and the empty asm statements keep the
// compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// WM x WN waves; each wave owns TM x TN MFMA tiles of 32 x 32; NS LDS stages.
// GS: grouped scales. When every run of prob.ga rows of A (prob.gb of B)
// shares one scale (a 32 x 32 block, or a whole pixel's N < 32 rows), a stage
// holds one scale per (K-block, group) instead of per (K-block, row), and
// one 64-lane load per operand fetches them: wave 0 the A scales, wave 1 the
// B scales; waves 2 and 3 issue a zero-reading load to keep every wave's
// load count equal.
// KH: every K-block has at most 16 valid codes (8-bit formats only): a
// stage holds only the first 16-byte piece of each run, which halves it, so
// the ring can be deeper for the same LDS.
// NG: wave groups of 4 waves per workgroup; group g runs the g-th part of
// the workgroup's K range in its own ring of stages, and the groups' sums
// are added (in group order) before the epilogue, so the workgroup covers
// NG times the K range with NG times the waves.
// At least two waves per SIMD: the register budget (VGPRs + accumulation
// registers) stays within 256, so two 256x128 workgroups share a CU.
// MX epilogue of one 32-row strip (rows ms.., columns c0.. of the wave, in
// LDS with pitch EP floats): lane l takes row l/2 and the 16 channels
// (l%2)*16.. of each 32-column block; the block maximum is a cross-lane
// maximum over the lanes of the block's rows; codes and scale bytes follow
// the element rule of the quantizer (scale_clamp16, convert_store_half_run).
// FP6 converts two blocks per instruction. The codes are packed in LDS
// (cst: 32 rows of TN runs) and leave as consecutive dwords of each row
// segment (whole rows are one contiguous stretch), not as scattered half
// runs.
// LEAN (tiles whose accumulators already fill most registers): one block
// (FP6: one pair) at a time and one copy piece at a time, so the epilogue
// needs few registers.
template <int F, int TN, bool LEAN, class P>
__device__ __forceinline__ void mx_store_strip(const P& p, const typename P::Ctx& cx, const float* strip, int EP,
                                               int ms, int c0, int lane, uint8_t* cst) {
  constexpr int RB = run_bytes_of(F), SEG = TN * RB;
  constexpr bool PAIR = Fmt<F>::bits == 6 && TN % 2 == 0;
  const int r = lane >> 1, half = lane & 1;
  const int m = ms + r;
  const int M = p.rows_a(cx);
  const int cb0 = c0 >> 5;
  const int nb = min(TN, p.ynCB - cb0);  // blocks of this wave inside the padded row (uniform)
  const int glanes = p.ymode == 0 ? 2 : (p.ymode == 1 ? 64 : 2 * p.N);  // lanes of one block
  // the scale bytes of this lane's blocks, written by the first lane of each
  // block's lane group (one address per strip, not one per block)
  const bool first = p.ymode == 0 ? half == 0 : (p.ymode == 1 ? lane == 0 : (lane & (2 * p.N - 1)) == 0);
  uint8_t* srow = nullptr;
  if (first && m < M) {
    const long long gm = p.out_index(cx, m);
    const long long pix = gm / p.N, n = gm - pix * p.N;
    const long long blk = p.ymode == 0 ? gm : pix * p.ynPB + (n >> 5);
    srow = p.ys + blk * p.ynCB + cb0;
  }
  typedef float v4f __attribute__((ext_vector_type(4)));
  // block j: this lane's 16 values scaled and clamped into v; returns the
  // block's scale byte (already stored)
  auto block = [&](int j, float (&v)[16]) -> uint32_t {
    float x[16];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const v4f t = *reinterpret_cast<const v4f*>(strip + r * EP + j * 32 + half * 16 + 4 * k);
      x[4 * k] = t[0]; x[4 * k + 1] = t[1]; x[4 * k + 2] = t[2]; x[4 * k + 3] = t[3];
    }
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) a = max(a, __float_as_uint(x[i]) & 0x7fffffffu);
    a = group_max(a, glanes);
    const uint32_t S = scale_byte_from_amax<F>(a);
    scale_clamp16<F>(x, S, v);
    if (srow) srow[j] = (uint8_t)S;
    return S;
  };
  uint8_t* const crow = cst + r * SEG + half * (RB / 2);
  if constexpr (PAIR) {
#pragma unroll(LEAN ? 1 : TN / 2)
    for (int j = 0; j < TN; j += 2) {
      if (j >= nb) break;  // uniform
      float v0[16], v1[16];
      const uint32_t S0 = block(j, v0);
      if (j + 1 < nb) {
        const uint32_t S1 = block(j + 1, v1);
        convert_store_two_half_runs6<F>(crow + j * RB, crow + (j + 1) * RB, v0, v1, code_keep(S0), code_keep(S1));
      } else {
        convert_store_half_run<F>(crow + j * RB, v0, code_keep(S0));
      }
    }
  } else {
#pragma unroll(LEAN ? 1 : TN)
    for (int j = 0; j < TN; j++) {
      if (j >= nb) break;  // uniform
      float v[16];
      const uint32_t S = block(j, v);
      convert_store_half_run<F>(crow + j * RB, v, code_keep(S));
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the packed codes are in LDS (same wave)
  __builtin_amdgcn_wave_barrier();
  // row segments: nb runs of each of the 32 rows, as VW-byte pieces (every
  // run, row and segment start is a multiple of VW)
  constexpr int VW = RB % 16 == 0 ? 16 : 8;
  typedef uint32_t vw_t __attribute__((ext_vector_type(VW / 4)));
  if (nb == TN) {  // the usual case: a piece count known at compile time
    constexpr int PR = SEG / VW, IT = (32 * PR + 63) / 64;
    if constexpr (LEAN) {
#pragma unroll
      for (int it = 0; it < IT; it++) {
        const int d = it * 64 + lane, row = d / PR, off = d - row * PR;
        if (d < 32 * PR && ms + row < M)
          *reinterpret_cast<vw_t*>(p.yc + p.out_index(cx, ms + row) * p.yrb + cb0 * RB + off * VW) =
              *reinterpret_cast<const vw_t*>(cst + row * SEG + off * VW);
      }
    } else {  // all reads first, then all stores
      vw_t val[IT];
#pragma unroll
      for (int it = 0; it < IT; it++) {
        const int d = min(it * 64 + lane, 32 * PR - 1), row = d / PR, off = d - row * PR;
        val[it] = *reinterpret_cast<const vw_t*>(cst + row * SEG + off * VW);
      }
#pragma unroll
      for (int it = 0; it < IT; it++) {
        const int d = it * 64 + lane, row = d / PR, off = d - row * PR;
        if (d < 32 * PR && ms + row < M)
          *reinterpret_cast<vw_t*>(p.yc + p.out_index(cx, ms + row) * p.yrb + cb0 * RB + off * VW) = val[it];
      }
    }
  } else {
    const int pr = nb * RB / VW;
    for (int d = lane; d < 32 * pr; d += 64) {
      const int row = d / pr, off = d - row * pr;
      if (ms + row < M)
        *reinterpret_cast<vw_t*>(p.yc + p.out_index(cx, ms + row) * p.yrb + cb0 * RB + off * VW) =
            *reinterpret_cast<const vw_t*>(cst + row * SEG + off * VW);
    }
  }
}

// The backward-data GEMM with fp32 output on its 256 x 128 tile runs
// persistent workgroups: as many as fit on the chip, each looping over
// tiles. Launched one per tile, the short-lived workgroups of the
// backward-data left the chip at 1.7 of the 3 workgroups per compute unit
// that fit its 128 x 128 tile (SQ_WAVE_CYCLES over the kernel's duration on
// the stride-2 layer, N 32, 128 -> 256 channels, 160 x 160); persistent, the
// 256 x 128 tile (two per CU, a quarter fewer operand bytes per FLOP through
// LDS) is the faster of the two.
template <class P, int WM, int WN, int TM, int TN, int NS>
constexpr bool gemm_persistent() {
  return std::is_base_of<DgradProb, P>::value && !MxOut<P>::value && WM == 2 && WN == 2 && TM == 4 && TN == 2 &&
         NS == 3;
}

template <int FA, int FB, class P, int WM, int WN, int TM, int TN, int NS, bool GS, bool KH, int KPS, int NG>
__global__ __launch_bounds__(256 * NG) __attribute__((amdgpu_waves_per_eu(2))) void mx_gemm_kernel(P prob) {
  static_assert(!KH || (FA <= 1 && FB <= 1), "half K-blocks only for 8-bit codes");
  // K-major operands (8-bit codes; 6/4-bit B codes without half K-blocks):
  // the staging order of the contraction's natural layout, read back with
  // transposing LDS reads
  constexpr bool TA = P::kKMajA, TB = P::kKMajB;
  static_assert(!TA || FA <= 1, "K-major A: 8-bit codes");
  static_assert(!TB || FB <= 1 || (SubB<P>::value && !KH), "K-major 6/4-bit B: its own problem, full K-blocks");
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  using OA = Op<FA>;
  using OB = Op<FB>;
  // KPS: K-blocks per step (a pair, or two pairs)
  static_assert(KPS == 2 || KPS == 4, "K-blocks per step");
  // 16-byte slots per row (row-major) or per 16-row chunk and 16 lines
  // (K-major: KL lines of BR bytes per K-block, whatever the code width)
  constexpr int NPKA = TA ? (KH ? 1 : 2) : (KH ? 1 : OA::NPK), NPKB = TB ? (KH ? 1 : 2) : (KH ? 1 : OB::NPK);
  constexpr int A_BYTES = KPS * BM * NPKA * 16, B_BYTES = KPS * BN * NPKB * 16;
  // slots per row of a row-major stage (K-major stages: unused)
  constexpr int SPRA = TA ? 2 : KPS * NPKA, SPRB = TB ? 2 : KPS * NPKB;
  constexpr int SA_BYTES = GS ? 256 : 4 * KPS * BM, SB_BYTES = GS ? 256 : 4 * KPS * BN;
  constexpr int OFF_B = A_BYTES, OFF_SA = OFF_B + B_BYTES, OFF_SB = OFF_SA + SA_BYTES;
  constexpr int STAGE = OFF_SB + SB_BYTES;
  // LDS-writing loads (64 lanes each) per stage and per wave; load g of a
  // kind belongs to K-block g / (loads per K-block)
  constexpr int NCA = KPS * BM * NPKA / 64, NCB = KPS * BN * NPKB / 64;
  constexpr int NSA = GS ? 1 : KPS * BM / 64, NSB = GS ? 1 : KPS * BN / 64;
  constexpr int WCA = (NCA + 3) / 4, WCB = (NCB + 3) / 4;
  constexpr int WSA = GS ? 1 : (NSA + 3) / 4, WSB = GS ? 0 : (NSB + 3) / 4;
  constexpr int WPS = WCA + WCB + WSA + WSB;
  // 1 KB sink for the loads a wave issues only to keep its count uniform
  constexpr int DUMMY = NG * NS * STAGE;
  constexpr int ZERO = DUMMY + 1024;  // KH: 16 zero bytes for the empty upper pieces
  constexpr int STRIP = 32 * (TN * 32 + 8) * 4;  // one wave's epilogue strip (bytes)
  constexpr int XCH = NG > 1 ? 4 * TM * TN * 16 * 64 * 4 : 0;  // group 1's accumulators
  // MX output: each wave packs a strip's codes (32 rows x TN runs) after the strips
  constexpr int CST = MxOut<P>::value ? 32 * TN * 32 : 0;
  constexpr int EPI = XCH > 4 * (STRIP + CST) ? XCH : 4 * (STRIP + CST);
  constexpr int ARENA = (ZERO + 16) > EPI ? (ZERO + 16) : EPI;
  __shared__ __attribute__((aligned(16))) uint8_t arena[ARENA];

  // XCD-aware tile order: the hardware hands consecutive workgroups to the 8
  // XCDs in turn, each with its own L2. Remap so that every XCD works on a
  // contiguous range of tiles (column tiles fastest, then row tiles):
  // neighbouring row tiles share the weight tile and the rows of the
  // implicit im2col, and now share an L2.
  // Persistent launch (prob.grid.gx > 0 workgroups per XCD, as many as fit
  // on the chip at once): workgroup j of an XCD takes, at its k-th pass,
  // local tile k*gx + (j + k) % gx, so a pass of the XCD's workgroups covers
  // gx consecutive tiles (the same L2 locality as one tile per workgroup)
  // and, with gx a multiple of the class count, each workgroup cycles
  // through the backward-data parity classes (whose K lengths differ).
  // (only the persistent backward-data tile is built with the loop; every
  // other kernel takes one tile and compiles as straight-line code)
  constexpr bool PERSIST = gemm_persistent<P, WM, WN, TM, TN, NS>();
  const int tnx = prob.grid.tx, tny = prob.grid.ty, tnz = prob.grid.tz, gx = PERSIST ? prob.grid.gx : 0;
  const int nb = tnx * tny * tnz;
  const int hw = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int xcd = hw % 8, jx = hw / 8, q8 = nb / 8, r8 = nb % 8;
  const int n_x = xcd < r8 ? q8 + 1 : q8;  // tiles of this XCD
  const int lo_x = xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8;
  for (int pass = 0; gx > 0 ? pass * gx < n_x : pass == 0; pass++) {
  const int u = gx > 0 ? pass * gx + (jx + pass) % gx : jx;
  if (u >= n_x) continue;  // (uniform)
  // the previous tile's epilogue may still read LDS that this tile's first
  // loads write
  if (pass > 0) stage_barrier();
  // The thread index passes through an empty asm each pass, so nothing
  // computed from it is hoisted out of the tile loop (values kept live
  // across the whole loop would exceed the register budget).
  int tid = threadIdx.x;
  if constexpr (PERSIST) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int grp = __builtin_amdgcn_readfirstlane(tid >> 8);          // wave group
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);   // wave within the group
  const int wm = wave % WM, wn = wave / WM;
  uint8_t* const ring = arena + grp * NS * STAGE;  // this group's stages
  int bx, by, z;
  {
    const int logical = lo_x + u;
    int rem;
    if constexpr (std::is_base_of<DgradProb, P>::value) {
      // backward-data: the stride-parity classes of one tile position run
      // side by side (they read the same dY rows through different taps)
      rem = logical / tnz;
      z = logical - rem * tnz;
    } else {
      z = (int)fdiv((unsigned)logical, prob.grid.nxy);
      rem = logical - z * tnx * tny;
    }
    // column tiles fastest: the column tiles of one row tile read the same
    // A rows, now from the same XCD's L2
    bx = rem / tny;
    by = rem - bx * tny;
  }
  const typename P::Ctx cx = prob.ctx(z);
  const int m0 = bx * BM, n0 = by * BN;
  if (m0 >= prob.rows_a(cx)) continue;  // whole tile beyond this class's rows (uniform)
  __amdgpu_buffer_rsrc_t rs[4];
  rsrcs(prob, rs);
  const PairDelta dA = prob.pd_a(), dB = prob.pd_b();
  const int la0 = prob.lim_a0(), la1 = prob.lim_a1(), lb0 = prob.lim_b0(), lb1 = prob.lim_b1();
  const GRange gA = prob.g_range_a(cx), gB = prob.g_range_b(cx);

  // Per-lane load descriptors. `inner` collects whether all of this wave's
  // rows stay inside the borders for every step of the problem.
  LaneLd ca[WCA], cb[WCB], sa[WSA], sb[WSB > 0 ? WSB : 1];
  bool innerA = true, innerB = true;
  // per-row scales: load g fills scale dwords [kb][row], 64 rows at a time
  auto make_lane_s = [&](LaneLd& l, int g, int ngl, int per_kb, bool is_a, bool& inner) {
    const bool real = g < ngl;
    const int kb = real ? (64 * g) / per_kb : 0;
    const int row = real ? 64 * g + lane - kb * per_kb : 0;
    const PairDelta& d = is_a ? dA : dB;
    const RowInfo r = is_a ? prob.row_a(cx, m0 + row) : prob.row_b(cx, n0 + row);
    const bool ok = r.ok & real;
    l.off = ok ? r.scale + kb * d.scale : kOOB;
    l.p0 = r.p0 + kb * d.g0;
    l.p1 = r.p1 + kb * d.g1;
    l.kb = 0;
    const GRange& gr = is_a ? gA : gB;
    const int L0 = is_a ? la0 : lb0, L1 = is_a ? la1 : lb1;
    inner = inner & (!ok | ((l.p0 + gr.min0 >= 0) & (l.p0 + gr.max0 < L0) & (l.p1 + gr.min1 >= 0) &
                            (l.p1 + gr.max1 < L1)));
  };
  // row-major codes: load g covers rows g * 64 / SPR .. of the [row][SPR]
  // stage; lane t writes physical slot u = t % SPR of its row, which holds
  // logical slot u ^ row_swz(row): K-block L / np, piece L % np
  auto make_lane_r = [&](LaneLd& l, int g, int ngl, auto SPRc, int np, int ch, bool is_a, bool& inner) {
    constexpr int SPR = decltype(SPRc)::value;
    const bool real = g < ngl;
    const int row = real ? g * (64 / SPR) + lane / SPR : 0;
    const int L = (lane % SPR) ^ row_swz<SPR>(row);
    const int kb = L / np, piece = L - kb * np;
    const PairDelta& d = is_a ? dA : dB;
    const RowInfo r = is_a ? prob.row_a(cx, m0 + row) : prob.row_b(cx, n0 + row);
    const bool ok = r.ok & real;
    l.off = ok ? r.code + piece * ch + kb * d.code : kOOB;
    l.p0 = r.p0 + kb * d.g0;
    l.p1 = r.p1 + kb * d.g1;
    l.kb = kb;
    const GRange& gr = is_a ? gA : gB;
    const int L0 = is_a ? la0 : lb0, L1 = is_a ? la1 : lb1;
    inner = inner & (!ok | ((l.p0 + gr.min0 >= 0) & (l.p0 + gr.max0 < L0) & (l.p1 + gr.min1 >= 0) &
                            (l.p1 + gr.max1 < L1)));
  };
  // K-major: slot t of the operand's stage holds K-block kb = t / (KL BR / 16),
  // line k and chunk c (rows 16c..16c+15), the chunk permuted by kswz(k);
  // KL = 32 lines per K-block (16 with KH); lines past the operand's K
  // extent read zeros
  auto make_lane_k = [&](LaneLd& l, int g, int ngl, auto BRc, auto IsA, bool& inner, const auto& pr) {
    constexpr int BR = decltype(BRc)::value, CPR = BR / 16, KBS = (KH ? 16 : 32) * CPR;
    constexpr bool is_a = decltype(IsA)::value;
    const bool real = g < ngl;
    const int t = real ? 64 * g + lane : 0;
    const int kb = t / KBS, u = t - kb * KBS;
    constexpr bool SUB = (is_a ? FA : FB) >= 2;
    const int k = u / CPR, chunk = (u - k * CPR) ^ kswz<SUB, CPR>(k);
    const PairDelta& d = is_a ? dA : dB;
    RowInfo r;
    int kext, ks;
    if constexpr (is_a) {
      r = pr.row_a(cx, m0 + 16 * chunk); kext = pr.kext_a(); ks = pr.kstride_a();
    } else {
      r = pr.row_b(cx, n0 + 16 * chunk); kext = pr.kext_b(); ks = pr.kstride_b();
    }
    const bool ok = r.ok & real & (k < kext);
    l.off = ok ? r.code + k * ks + kb * d.code : kOOB;
    l.p0 = r.p0 + kb * d.g0;
    l.p1 = r.p1 + kb * d.g1;
    l.kb = 0;
    const GRange& gr = is_a ? gA : gB;
    const int L0 = is_a ? la0 : lb0, L1 = is_a ? la1 : lb1;
    inner = inner & (!ok | ((l.p0 + gr.min0 >= 0) & (l.p0 + gr.max0 < L0) & (l.p1 + gr.min1 >= 0) &
                            (l.p1 + gr.max1 < L1)));
  };
#pragma unroll
  for (int k = 0; k < WCA; k++) {
    if constexpr (TA)
      make_lane_k(ca[k], wave + 4 * k, NCA, std::integral_constant<int, BM>{}, std::true_type{}, innerA, prob);
    else make_lane_r(ca[k], wave + 4 * k, NCA, std::integral_constant<int, SPRA>{}, NPKA, OA::CH, true, innerA);
  }
#pragma unroll
  for (int k = 0; k < WCB; k++) {
    if constexpr (TB)
      make_lane_k(cb[k], wave + 4 * k, NCB, std::integral_constant<int, BN>{}, std::false_type{}, innerB, prob);
    else make_lane_r(cb[k], wave + 4 * k, NCB, std::integral_constant<int, SPRB>{}, NPKB, OB::CH, false, innerB);
  }
  // grouped scales: lane e of wave 0 (A) or wave 1 (B) loads the scale of
  // group e % ngroups of K-block e / ngroups (e < KPS * ngroups <= 64)
  const int gsa = GS ? prob.ga : 1, gsb = GS ? prob.gb : 1;
  int s_kb = 0;  // K-block of this lane's grouped-scale load
  if constexpr (GS) {
    const bool isA = wave == 0, isB = wave == 1;
    const int rows = isA ? BM : BN, grp = isA ? gsa : gsb;
    const int ng = rows / grp;
    const bool real = (isA | isB) & (lane < KPS * ng);
    const int kb = real ? lane / ng : 0, row = real ? (lane - kb * ng) * grp : 0;
    const PairDelta& d = isA ? dA : dB;
    const RowInfo r = isA ? prob.row_a(cx, m0 + row) : prob.row_b(cx, n0 + row);
    const bool ok = r.ok & real;
    sa[0].off = ok ? r.scale + kb * d.scale : kOOB;
    sa[0].p0 = r.p0 + kb * d.g0;
    sa[0].p1 = r.p1 + kb * d.g1;
    sa[0].kb = 0;
    s_kb = kb;
    const GRange& gr = isA ? gA : gB;
    const int L0 = isA ? la0 : lb0, L1 = isA ? la1 : lb1;
    const bool inner = !ok | ((sa[0].p0 + gr.min0 >= 0) & (sa[0].p0 + gr.max0 < L0) & (sa[0].p1 + gr.min1 >= 0) &
                              (sa[0].p1 + gr.max1 < L1));
    if (isA) innerA = innerA & inner;
    if (isB) innerB = innerB & inner;
  } else {
#pragma unroll
    for (int k = 0; k < WSA; k++) make_lane_s(sa[k], wave + 4 * k, NSA, BM, true, innerA);
#pragma unroll
    for (int k = 0; k < WSB; k++) make_lane_s(sb[k], wave + 4 * k, NSB, BN, false, innerB);
  }
  // wave-uniform: no lane of this wave ever needs the border test
  const bool waveA = !P::kGeoA || __builtin_amdgcn_ballot_w64(!innerA) == 0;
  const bool waveB = !P::kGeoB || __builtin_amdgcn_ballot_w64(!innerB) == 0;

  int s_lo, s_hi;
  prob.steps(cx, z, s_lo, s_hi);
  // group g takes the g-th of NG equal parts; every group runs the same
  // number of iterations (steps past its part read zeros)
  const int per_grp = (s_hi - s_lo + NG - 1) / NG;
  s_lo = s_lo + grp * per_grp;
  s_hi = min(s_hi, s_lo + per_grp);
  // Step descriptors, 64 steps at a time: lane l of every wave holds those
  // of step tb + l (its K-block offsets and flags), and a step reads its own
  // into scalar registers with v_readlane. Steps past the last repeat it
  // (their loads read zeros).
  // descriptors of step s: K-block offsets of both operands, and flags
  // (valid K-blocks, step interior for A and for B)
  struct StepD { KInfo ka, kb; int fl; };
  auto step_desc = [&](int s_any) {
    const int s = min(s_any, max(s_hi - 1, s_lo));
    const typename P::KS k = prob.kstart(cx, s);
    return StepD{prob.k_a(cx, k), prob.k_b(cx, k),
                 prob.nvalid(cx, k) | (prob.step_interior_a(cx, k) ? 8 : 0) | (prob.step_interior_b(cx, k) ? 16 : 0)};
  };
  struct Tab { int ac, as, ag0, ag1, bc, bs, bg0, bg1, fl; };
  auto fill = [&](int base) {
    const StepD d = step_desc(base + lane);
    return Tab{d.ka.code, d.ka.scale, d.ka.g0, d.ka.g1, d.kb.code, d.kb.scale, d.kb.g0, d.kb.g1, d.fl};
  };
  Tab tab;
  int tb = s_lo;
  int s_next = s_lo;

  // lane offset of a load at this step (branch-free): the border test is
  // void when the wave or the step is known to be inside
  auto voff = [&](const LaneLd& l, const KInfo& k, bool geo, bool inside, int L0, int L1) {
    if (!geo) return l.off;
    const bool ok = inside | (((unsigned)(l.p0 + k.g0) < (unsigned)L0) & ((unsigned)(l.p1 + k.g1) < (unsigned)L1));
    return ok ? l.off : kOOB;
  };
  // uniform offset of a load of K-block kb at this step (kOOB: the load reads
  // zeros); nv = valid K-blocks of the step
  auto soff = [](int kofs, int kb, bool live, int nv) { return (live & (kb < nv)) ? kofs : kOOB; };

  // Issue the loads of the next step into stage `st`. Loads past the last
  // step read zeros, so every wave issues WPS loads per step.
  auto issue_d = [&](int st, const KInfo& ka, const KInfo& kb, int fl) {
    const bool live = s_next < s_hi;
    const int nv = fl & 7;
    const bool inA = waveA || (fl & 8);
    const bool inB = waveB || (fl & 16);
    uint8_t* const stage = ring + st * STAGE;
    // K-major loads belong to one K-block each (uniform validity); a
    // row-major load spans the step's K-blocks (validity per lane)
#pragma unroll
    for (int k = 0; k < WCA; k++) {
      const int g = wave + 4 * k;
      uint8_t* const dst = g < NCA ? stage + g * 64 * 16 : arena + DUMMY;
      const int v = voff(ca[k], ka, P::kGeoA, inA, la0, la1);
      if constexpr (TA) dma16(rs[0], dst, v, soff(ka.code, (g * 64) / (BM * NPKA), live, nv));
      else dma16(rs[0], dst, ca[k].kb < nv ? v : kOOB, live ? ka.code : kOOB);
    }
#pragma unroll
    for (int k = 0; k < WCB; k++) {
      const int g = wave + 4 * k;
      uint8_t* const dst = g < NCB ? stage + OFF_B + g * 64 * 16 : arena + DUMMY;
      const int v = voff(cb[k], kb, P::kGeoB, inB, lb0, lb1);
      if constexpr (TB) dma16(rs[2], dst, v, soff(kb.code, (g * 64) / (BN * NPKB), live, nv));
      else dma16(rs[2], dst, cb[k].kb < nv ? v : kOOB, live ? kb.code : kOOB);
    }
    if constexpr (GS) {
      // wave 0: A scales, wave 1: B scales, waves 2-3: zero-reading filler
      const bool isA = wave == 0;
      const int v = isA ? voff(sa[0], ka, P::kGeoA, inA, la0, la1) : voff(sa[0], kb, P::kGeoB, inB, lb0, lb1);
      const int vt = s_kb < nv ? v : kOOB;
      dma1(isA ? rs[1] : rs[3], wave == 0 ? stage + OFF_SA : (wave == 1 ? stage + OFF_SB : arena + DUMMY), vt,
           live ? (isA ? ka.scale : kb.scale) : kOOB);
    } else {
#pragma unroll
      for (int k = 0; k < WSA; k++) {
        const int g = wave + 4 * k, kbi = (g * 64) / BM;
        dma1(rs[1], g < NSA ? stage + OFF_SA + g * 256 : arena + DUMMY, voff(sa[k], ka, P::kGeoA, inA, la0, la1),
             soff(ka.scale, kbi, live, nv));
      }
#pragma unroll
      for (int k = 0; k < WSB; k++) {
        const int g = wave + 4 * k, kbi = (g * 64) / BN;
        dma1(rs[3], g < NSB ? stage + OFF_SB + g * 256 : arena + DUMMY, voff(sb[k], kb, P::kGeoB, inB, lb0, lb1),
             soff(kb.scale, kbi, live, nv));
      }
    }
    s_next++;
  };
  // a step of the ring: its descriptors from the table
  auto issue = [&](int st) {
    const int li = s_next - tb;
    auto rl = [li](int v) { return __builtin_amdgcn_readlane(v, li); };
    const KInfo ka{rl(tab.ac), rl(tab.as), P::kGeoA ? rl(tab.ag0) : 0, P::kGeoA ? rl(tab.ag1) : 0};
    const KInfo kb{rl(tab.bc), rl(tab.bs), P::kGeoB ? rl(tab.bg0) : 0, P::kGeoB ? rl(tab.bg1) : 0};
    issue_d(st, ka, kb, rl(tab.fl));
  };

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  const int r32 = lane & 31, q = lane >> 5;
  // row-major stages: tile rows start at multiples of 32, so row_swz of a
  // row is that of r32
  const int hA = row_swz<SPRA>(r32), hB = row_swz<SPRB>(r32);
  // operand images and scales of the step's KPS / 2 pairs of K-blocks; pair
  // p starts 2 K-blocks (KBA / KBB bytes each) into the operand's stage
  constexpr int NP = KPS / 2;
  constexpr int KBA = BM * NPKA * 16, KBB = BN * NPKB * 16;
  v8i a[NP][TM], b[NP][TN];
  int xa[NP][TM], xb[NP][TN];
  auto read_operands = [&](int st) {
    const uint8_t* const stage = ring + st * STAGE;
#pragma unroll
    for (int p = 0; p < NP; p++) {
      // K-major stages: pair p starts 2 K-blocks into the operand's stage
      const uint8_t* const sA = stage + p * 2 * KBA;
      const uint8_t* const sB = stage + OFF_B + p * 2 * KBB;
      const int kq = 2 * p + q;  // K-block whose scale this lane supplies
#pragma unroll
      for (int i = 0; i < TM; i++) {
        const int row = (wm * TM + i) * 32 + r32;
        if constexpr (TA) a[p][i] = lds_operand_k<BM, KH, true>(sA, (wm * TM + i) * 32, lane);
        else if constexpr (KH) a[p][i] = lds_operand_half<SPRA>(stage, arena + ZERO, row, hA, p, q);
        else a[p][i] = lds_operand<FA, SPRA>(stage, row, hA, p, q);
        xa[p][i] = *reinterpret_cast<const int*>(stage + OFF_SA + (GS ? kq * (BM / gsa) + row / gsa : kq * BM + row) * 4);
      }
#pragma unroll
      for (int j = 0; j < TN; j++) {
        const int row = (wn * TN + j) * 32 + r32;
        // (with KH the other operand's upper lanes are zero: a K-major A is
        // zeroed above, a row-major A reads the zero slot)
        if constexpr (TB && FB >= 2) b[p][j] = lds_operand_k_sub<FB, BN>(sB, (wn * TN + j) * 32, lane);
        else if constexpr (TB) b[p][j] = lds_operand_k<BN, KH, false>(sB, (wn * TN + j) * 32, lane);
        else if constexpr (KH) b[p][j] = lds_operand_half<SPRB>(stage + OFF_B, arena + ZERO, row, hB, p, q);
        else b[p][j] = lds_operand<FB, SPRB>(stage + OFF_B, row, hB, p, q);
        xb[p][j] = *reinterpret_cast<const int*>(stage + OFF_SB + (GS ? kq * (BN / gsb) + row / gsb : kq * BN + row) * 4);
      }
    }
  };
  auto mfmas = [&]() {
#pragma unroll
    for (int p = 0; p < NP; p++)
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
          acc[i][j] = mfma_scaled_32x32x64<FA, FB>(a[p][i], b[p][j], xa[p][i], xb[p][j], acc[i][j]);
  };

  // Ring of NS stages: at step s the loads of step s+NS-1 go into the stage
  // that step s-1 computed from. The barrier before them both completes
  // stage s (every wave has waited for its own loads of step s) and retires
  // every wave's reads of stage s-1.
  const int nsteps = per_grp;
  if constexpr (KH) {  // the zero slot; the first step's wait and barrier publish it
    if (tid == 0) {
      const v4i zero = {0, 0, 0, 0};
      *reinterpret_cast<v4i*>(arena + ZERO) = zero;
    }
  }
  // the first NS-1 steps' descriptors are computed directly (uniform, in
  // scalar registers), so their loads leave before the table is filled
#pragma unroll
  for (int i = 0; i < NS - 1; i++) {
    const StepD d = step_desc(s_lo + i);
    issue_d(i, d.ka, d.kb, d.fl);
  }
  tab = fill(s_lo);
  int cs = 0;
  // LDS reads per step of a wave, for the instruction schedule below
  constexpr int RDA = TA ? 4 : F_READS<FA>(), RDB = TB ? (FB <= 1 ? 4 : 2) : F_READS<FB>();
  constexpr int NDS = NP * (TM * (RDA + 1) + TN * (RDB + 1));
  constexpr int NMF = NP * TM * TN;
  constexpr int VPM = (WPS + NMF - 1) / NMF;  // loads issued after each MFMA
  // Chunks of the table: iteration s issues step s_lo + s + NS - 1, which
  // must lie in [tb, tb + 64); past that the table is refilled (outside the
  // inner loop, whose body stays one block for the schedule below).
  for (int s = 0; s < nsteps;) {
    const int chunk_end = min(nsteps, tb - s_lo + 65 - NS);
    for (; s < chunk_end; s++) {
      wait_vm_lgkm0<(NS - 2) * WPS>();
      stage_barrier();
      read_operands(cs);
      issue(cs == 0 ? NS - 1 : cs - 1);
      mfmas();
      // operand reads first, then the loads of the next stage spread between
      // the MFMAs so their issue overlaps the matrix pipe
      __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
#pragma unroll
      for (int i = 0; i < NMF; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, VPM, 0);
      }
      cs = cs + 1 == NS ? 0 : cs + 1;
    }
    if (s < nsteps) {
      tab = fill(s_next);
      tb = s_next;
    }
  }
  wait_vm_lgkm0<0>();
  stage_barrier();
  if constexpr (NG > 1) {
    // group 1 hands its sums to group 0 through LDS (lane-major, no bank
    // conflicts), group 0 adds them, and group 1 is done
    float* xch = reinterpret_cast<float*>(arena) + wave * (TM * TN * 16 * 64);
    if (grp == 1) {
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
          for (int e = 0; e < 16; e++) xch[((i * TN + j) * 16 + e) * 64 + lane] = acc[i][j][e];
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    stage_barrier();
    if (grp == 0) {
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
          for (int e = 0; e < 16; e++) acc[i][j][e] += xch[((i * TN + j) * 16 + e) * 64 + lane];
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    // the strips below reuse the exchange area: every group-0 wave must have
    // read its part first (all waves of both groups take this barrier)
    stage_barrier();
    if (grp == 1) continue;
  }

  // Epilogue through LDS (the stages are free now). For each 32-row strip i
  // a wave writes its TN accumulator tiles as a 32 x (TN*32) fp32 block
  // (lane = column r32 of rows 8*(e/4) + 4*q + e%4), then reads it back as
  // 16-byte row pieces and stores them: each output row segment goes out as
  // whole 16-byte vectors from consecutive lanes.
  constexpr int EW = TN * 32;        // strip width (columns)
  constexpr int EP = EW + 8;         // LDS pitch in floats (rows 4 apart land 32 banks apart)
  float* strip = reinterpret_cast<float*>(arena + wave * STRIP);
  const int ncols = prob.ncols();
  const int c_wave = n0 + wn * EW;  // first column of this wave
  const bool full_cols = (c_wave + EW <= ncols) && ((ncols & 3) == 0);
  typedef float v4f __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int i = 0; i < TM; i++) {
    if constexpr (!MxOut<P>::value && PERSIST) {
      // (persistent backward-data) A strip whose 32 rows all lie at a fixed stride from its first row
      // and whose columns are all in range goes out straight from the
      // accumulators: for each accumulator register, lanes 0-31 and 32-63
      // each write one whole 128-byte row segment (no LDS round trip, which
      // would compete with the K loops of the other workgroups on the CU).
      const int ms = m0 + (wm * TM + i) * 32;
      float* const sb = prob.out_row(cx, z, ms);
      const bool direct = sb != nullptr && c_wave + EW <= ncols && ms + 32 <= prob.rows_a(cx) &&
                          prob.row_run(cx, ms) >= 32;
      if (direct) {
        float* const col = sb + c_wave + r32;
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
          for (int e = 0; e < 16; e++)
            __builtin_nontemporal_store(acc[i][j][e],
                                        col + (long long)(8 * (e >> 2) + 4 * q + (e & 3)) * ncols + j * 32);
        continue;
      }
    }
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int e = 0; e < 16; e++)
        strip[(8 * (e >> 2) + 4 * q + (e & 3)) * EP + j * 32 + r32] = acc[i][j][e];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the strip is written (same wave)
    __builtin_amdgcn_wave_barrier();
    if constexpr (MxOut<P>::value) {
      const int ms = m0 + (wm * TM + i) * 32;
      uint8_t* const cst = arena + 4 * STRIP + wave * CST;
      constexpr bool LEAN = TM * TN >= 8;
      switch (prob.yfmt) {
        case 0: mx_store_strip<0, TN, LEAN>(prob, cx, strip, EP, ms, c_wave, lane, cst); break;
        case 1: mx_store_strip<1, TN, LEAN>(prob, cx, strip, EP, ms, c_wave, lane, cst); break;
        case 2: mx_store_strip<2, TN, LEAN>(prob, cx, strip, EP, ms, c_wave, lane, cst); break;
        case 3: mx_store_strip<3, TN, LEAN>(prob, cx, strip, EP, ms, c_wave, lane, cst); break;
        default: mx_store_strip<4, TN, LEAN>(prob, cx, strip, EP, ms, c_wave, lane, cst); break;
      }
      __builtin_amdgcn_wave_barrier();
      continue;
    }
    constexpr int V = 32 * EW / 4;  // float4 pieces in the strip
    // the strip's first row and the run of rows that follow it at a fixed
    // stride: one address computation per strip instead of one per row
    const int ms = m0 + (wm * TM + i) * 32;
    float* const sbase = prob.out_row(cx, z, ms);
    const int run = prob.row_run(cx, ms), mlim = prob.rows_a(cx);
#pragma unroll
    for (int t = 0; t < V / 64; t++) {
      const int flat = t * 64 + lane;
      const int rr = flat / (EW / 4), c4 = flat % (EW / 4);
      const int m = ms + rr;
      float* row = rr < run ? (m < mlim ? sbase + (long long)rr * ncols : nullptr) : prob.out_row(cx, z, m);
      const v4f val = *reinterpret_cast<const v4f*>(&strip[rr * EP + c4 * 4]);
      if (row) {
        const int c = c_wave + c4 * 4;
        if (full_cols) {
          __builtin_nontemporal_store(val, reinterpret_cast<v4f*>(row + c));
        } else {
#pragma unroll
          for (int u = 0; u < 4; u++)
            if (c + u < ncols) row[c + u] = val[u];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  }  // tiles of a persistent workgroup
}

// Workgroups of a kernel that fit on one compute unit at once (0 if the
// runtime cannot say; the query's error is cleared).
inline int kernel_occupancy(const void* kern, int threads) {
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return occ;
}
// Workgroups of a persistent launch: all that fit on the current device at
// once, a multiple of 8 * nz (eight XCDs, each pass of an XCD's workgroups
// spanning whole groups of nz parity classes); 0: launch one per tile.
inline int persistent_groups(int occ, int nz) {
  int dev = 0, cus = 0;
  if (occ <= 0 || hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int unit = 8 * (nz > 0 ? nz : 1);
  return occ * cus / unit * unit;
}

// The backward-weight tile that runs two wave groups per workgroup with full
// K-blocks (tile 2, 256 x 128).
template <int WM, int WN, int TM, int TN>
constexpr bool wgrad_two_groups() {
  return WM == 2 && WN == 2 && TM == 4 && TN == 2;
}

template <class P, int WM, int WN, int TM, int TN, int NS, bool GS, bool KH>
hipError_t launch_gemm(int fa, int fb, const P& prob, dim3 grid, hipStream_t st) {
  // the backward-weight problem with half K-blocks: four K-blocks per step
  // and two wave groups per workgroup
  constexpr int KPS = (P::kQuad && KH) ? 4 : 2;
  // and the 256 x 128 backward-weight tile too: two groups of four waves
  // split each slice's K range (one workgroup of eight waves per CU instead
  // of two of four), so half as many slices write fp32 partial sums
  constexpr int NG = (P::kQuad && (KH || wgrad_two_groups<WM, WN, TM, TN>())) ? 2 : 1;
  // persistent workgroups (see gemm_persistent)
  constexpr bool PERSIST = gemm_persistent<P, WM, WN, TM, TN, NS>();
#define MQ_CASE(A, B)                                                                                   \
  if (fa == A && fb == B) {                                                                             \
    const auto kern = mx_gemm_kernel<A, B, P, WM, WN, TM, TN, NS, GS, KH, KPS, NG>;                     \
    P pr = prob;                                                                                        \
    dim3 g = grid;                                                                                      \
    if (PERSIST) {                                                                                      \
      static const int occ = kernel_occupancy(reinterpret_cast<const void*>(kern), 256 * NG);          \
      const int G = persistent_groups(occ, (int)grid.z);                                                \
      if (G > 0 && (long long)grid.x * grid.y * grid.z > G) {                                           \
        pr.grid.gx = G / 8;                                                                             \
        g = dim3(G);                                                                                    \
      }                                                                                                 \
    }                                                                                                   \
    hipLaunchKernelGGL(kern, g, dim3(256 * NG), 0, st, pr);                                             \
    return launch_check();                                                                              \
  }
  if constexpr (SubB<P>::value) {  // 8-bit A, 6/4-bit B, full K-blocks only
    if constexpr (!KH) { MQ_CASE(0, 2) MQ_CASE(0, 3) MQ_CASE(0, 4) MQ_CASE(1, 2) MQ_CASE(1, 3) MQ_CASE(1, 4) }
    return hipErrorInvalidValue;
  } else if constexpr (KH || (P::kKMajA && P::kKMajB)) {
    MQ_CASE(0, 0) MQ_CASE(0, 1) MQ_CASE(1, 0) MQ_CASE(1, 1)
    return hipErrorInvalidValue;
  } else if constexpr (P::kKMajB) {
    MQ_CASE(0, 0) MQ_CASE(0, 1) MQ_CASE(1, 0) MQ_CASE(1, 1) MQ_CASE(2, 0) MQ_CASE(2, 1)
    MQ_CASE(3, 0) MQ_CASE(3, 1) MQ_CASE(4, 0) MQ_CASE(4, 1)
    return hipErrorInvalidValue;
  } else if constexpr (P::kKMajA) {
    MQ_CASE(0, 0) MQ_CASE(0, 1) MQ_CASE(0, 2) MQ_CASE(0, 3) MQ_CASE(0, 4)
    MQ_CASE(1, 0) MQ_CASE(1, 1) MQ_CASE(1, 2) MQ_CASE(1, 3) MQ_CASE(1, 4)
    return hipErrorInvalidValue;
  } else {
  MQ_CASE(0, 0) MQ_CASE(0, 1) MQ_CASE(0, 2) MQ_CASE(0, 3) MQ_CASE(0, 4)
  MQ_CASE(1, 0) MQ_CASE(1, 1) MQ_CASE(1, 2) MQ_CASE(1, 3) MQ_CASE(1, 4)
  MQ_CASE(2, 0) MQ_CASE(2, 1) MQ_CASE(2, 2) MQ_CASE(2, 3) MQ_CASE(2, 4)
  MQ_CASE(3, 0) MQ_CASE(3, 1) MQ_CASE(3, 2) MQ_CASE(3, 3) MQ_CASE(3, 4)
  MQ_CASE(4, 0) MQ_CASE(4, 1) MQ_CASE(4, 2) MQ_CASE(4, 3) MQ_CASE(4, 4)
  }
#undef MQ_CASE
  return hipErrorInvalidValue;
}

// Workgroup tile shapes (rows x cols of the output):
//   0: 256 x 64   (4 x 1 waves of 64 x 64)   narrow outputs
//   1: 128 x 128  (2 x 2 waves of 64 x 64)
//   2: 256 x 128  (2 x 2 waves of 128 x 64)
//   3: 64 x 256   (1 x 4 waves of 64 x 64)   short outputs
//   4: 64 x 192   (2 x 2 waves of 32 x 96)   short outputs of 3 x 64 columns
//   5: 128 x 128 with a 2-stage ring: a tile of few K-steps spends most of its
//      life outside the K-loop (set-up, first loads, epilogue), so smaller
//      workgroups that fit more per CU overlap those phases better (measured
//      on the stride-2 backward-data with the MX epilogue, 9 K-steps per tile
//      on average; the fp32 backward-data runs persistent 256 x 128 tiles)
struct TileChoice { int id, bm, bn; };
inline TileChoice tile_shape(int id) {
  switch (id) {
    case 0: return {0, 256, 64};
    case 1: return {1, 128, 128};
    case 2: return {2, 256, 128};
    case 4: return {4, 64, 192};
    case 5: return {5, 128, 128};
    default: return {3, 64, 256};
  }
}
// Picks the largest tile (fewest re-reads of the operands) that still gives
// about one workgroup per compute unit. Short outputs take the column width
// that pads the columns least (576 = 9 taps x 64 channels fills three
// 192-column tiles, but leaves a 256-column tile three quarters empty).
inline TileChoice choose_tile(long long M, long long Ncols, long long Z) {
  if (Ncols <= 64) return tile_shape(0);
  if (M <= 64) return ceil_div(Ncols, 192) * 192 < ceil_div(Ncols, 256) * 256 ? tile_shape(4) : tile_shape(3);
  const long long big = (long long)ceil_div(M, 256) * ceil_div(Ncols, 128) * Z;
  if (big >= 240) return tile_shape(2);
  return tile_shape(1);
}

// Stages in the ring (three: deeper rings measured slower).
template <class P, bool GS, bool KH>
hipError_t launch_tile_id(int id, int fa, int fb, const P& prob, dim3 grid, hipStream_t st) {
  constexpr int NS = 3;
  switch (id) {
    case 0: return launch_gemm<P, 4, 1, 2, 2, NS, GS, KH>(fa, fb, prob, grid, st);
    case 1: return launch_gemm<P, 2, 2, 2, 2, NS, GS, KH>(fa, fb, prob, grid, st);
    case 2:
      // not chosen (see launch_tiled), so not built
      if constexpr ((P::kQuad && KH) || !GS || (MxOut<P>::value && std::is_base_of<DgradProb, P>::value))
        return hipErrorInvalidValue;
      else return launch_gemm<P, 2, 2, 4, 2, NS, GS, KH>(fa, fb, prob, grid, st);
    case 4: return launch_gemm<P, 2, 2, 1, 3, NS, GS, KH>(fa, fb, prob, grid, st);
    case 5:  // 128 x 128 with a 2-deep ring (backward-data with few K-steps per tile)
      if constexpr (std::is_base_of<DgradProb, P>::value) return launch_gemm<P, 2, 2, 2, 2, 2, GS, KH>(fa, fb, prob, grid, st);
      else return hipErrorInvalidValue;
    default: return launch_gemm<P, 1, 4, 2, 2, NS, GS, KH>(fa, fb, prob, grid, st);
  }
}

// Rows sharing one scale in a tile of `rows` rows starting at a multiple of
// it: the block partner extent (32) when the partner size is a multiple of
// it, the whole partner extent when it divides 32, else 0 (per-row scales).
inline int scale_group_rows(int bp, int partner) {
  if (bp != 32) return 0;
  if (partner % 32 == 0) return 32;
  if (partner < 32 && 32 % partner == 0) return partner;
  return 0;
}

// The half-K-block kernel runs when both operands have grouped scales and
// 8-bit codes, and every K-block holds at most 16 valid codes. Re-laid
// operands then need only 16-byte runs.
inline bool half_k_blocks(int ga, int gb, int khalf, int fa, int fb) {
  return ga >= 8 && gb >= 8 && khalf && fa <= 1 && fb <= 1;
}

// ksteps: K-steps per tile (on average over the problem), when known
template <class P>
hipError_t launch_tiled(int fa, int fb, const P& prob_in, int M, int Ncols, int Z, hipStream_t st,
                        int ksteps = 1 << 30) {
  TileChoice t = choose_tile(M, Ncols, Z);
  // one scale per row (no grouped scales) needs more registers than the
  // 256 x 128 tile leaves at two waves per SIMD: 128 x 128 instead
  bool grouped = false;
  if constexpr (P::kCanGroup) grouped = prob_in.ga >= 8 && prob_in.gb >= 8;
  if (!grouped && t.id == 2) t = tile_shape(1);
  if constexpr (std::is_base_of<DgradProb, P>::value) {
    // the backward-data problem with the MX epilogue needs more registers
    // than the 256 x 128 tile leaves at two waves per SIMD (it would spill
    // to scratch memory): 128 x 128 instead, with a 2-deep ring for tiles
    // of few K-steps
    if (MxOut<P>::value && t.id == 2) t = tile_shape(ksteps <= 12 ? 5 : 1);
  }
  // four K-blocks per step double the operand registers: the 256 x 128 tile
  // would then exceed the budget of two waves per SIMD
  if constexpr (P::kQuad) {
    if (t.id == 2 && half_k_blocks(prob_in.ga, prob_in.gb, prob_in.khalf, fa, fb)) t = tile_shape(1);
  }
  dim3 grid(ceil_div(M, t.bm), ceil_div(Ncols, t.bn), Z);
  P prob = prob_in;
  prob.grid.nx = make_fastdiv(grid.x);
  prob.grid.nxy = make_fastdiv(grid.x * grid.y);
  prob.grid.tx = (int)grid.x;
  prob.grid.ty = (int)grid.y;
  prob.grid.tz = (int)grid.z;
  prob.grid.gx = 0;
  if constexpr (P::kCanGroup) {
    // one 64-lane load holds both K-blocks' group scales of a 256-row tile
    // when groups have at least 8 rows
    if (grouped) {
      if (half_k_blocks(prob.ga, prob.gb, prob.khalf, fa, fb))
        return launch_tile_id<P, true, true>(t.id, fa, fb, prob, grid, st);
      return launch_tile_id<P, true, false>(t.id, fa, fb, prob, grid, st);
    }
  }
  return launch_tile_id<P, false, false>(t.id, fa, fb, prob, grid, st);
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// A buffer and the bias in front of it must stay below the offset that
// marks invalid blocks.
inline bool offsets_fit(long long bytes, long long bias) { return bytes + bias < 0x7f000000LL; }

// Number of K slices for an output of Ma x Nb with nkb K-blocks: up to two
// workgroups per compute unit (a partial last wave of workgroups would
// double the time), while the fp32 partial sums that the slices write and
// the reduction reads stay below traffic_factor times the operand bytes.
// grouped: whether the launch will use grouped scales (without them it
// takes the 128 x 128 tile where choose_tile says 256 x 128).
inline int splitk_slices(long long Ma, long long Nb, long long nkb, long long operand_bytes, int traffic_factor = 2,
                         bool grouped = true) {
  auto pick = [&](long long z) {
    const TileChoice c = choose_tile(Ma, Nb, z);
    return (!grouped && c.id == 2) ? tile_shape(1) : c;
  };
  TileChoice t = pick(1);
  long long tiles = ceil_div(Ma, t.bm) * ceil_div(Nb, t.bn);
  long long s = 512 / tiles;
  // the launch picks its tile from the slice count too: count with that tile
  const TileChoice tz = pick(s > 0 ? s : 1);
  if (tz.id != t.id) {
    t = tz;
    tiles = ceil_div(Ma, t.bm) * ceil_div(Nb, t.bn);
    s = 512 / tiles;
  }
  // 2 x 4 bytes per partial, at most traffic_factor / 2 times the operand bytes
  const long long cap_traffic = operand_bytes * traffic_factor / (8 * Ma * Nb) + 1;
  if (s > cap_traffic) s = cap_traffic;
  if (s > nkb / 4) s = nkb / 4;  // at least 4 K-blocks per slice
  if (s < 1) s = 1;
  return (int)s;
}

}  // namespace mq
