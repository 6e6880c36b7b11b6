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
// Kernel: 256 threads = 4 waves in a WM x WN grid; each wave owns a 64 x 64
// output tile = 2 x 2 MFMA tiles of 32 x 32; a K-step covers two K-blocks.
// Every K-step the workgroup stages its BM x 2 and BN x 2 runs (and their
// scale bytes) in LDS with coalesced 16-byte (8-byte for 6-bit codes) loads,
// double-buffered: the global loads of step s+1 are in flight while the
// MFMAs of step s read their operands from LDS.
#pragma once
#include "mx_common.h"
#include "mqconv_internal.h"

#include <type_traits>

namespace mq {

// Byte offsets into a problem's code and scale buffers are the sum of a
// per-row part (computed once per thread) and a per-K-block part (uniform
// across the workgroup, advanced incrementally in scalar registers):
//   code  = row.code + k.code,   scale = row.scale + k.scale
// valid iff row.ok && k.ok && (row.p0 + k.g0) in [0, lim0) && (row.p1 + k.g1)
// in [0, lim1); the geometric test covers the image borders of the implicit
// im2col. Invalid (zero) blocks read from past the end of the buffer, where
// raw buffer loads return 0.
constexpr int kOOB = 0x7fffff00;
struct RowInfo { int code, scale, p0, p1; bool ok; };
struct KInfo { int code, scale, g0, g1; bool ok; };

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, long long bytes) {
  const int n = bytes < (long long)kOOB ? (int)bytes : kOOB;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}

// ---------------------------------------------------------------------------
// Problem descriptors
// ---------------------------------------------------------------------------
// Forward: rows m = (ho, wo, n), K-block (kh, kw, cb).
struct FwdProb {
  const uint8_t *xc, *xs, *wc, *ws;
  float* y;
  long long xc_bytes, xs_bytes, wc_bytes, ws_bytes;
  int N, H, W, Cin, Cout, KW, T, sh, sw, ph, pw, Wo, M;
  int xrb, xRB, xbp, xnPB, ncb;  // activation row bytes, run bytes, bp, partner blocks, channel blocks
  int wrb, wRB, wnCoB, wbp;       // weight row bytes, run bytes, Cout blocks, bp
  struct Ctx {};
  struct KS { int kh, kw, v; };
  __device__ Ctx ctx(int) const { return Ctx{}; }
  __device__ int rows_a(const Ctx&) const { return M; }
  __device__ int ncols() const { return Cout; }
  __device__ void krange(const Ctx&, int, int& lo, int& hi) const { lo = 0; hi = T * ncb; }
  __device__ KS kstart(const Ctx&, int kb) const {
    const int u = kb / ncb; KS k; k.v = kb - u * ncb; k.kh = u / KW; k.kw = u - k.kh * KW; return k;
  }
  __device__ void knext(const Ctx&, KS& k) const {
    if (++k.v == ncb) { k.v = 0; if (++k.kw == KW) { k.kw = 0; k.kh++; } }
  }
  __device__ RowInfo row_a(const Ctx&, int m) const {
    RowInfo r; r.ok = m < M; const int mm = r.ok ? m : 0;
    const int pix = mm / N, n = mm - pix * N, ho = pix / Wo, wo = pix - ho * Wo;
    r.p0 = ho * sh - ph; r.p1 = wo * sw - pw;
    const int p = r.p0 * W + r.p1;
    r.code = (p * N + n) * xrb; r.scale = (p * xnPB + n / xbp) * ncb; return r;
  }
  __device__ KInfo k_a(const Ctx&, const KS& k, bool ok) const {
    const int d = k.kh * W + k.kw;
    return KInfo{d * N * xrb + k.v * xRB, d * xnPB * ncb + k.v, k.kh, k.kw, ok};
  }
  __device__ RowInfo row_b(const Ctx&, int c) const {
    RowInfo r; r.ok = c < Cout; const int cc = r.ok ? c : 0;
    r.code = cc * T * wrb; r.scale = (cc / wbp) * ncb; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_b(const Ctx&, const KS& k, bool ok) const {
    const int tap = k.kh * KW + k.kw;
    return KInfo{tap * wrb + k.v * wRB, tap * wnCoB * ncb + k.v, 0, 0, ok};
  }
  __device__ int lim_a0() const { return H; }
  __device__ int lim_a1() const { return W; }
  __device__ float* out_row(const Ctx&, int, int m) const { return m < M ? y + (long long)m * Cout : nullptr; }
};

// Backward-data: rows of parity class z are h = hq*sh + ph_c, w = wq*sw + pw_c
// (and all n); the taps reaching them are kh = kh0 + sh*ih, kw = kw0 + sw*iw,
// from output pixel (ho0 - ih, wo0 - iw). K-block (ih, iw, cob).
struct DgradProb {
  const uint8_t *dyc, *dys, *wtc, *ws;
  float* dx;
  long long dyc_bytes, dys_bytes, wtc_bytes, ws_bytes;
  int N, H, W, Cin, Cout, KH, KW, sh, sw, ph, pw, Ho, Wo;
  int dyrb, dyRB, dybp, dynPB, ncob;  // gradient row bytes, run bytes, bp, partner blocks, Cout blocks
  int wRB, ncbi;                      // weight run bytes, Cin blocks
  struct Ctx { int ph_c, pw_c, Hc, Wc, kh0, kw0, nkh, nkw, M; };
  struct KS { int ih, iw, v; };
  __device__ Ctx ctx(int z) const {
    Ctx c; c.ph_c = z / sw; c.pw_c = z - c.ph_c * sw;
    c.Hc = H > c.ph_c ? (H - c.ph_c + sh - 1) / sh : 0;
    c.Wc = W > c.pw_c ? (W - c.pw_c + sw - 1) / sw : 0;
    c.kh0 = (c.ph_c + ph) % sh; c.kw0 = (c.pw_c + pw) % sw;
    c.nkh = c.kh0 < KH ? (KH - c.kh0 + sh - 1) / sh : 0;
    c.nkw = c.kw0 < KW ? (KW - c.kw0 + sw - 1) / sw : 0;
    c.M = c.Hc * c.Wc * N;
    return c;
  }
  __device__ int rows_a(const Ctx& c) const { return c.M; }
  __device__ int ncols() const { return Cin; }
  __device__ void krange(const Ctx& c, int, int& lo, int& hi) const { lo = 0; hi = c.nkh * c.nkw * ncob; }
  __device__ KS kstart(const Ctx& c, int kb) const {
    const int nkw = c.nkw > 0 ? c.nkw : 1;
    const int u = kb / ncob; KS k; k.v = kb - u * ncob; k.ih = u / nkw; k.iw = u - k.ih * nkw; return k;
  }
  __device__ void knext(const Ctx& c, KS& k) const {
    if (++k.v == ncob) { k.v = 0; if (++k.iw == c.nkw) { k.iw = 0; k.ih++; } }
  }
  __device__ RowInfo row_a(const Ctx& c, int m) const {
    RowInfo r; r.ok = m < c.M; const int mm = r.ok ? m : 0;
    const int wc = c.Wc > 0 ? c.Wc : 1;
    const int pix = mm / N, n = mm - pix * N, hq = pix / wc, wq = pix - hq * wc;
    // output pixel of tap (kh0, kw0); exact division by the class choice
    r.p0 = hq + (c.ph_c + ph - c.kh0) / sh;
    r.p1 = wq + (c.pw_c + pw - c.kw0) / sw;
    const int p = r.p0 * Wo + r.p1;
    r.code = (p * N + n) * dyrb; r.scale = (p * dynPB + n / dybp) * ncob; return r;
  }
  __device__ KInfo k_a(const Ctx&, const KS& k, bool ok) const {
    const int d = k.ih * Wo + k.iw;
    return KInfo{-d * N * dyrb + k.v * dyRB, -d * dynPB * ncob + k.v, -k.ih, -k.iw, ok};
  }
  __device__ RowInfo row_b(const Ctx&, int c) const {
    RowInfo r; r.ok = c < Cin; const int cc = r.ok ? c : 0;
    r.code = cc * ncob * wRB; r.scale = cc / 32; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_b(const Ctx& c, const KS& k, bool ok) const {
    const int tap = (c.kh0 + sh * k.ih) * KW + (c.kw0 + sw * k.iw);
    return KInfo{(tap * Cin * ncob + k.v) * wRB, (tap * ncob + k.v) * ncbi, 0, 0, ok};
  }
  __device__ int lim_a0() const { return Ho; }
  __device__ int lim_a1() const { return Wo; }
  __device__ float* out_row(const Ctx& c, int, int m) const {
    if (m >= c.M) return nullptr;
    const int pix = m / N, n = m - pix * N, hq = pix / c.Wc, wq = pix - hq * c.Wc;
    const int h = hq * sh + c.ph_c, w = wq * sw + c.pw_c;
    return dx + (((long long)h * W + w) * N + n) * Cin;
  }
};

// Backward-weight on codes re-laid with runs along N: rows co (A) and
// j = (kh, kw, ci) (B); K-block (ho, wo, nb) over the slice's output pixels.
struct WgradProb {
  const uint8_t *dytc, *dys, *xtc, *xs;
  float* part;
  long long dytc_bytes, dys_bytes, xtc_bytes, xs_bytes;
  int N, H, W, Cin, Cout, KW, T, sh, sw, ph, pw, Wo, nNB, ncob, ncbi;
  int dyRB, xRB;
  int npix;  // Ho*Wo
  int pix_per_split;
  struct Ctx {};
  struct KS { int ho, wo, v; };
  __device__ Ctx ctx(int) const { return Ctx{}; }
  __device__ int rows_a(const Ctx&) const { return Cout; }
  __device__ int ncols() const { return T * Cin; }
  __device__ void krange(const Ctx&, int z, int& lo, int& hi) const {
    int p0 = z * pix_per_split, p1 = min(npix, p0 + pix_per_split);
    lo = p0 * nNB; hi = max(p0, p1) * nNB;
  }
  __device__ KS kstart(const Ctx&, int kb) const {
    const int u = kb / nNB; KS k; k.v = kb - u * nNB; k.ho = u / Wo; k.wo = u - k.ho * Wo; return k;
  }
  __device__ void knext(const Ctx&, KS& k) const {
    if (++k.v == nNB) { k.v = 0; if (++k.wo == Wo) { k.wo = 0; k.ho++; } }
  }
  __device__ RowInfo row_a(const Ctx&, int m) const {
    RowInfo r; r.ok = m < Cout; const int co = r.ok ? m : 0;
    r.code = co * nNB * dyRB; r.scale = co / 32; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_a(const Ctx&, const KS& k, bool ok) const {
    const int pix = k.ho * Wo + k.wo;
    return KInfo{(pix * Cout * nNB + k.v) * dyRB, (pix * nNB + k.v) * ncob, 0, 0, ok};
  }
  __device__ RowInfo row_b(const Ctx&, int j) const {
    RowInfo r; r.ok = j < T * Cin; const int jj = r.ok ? j : 0;
    const int tap = jj / Cin, ci = jj - tap * Cin, kh = tap / KW, kw = tap - kh * KW;
    r.p0 = kh - ph; r.p1 = kw - pw;
    const int p = r.p0 * W + r.p1;
    r.code = (p * Cin + ci) * nNB * xRB; r.scale = p * nNB * ncbi + ci / 32; return r;
  }
  __device__ KInfo k_b(const Ctx&, const KS& k, bool ok) const {
    const int g0 = k.ho * sh, g1 = k.wo * sw, d = g0 * W + g1;
    return KInfo{(d * Cin * nNB + k.v) * xRB, (d * nNB + k.v) * ncbi, g0, g1, ok};
  }
  __device__ int lim_a0() const { return 1; }
  __device__ int lim_a1() const { return 1; }
  __device__ int lim_b0() const { return H; }
  __device__ int lim_b1() const { return W; }
  __device__ float* out_row(const Ctx&, int z, int m) const {
    return m < Cout ? part + ((long long)z * Cout + m) * ((long long)T * Cin) : nullptr;
  }
};

// Plain GEMM out[m][c] = sum_kb A[m][kb] . B[c][kb] over packed rows whose
// runs already follow the contraction (used by the naive comparison path).
// Slice z covers K-blocks [z*kb_per_split, (z+1)*kb_per_split) and writes its
// partial product to out + z*Ma*Nb.
struct PlainProb {
  const uint8_t *ac, *as, *bc, *bs;
  float* out;
  long long ac_bytes, as_bytes, bc_bytes, bs_bytes;
  int Ma, Nb, nkb, aRB, bRB, kb_per_split, arb, brb;
  struct Ctx {};
  struct KS { int u; };
  __device__ Ctx ctx(int) const { return Ctx{}; }
  __device__ int rows_a(const Ctx&) const { return Ma; }
  __device__ int ncols() const { return Nb; }
  __device__ void krange(const Ctx&, int z, int& lo, int& hi) const {
    lo = z * kb_per_split; hi = min(nkb, lo + kb_per_split); if (hi < lo) hi = lo;
  }
  __device__ KS kstart(const Ctx&, int kb) const { return KS{kb}; }
  __device__ void knext(const Ctx&, KS& k) const { k.u++; }
  __device__ RowInfo row_a(const Ctx&, int m) const {
    RowInfo r; r.ok = m < Ma; const int mm = r.ok ? m : 0;
    r.code = mm * arb; r.scale = mm * nkb; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_a(const Ctx&, const KS& k, bool ok) const { return KInfo{k.u * aRB, k.u, 0, 0, ok}; }
  __device__ RowInfo row_b(const Ctx&, int c) const {
    RowInfo r; r.ok = c < Nb; const int cc = r.ok ? c : 0;
    r.code = cc * brb; r.scale = cc * nkb; r.p0 = 0; r.p1 = 0; return r;
  }
  __device__ KInfo k_b(const Ctx&, const KS& k, bool ok) const { return KInfo{k.u * bRB, k.u, 0, 0, ok}; }
  __device__ int lim_a0() const { return 1; }
  __device__ int lim_a1() const { return 1; }
  __device__ float* out_row(const Ctx&, int z, int m) const {
    return m < Ma ? out + ((long long)z * Ma + m) * Nb : nullptr;
  }
};

// Default limits for the B side (weights and plain rows have no borders).
template <class P> __device__ __forceinline__ int lim_b0(const P&) { return 1; }
template <class P> __device__ __forceinline__ int lim_b1(const P&) { return 1; }
template <> __device__ __forceinline__ int lim_b0<WgradProb>(const WgradProb& p) { return p.lim_b0(); }
template <> __device__ __forceinline__ int lim_b1<WgradProb>(const WgradProb& p) { return p.lim_b1(); }

// Buffers of each problem: (A codes, A scales, B codes, B scales).
__device__ inline void rsrcs(const FwdProb& p, __amdgpu_buffer_rsrc_t (&r)[4]) {
  r[0] = make_rsrc(p.xc, p.xc_bytes); r[1] = make_rsrc(p.xs, p.xs_bytes);
  r[2] = make_rsrc(p.wc, p.wc_bytes); r[3] = make_rsrc(p.ws, p.ws_bytes);
}
__device__ inline void rsrcs(const DgradProb& p, __amdgpu_buffer_rsrc_t (&r)[4]) {
  r[0] = make_rsrc(p.dyc, p.dyc_bytes); r[1] = make_rsrc(p.dys, p.dys_bytes);
  r[2] = make_rsrc(p.wtc, p.wtc_bytes); r[3] = make_rsrc(p.ws, p.ws_bytes);
}
__device__ inline void rsrcs(const WgradProb& p, __amdgpu_buffer_rsrc_t (&r)[4]) {
  r[0] = make_rsrc(p.dytc, p.dytc_bytes); r[1] = make_rsrc(p.dys, p.dys_bytes);
  r[2] = make_rsrc(p.xtc, p.xtc_bytes); r[3] = make_rsrc(p.xs, p.xs_bytes);
}
__device__ inline void rsrcs(const PlainProb& p, __amdgpu_buffer_rsrc_t (&r)[4]) {
  r[0] = make_rsrc(p.ac, p.ac_bytes); r[1] = make_rsrc(p.as, p.as_bytes);
  r[2] = make_rsrc(p.bc, p.bc_bytes); r[3] = make_rsrc(p.bs, p.bs_bytes);
}

// ---------------------------------------------------------------------------
// Staging of one operand (BR rows x 2 runs) into LDS
// ---------------------------------------------------------------------------
template <int F, int BR>
struct Stage {
  static constexpr int RB = run_bytes_of(F);
  static constexpr int CH = (RB == 24) ? 8 : 16;       // bytes per load
  static constexpr int NC = 2 * RB / CH;               // loads per row
  // LDS row pitch: 2 runs plus a skew that keeps the 32 rows one MFMA tile
  // reads (16-byte reads for 8/4-bit codes, 8-byte reads for 6-bit) on
  // distinct banks
  static constexpr int PITCH = (RB == 24) ? 2 * RB + 8 : 2 * RB + 16;
  static constexpr int TOTAL = BR * NC;
  static constexpr int PER = (TOTAL + 255) / 256;      // loads per thread
  static constexpr int BYTES = BR * PITCH;
  typedef typename std::conditional<CH == 16, v4i, v2i>::type V;
};

template <class V>
__device__ __forceinline__ V buffer_load(__amdgpu_buffer_rsrc_t r, int off);
template <>
__device__ __forceinline__ v4i buffer_load<v4i>(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
template <>
__device__ __forceinline__ v2i buffer_load<v2i>(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

// Reads one 32x32x64 operand register image (see mx_common.h) of LDS row `base`.
template <int F>
__device__ __forceinline__ v8i lds_operand(const uint8_t* base, int q) {
  v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (F <= 1) {
    v4i lo = *reinterpret_cast<const v4i*>(base + 16 * q);
    v4i hi = *reinterpret_cast<const v4i*>(base + 32 + 16 * q);
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3]; r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  } else if constexpr (F <= 3) {
    const v2i* p = reinterpret_cast<const v2i*>(base + 24 * q);
    v2i x0 = p[0], x1 = p[1], x2 = p[2];
    r[0] = x0[0]; r[1] = x0[1]; r[2] = x1[0]; r[3] = x1[1]; r[4] = x2[0]; r[5] = x2[1];
  } else {
    v4i x = *reinterpret_cast<const v4i*>(base + 16 * q);
    r[0] = x[0]; r[1] = x[1]; r[2] = x[2]; r[3] = x[3];
  }
  return r;
}

// One K-step's staged loads of a thread, held in registers between the
// global load and the LDS write.
template <class SA, class SB>
struct StepRegs {
  typename SA::V ga[SA::PER];
  typename SB::V gb[SB::PER];
  // kept as bytes up to the LDS byte store: widening them would put a use
  // of the loaded value (and so a wait for the load) right after the load
  uint8_t sa[SA::PER], sb[SB::PER];
};

// WM x WN waves; each wave owns TM x TN MFMA tiles of 32 x 32.
template <int FA, int FB, class P, int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(256) void mx_gemm_kernel(P prob) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  using SA = Stage<FA, BM>;
  using SB = Stage<FB, BN>;
  // One LDS arena: the two staging stages (A runs, B runs, A scales, B
  // scales) during the K loop, the epilogue strips afterwards.
  constexpr int OFF_B = 2 * SA::BYTES, OFF_SA = OFF_B + 2 * SB::BYTES, OFF_SB = OFF_SA + 2 * BM * 2;
  constexpr int STAGING = OFF_SB + 2 * BN * 2;
  constexpr int STRIP = 32 * (TN * 32 + 8) * 4;  // one wave's epilogue strip (bytes)
  constexpr int ARENA = STAGING > 4 * STRIP ? STAGING : 4 * STRIP;
  __shared__ __attribute__((aligned(16))) uint8_t arena[ARENA];
  auto lds_a = reinterpret_cast<uint8_t(*)[SA::BYTES]>(arena);
  auto lds_b = reinterpret_cast<uint8_t(*)[SB::BYTES]>(arena + OFF_B);
  auto sc_a = reinterpret_cast<uint8_t(*)[BM * 2]>(arena + OFF_SA);
  auto sc_b = reinterpret_cast<uint8_t(*)[BN * 2]>(arena + OFF_SB);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  // XCD-aware tile order: the hardware hands consecutive workgroups to the 8
  // XCDs in turn, each with its own L2. Remap so that every XCD works on a
  // contiguous range of tiles (x fastest): neighbouring row tiles share the
  // weight tile and the rows of the implicit im2col, and now share an L2.
  int bx, by, z;
  {
    const int nx = gridDim.x, ny = gridDim.y;
    const int nb = nx * ny * gridDim.z;
    const int lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    const int xcd = lin % 8, idx = lin / 8, q8 = nb / 8, r8 = nb % 8;
    const int logical = xcd < r8 ? xcd * (q8 + 1) + idx : r8 * (q8 + 1) + (xcd - r8) * q8 + idx;
    bx = logical % nx;
    by = (logical / nx) % ny;
    z = logical / (nx * ny);
  }
  const typename P::Ctx cx = prob.ctx(z);
  const int m0 = bx * BM, n0 = by * BN;
  if (m0 >= prob.rows_a(cx)) return;  // whole tile beyond this class's rows (uniform)
  __amdgpu_buffer_rsrc_t rs[4];
  rsrcs(prob, rs);

  // Load c = tid + 256*i of a stage covers row c / NC and piece c % NC of
  // the row's two runs: K-block kbi of the pair, byte offset `off` in the run.
  RowInfo ra[SA::PER], rb[SB::PER];
  int rowa[SA::PER], kbia[SA::PER], offa[SA::PER];
  int rowb[SB::PER], kbib[SB::PER], offb[SB::PER];
#pragma unroll
  for (int i = 0; i < SA::PER; i++) {
    const int c = tid + 256 * i, part = c % SA::NC;
    rowa[i] = min(c / SA::NC, BM - 1);
    kbia[i] = part / (SA::NC / 2);
    offa[i] = (part % (SA::NC / 2)) * SA::CH;
    ra[i] = prob.row_a(cx, m0 + rowa[i]);
  }
#pragma unroll
  for (int i = 0; i < SB::PER; i++) {
    const int c = tid + 256 * i, part = c % SB::NC;
    rowb[i] = min(c / SB::NC, BN - 1);
    kbib[i] = part / (SB::NC / 2);
    offb[i] = (part % (SB::NC / 2)) * SB::CH;
    rb[i] = prob.row_b(cx, n0 + rowb[i]);
  }
  const int la0 = prob.lim_a0(), la1 = prob.lim_a1(), lb0 = lim_b0(prob), lb1 = lim_b1(prob);

  int kb_lo, kb_hi;
  prob.krange(cx, z, kb_lo, kb_hi);
  // K-block iterator over the fetch sequence (uniform)
  typename P::KS kit = prob.kstart(cx, kb_lo);
  int kb_next = kb_lo;

  // (bitwise &, not &&: straight-line selects instead of branches)
  auto offset = [&](const RowInfo& r, const KInfo& k, int lim0, int lim1, int& code, int& scale) {
    const bool ok = r.ok & k.ok & ((unsigned)(r.p0 + k.g0) < (unsigned)lim0) &
                    ((unsigned)(r.p1 + k.g1) < (unsigned)lim1);
    code = ok ? r.code + k.code : kOOB;
    scale = ok ? r.scale + k.scale : kOOB;
  };
  // global -> registers for the next K-block pair; no branches: zero blocks
  // (and pairs past the end) load from past the end of the buffer and read 0
  auto fetch = [&](StepRegs<SA, SB>& R) {
    const bool ok0 = kb_next < kb_hi, ok1 = kb_next + 1 < kb_hi;
    const KInfo a0 = prob.k_a(cx, kit, ok0), b0 = prob.k_b(cx, kit, ok0);
    if (ok0) prob.knext(cx, kit);
    const KInfo a1 = prob.k_a(cx, kit, ok1), b1 = prob.k_b(cx, kit, ok1);
    if (ok1) prob.knext(cx, kit);
    kb_next += 2;
    int oca[SA::PER], osa[SA::PER], ocb[SB::PER], osb[SB::PER];
#pragma unroll
    for (int i = 0; i < SA::PER; i++) offset(ra[i], kbia[i] ? a1 : a0, la0, la1, oca[i], osa[i]);
#pragma unroll
    for (int i = 0; i < SB::PER; i++) offset(rb[i], kbib[i] ? b1 : b0, lb0, lb1, ocb[i], osb[i]);
    // the loads leave together; their consumers (the LDS writes of commit)
    // stay behind the MFMAs that run meanwhile
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < SA::PER; i++) {
      R.ga[i] = buffer_load<typename SA::V>(rs[0], oca[i] + offa[i]);
      R.sa[i] = __builtin_amdgcn_raw_buffer_load_b8(rs[1], osa[i], 0, 0);
    }
#pragma unroll
    for (int i = 0; i < SB::PER; i++) {
      R.gb[i] = buffer_load<typename SB::V>(rs[2], ocb[i] + offb[i]);
      R.sb[i] = __builtin_amdgcn_raw_buffer_load_b8(rs[3], osb[i], 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // registers -> LDS stage st. Every load of a run carries the run's scale
  // byte, so all of them store it (same value, same address).
  auto commit = [&](const StepRegs<SA, SB>& R, int st) {
#pragma unroll
    for (int i = 0; i < SA::PER; i++) {
      if (SA::TOTAL % 256 == 0 || tid + 256 * i < SA::TOTAL) {
        *reinterpret_cast<typename SA::V*>(&lds_a[st][rowa[i] * SA::PITCH + kbia[i] * SA::RB + offa[i]]) = R.ga[i];
        sc_a[st][rowa[i] * 2 + kbia[i]] = R.sa[i];
      }
    }
#pragma unroll
    for (int i = 0; i < SB::PER; i++) {
      if (SB::TOTAL % 256 == 0 || tid + 256 * i < SB::TOTAL) {
        *reinterpret_cast<typename SB::V*>(&lds_b[st][rowb[i] * SB::PITCH + kbib[i] * SB::RB + offb[i]]) = R.gb[i];
        sc_b[st][rowb[i] * 2 + kbib[i]] = R.sb[i];
      }
    }
  };

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  const int r32 = lane & 31, q = lane >> 5;
  auto compute = [&](int st) {
    v8i a[TM], b[TN];
    int sa[TM], sb[TN];
#pragma unroll
    for (int i = 0; i < TM; i++) {
      const int row = (wm * TM + i) * 32 + r32;
      a[i] = lds_operand<FA>(&lds_a[st][row * SA::PITCH], q);
      sa[i] = sc_a[st][row * 2 + q];
    }
#pragma unroll
    for (int j = 0; j < TN; j++) {
      const int row = (wn * TN + j) * 32 + r32;
      b[j] = lds_operand<FB>(&lds_b[st][row * SB::PITCH], q);
      sb[j] = sc_b[st][row * 2 + q];
    }
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int j = 0; j < TN; j++)
        acc[i][j] = mfma_scaled_32x32x64<FA, FB>(a[i], b[j], sa[i], sb[j], acc[i][j]);
  };

  // Pipeline: LDS stages 0/1 and register sets R0/R1; the loads of step s+2
  // are issued before step s computes, so two steps of MFMAs cover each
  // load's latency. The step count is rounded up to even (a trailing zero
  // step adds nothing).
  const int nsteps = (kb_hi - kb_lo + 1) / 2;
  if (nsteps > 0) {
    StepRegs<SA, SB> R0, R1;
    fetch(R0);
    fetch(R1);
    commit(R0, 0);
    __syncthreads();
    for (int s = 0; s < nsteps; s += 2) {
      fetch(R0);
      compute(0);
      __builtin_amdgcn_sched_barrier(0);
      commit(R1, 1);
      __syncthreads();
      fetch(R1);
      compute(1);
      __builtin_amdgcn_sched_barrier(0);
      commit(R0, 0);
      __syncthreads();
    }
  }

  // Epilogue through LDS (the staging buffers are free now). For each 32-row
  // strip i a wave writes its TN accumulator tiles as a 32 x (TN*32) fp32
  // block (lane = column r32 of rows 8*(e/4) + 4*q + e%4), then reads it back
  // as 16-byte row pieces and stores them: each output row segment goes out
  // as whole 16-byte vectors from consecutive lanes.
  __syncthreads();
  constexpr int EW = TN * 32;        // strip width (columns)
  constexpr int EP = EW + 8;         // LDS pitch in floats (rows 4 apart land 32 banks apart)
  float* strip = reinterpret_cast<float*>(arena + wave * STRIP);
  const int ncols = prob.ncols();
  const int c_wave = n0 + wn * EW;  // first column of this wave
  const bool full_cols = (c_wave + EW <= ncols) && ((ncols & 3) == 0);
  typedef float v4f __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int i = 0; i < TM; i++) {
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int e = 0; e < 16; e++)
        strip[(8 * (e >> 2) + 4 * q + (e & 3)) * EP + j * 32 + r32] = acc[i][j][e];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the strip is written (same wave)
    __builtin_amdgcn_wave_barrier();
    constexpr int V = 32 * EW / 4;  // float4 pieces in the strip
#pragma unroll
    for (int t = 0; t < V / 64; t++) {
      const int flat = t * 64 + lane;
      const int rr = flat / (EW / 4), c4 = flat % (EW / 4);
      const int m = m0 + (wm * TM + i) * 32 + rr;
      float* row = prob.out_row(cx, z, m);
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
}

template <class P, int WM, int WN, int TM, int TN>
hipError_t launch_gemm(int fa, int fb, const P& prob, dim3 grid, hipStream_t st) {
#define MQ_CASE(A, B)                                                                               \
  if (fa == A && fb == B) {                                                                         \
    hipLaunchKernelGGL((mx_gemm_kernel<A, B, P, WM, WN, TM, TN>), grid, dim3(256), 0, st, prob);    \
    return hipGetLastError();                                                                       \
  }
  MQ_CASE(0, 0) MQ_CASE(0, 1) MQ_CASE(0, 2) MQ_CASE(0, 3) MQ_CASE(0, 4)
  MQ_CASE(1, 0) MQ_CASE(1, 1) MQ_CASE(1, 2) MQ_CASE(1, 3) MQ_CASE(1, 4)
  MQ_CASE(2, 0) MQ_CASE(2, 1) MQ_CASE(2, 2) MQ_CASE(2, 3) MQ_CASE(2, 4)
  MQ_CASE(3, 0) MQ_CASE(3, 1) MQ_CASE(3, 2) MQ_CASE(3, 3) MQ_CASE(3, 4)
  MQ_CASE(4, 0) MQ_CASE(4, 1) MQ_CASE(4, 2) MQ_CASE(4, 3) MQ_CASE(4, 4)
#undef MQ_CASE
  return hipErrorInvalidValue;
}

// Workgroup tile shapes (rows x cols of the output):
//   0: 256 x 64   (4 x 1 waves of 64 x 64)   narrow outputs
//   1: 128 x 128  (2 x 2 waves of 64 x 64)
//   2: 256 x 128  (2 x 2 waves of 128 x 64)
//   3: 64 x 256   (1 x 4 waves of 64 x 64)   short outputs
struct TileChoice { int id, bm, bn; };
inline TileChoice tile_shape(int id) {
  switch (id) {
    case 0: return {0, 256, 64};
    case 1: return {1, 128, 128};
    case 2: return {2, 256, 128};
    default: return {3, 64, 256};
  }
}
// Picks the largest tile (fewest re-reads of the operands) that still gives
// about one workgroup per compute unit.
inline TileChoice choose_tile(long long M, long long Ncols, long long Z) {
  if (Ncols <= 64) return tile_shape(0);
  if (M <= 64) return tile_shape(3);
  const long long big = (long long)ceil_div(M, 256) * ceil_div(Ncols, 128) * Z;
  if (big >= 240) return tile_shape(2);
  return tile_shape(1);
}

template <class P>
hipError_t launch_tiled(int fa, int fb, const P& prob, int M, int Ncols, int Z, hipStream_t st) {
  const TileChoice t = choose_tile(M, Ncols, Z);
  dim3 grid(ceil_div(M, t.bm), ceil_div(Ncols, t.bn), Z);
  switch (t.id) {
    case 0: return launch_gemm<P, 4, 1, 2, 2>(fa, fb, prob, grid, st);
    case 1: return launch_gemm<P, 2, 2, 2, 2>(fa, fb, prob, grid, st);
    case 2: return launch_gemm<P, 2, 2, 4, 2>(fa, fb, prob, grid, st);
    default: return launch_gemm<P, 1, 4, 2, 2>(fa, fb, prob, grid, st);
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Number of K slices for an output of Ma x Nb with nkb K-blocks: enough
// workgroups to cover the GPU about twice, while the fp32 partial sums that
// the slices write and the reduction reads stay below the operand bytes.
inline int splitk_slices(long long Ma, long long Nb, long long nkb, long long operand_bytes) {
  const TileChoice t = choose_tile(Ma, Nb, 1);
  const long long tiles = ceil_div(Ma, t.bm) * ceil_div(Nb, t.bn);
  long long s = (512 + tiles - 1) / tiles;
  const long long cap_traffic = operand_bytes / (8 * Ma * Nb) + 1;  // 2 x 4 bytes per partial
  if (s > cap_traffic) s = cap_traffic;
  if (s > nkb / 4) s = nkb / 4;  // at least 4 K-blocks per slice
  if (s < 1) s = 1;
  return (int)s;
}


}  // namespace mq
