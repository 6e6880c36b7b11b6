/*
 * mqref.c -- CPU oracle for the MicroQonv training hot path.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library. It shares no code with the GPU
 * library: it implements the same definitions independently, plainly and
 * slowly, in fp64.
 *
 * Source: "MicroQonv: Reshaping Convolution Tensors for Efficient
 * Microscaling in Training and Inference" (Facq, Ben-Ali, Sentieys).
 *   - element codec and block quantizer: §II-D (original microscaling
 *     format, power-of-two E8M0 block scale), §III-A (blocks of elements
 *     sharing one scale; fake quantization = code value times its scale),
 *     with the OCP MX scale rule (shared exponent = floor(log2 amax) minus
 *     the element format's largest exponent, round-to-nearest-even,
 *     saturation). The pages name E8M0 but do not print the rule.
 *   - block geometry: §IV-B (square blocks over the two GEMM directions),
 *     32 channels x bp partner indices.
 *   - channel-batch-first layout and im2col: §IV-A, Fig. 3.
 *   - convolution, input and weight gradients: §II-A, Eqs. (1)-(3), with
 *     stride and zero padding, kernel not flipped (§II-C1 patch definition).
 *   - classic im2col and kernel flattening: §II-C1, §II-C2.
 *   - stochastic rounding of the gradient: §III-A (Philox4x32-10 words).
 *   - two-level (NVFP-style) scaling: §II-D / §III-A, Eqs. (4)-(6), square
 *     blocks of 64 (§IV-B).
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared mqref.c -o libmqref.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

/* ------------------------------------------------------------------------
 * Element formats. Index = the ABI's mq_elem value.
 * ------------------------------------------------------------------------ */
typedef struct {
  int ebits, mbits, bias;
  double maxnorm;
} mqref_fmt;

static const mqref_fmt FMT[5] = {
    {4, 3, 7, 448.0},    /* E4M3: no Inf, S.1111.111 = NaN */
    {5, 2, 15, 57344.0}, /* E5M2: IEEE-like Inf/NaN at exponent 31 */
    {2, 3, 1, 7.5},      /* E2M3 */
    {3, 2, 3, 28.0},     /* E3M2 */
    {2, 1, 1, 6.0},      /* E2M1 */
};

#ifdef _OPENMP
#include <omp.h>
#endif
/* Number of threads the parallel loops use. */
int mqref_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int mqref_elem_bits(int f) { return 1 + FMT[f].ebits + FMT[f].mbits; }

/* Largest binade exponent of the element format: floor(log2(max normal)). */
int mqref_elem_emax(int f) {
  int k;
  frexp(FMT[f].maxnorm, &k);
  return k - 1;
}

double mqref_elem_max(int f) { return FMT[f].maxnorm; }

/* Value of a code (sign-magnitude float with the format's bias). */
double mqref_decode(int f, int code) {
  const mqref_fmt* F = &FMT[f];
  int nbits = 1 + F->ebits + F->mbits;
  int s = (code >> (nbits - 1)) & 1;
  int E = (code >> F->mbits) & ((1 << F->ebits) - 1);
  int M = code & ((1 << F->mbits) - 1);
  double mag;
  if (f == 0 && E == 15 && M == 7) return NAN;
  if (f == 1 && E == 31) {
    if (M != 0) return NAN;
    return s ? -INFINITY : INFINITY;
  }
  if (E == 0)
    mag = ldexp((double)M, 1 - F->bias - F->mbits); /* subnormal */
  else
    mag = ldexp(1.0 + ldexp((double)M, -F->mbits), E - F->bias);
  return s ? -mag : mag;
}

/* Code of an already-scaled finite value: round to the nearest point of the
 * element grid (ties to the even mantissa), saturate at the largest normal,
 * keep the sign of zero. */
int mqref_encode(int f, double v) {
  const mqref_fmt* F = &FMT[f];
  int sign = signbit(v) ? 1 : 0;
  int emin = 1 - F->bias; /* exponent of the smallest normal */
  double a = fabs(v);
  int code_mag;
  if (a != 0.0) {
    int k;
    frexp(a, &k);     /* a = m * 2^k with m in [0.5, 1) */
    int ex = k - 1;   /* floor(log2 a) */
    if (ex < emin) ex = emin; /* subnormals share the spacing of the first binade */
    double q = ldexp(1.0, ex - F->mbits);  /* grid spacing around a */
    double r = nearbyint(a / q) * q;       /* round half to even */
    if (r > F->maxnorm) r = F->maxnorm;    /* saturate */
    a = r;
  }
  if (a < ldexp(1.0, emin)) {
    code_mag = (int)(a / ldexp(1.0, emin - F->mbits)); /* exponent field 0 */
  } else {
    int k;
    double m = frexp(a, &k); /* a = (2m) * 2^(k-1), 2m in [1, 2) */
    int E = k - 1 + F->bias;
    int M = (int)((2.0 * m - 1.0) * (double)(1 << F->mbits));
    code_mag = (E << F->mbits) | M;
  }
  return (sign << (F->ebits + F->mbits)) | code_mag;
}

/* Encode many already-scaled values (a convenience loop over mqref_encode). */
void mqref_encode_array(int f, const double* v, long long n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < n; i++) out[i] = (uint8_t)mqref_encode(f, v[i]);
}

/* ------------------------------------------------------------------------
 * Block quantizer over a 4-D view [A][P][B][C]:
 *   element (a,p,b,c) at src[((a*P + p)*B + b)*C + c]
 *   block (a, b, pb, cb) = { p in [pb*bp, min(P,(pb+1)*bp)),
 *                            c in [32*cb, min(C, 32*cb+32)) }
 *   scale of that block at scales[((a*B + b)*nPB + pb)*nCB + cb]
 * Activations/gradients [H][W][N][C]: A = H*W, P = N, B = 1.
 * Weights [Cout][Kh][Kw][Cin]:         A = 1, P = Cout, B = Kh*Kw.
 * im2col output [Ho][Wo][N][Kh][Kw][C]: A = Ho*Wo, P = N, B = Kh*Kw.
 * Line blocks of 32 along the rows of a matrix [R][L]: A = R, P = 1, B = 1,
 *   bp = 1, C = L.
 * Logical codes (one byte per element, same index as src) go to `codes`.
 * Returns the number of element quantizations performed.
 * ------------------------------------------------------------------------ */
long long mqref_quantize_view(int f, int bp, const float* src, long long A, long long P,
                              long long B, long long C, uint8_t* codes, uint8_t* scales) {
  const long long nPB = (P + bp - 1) / bp, nCB = (C + 31) / 32;
  const int emax = mqref_elem_emax(f);
  long long count = 0;
#pragma omp parallel for collapse(2) reduction(+ : count) schedule(static)
  for (long long a = 0; a < A; a++)
    for (long long b = 0; b < B; b++)
      for (long long pb = 0; pb < nPB; pb++)
        for (long long cb = 0; cb < nCB; cb++) {
          long long p0 = pb * bp, p1 = p0 + bp < P ? p0 + bp : P;
          long long c0 = cb * 32, c1 = c0 + 32 < C ? c0 + 32 : C;
          /* amax over the block, and whether it holds a non-finite value */
          double amax = 0.0;
          int nonfinite = 0;
          for (long long p = p0; p < p1; p++)
            for (long long c = c0; c < c1; c++) {
              double x = src[((a * P + p) * B + b) * C + c];
              if (!isfinite(x)) nonfinite = 1;
              else if (fabs(x) > amax) amax = fabs(x);
            }
          int S;
          if (nonfinite) {
            S = 255;
          } else {
            int e;
            if (amax == 0.0) {
              e = -127;
            } else {
              int k;
              frexp(amax, &k);
              e = (k - 1) - emax; /* floor(log2 amax) - emax_elem */
              if (e < -127) e = -127;
              if (e > 127) e = 127;
            }
            S = e + 127;
          }
          scales[((a * B + b) * nPB + pb) * nCB + cb] = (uint8_t)S;
          for (long long p = p0; p < p1; p++)
            for (long long c = c0; c < c1; c++) {
              long long i = ((a * P + p) * B + b) * C + c;
              if (S == 255)
                codes[i] = 0;
              else
                codes[i] = (uint8_t)mqref_encode(f, ldexp((double)src[i], 127 - S));
            }
          count += (p1 - p0) * (c1 - c0);
        }
  return count;
}

/* ------------------------------------------------------------------------
 * Stochastic rounding of the gradient (§III-A: activations and weights round
 * to nearest, "stochastic rounding is performed on the gradient").
 * A scaled value between two neighbouring points lo < hi of the element grid
 * rounds up with probability (v - lo) / (hi - lo): with the random word r
 * (uniform 32-bit) and T = floor(2^32 (v - lo) / (hi - lo)), it takes hi when
 * r < T, else lo; points of the grid stay; results above the largest normal
 * saturate to it, as with round-to-nearest. The block scale follows the same
 * rule as round-to-nearest (the scale is not rounded stochastically).
 * ------------------------------------------------------------------------ */

/* Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
 * Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC'11): ten rounds of
 * two 32x32->64-bit multiplications with the published multipliers and key
 * increments, the first round with the original key. */
void mqref_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; r++) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1, n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The random word of element (memory row `row`, channel c) of a tensor
 * quantized with `seed`: word c mod 4 of Philox4x32-10 at counter
 * (row, floor(c / 4), 0, 0) with key (low, high 32 bits of seed). */
uint32_t mqref_sr_word(uint64_t seed, long long row, long long c) {
  const uint32_t ctr[4] = {(uint32_t)row, (uint32_t)(c >> 2), 0u, 0u};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  mqref_philox4x32_10(ctr, key, out);
  return out[c & 3];
}

/* Code of an already-scaled finite value, rounded stochastically with the
 * random word r. */
int mqref_encode_sr(int f, double v, uint32_t r) {
  const mqref_fmt* F = &FMT[f];
  const int emin = 1 - F->bias;
  const double a = fabs(v);
  double res = 0.0;
  if (a != 0.0) {
    int k;
    frexp(a, &k);
    int ex = k - 1;            /* floor(log2 a) */
    if (ex < emin) ex = emin;  /* subnormals share the spacing of the first binade */
    const double q = ldexp(1.0, ex - F->mbits); /* grid spacing around a */
    const double t = a / q, lo = floor(t);
    const double T = floor((t - lo) * 4294967296.0);
    res = ((double)r < T ? lo + 1.0 : lo) * q;
    if (res > F->maxnorm) res = F->maxnorm;
  }
  return mqref_encode(f, signbit(v) ? -res : res); /* res is a grid point: encoded exactly */
}

/* mqref_quantize_view with stochastic rounding of the elements; element
 * (a, p, b, c) lies on memory row (a*P + p)*B + b, which with c picks its
 * random word (mqref_sr_word). */
long long mqref_quantize_view_sr(int f, int bp, const float* src, long long A, long long P, long long B,
                                 long long C, uint64_t seed, uint8_t* codes, uint8_t* scales) {
  const long long nPB = (P + bp - 1) / bp, nCB = (C + 31) / 32;
  const int emax = mqref_elem_emax(f);
  long long count = 0;
#pragma omp parallel for collapse(2) reduction(+ : count) schedule(static)
  for (long long a = 0; a < A; a++)
    for (long long b = 0; b < B; b++)
      for (long long pb = 0; pb < nPB; pb++)
        for (long long cb = 0; cb < nCB; cb++) {
          long long p0 = pb * bp, p1 = p0 + bp < P ? p0 + bp : P;
          long long c0 = cb * 32, c1 = c0 + 32 < C ? c0 + 32 : C;
          double amax = 0.0;
          int nonfinite = 0;
          for (long long p = p0; p < p1; p++)
            for (long long c = c0; c < c1; c++) {
              double x = src[((a * P + p) * B + b) * C + c];
              if (!isfinite(x)) nonfinite = 1;
              else if (fabs(x) > amax) amax = fabs(x);
            }
          int S;
          if (nonfinite) {
            S = 255;
          } else {
            int e;
            if (amax == 0.0) {
              e = -127;
            } else {
              int k;
              frexp(amax, &k);
              e = (k - 1) - emax;
              if (e < -127) e = -127;
              if (e > 127) e = 127;
            }
            S = e + 127;
          }
          scales[((a * B + b) * nPB + pb) * nCB + cb] = (uint8_t)S;
          for (long long p = p0; p < p1; p++)
            for (long long c = c0; c < c1; c++) {
              const long long row = (a * P + p) * B + b, i = row * C + c;
              if (S == 255)
                codes[i] = 0;
              else
                codes[i] = (uint8_t)mqref_encode_sr(f, ldexp((double)src[i], 127 - S),
                                                    mqref_sr_word(seed, row, c));
            }
          count += (p1 - p0) * (c1 - c0);
        }
  return count;
}

/* ------------------------------------------------------------------------
 * Two-level (NVFP-style) microscaling, Eqs. (4)-(6) of §II-D / §III-A: one
 * FP32 scale for the whole tensor and one E4M3 scale per block,
 *   T   = max|X| / (448 * m)                     (m = largest element value)
 *   B_i = E4M3(max|X_i| / (T * m)), rounded to nearest
 *   q   = element code of X_i / (B_i * T), rounded to nearest even
 * with the pages' square blocks of B = 64 elements: 8 channels x 8 partner
 * indices inside one pixel (activations, gradients) or one tap (weights).
 * T, the divisions and products are fp32 operations, as the formula is
 * written for an FP32 tensor scale. Readings where the pages are silent: an
 * all-zero tensor gets T = 0 and all-zero codes; a block whose E4M3 scale
 * rounds to 0 gets all-zero codes; non-finite values are left out of T and
 * their block gets the E4M3 NaN scale (0x7F) and zero codes.
 * Block scale of block (a, b, pb, cb) at bscales[((a*B + b)*nPB8 + pb)*nCB8 + cb].
 * Returns T.
 * ------------------------------------------------------------------------ */
float mqref_nvfp_quantize_view(int f, const float* src, long long A, long long P, long long B, long long C,
                               uint8_t* codes, uint8_t* bscales) {
  const long long nPB = (P + 7) / 8, nCB = (C + 7) / 8, n = A * P * B * C;
  float amax = 0.0f;
  for (long long i = 0; i < n; i++)
    if (isfinite(src[i]) && fabsf(src[i]) > amax) amax = fabsf(src[i]);
  const float m = (float)FMT[f].maxnorm;
  const float T = amax / (448.0f * m);
  const float Tm = T * m;
#pragma omp parallel for collapse(2) schedule(static)
  for (long long a = 0; a < A; a++)
    for (long long b = 0; b < B; b++)
      for (long long pb = 0; pb < nPB; pb++)
        for (long long cb = 0; cb < nCB; cb++) {
          const long long p0 = pb * 8, p1 = p0 + 8 < P ? p0 + 8 : P;
          const long long c0 = cb * 8, c1 = c0 + 8 < C ? c0 + 8 : C;
          float bmax = 0.0f;
          int nonfinite = 0;
          for (long long p = p0; p < p1; p++)
            for (long long c = c0; c < c1; c++) {
              const float x = src[((a * P + p) * B + b) * C + c];
              if (!isfinite(x)) nonfinite = 1;
              else if (fabsf(x) > bmax) bmax = fabsf(x);
            }
          int sc;
          if (nonfinite) sc = 0x7F;
          else if (T == 0.0f) sc = 0;
          else sc = mqref_encode(0, (double)(bmax / Tm)); /* E4M3, nearest even, saturating */
          bscales[((a * B + b) * nPB + pb) * nCB + cb] = (uint8_t)sc;
          const float d = (float)mqref_decode(0, sc) * T;
          for (long long p = p0; p < p1; p++)
            for (long long c = c0; c < c1; c++) {
              const long long i = ((a * P + p) * B + b) * C + c;
              if (nonfinite || sc == 0) codes[i] = 0;
              else codes[i] = (uint8_t)mqref_encode(f, (double)(src[i] / d));
            }
        }
  return T;
}

/* Dequantized values of the same view: code value * B_i * T (fp64). */
void mqref_nvfp_dequant_view(int f, const uint8_t* codes, const uint8_t* bscales, float T, long long A, long long P,
                             long long B, long long C, double* out) {
  const long long nPB = (P + 7) / 8, nCB = (C + 7) / 8;
#pragma omp parallel for collapse(2) schedule(static)
  for (long long a = 0; a < A; a++)
    for (long long p = 0; p < P; p++)
      for (long long b = 0; b < B; b++)
        for (long long c = 0; c < C; c++) {
          const long long i = ((a * P + p) * B + b) * C + c;
          const int sc = bscales[((a * B + b) * nPB + p / 8) * nCB + c / 8];
          out[i] = mqref_decode(f, codes[i]) * mqref_decode(0, sc) * (double)T;
        }
}

/* Dequantize (fake quantization): code value times 2^(S-127). Same view. */
void mqref_dequant_view(int f, int bp, const uint8_t* codes, const uint8_t* scales, long long A,
                        long long P, long long B, long long C, double* out) {
  const long long nPB = (P + bp - 1) / bp, nCB = (C + 31) / 32;
#pragma omp parallel for collapse(2) schedule(static)
  for (long long a = 0; a < A; a++)
    for (long long p = 0; p < P; p++)
      for (long long b = 0; b < B; b++)
        for (long long c = 0; c < C; c++) {
          long long i = ((a * P + p) * B + b) * C + c;
          int S = scales[((a * B + b) * nPB + p / bp) * nCB + c / 32];
          out[i] = (S == 255) ? NAN : ldexp(mqref_decode(f, codes[i]), S - 127);
        }
}

/* ------------------------------------------------------------------------
 * Packing of logical codes into rows of 32-code runs (the library's byte
 * layout): run cb of a row holds channels 32cb..32cb+31; code j of a run
 * occupies bits [j*bits, (j+1)*bits) of the run read as a little-endian
 * integer; runs are 32*bits/8 bytes; padding channels are 0.
 * ------------------------------------------------------------------------ */
long long mqref_row_bytes(int f, long long C) {
  return ((C + 31) / 32) * (32LL * mqref_elem_bits(f) / 8);
}

void mqref_pack_rows(int f, const uint8_t* logical, long long rows, long long C, uint8_t* out) {
  const int bits = mqref_elem_bits(f);
  const long long rb = mqref_row_bytes(f, C), run = 32LL * bits / 8;
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; r++) {
    uint8_t* o = out + r * rb;
    memset(o, 0, (size_t)rb);
    for (long long c = 0; c < C; c++) {
      int code = logical[r * C + c];
      long long bit0 = (c / 32) * run * 8 + (c % 32) * bits;
      for (int i = 0; i < bits; i++)
        if ((code >> i) & 1) o[(bit0 + i) / 8] |= (uint8_t)(1u << ((bit0 + i) % 8));
    }
  }
}

void mqref_unpack_rows(int f, const uint8_t* packed, long long rows, long long C, uint8_t* logical) {
  const int bits = mqref_elem_bits(f);
  const long long rb = mqref_row_bytes(f, C), run = 32LL * bits / 8;
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; r++) {
    const uint8_t* in = packed + r * rb;
    for (long long c = 0; c < C; c++) {
      long long bit0 = (c / 32) * run * 8 + (c % 32) * bits;
      int code = 0;
      for (int i = 0; i < bits; i++)
        if ((in[(bit0 + i) / 8] >> ((bit0 + i) % 8)) & 1) code |= 1 << i;
      logical[r * C + c] = (uint8_t)code;
    }
  }
}

/* ------------------------------------------------------------------------
 * Convolution geometry: cv = {n, cin, h, w, cout, kh, kw, sh, sw, ph, pw}
 * ------------------------------------------------------------------------ */
enum { CN, CCI, CH, CW, CCO, CKH, CKW, CSH, CSW, CPH, CPW };
static long long out_h(const int* cv) { return (cv[CH] + 2 * cv[CPH] - cv[CKH]) / cv[CSH] + 1; }
static long long out_w(const int* cv) { return (cv[CW] + 2 * cv[CPW] - cv[CKW]) / cv[CSW] + 1; }

/* Channel-batch-first im2col (§IV-A) of logical codes and their scales:
 *   X'[ho][wo][n][kh][kw][c] = X[ho*s+kh-p][wo*s+kw-p][n][c]
 *   scale of X' block (ho,wo,kh,kw,nb,cb) = scale of X block (hi,wi,nb,cb)
 * Out-of-image positions: code 0, scale byte 0. */
void mqref_cbf_im2col_codes(const int* cv, int bp, const uint8_t* xc, const uint8_t* xs,
                            uint8_t* oc, uint8_t* os) {
  const long long N = cv[CN], C = cv[CCI], H = cv[CH], W = cv[CW], KH = cv[CKH], KW = cv[CKW];
  const long long Ho = out_h(cv), Wo = out_w(cv);
  const long long nPB = (N + bp - 1) / bp, nCB = (C + 31) / 32;
#pragma omp parallel for collapse(2) schedule(static)
  for (long long ho = 0; ho < Ho; ho++)
    for (long long wo = 0; wo < Wo; wo++)
      for (long long kh = 0; kh < KH; kh++)
        for (long long kw = 0; kw < KW; kw++) {
          long long hi = ho * cv[CSH] + kh - cv[CPH], wi = wo * cv[CSW] + kw - cv[CPW];
          int inside = hi >= 0 && hi < H && wi >= 0 && wi < W;
          for (long long n = 0; n < N; n++)
            for (long long c = 0; c < C; c++)
              oc[((((ho * Wo + wo) * N + n) * KH + kh) * KW + kw) * C + c] =
                  inside ? xc[((hi * W + wi) * N + n) * C + c] : 0;
          for (long long pb = 0; pb < nPB; pb++)
            for (long long cb = 0; cb < nCB; cb++)
              os[((((ho * Wo + wo) * KH + kh) * KW + kw) * nPB + pb) * nCB + cb] =
                  inside ? xs[((hi * W + wi) * nPB + pb) * nCB + cb] : 0;
        }
}

/* The same rearrangement of an fp32 CBF tensor (0.0 outside the image). */
void mqref_cbf_im2col_f32(const int* cv, const float* x, float* out) {
  const long long N = cv[CN], C = cv[CCI], H = cv[CH], W = cv[CW], KH = cv[CKH], KW = cv[CKW];
  const long long Ho = out_h(cv), Wo = out_w(cv);
#pragma omp parallel for collapse(2) schedule(static)
  for (long long ho = 0; ho < Ho; ho++)
    for (long long wo = 0; wo < Wo; wo++)
      for (long long n = 0; n < N; n++)
        for (long long kh = 0; kh < KH; kh++)
          for (long long kw = 0; kw < KW; kw++) {
            long long hi = ho * cv[CSH] + kh - cv[CPH], wi = wo * cv[CSW] + kw - cv[CPW];
            int inside = hi >= 0 && hi < H && wi >= 0 && wi < W;
            for (long long c = 0; c < C; c++)
              out[((((ho * Wo + wo) * N + n) * KH + kh) * KW + kw) * C + c] =
                  inside ? x[((hi * W + wi) * N + n) * C + c] : 0.0f;
          }
}

/* Classic im2col (§II-C1) with channel-major patch flattening (§II-C2):
 *   X'[m][k], m = (ho*Wo + wo)*N + n, k = (ci*KH + kh)*KW + kw,
 *   X'[m][k] = X[ho*s+kh-p][wo*s+kw-p][n][ci] (x in CBF order), 0 outside. */
void mqref_classic_im2col(const int* cv, const float* x, float* out) {
  const long long N = cv[CN], C = cv[CCI], H = cv[CH], W = cv[CW], KH = cv[CKH], KW = cv[CKW];
  const long long Ho = out_h(cv), Wo = out_w(cv), K = C * KH * KW;
#pragma omp parallel for collapse(2) schedule(static)
  for (long long ho = 0; ho < Ho; ho++)
    for (long long wo = 0; wo < Wo; wo++)
      for (long long n = 0; n < N; n++)
        for (long long ci = 0; ci < C; ci++)
          for (long long kh = 0; kh < KH; kh++)
            for (long long kw = 0; kw < KW; kw++) {
              long long hi = ho * cv[CSH] + kh - cv[CPH], wi = wo * cv[CSW] + kw - cv[CPW];
              int inside = hi >= 0 && hi < H && wi >= 0 && wi < W;
              out[((ho * Wo + wo) * N + n) * K + (ci * KH + kh) * KW + kw] =
                  inside ? x[((hi * W + wi) * N + n) * C + ci] : 0.0f;
            }
}

/* col2im: the adjoint of classic im2col. Every X' entry is added back to the
 * X position it was copied from; out-of-image entries are dropped.
 * gcol [M][K] as above, gx CBF [H][W][N][C]. */
void mqref_col2im(const int* cv, const double* gcol, double* gx) {
  const long long N = cv[CN], C = cv[CCI], H = cv[CH], W = cv[CW], KH = cv[CKH], KW = cv[CKW];
  const long long Ho = out_h(cv), Wo = out_w(cv), K = C * KH * KW;
  memset(gx, 0, sizeof(double) * (size_t)(H * W * N * C));
#pragma omp parallel for schedule(static)
  for (long long n = 0; n < N; n++) /* each thread owns one sample: no races */
    for (long long ho = 0; ho < Ho; ho++)
      for (long long wo = 0; wo < Wo; wo++)
        for (long long ci = 0; ci < C; ci++)
          for (long long kh = 0; kh < KH; kh++)
            for (long long kw = 0; kw < KW; kw++) {
              long long hi = ho * cv[CSH] + kh - cv[CPH], wi = wo * cv[CSW] + kw - cv[CPW];
              if (hi < 0 || hi >= H || wi < 0 || wi >= W) continue;
              gx[((hi * W + wi) * N + n) * C + ci] +=
                  gcol[((ho * Wo + wo) * N + n) * K + (ci * KH + kh) * KW + kw];
            }
}

/* ------------------------------------------------------------------------
 * Direct convolution, Eqs. (1)-(3), fp64, NCHW index order as in §II-A:
 *   x [N][Cin][H][W], w [Cout][Cin][Kh][Kw], y/dy [N][Cout][Ho][Wo]
 * ------------------------------------------------------------------------ */
#define X4(t, a, b, c, d, B_, C_, D_) t[(((long long)(a) * (B_) + (b)) * (C_) + (c)) * (D_) + (d)]

/* Eq. (1): Y = W * X */
void mqref_conv_fwd(const int* cv, const double* x, const double* w, double* y) {
  const long long N = cv[CN], CI = cv[CCI], H = cv[CH], W = cv[CW], CO = cv[CCO];
  const long long KH = cv[CKH], KW = cv[CKW], Ho = out_h(cv), Wo = out_w(cv);
#pragma omp parallel for collapse(2) schedule(static)
  for (long long n = 0; n < N; n++)
    for (long long co = 0; co < CO; co++)
      for (long long ho = 0; ho < Ho; ho++)
        for (long long wo = 0; wo < Wo; wo++) {
          double acc = 0.0;
          for (long long ci = 0; ci < CI; ci++)
            for (long long kh = 0; kh < KH; kh++)
              for (long long kw = 0; kw < KW; kw++) {
                long long hi = ho * cv[CSH] + kh - cv[CPH], wi = wo * cv[CSW] + kw - cv[CPW];
                if (hi < 0 || hi >= H || wi < 0 || wi >= W) continue;
                acc += X4(w, co, ci, kh, kw, CI, KH, KW) * X4(x, n, ci, hi, wi, CI, H, W);
              }
          X4(y, n, co, ho, wo, CO, Ho, Wo) = acc;
        }
}

/* Eq. (2): G_X = W^T * G_Y, as the scatter of every forward product back to
 * its input position. */
void mqref_conv_dgrad(const int* cv, const double* dy, const double* w, double* dx) {
  const long long N = cv[CN], CI = cv[CCI], H = cv[CH], W = cv[CW], CO = cv[CCO];
  const long long KH = cv[CKH], KW = cv[CKW], Ho = out_h(cv), Wo = out_w(cv);
#pragma omp parallel for collapse(2) schedule(static)
  for (long long n = 0; n < N; n++)
    for (long long ci = 0; ci < CI; ci++) { /* this thread owns dx[n][ci] */
      for (long long i = 0; i < H * W; i++) dx[(n * CI + ci) * H * W + i] = 0.0;
      for (long long co = 0; co < CO; co++)
        for (long long ho = 0; ho < Ho; ho++)
          for (long long wo = 0; wo < Wo; wo++)
            for (long long kh = 0; kh < KH; kh++)
              for (long long kw = 0; kw < KW; kw++) {
                long long hi = ho * cv[CSH] + kh - cv[CPH], wi = wo * cv[CSW] + kw - cv[CPW];
                if (hi < 0 || hi >= H || wi < 0 || wi >= W) continue;
                X4(dx, n, ci, hi, wi, CI, H, W) +=
                    X4(w, co, ci, kh, kw, CI, KH, KW) * X4(dy, n, co, ho, wo, CO, Ho, Wo);
              }
    }
}

/* Eq. (3): G_W[co,ci] = sum_n G_Y[n,co] * X[n,ci] (correlation). */
void mqref_conv_wgrad(const int* cv, const double* dy, const double* x, double* dw) {
  const long long N = cv[CN], CI = cv[CCI], H = cv[CH], W = cv[CW], CO = cv[CCO];
  const long long KH = cv[CKH], KW = cv[CKW], Ho = out_h(cv), Wo = out_w(cv);
#pragma omp parallel for collapse(2) schedule(static)
  for (long long co = 0; co < CO; co++)
    for (long long ci = 0; ci < CI; ci++)
      for (long long kh = 0; kh < KH; kh++)
        for (long long kw = 0; kw < KW; kw++) {
          double acc = 0.0;
          for (long long n = 0; n < N; n++)
            for (long long ho = 0; ho < Ho; ho++)
              for (long long wo = 0; wo < Wo; wo++) {
                long long hi = ho * cv[CSH] + kh - cv[CPH], wi = wo * cv[CSW] + kw - cv[CPW];
                if (hi < 0 || hi >= H || wi < 0 || wi >= W) continue;
                acc += X4(dy, n, co, ho, wo, CO, Ho, Wo) * X4(x, n, ci, hi, wi, CI, H, W);
              }
          X4(dw, co, ci, kh, kw, CI, KH, KW) = acc;
        }
}

/* Single outputs of the three operations, for sampled checks of large
 * problems. idx holds 4 ints per point:
 *   fwd   (n, co, ho, wo)   dgrad (n, ci, h, w)   wgrad (co, ci, kh, kw)
 * The dgrad point is the gather form of Eq. (2): input position h receives
 * tap kh from output row ho exactly when ho*s + kh - p = h. */
void mqref_conv_fwd_points(const int* cv, const double* x, const double* w, long long npts,
                           const int* idx, double* out) {
  const long long CI = cv[CCI], H = cv[CH], W = cv[CW], KH = cv[CKH], KW = cv[CKW];
#pragma omp parallel for schedule(dynamic, 16)
  for (long long t = 0; t < npts; t++) {
    long long n = idx[4 * t], co = idx[4 * t + 1], ho = idx[4 * t + 2], wo = idx[4 * t + 3];
    double acc = 0.0;
    for (long long ci = 0; ci < CI; ci++)
      for (long long kh = 0; kh < KH; kh++)
        for (long long kw = 0; kw < KW; kw++) {
          long long hi = ho * cv[CSH] + kh - cv[CPH], wi = wo * cv[CSW] + kw - cv[CPW];
          if (hi < 0 || hi >= H || wi < 0 || wi >= W) continue;
          acc += X4(w, co, ci, kh, kw, CI, KH, KW) * X4(x, n, ci, hi, wi, CI, H, W);
        }
    out[t] = acc;
  }
}

void mqref_conv_dgrad_points(const int* cv, const double* dy, const double* w, long long npts,
                             const int* idx, double* out) {
  const long long CI = cv[CCI], CO = cv[CCO], KH = cv[CKH], KW = cv[CKW];
  const long long Ho = out_h(cv), Wo = out_w(cv);
#pragma omp parallel for schedule(dynamic, 16)
  for (long long t = 0; t < npts; t++) {
    long long n = idx[4 * t], ci = idx[4 * t + 1], h = idx[4 * t + 2], wpos = idx[4 * t + 3];
    double acc = 0.0;
    for (long long co = 0; co < CO; co++)
      for (long long kh = 0; kh < KH; kh++)
        for (long long kw = 0; kw < KW; kw++) {
          long long th = h + cv[CPH] - kh, tw = wpos + cv[CPW] - kw;
          if (th < 0 || tw < 0 || th % cv[CSH] != 0 || tw % cv[CSW] != 0) continue;
          long long ho = th / cv[CSH], wo = tw / cv[CSW];
          if (ho >= Ho || wo >= Wo) continue;
          acc += X4(w, co, ci, kh, kw, CI, KH, KW) * X4(dy, n, co, ho, wo, CO, Ho, Wo);
        }
    out[t] = acc;
  }
}

void mqref_conv_wgrad_points(const int* cv, const double* dy, const double* x, long long npts,
                             const int* idx, double* out) {
  const long long N = cv[CN], CI = cv[CCI], H = cv[CH], W = cv[CW], CO = cv[CCO];
  const long long Ho = out_h(cv), Wo = out_w(cv);
#pragma omp parallel for schedule(dynamic, 4)
  for (long long t = 0; t < npts; t++) {
    long long co = idx[4 * t], ci = idx[4 * t + 1], kh = idx[4 * t + 2], kw = idx[4 * t + 3];
    double acc = 0.0;
    for (long long n = 0; n < N; n++)
      for (long long ho = 0; ho < Ho; ho++)
        for (long long wo = 0; wo < Wo; wo++) {
          long long hi = ho * cv[CSH] + kh - cv[CPH], wi = wo * cv[CSW] + kw - cv[CPW];
          if (hi < 0 || hi >= H || wi < 0 || wi >= W) continue;
          acc += X4(dy, n, co, ho, wo, CO, Ho, Wo) * X4(x, n, ci, hi, wi, CI, H, W);
        }
    out[t] = acc;
  }
}
