// gemm_wgrad.hip -- backward-weight GEMM launcher, split-K reduction and
// workspace sizes of the GEMM entry points.
#include "gemm_kernel.h"

namespace mq {

// The GEMM launch of the 6/4-bit in-place path (gemm_wgrad_sub.hip, its own
// translation unit so its kernels compile in parallel).
hipError_t launch_wgrad_nat_sub(int fa, int fb, const WgradNatSubProb& q, int Ma, int Nb, int S, hipStream_t st);

// out[i] = sum_z part[z][i] in a fixed order (deterministic): the G thread
// groups of a block sum the slices z = g, g+G, g+2G, ... in turn, then the G
// group sums are added in order g = 0..G-1. VEC: four consecutive outputs
// per thread with 16-byte loads (n a multiple of 4).
constexpr int kRedG = 16;
template <bool VEC>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            float* __restrict__ out, long long n,
                                                            int splits) {
  constexpr int C = 256 / kRedG;  // output columns per block
  constexpr int E = VEC ? 4 : 1;  // outputs per column
  __shared__ float red[kRedG][C][E];
  const int tc = threadIdx.x % C, g = threadIdx.x / C;
  const long long i0 = ((long long)blockIdx.x * C + tc) * E;
  float s[E];
#pragma unroll
  for (int e = 0; e < E; e++) s[e] = 0.0f;
  if (i0 < n) {
    // U slices in flight per thread: their loads go out together, then they
    // are added in slice order
    constexpr int U = 4;
    for (int z0 = g; z0 < splits; z0 += U * kRedG) {
      float v[U][E];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int z = z0 + u * kRedG;
        if constexpr (VEC) {
          typedef float v4f __attribute__((ext_vector_type(4)));
          v4f a = {0.0f, 0.0f, 0.0f, 0.0f};
          if (z < splits) a = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(part + (long long)z * n + i0));
          v[u][0] = a[0]; v[u][1] = a[1]; v[u][2] = a[2]; v[u][3] = a[3];
        } else {
          v[u][0] = z < splits ? __builtin_nontemporal_load(part + (long long)z * n + i0) : 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; u++)
        if (z0 + u * kRedG < splits) {
#pragma unroll
          for (int e = 0; e < E; e++) s[e] += v[u][e];
        }
    }
  }
#pragma unroll
  for (int e = 0; e < E; e++) red[g][tc][e] = s[e];
  __syncthreads();
  if (g == 0 && i0 < n) {
#pragma unroll
    for (int e = 0; e < E; e++) {
      float t = red[0][tc][e];
      for (int k = 1; k < kRedG; k++) t += red[k][tc][e];
      s[e] = t;
    }
    if constexpr (VEC) {
      *reinterpret_cast<float4*>(out + i0) = make_float4(s[0], s[1], s[2], s[3]);
    } else {
      out[i0] = s[0];
    }
  }
}

// ---------------------------------------------------------------------------
// Format and tile dispatch
// ---------------------------------------------------------------------------

// K-steps of the backward-weight GEMM: kps N blocks per output pixel, or
// kps output pixels along wo when N fits one block (kps = 4 when the
// K-blocks are half blocks, else 2).
struct WgradSteps { int pair_w, nsub, total; };
static WgradSteps wgrad_steps(const Conv& cv, int kps) {
  const int nNB = ceil_div(cv.n, 32);
  WgradSteps s;
  s.pair_w = nNB == 1;
  s.nsub = s.pair_w ? ceil_div(cv.wo(), kps) : ceil_div(nNB, kps);
  s.total = s.pair_w ? cv.ho() * s.nsub : cv.ho() * cv.wo() * s.nsub;
  return s;
}

static int wgrad_splits(const Conv& cv, int fdy, int fx) {
  const long long npix = (long long)cv.ho() * cv.wo();
  const long long nNB = ceil_div(cv.n, 32);
  const long long ops = npix * cv.cout * nNB * run_bytes(fdy) + (long long)cv.h * cv.w * cv.cin * nNB * run_bytes(fx);
  // the same count for either step size: capped by the number of four-block steps
  const WgradSteps ks = wgrad_steps(cv, 4);
  const long long nkb = (long long)cv.ho() * cv.wo() * ceil_div(cv.n, 32);
  // workgroups of one wave group (full K-blocks) run one per CU at the
  // two-times cap on the large layers; partial sums of up to eight times the
  // operand bytes let two run per CU, which measured faster despite the
  // extra bytes (3x3 stride-2 layer, N 32, 128 -> 256 channels, 160 x 160:
  // 97.8 -> 83.7 us at four times; 3x3 layer, N 128, 256 channels, 20 x 20:
  // 57.7 -> 49.2 us going from four to eight times); the two-group
  // half-block kernel keeps the tighter cap
  const int gb = cv.cin % 32 == 0 ? 32 : 0;
  const bool half = half_k_blocks(32, gb, cv.n <= 16, fdy, fx);
  int s = splitk_slices(cv.cout, (long long)cv.kh * cv.kw * cv.cin, nkb, ops, half ? 2 : 8, gb >= 8);
  if (s > ks.total) s = ks.total;
  if (s < 1) s = 1;
  return s;
}

// How the backward-weight GEMM reads its operands and how much workspace it
// uses: with 8-bit gradient codes, the codes are read where quantization
// left them (K-major staging) when a 16-channel chunk of B stays in one tap
// and a K-block's lines are the N values of one pixel (natural: 8-bit
// activation codes; natural_sub: 6- or 4-bit ones, read with the sub-byte
// transposing LDS reads); otherwise the activation (mixed: 8-bit gradient
// codes), or both, are first re-laid with runs along N. Workspace: [re-laid
// dY][re-laid X][fp32 partial sums of the S slices], each part present only
// when used.
struct WgradPlan {
  bool natural, natural_sub, mixed, half;
  int kps, S;
  size_t dyt_b, xt_b, part_b;
};
static WgradPlan wgrad_plan(const Conv& cv, int fdy, int fx) {
  WgradPlan w;
  const int ga = 32, gb = cv.cin % 32 == 0 ? 32 : 0, khalf = cv.n <= 16;
  const bool kext_ok = cv.n <= 32 || cv.n % 32 == 0;
  w.natural = fdy <= 1 && fx <= 1 && cv.cin % 16 == 0 && kext_ok;
  w.natural_sub = fdy <= 1 && fx >= 2 && cv.cin % 16 == 0 && kext_ok;
  w.mixed = !w.natural && !w.natural_sub && fdy <= 1 && kext_ok;
  w.half = !w.natural && !w.natural_sub && half_k_blocks(ga, gb, khalf, fdy, fx);
  // half K-blocks take four K-blocks per step and two wave groups per
  // workgroup, so half as many slices cover the K range
  w.kps = half_k_blocks(ga, gb, khalf, fdy, fx) ? 4 : 2;
  const int S0 = wgrad_splits(cv, fdy, fx);
  w.S = w.kps == 4 ? ceil_div(S0, 2) : S0;
  // the 256 x 128 tile runs two wave groups per workgroup as well (one
  // workgroup of eight waves per CU where two of four ran): half as many
  // slices, when the launch still takes that tile for them
  if (w.kps == 2 && cv.cin % 32 == 0 && w.S > 1) {
    const int S2 = ceil_div(w.S, 2);
    if (choose_tile(cv.cout, (long long)cv.kh * cv.kw * cv.cin, S2).id == 2) w.S = S2;
  }
  const long long npix_o = (long long)cv.ho() * cv.wo();
  const bool in_place = w.natural || w.natural_sub;
  w.dyt_b = (!in_place && !w.mixed) ? align256(transposed_bytes(fdy, npix_o, cv.n, 1, cv.cout)) : 0;
  w.xt_b = !in_place ? align256(transposed_bytes(fx, (long long)cv.h * cv.w, cv.n, 1, cv.cin)) : 0;
  w.part_b = w.S > 1 ? align256((size_t)w.S * cv.cout * cv.kh * cv.kw * cv.cin * 4) : 0;
  return w;
}

size_t gemm_workspace_bytes(const Conv& cv, int op, int fa, int fb) {
  if (op == 0) return 0;
  if (op == 1) {  // 6/4-bit W re-laid with runs along Cout (8-bit W is read in place)
    return fb <= 1 ? 0 : align256(transposed_bytes(fb, 1, cv.cout, (long long)cv.kh * cv.kw, cv.cin));
  }
  // op 2: fa = gradient format, fb = activation format
  const WgradPlan w = wgrad_plan(cv, fa, fb);
  return w.dyt_b + w.xt_b + w.part_b;
}

// Offsets of the kernels' buffer loads are 32-bit: every operand buffer plus
// the bias in front of it (padding, backward taps) must stay below the
// offset that marks invalid blocks. The same quantities as the launchers.
bool gemm_offsets_ok(const Conv& cv, int op, int fa, int fb, int bpa) {
  if (op == 0) {  // forward: fa = X format, bpa = X bp
    const long long ncb = ceil_div(cv.cin, 32), xrb = ncb * run_bytes(fa), xnPB = ceil_div(cv.n, bpa);
    const long long lead = (long long)cv.ph * cv.w + cv.pw;
    return offsets_fit((long long)cv.h * cv.w * cv.n * xrb, lead * cv.n * xrb) &&
           offsets_fit((long long)cv.h * cv.w * xnPB * ncb, lead * xnPB * ncb);
  }
  if (op == 1) {  // backward-data: fa = dY format, bpa = dY bp
    const long long ncob = ceil_div(cv.cout, 32), dyrb = ncob * run_bytes(fa), dynPB = ceil_div(cv.n, bpa);
    const long long dmax = (long long)(ceil_div(cv.kh, cv.sh) - 1) * cv.wo() + (ceil_div(cv.kw, cv.sw) - 1);
    return offsets_fit((long long)cv.ho() * cv.wo() * cv.n * dyrb, dmax * cv.n * dyrb) &&
           offsets_fit((long long)cv.ho() * cv.wo() * dynPB * ncob, dmax * dynPB * ncob);
  }
  // backward-weight: fa = dY format, fb = X format
  const WgradPlan w = wgrad_plan(cv, fa, fb);
  const long long nNB = ceil_div(cv.n, 32), ncbi = ceil_div(cv.cin, 32);
  const long long xRB = w.half ? 16 : run_bytes(fb);
  const long long lead = (long long)cv.ph * cv.w + cv.pw;
  bool ok = offsets_fit((long long)cv.h * cv.w * nNB * ncbi, lead * nNB * ncbi);
  if (w.natural || w.natural_sub) {
    const long long xrb = row_bytes(fb, cv.cin);
    ok = ok && offsets_fit((long long)cv.h * cv.w * cv.n * xrb, lead * cv.n * xrb);
  } else {
    ok = ok && offsets_fit((long long)cv.h * cv.w * cv.cin * nNB * xRB, lead * cv.cin * nNB * xRB);
  }
  return ok;
}

hipError_t launch_backward_weight(const Conv& cv, MxView dy, MxView x, float* dw, void* ws, size_t,
                                  hipStream_t st) {
  const WgradPlan plan = wgrad_plan(cv, dy.fmt, x.fmt);
  uint8_t* base = static_cast<uint8_t*>(ws);
  const long long npix_o = (long long)cv.ho() * cv.wo();
  uint8_t* dyt = base;
  uint8_t* xt = base + plan.dyt_b;
  float* part = reinterpret_cast<float*>(base + plan.dyt_b + plan.xt_b);
  const bool natural = plan.natural || plan.natural_sub, mixed = plan.mixed, half = plan.half;
  const int S = plan.S;
  WgradProb p;
  // rows of A are Cout (32 to a block); rows of B are (tap, Cin), whose
  // 32-channel blocks line up with 32-row groups when Cin is a multiple of 32
  p.khalf = cv.n <= 16;
  p.ga = 32;
  p.gb = cv.cin % 32 == 0 ? 32 : 0;
  p.kps = plan.kps;
  p.dytc = dyt; p.dys = dy.scales; p.xtc = xt; p.xs = x.scales; p.part = S > 1 ? part : dw;
  p.N = cv.n; p.H = cv.h; p.W = cv.w; p.Cin = cv.cin; p.Cout = cv.cout; p.KW = cv.kw;
  p.T = cv.kh * cv.kw; p.sh = cv.sh; p.sw = cv.sw; p.ph = cv.ph; p.pw = cv.pw; p.Ho = cv.ho(); p.Wo = cv.wo();
  p.nNB = ceil_div(cv.n, 32); p.ncob = ceil_div(cv.cout, 32); p.ncbi = ceil_div(cv.cin, 32);
  p.dyRB = half ? 16 : (int)run_bytes(dy.fmt); p.xRB = half ? 16 : (int)run_bytes(x.fmt);
  const WgradSteps ks = wgrad_steps(cv, p.kps);
  p.pair_w = ks.pair_w; p.nsub = ks.nsub; p.total_steps = ks.total; p.steps_per_split = ceil_div(ks.total, S);
  p.dytc_bytes = npix_o * cv.cout * p.nNB * p.dyRB; p.dys_bytes = npix_o * p.nNB * p.ncob;
  p.xtc_bytes = (long long)cv.h * cv.w * cv.cin * p.nNB * p.xRB; p.xs_bytes = (long long)cv.h * cv.w * p.nNB * p.ncbi;
  // padding moves the taps of the first output pixels before the buffer
  const long long lead = (long long)cv.ph * cv.w + cv.pw;
  p.xtcb = (int)(lead * cv.cin * p.nNB * p.xRB); p.xsb = (int)(lead * p.nNB * p.ncbi);
  // (gemm_offsets_ok has been checked by the caller; these never fail then)
  if (!offsets_fit(p.xtc_bytes, p.xtcb) || !offsets_fit(p.xs_bytes, p.xsb)) return hipErrorInvalidValue;
  p.dCin = make_fastdiv(cv.cin); p.dKW = make_fastdiv(cv.kw);
  p.dnsub = make_fastdiv(ks.nsub); p.dWo = make_fastdiv(p.Wo);
  const long long nj = (long long)p.T * cv.cin;
  WgradNatProb q;
  if (natural) {
    static_cast<WgradProb&>(q) = p;
    q.dyrb = (int)row_bytes(dy.fmt, cv.cout); q.xrb = (int)row_bytes(x.fmt, cv.cin);
    q.xbits = bits_of(x.fmt);
    q.dytc = dy.codes; q.dytc_bytes = npix_o * cv.n * q.dyrb;
    q.xtc = x.codes; q.xtc_bytes = (long long)cv.h * cv.w * cv.n * q.xrb;
    q.xtcb = (int)(lead * cv.n * q.xrb);
    if (!offsets_fit(q.xtc_bytes, q.xtcb)) return hipErrorInvalidValue;
  }
  // every check has passed: only now is anything enqueued
  hipError_t e = hipSuccess;
  if (!natural && !mixed) {
    e = launch_transpose_codes(dy.codes, dyt, dy.fmt, half, (int)npix_o, cv.n, 1, cv.cout, st);
    if (e != hipSuccess) return e;
  }
  if (!natural) {
    e = launch_transpose_codes(x.codes, xt, x.fmt, half, cv.h * cv.w, cv.n, 1, cv.cin, st);
    if (e != hipSuccess) return e;
  }
  if (plan.natural_sub) {
    WgradNatSubProb r;
    static_cast<WgradNatProb&>(r) = q;
    e = launch_wgrad_nat_sub(dy.fmt, x.fmt, r, cv.cout, (int)nj, S, st);
  } else if (natural) {
    e = launch_tiled(dy.fmt, x.fmt, q, cv.cout, (int)nj, S, st);
  } else if (mixed) {  // (half K-blocks need 8-bit activation codes: never here)
    WgradMixProb r;
    static_cast<WgradProb&>(r) = p;
    r.dyrb = (int)row_bytes(dy.fmt, cv.cout);
    r.dytc = dy.codes; r.dytc_bytes = npix_o * cv.n * r.dyrb;
    e = launch_tiled(dy.fmt, x.fmt, r, cv.cout, (int)nj, S, st);
  } else {
    e = launch_tiled(dy.fmt, x.fmt, p, cv.cout, (int)nj, S, st);
  }
  if (e != hipSuccess) return e;
  if (S > 1) {
    const long long n = (long long)cv.cout * nj;
    constexpr int C = 256 / kRedG;
    if ((n & 3) == 0) {
      hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3((unsigned)ceil_div(n / 4, C)), dim3(256), 0, st,
                         part, dw, n, S);
    } else {
      hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3((unsigned)ceil_div(n, C)), dim3(256), 0, st,
                         part, dw, n, S);
    }
    e = launch_check();
  }
  return e;
}


}  // namespace mq
