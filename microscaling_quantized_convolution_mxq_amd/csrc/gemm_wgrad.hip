// gemm_wgrad.hip -- backward-weight GEMM launcher, split-K reduction and
// workspace sizes of the GEMM entry points.
#include "gemm_kernel.h"

namespace mq {

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
  // the same count for either step size (the workspace size depends on it):
  // capped by the number of four-block steps
  const WgradSteps ks = wgrad_steps(cv, 4);
  const long long nkb = (long long)cv.ho() * cv.wo() * ceil_div(cv.n, 32);
  int s = splitk_slices(cv.cout, (long long)cv.kh * cv.kw * cv.cin, nkb, ops);
  if (s > ks.total) s = ks.total;
  if (s < 1) s = 1;
  return s;
}

size_t gemm_workspace_bytes(const Conv& cv, int op, int fa, int fb) {
  if (op == 0) return 0;
  if (op == 1) {  // W re-laid with runs along Cout
    return align256(transposed_bytes(fb, 1, cv.cout, (long long)cv.kh * cv.kw, cv.cin));
  }
  // op 2: fa = gradient format, fb = activation format
  const size_t dyt = align256(transposed_bytes(fa, (long long)cv.ho() * cv.wo(), cv.n, 1, cv.cout));
  const size_t xt = align256(transposed_bytes(fb, (long long)cv.h * cv.w, cv.n, 1, cv.cin));
  const int S = wgrad_splits(cv, fa, fb);
  const size_t part = S > 1 ? align256((size_t)S * cv.cout * cv.kh * cv.kw * cv.cin * 4) : 0;
  return dyt + xt + part;
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
  WgradProb p;
  // rows of A are Cout (32 to a block); rows of B are (tap, Cin), whose
  // 32-channel blocks line up with 32-row groups when Cin is a multiple of 32
  p.khalf = cv.n <= 16;
  p.ga = 32;
  p.gb = cv.cin % 32 == 0 ? 32 : 0;
  // 8-bit codes are read where quantization left them (K-major staging)
  // when a 16-channel chunk of B stays in one tap and a K-block's lines are
  // the N values of one pixel; otherwise both are first re-laid with runs
  // along N; with 8-bit gradient codes and other activation codes (mixed)
  // only the activation is re-laid
  const bool kext_ok = cv.n <= 32 || cv.n % 32 == 0;
  const bool natural = dy.fmt <= 1 && x.fmt <= 1 && cv.cin % 16 == 0 && kext_ok;
  const bool mixed = !natural && dy.fmt <= 1 && kext_ok;
  const bool half = !natural && half_k_blocks(p.ga, p.gb, p.khalf, dy.fmt, x.fmt);
  // as the kernel choice below: half K-blocks take four K-blocks per step and
  // two wave groups per workgroup, so half as many slices cover the K range
  p.kps = half_k_blocks(p.ga, p.gb, p.khalf, dy.fmt, x.fmt) ? 4 : 2;
  const int S0 = wgrad_splits(cv, dy.fmt, x.fmt);  // the workspace holds S0 slices
  const int S = p.kps == 4 ? ceil_div(S0, 2) : S0;
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
  if (!offsets_fit(p.xtc_bytes, p.xtcb) || !offsets_fit(p.xs_bytes, p.xsb)) return hipErrorInvalidValue;
  // every check of the re-laid path has passed: only now is anything enqueued
  // (the in-place path re-lays nothing; its own check follows)
  hipError_t e = hipSuccess;
  if (!natural && !mixed) {
    e = launch_transpose_codes(dy.codes, dyt, dy.fmt, half, (int)npix_o, cv.n, 1, cv.cout, st);
    if (e != hipSuccess) return e;
  }
  if (!natural) {
    e = launch_transpose_codes(x.codes, xt, x.fmt, half, cv.h * cv.w, cv.n, 1, cv.cin, st);
    if (e != hipSuccess) return e;
  }
  p.dCin = make_fastdiv(cv.cin); p.dKW = make_fastdiv(cv.kw);
  p.dnsub = make_fastdiv(ks.nsub); p.dWo = make_fastdiv(p.Wo);
  const long long nj = (long long)p.T * cv.cin;
  if (natural) {
    WgradNatProb q;
    static_cast<WgradProb&>(q) = p;
    q.dyrb = (int)row_bytes(dy.fmt, cv.cout); q.xrb = (int)row_bytes(x.fmt, cv.cin);
    q.dytc = dy.codes; q.dytc_bytes = npix_o * cv.n * q.dyrb;
    q.xtc = x.codes; q.xtc_bytes = (long long)cv.h * cv.w * cv.n * q.xrb;
    q.xtcb = (int)(lead * cv.n * q.xrb);
    if (!offsets_fit(q.xtc_bytes, q.xtcb)) return hipErrorInvalidValue;
    e = launch_tiled(dy.fmt, x.fmt, q, cv.cout, (int)nj, S, st);
  } else if (mixed) {  // (half K-blocks need 8-bit activation codes: never here)
    WgradMixProb q;
    static_cast<WgradProb&>(q) = p;
    q.dyrb = (int)row_bytes(dy.fmt, cv.cout);
    q.dytc = dy.codes; q.dytc_bytes = npix_o * cv.n * q.dyrb;
    e = launch_tiled(dy.fmt, x.fmt, q, cv.cout, (int)nj, S, st);
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
    e = hipGetLastError();
  }
  return e;
}


}  // namespace mq
