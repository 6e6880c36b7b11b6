// quantize.hip -- mxq_quantize: fp32 tensor -> packed MX codes + E8M0 scales,
// performed once per tensor (MicroQonv §III-A microscaling quantization,
// §IV-B square blocks along both GEMM directions).
//
// Tensor view [A][P][B][C] (C = channel, contiguous; P = partner dimension):
//   activations / gradients [H][W][N][C]: A = H*W, P = N, B = 1
//   weights [Cout][Kh][Kw][Cin]:          A = 1,   P = Cout, B = Kh*Kw
// memory row of (a, p, b) = (a*P + p)*B + b; a block is 32 channels x bp
// partner rows of one (a, b); its scale byte sits at
// ((a*B + b)*nPB + p/bp)*nCB + c/32.
//
// Mapping: one wave per tile of 32 rows x 32 channels; lane l takes row l/2
// and the channel half l%2 (16 consecutive fp32 = 64 contiguous bytes, so
// each row's 128-byte segment is read by two neighbouring lanes). The wave
// walks all channel blocks of its 32 rows, so every row's packed codes are
// written by one wave in consecutive iterations. The block maximum is a
// cross-lane max; the scaled values are clamped to the format's largest
// finite value and rounded by the hardware conversion instructions.
#include <algorithm>
#include <vector>

#include "mx_common.h"
#include "mqconv_internal.h"

namespace mq {

// MODE 0: line blocks (bp = 1), one block per row and channel block.
// MODE 1: square blocks (bp = 32): a tile is 32 partner rows of one (a, b).
// MODE 2: square blocks over a partner extent P in {1, 2, 4, 8, 16} with
//         B = 1: a tile is 32 consecutive memory rows = 32/P whole pixels,
//         and each pixel's P rows form one block (no idle lanes for small N).
// ST: the tile's 32 rows are consecutive in memory (B = 1) and short
// (at most 8 channel blocks): the wave packs them in LDS and writes the
// tile's bytes as one contiguous stretch, so every store covers whole
// cache lines (6-bit runs are 24 bytes, which direct stores would split).
// A workgroup quantizes 4 tiles (one per wave), tiles 4 wg .. 4 wg + 3, and
// of those the channel blocks cb0, cb0 + cbs, ...; `stage` is the wave's
// packing buffer (ST).
// ---------------------------------------------------------------------------
// Stochastic rounding (§III-A: the gradient is rounded stochastically). A
// scaled value between grid points lo < hi becomes hi when its random word r
// is below floor(2^32 (v - lo) / (hi - lo)), else lo; grid points stay, and
// results above the largest normal saturate. Element (memory row, channel c)
// takes word c mod 4 of Philox4x32-10 at counter (row, c / 4, 0, 0) with the
// seed's two halves as key (the generator of Salmon et al., SC'11: ten rounds
// of two 32 x 32 -> 64-bit products and key increments).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1, uint32_t (&o)[4]) {
#pragma unroll
  for (int r = 0; r < 10; r++) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
  }
  o[0] = c0; o[1] = c1; o[2] = c2; o[3] = c3;
}

// The 16 values x of half a block run (channels c0 .. c0 + 15 of memory row
// `row`, c0 a multiple of 16), divided by the block scale 2^(S - 127) and
// rounded stochastically onto the element grid; the results are grid points
// (or +-max), which the round-to-nearest conversions then encode exactly. A
// block holding a NaN or an infinity (S = 0xFF) is divided by 1 here and its
// codes are zeroed at conversion (code_keep).
template <int F>
__device__ __forceinline__ void sr_scale16(const float (&x)[16], uint32_t S, uint32_t row, int c0, uint32_t k0,
                                           uint32_t k1, float (&v)[16]) {
  using T = Fmt<F>;
  const float inv = inv_scale_from_byte(S == 255u ? 127u : S);
  uint32_t rw[16];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    uint32_t o[4];
    philox4x32_10(row, (uint32_t)(c0 >> 2) + q, 0u, 0u, k0, k1, o);
#pragma unroll
    for (int i = 0; i < 4; i++) rw[4 * q + i] = o[i];
  }
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const float t = x[i] * inv;
    const float a = fabsf(t);
    // grid spacing 2^e around a: e = max(floor(log2 a), emin) - M
    const int E = (int)(__float_as_uint(a) >> 23) - 127;
    const int e = max(E, T::emin) - T::M;
    const float u = a * __uint_as_float((uint32_t)(127 - e) << 23);  // a / 2^e, exact
    const float fl = floorf(u);
    const uint32_t thr = (uint32_t)floorf((u - fl) * 4294967296.0f);
    float r = (fl + (rw[i] < thr ? 1.0f : 0.0f)) * __uint_as_float((uint32_t)(127 + e) << 23);
    r = fminf(r, T::maxv);
    v[i] = copysignf(r, t);  // a block with S = 0xFF is zeroed at conversion
  }
}

constexpr int kStageCB = 8;
constexpr int kStageBytes = 32 * kStageCB * 32;
template <int F, int MODE, bool ST, bool SR = false>
__device__ __forceinline__ void quantize_tiles(const float* __restrict__ src, uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales, int A, int P, int B, int C,
                                               int bp, long long ntiles, long long wg, int cb0, int cbs,
                                               uint8_t* stage, uint32_t k0 = 0, uint32_t k1 = 0) {
  const int lane = threadIdx.x & 63;
  const long long tile = wg * 4 + (threadIdx.x >> 6);
  if (tile >= ntiles) return;
  const int r = lane >> 1, half = lane & 1;
  const int nCB = (C + 31) / 32;
  const int nPB = (P + bp - 1) / bp;
  long long row, sidx;  // memory row; scale byte index of channel block 0
  bool row_ok, writes_scale;
  if constexpr (MODE == 2) {
    row = tile * 32 + r;
    row_ok = row < (long long)A * P;
    const long long a = row / P;
    sidx = a * nCB;                                     // one partner block per pixel (P <= bp)
    writes_scale = (lane & (2 * P - 1)) == 0;           // first lane of the pixel's group
  } else {
    const int nPT = (P + 31) / 32;  // 32-row tiles along the partner dimension
    const int pt = (int)(tile % nPT);
    const long long ab = tile / nPT;  // = a*B + b
    const int b = (int)(ab % B);
    const long long a = ab / B;
    const int p = pt * 32 + r;
    row_ok = p < P;
    row = (a * P + p) * B + b;
    if constexpr (MODE == 1) {
      sidx = (ab * nPB + (long long)pt * 32 / bp) * nCB;
      writes_scale = lane == 0;
    } else {
      sidx = (ab * nPB + p) * nCB;
      writes_scale = half == 0;
    }
  }
  constexpr int RB = run_bytes_of(F);
  const long long row_bytes = (long long)nCB * RB;
  const float* srow = src + row * (long long)C;
  const bool vec = (C & 3) == 0;

  // cbs > 1 splits the channel blocks of small tensors over workgroups
  // (never with LDS staging, which needs a tile's whole rows)
  // the 16 values of channel block cb of this lane (zeros past the row or C)
  auto load16 = [&](int cb, float (&x)[16]) {
    const int c0 = cb * 32 + half * 16;
    if (row_ok && vec && c0 + 16 <= C) {
      const float4* s4 = reinterpret_cast<const float4*>(srow + c0);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        float4 t = s4[i];
        x[4 * i] = t.x; x[4 * i + 1] = t.y; x[4 * i + 2] = t.z; x[4 * i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; i++) x[i] = (row_ok && c0 + i < C) ? srow[c0 + i] : 0.0f;
    }
  };
  // software pipelined: the loads of the next channel block leave before the
  // current one is reduced, converted and stored
  float xn[16];
  if (cb0 < nCB) load16(cb0, xn);
  for (int cb = cb0; cb < nCB; cb += cbs) {
    const int c0 = cb * 32 + half * 16;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; i++) x[i] = xn[i];
    if (cb + cbs < nCB) load16(cb + cbs, xn);
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) m = max(m, __float_as_uint(x[i]) & 0x7fffffffu);
    // block max: the lane pair (a line of 32 channels), the whole wave
    // (32 partner rows) or the 2P lanes of one pixel
    m = group_max(m, MODE == 0 ? 2 : (MODE == 1 ? 64 : 2 * P));
    const uint32_t S = scale_byte_from_amax<F>(m);
    float v[16];
    if constexpr (SR) sr_scale16<F>(x, S, (uint32_t)row, c0, k0, k1, v);
    else scale_clamp16<F>(x, S, v);
    if constexpr (ST) {
      convert_store_half_run<F>(&stage[r * row_bytes + cb * RB + half * (RB / 2)], v, code_keep(S));
      if (row_ok && writes_scale) scales[sidx + cb] = (uint8_t)S;
    } else if (row_ok) {
      convert_store_half_run<F>(codes + row * row_bytes + (long long)cb * RB + half * (RB / 2), v, code_keep(S));
      if (writes_scale) scales[sidx + cb] = (uint8_t)S;
    }
  }
  if constexpr (ST) {
    // rows row0 .. row0 + nvalid - 1 of this tile are valid and consecutive
    const long long row0 = __shfl(row, 0);
    const int nvalid = __popcll(__ballot(row_ok && half == 0));
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's packed rows are in LDS
    __builtin_amdgcn_wave_barrier();
    const int words = (int)(nvalid * row_bytes / 4);
    const uint32_t* from = reinterpret_cast<const uint32_t*>(stage);
    uint32_t* to = reinterpret_cast<uint32_t*>(codes + row0 * row_bytes);
    for (int i = lane; i < words; i += 64) to[i] = from[i];
  }
}

template <int F, int MODE, bool ST, bool SR>
__global__ __launch_bounds__(256) void mxq_quantize_kernel(const float* __restrict__ src,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, int A, int P,
                                                          int B, int C, int bp, long long ntiles, uint32_t k0,
                                                          uint32_t k1) {
  __shared__ __attribute__((aligned(16))) uint8_t stage_buf[ST ? 4 : 1][ST ? kStageBytes : 16];
  quantize_tiles<F, MODE, ST, SR>(src, codes, scales, A, P, B, C, bp, ntiles, blockIdx.x, blockIdx.y, gridDim.y,
                                  stage_buf[ST ? threadIdx.x >> 6 : 0], k0, k1);
}

// Several tensors of one or two element formats in one launch (a small
// tensor, such as a weight, then runs beside a large one instead of after
// it): member i owns workgroups [begin, begin + nbx * gy) of the 1-D grid,
// nbx workgroups of tiles for each of its gy channel-block phases; its codes
// take the launch's first format, or the second one when alt is set.
struct QMember {
  const float* src;
  uint8_t *codes, *scales;
  long long ntiles;
  int A, P, B, C, bp, variant, nbx, gy, begin, alt;  // variant = 2 * MODE + ST
};
constexpr int kQGroupMax = 8;
struct QGroup {
  QMember m[kQGroupMax];
  int count;
};

template <int F0, int F1>
__global__ __launch_bounds__(256) void mxq_quantize_group_kernel(QGroup g) {
  __shared__ __attribute__((aligned(16))) uint8_t stage_buf[4][kStageBytes];
  const int b = blockIdx.x;
  QMember q = g.m[0];
#pragma unroll
  for (int j = 1; j < kQGroupMax; j++)
    if (j < g.count && b >= g.m[j].begin) q = g.m[j];
  const int lb = b - q.begin, by = lb / q.nbx, bx = lb - by * q.nbx;
  uint8_t* stage = stage_buf[threadIdx.x >> 6];
#define MQ_QT(F, MODE, ST) \
  quantize_tiles<F, MODE, ST>(q.src, q.codes, q.scales, q.A, q.P, q.B, q.C, q.bp, q.ntiles, bx, by, q.gy, stage)
#define MQ_QV(F)                          \
  switch (q.variant) {                    \
    case 0: MQ_QT(F, 0, false); break;    \
    case 1: MQ_QT(F, 0, true); break;     \
    case 2: MQ_QT(F, 1, false); break;    \
    case 3: MQ_QT(F, 1, true); break;     \
    case 4: MQ_QT(F, 2, false); break;    \
    default: MQ_QT(F, 2, true); break;    \
  }
  if constexpr (F0 == F1) {
    MQ_QV(F0)
  } else if (q.alt) {  // uniform: one member per workgroup
    MQ_QV(F1)
  } else {
    MQ_QV(F0)
  }
#undef MQ_QV
#undef MQ_QT
}

template <int F0>
static void launch_group_f0(int f1, const QGroup& g, unsigned blocks, hipStream_t st) {
  switch (f1) {
    case 0: hipLaunchKernelGGL((mxq_quantize_group_kernel<F0, 0>), dim3(blocks), dim3(256), 0, st, g); break;
    case 1: hipLaunchKernelGGL((mxq_quantize_group_kernel<F0, 1>), dim3(blocks), dim3(256), 0, st, g); break;
    case 2: hipLaunchKernelGGL((mxq_quantize_group_kernel<F0, 2>), dim3(blocks), dim3(256), 0, st, g); break;
    case 3: hipLaunchKernelGGL((mxq_quantize_group_kernel<F0, 3>), dim3(blocks), dim3(256), 0, st, g); break;
    default: hipLaunchKernelGGL((mxq_quantize_group_kernel<F0, 4>), dim3(blocks), dim3(256), 0, st, g); break;
  }
}
static void launch_group(int f0, int f1, const QGroup& g, unsigned blocks, hipStream_t st) {
  switch (f0) {
    case 0: launch_group_f0<0>(f1, g, blocks, st); break;
    case 1: launch_group_f0<1>(f1, g, blocks, st); break;
    case 2: launch_group_f0<2>(f1, g, blocks, st); break;
    case 3: launch_group_f0<3>(f1, g, blocks, st); break;
    default: launch_group_f0<4>(f1, g, blocks, st); break;
  }
}

// Block geometry of one tensor: MODE 0 for line blocks, 2 when a pixel's
// partner rows (P < 32 dividing 32) form whole square blocks, else 1; LDS
// staging (ST) when rows are consecutive and short; small tensors also
// spread their channel blocks over workgroups (gy, one memory round trip).
struct QPlan {
  int mode;
  bool st;
  long long ntiles, blocks;
  int gy;
};
static QPlan quantize_plan(int A, int P, int B, int C, int bp) {
  QPlan q;
  q.mode = bp != 32 ? 0 : (B == 1 && P < 32 && (32 % P) == 0) ? 2 : 1;
  q.ntiles = q.mode == 2 ? ((long long)A * P + 31) / 32 : (long long)A * B * ((P + 31) / 32);
  q.blocks = (q.ntiles + 3) / 4;
  q.st = B == 1 && (C + 31) / 32 <= kStageCB;
  q.gy = !q.st && q.blocks < 512 ? (C + 31) / 32 : 1;
  return q;
}

template <int F, int MODE, bool ST, bool SR>
static void launch_one(const QReq& r, const QPlan& q, uint64_t seed, hipStream_t st) {
  hipLaunchKernelGGL((mxq_quantize_kernel<F, MODE, ST, SR>), dim3((unsigned)q.blocks, (unsigned)q.gy), dim3(256), 0,
                     st, r.src, r.codes, r.scales, r.A, r.P, r.B, r.C, r.bp, q.ntiles, (uint32_t)seed,
                     (uint32_t)(seed >> 32));
}

template <int F, bool SR>
static hipError_t launch_f(const QReq& r, uint64_t seed, hipStream_t st) {
  const QPlan q = quantize_plan(r.A, r.P, r.B, r.C, r.bp);
  switch (2 * q.mode + q.st) {
    case 0: launch_one<F, 0, false, SR>(r, q, seed, st); break;
    case 1: launch_one<F, 0, true, SR>(r, q, seed, st); break;
    case 2: launch_one<F, 1, false, SR>(r, q, seed, st); break;
    case 3: launch_one<F, 1, true, SR>(r, q, seed, st); break;
    case 4: launch_one<F, 2, false, SR>(r, q, seed, st); break;
    default: launch_one<F, 2, true, SR>(r, q, seed, st); break;
  }
  return launch_check();
}

template <bool SR>
static hipError_t launch_fmt(const QReq& r, uint64_t seed, hipStream_t st) {
  switch (r.fmt) {
    case 0: return launch_f<0, SR>(r, seed, st);
    case 1: return launch_f<1, SR>(r, seed, st);
    case 2: return launch_f<2, SR>(r, seed, st);
    case 3: return launch_f<3, SR>(r, seed, st);
    default: return launch_f<4, SR>(r, seed, st);
  }
}

hipError_t launch_quantize(const float* src, uint8_t* codes, uint8_t* scales, int fmt, int bp, int A,
                           int P, int B, int C, hipStream_t st) {
  return launch_fmt<false>(QReq{src, codes, scales, fmt, bp, A, P, B, C}, 0, st);
}

hipError_t launch_quantize_sr(const float* src, uint8_t* codes, uint8_t* scales, int fmt, int bp, int A,
                              int P, int B, int C, uint64_t seed, hipStream_t st) {
  return launch_fmt<true>(QReq{src, codes, scales, fmt, bp, A, P, B, C}, seed, st);
}

// One grouped launch for up to kQGroupMax members of at most two element
// formats (more formats or members: one launch per format, per kQGroupMax
// members); members in increasing size, so the small ones are dispatched
// first and finish inside the large ones' time. A single tensor takes the
// single-tensor launch.
hipError_t launch_quantize_group(const QReq* reqs, int count, hipStream_t st) {
  std::vector<int> fmts;
  for (int i = 0; i < count; i++)
    if (std::find(fmts.begin(), fmts.end(), reqs[i].fmt) == fmts.end()) fmts.push_back(reqs[i].fmt);
  // the launches: lists of members and the (first, second) formats of each
  std::vector<std::vector<int>> sets;
  std::vector<std::pair<int, int>> fpair;
  if (fmts.size() <= 2 && count <= kQGroupMax) {
    std::vector<int> all(count);
    for (int i = 0; i < count; i++) all[i] = i;
    sets.push_back(all);
    fpair.push_back({fmts[0], fmts.size() > 1 ? fmts[1] : fmts[0]});
  } else {
    for (int f : fmts) {
      std::vector<int> idx;
      for (int i = 0; i < count; i++)
        if (reqs[i].fmt == f) idx.push_back(i);
      for (size_t c0 = 0; c0 < idx.size(); c0 += kQGroupMax) {
        sets.push_back(std::vector<int>(idx.begin() + c0, idx.begin() + std::min(idx.size(), c0 + kQGroupMax)));
        fpair.push_back({f, f});
      }
    }
  }
  for (size_t s = 0; s < sets.size(); s++) {
    std::vector<int>& idx = sets[s];
    if (idx.size() == 1) {
      const QReq& r = reqs[idx[0]];
      const hipError_t e = launch_quantize(r.src, r.codes, r.scales, r.fmt, r.bp, r.A, r.P, r.B, r.C, st);
      if (e != hipSuccess) return e;
      continue;
    }
    std::vector<QPlan> plans(count);
    for (int i : idx) plans[i] = quantize_plan(reqs[i].A, reqs[i].P, reqs[i].B, reqs[i].C, reqs[i].bp);
    std::stable_sort(idx.begin(), idx.end(),
                     [&](int a, int b) { return plans[a].blocks * plans[a].gy < plans[b].blocks * plans[b].gy; });
    QGroup g{};
    long long total = 0;
    g.count = (int)idx.size();
    for (int k = 0; k < g.count; k++) {
      const QReq& r = reqs[idx[k]];
      const QPlan& q = plans[idx[k]];
      QMember& m = g.m[k];
      m.src = r.src; m.codes = r.codes; m.scales = r.scales; m.ntiles = q.ntiles;
      m.A = r.A; m.P = r.P; m.B = r.B; m.C = r.C; m.bp = r.bp;
      m.variant = 2 * q.mode + q.st; m.nbx = (int)q.blocks; m.gy = q.gy; m.begin = (int)total;
      m.alt = r.fmt != fpair[s].first;
      total += q.blocks * q.gy;
      if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    }
    launch_group(fpair[s].first, fpair[s].second, g, (unsigned)total, st);
    const hipError_t e = launch_check();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mq
