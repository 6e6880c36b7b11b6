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
constexpr int kStageCB = 8;
constexpr int kStageBytes = 32 * kStageCB * 32;
template <int F, int MODE, bool ST>
__device__ __forceinline__ void quantize_tiles(const float* __restrict__ src, uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales, int A, int P, int B, int C,
                                               int bp, long long ntiles, long long wg, int cb0, int cbs,
                                               uint8_t* stage) {
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
  for (int cb = cb0; cb < nCB; cb += cbs) {
    const int c0 = cb * 32 + half * 16;
    float x[16];
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
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) m = max(m, __float_as_uint(x[i]) & 0x7fffffffu);
    // block max: the lane pair (a line of 32 channels), the whole wave
    // (32 partner rows) or the 2P lanes of one pixel
    m = max(m, (uint32_t)__shfl_xor((int)m, 1));
    if constexpr (MODE == 1) {
#pragma unroll
      for (int o = 2; o < 64; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    } else if constexpr (MODE == 2) {
#pragma unroll
      for (int o = 2; o < 32; o <<= 1)
        if (o < 2 * P) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    }
    const uint32_t S = scale_byte_from_amax<F>(m);
    float v[16];
    scale_clamp16<F>(x, S, v);
    if constexpr (ST) {
      convert_store_half_run<F>(&stage[r * row_bytes + cb * RB + half * (RB / 2)], v);
      if (row_ok && writes_scale) scales[sidx + cb] = (uint8_t)S;
    } else if (row_ok) {
      convert_store_half_run<F>(codes + row * row_bytes + (long long)cb * RB + half * (RB / 2), v);
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

template <int F, int MODE, bool ST>
__global__ __launch_bounds__(256) void mxq_quantize_kernel(const float* __restrict__ src,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, int A, int P,
                                                          int B, int C, int bp, long long ntiles) {
  __shared__ __attribute__((aligned(16))) uint8_t stage_buf[ST ? 4 : 1][ST ? kStageBytes : 16];
  quantize_tiles<F, MODE, ST>(src, codes, scales, A, P, B, C, bp, ntiles, blockIdx.x, blockIdx.y, gridDim.y,
                              stage_buf[ST ? threadIdx.x >> 6 : 0]);
}

// Several tensors of one element format in one launch (a small tensor, such
// as a weight, then runs beside a large one instead of after it): member i
// owns workgroups [begin, begin + nbx * gy) of the 1-D grid, nbx workgroups
// of tiles for each of its gy channel-block phases.
struct QMember {
  const float* src;
  uint8_t *codes, *scales;
  long long ntiles;
  int A, P, B, C, bp, variant, nbx, gy, begin;  // variant = 2 * MODE + ST
};
constexpr int kQGroupMax = 8;
struct QGroup {
  QMember m[kQGroupMax];
  int count;
};

template <int F>
__global__ __launch_bounds__(256) void mxq_quantize_group_kernel(QGroup g) {
  __shared__ __attribute__((aligned(16))) uint8_t stage_buf[4][kStageBytes];
  const int b = blockIdx.x;
  QMember q = g.m[0];
#pragma unroll
  for (int j = 1; j < kQGroupMax; j++)
    if (j < g.count && b >= g.m[j].begin) q = g.m[j];
  const int lb = b - q.begin, by = lb / q.nbx, bx = lb - by * q.nbx;
  uint8_t* stage = stage_buf[threadIdx.x >> 6];
#define MQ_QT(MODE, ST) \
  quantize_tiles<F, MODE, ST>(q.src, q.codes, q.scales, q.A, q.P, q.B, q.C, q.bp, q.ntiles, bx, by, q.gy, stage)
  switch (q.variant) {
    case 0: MQ_QT(0, false); break;
    case 1: MQ_QT(0, true); break;
    case 2: MQ_QT(1, false); break;
    case 3: MQ_QT(1, true); break;
    case 4: MQ_QT(2, false); break;
    default: MQ_QT(2, true); break;
  }
#undef MQ_QT
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

template <int F, int MODE, bool ST>
static void launch_one(const QReq& r, const QPlan& q, hipStream_t st) {
  hipLaunchKernelGGL((mxq_quantize_kernel<F, MODE, ST>), dim3((unsigned)q.blocks, (unsigned)q.gy), dim3(256), 0,
                     st, r.src, r.codes, r.scales, r.A, r.P, r.B, r.C, r.bp, q.ntiles);
}

template <int F>
static hipError_t launch_f(const QReq& r, hipStream_t st) {
  const QPlan q = quantize_plan(r.A, r.P, r.B, r.C, r.bp);
  switch (2 * q.mode + q.st) {
    case 0: launch_one<F, 0, false>(r, q, st); break;
    case 1: launch_one<F, 0, true>(r, q, st); break;
    case 2: launch_one<F, 1, false>(r, q, st); break;
    case 3: launch_one<F, 1, true>(r, q, st); break;
    case 4: launch_one<F, 2, false>(r, q, st); break;
    default: launch_one<F, 2, true>(r, q, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const float* src, uint8_t* codes, uint8_t* scales, int fmt, int bp, int A,
                           int P, int B, int C, hipStream_t st) {
  const QReq r{src, codes, scales, fmt, bp, A, P, B, C};
  switch (fmt) {
    case 0: return launch_f<0>(r, st);
    case 1: return launch_f<1>(r, st);
    case 2: return launch_f<2>(r, st);
    case 3: return launch_f<3>(r, st);
    default: return launch_f<4>(r, st);
  }
}

// One grouped launch per element format present (and per kQGroupMax
// members); members in increasing size, so the small ones are dispatched
// first and finish inside the large ones' time. A format with one member
// takes the single-tensor launch.
hipError_t launch_quantize_group(const QReq* reqs, int count, hipStream_t st) {
  for (int f = 0; f < 5; f++) {
    std::vector<int> idx;
    for (int i = 0; i < count; i++)
      if (reqs[i].fmt == f) idx.push_back(i);
    if (idx.empty()) continue;
    if (idx.size() == 1) {
      const hipError_t e = launch_quantize(reqs[idx[0]].src, reqs[idx[0]].codes, reqs[idx[0]].scales, f,
                                           reqs[idx[0]].bp, reqs[idx[0]].A, reqs[idx[0]].P, reqs[idx[0]].B,
                                           reqs[idx[0]].C, st);
      if (e != hipSuccess) return e;
      continue;
    }
    std::vector<QPlan> plans(count);
    for (int i : idx) plans[i] = quantize_plan(reqs[i].A, reqs[i].P, reqs[i].B, reqs[i].C, reqs[i].bp);
    std::stable_sort(idx.begin(), idx.end(),
                     [&](int a, int b) { return plans[a].blocks * plans[a].gy < plans[b].blocks * plans[b].gy; });
    for (size_t c0 = 0; c0 < idx.size(); c0 += kQGroupMax) {
      QGroup g{};
      long long total = 0;
      g.count = (int)std::min<size_t>(kQGroupMax, idx.size() - c0);
      for (int k = 0; k < g.count; k++) {
        const QReq& r = reqs[idx[c0 + k]];
        const QPlan& q = plans[idx[c0 + k]];
        QMember& m = g.m[k];
        m.src = r.src; m.codes = r.codes; m.scales = r.scales; m.ntiles = q.ntiles;
        m.A = r.A; m.P = r.P; m.B = r.B; m.C = r.C; m.bp = r.bp;
        m.variant = 2 * q.mode + q.st; m.nbx = (int)q.blocks; m.gy = q.gy; m.begin = (int)total;
        total += q.blocks * q.gy;
        if (total > 0x7fffffffLL) return hipErrorInvalidValue;
      }
      switch (f) {
        case 0: hipLaunchKernelGGL(mxq_quantize_group_kernel<0>, dim3((unsigned)total), dim3(256), 0, st, g); break;
        case 1: hipLaunchKernelGGL(mxq_quantize_group_kernel<1>, dim3((unsigned)total), dim3(256), 0, st, g); break;
        case 2: hipLaunchKernelGGL(mxq_quantize_group_kernel<2>, dim3((unsigned)total), dim3(256), 0, st, g); break;
        case 3: hipLaunchKernelGGL(mxq_quantize_group_kernel<3>, dim3((unsigned)total), dim3(256), 0, st, g); break;
        default: hipLaunchKernelGGL(mxq_quantize_group_kernel<4>, dim3((unsigned)total), dim3(256), 0, st, g); break;
      }
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace mq
