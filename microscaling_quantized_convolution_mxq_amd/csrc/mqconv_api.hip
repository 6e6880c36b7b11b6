// mqconv_api.hip -- the C ABI declared in include/mqconv.h.
// Validates every argument on the host before any HIP call (an invalid call
// enqueues nothing), converts descriptors and hands off to the launchers.
#include "mqconv.h"
#include "mqconv_internal.h"
#include "cuyckens.h"
#include "nvfp.h"

#include <limits.h>

#include <atomic>
#include <mutex>

using namespace mq;

namespace {

// Kernels address packed tensors with 32-bit byte offsets (buffer loads), so
// every tensor is limited to 2^30 elements (channel padding included).
const long long kMaxElems = 1LL << 30;

bool fmt_ok(int f) { return f >= MQ_E4M3 && f <= MQ_E2M1; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool dims_ok(int32_t d0, int32_t d1, int32_t d2, int32_t d3) {
  if (d0 < 1 || d1 < 1 || d2 < 1 || d3 < 1) return false;
  long long n = (long long)d0 * d1 * d2;
  if (n > kMaxElems) return false;
  long long cpad = ((long long)d3 + 31) / 32 * 32;
  return n * cpad <= kMaxElems;
}

// Element counts of the conv's tensors (0 if the geometry is invalid).
bool conv_ok(const mq_conv* c) {
  if (!c) return false;
  if (c->n < 1 || c->cin < 1 || c->h < 1 || c->w < 1 || c->cout < 1) return false;
  if (c->kh < 1 || c->kw < 1 || c->kh > 15 || c->kw > 15) return false;
  if (c->stride_h < 1 || c->stride_w < 1 || c->stride_h > 8 || c->stride_w > 8) return false;
  if (c->pad_h < 0 || c->pad_w < 0 || c->pad_h >= c->kh || c->pad_w >= c->kw) return false;
  long long ho = ((long long)c->h + 2LL * c->pad_h - c->kh) / c->stride_h + 1;
  long long wo = ((long long)c->w + 2LL * c->pad_w - c->kw) / c->stride_w + 1;
  if (c->h + 2LL * c->pad_h < c->kh || c->w + 2LL * c->pad_w < c->kw) return false;
  if (ho < 1 || wo < 1) return false;
  long long cpi = ((long long)c->cin + 31) / 32 * 32, cpo = ((long long)c->cout + 31) / 32 * 32;
  long long npad = ((long long)c->n + 31) / 32 * 32;
  if ((long long)c->h * c->w * npad * cpi > kMaxElems) return false;
  if (ho * wo * npad * cpo > kMaxElems) return false;
  if (ho * wo * c->n * (long long)c->kh * c->kw * cpi > kMaxElems) return false;
  if ((long long)c->cout * c->kh * c->kw * cpi > kMaxElems) return false;
  return true;
}

Conv to_conv(const mq_conv* c) {
  Conv v;
  v.n = c->n; v.cin = c->cin; v.h = c->h; v.w = c->w; v.cout = c->cout; v.kh = c->kh; v.kw = c->kw;
  v.sh = c->stride_h; v.sw = c->stride_w; v.ph = c->pad_h; v.pw = c->pad_w;
  return v;
}

// Checks a packed tensor view against a role and expected dims.
int check_mx(const mq_mx& t, mq_role role, int32_t d0, int32_t d1, int32_t d2, int32_t d3) {
  if (!t.codes || !t.scales) return MQ_ERR_NULL;
  if (!fmt_ok(t.fmt)) return MQ_ERR_FORMAT;
  if (t.role != role) return MQ_ERR_FORMAT;
  if (t.block_partner != 1 && t.block_partner != 32) return MQ_ERR_UNSUPPORTED;
  if (t.d0 != d0 || t.d1 != d1 || t.d2 != d2 || t.d3 != d3) return MQ_ERR_SHAPE;
  if (!aligned16(t.codes) || !aligned16(t.scales)) return MQ_ERR_ALIGN;
  return MQ_OK;
}

MxView view(const mq_mx& t) {
  MxView v;
  v.codes = static_cast<const uint8_t*>(t.codes);
  v.scales = t.scales;
  v.fmt = t.fmt;
  v.bp = t.block_partner;
  return v;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MQ_OK : MQ_ERR_HIP; }

// launch checks until the injected failure (0: none pending)
std::atomic<int> g_fail_countdown{0};

}  // namespace

hipError_t mq::launch_check() {
  const hipError_t e = hipGetLastError();
  int c = g_fail_countdown.load(std::memory_order_relaxed);
  while (c > 0 && !g_fail_countdown.compare_exchange_weak(c, c - 1, std::memory_order_relaxed)) {
  }
  return c == 1 ? hipErrorLaunchFailure : e;
}

// ---------------------------------------------------------------------------
// Backward-weight without any allocation: the scratch space (re-laid codes,
// split-K partial sums) is a fixed array of this library's code object in
// device memory. Every device the library runs on holds its own copy, at its
// own address, until the process ends; host code reaches it only through
// that per-device address, taken once per device with that device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[MQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per-device address of `scratch` (nullptr: not taken yet)

// Address of the current device's copy of `scratch` (nullptr on failure).
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int mqconv_abi_version(void) { return MQCONV_ABI_VERSION; }

int mqconv_inject_launch_failure(int n) {
  if (n < 0) return MQ_ERR_SHAPE;
  g_fail_countdown.store(n, std::memory_order_relaxed);
  return MQ_OK;
}

const char* mqconv_status_string(int status) {
  switch (status) {
    case MQ_OK: return "ok";
    case MQ_ERR_NULL: return "a required pointer is NULL";
    case MQ_ERR_SHAPE: return "invalid or inconsistent shape";
    case MQ_ERR_FORMAT: return "unknown element format or role mismatch";
    case MQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MQ_ERR_WORKSPACE: return "workspace too small";
    case MQ_ERR_UNSUPPORTED: return "unsupported combination";
    case MQ_ERR_HIP: return "HIP runtime or launch failure";
    default: return "unknown status";
  }
}

size_t mqconv_codes_bytes(mq_role role, mq_elem fmt, int32_t d0, int32_t d1, int32_t d2, int32_t d3) {
  if (!fmt_ok(fmt) || !dims_ok(d0, d1, d2, d3)) return 0;
  if (role != MQ_ROLE_ACT && role != MQ_ROLE_GRAD && role != MQ_ROLE_WEIGHT) return 0;
  return (size_t)((long long)d0 * d1 * d2 * row_bytes(fmt, d3));
}

size_t mqconv_scales_bytes(mq_role role, int32_t bp, int32_t d0, int32_t d1, int32_t d2, int32_t d3) {
  if ((bp != 1 && bp != 32) || !dims_ok(d0, d1, d2, d3)) return 0;
  const long long ncb = (d3 + 31) / 32;
  if (role == MQ_ROLE_ACT || role == MQ_ROLE_GRAD)
    return (size_t)((long long)d0 * d1 * ceil_div(d2, bp) * ncb);
  if (role == MQ_ROLE_WEIGHT) return (size_t)((long long)d1 * d2 * ceil_div(d0, bp) * ncb);
  return 0;
}

size_t mqconv_im2col_codes_bytes(const mq_conv* cv, mq_elem fmt) {
  if (!conv_ok(cv) || !fmt_ok(fmt)) return 0;
  Conv c = to_conv(cv);
  return (size_t)((long long)c.ho() * c.wo() * c.n * c.kh * c.kw * row_bytes(fmt, c.cin));
}

size_t mqconv_im2col_scales_bytes(const mq_conv* cv, int32_t bp) {
  if (!conv_ok(cv) || (bp != 1 && bp != 32)) return 0;
  Conv c = to_conv(cv);
  return (size_t)((long long)c.ho() * c.wo() * c.kh * c.kw * ceil_div(c.n, bp) * ceil_div(c.cin, 32));
}

// Checks one quantization request and maps its role to the [A][P][B] x C view.
static int quantize_req(const float* src, const mq_mx& dst, QReq* r) {
  if (!src || !dst.codes || !dst.scales) return MQ_ERR_NULL;
  if (!fmt_ok(dst.fmt)) return MQ_ERR_FORMAT;
  if (dst.role != MQ_ROLE_ACT && dst.role != MQ_ROLE_GRAD && dst.role != MQ_ROLE_WEIGHT) return MQ_ERR_FORMAT;
  if (dst.block_partner != 1 && dst.block_partner != 32) return MQ_ERR_UNSUPPORTED;
  if (!dims_ok(dst.d0, dst.d1, dst.d2, dst.d3)) return MQ_ERR_SHAPE;
  if (!aligned16(dst.codes) || !aligned16(dst.scales) || ((uintptr_t)src & 3u)) return MQ_ERR_ALIGN;
  int A, P, B;
  if (dst.role == MQ_ROLE_WEIGHT) { A = 1; P = dst.d0; B = dst.d1 * dst.d2; }
  else if (dst.block_partner == 1) { A = 1; P = dst.d0 * dst.d1 * dst.d2; B = 1; }  // rows independent
  else { A = dst.d0 * dst.d1; P = dst.d2; B = 1; }
  *r = QReq{src, static_cast<uint8_t*>(dst.codes), dst.scales, dst.fmt, dst.block_partner, A, P, B, dst.d3};
  return MQ_OK;
}

int mqconv_quantize(const float* src, mq_mx dst, void* stream) {
  QReq r;
  const int e = quantize_req(src, dst, &r);
  if (e != MQ_OK) return e;
  return hip_status(launch_quantize(r.src, r.codes, r.scales, r.fmt, r.bp, r.A, r.P, r.B, r.C, (hipStream_t)stream));
}

int mqconv_quantize_sr(const float* src, mq_mx dst, uint64_t seed, void* stream) {
  QReq r;
  const int e = quantize_req(src, dst, &r);
  if (e != MQ_OK) return e;
  return hip_status(launch_quantize_sr(r.src, r.codes, r.scales, r.fmt, r.bp, r.A, r.P, r.B, r.C, seed,
                                       (hipStream_t)stream));
}

int mqconv_quantize_group(int32_t count, const float* const* src, const mq_mx* dst, void* stream) {
  if (!src || !dst) return MQ_ERR_NULL;
  if (count < 1 || count > MQ_QUANTIZE_GROUP_MAX) return MQ_ERR_SHAPE;
  QReq r[MQ_QUANTIZE_GROUP_MAX];
  for (int i = 0; i < count; i++) {
    const int e = quantize_req(src[i], dst[i], &r[i]);
    if (e != MQ_OK) return e;
  }
  return hip_status(launch_quantize_group(r, count, (hipStream_t)stream));
}

int mqconv_cbf_im2col(const mq_conv* cv, mq_mx xq, void* col_codes, uint8_t* col_scales, void* stream) {
  if (!cv) return MQ_ERR_NULL;
  if (!conv_ok(cv)) return MQ_ERR_SHAPE;
  int s = check_mx(xq, MQ_ROLE_ACT, cv->h, cv->w, cv->n, cv->cin);
  if (s != MQ_OK) return s;
  if (!col_codes || !col_scales) return MQ_ERR_NULL;
  if (!aligned16(col_codes) || !aligned16(col_scales)) return MQ_ERR_ALIGN;
  return hip_status(launch_cbf_im2col(to_conv(cv), view(xq), static_cast<uint8_t*>(col_codes),
                                      col_scales, (hipStream_t)stream));
}

size_t mqconv_workspace_bytes(const mq_conv* cv, int op, mq_elem fa, mq_elem fb) {
  if (!conv_ok(cv) || !fmt_ok(fa) || !fmt_ok(fb) || op < 0 || op > 2) return 0;
  return gemm_workspace_bytes(to_conv(cv), op, fa, fb);
}

int mqconv_forward(const mq_conv* cv, mq_mx xq, mq_mx wq, float* y, void* ws, size_t ws_bytes, void* stream) {
  if (!cv) return MQ_ERR_NULL;
  if (!conv_ok(cv)) return MQ_ERR_SHAPE;
  int s = check_mx(xq, MQ_ROLE_ACT, cv->h, cv->w, cv->n, cv->cin);
  if (s != MQ_OK) return s;
  s = check_mx(wq, MQ_ROLE_WEIGHT, cv->cout, cv->kh, cv->kw, cv->cin);
  if (s != MQ_OK) return s;
  if (!y) return MQ_ERR_NULL;
  if ((uintptr_t)y & 3u) return MQ_ERR_ALIGN;
  if (!gemm_offsets_ok(to_conv(cv), 0, xq.fmt, wq.fmt, xq.block_partner)) return MQ_ERR_SHAPE;
  const size_t need = gemm_workspace_bytes(to_conv(cv), 0, xq.fmt, wq.fmt);
  if (need > 0 && (!ws || ws_bytes < need)) return MQ_ERR_WORKSPACE;
  return hip_status(launch_forward(to_conv(cv), view(xq), view(wq), y, ws, ws_bytes, (hipStream_t)stream));
}

int mqconv_forward_mx(const mq_conv* cv, mq_mx xq, mq_mx wq, mq_mx yq, void* ws, size_t ws_bytes, void* stream) {
  if (!cv) return MQ_ERR_NULL;
  if (!conv_ok(cv)) return MQ_ERR_SHAPE;
  const Conv c = to_conv(cv);
  int s = check_mx(xq, MQ_ROLE_ACT, cv->h, cv->w, cv->n, cv->cin);
  if (s != MQ_OK) return s;
  s = check_mx(wq, MQ_ROLE_WEIGHT, cv->cout, cv->kh, cv->kw, cv->cin);
  if (s != MQ_OK) return s;
  s = check_mx(yq, MQ_ROLE_ACT, c.ho(), c.wo(), cv->n, cv->cout);
  if (s != MQ_OK) return s;
  // a block of 32 batch rows must not straddle two 32-row groups of output rows
  if (yq.block_partner == 32 && cv->n % 32 != 0 && 32 % cv->n != 0) return MQ_ERR_UNSUPPORTED;
  if (!gemm_offsets_ok(c, 0, xq.fmt, wq.fmt, xq.block_partner)) return MQ_ERR_SHAPE;
  const size_t need = gemm_workspace_bytes(c, 0, xq.fmt, wq.fmt);
  if (need > 0 && (!ws || ws_bytes < need)) return MQ_ERR_WORKSPACE;
  MxOutView y{static_cast<uint8_t*>(yq.codes), yq.scales, yq.fmt, yq.block_partner};
  return hip_status(launch_forward_mx(c, view(xq), view(wq), y, (hipStream_t)stream));
}

int mqconv_backward_data(const mq_conv* cv, mq_mx dyq, mq_mx wq, float* dx, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!cv) return MQ_ERR_NULL;
  if (!conv_ok(cv)) return MQ_ERR_SHAPE;
  Conv c = to_conv(cv);
  int s = check_mx(dyq, MQ_ROLE_GRAD, c.ho(), c.wo(), cv->n, cv->cout);
  if (s != MQ_OK) return s;
  s = check_mx(wq, MQ_ROLE_WEIGHT, cv->cout, cv->kh, cv->kw, cv->cin);
  if (s != MQ_OK) return s;
  if (wq.block_partner != 32) return MQ_ERR_UNSUPPORTED;
  if (!dx) return MQ_ERR_NULL;
  if ((uintptr_t)dx & 3u) return MQ_ERR_ALIGN;
  if (!gemm_offsets_ok(c, 1, dyq.fmt, wq.fmt, dyq.block_partner)) return MQ_ERR_SHAPE;
  const size_t need = gemm_workspace_bytes(c, 1, dyq.fmt, wq.fmt);
  if (need > 0 && (!ws || ws_bytes < need)) return MQ_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return MQ_ERR_ALIGN;
  return hip_status(launch_backward_data(c, view(dyq), view(wq), dx, ws, ws_bytes, (hipStream_t)stream));
}

int mqconv_backward_data_mx(const mq_conv* cv, mq_mx dyq, mq_mx wq, mq_mx dxq, void* ws, size_t ws_bytes,
                            void* stream) {
  if (!cv) return MQ_ERR_NULL;
  if (!conv_ok(cv)) return MQ_ERR_SHAPE;
  const Conv c = to_conv(cv);
  int s = check_mx(dyq, MQ_ROLE_GRAD, c.ho(), c.wo(), cv->n, cv->cout);
  if (s != MQ_OK) return s;
  s = check_mx(wq, MQ_ROLE_WEIGHT, cv->cout, cv->kh, cv->kw, cv->cin);
  if (s != MQ_OK) return s;
  s = check_mx(dxq, MQ_ROLE_GRAD, cv->h, cv->w, cv->n, cv->cin);
  if (s != MQ_OK) return s;
  if (wq.block_partner != 32) return MQ_ERR_UNSUPPORTED;
  // a block of 32 batch rows must not straddle two 32-row groups of output rows
  if (dxq.block_partner == 32 && cv->n % 32 != 0 && 32 % cv->n != 0) return MQ_ERR_UNSUPPORTED;
  if (!gemm_offsets_ok(c, 1, dyq.fmt, wq.fmt, dyq.block_partner)) return MQ_ERR_SHAPE;
  const size_t need = gemm_workspace_bytes(c, 1, dyq.fmt, wq.fmt);
  if (need > 0 && (!ws || ws_bytes < need)) return MQ_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return MQ_ERR_ALIGN;
  MxOutView dx{static_cast<uint8_t*>(dxq.codes), dxq.scales, dxq.fmt, dxq.block_partner};
  return hip_status(launch_backward_data_mx(c, view(dyq), view(wq), dx, ws, ws_bytes, (hipStream_t)stream));
}

// Checks of the backward-weight call that need no workspace argument.
static int check_backward_weight(const mq_conv* cv, const mq_mx& dyq, const mq_mx& xq, const float* dw) {
  if (!cv) return MQ_ERR_NULL;
  if (!conv_ok(cv)) return MQ_ERR_SHAPE;
  const Conv c = to_conv(cv);
  int s = check_mx(dyq, MQ_ROLE_GRAD, c.ho(), c.wo(), cv->n, cv->cout);
  if (s != MQ_OK) return s;
  s = check_mx(xq, MQ_ROLE_ACT, cv->h, cv->w, cv->n, cv->cin);
  if (s != MQ_OK) return s;
  if (dyq.block_partner != 32 || xq.block_partner != 32) return MQ_ERR_UNSUPPORTED;
  if (!dw) return MQ_ERR_NULL;
  if ((uintptr_t)dw & 3u) return MQ_ERR_ALIGN;
  if (!gemm_offsets_ok(c, 2, dyq.fmt, xq.fmt, 32)) return MQ_ERR_SHAPE;
  return MQ_OK;
}

int mqconv_backward_weight(const mq_conv* cv, mq_mx dyq, mq_mx xq, float* dw, void* ws, size_t ws_bytes,
                           void* stream) {
  const int s = check_backward_weight(cv, dyq, xq, dw);
  if (s != MQ_OK) return s;
  const Conv c = to_conv(cv);
  const size_t need = gemm_workspace_bytes(c, 2, dyq.fmt, xq.fmt);
  if (need > 0 && (!ws || ws_bytes < need)) return MQ_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return MQ_ERR_ALIGN;
  return hip_status(launch_backward_weight(c, view(dyq), view(xq), dw, ws, ws_bytes, (hipStream_t)stream));
}

int mqconv_backward_weight_noalloc(const mq_conv* cv, mq_mx dyq, mq_mx xq, float* dw, void* stream) {
  const int s = check_backward_weight(cv, dyq, xq, dw);
  if (s != MQ_OK) return s;
  const Conv c = to_conv(cv);
  const size_t need = gemm_workspace_bytes(c, 2, dyq.fmt, xq.fmt);
  if (need > (size_t)MQ_NOALLOC_SCRATCH_BYTES) return MQ_ERR_WORKSPACE;
  void* ws = need > 0 ? scratch_for_current_device() : nullptr;
  if (need > 0 && !ws) return MQ_ERR_HIP;
  return hip_status(launch_backward_weight(c, view(dyq), view(xq), dw, ws, MQ_NOALLOC_SCRATCH_BYTES,
                                           (hipStream_t)stream));
}

size_t mqconv_naive_workspace_bytes(const mq_conv* cv, int op, mq_elem fa, mq_elem fb) {
  if (!conv_ok(cv) || !fmt_ok(fa) || !fmt_ok(fb) || op < 0 || op > 2) return 0;
  return naive_workspace_bytes(to_conv(cv), op, fa, fb);
}

static int naive_common(const mq_conv* cv, const void* a, const void* b, int fa, int fb, const void* out,
                        void* ws, size_t ws_bytes, int op) {
  if (!cv) return MQ_ERR_NULL;
  if (!conv_ok(cv)) return MQ_ERR_SHAPE;
  if (!a || !b || !out) return MQ_ERR_NULL;
  if (!fmt_ok(fa) || !fmt_ok(fb)) return MQ_ERR_FORMAT;
  if (((uintptr_t)a & 3u) || ((uintptr_t)b & 3u) || ((uintptr_t)out & 3u)) return MQ_ERR_ALIGN;
  const size_t need = naive_workspace_bytes(to_conv(cv), op, fa, fb);
  if (!ws || ws_bytes < need) return MQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return MQ_ERR_ALIGN;
  return MQ_OK;
}

int mqconv_naive_forward(const mq_conv* cv, const float* x, const float* w, mq_elem fx, mq_elem fw, float* y,
                         void* ws, size_t ws_bytes, void* stream) {
  int s = naive_common(cv, x, w, fx, fw, y, ws, ws_bytes, 0);
  if (s != MQ_OK) return s;
  return hip_status(launch_naive_forward(to_conv(cv), x, w, fx, fw, y, ws, (hipStream_t)stream));
}

int mqconv_naive_backward_data(const mq_conv* cv, const float* dy, const float* w, mq_elem fdy, mq_elem fw,
                               float* dx, void* ws, size_t ws_bytes, void* stream) {
  int s = naive_common(cv, dy, w, fdy, fw, dx, ws, ws_bytes, 1);
  if (s != MQ_OK) return s;
  return hip_status(launch_naive_backward_data(to_conv(cv), dy, w, fdy, fw, dx, ws, (hipStream_t)stream));
}

int mqconv_naive_backward_weight(const mq_conv* cv, const float* dy, const float* x, mq_elem fdy, mq_elem fx,
                                 float* dw, void* ws, size_t ws_bytes, void* stream) {
  int s = naive_common(cv, dy, x, fdy, fx, dw, ws, ws_bytes, 2);
  if (s != MQ_OK) return s;
  return hip_status(launch_naive_backward_weight(to_conv(cv), dy, x, fdy, fx, dw, ws, (hipStream_t)stream));
}

// ---- two-level (NVFP-style) quantization ---------------------------------------
size_t mqconv_nvfp_scales_bytes(mq_role role, int32_t d0, int32_t d1, int32_t d2, int32_t d3) {
  if (!dims_ok(d0, d1, d2, d3)) return 0;
  const long long nc8 = (d3 + 7) / 8;
  if (role == MQ_ROLE_ACT || role == MQ_ROLE_GRAD) return (size_t)((long long)d0 * d1 * ceil_div(d2, 8) * nc8);
  if (role == MQ_ROLE_WEIGHT) return (size_t)((long long)d1 * d2 * ceil_div(d0, 8) * nc8);
  return 0;
}

size_t mqconv_nvfp_workspace_bytes(void) { return nvfp_workspace_bytes(); }

int mqconv_nvfp_quantize(const float* src, mq_role role, mq_elem fmt, int32_t d0, int32_t d1, int32_t d2, int32_t d3,
                         void* codes, uint8_t* block_scales, float* tensor_scale, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!src || !codes || !block_scales || !tensor_scale) return MQ_ERR_NULL;
  if (!fmt_ok(fmt)) return MQ_ERR_FORMAT;
  if (role != MQ_ROLE_ACT && role != MQ_ROLE_GRAD && role != MQ_ROLE_WEIGHT) return MQ_ERR_FORMAT;
  if (!dims_ok(d0, d1, d2, d3)) return MQ_ERR_SHAPE;
  if (!ws || ws_bytes < nvfp_workspace_bytes()) return MQ_ERR_WORKSPACE;
  if (!aligned16(codes) || ((uintptr_t)src & 3u) || ((uintptr_t)tensor_scale & 3u) || ((uintptr_t)ws & 3u))
    return MQ_ERR_ALIGN;
  int A, P, B;
  if (role == MQ_ROLE_WEIGHT) { A = 1; P = d0; B = d1 * d2; }
  else { A = d0 * d1; P = d2; B = 1; }
  return hip_status(launch_nvfp_quantize(src, static_cast<uint8_t*>(codes), block_scales, tensor_scale, fmt, A, P, B,
                                         d3, ws, (hipStream_t)stream));
}

// ---- square-block comparator -------------------------------------------------
// the classic im2col extent M x K, and the GEMMs' 32-bit byte offsets over
// the expanded tensors (fp32 G_X' of the backward-data is the largest)
static bool cuyckens_fits(const mq_conv* cv) {
  const Conv c = to_conv(cv);
  const long long M = (long long)c.ho() * c.wo() * c.n, K = (long long)c.cin * c.kh * c.kw;
  return M * (long long)((K + 31) / 32 * 32) <= kMaxElems && M * K * 4 < 0x7f000000LL;
}

size_t mqconv_cuyckens_col_codes_bytes(const mq_conv* cv, mq_elem fx) {
  if (!conv_ok(cv) || !fmt_ok(fx) || !cuyckens_fits(cv)) return 0;
  return cuyckens_col_codes_bytes(to_conv(cv), fx);
}

size_t mqconv_cuyckens_col_scales_bytes(const mq_conv* cv) {
  if (!conv_ok(cv) || !cuyckens_fits(cv)) return 0;
  return cuyckens_col_scales_bytes(to_conv(cv));
}

size_t mqconv_cuyckens_workspace_bytes(const mq_conv* cv, int op, mq_elem fa, mq_elem fb) {
  if (!conv_ok(cv) || !fmt_ok(fa) || !fmt_ok(fb) || op < 0 || op > 2 || !cuyckens_fits(cv)) return 0;
  return cuyckens_workspace_bytes(to_conv(cv), op, fa, fb);
}

// common checks of the comparator's calls (pointers a, b, out; formats; workspace)
static int cuyckens_common(const mq_conv* cv, const void* a, const void* b, const void* out, int fa, int fb,
                           void* ws, size_t ws_bytes, int op) {
  if (!cv) return MQ_ERR_NULL;
  if (!conv_ok(cv) || !cuyckens_fits(cv)) return MQ_ERR_SHAPE;
  if (!a || !b || !out) return MQ_ERR_NULL;
  if (!fmt_ok(fa) || !fmt_ok(fb)) return MQ_ERR_FORMAT;
  if (((uintptr_t)a & 3u) || ((uintptr_t)b & 3u) || ((uintptr_t)out & 3u)) return MQ_ERR_ALIGN;
  if (op >= 0) {
    const size_t need = cuyckens_workspace_bytes(to_conv(cv), op, fa, fb);
    if (!ws || ws_bytes < need) return MQ_ERR_WORKSPACE;
    if (!aligned16(ws)) return MQ_ERR_ALIGN;
  }
  return MQ_OK;
}

int mqconv_cuyckens_im2col_quantize(const mq_conv* cv, const float* x, mq_elem fx, void* col_codes,
                                    uint8_t* col_scales, void* stream) {
  const int s = cuyckens_common(cv, x, col_codes, col_scales, fx, fx, nullptr, 0, -1);
  if (s != MQ_OK) return s;
  if (!aligned16(col_codes) || !aligned16(col_scales)) return MQ_ERR_ALIGN;
  return hip_status(launch_cuyckens_im2col_quantize(to_conv(cv), x, fx, static_cast<uint8_t*>(col_codes), col_scales,
                                                    (hipStream_t)stream));
}

int mqconv_cuyckens_forward(const mq_conv* cv, const void* col_codes, const uint8_t* col_scales, mq_elem fx,
                            const float* w, mq_elem fw, float* y, void* ws, size_t ws_bytes, void* stream) {
  if (!col_scales) return MQ_ERR_NULL;
  const int s = cuyckens_common(cv, col_codes, w, y, fx, fw, ws, ws_bytes, 0);
  if (s != MQ_OK) return s;
  if (!aligned16(col_codes) || !aligned16(col_scales)) return MQ_ERR_ALIGN;
  return hip_status(launch_cuyckens_forward(to_conv(cv), static_cast<const uint8_t*>(col_codes), col_scales, fx, w,
                                            fw, y, ws, (hipStream_t)stream));
}

int mqconv_cuyckens_backward_data(const mq_conv* cv, const float* dy, const float* w, mq_elem fdy, mq_elem fw,
                                  float* dx, void* ws, size_t ws_bytes, void* stream) {
  const int s = cuyckens_common(cv, dy, w, dx, fdy, fw, ws, ws_bytes, 1);
  if (s != MQ_OK) return s;
  return hip_status(launch_cuyckens_backward_data(to_conv(cv), dy, w, fdy, fw, dx, ws, (hipStream_t)stream));
}

int mqconv_cuyckens_backward_weight(const mq_conv* cv, const float* dy, const void* col_codes,
                                    const uint8_t* col_scales, mq_elem fdy, mq_elem fx, float* dw, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (!col_scales) return MQ_ERR_NULL;
  const int s = cuyckens_common(cv, dy, col_codes, dw, fdy, fx, ws, ws_bytes, 2);
  if (s != MQ_OK) return s;
  if (!aligned16(col_codes) || !aligned16(col_scales)) return MQ_ERR_ALIGN;
  return hip_status(launch_cuyckens_backward_weight(to_conv(cv), dy, static_cast<const uint8_t*>(col_codes),
                                                    col_scales, fdy, fx, dw, ws, (hipStream_t)stream));
}

}  // extern "C"
