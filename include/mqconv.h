/*
 * mqconv.h -- C ABI of the MI355X (gfx950) microscaled-convolution library.
 *
 * The library implements the training hot path of MicroQonv ("MicroQonv:
 * Reshaping Convolution Tensors for Efficient Microscaling in Training and
 * Inference", Facq, Ben-Ali, Sentieys):
 *   1. MX block quantization of each convolution tensor, performed once
 *      (§III-A microscaling quantization; §IV-B efficient quantization
 *      directions: square blocks spanning both GEMM directions);
 *   2. channel-batch-first (CBF) im2col applied to the already-quantized
 *      activation (§IV-A, Fig. 3);
 *   3. block-scaled GEMMs for the forward output Y, the input gradient G_X
 *      and the weight gradient G_W (§II-C3 matrix formulation, §IV-B,
 *      Eq. 7 block dot product);
 *   4. a naive path that expands with im2col first and quantizes each tensor
 *      twice along 1-D lines (§III-C limitations of related work, Table I),
 *      kept only to compare bytes moved.
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every entry point
 * ---------------------------------------------------------------------------
 * Pointers.   Every tensor pointer is a DEVICE pointer allocated and owned by
 *             the caller. The library never allocates, frees or retains
 *             memory, apart from the fixed scratch array of
 *             mqconv_backward_weight_noalloc (see there). `mq_conv`
 *             descriptors are HOST pointers, read during the call only.
 * Streams.    `stream` is a hipStream_t passed as void*; NULL means the
 *             default stream. Every call only enqueues work and returns.
 * Errors.     The return value is an mq_status. All argument validation
 *             happens before any HIP call; an invalid call returns an error
 *             and enqueues nothing. A failed launch returns MQ_ERR_HIP.
 *             No C++ exception crosses this interface.
 * Threading.  Functions keep no state between calls and may be called from
 *             several host threads on different streams.
 * Determinism. Equal inputs give bit-identical outputs (no float atomics).
 *
 * ---------------------------------------------------------------------------
 * Number formats (MicroQonv §II-D / §III-A; OCP MX element encodings)
 * ---------------------------------------------------------------------------
 * Element codes are sign-magnitude floats:
 *   MQ_E4M3  8 bit, bias 7,  max 448 (no Inf; S.1111.111 is NaN)
 *   MQ_E5M2  8 bit, bias 15, max 57344
 *   MQ_E2M3  6 bit, bias 1,  max 7.5
 *   MQ_E3M2  6 bit, bias 3,  max 28
 *   MQ_E2M1  4 bit, bias 1,  max 6
 * Block scales are E8M0 bytes: value 2^(S-127); 0xFF means NaN.
 *
 * Quantization of one block (the OCP MX rule with a power-of-two scale, the
 * original microscaling format named in §II-D):
 *   amax = max |x| over the block's elements;
 *   e    = floor(log2 amax) - emax_elem, clamped to [-127, 127]
 *          (emax_elem = 8, 15, 2, 4, 2 for the formats above);
 *          an all-zero block gets e = -127;
 *   S    = e + 127;
 *   code = round-to-nearest-even of x * 2^-e on the element grid
 *          (subnormals included), saturated to +-max; the sign of zero is
 *          kept; a block holding a NaN or Inf gets S = 0xFF and all codes 0.
 *
 * ---------------------------------------------------------------------------
 * Block geometry (§IV-B: square blocks, one side along the channel, the
 * other along the partner dimension of the second GEMM)
 * ---------------------------------------------------------------------------
 * A block is 32 consecutive channels x `block_partner` (bp) consecutive
 * partner indices, inside one pixel (activations, gradients) or one kernel
 * tap (weights). Channel blocks start at channel 0 and the last one is
 * truncated at C; partner blocks are truncated at the partner extent.
 * Partner dimension: N (batch) for ACT and GRAD, Cout for WEIGHT.
 * bp is 1 (a line along the channel) or 32 (a 32x32 square).
 *
 * ---------------------------------------------------------------------------
 * Packed layouts (channel-batch-first, §IV-A "each spatial location holds a
 * contiguous block of all channels across all batch elements")
 * ---------------------------------------------------------------------------
 * Cpad      = C rounded up to a multiple of 32; ncb = Cpad / 32.
 * run_bytes = bytes of 32 packed codes: 32 (8-bit), 24 (6-bit), 16 (4-bit).
 * row_bytes = ncb * run_bytes.
 * Inside a run, code j (channel 32*cb + j) sits at
 *   8-bit: byte j;
 *   6-bit: bits [6j, 6j+6) of the run read as a little-endian 192-bit word;
 *   4-bit: bits [4j, 4j+4) of the run read as a little-endian 128-bit word
 *          (code 2i in the low nibble of byte i).
 * Codes of padding channels (C <= c < Cpad) are 0.
 *
 *   role ACT / GRAD, dims (d0,d1,d2,d3) = (H, W, N, C):
 *     codes  [H][W][N][row_bytes]
 *     scales [H][W][ceil(N/bp)][ncb]
 *   role WEIGHT, dims (d0,d1,d2,d3) = (Cout, Kh, Kw, Cin):
 *     codes  [Cout][Kh][Kw][row_bytes]
 *     scales [Kh][Kw][ceil(Cout/bp)][ncb]
 *   CBF im2col output X' of an ACT tensor (mqconv_cbf_im2col):
 *     codes  [Ho][Wo][N][Kh][Kw][row_bytes]
 *     scales [Ho][Wo][Kh][Kw][ceil(N/bp)][ncb]
 *
 * fp32 tensors use the same orders: activations and gradients [H][W][N][C]
 * (C fastest), weights [Cout][Kh][Kw][Cin].
 *
 * Convolution (§II-A, Eqs. 1-3, with stride s and zero padding p; the kernel
 * is not flipped, as in the im2col patch definition of §II-C1):
 *   Ho = floor((H + 2p - Kh) / s) + 1  (same for Wo)
 *   Y[ho,wo,n,co]    = sum_{kh,kw,ci} W[co,kh,kw,ci] * X[ho*s+kh-p, wo*s+kw-p, n, ci]
 *   G_X[h,w,n,ci]    = sum over (co,kh,kw,ho,wo) with ho*s+kh-p = h, wo*s+kw-p = w
 *                      of W[co,kh,kw,ci] * G_Y[ho,wo,n,co]
 *   G_W[co,kh,kw,ci] = sum_{ho,wo,n} G_Y[ho,wo,n,co] * X[ho*s+kh-p, wo*s+kw-p, n, ci]
 * with out-of-image X taken as 0. The GEMMs use the dequantized operands
 * (code value * block scale, the fake-quantization view of §III-A) and
 * accumulate in fp32.
 */
#ifndef MQCONV_H
#define MQCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MQCONV_ABI_VERSION 1

typedef enum {
  MQ_OK = 0,
  MQ_ERR_NULL = -1,        /* a required pointer is NULL */
  MQ_ERR_SHAPE = -2,       /* a dimension is < 1, inconsistent, or too large */
  MQ_ERR_FORMAT = -3,      /* unknown element format or role mismatch */
  MQ_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  MQ_ERR_WORKSPACE = -5,   /* workspace smaller than the *_workspace_bytes query */
  MQ_ERR_UNSUPPORTED = -6, /* valid but unsupported combination (see each call) */
  MQ_ERR_HIP = -7          /* a HIP launch or runtime call failed */
} mq_status;

/* Element formats and tensor roles. mq_elem and mq_role are plain 32-bit
 * integers holding one of these constants, so that any value a caller passes
 * is representable and can be checked (an out-of-range value is rejected
 * with MQ_ERR_FORMAT, or a size of 0 from the size queries). */
enum { MQ_E4M3 = 0, MQ_E5M2 = 1, MQ_E2M3 = 2, MQ_E3M2 = 3, MQ_E2M1 = 4 };
typedef int32_t mq_elem;

enum { MQ_ROLE_ACT = 0, MQ_ROLE_WEIGHT = 1, MQ_ROLE_GRAD = 2 };
typedef int32_t mq_role;

/* Convolution geometry (host struct). All fields >= 1 except pads (>= 0).
 * Supported: kh, kw <= 15; stride <= 8; pad < kernel size; Ho, Wo >= 1;
 * every packed tensor and im2col output below 2^30 elements. */
typedef struct {
  int32_t n, cin, h, w, cout, kh, kw, stride_h, stride_w, pad_h, pad_w;
} mq_conv;

/* Packed MX tensor view (layouts above). Caller owns both buffers. */
typedef struct {
  void* codes;           /* device, 16-byte aligned */
  uint8_t* scales;       /* device, 16-byte aligned, one E8M0 byte per block */
  mq_elem fmt;
  int32_t block_partner; /* bp: 1 or 32 */
  mq_role role;
  int32_t d0, d1, d2, d3; /* ACT/GRAD: (H, W, N, C); WEIGHT: (Cout, Kh, Kw, Cin) */
} mq_mx;

/* Returns MQCONV_ABI_VERSION. */
int mqconv_abi_version(void);

/* Static English text for a status code; never NULL. */
const char* mqconv_status_string(int status);

/* Failure injection, for tests of the error paths (callers that must see
 * how an entry point behaves when a kernel launch fails). After
 * mqconv_inject_launch_failure(n), n >= 1, the n-th launch check from then
 * on (each entry point checks after each kernel it enqueues) reports a
 * launch failure: that entry point returns MQ_ERR_HIP at once, with the
 * kernels before it enqueued as usual and none after it, so its outputs
 * are undefined; later calls run normally. n = 0 cancels a pending
 * injection. Process-wide (one countdown shared by all threads and
 * devices). Returns MQ_OK, or MQ_ERR_SHAPE for n < 0. */
int mqconv_inject_launch_failure(int n);

/* Bytes of the packed code / scale buffers of a tensor with the given role
 * and dims (layouts above). 0 for invalid arguments. Host-only, no HIP call. */
size_t mqconv_codes_bytes(mq_role role, mq_elem fmt, int32_t d0, int32_t d1, int32_t d2,
                          int32_t d3);
size_t mqconv_scales_bytes(mq_role role, int32_t bp, int32_t d0, int32_t d1, int32_t d2,
                           int32_t d3);
/* Bytes of the CBF im2col output of an ACT tensor for conv `cv`. */
size_t mqconv_im2col_codes_bytes(const mq_conv* cv, mq_elem fmt);
size_t mqconv_im2col_scales_bytes(const mq_conv* cv, int32_t bp);

/* MX-quantize an fp32 tensor once (§III-A, §IV-B).
 * src: fp32 in the role's order ([H][W][N][C] or [Cout][Kh][Kw][Cin]).
 * dst: role, fmt, bp and dims select the block geometry; its code and scale
 *      buffers must hold mqconv_codes_bytes / mqconv_scales_bytes bytes and
 *      are fully overwritten (padding codes included). */
int mqconv_quantize(const float* src, mq_mx dst, void* stream);

/* mqconv_quantize with the elements rounded stochastically instead of to
 * nearest: §III-A rounds activations and weights to nearest and the
 * gradient stochastically. The block scale byte is the round-to-nearest
 * one; each scaled element x * 2^-e between neighbouring grid points
 * lo < hi becomes hi when its random word r satisfies
 * r < floor(2^32 * (x * 2^-e - lo) / (hi - lo)), else lo (grid points stay,
 * results above max normal saturate to it). The random word of the element
 * on memory row `row` (the element index divided by C in the role's fp32
 * order) and channel c is word (c mod 4) of Philox4x32-10 (Salmon et al.,
 * "Parallel random numbers: as easy as 1, 2, 3", SC'11) at counter
 * (row, c / 4, 0, 0) with key (seed & 0xffffffff, seed >> 32); equal
 * (src, seed) give equal codes. Arguments, layouts and errors: as
 * mqconv_quantize. */
int mqconv_quantize_sr(const float* src, mq_mx dst, uint64_t seed, void* stream);

/* mqconv_quantize of several tensors at once, e.g. a layer's activation and
 * weight before its forward pass (each still quantized once, §III-A, §IV-B):
 * src[i] -> dst[i] for i < count, every pair exactly as mqconv_quantize
 * would write it. Tensors of up to two element formats share one launch
 * (more formats: one launch per format), so a small tensor runs beside a
 * large one instead of after it.
 * src, dst: host arrays of count entries (read during the call only).
 * count: 1 .. MQ_QUANTIZE_GROUP_MAX, else MQ_ERR_SHAPE.
 * Every pair is checked (as mqconv_quantize) before anything is enqueued;
 * the first failing pair's status is returned. Output buffers of different
 * pairs must not overlap (their bytes would then be undefined). */
#define MQ_QUANTIZE_GROUP_MAX 8
int mqconv_quantize_group(int32_t count, const float* const* src, const mq_mx* dst, void* stream);

/* Channel-batch-first im2col of an already-quantized activation (§IV-A):
 *   X'[ho,wo,n,kh,kw,c] = X[ho*s+kh-p, wo*s+kw-p, n, c]
 * Codes and scales are moved unchanged (no requantization): every
 * (ho,wo,kh,kw, n-block, c-block) block of X' takes the scale of its source
 * block; positions outside the image get code 0 and scale byte 0.
 * xq must be an ACT tensor of dims (H, W, N, Cin) matching cv. */
int mqconv_cbf_im2col(const mq_conv* cv, mq_mx xq, void* col_codes, uint8_t* col_scales,
                      void* stream);

/* Workspace (device bytes) needed by the GEMM entry points.
 * op: 0 forward, 1 backward-data, 2 backward-weight. fa/fb: the formats of
 * the two operands in the order of the call's arguments. */
size_t mqconv_workspace_bytes(const mq_conv* cv, int op, mq_elem fa, mq_elem fb);

/* Forward GEMM Y_f = W_f . X'  (§IV-B), with X' generated on the fly from
 * the packed CBF activation (implicit CBF im2col).
 *   xq: ACT (H, W, N, Cin), bp 1 or 32;  wq: WEIGHT (Cout, Kh, Kw, Cin), bp 1 or 32.
 *   y:  fp32 [Ho][Wo][N][Cout], fully overwritten. */
int mqconv_forward(const mq_conv* cv, mq_mx xq, mq_mx wq, float* y, void* ws, size_t ws_bytes,
                   void* stream);

/* mqconv_forward whose output is Y MX-quantized (the next layer's
 * activation, quantized once: §III-A, §IV-B) instead of fp32: yq receives
 * exactly the codes and scales that mqconv_quantize of mqconv_forward's
 * fp32 Y would write, without the fp32 Y ever reaching memory.
 *   yq: ACT (Ho, Wo, N, Cout), any format; bp 1, or bp 32 when N is a
 *       multiple of 32 or divides 32 (otherwise MQ_ERR_UNSUPPORTED: a block
 *       would straddle two of the kernel's 32-row output groups). Its code
 *       and scale buffers are fully overwritten.
 *   xq, wq, ws, ws_bytes, errors: as mqconv_forward. */
int mqconv_forward_mx(const mq_conv* cv, mq_mx xq, mq_mx wq, mq_mx yq, void* ws, size_t ws_bytes,
                      void* stream);

/* Input-gradient GEMM G_X' = W_f^T . G_Yf (§IV-B) folded back to G_X
 * (Eq. 2: convolution of G_Y with the channel-transposed kernel).
 *   dyq: GRAD (Ho, Wo, N, Cout), any bp;  wq: WEIGHT, bp must be 32
 *        (the contraction runs along Cout, the weight's partner dimension;
 *        bp 1 returns MQ_ERR_UNSUPPORTED).
 *   dx: fp32 [H][W][N][Cin], fully overwritten. */
int mqconv_backward_data(const mq_conv* cv, mq_mx dyq, mq_mx wq, float* dx, void* ws,
                         size_t ws_bytes, void* stream);

/* mqconv_backward_data whose output is G_X MX-quantized (the gradient the
 * previous layer consumes, quantized once: §III-A, §IV-B) instead of fp32:
 * dxq receives exactly the codes and scales that mqconv_quantize of
 * mqconv_backward_data's fp32 G_X would write; the fp32 G_X never reaches
 * memory.
 *   dxq: GRAD (H, W, N, Cin), any format; bp 1, or bp 32 when N is a
 *        multiple of 32 or divides 32 (otherwise MQ_ERR_UNSUPPORTED). Its
 *        code and scale buffers are fully overwritten.
 *   dyq, wq, ws, ws_bytes, errors: as mqconv_backward_data. */
int mqconv_backward_data_mx(const mq_conv* cv, mq_mx dyq, mq_mx wq, mq_mx dxq, void* ws,
                            size_t ws_bytes, void* stream);

/* Weight-gradient GEMM G_Wf = G_Yf . X'^T (§IV-B; Eq. 3).
 *   dyq: GRAD (Ho, Wo, N, Cout) and xq: ACT (H, W, N, Cin), both bp 32
 *        (the contraction runs along N, the partner dimension; bp 1 returns
 *        MQ_ERR_UNSUPPORTED).
 *   dw: fp32 [Cout][Kh][Kw][Cin], fully overwritten. */
int mqconv_backward_weight(const mq_conv* cv, mq_mx dyq, mq_mx xq, float* dw, void* ws,
                           size_t ws_bytes, void* stream);

/* mqconv_backward_weight for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and result, bit for bit, with no workspace argument. Its
 * scratch space (re-laid codes and split-K partial sums) is a fixed array of
 * MQ_NOALLOC_SCRATCH_BYTES in device memory that this library holds on every
 * device it runs on until the process ends; the call itself allocates and
 * frees nothing.
 *   Arguments and errors: as mqconv_backward_weight, and MQ_ERR_WORKSPACE
 *   when the problem needs more scratch than MQ_NOALLOC_SCRATCH_BYTES
 *   (mqconv_workspace_bytes(cv, 2, dyq.fmt, xq.fmt) tells how much it
 *   needs); MQ_ERR_HIP if the scratch array's address cannot be taken.
 *   Every call on one device uses that device's one array: calls that
 *   overlap in time on one device (two streams, two host threads) race and
 *   give undefined results; calls ordered on one stream are safe. */
#define MQ_NOALLOC_SCRATCH_BYTES (96u << 20)
int mqconv_backward_weight_noalloc(const mq_conv* cv, mq_mx dyq, mq_mx xq, float* dw, void* stream);

/* ---------------------------------------------------------------------------
 * Naive comparison path (kept only to measure bytes moved; §III-C, Table I
 * "Dacapo" column). Every tensor stays fp32 in memory; im2col is explicit
 * and runs before quantization; 1-D blocks of 32 follow the GEMM direction,
 * so X' and W and G_Y are each quantized twice:
 *   X'  = classic im2col of X: rows m = (ho, wo, n), columns k = (ci, kh, kw)
 *         (channel-major patch flattening, §II-C1/§II-C2), zero outside.
 *   W_f = W flattened to [Cout][k] with the same k order.
 *   forward:  X' and W_f quantized along k;          Y  = X'q . W_fq^T
 *   backward-data: G_Y [m][Cout] and W_f quantized along Cout;
 *             G_X' = G_Yq . W_fq (fp32 [m][k]), then col2im into G_X
 *   backward-weight: G_Y and X' quantized along m;   G_W = G_Yq^T . X'q
 * Inputs and outputs are fp32 in the layouts above (x, dy, dx CBF; w, dw
 * [Cout][Kh][Kw][Cin]). The workspace holds the expanded and quantized
 * intermediates.
 * --------------------------------------------------------------------------- */
size_t mqconv_naive_workspace_bytes(const mq_conv* cv, int op, mq_elem fa, mq_elem fb);
int mqconv_naive_forward(const mq_conv* cv, const float* x, const float* w, mq_elem fx,
                         mq_elem fw, float* y, void* ws, size_t ws_bytes, void* stream);
int mqconv_naive_backward_data(const mq_conv* cv, const float* dy, const float* w, mq_elem fdy,
                               mq_elem fw, float* dx, void* ws, size_t ws_bytes, void* stream);
int mqconv_naive_backward_weight(const mq_conv* cv, const float* dy, const float* x,
                                 mq_elem fdy, mq_elem fx, float* dw, void* ws, size_t ws_bytes,
                                 void* stream);

/* ---------------------------------------------------------------------------
 * Two-level (NVFP-style) microscaling, §II-D / §III-A Eqs. (4)-(6), the
 * pages' experimental format: one FP32 scale for the whole tensor and one
 * E4M3 scale per square block of 64 elements (8 channels x 8 partner
 * indices inside one pixel or tap, §IV-B):
 *   T   = max|X| / (448 * m)             m = largest element value (6 for E2M1)
 *   B_i = E4M3(max|X_i| / (T * m))       rounded to nearest even, saturating
 *   q   = code of X_i / (B_i * T)        rounded to nearest even, saturating
 * evaluated in fp32 (IEEE division and products); dequantized value =
 * value(q) * B_i * T. An all-zero tensor gets T = 0 and zero codes; a block
 * whose scale rounds to 0 gets zero codes; non-finite values are left out of
 * T and their block gets the E4M3 NaN byte 0x7F and zero codes.
 * Codes: the packed layout of the role above (mqconv_codes_bytes).
 * Block scales (E4M3 bytes): ACT/GRAD [H][W][ceil(N/8)][ceil(C/8)],
 * WEIGHT [Kh][Kw][ceil(Cout/8)][ceil(Cin/8)] (mqconv_nvfp_scales_bytes).
 * tensor_scale: one fp32 on the device. ws: mqconv_nvfp_workspace_bytes()
 * bytes of device scratch (partial maxima).
 * The GEMMs of the path take E8M0 block scales (what gfx950's block-scaled
 * MFMA applies per 32 K-elements); this format is quantized and measured
 * (error against the E8M0 format at equal element bits), not multiplied.
 * --------------------------------------------------------------------------- */
size_t mqconv_nvfp_scales_bytes(mq_role role, int32_t d0, int32_t d1, int32_t d2, int32_t d3);
size_t mqconv_nvfp_workspace_bytes(void);
int mqconv_nvfp_quantize(const float* src, mq_role role, mq_elem fmt, int32_t d0, int32_t d1, int32_t d2, int32_t d3,
                         void* codes, uint8_t* block_scales, float* tensor_scale, void* ws, size_t ws_bytes,
                         void* stream);

/* ---------------------------------------------------------------------------
 * Square-block comparator (§III-C: the method of ref. [25], square blocks on
 * the im2col-expanded activation of a fully connected layer, extended to
 * convolution), kept to compare bytes moved and quantization error:
 *   X'  = classic im2col of X as in the naive path (rows m = (ho, wo, n),
 *         columns k = (ci, kh, kw)), quantized ONCE in 32 x 32 squares (32
 *         consecutive m x 32 consecutive k, truncated at the edges) and kept
 *         for the backward pass (the saved, expanded activation);
 *   W_f [Cout][k] and G_Y [m][Cout] quantized once in squares as well;
 *   forward:         Y    = X'q . W_fq^T
 *   backward-data:   G_X' = G_Yq . W_fq, then col2im into G_X
 *   backward-weight: G_W  = G_Yq^T . X'q (the saved X'q)
 * A square's codes serve the contraction along either of its sides: where a
 * GEMM contracts across the codes' runs it reads a copy re-laid in the
 * workspace (codes move, no value is quantized again).
 * Saved X'q: codes [M][ceil(K/32)] runs of 32 k (layout of packed rows as
 * above), scales [ceil(M/32)][ceil(K/32)] E8M0 bytes, M = Ho*Wo*N,
 * K = Cin*Kh*Kw. fp32 tensors x, dy, dx, w, dw as in the naive path.
 * op of the workspace query: 0 forward (fa = X format, fb = W format),
 * 1 backward-data (fa = dY, fb = W), 2 backward-weight (fa = dY, fb = X).
 * --------------------------------------------------------------------------- */
size_t mqconv_cuyckens_col_codes_bytes(const mq_conv* cv, mq_elem fx);
size_t mqconv_cuyckens_col_scales_bytes(const mq_conv* cv);
size_t mqconv_cuyckens_workspace_bytes(const mq_conv* cv, int op, mq_elem fa, mq_elem fb);
int mqconv_cuyckens_im2col_quantize(const mq_conv* cv, const float* x, mq_elem fx, void* col_codes,
                                    uint8_t* col_scales, void* stream);
int mqconv_cuyckens_forward(const mq_conv* cv, const void* col_codes, const uint8_t* col_scales, mq_elem fx,
                            const float* w, mq_elem fw, float* y, void* ws, size_t ws_bytes, void* stream);
int mqconv_cuyckens_backward_data(const mq_conv* cv, const float* dy, const float* w, mq_elem fdy, mq_elem fw,
                                  float* dx, void* ws, size_t ws_bytes, void* stream);
int mqconv_cuyckens_backward_weight(const mq_conv* cv, const float* dy, const void* col_codes,
                                    const uint8_t* col_scales, mq_elem fdy, mq_elem fx, float* dw, void* ws,
                                    size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MQCONV_H */
