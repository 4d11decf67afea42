/*
 * ttq.h - C ABI of the TTQ (activation-aware test-time quantization) q_proj
 * hot path for AMD Instinct MI355X (gfx950).
 *
 * What it computes (arXiv 2603.19296, "TTQ: Activation-Aware Test-Time
 * Quantization to Accelerate LLM Inference On The Fly"):
 *   per prompt X [T][d]:  d_j = (mean_t |x_tj|^p + lambda)^alpha
 *     (paper-daily.com deep reading, section 2, online AWQ diagonal;
 *      gist.science German summary, section 2, p-norm form)
 *   W_res = W - B A with static rank-r factors from the SVD of W
 *     (paper-daily.com section 2 low-rank compensation; gist.science French
 *      summary, section 2B)
 *   codes, scales, zeros = group RTN of W_res D^(1/2)
 *     (paper-daily.com section 2: RTN QDQ and the closed form Q[W D^(1/2)] D^(-1/2))
 *   Y = Q[W_res D^(1/2)] (D^(-1/2) X) + B (A X)
 *     (paper-daily.com section 5: a low-bit kernel on the pre-scaled input)
 * Quantisation parameters are computed at prefill and reused by decode
 * (paper-daily.com section 6).
 *
 * Conventions for every entry point
 *   - Tensors are row-major.  X is [T][ldx] (tokens x input channels, the
 *     first d columns used), W is [d_out][d_in] fp16, Y is [T][ldy].
 *   - Pointers marked "device" are HIP device (or managed) memory owned by
 *     the caller.  The library never allocates, frees or synchronises device
 *     memory; it only enqueues kernels on the caller's stream.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All calls are asynchronous; inputs must stay valid until the enqueued
 *     work has run.  Device faults surface at the caller's next
 *     synchronisation.
 *   - Every function validates all arguments before enqueuing anything; on
 *     error it returns a non-zero ttq_status, writes nothing, and leaves a
 *     thread-local message readable with ttq_last_error().
 *   - Alignment: every device base pointer must be 16-byte aligned, and row
 *     strides (ldx, ldy) must be multiples of 8 elements (TTQ_ERR_ALIGN).
 *   - NaN or Inf in X, W or D propagate or give unspecified codes; they are
 *     not checked.
 *   - No C++ exception crosses this interface.
 *
 * Packed code format (the pages fix none).  Codes: per output row, blocks
 * of 32 consecutive input channels; each block is q little-endian uint32
 * words forming one bitstream, slot k of the block at bits [q*k, q*k+q).
 * Inside every 8 channels, slots 0..7 hold the codes of channels
 * 0 2 4 6 1 3 5 7 (so slots j and j+4 hold the neighbours 2j and 2j+1).
 * The words are stored in a tiled order, so that one 64-channel step of 32
 * output rows is one contiguous chunk of 32 * 2q words:
 *   word w of block b of row n  ->  index ((nt * (d_in/64) + ks) * 32 + r) * 2q + pos
 *   nt = n / 32, r = n % 32, ks = b / 2, h = b % 2,
 *   pos = 4*(w % 2) + 2*h + w/2 for q = 4 (words b0w0 b0w2 b1w0 b1w2 b0w1
 *   b0w3 b1w1 b1w3), pos = q*h + w for q = 2, 3, 5.
 * Scales and zeros (fp16, zeros exact integers 0..2^q-1), one per row n and
 * group gi of g channels, are stored at index (nt * (d_in/g) + gi) * 32 + r.
 * codes hold d_out * (d_in/32) * q uint32; scales and zeros d_out * (d_in/g)
 * fp16 each.
 */
#ifndef TTQ_H
#define TTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTQ_ABI_VERSION 6

typedef enum ttq_status {
  TTQ_OK = 0,
  TTQ_ERR_INVALID_ARG = 1, /* a scalar argument out of its documented range */
  TTQ_ERR_UNSUPPORTED = 2, /* valid for the method, not built for the GPU (e.g. g=16) */
  TTQ_ERR_SHAPE = 3,       /* sizes inconsistent, or a buffer too small */
  TTQ_ERR_NULL = 4,        /* a required pointer is NULL */
  TTQ_ERR_ALIGN = 5,       /* a pointer or stride breaks the alignment rule */
  TTQ_ERR_HIP = 6          /* the HIP runtime refused a launch */
} ttq_status;

typedef enum ttq_dtype {
  TTQ_F32 = 0,
  TTQ_F16 = 1
} ttq_dtype;

/* Hyper-parameters of one q_proj.  Fixed per layer, no test-time search
 * (paper-daily.com section 2: alpha 0.5-0.75, lambda 0.4, p = 2).
 *   d_in  (d)  input channels,  multiple of 64 and of g
 *   d_out (d') output channels, multiple of 32
 *   q  bits per code: 2, 3, 4 or 5
 *   g  group size along d_in: 16, 32, 64 or 128 (8: TTQ_ERR_UNSUPPORTED)
 *   r  low-rank rank: 0 or 16
 *   alpha >= 0, p > 0, lambda > 0 unless alpha == 0 (a dead channel would
 *   otherwise get d_j = 0 and an infinite D^(-1/2)). */
typedef struct ttq_config {
  int32_t d_in;
  int32_t d_out;
  int32_t q;
  int32_t g;
  int32_t r;
  float alpha;
  float lambda;
  float p;
} ttq_config;

/* Byte sizes of every caller-owned buffer for a configuration and the
 * largest T a handle will see. */
typedef struct ttq_sizes {
  size_t codes_bytes;     /* uint32, d_out * (d_in/32) * q, tiled order  */
  size_t scales_bytes;    /* fp16, d_out * (d_in/g), tiled order         */
  size_t zeros_bytes;     /* fp16, d_out * (d_in/g), tiled order         */
  size_t d_bytes;         /* fp32   [d_in]   D                           */
  size_t dinvsqrt_bytes;  /* fp32   [d_in]   D^(-1/2), then its fp16     *
                          * copy [d_in] (read by ttq_linear)            */
  size_t wres_bytes;      /* fp16   [d_out][d_in] W - B A (0 when r = 0) */
  size_t workspace_bytes; /* prepare: column-statistic partial sums      */
  size_t linear_workspace_bytes; /* ttq_linear on any T <= T_max          */
  size_t wexp_bytes;      /* fp16   [d_out][d_in] effective weight W_hat  *
                          * (optional buffer, see ttq_buffers.wexp)      */
} ttq_sizes;

/* Device buffers a handle works in (all caller-owned, see ttq_sizes).
 * B (fp32 [d_out][r]) and A (fp32 [r][d_in]) are the static factors; they
 * and wres are ignored when r = 0.  The workspace serves ttq_prepare only.
 * wexp (optional, may be NULL): room for the effective fp16 weight
 * W_hat[n][j] = fp16(fp16((c - z) s) * fp16(d_j^(-1/2))), the pages' closed
 * form Q[(W - B A) D^(1/2)] D^(-1/2) (paper-daily.com deep reading, section
 * 2) in exactly the fp16 values the low-bit projection kernel dequantises.
 * With it, a prepare on an fp16 prompt of at least
 * ttq_dense_min_tokens(d_out) tokens also writes W_hat, and projections of
 * that many fp16 tokens run a dense fp16 GEMM on it: the dequantisation is
 * done once per prompt instead of once per 256-token tile, with the same
 * outputs bit for bit.  With r = 16 the buffer receives fp16(W_hat + B A)
 * instead (the fp32 sum rounded once; section 2's Y = W_hat X + B (A X) is
 * (W_hat + B A) X), so that GEMM is the whole projection, with no A X; its
 * outputs are then within the tolerance of the low-bit kernel's, not the
 * same bits.  Without it (NULL) every prompt runs the low-bit GEMM on the
 * codes, which on most MI355X boxes measured was as fast in the whole
 * prefill step and needs no d_out x d_in fp16 buffer. */
typedef struct ttq_buffers {
  uint32_t* codes;
  void* scales;
  void* zeros;
  float* D;
  float* dinvsqrt;
  void* wres;
  const float* B;
  const float* A;
  float* workspace;
  int64_t T_max;
  size_t workspace_bytes;
  void* wexp;
} ttq_buffers;

typedef struct ttq_handle ttq_handle;

/* ABI version the library was built with (TTQ_ABI_VERSION). */
int32_t ttq_abi_version(void);

/* Static text for a status code.  Never NULL. */
const char* ttq_status_string(ttq_status s);

/* Detail of the last error on the calling thread ("" if none).  Valid until
 * the next call into the library on this thread. */
const char* ttq_last_error(void);

/* Pure host: checks cfg and fills *out for prompts of up to T_max tokens.
 * (Bookkeeping of this library's buffers; the pages define no such call.) */
ttq_status ttq_query_sizes(const ttq_config* cfg, int64_t T_max, ttq_sizes* out);

/* Pure host: creates an opaque host object recording cfg and the device
 * pointers in *bufs (not owning them).  Buffers are checked against
 * ttq_query_sizes(cfg, bufs->T_max).  Destroy with ttq_destroy.  The handle
 * is the per-layer state the pages carry from prefill to decode: the
 * hyper-parameters fixed per layer (paper-daily.com deep reading, section 2)
 * and the quantisation computed at prefill (section 6). */
ttq_status ttq_create(const ttq_config* cfg, const ttq_buffers* bufs, ttq_handle** out);
void ttq_destroy(ttq_handle* h);

/* Binds the weight W (device fp16 [d_out][d_in]) once per layer.
 * r = 0: the handle borrows W (keep it alive and unchanged).
 * r > 0: enqueues W_res = fp16(W - B A) into bufs->wres, with the product
 *   accumulated in fp64 from the fp32 factors and rounded once (the factors
 *   come from a host SVD of W, computed once: paper-daily.com section 2,
 *   gist.science French summary section 2B). */
ttq_status ttq_set_weight(ttq_handle* h, const void* W, void* stream);

/* Per-prompt prefill step, prepare(X, W, q, g, alpha, lambda, p) with W and
 * the hyper-parameters bound in the handle:
 *   D, D^(-1/2) = colstats(X)  then  codes, scales, zeros = quantize(W_res, D)
 * (paper-daily.com deep reading, section 2: the diagonal from the prompt's own
 * activations, then group RTN of W D^(1/2); section 6: once per prompt at
 * prefill; nubint.ai review, proposed-method section: weights quantised on
 * the fly by group-wise RTN with QDQ).
 * D^(-1/2) is written as fp32 followed by an fp16 copy (ttq_sizes).
 * X: device [T][ldx] of dtype xdt, 1 <= T <= T_max. */
ttq_status ttq_prepare(ttq_handle* h, const void* X, ttq_dtype xdt, int64_t T,
                       int64_t ldx, void* stream);

/* The low-bit projection with the handle's current quantisation:
 *   Y = Q[W_res D^(1/2)] (D^(-1/2) X) + B (A X)
 * (paper-daily.com deep reading, section 2: the closed form and the low-rank
 * term; section 5: a low-bit kernel on the pre-scaled input; section 6:
 * decode steps reuse the prefill's parameters).
 * X: device [T][ldx] of dtype xdt; Y: device [T][ldy] of the same dtype,
 * fp32 accumulation.  Any T >= 0; T = 0 enqueues nothing.  Used for the
 * prefill tokens and, unchanged, for decode batches that reuse the prefill
 * quantisation.  fp16 input with T > 64: the dense GEMM on the effective
 * weight the last prepare formed (ttq_wexp_gemm, the rank-16 term already in
 * the weight; prompts of at least ttq_dense_min_tokens(d_out) tokens on a
 * handle with a wexp buffer), or ttq_lowrank_z into `workspace` when r > 0
 * and then ttq_wlowbit_gemm_raw on X itself (D^(-1/2) applied to the
 * dequantised weights, with the fp16 copy ttq_prepare wrote).  r = 0, T = 1: one dot-product kernel that pre-scales
 * the input itself (the same bits as ttq_prescale + ttq_wlowbit_gemm).  fp16
 * input, 2 <= T <= 16: one few-token kernel on X with D^(-1/2) on the weight
 * side (Z first when r > 0).  r = 0, 16 < T <= 64: a split-K kernel whose
 * 256-row workgroups share their input slice, fp32 partial products in
 * `workspace`, then a reduction in a fixed order (for d_in <= 5120 the
 * output equals ttq_wlowbit_gemm's bit for bit).  Otherwise (fp32 input, or
 * r > 0 with T <= 64 outside the cases above): ttq_prescale (fused with
 * ttq_lowrank_z when r > 0: one read of X) into `workspace`, then
 * ttq_wlowbit_gemm.
 * workspace: device memory of at least
 * ttq_linear_workspace_bytes(T, d_in, d_out, r) bytes, owned by the caller
 * (required for every T >= 1); the handle itself is only read, so calls on
 * one handle may run concurrently on different streams when each has its own
 * workspace. */
size_t ttq_linear_workspace_bytes(int64_t T, int32_t d_in, int32_t d_out, int32_t r);
ttq_status ttq_linear(const ttq_handle* h, const void* X, ttq_dtype xdt, int64_t T,
                      int64_t ldx, void* Y, int64_t ldy, void* workspace,
                      size_t workspace_bytes, void* stream);

/* The whole per-prompt prefill step in one call: ttq_prepare(X) then
 * ttq_linear(X) on the same prompt (paper-daily.com deep reading, section 6:
 * the quantisation parameters are computed from the prompt at prefill; the
 * projection of the prompt follows).  Writes D, D^(-1/2), codes, scales and
 * zeros into the handle (as ttq_prepare) and Y = the projection of X (as
 * ttq_linear).  With r = 16, fp16 input and 64 < T below the dense
 * projection's length (ttq_dense_min_tokens, or any T when the handle has
 * no wexp buffer) the column statistic and Z = X A^T come from one read of
 * X (the form the two separate calls cannot use, since ttq_linear may see
 * other inputs than the prompt); D and Z are then summed in other fixed
 * groupings than those of ttq_prepare and ttq_linear and may differ from
 * theirs in the last bits (D within 1e-5 of the exact statistic either way,
 * Z within fp32 rounding).  Otherwise it is exactly ttq_prepare followed by
 * ttq_linear (for a long prompt with r = 16: no Z at all, the rank-16 term
 * being folded into the effective weight).  workspace: device memory of
 * at least ttq_prefill_workspace_bytes(T, d_in, d_out, r, xdt) bytes, owned
 * by the caller; the handle's own workspace is used too (by the statistic of
 * the unfused form).  1 <= T <= T_max; the input stride ldx must stay below
 * 2^22 elements (as for ttq_linear). */
size_t ttq_prefill_workspace_bytes(int64_t T, int32_t d_in, int32_t d_out, int32_t r, ttq_dtype xdt);
ttq_status ttq_prefill(ttq_handle* h, const void* X, ttq_dtype xdt, int64_t T, int64_t ldx, void* Y,
                       int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);

/* ttq_prepare with an online refresh of the rank-16 factors first (r = 16
 * only).  The pages keep B, A static after their SVD initialisation and
 * note that an online PCA could update them at extra cost (paper-daily.com
 * deep reading, section 5, limitations; gist.science French summary,
 * section 2B).  Here, per prompt: D = colstats(X); one subspace-iteration
 * step of the right basis V toward the principal subspace of the
 * activation-weighted weight W D^(1/2) (ttq_lowrank_refresh); B, A from it,
 * written into the handle's B and A buffers (caller-owned device memory,
 * rewritten in place); W_res = fp16(W - B A) into the handle's wres buffer;
 * then quantize_pack as in ttq_prepare.  V: device fp32 [d_in][16], an
 * orthonormal basis on the first call (the right singular vectors of W give
 * back the static factors for a uniform D), updated in place.  workspace:
 * device memory of at least ttq_lowrank_refresh_workspace_bytes(d_out, d_in,
 * 16) bytes, owned by the caller.  The handle borrows W (ttq_set_weight):
 * keep it alive and unchanged.  d_in must be a multiple of 128.  Must not
 * overlap a ttq_linear on the same handle. */
ttq_status ttq_prepare_refresh(ttq_handle* h, const void* X, ttq_dtype xdt, int64_t T, int64_t ldx, float* V,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Smallest number of fp16 tokens for which a handle with a wexp buffer takes
 * the dense path (pure host; -1 for d_out <= 0). */
int64_t ttq_dense_min_tokens(int32_t d_out);

/* ---- Sub-steps, exported so each kernel can be checked on its own ---- */

/* Column statistic: D[j] = fp32((mean_{t<T} |X[t][j]|^p + lambda)^alpha) and
 * dinvsqrt[j] = fp32(1/sqrt(D[j])), j < d (paper-daily.com deep reading,
 * section 2: the online AWQ diagonal with shrinkage lambda and exponent
 * alpha; gist.science German summary, section 2: the p-norm of each input
 * channel over the prompt).  Partial sums go to workspace
 * (fp32, at least ttq_colstats_workspace_bytes(T, d) bytes).  Sums are
 * taken in a fixed order: the result is deterministic. */
size_t ttq_colstats_workspace_bytes(int64_t T, int64_t d);
ttq_status ttq_colstats(const void* X, ttq_dtype xdt, int64_t T, int64_t d, int64_t ldx,
                        float p, float lambda, float alpha, float* D, float* dinvsqrt,
                        float* workspace, size_t workspace_bytes, void* stream);

/* The column statistic of ttq_colstats without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the partial sums
 * live in a fixed array of the library on each GPU it runs on (8 MiB per
 * GPU, held until the process ends; nothing is allocated or freed per call).
 * Same arguments and results as ttq_colstats, bit for bit.  Limit: the
 * partial sums of d channels must fit, i.e. d <= 16384 (TTQ_ERR_SHAPE
 * otherwise).  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race; a call's results
 * never depend on what an earlier call left there.  The array of the device
 * the stream belongs to is used (looked up on the first call per device). */
ttq_status ttq_colstats_noalloc(const void* X, ttq_dtype xdt, int64_t T, int64_t d, int64_t ldx, float p,
                                float lambda, float alpha, float* D, float* dinvsqrt, void* stream);

/* One online step of the rank-16 factors (the sub-step of
 * ttq_prepare_refresh; same passages): with M = W D^(1/2),
 *   P = M^T (M V),  V' = P R^-1 where R^T R = P^T P (Cholesky, fp64),
 *   B = M V',  A = V'^T D^(-1/2)   (so B A = M V' V'^T D^(-1/2)).
 * W device fp16 [d_out][d_in]; D device fp32 [d_in]; V device fp32
 * [d_in][16] (orthonormal; replaced by V'); B device fp32 [d_out][16] and A
 * device fp32 [16][d_in] (written).  Products of W with the basis run on the
 * matrix cores with fp16 W and the fp32 basis split in two fp16 parts (about
 * 22 bits) or in fp32; the 16 x 16 algebra in fp64.  A direction the weighted
 * weight does not span gives zero columns of B and zero rows of A.  r must be
 * 16, d_in a multiple of 128, d_out of 32.  workspace: at least
 * ttq_lowrank_refresh_workspace_bytes(d_out, d_in, 16) bytes. */
size_t ttq_lowrank_refresh_workspace_bytes(int32_t d_out, int32_t d_in, int32_t r);
ttq_status ttq_lowrank_refresh(int32_t d_out, int32_t d_in, int32_t r, const void* W, const float* D, float* V,
                               float* B, float* A, void* workspace, size_t workspace_bytes, void* stream);

/* Quantise and pack W_src D^(1/2) (device fp16 [d_out][d_in], D device fp32
 * [d_in]), the group RTN of the activation-weighted weight
 * (paper-daily.com deep reading, section 2: RTN QDQ per group of W D^(1/2);
 * nubint.ai review, proposed-method section), with these rules: fp32 arithmetic, zero-inclusive
 * group range, fp16 scale rounded upward, z = rint(-mn/s),
 * c = clamp(rint(v/s) + z, 0, 2^q-1), round half to even, IEEE division.
 * Writes codes, scales, zeros (layouts above).  Any D > 0 may be supplied
 * (e.g. D = 1 gives plain RTN, a calibrated D gives static AWQ). */
ttq_status ttq_quantize_pack(int32_t d_out, int32_t d_in, int32_t q, int32_t g,
                             const void* W_src, const float* D, uint32_t* codes,
                             void* scales, void* zeros, void* stream);

/* W_res = fp16(W - B A): W device fp16 [d_out][d_in], B device fp32
 * [d_out][r], A device fp32 [r][d_in]; products summed in fp64
 * (paper-daily.com deep reading, section 2: W split into B A plus a
 * quantised residual; gist.science French summary, section 2B). */
ttq_status ttq_residual(int32_t d_out, int32_t d_in, int32_t r, const void* W,
                        const float* B, const float* A, void* W_res, void* stream);

/* Z = X A^T, the input of the low-rank term B (A X) (paper-daily.com deep
 * reading, section 2; gist.science French summary, section 2B):
 * X device [T][ldx] (dtype xdt), A device fp32 [r][d_in],
 * Z device fp32 [T][r], fp32 accumulation (A enters the matrix cores as two
 * fp16 parts, about 22 bits).  r must be 16. */
ttq_status ttq_lowrank_z(int64_t T, int32_t d_in, int32_t r, const void* X, ttq_dtype xdt,
                         int64_t ldx, const float* A, float* Z, void* stream);

/* Xs = fp16(dinvsqrt * X), the pre-scaled input D^(-1/2) X of the closed
 * form (paper-daily.com deep reading, section 2; section 5: the low-bit
 * kernel runs on the pre-scaled input): X device [T][ldx] (dtype xdt), dinvsqrt device
 * fp32 [d_in], Xs device fp16 [T][d_in] (dense rows, the channel order of
 * X).  Each product is taken in fp32 and rounded to fp16; d_in must be a
 * multiple of 64. */
ttq_status ttq_prescale(const void* X, ttq_dtype xdt, int64_t T, int32_t d_in, int64_t ldx,
                        const float* dinvsqrt, void* Xs, void* stream);

/* Y = V_hat Xs + B Z with V_hat[n][k] = (code - z) * s, fp16 operands on the
 * matrix cores and fp32 accumulation: Q[W_res D^(1/2)] (D^(-1/2) X) + B (A X)
 * on the pre-scaled input (paper-daily.com deep reading, sections 2 and 5;
 * thelatestinai.com, Tables 4-8: the query projection timed on the Qwen3
 * shapes of Table 15).  Xs: device fp16 [T][ldxs] as written
 * by ttq_prescale (ldxs >= d_in, a multiple of 8); codes/scales/zeros as
 * produced by ttq_quantize_pack; B device fp32 [d_out][r] and Z device fp32
 * [T][r] (both ignored when r = 0).  Y: device [T][ldy] of dtype ydt. */
ttq_status ttq_wlowbit_gemm(int64_t T, int32_t d_in, int32_t d_out, int32_t q, int32_t g,
                            int32_t r, const void* Xs, int64_t ldxs, const uint32_t* codes,
                            const void* scales, const void* zeros, const float* B,
                            const float* Z, void* Y, ttq_dtype ydt, int64_t ldy, void* stream);

/* The same projection straight from the raw fp16 input, the form ttq_linear
 * runs for fp16 X and T > 64: Y = (V_hat D^(-1/2)) X + B Z, D^(-1/2) applied
 * to each dequantised weight pair (paper-daily.com section 2: the closed form
 * Q[W D^(1/2)] D^(-1/2) X, here grouped as (Q[.] D^(-1/2)) X).
 * X device fp16 [T][ldx] (ldx >= d_in, a multiple of 8); dinv16 device fp16
 * [d_in], fp16(D^(-1/2)) (ttq_prepare writes it after the fp32 values in the
 * handle's dinvsqrt buffer); Y device fp16 [T][ldy].  T must exceed 64
 * (TTQ_ERR_SHAPE otherwise; fewer tokens go through ttq_linear).  Other
 * arguments as for ttq_wlowbit_gemm. */
ttq_status ttq_wlowbit_gemm_raw(int64_t T, int32_t d_in, int32_t d_out, int32_t q, int32_t g,
                                int32_t r, const void* X, int64_t ldx, const void* dinv16,
                                const uint32_t* codes, const void* scales, const void* zeros,
                                const float* B, const float* Z, void* Y, int64_t ldy, void* stream);

/* The dense projection on an effective fp16 weight, the form ttq_linear runs
 * for long fp16 prompts when the handle holds W_hat:
 *   Y = W_hat X + B Z   (paper-daily.com deep reading, section 2: the closed
 *   form Q[W D^(1/2)] D^(-1/2) applied to the raw input; B Z the static
 *   rank-16 term, gist.science French summary, section 2B)
 * X device fp16 [T][ldx] (ldx >= d_in, a multiple of 8, below 2^22); Wexp
 * device fp16 [d_out][d_in]; B device fp32 [d_out][r] and Z device fp32
 * [T][r] (ignored when r = 0); Y device fp16 [T][ldy].  fp16 operands on the
 * matrix cores, fp32 accumulation in the same K order as ttq_wlowbit_gemm_raw
 * (so on W_hat formed from that kernel's codes the outputs are identical).
 * Any T >= 0. */
ttq_status ttq_wexp_gemm(int64_t T, int32_t d_in, int32_t d_out, int32_t r, const void* X, int64_t ldx,
                         const void* Wexp, const float* B, const float* Z, void* Y, int64_t ldy, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TTQ_H */
