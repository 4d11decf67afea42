// libttq C ABI (include/ttq.h): argument validation, size queries, the
// handle that carries one q_proj's quantisation from prefill to decode, and
// dispatch to the HIP kernels.  Every check runs before anything is
// enqueued, so a rejected call leaves every output untouched.  No C++
// exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <new>
#include <string>

#include "../../include/ttq.h"
#include "ttq_internal.h"

struct ttq_handle {
  ttq_config cfg;
  ttq_buffers buf;
  const void* wsrc;  // W (r = 0) or buf.wres (r > 0)
  const void* w;     // W itself (the online refresh of the factors reads it)
  bool weight_bound;
  bool prepared;
  bool wexp_valid;  // the last prepare wrote the effective fp16 weight
};

namespace {

thread_local std::string g_last_error;

// The fp16 copy of D^(-1/2) that follows the fp32 values in the dinvsqrt
// buffer (4 d_in bytes in: 256-byte aligned, d_in being a multiple of 64).
void* dinv16(const ttq_handle* h) { return reinterpret_cast<char*>(h->buf.dinvsqrt) + (size_t)h->cfg.d_in * 4; }

ttq_status fail(ttq_status s, const char* fmt, ...) {
  char msg[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(msg, sizeof msg, fmt, ap);
  va_end(ap);
  g_last_error = msg;
  return s;
}

ttq_status ok() {
  g_last_error.clear();
  return TTQ_OK;
}

ttq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TTQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Longest row stride (elements) of a projection input: the prefill kernel
// addresses a 256-row input tile through a buffer resource whose byte
// offsets are 32-bit (at most 0x7FFFFFF0), so 256 * ld * 2 bytes must stay
// below 2^31.
constexpr int64_t kMaxGemmLd = (int64_t(1) << 22) - 8;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define TTQ_NEED(ptr)                                                          \
  do {                                                                         \
    if ((ptr) == nullptr) return fail(TTQ_ERR_NULL, "%s is NULL", #ptr);       \
    if (!aligned16(ptr)) return fail(TTQ_ERR_ALIGN, "%s is not 16-byte aligned", #ptr); \
  } while (0)

ttq_status check_qgr(int32_t q, int32_t g, int32_t r) {
  if (q < 2 || q > 5) return fail(TTQ_ERR_INVALID_ARG, "q=%d, expected 2, 3, 4 or 5", q);
  if (g == 8) return fail(TTQ_ERR_UNSUPPORTED, "group size 8 is not built (16, 32, 64 or 128)");
  if (g != 16 && g != 32 && g != 64 && g != 128) return fail(TTQ_ERR_INVALID_ARG, "g=%d, expected 16, 32, 64 or 128", g);
  if (r < 0) return fail(TTQ_ERR_INVALID_ARG, "r=%d is negative", r);
  if (r != 0 && r != 16) return fail(TTQ_ERR_UNSUPPORTED, "rank r=%d is not built (0 or 16)", r);
  return TTQ_OK;
}

ttq_status check_dims(int64_t d_in, int64_t d_out, int32_t g) {
  if (d_in <= 0 || d_in % 64 != 0) return fail(TTQ_ERR_SHAPE, "d_in=%lld must be a positive multiple of 64", (long long)d_in);
  if (d_in % g != 0) return fail(TTQ_ERR_SHAPE, "d_in=%lld is not a multiple of g=%d", (long long)d_in, g);
  if (d_in > kMaxGemmLd) return fail(TTQ_ERR_SHAPE, "d_in=%lld too large (at most %lld)", (long long)d_in, (long long)kMaxGemmLd);
  if (d_out <= 0 || d_out % 32 != 0) return fail(TTQ_ERR_SHAPE, "d_out=%lld must be a positive multiple of 32", (long long)d_out);
  if (d_out > (1 << 24)) return fail(TTQ_ERR_SHAPE, "d_out=%lld too large", (long long)d_out);
  return TTQ_OK;
}

ttq_status check_stats(float alpha, float lambda, float p) {
  if (!std::isfinite(alpha) || alpha < 0.f) return fail(TTQ_ERR_INVALID_ARG, "alpha=%g must be finite and >= 0", alpha);
  if (!std::isfinite(p) || p <= 0.f) return fail(TTQ_ERR_INVALID_ARG, "p=%g must be finite and > 0", p);
  if (!std::isfinite(lambda) || lambda < 0.f) return fail(TTQ_ERR_INVALID_ARG, "lambda=%g must be finite and >= 0", lambda);
  if (lambda == 0.f && alpha != 0.f)
    return fail(TTQ_ERR_INVALID_ARG, "lambda=0 with alpha>0 gives d_j=0 for a dead channel");
  return TTQ_OK;
}

ttq_status check_cfg(const ttq_config* cfg) {
  if (cfg == nullptr) return fail(TTQ_ERR_NULL, "cfg is NULL");
  ttq_status s = check_qgr(cfg->q, cfg->g, cfg->r);
  if (s != TTQ_OK) return s;
  s = check_dims(cfg->d_in, cfg->d_out, cfg->g);
  if (s != TTQ_OK) return s;
  return check_stats(cfg->alpha, cfg->lambda, cfg->p);
}

// Largest byte extent of a strided matrix argument, (rows - 1) * ld + cols
// elements: 2^48 bytes, beyond any device memory, so that no offset a kernel
// forms overflows 64 bits.
constexpr int64_t kMaxExtentBytes = int64_t(1) << 48;
bool extent_ok(int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
  if (rows <= 1) return cols <= kMaxExtentBytes / elem;
  const int64_t max_elems = kMaxExtentBytes / elem;
  return ld <= (max_elems - cols) / (rows - 1);
}

ttq_status check_x(const void* X, ttq_dtype xdt, int64_t T, int64_t d, int64_t ldx) {
  if (xdt != TTQ_F16 && xdt != TTQ_F32) return fail(TTQ_ERR_INVALID_ARG, "unknown dtype %d", (int)xdt);
  if (T < 0) return fail(TTQ_ERR_SHAPE, "T=%lld is negative", (long long)T);
  if (T > (int64_t(1) << 31)) return fail(TTQ_ERR_SHAPE, "T=%lld too large", (long long)T);
  if (ldx < d) return fail(TTQ_ERR_SHAPE, "ldx=%lld < d=%lld", (long long)ldx, (long long)d);
  if (ldx % 8 != 0) return fail(TTQ_ERR_ALIGN, "ldx=%lld is not a multiple of 8", (long long)ldx);
  if (!extent_ok(T, d, ldx, xdt == TTQ_F32 ? 4 : 2))
    return fail(TTQ_ERR_SHAPE, "T=%lld rows of stride ldx=%lld span more than 2^48 bytes", (long long)T,
                (long long)ldx);
  if (T > 0) TTQ_NEED(X);
  return TTQ_OK;
}

// Long prompts with fp16 input run the dense GEMM on the effective fp16
// weight W_hat when the caller gave the handle a buffer for it (opt-in): from
// a 256 x 256 tile grid of kDenseMinTiles tiles (two workgroups per CU) on,
// forming W_hat once per prompt can cost less than dequantising every weight
// fragment again for each token tile.  Whether it does depends on the
// machine: the low-bit GEMM measured as fast or faster on most MI355X boxes,
// so handles without the buffer, the default, keep it.
constexpr int64_t kDenseMinTiles = 512;
int64_t dense_min_tokens(int64_t d_out) {
  const int64_t tn = (d_out + 255) / 256;
  return 256 * ((kDenseMinTiles + tn - 1) / tn - 1) + 1;
}
bool use_dense(const ttq_handle* h, ttq_dtype xdt, int64_t T) {
  return h->buf.wexp != nullptr && xdt == TTQ_F16 && T > ttq::kDecodeMaxT && T >= dense_min_tokens(h->cfg.d_out);
}

// Codes, scales and zeros of W_src D^(1/2) for the prompt just measured; for
// a prompt that takes the dense projection also the effective weight, with
// the rank-16 term folded in when r > 0 (fp16(W_hat + B A)), so that the
// dense GEMM on it is the whole projection.
hipError_t quantize(const ttq_handle* h, ttq_dtype xdt, int64_t T, const void* W_src, hipStream_t st) {
  const ttq_config& c = h->cfg;
  const bool expand = use_dense(h, xdt, T);
  const bool fold = expand && c.r > 0;
  return ttq::launch_quantize_pack(c.d_out, c.d_in, c.q, c.g, W_src, h->buf.D, h->buf.codes, h->buf.scales,
                                   h->buf.zeros, expand ? dinv16(h) : nullptr, expand ? h->buf.wexp : nullptr,
                                   fold ? h->buf.B : nullptr, fold ? h->buf.A : nullptr, st);
}

size_t colstats_ws_bytes(int64_t T, int64_t d) {
  return (size_t)ttq::colstats_chunks(T < 1 ? 1 : T) * (size_t)d * sizeof(float);
}

// ttq_linear's workspace: Xs (fp16 [T][d_in]) then, for r > 0, Z (fp32 [T][r]);
// for r = 0 and a few tokens (kFewTokMaxT < T <= kDecodeMaxT) the split-K
// partial products instead, when they are larger
size_t xs_bytes(int64_t T, int64_t d) { return ((size_t)T * (size_t)d * 2 + 255) & ~(size_t)255; }
size_t linear_ws_bytes(int64_t T, int64_t d, int64_t d_out, int32_t r) {
  size_t b = xs_bytes(T, d) + (r > 0 ? (size_t)T * (size_t)r * 4 : 0);
  if (r == 0 && d >= 64 && d_out > 0) b = std::max(b, ttq::decode_splitk_ws_bytes(T, (int)d, (int)d_out));
  return b;
}

// the row stride of a projection input (X, or the pre-scaled Xs)
ttq_status check_gemm_ld(int64_t ld, const char* name) {
  if (ld > kMaxGemmLd)
    return fail(TTQ_ERR_SHAPE, "%s=%lld too large (at most %lld elements)", name, (long long)ld, (long long)kMaxGemmLd);
  return TTQ_OK;
}

// ttq_prefill's workspace: with the rank-16 term and fp16 input of more than
// kDecodeMaxT tokens, the fused statistic pass's partial sums, then Z (fp32
// [T][r]); otherwise what ttq_linear needs (the handle's own workspace takes
// the statistic)
bool prefill_fused(int64_t T, int32_t r, ttq_dtype xdt) { return r > 0 && xdt == TTQ_F16 && T > ttq::kDecodeMaxT; }
size_t fused_partial_bytes(int64_t T, int64_t d) {
  return ((size_t)ttq::colstats_z_chunks(T) * (size_t)d * 4 + 255) & ~(size_t)255;
}
size_t prefill_ws_bytes(int64_t T, int64_t d, int64_t d_out, int32_t r, ttq_dtype xdt) {
  if (prefill_fused(T, r, xdt)) return fused_partial_bytes(T, d) + (size_t)T * (size_t)r * 4;
  return linear_ws_bytes(T, d, d_out, r);
}

ttq_status check_y(const void* Y, ttq_dtype ydt, int64_t T, int64_t d_out, int64_t ldy) {
  if (ydt != TTQ_F16 && ydt != TTQ_F32) return fail(TTQ_ERR_INVALID_ARG, "unknown dtype %d", (int)ydt);
  if (ldy < d_out) return fail(TTQ_ERR_SHAPE, "ldy=%lld < d_out=%lld", (long long)ldy, (long long)d_out);
  if (ldy % 8 != 0) return fail(TTQ_ERR_ALIGN, "ldy=%lld is not a multiple of 8", (long long)ldy);
  if (!extent_ok(T, d_out, ldy, ydt == TTQ_F32 ? 4 : 2))
    return fail(TTQ_ERR_SHAPE, "T=%lld rows of stride ldy=%lld span more than 2^48 bytes", (long long)T,
                (long long)ldy);
  if (T > 0) TTQ_NEED(Y);
  return TTQ_OK;
}

}  // namespace

extern "C" {

int32_t ttq_abi_version(void) { return TTQ_ABI_VERSION; }

const char* ttq_status_string(ttq_status s) {
  switch (s) {
    case TTQ_OK: return "TTQ_OK";
    case TTQ_ERR_INVALID_ARG: return "TTQ_ERR_INVALID_ARG: argument out of range";
    case TTQ_ERR_UNSUPPORTED: return "TTQ_ERR_UNSUPPORTED: not built for the GPU";
    case TTQ_ERR_SHAPE: return "TTQ_ERR_SHAPE: inconsistent sizes";
    case TTQ_ERR_NULL: return "TTQ_ERR_NULL: required pointer is NULL";
    case TTQ_ERR_ALIGN: return "TTQ_ERR_ALIGN: misaligned pointer or stride";
    case TTQ_ERR_HIP: return "TTQ_ERR_HIP: HIP runtime error";
  }
  return "unknown ttq_status";
}

const char* ttq_last_error(void) { return g_last_error.c_str(); }

size_t ttq_colstats_workspace_bytes(int64_t T, int64_t d) {
  if (T < 0 || d <= 0) return 0;
  return colstats_ws_bytes(T, d);
}

ttq_status ttq_query_sizes(const ttq_config* cfg, int64_t T_max, ttq_sizes* out) {
  ttq_status s = check_cfg(cfg);
  if (s != TTQ_OK) return s;
  if (out == nullptr) return fail(TTQ_ERR_NULL, "out is NULL");
  if (T_max < 1) return fail(TTQ_ERR_SHAPE, "T_max=%lld must be >= 1", (long long)T_max);
  const size_t din = (size_t)cfg->d_in, dout = (size_t)cfg->d_out;
  out->codes_bytes = dout * (din / 32) * (size_t)cfg->q * 4;
  out->scales_bytes = dout * (din / (size_t)cfg->g) * 2;
  out->zeros_bytes = out->scales_bytes;
  out->d_bytes = din * 4;
  out->dinvsqrt_bytes = din * 4 + din * 2;  // fp32, then the fp16 copy
  out->wres_bytes = cfg->r > 0 ? dout * din * 2 : 0;
  out->wexp_bytes = dout * din * 2;
  out->workspace_bytes = colstats_ws_bytes(T_max, cfg->d_in);
  // the largest need over 1 <= T <= T_max: the prefill form grows with T, the
  // split-K form with T up to kDecodeMaxT
  out->linear_workspace_bytes =
      std::max(linear_ws_bytes(T_max, cfg->d_in, cfg->d_out, cfg->r),
               linear_ws_bytes(std::min<int64_t>(T_max, ttq::kDecodeMaxT), cfg->d_in, cfg->d_out, cfg->r));
  return ok();
}

ttq_status ttq_create(const ttq_config* cfg, const ttq_buffers* bufs, ttq_handle** out) {
  if (out == nullptr) return fail(TTQ_ERR_NULL, "out is NULL");
  if (bufs == nullptr) return fail(TTQ_ERR_NULL, "bufs is NULL");
  ttq_sizes sz;
  ttq_status s = ttq_query_sizes(cfg, bufs->T_max, &sz);
  if (s != TTQ_OK) return s;
  TTQ_NEED(bufs->codes);
  TTQ_NEED(bufs->scales);
  TTQ_NEED(bufs->zeros);
  TTQ_NEED(bufs->D);
  TTQ_NEED(bufs->dinvsqrt);
  TTQ_NEED(bufs->workspace);
  if (bufs->workspace_bytes < sz.workspace_bytes)
    return fail(TTQ_ERR_SHAPE, "workspace %zu bytes < %zu needed", bufs->workspace_bytes, sz.workspace_bytes);
  if (bufs->wexp != nullptr && !aligned16(bufs->wexp)) return fail(TTQ_ERR_ALIGN, "bufs->wexp is not 16-byte aligned");
  if (cfg->r > 0) {
    TTQ_NEED(bufs->wres);
    TTQ_NEED(bufs->B);
    TTQ_NEED(bufs->A);
  }
  ttq_handle* h = new (std::nothrow) ttq_handle;
  if (h == nullptr) return fail(TTQ_ERR_INVALID_ARG, "host allocation of the handle failed");
  h->cfg = *cfg;
  h->buf = *bufs;
  h->wsrc = nullptr;
  h->w = nullptr;
  h->weight_bound = false;
  h->prepared = false;
  h->wexp_valid = false;
  *out = h;
  return ok();
}

void ttq_destroy(ttq_handle* h) { delete h; }

ttq_status ttq_set_weight(ttq_handle* h, const void* W, void* stream) {
  if (h == nullptr) return fail(TTQ_ERR_NULL, "handle is NULL");
  TTQ_NEED(W);
  h->w = W;
  if (h->cfg.r == 0) {
    h->wsrc = W;
    h->weight_bound = true;
    return ok();
  }
  hipError_t e = ttq::launch_residual(h->cfg.d_out, h->cfg.d_in, h->cfg.r, W, h->buf.B, h->buf.A,
                                      h->buf.wres, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "residual launch");
  h->wsrc = h->buf.wres;
  h->weight_bound = true;
  return ok();
}

ttq_status ttq_colstats(const void* X, ttq_dtype xdt, int64_t T, int64_t d, int64_t ldx, float p,
                        float lambda, float alpha, float* D, float* dinvsqrt, float* workspace,
                        size_t workspace_bytes, void* stream) {
  if (d <= 0 || d % 8 != 0) return fail(TTQ_ERR_SHAPE, "d=%lld must be a positive multiple of 8", (long long)d);
  ttq_status s = check_x(X, xdt, T, d, ldx);
  if (s != TTQ_OK) return s;
  if (T < 1) return fail(TTQ_ERR_SHAPE, "T=%lld: the statistic needs at least one token", (long long)T);
  s = check_stats(alpha, lambda, p);
  if (s != TTQ_OK) return s;
  TTQ_NEED(D);
  TTQ_NEED(dinvsqrt);
  TTQ_NEED(workspace);
  if (workspace_bytes < colstats_ws_bytes(T, d))
    return fail(TTQ_ERR_SHAPE, "workspace %zu bytes < %zu needed", workspace_bytes, colstats_ws_bytes(T, d));
  hipError_t e = ttq::launch_colstats(X, xdt == TTQ_F32, T, d, ldx, p, lambda, alpha, D, dinvsqrt, nullptr,
                                      workspace, static_cast<hipStream_t>(stream));
  return hip_status(e, "colstats launch");
}

ttq_status ttq_colstats_noalloc(const void* X, ttq_dtype xdt, int64_t T, int64_t d, int64_t ldx, float p,
                                float lambda, float alpha, float* D, float* dinvsqrt, void* stream) {
  if (d <= 0 || d % 8 != 0) return fail(TTQ_ERR_SHAPE, "d=%lld must be a positive multiple of 8", (long long)d);
  ttq_status s = check_x(X, xdt, T, d, ldx);
  if (s != TTQ_OK) return s;
  if (T < 1) return fail(TTQ_ERR_SHAPE, "T=%lld: the statistic needs at least one token", (long long)T);
  s = check_stats(alpha, lambda, p);
  if (s != TTQ_OK) return s;
  TTQ_NEED(D);
  TTQ_NEED(dinvsqrt);
  if (d > ttq::kColstatsScratchMaxD)
    return fail(TTQ_ERR_SHAPE, "d=%lld: the fixed scratch (%zu bytes) holds the partial sums of at most %d channels",
                (long long)d, ttq::kColstatsScratchBytes, ttq::kColstatsScratchMaxD);
  hipError_t e = ttq::launch_colstats_noalloc(X, xdt == TTQ_F32, T, d, ldx, p, lambda, alpha, D, dinvsqrt,
                                              static_cast<hipStream_t>(stream));
  return hip_status(e, "colstats launch (fixed scratch)");
}

ttq_status ttq_quantize_pack(int32_t d_out, int32_t d_in, int32_t q, int32_t g, const void* W_src,
                             const float* D, uint32_t* codes, void* scales, void* zeros,
                             void* stream) {
  ttq_status s = check_qgr(q, g, 0);
  if (s != TTQ_OK) return s;
  s = check_dims(d_in, d_out, g);
  if (s != TTQ_OK) return s;
  TTQ_NEED(W_src);
  TTQ_NEED(D);
  TTQ_NEED(codes);
  TTQ_NEED(scales);
  TTQ_NEED(zeros);
  hipError_t e = ttq::launch_quantize_pack(d_out, d_in, q, g, W_src, D, codes, scales, zeros, nullptr, nullptr,
                                           nullptr, nullptr, static_cast<hipStream_t>(stream));
  return hip_status(e, "quantize_pack launch");
}

ttq_status ttq_residual(int32_t d_out, int32_t d_in, int32_t r, const void* W, const float* B,
                        const float* A, void* W_res, void* stream) {
  ttq_status s = check_dims(d_in, d_out, 32);
  if (s != TTQ_OK) return s;
  if (r != 16) return fail(r <= 0 ? TTQ_ERR_INVALID_ARG : TTQ_ERR_UNSUPPORTED, "r=%d, the residual kernel is built for r=16", r);
  TTQ_NEED(W);
  TTQ_NEED(B);
  TTQ_NEED(A);
  TTQ_NEED(W_res);
  hipError_t e = ttq::launch_residual(d_out, d_in, r, W, B, A, W_res, static_cast<hipStream_t>(stream));
  return hip_status(e, "residual launch");
}

ttq_status ttq_lowrank_z(int64_t T, int32_t d_in, int32_t r, const void* X, ttq_dtype xdt,
                         int64_t ldx, const float* A, float* Z, void* stream) {
  if (d_in <= 0 || d_in % 64 != 0) return fail(TTQ_ERR_SHAPE, "d_in=%d must be a positive multiple of 64", d_in);
  if (r != 16) return fail(r <= 0 ? TTQ_ERR_INVALID_ARG : TTQ_ERR_UNSUPPORTED, "r=%d, the kernel is built for r=16", r);
  ttq_status s = check_x(X, xdt, T, d_in, ldx);
  if (s != TTQ_OK) return s;
  if (T == 0) return ok();
  TTQ_NEED(A);
  TTQ_NEED(Z);
  hipError_t e = ttq::launch_prescale_z(T, d_in, X, xdt == TTQ_F32, ldx, nullptr, nullptr, A, Z,
                                        static_cast<hipStream_t>(stream));
  return hip_status(e, "lowrank_z launch");
}

ttq_status ttq_prescale(const void* X, ttq_dtype xdt, int64_t T, int32_t d_in, int64_t ldx,
                        const float* dinvsqrt, void* Xs, void* stream) {
  if (d_in <= 0 || d_in % 64 != 0) return fail(TTQ_ERR_SHAPE, "d_in=%d must be a positive multiple of 64", d_in);
  ttq_status s = check_x(X, xdt, T, d_in, ldx);
  if (s != TTQ_OK) return s;
  if (T == 0) return ok();
  TTQ_NEED(dinvsqrt);
  TTQ_NEED(Xs);
  hipError_t e = ttq::launch_prescale_z(T, d_in, X, xdt == TTQ_F32, ldx, dinvsqrt, Xs, nullptr, nullptr,
                                        static_cast<hipStream_t>(stream));
  return hip_status(e, "prescale launch");
}

ttq_status ttq_wlowbit_gemm(int64_t T, int32_t d_in, int32_t d_out, int32_t q, int32_t g, int32_t r,
                            const void* Xs, int64_t ldxs, const uint32_t* codes, const void* scales,
                            const void* zeros, const float* B, const float* Z, void* Y, ttq_dtype ydt,
                            int64_t ldy, void* stream) {
  ttq_status s = check_qgr(q, g, r);
  if (s != TTQ_OK) return s;
  s = check_dims(d_in, d_out, g);
  if (s != TTQ_OK) return s;
  s = check_x(Xs, TTQ_F16, T, d_in, ldxs);
  if (s != TTQ_OK) return s;
  s = check_gemm_ld(ldxs, "ldxs");
  if (s != TTQ_OK) return s;
  s = check_y(Y, ydt, T, d_out, ldy);
  if (s != TTQ_OK) return s;
  if (T == 0) return ok();
  TTQ_NEED(codes);
  TTQ_NEED(scales);
  TTQ_NEED(zeros);
  if (r > 0) {
    TTQ_NEED(B);
    TTQ_NEED(Z);
  }
  hipError_t e = ttq::launch_wlowbit_gemm(T, d_in, d_out, q, g, r, Xs, ldxs, codes, scales, zeros, B, Z,
                                          Y, ydt == TTQ_F32, ldy, static_cast<hipStream_t>(stream));
  return hip_status(e, "wlowbit_gemm launch");
}

ttq_status ttq_wlowbit_gemm_raw(int64_t T, int32_t d_in, int32_t d_out, int32_t q, int32_t g, int32_t r,
                                const void* X, int64_t ldx, const void* dinv16, const uint32_t* codes,
                                const void* scales, const void* zeros, const float* B, const float* Z, void* Y,
                                int64_t ldy, void* stream) {
  ttq_status s = check_qgr(q, g, r);
  if (s != TTQ_OK) return s;
  s = check_dims(d_in, d_out, g);
  if (s != TTQ_OK) return s;
  s = check_x(X, TTQ_F16, T, d_in, ldx);
  if (s != TTQ_OK) return s;
  s = check_gemm_ld(ldx, "ldx");
  if (s != TTQ_OK) return s;
  if (T <= ttq::kDecodeMaxT)
    return fail(TTQ_ERR_SHAPE, "T=%lld: the raw-input form is for T > %d (use ttq_linear)", (long long)T,
                ttq::kDecodeMaxT);
  s = check_y(Y, TTQ_F16, T, d_out, ldy);
  if (s != TTQ_OK) return s;
  TTQ_NEED(dinv16);
  TTQ_NEED(codes);
  TTQ_NEED(scales);
  TTQ_NEED(zeros);
  if (r > 0) {
    TTQ_NEED(B);
    TTQ_NEED(Z);
  }
  hipError_t e = ttq::launch_wlowbit_gemm_rawx(T, d_in, d_out, q, g, r, X, ldx, dinv16, codes, scales, zeros, B,
                                               Z, Y, ldy, static_cast<hipStream_t>(stream));
  return hip_status(e, "wlowbit_gemm launch");
}

ttq_status ttq_prepare(ttq_handle* h, const void* X, ttq_dtype xdt, int64_t T, int64_t ldx,
                       void* stream) {
  if (h == nullptr) return fail(TTQ_ERR_NULL, "handle is NULL");
  if (!h->weight_bound) return fail(TTQ_ERR_INVALID_ARG, "ttq_set_weight has not been called");
  const ttq_config& c = h->cfg;
  ttq_status s = check_x(X, xdt, T, c.d_in, ldx);
  if (s != TTQ_OK) return s;
  if (T < 1) return fail(TTQ_ERR_SHAPE, "T=%lld: prepare needs at least one token", (long long)T);
  if (T > h->buf.T_max) return fail(TTQ_ERR_SHAPE, "T=%lld exceeds the handle's T_max=%lld", (long long)T, (long long)h->buf.T_max);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = ttq::launch_colstats(X, xdt == TTQ_F32, T, c.d_in, ldx, c.p, c.lambda, c.alpha, h->buf.D,
                                      h->buf.dinvsqrt, dinv16(h), h->buf.workspace, st);
  if (e != hipSuccess) return hip_status(e, "colstats launch");
  e = quantize(h, xdt, T, h->wsrc, st);
  if (e != hipSuccess) return hip_status(e, "quantize_pack launch");
  h->prepared = true;
  h->wexp_valid = use_dense(h, xdt, T);
  return ok();
}

size_t ttq_linear_workspace_bytes(int64_t T, int32_t d_in, int32_t d_out, int32_t r) {
  if (T < 0 || d_in <= 0 || d_out < 0 || r < 0) return 0;
  return linear_ws_bytes(T, d_in, d_out, r);
}

ttq_status ttq_linear(const ttq_handle* h, const void* X, ttq_dtype xdt, int64_t T, int64_t ldx,
                      void* Y, int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  if (h == nullptr) return fail(TTQ_ERR_NULL, "handle is NULL");
  const ttq_config& c = h->cfg;
  ttq_status s = check_x(X, xdt, T, c.d_in, ldx);
  if (s != TTQ_OK) return s;
  s = check_gemm_ld(ldx, "ldx");
  if (s != TTQ_OK) return s;
  s = check_y(Y, xdt, T, c.d_out, ldy);
  if (s != TTQ_OK) return s;
  if (!h->prepared) return fail(TTQ_ERR_INVALID_ARG, "ttq_prepare has not been called on this handle");
  if (T == 0) return ok();
  TTQ_NEED(workspace);
  const size_t need = linear_ws_bytes(T, c.d_in, c.d_out, c.r);
  if (workspace_bytes < need) return fail(TTQ_ERR_SHAPE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (c.r == 0 && T == 1) {
    // one token: the dot-product form, pre-scaling the input itself
    hipError_t e = ttq::launch_wlowbit_gemv_raw(c.d_in, c.d_out, c.q, c.g, X, xdt == TTQ_F32, h->buf.dinvsqrt,
                                                h->buf.codes, h->buf.scales, h->buf.zeros, Y, st);
    return hip_status(e, "wlowbit_gemv launch");
  }
  if (xdt == TTQ_F16 && T >= 2 && T <= ttq::kFewTokMaxT) {
    // a few fp16 tokens: the few-token form on X itself, D^(-1/2) applied on
    // the weight side (Z = X A^T first when r > 0)
    float* z = c.r > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + xs_bytes(T, c.d_in)) : nullptr;
    hipError_t e = hipSuccess;
    if (c.r > 0) e = ttq::launch_prescale_z(T, c.d_in, X, false, ldx, h->buf.dinvsqrt, nullptr, h->buf.A, z, st);
    if (e != hipSuccess) return hip_status(e, "lowrank_z launch");
    e = ttq::launch_wlowbit_fewtok(T, c.d_in, c.d_out, c.q, c.g, c.r, X, ldx, dinv16(h), h->buf.codes,
                                   h->buf.scales, h->buf.zeros, h->buf.B, z, Y, false, ldy, st);
    return hip_status(e, "wlowbit_fewtok launch");
  }
  if (c.r == 0 && T > ttq::kFewTokMaxT && T <= ttq::kDecodeMaxT) {
    // up to 64 tokens: split-K over 256-row workgroups, partials in the workspace
    hipError_t e = ttq::launch_wlowbit_decode_splitk(T, c.d_in, c.d_out, c.q, c.g, X, xdt == TTQ_F32, ldx,
                                                     h->buf.dinvsqrt, h->buf.codes, h->buf.scales,
                                                     h->buf.zeros, Y, ldy, workspace, st);
    return hip_status(e, "wlowbit_decode_splitk launch");
  }
  void* xs = workspace;
  float* z = c.r > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + xs_bytes(T, c.d_in)) : nullptr;
  if (h->wexp_valid && use_dense(h, xdt, T)) {
    // a long prompt: the dense GEMM on the effective weight the last prepare
    // formed (r = 0: the raw-input GEMM's results on the codes bit for bit;
    // r > 0: B A is already in the weight)
    hipError_t e = ttq::launch_dense_gemm(T, c.d_in, c.d_out, 0, X, ldx, h->buf.wexp, nullptr, nullptr, Y, ldy, st);
    return hip_status(e, "dense_gemm launch");
  }
  if (xdt == TTQ_F16 && T > ttq::kDecodeMaxT) {
    // fp16 input: the GEMM reads X itself, D^(-1/2) applied on the weight side
    hipError_t e = hipSuccess;
    if (c.r > 0) e = ttq::launch_prescale_z(T, c.d_in, X, false, ldx, h->buf.dinvsqrt, nullptr, h->buf.A, z, st);
    if (e != hipSuccess) return hip_status(e, "lowrank_z launch");
    e = ttq::launch_wlowbit_gemm_rawx(T, c.d_in, c.d_out, c.q, c.g, c.r, X, ldx, dinv16(h), h->buf.codes,
                                      h->buf.scales, h->buf.zeros, h->buf.B, z, Y, ldy, st);
    return hip_status(e, "wlowbit_gemm launch");
  }
  hipError_t e = ttq::launch_prescale_z(T, c.d_in, X, xdt == TTQ_F32, ldx, h->buf.dinvsqrt, xs,
                                        c.r > 0 ? h->buf.A : nullptr, z, st);
  if (e != hipSuccess) return hip_status(e, "prescale launch");
  e = ttq::launch_wlowbit_gemm(T, c.d_in, c.d_out, c.q, c.g, c.r, xs, c.d_in, h->buf.codes, h->buf.scales,
                               h->buf.zeros, h->buf.B, z, Y, xdt == TTQ_F32, ldy, st);
  return hip_status(e, "wlowbit_gemm launch");
}

size_t ttq_prefill_workspace_bytes(int64_t T, int32_t d_in, int32_t d_out, int32_t r, ttq_dtype xdt) {
  if (T < 0 || d_in <= 0 || d_out < 0 || r < 0 || (xdt != TTQ_F16 && xdt != TTQ_F32)) return 0;
  return prefill_ws_bytes(T, d_in, d_out, r, xdt);
}

ttq_status ttq_prefill(ttq_handle* h, const void* X, ttq_dtype xdt, int64_t T, int64_t ldx, void* Y, int64_t ldy,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (h == nullptr) return fail(TTQ_ERR_NULL, "handle is NULL");
  const ttq_config& c = h->cfg;
  ttq_status s = check_x(X, xdt, T, c.d_in, ldx);
  if (s != TTQ_OK) return s;
  s = check_gemm_ld(ldx, "ldx");
  if (s != TTQ_OK) return s;
  s = check_y(Y, xdt, T, c.d_out, ldy);
  if (s != TTQ_OK) return s;
  if (!h->weight_bound) return fail(TTQ_ERR_INVALID_ARG, "ttq_set_weight has not been called");
  if (T < 1) return fail(TTQ_ERR_SHAPE, "T=%lld: prefill needs at least one token", (long long)T);
  if (T > h->buf.T_max) return fail(TTQ_ERR_SHAPE, "T=%lld exceeds the handle's T_max=%lld", (long long)T, (long long)h->buf.T_max);
  TTQ_NEED(workspace);
  const size_t need = prefill_ws_bytes(T, c.d_in, c.d_out, c.r, xdt);
  if (workspace_bytes < need) return fail(TTQ_ERR_SHAPE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  if (!prefill_fused(T, c.r, xdt)) {
    // no rank-16 term to fuse: exactly ttq_prepare then ttq_linear
    s = ttq_prepare(h, X, xdt, T, ldx, stream);
    if (s != TTQ_OK) return s;
    return ttq_linear(h, X, xdt, T, ldx, Y, ldy, workspace, workspace_bytes, stream);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (use_dense(h, xdt, T)) {
    // a long prompt: B A is folded into the effective weight, so the
    // statistic, the quantisation and one dense GEMM are the whole step
    s = ttq_prepare(h, X, xdt, T, ldx, stream);
    if (s != TTQ_OK) return s;
    hipError_t e = ttq::launch_dense_gemm(T, c.d_in, c.d_out, 0, X, ldx, h->buf.wexp, nullptr, nullptr, Y, ldy, st);
    return hip_status(e, "dense_gemm launch");
  }
  float* partial = static_cast<float*>(workspace);
  float* z = reinterpret_cast<float*>(static_cast<char*>(workspace) + fused_partial_bytes(T, c.d_in));
  hipError_t e = ttq::launch_colstats_z(X, T, c.d_in, ldx, c.p, c.lambda, c.alpha, h->buf.A, h->buf.D,
                                        h->buf.dinvsqrt, dinv16(h), partial, z, st);
  if (e != hipSuccess) return hip_status(e, "colstats_z launch");
  e = quantize(h, xdt, T, h->wsrc, st);
  if (e != hipSuccess) return hip_status(e, "quantize_pack launch");
  h->prepared = true;
  h->wexp_valid = false;
  e = ttq::launch_wlowbit_gemm_rawx(T, c.d_in, c.d_out, c.q, c.g, c.r, X, ldx, dinv16(h), h->buf.codes,
                                    h->buf.scales, h->buf.zeros, h->buf.B, z, Y, ldy, st);
  return hip_status(e, "projection launch");
}

int64_t ttq_dense_min_tokens(int32_t d_out) {
  if (d_out <= 0) return -1;
  return std::max<int64_t>(dense_min_tokens(d_out), ttq::kDecodeMaxT + 1);
}

ttq_status ttq_wexp_gemm(int64_t T, int32_t d_in, int32_t d_out, int32_t r, const void* X, int64_t ldx,
                         const void* Wexp, const float* B, const float* Z, void* Y, int64_t ldy, void* stream) {
  ttq_status s = check_qgr(4, 32, r);
  if (s != TTQ_OK) return s;
  s = check_dims(d_in, d_out, 32);
  if (s != TTQ_OK) return s;
  s = check_x(X, TTQ_F16, T, d_in, ldx);
  if (s != TTQ_OK) return s;
  s = check_gemm_ld(ldx, "ldx");
  if (s != TTQ_OK) return s;
  s = check_y(Y, TTQ_F16, T, d_out, ldy);
  if (s != TTQ_OK) return s;
  if (T == 0) return ok();
  TTQ_NEED(Wexp);
  if (r > 0) {
    TTQ_NEED(B);
    TTQ_NEED(Z);
  }
  hipError_t e = ttq::launch_dense_gemm(T, d_in, d_out, r, X, ldx, Wexp, B, Z, Y, ldy,
                                        static_cast<hipStream_t>(stream));
  return hip_status(e, "dense_gemm launch");
}

size_t ttq_lowrank_refresh_workspace_bytes(int32_t d_out, int32_t d_in, int32_t r) {
  if (d_out <= 0 || d_in <= 0 || r != 16) return 0;
  return ttq::lowrank_refresh_ws_bytes(d_out, d_in);
}

namespace {
ttq_status check_refresh(int32_t d_out, int32_t d_in, int32_t r, const void* W, const float* D, const float* V,
                         const float* B, const float* A, const void* workspace, size_t workspace_bytes) {
  if (r != 16) return fail(r <= 0 ? TTQ_ERR_INVALID_ARG : TTQ_ERR_UNSUPPORTED, "r=%d, the refresh is built for r=16", r);
  ttq_status s = check_dims(d_in, d_out, 32);
  if (s != TTQ_OK) return s;
  if (d_in % 128 != 0) return fail(TTQ_ERR_SHAPE, "d_in=%d must be a multiple of 128 for the refresh", d_in);
  TTQ_NEED(W);
  TTQ_NEED(D);
  TTQ_NEED(V);
  TTQ_NEED(B);
  TTQ_NEED(A);
  TTQ_NEED(workspace);
  const size_t need = ttq::lowrank_refresh_ws_bytes(d_out, d_in);
  if (workspace_bytes < need) return fail(TTQ_ERR_SHAPE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  return TTQ_OK;
}
}  // namespace

ttq_status ttq_lowrank_refresh(int32_t d_out, int32_t d_in, int32_t r, const void* W, const float* D, float* V,
                               float* B, float* A, void* workspace, size_t workspace_bytes, void* stream) {
  ttq_status s = check_refresh(d_out, d_in, r, W, D, V, B, A, workspace, workspace_bytes);
  if (s != TTQ_OK) return s;
  hipError_t e = ttq::launch_lowrank_refresh(d_out, d_in, W, D, V, B, A, workspace, static_cast<hipStream_t>(stream));
  return hip_status(e, "lowrank_refresh launch");
}

ttq_status ttq_prepare_refresh(ttq_handle* h, const void* X, ttq_dtype xdt, int64_t T, int64_t ldx, float* V,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (h == nullptr) return fail(TTQ_ERR_NULL, "handle is NULL");
  if (!h->weight_bound) return fail(TTQ_ERR_INVALID_ARG, "ttq_set_weight has not been called");
  const ttq_config& c = h->cfg;
  ttq_status s = check_x(X, xdt, T, c.d_in, ldx);
  if (s != TTQ_OK) return s;
  if (T < 1) return fail(TTQ_ERR_SHAPE, "T=%lld: prepare needs at least one token", (long long)T);
  if (T > h->buf.T_max) return fail(TTQ_ERR_SHAPE, "T=%lld exceeds the handle's T_max=%lld", (long long)T, (long long)h->buf.T_max);
  // the handle's factor buffers are caller-owned device memory; the refresh rewrites them
  float* B = const_cast<float*>(h->buf.B);
  float* A = const_cast<float*>(h->buf.A);
  s = check_refresh(c.d_out, c.d_in, c.r, h->w, h->buf.D, V, B, A, workspace, workspace_bytes);
  if (s != TTQ_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = ttq::launch_colstats(X, xdt == TTQ_F32, T, c.d_in, ldx, c.p, c.lambda, c.alpha, h->buf.D,
                                      h->buf.dinvsqrt, dinv16(h), h->buf.workspace, st);
  if (e != hipSuccess) return hip_status(e, "colstats launch");
  e = ttq::launch_lowrank_refresh(c.d_out, c.d_in, h->w, h->buf.D, V, B, A, workspace, st);
  if (e != hipSuccess) return hip_status(e, "lowrank_refresh launch");
  e = ttq::launch_residual(c.d_out, c.d_in, c.r, h->w, B, A, h->buf.wres, st);
  if (e != hipSuccess) return hip_status(e, "residual launch");
  e = quantize(h, xdt, T, h->buf.wres, st);
  if (e != hipSuccess) return hip_status(e, "quantize_pack launch");
  h->prepared = true;
  h->wexp_valid = use_dense(h, xdt, T);
  return ok();
}

}  // extern "C"
