// C ABI (include/wq.h): argument validation, layout queries and dispatch to
// the kernel launchers.  Host-side checks run before any HIP call, so every
// error path is reachable without a GPU.
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "wq.h"
#include "wq_internal.hpp"

namespace {

thread_local char g_err[512] = {0};

wq_status fail(wq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

wq_status ok() {
  g_err[0] = 0;
  return WQ_OK;
}

wq_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(WQ_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

const char* fmt_name(int f) {
  switch (f) {
    case WQ_BF16: return "BF16";
    case WQ_INT4: return "INT4";
    case WQ_FP8: return "FP8";
    case WQ_NVFP4: return "NVFP4";
    case WQ_MXFP4: return "MXFP4";
    case WQ_INT4_ASYM: return "INT4_ASYM";
    default: return "?";
  }
}

bool valid_fmt(int f) { return f >= WQ_BF16 && f <= WQ_INT4_ASYM; }

// Kernel-side format id (the public ids coincide with the kernels' except the
// asymmetric INT4, whose kernel id follows the static-FP8 GEMM's).
int kfmt_of(int f) { return f == WQ_INT4_ASYM ? wq::KF_INT4A : f; }

// Divisibility rules of each format (INT4: group 128 along K; NVFP4: last two
// weight dims % 16; MXFP4: K and N % 32).
wq_status check_shape_rule(int f, int64_t N, int64_t K) {
  if (N < 0 || K < 0) return fail(WQ_EINVAL, "negative size N=%lld K=%lld", (long long)N, (long long)K);
  if ((f == WQ_INT4 || f == WQ_INT4_ASYM) && K % 128)
    return fail(WQ_ESHAPE, "INT4 needs K %% 128 == 0 (K=%lld)", (long long)K);
  if (f == WQ_NVFP4 && (N % 16 || K % 16))
    return fail(WQ_ESHAPE, "NVFP4 needs N %% 16 == 0 and K %% 16 == 0 (N=%lld K=%lld)", (long long)N, (long long)K);
  if (f == WQ_MXFP4 && (N % 32 || K % 32))
    return fail(WQ_ESHAPE, "MXFP4 needs N %% 32 == 0 and K %% 32 == 0 (N=%lld K=%lld)", (long long)N, (long long)K);
  return WQ_OK;
}

// Weight layouts: rows (0) for every format; tile order (1) for the quantized
// formats when whole 16-row x 64-byte tiles cover the weight.
wq_status check_layout(int f, int32_t layout, int64_t N, int64_t K) {
  if (layout != WQ_LAYOUT_ROWS && layout != WQ_LAYOUT_TILES) return fail(WQ_EINVAL, "unknown layout %d", (int)layout);
  if (layout == WQ_LAYOUT_TILES) {
    if (f == WQ_BF16) return fail(WQ_EUNSUPPORTED, "BF16 weights have only the rows layout");
    const int64_t kmul = f == WQ_FP8 ? 64 : 128;
    if (N % 16 || K % kmul)
      return fail(WQ_EUNSUPPORTED, "tile order needs N %% 16 == 0 and K %% %lld == 0 (N=%lld K=%lld)", (long long)kmul,
                  (long long)N, (long long)K);
  }
  return WQ_OK;
}

int kernel_k_multiple(int f) {
  switch (f) {
    case WQ_BF16: return 8;
    case WQ_FP8: return 16;
    default: return 32;
  }
}

constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int64_t kMaxBufferBytes = (int64_t)1 << 31;

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

extern "C" {

int wq_abi_version(void) { return WQ_ABI_VERSION; }

const char* wq_status_str(int s) {
  switch (s) {
    case WQ_OK: return "WQ_OK";
    case WQ_EINVAL: return "WQ_EINVAL";
    case WQ_ESHAPE: return "WQ_ESHAPE";
    case WQ_EALIGN: return "WQ_EALIGN";
    case WQ_EUNSUPPORTED: return "WQ_EUNSUPPORTED";
    case WQ_EWORKSPACE: return "WQ_EWORKSPACE";
    case WQ_EHIP: return "WQ_EHIP";
    default: return "WQ_UNKNOWN";
  }
}

const char* wq_last_error(void) { return g_err; }

wq_status wq_layout(int fmt, int64_t N, int64_t K, size_t* codes_bytes, size_t* packed_bytes,
                    size_t* scale_bytes, size_t* global_bytes) {
  if (!valid_fmt(fmt)) return fail(WQ_EINVAL, "unknown format %d", fmt);
  wq_status st = check_shape_rule(fmt, N, K);
  if (st != WQ_OK) return st;
  const size_t nk = (size_t)N * (size_t)K;
  size_t cb = 0, pb = 0, sb = 0, gb = 0;
  switch (fmt) {
    case WQ_BF16: cb = pb = 2 * nk; break;
    case WQ_INT4: cb = nk; pb = nk / 2; sb = (size_t)N * (size_t)(K / 128) * 2; break;
    case WQ_FP8: cb = pb = nk; sb = (size_t)N * 4; break;
    case WQ_NVFP4: cb = nk; pb = nk / 2; sb = (size_t)N * (size_t)(K / 16); gb = 4; break;
    case WQ_MXFP4: cb = nk; pb = nk / 2; sb = (size_t)N * (size_t)(K / 32); break;
    case WQ_INT4_ASYM: cb = nk; pb = nk / 2; sb = (size_t)N * (size_t)(K / 128) * 4; break;
  }
  if (codes_bytes) *codes_bytes = cb;
  if (packed_bytes) *packed_bytes = pb;
  if (scale_bytes) *scale_bytes = sb;
  if (global_bytes) *global_bytes = gb;
  return ok();
}

wq_status wq_quantize(int fmt, const void* W, int64_t N, int64_t K, void* codes, void* scales,
                      float* global_scale, void* stream) {
  if (!valid_fmt(fmt) || fmt == WQ_BF16) return fail(WQ_EINVAL, "wq_quantize: unsupported format %d", fmt);
  wq_status st = check_shape_rule(fmt, N, K);
  if (st != WQ_OK) return st;
  if (N > kMaxDim || K > kMaxDim) return fail(WQ_EUNSUPPORTED, "dimension above 2^30");
  if (N == 0 || K == 0) return ok();
  if (!W || !codes || !scales) return fail(WQ_EINVAL, "wq_quantize: null pointer");
  if ((fmt == WQ_NVFP4) != (global_scale != nullptr))
    return fail(WQ_EINVAL, "wq_quantize: global_scale is required for NVFP4 and must be NULL otherwise");
  if (!aligned16(W) || !aligned16(codes)) return fail(WQ_EALIGN, "wq_quantize: W and codes must be 16-byte aligned");
  return hip_status(wq::launch_quantize(kfmt_of(fmt), (const uint16_t*)W, N, K, codes, scales, global_scale,
                                        (hipStream_t)stream),
                    "wq_quantize launch");
}

wq_status wq_pack(int fmt, const void* codes, int64_t N, int64_t K, void* packed, void* stream) {
  if (!valid_fmt(fmt) || fmt == WQ_BF16) return fail(WQ_EINVAL, "wq_pack: unsupported format %d", fmt);
  wq_status st = check_shape_rule(fmt, N, K);
  if (st != WQ_OK) return st;
  if (N > kMaxDim || K > kMaxDim) return fail(WQ_EUNSUPPORTED, "dimension above 2^30");
  if (N == 0 || K == 0) return ok();
  if (!codes || !packed) return fail(WQ_EINVAL, "wq_pack: null pointer");
  if (!aligned16(codes) || !aligned16(packed)) return fail(WQ_EALIGN, "wq_pack: buffers must be 16-byte aligned");
  const int64_t nk = N * K;
  if (fmt == WQ_FP8 ? (nk % 16) : (nk % 32))
    return fail(WQ_EUNSUPPORTED, "wq_pack: N*K must be a multiple of %d", fmt == WQ_FP8 ? 16 : 32);
  return hip_status(wq::launch_pack(kfmt_of(fmt), (const uint8_t*)codes, N, K, (uint8_t*)packed, (hipStream_t)stream),
                    "wq_pack launch");
}

wq_status wq_dequantize(int fmt, const void* packed, int32_t layout, const void* scales, const float* global_scale,
                        int64_t N, int64_t K, void* W_out, void* stream) {
  if (!valid_fmt(fmt)) return fail(WQ_EINVAL, "wq_dequantize: unknown format %d", fmt);
  wq_status st = check_shape_rule(fmt, N, K);
  if (st != WQ_OK) return st;
  st = check_layout(fmt, layout, N, K);
  if (st != WQ_OK) return st;
  if (N > kMaxDim || K > kMaxDim) return fail(WQ_EUNSUPPORTED, "dimension above 2^30");
  if (N == 0 || K == 0) return ok();
  if (!packed || !W_out || (fmt != WQ_BF16 && !scales)) return fail(WQ_EINVAL, "wq_dequantize: null pointer");
  if (fmt == WQ_NVFP4 && !global_scale) return fail(WQ_EINVAL, "wq_dequantize: NVFP4 needs global_scale");
  if (K % 8) return fail(WQ_EUNSUPPORTED, "wq_dequantize: K %% 8 != 0");
  if (!aligned16(packed) || !aligned16(W_out)) return fail(WQ_EALIGN, "wq_dequantize: buffers must be 16-byte aligned");
  return hip_status(wq::launch_dequantize(kfmt_of(fmt), layout, packed, scales, global_scale, N, K, (uint16_t*)W_out,
                                          (hipStream_t)stream),
                    "wq_dequantize launch");
}

wq_status wq_repack(int fmt, int64_t N, int64_t K, int32_t src_layout, const void* src_packed, const void* src_scales,
                    int32_t dst_layout, void* dst_packed, void* dst_scales, void* stream) {
  if (!valid_fmt(fmt) || fmt == WQ_BF16) return fail(WQ_EINVAL, "wq_repack: unsupported format %d", fmt);
  wq_status st = check_shape_rule(fmt, N, K);
  if (st != WQ_OK) return st;
  st = check_layout(fmt, src_layout, N, K);
  if (st != WQ_OK) return st;
  st = check_layout(fmt, dst_layout, N, K);
  if (st != WQ_OK) return st;
  if (N > kMaxDim || K > kMaxDim) return fail(WQ_EUNSUPPORTED, "dimension above 2^30");
  if (N == 0 || K == 0) return ok();
  if (!src_packed || !src_scales || !dst_packed || !dst_scales) return fail(WQ_EINVAL, "wq_repack: null pointer");
  if (src_packed == dst_packed || src_scales == dst_scales)
    return fail(WQ_EINVAL, "wq_repack: source and destination must be distinct buffers");
  if (!aligned16(src_packed) || !aligned16(dst_packed) || !aligned16(src_scales) || !aligned16(dst_scales))
    return fail(WQ_EALIGN, "wq_repack: buffers must be 16-byte aligned");
  // rows layout with row bytes not a multiple of 16 is copied in 16-byte chunks: keep whole chunks per row
  if ((fmt == WQ_FP8 ? K : K / 2) % 16)
    return fail(WQ_EUNSUPPORTED, "wq_repack: rows of a multiple of 16 bytes needed (K=%lld)", (long long)K);
  if (fmt != WQ_FP8 && K % 128)
    return fail(WQ_EUNSUPPORTED, "wq_repack: block scales are moved per 128-K tile (K=%lld)", (long long)K);
  return hip_status(wq::launch_repack(kfmt_of(fmt), N, K, src_layout, src_packed, src_scales, dst_layout, dst_packed,
                                      dst_scales, (hipStream_t)stream),
                    "wq_repack launch");
}

size_t wq_linear_workspace(int fmt, int64_t M, int64_t N, int64_t K) {
  if (!valid_fmt(fmt) || M <= 0 || N <= 0 || K <= 0) return 0;
  return wq::plan_linear(kfmt_of(fmt), M, N, K).ws_bytes;
}

// Host-side checks of a dequant-GEMM call; on success fills the launch
// arguments and the plan.  Nothing is enqueued here, so callers that launch
// more than one kernel validate every launch before the first one.
static wq_status linear_check(int kfmt, int fmt, const void* X, int64_t M, int64_t K, const void* W, int32_t layout,
                              const void* scales, const float* gscale, const float* act_scale, const void* bias,
                              int64_t N, void* Y, void* ws, size_t ws_bytes, wq::LinearArgs* a, wq::LinearPlan* p,
                              bool* empty) {
  *empty = false;
  if (!valid_fmt(fmt)) return fail(WQ_EINVAL, "unknown format %d", fmt);
  if (M < 0 || N < 0 || K < 0) return fail(WQ_EINVAL, "negative size");
  wq_status st = check_shape_rule(fmt, N, K);
  if (st != WQ_OK) return st;
  st = check_layout(fmt, layout, N, K);
  if (st != WQ_OK) return st;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(WQ_EUNSUPPORTED, "dimension above 2^30");
  if (M == 0 || N == 0) {
    *empty = true;
    return ok();
  }
  if (K == 0) return fail(WQ_EUNSUPPORTED, "K == 0");
  if (K % kernel_k_multiple(fmt))
    return fail(WQ_EUNSUPPORTED, "%s linear kernels need K %% %d == 0 (K=%lld)", fmt_name(fmt),
                kernel_k_multiple(fmt), (long long)K);
  {
    // the kernels address X and the packed weight with 32-bit buffer offsets
    const int64_t wbytes = fmt == WQ_BF16 ? 2 * N * K : (fmt == WQ_FP8 ? N * K : N * K / 2);
    const int64_t xbytes = kfmt == wq::KF_FP8S ? M * K : 2 * M * K;
    if (wbytes >= kMaxBufferBytes || xbytes >= kMaxBufferBytes)
      return fail(WQ_EUNSUPPORTED, "weight or activation buffer of 2^31 bytes or more");
    // tile overhang past the last row/column must not wrap a 32-bit offset
    if (K >= ((int64_t)1 << 22)) return fail(WQ_EUNSUPPORTED, "K of 2^22 or more");
  }
  if (!X || !W || !Y) return fail(WQ_EINVAL, "null X, weight or Y");
  if (fmt != WQ_BF16 && !scales) return fail(WQ_EINVAL, "null scales");
  if (kfmt == wq::KF_NVFP4 && !gscale) return fail(WQ_EINVAL, "NVFP4 needs global_scale");
  if (kfmt != wq::KF_NVFP4 && gscale) return fail(WQ_EINVAL, "global_scale must be NULL for %s", fmt_name(fmt));
  if (kfmt == wq::KF_FP8S && !act_scale) return fail(WQ_EINVAL, "null act_scale");
  if (!aligned16(X) || !aligned16(W) || !aligned16(Y)) return fail(WQ_EALIGN, "X, weight and Y must be 16-byte aligned");
  *p = wq::plan_linear(kfmt, M, N, K, layout);
  if (p->ws_bytes > 0) {
    if (!ws || ws_bytes < p->ws_bytes)
      return fail(WQ_EWORKSPACE, "workspace of %zu bytes required (got %zu)", p->ws_bytes, ws ? ws_bytes : (size_t)0);
    if (!aligned16(ws)) return fail(WQ_EALIGN, "workspace must be 16-byte aligned");
  }
  *a = wq::LinearArgs{};
  a->X = X;
  a->W = W;
  a->scales = scales;
  a->gscale = gscale;
  a->act_scale = act_scale;
  a->bias = (const uint16_t*)bias;
  a->Y = (uint16_t*)Y;
  a->part = p->ws_bytes ? (float*)ws : nullptr;
  a->M = (int)M;
  a->N = (int)N;
  a->K = (int)K;
  a->wl = layout;
  return WQ_OK;
}

static wq_status linear_common(int kfmt, int fmt, const void* X, int64_t M, int64_t K, const void* W,
                               int32_t layout, const void* scales, const float* gscale, const float* act_scale,
                               const void* bias, int64_t N, void* Y, void* ws, size_t ws_bytes, void* stream) {
  wq::LinearArgs a;
  wq::LinearPlan p;
  bool empty;
  wq_status st = linear_check(kfmt, fmt, X, M, K, W, layout, scales, gscale, act_scale, bias, N, Y, ws, ws_bytes, &a,
                              &p, &empty);
  if (st != WQ_OK || empty) return st;
  return hip_status(wq::launch_linear(kfmt, a, p, (hipStream_t)stream), "wq_linear launch");
}

wq_status wq_linear(int fmt, const void* X, int64_t M, int64_t K, const void* packed, int32_t layout,
                    const void* scales, const float* global_scale, const void* bias, int64_t N, void* Y,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return linear_common(kfmt_of(fmt), fmt, X, M, K, packed, layout, scales, global_scale, nullptr, bias, N, Y,
                       workspace, workspace_bytes, stream);
}

// Two-kernel form: [dense GEMM split-K partials][bf16 W, N*K*2]
static size_t dq_gemm_w_offset(int64_t M, int64_t N, int64_t K) {
  return align256(wq::plan_linear(wq::KF_BF16, M, N, K).ws_bytes);
}

size_t wq_linear_dq_gemm_workspace(int fmt, int64_t M, int64_t N, int64_t K) {
  if (!valid_fmt(fmt) || fmt == WQ_BF16 || M <= 0 || N <= 0 || K <= 0) return 0;
  return dq_gemm_w_offset(M, N, K) + align256((size_t)N * (size_t)K * 2);
}

wq_status wq_linear_dq_gemm(int fmt, const void* X, int64_t M, int64_t K, const void* packed, int32_t layout,
                            const void* scales, const float* global_scale, const void* bias, int64_t N, void* Y,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_fmt(fmt) || fmt == WQ_BF16) return fail(WQ_EINVAL, "wq_linear_dq_gemm: unsupported format %d", fmt);
  // the quantized weight's own checks (shape rule, layout, pointers), as the fused call makes them
  wq::LinearArgs qa;
  wq::LinearPlan qp;
  bool empty;
  wq_status st = linear_check(kfmt_of(fmt), fmt, X, M, K, packed, layout, scales, global_scale, nullptr, bias, N, Y,
                              nullptr, 0, &qa, &qp, &empty);
  if (st == WQ_EWORKSPACE) st = WQ_OK;  // the fused kernel's split-K needs do not apply here
  if (st != WQ_OK || empty) return st;
  const size_t need = wq_linear_dq_gemm_workspace(fmt, M, N, K);
  if (!workspace || workspace_bytes < need)
    return fail(WQ_EWORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(WQ_EALIGN, "workspace must be 16-byte aligned");
  if (2 * N * K >= kMaxBufferBytes) return fail(WQ_EUNSUPPORTED, "bf16 weight of 2^31 bytes or more");
  // the dense GEMM on the dequantized weight, checked before anything is enqueued
  void* wd = (char*)workspace + dq_gemm_w_offset(M, N, K);
  wq::LinearArgs a;
  wq::LinearPlan p;
  st = linear_check(wq::KF_BF16, WQ_BF16, X, M, K, wd, WQ_LAYOUT_ROWS, nullptr, nullptr, nullptr, bias, N, Y,
                    workspace, workspace_bytes, &a, &p, &empty);
  if (st != WQ_OK || empty) return st;
  st = hip_status(wq::launch_dequantize(kfmt_of(fmt), layout, packed, scales, global_scale, N, K, (uint16_t*)wd,
                                        (hipStream_t)stream),
                  "wq_linear_dq_gemm dequantize launch");
  if (st != WQ_OK) return st;
  return hip_status(wq::launch_linear(wq::KF_BF16, a, p, (hipStream_t)stream), "wq_linear_dq_gemm GEMM launch");
}

wq_status wq_absmax(const void* X, int64_t numel, float* amax, void* stream) {
  if (numel < 0) return fail(WQ_EINVAL, "negative numel");
  if (numel == 0) return ok();
  if (!X || !amax) return fail(WQ_EINVAL, "wq_absmax: null pointer");
  return hip_status(wq::launch_absmax((const uint16_t*)X, numel, amax, (hipStream_t)stream), "wq_absmax launch");
}

wq_status wq_fp8_scale(const float* amax, float* scale, int64_t count, void* stream) {
  if (count < 0) return fail(WQ_EINVAL, "negative count");
  if (count == 0) return ok();
  if (!amax || !scale) return fail(WQ_EINVAL, "wq_fp8_scale: null pointer");
  return hip_status(wq::launch_fp8_scale(amax, scale, count, (hipStream_t)stream), "wq_fp8_scale launch");
}

wq_status wq_fp8_quantize_act(const void* X, int64_t M, int64_t K, const float* act_scale, void* Xq,
                              void* stream) {
  if (M < 0 || K < 0) return fail(WQ_EINVAL, "negative size");
  if (M > kMaxDim || K > kMaxDim) return fail(WQ_EUNSUPPORTED, "dimension above 2^30");
  if (M == 0 || K == 0) return ok();
  if (M * K >= ((int64_t)1 << 43)) return fail(WQ_EUNSUPPORTED, "wq_fp8_quantize_act: 2^43 elements or more");
  if (!X || !Xq || !act_scale) return fail(WQ_EINVAL, "wq_fp8_quantize_act: null pointer");
  if (!aligned16(X) || !aligned16(Xq)) return fail(WQ_EALIGN, "X and Xq must be 16-byte aligned");
  return hip_status(wq::launch_quantize_act((const uint16_t*)X, M * K, act_scale, (uint8_t*)Xq,
                                            (hipStream_t)stream),
                    "wq_fp8_quantize_act launch");
}

// Static-FP8 workspace: [split-K partials][quantized X].
static size_t static_xq_offset(int64_t M, int64_t N, int64_t K) {
  return align256(wq::plan_linear(wq::KF_FP8S, M, N, K).part_bytes);
}

size_t wq_fp8_static_workspace(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return static_xq_offset(M, N, K) + align256((size_t)M * (size_t)K);
}

wq_status wq_fp8_static_linear(const void* X, int64_t M, int64_t K, const float* act_scale, const void* Wq,
                               int32_t layout, const float* w_scale, const void* bias, int64_t N, void* Y,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0 || K < 0) return fail(WQ_EINVAL, "negative size");
  if (M == 0 || N == 0) return ok();
  if (K > 0 && K % 16) return fail(WQ_EUNSUPPORTED, "static FP8 linear needs K %% 16 == 0 (K=%lld)", (long long)K);
  const size_t need = wq_fp8_static_workspace(M, N, K);
  if (!workspace || workspace_bytes < need)
    return fail(WQ_EWORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(WQ_EALIGN, "workspace must be 16-byte aligned");
  if (K == 0) return fail(WQ_EUNSUPPORTED, "K == 0");
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(WQ_EUNSUPPORTED, "dimension above 2^30");
  if (!X || !act_scale || !Wq || !w_scale || !Y) return fail(WQ_EINVAL, "wq_fp8_static_linear: null pointer");
  if (!aligned16(X) || !aligned16(Wq) || !aligned16(Y))
    return fail(WQ_EALIGN, "X, Wq and Y must be 16-byte aligned");
  if (M * K >= ((int64_t)1 << 43)) return fail(WQ_EUNSUPPORTED, "wq_fp8_static_linear: 2^43 activations or more");
  // both launches are validated before the first is enqueued
  void* xq = (char*)workspace + static_xq_offset(M, N, K);
  wq::LinearArgs a;
  wq::LinearPlan p;
  bool empty;
  wq_status st = linear_check(wq::KF_FP8S, WQ_FP8, xq, M, K, Wq, layout, w_scale, nullptr, act_scale, bias, N, Y,
                              workspace, workspace_bytes, &a, &p, &empty);
  if (st != WQ_OK) return st;
  st = hip_status(wq::launch_quantize_act((const uint16_t*)X, M * K, act_scale, (uint8_t*)xq, (hipStream_t)stream),
                  "wq_fp8_quantize_act launch");
  if (st != WQ_OK) return st;
  return hip_status(wq::launch_linear(wq::KF_FP8S, a, p, (hipStream_t)stream), "wq_linear launch");
}

wq_status wq_fp8_static_linear_noalloc(const void* X, int64_t M, int64_t K, const float* act_scale, const void* Wq,
                                       int32_t layout, const float* w_scale, const void* bias, int64_t N, void* Y,
                                       void* stream) {
  if (M < 0 || N < 0 || K < 0) return fail(WQ_EINVAL, "negative size");
  if (M == 0 || N == 0) return ok();
  if (K > 0 && K % 16) return fail(WQ_EUNSUPPORTED, "static FP8 linear needs K %% 16 == 0 (K=%lld)", (long long)K);
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(WQ_EUNSUPPORTED, "dimension above 2^30");
  const size_t need = wq_fp8_static_workspace(M, N, K);
  if (need > wq::kNoAllocScratchBytes)
    return fail(WQ_EUNSUPPORTED, "wq_fp8_static_linear_noalloc: needs %zu scratch bytes, the limit is %zu", need,
                wq::kNoAllocScratchBytes);
  void* scratch = nullptr;
  wq_status st = hip_status(wq::noalloc_scratch(&scratch), "wq_fp8_static_linear_noalloc scratch");
  if (st != WQ_OK) return st;
  return wq_fp8_static_linear(X, M, K, act_scale, Wq, layout, w_scale, bias, N, Y, scratch,
                              wq::kNoAllocScratchBytes, stream);
}

size_t wq_fp8_linear_workspace(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return wq::plan_linear(wq::KF_FP8S, M, N, K).ws_bytes;
}

wq_status wq_fp8_linear(const void* Xq, int64_t M, int64_t K, const float* act_scale, const void* Wq, int32_t layout,
                        const float* w_scale, const void* bias, int64_t N, void* Y, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0 || K < 0) return fail(WQ_EINVAL, "negative size");
  if (M == 0 || N == 0) return ok();
  if (K > 0 && K % 16) return fail(WQ_EUNSUPPORTED, "FP8 linear needs K %% 16 == 0 (K=%lld)", (long long)K);
  if (!Xq || !act_scale || !Wq || !w_scale || !Y) return fail(WQ_EINVAL, "wq_fp8_linear: null pointer");
  return linear_common(wq::KF_FP8S, WQ_FP8, Xq, M, K, Wq, layout, w_scale, nullptr, act_scale, bias, N, Y, workspace,
                       workspace_bytes, stream);
}

wq_status wq_mx_quantize_act(const void* X, int64_t M, int64_t K, void* Xq, void* Xs, void* stream) {
  if (M < 0 || K < 0) return fail(WQ_EINVAL, "negative size");
  if (K % 32) return fail(WQ_ESHAPE, "MX activation blocks need K %% 32 == 0 (K=%lld)", (long long)K);
  if (M > kMaxDim || K > kMaxDim) return fail(WQ_EUNSUPPORTED, "dimension above 2^30");
  if (M == 0 || K == 0) return ok();
  if (2 * M * K >= kMaxBufferBytes) return fail(WQ_EUNSUPPORTED, "activation buffer of 2^31 bytes or more");
  if (!X || !Xq || !Xs) return fail(WQ_EINVAL, "wq_mx_quantize_act: null pointer");
  if (!aligned16(X) || !aligned16(Xq)) return fail(WQ_EALIGN, "X and Xq must be 16-byte aligned");
  return hip_status(wq::launch_mx_quantize_act((const uint16_t*)X, M, K, (uint8_t*)Xq, (uint8_t*)Xs,
                                               (hipStream_t)stream),
                    "wq_mx_quantize_act launch");
}

wq_status wq_mx_linear(const void* Xq, const void* Xs, int64_t M, int64_t K, const void* Wq, int32_t layout,
                       const void* Ws, const void* bias, int64_t N, void* Y, void* stream) {
  if (M < 0 || N < 0 || K < 0) return fail(WQ_EINVAL, "negative size");
  wq_status st = check_shape_rule(WQ_MXFP4, N, K);
  if (st != WQ_OK) return st;
  st = check_layout(WQ_MXFP4, layout, N, K);
  if (st != WQ_OK) return st;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(WQ_EUNSUPPORTED, "dimension above 2^30");
  if (M == 0 || N == 0) return ok();
  if (K == 0) return fail(WQ_EUNSUPPORTED, "K == 0");
  if (N * K / 2 >= kMaxBufferBytes || M * K / 2 >= kMaxBufferBytes)
    return fail(WQ_EUNSUPPORTED, "weight or activation buffer of 2^31 bytes or more");
  if (K >= ((int64_t)1 << 22)) return fail(WQ_EUNSUPPORTED, "K of 2^22 or more");
  if (!Xq || !Xs || !Wq || !Ws || !Y) return fail(WQ_EINVAL, "wq_mx_linear: null pointer");
  if (!aligned16(Xq) || !aligned16(Wq) || !aligned16(Y)) return fail(WQ_EALIGN, "Xq, Wq and Y must be 16-byte aligned");
  wq::LinearArgs a{};
  a.X = Xq;
  a.xscales = (const uint8_t*)Xs;
  a.W = Wq;
  a.scales = Ws;
  a.bias = (const uint16_t*)bias;
  a.Y = (uint16_t*)Y;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.wl = layout;
  return hip_status(wq::launch_mx_linear(a, (hipStream_t)stream), "wq_mx_linear launch");
}

size_t wq_mxfp4_dynamic_workspace(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  return align256((size_t)M * (size_t)K / 2) + align256((size_t)M * (size_t)(K / 32));
}

wq_status wq_mxfp4_dynamic_linear(const void* X, int64_t M, int64_t K, const void* Wq, int32_t layout, const void* Ws,
                                  const void* bias, int64_t N, void* Y, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (M < 0 || N < 0 || K < 0) return fail(WQ_EINVAL, "negative size");
  wq_status st = check_shape_rule(WQ_MXFP4, N, K);
  if (st != WQ_OK) return st;
  st = check_layout(WQ_MXFP4, layout, N, K);
  if (st != WQ_OK) return st;
  if (M == 0 || N == 0) return ok();
  const size_t need = wq_mxfp4_dynamic_workspace(M, K);
  if (!workspace || workspace_bytes < need)
    return fail(WQ_EWORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(WQ_EALIGN, "workspace must be 16-byte aligned");
  if (!X || !Wq || !Ws || !Y) return fail(WQ_EINVAL, "wq_mxfp4_dynamic_linear: null pointer");
  // validate the GEMM before anything is enqueued
  void* xq = workspace;
  void* xs = (char*)workspace + align256((size_t)M * (size_t)K / 2);
  if (K == 0) return fail(WQ_EUNSUPPORTED, "K == 0");
  if (!aligned16(X) || !aligned16(Wq) || !aligned16(Y)) return fail(WQ_EALIGN, "X, Wq and Y must be 16-byte aligned");
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(WQ_EUNSUPPORTED, "dimension above 2^30");
  if (N * K / 2 >= kMaxBufferBytes || 2 * M * K >= kMaxBufferBytes || K >= ((int64_t)1 << 22))
    return fail(WQ_EUNSUPPORTED, "buffer of 2^31 bytes or more, or K of 2^22 or more");
  st = wq_mx_quantize_act(X, M, K, xq, xs, stream);
  if (st != WQ_OK) return st;
  return wq_mx_linear(xq, xs, M, K, Wq, layout, Ws, bias, N, Y, stream);
}

wq_status wq_fp8_static_mlp2(const void* X, int64_t M, int64_t K1, const float* act_scale1, const void* W1q,
                             const float* w1_scale, const void* b1, int64_t N1, const float* act_scale2,
                             const void* W2q, const float* w2_scale, const void* b2, int64_t N2, void* Y,
                             void* stream) {
  if (M < 0 || K1 < 0 || N1 < 0 || N2 < 0) return fail(WQ_EINVAL, "negative size");
  if (M == 0 || N2 == 0) return ok();
  if (K1 == 0 || N1 == 0) return fail(WQ_EUNSUPPORTED, "K1 == 0 or N1 == 0");
  if (K1 % 16 || N1 % 16)
    return fail(WQ_EUNSUPPORTED, "fused MLP needs K1 %% 16 == 0 and N1 %% 16 == 0 (K1=%lld N1=%lld)", (long long)K1,
                (long long)N1);
  if (M > kMaxDim || K1 > kMaxDim || N1 > kMaxDim || N2 > kMaxDim) return fail(WQ_EUNSUPPORTED, "dimension above 2^30");
  if (wq::mlp2_smem_bytes(K1, N1, N2) > (size_t)160 * 1024)
    return fail(WQ_EUNSUPPORTED, "fused MLP: 16 rows of K1 + N1 codes exceed the LDS of a CU");
  if (N1 * K1 >= kMaxBufferBytes || N2 * N1 >= kMaxBufferBytes || M * K1 * 2 >= kMaxBufferBytes)
    return fail(WQ_EUNSUPPORTED, "weight or activation buffer of 2^31 bytes or more");
  if (!X || !act_scale1 || !W1q || !w1_scale || !act_scale2 || !W2q || !w2_scale || !Y)
    return fail(WQ_EINVAL, "wq_fp8_static_mlp2: null pointer");
  if (!aligned16(X) || !aligned16(W1q) || !aligned16(W2q) || !aligned16(Y))
    return fail(WQ_EALIGN, "X, W1q, W2q and Y must be 16-byte aligned");
  wq::Mlp2Args a{};
  a.X = (const uint16_t*)X;
  a.act_scale1 = act_scale1;
  a.W1 = (const uint8_t*)W1q;
  a.w1_scale = w1_scale;
  a.b1 = (const uint16_t*)b1;
  a.act_scale2 = act_scale2;
  a.W2 = (const uint8_t*)W2q;
  a.w2_scale = w2_scale;
  a.b2 = (const uint16_t*)b2;
  a.Y = (uint16_t*)Y;
  a.M = (int)M;
  a.K1 = (int)K1;
  a.N1 = (int)N1;
  a.N2 = (int)N2;
  return hip_status(wq::launch_static_mlp2(a, (hipStream_t)stream), "wq_fp8_static_mlp2 launch");
}

size_t wq_read_stream_words(size_t bytes) { return (bytes + 16383) / 16384; }

wq_status wq_read_stream(const void* p, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return ok();
  if (!p || !sink) return fail(WQ_EINVAL, "wq_read_stream: null pointer");
  if (!aligned16(p)) return fail(WQ_EALIGN, "wq_read_stream: p must be 16-byte aligned");
  if (bytes % 16) return fail(WQ_EUNSUPPORTED, "wq_read_stream: bytes %% 16 != 0");
  if (bytes >= (size_t)kMaxBufferBytes) return fail(WQ_EUNSUPPORTED, "wq_read_stream: 2^31 bytes or more");
  return hip_status(wq::launch_read_stream(p, bytes, sink, (hipStream_t)stream), "wq_read_stream launch");
}

}  // extern "C"
