/*
 * wq.h -- C ABI of the MI355X (gfx950) weight-only low-bit quantized Linear
 * and the static-FP8 Linear.
 *
 * What the library computes (the Torch-TensorRT "TorchAO ... (Linear)"
 * tutorial pages are the source of the method; each entry point cites its page
 * and section):
 *   - weight quantizers for four packed formats and their nibble packing,
 *   - y = x . deq(W)^T + b with the dequantization fused ahead of a bf16 matrix
 *     multiply (the "DQ prologue into GEMM" of every weight-only page),
 *   - the static-FP8 path: absmax calibration, per-tensor activation
 *     quantization to E4M3 and an FP8 x FP8 GEMM.
 *
 * Conventions for every entry point
 *   - Shapes follow nn.Linear(in_features=K, out_features=N): weights W[N][K]
 *     (rows contiguous along K), activations X[M][K], outputs Y[M][N]; all
 *     row-major and contiguous.  bf16 is stored as uint16 bit patterns.
 *   - Every pointer is a DEVICE pointer, allocated and owned by the caller.  The
 *     library never allocates or frees device memory and keeps no pointer after
 *     a call returns.  Scales, including the NVFP4 global scale and static-FP8
 *     activation scales, stay on the device (no host synchronisation).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it; calls return without waiting for the GPU.
 *   - The return value reports host-side validation and the launch itself
 *     (hipGetLastError), not kernel completion.  Nothing is enqueued when a
 *     check fails.  wq_last_error() gives a readable reason for the last
 *     non-OK status on the calling thread.  No call throws or aborts.
 *   - M == 0 or N == 0 is a valid empty call (nothing is launched).
 *   - Base pointers of X, W/codes/packed and Y must be 16-byte aligned.
 *
 * Formats (scale layouts are row-major):
 *   WQ_BF16  dense bf16 weight W[N][K] (the unquantized Linear; no scales)
 *   WQ_INT4  symmetric group-wise INT4, group 128 along K, zero-point 0;
 *            codes int8 [N][K] (-8..7), packed uint8 [N][K/2],
 *            scales bf16 [N][K/128]
 *   WQ_FP8   E4M3 (OCP, max 448) codes uint8 [N][K], one fp32 scale per
 *            output row: scales float [N]
 *   WQ_NVFP4 E2M1 codes (one per byte) [N][K], packed [N][K/2],
 *            E4M3 block scales uint8 [N][K/16], one fp32 global scale
 *   WQ_MXFP4 E2M1 codes [N][K], packed [N][K/2], E8M0 block scales
 *            uint8 [N][K/32]
 *   WQ_INT4_ASYM asymmetric group-wise INT4 ("TorchAO INT4 Weight-Only
 *            Quantization (Linear)", intro: TorchAO's default scheme, with a
 *            nonzero zero-point), group 128 along K: codes uint8 [N][K]
 *            (0..15), packed [N][K/2]; per group one uint32 word: bf16 scale
 *            in bits 0-15, zero-point in bits 16-19 -> scales uint32
 *            [N][K/128].  s = bf16((hi - lo) / 15) with lo = min(min w, 0),
 *            hi = max(max w, 0); z = clamp(rint(-lo / s), 0, 15); code =
 *            clamp(rint(w / s) + z, 0, 15); value (code - z) * s.
 * Packing: byte j of a packed row holds element 2j in its low nibble and
 * element 2j+1 in its high nibble.
 *
 * Weight layouts (the `layout` argument of the calls that read a packed weight):
 *   WQ_LAYOUT_ROWS  (0) canonical: packed row n at n * row_bytes (row_bytes =
 *                   K/2 for 4-bit formats, K for FP8), scales row-major as
 *                   listed above.  These are the bytes wq_pack writes.
 *   WQ_LAYOUT_TILES (1) kernel tile order ("TorchAO INT4 Weight-Only
 *                   Quantization (Linear)", "Export and compile": the packed
 *                   constant is re-laid-out once for the engine): the packed
 *                   weight is cut into tiles of 16 rows x 64 bytes (128 K of a
 *                   4-bit format, 64 K of E4M3); tile (n / 16, b / 64) starts
 *                   at ((n / 16) * (row_bytes / 64) + b / 64) * 1024 and holds
 *                   its 16 rows' 64 bytes one after the other, so byte b of row
 *                   n is at that start + 64 * (n % 16) + b % 64.  Block scales
 *                   follow the same tiles: for tile (n / 16, j), the 16 rows'
 *                   scale bytes of K range [128 j, 128 j + 128) one after the
 *                   other -- INT4 2, INT4_ASYM 4, NVFP4 8, MXFP4 4 bytes per row
 *                   -- starting at ((n / 16) * (K / 128) + j) * 16 * that size.
 *                   FP8 row scales and the NVFP4 global scale are the same in
 *                   both layouts.  Sizes are those of WQ_LAYOUT_ROWS.  Needs
 *                   N % 16 == 0 and K % 128 == 0 (4-bit) or K % 64 == 0 (FP8)
 *                   (WQ_EUNSUPPORTED otherwise); BF16 has only layout 0.  One
 *                   16-byte load per lane of a 64-lane wave then reads a whole
 *                   tile (8 full cache lines) instead of 16 half lines.
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WQ_ABI_VERSION 2

typedef enum wq_format {
  WQ_BF16 = 0,
  WQ_INT4 = 1,
  WQ_FP8 = 2,
  WQ_NVFP4 = 3,
  WQ_MXFP4 = 4,
  WQ_INT4_ASYM = 5
} wq_format;

typedef enum wq_layout_kind { WQ_LAYOUT_ROWS = 0, WQ_LAYOUT_TILES = 1 } wq_layout_kind;

typedef enum wq_status {
  WQ_OK = 0,
  WQ_EINVAL = 1,       /* null pointer, negative size, unknown format        */
  WQ_ESHAPE = 2,       /* a format's divisibility rule is violated           */
  WQ_EALIGN = 3,       /* a base pointer is not 16-byte aligned              */
  WQ_EUNSUPPORTED = 4, /* valid for the format, not supported by the kernels */
  WQ_EWORKSPACE = 5,   /* workspace missing or too small                     */
  WQ_EHIP = 6          /* the HIP runtime reported an error                  */
} wq_status;

/* ABI version of the loaded library (WQ_ABI_VERSION at build time). */
int wq_abi_version(void);

/* Static string naming a status code. */
const char* wq_status_str(int status);

/* Reason for the last non-OK status returned on the calling thread ("" if none). */
const char* wq_last_error(void);

/*
 * Byte sizes of the buffers of format `fmt` for a weight W[N][K]:
 *   codes_bytes  : unpacked codes, one per byte (N*K; BF16: 2*N*K)
 *   packed_bytes : what wq_linear reads (N*K/2 for 4-bit formats, N*K for FP8,
 *                  2*N*K for BF16)
 *   scale_bytes  : block/row scales (0 for BF16)
 *   global_bytes : 4 for NVFP4's global scale, else 0
 * Any output pointer may be NULL.  Returns WQ_ESHAPE if (N, K) break the
 * format's divisibility rule.
 */
wq_status wq_layout(int fmt, int64_t N, int64_t K, size_t* codes_bytes, size_t* packed_bytes,
                    size_t* scale_bytes, size_t* global_bytes);

/*
 * Quantize a bf16 weight W[N][K] to unpacked codes (one per byte) and scales.
 *   INT4  -- "TorchAO INT4 Weight-Only Quantization (Linear)", intro and
 *            "Define a linear model and quantize weights to symmetric INT4":
 *            symmetric, zero-point 0, group 128.  s = bf16(max|w_group| / 7),
 *            code = clamp(round(w / s), -8, 7) (the division uses the bf16
 *            scale); an all-zero group has s = 0 and codes 0.  K % 128 == 0.
 *   FP8   -- "TorchAO FP8 Weight-Only Quantization (Linear)", intro: per-row
 *            s = max|w_row| / 448, code = E4M3(clamp(w / s, +-448)).
 *   NVFP4 -- "TorchAO NVFP4 Weight-Only Quantization (Linear)", intro: with
 *            A = max|W|, g = A / 2688; per 16-element block t = (amax/6)/g,
 *            scale = E4M3(clamp(t, 2^-9, 448)), S = dec(scale) * g,
 *            code = E2M1(clamp(w / S, +-6)).  N % 16 == 0 and K % 16 == 0.
 *            `global_scale` (1 float, device) receives g.
 *   MXFP4 -- "TorchAO MXFP4 Dynamic Activation + MX Weight (Linear)", intro:
 *            per 32-element block e = floor(log2 amax) - 2 clamped to
 *            [-127, 127] (an all-zero block gets -127), scale code e + 127,
 *            code = E2M1(clamp(w / 2^e, +-6)).  N % 32 == 0 and K % 32 == 0.
 * Every step is an IEEE fp32 operation and every cast rounds to nearest-even
 * after clamping, keeping the sign of zero.  `global_scale` must be NULL for
 * formats other than NVFP4.  WQ_BF16 is rejected (WQ_EINVAL).
 */
wq_status wq_quantize(int fmt, const void* W, int64_t N, int64_t K, void* codes, void* scales,
                      float* global_scale, void* stream);

/*
 * Pack unpacked codes into the canonical byte stream (WQ_LAYOUT_ROWS)
 * ("TorchAO INT4 Weight-Only Quantization (Linear)", "Export and compile":
 * one-code-per-byte int8 data re-packed into a 4-bit constant).  4-bit formats:
 * two codes per byte, low nibble = even element; FP8: a plain copy.
 * Packing is done once; there is no in-place update of a packed weight.
 */
wq_status wq_pack(int fmt, const void* codes, int64_t N, int64_t K, void* packed, void* stream);

/*
 * Convert a packed weight and its block scales from layout `src_layout` to
 * `dst_layout` (see "Weight layouts" above; the same page and section as
 * wq_pack: the one-time re-layout of the packed constant).  src and dst are
 * distinct buffers of the sizes wq_layout reports.  FP8 row scales are copied
 * unchanged; the NVFP4 global scale is not touched (it is the same in both
 * layouts).  Converting back reproduces the source bytes exactly.  Both
 * layouts' constraints apply (WQ_EUNSUPPORTED); BF16 is rejected (WQ_EINVAL).
 */
wq_status wq_repack(int fmt, int64_t N, int64_t K, int32_t src_layout, const void* src_packed, const void* src_scales,
                    int32_t dst_layout, void* dst_packed, void* dst_scales, void* stream);

/*
 * Dequantize packed weights (in `layout`) to bf16 W_out[N][K], row-major (the
 * DQ of the two-kernel form, "TorchAO FP8 Weight-Only Quantization (Linear)",
 * intro).  Each element is bf16(fp32 product) of the code's value and its
 * scale(s), evaluated in the order code * block-scale * global-scale.
 */
wq_status wq_dequantize(int fmt, const void* packed, int32_t layout, const void* scales, const float* global_scale,
                        int64_t N, int64_t K, void* W_out, void* stream);

/*
 * Workspace bytes wq_linear needs for (M, N, K); 0 means none.  It holds
 * fp32 split-K partial sums when the launch plan splits K across workgroups
 * (small problems); no initialisation is needed.  Calls that may run
 * concurrently (different streams) need different workspaces.
 */
size_t wq_linear_workspace(int fmt, int64_t M, int64_t N, int64_t K);

/*
 * Y[M][N] = bf16( X[M][K] . deq(W)^T (+ bias[N]) ), fp32 accumulation, bias
 * added in fp32, one round-to-nearest-even to bf16.  The weight stays packed
 * in device memory and is dequantized in registers ahead of the bf16 matrix
 * cores (every weight-only page's intro: a DQ prologue into a high-precision
 * GEMM; activations stay bf16).
 *   packed       : packed codes (BF16: the dense weight)
 *   layout       : layout of `packed` and `scales` (WQ_LAYOUT_ROWS as wq_pack
 *                  writes them, or WQ_LAYOUT_TILES after wq_repack)
 *   scales       : the format's scales (NULL for BF16)
 *   global_scale : NVFP4's device float, else NULL
 *   bias         : bf16 [N] or NULL
 * Kernel constraints: K % 32 == 0 for 4-bit formats, K % 16 for FP8, K % 8
 * for BF16 (WQ_EUNSUPPORTED otherwise).
 * Numerics by M: up to 128 rows (the small-M kernels) INT4 groups are summed
 * exactly as s * (sum_k x_k (code_k + 136) - 136 sum_k x_k) in fp32 (the
 * INT4_ASYM bias is 128 + zero-point), i.e. the scale multiplies the group's
 * fp32 partial sum; above that (the mid-M and LDS-tiled kernels) each INT4 weight is
 * first rounded to bf16(code * s) -- the wq_dequantize value -- and then
 * multiplied.  The other formats' decoded weights are exact in bf16 at every
 * M, so only the accumulation order differs.
 */
wq_status wq_linear(int fmt, const void* X, int64_t M, int64_t K, const void* packed, int32_t layout,
                    const void* scales, const float* global_scale, const void* bias, int64_t N, void* Y,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two-kernel form of the same Linear ("TorchAO FP8 Weight-Only
 * Quantization (Linear)", intro: where the DQ is not fused into the GEMM, DQ
 * and GEMM run as two kernels): wq_dequantize writes the bf16 weight into the
 * workspace, then the dense bf16 GEMM computes
 * Y = bf16(X . W_bf16^T (+ bias)) with fp32 accumulation.  The weight is
 * rounded to bf16 before the product (the wq_dequantize value), so results
 * differ from wq_linear's by that rounding: FP8 row scales and the NVFP4
 * global scale, which wq_linear applies exactly in its epilogue, and INT4
 * group scales enter through bf16(code * scale).  Same arguments as
 * wq_linear; the workspace holds the N*K bf16 weight (and the dense GEMM's
 * split-K partials): wq_linear_dq_gemm_workspace bytes.  Both launches are
 * checked before the first is enqueued.
 */
size_t wq_linear_dq_gemm_workspace(int fmt, int64_t M, int64_t N, int64_t K);
wq_status wq_linear_dq_gemm(int fmt, const void* X, int64_t M, int64_t K, const void* packed, int32_t layout,
                            const void* scales, const float* global_scale, const void* bias, int64_t N, void* Y,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Calibration observer ("TorchAO Static FP8 Quantization (Linear)", "Calibrate,
 * then insert static FP8 Q/DQ": per-tensor activation min/max over the
 * calibration forwards, read symmetrically): amax = max(amax, max|X|) over
 * `numel` bf16 values.  `amax` (1 float, device) must start at 0 before the
 * first batch.
 */
wq_status wq_absmax(const void* X, int64_t numel, float* amax, void* stream);

/* scale[i] = fp32(amax[i] / 448) for i < count (device arrays). */
wq_status wq_fp8_scale(const float* amax, float* scale, int64_t count, void* stream);

/*
 * Static activation Q ("TorchAO Static FP8 Quantization (Linear)", intro and
 * "Graph after export" figure: bf16 activation -> Q -> FP8):
 * Xq = E4M3(clamp(fp32(x / act_scale), +-448)), nearest-even; act_scale is one
 * device float (0 keeps x).  X bf16 [M][K] -> Xq uint8 [M][K]; M * K < 2^43
 * (else WQ_EUNSUPPORTED).
 */
wq_status wq_fp8_quantize_act(const void* X, int64_t M, int64_t K, const float* act_scale, void* Xq,
                              void* stream);

/*
 * Static-FP8 Linear (same page, intro: after Q/DQ fusion the GEMM itself runs
 * in FP8): quantizes X with wq_fp8_quantize_act's rule, multiplies E4M3 x E4M3
 * on the FP8 matrix cores with fp32 accumulation, then
 * Y = bf16(acc * act_scale * w_scale[n] (+ bias[n])).
 * Wq: E4M3 codes [N][K] (wq_quantize(WQ_FP8) output) in `layout`, w_scale:
 * float [N].  K % 16 == 0.  Workspace: wq_linear_workspace(WQ_FP8, M, N, K)
 * plus M*K bytes for the quantized activations -- query
 * wq_fp8_static_workspace.  Every check of both launches runs before the
 * first is enqueued.
 */
size_t wq_fp8_static_workspace(int64_t M, int64_t N, int64_t K);
wq_status wq_fp8_static_linear(const void* X, int64_t M, int64_t K, const float* act_scale, const void* Wq,
                               int32_t layout, const float* w_scale, const void* bias, int64_t N, void* Y,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * wq_fp8_static_linear without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The quantized activations and split-K partials go
 * to a scratch array of 16 MiB that the library holds on each GPU it runs on
 * until the process ends: wq_fp8_static_workspace(M, N, K) must not exceed
 * 16 MiB (M * K up to about 16 Mi elements; WQ_EUNSUPPORTED otherwise).  The
 * call allocates nothing.  Every call on a GPU shares that GPU's scratch, so
 * calls that overlap on one GPU (different streams, or threads without
 * ordering) race and must be serialized by the caller.  The scratch needs no
 * initialisation.  Same arguments and results as wq_fp8_static_linear.
 */
wq_status wq_fp8_static_linear_noalloc(const void* X, int64_t M, int64_t K, const float* act_scale, const void* Wq,
                                       int32_t layout, const float* w_scale, const void* bias, int64_t N, void* Y,
                                       void* stream);

/*
 * The FP8 x FP8 GEMM of the static path on activations that are already
 * quantized (same page, "Graph after export": the Q node's E4M3 output and the
 * E4M3 weight each pass a DQ into the linear; intro: that pair runs as one FP8
 * GEMM): Y = bf16(sum_k dec(Xq[m][k]) dec(Wq[n][k]) * act_scale * w_scale[n]
 * (+ bias[n])).  Xq: E4M3 codes uint8 [M][K] (wq_fp8_quantize_act output, or
 * any E4M3 tensor quantized with act_scale).  wq_fp8_static_linear is
 * wq_fp8_quantize_act followed by this call.  K % 16 == 0.  Workspace:
 * wq_fp8_linear_workspace bytes (0 for most shapes).
 */
size_t wq_fp8_linear_workspace(int64_t M, int64_t N, int64_t K);
wq_status wq_fp8_linear(const void* Xq, int64_t M, int64_t K, const float* act_scale, const void* Wq, int32_t layout,
                        const float* w_scale, const void* bias, int64_t N, void* Y, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Fused two-layer static-FP8 MLP ("TorchAO Static FP8 Quantization (Linear)",
 * model and "Calibrate, then insert static FP8 Q/DQ": Linear(K1, N1) ->
 * Linear(N1, N2), each input quantized with its calibrated act_scale and each
 * GEMM run in FP8).  Computes, in one kernel,
 *   H = bf16(Q(X, act_scale1) . deq(W1q)^T * act_scale1 * w1_scale[n] (+ b1))
 *   Y = bf16(Q(H, act_scale2) . deq(W2q)^T * act_scale2 * w2_scale[n] (+ b2))
 * with the same per-step arithmetic as two wq_fp8_static_linear calls (results
 * differ only by fp32 accumulation order); H never leaves the chip.
 * W1q E4M3 [N1][K1], W2q E4M3 [N2][N1] (WQ_LAYOUT_ROWS), scales float [N1] / [N2], biases bf16
 * or NULL.  K1 % 16 == 0, N1 % 16 == 0, M * K1 * 2 < 2^31, and 16 rows of the
 * input and hidden codes plus both layers' column scales and biases must fit
 * in the 160 KiB LDS of a CU (K1 + N1 up to about 9.5K; else WQ_EUNSUPPORTED --
 * use two wq_fp8_static_linear calls).  No workspace.
 */
wq_status wq_fp8_static_mlp2(const void* X, int64_t M, int64_t K1, const float* act_scale1, const void* W1q,
                             const float* w1_scale, const void* b1, int64_t N1, const float* act_scale2,
                             const void* W2q, const float* w2_scale, const void* b2, int64_t N2, void* Y,
                             void* stream);

/*
 * MXFP4 dynamic-activation x MXFP4-weight Linear ("TorchAO MXFP4 Dynamic
 * Activation + MX Weight (Linear)", intro: weights MXFP4, activations
 * quantized to MX on every call, the GEMM on native MXFP4 matrix units).
 *
 * wq_mx_quantize_act: X bf16 [M][K] -> Xq packed E2M1 [M][K/2] (element 2j in
 * the low nibble of byte j) and Xs E8M0 [M][K/32], with the MXFP4 weight rule
 * applied to each 32-element block of a row (e = floor(log2 max|x|) - 2,
 * clamped to [-127, 127]; codes E2M1(clamp(x / 2^e, +-6)), nearest even, sign
 * kept).  K % 32 == 0; any M.
 *
 * wq_mx_linear: Y = bf16(sum_k deq(Xq)[m][k] deq(Wq)[n][k] (+ bias[n])) on the
 * E2M1 x E2M1 scaled matrix cores (fp32 accumulation).  Wq/Ws: the packed
 * weight and E8M0 scales of wq_quantize + wq_pack for WQ_MXFP4, in `layout`
 * (the activations Xq/Xs are always row-major).  N % 32 == 0, K % 32 == 0.
 * No workspace.  With K % 128 == 0 and 4-byte aligned Xs and Ws the kernels
 * load the block scales as dwords (and from 9 rows with K % 512 == 0 copy the
 * activation rows into LDS); other shapes and alignments take byte loads.  Up
 * to 64 rows both forms give the same bits; above, the kernel (and with it
 * the fp32 summation order) can differ between them.
 *
 * wq_mxfp4_dynamic_linear: wq_mx_quantize_act into the workspace, then
 * wq_mx_linear.  Workspace: wq_mxfp4_dynamic_workspace(M, K) bytes.
 */
wq_status wq_mx_quantize_act(const void* X, int64_t M, int64_t K, void* Xq, void* Xs, void* stream);
wq_status wq_mx_linear(const void* Xq, const void* Xs, int64_t M, int64_t K, const void* Wq, int32_t layout,
                       const void* Ws, const void* bias, int64_t N, void* Y, void* stream);
size_t wq_mxfp4_dynamic_workspace(int64_t M, int64_t K);
wq_status wq_mxfp4_dynamic_linear(const void* X, int64_t M, int64_t K, const void* Wq, int32_t layout, const void* Ws,
                                  const void* bias, int64_t N, void* Y, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Measurement aid (not part of the method): reads `bytes` bytes at `p` with
 * 16-byte vector loads, as the plain read-only stream that a weight stream of
 * the same size is compared against.  sink[b] (device, wq_read_stream_words
 * entries) receives the XOR of the 32-bit words of the b-th 16 KiB block, so
 * every byte read reaches the output.  p 16-byte aligned, bytes % 16 == 0.
 */
size_t wq_read_stream_words(size_t bytes);
wq_status wq_read_stream(const void* p, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
