// Internal launch interface between the C ABI (wq_api.hip) and the kernels.
// Launchers assume their arguments were validated by the ABI layer.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace wq {

// Kernel-side format ids (the ABI's wq_format values plus the FP8-activation
// variant used by the static path).
enum KFmt { KF_BF16 = 0, KF_INT4 = 1, KF_FP8 = 2, KF_NVFP4 = 3, KF_MXFP4 = 4, KF_FP8S = 5, KF_INT4A = 6 };

// Workspace: split-K partial sums (fp32) when a plan splits K across
// workgroups; the static path appends its quantized activations.
constexpr int kMaxSplit = 8;  // K splits across workgroups of one column tile

// Launch plan of the small-M dequant-GEMM (shared by the workspace query and
// the launch so both always agree).
// Tile configurations of the small-M kernel:
//  kCfgSplit   : 64 columns x 4 waves per workgroup, K split across workgroups
//  kCfgNoSplit : 16 columns x 12 waves per workgroup covering all of K
//  kCfgTiled   : LDS-tiled GEMM for larger M (BM x BN tiles, weights decoded
//                once per tile)
//  kCfgMid     : 64 x 64 tiles of 8 waves that split K, weights in registers,
//                activations loaded straight into LDS (wq_gemm_mid.hip)
constexpr int kCfgSplit = 0;
constexpr int kCfgNoSplit = 1;
constexpr int kCfgTiled = 2;
constexpr int kCfgMid = 3;
constexpr int64_t kMidMaxK = 16384;  // K limit of the mid-M kernel (16 K blocks per wave)

// Packed-weight layouts (the ABI's `layout` argument; see wq_kernel_common.hpp)
constexpr int kLayoutRows = 0;   // canonical: row n of the packed weight at n * row_bytes
constexpr int kLayoutTiles = 1;  // tile order: 16 rows x 64 bytes per tile

struct LinearPlan {
  int cfg;        // kCfgSplit, kCfgNoSplit, kCfgTiled or kCfgMid
  int mt;         // 16-row MFMA tiles per workgroup (1 or 2)
  int ntw;        // 16-column tiles per wave (= per workgroup)
  int nwaves;     // waves per workgroup
  int spw;        // K macro-steps per wave whose loads are issued together
  int gx, gz;     // workgroups along N and along M
  int S;          // K splits across workgroups
  int bm, bn;     // output tile of the tiled configuration
  int ks;         // K groups inside a tiled workgroup (1 or 2)
  size_t part_bytes, ws_bytes;  // split-K partials (0 without a split)
};

// `wl` (the weight layout) picks among tile shapes of the same workspace
// needs: the workspace size never depends on it.
LinearPlan plan_linear(int kfmt, int64_t M, int64_t N, int64_t K, int wl = kLayoutRows);


struct LinearArgs {
  const void* X;         // bf16 [M][K], or E4M3 [M][K] for KF_FP8S
  const void* W;         // packed weight
  const void* scales;    // format scales
  const float* gscale;   // NVFP4 global scale (device)
  const float* act_scale;  // static FP8 activation scale (device)
  const uint8_t* xscales;  // E8M0 activation block scales [M][K/32] (MX path)
  const uint16_t* bias;  // bf16 [N] or null
  uint16_t* Y;           // bf16 [M][N]
  float* part;           // split-K partials (workspace)
  int M, N, K;
  int wl;                // layout of W and its block scales (kLayoutRows / kLayoutTiles)
};

hipError_t launch_linear(int kfmt, const LinearArgs& a, const LinearPlan& p, hipStream_t s);

// Scratch of the allocation-free static-FP8 Linear: a device array of this
// size per GPU; noalloc_scratch gives its address on the current device.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_gemm_tiled(int kfmt, const LinearArgs& a, const LinearPlan& p, hipStream_t s);
hipError_t launch_gemm_mid(int kfmt, const LinearArgs& a, hipStream_t s);

hipError_t launch_quantize(int fmt, const uint16_t* W, int64_t N, int64_t K, void* codes, void* scales,
                           float* gscale, hipStream_t s);
hipError_t launch_read_stream(const void* p, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_pack(int fmt, const uint8_t* codes, int64_t N, int64_t K, uint8_t* packed, hipStream_t s);
hipError_t launch_dequantize(int fmt, int wl, const void* packed, const void* scales, const float* gscale, int64_t N,
                             int64_t K, uint16_t* out, hipStream_t s);
// layout conversion of a packed weight and its block scales (src -> dst layout)
hipError_t launch_repack(int fmt, int64_t N, int64_t K, int src_wl, const void* src_packed, const void* src_scales,
                         int dst_wl, void* dst_packed, void* dst_scales, hipStream_t s);
hipError_t launch_absmax(const uint16_t* X, int64_t numel, float* amax, hipStream_t s);
hipError_t launch_fp8_scale(const float* amax, float* scale, int64_t count, hipStream_t s);
hipError_t launch_quantize_act(const uint16_t* X, int64_t numel, const float* act_scale, uint8_t* Xq,
                               hipStream_t s);
// Fused two-layer static-FP8 MLP
struct Mlp2Args {
  const uint16_t* X;                 // bf16 [M][K1]
  const float* act_scale1;           // layer-1 activation scale (device)
  const uint8_t* W1;                 // E4M3 [N1][K1]
  const float* w1_scale;             // [N1]
  const uint16_t* b1;                // bf16 [N1] or null
  const float* act_scale2;           // layer-2 activation scale (device)
  const uint8_t* W2;                 // E4M3 [N2][N1]
  const float* w2_scale;             // [N2]
  const uint16_t* b2;                // bf16 [N2] or null
  uint16_t* Y;                       // bf16 [M][N2]
  int M, K1, N1, N2;
};
size_t mlp2_smem_bytes(int64_t K1, int64_t N1, int64_t N2);
hipError_t launch_static_mlp2(const Mlp2Args& a, hipStream_t s);

// MXFP4 dynamic-activation path
hipError_t launch_mx_quantize_act(const uint16_t* X, int64_t M, int64_t K, uint8_t* Xq, uint8_t* Xs, hipStream_t s);
hipError_t launch_mx_linear(const LinearArgs& a, hipStream_t s);
// static FP8 tiled GEMM on the scaled matrix cores (E4M3 x E4M3, unit scales)
hipError_t launch_f8_gemm_tiled(const LinearArgs& a, hipStream_t s);

}  // namespace wq
