// Shared device helpers of the GEMM kernels: format traits, operand decoders,
// MFMA wrappers, buffer loads and the output epilogue.
#pragma once

#include <atomic>

#include "wq_device.hpp"
#include "wq_internal.hpp"

namespace wq {

template <int F>
struct FmtT;
template <>
struct FmtT<KF_BF16> {
  static constexpr int KPL = 8;  // K elements per 16-byte weight chunk
};
template <>
struct FmtT<KF_INT4> {
  static constexpr int KPL = 32;
};
template <>
struct FmtT<KF_FP8> {
  static constexpr int KPL = 16;
};
template <>
struct FmtT<KF_NVFP4> {
  static constexpr int KPL = 32;
};
template <>
struct FmtT<KF_MXFP4> {
  static constexpr int KPL = 32;
};
template <>
struct FmtT<KF_FP8S> {
  static constexpr int KPL = 16;
};
template <>
struct FmtT<KF_INT4A> {
  static constexpr int KPL = 32;
};

template <int F>
__device__ __forceinline__ int64_t kbyte(int64_t k) {
  if constexpr (F == KF_BF16) return 2 * k;
  else if constexpr (F == KF_FP8 || F == KF_FP8S) return k;
  else return k / 2;
}

// Packed-weight layouts.  kLayoutRows: row n of the packed weight starts at
// n * row_bytes and the block scales are [N][K / block] row-major.
// kLayoutTiles (kernel tile order): the weight is cut into tiles of 16 rows x
// 64 bytes (128 K of a 4-bit format, 64 K of E4M3); tile (n / 16, kb / 64)
// starts at ((n / 16) * (row_bytes / 64) + kb / 64) * 1024 and holds its 16
// rows one after the other, so one 16-byte load per lane of a wave reads a
// whole tile, 1 KiB in 8 full cache lines.  The block scales of each tile
// follow the same order: SB bytes per row and tile (INT4 2, INT4_ASYM 4,
// NVFP4 8, MXFP4 4).  The E4M3 row scales and the NVFP4 global scale do not
// depend on the layout.  Tile order needs N % 16 == 0 and row_bytes % 64 == 0.
template <int WL>
__device__ __forceinline__ uint32_t w_off(uint32_t n, uint32_t kb, uint32_t row_bytes) {
  if constexpr (WL == kLayoutTiles)
    return ((((n >> 4) * (row_bytes >> 6) + (kb >> 6)) << 10) | ((n & 15u) << 6)) + (kb & 63u);
  else
    return n * row_bytes + kb;
}

// Block-scale geometry of the 4-bit formats: K elements per scale, bytes per scale.
template <int F>
struct ScaleT {
  static constexpr uint32_t BLK = (F == KF_NVFP4) ? 16u : ((F == KF_MXFP4) ? 32u : 128u);
  static constexpr uint32_t ES = (F == KF_INT4) ? 2u : ((F == KF_INT4A) ? 4u : 1u);
  static constexpr uint32_t SB = 128u / BLK * ES;  // bytes per row of one 128-K tile
};

// Byte offset of the block scale that covers K element k of row n.
template <int F, int WL>
__device__ __forceinline__ uint32_t s_off(uint32_t n, uint32_t k, uint32_t K) {
  using S = ScaleT<F>;
  if constexpr (WL == kLayoutTiles)
    return (((n >> 4) * (K >> 7) + (k >> 7)) * 16u + (n & 15u)) * S::SB + ((k & 127u) / S::BLK) * S::ES;
  else
    return (n * (K / S::BLK) + k / S::BLK) * S::ES;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// INT4: 8 nibbles (K order 0..7) -> bf16 values 136 + code, K order kept.
__device__ __forceinline__ bf16x8 dec_int4_biased(uint32_t w) {
  const uint32_t u = w ^ 0x88888888u;
  const uint32_t v = u >> 4;
  u32x4 p;
  p.x = (__builtin_amdgcn_perm(v, u, 0x0C040C00u) & 0x000F000Fu) | 0x43004300u;
  p.y = (__builtin_amdgcn_perm(v, u, 0x0C050C01u) & 0x000F000Fu) | 0x43004300u;
  p.z = (__builtin_amdgcn_perm(v, u, 0x0C060C02u) & 0x000F000Fu) | 0x43004300u;
  p.w = (__builtin_amdgcn_perm(v, u, 0x0C070C03u) & 0x000F000Fu) | 0x43004300u;
  return as_bf16x8(p);
}

// Unsigned INT4: 8 nibbles (K order 0..7) -> bf16 values 128 + code.
__device__ __forceinline__ bf16x8 dec_uint4_biased(uint32_t u) {
  const uint32_t v = u >> 4;
  u32x4 p;
  p.x = (__builtin_amdgcn_perm(v, u, 0x0C040C00u) & 0x000F000Fu) | 0x43004300u;
  p.y = (__builtin_amdgcn_perm(v, u, 0x0C050C01u) & 0x000F000Fu) | 0x43004300u;
  p.z = (__builtin_amdgcn_perm(v, u, 0x0C060C02u) & 0x000F000Fu) | 0x43004300u;
  p.w = (__builtin_amdgcn_perm(v, u, 0x0C070C03u) & 0x000F000Fu) | 0x43004300u;
  return as_bf16x8(p);
}

// E2M1 x 8 times an arbitrary fp32 scale d (the product is exact in bf16).
__device__ __forceinline__ bf16x8 dec_fp4_mul(uint32_t w, float d) {
  bf16x8 r;
  f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  r[0] = (__bf16)(f0.x * d);
  r[1] = (__bf16)(f0.y * d);
  r[2] = (__bf16)(f1.x * d);
  r[3] = (__bf16)(f1.y * d);
  r[4] = (__bf16)(f2.x * d);
  r[5] = (__bf16)(f2.y * d);
  r[6] = (__bf16)(f3.x * d);
  r[7] = (__bf16)(f3.y * d);
  return r;
}

// E2M1 x 8 times a power-of-two scale p.
__device__ __forceinline__ bf16x8 dec_fp4_pow2(uint32_t w, float p) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, p, 0);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, p, 1);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, p, 2);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, p, 3);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// E4M3 x 8 (two words) -> bf16, exact.
__device__ __forceinline__ bf16x8 dec_fp8(uint32_t w0, uint32_t w1) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_fp8(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4 c) {
  const long a = (long)(((uint64_t)a1 << 32) | a0);
  const long b = (long)(((uint64_t)b1 << 32) | b0);
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

// Buffer loads: an offset at or beyond the resource size reads as zero, which
// masks the M, N and K tails without branches (a branch per masked load makes
// the compiler wait for every outstanding load at each join).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
// Non-temporal (streaming) 16-byte load, for data read once.
__device__ __forceinline__ u32x4 bload128_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}
__device__ __forceinline__ uint32_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t bload32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

constexpr uint32_t kOOB = 0x80000000u;  // beyond every resource (sizes are < 2^31)

// s_waitcnt immediates (gfx9 encoding): vmcnt(0) with the other counters left
// alone, and lgkmcnt(0) likewise.  Loads into LDS (buffer_load ... lds) count
// in vmcnt, so vmcnt(0) also means this wave's LDS copies have landed.
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;

// `off` when `ok`, else an offset past every resource -- computed with bit
// operations so the compiler cannot split the load into guarded branches
// (each branch join would drain the loads in flight).
__device__ __forceinline__ uint32_t off_if(bool ok, uint32_t off) { return off | ((uint32_t)(!ok) << 31); }

// Output epilogue: y = acc * column scale (+ bias) -> bf16 (nearest even).
// Column scale: FP8 row scale, NVFP4 global scale, static FP8
// act_scale * w_scale[n]; 1 otherwise.  The tensor-wide factor (NVFP4 global,
// static act_scale) is read by uniform_scale() at kernel start so that its
// load travels with the main loads instead of after the reduction.
template <int F>
struct Epilogue {
  float scale1, scale2, bias;
  __device__ __forceinline__ static float uniform_scale(const LinearArgs& a) {
    if constexpr (F == KF_NVFP4) return a.gscale[0];
    else if constexpr (F == KF_FP8S) return a.act_scale[0];
    else return 1.0f;
  }
  __device__ __forceinline__ Epilogue(int en, uint32_t bias_bits, uint32_t cs_bits, float uscale) {
    (void)en;
    bias = bitsf(bias_bits << 16);
    scale2 = 1.0f;
    if constexpr (F == KF_FP8) scale1 = bitsf(cs_bits);
    else if constexpr (F == KF_NVFP4) scale1 = uscale;
    else if constexpr (F == KF_FP8S) {
      scale1 = uscale;
      scale2 = bitsf(cs_bits);
    } else scale1 = 1.0f;
  }
  __device__ __forceinline__ void store(const LinearArgs& a, int m0, int en, int e, int E, int NT, float v) const {
    const int m = m0 + e / NT;
    if (e < E && m < a.M && en < a.N) {
      float y = v * scale1;
      if constexpr (F == KF_FP8S) y = y * scale2;
      a.Y[(int64_t)m * a.N + en] = f32_to_bf16(y + bias);
    }
  }
};

// Output tiles of the tiled GEMMs leave through LDS: a wave writes its ROWS x
// COLS (COLS = 32 or 64) bf16 tile in row-major order (rows padded to
// kTileRowBytes: the four row groups 4g + r of a 16 x 16 result, or the two of
// a 32 x 32 one, land 64 bytes apart in the banks), then stores it as 16-byte
// row pieces, 64 lanes x 16 bytes per store instruction, instead of one
// 2-byte store per element.  Measured on the static FP8 GEMM at
// M = N = 4096, K = 3072: 49.8 -> 47.2 us.
constexpr int kTileRowBytes = 64 * 2 + 16;

__device__ __forceinline__ void tile_put(unsigned char* et, int row, int col, float y) {
  *reinterpret_cast<uint16_t*>(et + row * kTileRowBytes + col * 2) = f32_to_bf16(y);
}

// Rows mw .. mw+ROWS-1, columns nw .. nw+COLS-1 of Y from the wave's LDS
// tile; whole tiles with N % 8 == 0 take 16-byte stores (the ABI's 16-byte
// aligned Y makes them aligned), edge tiles store the elements inside M x N.
template <int ROWS, int COLS = 64>
__device__ __forceinline__ void tile_store(uint16_t* Y, int M, int N, int mw, int nw, const unsigned char* et, int lane) {
  static_assert(COLS == 32 || COLS == 64, "32 or 64 columns");
  constexpr int LPR = COLS / 8, RPI = 64 / LPR;  // lanes per row, rows per instruction
  static_assert(ROWS % RPI == 0, "whole store instructions");
  const bool full = mw + ROWS <= M && nw + COLS <= N && (N & 7) == 0;
#pragma unroll
  for (int q = 0; q < ROWS / RPI; ++q) {
    const int row = RPI * q + lane / LPR, col = 8 * (lane % LPR);
    const u32x4 v = *reinterpret_cast<const u32x4*>(et + row * kTileRowBytes + col * 2);
    const int m = mw + row, n = nw + col;
    if (full) {
      // non-temporal: the output is not read again by this kernel (MXFP4 at
      // M = N = 4096, K = 3072: 97-99 -> 93 us)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(Y + (int64_t)m * N + n));
    } else if (m < M) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < N) Y[(int64_t)m * N + n + e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// Dynamic LDS above 64 KiB must be allowed per kernel once per process.
template <typename Kern>
hipError_t allow_smem(Kern k, int bytes, std::atomic<int>& done) {
  if (bytes <= 65536 || done.load(std::memory_order_acquire)) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.store(1, std::memory_order_release);
  return e;
}

}  // namespace wq
