// Offline and calibration kernels: weight quantizers, packing, dequantization
// to bf16, absmax observers and the static activation Q.
//
// Quantizer arithmetic is IEEE fp32 (correctly rounded division; the library
// is built with -fhip-fp32-correctly-rounded-divide-sqrt and without
// denormal flushing) followed by clamp-then-nearest-even casts, so codes and
// scales are bit-identical to an IEEE reference.
#include <type_traits>

#include "wq_device.hpp"
#include "wq_internal.hpp"
#include "wq_kernel_common.hpp"

namespace wq {

namespace {

constexpr int kThreads = 256;

inline unsigned grid_for(int64_t items, int per_block = kThreads) {
  int64_t g = (items + per_block - 1) / per_block;
  return (unsigned)(g < 1 ? 1 : g);
}

// 16 consecutive bf16 -> fp32 (two 16-byte loads).
__device__ __forceinline__ void load16_bf16(const uint16_t* p, float* out) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  u32x4 a = q[0], b = q[1];
  uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out[2 * i] = bitsf(w[i] << 16);
    out[2 * i + 1] = bitsf(w[i] & 0xFFFF0000u);
  }
}

// ---------------------------------------------------------------- INT4
// "TorchAO INT4 Weight-Only Quantization (Linear)": symmetric, zero-point 0,
// group 128 along K.  One thread per (row, group).
__global__ __launch_bounds__(kThreads) void k_quant_int4(const uint16_t* __restrict__ W, int64_t N, int64_t K,
                                                         int8_t* __restrict__ codes,
                                                         uint16_t* __restrict__ scales) {
  const int64_t G = K / 128;
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= N * G) return;
  const int64_t n = id / G, gi = id % G;
  const uint16_t* w = W + n * K + gi * 128;
  float v[128];
#pragma unroll
  for (int i = 0; i < 8; ++i) load16_bf16(w + 16 * i, v + 16 * i);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 128; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint16_t sb = f32_to_bf16(amax / 7.0f);
  const float s = bf16_to_f32(sb);
  scales[n * G + gi] = sb;
  uint32_t packed[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) packed[i] = 0;
#pragma unroll
  for (int i = 0; i < 128; ++i) {
    float q = (s > 0.f) ? v[i] / s : 0.f;
    int c = (int)__builtin_rintf(q);
    c = c < -8 ? -8 : (c > 7 ? 7 : c);
    packed[i >> 2] |= ((uint32_t)(uint8_t)(int8_t)c) << (8 * (i & 3));
  }
  u32x4* out = reinterpret_cast<u32x4*>(codes + n * K + gi * 128);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = u32x4{packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]};
}

// ---------------------------------------------------------------- INT4, asymmetric
// The INT4 page's intro names TorchAO's default asymmetric scheme (nonzero
// zero-point).  Per (row, group of 128 K): lo = min(min w, 0), hi = max(max w,
// 0), s = bf16((hi - lo) / 15), z = clamp(rint(-lo / s), 0, 15), code =
// clamp(rint(w / s) + z, 0, 15); the group's word holds s | z << 16.  One
// thread per (row, group).
__global__ __launch_bounds__(kThreads) void k_quant_int4a(const uint16_t* __restrict__ W, int64_t N, int64_t K,
                                                          uint8_t* __restrict__ codes,
                                                          uint32_t* __restrict__ scales) {
  const int64_t G = K / 128;
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= N * G) return;
  const int64_t n = id / G, gi = id % G;
  const uint16_t* w = W + n * K + gi * 128;
  float v[128];
#pragma unroll
  for (int i = 0; i < 8; ++i) load16_bf16(w + 16 * i, v + 16 * i);
  float lo = 0.f, hi = 0.f;
#pragma unroll
  for (int i = 0; i < 128; ++i) {
    lo = fminf(lo, v[i]);
    hi = fmaxf(hi, v[i]);
  }
  const uint16_t sb = f32_to_bf16((hi - lo) / 15.0f);
  const float s = bf16_to_f32(sb);
  int z = 0;
  if (s > 0.f) {
    z = (int)__builtin_rintf(-lo / s);
    z = z < 0 ? 0 : (z > 15 ? 15 : z);
  }
  scales[n * G + gi] = (uint32_t)sb | ((uint32_t)z << 16);
  uint32_t packed[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) packed[i] = 0;
#pragma unroll
  for (int i = 0; i < 128; ++i) {
    int c = (s > 0.f) ? (int)__builtin_rintf(v[i] / s) + z : 0;
    c = c < 0 ? 0 : (c > 15 ? 15 : c);
    packed[i >> 2] |= (uint32_t)c << (8 * (i & 3));
  }
  u32x4* out = reinterpret_cast<u32x4*>(codes + n * K + gi * 128);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = u32x4{packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]};
}

// ---------------------------------------------------------------- FP8 row
// "TorchAO FP8 Weight-Only Quantization (Linear)": one fp32 scale per output
// row, s = max|w| / 448.  One workgroup per row.
__device__ __forceinline__ float block_max(float v, float* lds) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) lds[wv] = v;
  __syncthreads();
  float r = lds[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fmaxf(r, lds[i]);
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void k_quant_fp8row(const uint16_t* __restrict__ W, int64_t K,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ scales) {
  __shared__ float lds[kThreads / 64];
  const int64_t n = blockIdx.x;
  const uint16_t* w = W + n * K;
  float amax = 0.f;
  for (int64_t k = threadIdx.x; k < K; k += kThreads) amax = fmaxf(amax, fabsf(bf16_to_f32(w[k])));
  amax = block_max(amax, lds);
  const float s = amax / 448.0f;
  if (threadIdx.x == 0) scales[n] = s;
  for (int64_t k = threadIdx.x; k < K; k += kThreads) {
    float x = bf16_to_f32(w[k]);
    float q = (s > 0.f) ? x / s : x;
    codes[n * K + k] = (uint8_t)e4m3_encode(clampf(q, -448.f, 448.f));
  }
}

// ---------------------------------------------------------------- NVFP4
// "TorchAO NVFP4 Weight-Only Quantization (Linear)": E2M1 codes, E4M3 scale per
// 16 consecutive K, fp32 global scale g = max|W| / (448 * 6).
__global__ void k_fill_f32(float* p, float v, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(kThreads) void k_absmax_bf16(const uint16_t* __restrict__ X, int64_t n,
                                                          float* __restrict__ amax) {
  __shared__ float lds[kThreads / 64];
  float m = 0.f;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
    m = fmaxf(m, fabsf(bf16_to_f32(X[i])));
  m = block_max(m, lds);
  if (threadIdx.x == 0) atomic_max_nonneg(amax, m);
}

__global__ __launch_bounds__(kThreads) void k_quant_nvfp4(const uint16_t* __restrict__ W, int64_t N, int64_t K,
                                                          const float* __restrict__ tensor_amax,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int64_t B = K / 16;
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= N * B) return;
  const int64_t n = id / B, bi = id % B;
  float v[16];
  load16_bf16(W + n * K + bi * 16, v);
  float ab = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ab = fmaxf(ab, fabsf(v[i]));
  const float g = tensor_amax[0] / 2688.0f;
  float t = (g > 0.f) ? (ab / 6.0f) / g : 0.f;
  t = clampf(t, 0.001953125f, 448.f);
  const uint32_t sc = e4m3_encode(t);
  const float S = e4m3_decode(sc) * g;
  scales[n * B + bi] = (uint8_t)sc;
  uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float q = (S > 0.f) ? v[i] / S : v[i];
    out[i >> 2] |= e2m1_encode(clampf(q, -6.f, 6.f)) << (8 * (i & 3));
  }
  *reinterpret_cast<u32x4*>(codes + n * K + bi * 16) = u32x4{out[0], out[1], out[2], out[3]};
}

__global__ void k_nvfp4_global(float* gscale) {
  if (threadIdx.x == 0 && blockIdx.x == 0) gscale[0] = gscale[0] / 2688.0f;
}

// ---------------------------------------------------------------- MXFP4
// "TorchAO MXFP4 Dynamic Activation + MX Weight (Linear)": E2M1 codes, E8M0
// scale per 32 consecutive K; shared exponent floor(log2 amax) - 2.
__global__ __launch_bounds__(kThreads) void k_quant_mxfp4(const uint16_t* __restrict__ W, int64_t N, int64_t K,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int64_t B = K / 32;
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= N * B) return;
  const int64_t n = id / B, bi = id % B;
  float v[32];
  load16_bf16(W + n * K + bi * 32, v);
  load16_bf16(W + n * K + bi * 32 + 16, v + 16);
  float ab = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) ab = fmaxf(ab, fabsf(v[i]));
  const uint32_t ebits = fbits(ab) >> 23;  // biased exponent; 0 for zero and subnormals
  int e = (ebits == 0u) ? -127 : (int)ebits - 127 - 2;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  scales[n * B + bi] = (uint8_t)(e + 127);
  const float p = (e == -127) ? bitsf(0x00400000u) : bitsf((uint32_t)(e + 127) << 23);
  uint32_t out[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float q = v[i] / p;
    out[i >> 2] |= e2m1_encode(clampf(q, -6.f, 6.f)) << (8 * (i & 3));
  }
  u32x4* o = reinterpret_cast<u32x4*>(codes + n * K + bi * 32);
  o[0] = u32x4{out[0], out[1], out[2], out[3]};
  o[1] = u32x4{out[4], out[5], out[6], out[7]};
}

// ---------------------------------------------------------------- packing
// Two 4-bit codes per byte along K, even element in the low nibble.  One
// thread per 16 output bytes (32 codes).
__global__ __launch_bounds__(kThreads) void k_pack4(const uint8_t* __restrict__ codes, int64_t n16,
                                                    uint8_t* __restrict__ packed) {
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= n16) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(codes + id * 32);
  u32x4 a = src[0], b = src[1];
  uint32_t in[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = in[2 * i], hi = in[2 * i + 1];
    // bytes b0..b3 of lo -> two output bytes; same for hi
    uint32_t r = 0;
    r |= ((lo & 0xFu) | ((lo >> 4) & 0xF0u));
    r |= (((lo >> 16) & 0xFu) | ((lo >> 20) & 0xF0u)) << 8;
    r |= ((hi & 0xFu) | ((hi >> 4) & 0xF0u)) << 16;
    r |= (((hi >> 16) & 0xFu) | ((hi >> 20) & 0xF0u)) << 24;
    out[i] = r;
  }
  *reinterpret_cast<u32x4*>(packed + id * 16) = u32x4{out[0], out[1], out[2], out[3]};
}

__global__ __launch_bounds__(kThreads) void k_copy16(const u32x4* __restrict__ src, int64_t n16,
                                                     u32x4* __restrict__ dst) {
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id < n16) dst[id] = src[id];
}

__global__ __launch_bounds__(kThreads) void k_copy_bytes(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                         int64_t n) {
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id < n) dst[id] = src[id];
}

// ---------------------------------------------------------------- dequantize to bf16
// bf16(fp32(code value * block scale (* global))).  One thread per 8 outputs;
// the packed weight and its block scales are read in layout WL.
template <int F, int WL>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t* __restrict__ P, const void* __restrict__ scales,
                                                      const float* __restrict__ gscale, int64_t N, int64_t K,
                                                      uint16_t* __restrict__ out) {
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t per_row = K / 8;
  if (id >= N * per_row) return;
  const int64_t n = id / per_row, k0 = (id % per_row) * 8;
  const unsigned char* S = reinterpret_cast<const unsigned char*>(scales);
  uint16_t r[8];
  if constexpr (F == KF_FP8) {
    const float s = reinterpret_cast<const float*>(scales)[n];
    const uint8_t* c = P + w_off<WL>((uint32_t)n, (uint32_t)k0, (uint32_t)K);
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = f32_to_bf16(e4m3_decode(c[i]) * s);
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(P + w_off<WL>((uint32_t)n, (uint32_t)k0 / 2u, (uint32_t)K / 2u));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = (w >> (4 * i)) & 0xFu;
      const uint32_t so = s_off<F, WL>((uint32_t)n, (uint32_t)(k0 + i), (uint32_t)K);
      float v;
      if constexpr (F == KF_INT4) {
        const float s = bf16_to_f32(*reinterpret_cast<const uint16_t*>(S + so));
        v = (float)((int)c - ((c & 8u) ? 16 : 0)) * s;
      } else if constexpr (F == KF_INT4A) {
        const uint32_t sw = *reinterpret_cast<const uint32_t*>(S + so);
        v = (float)((int)c - (int)((sw >> 16) & 15u)) * bitsf(sw << 16);
      } else if constexpr (F == KF_NVFP4) {
        const float d = e4m3_decode(S[so]);
        v = (e2m1_decode(c) * d) * gscale[0];
      } else {  // MXFP4
        const float p = e8m0_decode(S[so]);
        v = e2m1_decode(c) * p;
      }
      r[i] = f32_to_bf16(v);
    }
  }
  *reinterpret_cast<u32x4*>(out + n * K + k0) =
      u32x4{r[0] | ((uint32_t)r[1] << 16), r[2] | ((uint32_t)r[3] << 16), r[4] | ((uint32_t)r[5] << 16),
            r[6] | ((uint32_t)r[7] << 16)};
}

// ---------------------------------------------------------------- layout conversion
// One thread per 16-byte chunk of packed weight (canonical chunk c = row n,
// bytes 16 (c % (row_bytes / 16)) ..): copied from its place in layout SRC to
// its place in layout DST.
template <int SRC, int DST>
__global__ __launch_bounds__(kThreads) void k_repack_codes(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                           int64_t N, uint32_t row_bytes) {
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const uint32_t cpr = row_bytes / 16u;
  if (id >= N * (int64_t)cpr) return;
  const uint32_t n = (uint32_t)(id / cpr), kb = (uint32_t)(id % cpr) * 16u;
  *reinterpret_cast<u32x4*>(dst + w_off<DST>(n, kb, row_bytes)) =
      *reinterpret_cast<const u32x4*>(src + w_off<SRC>(n, kb, row_bytes));
}

// One thread per (row, 128-K tile) piece of block scales (ScaleT<F>::SB bytes:
// 2, 4 or 8, contiguous in both layouts).
template <int F, int SRC, int DST>
__global__ __launch_bounds__(kThreads) void k_repack_scales(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                            int64_t N, uint32_t K) {
  using P = typename std::conditional<ScaleT<F>::SB == 2, uint16_t,
                                      typename std::conditional<ScaleT<F>::SB == 4, uint32_t, uint64_t>::type>::type;
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const uint32_t tiles = K / 128u;
  if (id >= N * (int64_t)tiles) return;
  const uint32_t n = (uint32_t)(id / tiles), k = (uint32_t)(id % tiles) * 128u;
  *reinterpret_cast<P*>(dst + s_off<F, DST>(n, k, K)) = *reinterpret_cast<const P*>(src + s_off<F, SRC>(n, k, K));
}

template <int SRC, int DST>
hipError_t repack_l(int fmt, int64_t N, int64_t K, const void* sp, const void* ss, void* dp, void* ds, hipStream_t s) {
  const uint32_t row_bytes = (fmt == KF_FP8) ? (uint32_t)K : (uint32_t)K / 2u;
  k_repack_codes<SRC, DST><<<grid_for(N * (row_bytes / 16)), kThreads, 0, s>>>((const uint8_t*)sp, (uint8_t*)dp, N,
                                                                                  row_bytes);
  const unsigned gs = grid_for(N * (K / 128));
  const uint8_t* a = (const uint8_t*)ss;
  uint8_t* b = (uint8_t*)ds;
  switch (fmt) {
    case KF_FP8: k_copy_bytes<<<grid_for(N * 4), kThreads, 0, s>>>(a, b, N * 4); break;  // row scales
    case KF_INT4: k_repack_scales<KF_INT4, SRC, DST><<<gs, kThreads, 0, s>>>(a, b, N, (uint32_t)K); break;
    case KF_INT4A: k_repack_scales<KF_INT4A, SRC, DST><<<gs, kThreads, 0, s>>>(a, b, N, (uint32_t)K); break;
    case KF_NVFP4: k_repack_scales<KF_NVFP4, SRC, DST><<<gs, kThreads, 0, s>>>(a, b, N, (uint32_t)K); break;
    case KF_MXFP4: k_repack_scales<KF_MXFP4, SRC, DST><<<gs, kThreads, 0, s>>>(a, b, N, (uint32_t)K); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- static FP8 helpers
__global__ void k_fp8_scale(const float* __restrict__ amax, float* __restrict__ scale, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) scale[i] = amax[i] / 448.0f;
}

// "TorchAO Static FP8 Quantization (Linear)": x -> E4M3(clamp(x / act_scale, +-448)).
// One 8-element chunk per thread (chunk c = block * 256 + thread); the
// element tail (numel % 8) goes to the thread whose chunk index equals the
// chunk count.  Grids are capped at kQActMaxBlocks: beyond that (STRIDE) the
// threads stride over the rest.  Four chunks per thread with all four loads in
// flight measured slower at every size (K = 3072, M = 1 / 32 / 256 / 4096:
// 2.05 / 2.4 / 2.5 / 9.6 us against 1.62 / 1.65 / 1.86 / 8.8 us on one box).
constexpr int64_t kQActMaxBlocks = 1 << 16;
template <bool STRIDE>
__global__ __launch_bounds__(kThreads) void k_quant_act(const uint16_t* __restrict__ X, int64_t numel,
                                                        const float* __restrict__ act_scale,
                                                        uint8_t* __restrict__ Xq) {
  const float s = act_scale[0];
  const int64_t full = numel / 8;
  const u32x4* X16 = reinterpret_cast<const u32x4*>(X);
  u32x2* Q8 = reinterpret_cast<u32x2*>(Xq);
  const int64_t c0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t step = STRIDE ? (int64_t)gridDim.x * kThreads : full + 1;
  for (int64_t c = c0; c <= full; c += step) {
    if (c < full) {
      Q8[c] = act_q8(X16[c], s);
    } else {
      for (int64_t i = full * 8; i < numel; ++i) Xq[i] = (uint8_t)e4m3_encode(act_q_val(bf16_to_f32(X[i]), s));
    }
    if constexpr (!STRIDE) break;
  }
}

}  // namespace

// ---------------------------------------------------------------- launchers

hipError_t launch_quantize(int fmt, const uint16_t* W, int64_t N, int64_t K, void* codes, void* scales,
                           float* gscale, hipStream_t s) {
  switch (fmt) {
    case KF_INT4:
      k_quant_int4<<<grid_for(N * (K / 128)), kThreads, 0, s>>>(W, N, K, (int8_t*)codes, (uint16_t*)scales);
      break;
    case KF_INT4A:
      k_quant_int4a<<<grid_for(N * (K / 128)), kThreads, 0, s>>>(W, N, K, (uint8_t*)codes, (uint32_t*)scales);
      break;
    case KF_FP8:
      k_quant_fp8row<<<(unsigned)N, kThreads, 0, s>>>(W, K, (uint8_t*)codes, (float*)scales);
      break;
    case KF_NVFP4: {
      k_fill_f32<<<1, 64, 0, s>>>(gscale, 0.f, 1);
      const int64_t n = N * K;
      unsigned g = grid_for(n, kThreads * 16);
      if (g > 4096) g = 4096;
      k_absmax_bf16<<<g, kThreads, 0, s>>>(W, n, gscale);
      k_quant_nvfp4<<<grid_for(N * (K / 16)), kThreads, 0, s>>>(W, N, K, gscale, (uint8_t*)codes,
                                                                  (uint8_t*)scales);
      k_nvfp4_global<<<1, 64, 0, s>>>(gscale);
      break;
    }
    case KF_MXFP4:
      k_quant_mxfp4<<<grid_for(N * (K / 32)), kThreads, 0, s>>>(W, N, K, (uint8_t*)codes, (uint8_t*)scales);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pack(int fmt, const uint8_t* codes, int64_t N, int64_t K, uint8_t* packed, hipStream_t s) {
  if (fmt == KF_FP8) {
    const int64_t n16 = N * K / 16;
    k_copy16<<<grid_for(n16), kThreads, 0, s>>>((const u32x4*)codes, n16, (u32x4*)packed);
  } else {
    const int64_t n16 = N * K / 32;
    k_pack4<<<grid_for(n16), kThreads, 0, s>>>(codes, n16, packed);
  }
  return hipGetLastError();
}

template <int WL>
hipError_t dequantize_l(int fmt, const void* packed, const void* scales, const float* gscale, int64_t N, int64_t K,
                        uint16_t* out, hipStream_t s) {
  const unsigned g = grid_for(N * (K / 8));
  const uint8_t* P = (const uint8_t*)packed;
  switch (fmt) {
    case KF_BF16: {
      const int64_t n16 = N * K / 8;
      k_copy16<<<grid_for(n16), kThreads, 0, s>>>((const u32x4*)packed, n16, (u32x4*)out);
      break;
    }
    case KF_INT4: k_dequant<KF_INT4, WL><<<g, kThreads, 0, s>>>(P, scales, gscale, N, K, out); break;
    case KF_INT4A: k_dequant<KF_INT4A, WL><<<g, kThreads, 0, s>>>(P, scales, gscale, N, K, out); break;
    case KF_FP8: k_dequant<KF_FP8, WL><<<g, kThreads, 0, s>>>(P, scales, gscale, N, K, out); break;
    case KF_NVFP4: k_dequant<KF_NVFP4, WL><<<g, kThreads, 0, s>>>(P, scales, gscale, N, K, out); break;
    case KF_MXFP4: k_dequant<KF_MXFP4, WL><<<g, kThreads, 0, s>>>(P, scales, gscale, N, K, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(int fmt, int wl, const void* packed, const void* scales, const float* gscale, int64_t N,
                             int64_t K, uint16_t* out, hipStream_t s) {
  return wl == kLayoutTiles ? dequantize_l<kLayoutTiles>(fmt, packed, scales, gscale, N, K, out, s)
                            : dequantize_l<kLayoutRows>(fmt, packed, scales, gscale, N, K, out, s);
}

hipError_t launch_repack(int fmt, int64_t N, int64_t K, int src_wl, const void* src_packed, const void* src_scales,
                         int dst_wl, void* dst_packed, void* dst_scales, hipStream_t s) {
  if (src_wl == kLayoutRows && dst_wl == kLayoutTiles)
    return repack_l<kLayoutRows, kLayoutTiles>(fmt, N, K, src_packed, src_scales, dst_packed, dst_scales, s);
  if (src_wl == kLayoutTiles && dst_wl == kLayoutRows)
    return repack_l<kLayoutTiles, kLayoutRows>(fmt, N, K, src_packed, src_scales, dst_packed, dst_scales, s);
  if (src_wl == kLayoutTiles)
    return repack_l<kLayoutTiles, kLayoutTiles>(fmt, N, K, src_packed, src_scales, dst_packed, dst_scales, s);
  return repack_l<kLayoutRows, kLayoutRows>(fmt, N, K, src_packed, src_scales, dst_packed, dst_scales, s);
}

hipError_t launch_absmax(const uint16_t* X, int64_t numel, float* amax, hipStream_t s) {
  unsigned g = grid_for(numel, kThreads * 16);
  if (g > 4096) g = 4096;
  k_absmax_bf16<<<g, kThreads, 0, s>>>(X, numel, amax);
  return hipGetLastError();
}

hipError_t launch_fp8_scale(const float* amax, float* scale, int64_t count, hipStream_t s) {
  k_fp8_scale<<<grid_for(count, 64), 64, 0, s>>>(amax, scale, count);
  return hipGetLastError();
}

hipError_t launch_quantize_act(const uint16_t* X, int64_t numel, const float* act_scale, uint8_t* Xq,
                               hipStream_t s) {
  const int64_t blocks = (numel / 8 + kThreads) / kThreads;  // chunks + the tail's thread
  if (blocks <= kQActMaxBlocks)
    k_quant_act<false><<<(unsigned)blocks, kThreads, 0, s>>>(X, numel, act_scale, Xq);
  else
    k_quant_act<true><<<(unsigned)kQActMaxBlocks, kThreads, 0, s>>>(X, numel, act_scale, Xq);
  return hipGetLastError();
}

// Read-only stream (measurement aid): workgroup b reads the 16 KiB block b
// (1024 chunks of 16 bytes, four per thread, all issued before the first use,
// non-temporal like the 4-bit weight loads) and stores the XOR of its 32-bit
// words to sink[b].  Offsets past the end read zero (neutral for XOR).  One
// plain store per workgroup: no atomics on a shared address, which would
// serialize the workgroups.  Of thirteen variants measured as graphs of 200
// launches over cold copies (256 to 3076 workgroups of 256 to 1024 threads,
// 1 to 16 loads per thread in flight, with and without non-temporal loads;
// the best of three replays): this form was fastest at both sizes, 3.06 us
// for 6.68 MB and 3.83 us for 12.6 MB; with ordinary loads 3.30 and 4.10 us;
// grids of about one workgroup per CU (102-272 workgroups of 256-1024
// threads, 3-16 loads per thread) 3.27-3.64 us and 4.10-4.21 us; an empty
// kernel in the same graph 1.6 us.
namespace {
__global__ __launch_bounds__(256) void k_read_stream(const void* p, uint32_t bytes, uint32_t* sink) {
  __shared__ uint32_t part[4];
  const __amdgpu_buffer_rsrc_t r = make_rsrc(p, bytes);
  const uint32_t base = (uint32_t)blockIdx.x * 1024u + threadIdx.x;
  u32x4 v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = bload128_nt(r, (base + 256u * q) * 16u);
  uint32_t h = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) h ^= v[q].x ^ v[q].y ^ v[q].z ^ v[q].w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) h ^= __shfl_xor(h, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = h;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}
}  // namespace

hipError_t launch_read_stream(const void* p, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t chunks = bytes / 16;
  const unsigned grid = (unsigned)((chunks + 1023) / 1024);
  k_read_stream<<<grid, 256, 0, s>>>(p, (uint32_t)bytes, sink);
  return hipGetLastError();
}

}  // namespace wq
