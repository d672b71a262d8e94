// Dequant-GEMM for small and moderate M: Y = X . deq(W)^T (+ b).
//
// Every weight-only page's intro describes the engine it wants: the weight stays
// packed in device memory and a dequantization prologue feeds a high-precision
// GEMM while activations stay bf16 (NVFP4 adds a two-level block x global
// scale).  The static-FP8 page's intro runs the GEMM itself in FP8.  Here:
//
//  * one workgroup = 4 waves = 64 output columns x a contiguous K range;
//    each wave owns a quarter of that K range (split-K inside the workgroup);
//  * per K macro-step each lane issues one 16-byte load per 16-column tile of
//    packed weight and 16-byte loads of its activation rows straight into
//    registers (no LDS staging at small M: every activation element is used
//    by exactly the 64 columns of this workgroup);
//  * codes are decoded in registers and fed to v_mfma_f32_16x16x32_bf16
//    (v_mfma_f32_16x16x32_fp8_fp8 for the static path) with fp32
//    accumulation.  Lane (g, c) with g = lane/16, c = lane%16 supplies
//    8 consecutive K of its own 16-byte chunk to each MFMA, so the K order
//    inside an MFMA is a permutation shared by both operands;
//  * wave partials are reduced through LDS; with S > 1 K-splits the
//    workgroups of one column tile write fp32 partials to the workspace and
//    the last one to arrive (device-scope counter) sums them in a fixed
//    order, applies the epilogue and resets the counter;
//  * epilogue: x row/global scale, + bias, one nearest-even rounding to bf16.
//
// Decode per format (all exact in bf16):
//  INT4  : nibble XOR 8 ORed into bf16 0x4300 gives 136 + code; the group
//          (= one 128-K macro-step) is accumulated on its own, the bias is
//          removed with a row-sum MFMA against ones and the bf16 group scale
//          is applied to the group partial: acc += s * (P - 136 * rowsum).
//  FP8   : v_cvt_scalef32_pk_bf16_fp8 (scale 1); the row scale goes to the
//          epilogue.
//  NVFP4 : E2M1 -> fp32 (v_cvt_scalef32_pk_f32_fp4), x E4M3 block scale in
//          fp32 (exact: <= 6 significant bits), -> bf16; the fp32 global
//          scale goes to the epilogue.  (The scaled converts apply only the
//          exponent of their scale operand, so the E4M3 mantissa is applied
//          with a multiply.)
//  MXFP4 : v_cvt_scalef32_pk_bf16_fp4 with the power-of-two E8M0 scale.
//  BF16  : the dense weight (the unquantized Linear), no decode.
#include "wq_device.hpp"
#include "wq_internal.hpp"

namespace wq {

namespace {

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

template <int F>
__device__ __forceinline__ int64_t kbyte(int64_t k) {
  if constexpr (F == KF_BF16) return 2 * k;
  else if constexpr (F == KF_FP8 || F == KF_FP8S) return k;
  else return k / 2;
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

template <int F>
__device__ __forceinline__ float column_scale(const LinearArgs& a, int n) {
  if constexpr (F == KF_FP8) return reinterpret_cast<const float*>(a.scales)[n];
  else if constexpr (F == KF_NVFP4) return a.gscale[0];
  else return 1.0f;
}

template <int F, int MT>
__global__ __launch_bounds__(256) void k_linear_small(LinearArgs a, int S, int spw) {
  constexpr int KPL = FmtT<F>::KPL;
  constexpr int MACRO = 4 * KPL;
  constexpr bool ACT8 = (F == KF_FP8S);
  constexpr int XL = ACT8 ? 1 : KPL / 8;  // 16-byte activation loads per m-tile
  constexpr int E = MT * 16 * 64;         // outputs of the workgroup tile
  __shared__ float red[3 * E];
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int n0 = blockIdx.x * 64;
  const int split = blockIdx.y;
  const int m0 = blockIdx.z * (16 * MT);
  const int M = a.M, N = a.N, K = a.K;
  const int T = (K + MACRO - 1) / MACRO;
  const int t0 = (split * 4 + wave) * spw;
  const int t1 = min(t0 + spw, T);

  const uint8_t* __restrict__ Wb = reinterpret_cast<const uint8_t*>(a.W);
  const int64_t wrow = kbyte<F>(K);

  f32x4 acc[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ts = t0; ts < t1; ++ts) {
    const int kl = ts * MACRO + g * KPL;
    const bool kv = kl < K;
    u32x4 w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = n0 + 16 * t + c;
      w[t] = (kv && n < N) ? *reinterpret_cast<const u32x4*>(Wb + (int64_t)n * wrow + kbyte<F>(kl))
                           : u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 xv[MT][XL];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = m0 + 16 * i + c;
      const bool ok = kv && m < M;
#pragma unroll
      for (int j = 0; j < XL; ++j) {
        if constexpr (ACT8)
          xv[i][j] = ok ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(a.X) + (int64_t)m * K + kl)
                        : u32x4{0u, 0u, 0u, 0u};
        else
          xv[i][j] = ok ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.X) + (int64_t)m * K +
                                                          kl + 8 * j)
                        : u32x4{0u, 0u, 0u, 0u};
      }
    }

    if constexpr (F == KF_INT4) {
      float sc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = n0 + 16 * t + c;
        sc[t] = (kv && n < N)
                    ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.scales)[(int64_t)n * (K / 128) + kl / 128])
                    : 0.f;
      }
      f32x4 tmp[MT][4], rs[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        rs[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) tmp[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      const bf16x8 ones = as_bf16x8(u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) b[t] = dec_int4_biased(w[t][j]);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const bf16x8 A = as_bf16x8(xv[i][j]);
          rs[i] = mfma_bf16(A, ones, rs[i]);
#pragma unroll
          for (int t = 0; t < 4; ++t) tmp[i][t] = mfma_bf16(A, b[t], tmp[i][t]);
        }
      }
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][t][r] = fmaf(sc[t], fmaf(-136.f, rs[i][r], tmp[i][t][r]), acc[i][t][r]);
    } else if constexpr (F == KF_NVFP4) {
      float d0[4], d1[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = n0 + 16 * t + c;
        const uint8_t* sp = reinterpret_cast<const uint8_t*>(a.scales) + (int64_t)n * (K / 16) + kl / 16;
        const bool ok = kv && n < N;
        d0[t] = ok ? e4m3_decode(sp[0]) : 0.f;
        d1[t] = ok ? e4m3_decode(sp[1]) : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) b[t] = dec_fp4_mul(w[t][j], j < 2 ? d0[t] : d1[t]);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[i][t] = mfma_bf16(as_bf16x8(xv[i][j]), b[t], acc[i][t]);
      }
    } else if constexpr (F == KF_MXFP4) {
      float p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = n0 + 16 * t + c;
        p[t] = (kv && n < N) ? e8m0_decode(reinterpret_cast<const uint8_t*>(a.scales)[(int64_t)n * (K / 32) + kl / 32])
                             : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) b[t] = dec_fp4_pow2(w[t][j], p[t]);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[i][t] = mfma_bf16(as_bf16x8(xv[i][j]), b[t], acc[i][t]);
      }
    } else if constexpr (F == KF_FP8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8 b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) b[t] = dec_fp8(w[t][2 * j], w[t][2 * j + 1]);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[i][t] = mfma_bf16(as_bf16x8(xv[i][j]), b[t], acc[i][t]);
      }
    } else if constexpr (F == KF_BF16) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][t] = mfma_bf16(as_bf16x8(xv[i][0]), as_bf16x8(w[t]), acc[i][t]);
    } else {  // KF_FP8S: E4M3 activations x E4M3 weights
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            acc[i][t] = mfma_fp8(xv[i][0][2 * j], xv[i][0][2 * j + 1], w[t][2 * j], w[t][2 * j + 1], acc[i][t]);
    }
  }

  // ---- reduce the 4 wave partials: waves 1..3 through LDS into wave 0
  if (wave > 0) {
    float* dst = red + (wave - 1) * E;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * i + 4 * g + r) * 64 + 16 * t + c] = acc[i][t][r];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = (16 * i + 4 * g + r) * 64 + 16 * t + c;
          red[e] = acc[i][t][r] + red[e] + red[E + e] + red[2 * E + e];
        }
  }
  __syncthreads();

  // ---- epilogue (directly, or after the cross-workgroup split-K reduction)
  auto store = [&](int e, float v) {
    const int m = m0 + (e >> 6), n = n0 + (e & 63);
    if (m < M && n < N) {
      float y;
      if constexpr (F == KF_FP8S) y = (v * a.act_scale[0]) * reinterpret_cast<const float*>(a.scales)[n];
      else y = v * column_scale<F>(a, n);
      if (a.bias) y += bf16_to_f32(a.bias[n]);
      a.Y[(int64_t)m * N + n] = f32_to_bf16(y);
    }
  };

  if (S == 1) {
    for (int e = tid; e < E; e += 256) store(e, red[e]);
    return;
  }
  const int tile = blockIdx.z * gridDim.x + blockIdx.x;
  float* mine = a.part + ((int64_t)tile * S + split) * E;
  for (int e = tid; e < E; e += 256) mine[e] = red[e];
  __threadfence();
  __syncthreads();
  if (tid == 0) last_flag = (atomicAdd(&a.cnt[tile], 1u) == (unsigned)(S - 1));
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  const float* base = a.part + (int64_t)tile * S * E;
  for (int e = tid; e < E; e += 256) {
    float v = 0.f;
    for (int s2 = 0; s2 < S; ++s2) v += base[(int64_t)s2 * E + e];
    store(e, v);
  }
  if (tid == 0) a.cnt[tile] = 0u;
}

template <int F>
hipError_t launch_f(const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  dim3 grid(p.gx, p.S, p.gz);
  switch (p.mt) {
    case 1: k_linear_small<F, 1><<<grid, 256, 0, s>>>(a, p.S, p.spw); break;
    case 2: k_linear_small<F, 2><<<grid, 256, 0, s>>>(a, p.S, p.spw); break;
    default: k_linear_small<F, 4><<<grid, 256, 0, s>>>(a, p.S, p.spw); break;
  }
  return hipGetLastError();
}

int kpl_of(int kfmt) {
  switch (kfmt) {
    case KF_BF16: return 8;
    case KF_FP8:
    case KF_FP8S: return 16;
    default: return 32;
  }
}

}  // namespace

LinearPlan plan_linear(int kfmt, int64_t M, int64_t N, int64_t K) {
  LinearPlan p{};
  p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.gz = (int)((M + 16 * p.mt - 1) / (16 * p.mt));
  p.gx = (int)((N + 63) / 64);
  const int64_t macro = 4 * kpl_of(kfmt);
  const int64_t T = (K + macro - 1) / macro;
  int spw = (kfmt == KF_BF16) ? 4 : ((kfmt == KF_FP8 || kfmt == KF_FP8S) ? 2 : 1);
  int64_t S = (T + 4 * spw - 1) / (4 * spw);
  const int64_t base = (int64_t)p.gx * p.gz;
  if (base >= 256) S = 1;
  if (S < 1) S = 1;
  spw = (int)((T + 4 * S - 1) / (4 * S));
  if (spw < 1) spw = 1;
  S = (T + 4 * spw - 1) / (4 * spw);
  if (S < 1) S = 1;
  p.S = (int)S;
  p.spw = spw;
  const int64_t E = (int64_t)p.mt * 16 * 64;
  if (p.S > 1) {
    p.part_bytes = (size_t)(base * p.S * E * 4);
    p.cnt_bytes = (size_t)(((base * 4) + 255) / 256 * 256);
  } else {
    p.part_bytes = 0;
    p.cnt_bytes = 0;
  }
  p.ws_bytes = p.part_bytes + p.cnt_bytes;
  return p;
}

hipError_t launch_linear(int kfmt, const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  switch (kfmt) {
    case KF_BF16: return launch_f<KF_BF16>(a, p, s);
    case KF_INT4: return launch_f<KF_INT4>(a, p, s);
    case KF_FP8: return launch_f<KF_FP8>(a, p, s);
    case KF_NVFP4: return launch_f<KF_NVFP4>(a, p, s);
    case KF_MXFP4: return launch_f<KF_MXFP4>(a, p, s);
    case KF_FP8S: return launch_f<KF_FP8S>(a, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wq
