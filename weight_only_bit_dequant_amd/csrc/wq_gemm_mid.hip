// Dequant-GEMM for mid-size M (129 rows up to about three rounds of 64 x 64
// tiles on the chip), weight-only formats.
//
// One workgroup of 8 waves owns a 64 x 64 output tile.  K is split over the
// waves, not over workgroups: wave w takes the 128-K blocks w, w + 8, ...
// of the tile and accumulates all 64 x 64 outputs of its blocks, so the waves
// run independently until one LDS reduction at the end.  Per block a wave
//  * loads the 64 activation rows of the block (256 bytes each) straight into
//    its own LDS slot with buffer_load ... lds (no registers), in a chunk
//    order that keeps the operand reads free of bank conflicts;
//  * loads its four 16-column weight tiles into registers: lane (g, c) takes
//    the 16 packed bytes of column c that hold K 32g .. 32g+31 of the block
//    (in tile order one load instruction reads one whole 1 KiB weight tile);
//    E4M3 weights take two such loads, one per 64-K half;
//  * loads the block scales with one aligned dword per lane and tile, the
//    lane's bytes selected in the decode (byte loads of the scales cost about
//    0.8 us more per launch);
//  * decodes each weight chunk to bf16 once and feeds it to four
//    v_mfma_f32_16x16x32_bf16 (the 64 rows), K order shared by both operands;
//    INT4, INT4_ASYM and NVFP4 (the longer decodes) load the weights first and
//    decode the whole block while its activations are still landing.
// After the last block the waves write their fp32 partials to LDS and every
// thread sums the 8 partials of 8 outputs in wave order, applies the column
// scale and bias, rounds to bf16 once and stores 16 bytes.
//
// Measured against the LDS-tiled kernel at N = 4096, K = 3072 (graphs, cold
// weight copies): M = 256 MXFP4 15.9 -> 10.7 us, FP8 15.0 -> 12.2, NVFP4 17.6
// -> 12.8, INT4 18.0 -> 14.0; M = 768 MXFP4 34.0 -> 28.6 us.  At 1024 tiles
// (four rounds) the 128 x 128 tiles win again.  Variants measured and
// dropped: 32 x 128 tiles (twice the decode per MFMA: 0.5-1.7 us slower);
// two blocks in flight per wave (in a rolled loop the compiler's waits for the
// register loads at the loop head also cover the next block; unrolled, with 4
// waves, MXFP4 and FP8 were within 0.3 us and NVFP4 and INT4 1.5-2.2 us
// slower); 4 or 6 waves; activations staged through registers.
//
// Numerics: as the tiled kernel -- MXFP4, NVFP4 and E4M3 weights are exact
// in bf16, INT4 is rounded to bf16(code * s) per weight; fp32 accumulation.
#include "wq_kernel_common.hpp"

namespace wq {

namespace {

constexpr int kMidWaves = 8;
constexpr int kMidBM = 64, kMidBN = 64;
constexpr int kMidMT = kMidBM / 16, kMidNT = kMidBN / 16;
constexpr int kMidSlot = kMidBM * 256;  // one 128-K block of 64 activation rows
constexpr int kMidPW = kMidBN + 4;      // partial row stride (floats)


// LDS position of 16-byte chunk k of activation row r (16 chunks per row): the
// reads of lane groups g (chunk 4g + kk) of 16 rows hit 16 distinct 16-byte
// bank groups; the map is its own inverse
__device__ __forceinline__ int mid_xpos(int r, int k) { return k ^ ((r & 3) | (((r >> 2) & 1) << 3)); }

template <int F>
struct MidW {
  static constexpr int NL = (F == KF_FP8) ? 2 : 1;  // 16-byte loads per tile and block
  u32x4 w[NL];
  uint32_t sc;
};

// formats whose block scales load as one aligned dword per lane
template <int F, int WL>
constexpr bool mid_dword_scales() {
  return F == KF_MXFP4 || F == KF_NVFP4 || (F == KF_INT4 && WL == kLayoutTiles);
}

// bit position of a lane's scale bytes in that dword; the same for every tile
// and block (K % 128 == 0)
template <int F, int WL>
__device__ __forceinline__ uint32_t mid_scale_shift(int g, int c) {
  if constexpr (!mid_dword_scales<F, WL>()) return 0u;
  else if constexpr (F == KF_MXFP4) return 8u * (uint32_t)g;
  else if constexpr (F == KF_NVFP4) return 16u * (uint32_t)(g & 1);
  else return 16u * (uint32_t)(c & 1);
}

template <int F, int WL>
__device__ __forceinline__ void mid_load_w(MidW<F>& r, __amdgpu_buffer_rsrc_t Wr, __amdgpu_buffer_rsrc_t Sr, uint32_t n,
                                           int kb, uint32_t K, int g, bool ok) {
  const uint32_t rb = (F == KF_FP8) ? K : K / 2u;
  if constexpr (F == KF_FP8) {
    // K 16g .. 16g+15 of each 64-K half of the block
#pragma unroll
    for (int h = 0; h < 2; ++h) r.w[h] = bload128(Wr, off_if(ok, w_off<WL>(n, (uint32_t)(kb * 128 + 64 * h + 16 * g), rb)));
    r.sc = 0u;
  } else {
    r.w[0] = bload128(Wr, off_if(ok, w_off<WL>(n, (uint32_t)(kb * 64 + 16 * g), rb)));
    const uint32_t so = s_off<F, WL>(n, (uint32_t)(kb * 128 + 32 * g), K);
    if constexpr (mid_dword_scales<F, WL>()) r.sc = bload32(Sr, off_if(ok, so & ~3u));
    else if constexpr (F == KF_INT4) r.sc = bload16(Sr, off_if(ok, so));
    else r.sc = bload32(Sr, off_if(ok, so));  // INT4_ASYM: bf16 scale + zero point
  }
}

// bf16 operand of sub-step kk (8 K): 4-bit formats K 32g + 8kk .. +7, E4M3
// K 16g + 8(kk & 1) .. +7 of half kk / 2
template <int F>
__device__ __forceinline__ bf16x8 mid_decode(const MidW<F>& r, int kk, uint32_t sh) {
  const uint32_t sc = r.sc >> sh;
  if constexpr (F == KF_MXFP4) return dec_fp4_pow2(r.w[0][kk], e8m0_decode(sc & 0xFFu));
  else if constexpr (F == KF_NVFP4) return dec_fp4_mul(r.w[0][kk], e4m3_decode(kk < 2 ? (sc & 0xFFu) : ((sc >> 8) & 0xFFu)));
  else if constexpr (F == KF_FP8) return dec_fp8(r.w[kk >> 1][2 * (kk & 1)], r.w[kk >> 1][2 * (kk & 1) + 1]);
  else {
    // (code - z) * s, exact in fp32, then one bf16 rounding
    const float s = bitsf(sc << 16);
    const float bias = (F == KF_INT4) ? 136.f : (float)(128u + ((sc >> 16) & 15u));
    const bf16x8 biased = (F == KF_INT4) ? dec_int4_biased(r.w[0][kk]) : dec_uint4_biased(r.w[0][kk]);
    const u32x4 bb = __builtin_bit_cast(u32x4, biased);
    bf16x8 r8;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float lo = bitsf(bb[p] << 16), hi = bitsf(bb[p] & 0xFFFF0000u);
      r8[2 * p] = (__bf16)fmaf(lo, s, -bias * s);
      r8[2 * p + 1] = (__bf16)fmaf(hi, s, -bias * s);
    }
    return r8;
  }
}

// activation chunk (8 K, 16 bytes) that matches mid_decode's sub-step kk
template <int F>
__device__ __forceinline__ int mid_chunk(int g, int kk) {
  if constexpr (F == KF_FP8) return 8 * (kk >> 1) + 2 * g + (kk & 1);
  else return 4 * g + kk;
}

// NBMAX: compile-time bound on the blocks per wave; up to 8 the block loop is
// unrolled into straight-line code
template <int F, int WL, int NBMAX>
__global__ __launch_bounds__(kMidWaves * 64) void k_gemm_mid(LinearArgs a) {
  constexpr int MT = kMidMT, NT = kMidNT, BM = kMidBM, BN = kMidBN;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int M = a.M, N = a.N, K = a.K;
  // column tiles along x: the row blocks of one column tile have ids gx apart,
  // which with gx % 8 == 0 puts them on one XCD, sharing its L2 copy of the
  // weight tiles
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int KT = K / 128;
  const int nb = (KT + kMidWaves - 1) / kMidWaves;

  const uint32_t rb = (F == KF_FP8) ? (uint32_t)K : (uint32_t)K / 2u;
  const __amdgpu_buffer_rsrc_t Wr = make_rsrc(a.W, (uint32_t)N * rb);
  const __amdgpu_buffer_rsrc_t Xr = make_rsrc(a.X, (uint32_t)M * (uint32_t)K * 2u);
  uint32_t sbytes;
  if constexpr (F == KF_FP8) sbytes = (uint32_t)N * 4u;
  else sbytes = (uint32_t)N * (uint32_t)(K / 128) * ScaleT<F>::SB;
  const __amdgpu_buffer_rsrc_t Sr = make_rsrc(a.scales, sbytes);
  const uint32_t sh = mid_scale_shift<F, WL>(g, c);
  unsigned char* slot = smem + wave * kMidSlot;

  MidW<F> wr[NT];
  // EW (the formats with the longer decodes): the weights are loaded first,
  // return first, and their decode overlaps the activation loads.  Measured
  // at N = 4096, K = 3072, M = 256 / 512: INT4 15.0 / 26.3 -> 14.1 / 24.5 us,
  // INT4_ASYM 14.6 / 25.6 -> 14.4 / 24.2, NVFP4 13.8 / 24.3 -> 13.4 / 23.2;
  // MXFP4 and FP8 were up to 0.4 us slower with it
  constexpr bool EW = F == KF_INT4 || F == KF_INT4A || F == KF_NVFP4;
  auto issue = [&](int j) {
    const int kb = wave + j * kMidWaves;
    const bool ok = kb < KT;
    if constexpr (EW) {
#pragma unroll
      for (int t = 0; t < NT; ++t) mid_load_w<F, WL>(wr[t], Wr, Sr, (uint32_t)(n0 + 16 * t + c), kb, (uint32_t)K, g, ok);
    }
    // activation rows 4q .. 4q+3 of the block: lane L fills position L % 16 of
    // row 4q + L / 16 with the chunk mid_xpos maps there; rows past M and
    // blocks past K read zero
#pragma unroll
    for (int q = 0; q < BM / 4; ++q) {
      const int row = 4 * q + (lane >> 4);
      const int kx = kb * 128 + 8 * mid_xpos(row, lane & 15);
      const uint32_t off = off_if(ok, ((uint32_t)(m0 + row) * (uint32_t)K + (uint32_t)kx) * 2u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Xr, (__attribute__((address_space(3))) void*)(slot + q * 1024), 16, off, 0, 0,
                                               0);
    }
    if constexpr (!EW) {
#pragma unroll
      for (int t = 0; t < NT; ++t) mid_load_w<F, WL>(wr[t], Wr, Sr, (uint32_t)(n0 + 16 * t + c), kb, (uint32_t)K, g, ok);
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto block = [&](int j) {
    // EW: decode the block's weights as soon as they have returned (the
    // compiler waits for them alone), while the activation loads still land
    bf16x8 bw[EW ? 4 : 1][NT];
    if constexpr (EW) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int t = 0; t < NT; ++t) bw[kk][t] = mid_decode<F>(wr[t], kk, sh);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the block's activations are in LDS once its loads have returned
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 bf[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) bf[t] = EW ? bw[EW ? kk : 0][t] : mid_decode<F>(wr[t], kk, sh);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int row = 16 * i + c;
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(slot + row * 256 + mid_xpos(row, mid_chunk<F>(g, kk)) * 16);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = mfma_bf16(af, bf[t], acc[i][t]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (j + 1 < nb) {
      // the slot's operand reads are complete before the next block lands there
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      issue(j + 1);
    }
  };
  issue(0);
  if constexpr (NBMAX <= 8) {
#pragma unroll
    for (int j = 0; j < NBMAX; ++j) {
      if (j >= nb) break;  // wave-uniform
      block(j);
    }
  } else {
    // long K: a rolled loop (every block waits for all of its loads anyway)
    for (int j = 0; j < nb; ++j) block(j);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();  // every wave is done with its slot

  // partials of wave w: rows w * BM .. w * BM + BM-1 (stride kMidPW floats)
  float* part = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[(wave * BM + 16 * i + 4 * g + r) * kMidPW + 16 * t + c] = acc[i][t][r];
  __syncthreads();

  float gscale = 1.0f;
  if constexpr (F == KF_NVFP4) gscale = a.gscale[0];
  const __amdgpu_buffer_rsrc_t Br = make_rsrc(a.bias ? (const void*)a.bias : a.W, a.bias ? (uint32_t)N * 2u : 0u);
  // one item per thread: 8 consecutive outputs of one row
  static_assert(BM * (BN / 8) == kMidWaves * 64, "one output item per thread");
  {
    const int row = tid / (BN / 8), cg = tid % (BN / 8);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
#pragma unroll
    for (int w = 0; w < kMidWaves; ++w) {
      const float* p = part + (w * BM + row) * kMidPW + 8 * cg;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(p), hi = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] += lo[e];
        v[4 + e] += hi[e];
      }
    }
    const int m = m0 + row, nn = n0 + 8 * cg;
    const u32x4 bb = bload128(Br, (uint32_t)nn * 2u);  // zero past N and without bias
    f32x4 cs0 = f32x4{1.f, 1.f, 1.f, 1.f}, cs1 = cs0;
    if constexpr (F == KF_FP8) {  // E4M3 row scales
      cs0 = __builtin_bit_cast(f32x4, bload128(Sr, (uint32_t)nn * 4u));
      cs1 = __builtin_bit_cast(f32x4, bload128(Sr, (uint32_t)nn * 4u + 16u));
    }
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float y0 = v[2 * p], y1 = v[2 * p + 1];
      if constexpr (F == KF_FP8) {
        y0 = y0 * (p < 2 ? cs0[2 * p] : cs1[2 * p - 4]);
        y1 = y1 * (p < 2 ? cs0[2 * p + 1] : cs1[2 * p - 3]);
      } else if constexpr (F == KF_NVFP4) {
        y0 = y0 * gscale;
        y1 = y1 * gscale;
      }
      const float b0 = bitsf(bb[p] << 16), b1 = bitsf(bb[p] & 0xFFFF0000u);
      o[p] = (uint32_t)f32_to_bf16(y0 + b0) | ((uint32_t)f32_to_bf16(y1 + b1) << 16);
    }
    if (m < M) {
      if (nn + 8 <= N && (N & 7) == 0) {
        __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<u32x4*>(a.Y + (int64_t)m * N + nn));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (nn + e < N) a.Y[(int64_t)m * N + nn + e] = (uint16_t)(o[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

template <int F, int WL, int NBMAX>
hipError_t launch_mid_nb(const LinearArgs& a, hipStream_t s) {
  constexpr int ring = kMidWaves * kMidSlot;
  constexpr int part = kMidWaves * kMidBM * kMidPW * 4;
  constexpr int sm = ring > part ? ring : part;
  static_assert(sm <= 160 * 1024, "exceeds the LDS of a CU");
  static std::atomic<int> done{0};
  auto k = k_gemm_mid<F, WL, NBMAX>;
  hipError_t e = allow_smem(k, sm, done);
  if (e != hipSuccess) return e;
  k<<<dim3((a.N + kMidBN - 1) / kMidBN, (a.M + kMidBM - 1) / kMidBM), kMidWaves * 64, sm, s>>>(a);
  return hipGetLastError();
}

template <int F, int WL>
hipError_t launch_mid_f(const LinearArgs& a, hipStream_t s) {
  const int nb = (a.K / 128 + kMidWaves - 1) / kMidWaves;
  if (nb <= 4) return launch_mid_nb<F, WL, 4>(a, s);
  if (nb <= 8) return launch_mid_nb<F, WL, 8>(a, s);
  if (nb <= 16) return launch_mid_nb<F, WL, 16>(a, s);
  return hipErrorInvalidValue;  // the plan keeps K <= kMidMaxK
}

template <int F>
hipError_t launch_mid_fl(const LinearArgs& a, hipStream_t s) {
  if (a.wl == kLayoutTiles) return launch_mid_f<F, kLayoutTiles>(a, s);
  return launch_mid_f<F, kLayoutRows>(a, s);
}

}  // namespace

hipError_t launch_gemm_mid(int kfmt, const LinearArgs& a, hipStream_t s) {
  if (a.K % 128 != 0 || a.K > kMidMaxK) return hipErrorInvalidValue;
  switch (kfmt) {
    case KF_INT4: return launch_mid_fl<KF_INT4>(a, s);
    case KF_INT4A: return launch_mid_fl<KF_INT4A>(a, s);
    case KF_FP8: return launch_mid_fl<KF_FP8>(a, s);
    case KF_NVFP4: return launch_mid_fl<KF_NVFP4>(a, s);
    case KF_MXFP4: return launch_mid_fl<KF_MXFP4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wq
