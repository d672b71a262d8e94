// GEMMs on the gfx950 scaled matrix cores (v_mfma_scale_f32_*_f8f6f4):
//  * the MXFP4 dynamic-activation x MXFP4-weight Linear (below);
//  * the static-FP8 (E4M3 x E4M3) GEMM for larger M, with unit block scales
//    ("TorchAO Static FP8 Quantization (Linear)": after Q/DQ fusion the GEMM
//    runs in FP8), further down.
//
// "TorchAO MXFP4 Dynamic Activation + MX Weight (Linear)", intro: the weights
// are MXFP4 (E2M1 codes, E8M0 scale per 32 K); the activations are quantized
// to MX on every call, and on hardware with MXFP4 matrix units the GEMM
// multiplies the two MX operands directly.  Here the activations get the same
// MXFP4 rule as the weights, and v_mfma_scale_f32_16x16x128_f8f6f4 takes both
// E2M1 operands and their E8M0 block scales as they are stored: no decode.
//
// Operand layout (checked on the device against a host model): in one
// 16x16x128 MFMA, lane (g, c) supplies 16 bytes = 32 E2M1 codes of row c (A)
// or column c (B), K 32g .. 32g+31 of the step, low nibble first, plus the
// E8M0 scale of exactly that 32-element block; the result D[4g + r][c] lands
// in element r of lane (g, c).  A packed row of K/2 bytes and its [K/32]
// scale row therefore feed the MFMA with one 16-byte and one 1-byte load per
// lane and step.
#include "wq_kernel_common.hpp"

namespace wq {

namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x4 mfma_mx4(u32x4 a, uint32_t sa, u32x4 b, uint32_t sb, f32x4 c) {
  const i32x8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const i32x8 bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // cbsz = blgp = 4: both operands E2M1; byte 0 of each scale register
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// E4M3 x E4M3 on the same instruction (cbsz = blgp = 0): lane (g, c) supplies
// 32 codes of row/column c, K 32g .. 32g+31 (byte j of the 32 = K 32g + j),
// both block scales 2^0 (code 127).  A device probe confirmed the layout
// against a host model.
__device__ __forceinline__ f32x4 mfma_f8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// ---------------------------------------------------------------- activation quantizer
// One thread per 32-element block of a row: the block's max |x| sets
// e = floor(log2 amax) - 2 (from the bf16 exponent field; zero and subnormal
// maxima give the clamp value -127), scale code e + 127, and the codes are
// E2M1(x * 2^-e) -- an exact power-of-two product -- converted with
// v_cvt_scalef32_pk_fp4_f32 (nearest even, saturating at 6, sign kept:
// checked against the reference encoder on the device).  The 32 codes are
// stored packed (element 2j in the low nibble of byte j).
__global__ __launch_bounds__(256) void k_mx_quant_act(const uint16_t* __restrict__ X, uint32_t nblk,
                                                      uint8_t* __restrict__ Xq, uint8_t* __restrict__ Xs) {
  const uint32_t blk = blockIdx.x * 256u + threadIdx.x;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(X, nblk * 64u);
  u32x4 v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = bload128(r, blk * 64u + 16u * q);
  uint32_t amax = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = v[q][w] & 0x7FFFu, hi = (v[q][w] >> 16) & 0x7FFFu;
      amax = max(amax, max(lo, hi));
    }
  const int E = (int)(amax >> 7);
  const int e = max(E - 129, -127);  // zero, subnormal and [2^-126, 2^-125) maxima clamp to -127
  const float inv = bitsf((uint32_t)(127 - e) << 23);  // 2^-e, e in [-127, 125]
  // bf16 pair word -> two scaled fp32 values (element 2j in the low half)
#define WQ_LO(u) (bitsf((u) << 16) * inv)
#define WQ_HI(u) (bitsf((u) & 0xFFFF0000u) * inv)
  u32x4 out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t word = 0;
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, WQ_LO(v[q].x), WQ_HI(v[q].x), 1.0f, 0);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, WQ_LO(v[q].y), WQ_HI(v[q].y), 1.0f, 1);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, WQ_LO(v[q].z), WQ_HI(v[q].z), 1.0f, 2);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, WQ_LO(v[q].w), WQ_HI(v[q].w), 1.0f, 3);
    out[q] = word;
  }
#undef WQ_LO
#undef WQ_HI
  if (blk < nblk) {
    *reinterpret_cast<u32x4*>(Xq + (size_t)blk * 16) = out;
    Xs[blk] = (uint8_t)(e + 127);
  }
}

// ---------------------------------------------------------------- small-M GEMM
// One workgroup = 12 waves = 16 output columns x 16*MT rows x all of K; wave w
// owns 128-K steps w*SPW .. w*SPW+SPW-1 (+ 12*SPW per pass).  Every load of a
// pass (packed weight, weight scales, packed activations, activation scales)
// is issued before the first MFMA; out-of-range offsets read zero codes and
// zero scale bytes, whose products are zero.  Wave partials are reduced
// through LDS as in the bf16 kernel.
// DW (K % 128 == 0): the block scales load as one aligned dword per lane
// (the step's four E8M0 bytes of the row) and lane group g shifts its byte
// down; a byte load per lane costs the address unit as much as a 16-byte one.
template <int MT, int WL, bool DW>
__global__ __launch_bounds__(768) void k_mx_linear(LinearArgs a) {
  constexpr int NW = 12, SPW = 2, NT = 16;
  constexpr int E = MT * 16 * NT;
  __shared__ __attribute__((aligned(16))) float red[NW * E];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int n0 = blockIdx.x * NT, m0 = blockIdx.z * (16 * MT);
  const int M = a.M, N = a.N, K = a.K;
  const int T = (K + 127) / 128;
  const uint32_t rowb = (uint32_t)K / 2u, srow = (uint32_t)K / 32u;
  const __amdgpu_buffer_rsrc_t Wr = make_rsrc(a.W, (uint32_t)N * rowb);
  const __amdgpu_buffer_rsrc_t Wsr = make_rsrc(a.scales, (uint32_t)N * srow);
  const __amdgpu_buffer_rsrc_t Xr = make_rsrc(a.X, (uint32_t)M * rowb);
  const __amdgpu_buffer_rsrc_t Xsr = make_rsrc(a.xscales, (uint32_t)M * srow);
  const __amdgpu_buffer_rsrc_t Br = make_rsrc(a.bias ? (const void*)a.bias : a.W, a.bias ? (uint32_t)N * 2u : 0u);
  const int ecol = tid % NT, en = n0 + ecol;
  const uint32_t bias_bits = bload16(Br, (uint32_t)en * 2u);

  f32x4 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s0 = wave * SPW; s0 < T; s0 += NW * SPW) {
    u32x4 w[SPW], x[SPW][MT];
    uint32_t ws[SPW], xs[SPW][MT];
#pragma unroll
    for (int st = 0; st < SPW; ++st) {
      const int k = (s0 + st) * 128 + 32 * g;  // first K of this lane's block
      const bool kv = k < K;
      const uint32_t n = (uint32_t)(n0 + c);
      w[st] = bload128(Wr, off_if(kv, w_off<WL>(n, (uint32_t)k / 2u, rowb)));
      const uint32_t wso = s_off<KF_MXFP4, WL>(n, (uint32_t)k, (uint32_t)K);
      if constexpr (DW) ws[st] = bload32(Wsr, off_if(kv, wso & ~3u));
      else ws[st] = bload8(Wsr, off_if(kv, wso));
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const uint32_t m = (uint32_t)(m0 + 16 * i + c);
        x[st][i] = bload128(Xr, off_if(kv, m * rowb + (uint32_t)k / 2u));
        const uint32_t xso = m * srow + (uint32_t)k / 32u;
        if constexpr (DW) xs[st][i] = bload32(Xsr, off_if(kv, xso & ~3u));
        else xs[st][i] = bload8(Xsr, off_if(kv, xso));
      }
    }
    const uint32_t sh = DW ? 8u * (uint32_t)g : 0u;  // byte g of the dword: K block 32g of the step
#pragma unroll
    for (int st = 0; st < SPW; ++st)
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[i] = mfma_mx4(x[st][i], xs[st][i] >> sh, w[st], ws[st] >> sh, acc[i]);
  }

  // wave partials -> LDS, one barrier, per-thread sums in wave order
#pragma unroll
  for (int i = 0; i < MT; ++i) *reinterpret_cast<f32x4*>(red + ((wave * MT + i) * 64 + lane) * 4) = acc[i];
  __syncthreads();
  if (tid < E) {
    const int row = tid / NT, col = tid % NT;
    const int idx = ((row >> 4) * 64 + 16 * ((row >> 2) & 3) + col) * 4 + (row & 3);
    float v = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) v += red[w2 * E + idx];
    const int m = m0 + row;
    if (m < M && en < N) a.Y[(int64_t)m * N + en] = f32_to_bf16(v + bitsf(bias_bits << 16));
  }
}

// ---------------------------------------------------------------- mid-M GEMM
// One workgroup of 8 waves owns a 64 x 64 output tile and its waves split K:
// wave w takes the 128-K blocks w, w + 8, ... and accumulates all 16 of the
// tile's 16 x 16 outputs for them, so the waves meet only twice: once when
// the activations are in LDS and once for the reduction at the end.
//  * The workgroup's 64 packed activation rows (all of K) and the block scales
//    of its rows and columns go from memory straight into LDS (buffer_load
//    ... lds), 64 lanes x 16 bytes per instruction: every instruction reads
//    whole 128-byte lines.  Loaded in the MFMA operand layout instead, each
//    instruction would touch 16 rows for 64 bytes each, and each scale dword
//    load 16 lines for 4 bytes each; those requests, not the bytes, bound
//    that form (10.6 us at M = 256, N = 4096, K = 3072, the same as the
//    64 x 64 LDS-tiled kernel; 8.0 us without the scale loads, 7.8 us without
//    the activation loads, 10.6 us without the MFMAs).
//  * The packed weights of the wave's blocks are loaded into registers up
//    front: lane (g, c) takes the 16 bytes of column c at K 32g .. 32g+31 of
//    the block (in tile order one instruction reads one whole 1 KiB tile).
//  * Activation rows in LDS keep the memory order of their 16-byte chunks
//    except for an XOR of chunk bits 1-3 with row bits 0-2: the operand reads
//    of rows c = 0..7 by lane groups g and g + 1 (one ds_read_b128 cycle) then
//    hit 16 distinct bank groups.  Needs K % 512 == 0 (16-chunk row groups).
// Rows past M, columns past N read zeros.  K % 512 == 0, K <= kMxMidMaxK,
// 4-byte aligned scale arrays.
constexpr int kMxMidWaves = 8, kMxMidT = 64, kMxMidPW = kMxMidT + 4;
constexpr int kMxMidMaxK = 4096;
constexpr int kMxMidNB = kMxMidMaxK / 128 / kMxMidWaves;  // blocks per wave at most
constexpr int kMxMidXBytes = kMxMidT * kMxMidMaxK / 2;     // activation rows
constexpr int kMxMidSBytes = kMxMidT * kMxMidMaxK / 32;    // one scale plane
constexpr int kMxMidPart = kMxMidWaves * kMxMidT * kMxMidPW * 4;
constexpr int kMxMidSmem = (kMxMidXBytes + 2 * kMxMidSBytes) > kMxMidPart ? (kMxMidXBytes + 2 * kMxMidSBytes) : kMxMidPart;

__device__ __forceinline__ uint32_t mx_mid_swz(uint32_t row, uint32_t chunk) { return chunk ^ ((row & 7u) << 1); }

// copy `bytes` (a multiple of 16) from r at `src` to LDS at `dst`, 16 bytes
// per lane, the workgroup's 512 lanes in turn; chunks past the resource read zero
__device__ __forceinline__ void mx_mid_copy(unsigned char* dst, __amdgpu_buffer_rsrc_t r, uint32_t src, uint32_t bytes,
                                            int wave, int lane) {
  for (uint32_t p = (uint32_t)wave * 64u; p < bytes / 16u; p += kMxMidWaves * 64u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + p * 16u), 16,
                                             src + (p + (uint32_t)lane) * 16u, 0, 0, 0);
}

template <int WL, int NB>
__global__ __launch_bounds__(kMxMidWaves * 64) void k_mx_mid(LinearArgs a) {
  constexpr int T = kMxMidT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int M = a.M, N = a.N, K = a.K;
  const int n0 = blockIdx.x * T, m0 = blockIdx.y * T;
  const int KT = K / 128;
  const uint32_t rowb = (uint32_t)K / 2u, srow = (uint32_t)K / 32u, C = rowb / 16u;  // C: chunks per row
  const __amdgpu_buffer_rsrc_t Wr = make_rsrc(a.W, (uint32_t)N * rowb);
  const __amdgpu_buffer_rsrc_t Wsr = make_rsrc(a.scales, (uint32_t)N * srow);
  const __amdgpu_buffer_rsrc_t Xr = make_rsrc(a.X, (uint32_t)M * rowb);
  const __amdgpu_buffer_rsrc_t Xsr = make_rsrc(a.xscales, (uint32_t)M * srow);
  unsigned char* xl = smem;                       // [64][K/2] activation rows, swizzled chunks
  unsigned char* xsl = smem + 64 * rowb;          // [64][K/32] activation block scales
  unsigned char* wsl = xsl + 64 * srow;           // the weight block scales of the 64 columns

  // weights of this wave's blocks into registers
  u32x4 w[NB][4];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int kb = wave + j * kMxMidWaves;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      w[j][t] = bload128(Wr, off_if(kb < KT, w_off<WL>((uint32_t)(n0 + 16 * t + c), (uint32_t)(kb * 64 + 16 * g), rowb)));
  }
  // activation rows: LDS chunk p = row * C + k holds memory chunk k ^ swz of that row
  {
    const uint32_t step = kMxMidWaves * 64u, dq = step / C, dr = step % C;  // C is a multiple of 16, <= 128
    uint32_t p = (uint32_t)wave * 64u + (uint32_t)lane;
    uint32_t row = p / C, k = p % C;
    for (uint32_t p0 = (uint32_t)wave * 64u; p0 < 64u * C; p0 += step) {
      const uint32_t src = (((uint32_t)m0 + row) * C + mx_mid_swz(row, k)) * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Xr, (__attribute__((address_space(3))) void*)(xl + p0 * 16u), 16, src, 0, 0, 0);
      row += dq;
      k += dr;
      if (k >= C) {
        k -= C;
        ++row;
      }
    }
  }
  // block scales: the 64 activation rows are contiguous, and so are the 64
  // columns' weight scales in either layout
  mx_mid_copy(xsl, Xsr, (uint32_t)m0 * srow, 64u * srow, wave, lane);
  mx_mid_copy(wsl, Wsr, WL == kLayoutTiles ? (uint32_t)(n0 / 16) * (uint32_t)KT * 64u : (uint32_t)n0 * srow, 64u * srow, wave,
              lane);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's loads, LDS ones included
  __syncthreads();

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t sh = 8u * (uint32_t)g;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int kb = wave + j * kMxMidWaves;
    if (kb >= KT) break;  // wave-uniform
    u32x4 x[4];
    uint32_t xs[4], ws[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t row = (uint32_t)(16 * i + c);
      x[i] = *reinterpret_cast<const u32x4*>(xl + (row * C + mx_mid_swz(row, (uint32_t)(4 * kb + g))) * 16u);
      xs[i] = *reinterpret_cast<const uint32_t*>(xsl + row * srow + 4u * (uint32_t)kb);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t so = WL == kLayoutTiles ? (((uint32_t)t * (uint32_t)KT + (uint32_t)kb) * 16u + (uint32_t)c) * 4u
                                             : (uint32_t)(16 * t + c) * srow + 4u * (uint32_t)kb;
      ws[t] = *reinterpret_cast<const uint32_t*>(wsl + so);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[i][t] = mfma_mx4(x[i], xs[i] >> sh, w[j][t], ws[t] >> sh, acc[i][t]);
  }
  __syncthreads();  // every wave is done with the operands in LDS

  // partials of wave w: rows w * 64 .. w * 64 + 63 (stride kMxMidPW floats)
  float* part = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[(wave * T + 16 * i + 4 * g + r) * kMxMidPW + 16 * t + c] = acc[i][t][r];
  __syncthreads();

  const __amdgpu_buffer_rsrc_t Br = make_rsrc(a.bias ? (const void*)a.bias : a.W, a.bias ? (uint32_t)N * 2u : 0u);
  // one item per thread: 8 consecutive outputs of one row, wave partials summed in wave order
  static_assert(T * (T / 8) == kMxMidWaves * 64, "one output item per thread");
  const int row = tid / (T / 8), cg = tid % (T / 8);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < kMxMidWaves; ++w2) {
    const float* pp = part + (w2 * T + row) * kMxMidPW + 8 * cg;
    const f32x4 lo = *reinterpret_cast<const f32x4*>(pp), hi = *reinterpret_cast<const f32x4*>(pp + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] += lo[e];
      v[4 + e] += hi[e];
    }
  }
  const int m = m0 + row, nn = n0 + 8 * cg;
  const u32x4 bb = bload128(Br, (uint32_t)nn * 2u);  // zero past N and without bias
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float b0 = bitsf(bb[q] << 16), b1 = bitsf(bb[q] & 0xFFFF0000u);
    o[q] = (uint32_t)f32_to_bf16(v[2 * q] + b0) | ((uint32_t)f32_to_bf16(v[2 * q + 1] + b1) << 16);
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

template <int WL, int NB>
hipError_t launch_mx_mid_nb(const LinearArgs& a, hipStream_t s) {
  static_assert(kMxMidSmem <= 160 * 1024, "exceeds the LDS of a CU");
  static std::atomic<int> done{0};
  auto k = k_mx_mid<WL, NB>;
  hipError_t e = allow_smem(k, kMxMidSmem, done);
  if (e != hipSuccess) return e;
  k<<<dim3((a.N + kMxMidT - 1) / kMxMidT, (a.M + kMxMidT - 1) / kMxMidT), kMxMidWaves * 64, kMxMidSmem, s>>>(a);
  return hipGetLastError();
}

template <int WL>
hipError_t launch_mx_mid(const LinearArgs& a, hipStream_t s) {
  const int nb = (a.K / 128 + kMxMidWaves - 1) / kMxMidWaves;
  if (nb <= 2) return launch_mx_mid_nb<WL, 2>(a, s);
  if (nb <= 3) return launch_mx_mid_nb<WL, 3>(a, s);
  return launch_mx_mid_nb<WL, kMxMidNB>(a, s);
}

// ---------------------------------------------------------------- small-M GEMM, activations through LDS
// k_mx_linear's workgroup (12 waves, 16 columns x 16*MT rows x all of K, wave
// w taking the 128-K steps 2w, 2w + 1, 2w + 24, ...) with its activations
// copied into LDS first: the 16*MT packed rows (all of K) and their block
// scale rows go from memory straight into LDS as whole 128-byte lines
// (buffer_load ... lds, chunks swizzled as in the mid-M kernel), instead of
// 16 rows x 64 bytes and 16 rows x 4 bytes per instruction.  Each wave loads
// its steps' packed weights and weight scale dwords into registers up front,
// waits at one barrier and runs its MFMAs from LDS and registers.  NS: steps
// per wave at most (2 per 24-step pass).  K % 512 == 0, K <= kMxSmallMaxK.
constexpr int kMxSmallMaxK = 8192;

template <int MT, int WL, int NS>
__global__ __launch_bounds__(768) void k_mx_small(LinearArgs a) {
  constexpr int NW = 12, NT = 16, R = 16 * MT;
  constexpr int E = MT * 16 * NT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int n0 = blockIdx.x * NT, m0 = blockIdx.z * R;
  const int M = a.M, N = a.N, K = a.K;
  const int T = K / 128;
  const uint32_t rowb = (uint32_t)K / 2u, srow = (uint32_t)K / 32u, C = rowb / 16u;
  const __amdgpu_buffer_rsrc_t Wr = make_rsrc(a.W, (uint32_t)N * rowb);
  const __amdgpu_buffer_rsrc_t Wsr = make_rsrc(a.scales, (uint32_t)N * srow);
  const __amdgpu_buffer_rsrc_t Xr = make_rsrc(a.X, (uint32_t)M * rowb);
  const __amdgpu_buffer_rsrc_t Xsr = make_rsrc(a.xscales, (uint32_t)M * srow);
  const __amdgpu_buffer_rsrc_t Br = make_rsrc(a.bias ? (const void*)a.bias : a.W, a.bias ? (uint32_t)N * 2u : 0u);
  const int en = n0 + tid % NT;
  const uint32_t bias_bits = bload16(Br, (uint32_t)en * 2u);
  unsigned char* xl = smem;                       // [R][K/2] activation rows, swizzled chunks
  unsigned char* xsl = smem + R * rowb;           // [R][K/32] activation block scales
  auto step_of = [&](int j) { return 2 * wave + (j & 1) + (j >> 1) * (2 * NW); };

  // this wave's packed weights and weight scale dwords
  const uint32_t n = (uint32_t)(n0 + c);
  u32x4 w[NS];
  uint32_t ws[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int st = step_of(j);
    const bool ok = st < T;
    w[j] = bload128(Wr, off_if(ok, w_off<WL>(n, (uint32_t)(st * 64 + 16 * g), rowb)));
    ws[j] = bload32(Wsr, off_if(ok, s_off<KF_MXFP4, WL>(n, (uint32_t)(st * 128), (uint32_t)K)));
  }
  // activation rows: LDS chunk p = row * C + k holds memory chunk k ^ swz of that row
  {
    const uint32_t step = NW * 64u, dq = step / C, dr = step % C;
    uint32_t p = (uint32_t)wave * 64u + (uint32_t)lane;
    uint32_t row = p / C, k = p % C;
    for (uint32_t p0 = (uint32_t)wave * 64u; p0 < (uint32_t)R * C; p0 += step) {
      const uint32_t src = (((uint32_t)m0 + row) * C + mx_mid_swz(row, k)) * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Xr, (__attribute__((address_space(3))) void*)(xl + p0 * 16u), 16, src, 0, 0, 0);
      row += dq;
      k += dr;
      if (k >= C) {
        k -= C;
        ++row;
      }
    }
  }
  // the rows' block scales (contiguous); the LDS region is rounded up to whole
  // 1 KiB instructions
  for (uint32_t p0 = (uint32_t)wave * 64u; p0 * 16u < (uint32_t)R * srow; p0 += NW * 64u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(Xsr, (__attribute__((address_space(3))) void*)(xsl + p0 * 16u), 16,
                                             (uint32_t)m0 * srow + (p0 + (uint32_t)lane) * 16u, 0, 0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's loads, LDS ones included
  __syncthreads();

  f32x4 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t sh = 8u * (uint32_t)g;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int st = step_of(j);
    if (st >= T) break;  // wave-uniform; steps grow with j
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const uint32_t row = (uint32_t)(16 * i + c);
      const u32x4 x = *reinterpret_cast<const u32x4*>(xl + (row * C + mx_mid_swz(row, (uint32_t)(4 * st + g))) * 16u);
      const uint32_t xs = *reinterpret_cast<const uint32_t*>(xsl + row * srow + 4u * (uint32_t)st);
      acc[i] = mfma_mx4(x, xs >> sh, w[j], ws[j] >> sh, acc[i]);
    }
  }
  __syncthreads();  // the partials reuse the activation rows' LDS

  // wave partials -> LDS, one barrier, per-thread sums in wave order
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < MT; ++i) *reinterpret_cast<f32x4*>(red + ((wave * MT + i) * 64 + lane) * 4) = acc[i];
  __syncthreads();
  if (tid < E) {
    const int row = tid / NT, col = tid % NT;
    const int idx = ((row >> 4) * 64 + 16 * ((row >> 2) & 3) + col) * 4 + (row & 3);
    float v = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) v += red[w2 * E + idx];
    const int m = m0 + row;
    if (m < M && en < N) a.Y[(int64_t)m * N + en] = f32_to_bf16(v + bitsf(bias_bits << 16));
  }
}

// LDS bytes of k_mx_small: activation rows plus scale rows (rounded up to
// 1 KiB), or the wave partials if larger
__host__ __device__ constexpr int mx_small_smem(int MT, int K) {
  const int rows = 16 * MT * K / 2 + (16 * MT * K / 32 + 1023) / 1024 * 1024;
  const int red = 12 * MT * 16 * 16 * 4;
  return rows > red ? rows : red;
}

template <int MT, int WL, int NS>
hipError_t launch_mx_small_ns(const LinearArgs& a, hipStream_t s) {
  static_assert(mx_small_smem(MT, kMxSmallMaxK) <= 160 * 1024, "exceeds the LDS of a CU");
  static std::atomic<int> done{0};
  auto k = k_mx_small<MT, WL, NS>;
  hipError_t e = allow_smem(k, mx_small_smem(MT, kMxSmallMaxK), done);
  if (e != hipSuccess) return e;
  k<<<dim3((a.N + 15) / 16, 1, (a.M + 16 * MT - 1) / (16 * MT)), 768, mx_small_smem(MT, a.K), s>>>(a);
  return hipGetLastError();
}

template <int MT, int WL>
hipError_t launch_mx_small(const LinearArgs& a, hipStream_t s) {
  const int passes = (a.K / 128 + 23) / 24;
  if (passes <= 1) return launch_mx_small_ns<MT, WL, 2>(a, s);
  if (passes <= 2) return launch_mx_small_ns<MT, WL, 4>(a, s);
  return launch_mx_small_ns<MT, WL, 6>(a, s);  // K <= 8192: 64 steps
}

// ---------------------------------------------------------------- tiled GEMM (larger M)
// One workgroup (4 waves, 2 x 2) computes a BM x BN tile; K advances 128 per
// step (one scaled MFMA deep).  Per step every thread loads its share of the
// packed activation and weight tiles (16-byte chunks, 64 bytes per row) one
// step ahead and stores them to a double-buffered LDS tile as they are:
// nothing is decoded.  Each wave then reads 16-byte operand chunks and scale
// bytes from LDS and issues (BM/32) x (BN/32) MFMAs.  LDS rows hold their four
// 16-byte chunks XOR-swizzled with row bits 1-2, which keeps both the operand
// reads and the row writes free of bank conflicts.
//
// Scales: with PRE, the workgroup copies its BM activation and BN weight
// scale rows (K/32 bytes each, contiguous in memory) into LDS once, with
// 16-byte loads, before the K loop.  Without PRE (scale rows not 16-byte
// multiples, or too long for LDS) every step loads 4 scale bytes per row;
// those loads touch a different row per lane and were measured to dominate
// the step time when they are used.
template <int BM, int BN, int GT, bool F8>
struct MxTile {
  static constexpr int ROWB = F8 ? 128 : 64;            // operand bytes of one row per step
  static constexpr int CPR = ROWB / 16;                 // 16-byte chunks per row and step
  static constexpr int KPC = F8 ? 16 : 32;              // K elements per chunk
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  static constexpr int AS_BYTES = F8 ? 0 : BM * 4, BS_BYTES = F8 ? 0 : BN * 4;  // per-step scale planes (no PRE)
  static constexpr int BUF = A_BYTES + B_BYTES + AS_BYTES + BS_BYTES;
  static constexpr int TILES = 2 * BUF;
  static constexpr int NA = BM * CPR / GT, NB = BN * CPR / GT;  // 16-byte chunks per thread
  // LDS slot of chunk k of row r.  A ds_read_b128 serves lanes 0-7 with
  // 16-23 (8-15 with 24-31, ...) together: the 16 reads of rows c = 0..7 by
  // lane groups g and g+1 must hit distinct 16-byte bank groups of the row
  // window they fall in.  E2M1 rows (64 bytes, lane reads chunk g): XOR with
  // row bits 1-2.  E4M3 rows (128 bytes, lane reads chunks 2g and 2g+1): XOR
  // with row bits 1 and 2 as 1 and 4.  Whole-row writes are conflict-free
  // under any XOR.
  __device__ static __forceinline__ int pos(int r, int k) {
    return F8 ? (k ^ (((r >> 1) & 1) | (r & 4))) : (k ^ ((r >> 1) & 3));
  }
  // LDS for the whole-K scale rows (PRE)
  static size_t pre_bytes(int K) { return (size_t)(BM + BN) * (size_t)(K / 32); }
};

// WGN waves along N (2 x WGN wave grid, GT = 128 * WGN threads); each wave
// owns a (BM/2) x (BN/WGN) block.  F8: E4M3 operands (static FP8 path): 128
// bytes per row and step, no block scales (the MFMA takes 2^0 for both), the
// epilogue applies act_scale * w_scale[n].
template <int BM, int BN, int WGN, bool PRE, bool F8, int WL>
__global__ __launch_bounds__(128 * WGN) void k_mx_gemm_tiled(LinearArgs a) {
  constexpr int GT = 128 * WGN, WBN = BN / WGN;
  using TT = MxTile<BM, BN, GT, F8>;
  constexpr int TM = BM / 32, TN = WBN / 16;
  constexpr int CPR = TT::CPR;
  static_assert(!(PRE && F8), "E4M3 operands have no block scales");
  static_assert(TT::NA >= 1 && TT::NB >= 1 && TT::NA * GT == BM * CPR && TT::NB * GT == BN * CPR,
                "tile rows must split evenly over the threads");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave / WGN, wn = wave % WGN;
  const int M = a.M, N = a.N, K = a.K;

  // XCD-aware tile order (see the bf16 tiled kernel)
  const int gx = gridDim.x, G = gx * gridDim.y;
  int b = blockIdx.y * gx + blockIdx.x;
  if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
  const int n0 = (b % gx) * BN, m0 = (b / gx) * BM;

  const uint32_t rowb = F8 ? (uint32_t)K : (uint32_t)K / 2u, srow = (uint32_t)K / 32u;
  const __amdgpu_buffer_rsrc_t Xr = make_rsrc(a.X, (uint32_t)M * rowb);
  const __amdgpu_buffer_rsrc_t Wr = make_rsrc(a.W, (uint32_t)N * rowb);
  const __amdgpu_buffer_rsrc_t Xsr = make_rsrc(F8 ? a.X : (const void*)a.xscales, F8 ? 0u : (uint32_t)M * srow);
  const __amdgpu_buffer_rsrc_t Wsr = make_rsrc(a.scales, F8 ? (uint32_t)N * 4u : (uint32_t)N * srow);
  const __amdgpu_buffer_rsrc_t Br = make_rsrc(a.bias ? (const void*)a.bias : a.W, a.bias ? (uint32_t)N * 2u : 0u);
  const int KT = (K + 127) / 128;
  unsigned char* XS = smem + TT::TILES;    // PRE: [BM][srow] activation scale rows
  unsigned char* WS = XS + BM * srow;      //      [BN][srow] weight scale rows

  if constexpr (PRE) {
    // rows m0 .. m0+BM-1 of the scale matrix are one contiguous byte range
    // (in tile order too: a 16-row group's scales are consecutive); 16-byte
    // chunks, rows past M / N read zero
    const int xchunks = BM * (int)srow / 16, wchunks = BN * (int)srow / 16;
    for (int q = tid; q < xchunks; q += GT)
      *reinterpret_cast<u32x4*>(XS + 16 * q) = bload128(Xsr, (uint32_t)m0 * srow + 16u * q);
    for (int q = tid; q < wchunks; q += GT)
      *reinterpret_cast<u32x4*>(WS + 16 * q) = bload128(Wsr, (uint32_t)n0 * srow + 16u * q);
  }

  // loads of one step: chunk q of this thread is row (q*GT + tid) / CPR, part % CPR
  u32x4 xa[2][TT::NA], wb[2][TT::NB];
  uint32_t xsb[2][4], wsb[2][4];  // raw scale bytes (MX without PRE)
  auto gload = [&](int kt, int st) {
    const uint32_t kb = (uint32_t)kt * (uint32_t)TT::ROWB;  // byte offset of the step in a row
#pragma unroll
    for (int q = 0; q < TT::NA; ++q) {
      const int id = q * GT + tid, row = id / CPR, part = id % CPR;
      const bool ok = kt * 128 + part * TT::KPC < K;
      xa[st][q] = bload128(Xr, off_if(ok, (uint32_t)(m0 + row) * rowb + kb + 16u * part));
    }
#pragma unroll
    for (int q = 0; q < TT::NB; ++q) {
      const int id = q * GT + tid, row = id / CPR, part = id % CPR;
      const bool ok = kt * 128 + part * TT::KPC < K;
      wb[st][q] = bload128(Wr, off_if(ok, w_off<WL>((uint32_t)(n0 + row), kb + 16u * part, rowb)));
    }
    if constexpr (!PRE && !F8) {
      // thread t reads the step's 4 scale bytes of activation row t % BM and
      // weight row t % BN (threads past the row count repeat a row, so no
      // thread needs a branch); bytes past K read zero
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool okj = kt * 128 + 32 * j < K;
        xsb[st][j] = bload8(Xsr, off_if(okj, (uint32_t)(m0 + tid % BM) * srow + (uint32_t)kt * 4u + j));
        wsb[st][j] = bload8(Wsr, off_if(okj, s_off<KF_MXFP4, WL>((uint32_t)(n0 + tid % BN), (uint32_t)(kt * 128 + 32 * j),
                                                                   (uint32_t)K)));
      }
    }
  };
  auto lstore = [&](int buf, int st) {
    unsigned char* A = smem + buf * TT::BUF;
    unsigned char* B = A + TT::A_BYTES;
#pragma unroll
    for (int q = 0; q < TT::NA; ++q) {
      const int id = q * GT + tid, row = id / CPR, part = id % CPR;
      *reinterpret_cast<u32x4*>(A + row * TT::ROWB + TT::pos(row, part) * 16) = xa[st][q];
    }
#pragma unroll
    for (int q = 0; q < TT::NB; ++q) {
      const int id = q * GT + tid, row = id / CPR, part = id % CPR;
      *reinterpret_cast<u32x4*>(B + row * TT::ROWB + TT::pos(row, part) * 16) = wb[st][q];
    }
    if constexpr (!PRE && !F8) {
      // scale planes [block j][row]: byte stores straight from the loaded
      // registers, BM apart, so the compiler does not merge them into words
      // (which would make it wait for all four loads); repeated rows store
      // identical bytes
      unsigned char* AS = B + TT::B_BYTES;
      unsigned char* BS = AS + TT::AS_BYTES;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        AS[j * BM + tid % BM] = (unsigned char)xsb[st][j];
        BS[j * BN + tid % BN] = (unsigned char)wsb[st][j];
      }
    }
  };

  uint32_t bias_bits[TN], cs_bits[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const uint32_t n = (uint32_t)(n0 + wn * WBN + 16 * t + c);
    bias_bits[t] = bload16(Br, n * 2u);
    cs_bits[t] = F8 ? bload32(Wsr, n * 4u) : 0x3F800000u;
  }
  const float s1 = F8 ? a.act_scale[0] : 1.0f;

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf, int kt) {
    const unsigned char* A = smem + buf * TT::BUF;
    const unsigned char* B = A + TT::A_BYTES;
    if constexpr (F8) {
      // lane (g, c): row/column c, K 32g .. 32g+31 of the step = chunks 2g and
      // 2g+1 of the row
      i32x8 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * (BM / 2) + 16 * i + c;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(A + r * TT::ROWB + TT::pos(r, 2 * g) * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(A + r * TT::ROWB + TT::pos(r, 2 * g + 1) * 16);
        af[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int r = wn * WBN + 16 * t + c;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(B + r * TT::ROWB + TT::pos(r, 2 * g) * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(B + r * TT::ROWB + TT::pos(r, 2 * g + 1) * 16);
        bf[t] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[i][t] = mfma_f8(af[i], bf[t], acc[i][t]);
    } else {
      const unsigned char* AS = B + TT::B_BYTES;
      const unsigned char* BS = AS + TT::AS_BYTES;
      u32x4 af[TM], bf[TN];
      uint32_t as[TM], bs[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * (BM / 2) + 16 * i + c;
        af[i] = *reinterpret_cast<const u32x4*>(A + r * TT::ROWB + TT::pos(r, g) * 16);
        // blocks past K have zero codes; their scale is taken as 2^0
        as[i] = PRE ? ((4 * kt + g < (int)srow) ? XS[r * srow + min(4 * kt + g, (int)srow - 1)] : 127u) : AS[g * BM + r];
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int r = wn * WBN + 16 * t + c;
        bf[t] = *reinterpret_cast<const u32x4*>(B + r * TT::ROWB + TT::pos(r, g) * 16);
        // (tile order: the copied range holds each 16-row group's 128-K tiles
        // one after the other, 4 scale bytes per row and tile)
        const int wsi = (WL == kLayoutTiles) ? (((r >> 4) * ((int)srow >> 2) + min(kt, ((int)srow >> 2) - 1)) * 64 + (r & 15) * 4 + g)
                                             : r * srow + min(4 * kt + g, (int)srow - 1);
        bs[t] = PRE ? ((4 * kt + g < (int)srow) ? WS[wsi] : 127u) : BS[g * BN + r];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[i][t] = mfma_mx4(af[i], as[i], bf[t], bs[t], acc[i][t]);
    }
  };

  // two register stages, two LDS buffers; the step count is even so both
  // indices are compile-time constants in the unrolled pair (steps past K
  // read zero codes)
  const int KTP = (KT + 1) / 2 * 2;
  gload(0, 0);
  gload(1, 1);
  lstore(0, 0);
  gload(2, 0);
  __syncthreads();
  for (int kt = 0; kt < KTP; kt += 2) {
    compute(0, kt);
    lstore(1, 1);
    gload(kt + 3, 1);
    __syncthreads();
    compute(1, kt + 1);
    lstore(0, 0);
    gload(kt + 4, 0);
    __syncthreads();
  }

#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = n0 + wn * WBN + 16 * t + c;
    const float bias = bitsf(bias_bits[t] << 16), cs = bitsf(cs_bits[t]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * (BM / 2) + 16 * i + 4 * g + r;
        const float y = F8 ? (acc[i][t][r] * s1) * cs : acc[i][t][r];
        if (m < M && n < N) a.Y[(int64_t)m * N + n] = f32_to_bf16(y + bias);
      }
  }
}

// ---------------------------------------------------------------- static FP8, 256 x 256 tiles
// For large M x N: a workgroup of 16 waves (4 x 4 wave grid, 64 x 64 outputs
// per wave; 16 waves measured 7 % faster than 8 waves of 128 x 64) owns a
// 256 x 256 tile; K advances 128 per step on the E4M3 scaled MFMA.  Operand
// rows go from memory straight into LDS (buffer_load_dwordx4 ... lds writes
// lane i's 16 bytes at the wave's LDS base + 16 i): one load moves 8 whole
// 128-byte rows, and the bank swizzle is applied by choosing which 16-byte
// chunk of its row each lane reads.  Two LDS stages of 64 KiB.
// Per step a wave waits for its loads and meets the others at the one barrier
// of the step, issues the loads of the next step into the other stage, then
// reads its operands and runs its 16 MFMAs.
constexpr int kF8T = 256;                 // tile rows and columns
constexpr int kF8Stage = 2 * kF8T * 128;  // one LDS stage: A then B, 128 codes per row
constexpr int kF8Colv = (2 * kF8Stage > 16 * 64 * kTileRowBytes) ? 2 * kF8Stage : 16 * 64 * kTileRowBytes;
constexpr int kF8Smem = kF8Colv + kF8T * 8;  // stages or output tiles, then the column scales and biases

// LDS slot of 16-byte chunk k (0..7) of tile row r.  An operand read has lane
// (g, c) take chunks 2g and 2g+1 of row c; a ds_read_b128 serves lanes 0-7
// with 16-23 (and 8-15 with 24-31, ...) together, so rows 0..7 with chunks
// {0, 2} (or {1, 3}, {4, 6}, {5, 7}) must land on 16 distinct 16-byte bank
// groups: rows of one parity share a 256-byte bank window, and within it the
// XOR with row bits 1 and 2 (as 1 and 4) spreads the four rows' two chunks
// over all eight slots.
__device__ __forceinline__ int f8pos(int r, int k) { return k ^ (((r >> 1) & 1) | (r & 4)); }

constexpr int kF8Waves = 16;

template <int WL>
__global__ __launch_bounds__(kF8Waves * 64) void k_f8_gemm256(LinearArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // 16 x 16 tiles per wave (WBM x 64 outputs); the first half of the waves
  // loads activation rows, the second half weight rows, LROWS rows each, in
  // LJ loads of 8 rows per step
  constexpr int NW = kF8Waves, WBM = 1024 / NW, TM = WBM / 16, TN = 4;
  constexpr int HALF = NW / 2, LROWS = kF8T / HALF, LJ = LROWS / 8;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave >> 2, wn = wave & 3;  // NW/4 x 4 wave grid
  const int M = a.M, N = a.N, K = a.K;

  // XCD-aware tile order (see the bf16 tiled kernel)
  const int gx = gridDim.x, G = gx * gridDim.y;
  int b = blockIdx.y * gx + blockIdx.x;
  if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
  const int n0 = (b % gx) * kF8T, m0 = (b / gx) * kF8T;

  const __amdgpu_buffer_rsrc_t Xr = make_rsrc(a.X, (uint32_t)M * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t Wr = make_rsrc(a.W, (uint32_t)N * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t Sr = make_rsrc(a.scales, (uint32_t)N * 4u);
  const __amdgpu_buffer_rsrc_t Br = make_rsrc(a.bias ? (const void*)a.bias : a.W, a.bias ? (uint32_t)N * 2u : 0u);
  const int KT = (K + 127) / 128;

  // wave w < HALF loads activation rows LROWS*w .., wave w >= HALF weight rows
  // LROWS*(w-HALF) ..; load j covers rows +8j .. +8j+7, lane L fills LDS slot
  // L % 8 of row L / 8 with the chunk stored there (the slot map is its own
  // inverse); chunks past K and rows past M / N read zero
  const bool loadA = wave < HALF;
  const __amdgpu_buffer_rsrc_t Lr = loadA ? Xr : Wr;
  const int lrow0 = LROWS * (wave % HALF);
  const uint32_t lbase = (uint32_t)((loadA ? m0 : n0) + lrow0);
  auto issue = [&](int kt, int st) {
    unsigned char* dst0 = smem + st * kF8Stage + (loadA ? 0 : kF8T * 128) + lrow0 * 128;
#pragma unroll
    for (int j = 0; j < LJ; ++j) {
      const int r = lrow0 + 8 * j + (lane >> 3);
      const int kc = f8pos(r, lane & 7);
      const bool ok = kt * 128 + 16 * kc < K;
      const uint32_t row = lbase + 8u * j + (uint32_t)(lane >> 3), kb = (uint32_t)kt * 128u + 16u * kc;
      const uint32_t off = off_if(ok, loadA ? row * (uint32_t)K + kb : w_off<WL>(row, kb, (uint32_t)K));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Lr, (__attribute__((address_space(3))) void*)(dst0 + j * 1024), 16, off, 0,
                                               0, 0);
    }
  };

  const float s1 = a.act_scale[0];

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // lane (g, c): row/column c, K 32g .. 32g+31 of the step = chunks 2g, 2g+1
  auto operand = [&](const unsigned char* T, int r) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(T + r * 128 + f8pos(r, 2 * g) * 16);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(T + r * 128 + f8pos(r, 2 * g + 1) * 16);
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };

  issue(0, 0);
  // the tile's column scales and biases wait in LDS for the epilogue (the
  // loop's first barrier publishes them; issued after the first step's loads), which keeps registers free
  float* colv = reinterpret_cast<float*>(smem + kF8Colv);  // [0][256] scale, [1][256] bias
  if (tid < kF8T) {
    colv[tid] = bitsf(bload32(Sr, (uint32_t)(n0 + tid) * 4u));
    colv[kF8T + tid] = bitsf(bload16(Br, (uint32_t)(n0 + tid) * 2u) << 16);
  }
  for (int kt = 0; kt < KT; ++kt) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's loads of step kt are in LDS
    __syncthreads();                     // ... and every wave's; stage (kt+1)&1 is no longer read
    if (kt + 1 < KT) issue(kt + 1, (kt + 1) & 1);
    const unsigned char* A = smem + (kt & 1) * kF8Stage;
    const unsigned char* B = A + kF8T * 128;
    i32x8 bf[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) bf[t] = operand(B, wn * 64 + 16 * t + c);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const i32x8 af = operand(A, wm * WBM + 16 * i + c);
#pragma unroll
      for (int t = 0; t < TN; ++t) acc[i][t] = mfma_f8(af, bf[t], acc[i][t]);
    }
  }

  // epilogue through LDS (no load is in flight: the last step issued none)
  static_assert(WBM == 64, "64 x 64 wave tiles");
  __syncthreads();  // every wave is done with the operand stages
  unsigned char* et = smem + wave * (64 * kTileRowBytes);
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const float cs = colv[wn * 64 + 16 * t + c], bias = colv[kF8T + wn * 64 + 16 * t + c];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) tile_put(et, 16 * i + 4 * g + r, 16 * t + c, (acc[i][t][r] * s1) * cs + bias);
  }
  tile_store<64>(a.Y, M, N, m0 + wm * 64, n0 + wn * 64, et, lane);
}

// ---------------------------------------------------------------- MXFP4 x MXFP4, 256 x 256 tiles
// For large M x N: 16 waves (4 x 4 grid, 64 x 64 outputs per wave) own a
// 256 x 256 tile and K advances 256 per step, twice the K per barrier of the
// E4M3 kernel above at the same LDS stage size (128 packed bytes per row).
// Packed rows and their E8M0 scale bytes go from memory straight into LDS
// (buffer_load_dwordx4 / buffer_load_dword ... lds; lane i's bytes land at the
// wave's LDS base + 16 i or 4 i).  Stage layout: activation codes [256][128],
// weight codes [256][128], activation scales [256][8], weight scales [256][8];
// two stages.  The MFMA is the 32 x 32 x 64 form
// (v_mfma_scale_f32_32x32x64_f8f6f4, E2M1 x E2M1): lane (g, c) = (lane/32,
// lane%32) supplies 32 codes of row c, K 32g .. 32g+31 of the 64-K sub-step,
// and the result D[8(r/4) + 4g + r%4][c] lands in element r (both layouts
// checked on the device against a host model); per output it reads half the
// LDS bytes of the 16 x 16 x 128 form and measured 8 % faster (34.6 against
// 37.7 us at M = N = 4096, K = 3072).  LDS rows XOR their chunk index with row
// bits 0-2 and row bit 4: the rows c and c + 16 that one ds_read_b128 serves
// together land in different bank groups.  Needs K % 128 == 0 (whole scale
// dwords per row) and 4-byte aligned scale arrays.
constexpr int kMxT = 256;
constexpr int kMxCodes = kMxT * 128;                  // one operand's codes per step
constexpr int kMxStage = 2 * kMxCodes + 2 * kMxT * 8;  // codes, then scales
constexpr int kMxColb = (2 * kMxStage > 16 * 64 * kTileRowBytes) ? 2 * kMxStage : 16 * 64 * kTileRowBytes;
constexpr int kMxSmem = kMxColb + kMxT * 4;  // stages or output tiles, then the tile's biases

template <int WL>
__global__ __launch_bounds__(1024) void k_mx_gemm256(LinearArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int TM = 2, TN = 2;  // 32 x 32 tiles per wave
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  const int wm = wave >> 2, wn = wave & 3;
  const int M = a.M, N = a.N, K = a.K;

  // XCD-aware tile order (see the bf16 tiled kernel)
  const int gx = gridDim.x, G = gx * gridDim.y;
  int b = blockIdx.y * gx + blockIdx.x;
  if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
  const int n0 = (b % gx) * kMxT, m0 = (b / gx) * kMxT;

  const uint32_t rowb = (uint32_t)K / 2u, srow = (uint32_t)K / 32u;
  const __amdgpu_buffer_rsrc_t Xr = make_rsrc(a.X, (uint32_t)M * rowb);
  const __amdgpu_buffer_rsrc_t Wr = make_rsrc(a.W, (uint32_t)N * rowb);
  const __amdgpu_buffer_rsrc_t Xsr = make_rsrc(a.xscales, (uint32_t)M * srow);
  const __amdgpu_buffer_rsrc_t Wsr = make_rsrc(a.scales, (uint32_t)N * srow);
  const __amdgpu_buffer_rsrc_t Br = make_rsrc(a.bias ? (const void*)a.bias : a.W, a.bias ? (uint32_t)N * 2u : 0u);
  const int KT = (K + 255) / 256;

  // waves 0-7 load activation rows 32w .., waves 8-15 weight rows 32(w-8) ..:
  // four code loads of 8 rows (lane L fills slot L % 8 of row L / 8 with the
  // chunk stored there; the slot map is its own inverse) and one scale load
  // (lane L: dword L % 2 of row L / 2's 8 scale bytes); K past the end and
  // rows past M / N read zero
  const bool loadA = wave < 8;
  const __amdgpu_buffer_rsrc_t Lr = loadA ? Xr : Wr;
  const __amdgpu_buffer_rsrc_t Lsr = loadA ? Xsr : Wsr;
  const int lrow0 = 32 * (wave & 7);
  const uint32_t lbase = (uint32_t)((loadA ? m0 : n0) + lrow0);
  auto issue = [&](int kt, int st) {
    unsigned char* base = smem + st * kMxStage;
    unsigned char* dst0 = base + (loadA ? 0 : kMxCodes) + lrow0 * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = lrow0 + 8 * j + (lane >> 3);
      const int kc = (lane & 7) ^ (r & 7) ^ ((r >> 4) & 1);
      const bool ok = kt * 256 + 32 * kc < K;
      const uint32_t row = lbase + 8u * j + (uint32_t)(lane >> 3), kb = (uint32_t)kt * 128u + 16u * kc;
      const uint32_t off = off_if(ok, loadA ? row * rowb + kb : w_off<WL>(row, kb, rowb));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Lr, (__attribute__((address_space(3))) void*)(dst0 + j * 1024), 16, off, 0,
                                               0, 0);
    }
    const int h = lane & 1;
    const bool sok = kt * 8 + 4 * h < (int)srow;
    const uint32_t srw = lbase + (uint32_t)(lane >> 1);
    const uint32_t soff = off_if(sok, loadA ? srw * srow + (uint32_t)kt * 8u + 4u * h
                                            : s_off<KF_MXFP4, WL>(srw, (uint32_t)(kt * 256 + 128 * h), (uint32_t)K));
    unsigned char* sdst = base + 2 * kMxCodes + (loadA ? 0 : kMxT * 8) + lrow0 * 8;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(Lsr, (__attribute__((address_space(3))) void*)sdst, 4, soff, 0, 0, 0);
  };


  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][t][e] = 0.f;

  issue(0, 0);
  // the tile's biases wait in LDS for the epilogue (the loop's first barrier
  // publishes them), which keeps registers free
  float* colb = reinterpret_cast<float*>(smem + kMxColb);
  if (tid < kMxT) colb[tid] = bitsf(bload16(Br, (uint32_t)(n0 + tid) * 2u) << 16);
  for (int kt = 0; kt < KT; ++kt) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's loads of step kt are in LDS
    __syncthreads();                     // ... and every wave's; stage (kt+1)&1 is no longer read
    if (kt + 1 < KT) issue(kt + 1, (kt + 1) & 1);
    const unsigned char* base = smem + (kt & 1) * kMxStage;
    const unsigned char* A = base;
    const unsigned char* B = base + kMxCodes;
    const unsigned char* AS = base + 2 * kMxCodes;
    const unsigned char* BS = AS + kMxT * 8;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      // lane (g, c): row/column c of the 32-row tile, K 64 s4 + 32g .. +31 =
      // chunk 2 s4 + g of the row and scale byte 2 s4 + g
      i32x8 bf[TN];
      uint32_t bs[TN];
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int r = wn * 64 + 32 * t + c;
        const u32x4 v = *reinterpret_cast<const u32x4*>(B + r * 128 + ((2 * s4 + g) ^ (r & 7) ^ ((r >> 4) & 1)) * 16);
        bf[t] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        bs[t] = BS[r * 8 + 2 * s4 + g];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * 64 + 32 * i + c;
        const u32x4 v = *reinterpret_cast<const u32x4*>(A + r * 128 + ((2 * s4 + g) ^ (r & 7) ^ ((r >> 4) & 1)) * 16);
        const i32x8 af = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        const uint32_t as = AS[r * 8 + 2 * s4 + g];
#pragma unroll
        for (int t = 0; t < TN; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf[t], acc[i][t], 4, 4, 0, (int)as, 0, (int)bs[t]);
      }
    }
  }

  // epilogue through LDS (no load is in flight: the last step issued none)
  __syncthreads();  // every wave is done with the operand stages
  unsigned char* et = smem + wave * (64 * kTileRowBytes);
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const float bias = colb[wn * 64 + 32 * t + c];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) tile_put(et, 32 * i + 8 * (r >> 2) + 4 * g + (r & 3), 32 * t + c, acc[i][t][r] + bias);
  }
  tile_store<64>(a.Y, M, N, m0 + wm * 64, n0 + wn * 64, et, lane);
}

template <int BM, int BN, int WL, int WGN = 2>
hipError_t launch_mx_tile(const LinearArgs& a, hipStream_t s) {
  using TT = MxTile<BM, BN, 128 * WGN, false>;
  dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM);
  const size_t pre = TT::pre_bytes(a.K);
  constexpr int limit = 128 * 1024;
  if ((a.K / 32) % 16 == 0 && TT::TILES + pre <= (size_t)limit) {
    static std::atomic<int> done{0};
    const int sm = (int)(TT::TILES + pre);
    auto k = k_mx_gemm_tiled<BM, BN, WGN, true, false, WL>;
    if (sm > 65536 && !done.load(std::memory_order_acquire)) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                         limit);
      if (e != hipSuccess) return e;
      done.store(1, std::memory_order_release);
    }
    k<<<grid, 128 * WGN, sm, s>>>(a);
  } else {
    static std::atomic<int> done{0};
    auto k = k_mx_gemm_tiled<BM, BN, WGN, false, false, WL>;
    hipError_t e = allow_smem(k, TT::TILES, done);
    if (e != hipSuccess) return e;
    k<<<grid, 128 * WGN, TT::TILES, s>>>(a);
  }
  return hipGetLastError();
}

template <int BM, int BN, int WL, int WGN = 2>
hipError_t launch_f8_tile(const LinearArgs& a, hipStream_t s) {
  using TT = MxTile<BM, BN, 128 * WGN, true>;
  static std::atomic<int> done{0};
  auto k = k_mx_gemm_tiled<BM, BN, WGN, false, true, WL>;
  hipError_t e = allow_smem(k, TT::TILES, done);
  if (e != hipSuccess) return e;
  k<<<dim3((a.N + BN - 1) / BN, (a.M + BM - 1) / BM), 128 * WGN, TT::TILES, s>>>(a);
  return hipGetLastError();
}

template <int WL>
hipError_t launch_f8_gemm_tiled_l(const LinearArgs& a, hipStream_t s) {
  // the largest tiles that still give most CUs a workgroup
  const int64_t t256 = (int64_t)((a.M + 255) / 256) * ((a.N + 255) / 256);
  if (t256 >= 192) {
    static std::atomic<int> done{0};
    hipError_t e = allow_smem(k_f8_gemm256<WL>, kF8Smem, done);
    if (e != hipSuccess) return e;
    k_f8_gemm256<WL><<<dim3((a.N + kF8T - 1) / kF8T, (a.M + kF8T - 1) / kF8T), kF8Waves * 64, kF8Smem, s>>>(a);
    return hipGetLastError();
  }
  const int64_t t128 = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128);
  return t128 >= 192 ? launch_f8_tile<128, 128, WL>(a, s) : launch_f8_tile<64, 64, WL>(a, s);
}

template <int WL>
hipError_t launch_mx_linear_l(const LinearArgs& a, hipStream_t s) {
  if (a.M > 64) {
    // 256 x 256 tiles straight into LDS when they fill the chip (whole scale
    // dwords per row needed); up to one round of 64 x 64 tiles the mid-M
    // kernel; else 128 x 128 or 64 x 64 through registers
    const int64_t t256 = (int64_t)((a.M + 255) / 256) * ((a.N + 255) / 256);
    if (t256 >= 192 && a.K % 128 == 0 && (reinterpret_cast<uintptr_t>(a.xscales) & 3) == 0 &&
        (reinterpret_cast<uintptr_t>(a.scales) & 3) == 0) {
      static std::atomic<int> done{0};
      hipError_t e = allow_smem(k_mx_gemm256<WL>, kMxSmem, done);
      if (e != hipSuccess) return e;
      k_mx_gemm256<WL><<<dim3((a.N + kMxT - 1) / kMxT, (a.M + kMxT - 1) / kMxT), 1024, kMxSmem, s>>>(a);
      return hipGetLastError();
    }
    const int64_t t64 = (int64_t)((a.M + 63) / 64) * ((a.N + 63) / 64);
    if (t64 <= 256 && a.K % 512 == 0 && a.K >= 1024 && a.K <= kMxMidMaxK && (reinterpret_cast<uintptr_t>(a.xscales) & 3) == 0 &&
        (reinterpret_cast<uintptr_t>(a.scales) & 3) == 0)
      return launch_mx_mid<WL>(a, s);
    const int64_t t128 = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128);
    return t128 >= 192 ? launch_mx_tile<128, 128, WL>(a, s) : launch_mx_tile<64, 64, WL>(a, s);
  }
  const int gx = (a.N + 15) / 16;
  const bool dw = a.K % 128 == 0 && (reinterpret_cast<uintptr_t>(a.xscales) & 3) == 0 &&
                  (reinterpret_cast<uintptr_t>(a.scales) & 3) == 0;
  // activations through LDS from 9 rows on (M = 1 / 8 / 12 / 32 at N = 4096,
  // K = 3072: 3.48 / 3.74 / 4.01 / 5.81 us straight into registers against
  // 3.65 / 3.75 / 3.82 / 4.42 us through LDS)
  if (dw && a.M > 8 && a.K % 512 == 0 && a.K <= kMxSmallMaxK)
    return a.M <= 16 ? launch_mx_small<1, WL>(a, s) : launch_mx_small<2, WL>(a, s);
  if (a.M <= 16) {
    if (dw) k_mx_linear<1, WL, true><<<dim3(gx, 1, (a.M + 15) / 16), 768, 0, s>>>(a);
    else k_mx_linear<1, WL, false><<<dim3(gx, 1, (a.M + 15) / 16), 768, 0, s>>>(a);
  } else {
    if (dw) k_mx_linear<2, WL, true><<<dim3(gx, 1, (a.M + 31) / 32), 768, 0, s>>>(a);
    else k_mx_linear<2, WL, false><<<dim3(gx, 1, (a.M + 31) / 32), 768, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_quantize_act(const uint16_t* X, int64_t M, int64_t K, uint8_t* Xq, uint8_t* Xs, hipStream_t s) {
  const uint32_t nblk = (uint32_t)(M * (K / 32));
  k_mx_quant_act<<<(nblk + 255) / 256, 256, 0, s>>>(X, nblk, Xq, Xs);
  return hipGetLastError();
}

hipError_t launch_f8_gemm_tiled(const LinearArgs& a, hipStream_t s) {
  return a.wl == kLayoutTiles ? launch_f8_gemm_tiled_l<kLayoutTiles>(a, s) : launch_f8_gemm_tiled_l<kLayoutRows>(a, s);
}

hipError_t launch_mx_linear(const LinearArgs& a, hipStream_t s) {
  return a.wl == kLayoutTiles ? launch_mx_linear_l<kLayoutTiles>(a, s) : launch_mx_linear_l<kLayoutRows>(a, s);
}

}  // namespace wq
