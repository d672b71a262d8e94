// Tiled dequant-GEMM for larger M, where the contraction (2*M*N*K FLOP)
// rather than the weight stream bounds the time.
//
// One workgroup (4 waves, 2 x 2) computes a BM x BN output tile.  K advances in
// steps of 64.  Per step:
//  * every thread loads its share of the activation tile (contiguous 16-byte
//    loads) and of the packed weight tile for the NEXT step, so global
//    latency overlaps the current step's matrix-core work;
//  * the weight chunk is decoded once per workgroup into bf16 and written to
//    LDS next to the activation tile (double
//    buffered; the 16-byte chunks of each row are XOR-swizzled with row bits
//    so that operand reads and tile writes are free of bank conflicts);
//  * each wave reads 16x32 operand fragments from LDS and issues
//    v_mfma_f32_16x16x32_bf16.
// Decode: FP8 weights, NVFP4 (E2M1 x E4M3 block scale) and MXFP4 (E2M1 x
// 2^e) are exact in bf16; the FP8 row scale and the NVFP4 global scale go to
// the epilogue.  (The static FP8 path, E4M3 x E4M3, runs on the scaled
// matrix cores in wq_mx.hip.)  INT4 is decoded as
// bf16(code * s), the dequantized weight of the two-kernel form (at most one
// bf16 rounding per weight).  Workgroups are mapped to tiles so that the
// tiles resident on one XCD share activation rows in that XCD's L2.
#include "wq_kernel_common.hpp"

namespace wq {

namespace {

constexpr int kBK = 64;  // K elements per step

// Global-load steps in flight per tile shape (measured on MI355X): the large
// 128 x 128 tile keeps two stages so two workgroups fit per CU (registers);
// smaller tiles, used when there are few tiles, keep four.
template <int BM, int BN>
constexpr int tile_stages() {
  return (BM >= 128 && BN >= 128) ? 2 : 4;
}

template <int F>
struct TileFmt {
  static constexpr int XB = 2;  // bytes per activation element in LDS (bf16)
  static constexpr int OB = 2;  // bytes per weight operand element in LDS (bf16)
  // packed weight bytes per column per step
  static constexpr int WSTEP = (F == KF_BF16) ? 128 : (F == KF_FP8 ? 64 : 32);
  static constexpr int ARS = kBK * XB;  // LDS row strides (bytes)
  static constexpr int BRS = kBK * OB;
  static_assert(ARS == BRS, "activation and weight rows share one swizzle");
  // Position of 16-byte chunk k in LDS row r (rows of 8 chunks): the chunk
  // index XOR r & 7.  With it, the operand reads (lane (g, c) takes chunk
  // 4kk + g of row c) and a wave writing whole rows hit every LDS bank once
  // (measured with the SQ_LDS_BANK_CONFLICT counter on gfx950; padding rows by
  // 16 bytes instead doubles the read cycles).
  __device__ static __forceinline__ int pos(int r, int k) { return k ^ (r & 7); }
};

template <int F, int BM, int BN>
constexpr int tile_smem() {
  return 2 * (BM * TileFmt<F>::ARS + BN * TileFmt<F>::BRS);
}

// Decode one 16-byte packed chunk of a weight column into operand bytes in
// LDS: `row` is the column's LDS row, k0 the index of its first 16-byte output
// chunk in that row (`sc` holds the chunk's scale codes).  SEQ stores each
// NVFP4 chunk before decoding the next, which bounds the fp32 temporaries
// where registers are scarce.
template <int F, bool SEQ = false>
__device__ __forceinline__ void decode_store(unsigned char* row, int r, int k0, u32x4 w, uint32_t sc) {
  using TF = TileFmt<F>;
  auto at = [&](int p) { return reinterpret_cast<bf16x8*>(row + TF::pos(r, k0 + p) * 16); };
  if constexpr (F == KF_INT4 || F == KF_INT4A) {
    // signed codes: 136 + code after XOR 8; unsigned: 128 + code, value
    // (code - z) * s -- both exact in fp32 before the bf16 rounding
    const float s = bitsf(sc << 16);
    const float bias = (F == KF_INT4) ? 136.f : (float)(128u + ((sc >> 16) & 15u));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // 8 nibbles -> bf16(value), K order kept
      const bf16x8 biased = (F == KF_INT4) ? dec_int4_biased(w[j]) : dec_uint4_biased(w[j]);
      const u32x4 bb = __builtin_bit_cast(u32x4, biased);
      bf16x8 r8;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float lo = bitsf(bb[p] << 16), hi = bitsf(bb[p] & 0xFFFF0000u);
        r8[2 * p] = (__bf16)fmaf(lo, s, -bias * s);
        r8[2 * p + 1] = (__bf16)fmaf(hi, s, -bias * s);
      }
      *at(j) = r8;
    }
  } else if constexpr (F == KF_NVFP4) {
    const float d0 = e4m3_decode(sc & 0xFFu), d1 = e4m3_decode((sc >> 8) & 0xFFu);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *at(j) = dec_fp4_mul(w[j], j < 2 ? d0 : d1);
      if constexpr (SEQ) __builtin_amdgcn_sched_barrier(0);
    }
  } else if constexpr (F == KF_MXFP4) {
    const float p = e8m0_decode(sc);
#pragma unroll
    for (int j = 0; j < 4; ++j) *at(j) = dec_fp4_pow2(w[j], p);
  } else if constexpr (F == KF_FP8) {
    *at(0) = dec_fp8(w[0], w[1]);
    *at(1) = dec_fp8(w[2], w[3]);
  } else {  // BF16 weights are stored as they are
    *reinterpret_cast<u32x4*>(at(0)) = w;
  }
}

// bytes of decoded operand written per 16-byte packed chunk
template <int F>
constexpr int decoded_bytes() {
  return (F == KF_INT4 || F == KF_INT4A || F == KF_NVFP4 || F == KF_MXFP4) ? 64 : ((F == KF_FP8) ? 32 : 16);
}

// WGN: waves along N in a 2 x WGN wave grid (GT = 128 * WGN threads per K
// group); each wave owns a (BM/2) x (BN/WGN) block of the tile.
template <int F, int BM, int BN, int STG, int KS, int WGN, int WL>
__global__ __launch_bounds__(128 * WGN * KS) void k_gemm_tiled(LinearArgs a) {
  using TF = TileFmt<F>;
  constexpr int GT = 128 * WGN;                // threads per K group
  constexpr int WBN = BN / WGN;                // columns per wave
  constexpr int TM = BM / 32, TN = WBN / 16;   // 16x16 tiles per wave
  constexpr int LA = kBK * TF::XB / 16;       // 16-byte chunks per activation row per step
  constexpr int NA = BM * LA / GT;            // activation loads per thread per step
  constexpr int LB = TF::WSTEP / 16;          // 16-byte chunks per weight column per step
  constexpr int CB = BN * LB;                 // weight chunks per step
  constexpr int NB = (CB + GT - 1) / GT;      // weight loads per thread per step
  constexpr int DB = decoded_bytes<F>();
  static_assert(NA * GT == BM * LA, "activation tile must split evenly over the group's threads");
  static_assert(CB % 64 == 0, "whole waves own the weight chunks");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // KS groups of 4 waves split K inside the workgroup: group kg owns a
  // contiguous range of K steps and its own double-buffered tiles; all groups
  // step in lockstep (one workgroup barrier per step) and are summed through
  // LDS at the end.
  const int kg = (int)threadIdx.x / GT;
  unsigned char* As = smem + kg * tile_smem<F, BM, BN>();  // [2][BM][ARS]
  unsigned char* Bs = As + 2 * BM * TF::ARS;                // [2][BN][BRS]

  const int tid = (int)threadIdx.x % GT, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave / WGN, wn = wave % WGN;
  const int M = a.M, N = a.N, K = a.K;

  // XCD-aware tile order: consecutive workgroups go round-robin to the 8 XCDs;
  // give each XCD a contiguous band of tiles (N fastest) so its resident
  // tiles share activation rows.
  const int gx = gridDim.x, gy = gridDim.y;
  const int G = gx * gy;
  int b = blockIdx.y * gx + blockIdx.x;
  if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
  const int n0 = (b % gx) * BN, m0 = (b / gx) * BM;

  const uint32_t wrow = (F == KF_BF16) ? 2u * (uint32_t)K : ((F == KF_FP8) ? (uint32_t)K : (uint32_t)K / 2u);
  const __amdgpu_buffer_rsrc_t Wr = make_rsrc(a.W, (uint32_t)N * wrow);
  const __amdgpu_buffer_rsrc_t Xr = make_rsrc(a.X, (uint32_t)M * (uint32_t)K * (uint32_t)TF::XB);
  uint32_t sbytes = 0;
  if constexpr (F == KF_INT4) sbytes = (uint32_t)N * (uint32_t)(K / 128) * 2u;
  else if constexpr (F == KF_INT4A) sbytes = (uint32_t)N * (uint32_t)(K / 128) * 4u;
  else if constexpr (F == KF_NVFP4) sbytes = (uint32_t)N * (uint32_t)(K / 16);
  else if constexpr (F == KF_MXFP4) sbytes = (uint32_t)N * (uint32_t)(K / 32);
  else if constexpr (F == KF_FP8) sbytes = (uint32_t)N * 4u;
  const __amdgpu_buffer_rsrc_t Sr = make_rsrc(a.scales ? a.scales : a.W, a.scales ? sbytes : 0u);
  const __amdgpu_buffer_rsrc_t Br = make_rsrc(a.bias ? (const void*)a.bias : a.W, a.bias ? (uint32_t)N * 2u : 0u);

  const int KT = (K + kBK - 1) / kBK;
  const int KTg = (KT + KS - 1) / KS;  // steps per group
  const int kbeg = kg * KTg * kBK;     // this group's K range [kbeg, kend)
  const int kend = min(K, kbeg + KTg * kBK);

  // STG register stages of global loads are in flight: the loads of step k
  // live in stage k % STG from the moment they are issued (STG steps ahead)
  // until their decode into LDS.
  u32x4 xa[STG][NA];
  u32x4 wb[STG][NB];
  uint32_t sb[STG][NB];

  auto gload = [&](int kt, u32x4 (&xa)[NA], u32x4 (&wb)[NB], uint32_t (&sb)[NB]) {
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      const int row = q * (GT / LA) + tid / LA;
      const int kx = kbeg + kt * kBK + (tid % LA) * (16 / TF::XB);
      xa[q] = bload128(Xr, off_if(kx < kend, ((uint32_t)(m0 + row) * (uint32_t)K + (uint32_t)kx) * (uint32_t)TF::XB));
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      // threads beyond the chunk count repeat a chunk (identical bytes): no
      // divergent branch, which would make the compiler drain every load
      const int id = (q * GT + tid) % CB;
      const int col = id / LB, part = id % LB;
      const uint32_t n = (uint32_t)(n0 + col);
      // K elements per 16-byte chunk: 4-bit 32, FP8 16, BF16 8; k0 is the chunk's first K
      const int kpc = (F == KF_BF16) ? 8 : ((F == KF_FP8) ? 16 : 32);
      const int k0 = kbeg + kt * kBK + part * kpc;
      const bool ok = k0 < kend;
      const uint32_t byte0 = (F == KF_BF16) ? 2u * (uint32_t)k0 : ((F == KF_FP8) ? (uint32_t)k0 : (uint32_t)k0 / 2u);
      wb[q] = bload128(Wr, off_if(ok, w_off<WL>(n, byte0, wrow)));
      if constexpr (F == KF_INT4 || F == KF_NVFP4) sb[q] = bload16(Sr, off_if(ok, s_off<F, WL>(n, (uint32_t)k0, (uint32_t)K)));
      else if constexpr (F == KF_INT4A) sb[q] = bload32(Sr, off_if(ok, s_off<F, WL>(n, (uint32_t)k0, (uint32_t)K)));
      else if constexpr (F == KF_MXFP4) sb[q] = bload8(Sr, off_if(ok, s_off<F, WL>(n, (uint32_t)k0, (uint32_t)K)));
      else sb[q] = 0u;
    }
  };
  auto lstore = [&](int buf, const u32x4 (&xa)[NA], const u32x4 (&wb)[NB], const uint32_t (&sb)[NB]) {
    unsigned char* A = As + buf * BM * TF::ARS;
    unsigned char* B = Bs + buf * BN * TF::BRS;
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      const int row = q * (GT / LA) + tid / LA;
      *reinterpret_cast<u32x4*>(A + row * TF::ARS + TF::pos(row, tid % LA) * 16) = xa[q];
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      // threads past the chunk count loaded a repeat; they store nothing
      // (wave-uniform: CB is a multiple of 64).  Measured at M = 128 and 256
      // (N = 4096, K = 3072, 64 x 64 tiles): MXFP4 17.5 -> 16.2 us and 18.9 ->
      // 17.6 us, NVFP4 21.5 -> 20.8 us.
      const int id = (q * GT + tid) % CB;
      const int col = id / LB, part = id % LB;
      if (CB % GT == 0 || q * GT + tid < CB) decode_store<F>(B + col * TF::BRS, col, part * (DB / 16), wb[q], sb[q]);
    }
  };

  // epilogue operands of this lane's columns, loaded up front
  uint32_t bias_bits[TN], cs_bits[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const uint32_t n = (uint32_t)(n0 + wn * WBN + 16 * t + c);
    bias_bits[t] = bload16(Br, n * 2u);
    cs_bits[t] = (F == KF_FP8) ? bload32(Sr, n * 4u) : 0x3F800000u;
  }

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
    const unsigned char* A = As + buf * BM * TF::ARS;
    const unsigned char* B = Bs + buf * BN * TF::BRS;
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      // lane (g, c): K 32kk + 8g .. +7 of the step = 16-byte chunk 4kk + g
      bf16x8 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * (BM / 2) + 16 * i + c;
        af[i] = *reinterpret_cast<const bf16x8*>(A + r * TF::ARS + TF::pos(r, 4 * kk + g) * 16);
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int r = wn * WBN + 16 * t + c;
        bf[t] = *reinterpret_cast<const bf16x8*>(B + r * TF::BRS + TF::pos(r, 4 * kk + g) * 16);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[i][t] = mfma_bf16(af[i], bf[t], acc[i][t]);
    }
  };

  // The step count is padded to a multiple of STG: steps past K read zeros
  // (their loads fall outside the buffers) and add nothing, which keeps the
  // loop body free of branches -- a branch makes the compiler drain all loads
  // in flight.  STG is even, so the LDS buffer index kt % 2 = st % 2 is a
  // compile-time constant.
  static_assert(STG % 2 == 0, "even number of load stages");
  const int KTP = (KTg + STG - 1) / STG * STG;

  // prologue: steps 0 .. STG-1 in flight, step 0 decoded into LDS buffer 0,
  // then its register stage refilled with step STG
#pragma unroll
  for (int st = 0; st < STG; ++st) gload(st, xa[st], wb[st], sb[st]);
  lstore(0, xa[0], wb[0], sb[0]);
  gload(STG, xa[0], wb[0], sb[0]);
  __syncthreads();

  // step kt computes from LDS buffer kt % 2, decodes step kt + 1 (register
  // stage (kt + 1) % STG) into the other buffer and refills that stage with
  // step kt + 1 + STG
  for (int kt0 = 0; kt0 < KTP; kt0 += STG) {
#pragma unroll
    for (int st = 0; st < STG; ++st) {
      const int kt = kt0 + st;
      const int nx = (st + 1) % STG;
      compute(st & 1);
      lstore((st + 1) & 1, xa[nx], wb[nx], sb[nx]);
      gload(kt + 1 + STG, xa[nx], wb[nx], sb[nx]);
      __syncthreads();
    }
  }

  // ---- sum the K groups: groups 1.. store their tiles into the (now idle)
  // tile buffers, group 0 adds them in group order
  if constexpr (KS > 1) {
    float* red = reinterpret_cast<float*>(smem);
    if (kg > 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
          *reinterpret_cast<f32x4*>(red + ((((kg - 1) * (2 * WGN) + wave) * TM * TN + i * TN + t) * 64 + lane) * 4) = acc[i][t];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int g2 = 1; g2 < KS; ++g2)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          const f32x4 o = *reinterpret_cast<const f32x4*>(red + ((((g2 - 1) * (2 * WGN) + wave) * TM * TN + i * TN + t) * 64 + lane) * 4);
          acc[i][t] += o;
        }
  }

  // ---- epilogue: lane holds D[4g + r][c] of every 16x16 tile; the column
  // operands were fetched before the main loop.  The output tile leaves
  // through LDS past the group partials (idle: the loop's last barrier is
  // behind every wave, and only group 0, each wave in its own region, is
  // left).  Measured at N = 4096, K = 3072, M = 128-1024: 0.3-1.3 us faster
  // for the 4-bit formats; FP8 on 128 x 128 tiles was 1-2 us slower and keeps
  // the element stores.
  float s1 = 1.0f;
  if constexpr (F == KF_NVFP4) s1 = a.gscale[0];
  if constexpr (F == KF_FP8 || F == KF_BF16) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int n = n0 + wn * WBN + 16 * t + c;
      const float bias = bitsf(bias_bits[t] << 16);
      const float cs = bitsf(cs_bits[t]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * (BM / 2) + 16 * i + 4 * g + r;
          const float y = (F == KF_FP8) ? acc[i][t][r] * cs : acc[i][t][r];
          if (m < M && n < N) a.Y[(int64_t)m * N + n] = f32_to_bf16(y + bias);
        }
    }
    return;
  }
  constexpr int EOFF = (KS - 1) * BM * BN * 4;
  static_assert(EOFF + 2 * WGN * (BM / 2) * kTileRowBytes <= KS * tile_smem<F, BM, BN>(), "output tiles fit in LDS");
  unsigned char* et = smem + EOFF + wave * ((BM / 2) * kTileRowBytes);
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const float bias = bitsf(bias_bits[t] << 16);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        tile_put(et, 16 * i + 4 * g + r, 16 * t + c, acc[i][t][r] * s1 + bias);
      }
  }
  tile_store<BM / 2, WBN>(a.Y, M, N, m0 + wm * (BM / 2), n0 + wn * WBN, et, lane);
}

// ---------------------------------------------------------------- 256 x 256 tiles
// For large M x N: one workgroup of NW waves (NW/4 x 4 grid, 256/(NW/4) x 64
// outputs per wave) owns a 256 x 256 tile; K advances 64 per step.
// Activation rows go from memory straight into LDS (buffer_load_dwordx4 ...
// lds writes lane i's 16 bytes at the wave's LDS base + 16 i: one load moves 8
// whole 128-byte rows, and the row swizzle is applied by choosing which chunk
// of its row each lane fetches).  The packed weight chunks of step k+2 are
// loaded into registers during step k, and those of step k+1 are decoded into
// the other LDS stage at the end of step k.  Two LDS stages of 64 KiB, one
// barrier per step: after it a wave issues the next step's activation loads
// and the weight loads two steps ahead, runs its MFMAs, then decodes.
template <int F, int NW, int WL>
__global__ __launch_bounds__(NW * 64) void k_woq_gemm256(LinearArgs a) {
  using TF = TileFmt<F>;
  static_assert(TF::ARS == 128 && TF::BRS == 128, "128-byte LDS rows");
  constexpr int T = 256, NT = NW * 64;
  constexpr int WBM = T / (NW / 4), TM = WBM / 16, TN = 4;
  constexpr int STAGE = 2 * T * 128;                 // A rows then B rows
  constexpr int XJ = 32 / NW;                        // activation loads (8 rows each) per wave and step
  constexpr int LB = TF::WSTEP / 16;                 // packed 16-byte chunks per column and step
  constexpr int CB = T * LB;                         // packed chunks per step
  constexpr int NB = (CB + NT - 1) / NT;             // per thread
  constexpr int DB = decoded_bytes<F>();
  constexpr int kpc = (F == KF_BF16) ? 8 : (F == KF_FP8 ? 16 : 32);  // K per packed chunk
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave >> 2, wn = wave & 3;
  const int M = a.M, N = a.N, K = a.K;

  // XCD-aware tile order (consecutive workgroups go round-robin to the XCDs)
  const int gx = gridDim.x, G = gx * gridDim.y;
  int b = blockIdx.y * gx + blockIdx.x;
  if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
  const int n0 = (b % gx) * T, m0 = (b / gx) * T;

  const uint32_t wrow = (F == KF_BF16) ? 2u * (uint32_t)K : (F == KF_FP8 ? (uint32_t)K : (uint32_t)K / 2u);
  const __amdgpu_buffer_rsrc_t Wr = make_rsrc(a.W, (uint32_t)N * wrow);
  const __amdgpu_buffer_rsrc_t Xr = make_rsrc(a.X, (uint32_t)M * (uint32_t)K * 2u);
  uint32_t sbytes = 0;
  if constexpr (F == KF_INT4) sbytes = (uint32_t)N * (uint32_t)(K / 128) * 2u;
  else if constexpr (F == KF_INT4A) sbytes = (uint32_t)N * (uint32_t)(K / 128) * 4u;
  else if constexpr (F == KF_NVFP4) sbytes = (uint32_t)N * (uint32_t)(K / 16);
  else if constexpr (F == KF_MXFP4) sbytes = (uint32_t)N * (uint32_t)(K / 32);
  else if constexpr (F == KF_FP8) sbytes = (uint32_t)N * 4u;
  const __amdgpu_buffer_rsrc_t Sr = make_rsrc(a.scales ? a.scales : a.W, a.scales ? sbytes : 0u);
  const __amdgpu_buffer_rsrc_t Br = make_rsrc(a.bias ? (const void*)a.bias : a.W, a.bias ? (uint32_t)N * 2u : 0u);
  const int KT = (K + 63) / 64;

  // activation rows (256/NW)*w .. of step kt into LDS stage st; K past the end
  // and rows past M read zero
  auto issueX = [&](int kt, int st) {
    unsigned char* dst0 = smem + st * STAGE + (T / NW) * wave * 128;
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
      const int r = (T / NW) * wave + 8 * j + (lane >> 3);
      const int kx = kt * 64 + 8 * TF::pos(r, lane & 7);  // the slot map is its own inverse
      const uint32_t off = off_if(kx < K, ((uint32_t)(m0 + r) * (uint32_t)K + (uint32_t)kx) * 2u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Xr, (__attribute__((address_space(3))) void*)(dst0 + j * 1024), 16, off, 0,
                                               0, 0);
    }
  };
  // packed weight chunks of step kt (threads past the chunk count repeat a
  // chunk: identical bytes, no divergent branch)
  u32x4 wb[2][NB];
  uint32_t sb[2][NB];
  auto loadW = [&](int kt, u32x4 (&w)[NB], uint32_t (&sc)[NB]) {
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int id = (q * NT + tid) % CB;
      const int col = id / LB, part = id % LB;
      const uint32_t n = (uint32_t)(n0 + col);
      const int k0 = kt * 64 + part * kpc;
      const bool ok = k0 < K;
      const uint32_t byte0 = (F == KF_BF16) ? 2u * (uint32_t)k0 : (F == KF_FP8 ? (uint32_t)k0 : (uint32_t)k0 / 2u);
      w[q] = bload128(Wr, off_if(ok, w_off<WL>(n, byte0, wrow)));
      if constexpr (F == KF_INT4 || F == KF_NVFP4) sc[q] = bload16(Sr, off_if(ok, s_off<F, WL>(n, (uint32_t)k0, (uint32_t)K)));
      else if constexpr (F == KF_INT4A) sc[q] = bload32(Sr, off_if(ok, s_off<F, WL>(n, (uint32_t)k0, (uint32_t)K)));
      else if constexpr (F == KF_MXFP4) sc[q] = bload8(Sr, off_if(ok, s_off<F, WL>(n, (uint32_t)k0, (uint32_t)K)));
      else sc[q] = 0u;
    }
  };
  auto decodeW = [&](int st, const u32x4 (&w)[NB], const uint32_t (&sc)[NB]) {
    unsigned char* B = smem + st * STAGE + T * 128;
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int id = (q * NT + tid) % CB;
      const int col = id / LB, part = id % LB;
      // (NVFP4: chunk by chunk; decoded all at once, its fp32 temporaries
      // pushed the kernel past 256 registers and spilled, 145 against 116 us
      // at M = N = 4096, K = 3072)
      decode_store<F, true>(B + col * 128, col, part * (DB / 16), w[q], sc[q]);
    }
  };

  uint32_t bias_bits[TN], cs_bits[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const uint32_t n = (uint32_t)(n0 + wn * 64 + 16 * t + c);
    bias_bits[t] = bload16(Br, n * 2u);
    cs_bits[t] = (F == KF_FP8) ? bload32(Sr, n * 4u) : 0x3F800000u;
  }

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int st) {
    const unsigned char* A = smem + st * STAGE;
    const unsigned char* B = A + T * 128;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // lane (g, c): K 32kk + 8g .. +7 of the step = 16-byte chunk 4kk + g
      bf16x8 bf[TN];
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int r = wn * 64 + 16 * t + c;
        bf[t] = *reinterpret_cast<const bf16x8*>(B + r * 128 + TF::pos(r, 4 * kk + g) * 16);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WBM + 16 * i + c;
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(A + r * 128 + TF::pos(r, 4 * kk + g) * 16);
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[i][t] = mfma_bf16(af, bf[t], acc[i][t]);
      }
    }
  };

  // steps past K read zeros and add nothing: the step count is padded to an
  // even number so that both register stages are compile-time indices
  const int KTP = (KT + 1) / 2 * 2;
  issueX(0, 0);
  loadW(0, wb[0], sb[0]);
  loadW(1, wb[1], sb[1]);
  decodeW(0, wb[0], sb[0]);
  for (int kt = 0; kt < KTP; kt += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // this wave's loads are done: activations of step kt+h in LDS, weight
      // registers of step kt+h+1; after the barrier every wave's are, and
      // stage (kt+h+1)&1 is no longer read
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      issueX(kt + h + 1, (h + 1) & 1);
      loadW(kt + h + 2, wb[h], sb[h]);
      compute(h);
      decodeW((h + 1) & 1, wb[(h + 1) & 1], sb[(h + 1) & 1]);
    }
  }
  // no LDS write may still be in flight when the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  float s1 = 1.0f;
  if constexpr (F == KF_NVFP4) s1 = a.gscale[0];
  // epilogue through LDS
  __syncthreads();  // every wave is done with the tile stages
  unsigned char* et = smem + wave * (WBM * kTileRowBytes);
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const float bias = bitsf(bias_bits[t] << 16), cs = bitsf(cs_bits[t]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float y = (F == KF_FP8) ? acc[i][t][r] * cs : acc[i][t][r] * s1;
        tile_put(et, 16 * i + 4 * g + r, 16 * t + c, y + bias);
      }
  }
  tile_store<WBM>(a.Y, M, N, m0 + wm * WBM, n0 + wn * 64, et, lane);
}

// ---------------------------------------------------------------- MXFP4, 256 x 256 tiles, weights in registers
// For large M x N: one workgroup of 8 waves (2 x 4 grid, 128 x 64 outputs per
// wave) owns a 256 x 256 tile and K advances 128 per step, twice the K per
// barrier of k_woq_gemm256: only the activations pass through LDS (256 rows x
// 256 bytes per step, loaded straight into LDS), while every wave loads and
// decodes its own 64 weight columns in registers.  Lane (g, c) of a wave holds
// K 32g .. 32g+31 of the step for its columns (16 packed bytes and their E8M0
// scale) and, in sub-step kk, feeds K 32g + 8kk .. +7 to the MFMA; it reads
// the activations with the same K order (16-byte chunk 4g + kk of the row).
// The two waves of a column block load the same weight bytes (from L1) and
// decode them twice.  Measured at M = 4096 (N = 4096, K = 3072): 98-102 us
// against 104-107 us for k_woq_gemm256.  The same scheme spilled registers for
// the other formats (their decodes need more), which stay on k_woq_gemm256.
struct MxWReg {
  uint32_t w[4];  // 32 E2M1 codes, K order, low nibble first
  uint32_t sc;    // E8M0 scale byte of the 32-element block (DW: the aligned dword holding it)
};

template <int WL, bool DW>
__device__ __forceinline__ void mxwreg_load(MxWReg& r, __amdgpu_buffer_rsrc_t Wr, __amdgpu_buffer_rsrc_t Sr, uint32_t n,
                                            int kb, int K) {
  const bool ok = kb < K;
  const u32x4 v = bload128(Wr, off_if(ok, w_off<WL>(n, (uint32_t)kb / 2u, (uint32_t)K / 2u)));
  r.w[0] = v.x;
  r.w[1] = v.y;
  r.w[2] = v.z;
  r.w[3] = v.w;
  // DW (K % 128 == 0): one aligned dword per lane, which holds the 4 block
  // scales of the 128-K step (a byte load costs the address unit as much as a
  // 16-byte one); the decode shifts the block's byte down.  Measured at
  // M = N = 4096, K = 3072: 84.7 -> 79.7 us
  const uint32_t so = s_off<KF_MXFP4, WL>(n, (uint32_t)kb, (uint32_t)K);
  if constexpr (DW) r.sc = bload32(Sr, off_if(ok, so & ~3u));
  else r.sc = bload8(Sr, off_if(ok, so));
}

// LDS slot of 16-byte chunk k (0..15) of activation row r (256-byte rows): the
// 16 reads of rows c = 0..7 by lane groups g and g+1 (chunks 4g + kk) land on
// 16 distinct 16-byte bank groups
__device__ __forceinline__ int wreg_pos(int r, int k) { return k ^ ((r & 3) | (((r >> 2) & 1) << 3)); }

template <int WL, bool DW>
__global__ __launch_bounds__(512) void k_mx_wreg(LinearArgs a) {
  constexpr int T = 256, TM = 8, TN = 4;
  constexpr int STAGE = T * 256;  // activation rows of one step
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave >> 2, wn = wave & 3;
  const int M = a.M, N = a.N, K = a.K;

  // XCD-aware tile order (consecutive workgroups go round-robin to the XCDs)
  const int gx = gridDim.x, G = gx * gridDim.y;
  int b = blockIdx.y * gx + blockIdx.x;
  if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
  const int n0 = (b % gx) * T, m0 = (b / gx) * T;

  const __amdgpu_buffer_rsrc_t Wr = make_rsrc(a.W, (uint32_t)N * ((uint32_t)K / 2u));
  const __amdgpu_buffer_rsrc_t Xr = make_rsrc(a.X, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t Sr = make_rsrc(a.scales, (uint32_t)N * (uint32_t)(K / 32));
  const __amdgpu_buffer_rsrc_t Br = make_rsrc(a.bias ? (const void*)a.bias : a.W, a.bias ? (uint32_t)N * 2u : 0u);
  const int KT = (K + 127) / 128;

  // activation rows 32w .. 32w+31 of step kt into LDS stage st: load j moves
  // rows +4j .. +4j+3, lane L filling slot L % 16 of row L / 16 with the chunk
  // stored there (the slot map is its own inverse); K past the end and rows
  // past M read zero
  auto issueX = [&](int kt, int st) {
    unsigned char* dst0 = smem + st * STAGE + 32 * wave * 256;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 32 * wave + 4 * j + (lane >> 4);
      const int kx = kt * 128 + 8 * wreg_pos(r, lane & 15);
      const uint32_t off = off_if(kx < K, ((uint32_t)(m0 + r) * (uint32_t)K + (uint32_t)kx) * 2u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Xr, (__attribute__((address_space(3))) void*)(dst0 + j * 1024), 16, off, 0,
                                               0, 0);
    }
  };
  MxWReg wr[2][TN];
  auto loadW = [&](int kt, MxWReg (&r)[TN]) {
#pragma unroll
    for (int t = 0; t < TN; ++t)
      mxwreg_load<WL, DW>(r[t], Wr, Sr, (uint32_t)(n0 + wn * 64 + 16 * t + c), kt * 128 + 32 * g, K);
  };

  uint32_t bias_bits[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) bias_bits[t] = bload16(Br, (uint32_t)(n0 + wn * 64 + 16 * t + c) * 2u);
  // with DW the block of lane group g is byte g of its scale dword in both
  // layouts (K % 128 == 0)
  const uint32_t ssh = DW ? 8u * (uint32_t)g : 0u;

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int st, const MxWReg (&r)[TN]) {
    const unsigned char* A = smem + st * STAGE;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 bf[TN];
#pragma unroll
      for (int t = 0; t < TN; ++t) bf[t] = dec_fp4_pow2(r[t].w[kk], e8m0_decode((r[t].sc >> ssh) & 0xFFu));
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * 128 + 16 * i + c;
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(A + row * 256 + wreg_pos(row, 4 * g + kk) * 16);
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[i][t] = mfma_bf16(af, bf[t], acc[i][t]);
      }
      // keep each sub-step's decode and operand reads next to its MFMAs
      // (hoisting them all over-commits the registers)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // steps past K read zeros and add nothing; the step count is padded to an
  // even number so that both register stages are compile-time indices
  const int KTP = (KT + 1) / 2 * 2;
  issueX(0, 0);
  loadW(0, wr[0]);
  for (int kt = 0; kt < KTP; kt += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // this wave's loads of step kt+h are done; after the barrier every
      // wave's are, and stage (kt+h+1)&1 is no longer read
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      issueX(kt + h + 1, (h + 1) & 1);
      loadW(kt + h + 1, wr[(h + 1) & 1]);
      compute(h, wr[h]);
    }
  }
  // no LDS write may still be in flight when the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  // epilogue through LDS
  __syncthreads();  // every wave is done with the activation stages
  unsigned char* et = smem + wave * (128 * kTileRowBytes);
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const float bias = bitsf(bias_bits[t] << 16);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) tile_put(et, 16 * i + 4 * g + r, 16 * t + c, acc[i][t][r] + bias);
  }
  tile_store<128>(a.Y, M, N, m0 + wm * 128, n0 + wn * 64, et, lane);
}

template <int F, int WL, int BM, int BN, int KS, int WGN = 2>
hipError_t launch_tile(const LinearArgs& a, hipStream_t s) {
  constexpr int sm = KS * tile_smem<F, BM, BN>();
  static_assert(sm <= 160 * 1024, "tile exceeds the LDS of a CU");
  static_assert(KS == 1 || (KS - 1) * BM * BN * 4 <= sm, "group partials must fit in the tile buffers");
  static std::atomic<int> done{0};
  auto k = k_gemm_tiled<F, BM, BN, tile_stages<BM, BN>(), KS, WGN, WL>;
  hipError_t e = allow_smem(k, sm, done);
  if (e != hipSuccess) return e;
  dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM);
  k<<<grid, 128 * WGN * KS, sm, s>>>(a);
  return hipGetLastError();
}

// 8 waves of 128 x 64 outputs: with 16 waves of 64 x 64 every format spilled
// registers (128 per wave at four waves per SIMD)
constexpr int kWoqWaves = 8;

template <int F, int WL>
hipError_t launch_tiled_f(const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  // 256 x 256 and 128 x 128 tiles are planned only when there are enough of
  // them (no K groups); the other shapes run with one or two K groups
  if constexpr (F == KF_MXFP4) {
    if (p.bm == 256) {
      static std::atomic<int> done_dw{0}, done_b{0};
      constexpr int sm = (2 * 256 * 256 > 8 * 128 * kTileRowBytes) ? 2 * 256 * 256 : 8 * 128 * kTileRowBytes;
      const bool dw = a.K % 128 == 0;
      auto k = dw ? k_mx_wreg<WL, true> : k_mx_wreg<WL, false>;
      hipError_t e = allow_smem(k, sm, dw ? done_dw : done_b);
      if (e != hipSuccess) return e;
      k<<<dim3((a.N + 255) / 256, (a.M + 255) / 256), 512, sm, s>>>(a);
      return hipGetLastError();
    }
  }
  if (p.bm == 256) {
    static std::atomic<int> done{0};
    constexpr int sm = (2 * 2 * 256 * 128 > kWoqWaves * 128 * kTileRowBytes) ? 2 * 2 * 256 * 128 : kWoqWaves * 128 * kTileRowBytes;
    auto k = k_woq_gemm256<F, kWoqWaves, WL>;
    hipError_t e = allow_smem(k, sm, done);
    if (e != hipSuccess) return e;
    k<<<dim3((a.N + 255) / 256, (a.M + 255) / 256), kWoqWaves * 64, sm, s>>>(a);
    return hipGetLastError();
  }
  if (p.bm == 128 && p.bn == 128) return launch_tile<F, WL, 128, 128, 1>(a, s);
  if (p.bm == 128) return p.ks >= 2 ? launch_tile<F, WL, 128, 64, 2>(a, s) : launch_tile<F, WL, 128, 64, 1>(a, s);
  if (p.bn == 128) return p.ks >= 2 ? launch_tile<F, WL, 64, 128, 2>(a, s) : launch_tile<F, WL, 64, 128, 1>(a, s);
  if (p.ks >= 2) {
    // 4-bit weights: four K groups of two waves (32 x 64 outputs each)
    // rather than two groups of four; each activation row is then read from
    // LDS by one wave instead of two.  Measured at N = 4096, K = 3072, M = 128
    // and 256: INT4 23.4 -> 17.8 and 24.8 -> 19.9 us, NVFP4 20.8 -> 17.5 and
    // 22.6 -> 19.7 us, MXFP4 16.2 -> 14.9 and 17.6 -> 16.8 us; FP8 (twice the
    // weight bytes per step) was 1.5-3.4 us slower and keeps two groups.
    constexpr bool four_bit = F == KF_INT4 || F == KF_INT4A || F == KF_NVFP4 || F == KF_MXFP4;
    if constexpr (four_bit) return launch_tile<F, WL, 64, 64, 4, 1>(a, s);
    else return launch_tile<F, WL, 64, 64, 2>(a, s);
  }
  return launch_tile<F, WL, 64, 64, 1>(a, s);
}

template <int F>
hipError_t launch_tiled_fl(const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  if constexpr (F != KF_BF16) {
    if (a.wl == kLayoutTiles) return launch_tiled_f<F, kLayoutTiles>(a, p, s);
  }
  return launch_tiled_f<F, kLayoutRows>(a, p, s);
}

}  // namespace

hipError_t launch_gemm_tiled(int kfmt, const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  switch (kfmt) {
    case KF_BF16: return launch_tiled_fl<KF_BF16>(a, p, s);
    case KF_INT4: return launch_tiled_fl<KF_INT4>(a, p, s);
    case KF_INT4A: return launch_tiled_fl<KF_INT4A>(a, p, s);
    case KF_FP8: return launch_tiled_fl<KF_FP8>(a, p, s);
    case KF_NVFP4: return launch_tiled_fl<KF_NVFP4>(a, p, s);
    case KF_MXFP4: return launch_tiled_fl<KF_MXFP4>(a, p, s);
    case KF_FP8S: return launch_f8_gemm_tiled(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wq
