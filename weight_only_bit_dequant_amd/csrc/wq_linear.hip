// Dequant-GEMM for small M (M <= 64, and up to 128 on wide layers):
// Y = X . deq(W)^T (+ b).
//
// Every weight-only page's intro describes the engine it wants: the weight stays
// packed in device memory and a dequantization prologue feeds a high-precision
// GEMM while activations stay bf16 (NVFP4 adds a two-level block x global
// scale).  The static-FP8 page's intro runs the GEMM itself in FP8.  Here:
//
//  * no-split tiles (whenever they give at least 128 workgroups, and at any
//    width for K <= 3072): one workgroup = 12 waves = 16 output columns (32
//    for two row blocks) x all of K; each wave owns a contiguous K range
//    (split-K inside the workgroup).  Split tiles (narrow layers with
//    K > 3072): 4 waves = 64 columns x a K range, with the K ranges of one
//    column tile spread over S workgroups;
//  * each wave issues every load of its K range (activations, packed weights
//    and block scales; bias and column scale at the start) before the first
//    wait, as buffer loads whose out-of-range offsets read
//    zero (no branches around loads);
//  * activations (M <= 32 rows per workgroup) are loaded with contiguous
//    16-byte loads into a private LDS slot per wave (for the 4-bit formats
//    with 16-row blocks straight from memory, one slot per K step) and read
//    back in the MFMA operand layout;
//  * codes are decoded in registers and fed to v_mfma_f32_16x16x32_bf16
//    (v_mfma_f32_16x16x32_fp8_fp8 for the static path) with fp32
//    accumulation.  Lane (g, c) with g = lane/16, c = lane%16 supplies
//    8 consecutive K of its own 16-byte chunk to each MFMA, so the K order
//    inside an MFMA is a permutation shared by both operands;
//  * every wave writes its partial tile to LDS; after one barrier each thread
//    sums the wave partials of its output in a fixed order.  With S > 1 the
//    workgroup partials go to the workspace and k_splitk_reduce, launched
//    next on the same stream, sums them;
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
#include <atomic>

#include "wq_kernel_common.hpp"

namespace wq {

namespace {

// Activation staging through LDS (XLDS): the MFMA operand layout wants lane
// (g, c) to hold row c, K-chunk g, so loading it straight from a row-major X
// touches 16 rows per load instruction.  With XLDS each wave instead loads
// its [16*MT rows x one K macro-step] slice with contiguous 16-byte loads
// (L lanes per row, R rows per instruction), writes it into a private LDS slot
// and reads it back in the operand layout.
//
// Slot layout: row r holds its L 16-byte chunks in the order pos(r, k) -- an
// XOR of the chunk index with a few row bits, chosen so that the operand
// reads (each quarter-wave reads 16 different rows) and the contiguous writes
// are free of LDS bank conflicts on gfx950 (checked with the
// SQ_LDS_BANK_CONFLICT counter: an unswizzled or padded row costs the reads
// twice the LDS cycles).
template <int F, int MT>
struct XStage {
  static constexpr int KPL = FmtT<F>::KPL;
  static constexpr int MACRO = 4 * KPL;
  static constexpr int XB = (F == KF_FP8S) ? 1 : 2;  // bytes per activation element
  static constexpr int ROWB = MACRO * XB;             // LDS row (no padding)
  static constexpr int SLOT = 16 * MT * ROWB;         // one wave's slice
  static constexpr int L = MACRO * XB / 16;           // lanes per row = chunks per row
  static constexpr int R = 64 / L;                    // rows per load instruction
  static_assert(L == 4 || L == 8 || L == 16, "slot rows of 4, 8 or 16 chunks");
  __device__ static __forceinline__ int pos(int r, int k) {
    if constexpr (L == 16) return k ^ ((r & 3) | (((r >> 3) & 1) << 3));
    else if constexpr (L == 8) return k ^ (((r >> 1) & 1) | (((r >> 3) & 1) << 2));
    else return k ^ ((r >> 1) & 3);
  }
};

// XDMA: the activation slices go from memory straight into LDS (buffer_load
// ... lds), one slot per K step of the wave, instead of through registers and
// a write into one slot (16-row blocks of 32-column tiles in tile order).
// Measured at N = 4096, K = 3072, M = 32 (two alternating bench runs):
// MXFP4 5.39 -> 5.24-5.26 us, INT4 6.01-6.02 -> 5.99-6.00 us; FP8 did not
// change (6.16-6.18 against 6.16 us) and keeps the register staging
template <int F, int MT, int NTW, int WL>
constexpr bool x_dma() {
  return MT == 1 && NTW == 2 && WL == kLayoutTiles && (F == KF_INT4 || F == KF_INT4A || F == KF_MXFP4);
}

// LDS: [activation slots of the NW waves (XLDS)][NW wave partials, fp32]
template <int F, int MT, int NTW, int NW, int WL, int SPW>
constexpr int xslots_bytes(bool xlds) {
  return xlds ? NW * XStage<F, MT>::SLOT * (x_dma<F, MT, NTW, WL>() ? SPW : 1) : 0;
}
template <int F, int MT, int NTW, int NW, int WL, int SPW>
constexpr int smem_bytes(bool xlds) {
  return xslots_bytes<F, MT, NTW, NW, WL, SPW>(xlds) + NW * (MT * 16 * 16 * NTW) * 4;
}

// Weights before activations (no-split tiles): every wave issues its packed
// weight and scale loads, the workgroup meets at a barrier, and only then are
// the activation loads issued, so that the long-latency weight stream is not
// queued behind the CU's activation traffic (192 KiB per CU at M = 32,
// K = 3072).  Measured at N = 4096, K = 3072, M = 32 (cold weights): rows
// layout INT4 6.52 -> 6.35 us, FP8 7.03 -> 6.57, NVFP4 6.90 -> 6.51, MXFP4
// 6.55 -> 6.20; in tile order only MXFP4 (5.73 -> 5.65) and NVFP4 (6.08 ->
// 6.03) gain, while INT4 (5.82 -> 6.01) and FP8 (6.34 -> 6.40) lose.
template <int F, int WL, int MT, int NTW>
constexpr bool weights_first() {
  if constexpr (WL == kLayoutRows) return true;
  // tile order with 16-row blocks of 32-column tiles (17..32 rows), measured
  // at N = 4096, K = 3072, M = 32 without -> with: MXFP4 5.42 -> 5.26 us,
  // FP8 6.15 -> 6.06 us, INT4 5.39 -> 5.71 us (INT4_ASYM follows INT4)
  else if constexpr (MT == 1 && NTW == 2) return F == KF_MXFP4 || F == KF_FP8;
  // 32-row tiles: MXFP4 and NVFP4 as above; the static FP8 GEMM measured
  // 5.95 -> 5.63 us (its 16-row blocks, 5.72 us, lost)
  else return F == KF_MXFP4 || F == KF_NVFP4 || F == KF_FP8S;
}

// K-split plan of one workgroup: NW waves x SPW macro-steps each per block;
// the S workgroups of a column tile interleave their blocks.
//
// Template parameters: F format, MT 16-row tiles, NTW 16-column tiles per wave,
// NW waves per workgroup, SPW macro-steps whose loads are issued together, WL
// weight layout.
template <int F, int MT, int NTW, int NW, int SPW, bool XLDS, int WL>
__global__ __launch_bounds__(NW * 64) void k_linear(LinearArgs a, int S) {
  constexpr int KPL = FmtT<F>::KPL;
  constexpr int MACRO = 4 * KPL;
  constexpr bool ACT8 = (F == KF_FP8S);
  constexpr int XL = ACT8 ? 1 : KPL / 8;  // 16-byte activation loads per m-tile per step
  constexpr int NT = 16 * NTW;            // columns per workgroup
  constexpr int E = MT * 16 * NT;         // outputs per workgroup
  constexpr int NTHR = NW * 64;
  using XS = XStage<F, MT>;
  static_assert(!XLDS || XS::R * MT * XL == 16 * MT, "XLDS: load instructions must cover the slice rows");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* red = reinterpret_cast<float*>(smem + xslots_bytes<F, MT, NTW, NW, WL, SPW>(XLDS));
  constexpr bool XDMA = XLDS && x_dma<F, MT, NTW, WL>();

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int n0 = blockIdx.x * NT;
  const int split = blockIdx.y;
  const int m0 = blockIdx.z * (16 * MT);
  const int M = a.M, N = a.N, K = a.K;
  const int T = (K + MACRO - 1) / MACRO;
  const uint32_t wrow = (uint32_t)kbyte<F>(K);

  const __amdgpu_buffer_rsrc_t Wr = make_rsrc(a.W, (uint32_t)N * wrow);
  const __amdgpu_buffer_rsrc_t Xr = make_rsrc(a.X, (uint32_t)M * (uint32_t)K * (ACT8 ? 1u : 2u));
  uint32_t sbytes = 0;
  if constexpr (F == KF_INT4) sbytes = (uint32_t)N * (uint32_t)(K / 128) * 2u;
  else if constexpr (F == KF_INT4A) sbytes = (uint32_t)N * (uint32_t)(K / 128) * 4u;
  else if constexpr (F == KF_NVFP4) sbytes = (uint32_t)N * (uint32_t)(K / 16);
  else if constexpr (F == KF_MXFP4) sbytes = (uint32_t)N * (uint32_t)(K / 32);
  else if constexpr (F == KF_FP8 || F == KF_FP8S) sbytes = (uint32_t)N * 4u;
  const __amdgpu_buffer_rsrc_t Sr = make_rsrc(a.scales ? a.scales : a.W, a.scales ? sbytes : 0u);
  const __amdgpu_buffer_rsrc_t Br = make_rsrc(a.bias ? (const void*)a.bias : a.W, a.bias ? (uint32_t)N * 2u : 0u);

  // epilogue operands of this thread's column, fetched early so they travel
  // with the main loads
  const int ecol = tid % NT;
  const int en = n0 + ecol;
  const uint32_t bias_bits = bload16(Br, (uint32_t)en * 2u);
  uint32_t cs_bits = 0x3F800000u;  // 1.0f
  if constexpr (F == KF_FP8 || F == KF_FP8S) cs_bits = bload32(Sr, (uint32_t)en * 4u);
  const float uscale = Epilogue<F>::uniform_scale(a);
  // Block scales in tile order (MXFP4, NVFP4) load as one aligned dword per
  // lane and tile; the decode shifts the lane's bytes down (ssh, the same for
  // every tile and K step).  A byte or half-word load per lane cost the
  // address unit as much as a 16-byte one: measured at N = 4096, K = 3072,
  // M = 32, MXFP4 5.43 -> 5.26 us and NVFP4 6.06 -> 5.98 us.
  constexpr bool DWS = WL == kLayoutTiles && (F == KF_MXFP4 || F == KF_NVFP4);
  uint32_t ssh = 0u;
  if constexpr (DWS) ssh = (F == KF_MXFP4) ? 8u * (uint32_t)g : 16u * (uint32_t)(g & 1);

  f32x4 acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // No-split tiles rotate their waves' K blocks by workgroup, so that the
  // CUs of an XCD do not all request the same activation and weight lines at
  // once (measured at N = 4096, K = 3072, M = 32: FP8 7.4 -> 7.15-7.25 us,
  // the other formats unchanged; the one/two-row kernel keeps the plain order)
  const int rot = (XLDS && S == 1) ? (int)(blockIdx.x % NW) : 0;  // K-block rotation of the waves
  const int wi = (XLDS && S == 1) ? (wave + rot) % NW : split * NW + wave;
  constexpr bool WFB = XLDS && weights_first<F, WL, MT, NTW>();
  // early weight decode: weights-first tiles of the float weight formats
  // whose decoded weights fit beside the activations in registers (at most
  // 64 VGPRs of them, and 16 or 32 rows x one or two 16-column tiles: with two
  // row tiles and two column tiles it spilled 13-27 registers)
  constexpr int EDJ = (F == KF_FP8) ? 2 : 4;  // decoded 8-element chunks per tile and K step
  constexpr bool EDW = WFB && (F == KF_NVFP4 || F == KF_MXFP4 || F == KF_FP8) && MT * NTW <= 2 &&
                       SPW * NTW * EDJ <= 16;
  for (int blk = wi; blk * SPW < T; blk += S * NW) {
    // ---- issue every load of this block before any wait: the activation
    // slices (cache hits; loads return in issue order, so their LDS staging
    // can start while the weight stream is still in flight) and the packed
    // weights and block scales
    u32x4 w[SPW][NTW];
    u32x4 xv[SPW][MT][XL];
    uint32_t sc[SPW][NTW];
    auto load_x = [&]() {
      // XDMA: the slots' reads of the previous pass are done before they refill
      if constexpr (XDMA) __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
      for (int st = 0; st < SPW; ++st) {
        const int kl = (blk * SPW + st) * MACRO + g * KPL;
        const bool kv = kl < K;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const uint32_t m = (uint32_t)(m0 + 16 * i + c);
#pragma unroll
          for (int j = 0; j < XL; ++j) {
            if constexpr (XDMA) {
              // instruction q fills rows q*R .. q*R+R-1 of step st's slot:
              // lane L writes position L % L_ of its row, so it loads the
              // chunk the slot map puts there (the map is its own inverse)
              const int q = i * XL + j;
              const int rr = q * XS::R + lane / XS::L;
              const uint32_t row = (uint32_t)(m0 + rr);
              const int kx = (blk * SPW + st) * MACRO + XS::pos(rr, lane % XS::L) * (16 / XS::XB);
              unsigned char* dst = smem + (wave * SPW + st) * XS::SLOT + q * 1024;
              __builtin_amdgcn_raw_ptr_buffer_load_lds(
                  Xr, (__attribute__((address_space(3))) void*)dst, 16,
                  off_if(kx < K, (row * (uint32_t)K + (uint32_t)kx) * (uint32_t)XS::XB), 0, 0, 0);
            } else if constexpr (XLDS) {
              // contiguous: instruction q covers rows q*R .. q*R+R-1 of the slice
              const int q = i * XL + j;
              const uint32_t row = (uint32_t)(m0 + q * XS::R + lane / XS::L);
              const int kx = (blk * SPW + st) * MACRO + (lane % XS::L) * (16 / XS::XB);
              xv[st][i][j] = bload128(Xr, off_if(kx < K, (row * (uint32_t)K + (uint32_t)kx) * (uint32_t)XS::XB));
            } else if constexpr (ACT8) {
              xv[st][i][j] = bload128(Xr, off_if(kv, m * (uint32_t)K + (uint32_t)kl));
            } else {
              xv[st][i][j] = bload128(Xr, off_if(kv, (m * (uint32_t)K + (uint32_t)kl + 8u * j) * 2u));
            }
          }
        }
      }
    };
    auto load_w = [&]() {
#pragma unroll
      for (int st = 0; st < SPW; ++st) {
        const int kl = (blk * SPW + st) * MACRO + g * KPL;
        const bool kv = kl < K;
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const uint32_t n = (uint32_t)(n0 + 16 * t + c);
          // 4-bit weights stream past the caches (non-temporal), which keeps
          // the activations, read by every workgroup, resident: measured at
          // N = 4096, K = 3072, M = 32: INT4 6.7 -> 6.55 us, NVFP4 7.4 -> 7.2,
          // MXFP4 6.8 -> 6.7.  FP8 gained nothing at M = 32 with 32-row blocks
          // in the rows layout and lost 0.3 us at M = 1, but gains in tile
          // order with 16-row blocks (6.20 -> 5.94 us), where it is used
          const uint32_t wo = off_if(kv, w_off<WL>(n, (uint32_t)kbyte<F>(kl), wrow));
          if constexpr (F == KF_INT4 || F == KF_INT4A || F == KF_NVFP4 || F == KF_MXFP4 ||
                        (F == KF_FP8 && WL == kLayoutTiles && MT == 1 && NTW == 2))
            w[st][t] = bload128_nt(Wr, wo);
          else
            w[st][t] = bload128(Wr, wo);
          // (NVFP4: the lane's 32 K span two 16-K blocks, whose scales are
          // adjacent bytes in both layouts)
          if constexpr (DWS)
            sc[st][t] = bload32(Sr, off_if(kv, s_off<F, WL>(n, (uint32_t)kl, (uint32_t)K) & ~3u));
          else if constexpr (F == KF_INT4 || F == KF_NVFP4)
            sc[st][t] = bload16(Sr, off_if(kv, s_off<F, WL>(n, (uint32_t)kl, (uint32_t)K)));
          else if constexpr (F == KF_INT4A)
            sc[st][t] = bload32(Sr, off_if(kv, s_off<F, WL>(n, (uint32_t)kl, (uint32_t)K)));
          else if constexpr (F == KF_MXFP4)
            sc[st][t] = bload8(Sr, off_if(kv, s_off<F, WL>(n, (uint32_t)kl, (uint32_t)K)));
          else
            sc[st][t] = 0u;
        }
      }
    };
    if constexpr (WFB) {
      load_w();
      __builtin_amdgcn_sched_barrier(0);
      if (blk == wi) __builtin_amdgcn_s_barrier();  // once per wave (see after the loop)
      __builtin_amdgcn_sched_barrier(0);
      load_x();
    } else if constexpr (F == KF_NVFP4) {
      // NVFP4 issues its weights first per wave: measured at N = 4096,
      // K = 3072, M = 32, 7.3-7.4 -> 7.0-7.1 us
      load_w();
      load_x();
    } else {
      load_x();
      load_w();
    }
    // Keep every load above in flight together: left alone, the scheduler
    // sinks them towards their uses to save registers, which leaves only 6-10
    // of the ~20 loads of a wave outstanding at a time.
    __builtin_amdgcn_sched_barrier(0);

    // Early decode (EDW): the weights were issued before the activations and
    // land first, so the float formats decode them while the activation loads
    // are still in flight.  Same values, same MFMA order.  Measured at
    // N = 4096, K = 3072, M = 32: NVFP4 6.14-6.28 -> 6.07-6.17 us, MXFP4 5.29
    // -> 5.11 us, FP8 6.20 -> 6.03 us.
    bf16x8 bw[EDW ? SPW : 1][EDW ? NTW : 1][EDW ? EDJ : 1];
    if constexpr (EDW) {
#pragma unroll
      for (int st = 0; st < SPW; ++st)
#pragma unroll
        for (int t = 0; t < NTW; ++t)
#pragma unroll
          for (int j = 0; j < EDJ; ++j) {
            if constexpr (F == KF_NVFP4)
              bw[st][t][j] = dec_fp4_mul(w[st][t][j], e4m3_decode((sc[st][t] >> (ssh + (j < 2 ? 0u : 8u))) & 0xFFu));
            else if constexpr (F == KF_MXFP4)
              bw[st][t][j] = dec_fp4_pow2(w[st][t][j], e8m0_decode((sc[st][t] >> ssh) & 0xFFu));
            else
              bw[st][t][j] = dec_fp8(w[st][t][2 * j], w[st][t][2 * j + 1]);
          }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- decode and multiply
    // XDMA: every activation load of the block has landed in LDS (they were
    // issued after the weights, whose registers the decode has waited for)
    if constexpr (XDMA) __builtin_amdgcn_s_waitcnt(kWaitVm0);
#pragma unroll
    for (int st = 0; st < SPW; ++st) {
      if constexpr (XLDS) {
        // through this wave's LDS slot into the operand layout (a wave's LDS
        // operations execute in order, so no barrier is needed here)
        unsigned char* slot = smem + (wave * (XDMA ? SPW : 1) + (XDMA ? st : 0)) * XS::SLOT;
        if constexpr (!XDMA) {
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < XL; ++j) {
              const int row = (i * XL + j) * XS::R + lane / XS::L;
              *reinterpret_cast<u32x4*>(slot + row * XS::ROWB + XS::pos(row, lane % XS::L) * 16) = xv[st][i][j];
            }
        }
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < XL; ++j)
            xv[st][i][j] = *reinterpret_cast<const u32x4*>(
                slot + (16 * i + c) * XS::ROWB + XS::pos(16 * i + c, (g * KPL + 8 * j) * XS::XB / 16) * 16);
      }
      if constexpr (F == KF_INT4 || F == KF_INT4A) {
        // bias: 136 for signed codes (XOR 8), 128 + zero-point for unsigned ones
        f32x4 tmp[MT][NTW], rs[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          rs[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < NTW; ++t) tmp[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const bf16x8 ones = as_bf16x8(u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x8 b[NTW];
#pragma unroll
          for (int t = 0; t < NTW; ++t) b[t] = (F == KF_INT4) ? dec_int4_biased(w[st][t][j]) : dec_uint4_biased(w[st][t][j]);
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            const bf16x8 A = as_bf16x8(xv[st][i][j]);
            rs[i] = mfma_bf16(A, ones, rs[i]);
#pragma unroll
            for (int t = 0; t < NTW; ++t) tmp[i][t] = mfma_bf16(A, b[t], tmp[i][t]);
          }
        }
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const float s = bitsf(sc[st][t] << 16);
          const float nb = (F == KF_INT4) ? -136.f : -(float)(128u + ((sc[st][t] >> 16) & 15u));
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][t][r] = fmaf(s, fmaf(nb, rs[i][r], tmp[i][t][r]), acc[i][t][r]);
        }
      } else if constexpr (F == KF_NVFP4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x8 b[NTW];
#pragma unroll
          for (int t = 0; t < NTW; ++t) {
            if constexpr (EDW) b[t] = bw[st][t][j];
            else b[t] = dec_fp4_mul(w[st][t][j], e4m3_decode((sc[st][t] >> (ssh + (j < 2 ? 0u : 8u))) & 0xFFu));
          }
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int t = 0; t < NTW; ++t) acc[i][t] = mfma_bf16(as_bf16x8(xv[st][i][j]), b[t], acc[i][t]);
        }
      } else if constexpr (F == KF_MXFP4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x8 b[NTW];
#pragma unroll
          for (int t = 0; t < NTW; ++t) {
            if constexpr (EDW) b[t] = bw[st][t][j];
            else b[t] = dec_fp4_pow2(w[st][t][j], e8m0_decode((sc[st][t] >> ssh) & 0xFFu));
          }
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int t = 0; t < NTW; ++t) acc[i][t] = mfma_bf16(as_bf16x8(xv[st][i][j]), b[t], acc[i][t]);
        }
      } else if constexpr (F == KF_FP8) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          bf16x8 b[NTW];
#pragma unroll
          for (int t = 0; t < NTW; ++t) {
            if constexpr (EDW) b[t] = bw[st][t][j];
            else b[t] = dec_fp8(w[st][t][2 * j], w[st][t][2 * j + 1]);
          }
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int t = 0; t < NTW; ++t) acc[i][t] = mfma_bf16(as_bf16x8(xv[st][i][j]), b[t], acc[i][t]);
        }
      } else if constexpr (F == KF_BF16) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int t = 0; t < NTW; ++t) acc[i][t] = mfma_bf16(as_bf16x8(xv[st][i][0]), as_bf16x8(w[st][t]), acc[i][t]);
      } else {  // KF_FP8S: E4M3 activations x E4M3 weights
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int t = 0; t < NTW; ++t)
              acc[i][t] = mfma_fp8(xv[st][i][0][2 * j], xv[st][i][0][2 * j + 1], w[st][t][2 * j],
                                   w[st][t][2 * j + 1], acc[i][t]);
      }
    }
  }

  // a wave without a K block still meets the weights-first barrier once
  if constexpr (WFB) {
    if (wi * SPW >= T) __builtin_amdgcn_s_barrier();
  }

  // ---- reduce the wave partials: every wave stores its tile (one 16-byte
  // vector per lane and MFMA tile), then thread tid sums the NW partials of
  // the outputs e = tid + q * NTHR (row-major in the workgroup tile, column
  // n0 + tid % NT) in the order of their K blocks (wave (j - rot) mod NW holds
  // block j), so that every tile configuration with the same K blocks per
  // wave adds the same partials in the same order and gives the same bits.
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NTW; ++t)
      *reinterpret_cast<f32x4*>(red + ((wave * MT * NTW + i * NTW + t) * 64 + lane) * 4) = acc[i][t];
  __syncthreads();
  constexpr int EPT = (E + NTHR - 1) / NTHR;
  float v[EPT];
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    const int e = tid + q * NTHR;
    const int row = e / NT, col = e % NT;
    // lane (g, c) of MFMA tile (i, t) holds rows 16i + 4g + r, column 16t + c
    const int idx = (((row >> 4) * NTW + (col >> 4)) * 64 + 16 * ((row >> 2) & 3) + (col & 15)) * 4 + (row & 3);
    float sum = 0.f;
    if (e < E) {
#pragma unroll
      for (int j = 0; j < NW; ++j) sum += red[((j + NW - rot) % NW) * E + idx];
    }
    v[q] = sum;
  }
  if (S == 1) {
    const Epilogue<F> ep(en, bias_bits, cs_bits, uscale);
#pragma unroll
    for (int q = 0; q < EPT; ++q) ep.store(a, m0, en, tid + q * NTHR, E, NT, v[q]);
    return;
  }
  // ---- split-K: publish this workgroup's partial (thread-major, 16-byte
  // vectors); k_splitk_reduce, launched next on the same stream, sums the S
  // partials of each tile in a fixed order.  Stream order makes the partials
  // visible to it without any device-wide fence here.
  constexpr int V4 = (EPT + 3) / 4;
  const int tile = blockIdx.z * gridDim.x + blockIdx.x;
  float* mine = a.part + ((int64_t)tile * S + split) * (NTHR * V4 * 4);
#pragma unroll
  for (int q4 = 0; q4 < V4; ++q4) {
    f32x4 o{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * q4 + r < EPT) o[r] = v[4 * q4 + r];
    *reinterpret_cast<f32x4*>(mine + (tid * V4 + q4) * 4) = o;
  }
}

// Sums the S split-K partials of each column tile (same thread mapping as the
// producing kernel) and applies the epilogue.  All partial loads of a thread
// are issued before the first add.
template <int F, int MT, int NTW, int NW>
__global__ __launch_bounds__(NW * 64) void k_splitk_reduce(LinearArgs a, int S) {
  constexpr int NT = 16 * NTW;
  constexpr int E = MT * 16 * NT;
  constexpr int NTHR = NW * 64;
  constexpr int EPT = (E + NTHR - 1) / NTHR;
  constexpr int V4 = (EPT + 3) / 4;
  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * NT, m0 = blockIdx.z * (16 * MT);
  const int en = n0 + tid % NT;
  const int N = a.N;
  const __amdgpu_buffer_rsrc_t Br = make_rsrc(a.bias ? (const void*)a.bias : a.W, a.bias ? (uint32_t)N * 2u : 0u);
  const uint32_t bias_bits = bload16(Br, (uint32_t)en * 2u);
  uint32_t cs_bits = 0x3F800000u;
  if constexpr (F == KF_FP8 || F == KF_FP8S) {
    const __amdgpu_buffer_rsrc_t Sr = make_rsrc(a.scales, (uint32_t)N * 4u);
    cs_bits = bload32(Sr, (uint32_t)en * 4u);
  }
  const int tile = blockIdx.z * gridDim.x + blockIdx.x;
  const uint32_t slab = (uint32_t)(NTHR * V4 * 16);
  const __amdgpu_buffer_rsrc_t Pr = make_rsrc(a.part + (int64_t)tile * S * (NTHR * V4 * 4), (uint32_t)S * slab);
  u32x4 pv[kMaxSplit][V4];
#pragma unroll
  for (int s2 = 0; s2 < kMaxSplit; ++s2)
#pragma unroll
    for (int q4 = 0; q4 < V4; ++q4) pv[s2][q4] = bload128(Pr, (uint32_t)s2 * slab + (uint32_t)(tid * V4 + q4) * 16u);
  float v[EPT];
#pragma unroll
  for (int q = 0; q < EPT; ++q) v[q] = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < kMaxSplit; ++s2)
#pragma unroll
    for (int q = 0; q < EPT; ++q) v[q] += bitsf(pv[s2][q / 4][q % 4]);
  const Epilogue<F> ep(en, bias_bits, cs_bits, Epilogue<F>::uniform_scale(a));
#pragma unroll
  for (int q = 0; q < EPT; ++q) ep.store(a, m0, en, tid + q * NTHR, E, NT, v[q]);
}

// Steps per wave whose loads are issued together: one 16-byte weight chunk
// per tile and step, sized so that a no-split workgroup of 12 waves covers a
// 3072-deep K in one pass.
template <int F>
constexpr int spw_nosplit() {
  return (F == KF_BF16) ? 8 : ((F == KF_FP8 || F == KF_FP8S) ? 4 : 2);
}
template <int F>
constexpr int spw_split() {
  return (F == KF_BF16) ? 4 : ((F == KF_FP8 || F == KF_FP8S) ? 2 : 1);
}

// 64-column tiles (NTW = 4) run 8 waves of 1.5x the K: at 12 waves their
// loads and accumulators spilled registers.
template <int F, int MT, int NTW, int WL>
hipError_t launch_nosplit(const LinearArgs& a, dim3 grid, hipStream_t s) {
  constexpr int NW = (NTW == 4) ? 8 : 12;
  constexpr int SPW = spw_nosplit<F>() * 12 / NW;
  constexpr int sm = smem_bytes<F, MT, NTW, NW, WL, SPW>(true);
  static_assert(sm <= 160 * 1024, "no-split tile exceeds the LDS of a CU");
  static std::atomic<int> done{0};
  auto k = k_linear<F, MT, NTW, NW, SPW, true, WL>;
  hipError_t e = allow_smem(k, sm, done);
  if (e != hipSuccess) return e;
  k<<<grid, NW * 64, sm, s>>>(a, 1);
  return hipGetLastError();
}

template <int F, int MT, int WL>
hipError_t launch_mt(const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  dim3 grid(p.gx, p.S, p.gz);
  if (p.cfg == kCfgSplit) {
    constexpr int sm = smem_bytes<F, MT, 4, 4, WL, spw_split<F>()>(false);
    k_linear<F, MT, 4, 4, spw_split<F>(), false, WL><<<grid, 256, sm, s>>>(a, p.S);
    if (p.S > 1) k_splitk_reduce<F, MT, 4, 4><<<dim3(p.gx, 1, p.gz), 256, 0, s>>>(a, p.S);
  } else {
    if constexpr (MT == 1) {
      if (a.M <= 2) {
        // one or two rows: the activation slice is a few KiB, and loading it
        // in the operand layout directly beats staging it through LDS; with
        // so little work per column tile, 6 waves of twice the K beat 12
        // (measured at N = 4096, K = 3072, MXFP4, M = 1, weights in cache:
        // 12 waves staged 5.2 us, direct 5.0 us, 6 waves direct 4.5 us; with
        // cold weights both direct forms take 4.8 us; from four rows up the
        // 12 staged waves win)
        constexpr int sm = smem_bytes<F, MT, 1, 6, WL, 2 * spw_nosplit<F>()>(false);
        k_linear<F, MT, 1, 6, 2 * spw_nosplit<F>(), false, WL><<<grid, 384, sm, s>>>(a, p.S);
        return hipGetLastError();
      }
    }
    // no-split tiles with activations staged through LDS
    if constexpr (MT == 1 && WL == kLayoutTiles && (F == KF_INT4 || F == KF_INT4A || F == KF_MXFP4 || F == KF_FP8)) {
      if (p.ntw == 2) return launch_nosplit<F, MT, 2, WL>(a, grid, s);
    }
    if constexpr (MT == 2) {
      if (p.ntw == 2) return launch_nosplit<F, MT, 2, WL>(a, grid, s);
      if constexpr (F != KF_BF16 && F != KF_FP8S) {
        if (p.ntw == 4) return launch_nosplit<F, MT, 4, WL>(a, grid, s);
      }
    }
    return launch_nosplit<F, MT, 1, WL>(a, grid, s);
  }
  return hipGetLastError();
}

template <int F>
hipError_t launch_f(const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  if constexpr (F != KF_BF16) {
    if (a.wl == kLayoutTiles) return p.mt == 1 ? launch_mt<F, 1, kLayoutTiles>(a, p, s) : launch_mt<F, 2, kLayoutTiles>(a, p, s);
  }
  return p.mt == 1 ? launch_mt<F, 1, kLayoutRows>(a, p, s) : launch_mt<F, 2, kLayoutRows>(a, p, s);
}

}  // namespace

hipError_t launch_linear(int kfmt, const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  if (p.cfg == kCfgTiled) return launch_gemm_tiled(kfmt, a, p, s);
  if (p.cfg == kCfgMid) return launch_gemm_mid(kfmt, a, s);
  switch (kfmt) {
    case KF_BF16: return launch_f<KF_BF16>(a, p, s);
    case KF_INT4: return launch_f<KF_INT4>(a, p, s);
    case KF_INT4A: return launch_f<KF_INT4A>(a, p, s);
    case KF_FP8: return launch_f<KF_FP8>(a, p, s);
    case KF_NVFP4: return launch_f<KF_NVFP4>(a, p, s);
    case KF_MXFP4: return launch_f<KF_MXFP4>(a, p, s);
    case KF_FP8S: return launch_f<KF_FP8S>(a, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wq
