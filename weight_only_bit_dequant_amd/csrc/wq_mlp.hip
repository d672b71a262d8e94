// Fused two-layer static-FP8 MLP: Q -> FP8 GEMM -> bf16 -> Q -> FP8 GEMM in one
// kernel.
//
// "TorchAO Static FP8 Quantization (Linear)": the page's model is
// Linear(256, 512) -> Linear(512, 128); after calibration each Linear input
// gets a static Q node (activation scale) and both GEMMs run in FP8.  The
// unfused path launches four kernels (act Q, GEMM, act Q, GEMM) and writes
// the bf16 hidden layer to memory between them.  Here one workgroup of 16
// waves owns 16 rows and keeps them on chip end to end:
//   1. X rows -> E4M3 codes with act_scale1 (fp32 division, clamp, nearest
//      even) into LDS;
//   2. layer 1 on v_mfma_f32_16x16x32_fp8_fp8 over K1; epilogue
//      h = bf16(acc * act_scale1 * w1_scale[n] (+ b1)), then the layer-2 Q
//      (h / act_scale2 -> E4M3) straight into LDS;
//   3. layer 2 the same way over the hidden codes; y = bf16(acc * act_scale2 *
//      w2_scale[n] (+ b2)) is the only store.
// Two forms: a single-pass kernel for models one workgroup covers in one pass
// (the page's model), with every global load issued up front, and a looped
// kernel for larger layers (up to the LDS limit).  Every step uses the
// unfused path's arithmetic, so results differ from it only through the order
// of fp32 accumulation.
#include "wq_kernel_common.hpp"

namespace wq {

namespace {

__device__ __forceinline__ u32x2 bload64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}

constexpr int kWaves = 16;  // 1024 threads: every wave keeps its weight loads in flight at once
constexpr int kTPW = 2;     // 16-column tiles per wave and pass

// Weight codes of one 256-K chunk for kTPW 16-column tiles: lane (g, c) holds
// 8 codes of row n0[j] + c at K k0 + 32s + 8g (s = 0..7).  Rows past N and K
// past the end read zero.
struct Chunk {
  u32x2 b[kTPW][8];
};

__device__ __forceinline__ void load_chunk(Chunk& ch, __amdgpu_buffer_rsrc_t Br, const int* n0, int K, int k0, int g,
                                           int c) {
#pragma unroll
  for (int j = 0; j < kTPW; ++j)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int k = k0 + 32 * s + 8 * g;
      ch.b[j][s] = bload64(Br, off_if(k < K, (uint32_t)(n0[j] + c) * (uint32_t)K + (uint32_t)k));
    }
}

// acc[j] += A (16 rows of codes in LDS, row stride RS) x chunk; K past the
// end multiplies zero codes on both sides (the LDS rows are zero-padded)
__device__ __forceinline__ void mma_chunk(const unsigned char* A, int RS, const Chunk& ch, int k0, int g, int c,
                                          f32x4* acc) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const u32x2 a = *reinterpret_cast<const u32x2*>(A + c * RS + k0 + 32 * s + 8 * g);
#pragma unroll
    for (int j = 0; j < kTPW; ++j) acc[j] = mfma_fp8(a.x, a.y, ch.b[j][s].x, ch.b[j][s].y, acc[j]);
  }
}

// Single-pass form, for models whose layers one workgroup covers in one pass
// (K1 <= 256, N1 <= 512, N2 <= 128; the page's 256 -> 512 -> 128 model).
// Every global load of the kernel -- X, the wave's weight rows of both
// layers, the epilogue operands -- is issued before the first wait, so the
// MLP costs one memory round trip.  Weight rows are read as whole 256-byte
// K spans (16 lanes x 16 bytes per row, four rows per load: contiguous cache
// lines) and reach the matrix-core layout through a wave-private LDS slab
// (one row per lane group there), which the wave reuses for layer 2.  Layer 2
// splits its K (= N1) into 256-wide slices across waves; the slices' fp32
// partial sums meet in LDS and are added in slice order.
constexpr int kSpK1 = 256, kSpN1 = 512, kSpN2 = 128;
constexpr int kSpRS1 = kSpK1 + 16, kSpRS2 = kSpN1 + 16;  // code-row strides (bytes)
constexpr int kSpPS = kSpN2 + 4;                        // partial-sum row stride (floats)
constexpr int kSpSlab = 32 * 256;                       // per wave: 32 weight rows x 256 codes
constexpr size_t kSpSmem = (size_t)kWaves * kSpSlab + 16 * (kSpRS1 + kSpRS2) + 2 * 16 * kSpPS * 4;
static_assert(kSpSmem <= 160 * 1024, "single-pass MLP exceeds the LDS of a CU");

// Byte offset of 16-byte piece q of row r in a slab: pieces XOR-swizzled by
// the row so that 16 lanes reading one piece index of 16 rows hit all banks.
__device__ __forceinline__ int slab_off(int r, int q) { return r * 256 + ((q ^ (r & 15)) << 4); }

// Load 32 weight rows of up to 256 codes; row r starts at byte base + r *
// stride, codes at K >= klen and rows past the resource read zero.  Load i,
// lane L -> row 4i + L/16, 16-byte piece L%16.
__device__ __forceinline__ void load_slab(u32x4* v, __amdgpu_buffer_rsrc_t r, uint32_t base, uint32_t stride, int klen,
                                          int lane) {
  const int q = lane & 15;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 4 * i + (lane >> 4);
    v[i] = bload128(r, off_if(16 * q < klen, base + (uint32_t)row * stride + 16u * q));
  }
}
__device__ __forceinline__ void store_slab(unsigned char* slab, const u32x4* v, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(slab + slab_off(4 * i + (lane >> 4), lane & 15)) = v[i];
}
// acc[j] += A (16 code rows in LDS, stride RS, from column k0) x slab rows
// 16j..16j+15 over 256 K
__device__ __forceinline__ void mma_slab(const unsigned char* A, int RS, int k0, const unsigned char* slab, int g, int c,
                                         f32x4* acc) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const u32x2 a = *reinterpret_cast<const u32x2*>(A + c * RS + k0 + 32 * s + 8 * g);
#pragma unroll
    for (int j = 0; j < kTPW; ++j) {
      const u32x2 b = *reinterpret_cast<const u32x2*>(slab + slab_off(16 * j + c, 2 * s + (g >> 1)) + 8 * (g & 1));
      acc[j] = mfma_fp8(a.x, a.y, b.x, b.y, acc[j]);
    }
  }
}

__global__ __launch_bounds__(kWaves * 64) void k_static_mlp2_sp(Mlp2Args a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int m0 = blockIdx.x * 16;
  const int K1 = a.K1, N1 = a.N1, N2 = a.N2;
  unsigned char* slab = smem + wave * kSpSlab;                                // [32][256], this wave's
  unsigned char* Xq = smem + kWaves * kSpSlab;                                // [16][kSpRS1]
  unsigned char* Hq = Xq + 16 * kSpRS1;                                       // [16][kSpRS2]
  float* P = reinterpret_cast<float*>(Hq + 16 * kSpRS2);                      // [2][16][kSpPS]
  const float s1 = a.act_scale1[0], s2 = a.act_scale2[0];

  // ---- all global loads (rows past M, columns past N and K past the end
  // read zero)
  // X: threads 0..511 take 8 elements of row tid/32 at K 8*(tid%32), the whole
  // 256-wide LDS row (zeros past K1)
  const int xr = tid >> 5, xk = (tid & 31) * 8;
  const __amdgpu_buffer_rsrc_t Xr = make_rsrc(a.X, (uint32_t)a.M * (uint32_t)K1 * 2u);
  const u32x4 xv = bload128(Xr, off_if(xr < 16 && xk < K1, ((uint32_t)(m0 + xr) * (uint32_t)K1 + (uint32_t)xk) * 2u));
  // layer 1: hidden columns 32*wave .. +31 (two 16-column tiles), all of K1
  u32x4 w1[8];
  load_slab(w1, make_rsrc(a.W1, (uint32_t)N1 * (uint32_t)K1), (uint32_t)(32 * wave) * (uint32_t)K1, (uint32_t)K1, K1,
            lane);
  const __amdgpu_buffer_rsrc_t S1r = make_rsrc(a.w1_scale, (uint32_t)N1 * 4u);
  const __amdgpu_buffer_rsrc_t B1r = make_rsrc(a.b1, a.b1 ? (uint32_t)N1 * 2u : 0u);
  uint32_t e1s[kTPW], e1b[kTPW];
#pragma unroll
  for (int j = 0; j < kTPW; ++j) {
    const uint32_t n = (uint32_t)(32 * wave + 16 * j + c);
    e1s[j] = bload32(S1r, n * 4u);
    e1b[j] = bload16(B1r, n * 2u);
  }
  // layer 2: unit = (column pair tp, K slice sl); slices past N1 read zero
  const int TP2 = (N2 + 31) / 32, nsl = (N1 + 255) / 256;
  const int sl = wave / TP2, tp = wave - sl * TP2;
  u32x4 w2[8];
  load_slab(w2, make_rsrc(a.W2, (uint32_t)N2 * (uint32_t)N1), (uint32_t)(32 * tp) * (uint32_t)N1 + 256u * sl,
            (uint32_t)N1, N1 - 256 * sl, lane);
  // final epilogue: thread takes outputs tid and tid + 1024 of the 16 x N2 block
  const __amdgpu_buffer_rsrc_t S2r = make_rsrc(a.w2_scale, (uint32_t)N2 * 4u);
  const __amdgpu_buffer_rsrc_t B2r = make_rsrc(a.b2, a.b2 ? (uint32_t)N2 * 2u : 0u);
  uint32_t e2s[2], e2b[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int o = tid + i * kWaves * 64, n = o % N2;
    e2s[i] = bload32(S2r, off_if(o < 16 * N2, (uint32_t)n * 4u));
    e2b[i] = bload16(B2r, off_if(o < 16 * N2, (uint32_t)n * 2u));
  }

  // ---- X -> E4M3 codes; layer-1 weight rows -> the wave's slab
  if (xr < 16) {
    *reinterpret_cast<u32x2*>(Xq + xr * kSpRS1 + xk) = act_q8(xv, s1);
  }
  store_slab(slab, w1, lane);
  __syncthreads();

  // ---- layer 1 -> hidden codes; every column below 512 is written (zero
  // past N1), so layer 2's K tail multiplies zeros
  {
    f32x4 acc[kTPW];
#pragma unroll
    for (int j = 0; j < kTPW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    mma_slab(Xq, kSpRS1, 0, slab, g, c, acc);
#pragma unroll
    for (int j = 0; j < kTPW; ++j) {
      const int n = 32 * wave + 16 * j + c;
      const float ws = bitsf(e1s[j]), b = bitsf(e1b[j] << 16);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float h = bf16_to_f32(f32_to_bf16((acc[j][r] * s1) * ws + b));
        Hq[(4 * g + r) * kSpRS2 + n] = n < N1 ? (uint8_t)act_q(h, s2) : (uint8_t)0;
      }
    }
  }
  // the wave's layer-1 slab reads are done (in-order LDS per wave): reuse it
  store_slab(slab, w2, lane);
  __syncthreads();

  // ---- layer 2 partial sums of slice sl -> LDS
  if (sl < nsl) {
    f32x4 acc[kTPW];
#pragma unroll
    for (int j = 0; j < kTPW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    mma_slab(Hq, kSpRS2, 256 * sl, slab, g, c, acc);
#pragma unroll
    for (int j = 0; j < kTPW; ++j) {
      const int n = 32 * tp + 16 * j + c;
      if (n < N2) {
#pragma unroll
        for (int r = 0; r < 4; ++r) P[(sl * 16 + 4 * g + r) * kSpPS + n] = acc[j][r];
      }
    }
  }
  __syncthreads();

  // ---- slices summed in order, epilogue, the only store
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int o = tid + i * kWaves * 64;
    if (o < 16 * N2) {
      const int row = o / N2, n = o - row * N2;
      float v = P[row * kSpPS + n];
      if (nsl > 1) v += P[(16 + row) * kSpPS + n];
      if (m0 + row < a.M)
        a.Y[(int64_t)(m0 + row) * N2 + n] = f32_to_bf16((v * s2) * bitsf(e2s[i]) + bitsf(e2b[i] << 16));
    }
  }
}

__global__ __launch_bounds__(kWaves * 64) void k_static_mlp2(Mlp2Args a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int NTHR = kWaves * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int m0 = blockIdx.x * 16;
  const int K1 = a.K1, N1 = a.N1, N2 = a.N2;
  // LDS: X codes [16][RS1], hidden codes [16][RS2] (rows padded to a multiple
  // of 256 codes + 16 bytes against bank conflicts; the padding stays zero),
  // then the column operands of both epilogues (scale, bias) as fp32
  const int RS1 = (K1 + 255) / 256 * 256 + 16, RS2 = (N1 + 255) / 256 * 256 + 16;
  unsigned char* Xq = smem;
  unsigned char* Hq = smem + 16 * RS1;
  float* E1 = reinterpret_cast<float*>(Hq + 16 * RS2);  // [2][N1]: w1_scale, b1
  float* E2 = E1 + 2 * N1;                              // [2][N2]: w2_scale, b2
  const float s1 = a.act_scale1[0], s2 = a.act_scale2[0];

  // ---- every global load that does not depend on a result goes out first:
  // the first weight chunk of this wave's layer-2 tiles, the epilogue
  // operands, the X rows
  const __amdgpu_buffer_rsrc_t W1r = make_rsrc(a.W1, (uint32_t)N1 * (uint32_t)K1);
  const __amdgpu_buffer_rsrc_t W2r = make_rsrc(a.W2, (uint32_t)N2 * (uint32_t)N1);
  int n2[kTPW];
#pragma unroll
  for (int j = 0; j < kTPW; ++j) n2[j] = (wave * kTPW + j) * 16;
  Chunk w2first;
  load_chunk(w2first, W2r, n2, N1, 0, g, c);
  {
    // a null bias reads as zero through an empty resource
    const __amdgpu_buffer_rsrc_t S1r = make_rsrc(a.w1_scale, (uint32_t)N1 * 4u);
    const __amdgpu_buffer_rsrc_t B1r = make_rsrc(a.b1, a.b1 ? (uint32_t)N1 * 2u : 0u);
    const __amdgpu_buffer_rsrc_t S2r = make_rsrc(a.w2_scale, (uint32_t)N2 * 4u);
    const __amdgpu_buffer_rsrc_t B2r = make_rsrc(a.b2, a.b2 ? (uint32_t)N2 * 2u : 0u);
    for (int i = tid; i < N1; i += NTHR) {
      E1[i] = bitsf(bload32(S1r, (uint32_t)i * 4u));
      E1[N1 + i] = bitsf(bload16(B1r, (uint32_t)i * 2u) << 16);
    }
    for (int i = tid; i < N2; i += NTHR) {
      E2[i] = bitsf(bload32(S2r, (uint32_t)i * 4u));
      E2[N2 + i] = bitsf(bload16(B2r, (uint32_t)i * 2u) << 16);
    }
  }
  for (int i = tid; i < 16 * (RS1 + RS2) / 4; i += NTHR) reinterpret_cast<uint32_t*>(smem)[i] = 0u;
  __syncthreads();
  // X rows -> E4M3 codes, 8 elements per thread (K1 % 16 == 0)
  const __amdgpu_buffer_rsrc_t Xr = make_rsrc(a.X, (uint32_t)a.M * (uint32_t)K1 * 2u);
  for (int i = tid; i < 16 * K1 / 8; i += NTHR) {
    const int r = (i * 8) / K1, k = (i * 8) % K1;
    const u32x4 v = bload128(Xr, ((uint32_t)(m0 + r) * (uint32_t)K1 + (uint32_t)k) * 2u);  // rows past M read 0
    *reinterpret_cast<u32x2*>(Xq + r * RS1 + k) = act_q8(v, s1);
  }
  __syncthreads();

  // ---- layer 1 -> hidden codes
  for (int t0 = wave * kTPW; t0 * 16 < N1; t0 += kWaves * kTPW) {
    int n0[kTPW];
#pragma unroll
    for (int j = 0; j < kTPW; ++j) n0[j] = (t0 + j) * 16;
    f32x4 acc[kTPW];
#pragma unroll
    for (int j = 0; j < kTPW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < K1; k0 += 256) {
      Chunk ch;
      load_chunk(ch, W1r, n0, K1, k0, g, c);
      mma_chunk(Xq, RS1, ch, k0, g, c, acc);
    }
#pragma unroll
    for (int j = 0; j < kTPW; ++j) {
      const int n = n0[j] + c;
      if (n < N1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float h = bf16_to_f32(f32_to_bf16((acc[j][r] * s1) * E1[n] + E1[N1 + n]));
          Hq[(4 * g + r) * RS2 + n] = (uint8_t)act_q(h, s2);
        }
      }
    }
  }
  __syncthreads();

  // ---- layer 2 -> Y (the first pass uses the chunk loaded at the start)
  for (int t0 = wave * kTPW; t0 * 16 < N2; t0 += kWaves * kTPW) {
    int n0[kTPW];
#pragma unroll
    for (int j = 0; j < kTPW; ++j) n0[j] = (t0 + j) * 16;
    f32x4 acc[kTPW];
#pragma unroll
    for (int j = 0; j < kTPW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < N1; k0 += 256) {
      if (t0 == wave * kTPW && k0 == 0) {
        mma_chunk(Hq, RS2, w2first, 0, g, c, acc);
      } else {
        Chunk ch;
        load_chunk(ch, W2r, n0, N1, k0, g, c);
        mma_chunk(Hq, RS2, ch, k0, g, c, acc);
      }
    }
#pragma unroll
    for (int j = 0; j < kTPW; ++j) {
      const int n = n0[j] + c;
      if (n < N2) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + 4 * g + r;
          if (m < a.M) a.Y[(int64_t)m * N2 + n] = f32_to_bf16((acc[j][r] * s2) * E2[n] + E2[N2 + n]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_static_mlp2(const Mlp2Args& a, hipStream_t s) {
  const unsigned grid = (unsigned)((a.M + 15) / 16);
  if (a.K1 <= kSpK1 && a.N1 <= kSpN1 && a.N2 <= kSpN2) {
    static std::atomic<int> done_sp{0};
    hipError_t e = allow_smem(k_static_mlp2_sp, (int)kSpSmem, done_sp);
    if (e != hipSuccess) return e;
    k_static_mlp2_sp<<<grid, kWaves * 64, kSpSmem, s>>>(a);
    return hipGetLastError();
  }
  const size_t sm = mlp2_smem_bytes(a.K1, a.N1, a.N2);
  static std::atomic<int> done{0};
  hipError_t e = allow_smem(k_static_mlp2, sm > 65536 ? 160 * 1024 : (int)sm, done);
  if (e != hipSuccess) return e;
  k_static_mlp2<<<grid, kWaves * 64, sm, s>>>(a);
  return hipGetLastError();
}

}  // namespace wq
