// Host-side launch planning shared by the C ABI (workspace queries, argument
// checks) and the kernel launchers: which kernel configuration a dequant-GEMM
// call runs and how much scratch it needs.  Plain C++ with no device code, so
// the ABI's host logic also builds and runs without the GPU toolchain's device
// pass (the sanitizer build of the CPU tests).
#include "wq_internal.hpp"

namespace wq {

namespace {

int kpl_of(int kfmt) {
  switch (kfmt) {
    case KF_BF16: return 8;
    case KF_FP8:
    case KF_FP8S: return 16;
    default: return 32;
  }
}

int spw_of(int kfmt, int cfg) {
  const bool b16 = kfmt == KF_BF16, f8 = (kfmt == KF_FP8 || kfmt == KF_FP8S);
  if (cfg == kCfgSplit) return b16 ? 4 : (f8 ? 2 : 1);
  return b16 ? 8 : (f8 ? 4 : 2);
}

}  // namespace

LinearPlan plan_linear(int kfmt, int64_t M, int64_t N, int64_t K, int wl) {
  LinearPlan p{};
  // 65..128 rows of a wide layer (weight-only formats): three or four row
  // blocks of 64-column tiles (at least 192 workgroups) load everything up
  // front like the smaller M do, instead of stepping K through LDS tiles.
  // Measured at N = 4096, K = 3072, M = 72 / 96 / 128: INT4 18.1 -> 12.5 /
  // 12.6 / 13.2 us, NVFP4 18.4 -> 13.5 / 13.6 / 14.0, MXFP4 15.6 -> 12.3 /
  // 12.4 / 12.7, FP8 13.9 -> 13.0 / 13.2 / 13.4.
  const bool wide64 = M > 64 && M <= 128 && kfmt != KF_BF16 && kfmt != KF_FP8S &&
                      ((N + 63) / 64) * ((M + 31) / 32) >= 192;
  // 129 rows and more, up to three rounds of 64 x 64 tiles on the chip: the
  // mid-M kernel (8 waves split K inside the workgroup, no barrier per K
  // step).  Measured against the LDS-tiled kernels (graphs, cold weights):
  // N = 4096, K = 3072, M = 160 / 256 / 512 / 768: MXFP4 15.8 / 15.9 / 23.0 /
  // 34.0 -> 10.7 / 10.7 / 19.8 / 28.6 us, INT4 17.3 / 18.0 / 28.9 / 44.2 ->
  // 13.5 / 14.0 / 26.2 / 38.0; N = 512 .. 2048, K = 1024 .. 4096, M = 160 ..
  // 512: 13-38 % faster in every case.  At 1024 tiles (M = 1024 at N = 4096,
  // M = 512 at N = 8192) the 128 x 128 tiles win by 5-30 %.  The kernel needs
  // K % 128 == 0; with fewer than 8 K blocks some of its waves would idle.
  const bool mid_fmt = kfmt == KF_INT4 || kfmt == KF_INT4A || kfmt == KF_FP8 || kfmt == KF_NVFP4 || kfmt == KF_MXFP4;
  if (mid_fmt && M > 128 && K % 128 == 0 && K >= 1024 && K <= kMidMaxK &&
      ((M + 63) / 64) * ((N + 63) / 64) <= 768) {
    p.cfg = kCfgMid;
    p.S = 1;
    p.bm = 64;
    p.bn = 64;
    p.ks = 1;
    p.part_bytes = 0;
    p.ws_bytes = 0;
    return p;
  }
  if (M > 64 && !wide64) {
    // MFMA-bound: LDS-tiled GEMM; the largest tile that still gives about
    // 192 workgroups.  (The static FP8 GEMM's tiled kernels choose their own
    // tiles by the same rule; for it only cfg and the zero workspace matter.)
    p.cfg = kCfgTiled;
    p.S = 1;
    p.bm = 64;
    p.bn = 64;
    // 256 x 256 tiles: k_woq_gemm256 (activations loaded straight into LDS);
    // measured at M = 4096 (N = 4096, K = 3072): INT4 157 -> 114 us against
    // 128 x 128 tiles, MXFP4 and FP8 on par with the register-staged 256 x 256
    // kernel it replaced.
    const int cand[4][2] = {{256, 256}, {128, 128}, {128, 64}, {64, 128}};
    for (const auto& cb : cand) {
      const int64_t tiles = ((M + cb[0] - 1) / cb[0]) * ((N + cb[1] - 1) / cb[1]);
      if (tiles >= 192) {
        p.bm = cb[0];
        p.bn = cb[1];
        break;
      }
    }
    // few tiles: split K over two groups of waves inside each workgroup, so
    // that each CU runs 8 waves (the K steps are latency-bound otherwise).
    // Measured at M = 128 and 256 (N = 4096, K = 3072): two groups beat one by
    // 10-25 %; four groups (64 x 64 tiles only) were slower than two.
    const int64_t tiles = ((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
    const int64_t steps = (K + 63) / 64;
    p.ks = 1;
    if (p.bm < 128 || p.bn < 128) {
      if (tiles <= 512 && steps >= 16) p.ks = 2;
    }
    p.part_bytes = 0;
    p.ws_bytes = 0;
    return p;
  }
  // 16 or 32 rows per workgroup; 33..64 rows take two row blocks (grid z)
  // that read the same packed columns, 65..128 three or four.  Workgroup ids of one column tile
  // differ by gx, so with gx a multiple of 8 both blocks run on the same XCD
  // (workgroups are dealt to the 8 XCDs round robin) and share its L2 copy.
  p.mt = M <= 16 ? 1 : 2;
  p.gz = (int)((M + 16 * p.mt - 1) / (16 * p.mt));
  // No-split (16 columns x all of K per workgroup) whenever it yields enough
  // workgroups to cover the chip, or K <= 3072; otherwise 64-column tiles with
  // K split across workgroups and a second, stream-ordered reduction kernel.
  // On narrow layers the second launch costs more than the idle CUs: measured
  // at K = 3072, N = 256 / 512 / 1024, M = 4..64, no-split is 1.2-2.0 us
  // faster in every format (N = 512, M = 32: FP8 7.6 -> 6.05 us, INT4 7.3 ->
  // 5.9); at K = 4096 only FP8 gained, and from K = 6144 split wins.
  const int64_t gx_nosplit = (N + 15) / 16;
  p.cfg = (gx_nosplit * p.gz >= 128 || K <= 3072) ? kCfgNoSplit : kCfgSplit;
  const int64_t T = (K + 4 * kpl_of(kfmt) - 1) / (4 * kpl_of(kfmt));
  if (p.cfg == kCfgSplit) {
    p.ntw = 4;
    p.nwaves = 4;
  } else {
    // two row blocks (33..64 rows): 32 columns per workgroup when that still
    // gives 256 workgroups, so that a CU reads one 32-row activation block
    // (192 KiB at K = 3072) rather than two workgroups' worth; measured at
    // N = 4096, K = 3072, M = 64: 11.1-12.2 -> 8.6-9.8 us for every format.
    // (With one row block, 32-column tiles leave half the CUs idle: 1.3-1.8 us
    // slower at M = 16 and 32.)
    p.ntw = (p.gz == 2 && ((N + 31) / 32) * p.gz >= 256) ? 2 : 1;
    if (p.gz >= 3) p.ntw = 4;  // wide64 above
    // 17..32 rows, weights in tile order: two 16-row blocks of 32-column
    // tiles instead of one 32-row block of 16-column tiles (each CU reads half
    // the activation rows; the two blocks of a column tile run on one XCD and
    // read the same weight tiles).  Measured at N = 4096, K = 3072, M = 32:
    // MXFP4 5.53 -> 5.26 us, FP8 6.34 -> 6.06 us, INT4 5.78 -> 5.39 us; NVFP4
    // lost (6.02 -> 6.13 us) and keeps 32-row blocks.
    const bool rb16 = wl == kLayoutTiles && M > 16 && M <= 32 &&
                      (kfmt == KF_INT4 || kfmt == KF_INT4A || kfmt == KF_MXFP4 || kfmt == KF_FP8) &&
                      ((N + 31) / 32) * 2 >= 256;
    if (rb16) {
      p.mt = 1;
      p.gz = 2;
      p.ntw = 2;
    }
    p.nwaves = (p.ntw == 4) ? 8 : 12;
  }
  p.spw = (p.cfg == kCfgNoSplit) ? spw_of(kfmt, p.cfg) * 12 / p.nwaves : spw_of(kfmt, p.cfg);
  p.gx = (int)((N + 16 * p.ntw - 1) / (16 * p.ntw));
  const int64_t base = (int64_t)p.gx * p.gz;
  int64_t S = 1;
  if (p.cfg == kCfgSplit) S = (T + (int64_t)p.nwaves * p.spw - 1) / ((int64_t)p.nwaves * p.spw);
  if (S > kMaxSplit) S = kMaxSplit;  // the waves then loop over several blocks
  if (S < 1) S = 1;
  p.S = (int)S;
  const int64_t E = (int64_t)p.mt * 16 * 16 * p.ntw;
  const int64_t nthr = 64 * (int64_t)p.nwaves;
  const int64_t ept = (E + nthr - 1) / nthr;
  const int64_t slab = nthr * ((ept + 3) / 4) * 16;  // bytes of one workgroup partial
  p.part_bytes = p.S > 1 ? (size_t)(base * p.S * slab) : 0;
  p.ws_bytes = p.part_bytes;
  return p;
}

// LDS bytes of the looped fused-MLP kernel: 16 rows of K1 and of N1 E4M3 codes
// (each rounded up to 256 plus 16 bytes of padding) and the two layers' column
// scales and biases.
size_t mlp2_smem_bytes(int64_t K1, int64_t N1, int64_t N2) {
  return (size_t)16 * (size_t)(((K1 + 255) / 256 * 256 + 16) + ((N1 + 255) / 256 * 256 + 16)) +
         (size_t)8 * (size_t)(N1 + N2);
}

}  // namespace wq
