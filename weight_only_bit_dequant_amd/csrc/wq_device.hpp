// Device-side element codecs and small helpers for gfx950.
//
// Encoders are written on the fp32 bit pattern with integer round-to-nearest-
// even, so that quantized codes are bit-identical to an IEEE reference: every
// value is clamped to the format's largest finite magnitude first, the sign bit
// is kept (a negative zero or a negative value that rounds to zero gives the
// negative-zero code).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }

// bf16 (bit pattern) -> fp32, exact.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return bitsf(((uint32_t)h) << 16); }

// fp32 -> bf16 bit pattern, round to nearest even, on the gfx950 converter
// (v_cvt_pk_bf16_f32).  An exhaustive device comparison found it equal, on
// every non-NaN fp32 input, to the integer rounding
//   u + 0x7FFF + ((u >> 16) & 1), upper half;
// a NaN gives a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Round the integer `mant` (the dropped low bits are `drop` wide) to nearest
// even; returns the kept value (may carry to 1 << (23 - drop)).
__device__ __forceinline__ uint32_t rne_shift(uint32_t mant, int drop) {
  uint32_t kept = mant >> drop;
  uint32_t rem = mant & ((1u << drop) - 1u);
  uint32_t half = 1u << (drop - 1);
  return kept + ((rem > half) || (rem == half && (kept & 1u)));
}

// E4M3 ("fn", bias 7, max 448): x must already be clamped to [-448, 448].
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  uint32_t u = fbits(x);
  uint32_t sign = (u >> 31) << 7;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a < 0x3C800000u) {  // |x| < 2^-6: subnormal grid of 2^-9 (exact scaling)
    code = (uint32_t)__builtin_rintf(bitsf(a) * 512.0f);
  } else {
    int e = (int)(a >> 23) - 127;  // -6 .. 8
    uint32_t m = rne_shift(a & 0x7FFFFFu, 20);
    if (m == 8u) { m = 0u; e += 1; }
    code = ((uint32_t)(e + 7) << 3) | m;
  }
  return sign | code;
}

// The same E4M3 rounding on the gfx950 converter (v_cvt_pk_fp8_f32, OCP
// E4M3, nearest even), two values per instruction.  An exhaustive device
// comparison over every fp32 input with |x| <= 448 (both signs, zeros and
// subnormals included) found it equal to e4m3_encode.  Inputs must already be
// clamped to [-448, 448].
__device__ __forceinline__ uint32_t e4m3_cvt(float x) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, x, 0, false) & 0xFFu;
}
// four values -> one word, value i in byte i
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// E2M1 (bias 1, max 6): x must already be clamped to [-6, 6].
__device__ __forceinline__ uint32_t e2m1_encode(float x) {
  uint32_t u = fbits(x);
  uint32_t sign = (u >> 31) << 3;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a < 0x3F800000u) {  // |x| < 1: subnormal grid of 0.5
    code = (uint32_t)__builtin_rintf(bitsf(a) * 2.0f);
  } else {
    int e = (int)(a >> 23) - 127;  // 0 .. 2
    uint32_t m = rne_shift(a & 0x7FFFFFu, 22);
    if (m == 2u) { m = 0u; e += 1; }
    code = ((uint32_t)(e + 1) << 1) | m;
  }
  return sign | code;
}

// Decoders (exact).  Written with selects only: a data-dependent branch in a
// kernel's main loop makes the compiler drain every memory load in flight.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float sub = (float)m * 0.001953125f;  // m * 2^-9
  const float nrm = bitsf(((e + 120u) << 23) | (m << 20));
  float mag = (e == 0u) ? sub : nrm;
  mag = ((c & 0x7Fu) == 0x7Fu) ? __builtin_nanf("") : mag;
  return bitsf(fbits(mag) | ((c & 0x80u) << 24));
}

__device__ __forceinline__ float e2m1_decode(uint32_t c) {
  const float t[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
  float v = t[c & 7u];
  return (c & 8u) ? -v : v;
}

// 2^(c - 127) for an E8M0 code (0xFF -> NaN; 0 -> 2^-127, an fp32 subnormal).
__device__ __forceinline__ float e8m0_decode(uint32_t c) {
  const uint32_t bits = (c == 0u) ? 0x00400000u : ((c == 0xFFu) ? 0x7FC00000u : (c << 23));
  return bitsf(bits);
}

__device__ __forceinline__ float clampf(float x, float lo, float hi) { return fminf(fmaxf(x, lo), hi); }

// Static FP8 activation Q ("TorchAO Static FP8 Quantization (Linear)": the
// calibrated per-tensor scale divides x, the quotient is clamped to the E4M3
// range and rounded to nearest even): the value before rounding, x itself when
// s == 0.  One IEEE fp32 division, as in every kernel that applies this Q.
__device__ __forceinline__ float act_q_val(float x, float s) {
  return clampf((s > 0.f) ? x / s : x, -448.f, 448.f);
}
__device__ __forceinline__ uint32_t act_q(float x, float s) { return e4m3_cvt(act_q_val(x, s)); }
// eight bf16 values (four words, K order) -> eight E4M3 codes, value i in byte i
__device__ __forceinline__ u32x2 act_q8(u32x4 v, float s) {
  return u32x2{e4m3_pack4(act_q_val(bitsf(v.x << 16), s), act_q_val(bitsf(v.x & 0xFFFF0000u), s),
                          act_q_val(bitsf(v.y << 16), s), act_q_val(bitsf(v.y & 0xFFFF0000u), s)),
               e4m3_pack4(act_q_val(bitsf(v.z << 16), s), act_q_val(bitsf(v.z & 0xFFFF0000u), s),
                          act_q_val(bitsf(v.w << 16), s), act_q_val(bitsf(v.w & 0xFFFF0000u), s))};
}

// Nonnegative float atomic max via the ordered integer view (valid for x >= 0, not NaN).
__device__ __forceinline__ void atomic_max_nonneg(float* p, float x) {
  atomicMax(reinterpret_cast<unsigned int*>(p), fbits(x));
}

}  // namespace wq
