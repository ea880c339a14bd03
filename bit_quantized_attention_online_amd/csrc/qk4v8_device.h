// Device-side building blocks of the QK4V8 kernels for gfx950 (CDNA4).
//
// Formats: MXFP4 = E2M1 codes with one E8M0 scale per 32 elements (the block
// size of "小米MiMo-V2.5-Pro-FP4-DFlash：FP4+推测解码的万亿推理提速指南", section
// "MXFP4专家量化"); V in FP8 E4M3FN with one E8M0 scale per tile of rows
// ("MpFA免训练量化：QK4V8混合精度在Blackwell上的推理加速实践" §2.2 keeps V at 8
// bits, §3.2 computes each block's scale online from the block itself).
//
// Hardware facts these helpers rely on (gfx950):
//  * v_cvt_scalef32_pk_fp4_f32 / _pk_fp8_f32 compute fmt(x / scale) with
//    round-to-nearest-even.  The fp4 form saturates to +-6; the fp8 form does
//    NOT saturate (an overflow becomes NaN), so callers clamp to +-448 first.
//    The sign of a zero result is kept.
//  * v_cvt_scalef32_pk_f32_fp8 computes decode(code) * scale.
//  * v_mfma_scale_f32_16x16x128_f8f6f4: lane l holds row/column (l % 16) and
//    supplies the E8M0 scale of block (l / 16) (32 consecutive k) for that
//    row/column.  With fp4 operands lane l holds k = 32*(l/16) + j in nibble j
//    of dwords 0..3.  With fp8 operands byte j of the lane's 8 dwords is
//    k = 64*(j/16) + 16*(l/16) + (j%16).  The 4 results of lane l are
//    C[4*(l/16) + i][l % 16].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qk4v8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v2s __attribute__((ext_vector_type(2)));

constexpr int kFmtFp8 = 0;   // E4M3 operand format code of the scaled MFMA
constexpr int kFmtFp4 = 4;   // E2M1 operand format code

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 2^e for e in [-126, 127] built from its exponent bits (exact).
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// OCP MX shared exponent X = floor(log2(amax)) - emax, clamped to [-127, 127];
// -127 for an all-zero block.  amax is the (non-negative) fp32 maximum of the
// block's magnitudes.  Subnormal amax (exponent field 0) has floor(log2) <= -127,
// so it also clamps to -127.
__device__ __forceinline__ int mx_shared_exp(float amax, int emax) {
  int ebits = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  if (ebits == 0) return -127;
  int x = ebits - 127 - emax;
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// Two fp32 values (already divided by the block scale, |y| < 8) -> one byte of
// two E2M1 codes, low nibble = first value.  RNE, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_pack2(float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}

// Two fp32 values -> two E4M3FN bytes (low byte = a) with RNE after dividing
// by `scale`; the caller guarantees |x / scale| <= 448.
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b, float scale) {
  v2s z = {0, 0};
  v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a, b, scale, false);
  return (uint32_t)(uint16_t)r[0];
}

__device__ __forceinline__ float clamp448(float y) { return fminf(fmaxf(y, -448.0f), 448.0f); }

// Quantize 32 bf16 values held as 16 packed dwords (element 2i in the low half
// of word i) into 16 bytes of E2M1 codes (4 dwords) and return the scale byte.
__device__ __forceinline__ uint32_t mxfp4_quantize32(const uint32_t (&w)[16], uint32_t (&codes)[4]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  int X = mx_shared_exp(amax, 2);
  float inv = exp2i(-X);   // -X in [-127, 127]; X = -127 gives 2^127
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t ww = w[4 * i + j];
      c |= e2m1_pack2(bf16_lo(ww) * inv, bf16_hi(ww) * inv) << (8 * j);
    }
    codes[i] = c;
  }
  return (uint32_t)(X + 127);
}

// Scaled MFMA wrappers.  `sa`/`sb` hold E8M0 bytes; OPA/OPB select the byte.
template <int FA, int FB, int OPA = 0, int OPB = 0>
__device__ __forceinline__ v4f mfma16x16x128(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, OPA, sa, OPB, sb);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace qk4v8
