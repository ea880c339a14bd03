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
//  * The unscaled v_cvt_pk_fp8_f32 / v_cvt_pk_f32_fp8 use the same OCP E4M3
//    code (RNE).  Measured issue cost with four waves per SIMD: the E4M3
//    conversions and v_exp_f32 take about 2.7x the cycles of an fp32 FMA,
//    except the unscaled E4M3 -> f32 back conversion (about 1.6x).
//  * v_mfma_scale_f32_16x16x128_f8f6f4: lane l holds row/column (l % 16) and
//    supplies the E8M0 scale of block (l / 16) (32 consecutive k) for that
//    row/column.  With fp4 operands lane l holds k = 32*(l/16) + j in nibble j
//    of dwords 0..3.  With fp8 operands byte j of the lane's 8 dwords is
//    k = 64*(j/16) + 16*(l/16) + (j%16).  The 4 results of lane l are
//    C[4*(l/16) + i][l % 16].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace qk4v8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v2s __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (a in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  const v2bf r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

// Compile-time loop: f(std::integral_constant<int, 0>{}) ... f(<N-1>), so the
// index can feed instruction immediates (e.g. the MFMA scale byte select).
template <int... I, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// An FP4 MFMA operand: 16 bytes of E2M1 codes in the low half of the 8-dword
// operand; the upper half is left undefined so the backend passes 4 VGPRs.
__device__ __forceinline__ v8i fp4_operand(v4i v) {
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}
__device__ __forceinline__ v8i fp4_operand(uint4 x) {
  return fp4_operand(v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w});
}

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
// The block maximum is taken on the bf16 bit patterns (magnitudes of finite
// bf16 values order as unsigned integers, two per v_pk_max_u16), and the
// codes come from the packed bf16 pairs through the scaled convert (x / 2^X,
// RNE, saturating at 6), one instruction per byte.  Blocks with X < -120
// (only tiny or zero values) take the fp32 route, so a bf16 subnormal never
// meets the scaled convert.
__device__ __forceinline__ uint32_t mxfp4_quantize32(const uint32_t (&w)[16], uint32_t (&codes)[4]) {
  typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  v2u16 m = __builtin_bit_cast(v2u16, w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < 16; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(v2u16, w[i] & 0x7FFF7FFFu));
  const uint32_t mag = max((uint32_t)m[0], (uint32_t)m[1]);
  const int X = mx_shared_exp(__uint_as_float(mag << 16), 2);
  if (X >= -120) {
    const float scale = exp2i(X);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(v2bf, w[4 * i]), scale, 0);
      c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(v2bf, w[4 * i + 1]), scale, 1);
      c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(v2bf, w[4 * i + 2]), scale, 2);
      codes[i] = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(v2bf, w[4 * i + 3]), scale, 3);
    }
  } else {
    const float inv = exp2i(-X);   // -X in [121, 127]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t ww = w[4 * i + j];
        c |= e2m1_pack2(bf16_lo(ww) * inv, bf16_hi(ww) * inv) << (8 * j);
      }
      codes[i] = c;
    }
  }
  return (uint32_t)(X + 127);
}

// MXFP4 of 32 fp32 values (exact float32 inputs, e.g. rotated rows): the same
// rule as mxfp4_quantize32 on values that are not bf16.
__device__ __forceinline__ uint32_t mxfp4_quantize32f(const float (&x)[32], uint32_t (&codes)[4]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const int X = mx_shared_exp(amax, 2);
  const float inv = exp2i(-X);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) c |= e2m1_pack2(x[8 * i + 2 * j] * inv, x[8 * i + 2 * j + 1] * inv) << (8 * j);
    codes[i] = c;
  }
  return (uint32_t)(X + 127);
}

// 32 bf16 (16 packed dwords, element 2i in the low half of word i) -> fp32.
__device__ __forceinline__ void unpack_bf16x32(const uint32_t (&w)[16], float (&x)[32]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
}

// Sylvester-Hadamard transform of head_dim rows ("MpFA免训练量化：QK4V8混合精度在
// Blackwell上的推理加速实践" §3.1: a rotation spreads outlier channels over
// all channels before 4-bit quantization).  Butterfly stages h = 1, 2, ...,
// d/2 in that order, (x_i, x_{i+h}) -> (x_i + x_{i+h}, x_i - x_{i+h}), in
// fp32; a lane holds one 32-element block, so stages h < 32 run in the lane
// and stage h = 32 * 2^k pairs the lane with the lane holding block b ^ 2^k.
__device__ __forceinline__ void fwht32(float (&x)[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1)
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
}

// One cross-lane butterfly stage: `partner` is the value the other lane of the
// pair holds at the same position; the lane with the lower block index keeps
// the sum, the other the difference (lower - upper).
__device__ __forceinline__ float hadamard_pair(float own, float partner, bool upper) {
  return upper ? partner - own : own + partner;
}

// The partner's value out of a lane-swap result pair (whichever of the two is
// not this lane's own bits; when both are, the partner holds the same value).
__device__ __forceinline__ float swap_partner(float own, uint32_t r0, uint32_t r1) {
  return __uint_as_float(r0 != __float_as_uint(own) ? r0 : r1);
}

// Stage h = 32 * 2^k with the pair lanes l and l ^ 16 (k chosen by the caller's
// layout), using v_permlane16_swap.
__device__ __forceinline__ void hadamard_stage_lane_xor16(float (&x)[32], bool upper) {
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[i]), __float_as_uint(x[i]), false, false);
    x[i] = hadamard_pair(x[i], swap_partner(x[i], r[0], r[1]), upper);
  }
}

// The same with the pair lanes l and l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ void hadamard_stage_lane_xor32(float (&x)[32], bool upper) {
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[i]), __float_as_uint(x[i]), false, false);
    x[i] = hadamard_pair(x[i], swap_partner(x[i], r[0], r[1]), upper);
  }
}

// Key (0..127 of a 128-key tile) behind row r of QK^T subtile t in the
// 16x16x128 layout.  S^T = K·Q^T puts row 4*(l/16) + i of the 16x16 result in
// element i of lane l, so lane l holds the keys 64*(t/4) + 16*(l/16) +
// 4*(t%4) + i of its query: with the FP8 operand order above, dword t of the
// P·V operand built from them needs no lane exchange.
__host__ __device__ constexpr int subtile_key(int t, int r) {
  return (t >> 2) * 64 + 16 * (r >> 2) + 4 * (t & 3) + (r & 3);
}

// Workgroup barrier inside a tile loop whose callers have already waited for
// the LDS data it orders (their own direct loads or staging writes), with
// every LDS read before it consumed, so no memory fence is needed (a fence
// would wait for the loads still in flight); the empty asm statements keep
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// An empty asm that reads x: the value has to be computed at this point of
// the program, which pins pure computations (matrix instructions) in place.
template <class T>
__device__ __forceinline__ void keep_in_vgprs(const T& x) {
#if __HIP_DEVICE_COMPILE__
  asm volatile("" ::"v"(x));
#else
  (void)x;
#endif
}

// Scaled MFMA wrappers.  `sa`/`sb` hold E8M0 bytes; OPA/OPB select the byte.
template <int FA, int FB, int OPA = 0, int OPB = 0>
__device__ __forceinline__ v4f mfma16x16x128(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, OPA, sa, OPB, sb);
}

template <int FA, int FB, int OPA = 0, int OPB = 0>
__device__ __forceinline__ v16f mfma32x32x64(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, OPA, sa, OPB, sb);
}

// v_mfma_f32_32x32x16_bf16: A (32 x 16) and B (16 x 32) as 8 bf16 per lane
// (4 dwords: row or column lane % 32, k half lane / 32), fp32 32x32 result in
// the same lane layout as the scaled 32x32x64 instruction.
__device__ __forceinline__ v16f mfma32x32x16_bf16(const v4i& a, const v4i& b, const v16f& c) {
  typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                  0);
}

// Two fp32 values -> two E4M3 bytes written into the low (HI=false) or high
// (HI=true) 16 bits of `old`, after dividing by `scale` (|x/scale| <= 448).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_put2(uint32_t old, float a, float b, float scale) {
  v2s o = __builtin_bit_cast(v2s, old);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, scale, HI);
  return __builtin_bit_cast(uint32_t, o);
}

// The same without a scale (RNE to E4M3 of the values themselves): the
// unscaled E4M3 <-> f32 conversions run faster than the scaled ones for the
// back conversion, and the P split works on p / 2^X directly.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_put2_unscaled(uint32_t old, float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// Causal / window / length mask: the score of the key at offset x survives
// when low <= x <= low + span, one unsigned range compare (x - low wraps to
// a huge value below low); masked scores become -inf.
__device__ __forceinline__ float mask_range(float s, int x, int low, uint32_t span) {
  return (uint32_t)(x - low) <= span ? s : -INFINITY;
}

constexpr float kLazyRescale = 8.0f;   // log2 headroom before the accumulator is rescaled
constexpr uint32_t kFp8Ones = 0x38383838u;   // four E4M3 1.0 bytes

// Maximum over the two lanes l and l^32 (v_permlane32_swap exchanges the
// halves of the wave without an LDS round trip; max is symmetric, so the pair
// of results gives the partner's value whichever way round they come).
__device__ __forceinline__ float max_with_lane_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over the two lanes l and l^32 (as above; the sum is commutative, so
// both lanes of a pair get the same bits).
__device__ __forceinline__ float sum_with_lane_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum over the two lanes l and l^16 (v_permlane16_swap exchanges the
// odd and even 16-lane rows; as above, the pair holds the partner's value).
__device__ __forceinline__ float max_with_lane_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Online-softmax step for one 16-query block and one 128-key tile, followed
// by the two-term FP8 split of the probabilities ("MpFA免训练量化：QK4V8混合精度
// 在Blackwell上的推理加速实践" §2.3: scores, normalizer and V accumulation in one
// loop; §3.3: FP32 accumulator).
//
// S: the 8 QK^T subtile results of this lane (32 scores of query lane%16;
//    masked entries -inf).  c = softmax_scale * log2(e).  m_run: running
//    maximum in the log2 domain.  The running max only moves when it grows by
//    more than kLazyRescale, so most tiles skip the rescale of O and L.
// Outputs: Phi / Plo = the E4M3 codes of p / 2^X and of the residual
//    (p - hi) / 2^(X-4), byte 4t+i holding subtile t, element i (the order of
//    the FP8 MFMA k index), and psc = X + 127 (E8M0) with X chosen from the
//    tile's largest p so that p / 2^X < 256.
template <int ND>
__device__ __forceinline__ void softmax_tile(v4f (&S)[8], float c, float& m_run, v4f (&O)[ND], v4f& L, v8i& Phi,
                                             v8i& Plo, int& psc) {
  // row maximum over the lane's 32 scores (independent chains, then a tree),
  // then across the 4 lanes that hold the same query (l ^ 16, l ^ 32), by lane
  // swaps rather than LDS permutes
  float m4[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) m4[g] = fmaxf(fmaxf(S[2 * g][0], S[2 * g][1]), fmaxf(S[2 * g][2], S[2 * g][3]));
#pragma unroll
  for (int g = 0; g < 4; ++g) m4[g] = fmaxf(m4[g], fmaxf(fmaxf(S[2 * g + 1][0], S[2 * g + 1][1]),
                                                       fmaxf(S[2 * g + 1][2], S[2 * g + 1][3])));
  float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
  mx = max_with_lane_xor16(mx);
  mx = max_with_lane_xor32(mx);
  const float tmax = mx * c;
  const float m_new = fmaxf(m_run, tmax);
  // wave-uniform, rarely taken: move the running max only when it grew by more
  // than kLazyRescale somewhere in the wave
  const bool grow = __builtin_amdgcn_ballot_w64(m_new > m_run + kLazyRescale) != 0;
  if (__builtin_expect(grow, 0)) {
    const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
    for (int dd = 0; dd < ND; ++dd) O[dd] *= alpha;
    L *= alpha;
    m_run = m_new;
  }
  const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
  const int X = (int)floorf(fmaxf(tmax - m_use, -100.0f)) - 7;
  psc = X + 127;
  // p / 2^X = 2^(s*c - (m_use + X)): the range scale folds into the
  // exponent, so hi and its back conversion need no scale operand
  const float mX = m_use + (float)X;
  // independent passes over the 32 scores, in place: weights, hi codes (the
  // previous tile's codes are dead here and are overwritten), residuals, lo
  // codes (lo = E4M3(16 * residual), the scaled convert's 2^-4)
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) S[t][i] = __builtin_amdgcn_exp2f(fmaf(S[t][i], c, -mX));
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t h = e4m3_put2_unscaled<false>((uint32_t)Phi[t], S[t][0], S[t][1]);
    Phi[t] = (int)e4m3_put2_unscaled<true>(h, S[t][2], S[t][3]);
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const auto b01 = __builtin_amdgcn_cvt_pk_f32_fp8(Phi[t], false);
    const auto b23 = __builtin_amdgcn_cvt_pk_f32_fp8(Phi[t], true);
    S[t][0] -= b01[0];
    S[t][1] -= b01[1];
    S[t][2] -= b23[0];
    S[t][3] -= b23[1];
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t l = e4m3_put2<false>((uint32_t)Plo[t], S[t][0], S[t][1], 0.0625f);
    Plo[t] = (int)e4m3_put2<true>(l, S[t][2], S[t][3], 0.0625f);
  }
}

// softmax_tile in two parts with identical arithmetic, for a schedule that
// runs the second part elsewhere: (1) the online-softmax step, with the
// weights p / 2^X left in W; (2) the hi codes, residuals and lo codes.
template <int ND>
__device__ __forceinline__ void softmax_tile_hi(v4f (&S)[8], v4f (&W)[8], float c, float& m_run, v4f (&O)[ND],
                                                v4f& L, int& psc) {
  float m4[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) m4[g] = fmaxf(fmaxf(S[2 * g][0], S[2 * g][1]), fmaxf(S[2 * g][2], S[2 * g][3]));
#pragma unroll
  for (int g = 0; g < 4; ++g) m4[g] = fmaxf(m4[g], fmaxf(fmaxf(S[2 * g + 1][0], S[2 * g + 1][1]),
                                                       fmaxf(S[2 * g + 1][2], S[2 * g + 1][3])));
  float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
  mx = max_with_lane_xor16(mx);
  mx = max_with_lane_xor32(mx);
  const float tmax = mx * c;
  const float m_new = fmaxf(m_run, tmax);
  const bool grow = __builtin_amdgcn_ballot_w64(m_new > m_run + kLazyRescale) != 0;
  if (__builtin_expect(grow, 0)) {
    const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
    for (int dd = 0; dd < ND; ++dd) O[dd] *= alpha;
    L *= alpha;
    m_run = m_new;
  }
  const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
  const int X = (int)floorf(fmaxf(tmax - m_use, -100.0f)) - 7;
  psc = X + 127;
  const float mX = m_use + (float)X;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) W[t][i] = __builtin_amdgcn_exp2f(fmaf(S[t][i], c, -mX));
}

__device__ __forceinline__ void softmax_tile_lo(v4f (&W)[8], v8i& Phi, v8i& Plo) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t h = e4m3_put2_unscaled<false>((uint32_t)Phi[t], W[t][0], W[t][1]);
    Phi[t] = (int)e4m3_put2_unscaled<true>(h, W[t][2], W[t][3]);
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const auto b01 = __builtin_amdgcn_cvt_pk_f32_fp8(Phi[t], false);
    const auto b23 = __builtin_amdgcn_cvt_pk_f32_fp8(Phi[t], true);
    W[t][0] -= b01[0];
    W[t][1] -= b01[1];
    W[t][2] -= b23[0];
    W[t][3] -= b23[1];
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t l = e4m3_put2<false>((uint32_t)Plo[t], W[t][0], W[t][1], 0.0625f);
    Plo[t] = (int)e4m3_put2<true>(l, W[t][2], W[t][3], 0.0625f);
  }
}

// The same step for the 32x32x64 layout: S holds the 4 key-block results of
// this lane (64 scores of query lane%32, split with lane^32), P byte j of the
// 8-dword operand of P·V step s2 holds key-block 2*s2 + j/16, element j%16.
// One wave runs this alone on its SIMD while the other feeds the matrix core,
// so it is written as independent passes over all 64 scores (in place in S):
// the exponentials, then the hi codes, then the residuals, then the lo codes,
// which lets the scheduler hide the latency of the transcendental and convert
// instructions behind independent work.
template <int NO>
__device__ __forceinline__ void softmax_tile32(v16f (&S)[4], float c, float& m_run, v16f (&O)[NO], v16f& L,
                                               v8i (&Phi)[2], v8i (&Plo)[2], int (&psc)[2]) {
  // row maximum: four independent chains, then a tree
  float m4[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    float a = fmaxf(S[kb][0], S[kb][1]), b = fmaxf(S[kb][2], S[kb][3]);
#pragma unroll
    for (int i = 4; i < 16; i += 4) {
      a = fmaxf(a, fmaxf(S[kb][i], S[kb][i + 1]));
      b = fmaxf(b, fmaxf(S[kb][i + 2], S[kb][i + 3]));
    }
    m4[kb] = fmaxf(a, b);
  }
  const float mx = max_with_lane_xor32(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
  const float tmax = mx * c;
  const float m_new = fmaxf(m_run, tmax);
  const bool grow = __builtin_amdgcn_ballot_w64(m_new > m_run + kLazyRescale) != 0;
  if (__builtin_expect(grow, 0)) {
    const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
    for (int o = 0; o < NO; ++o) O[o] *= alpha;
    L *= alpha;
    m_run = m_new;
  }
  const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
  const int X = (int)floorf(fmaxf(tmax - m_use, -100.0f)) - 7;
  psc[0] = psc[1] = X + 127;   // one range exponent per (row, tile)
  const float mX = m_use + (float)X;
  // p / 2^X = 2^(s*c - (m_use + X)), in place
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) S[kb][i] = __builtin_amdgcn_exp2f(fmaf(S[kb][i], c, -mX));
  // hi = E4M3(p / 2^X)
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int dw = 4 * (kb & 1) + w;
      uint32_t h = e4m3_put2_unscaled<false>((uint32_t)Phi[kb >> 1][dw], S[kb][4 * w], S[kb][4 * w + 1]);
      Phi[kb >> 1][dw] = (int)e4m3_put2_unscaled<true>(h, S[kb][4 * w + 2], S[kb][4 * w + 3]);
    }
  // residual p / 2^X - hi, in place
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int h = Phi[kb >> 1][4 * (kb & 1) + w];
      const auto b01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
      const auto b23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
      S[kb][4 * w] -= b01[0];
      S[kb][4 * w + 1] -= b01[1];
      S[kb][4 * w + 2] -= b23[0];
      S[kb][4 * w + 3] -= b23[1];
    }
  // lo = E4M3(16 * residual) (scale 2^-4)
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int dw = 4 * (kb & 1) + w;
      uint32_t l = e4m3_put2<false>((uint32_t)Plo[kb >> 1][dw], S[kb][4 * w], S[kb][4 * w + 1], 0.0625f);
      Plo[kb >> 1][dw] = (int)e4m3_put2<true>(l, S[kb][4 * w + 2], S[kb][4 * w + 3], 0.0625f);
    }
}

// Single-term variant of softmax_tile32 (fast mode): P is one E4M3 term per
// weight, with one E8M0 range exponent per row and aligned 32-key block (the
// MX block size).  Key block kb of the tile (keys 32*kb .. 32*kb + 31) is
// S[kb] of this lane and of lane ^ 32, so its maximum takes one lane swap;
// P·V step s2 applies lane half h's exponent to key block 2*s2 + h.  The
// running maximum is kept integral, so every rescale is an exact power of
// two, and the E4M3 rounding of p / 2^X_B = 2^(s*c - floor(max_B) + 7)
// depends only on the scores and on the block's maximum, not on when the
// running maximum moved: the result is the same for any order of the tiles
// and any tiling that keeps the aligned 32-key blocks whole.
template <int NO>
__device__ __forceinline__ void softmax_tile32_single(v16f (&S)[4], float c, float& m_run, v16f (&O)[NO], v16f& L,
                                                      v8i (&Phi)[2], int (&psc)[2], int lh) {
  float bm[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    float a = fmaxf(S[kb][0], S[kb][1]), b = fmaxf(S[kb][2], S[kb][3]);
#pragma unroll
    for (int i = 4; i < 16; i += 4) {
      a = fmaxf(a, fmaxf(S[kb][i], S[kb][i + 1]));
      b = fmaxf(b, fmaxf(S[kb][i + 2], S[kb][i + 3]));
    }
    bm[kb] = max_with_lane_xor32(fmaxf(a, b));   // the whole 32-key block of this row
  }
  const float mx = fmaxf(fmaxf(bm[0], bm[1]), fmaxf(bm[2], bm[3]));
  const float tmax = mx * c;
  const float m_new = ceilf(fmaxf(m_run, tmax));           // integral (or -inf)
  const bool grow = __builtin_amdgcn_ballot_w64(m_new > m_run + kLazyRescale) != 0;
  if (__builtin_expect(grow, 0)) {
    // 2^(m_run - m_new) built from its exponent bits: exact
    const float alpha = (m_run == -INFINITY) ? 0.0f : exp2i((int)fmaxf(m_run - m_new, -126.0f));
#pragma unroll
    for (int o = 0; o < NO; ++o) O[o] *= alpha;
    L *= alpha;
    m_run = m_new;
  }
  const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
  int X[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) X[kb] = (int)floorf(fmaxf(bm[kb] * c - m_use, -100.0f)) - 7;
  psc[0] = (lh ? X[1] : X[0]) + 127;
  psc[1] = (lh ? X[3] : X[2]) + 127;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const float mX = m_use + (float)X[kb];   // integral: p / 2^X exactly
#pragma unroll
    for (int i = 0; i < 16; ++i) S[kb][i] = __builtin_amdgcn_exp2f(fmaf(S[kb][i], c, -mX));
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int dw = 4 * (kb & 1) + w;
      uint32_t h = e4m3_put2_unscaled<false>((uint32_t)Phi[kb >> 1][dw], S[kb][4 * w], S[kb][4 * w + 1]);
      Phi[kb >> 1][dw] = (int)e4m3_put2_unscaled<true>(h, S[kb][4 * w + 2], S[kb][4 * w + 3]);
    }
}

// BF16 variant of softmax_tile32: the probabilities feed the bf16 matrix core
// (v_mfma_f32_32x32x16_bf16) against V widened exactly to bf16, so each
// weight is one RNE bf16 rounding of p (8 significant bits) and needs no range
// scale: with the lazy rescale p < 2^8, well inside bf16's exponent range.
// P^T operand of MFMA step st (16 keys): lane (q, h) supplies elements
// 8*(st%2) .. +7 of key block st/2, i.e. dwords P[st][0..3] hold the bf16
// pairs of S[st/2][8*(st%2) + 2w], S[st/2][8*(st%2) + 2w + 1].
// Lh is the lane's share of its row's sum of weights, rescaled with O.
template <int NO>
__device__ __forceinline__ void softmax_tile32_bf16(v16f (&S)[4], float c, float& m_run, v16f (&O)[NO], float& Lh,
                                                    v4i (&P)[8]) {
  float m4[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    float a = fmaxf(S[kb][0], S[kb][1]), b = fmaxf(S[kb][2], S[kb][3]);
#pragma unroll
    for (int i = 4; i < 16; i += 4) {
      a = fmaxf(a, fmaxf(S[kb][i], S[kb][i + 1]));
      b = fmaxf(b, fmaxf(S[kb][i + 2], S[kb][i + 3]));
    }
    m4[kb] = fmaxf(a, b);
  }
  const float mx = max_with_lane_xor32(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
  const float tmax = mx * c;
  const float m_new = fmaxf(m_run, tmax);
  const bool grow = __builtin_amdgcn_ballot_w64(m_new > m_run + kLazyRescale) != 0;
  if (__builtin_expect(grow, 0)) {
    const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
    for (int o = 0; o < NO; ++o) O[o] *= alpha;
    Lh *= alpha;
    m_run = m_new;
  }
  const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) S[kb][i] = __builtin_amdgcn_exp2f(fmaf(S[kb][i], c, -m_use));
#pragma unroll
  for (int st = 0; st < 8; ++st)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int i = 8 * (st & 1) + 2 * w;
      P[st][w] = (int)bf16x2(S[st >> 1][i], S[st >> 1][i + 1]);
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide max over 256 threads (4 waves).
__device__ __forceinline__ float block_max256(float v, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) red[wv] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  return v;
}

// Quantize 8 bf16 (one uint4) with the tile's inverse scale -> 8 E4M3 bytes.
__device__ __forceinline__ uint2 e4m3_quantize8(uint4 w, float inv) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    b[i] = e4m3_pack2(clamp448(bf16_lo(ws[i]) * inv), clamp448(bf16_hi(ws[i]) * inv), 1.0f);
  return make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
}

// Streaming access for the quantizers: loads of inputs read once and stores
// of codes that another kernel reads later carry the non-temporal bit, so
// the stream does not displace cached lines (the V quantizer: 9.6 -> 7.7 us
// for 50 MB), where each wave's stores cover whole 128-byte lines.  The KV
// append ran slower with the hint on its loads and code stores (16.9 ->
// 22.4 us for a 4096-token prompt; its K-code rows are 64-byte pieces spread
// over the cache, its inputs token-major rows) and keeps plain accesses.
typedef uint32_t v4u_nt __attribute__((ext_vector_type(4)));
typedef uint32_t v2u_nt __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const v4u_nt r = __builtin_nontemporal_load(reinterpret_cast<const v4u_nt*>(p));
  return make_uint4(r[0], r[1], r[2], r[3]);
}
__device__ __forceinline__ void store_nt16(void* p, uint4 v) {
  __builtin_nontemporal_store(v4u_nt{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u_nt*>(p));
}
__device__ __forceinline__ void store_nt8(void* p, uint2 v) {
  __builtin_nontemporal_store(v2u_nt{v.x, v.y}, reinterpret_cast<v2u_nt*>(p));
}
__device__ __forceinline__ void store_nt4(void* p, uint32_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}


}  // namespace qk4v8
