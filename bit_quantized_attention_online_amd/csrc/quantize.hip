// Online quantizers (HBM-streaming): MXFP4 for Q/K rows and per-tile FP8 for V.
//
// "MpFA免训练量化：QK4V8混合精度在Blackwell上的推理加速实践" §3.2: the scale of a
// block is computed at run time from that block while it is loaded; here the
// block is 32 elements along head_dim for Q/K (MXFP4, block size from
// "小米MiMo-V2.5-Pro-FP4-DFlash：FP4+推测解码的万亿推理提速指南", section
// "MXFP4专家量化") and a tile of rows of one (batch, kv-head) for V (§2.2 keeps V
// at 8 bits).
#include "qk4v8_device.h"
#include "qk4v8_launch.h"

namespace qk4v8 {

// One lane per 8 consecutive elements; 4 adjacent lanes own one 32-element
// block and combine their maxima with two xor-shuffles.  Loads are 16 B per
// lane and the code stores 4 B per lane, both contiguous across the wave.
// Each thread takes CPT such chunks a grid apart, all loads issued before
// any encode, so a wave keeps CPT KB of reads in flight.
// cpr_shift: log2 of the chunks per row when that is a power of two (a
// shift instead of a 64-bit division), else -1.
template <int CPT>
__global__ void __launch_bounds__(256) quantize_qk_kernel(const uint16_t* __restrict__ x, int64_t rows, int d,
                                                          int64_t ld, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, int cpr_shift) {
  const int64_t chunks_per_row = d >> 3;
  auto row_of = [&](int64_t idx) __attribute__((always_inline)) {
    return cpr_shift >= 0 ? idx >> cpr_shift : idx / chunks_per_row;
  };
  const int64_t total = rows * chunks_per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t idx0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint4 w[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int64_t idx = idx0 + i * stride;
    w[i] = make_uint4(0, 0, 0, 0);
    if (idx < total) {
      const int64_t row = row_of(idx);
      w[i] = load_nt16(x + row * ld + (idx - row * chunks_per_row) * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    // a group of 4 lanes is all inside or all past the end (total is a
    // multiple of 4 chunks), so the shuffles below stay within live groups
    const int64_t idx = idx0 + i * stride;
    const bool live = idx < total;
    const int64_t row = live ? row_of(idx) : 0;
    const int chunk = live ? (int)(idx - row * chunks_per_row) : 0;
    const uint32_t ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(ws[k])), fabsf(bf16_hi(ws[k]))));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int X = mx_shared_exp(amax, 2);
    uint32_t c = 0;
    if (X >= -120) {
      // the bf16 pairs straight through the scaled convert (x / 2^X), as in
      // mxfp4_quantize32
      typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
      const float scale = exp2i(X);
      c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(v2bf, ws[0]), scale, 0);
      c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(v2bf, ws[1]), scale, 1);
      c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(v2bf, ws[2]), scale, 2);
      c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(v2bf, ws[3]), scale, 3);
    } else {
      const float inv = exp2i(-X);
#pragma unroll
      for (int k = 0; k < 4; ++k) c |= e2m1_pack2(bf16_lo(ws[k]) * inv, bf16_hi(ws[k]) * inv) << (8 * k);
    }
    if (live) {
      store_nt4(codes + row * (d >> 1) + chunk * 4, c);
      if ((chunk & 3) == 0) scales[row * (d >> 5) + (chunk >> 2)] = (uint8_t)(X + 127);
    }
  }
}

// One workgroup (256 threads) per (group, tile of R rows).  The tile stays in
// registers (VPT uint4 per thread) between the absmax and the encode phase.
template <int VPT>
__global__ void __launch_bounds__(256) quantize_v_kernel(const uint16_t* __restrict__ v, int64_t n, int d,
                                                         int64_t group_stride, int64_t row_stride, int R,
                                                         int64_t n_tiles, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t g = blockIdx.x / n_tiles;
  const int64_t t = blockIdx.x - g * n_tiles;
  const int64_t r0 = t * R;
  const int rows = (int)min((int64_t)R, n - r0);
  const int cpr = d >> 3;                    // uint4 chunks per row
  const int nvec = rows * cpr;
  const uint16_t* src = v + g * group_stride + r0 * row_stride;
  uint4 w[VPT];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int vi = threadIdx.x + i * 256;
    w[i] = make_uint4(0, 0, 0, 0);
    if (vi < nvec) {
      const int rr = vi / cpr, cc = vi - rr * cpr;
      w[i] = load_nt16(src + rr * row_stride + cc * 8);
    }
    const uint32_t ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(ws[k])), fabsf(bf16_hi(ws[k]))));
  }
  amax = block_max256(amax, red);
  const int X = mx_shared_exp(amax, 8);
  const float inv = exp2i(-X);
  uint8_t* dst = codes + (g * n + r0) * d;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int vi = threadIdx.x + i * 256;
    if (vi < nvec) store_nt8(dst + (int64_t)vi * 8, e4m3_quantize8(w[i], inv));
  }
  if (threadIdx.x == 0) scales[g * n_tiles + t] = (uint8_t)(X + 127);
}

// Same contract for tiles too large to keep in registers: two passes over the
// tile (the second pass mostly hits L2).
__global__ void __launch_bounds__(256) quantize_v_kernel_2pass(const uint16_t* __restrict__ v, int64_t n, int d,
                                                               int64_t group_stride, int64_t row_stride, int R,
                                                               int64_t n_tiles, uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t g = blockIdx.x / n_tiles, t = blockIdx.x - g * n_tiles, r0 = t * R;
  const int rows = (int)min((int64_t)R, n - r0);
  const int cpr = d >> 3, nvec = rows * cpr;
  const uint16_t* src = v + g * group_stride + r0 * row_stride;
  float amax = 0.0f;
  for (int vi = threadIdx.x; vi < nvec; vi += 256) {
    const int rr = vi / cpr, cc = vi - rr * cpr;
    const uint4 w = *reinterpret_cast<const uint4*>(src + rr * row_stride + cc * 8);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(ws[k])), fabsf(bf16_hi(ws[k]))));
  }
  amax = block_max256(amax, red);
  const int X = mx_shared_exp(amax, 8);
  const float inv = exp2i(-X);
  uint8_t* dst = codes + (g * n + r0) * d;
  for (int vi = threadIdx.x; vi < nvec; vi += 256) {
    const int rr = vi / cpr, cc = vi - rr * cpr;
    const uint4 w = *reinterpret_cast<const uint4*>(src + rr * row_stride + cc * 8);
    *reinterpret_cast<uint2*>(dst + (int64_t)vi * 8) = e4m3_quantize8(w, inv);
  }
  if (threadIdx.x == 0) scales[g * n_tiles + t] = (uint8_t)(X + 127);
}

hipError_t launch_quantize_qk(const uint16_t* x, int64_t rows, int d, int64_t ld, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream) {
  constexpr int kCpt = 4;   // chunks per thread
  const int64_t total = rows * (d >> 3);
  const int64_t blocks = (total + 256 * kCpt - 1) / (256 * kCpt);
  const int cpr = d >> 3;
  const int cpr_shift = (cpr & (cpr - 1)) == 0 ? __builtin_ctz((unsigned)cpr) : -1;
  hipLaunchKernelGGL((quantize_qk_kernel<kCpt>), dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, d, ld, codes,
                     scales, cpr_shift);
  return hipGetLastError();
}

hipError_t launch_quantize_v(const uint16_t* v, int64_t groups, int64_t n, int d, int64_t group_stride,
                             int64_t row_stride, int R, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t n_tiles = (n + R - 1) / R;
  const int64_t nvec = (int64_t)R * (d >> 3);
  const dim3 grid((unsigned)(n_tiles * groups));
  if (nvec <= 256 * 4)
    hipLaunchKernelGGL((quantize_v_kernel<4>), grid, dim3(256), 0, stream, v, n, d, group_stride, row_stride, R,
                       n_tiles, codes, scales);
  else if (nvec <= 256 * 16)
    hipLaunchKernelGGL((quantize_v_kernel<16>), grid, dim3(256), 0, stream, v, n, d, group_stride, row_stride, R,
                       n_tiles, codes, scales);
  else
    hipLaunchKernelGGL(quantize_v_kernel_2pass, grid, dim3(256), 0, stream, v, n, d, group_stride, row_stride, R,
                       n_tiles, codes, scales);
  return hipGetLastError();
}

}  // namespace qk4v8
