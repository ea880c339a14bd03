// Peak microbenchmarks for gfx950 (see include/qk4v8_peaks.h): HBM streaming
// read, scaled FP4 / FP8 and bf16 MFMA issue rate, v_exp_f32 rate.  The QK4V8 kernels'
// roofline fractions are reported against both the vendor's nominal peaks and
// these measured ones ("MpFA免训练量化：QK4V8混合精度在Blackwell上的推理加速实践"
// §5.1 compares compute and bandwidth utilisation with what the hardware
// delivers).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qk4v8_peaks.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;         // 16-byte loads in flight per thread
constexpr int kLoopThreads = 512;      // 8 waves per CU for the MFMA and exp loops

// Each workgroup streams one contiguous slice of the buffer, kReadUnroll
// 16-byte non-temporal buffer loads per thread in flight, and folds the words
// into one value per thread; the slices cover the buffer exactly once.
__global__ void __launch_bounds__(kReadThreads) hbm_read_kernel(const uint8_t* buf, uint64_t n16,
                                                                uint64_t per_wg, uint32_t* sink) {
  const uint64_t first = (uint64_t)blockIdx.x * per_wg;
  const uint64_t last = first + per_wg < n16 ? first + per_wg : n16;
  uint32_t acc = 0;
  for (uint64_t base = first; base < last; base += (uint64_t)kReadThreads * kReadUnroll) {
    // a buffer resource bounded to the slice's remaining bytes: loads past it return zeros
    const uint64_t left = (last - base) * 16;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(buf + base * 16), (short)0, (int)(left < 0x7FFFFFF0ull ? left : 0x7FFFFFF0ull),
        0x00020000);
    v4i x[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      x[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (threadIdx.x + u * kReadThreads) * 16, 0, 2);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= (uint32_t)(x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3]);
  }
  sink[(blockIdx.x * kReadThreads + threadIdx.x) & 4095] = acc;
}

template <int FMT>
__global__ void __launch_bounds__(kLoopThreads) mfma_loop_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  const v8i a = v8i{lane, lane * 3, lane ^ 5, 7, lane, 1, 2, 3};
  const v8i b = v8i{lane * 5, lane, 9, lane ^ 3, 4, 5, 6, lane};
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, FMT, FMT, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, FMT, FMT, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, FMT, FMT, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, FMT, FMT, 0, 127, 0, 127);
  }
  sink[blockIdx.x * kLoopThreads + threadIdx.x] = c0[0] + c1[1] + c2[2] + c3[3];
}

__global__ void __launch_bounds__(kLoopThreads) mfma_bf16_loop_kernel(int iters, float* sink) {
  typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
  const int lane = threadIdx.x & 63;
  const v4i ai = v4i{lane, lane * 3, 0x3F803F80, 7};
  const v4i bi = v4i{lane * 5, 0x3F803F80, 9, lane};
  const v8bf a = __builtin_bit_cast(v8bf, ai), b = __builtin_bit_cast(v8bf, bi);
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  sink[blockIdx.x * kLoopThreads + threadIdx.x] = c0[0] + c1[1] + c2[2] + c3[3];
}

__global__ void __launch_bounds__(kLoopThreads) exp2_loop_kernel(int iters, float* sink) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = -0.001f * (float)(threadIdx.x + j);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(x[j]);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  sink[blockIdx.x * kLoopThreads + threadIdx.x] = s;
}

int cu_count(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 6;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || *cus < 1) return 6;
  return 0;
}

}  // namespace

extern "C" {

int qk4v8_peak_hbm_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (buf == nullptr || sink == nullptr) return 1;
  if (bytes < 16 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0) return 2;
  int cus = 0;
  if (int st = cu_count(&cus)) return st;
  const uint64_t n16 = bytes / 16;
  const uint64_t wgs = (uint64_t)cus * 8;
  const uint64_t per_wg = (n16 + wgs - 1) / wgs;
  const uint64_t grid = (n16 + per_wg - 1) / per_wg;
  hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)grid), dim3(kReadThreads), 0, stream,
                     static_cast<const uint8_t*>(buf), n16, per_wg, sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

int qk4v8_peak_mfma(int fmt, int iters, float* sink, double* flops, hipStream_t stream) {
  if (sink == nullptr || flops == nullptr) return 1;
  if ((fmt != 0 && fmt != 4 && fmt != 16) || iters < 1 || iters > (1 << 24)) return 2;
  int cus = 0;
  if (int st = cu_count(&cus)) return st;
  if (fmt == 4)
    hipLaunchKernelGGL(mfma_loop_kernel<4>, dim3(cus), dim3(kLoopThreads), 0, stream, iters, sink);
  else if (fmt == 0)
    hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(cus), dim3(kLoopThreads), 0, stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_bf16_loop_kernel, dim3(cus), dim3(kLoopThreads), 0, stream, iters, sink);
  *flops = (double)cus * (kLoopThreads / 64) * iters * 4.0 * (2.0 * 32 * 32 * (fmt == 16 ? 16 : 64));
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

int qk4v8_peak_exp2(int iters, float* sink, double* exps, hipStream_t stream) {
  if (sink == nullptr || exps == nullptr) return 1;
  if (iters < 1 || iters > (1 << 24)) return 2;
  int cus = 0;
  if (int st = cu_count(&cus)) return st;
  hipLaunchKernelGGL(exp2_loop_kernel, dim3(cus), dim3(kLoopThreads), 0, stream, iters, sink);
  *exps = (double)cus * kLoopThreads * iters * 8.0;
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
