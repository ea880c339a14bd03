// KV-cache append: new tokens' K rows to MXFP4 and V rows to per-tile FP8,
// written into the cache layout the decode kernel reads.
//
// "MpFA免训练量化：QK4V8混合精度在Blackwell上的推理加速实践" §6.1: the KV cache is
// kept quantized, so every new token is quantized when it is written; §3.2:
// each block's scale comes from the block itself.  For V the block is a tile of
// R rows of one (batch, kv-head), so the last tile of a sequence keeps growing
// as tokens arrive and its scale must always be that of all the rows it holds.
// E8M0 scales are monotone in the absolute maximum, so the new scale of a
// filling tile is max(old, scale of the new rows): when it does not change,
// only the new rows are encoded (their codes are the same as a full
// re-quantization would give); when it grows, the tile is re-quantized from
// the bf16 rows the caller's tail buffer keeps for the partial tile.
//
// One launch: workgroups [0, bh * slots) handle the V tiles touched by the
// append, one per (b, kv-head, tile); the rest quantize the new K rows, one
// thread per (b, token, kv-head, 32-element block).  Only the workgroup of the
// first touched tile of a sequence reads that sequence's tail buffer, and the
// same workgroup writes the new tail rows after a barrier, so no other
// workgroup races with it.
#include "qk4v8_device.h"
#include "qk4v8_launch.h"

namespace qk4v8 {

namespace {

// Cache length of sequence b, or -1 when the append does not fit.
__device__ __forceinline__ int append_len(const AppendParams& p, int b) {
  const int len = p.kv_lens ? p.kv_lens[b] : p.kv_len;
  return (len < 0 || (int64_t)len + p.n_new > p.cap) ? -1 : len;
}

// Cache row of position pos of (b, h): rows [b][h][cap] in a contiguous
// cache, [page][h][page_size] in a paged one (page ids from the block table).
__device__ __forceinline__ int64_t cache_row(const AppendParams& p, int b, int h, int pos) {
  if (p.block_table == nullptr) return ((int64_t)b * p.kv_heads + h) * p.cap + pos;
  const int64_t page = p.block_table[(int64_t)b * p.pages_per_seq + pos / p.page_size];
  return (page * p.kv_heads + h) * p.page_size + pos % p.page_size;
}

// Index of the E8M0 scale of V tile `tile` (R rows) of (b, h); a page holds
// whole V tiles.
__device__ __forceinline__ int64_t vscale_index(const AppendParams& p, int b, int h, int tile) {
  if (p.block_table == nullptr) return ((int64_t)b * p.kv_heads + h) * p.n_vtiles_cap + tile;
  const int pos = tile * p.R;
  const int64_t page = p.block_table[(int64_t)b * p.pages_per_seq + pos / p.page_size];
  return (page * p.kv_heads + h) * (p.page_size / p.R) + (pos % p.page_size) / p.R;
}

template <int D>
__device__ __forceinline__ void append_k(const AppendParams& p, int64_t id, int64_t total) {
  constexpr int NB = D / 32;
  if (id >= total) return;
  const int g = (int)(id % NB);
  const int64_t rest = id / NB;
  const int h = (int)(rest % p.kv_heads);
  const int64_t bt = rest / p.kv_heads;
  const int t = (int)(bt % p.n_new);
  const int b = (int)(bt / p.n_new);
  const int len = append_len(p, b);
  if (len < 0) return;
  const uint4* src = reinterpret_cast<const uint4*>(p.k_new + b * p.ks[0] + t * p.ks[1] + h * p.ks[2] + 32 * g);
  uint32_t w[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 x = src[q];
    w[4 * q] = x.x; w[4 * q + 1] = x.y; w[4 * q + 2] = x.z; w[4 * q + 3] = x.w;
  }
  uint32_t codes[4];
  uint32_t scale;
  if (!p.hadamard) {
    scale = mxfp4_quantize32(w, codes);
  } else {
    // rotated K rows: the NB threads of a row are adjacent lanes (g fastest),
    // and every exit above is taken by whole rows, so the pairs are complete
    float x[32];
    unpack_bf16x32(w, x);
    fwht32(x);
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = hadamard_pair(x[i], __shfl_xor(x[i], 1, 64), (g & 1) != 0);
    if constexpr (NB == 4) {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = hadamard_pair(x[i], __shfl_xor(x[i], 2, 64), (g & 2) != 0);
    }
    scale = mxfp4_quantize32f(x, codes);
  }
  const int64_t row = cache_row(p, b, h, len + t);
  *reinterpret_cast<uint4*>(p.k_codes + row * (D / 2) + 16 * g) = make_uint4(codes[0], codes[1], codes[2], codes[3]);
  p.k_scales[row * NB + g] = (uint8_t)scale;
}

// Workgroup per (b, h, slot): slot s handles tile floor(len/R) + s.  Rows of
// the tile in [len, end) are new (from v_new); rows in [tile*R, len) were
// cached earlier and their bf16 values are in the tail buffer.  With REG
// (appends of many rows) the new rows stay in registers between the maximum
// and the encode (a tile holds at most 256 rows: VPT 16-byte chunks per
// thread), all requested at once; otherwise (a few rows per tile, where the
// registers would only lower occupancy) they are read twice, the second time
// from L2.
template <int D, bool REG>
__device__ __forceinline__ void append_v(const AppendParams& p, int64_t wg, int slots, float* red) {
  constexpr int CPR = D / 8;                        // 16-byte chunks per row
  constexpr int VPT = REG ? 256 * CPR / 256 : 1;    // chunks per thread for the largest tile
  const int slot = (int)(wg % slots);
  const int64_t bh = wg / slots;
  const int b = (int)(bh / p.kv_heads), h = (int)(bh - (int64_t)b * p.kv_heads);
  const int len = append_len(p, b);
  if (len < 0) return;
  const int R = p.R;
  const int end = len + p.n_new;
  const int tile = len / R + slot;
  const int r0 = tile * R;
  if (r0 >= end) return;                            // uniform across the workgroup
  const int r1 = min(r0 + R, end);
  const int first_new = max(r0, len);
  // absolute maximum of the new rows of this tile
  float amax = 0.0f;
  const int nvec_new = (r1 - first_new) * CPR;
  auto new_chunk = [&](int vi) -> uint4 {
    const int r = first_new + vi / CPR, cc = vi % CPR;
    return *reinterpret_cast<const uint4*>(p.v_new + b * p.vs[0] + (int64_t)(r - len) * p.vs[1] + h * p.vs[2] + cc * 8);
  };
  auto absmax8 = [&](const uint4& w) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(ws[k])), fabsf(bf16_hi(ws[k]))));
  };
  uint4 wv[VPT];
  if constexpr (REG) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int vi = (int)threadIdx.x + 256 * i;
      wv[i] = vi < nvec_new ? new_chunk(vi) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) absmax8(wv[i]);
  } else {
    for (int vi = threadIdx.x; vi < nvec_new; vi += 256) absmax8(new_chunk(vi));
  }
  amax = block_max256(amax, red);
  uint8_t* const scale_ptr = p.v_scales + vscale_index(p, b, h, tile);
  const bool has_old = len > r0;                    // the tile was partly filled before
  int X = mx_shared_exp(amax, 8);
  const int X_old = has_old ? (int)*scale_ptr - 127 : -127;
  const bool requant = has_old && X > X_old;
  X = max(X, X_old);
  const float inv = exp2i(-X);
  // codes of the tile's first row; its rows are consecutive cache rows
  uint8_t* const codes = p.v_codes + cache_row(p, b, h, r0) * D;
  // re-encode the earlier rows from their bf16 values when the scale grew
  if (requant) {
    const uint16_t* tail = p.v_tail + bh * R * D;
    const int nvec_old = (len - r0) * CPR;
    for (int vi = threadIdx.x; vi < nvec_old; vi += 256) {
      const int i = vi / CPR, cc = vi % CPR;
      const uint4 w = *reinterpret_cast<const uint4*>(tail + (int64_t)i * D + cc * 8);
      *reinterpret_cast<uint2*>(codes + (int64_t)i * D + cc * 8) = e4m3_quantize8(w, inv);
    }
  }
  auto put_chunk = [&](int vi, const uint4& w) {
    const int r = first_new + vi / CPR, cc = vi % CPR;
    *reinterpret_cast<uint2*>(codes + (int64_t)(r - r0) * D + cc * 8) = e4m3_quantize8(w, inv);
  };
  if constexpr (REG) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int vi = (int)threadIdx.x + 256 * i;
      if (vi < nvec_new) put_chunk(vi, wv[i]);
    }
  } else {
    for (int vi = threadIdx.x; vi < nvec_new; vi += 256) put_chunk(vi, new_chunk(vi));
  }
  if (threadIdx.x == 0) *scale_ptr = (uint8_t)(X + 127);
  if (slot != 0) return;
  // the new rows of the sequence's last, partial tile go to the tail buffer,
  // after every read of it above (rows already there stay)
  __syncthreads();
  const int t_last = end / R;
  const int first = max(t_last * R, len);
  const int nvec_tail = (end - first) * CPR;
  uint16_t* const tail = p.v_tail + bh * R * D;
  for (int vi = threadIdx.x; vi < nvec_tail; vi += 256) {
    const int r = first + vi / CPR, cc = vi % CPR;
    const uint4 w = *reinterpret_cast<const uint4*>(p.v_new + b * p.vs[0] + (int64_t)(r - len) * p.vs[1] +
                                                    h * p.vs[2] + cc * 8);
    *reinterpret_cast<uint4*>(tail + (int64_t)(r - t_last * R) * D + cc * 8) = w;
  }
}

template <int D, bool REG>
__global__ void __launch_bounds__(256) append_kernel(AppendParams p, int slots, int64_t v_wgs, int64_t total_k) {
  __shared__ float red[4];
  if ((int64_t)blockIdx.x < v_wgs)
    append_v<D, REG>(p, blockIdx.x, slots, red);
  else
    append_k<D>(p, ((int64_t)blockIdx.x - v_wgs) * 256 + threadIdx.x, total_k);
}

}  // namespace

template <int D>
static hipError_t launch_append_d(const AppendParams& p, hipStream_t stream) {
  const int64_t bh = (int64_t)p.batch * p.kv_heads;
  // tiles touched per sequence: at most ceil(n_new / R) + 1
  const int slots = (p.n_new + p.R - 1) / p.R + 1;
  const int64_t v_wgs = bh * slots;
  const int64_t total_k = bh * p.n_new * (D / 32);
  const int64_t k_wgs = (total_k + 255) / 256;
  const dim3 grid((unsigned)(v_wgs + k_wgs));
  // tiles of many new rows keep them in registers (prompts); a few rows per
  // sequence (decode steps, drafted blocks) take the low-register variant
  if (p.n_new >= 64)
    hipLaunchKernelGGL((append_kernel<D, true>), grid, dim3(256), 0, stream, p, slots, v_wgs, total_k);
  else
    hipLaunchKernelGGL((append_kernel<D, false>), grid, dim3(256), 0, stream, p, slots, v_wgs, total_k);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  return p.head_dim == 64 ? launch_append_d<64>(p, stream) : launch_append_d<128>(p, stream);
}

}  // namespace qk4v8
