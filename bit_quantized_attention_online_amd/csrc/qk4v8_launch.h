// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qk4v8_split.h"

namespace qk4v8 {

constexpr int kKvTile = 128;    // keys per attention KV tile
constexpr int kWsAlign = 256;   // workspace sub-buffer alignment (bytes)

hipError_t launch_quantize_qk(const uint16_t* x, int64_t rows, int d, int64_t ld, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream);
hipError_t launch_quantize_v(const uint16_t* v, int64_t groups, int64_t n, int d, int64_t group_stride,
                             int64_t row_stride, int R, uint8_t* codes, uint8_t* scales, hipStream_t stream);

// Prefill: the quantized copies of K and V live in the caller's workspace in
// the layouts the attention kernel consumes (see prefill.hip).
// How the probabilities enter P·V.
enum PMode {
  kPTwoTerm = 0,   // FP8 MFMA, two E4M3 terms per weight
  kPSingle = 1,    // FP8 MFMA, one E4M3 term (fast mode)
  kPBf16 = 2       // BF16 MFMA: bf16 weights against V widened exactly to bf16
};

struct PrefillLayout {
  int64_t n_tiles;        // ceil(seq_k / 128)
  int64_t n_vtiles;       // ceil(seq_k / v_tile_rows)
  int64_t rec_bytes;      // one packed K/V tile record
  size_t off_rec, off_vtile, total;
};
// bf16_v: the records hold V as bf16 values (kPBf16) instead of E4M3 codes.
PrefillLayout prefill_layout(int batch, int kv_heads, int seq_k, int head_dim, int v_tile_rows, bool bf16_v);

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int64_t qs[3], ks[3], vs[3], os[3];
  int batch, q_heads, kv_heads, seq_q, seq_k, head_dim, v_tile_rows, causal;
  int p_mode;                // PMode
  int hadamard;              // 1: Q and K rotated by the Sylvester-Hadamard H_d
  int window;                // causal sliding window (0: none)
  float softmax_scale;
  uint8_t* ws;
};
hipError_t launch_prefill_pack(const PrefillParams& p, hipStream_t stream);
hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t stream);

struct DecodeParams {
  const uint16_t* q;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  const int32_t* kv_lens;
  uint16_t* o;
  float* lse;
  int64_t qs[3], os[3];
  int batch, q_len, q_heads, kv_heads, kv_len, cap, head_dim, v_tile_rows, num_splits;
  int hadamard;              // 1: queries rotated by H_d (the cache K was written rotated)
  int window;                // sliding window (0: none)
  const int32_t* block_table;  // paged cache: [batch, pages_per_seq] page ids, or NULL
  int page_size, pages_per_seq;
  float softmax_scale;
  uint8_t* ws;
};
// Splits of the KV range per (batch, kv-head); rows = (q_heads / kv_heads) * q_len.
// With requested == 0 the count comes from the current device's CU count and
// the split kernel's occupancy; 0 when that query fails.
int decode_num_splits(int batch, int kv_heads, int rows, int head_dim, int span, int requested);
size_t decode_workspace_bytes(int batch, int q_len, int q_heads, int kv_heads, int head_dim, int splits);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
// The same launch with the split partials in the library's fixed per-device
// array instead of p.ws (no allocation); `need` bytes must fit it.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t launch_decode_noalloc(DecodeParams p, size_t need, hipStream_t stream);

// KV-cache append: new K rows to MXFP4 and V rows to per-tile FP8 in the
// decode cache layout (see append.hip).
struct AppendParams {
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t ks[3], vs[3];      // {batch, token, head} element strides
  uint8_t* k_codes;
  uint8_t* k_scales;
  uint8_t* v_codes;
  uint8_t* v_scales;
  uint16_t* v_tail;          // [batch * kv_heads, R, head_dim]
  const int32_t* kv_lens;
  int batch, kv_heads, n_new, kv_len, cap, head_dim, R;
  int hadamard;              // 1: K rows rotated by H_d before quantization
  int64_t n_vtiles_cap;      // ceil(cap / R)
  const int32_t* block_table;  // paged cache: [batch, pages_per_seq] page ids, or NULL
  int page_size, pages_per_seq;
};
hipError_t launch_append(const AppendParams& p, hipStream_t stream);

}  // namespace qk4v8
