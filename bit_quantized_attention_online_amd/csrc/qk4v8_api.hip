// C-ABI host layer of libqk4v8: argument validation, device check, launches.
//
// The MpFA page ("MpFA免训练量化：QK4V8混合精度在Blackwell上的推理加速实践") §4.2
// and §5.2 warn that a Q/K/V stride or layout mismatch shows up as an illegal
// memory access; every size, stride and alignment is therefore checked on the
// host before anything is enqueued, and a failed check returns a status.
#include <atomic>
#include <cmath>
#include <cstring>

#include "qk4v8.h"
#include "qk4v8_launch.h"

using namespace qk4v8;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_v_tile(int r) { return r == 32 || r == 64 || r == 128 || r == 256; }

// gfx950 check, memoised per device ordinal (the only state the library keeps).
qk4v8_status check_device() {
  static std::atomic<int> verdict[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QK4V8_ERR_HIP;
  if (dev >= 0 && dev < 64) {
    const int v = verdict[dev].load(std::memory_order_relaxed);
    if (v == 1) return QK4V8_OK;
    if (v == 2) return QK4V8_ERR_UNSUPPORTED;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QK4V8_ERR_HIP;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) verdict[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? QK4V8_OK : QK4V8_ERR_UNSUPPORTED;
}

qk4v8_status from_hip(hipError_t e) { return e == hipSuccess ? QK4V8_OK : QK4V8_ERR_HIP; }

bool good_scale(float s) { return std::isfinite(s) && s > 0.0f; }

// A paged cache: pages of page_size keys (a multiple of the 128-key tile and
// of the V tile), pages_per_seq entries per sequence in the block table, and
// the per-sequence capacity equal to pages_per_seq * page_size.
bool valid_paging(const int32_t* block_table, int page_size, int pages_per_seq, int v_tile_rows, int cap) {
  if (block_table == nullptr) return true;
  if (page_size < 128 || page_size % 128 != 0 || page_size % v_tile_rows != 0 || pages_per_seq < 1) return false;
  return (int64_t)page_size * pages_per_seq == cap && (reinterpret_cast<uintptr_t>(block_table) & 3) == 0;
}

// The kernel mode of a call's p_mode (QK4V8_P_DEFAULT picks the library's
// default, QK4V8_P_DEFAULT_MODE).
PMode prefill_mode(const qk4v8_prefill_args* a) {
  const int m = a->p_mode == QK4V8_P_DEFAULT ? QK4V8_P_DEFAULT_MODE : a->p_mode;
  return m == QK4V8_P_FP8_SINGLE ? kPSingle : m == QK4V8_P_BF16 ? kPBf16 : kPTwoTerm;
}

qk4v8_status validate_prefill(const qk4v8_prefill_args* a) {
  if (a == nullptr) return QK4V8_ERR_NULL;
  if (a->batch < 0 || a->q_heads < 1 || a->kv_heads < 1 || a->seq_q < 0 || a->seq_k < 0) return QK4V8_ERR_SHAPE;
  if (a->q_heads % a->kv_heads != 0) return QK4V8_ERR_SHAPE;
  if (a->head_dim != 64 && a->head_dim != 128) return QK4V8_ERR_SHAPE;
  if (!valid_v_tile(a->v_tile_rows)) return QK4V8_ERR_SHAPE;
  if (a->causal != 0 && a->causal != 1) return QK4V8_ERR_SHAPE;
  if (a->seq_q > 0 && a->seq_k < 1) return QK4V8_ERR_SHAPE;
  if (a->causal && a->seq_q > a->seq_k) return QK4V8_ERR_SHAPE;
  if (!good_scale(a->softmax_scale)) return QK4V8_ERR_SHAPE;
  if (a->seq_q > (1 << 30) || a->seq_k > (1 << 30)) return QK4V8_ERR_SHAPE;
  if (a->p_mode < QK4V8_P_DEFAULT || a->p_mode > QK4V8_P_BF16) return QK4V8_ERR_SHAPE;
  if (a->hadamard != 0 && a->hadamard != 1) return QK4V8_ERR_SHAPE;
  if (a->window < 0 || (a->window > 0 && !a->causal)) return QK4V8_ERR_SHAPE;
  return QK4V8_OK;
}

qk4v8_status validate_prefill_memory(const qk4v8_prefill_args* a) {
  if (!a->q || !a->k || !a->v || !a->o) return QK4V8_ERR_NULL;
  const int64_t* strides[4] = {a->q_stride, a->k_stride, a->v_stride, a->o_stride};
  for (auto s : strides)
    for (int i = 0; i < 3; ++i)
      if (s[i] < 0 || s[i] % 8 != 0) return QK4V8_ERR_STRIDE;
  if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->o, 16)) return QK4V8_ERR_STRIDE;
  if (a->lse && !aligned(a->lse, 4)) return QK4V8_ERR_STRIDE;
  // rows of one head must not overlap, nor may heads of the output
  const int d = a->head_dim;
  if (a->seq_q > 1 && (a->q_stride[2] < d || a->o_stride[2] < d)) return QK4V8_ERR_STRIDE;
  if (a->seq_k > 1 && (a->k_stride[2] < d || a->v_stride[2] < d)) return QK4V8_ERR_STRIDE;
  if (a->q_heads > 1 && a->o_stride[1] < d) return QK4V8_ERR_STRIDE;
  if (a->workspace == nullptr || !aligned(a->workspace, kWsAlign)) return QK4V8_ERR_WORKSPACE;
  const PrefillLayout L =
      prefill_layout(a->batch, a->kv_heads, a->seq_k, a->head_dim, a->v_tile_rows, prefill_mode(a) == kPBf16);
  if (a->workspace_bytes < L.total) return QK4V8_ERR_WORKSPACE;
  return QK4V8_OK;
}

qk4v8_status validate_decode(const qk4v8_decode_args* a) {
  if (a == nullptr) return QK4V8_ERR_NULL;
  if (a->batch < 0 || a->q_heads < 1 || a->kv_heads < 1 || a->q_len < 1) return QK4V8_ERR_SHAPE;
  if (a->q_heads % a->kv_heads != 0) return QK4V8_ERR_SHAPE;
  if (a->head_dim != 64 && a->head_dim != 128) return QK4V8_ERR_SHAPE;
  if (!valid_v_tile(a->v_tile_rows)) return QK4V8_ERR_SHAPE;
  if (a->kv_len < a->q_len || a->cap < a->kv_len || a->cap > (1 << 30)) return QK4V8_ERR_SHAPE;
  if ((int64_t)(a->q_heads / a->kv_heads) * a->q_len > 64) return QK4V8_ERR_SHAPE;
  if (a->num_splits < 0) return QK4V8_ERR_SHAPE;
  if (!good_scale(a->softmax_scale)) return QK4V8_ERR_SHAPE;
  if (a->hadamard != 0 && a->hadamard != 1) return QK4V8_ERR_SHAPE;
  if (a->window < 0) return QK4V8_ERR_SHAPE;
  if (!valid_paging(a->block_table, a->page_size, a->pages_per_seq, a->v_tile_rows, a->cap)) return QK4V8_ERR_SHAPE;
  return QK4V8_OK;
}

int decode_splits(const qk4v8_decode_args* a) {
  return decode_num_splits(a->batch, a->kv_heads, (a->q_heads / a->kv_heads) * a->q_len, a->head_dim,
                           decode_key_span(a->kv_len, a->q_len, a->window), a->num_splits);
}

// Buffers of a decode call.  `caller_ws`: the partials go to the caller's
// workspace (checked here); otherwise to the library's fixed array, whose
// size bounds the call.  *need receives the partials' bytes.
qk4v8_status validate_decode_memory(const qk4v8_decode_args* a, bool caller_ws, size_t* need) {
  if (!a->q || !a->k_codes || !a->k_scales || !a->v_codes || !a->v_scales || !a->o) return QK4V8_ERR_NULL;
  for (int i = 0; i < 3; ++i)
    if (a->q_stride[i] < 0 || a->q_stride[i] % 8 != 0 || a->o_stride[i] < 0) return QK4V8_ERR_STRIDE;
  if (!aligned(a->q, 16) || !aligned(a->o, 2) || !aligned(a->k_codes, 16) || !aligned(a->v_codes, 16))
    return QK4V8_ERR_STRIDE;
  if (!aligned(a->k_scales, a->head_dim == 128 ? 4 : 2)) return QK4V8_ERR_STRIDE;
  if (a->kv_lens && !aligned(a->kv_lens, 4)) return QK4V8_ERR_STRIDE;
  if (a->lse && !aligned(a->lse, 4)) return QK4V8_ERR_STRIDE;
  if (a->q_heads > 1 && a->o_stride[2] < a->head_dim) return QK4V8_ERR_STRIDE;
  if (a->q_len > 1 && a->o_stride[1] < a->head_dim) return QK4V8_ERR_STRIDE;
  const int splits = decode_splits(a);
  if (splits < 1) return QK4V8_ERR_HIP;   // the device's occupancy query failed
  *need = decode_workspace_bytes(a->batch, a->q_len, a->q_heads, a->kv_heads, a->head_dim, splits);
  if (caller_ws) {
    if (a->workspace == nullptr || !aligned(a->workspace, kWsAlign)) return QK4V8_ERR_WORKSPACE;
    if (a->workspace_bytes < *need) return QK4V8_ERR_WORKSPACE;
  } else if (*need > kNoAllocScratchBytes) {
    return QK4V8_ERR_WORKSPACE;
  }
  return QK4V8_OK;
}

}  // namespace

extern "C" {

int qk4v8_abi_version(void) { return QK4V8_ABI_VERSION; }

const char* qk4v8_status_string(int status) {
  switch (status) {
    case QK4V8_OK: return "ok";
    case QK4V8_ERR_NULL: return "null pointer";
    case QK4V8_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case QK4V8_ERR_STRIDE: return "misaligned pointer or invalid stride";
    case QK4V8_ERR_UNSUPPORTED: return "device is not gfx950";
    case QK4V8_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case QK4V8_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

qk4v8_status qk4v8_quantize_qk(const uint16_t* x, int64_t rows, int32_t d, int64_t ld, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream) {
  if (rows < 0 || d <= 0 || d % 32 != 0 || d > 1024) return QK4V8_ERR_SHAPE;
  if (rows > ((int64_t)1 << 40) / d) return QK4V8_ERR_SHAPE;
  if (ld < d || ld % 8 != 0) return QK4V8_ERR_STRIDE;
  if (rows == 0) return QK4V8_OK;
  if (!x || !codes || !scales) return QK4V8_ERR_NULL;
  if (!aligned(x, 16) || !aligned(codes, 4)) return QK4V8_ERR_STRIDE;
  if ((rows * (d / 8) + 255) / 256 > 0x7FFFFFFF) return QK4V8_ERR_SHAPE;
  qk4v8_status st = check_device();
  if (st != QK4V8_OK) return st;
  return from_hip(launch_quantize_qk(x, rows, d, ld, codes, scales, stream));
}

qk4v8_status qk4v8_quantize_v(const uint16_t* v, int64_t groups, int64_t n, int32_t d, int64_t group_stride,
                              int64_t row_stride, int32_t tile_rows, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream) {
  if (groups < 0 || n < 0 || d <= 0 || d % 8 != 0 || d > 512 || !valid_v_tile(tile_rows)) return QK4V8_ERR_SHAPE;
  if (row_stride < d || row_stride % 8 != 0 || group_stride < 0 || group_stride % 8 != 0) return QK4V8_ERR_STRIDE;
  if (groups == 0 || n == 0) return QK4V8_OK;
  if (!v || !codes || !scales) return QK4V8_ERR_NULL;
  if (!aligned(v, 16) || !aligned(codes, 8)) return QK4V8_ERR_STRIDE;
  if (groups * ((n + tile_rows - 1) / tile_rows) > 0x7FFFFFFF) return QK4V8_ERR_SHAPE;
  qk4v8_status st = check_device();
  if (st != QK4V8_OK) return st;
  return from_hip(launch_quantize_v(v, groups, n, d, group_stride, row_stride, tile_rows, codes, scales, stream));
}

size_t qk4v8_prefill_workspace_bytes(const qk4v8_prefill_args* a) {
  if (validate_prefill(a) != QK4V8_OK) return 0;
  return prefill_layout(a->batch, a->kv_heads, a->seq_k, a->head_dim, a->v_tile_rows, prefill_mode(a) == kPBf16).total;
}

}  // extern "C"

namespace {

// A decode call; caller_ws false: the partials live in the library's fixed
// per-device array (qk4v8_attn_decode_noalloc), nothing is allocated.
qk4v8_status run_decode(const qk4v8_decode_args* a, hipStream_t stream, bool caller_ws) {
  qk4v8_status st = validate_decode(a);
  if (st != QK4V8_OK) return st;
  if (a->batch == 0) return QK4V8_OK;
  size_t need = 0;
  st = validate_decode_memory(a, caller_ws, &need);
  if (st != QK4V8_OK) return st;
  st = check_device();
  if (st != QK4V8_OK) return st;
  DecodeParams p;
  p.q = a->q; p.k_codes = a->k_codes; p.k_scales = a->k_scales; p.v_codes = a->v_codes; p.v_scales = a->v_scales;
  p.kv_lens = a->kv_lens; p.o = a->o; p.lse = a->lse;
  for (int i = 0; i < 3; ++i) { p.qs[i] = a->q_stride[i]; p.os[i] = a->o_stride[i]; }
  p.batch = a->batch; p.q_len = a->q_len; p.q_heads = a->q_heads; p.kv_heads = a->kv_heads; p.kv_len = a->kv_len;
  p.cap = a->cap; p.head_dim = a->head_dim; p.v_tile_rows = a->v_tile_rows;
  p.num_splits = a->num_splits; p.softmax_scale = a->softmax_scale;
  p.hadamard = a->hadamard;
  p.window = a->window;
  p.block_table = a->block_table; p.page_size = a->page_size; p.pages_per_seq = a->pages_per_seq;
  p.ws = static_cast<uint8_t*>(a->workspace);
  return from_hip(caller_ws ? launch_decode(p, stream) : launch_decode_noalloc(p, need, stream));
}

enum PrefillPart { kPack = 1, kAttn = 2 };

qk4v8_status run_prefill(const qk4v8_prefill_args* a, hipStream_t stream, int parts) {
  qk4v8_status st = validate_prefill(a);
  if (st != QK4V8_OK) return st;
  if (a->batch == 0 || a->seq_q == 0) return QK4V8_OK;
  st = validate_prefill_memory(a);
  if (st != QK4V8_OK) return st;
  st = check_device();
  if (st != QK4V8_OK) return st;
  PrefillParams p;
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o; p.lse = a->lse;
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = a->q_stride[i]; p.ks[i] = a->k_stride[i]; p.vs[i] = a->v_stride[i]; p.os[i] = a->o_stride[i];
  }
  p.batch = a->batch; p.q_heads = a->q_heads; p.kv_heads = a->kv_heads; p.seq_q = a->seq_q; p.seq_k = a->seq_k;
  p.head_dim = a->head_dim; p.v_tile_rows = a->v_tile_rows; p.causal = a->causal;
  p.p_mode = prefill_mode(a);
  p.hadamard = a->hadamard;
  p.window = a->window;
  p.softmax_scale = a->softmax_scale;
  p.ws = static_cast<uint8_t*>(a->workspace);
  if (parts & kPack) {
    st = from_hip(launch_prefill_pack(p, stream));
    if (st != QK4V8_OK) return st;
  }
  if (parts & kAttn) st = from_hip(launch_prefill_attn(p, stream));
  return st;
}

}  // namespace

extern "C" {

qk4v8_status qk4v8_attn_prefill(const qk4v8_prefill_args* a, hipStream_t stream) {
  return run_prefill(a, stream, kPack | kAttn);
}

qk4v8_status qk4v8_prefill_pack_kv(const qk4v8_prefill_args* a, hipStream_t stream) {
  return run_prefill(a, stream, kPack);
}

qk4v8_status qk4v8_attn_prefill_packed(const qk4v8_prefill_args* a, hipStream_t stream) {
  return run_prefill(a, stream, kAttn);
}

size_t qk4v8_decode_workspace_bytes(const qk4v8_decode_args* a) {
  if (validate_decode(a) != QK4V8_OK) return 0;
  const int splits = decode_splits(a);
  if (splits < 1) return 0;
  return decode_workspace_bytes(a->batch, a->q_len, a->q_heads, a->kv_heads, a->head_dim, splits);
}

qk4v8_status qk4v8_kv_append(const qk4v8_append_args* a, hipStream_t stream) {
  if (a == nullptr) return QK4V8_ERR_NULL;
  if (a->batch < 0 || a->kv_heads < 1 || a->n_new < 0 || a->cap < 0) return QK4V8_ERR_SHAPE;
  if (a->head_dim != 64 && a->head_dim != 128) return QK4V8_ERR_SHAPE;
  if (!valid_v_tile(a->v_tile_rows)) return QK4V8_ERR_SHAPE;
  if (a->kv_lens == nullptr && (a->kv_len < 0 || (int64_t)a->kv_len + a->n_new > a->cap)) return QK4V8_ERR_SHAPE;
  if (a->cap > (1 << 30)) return QK4V8_ERR_SHAPE;
  if (a->hadamard != 0 && a->hadamard != 1) return QK4V8_ERR_SHAPE;
  if (!valid_paging(a->block_table, a->page_size, a->pages_per_seq, a->v_tile_rows, a->cap)) return QK4V8_ERR_SHAPE;
  for (int i = 0; i < 3; ++i)
    if (a->k_stride[i] < 0 || a->k_stride[i] % 8 != 0 || a->v_stride[i] < 0 || a->v_stride[i] % 8 != 0)
      return QK4V8_ERR_STRIDE;
  if (a->batch == 0 || a->n_new == 0) return QK4V8_OK;
  if (!a->k_new || !a->v_new || !a->k_codes || !a->k_scales || !a->v_codes || !a->v_scales || !a->v_tail)
    return QK4V8_ERR_NULL;
  if (!aligned(a->k_new, 16) || !aligned(a->v_new, 16) || !aligned(a->v_tail, 16) || !aligned(a->k_codes, 16) ||
      !aligned(a->v_codes, 8))
    return QK4V8_ERR_STRIDE;
  if (a->kv_lens && !aligned(a->kv_lens, 4)) return QK4V8_ERR_STRIDE;
  const int64_t bh = (int64_t)a->batch * a->kv_heads;
  if (bh * ((a->n_new + a->v_tile_rows - 1) / a->v_tile_rows + 1) > 0x7FFFFFFF ||
      (bh * a->n_new * (a->head_dim / 32) + 255) / 256 > 0x7FFFFFFF)
    return QK4V8_ERR_SHAPE;
  qk4v8_status st = check_device();
  if (st != QK4V8_OK) return st;
  AppendParams p;
  p.k_new = a->k_new; p.v_new = a->v_new;
  for (int i = 0; i < 3; ++i) { p.ks[i] = a->k_stride[i]; p.vs[i] = a->v_stride[i]; }
  p.k_codes = a->k_codes; p.k_scales = a->k_scales; p.v_codes = a->v_codes; p.v_scales = a->v_scales;
  p.v_tail = a->v_tail; p.kv_lens = a->kv_lens;
  p.batch = a->batch; p.kv_heads = a->kv_heads; p.n_new = a->n_new; p.kv_len = a->kv_len; p.cap = a->cap;
  p.head_dim = a->head_dim; p.R = a->v_tile_rows; p.hadamard = a->hadamard;
  p.n_vtiles_cap = (a->cap + a->v_tile_rows - 1) / a->v_tile_rows;
  p.block_table = a->block_table; p.page_size = a->page_size; p.pages_per_seq = a->pages_per_seq;
  return from_hip(launch_append(p, stream));
}

qk4v8_status qk4v8_attn_decode(const qk4v8_decode_args* a, hipStream_t stream) {
  return run_decode(a, stream, true);
}

qk4v8_status qk4v8_attn_decode_noalloc(const qk4v8_decode_args* a, hipStream_t stream) {
  return run_decode(a, stream, false);
}

}  // extern "C"
