/*
 * qk4v8.h - C ABI of the QK4V8 attention library for MI355X (gfx950).
 *
 * QK4V8 is the training-free mixed-precision attention of the page
 * "MpFA免训练量化：QK4V8混合精度在Blackwell上的推理加速实践" (mhpn.cn/news/2564245,
 * below "MpFA page"): Q and K are quantized to 4 bits and V to 8 bits (§1.1,
 * §2.1, §2.2), each block's scale is computed at run time from the block itself
 * with no calibration data (§1.2, §3.2), and attention runs as a tiled online
 * softmax with an FP32 accumulator whose result is cast back to 16 bits (§2.3,
 * §3.3).  The 4-bit format is MXFP4: E2M1 values sharing one E8M0 scale per 32
 * elements, the block size named in "小米MiMo-V2.5-Pro-FP4-DFlash：FP4+推测解码的
 * 万亿推理提速指南" (wmrh.cn/news/72329, below "MiMo page"), section
 * "MXFP4专家量化".  V is FP8 E4M3FN with one power-of-two (E8M0) scale per tile of
 * rows.  The MpFA page §4.2 describes shipping the kernel as a standalone
 * extension whose Q/K/V strides must match the caller's layout; §5.2 lists a
 * stride mismatch as the cause of illegal memory accesses, so every stride is
 * validated here before any launch.
 *
 * Formats (bit layouts of the OCP MX v1.0 / OFP8 specifications):
 *   bf16 input        : uint16 bit patterns.
 *   MXFP4 codes       : uint8, two E2M1 codes per byte; byte k of a row holds
 *                       element 2k in its low nibble and element 2k+1 in its
 *                       high nibble.
 *   MXFP4 scales      : uint8 E8M0, one per 32 consecutive elements of a row;
 *                       byte b means 2^(b-127).  X = floor(log2 amax) - 2,
 *                       clamped to [-127, 127]; an all-zero block has b = 0.
 *   FP8 V codes       : uint8 E4M3FN, one per element.
 *   FP8 V scales      : uint8 E8M0, one per tile of `tile_rows` rows of one
 *                       (batch, kv-head); X = floor(log2 amax) - 8.
 *   Rounding          : round to nearest, ties to even, after saturating the
 *                       magnitude to the format's largest finite value (6 for
 *                       E2M1, 448 for E4M3FN).  The sign bit of a value that
 *                       rounds to zero is kept.
 *
 * Conventions for every call:
 *   - All data pointers are DEVICE pointers; the caller owns every buffer,
 *     including the workspace sized by the *_workspace_bytes queries.  The
 *     library allocates no device memory and keeps no data between calls
 *     (nothing is calibrated).  Its only state is per device ordinal and
 *     read-only once set: whether the device is a gfx950, the CU count times
 *     the decode kernels' occupancy (which sizes decode's automatic split
 *     count), and the address of the fixed array of
 *     qk4v8_attn_decode_noalloc.
 *   - Work is enqueued on `stream` and is asynchronous; the library never
 *     synchronizes the host.
 *   - Arguments are validated on the host before any launch; a failed check
 *     returns its status and enqueues nothing.  Nothing is printed and no
 *     C++ exception crosses the ABI.  A launch failure returns QK4V8_ERR_HIP.
 *   - NaN or Inf inputs are outside the contract.
 *   - The same inputs give the same bits on the same device.
 *   - Element strides are in elements of the pointed-to type; the innermost
 *     stride is always 1.  Row strides and base pointers of bf16 inputs must be
 *     16-byte aligned (row stride a multiple of 8 elements).
 */
#ifndef QK4V8_H
#define QK4V8_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QK4V8_ABI_VERSION 8

typedef enum {
  QK4V8_OK = 0,
  QK4V8_ERR_NULL = 1,        /* a required pointer is NULL                     */
  QK4V8_ERR_SHAPE = 2,       /* a size is negative, zero where it may not be,
                                or outside the supported set                    */
  QK4V8_ERR_STRIDE = 3,      /* a stride or pointer is misaligned or overlaps  */
  QK4V8_ERR_UNSUPPORTED = 4, /* the current device is not gfx950               */
  QK4V8_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required        */
  QK4V8_ERR_HIP = 6          /* a HIP launch or query failed                   */
} qk4v8_status;

/* Version of this ABI (QK4V8_ABI_VERSION of the library that was built). */
int qk4v8_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* qk4v8_status_string(int status);

/*
 * MXFP4 quantizer, the online per-block scale of MpFA page §3.2 applied to Q
 * or K along head_dim (blocks of 32 per the MiMo page, "MXFP4专家量化").
 *   x      : bf16 [rows, d], row stride `ld` elements (ld >= d, ld % 8 == 0).
 *   codes  : out, uint8 [rows, d/2], contiguous.
 *   scales : out, uint8 [rows, d/32], contiguous.
 *   d      : multiple of 32, at most 1024.  rows >= 0 (0 is a no-op).
 */
qk4v8_status qk4v8_quantize_qk(const uint16_t* x, int64_t rows, int32_t d, int64_t ld,
                               uint8_t* codes, uint8_t* scales, hipStream_t stream);

/*
 * FP8 E4M3FN quantizer for V with one E8M0 scale per tile of `tile_rows` rows
 * (MpFA page §2.2 keeps V at 8 bits; the per-tile scale is the online block
 * scale of §3.2).
 *   v            : bf16, element (g, i, c) at v[g*group_stride + i*row_stride + c]
 *                  (row_stride >= d, both multiples of 8).
 *   groups       : number of (batch, kv-head) pairs, >= 0.
 *   n            : rows per group, >= 0.  The last tile of a group may be
 *                  shorter than tile_rows.
 *   d            : multiple of 8, at most 512.
 *   tile_rows    : one of 32, 64, 128, 256.
 *   codes        : out, uint8 [groups, n, d], contiguous.
 *   scales       : out, uint8 [groups, ceil(n / tile_rows)], contiguous.
 */
qk4v8_status qk4v8_quantize_v(const uint16_t* v, int64_t groups, int64_t n, int32_t d,
                              int64_t group_stride, int64_t row_stride, int32_t tile_rows,
                              uint8_t* codes, uint8_t* scales, hipStream_t stream);

/* Probability formats of the prefill P·V product (qk4v8_prefill_args.p_mode). */
#define QK4V8_P_DEFAULT 0
#define QK4V8_P_FP8_SINGLE 1
#define QK4V8_P_FP8_TWO_TERM 2
#define QK4V8_P_BF16 3
#define QK4V8_P_DEFAULT_MODE QK4V8_P_BF16

/*
 * Prefill attention (MpFA page §2.3, §3.3): Q and K are quantized to MXFP4 and
 * V to FP8 (per-tile E8M0 scale) inside the call, then
 *   o_i = sum_j softmax_j(softmax_scale * q̂_i·k̂_j) v̂_j
 * with an FP32 online softmax and FP32 accumulator, stored as bf16.
 *
 *   q : bf16 [batch, q_heads, seq_q, head_dim], strides q_stride = {batch, head, token}
 *   k : bf16 [batch, kv_heads, seq_k, head_dim], strides k_stride
 *   v : bf16 [batch, kv_heads, seq_k, head_dim], strides v_stride
 *   o : out bf16 [batch, q_heads, seq_q, head_dim], strides o_stride
 *   lse : out fp32 [batch, q_heads, seq_q] contiguous, natural-log
 *         log-sum-exp of the scaled scores of each row; may be NULL.
 *   head_dim ∈ {64, 128}; q_heads % kv_heads == 0 and query head h reads KV
 *   head h / (q_heads / kv_heads) (GQA); v_tile_rows ∈ {32, 64, 128, 256};
 *   causal ∈ {0, 1}: row i sees keys j <= i + seq_k - seq_q (bottom-right),
 *   and needs seq_q <= seq_k.  seq_k >= 1 when seq_q >= 1.
 *   softmax_scale: applied in fp32 to the dequantized dot products.
 *   workspace : device scratch of at least qk4v8_prefill_workspace_bytes()
 *               bytes, 256-byte aligned; it receives the call's quantized
 *               copies of K and V.  Contents on return are unspecified.
 *   p_mode    : how the probabilities enter the P·V product (QK4V8_P_*):
 *               QK4V8_P_FP8_TWO_TERM (2): FP8 MFMA with two E4M3 terms per
 *               weight, hi = E4M3(p/2^X) and lo = E4M3((p - hi*2^X) / 2^(X-4)),
 *               one E8M0 range exponent X per query row and 128-key tile;
 *               about 2e-3 relative L2 from exact attention on the quantized
 *               operands.
 *               QK4V8_P_BF16 (3): bf16 weights (one RNE rounding of p) on the
 *               bf16 matrix core against V̂ widened to bf16: V is still
 *               quantized to E4M3 with its per-tile E8M0 scale (the same codes),
 *               and E4M3 * 2^X fits bf16 exactly, so only the weights' rounding
 *               differs; about 2e-3 relative L2 as well, with half the vector
 *               instructions per score of the two-term split.
 *               QK4V8_P_FP8_SINGLE (1, fast mode): FP8 MFMA with one E4M3 term
 *               per weight, an integral running maximum (every rescale an exact
 *               power of two) and one E8M0 range exponent per query row and
 *               aligned 32-key block (the MX block size); half the P·V matrix
 *               work, at about 2e-2 relative L2 from exact attention.  Its
 *               result is independent of the tiling: with base-2 scores
 *               t = s*log2(e) and 32-key blocks B aligned at multiples of 32,
 *               p~_j = 2^X_B * E4M3(2^(t_j - X_B)), X_B = floor(max_B t) - 7, and
 *               o = sum_j p~_j v_j / sum_j p~_j.
 *               QK4V8_P_DEFAULT (0): QK4V8_P_DEFAULT_MODE.
 *               The workspace holds V in the mode's format, so a pack call and
 *               the attention call that reads it must use the same p_mode.
 *   hadamard  : 1 rotates every Q and K row by the Sylvester-Hadamard matrix
 *               H_d (+-1 entries, H_2n = [[H_n, H_n], [H_n, -H_n]]) before its
 *               MXFP4 quantization (MpFA page §3.1: a rotation spreads outlier
 *               channels over all channels).  The rotation is evaluated in fp32
 *               with the butterfly stages h = 1, 2, ..., d/2 in that order, and
 *               the scores are multiplied by softmax_scale / d, since
 *               (H q).(H k) = d (q.k): exact attention is unchanged and only
 *               the quantization error moves.  0: no rotation.
 *   window    : causal sliding window (MiMo page, section "DFlash块扩散推测解码":
 *               the drafter attends to the most recent 1024 keys only).  0: no
 *               window; W > 0 (needs causal = 1): row i sees keys j with
 *               i + seq_k - seq_q - W < j <= i + seq_k - seq_q, and the call
 *               reads only the key tiles some row of a workgroup can see.
 *               W >= seq_k is the same as 0.
 */
typedef struct {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  int32_t batch, q_heads, kv_heads, seq_q, seq_k, head_dim, v_tile_rows, causal;
  float softmax_scale;
  void* workspace;
  size_t workspace_bytes;
  int32_t p_mode;
  int32_t hadamard;
  int32_t window;
} qk4v8_prefill_args;

/* Workspace bytes qk4v8_attn_prefill needs for these sizes (0 on bad sizes). */
size_t qk4v8_prefill_workspace_bytes(const qk4v8_prefill_args* a);
qk4v8_status qk4v8_attn_prefill(const qk4v8_prefill_args* a, hipStream_t stream);

/*
 * The two halves of qk4v8_attn_prefill, for callers that reuse one quantized
 * K/V for several query chunks, or time the attention kernel alone:
 *   qk4v8_prefill_pack_kv      quantizes K (MXFP4) and V (per-tile FP8) into the
 *                              workspace; reads k, v; ignores q, o and lse.
 *   qk4v8_attn_prefill_packed  runs the attention from a workspace filled by a
 *                              pack call with the same batch, kv_heads, seq_k,
 *                              head_dim and v_tile_rows; reads q, writes o and
 *                              lse; ignores k and v.
 * Validation and status codes are those of qk4v8_attn_prefill.
 */
qk4v8_status qk4v8_prefill_pack_kv(const qk4v8_prefill_args* a, hipStream_t stream);
qk4v8_status qk4v8_attn_prefill_packed(const qk4v8_prefill_args* a, hipStream_t stream);

/*
 * Decode / block-verify attention over a quantized KV cache (MpFA page §1.3:
 * decode is memory-bound and 4-bit K cuts its traffic; §6.1: combined with a
 * quantized KV cache).  q_len new query tokens per sequence (1 for decode, or a
 * drafted block verified in one pass as in the MiMo page, section
 * "DFlash块扩散推测解码"); query t of the block sees cache keys
 * j <= kv_len_b - q_len + t (bottom-right causal).  The queries are quantized
 * to MXFP4 inside the call.  The KV range is split across workgroups and the
 * partial results merged by log-sum-exp.
 *
 *   q        : bf16 [batch, q_len, q_heads, head_dim], strides q_stride = {batch, token, head}
 *   k_codes  : uint8 [batch, kv_heads, cap, head_dim/2]   (MXFP4, as qk4v8_quantize_qk)
 *   k_scales : uint8 [batch, kv_heads, cap, head_dim/32]
 *   v_codes  : uint8 [batch, kv_heads, cap, head_dim]     (E4M3FN, as qk4v8_quantize_v)
 *   v_scales : uint8 [batch, kv_heads, ceil(cap / v_tile_rows)]
 *   kv_lens  : device int32 [batch] with q_len <= kv_lens[b] <= kv_len, or NULL
 *              for every sequence having kv_len entries.  Cache rows at or
 *              past a sequence's length are never read (their bytes, and the
 *              V scales of tiles that start there, may be anything).  A
 *              length outside that range is outside the contract and is read
 *              on the device as follows: above kv_len it is taken as kv_len
 *              (no read past the capacity or the block-table row), below
 *              q_len the sequence is empty (zero output rows, lse -inf).
 *   o        : out bf16 [batch, q_len, q_heads, head_dim], strides o_stride
 *   lse      : out fp32 [batch, q_len, q_heads] contiguous, natural log; may be NULL.
 *   head_dim ∈ {64, 128}; v_tile_rows ∈ {32, 64, 128, 256};
 *   1 <= q_len <= kv_len <= cap; (q_heads / kv_heads) * q_len <= 64.
 *   num_splits: KV splits per (batch, kv-head), 0 = chosen by the library
 *              from the current device (one round of resident workgroups:
 *              CU count times the occupancy of the kernel that runs, at
 *              least 8 tiles of 128 keys per split; on MI355X 2 splits for
 *              decode at 32768 keys and 1 for a block of 64 query rows per
 *              KV head at head_dim 128, whose kernel holds one workgroup per
 *              CU); with 0 the workspace query and
 *              the call return 0 / QK4V8_ERR_HIP when no device answers.
 *   workspace : at least qk4v8_decode_workspace_bytes() bytes, 256-byte aligned
 *               (fp32 partial outputs and log-sum-exps of the splits; with a
 *               single split and an 8-byte aligned o whose strides are
 *               multiples of 4, o and lse are written directly and the
 *               workspace is not touched).
 *   hadamard  : 1 when the cache's K rows were rotated before quantization
 *               (qk4v8_kv_append with hadamard = 1); the queries are then
 *               rotated the same way and the scores multiplied by
 *               softmax_scale / head_dim (see qk4v8_prefill_args).  0: neither.
 *   window    : sliding window W (see qk4v8_prefill_args); 0: none.  Query t
 *               sees keys j with kv_len_b - q_len + t - W < j <= kv_len_b -
 *               q_len + t; the splits cover only the keys from the 128-key tile
 *               holding query 0's first visible key, so the traffic and the
 *               workspace are bounded by W + q_len + 126 keys per sequence.
 *   block_table, page_size, pages_per_seq : paged cache (pages of whole tiles
 *               named per sequence by a block table), or block_table = NULL
 *               for the contiguous layout above.  Paged: the four cache arrays are page pools
 *               k_codes [pages, kv_heads, page_size, head_dim/2],
 *               k_scales [pages, kv_heads, page_size, head_dim/32],
 *               v_codes [pages, kv_heads, page_size, head_dim],
 *               v_scales [pages, kv_heads, page_size / v_tile_rows];
 *               key j of sequence b is slot j % page_size of page
 *               block_table[b * pages_per_seq + j / page_size] (device int32,
 *               every entry a sequence reaches must name a valid page).
 *               page_size is a multiple of 128 and of v_tile_rows, and cap
 *               must equal pages_per_seq * page_size.  The result is the same
 *               bits as the contiguous cache holding the same rows.
 */
typedef struct {
  const uint16_t* q;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  const int32_t* kv_lens;
  uint16_t* o;
  float* lse;
  int64_t q_stride[3];
  int64_t o_stride[3];
  int32_t batch, q_len, q_heads, kv_heads, kv_len, cap, head_dim, v_tile_rows, num_splits;
  float softmax_scale;
  void* workspace;
  size_t workspace_bytes;
  int32_t hadamard;
  int32_t window;
  const int32_t* block_table;
  int32_t page_size;
  int32_t pages_per_seq;
} qk4v8_decode_args;

/* Workspace bytes qk4v8_attn_decode needs for these sizes (0 on bad sizes). */
size_t qk4v8_decode_workspace_bytes(const qk4v8_decode_args* a);
qk4v8_status qk4v8_attn_decode(const qk4v8_decode_args* a, hipStream_t stream);

/*
 * qk4v8_attn_decode without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  `workspace` and `workspace_bytes` are
 * ignored; the split partials go to a fixed device array of
 * QK4V8_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  The call allocates nothing and otherwise behaves
 * as qk4v8_attn_decode: the same arguments, validation, kernels and result
 * bits.  QK4V8_ERR_WORKSPACE when the partials (the bytes
 * qk4v8_decode_workspace_bytes reports) exceed the array; pass a smaller
 * num_splits then.  Calls on one GPU share its array and it keeps the last
 * call's partials: calls that overlap in time on one GPU (on different
 * streams, or from several host threads) race and may return wrong results.
 */
#define QK4V8_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
qk4v8_status qk4v8_attn_decode_noalloc(const qk4v8_decode_args* a, hipStream_t stream);

/*
 * KV-cache append (MpFA page §6.1: the cache is kept quantized, so new tokens
 * are quantized as they are written; §5.2).  Writes n_new new tokens per
 * sequence into the cache layout that qk4v8_attn_decode reads: K rows to MXFP4
 * (each row independently) and V rows to E4M3FN in the per-(batch, kv-head)
 * tiles of v_tile_rows rows.  A V tile that is still filling carries the scale
 * of all the rows it holds so far, so after any sequence of appends the cache
 * holds exactly what qk4v8_quantize_qk / qk4v8_quantize_v give for the whole
 * sequence.  When new rows raise a tile's E8M0 exponent, its earlier rows are
 * re-quantized from their bf16 values, which `v_tail` keeps for the last,
 * partial tile of every sequence.
 *
 *   k_new, v_new : bf16 [batch, n_new, kv_heads, head_dim], strides
 *                  k_stride / v_stride = {batch, token, head} (multiples of 8).
 *   kv_lens      : device int32 [batch]: tokens in each sequence's cache before
 *                  this call (NULL: kv_len for every sequence).  Not modified;
 *                  the caller advances it.  A sequence whose length is negative
 *                  or whose length + n_new exceeds cap is left untouched.
 *   k_codes, k_scales, v_codes, v_scales : the cache (qk4v8_attn_decode layout,
 *                  capacity cap tokens), updated in place.
 *   v_tail       : bf16 [batch, kv_heads, v_tile_rows, head_dim], contiguous,
 *                  owned by the caller and updated by the call.  Before the
 *                  call, row i of (b, h) must hold the source V row
 *                  R * floor(len_b / R) + i for i < len_b % R (as the previous
 *                  append left it; nothing is needed when len_b % R == 0).
 *   head_dim ∈ {64, 128}; v_tile_rows ∈ {32, 64, 128, 256}; n_new >= 0 (0 is a
 *   no-op); with kv_lens NULL, 0 <= kv_len and kv_len + n_new <= cap.
 *   hadamard     : 1 rotates the new K rows by H_d before quantization (for a
 *                  cache read by qk4v8_attn_decode with hadamard = 1); 0: not.
 *   block_table, page_size, pages_per_seq : a paged cache, laid out and
 *                  addressed as in qk4v8_decode_args; NULL: contiguous.
 */
typedef struct {
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t k_stride[3];
  int64_t v_stride[3];
  uint8_t* k_codes;
  uint8_t* k_scales;
  uint8_t* v_codes;
  uint8_t* v_scales;
  uint16_t* v_tail;
  const int32_t* kv_lens;
  int32_t batch, kv_heads, n_new, kv_len, cap, head_dim, v_tile_rows;
  int32_t hadamard;
  const int32_t* block_table;
  int32_t page_size;
  int32_t pages_per_seq;
} qk4v8_append_args;

qk4v8_status qk4v8_kv_append(const qk4v8_append_args* a, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QK4V8_H */
