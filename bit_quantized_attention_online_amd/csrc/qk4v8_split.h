// Split-K sizing of the decode / block-verify kernel: plain C++ with no HIP
// dependency, so the formula can be checked on the host with any CU count and
// occupancy.
//
// Split-K is the decode parallelisation of "MpFA免训练量化：QK4V8混合精度在
// Blackwell上的推理加速实践" §1.3 / §6.1 (decode is memory-bound: the KV range of
// one sequence is read by several workgroups at once and their partial results
// are merged by log-sum-exp).
#pragma once

#include <stdint.h>

namespace qk4v8 {

// Keys the split range of one sequence covers at most: kv_len, or with a
// sliding window the window, the query block and up to 127 keys before the
// window's first key (the range starts at a 128-key tile boundary).
inline int decode_key_span(int kv_len, int q_len, int window) {
  if (window > 0 && (int64_t)window + q_len + 126 < kv_len) return window + q_len + 126;
  return kv_len;
}

// Query rows of one KV head -> 16-row blocks, one wave each (1..4).
inline int decode_row_blocks(int rows) { return rows <= 16 ? 1 : rows <= 32 ? 2 : rows <= 48 ? 3 : 4; }

// Splits of the KV range per (batch, kv-head).
//   units    : batch * kv_heads (independent workgroup columns)
//   span     : keys per sequence the splits cover (decode_key_span)
//   capacity : workgroups the device holds at once (CUs x resident
//              workgroups per CU of the kernel that will run)
//   requested: > 0 forces that count (at most one split per 128-key tile)
// With requested == 0 the splits fill one round of resident workgroups (a
// second, partial round and larger fp32 partials cost more than they balance),
// each split keeping at least 8 tiles of work (below that the merge pass costs
// more than the parallelism gains; one split writes the output without it).
// Returns 0 when capacity is unknown (0) and no count was requested.
inline int decode_split_count(int64_t units, int span, int64_t capacity, int requested) {
  const int tiles = (span + 127) / 128;
  if (requested > 0) return requested < tiles ? requested : (tiles > 0 ? tiles : 1);
  if (capacity <= 0) return 0;
  if (units < 1) units = 1;
  int64_t s = (capacity + units / 2) / units;
  const int max_s = tiles / 8 > 0 ? tiles / 8 : 1;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return (int)s;
}

}  // namespace qk4v8
