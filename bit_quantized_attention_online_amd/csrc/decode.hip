// QK4V8 decode / block-verify attention over a quantized KV cache (gfx950).
//
// "MpFA免训练量化：QK4V8混合精度在Blackwell上的推理加速实践" §1.3: decode attention
// is memory-bound and 4-bit K cuts its traffic; §6.1: pair it with a quantized
// KV cache.  "小米MiMo-V2.5-Pro-FP4-DFlash：FP4+推测解码的万亿推理提速指南", section
// "DFlash块扩散推测解码": a drafted block of tokens is verified by one backbone
// pass, i.e. q_len queries with a bottom-right causal mask over the cache.
//
// Split-K: one workgroup per (batch, KV head, split of the KV range).  The
// G*q_len query rows of a KV head (G = q_heads / kv_heads) form up to four
// 16-row blocks, one wave each; every wave streams the same 128-key tiles
// through LDS:
//   K codes (row-major, 16-byte chunks XOR-swizzled by row) -> QK^T A operand
//   (16 B per lane),
//   V codes (row-major, 16-byte chunks XOR-swizzled by row) -> ds_read_tr8_b64
//   gathers 8 keys of one column per lane, which is the P·V A operand layout.
// The next tile is fetched into registers while one computes, by buffer loads
// bounded to the sequence and marked non-temporal (the cache is streamed
// once).  Each split writes its normalized fp32 partial output and
// log2-sum-exp; the merge kernel combines splits with log-sum-exp weights.
//
// Four row blocks at head_dim 128 (a drafted block of 8 tokens over 8 query
// heads per KV head) run verify_pingpong_kernel instead: two 4-wave groups
// per workgroup, one workgroup per CU, that take turns between matrix and
// vector work, with tiles copied from global memory straight into LDS.
//
// Sliding window (MiMo page, section "DFlash块扩散推测解码": the drafter keeps
// only the most recent 1024 keys): the splits cover the keys from the tile
// holding the first query's first visible key to the end of the sequence, so
// the work and the traffic do not grow with the length of the cache.
#include <atomic>

#include "qk4v8_device.h"
#include "qk4v8_launch.h"

namespace qk4v8 {

namespace {

constexpr int kMaxDevices = 64;   // device ordinals the per-device caches cover

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNT = 2;      // buffer-load cache policy: non-temporal (nt)

typedef int v2i __attribute__((ext_vector_type(2)));
typedef v2i __attribute__((address_space(3))) * lds_v2i_ptr;

}  // namespace

struct DecodeArgs {
  const uint16_t* q;
  const uint8_t* kc;
  const uint8_t* ksc;
  const uint8_t* vc;
  const uint8_t* vsc;
  const int32_t* kv_lens;
  float* part_o;      // [bk][split][M][D]
  float* part_lse;    // [bk][split][M]  (log2 domain)
  uint16_t* o;        // final output and lse, written directly by a single split
  float* lse;
  int64_t os0, os1, os2;
  int q_heads;
  int direct;         // one split and an 8-byte aligned output: no merge pass
  int64_t qs0, qs1, qs2;
  int kv_heads, group, q_len, M, kv_len, cap, R, splits, tiles_per_split;
  int64_t n_vtiles_cap;
  int log2R;        // log2 of the V tile rows R
  float c;          // softmax_scale * log2(e), divided by D for rotated queries
  int hadamard;
  int window;       // > 0: query t sees only the `window` most recent keys up to its position
  const int32_t* block_table;   // paged cache: page ids [batch][pages_per_seq], or NULL
  int page_size, pages_per_seq;
};

template <int D>
struct DecTile {
  static constexpr int NB = D / 32;             // MXFP4 blocks per key
  static constexpr int NC = D / 16;             // 16-byte V chunks per key
  static constexpr int KRB = D / 2;             // K row bytes in LDS (16-byte chunks swizzled, kswz)
  static constexpr int K = 128 * KRB;
  static constexpr int KS = 128 * 4;            // one dword of scales per key
  static constexpr int V = 128 * D;
  static constexpr int VS = 16;                 // V scales of the four 32-key groups
  static constexpr int BYTES = K + KS + V + VS;
};

// K rows in LDS: the 16-byte chunk c of key row r sits at chunk position
// c ^ ((r / 16) % NB).  The QK^T operand read of one 16-lane group touches
// keys K0 + 16*a + b (a, b = 0..3, subtile_key), which with any 16-byte row
// stride share their banks across a: the XOR puts the four keys of equal b in
// four different chunk positions, so the group covers every bank once
// (measured without it: some 25M LDS bank-conflict cycles per block-verify
// launch).
template <int D>
__device__ __forceinline__ int kswz(int row, int chunk) {
  return chunk ^ ((row >> 4) & (DecTile<D>::NB - 1));
}

template <int D>
__device__ __forceinline__ int vswz(int row, int chunk) {
  return chunk ^ (row & (DecTile<D>::NC - 1));
}

// ---- pieces of the block-verify kernel below ----

// The sequence length a workgroup sees.  A length outside [q_len, kv_len] is
// outside the contract: above kv_len it is clamped to kv_len, so every read
// stays inside the cache's capacity (and a paged sequence inside its
// block-table row); below q_len the sequence is empty (zero output rows, lse
// -inf).
__device__ __forceinline__ int sequence_length(const DecodeArgs& a, int b) {
  const int n = a.kv_lens ? a.kv_lens[b] : a.kv_len;
  return n > a.kv_len ? a.kv_len : (n < a.q_len ? 0 : n);
}

// The keys [j_begin, j_end) split s covers, in ntiles 128-key tiles.  The
// splits share a range that starts at key 0, or with a window at the tile
// holding query 0's first visible key.
struct SplitRange {
  int j_begin, j_end, ntiles;
};
__device__ __forceinline__ SplitRange split_range(const DecodeArgs& a, int kvlen, int s) {
  SplitRange r;
  const int j_base = a.window > 0 ? max(0, kvlen - a.q_len + 1 - a.window) & ~127 : 0;
  r.j_begin = j_base + s * a.tiles_per_split * 128;
  r.j_end = min(kvlen, r.j_begin + a.tiles_per_split * 128);
  r.ntiles = r.j_end > r.j_begin ? (r.j_end - r.j_begin + 127) / 128 : 0;
  return r;
}

// Query row mrow = t * G + (head within the group) of a KV head: its position
// t, head, and the keys it sees, [low, low + span] (rows past M see none).
struct QueryRow {
  bool ok;
  int qt, head, low;
  uint32_t span;
};
__device__ __forceinline__ QueryRow query_row(const DecodeArgs& a, int kvh, int kvlen, int mrow) {
  QueryRow r;
  r.ok = mrow < a.M;
  r.qt = r.ok ? mrow / a.group : 0;
  r.head = kvh * a.group + (r.ok ? mrow - r.qt * a.group : 0);
  const int lim = r.ok ? kvlen - a.q_len + r.qt : -1;   // last visible key
  r.low = !r.ok ? (1 << 30) : a.window > 0 ? max(0, lim - a.window + 1) : 0;
  r.span = r.ok ? (uint32_t)(lim - r.low) : 0u;
  return r;
}

// The QK^T B operand of lane (row, k-block lg): the row's MXFP4 codes of
// head_dim block lg (zero past the row count and for lg >= NB) and their
// E8M0 scale.  Rotated queries: lane (q, g) holds block g, so the Hadamard
// stage across 32-element blocks pairs lanes l and l ^ 16 and the one across
// 64-element blocks lanes l and l ^ 32.
template <int D>
__device__ __forceinline__ v8i query_operand(const DecodeArgs& a, int b, const QueryRow& r, int lg, int& qsc) {
  constexpr int NB = D / 32;
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = 0;
  if (r.ok && lg < NB) {
    const uint4* src = reinterpret_cast<const uint4*>(a.q + b * a.qs0 + r.qt * a.qs1 + (int64_t)r.head * a.qs2 + 32 * lg);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 x = src[i];
      w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
    }
  }
  uint32_t cq[4] = {0, 0, 0, 0};
  qsc = 127;
  if (!a.hadamard) {
    if (r.ok && lg < NB) qsc = (int)mxfp4_quantize32(w, cq);
  } else {
    float x[32];
    unpack_bf16x32(w, x);
    fwht32(x);
    hadamard_stage_lane_xor16(x, (lg & 1) != 0);
    if constexpr (NB == 4) hadamard_stage_lane_xor32(x, (lg & 2) != 0);
    if (r.ok && lg < NB) qsc = (int)mxfp4_quantize32f(x, cq);
  }
  return fp4_operand(make_uint4(cq[0], cq[1], cq[2], cq[3]));
}

// Split s's rows of one wave: the normalized fp32 partial and its log2-sum-
// exp, or with one split (direct) the final bf16 output and natural-log lse,
// as the merge would write them.  Element i of column block dd in lane
// (row, lg) is column 16 dd + 4 lg + i.
template <int D>
__device__ __forceinline__ void store_split_rows(const DecodeArgs& a, const v4f (&O)[D / 16], const v4f& L, float m_run,
                                                 int64_t bk, int s, int b, int mrow, const QueryRow& r, int lg) {
  constexpr int ND = D / 16;
  if (!r.ok) return;
  const float l = L[0];
  const bool empty = !(l > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / l;
  if (a.direct) {
    uint16_t* orow = a.o + b * a.os0 + r.qt * a.os1 + (int64_t)r.head * a.os2;
#pragma unroll
    for (int dd = 0; dd < ND; ++dd) {
      const v4f v = O[dd] * inv;
      *reinterpret_cast<uint2*>(orow + dd * 16 + 4 * lg) = make_uint2(bf16x2(v[0], v[1]), bf16x2(v[2], v[3]));
    }
    if (a.lse != nullptr && lg == 0)
      a.lse[((int64_t)b * a.q_len + r.qt) * a.q_heads + r.head] = empty ? -INFINITY : (m_run + __log2f(l)) * kLn2;
    return;
  }
  const int64_t prow = (bk * a.splits + s) * a.M + mrow;
  float* dst = a.part_o + prow * D;
#pragma unroll
  for (int dd = 0; dd < ND; ++dd) *reinterpret_cast<v4f*>(dst + dd * 16 + 4 * lg) = O[dd] * inv;
  if (lg == 0) a.part_lse[prow] = empty ? -INFINITY : (m_run + __log2f(l));
}

template <int D, int MB>
__global__ void __launch_bounds__(MB * 64) __attribute__((amdgpu_waves_per_eu(MB == 4 ? 3 : 1, 8)))
decode_split_kernel(DecodeArgs a) {
  using T = DecTile<D>;
  constexpr int NB = T::NB, NC = T::NC, ND = D / 16;
  constexpr int NT = MB * 64;
  __shared__ __attribute__((aligned(16))) uint8_t lds[T::BYTES];
  uint8_t* lk = lds;
  uint8_t* lks = lds + T::K;
  uint8_t* lv = lds + T::K + T::KS;
  uint8_t* lvs = lds + T::K + T::KS + T::V;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 15, lg = lane >> 4;
  const int s = blockIdx.x % a.splits;
  const int64_t bk = blockIdx.x / a.splits;
  const int b = (int)(bk / a.kv_heads), kvh = (int)(bk - (int64_t)b * a.kv_heads);
  // a length outside [q_len, kv_len] is outside the contract: above kv_len
  // it is clamped to kv_len, so every read stays inside the cache's capacity
  // (and a paged sequence inside its block-table row); below q_len the
  // sequence is empty (zero output rows, lse -inf)
  int kvlen = a.kv_lens ? a.kv_lens[b] : a.kv_len;
  kvlen = kvlen > a.kv_len ? a.kv_len : (kvlen < a.q_len ? 0 : kvlen);
  // first key of the range the splits share: 0, or with a window the start of
  // the tile holding query 0's first visible key
  const int j_base = a.window > 0 ? max(0, kvlen - a.q_len + 1 - a.window) & ~127 : 0;
  const int j_begin = j_base + s * a.tiles_per_split * 128;
  const int j_end = min(kvlen, j_begin + a.tiles_per_split * 128);
  const int ntiles = j_end > j_begin ? (j_end - j_begin + 127) / 128 : 0;

  // ---- this wave's 16 query rows: row m = t * G + (head within group) ----
  const int mrow = wave * 16 + ql;
  const bool row_ok = mrow < a.M;
  const int qt = row_ok ? mrow / a.group : 0;
  const int head = kvh * a.group + (row_ok ? mrow - qt * a.group : 0);
  const int lim = row_ok ? kvlen - a.q_len + qt : -1;   // last visible key
  // first visible key (clamped at 0) and the count after it; rows past M see nothing
  const int low = !row_ok ? (1 << 30) : a.window > 0 ? max(0, lim - a.window + 1) : 0;
  const uint32_t span = row_ok ? (uint32_t)(lim - low) : 0u;
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = 0;
  if (row_ok && lg < NB) {
    const uint4* src = reinterpret_cast<const uint4*>(a.q + b * a.qs0 + qt * a.qs1 + (int64_t)head * a.qs2 + 32 * lg);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 x = src[i];
      w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
    }
  }
  uint32_t cq[4] = {0, 0, 0, 0};
  int qsc = 127;
  if (!a.hadamard) {
    if (row_ok && lg < NB) qsc = (int)mxfp4_quantize32(w, cq);
  } else {
    // rotated queries: lane (q, g) holds block g, so stage 32 pairs lanes
    // l and l ^ 16 and stage 64 lanes l and l ^ 32
    float x[32];
    unpack_bf16x32(w, x);
    fwht32(x);
    hadamard_stage_lane_xor16(x, (lg & 1) != 0);
    if constexpr (NB == 4) hadamard_stage_lane_xor32(x, (lg & 2) != 0);
    if (row_ok && lg < NB) qsc = (int)mxfp4_quantize32f(x, cq);
  }
  const v8i qf = fp4_operand(make_uint4(cq[0], cq[1], cq[2], cq[3]));

  v4f O[ND];
#pragma unroll
  for (int dd = 0; dd < ND; ++dd) O[dd] = v4f{0.f, 0.f, 0.f, 0.f};
  v4f L = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  v8i Phi = v8i{}, Plo = v8i{};
  const v8i ones = v8i{(int)kFp8Ones, (int)kFp8Ones, (int)kFp8Ones, (int)kFp8Ones,
                       (int)kFp8Ones, (int)kFp8Ones, (int)kFp8Ones, (int)kFp8Ones};
  const int klg = lg & (NB - 1);    // D = 64: lanes of k-blocks 2, 3 reread blocks 0, 1 (their Q is zero)
  // swizzled position of this lane's K chunk: (key / 16) % 4 is (ql / 4) % 4
  // for every key subtile_key(t, ql) gives, so it is the same for all t
  const int kchunk = kswz<D>(subtile_key(0, ql), klg) * 16;

  // ---- tile staging: the next tile is held in registers while this one
  // computes, then written to LDS (K rows padded, V chunks XOR-swizzled).
  // Buffer loads bounded to the rows inside the sequence: rows past kv_len
  // read as zero, so no cache byte beyond it (E4M3 NaN included) reaches the
  // accumulator, where 0 * NaN would survive the mask.  The loads are
  // unconditional (a tile past the range has no rows and touches no memory),
  // so the staged values need no copies at the loop's back edge, which would
  // wait for every load in flight. ----
  constexpr int KCH = 128 * NB;          // 16-byte K chunks per tile
  constexpr int VCH = 128 * NC;          // 16-byte V chunks per tile
  constexpr int KPT = (KCH + NT - 1) / NT, VPT = (VCH + NT - 1) / NT, SPT = (128 + NT - 1) / NT;
  v4i rk[KPT], rv[VPT];   // clang vectors (not HIP's uint4 struct) so SROA keeps them in VGPRs
  uint32_t rs[SPT];
  uint8_t rvs;            // V scale of 32-key group tid & 3
  // Load cursor: the next tile starts at key ld_j of this sequence and KV
  // head.  Contiguous cache: rows [bk][cap] (row bk * cap + ld_j), V scales
  // [bk][cap / R]; paged cache: rows [page][kv_head][page_size] (slot
  // ld_slot of the sequence's page ld_page), V scales
  // [page][kv_head][page_size / R], and a page (a multiple of 128 keys and
  // of R) holds whole 128-key tiles and whole V tiles.
  const bool paged = a.block_table != nullptr;
  int ld_j = j_begin;
  int ld_page = paged ? j_begin / a.page_size : 0;
  int ld_slot = paged ? j_begin - ld_page * a.page_size : j_begin;
  // all accesses to the staging arrays use compile-time indices (static_for)
  // so they stay in registers
  auto dload = [&]() __attribute__((always_inline)) {
    const int rows = ld_j < j_end ? min(128, kvlen - ld_j) : 0;
    int64_t row0, vs0;
    if (!paged) {
      row0 = bk * (int64_t)a.cap;
      vs0 = bk * a.n_vtiles_cap;
    } else {
      const int64_t page = rows > 0 ? a.block_table[(int64_t)b * a.pages_per_seq + ld_page] : 0;
      row0 = (page * a.kv_heads + kvh) * a.page_size;
      vs0 = (page * a.kv_heads + kvh) * (a.page_size >> a.log2R);
    }
    const int64_t row = row0 + ld_slot;
    const __amdgpu_buffer_rsrc_t bk_ = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.kc + row * (D / 2)), (short)0, rows * (D / 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t bv_ = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.vc + row * D), (short)0, rows * D, 0x00020000);
    const __amdgpu_buffer_rsrc_t bs_ = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.ksc + row * NB), (short)0, rows * NB, 0x00020000);
    // V tiles of this tile's rows; a 32-key group past the sequence takes
    // the last row's scale (its V rows are zero)
    const __amdgpu_buffer_rsrc_t bvs_ = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.vsc + vs0 + (ld_slot >> a.log2R)), (short)0, rows > 0 ? 8 : 0, 0x00020000);
    // chunk ci of a tile is bytes [16 ci, 16 ci + 16) of its row-major rows;
    // the cache is streamed once, so the loads carry the non-temporal hint
    // (measured: ~15% more read bandwidth for streams of this shape)
    static_for<KPT>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int ci = tid + i * NT;
      if (KCH % NT == 0 || ci < KCH) rk[i] = __builtin_amdgcn_raw_buffer_load_b128(bk_, ci * 16, 0, kNT);
    });
    static_for<VPT>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int ci = tid + i * NT;
      if (VCH % NT == 0 || ci < VCH) rv[i] = __builtin_amdgcn_raw_buffer_load_b128(bv_, ci * 16, 0, kNT);
    });
    static_for<SPT>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int ki = tid + i * NT;
      if (128 % NT == 0 || ki < 128)
        rs[i] = NB == 4 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(bs_, ki * 4, 0, kNT)
                           : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(bs_, ki * 2, 0, kNT);
    });
    const int vrow = (ld_slot & ((1 << a.log2R) - 1)) + min(32 * (tid & 3), max(rows, 1) - 1);
    rvs = __builtin_amdgcn_raw_buffer_load_b8(bvs_, vrow >> a.log2R, 0, 0);
    ld_j += 128;
    ld_slot += 128;
    if (paged && ld_slot == a.page_size) { ld_slot = 0; ++ld_page; }
  };
  auto stage_to_lds = [&]() __attribute__((always_inline)) {
    static_for<KPT>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int ci = tid + i * NT;
      if (KCH % NT == 0 || ci < KCH) {
        const int row = ci / NB;
        *reinterpret_cast<v4i*>(lk + row * T::KRB + kswz<D>(row, ci % NB) * 16) = rk[i];
      }
    });
    static_for<VPT>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int ci = tid + i * NT;
      if (VCH % NT == 0 || ci < VCH) {
        const int row = ci / NC;
        *reinterpret_cast<v4i*>(lv + row * D + vswz<D>(row, ci % NC) * 16) = rv[i];
      }
    });
    static_for<SPT>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int ki = tid + i * NT;
      if (128 % NT == 0 || ki < 128) reinterpret_cast<uint32_t*>(lks)[ki] = rs[i];
    });
    // the V scales go through LDS too: a register holding one past the next
    // load would be copied at the back edge, after a wait for every load.
    // Threads with equal tid & 3 hold the same byte; all write it, so no
    // branch leaves the load pending for the compiler's wait counting.
    lvs[tid & 3] = rvs;
  };

  auto tile_step = [&](int it) __attribute__((always_inline)) {
    const int j0 = j_begin + it * 128;
    __syncthreads();            // previous tile fully consumed
    stage_to_lds();
    __syncthreads();            // this tile visible
    dload();

    // Wave priorities (workgroups of several waves, three resident per
    // SIMD): a wave issuing its QK^T reads and MFMAs runs at priority 1, one
    // issuing P·V at 2, the softmax at 0, so the matrix sections of the
    // waves on a SIMD go first and its vector work fills the gaps (block
    // verify 182 -> 175 us; a single-wave decode workgroup is alone on its
    // SIMD and skips this).
    if constexpr (MB >= 2) __builtin_amdgcn_s_setprio(1);
    // ---- S^T = K · Q^T ----
    v4f S[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int key = subtile_key(t, ql);
      const v8i af = fp4_operand(*reinterpret_cast<const uint4*>(lk + key * T::KRB + kchunk));
      const int sa = (int)((reinterpret_cast<const uint32_t*>(lks)[key] >> (8 * klg)) & 0xFF);
      S[t] = mfma16x16x128<kFmtFp4, kFmtFp4>(af, qf, v4f{0.f, 0.f, 0.f, 0.f}, sa, qsc);
    }
    if constexpr (MB >= 2) __builtin_amdgcn_s_setprio(0);
    // ---- mask: keys past this row's limit (covers kv_len and the causal
    // block) or, with a window, before its first visible key ----
    if (j0 + 127 > kvlen - a.q_len || !row_ok || (a.window > 0 && j0 < kvlen - a.window)) {
      // key(t, 4*lg + i) = j0 + 16*lg + subtile_key(t, i)
      const int low_l = low - j0 - 16 * lg;
      static_for<8>([&](auto T) {
        constexpr int t = decltype(T)::value;
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t][i] = mask_range(S[t][i], subtile_key(t, i), low_l, span);
      });
    }
    // ---- online softmax + two-term FP8 P ----
    int psc;
    softmax_tile<ND>(S, a.c, m_run, O, L, Phi, Plo, psc);
    if constexpr (MB >= 2) __builtin_amdgcn_s_setprio(2);
    // ---- O^T += V^T · P^T, L += 1 · P^T ----
    const int vs = lvs[lg];
    const int src_row_in_piece = ql >> 1, src_half = ql & 1;
#pragma unroll
    for (int dd = 0; dd < ND; ++dd) {
      v8i av;
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
        const int row = (pc >> 1) * 64 + 16 * lg + (pc & 1) * 8 + src_row_in_piece;
        const int addr = row * D + vswz<D>(row, dd) * 16 + src_half * 8;
        const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_ptr)(lv + addr));
        av[2 * pc] = r[0];
        av[2 * pc + 1] = r[1];
      }
      O[dd] = mfma16x16x128<kFmtFp8, kFmtFp8>(av, Phi, O[dd], vs, psc);
      O[dd] = mfma16x16x128<kFmtFp8, kFmtFp8>(av, Plo, O[dd], vs, psc - 4);
    }
    L = mfma16x16x128<kFmtFp8, kFmtFp8>(ones, Phi, L, 127, psc);
    L = mfma16x16x128<kFmtFp8, kFmtFp8>(ones, Plo, L, 127, psc - 4);
    if constexpr (MB >= 2) __builtin_amdgcn_s_setprio(0);
  };

  dload();
  for (int it = 0; it < ntiles; ++it) tile_step(it);

  // ---- write this split's normalized partial and its log2-sum-exp (one
  // split: the final bf16 output and natural-log lse, as the merge would) ----
  if (!row_ok) return;
  const float l = L[0];
  const int64_t prow = (bk * a.splits + s) * a.M + mrow;
  const bool empty = !(l > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / l;
  if (a.direct) {
    uint16_t* orow = a.o + b * a.os0 + qt * a.os1 + (int64_t)head * a.os2;
#pragma unroll
    for (int dd = 0; dd < ND; ++dd) {
      const v4f v = O[dd] * inv;
      *reinterpret_cast<uint2*>(orow + dd * 16 + 4 * lg) =
          make_uint2(bf16x2(v[0], v[1]), bf16x2(v[2], v[3]));
    }
    if (a.lse != nullptr && lg == 0)
      a.lse[((int64_t)b * a.q_len + qt) * a.q_heads + head] = empty ? -INFINITY : (m_run + __log2f(l)) * kLn2;
    return;
  }
  float* dst = a.part_o + prow * D;
#pragma unroll
  for (int dd = 0; dd < ND; ++dd) *reinterpret_cast<v4f*>(dst + dd * 16 + 4 * lg) = O[dd] * inv;
  if (lg == 0) a.part_lse[prow] = empty ? -INFINITY : (m_run + __log2f(l));
}

// ds_read_tr8_b64 through a restrict pointer: once inlined, the read carries
// alias metadata, without which the compiler's wait-count pass assumes it may
// alias any direct global->LDS load in flight and waits for all of them.
__device__ __forceinline__ v2i lds_read_tr8(const uint8_t* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_ptr)p);
}

// One 16-byte piece per lane from global memory straight into LDS, through
// a buffer resource (a load with the LDS bit): lane l copies bytes voffset ..
// voffset + 15 of the resource's range to lds_base + 16 l (lds_base
// wave-uniform).  Lanes past the range read nothing from memory.  Completion
// is counted in vmcnt like any other load.  The 4-byte form copies bytes
// voffset .. voffset + 3 to lds_base + 4 l; the 1-byte form writes the byte
// zero-extended to the dword at lds_base + 4 l.
__device__ __forceinline__ void load_to_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint8_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(lds_base)), 16,
      voffset, 0, 0, kNT);
}
__device__ __forceinline__ void load_to_lds4(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint8_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(lds_base)), 4,
      voffset, 0, 0, kNT);
}
__device__ __forceinline__ void load_to_lds1(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint8_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(lds_base)), 1,
      voffset, 0, 0, 0);
}

// vmcnt(N) on gfx9: vm_cnt[3:0] | exp_cnt[6:4] | lgkm_cnt[11:8] | vm_cnt[5:4]
// << 14, the other counters left at their maximum (no wait).
template <int N>
__device__ __forceinline__ void wait_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Block verify with four 16-row blocks at head_dim 128: a workgroup of two
// 4-wave groups that walk the even and the odd tiles of the split's key range
// in a ping-pong, one phase apart, so that in every phase one wave on each
// SIMD issues matrix instructions while the other runs the softmax.  Tiles go
// from global memory straight into LDS, three K and three V buffers per
// group, so no tile passes through registers; the two groups hold the same
// query rows and merge them through LDS at the end.
template <int D>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
verify_pingpong_kernel(DecodeArgs a) {
  using T = DecTile<D>;
  constexpr int NB = T::NB, ND = D / 16;
  static_assert(NB == 4 && D == 128, "one dword of K scales per key; 1 KB holds 16 K rows or 8 V rows");
  constexpr int KBUF = T::K + 1024;   // K codes, then the scales (in the order the QK^T reads them)
  constexpr int VBUF = T::V + 256;    // V codes, then the 32-key scales (group g's byte at 4 g)
  constexpr int GRP = 3 * KBUF + 3 * VBUF;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * GRP];

  // the wave index through readfirstlane: known wave-uniform, so the load
  // cursors and buffer resources stay in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;          // group 0 runs one phase ahead of group 1
  const int rb = wave & 3;            // this wave's 16-row block
  // loads one wave issues per vector phase: the K and V codes (2 + 4), and
  // half of the tile's K scales (waves 0 and 2) or its V scales (wave 1)
  const int phase_loads = rb < 3 ? 7 : 6;
  uint8_t* gk = lds + grp * GRP;      // K buffer i at gk + i * KBUF
  uint8_t* gv = gk + 3 * KBUF;        // V buffer i at gv + i * VBUF
  const int ql = lane & 15, lg = lane >> 4;
  const int s = blockIdx.x % a.splits;
  const int64_t bk = blockIdx.x / a.splits;
  const int b = (int)(bk / a.kv_heads), kvh = (int)(bk - (int64_t)b * a.kv_heads);
  const int kvlen = sequence_length(a, b);
  const SplitRange sr = split_range(a, kvlen, s);
  const int j_begin = sr.j_begin, j_end = sr.j_end, ntiles = sr.ntiles;

  const int mrow = rb * 16 + ql;
  const QueryRow qr = query_row(a, kvh, kvlen, mrow);
  const bool row_ok = qr.ok;
  const int low = qr.low;
  const uint32_t span = qr.span;
  int qsc;
  const v8i qf = query_operand<D>(a, b, qr, lg, qsc);

  v4f O[ND];
#pragma unroll
  for (int dd = 0; dd < ND; ++dd) O[dd] = v4f{0.f, 0.f, 0.f, 0.f};
  v4f L = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  v8i Phi = v8i{}, Plo = v8i{};
  const v8i ones = v8i{(int)kFp8Ones, (int)kFp8Ones, (int)kFp8Ones, (int)kFp8Ones,
                       (int)kFp8Ones, (int)kFp8Ones, (int)kFp8Ones, (int)kFp8Ones};
  const int kchunk = kswz<D>(subtile_key(0, ql), lg) * 16;

  // ---- loads: in vector phase k a group requests its tile k + 3's K and
  // tile k + 2's V, so each has two iterations to land.  Contiguous cache:
  // rows [bk][cap], V scales [bk][cap / R]; paged cache: rows
  // [page][kv_head][page_size], V scales [page][kv_head][page_size / R].
  // Resources bounded to the rows inside the sequence, so a tile past the
  // range, or the rows of the last tile past kv_len, touch no memory.  A
  // group's k-th tile is tile 2k + grp of the range, so its cursors step by
  // 256 keys. ----
  const bool paged = a.block_table != nullptr;
  struct Cursor { int j, page, slot; };
  auto cursor_at = [&](int j) __attribute__((always_inline)) {
    Cursor c;
    c.j = j;
    c.page = paged ? j / a.page_size : 0;
    c.slot = paged ? j - c.page * a.page_size : j;
    return c;
  };
  auto advance = [&](Cursor& c) __attribute__((always_inline)) {
    c.j += 256;
    c.slot += 256;
    while (paged && c.slot >= a.page_size) { c.slot -= a.page_size; ++c.page; }
  };
  auto locate = [&](const Cursor& c, int& rows, int64_t& row, int64_t& vs0) __attribute__((always_inline)) {
    rows = c.j < j_end ? min(128, kvlen - c.j) : 0;
    if (!paged) {
      row = bk * (int64_t)a.cap + c.slot;
      vs0 = bk * a.n_vtiles_cap;
    } else {
      // a scalar load through the constant address space (the table is
      // read-only here): a vector load would be counted with the tile loads
      // in flight, and waiting for the page id would wait for all of them
      typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
      const int64_t page = rows > 0 ? ((const_i32_ptr)(a.block_table))[(int64_t)b * a.pages_per_seq + c.page] : 0;
      const int64_t base = page * a.kv_heads + kvh;
      row = base * a.page_size + c.slot;
      vs0 = base * (a.page_size >> a.log2R);
    }
  };
  Cursor kcur = cursor_at(j_begin + grp * 128), vcur = kcur;
  // K codes: wave rb fills LDS kilobytes 2 rb and 2 rb + 1 (16 rows each);
  // the lane writing LDS chunk position p of row r fetches chunk p ^ ((r /
  // 16) % 4), the K-row swizzle.  K scales: waves 0 and 2, one dword per
  // lane, in the order the QK^T reads them (dword 8 q + t is the scale of
  // key subtile_key(t, q), so a lane reads its eight as two 16-byte
  // pieces); two waves rather than one or four, since every load
  // instruction costs the issuing SIMD time whatever its size.
  auto issue_k = [&](uint8_t* kb) __attribute__((always_inline)) {
    int rows;
    int64_t row, vs0;
    locate(kcur, rows, row, vs0);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.kc + row * (D / 2)), (short)0, rows * (D / 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.ksc + row * NB), (short)0, rows * NB, 0x00020000);
    static_for<2>([&](auto I) {
      const int c = rb * 2 + decltype(I)::value;
      load_to_lds16(rk, (uint32_t)(c * 1024 + (lane >> 2) * 64 + (((lane & 3) ^ (c & 3)) * 16)), kb + c * 1024);
    });
    if ((rb & 1) == 0) {
      const int slot = (rb >> 1) * 64 + lane;
      load_to_lds4(rs, (uint32_t)(subtile_key(slot & 7, slot >> 3) * 4), kb + T::K + (rb >> 1) * 256);
    }
    advance(kcur);
  };
  // V codes: wave rb fills LDS kilobytes 4 rb .. 4 rb + 3 (8 rows each);
  // the lane writing chunk position p of row r fetches chunk p ^ (r % 8).
  // V scales: wave 1 alone, lane l the byte of 32-key group l % 4 (a group
  // past the sequence takes the last row's scale) into LDS dword l,
  // zero-extended, so dword g holds group g's scale.
  auto issue_v = [&](uint8_t* vb) __attribute__((always_inline)) {
    int rows;
    int64_t row, vs0;
    locate(vcur, rows, row, vs0);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.vc + row * D), (short)0, rows * D, 0x00020000);
    const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.vsc + vs0 + (vcur.slot >> a.log2R)), (short)0, rows > 0 ? 8 : 0, 0x00020000);
    const int vrow = (vcur.slot & ((1 << a.log2R) - 1)) + min(32 * (lane & 3), max(rows, 1) - 1);
    if (rb == 1) load_to_lds1(rvs, (uint32_t)(vrow >> a.log2R), vb + T::V);
    static_for<4>([&](auto I) {
      const int c = rb * 4 + decltype(I)::value;
      load_to_lds16(rv, (uint32_t)(c * 1024 + (lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3)) * 16)), vb + c * 1024);
    });
    advance(vcur);
  };
  // Rows of the sequence's last tile past kv_len: the loads leave them
  // untouched or zero; they are cleared here, after this wave's loads of the
  // tile have landed, so no stale byte (an E4M3 NaN among them) meets a zero
  // weight in the P·V product.
  auto clear_tail = [&](uint8_t* vb, int tile) __attribute__((always_inline)) {
    const int rows = kvlen - (j_begin + tile * 128);
    if (rows < 128) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ci = (tid & 255) + 256 * i;   // 16-byte chunk of the tile
        if ((ci >> 3) >= rows) *reinterpret_cast<v4i*>(vb + ci * 16) = v4i{0, 0, 0, 0};
      }
    }
  };

  v4f S[8];
  int psc = 127;
  auto qk_tile = [&](const uint8_t* kb) __attribute__((always_inline)) {
    const v4i* ks = reinterpret_cast<const v4i*>(kb + T::K + ql * 32);
    const v4i ks0 = ks[0], ks1 = ks[1];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int key = subtile_key(t, ql);
      const v4i kv = *reinterpret_cast<const v4i*>(kb + key * T::KRB + kchunk);
      const v8i af = fp4_operand(make_uint4((uint32_t)kv[0], (uint32_t)kv[1], (uint32_t)kv[2], (uint32_t)kv[3]));
      const int sa = (int)(((uint32_t)(t < 4 ? ks0[t & 3] : ks1[t & 3]) >> (8 * lg)) & 0xFF);
      S[t] = mfma16x16x128<kFmtFp4, kFmtFp4>(af, qf, v4f{0.f, 0.f, 0.f, 0.f}, sa, qsc);
    }
  };
  auto mask_tile = [&](int it) __attribute__((always_inline)) {
    const int j0 = j_begin + it * 128;
    if (j0 + 127 > kvlen - a.q_len || !row_ok || (a.window > 0 && j0 < kvlen - a.window)) {
      const int low_l = low - j0 - 16 * lg;
      static_for<8>([&](auto TT) {
        constexpr int t = decltype(TT)::value;
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t][i] = mask_range(S[t][i], subtile_key(t, i), low_l, span);
      });
    }
  };
  // column blocks in pairs: the hi and the lo instruction of one block
  // accumulate into the same registers, so an independent instruction
  // between them keeps a wave alone on its SIMD from stalling
  auto pv_tile = [&](const uint8_t* vb) __attribute__((always_inline)) {
    const int vs = reinterpret_cast<const uint32_t*>(vb + T::V)[lg];
    const int src_row_in_piece = ql >> 1, src_half = ql & 1;
    auto v_operand = [&](int dd) __attribute__((always_inline)) {
      v8i av;
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
        const int row = (pc >> 1) * 64 + 16 * lg + (pc & 1) * 8 + src_row_in_piece;
        const int addr = row * D + vswz<D>(row, dd) * 16 + src_half * 8;
        const v2i r = lds_read_tr8(vb + addr);
        av[2 * pc] = r[0];
        av[2 * pc + 1] = r[1];
      }
      return av;
    };
#pragma unroll
    for (int dd = 0; dd < ND; dd += 2) {
      const v8i a0 = v_operand(dd), a1 = v_operand(dd + 1);
      O[dd] = mfma16x16x128<kFmtFp8, kFmtFp8>(a0, Phi, O[dd], vs, psc);
      O[dd + 1] = mfma16x16x128<kFmtFp8, kFmtFp8>(a1, Phi, O[dd + 1], vs, psc);
      O[dd] = mfma16x16x128<kFmtFp8, kFmtFp8>(a0, Plo, O[dd], vs, psc - 4);
      O[dd + 1] = mfma16x16x128<kFmtFp8, kFmtFp8>(a1, Plo, O[dd + 1], vs, psc - 4);
    }
    L = mfma16x16x128<kFmtFp8, kFmtFp8>(ones, Phi, L, 127, psc);
    L = mfma16x16x128<kFmtFp8, kFmtFp8>(ones, Plo, L, 127, psc - 4);
  };

  // ---- the ping-pong.  Iteration k of a group: a matrix phase (the two-term
  // split of tile k - 1's weights, the QK^T of tile k, the P·V of tile
  // k - 1) and a vector phase (tile k's V scales and tail, the loads of phase
  // k, the mask and softmax of tile k), each ended by a workgroup barrier;
  // group 1 runs one phase behind group 0.  Tile k's K sits in K buffer k % 3
  // and its V in V buffer k % 3: the K buffer of tile k is free once this
  // phase's QK^T has run, the V buffer of tile k - 1 once its P·V has. ----
  const int nk = (ntiles - grp + 1) / 2;      // this group's tiles
  const int n_it = (ntiles + 1) / 2;          // group 0's: both groups run n_it + 1 iterations, rounded up to pairs
  issue_k(gk);                                // tile 0's K
  issue_k(gk + KBUF);                         // "phase -2": tile 1's K, tile 0's V
  issue_v(gv);
  issue_k(gk + 2 * KBUF);                     // "phase -1": tile 2's K, tile 1's V
  issue_v(gv + VBUF);
  // this wave's part of tile 0's K has landed
  if (phase_loads == 7) wait_loads<14>(); else wait_loads<12>();   // after tile 0's K
  phase_barrier();
  if (grp == 1) phase_barrier();
  v4f W[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) W[t] = v4f{0.f, 0.f, 0.f, 0.f};
  int b3 = 0;                                 // k % 3
  auto iteration = [&](int k) __attribute__((always_inline)) {
    const int bm1 = b3 == 0 ? 2 : b3 - 1;     // (k - 1) % 3, also (k + 2) % 3
    __builtin_amdgcn_s_setprio(1);
    // unconditional (their results are used only when the P·V and the
    // softmax run), so that both form one block the scheduler can
    // interleave: the K operand reads first, then each QK^T instruction
    // followed by an eighth of the split's vector work
    softmax_tile_lo(W, Phi, Plo);
    qk_tile(gk + b3 * KBUF);
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
    static_for<8>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 11, 0);
    });
    if (k >= 1 && k - 1 < nk) pv_tile(gv + bm1 * VBUF);
    __builtin_amdgcn_s_setprio(0);
    // the matrix instructions are pure values to the compiler, which would
    // sink them past the barrier into the vector phase
    static_for<ND>([&](auto DD) { keep_in_vgprs(O[decltype(DD)::value]); });
    keep_in_vgprs(L);
    static_for<8>([&](auto TT) { keep_in_vgprs(S[decltype(TT)::value]); });
    phase_barrier();
    // the loads of phase k - 2 have landed: tile k's V (read by the next
    // P·V) and tile k + 1's K (the next QK^T)
    if (phase_loads == 7) wait_loads<7>(); else wait_loads<6>();
    if (k < nk) clear_tail(gv + b3 * VBUF, 2 * k + grp);
    // the next loads before the softmax (measured: 2-3% faster than after it,
    // where the waves of a group wait for the memory pipeline at the barrier)
    issue_k(gk + b3 * KBUF);                  // tile k + 3's K
    issue_v(gv + bm1 * VBUF);                 // tile k + 2's V
    if (k < nk) {
      mask_tile(2 * k + grp);
      softmax_tile_hi<ND>(S, W, a.c, m_run, O, L, psc);
    }
    static_for<8>([&](auto TT) { keep_in_vgprs(W[decltype(TT)::value]); });
    __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): LDS writes done before the barrier
    phase_barrier();
    b3 = b3 == 2 ? 0 : b3 + 1;
  };
  // unrolled by two, always whole pairs (an iteration past n_it does nothing but its barriers and
  // empty loads), so the compiler knows at the back edge which loads are in
  // flight
  for (int k = 0; k <= n_it; k += 2) {
    iteration(k);
    iteration(k + 1);
  }
  wait_loads<0>();                            // the empty loads past the range still write LDS
  if (grp == 0) phase_barrier();              // matches group 1's initial wait
  // ---- both groups hold the same rows: group 1 hands its (m, l, O) to
  // group 0 through LDS (every tile has been consumed) ----
  float* xf = reinterpret_cast<float*>(lds);
  const int idx = rb * 64 + lane;
  if (grp == 1) {
#pragma unroll
    for (int dd = 0; dd < ND; ++dd)
#pragma unroll
      for (int i = 0; i < 4; ++i) xf[(dd * 4 + i) * 256 + idx] = O[dd][i];
#pragma unroll
    for (int i = 0; i < 4; ++i) xf[(ND * 4 + i) * 256 + idx] = L[i];
    xf[(ND * 4 + 4) * 256 + idx] = m_run;
  }
  __syncthreads();
  if (grp == 1) return;
  const float m1 = xf[(ND * 4 + 4) * 256 + idx];
  const float mm = fmaxf(m_run, m1);
  if (mm != -INFINITY) {
    const float a0 = __builtin_amdgcn_exp2f(m_run - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
    for (int dd = 0; dd < ND; ++dd)
#pragma unroll
      for (int i = 0; i < 4; ++i) O[dd][i] = O[dd][i] * a0 + xf[(dd * 4 + i) * 256 + idx] * a1;
#pragma unroll
    for (int i = 0; i < 4; ++i) L[i] = L[i] * a0 + xf[(ND * 4 + i) * 256 + idx] * a1;
    m_run = mm;
  }

  store_split_rows<D>(a, O, L, m_run, bk, s, b, mrow, qr, lg);
}

// Combine the splits' partials with weights 2^(lse_s - max).  A query row
// is D/4 threads of four elements each (16-byte partial loads, one 8-byte
// bf16 store when the output allows it); a workgroup of 256 threads covers
// 256 / (D/4) rows.
template <int D>
__global__ void __launch_bounds__(256) decode_merge_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_lse, int kv_heads, int group,
                                                           int M, int splits, int64_t rows, uint16_t* __restrict__ o,
                                                           int64_t os0, int64_t os1, int64_t os2, int aligned8,
                                                           float* __restrict__ lse, int q_heads, int q_len) {
  constexpr int TPR = D / 4;
  const int64_t r = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;   // (bk, mrow)
  if (r >= rows) return;
  const int e = (threadIdx.x % TPR) * 4;
  const int64_t bk = r / M;
  const int mrow = (int)(r - bk * M);
  const int b = (int)(bk / kv_heads), kvh = (int)(bk - (int64_t)b * kv_heads);
  const int qt = mrow / group, head = kvh * group + (mrow - qt * group);
  const float* pl = part_lse + bk * splits * M + mrow;
  // splits in groups of four, all eight loads of a group in flight at once
  // (one memory round trip per group rather than one for the sums' maximum
  // and another for the partials), merged into a running maximum; an empty
  // split has lse -inf and a zero partial, so it adds nothing
  float mx = -INFINITY, wsum = 0.f;
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += 4) {
    float ls[4];
    v4f po[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = s0 + k < splits ? s0 + k : splits - 1;
      ls[k] = s0 + k < splits ? pl[(int64_t)s * M] : -INFINITY;
      po[k] = *reinterpret_cast<const v4f*>(part_o + ((bk * splits + s) * M + mrow) * D + e);
    }
    const float m_new = fmaxf(fmaxf(mx, fmaxf(ls[0], ls[1])), fmaxf(ls[2], ls[3]));
    if (m_new == -INFINITY) continue;
    const float sc = __builtin_amdgcn_exp2f(mx - m_new);   // 0 while mx is -inf
    wsum *= sc;
    acc *= sc;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float w = __builtin_amdgcn_exp2f(ls[k] - m_new);
      wsum += w;
      acc += w * po[k];
    }
    mx = m_new;
  }
  const v4f val = wsum > 0.f ? acc / wsum : v4f{0.f, 0.f, 0.f, 0.f};
  uint16_t* dst = o + b * os0 + qt * os1 + (int64_t)head * os2 + e;
  if (aligned8) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(bf16x2(val[0], val[1]), bf16x2(val[2], val[3]));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = (uint16_t)f32_to_bf16(val[i]);
  }
  if (lse != nullptr && e == 0)
    lse[((int64_t)b * q_len + qt) * q_heads + head] = wsum > 0.f ? (mx + __log2f(wsum)) * kLn2 : -INFINITY;
}

// Four row blocks at head_dim 128 run the ping-pong workgroup.
template <int D, int MB>
constexpr bool kPingPong = MB == 4 && D == 128;

// Workgroups of decode_split_kernel<D, MB> the current device holds at once:
// its CU count times the runtime's occupancy figure for the compiled kernel
// (register and LDS use), so a different compiler, register budget or device
// partition changes the split count with it.  Cached per device ordinal (a
// read-only property of the device and the loaded code); 0 when a query fails.
template <int D, int MB>
static int64_t decode_capacity_of(int dev) {
  static std::atomic<int64_t> cache[kMaxDevices];
  if (dev >= 0 && dev < kMaxDevices) {
    const int64_t c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  constexpr bool pp = kPingPong<D, MB>;
  const void* fn = pp ? reinterpret_cast<const void*>(&verify_pingpong_kernel<128>)
                      : reinterpret_cast<const void*>(&decode_split_kernel<D, MB>);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, pp ? 512 : MB * 64, 0) != hipSuccess) return 0;
  const int64_t c = (int64_t)cus * per_cu;
  if (c > 0 && dev >= 0 && dev < kMaxDevices) cache[dev].store(c, std::memory_order_relaxed);
  return c;
}

static int64_t decode_capacity(int head_dim, int MB) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (head_dim == 64) {
    switch (MB) {
      case 1: return decode_capacity_of<64, 1>(dev);
      case 2: return decode_capacity_of<64, 2>(dev);
      case 3: return decode_capacity_of<64, 3>(dev);
      default: return decode_capacity_of<64, 4>(dev);
    }
  }
  switch (MB) {
    case 1: return decode_capacity_of<128, 1>(dev);
    case 2: return decode_capacity_of<128, 2>(dev);
    case 3: return decode_capacity_of<128, 3>(dev);
    default: return decode_capacity_of<128, 4>(dev);
  }
}

int decode_num_splits(int batch, int kv_heads, int rows, int head_dim, int span, int requested) {
  const int64_t capacity = requested > 0 ? 0 : decode_capacity(head_dim, decode_row_blocks(rows));
  return decode_split_count((int64_t)batch * kv_heads, span, capacity, requested);
}

size_t decode_workspace_bytes(int batch, int q_len, int q_heads, int kv_heads, int head_dim, int splits) {
  const size_t M = (size_t)(q_heads / kv_heads) * q_len;
  const size_t rows = (size_t)batch * kv_heads * splits * M;
  const size_t o_bytes = (rows * head_dim * 4 + kWsAlign - 1) / kWsAlign * kWsAlign;
  return o_bytes + (rows * 4 + kWsAlign - 1) / kWsAlign * kWsAlign;
}

template <int D>
static hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream) {
  DecodeArgs a;
  const int G = p.q_heads / p.kv_heads;
  const int M = G * p.q_len;
  const int span = decode_key_span(p.kv_len, p.q_len, p.window);
  const int splits = decode_num_splits(p.batch, p.kv_heads, M, D, span, p.num_splits);
  const int tiles = (span + 127) / 128;
  a.q = p.q; a.kc = p.k_codes; a.ksc = p.k_scales; a.vc = p.v_codes; a.vsc = p.v_scales; a.kv_lens = p.kv_lens;
  const size_t rows = (size_t)p.batch * p.kv_heads * splits * M;
  a.part_o = reinterpret_cast<float*>(p.ws);
  a.part_lse = reinterpret_cast<float*>(p.ws + (rows * D * 4 + kWsAlign - 1) / kWsAlign * kWsAlign);
  a.qs0 = p.qs[0]; a.qs1 = p.qs[1]; a.qs2 = p.qs[2];
  a.kv_heads = p.kv_heads; a.group = G; a.q_len = p.q_len; a.M = M; a.kv_len = p.kv_len; a.cap = p.cap;
  a.R = p.v_tile_rows; a.log2R = __builtin_ctz((unsigned)p.v_tile_rows); a.splits = splits; a.tiles_per_split = (tiles + splits - 1) / splits;
  a.n_vtiles_cap = (p.cap + p.v_tile_rows - 1) / p.v_tile_rows;
  a.c = p.softmax_scale * kLog2e / (p.hadamard ? (float)D : 1.0f);
  a.hadamard = p.hadamard;
  a.window = p.window < p.kv_len ? p.window : 0;   // a window of kv_len or more keeps every key
  a.o = p.o; a.lse = p.lse; a.os0 = p.os[0]; a.os1 = p.os[1]; a.os2 = p.os[2]; a.q_heads = p.q_heads;
  a.block_table = p.block_table; a.page_size = p.page_size; a.pages_per_seq = p.pages_per_seq;
  a.direct = splits == 1 && (reinterpret_cast<uintptr_t>(p.o) & 7) == 0 && p.os[0] % 4 == 0 && p.os[1] % 4 == 0 &&
             p.os[2] % 4 == 0;
  const dim3 grid((unsigned)((int64_t)p.batch * p.kv_heads * splits));
  const int MB = (M + 15) / 16;
  switch (MB) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<D, 1>), grid, dim3(64), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2>), grid, dim3(128), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((decode_split_kernel<D, 3>), grid, dim3(192), 0, stream, a); break;
    default:
      if constexpr (kPingPong<D, 4>)
        hipLaunchKernelGGL((verify_pingpong_kernel<D>), grid, dim3(512), 0, stream, a);
      else
        hipLaunchKernelGGL((decode_split_kernel<D, 4>), grid, dim3(256), 0, stream, a);
      break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.direct) return e;
  const int64_t mrows = (int64_t)p.batch * p.kv_heads * M;
  constexpr int rows_per_wg = 256 / (D / 4);
  const int aligned8 = (reinterpret_cast<uintptr_t>(p.o) & 7) == 0 && p.os[0] % 4 == 0 && p.os[1] % 4 == 0 &&
                       p.os[2] % 4 == 0;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)((mrows + rows_per_wg - 1) / rows_per_wg)), dim3(256),
                     0, stream, a.part_o, a.part_lse, p.kv_heads, G, M, splits, mrows, p.o, p.os[0], p.os[1], p.os[2],
                     aligned8, p.lse, p.q_heads, p.q_len);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  return p.head_dim == 64 ? launch_decode_d<64>(p, stream) : launch_decode_d<128>(p, stream);
}

// Split partials of the allocation-free decode entry point.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: the kernels get
// the device address that hipGetSymbolAddress returns for the current device,
// looked up on the first call on each device and kept per device ordinal.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static hipError_t scratch_address(uint8_t** out) {
  static std::atomic<uint8_t*> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uint8_t* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* sym = nullptr;
    e = hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    p = static_cast<uint8_t*>(sym);
    addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_decode_noalloc(DecodeParams p, size_t need, hipStream_t stream) {
  if (need > kNoAllocScratchBytes) return hipErrorInvalidValue;
  uint8_t* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  // every split writes all of its partial rows before the merge reads them,
  // so nothing in the array needs clearing between calls
  p.ws = ws;
  return launch_decode(p, stream);
}

}  // namespace qk4v8
