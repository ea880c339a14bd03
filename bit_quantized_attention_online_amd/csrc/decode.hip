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
//   K codes (row-major, padded rows) -> QK^T A operand (16 B per lane),
//   V codes (row-major, 16-byte chunks XOR-swizzled by row) -> ds_read_tr8_b64
//   gathers 8 keys of one column per lane, which is the P·V A operand layout.
// The next tile is fetched into registers while one computes, by buffer loads
// bounded to the sequence and marked non-temporal (the cache is streamed
// once).  Each split writes its normalized fp32 partial output and
// log2-sum-exp; the merge kernel combines splits with log-sum-exp weights.
//
// Sliding window (MiMo page, section "DFlash块扩散推测解码": the drafter keeps
// only the most recent 1024 keys): the splits cover the keys from the tile
// holding the first query's first visible key to the end of the sequence, so
// the work and the traffic do not grow with the length of the cache.
#include "qk4v8_device.h"
#include "qk4v8_launch.h"

namespace qk4v8 {

namespace {

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
  static constexpr int KRB = D / 2 + 16;        // padded K row bytes in LDS
  static constexpr int K = 128 * KRB;
  static constexpr int KS = 128 * 4;            // one dword of scales per key
  static constexpr int V = 128 * D;
  static constexpr int VS = 16;                 // V scales of the four 32-key groups
  static constexpr int BYTES = K + KS + V + VS;
};

template <int D>
__device__ __forceinline__ int vswz(int row, int chunk) {
  return chunk ^ (row & (DecTile<D>::NC - 1));
}

// Resident workgroups per CU (4 SIMDs x waves per SIMD / MB), from the
// kernels' register use: at head_dim 128 one wave per SIMD for MB = 1, 2
// (the next tile is staged in registers), two for MB = 3 and three for MB = 4
// (register budget 168); at head_dim 64 two for MB <= 3 and three for MB = 4.
__host__ __device__ constexpr int decode_wgs_per_cu(int D, int MB) {
  return MB == 4 ? 3 : (D == 128 ? (MB == 3 ? 8 : 4) : 8) / MB;
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
  const int kvlen = a.kv_lens ? a.kv_lens[b] : a.kv_len;
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
      if (KCH % NT == 0 || ci < KCH) *reinterpret_cast<v4i*>(lk + (ci / NB) * T::KRB + (ci % NB) * 16) = rk[i];
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
      const v8i af = fp4_operand(*reinterpret_cast<const uint4*>(lk + key * T::KRB + klg * 16));
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
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, pl[(int64_t)s * M]);
  float wsum = 0.f;
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  if (mx != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const float w = __builtin_amdgcn_exp2f(pl[(int64_t)s * M] - mx);
      wsum += w;
      acc += w * *reinterpret_cast<const v4f*>(part_o + ((bk * splits + s) * M + mrow) * D + e);
    }
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

int decode_key_span(int kv_len, int q_len, int window) {
  // with a window the range starts at most 127 keys before query 0's first key
  if (window > 0 && (int64_t)window + q_len + 126 < kv_len) return window + q_len + 126;
  return kv_len;
}

int decode_num_splits(int batch, int kv_heads, int rows, int head_dim, int span, int requested) {
  const int tiles = (span + 127) / 128;
  if (requested > 0) return requested < tiles ? requested : tiles;
  // one round of workgroups: as many as the 256 CUs hold at once (a second,
  // partial round and larger split partials cost more than they balance),
  // each with >= 8 tiles of work (below that the merge pass costs more than
  // the parallelism gains; one split writes the output without it)
  const int MB = rows <= 16 ? 1 : rows <= 32 ? 2 : rows <= 48 ? 3 : 4;
  const int64_t units = (int64_t)batch * kv_heads;
  const int64_t capacity = 256 * (int64_t)decode_wgs_per_cu(head_dim, MB);
  int s = (int)((capacity + units / 2) / units);
  const int max_s = tiles / 8 > 0 ? tiles / 8 : 1;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return s;
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
    default: hipLaunchKernelGGL((decode_split_kernel<D, 4>), grid, dim3(256), 0, stream, a); break;
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

}  // namespace qk4v8
