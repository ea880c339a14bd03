// QK4V8 prefill attention for gfx950.
//
// What is computed ("MpFA免训练量化：QK4V8混合精度在Blackwell上的推理加速实践"):
// Q and K quantized to 4 bits, V to 8 bits (§2.1, §2.2), each block's scale
// computed online from the block (§3.2), scores dequantized right after each
// tile's QK^T (§3.3; here the block-scaled MFMA applies both operands' E8M0
// scales inside the instruction), an online softmax and FP32 accumulation of
// P·V in the same loop (§2.3), output cast back to 16 bits (§3.3).
//
// Structure on the GPU:
//  1. pack_k: K -> MXFP4, written once per call into the workspace in the
//     exact lane order of the QK^T MFMA A operand (16 B per lane per subtile).
//  2. vtile_scale + pack_v: V -> per-tile E8M0 + E4M3 codes, written
//     transposed (keys contiguous per head_dim column) in the lane order of
//     the P·V MFMA A operand.
//  3. attn: one workgroup of 8 waves per (batch, KV head, head group,
//     position block); every wave owns 32 query rows of one query head, all
//     waves of the workgroup share each 128-key K/V tile staged in LDS
//     (double-buffered).  Per tile and wave:
//       S^T = K·Q^T on v_mfma_scale_f32_16x16x128_f8f6f4 (FP4 x FP4),
//       FP32 online softmax in the log2 domain with lazy rescaling,
//       P split into two E4M3 terms (hi + residual) with a per-(row, tile)
//       E8M0 range scale,
//       O^T += V^T·P^T on the same instruction in FP8 x FP8 (twice: hi, lo).
//     Computing S^T and O^T (instead of S and O) puts one query per lane
//     column in both, so the softmax state, the P operand and the output rows
//     need no cross-lane transposes.
#include "qk4v8_device.h"
#include "qk4v8_launch.h"

namespace qk4v8 {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;          // two 16-row query blocks
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Key offset (0..127 in a KV tile) held by row r of S^T subtile t.  Chosen so
// that the 32 scores a lane holds after the 8 QK^T MFMAs are exactly the 32
// keys the FP8 P·V MFMA expects in that lane (keys 16g..16g+15 and
// 64+16g..64+16g+15 for lane group g), in byte order 4t + i.
__host__ __device__ constexpr int subtile_key(int t, int r) {
  return (t >> 2) * 64 + 16 * (r >> 2) + 4 * (t & 3) + (r & 3);
}

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

}  // namespace

PrefillLayout prefill_layout(int batch, int kv_heads, int seq_k, int head_dim, int v_tile_rows) {
  PrefillLayout L;
  const int64_t bk = (int64_t)batch * kv_heads;
  L.n_tiles = (seq_k + kKvTile - 1) / kKvTile;
  L.n_vtiles = (seq_k + v_tile_rows - 1) / v_tile_rows;
  size_t off = 0;
  L.off_k = off;     off = align_up(off + (size_t)bk * L.n_tiles * kKvTile * (head_dim / 2));
  L.off_ks = off;    off = align_up(off + (size_t)bk * L.n_tiles * (head_dim / 32) * 16 * 8);
  L.off_v = off;     off = align_up(off + (size_t)bk * L.n_tiles * kKvTile * head_dim);
  L.off_vs = off;    off = align_up(off + (size_t)bk * L.n_tiles * 4);
  L.off_vtile = off; off = align_up(off + (size_t)bk * L.n_vtiles);
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// Pre-pass 1: K -> MXFP4 in MFMA-operand order.
// Thread per (group bk, padded key j, 32-element block g).  Keys past seq_k
// are written as zero codes.
//   codes: [bk][tile][t][g][r][16 B]   scales: [bk][tile][g*16 + r][t]
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) pack_k_kernel(const uint16_t* __restrict__ k, int64_t ks0, int64_t ks1,
                                                     int64_t ks2, int kv_heads, int seq_k, int64_t n_tiles,
                                                     uint8_t* __restrict__ wk, uint8_t* __restrict__ wks,
                                                     int64_t total) {
  constexpr int NB = D / 32;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= total) return;
  const int g = (int)(id % NB);
  const int64_t jj = (id / NB) % (n_tiles * kKvTile);
  const int64_t bk = id / (NB * n_tiles * kKvTile);
  const int64_t b = bk / kv_heads, h = bk - b * kv_heads;
  const int64_t tile = jj / kKvTile;
  const int kk = (int)(jj - tile * kKvTile);
  // invert subtile_key: kk = 64a + 16b + 4c + e  ->  t = 4a + c, r = 4b + e
  const int t = 4 * (kk >> 6) + ((kk >> 2) & 3);
  const int r = 4 * ((kk >> 4) & 3) + (kk & 3);
  uint32_t codes[4] = {0, 0, 0, 0};
  uint32_t scale = 127;
  if (jj < seq_k) {
    const uint4* src = reinterpret_cast<const uint4*>(k + b * ks0 + h * ks1 + jj * ks2 + 32 * g);
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 x = src[i];
      w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
    }
    scale = mxfp4_quantize32(w, codes);
  }
  const int64_t tb = bk * n_tiles + tile;
  *reinterpret_cast<uint4*>(wk + ((tb * 8 + t) * (NB * 16) + g * 16 + r) * 16) =
      make_uint4(codes[0], codes[1], codes[2], codes[3]);
  wks[(tb * (NB * 16) + g * 16 + r) * 8 + t] = (uint8_t)scale;
}

// ---------------------------------------------------------------------------
// Pre-pass 2: E8M0 scale of each V tile of R rows (absmax over R x D).
// One workgroup (256 threads) per (group, tile).
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) vtile_scale_kernel(const uint16_t* __restrict__ v, int64_t vs0, int64_t vs1,
                                                          int64_t vs2, int kv_heads, int seq_k, int R,
                                                          int64_t n_vtiles, uint8_t* __restrict__ out) {
  __shared__ float red[4];
  const int64_t bk = blockIdx.x / n_vtiles, vt = blockIdx.x - bk * n_vtiles;
  const int64_t b = bk / kv_heads, h = bk - b * kv_heads;
  const int64_t r0 = vt * R;
  const int rows = (int)min((int64_t)R, (int64_t)seq_k - r0);
  constexpr int CPR = D / 8;
  float amax = 0.0f;
  for (int vi = threadIdx.x; vi < rows * CPR; vi += 256) {
    const int rr = vi / CPR, cc = vi - rr * CPR;
    const uint4 x = *reinterpret_cast<const uint4*>(v + b * vs0 + h * vs1 + (r0 + rr) * vs2 + cc * 8);
    const uint32_t ws[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(ws[i])), fabsf(bf16_hi(ws[i]))));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0) {
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    out[bk * n_vtiles + vt] = (uint8_t)(mx_shared_exp(amax, 8) + 127);
  }
}

// ---------------------------------------------------------------------------
// Pre-pass 3: V -> E4M3 codes, transposed per 128-key tile.
// One workgroup per (group, tile): quantize row-major into LDS, then gather
// 16 consecutive keys of one column per output chunk.
//   codes : [bk][tile][dd = D/16][half][g][m][16 keys]  (column d = 16dd+m,
//           keys 64*half + 16g .. +15)
//   scales: [bk][tile] u32, byte b = E8M0 of the V tile holding key 32b
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) pack_v_kernel(const uint16_t* __restrict__ v, int64_t vs0, int64_t vs1,
                                                     int64_t vs2, int kv_heads, int seq_k, int R, int64_t n_tiles,
                                                     int64_t n_vtiles, const uint8_t* __restrict__ vtile,
                                                     uint8_t* __restrict__ wv, uint32_t* __restrict__ wvs) {
  constexpr int LDSROW = D + 4;   // bytes per key row in LDS (padding spreads banks)
  __shared__ uint8_t tileb[kKvTile * LDSROW];
  const int64_t bk = blockIdx.x / n_tiles, tile = blockIdx.x - bk * n_tiles;
  const int64_t b = bk / kv_heads, h = bk - b * kv_heads;
  const uint8_t* vts = vtile + bk * n_vtiles;
  constexpr int CPR = D / 8;
  for (int vi = threadIdx.x; vi < kKvTile * CPR; vi += 256) {
    const int kk = vi / CPR, cc = vi - kk * CPR;
    const int64_t j = tile * kKvTile + kk;
    uint32_t lo = 0, hi = 0;
    if (j < seq_k) {
      const uint4 x = *reinterpret_cast<const uint4*>(v + b * vs0 + h * vs1 + j * vs2 + cc * 8);
      const float inv = exp2i(127 - (int)vts[j / R]);
      const uint32_t ws[4] = {x.x, x.y, x.z, x.w};
      uint32_t bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bb[i] = e4m3_pack2(clamp448(bf16_lo(ws[i]) * inv), clamp448(bf16_hi(ws[i]) * inv), 1.0f);
      lo = bb[0] | (bb[1] << 16);
      hi = bb[2] | (bb[3] << 16);
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(tileb + kk * LDSROW + cc * 8);
    dst[0] = lo;
    dst[1] = hi;
  }
  __syncthreads();
  constexpr int ND = D / 16;
  uint8_t* out = wv + (bk * n_tiles + tile) * (int64_t)(kKvTile * D);
  for (int o = threadIdx.x; o < ND * 128; o += 256) {
    const int dd = o >> 7, half = (o >> 6) & 1, lane = o & 63;
    const int g = lane >> 4, m = lane & 15;
    const int col = dd * 16 + m, k0 = half * 64 + g * 16;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t acc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc |= (uint32_t)tileb[(k0 + 4 * q + e) * LDSROW + col] << (8 * e);
      w[q] = acc;
    }
    *reinterpret_cast<uint4*>(out + (int64_t)o * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (threadIdx.x == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      int64_t j = tile * kKvTile + 32 * blk;
      if (j >= seq_k) j = seq_k - 1;
      s |= (uint32_t)vts[j / R] << (8 * blk);
    }
    wvs[bk * n_tiles + tile] = s;
  }
}

// ---------------------------------------------------------------------------
// Attention kernel.
// ---------------------------------------------------------------------------
struct AttnArgs {
  const uint16_t* q;
  uint16_t* o;
  float* lse;
  const uint8_t* wk;
  const uint8_t* wks;
  const uint8_t* wv;
  const uint32_t* wvs;
  int64_t qs0, qs1, qs2, os0, os1, os2;
  int q_heads, kv_heads, group, heads_per_wg, pos_blocks, seq_q, seq_k;
  int xblocks, pos_groups;   // 1-D grid = pos_groups x xblocks, xblocks fastest
  int64_t n_tiles;
  float c;          // softmax_scale * log2(e)
};

template <int D>
struct TileBytes {
  static constexpr int NB = D / 32;
  static constexpr int K = 8 * NB * 16 * 16;      // codes of one 128-key tile
  static constexpr int KS = NB * 16 * 8;          // K scales of one tile
  static constexpr int V = kKvTile * D;           // V^T codes of one tile
  static constexpr int STAGE = K + KS + V + 16;   // + V scale word (padded)
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) attn_kernel(AttnArgs a) {
  using TB = TileBytes<D>;
  constexpr int NB = TB::NB;
  constexpr int ND = D / 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * TB::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 15;     // query column of this lane within a 16-block
  const int lg = lane >> 4;     // lane group (k-block / d sub-row group)

  // workgroup -> (b, kv head, head group); position block reversed so the
  // longest causal rows start first
  const int hgroups = a.group / a.heads_per_wg;
  const int bx = (int)(blockIdx.x % (unsigned)a.xblocks);
  const int hg = bx % hgroups;
  const int kvh = (bx / hgroups) % a.kv_heads;
  const int b = bx / (hgroups * a.kv_heads);
  const int pg = a.pos_groups - 1 - (int)(blockIdx.x / (unsigned)a.xblocks);
  const int P0 = pg * a.pos_blocks * kRowsPerWave;
  const int hw = wave % a.heads_per_wg, pb = wave / a.heads_per_wg;
  const int head = kvh * a.group + hg * a.heads_per_wg + hw;
  const int p0w = P0 + pb * kRowsPerWave;
  const int off = a.seq_k - a.seq_q;

  // key range of the workgroup and of this wave
  const int wg_last_row = min(P0 + a.pos_blocks * kRowsPerWave, a.seq_q) - 1;
  const int kend_wg = CAUSAL ? min(a.seq_k, wg_last_row + off + 1) : a.seq_k;
  const int nt_wg = (kend_wg + kKvTile - 1) / kKvTile;
  const bool wave_live = p0w < a.seq_q;
  const int w_last_row = min(p0w + kRowsPerWave, a.seq_q) - 1;
  const int kend_w = wave_live ? (CAUSAL ? min(a.seq_k, w_last_row + off + 1) : a.seq_k) : 0;
  const int nt_w = (kend_w + kKvTile - 1) / kKvTile;
  // tiles whose last key exceeds this bound need the element mask
  const int mask_lim = CAUSAL ? min(a.seq_k - 1, p0w + off) : a.seq_k - 1;

  const int64_t bk = (int64_t)b * a.kv_heads + kvh;
  const uint8_t* gk = a.wk + bk * a.n_tiles * TB::K;
  const uint8_t* gks = a.wks + bk * a.n_tiles * TB::KS;
  const uint8_t* gv = a.wv + bk * a.n_tiles * TB::V;
  const uint32_t* gvs = a.wvs + bk * a.n_tiles;

  // ---- Q prologue: quantize this wave's 32 rows to MXFP4 in registers.
  // Lanes of k-blocks past head_dim (D = 64) hold zero codes, so whatever K
  // codes those lanes read contribute nothing.
  v8i qf[2];
  int qsc[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    uint4 qc = make_uint4(0, 0, 0, 0);
    qsc[qb] = 127;
    const int row = p0w + qb * 16 + ql;
    if (row < a.seq_q && lg < NB) {
      const uint4* src = reinterpret_cast<const uint4*>(a.q + b * a.qs0 + (int64_t)head * a.qs1 + row * a.qs2 + 32 * lg);
      uint32_t w[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 x = src[i];
        w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
      }
      uint32_t c[4];
      qsc[qb] = (int)mxfp4_quantize32(w, c);
      qc = make_uint4(c[0], c[1], c[2], c[3]);
    }
    qf[qb] = fp4_operand(qc);
  }

  v4f O[2][ND];
  v4f L[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    L[qb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dd = 0; dd < ND; ++dd) O[qb][dd] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  float m_run[2] = {-INFINITY, -INFINITY};
  v8i Phi[2] = {v8i{}, v8i{}}, Plo[2] = {v8i{}, v8i{}};
  const v8i ones = v8i{(int)kFp8Ones, (int)kFp8Ones, (int)kFp8Ones, (int)kFp8Ones,
                       (int)kFp8Ones, (int)kFp8Ones, (int)kFp8Ones, (int)kFp8Ones};
  const int klane = lane & (NB * 16 - 1);   // K fragment lane (D = 64 reuses lanes 0..31)

  // ---- tile staging: global -> registers -> LDS (double-buffered LDS) ----
  constexpr int KV4 = TB::K / 16, VV4 = TB::V / 16, KSV4 = TB::KS / 16;
  uint4 rk = make_uint4(0, 0, 0, 0), rv0 = rk, rv1 = rk, rks = rk;
  uint32_t rvs = 0;
#define QK4V8_GLOAD(tile)                                                                    \
  do {                                                                                       \
    const uint4* sk_ = reinterpret_cast<const uint4*>(gk + (int64_t)(tile) * TB::K);        \
    const uint4* sv_ = reinterpret_cast<const uint4*>(gv + (int64_t)(tile) * TB::V);        \
    const uint4* sks_ = reinterpret_cast<const uint4*>(gks + (int64_t)(tile) * TB::KS);     \
    if (tid < KV4) rk = sk_[tid];                                                            \
    if (tid < VV4) rv0 = sv_[tid];                                                           \
    if (tid + kThreads < VV4) rv1 = sv_[tid + kThreads];                                     \
    if (tid < KSV4) rks = sks_[tid];                                                         \
    if (tid == 0) rvs = gvs[(tile)];                                                         \
  } while (0)
#define QK4V8_SSTORE(buf)                                                                    \
  do {                                                                                       \
    uint8_t* base_ = lds + (buf) * TB::STAGE;                                                \
    if (tid < KV4) reinterpret_cast<uint4*>(base_)[tid] = rk;                                \
    if (tid < VV4) reinterpret_cast<uint4*>(base_ + TB::K + TB::KS)[tid] = rv0;              \
    if (tid + kThreads < VV4) reinterpret_cast<uint4*>(base_ + TB::K + TB::KS)[tid + kThreads] = rv1; \
    if (tid < KSV4) reinterpret_cast<uint4*>(base_ + TB::K)[tid] = rks;                      \
    if (tid == 0) *reinterpret_cast<uint32_t*>(base_ + TB::K + TB::KS + TB::V) = rvs;        \
  } while (0)

  if (nt_wg > 0) {
    QK4V8_GLOAD(0);
    QK4V8_SSTORE(0);
  }
  __syncthreads();

  for (int j = 0; j < nt_wg; ++j) {
    const int buf = j & 1;
    if (j + 1 < nt_wg) QK4V8_GLOAD(j + 1);
    if (j < nt_w) {
      const uint8_t* base = lds + buf * TB::STAGE;
      const uint8_t* lk = base;
      const uint8_t* lks = base + TB::K;
      const uint8_t* lv = base + TB::K + TB::KS;
      const uint32_t vsw = *reinterpret_cast<const uint32_t*>(base + TB::K + TB::KS + TB::V);

      // ---- S^T = K · Q^T  (FP4 x FP4; both operands' E8M0 scales applied
      // inside the instruction, i.e. the scores come out dequantized) ----
      v4f S[2][8];
      const uint2 ksc = *reinterpret_cast<const uint2*>(lks + klane * 8);
      static_for<8>([&](auto T) {
        constexpr int t = decltype(T)::value;
        const v8i af = fp4_operand(*reinterpret_cast<const uint4*>(lk + (t * NB * 16 + klane) * 16));
        const int sa = (int)(t < 4 ? ksc.x : ksc.y);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          S[qb][t] = mfma16x16x128<kFmtFp4, kFmtFp4, t & 3, 0>(af, qf[qb], v4f{0.f, 0.f, 0.f, 0.f}, sa, qsc[qb]);
      });

      // ---- mask (only tiles that cross the causal diagonal or seq_k) ----
      if (j * kKvTile + kKvTile - 1 > mask_lim) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int row = p0w + qb * 16 + ql;
          const int lim = (CAUSAL ? min(a.seq_k - 1, row + off) : a.seq_k - 1) - j * kKvTile;
#pragma unroll
          for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (subtile_key(t, 4 * lg + i) > lim) S[qb][t][i] = -INFINITY;
        }
      }

      // ---- online softmax and two-term FP8 P ----
      int psc[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) softmax_tile<ND>(S[qb], a.c, m_run[qb], O[qb], L[qb], Phi[qb], Plo[qb], psc[qb]);

      // ---- O^T += V^T · P^T and L += 1 · P^T  (FP8 x FP8) ----
      const int vsc = (int)((vsw >> (8 * lg)) & 0xFF);
#pragma unroll
      for (int dd = 0; dd < ND; ++dd) {
        const uint4 v0 = *reinterpret_cast<const uint4*>(lv + ((dd * 2 + 0) * 64 + lane) * 16);
        const uint4 v1 = *reinterpret_cast<const uint4*>(lv + ((dd * 2 + 1) * 64 + lane) * 16);
        const v8i av = v8i{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          O[qb][dd] = mfma16x16x128<kFmtFp8, kFmtFp8>(av, Phi[qb], O[qb][dd], vsc, psc[qb]);
          O[qb][dd] = mfma16x16x128<kFmtFp8, kFmtFp8>(av, Plo[qb], O[qb][dd], vsc, psc[qb] - 4);
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        L[qb] = mfma16x16x128<kFmtFp8, kFmtFp8>(ones, Phi[qb], L[qb], 127, psc[qb]);
        L[qb] = mfma16x16x128<kFmtFp8, kFmtFp8>(ones, Plo[qb], L[qb], 127, psc[qb] - 4);
      }
    }
    if (j + 1 < nt_wg) QK4V8_SSTORE(buf ^ 1);
    __syncthreads();
  }
#undef QK4V8_GLOAD
#undef QK4V8_SSTORE

  // ---- epilogue: normalize by the sum of the quantized weights, store bf16
  // rows and the log-sum-exp ----
  if (!wave_live) return;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = L[qb][0];     // every row of the ones-MFMA holds the same sum
    const int row = p0w + qb * 16 + ql;
    if (row >= a.seq_q) continue;
    const float inv = 1.0f / l;
    uint16_t* dst = a.o + b * a.os0 + (int64_t)head * a.os1 + row * a.os2;
#pragma unroll
    for (int dd = 0; dd < ND; ++dd) {
      const v4f x = O[qb][dd] * inv;
      const uint32_t w0 = f32_to_bf16(x[0]) | (f32_to_bf16(x[1]) << 16);
      const uint32_t w1 = f32_to_bf16(x[2]) | (f32_to_bf16(x[3]) << 16);
      *reinterpret_cast<uint2*>(dst + dd * 16 + 4 * lg) = make_uint2(w0, w1);
    }
    if (a.lse != nullptr && lg == 0) {
      const float m_use = (m_run[qb] == -INFINITY) ? 0.0f : m_run[qb];
      a.lse[((int64_t)b * a.q_heads + head) * a.seq_q + row] = (m_use + __log2f(l)) * kLn2;
    }
  }
}

static int gcd_int(int x, int y) {
  while (y) { int t = x % y; x = y; y = t; }
  return x;
}

template <int D>
static hipError_t launch_pack_d(const PrefillParams& p, hipStream_t stream) {
  const PrefillLayout L = prefill_layout(p.batch, p.kv_heads, p.seq_k, D, p.v_tile_rows);
  uint8_t* wvt = p.ws + L.off_vtile;
  const int64_t bk = (int64_t)p.batch * p.kv_heads;
  const int64_t total_k = bk * L.n_tiles * kKvTile * (D / 32);
  hipLaunchKernelGGL((pack_k_kernel<D>), dim3((unsigned)((total_k + 255) / 256)), dim3(256), 0, stream, p.k,
                     p.ks[0], p.ks[1], p.ks[2], p.kv_heads, p.seq_k, L.n_tiles, p.ws + L.off_k, p.ws + L.off_ks,
                     total_k);
  hipLaunchKernelGGL((vtile_scale_kernel<D>), dim3((unsigned)(bk * L.n_vtiles)), dim3(256), 0, stream, p.v,
                     p.vs[0], p.vs[1], p.vs[2], p.kv_heads, p.seq_k, p.v_tile_rows, L.n_vtiles, wvt);
  hipLaunchKernelGGL((pack_v_kernel<D>), dim3((unsigned)(bk * L.n_tiles)), dim3(256), 0, stream, p.v, p.vs[0],
                     p.vs[1], p.vs[2], p.kv_heads, p.seq_k, p.v_tile_rows, L.n_tiles, L.n_vtiles, wvt,
                     p.ws + L.off_v, reinterpret_cast<uint32_t*>(p.ws + L.off_vs));
  return hipGetLastError();
}

template <int D>
static hipError_t launch_attn_d(const PrefillParams& p, hipStream_t stream) {
  const PrefillLayout L = prefill_layout(p.batch, p.kv_heads, p.seq_k, D, p.v_tile_rows);
  AttnArgs a;
  a.q = p.q; a.o = p.o; a.lse = p.lse;
  a.wk = p.ws + L.off_k; a.wks = p.ws + L.off_ks; a.wv = p.ws + L.off_v;
  a.wvs = reinterpret_cast<const uint32_t*>(p.ws + L.off_vs);
  a.qs0 = p.qs[0]; a.qs1 = p.qs[1]; a.qs2 = p.qs[2];
  a.os0 = p.os[0]; a.os1 = p.os[1]; a.os2 = p.os[2];
  a.q_heads = p.q_heads; a.kv_heads = p.kv_heads;
  a.group = p.q_heads / p.kv_heads;
  a.heads_per_wg = gcd_int(a.group, kWaves);
  a.pos_blocks = kWaves / a.heads_per_wg;
  a.seq_q = p.seq_q; a.seq_k = p.seq_k;
  a.n_tiles = L.n_tiles;
  a.c = p.softmax_scale * kLog2e;
  const int rows_per_wg = a.pos_blocks * kRowsPerWave;
  a.xblocks = p.batch * p.kv_heads * (a.group / a.heads_per_wg);
  a.pos_groups = (p.seq_q + rows_per_wg - 1) / rows_per_wg;
  const dim3 grid((unsigned)((int64_t)a.xblocks * a.pos_groups));
  if (p.causal)
    hipLaunchKernelGGL((attn_kernel<D, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_kernel<D, false>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill_pack(const PrefillParams& p, hipStream_t stream) {
  return p.head_dim == 64 ? launch_pack_d<64>(p, stream) : launch_pack_d<128>(p, stream);
}

hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t stream) {
  return p.head_dim == 64 ? launch_attn_d<64>(p, stream) : launch_attn_d<128>(p, stream);
}

}  // namespace qk4v8
