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
//     exact lane order of the QK^T MFMA A operand (16 B per lane).
//  2. vtile_scale + pack_v: V -> per-tile E8M0 + E4M3 codes, written
//     transposed (keys contiguous per head_dim column) in the lane order of
//     the P·V MFMA A operand.
//  3. attn: one workgroup of 8 waves per (batch, KV head, head group,
//     position block); every wave owns 32 query rows of one query head, all
//     waves share each 128-key K/V tile staged in LDS.  Per tile and wave:
//       S^T = K·Q^T on v_mfma_scale_f32_32x32x64_f8f6f4 (FP4 x FP4),
//       FP32 online softmax in the log2 domain with lazy rescaling,
//       P split into two E4M3 terms (hi + residual) with a per-(row, tile)
//       E8M0 range scale,
//       O^T += V^T·P^T on the same instruction in FP8 x FP8 (twice: hi, lo),
//       and the row sums of the quantized weights as 1·P^T.
//     Computing S^T and O^T (instead of S and O) puts one query per lane
//     column in both, so the softmax state, the P operand and the output rows
//     need no cross-lane transposes.  The 32x32x64 shape keeps the matrix
//     core busy long enough per instruction for the vector ALU work of the
//     other wave on the SIMD to issue alongside it.
#include "qk4v8_device.h"
#include "qk4v8_launch.h"

namespace qk4v8 {

namespace {

constexpr int kWaves = 8;                 // waves per attention workgroup (two ping-pong groups)
constexpr int kRowsPerWave = 32;          // two 16-row query blocks
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Key offset (0..127 in a KV tile) of row rho of the QK^T output for key block
// kb (32 keys each).  The 32x32 result puts row (i/4)*8 + 4h + i%4 in element
// i of lane (q, h); with this order that element is key 32*kb + 16*h + i, so
// the 64 scores of lane (q, h) are exactly the keys 64*s2 + 32*(j/16) + 16*h
// + j%16 (j = 0..31, s2 = kb/2) that the FP8 P·V MFMA expects from it, in
// byte order j = 16*(kb%2) + i.
__host__ __device__ constexpr int block_key(int kb, int rho) {
  return 32 * kb + 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3);
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
  L.off_ks = off;    off = align_up(off + (size_t)bk * L.n_tiles * 256 * (head_dim / 64));
  L.off_v = off;     off = align_up(off + (size_t)bk * L.n_tiles * kKvTile * head_dim);
  L.off_vs = off;    off = align_up(off + (size_t)bk * L.n_tiles * 4);
  L.off_vtile = off; off = align_up(off + (size_t)bk * L.n_vtiles);
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// Pre-pass 1: K -> MXFP4 in MFMA-operand order.
// Thread per (group bk, padded key j, 32-element block g).  Keys past seq_k
// are written as zero codes.  With NS = D/64 contraction steps, block g is
// step s = g/2 of lane half h = g%2:
//   codes : [bk][tile][kb][s][lane = rho + 32h][16 B]
//   scales: [bk][tile][lane][kb*NS + s]
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) pack_k_kernel(const uint16_t* __restrict__ k, int64_t ks0, int64_t ks1,
                                                     int64_t ks2, int kv_heads, int seq_k, int64_t n_tiles,
                                                     uint8_t* __restrict__ wk, uint8_t* __restrict__ wks,
                                                     int64_t total) {
  constexpr int NB = D / 32, NS = D / 64;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= total) return;
  const int g = (int)(id % NB);
  const int64_t jj = (id / NB) % (n_tiles * kKvTile);
  const int64_t bk = id / (NB * n_tiles * kKvTile);
  const int64_t b = bk / kv_heads, h = bk - b * kv_heads;
  const int64_t tile = jj / kKvTile;
  const int kk = (int)(jj - tile * kKvTile);
  // invert block_key: kk = 32*kb + 16*hh + i  ->  rho = (i/4)*8 + 4*hh + i%4
  const int kb = kk >> 5, hh = (kk >> 4) & 1, i = kk & 15;
  const int rho = (i >> 2) * 8 + 4 * hh + (i & 3);
  const int step = g >> 1, lane = rho + 32 * (g & 1);
  uint32_t codes[4] = {0, 0, 0, 0};
  uint32_t scale = 127;
  if (jj < seq_k) {
    const uint4* src = reinterpret_cast<const uint4*>(k + b * ks0 + h * ks1 + jj * ks2 + 32 * g);
    uint32_t w[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 x = src[q];
      w[4 * q] = x.x; w[4 * q + 1] = x.y; w[4 * q + 2] = x.z; w[4 * q + 3] = x.w;
    }
    scale = mxfp4_quantize32(w, codes);
  }
  const int64_t tb = bk * n_tiles + tile;
  *reinterpret_cast<uint4*>(wk + ((tb * 4 + kb) * NS + step) * 1024 + lane * 16) =
      make_uint4(codes[0], codes[1], codes[2], codes[3]);
  wks[(tb * 64 + lane) * (4 * NS) + kb * NS + step] = (uint8_t)scale;
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
//   codes : [bk][tile][db = D/32][s2][half][lane = m + 32h][16 keys]
//           (column d = 32*db + m, keys 64*s2 + 32*half + 16*h .. +15)
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
  uint8_t* out = wv + (bk * n_tiles + tile) * (int64_t)(kKvTile * D);
  for (int o = threadIdx.x; o < D * 8; o += 256) {
    const int lane = o & 63, half = (o >> 6) & 1, s2 = (o >> 7) & 1, db = o >> 8;
    const int col = db * 32 + (lane & 31), k0 = 64 * s2 + 32 * half + 16 * (lane >> 5);
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
  static constexpr int NS = D / 64;               // 64-wide contraction steps of QK^T
  static constexpr int K = 4 * NS * 1024;         // codes of one 128-key tile
  static constexpr int KS = 64 * 4 * NS;          // K scales of one tile
  static constexpr int V = kKvTile * D;           // V^T codes of one tile
  static constexpr int STAGE = K + KS + V + 16;   // + V scale word (padded)
};

// Ping-pong schedule.  The 8 waves form two groups of 4 (one wave of each on
// every SIMD).  Per KV tile k a group runs an MFMA step (P·V of tile k-1, then
// QK^T of tile k) and a VALU step (mask + softmax + FP8 split of tile k),
// separated by workgroup barriers.  Both groups run the same instruction
// stream, but group 1 starts one barrier late (group 0 takes one extra barrier
// at the end), so in every phase one wave per SIMD feeds the matrix core while
// the other keeps the vector ALU busy.  Tile k is read in phases 2k .. 2k+3,
// so three LDS stages rotate.  Each thread fetches its share of tile k+1 into
// registers at the start of its iteration k; group 0 writes it to LDS after
// its VALU step and group 1 after its MFMA step, both at the end of phase
// 2k+1, before either group's QK^T of tile k+1.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_kernel(AttnArgs a) {
  constexpr int W = 8;
  constexpr int kThreads = W * 64;
  using TB = TileBytes<D>;
  constexpr int NS = TB::NS;        // QK^T contraction steps (64 head_dim each)
  constexpr int NDB = D / 32;       // 32-row head_dim blocks of O^T
  constexpr int kStages = 3;
  constexpr int kOnes = kStages * TB::STAGE;   // 1 KB of E4M3 1.0: the row-sum MFMA operand
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * TB::STAGE + 1024];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;    // 0: MFMA step first, 1: one phase behind
  const int ql = lane & 31;     // query column of this lane
  const int lh = lane >> 5;     // lane half (k-block of the MFMA operands)

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

  // every wave walks the workgroup's tiles; rows that cannot see a tile's
  // keys are masked
  const int wg_last_row = min(P0 + a.pos_blocks * kRowsPerWave, a.seq_q) - 1;
  const int kend_wg = CAUSAL ? min(a.seq_k, wg_last_row + off + 1) : a.seq_k;
  const int nt = (kend_wg + kKvTile - 1) / kKvTile;
  const bool wave_live = p0w < a.seq_q;
  const int mask_lim = CAUSAL ? min(a.seq_k - 1, p0w + off) : a.seq_k - 1;   // tiles past it need the mask
  const int row = p0w + ql;
  const int row_lim = (CAUSAL ? min(a.seq_k - 1, row + off) : a.seq_k - 1) - 16 * lh;

  const int64_t bk = (int64_t)b * a.kv_heads + kvh;
  const uint8_t* gk = a.wk + bk * a.n_tiles * TB::K;
  const uint8_t* gks = a.wks + bk * a.n_tiles * TB::KS;
  const uint8_t* gv = a.wv + bk * a.n_tiles * TB::V;
  const uint32_t* gvs = a.wvs + bk * a.n_tiles;

  // ---- Q prologue: this wave's 32 rows to MXFP4 in registers; lane (q, h)
  // holds head_dim block 2s + h of row q for contraction step s ----
  v8i qf[NS];
  int qsc[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    uint4 qc = make_uint4(0, 0, 0, 0);
    qsc[st] = 127;
    if (row < a.seq_q) {
      const uint4* src =
          reinterpret_cast<const uint4*>(a.q + b * a.qs0 + (int64_t)head * a.qs1 + row * a.qs2 + 32 * (2 * st + lh));
      uint32_t w[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 x = src[i];
        w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
      }
      uint32_t c[4];
      qsc[st] = (int)mxfp4_quantize32(w, c);
      qc = make_uint4(c[0], c[1], c[2], c[3]);
    }
    qf[st] = fp4_operand(qc);
  }

  v16f O[NDB];
  v16f L = v16f{};
  v16f S[4];
#pragma unroll
  for (int db = 0; db < NDB; ++db) O[db] = v16f{};
  float m_run = -INFINITY;
  v8i Phi[2] = {v8i{}, v8i{}}, Plo[2] = {v8i{}, v8i{}};
  int psc = 127;
  if (tid < 256) reinterpret_cast<uint32_t*>(lds + kOnes)[tid] = kFp8Ones;

  // output addressing, computed here so the argument block is dead in the loop
  uint16_t* const orow = a.o + b * a.os0 + (int64_t)head * a.os1 + (int64_t)row * a.os2;
  float* const lse_row = a.lse ? a.lse + ((int64_t)b * a.q_heads + head) * a.seq_q + row : nullptr;
  const bool row_live = row < a.seq_q;
  const float cexp = a.c;

  // ---- tile staging: global -> registers -> LDS.  The staging arrays are
  // clang vectors indexed only at compile time, so they stay in VGPRs. ----
  constexpr int KV4 = TB::K / 16, VV4 = TB::V / 16, KSV4 = TB::KS / 16;
  constexpr int KPT = (KV4 + kThreads - 1) / kThreads, VPT = (VV4 + kThreads - 1) / kThreads;
  v4i rk[KPT], rv[VPT], rks;
  uint32_t rvs = 0;
  auto gload = [&](int tile) __attribute__((always_inline)) {
    const v4i* sk = reinterpret_cast<const v4i*>(gk + (int64_t)tile * TB::K);
    const v4i* sv = reinterpret_cast<const v4i*>(gv + (int64_t)tile * TB::V);
    static_for<KPT>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if (KV4 % kThreads == 0 || tid + i * kThreads < KV4) rk[i] = sk[tid + i * kThreads];
    });
    static_for<VPT>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if (VV4 % kThreads == 0 || tid + i * kThreads < VV4) rv[i] = sv[tid + i * kThreads];
    });
    if (tid < KSV4) rks = reinterpret_cast<const v4i*>(gks + (int64_t)tile * TB::KS)[tid];
    if (tid == 0) rvs = gvs[tile];
  };
  auto sstore = [&](int stage) __attribute__((always_inline)) {
    uint8_t* base = lds + stage * TB::STAGE;
    static_for<KPT>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if (KV4 % kThreads == 0 || tid + i * kThreads < KV4) reinterpret_cast<v4i*>(base)[tid + i * kThreads] = rk[i];
    });
    static_for<VPT>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if (VV4 % kThreads == 0 || tid + i * kThreads < VV4)
        reinterpret_cast<v4i*>(base + TB::K + TB::KS)[tid + i * kThreads] = rv[i];
    });
    if (tid < KSV4) reinterpret_cast<v4i*>(base + TB::K)[tid] = rks;
    if (tid == 0) *reinterpret_cast<uint32_t*>(base + TB::K + TB::KS + TB::V) = rvs;
  };

  // MFMA step k: O^T += V^T·P^T and L += 1·P^T for tile k-1 (FP8 x FP8),
  // then S^T = K·Q^T for tile k (FP4 x FP4; both operands' E8M0 scales are
  // applied inside the instruction, so the scores come out dequantized).
  auto mfma_step = [&](int k) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    if (k >= 1) {
      const uint8_t* base = lds + ((k - 1) % kStages) * TB::STAGE;
      const uint8_t* lv = base + TB::K + TB::KS;
      const uint32_t vsw = *reinterpret_cast<const uint32_t*>(base + TB::K + TB::KS + TB::V);
      const v4i o0 = *reinterpret_cast<const v4i*>(lds + kOnes + (lane & 31) * 16);
      const v8i ones = __builtin_shufflevector(o0, o0, 0, 1, 2, 3, 0, 1, 2, 3);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int vsc = (int)((vsw >> (8 * (2 * s2 + lh))) & 0xFF);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint8_t* src = lv + (db * 2 + s2) * 2048 + lane * 16;
          const v4i v0 = *reinterpret_cast<const v4i*>(src);
          const v4i v1 = *reinterpret_cast<const v4i*>(src + 1024);
          const v8i av = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          O[db] = mfma32x32x64<kFmtFp8, kFmtFp8>(av, Phi[s2], O[db], vsc, psc);
          O[db] = mfma32x32x64<kFmtFp8, kFmtFp8>(av, Plo[s2], O[db], vsc, psc - 4);
        }
        L = mfma32x32x64<kFmtFp8, kFmtFp8>(ones, Phi[s2], L, 127, psc);
        L = mfma32x32x64<kFmtFp8, kFmtFp8>(ones, Plo[s2], L, 127, psc - 4);
      }
    }
    if (k < nt) {
      const uint8_t* base = lds + (k % kStages) * TB::STAGE;
      const uint32_t* ksw = reinterpret_cast<const uint32_t*>(base + TB::K + lane * (4 * NS));
      uint32_t ks[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) ks[i] = ksw[i];
      static_for<4 * NS>([&](auto I) {
        constexpr int idx = decltype(I)::value;           // kb * NS + st
        constexpr int kb = idx / NS, st = idx % NS;
        const v8i af = fp4_operand(*reinterpret_cast<const uint4*>(base + (idx * 64 + lane) * 16));
        S[kb] = mfma32x32x64<kFmtFp4, kFmtFp4, idx & 3, 0>(af, qf[st], st == 0 ? v16f{} : S[kb],
                                                          (int)ks[idx >> 2], qsc[st]);
      });
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // VALU step k: mask, online softmax and two-term FP8 split of tile k.
  auto valu_step = [&](int k) __attribute__((always_inline)) {
    if (k < 0 || k >= nt) return;
    if (k * kKvTile + kKvTile - 1 > mask_lim) {      // tiles crossing the diagonal or seq_k
      // element i of key block kb in this lane is key 32*kb + 16*h + i
      const int lim = row_lim - k * kKvTile;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[kb][i] = mask_score(S[kb][i], lim - (32 * kb + i));
    }
    softmax_tile32<NDB>(S, cexp, m_run, O, L, Phi, Plo, psc);
  };

  gload(0);
  sstore(0);
  __syncthreads();
  if (grp == 1) __syncthreads();       // group 1 runs one phase behind
  for (int k = 0; k <= nt; ++k) {
    const bool next = k + 1 < nt;
    if (next) gload(k + 1);
    mfma_step(k);
    if (grp == 1 && next) sstore((k + 1) % kStages);
    __syncthreads();
    valu_step(k);
    if (grp == 0 && next) sstore((k + 1) % kStages);
    __syncthreads();
  }
  if (grp == 0) __syncthreads();       // matches group 1's initial wait

  // ---- epilogue: normalize by the sum of the quantized weights, store bf16
  // rows and the log-sum-exp.  Element i of head_dim block db in lane (q, h)
  // is column 32*db + 8*(i/4) + 4*h + i%4. ----
  if (!wave_live || !row_live) return;
  const float l = L[0];     // every row of the ones-MFMA holds the same sum
  const float inv = 1.0f / l;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const uint32_t w0 = f32_to_bf16(O[db][4 * g4] * inv) | (f32_to_bf16(O[db][4 * g4 + 1] * inv) << 16);
      const uint32_t w1 = f32_to_bf16(O[db][4 * g4 + 2] * inv) | (f32_to_bf16(O[db][4 * g4 + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + 32 * db + 8 * g4 + 4 * lh) = make_uint2(w0, w1);
    }
  if (lse_row != nullptr && lh == 0) {
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    *lse_row = (m_use + __log2f(l)) * kLn2;
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
    hipLaunchKernelGGL((attn_kernel<D, true>), grid, dim3(kWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_kernel<D, false>), grid, dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill_pack(const PrefillParams& p, hipStream_t stream) {
  return p.head_dim == 64 ? launch_pack_d<64>(p, stream) : launch_pack_d<128>(p, stream);
}

hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t stream) {
  return p.head_dim == 64 ? launch_attn_d<64>(p, stream) : launch_attn_d<128>(p, stream);
}

}  // namespace qk4v8
