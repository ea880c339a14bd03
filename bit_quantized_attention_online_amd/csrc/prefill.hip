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
//     Both write one contiguous record per (batch x KV head, 128-key tile):
//     K codes | 1 KB of scales | V codes, i.e. the tile's LDS image, so the
//     attention kernel moves it with direct global->LDS loads in 1 KB chunks.
//  3. attn: one workgroup of 8 waves per (batch, KV head, head group,
//     position block); every wave owns 32 query rows of one query head, all
//     waves share each 128-key K/V tile staged in LDS.  Per tile and wave:
//       S^T = K·Q^T on v_mfma_scale_f32_32x32x64_f8f6f4 (FP4 x FP4),
//       FP32 online softmax in the log2 domain with lazy rescaling,
//       then by default P rounded to bf16 and O^T += V^T·P^T on
//       v_mfma_f32_32x32x16_bf16 against V widened exactly to bf16 (the
//       records then hold bf16 V), the row sums of the bf16 weights by
//       v_dot2_f32_bf16 on the vector unit; or, in the FP8 formats, P split
//       into two E4M3 terms (hi + residual) with a per-(row, tile) E8M0
//       range scale, O^T += V^T·P^T on the scaled FP8 x FP8 instruction
//       (twice: hi, lo) and the row sums as 1·P^T on the same instruction.
//     Computing S^T and O^T (instead of S and O) puts one query per lane
//     column in both, so the softmax state, the P operand and the output rows
//     need no cross-lane transposes.  The 32x32x64 shape keeps the matrix
//     core busy long enough per instruction for the vector ALU work of the
//     other wave on the SIMD to issue alongside it.
#include <algorithm>
#include <climits>

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

// vmcnt(N) on gfx9: vm_cnt[3:0] | exp_cnt[6:4] | lgkm_cnt[11:8] | vm_cnt[5:4]
// << 14, the other counters left at their maximum (no wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 16 bytes per lane from global memory straight into LDS through a buffer
// resource (MUBUF load with the LDS bit): lane l copies bytes voffset ..
// voffset + 15 of the `bytes`-long range at `base` (wave-uniform) to lds_base
// + 16*l (lds_base wave-uniform); reads past the range return zeros.
// Completion is tracked by vmcnt, not by the compiler.  The compiler counts
// these in vmcnt only, so the LDS reads of the MFMA step keep exact lgkmcnt
// waits; with the FLAT-encoded global_load_lds it waits for every
// outstanding LDS read instead, which defeats the operand prefetch.
__device__ __forceinline__ void buffer_to_lds16(const uint8_t* base, uint32_t bytes, uint32_t voffset,
                                                uint8_t* lds_base) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(lds_base)), 16,
      voffset, 0, 0, 0);
}


}  // namespace

// Bytes of one packed 128-key tile record (the LDS image of the tile).  BV:
// V^T as bf16 values (the E4M3 codes times the tile's E8M0 scale, exact)
// for the bf16 P·V product, else as E4M3 codes.
template <int D, bool BV = false>
struct TileBytes {
  static constexpr int NS = D / 64;               // 64-wide contraction steps of QK^T
  static constexpr int K = 4 * NS * 1024;         // K codes: [kb][step][lane][16 B]
  static constexpr int SC = 1024;                 // K scales [lane][kb*NS+step], then the V scale word
  static constexpr int KS = 64 * 4 * NS;          // K scale bytes at the start of SC
  static constexpr int VS_OFF = 512;              // V scale word inside SC
  static constexpr int V = kKvTile * D * (BV ? 2 : 1);   // V^T codes (or bf16 values)
  static constexpr int REC = K + SC + V;          // a multiple of 1 KB
  static constexpr int CHUNKS = REC / 1024;       // 1 KB direct-load chunks
};

PrefillLayout prefill_layout(int batch, int kv_heads, int seq_k, int head_dim, int v_tile_rows, bool bf16_v) {
  PrefillLayout L;
  const int64_t bk = (int64_t)batch * kv_heads;
  L.n_tiles = (seq_k + kKvTile - 1) / kKvTile;
  L.n_vtiles = (seq_k + v_tile_rows - 1) / v_tile_rows;
  if (head_dim == 64)
    L.rec_bytes = bf16_v ? TileBytes<64, true>::REC : TileBytes<64>::REC;
  else
    L.rec_bytes = bf16_v ? TileBytes<128, true>::REC : TileBytes<128>::REC;
  size_t off = 0;
  L.off_rec = off;   off = align_up(off + (size_t)bk * L.n_tiles * L.rec_bytes);
  L.off_vtile = off; off = align_up(off + (size_t)bk * L.n_vtiles);
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// Pre-pass 1: K -> MXFP4 in MFMA-operand order.
// Thread per (group bk, padded key j, 32-element block g).  Keys past seq_k
// are written as zero codes.  With NS = D/64 contraction steps, block g is
// step s = g/2 of lane half h = g%2.  In the record of tile (bk, tile):
//   codes : [kb][s][lane = rho + 32h][16 B]          at 0
//   scales: [lane][kb*NS + s]                         at K
// ---------------------------------------------------------------------------
template <int D, bool BV>
__device__ __forceinline__ void pack_k_block(const uint16_t* __restrict__ k, int64_t ks0, int64_t ks1, int64_t ks2,
                                             int kv_heads, int seq_k, int64_t n_tiles, uint8_t* __restrict__ rec,
                                             int hadamard, int64_t id) {
  using TB = TileBytes<D, BV>;
  constexpr int NB = D / 32, NS = D / 64;
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
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = 0;
  if (jj < seq_k) {
    const uint4* src = reinterpret_cast<const uint4*>(k + b * ks0 + h * ks1 + jj * ks2 + 32 * g);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 x = src[q];
      w[4 * q] = x.x; w[4 * q + 1] = x.y; w[4 * q + 2] = x.z; w[4 * q + 3] = x.w;
    }
  }
  if (!hadamard) {
    if (jj < seq_k) scale = mxfp4_quantize32(w, codes);
  } else {
    // the NB threads of a key row are adjacent lanes (g fastest): stage 32
    // pairs lanes ^ 1, stage 64 lanes ^ 2
    float x[32];
    unpack_bf16x32(w, x);
    fwht32(x);
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = hadamard_pair(x[i], __shfl_xor(x[i], 1, 64), (g & 1) != 0);
    if constexpr (NB == 4) {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = hadamard_pair(x[i], __shfl_xor(x[i], 2, 64), (g & 2) != 0);
    }
    if (jj < seq_k) scale = mxfp4_quantize32f(x, codes);
  }
  uint8_t* r = rec + (bk * n_tiles + tile) * TB::REC;
  *reinterpret_cast<uint4*>(r + (kb * NS + step) * 1024 + lane * 16) = make_uint4(codes[0], codes[1], codes[2], codes[3]);
  r[TB::K + lane * (4 * NS) + kb * NS + step] = (uint8_t)scale;
}

template <int D, bool BV>
__global__ void __launch_bounds__(256) pack_k_kernel(const uint16_t* __restrict__ k, int64_t ks0, int64_t ks1,
                                                     int64_t ks2, int kv_heads, int seq_k, int64_t n_tiles,
                                                     uint8_t* __restrict__ rec, int64_t total, int hadamard) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id < total) pack_k_block<D, BV>(k, ks0, ks1, ks2, kv_heads, seq_k, n_tiles, rec, hadamard, id);
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
// 16 consecutive keys of one column per output chunk.  In the tile record:
//   codes : [db = D/32][s2][half][lane = m + 32h][16 keys]      at K + SC
//           (column d = 32*db + m, keys 64*s2 + 32*half + 16*h .. +15)
//   scales: u32, byte b = E8M0 of the V tile holding key 32b    at K + VS_OFF
// ---------------------------------------------------------------------------
// FUSED (V tiles of R <= 128 rows, which never straddle a 128-key tile): the
// workgroup computes the scales of its own V tiles from the rows it holds in
// registers instead of reading them from the vtile_scale pre-pass.
template <int D>
struct PackVShared {
  static constexpr int LDSROW = D + 4;   // bytes per key row in LDS (padding spreads banks)
  uint8_t tileb[kKvTile * LDSROW];
  float red[4][4];
  uint8_t own[4];                        // E8M0 of this tile's V tiles (FUSED)
};

template <int D, bool FUSED, bool BV>
__device__ __forceinline__ void pack_v_tile(const uint16_t* __restrict__ v, int64_t vs0, int64_t vs1, int64_t vs2,
                                            int kv_heads, int seq_k, int R, int64_t n_tiles, int64_t n_vtiles,
                                            const uint8_t* __restrict__ vtile, uint8_t* __restrict__ rec,
                                            int64_t blk, PackVShared<D>& sh) {
  using TB = TileBytes<D, BV>;
  constexpr int LDSROW = PackVShared<D>::LDSROW;
  constexpr int CPR = D / 8;
  constexpr int PER = kKvTile * CPR / 256;   // 16-byte chunks per thread (rows tid/CPR + (256/CPR)*i)
  uint8_t* tileb = sh.tileb;
  float (*red)[4] = sh.red;
  uint8_t* own = sh.own;
  const int64_t bk = blk / n_tiles, tile = blk - bk * n_tiles;
  const int64_t b = bk / kv_heads, h = bk - b * kv_heads;
  const uint8_t* vts = vtile + bk * n_vtiles;
  uint4 x[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int vi = threadIdx.x + 256 * i;
    const int kk = vi / CPR, cc = vi - kk * CPR;
    const int64_t j = tile * kKvTile + kk;
    x[i] = j < seq_k ? *reinterpret_cast<const uint4*>(v + b * vs0 + h * vs1 + j * vs2 + cc * 8)
                     : make_uint4(0, 0, 0, 0);
  }
  if constexpr (FUSED) {
    // absolute maximum of each V tile (up to 4 of R >= 32 rows) of this key tile
    float am[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int kk = (threadIdx.x + 256 * i) / CPR;
      const uint32_t ws[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(fabsf(bf16_lo(ws[e])), fabsf(bf16_hi(ws[e]))));
      const int t = kk / R;
#pragma unroll
      for (int q = 0; q < 4; ++q) am[q] = fmaxf(am[q], q == t ? m : 0.f);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float w = wave_max(am[q]);
      if ((threadIdx.x & 63) == 0) red[q][threadIdx.x >> 6] = w;
    }
    __syncthreads();
    if (threadIdx.x < 4)
      own[threadIdx.x] = (uint8_t)(mx_shared_exp(fmaxf(fmaxf(red[threadIdx.x][0], red[threadIdx.x][1]),
                                                       fmaxf(red[threadIdx.x][2], red[threadIdx.x][3])),
                                                 8) + 127);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int vi = threadIdx.x + 256 * i;
    const int kk = vi / CPR, cc = vi - kk * CPR;
    const int64_t j = tile * kKvTile + kk;
    uint32_t lo = 0, hi = 0;
    if (j < seq_k) {
      const float inv = exp2i(127 - (int)(FUSED ? own[kk / R] : vts[j / R]));
      const uint32_t ws[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
      uint32_t bb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        bb[e] = e4m3_pack2(clamp448(bf16_lo(ws[e]) * inv), clamp448(bf16_hi(ws[e]) * inv), 1.0f);
      lo = bb[0] | (bb[1] << 16);
      hi = bb[2] | (bb[3] << 16);
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(tileb + kk * LDSROW + cc * 8);
    dst[0] = lo;
    dst[1] = hi;
  }
  __syncthreads();
  uint8_t* const r = rec + (bk * n_tiles + tile) * TB::REC;
  uint8_t* out = r + TB::K + TB::SC;
  if constexpr (BV) {
    // bf16 V^T in the operand order of the 32x32x16 bf16 MFMA: chunk
    // [db][st][lane = m + 32h] holds column 32*db + m at the 8 keys
    // 32*(st/2) + 16*h + 8*(st%2) .. +7, each the E4M3 value times 2^X_V of
    // its V tile, exact in fp32 and then in bf16 (bf16 keeps fp32's exponent
    // range; only values below 2^-126 round, by at most 2^-134).  Keys past
    // seq_k have zero codes.
    for (int o = threadIdx.x; o < D * 16; o += 256) {
      const int lane = o & 63, st = (o >> 6) & 7, db = o >> 9;
      const int col = db * 32 + (lane & 31), k0 = 32 * (st >> 1) + 16 * (lane >> 5) + 8 * (st & 1);
      int64_t j = tile * kKvTile + k0;
      if (j >= seq_k) j = seq_k - 1;
      const int X = (int)(FUSED ? own[k0 / R] : vts[j / R]) - 127;
      const float s1 = exp2i(X / 2), s2 = exp2i(X - X / 2);   // each factor in range for X = -127
      uint32_t wv[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        uint32_t acc = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc |= (uint32_t)tileb[(k0 + 4 * q + e) * LDSROW + col] << (8 * e);
        wv[q] = acc;
      }
      uint32_t outw[4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[q], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[q], true);
        outw[2 * q] = bf16x2(lo[0] * s1 * s2, lo[1] * s1 * s2);
        outw[2 * q + 1] = bf16x2(hi[0] * s1 * s2, hi[1] * s1 * s2);
      }
      *reinterpret_cast<uint4*>(out + (int64_t)o * 16) = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    }
  } else
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
      s |= (uint32_t)(FUSED ? own[(j - tile * kKvTile) / R] : vts[j / R]) << (8 * blk);
    }
    *reinterpret_cast<uint32_t*>(r + TB::K + TB::VS_OFF) = s;
  }
}

template <int D, bool FUSED, bool BV>
__global__ void __launch_bounds__(256) pack_v_kernel(const uint16_t* __restrict__ v, int64_t vs0, int64_t vs1,
                                                     int64_t vs2, int kv_heads, int seq_k, int R, int64_t n_tiles,
                                                     int64_t n_vtiles, const uint8_t* __restrict__ vtile,
                                                     uint8_t* __restrict__ rec) {
  __shared__ PackVShared<D> sh;
  pack_v_tile<D, FUSED, BV>(v, vs0, vs1, vs2, kv_heads, seq_k, R, n_tiles, n_vtiles, vtile, rec, blockIdx.x, sh);
}

// Both packs in one launch (V tiles of R <= 128 rows, whose scales the V
// workgroups compute themselves): the first nblk_k workgroups pack K, the
// rest pack one V tile each, so V work starts as K workgroups retire and
// the step pays one launch instead of two.
struct PackKVArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t ks0, ks1, ks2, vs0, vs1, vs2;
  int kv_heads, seq_k, R, hadamard;
  int64_t n_tiles, n_vtiles, total_k, nblk_k;
  const uint8_t* vtile;    // unused by the V workgroups here (they compute their scales)
  uint8_t* rec;
};

template <int D, bool BV>
__global__ void __launch_bounds__(256) pack_kv_kernel(PackKVArgs a) {
  __shared__ PackVShared<D> sh;
  if ((int64_t)blockIdx.x < a.nblk_k) {
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id < a.total_k)
      pack_k_block<D, BV>(a.k, a.ks0, a.ks1, a.ks2, a.kv_heads, a.seq_k, a.n_tiles, a.rec, a.hadamard, id);
    return;
  }
  pack_v_tile<D, true, BV>(a.v, a.vs0, a.vs1, a.vs2, a.kv_heads, a.seq_k, a.R, a.n_tiles, a.n_vtiles, a.vtile, a.rec,
                           (int64_t)blockIdx.x - a.nblk_k, sh);
}

// ---------------------------------------------------------------------------
// Attention kernel.
// ---------------------------------------------------------------------------
struct AttnArgs {
  const uint16_t* q;
  uint16_t* o;
  float* lse;
  const uint8_t* rec;      // packed tile records [bk][tile]
  int64_t qs0, qs1, qs2, os0, os1, os2;
  int q_heads, kv_heads, group, heads_per_wg, pos_blocks, seq_q, seq_k;
  int xblocks, pos_groups;   // work items = pos_groups x xblocks, xblocks fastest
  int64_t n_tiles;
  float c;          // softmax_scale * log2(e), divided by D for rotated Q/K
  int hadamard;     // Q (and the packed K) rotated by H_D
  int window;       // causal only: > 0 keeps the `window` most recent keys of each row
};

// Persistent schedule.  The grid holds one workgroup per CU; workgroup w
// walks the work items (batch, KV head, head group, position block) in rounds
// of G = gridDim.x, item w of round 0, item G - 1 - w of round 1, and so on:
// items come longest first (causal), and the alternating order evens out the
// rounds (each workgroup starts at a different round).  Within an item nothing changes from a one-item workgroup: the waves
// run the item's tiles t0 .. t0 + nt - 1 as nt + 1 iterations (QK^T only,
// P·V + QK^T, ..., P·V only).  Across items three things carry over:
//  * the tile feed is one stream: the direct loads run two tiles ahead of the
//    QK^T, into the next item's first tiles during the current item's last
//    iterations, and the LDS stage of a tile is its index in the stream mod 4;
//  * the next item's query rows are read at the start of the P·V-only
//    iteration (the score registers are free there) and quantized in its
//    VALU phase, which also stores the finished item's rows;
//  * workgroup start-up (and its wait for the first query rows and tiles) is
//    paid once per CU, not once per item.
//
// Ping-pong schedule.  The 8 waves form two groups of 4 (one wave of each on
// every SIMD).  Per KV tile k a group runs an MFMA step (P·V of tile k-1, then
// QK^T of tile k) and a VALU step (mask + softmax + FP8 split of tile k),
// separated by workgroup barriers.  Both groups run the same instruction
// stream, but group 1 starts one barrier late (group 0 takes one extra barrier
// at the end), so in every phase one wave per SIMD feeds the matrix core while
// the other keeps the vector ALU busy.
//
// Tiles reach LDS by direct global->LDS loads (no registers involved): every
// wave copies its share of the 1 KB chunks of stream tile T+2 at the start of
// the iteration that runs QK^T on stream tile T, into stage (T+2) % 4, whose
// previous tile T-2 was last read by the P·V of an earlier iteration.  Before
// the barrier that ends that iteration's second phase every wave waits until
// its chunks of tile T+1 have landed (the loads complete in order, so at most
// its chunks of tile T+2 may still be in flight), which publishes tile T+1
// before its first QK^T.  A tile thus has about three phases to arrive.
// (Measured: group 1's MFMA phase, which ends with its wait, runs some 400
// cycles longer than group 0's; running the feed three tiles ahead in five
// stages left that gap unchanged, so it is not the loads' latency.)
// PM = kPSingle: single-term E4M3 probabilities (integral running maximum, no
// lo term).  PM = kPBf16: bf16 probabilities on the bf16 matrix core against
// V^T stored as exact bf16 values; its records are 16 KB larger at head_dim
// 128, so three LDS stages hold them (41 KB each) and the feed runs one tile
// ahead: the four waves of group 0 copy all of stream tile T+1 at the start of
// their MFMA phase for tile T, into the stage of tile T-2, whose last reader
// (group 1's P·V) ran in the phase before, and wait for it at the barrier
// that ends their VALU phase, so a tile has two phases to arrive.  Group 1
// copies nothing.  Measured: a direct load costs the issuing wave some 20 - 45
// cycles in an MFMA phase but about 90 inside a VALU phase, which in this
// mode is the longer one, where group 1 would have to issue; splitting each
// tile between both groups' MFMA phases instead (the V part is needed one
// iteration after the K part) left group 1 waiting some 1700 cycles per
// phase for its copies, with the records in L2 or not.
template <int D, bool CAUSAL, int PM>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_kernel(AttnArgs a) {
  constexpr bool FAST = PM == kPSingle;
  constexpr bool BF = PM == kPBf16;
  using TB = TileBytes<D, BF>;
  constexpr int NS = TB::NS;        // QK^T contraction steps (64 head_dim each)
  constexpr int NDB = D / 32;       // 32-row head_dim blocks of O^T
  constexpr int kStages = BF ? 3 : 4;
  constexpr int kOnes = kStages * TB::REC;   // 1 KB of E4M3 1.0: the row-sum MFMA operand (FP8 modes)
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * TB::REC + (BF ? 0 : 1024)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;    // 0: MFMA step first, 1: one phase behind
  const int ql = lane & 31;     // query column of this lane
  const int lh = lane >> 5;     // lane half (k-block of the MFMA operands)
  const int hgroups = a.group / a.heads_per_wg;
  const int hw = wave % a.heads_per_wg, pb = wave / a.heads_per_wg;
  const int off = a.seq_k - a.seq_q;
  const int W = CAUSAL ? a.window : 0;
  const int n_items = a.xblocks * a.pos_groups;
  const int G = (int)gridDim.x;

  // ---- work items ----
  const int R = (n_items + G - 1) / G;
  auto round_item = [&](int r) -> int { return r * G + ((r & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x); };
  // the workgroup takes its rounds starting at round (blockIdx.x mod 8) mod
  // R, so workgroups switch items (and read query rows, store output rows) at
  // different times, while the workgroups of one XCD (blockIdx.x mod 8) stay
  // on the same rounds and share their K/V tiles in its L2; seq_item(i) is
  // the i-th item of that sequence (i is advanced past a round without an
  // item for this workgroup), n_items at the end
  auto seq_item = [&](int& i) -> int {
    for (; i < R; ++i) {
      const int j = round_item((i + ((int)blockIdx.x & 7)) % R);
      if (j < n_items) return j;
    }
    return n_items;
  };
  // first row of item j's position block, and its tiles t0 .. t0 + nt - 1:
  // every wave walks them all; rows that cannot see a tile's keys are masked.
  // With a sliding window the walk starts at the tile holding the first key
  // the item's first row sees.
  auto item_p0 = [&](int j) -> int { return (a.pos_groups - 1 - j / a.xblocks) * a.pos_blocks * kRowsPerWave; };
  auto item_tiles = [&](int j, int& t0_, int& nt_) __attribute__((always_inline)) {
    const int p0 = item_p0(j);
    const int last_row = min(p0 + a.pos_blocks * kRowsPerWave, a.seq_q) - 1;
    const int kend = CAUSAL ? min(a.seq_k, last_row + off + 1) : a.seq_k;
    t0_ = W > 0 ? max(0, p0 + off - W + 1) / kKvTile : 0;
    nt_ = (kend + kKvTile - 1) / kKvTile - t0_;
  };
  // (batch * kv_heads + kv head) and this wave's query head for item j
  auto item_bk = [&](int j) -> int64_t {
    const int bx = j % a.xblocks;
    return (int64_t)(bx / (hgroups * a.kv_heads)) * a.kv_heads + (bx / hgroups) % a.kv_heads;
  };
  auto item_head = [&](int j) -> int {
    const int bx = j % a.xblocks;
    return ((bx / hgroups) % a.kv_heads) * a.group + (bx % hgroups) * a.heads_per_wg + hw;
  };

  // ---- the current item (set by setup) ----
  int b, head, t0, nt, p0w, mask_lim, mask_low, row, row_low;
  uint32_t row_span;
  uint32_t g0 = 0;   // stream index of the item's first tile
  auto setup = [&](int j) __attribute__((always_inline)) {
    const int64_t bk = item_bk(j);
    b = (int)(bk / a.kv_heads);
    head = item_head(j);
    item_tiles(j, t0, nt);
    p0w = item_p0(j) + pb * kRowsPerWave;
    mask_lim = CAUSAL ? min(a.seq_k - 1, p0w + off) : a.seq_k - 1;   // tiles past it need the mask
    // tiles starting before the window's lower edge of the wave's last row need it too
    mask_low = W > 0 ? p0w + kRowsPerWave + off - W : -1;
    row = p0w + ql;
    const int row_lim = (CAUSAL ? min(a.seq_k - 1, row + off) : a.seq_k - 1) - 16 * lh;
    row_low = (W > 0 ? max(0, row + off - W + 1) : 0) - 16 * lh;   // first visible key (clamped at 0)
    // visible keys row_low .. row_low + row_span (rows past seq_q are never stored)
    row_span = (uint32_t)max(row_lim - row_low, 0);
  };
  auto stage_of = [&](int k) -> uint32_t { return (g0 + (uint32_t)k) % kStages; };

  // ---- tile feed: direct global->LDS loads of 1 KB chunks, two tiles ahead
  // of the QK^T (one in bf16 mode) along the stream of this workgroup's
  // items; wave w copies chunks w, w+8, ... of each tile record ----
  // chunks this wave copies per tile: every 8th of the record, or in bf16
  // mode every 4th for the waves of group 0 and none for group 1
  constexpr int kFeeders = BF ? kWaves / 2 : kWaves;
  const int my_chunks = BF && wave >= kFeeders ? 0 : (TB::CHUNKS - wave + kFeeders - 1) / kFeeders;
  // feed state: the next record to copy, the copies left in its item, the
  // LDS stage it goes to (its stream index mod kStages)
  int feed_i = 0;
  const uint8_t* feed_src = nullptr;
  int feed_left = 0;
  uint32_t feed_stage = 0;
  auto feed_item = [&]() __attribute__((always_inline)) {
    const int j = seq_item(feed_i);
    if (j < n_items) {
      int t0_, nt_;
      item_tiles(j, t0_, nt_);
      feed_src = a.rec + (item_bk(j) * a.n_tiles + t0_) * TB::REC;
      feed_left = nt_;
    }
  };
  feed_item();
  auto feed = [&]() -> bool __attribute__((always_inline)) {
    if (feed_left == 0) return false;   // past the last item
    uint8_t* dst = lds + feed_stage * TB::REC;
    static_for<(TB::CHUNKS + kFeeders - 1) / kFeeders>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int c = wave + kFeeders * i;
      if (kFeeders * (i + 1) <= TB::CHUNKS || c < TB::CHUNKS)
        buffer_to_lds16(feed_src, TB::REC, (uint32_t)(c * 1024 + lane * 16), dst + c * 1024);
    });
    feed_src += TB::REC;
    feed_stage = feed_stage + 1 == kStages ? 0 : feed_stage + 1;
    if (--feed_left == 0) {
      ++feed_i;
      feed_item();
    }
    return true;
  };
  // wait until at most `pending` of this wave's memory operations are in flight
  auto wait_dma = [&](int pending) __attribute__((always_inline)) {
    switch (pending) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<1>(); break;
      case 2: wait_vmcnt<2>(); break;
      case 3: wait_vmcnt<3>(); break;
      case 4: wait_vmcnt<4>(); break;
      case 5: wait_vmcnt<5>(); break;
      case 6: wait_vmcnt<6>(); break;
      case 7: wait_vmcnt<7>(); break;
      case 8: wait_vmcnt<8>(); break;
      case 9: wait_vmcnt<9>(); break;
      case 10: wait_vmcnt<10>(); break;
      case 11: wait_vmcnt<11>(); break;
      case 12: wait_vmcnt<12>(); break;
      case 13: wait_vmcnt<13>(); break;
      case 14: wait_vmcnt<14>(); break;
      case 15: wait_vmcnt<15>(); break;
      case 16: wait_vmcnt<16>(); break;
      case 17: wait_vmcnt<17>(); break;
      case 18: wait_vmcnt<18>(); break;
      case 19: wait_vmcnt<19>(); break;
      case 20: wait_vmcnt<20>(); break;
      case 21: wait_vmcnt<21>(); break;
      case 22: wait_vmcnt<22>(); break;
      case 23: wait_vmcnt<23>(); break;
      default: wait_vmcnt<24>(); break;
    }
  };


  // ---- query rows: item j's 32 rows of this wave, bf16, lane (q, h) holding
  // head_dim block 2s + h of row q for contraction step s ----
  auto load_q = [&](int j, uint32_t (&w)[NS][16]) __attribute__((always_inline)) {
    const int r = item_p0(j) + pb * kRowsPerWave + ql;
    const int64_t qbase = (int64_t)(item_bk(j) / a.kv_heads) * a.qs0 + (int64_t)item_head(j) * a.qs1 + (int64_t)r * a.qs2;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
#pragma unroll
      for (int i = 0; i < 16; ++i) w[st][i] = 0;
      if (r < a.seq_q) {
        const uint4* src = reinterpret_cast<const uint4*>(a.q + qbase + 32 * (2 * st + lh));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 x = src[i];
          w[st][4 * i] = x.x; w[st][4 * i + 1] = x.y; w[st][4 * i + 2] = x.z; w[st][4 * i + 3] = x.w;
        }
      }
    }
  };
  // ... to MXFP4 in MFMA operand registers (rows past seq_q quantize zeros)
  v8i qf[NS];
  int qsc[NS];
  auto quantize_q = [&](uint32_t (&w)[NS][16]) __attribute__((always_inline)) {
    if (!a.hadamard) {
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        uint32_t c[4] = {0, 0, 0, 0};
        qsc[st] = (int)mxfp4_quantize32(w[st], c);
        qf[st] = fp4_operand(v4i{(int)c[0], (int)c[1], (int)c[2], (int)c[3]});
      }
    } else {
      // rotated rows: lane (q, h) holds blocks h (step 0) and 2 + h (step 1),
      // so stage 32 pairs the lane with lane ^ 32 and stage 64 pairs its two
      // steps
      float x[NS][32];
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        unpack_bf16x32(w[st], x[st]);
        fwht32(x[st]);
        hadamard_stage_lane_xor32(x[st], lh == 1);
      }
      if constexpr (NS == 2) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const float u = x[0][i], v = x[1][i];
          x[0][i] = u + v;
          x[1][i] = u - v;
        }
      }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        uint32_t c[4];
        qsc[st] = (int)mxfp4_quantize32f(x[st], c);
        qf[st] = fp4_operand(v4i{(int)c[0], (int)c[1], (int)c[2], (int)c[3]});
      }
    }
  };

  v16f O[NDB];
  v16f L;       // FP8 modes: row sums from the ones-operand MFMA (every row holds the sum)
  float Lh;     // bf16 mode: this lane's share of its row's sum (the keys of its lane half)
  v16f S[4];
  float m_run;
  auto reset_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) O[db] = v16f{};
    L = v16f{};
    Lh = 0.f;
    m_run = -INFINITY;
  };
  v8i Phi[2] = {v8i{}, v8i{}}, Plo[2] = {v8i{}, v8i{}};   // FP8 modes
  v4i Pb[8];                                                 // bf16 mode: P^T operands of the 8 steps
  // E8M0 range exponent of the probabilities this lane supplies for P·V
  // steps 0 and 1 (the MFMA applies lane half h's byte to k-block h, the
  // keys 64*s2 + 32*h .. +31)
  int psc[2] = {127, 127};
  const float cexp = a.c;


  // ---- store the finished item's rows: normalize by the sum of the
  // quantized weights, bf16 rows and the log-sum-exp.  Element i of head_dim
  // block db in lane (q, h) is column 32*db + 8*(i/4) + 4*h + i%4.  Buffer
  // stores bounded to the rows below seq_q: every wave issues the same
  // stores and the hardware drops the ones past the bound, so no branch
  // makes the compiler's vmcnt bookkeeping for the next query rows wait for
  // the stores to complete. ----
  auto store_rows = [&]() __attribute__((always_inline)) {
    const int live_rows = max(0, min(kRowsPerWave, a.seq_q - p0w));
    const uint16_t* obase = a.o + b * a.os0 + (int64_t)head * a.os1 + (int64_t)p0w * a.os2;
    const uint32_t obytes = live_rows > 0 ? (uint32_t)(((int64_t)(live_rows - 1) * a.os2 + D) * 2) : 0u;
    const __amdgpu_buffer_rsrc_t ro =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(obase), (short)0, (int)obytes, 0x00020000);
    const uint32_t orow_off = (uint32_t)((int64_t)ql * a.os2 * 2) + 8u * lh;
    const float l = BF ? sum_with_lane_xor32(Lh) : L[0];
    const float inv = 1.0f / l;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const uint32_t w0 = bf16x2(O[db][4 * g4] * inv, O[db][4 * g4 + 1] * inv);
        const uint32_t w1 = bf16x2(O[db][4 * g4 + 2] * inv, O[db][4 * g4 + 3] * inv);
        typedef int v2i_t __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(v2i_t{(int)w0, (int)w1}, ro, orow_off, (32 * db + 8 * g4) * 2, 0);
      }
    if (a.lse != nullptr) {
      // lane half 1 holds the same row: its offset is past the bound
      float* lbase = a.lse + ((int64_t)b * a.q_heads + head) * a.seq_q + p0w;
      const __amdgpu_buffer_rsrc_t rl =
          __builtin_amdgcn_make_buffer_rsrc(lbase, (short)0, live_rows * 4, 0x00020000);
      const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int((m_use + __log2f(l)) * kLn2), rl,
                                            lh == 0 ? (uint32_t)ql * 4 : 0x80000000u, 0, 0);
    }
  };


  // MFMA step k: O^T += V^T·P^T and the row sums for tile k-1,
  // then S^T = K·Q^T for tile k (FP4 x FP4; both operands' E8M0 scales are
  // applied inside the instruction, so the scores come out dequantized).
  // LDS reads are software-pipelined against the matrix instructions: the V
  // operands of head_dim block db+1 are read while the four P·V instructions
  // of block db run, and the K operands of the QK^T while the row sums run,
  // so no LDS round trip sits between two matrix instructions.  (The four instructions of a block accumulate into one
  // register block back to back, which the matrix core chains directly.)
  auto mfma_step = [&](int k, auto with_pv, auto with_qk) __attribute__((always_inline)) {
    constexpr bool PV = decltype(with_pv)::value, QK = decltype(with_qk)::value;
    __builtin_amdgcn_s_setprio(1);
    v4i kf[4 * NS];
    uint32_t ks[NS];
    auto kload = [&]() __attribute__((always_inline)) {
      const uint8_t* base = lds + stage_of(k) * TB::REC;
      static_for<4 * NS>([&](auto I) {
        constexpr int idx = decltype(I)::value;
        kf[idx] = *reinterpret_cast<const v4i*>(base + (idx * 64 + lane) * 16);
      });
      const uint32_t* ksw = reinterpret_cast<const uint32_t*>(base + TB::K + lane * (4 * NS));
#pragma unroll
      for (int i = 0; i < NS; ++i) ks[i] = ksw[i];
    };
    if constexpr (PV && BF) {
      // bf16 P·V: head_dim block db, steps 4*half .. 4*half + 3 (16 keys
      // each) form one unit of four MFMAs; the unit's V^T operands (16 B per
      // lane and step, [db][st][lane] in the record) are read one unit ahead
      const uint8_t* lv = lds + stage_of(k - 1) * TB::REC + TB::K + TB::SC + lane * 16;
      v4i bv[2][4];
      auto bvload = [&](auto U) __attribute__((always_inline)) {
        constexpr int u = decltype(U)::value;
        static_for<4>([&](auto J) {
          constexpr int j = decltype(J)::value;
          bv[u & 1][j] = *reinterpret_cast<const v4i*>(lv + ((u >> 1) * 8 + 4 * (u & 1) + j) * 1024);
        });
      };
      constexpr uint32_t kBf16Ones = 0x3F803F80u;   // two bf16 1.0
      bvload(std::integral_constant<int, 0>{});
      static_for<2 * NDB + 1>([&](auto J) {
        constexpr int u = decltype(J)::value;
        if constexpr (u < 2 * NDB - 1) bvload(std::integral_constant<int, u + 1>{});
        if constexpr (u == 2 * NDB && QK) kload();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (u < 2 * NDB) {
          constexpr int db = u >> 1, h4 = 4 * (u & 1);
          static_for<4>([&](auto JJ) {
            constexpr int j = decltype(JJ)::value;
            O[db] = mfma32x32x16_bf16(bv[u & 1][j], Pb[h4 + j], O[db]);
          });
        } else {
          // row sums of the bf16 weights on the vector unit, two weights per
          // v_dot2_f32_bf16 against (1, 1) in four independent chains; they
          // run between the K operand reads and the QK^T, which wait on those
          // reads anyway (a ones-operand MFMA here cost a fifth of the P·V's
          // matrix cycles)
          typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
          typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
          const bf2_t one2 = __builtin_bit_cast(bf2_t, kBf16Ones);
          float l4[4] = {0.f, 0.f, 0.f, 0.f};
          static_for<8>([&](auto ST) {
            // the pairs through a bf16x8 view and shuffles: a bit_cast of a
            // single dword of the v4i compiled to the wrong dword
            const bf8_t x = __builtin_bit_cast(bf8_t, Pb[decltype(ST)::value]);
            l4[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), one2, l4[0], false);
            l4[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), one2, l4[1], false);
            l4[2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), one2, l4[2], false);
            l4[3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), one2, l4[3], false);
          });
          Lh += (l4[0] + l4[1]) + (l4[2] + l4[3]);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    } else if constexpr (PV) {
      const uint8_t* base = lds + stage_of(k - 1) * TB::REC;
      const uint8_t* lv = base + TB::K + TB::SC + lane * 16;
      const uint32_t vsw = *reinterpret_cast<const uint32_t*>(base + TB::K + TB::VS_OFF);
      const v4i o0 = *reinterpret_cast<const v4i*>(lds + kOnes + (lane & 31) * 16);
      const v8i ones = __builtin_shufflevector(o0, o0, 0, 1, 2, 3, 0, 1, 2, 3);
      const int vsc0 = (int)((vsw >> (8 * lh)) & 0xFF), vsc1 = (int)((vsw >> (8 * (2 + lh))) & 0xFF);
      // head_dim block db: operands for both 64-key halves, read one block ahead
      v8i av[2][2];
      auto vload = [&](auto DB) __attribute__((always_inline)) {
        constexpr int db = decltype(DB)::value;
        static_for<2>([&](auto S2) {
          constexpr int s2 = decltype(S2)::value;
          const v4i v0 = *reinterpret_cast<const v4i*>(lv + (db * 2 + s2) * 2048);
          const v4i v1 = *reinterpret_cast<const v4i*>(lv + (db * 2 + s2) * 2048 + 1024);
          av[db & 1][s2] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        });
      };
      vload(std::integral_constant<int, 0>{});
      static_for<NDB + 1>([&](auto J) {
        constexpr int j = decltype(J)::value;
        if constexpr (j < NDB - 1) vload(std::integral_constant<int, j + 1>{});
        if constexpr (j == NDB && QK) kload();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (j < NDB) {
          O[j] = mfma32x32x64<kFmtFp8, kFmtFp8>(av[j & 1][0], Phi[0], O[j], vsc0, psc[0]);
          if constexpr (!FAST) O[j] = mfma32x32x64<kFmtFp8, kFmtFp8>(av[j & 1][0], Plo[0], O[j], vsc0, psc[0] - 4);
          O[j] = mfma32x32x64<kFmtFp8, kFmtFp8>(av[j & 1][1], Phi[1], O[j], vsc1, psc[1]);
          if constexpr (!FAST) O[j] = mfma32x32x64<kFmtFp8, kFmtFp8>(av[j & 1][1], Plo[1], O[j], vsc1, psc[1] - 4);
        } else {
          L = mfma32x32x64<kFmtFp8, kFmtFp8>(ones, Phi[0], L, 127, psc[0]);
          if constexpr (!FAST) L = mfma32x32x64<kFmtFp8, kFmtFp8>(ones, Plo[0], L, 127, psc[0] - 4);
          L = mfma32x32x64<kFmtFp8, kFmtFp8>(ones, Phi[1], L, 127, psc[1]);
          if constexpr (!FAST) L = mfma32x32x64<kFmtFp8, kFmtFp8>(ones, Plo[1], L, 127, psc[1] - 4);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    } else if constexpr (QK) {
      kload();
    }
    if constexpr (QK) {
      static_for<4 * NS>([&](auto I) {
        constexpr int st = decltype(I)::value / 4, kb = decltype(I)::value % 4;
        constexpr int idx = kb * NS + st;
        S[kb] = mfma32x32x64<kFmtFp4, kFmtFp4, idx & 3, 0>(fp4_operand(kf[idx]), qf[st], st == 0 ? v16f{} : S[kb],
                                                          (int)ks[idx >> 2], qsc[st]);
      });
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // VALU step k: mask, online softmax and two-term FP8 split of tile k
  // (the workgroup's k-th tile, t0 + k).
  auto valu_step = [&](int k) __attribute__((always_inline)) {
    const int j0 = (t0 + k) * kKvTile;
    if (j0 + kKvTile - 1 > mask_lim || j0 < mask_low) {   // tiles crossing the diagonal, seq_k or the window edge
      // element i of key block kb in this lane is key j0 + 32*kb + 16*h + i
      const int low = row_low - j0;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[kb][i] = mask_range(S[kb][i], 32 * kb + i, low, row_span);
    }
    if constexpr (BF)
      softmax_tile32_bf16<NDB>(S, cexp, m_run, O, Lh, Pb);
    else if constexpr (FAST)
      softmax_tile32_single<NDB>(S, cexp, m_run, O, L, Phi, psc, lh);
    else
      softmax_tile32<NDB>(S, cexp, m_run, O, L, Phi, Plo, psc);
  };

  // one iteration of the schedule for tile k of the current item; the first
  // (no P·V yet) is peeled so the steady state has no branches
  auto iteration = [&](int k, auto with_pv) __attribute__((always_inline)) {
    // stream tile T+2 (bf16 mode: T+1, copied by group 0 alone)
    int pending = 0;
    if constexpr (BF) {
      if (grp == 0) feed();
    } else {
      pending = feed() ? my_chunks : 0;
    }
    mfma_step(k, with_pv, std::true_type{});
    // The matrix instructions are pure values to the compiler, which would
    // otherwise sink them past the barrier into the other phase: an empty asm
    // that reads the accumulators keeps them (and the softmax below) on their
    // side of it.
    if constexpr (decltype(with_pv)::value) {
      static_for<NDB>([&](auto DB) { keep_in_vgprs(O[decltype(DB)::value]); });
      if constexpr (BF) keep_in_vgprs(Lh); else keep_in_vgprs(L);
    }
    static_for<4>([&](auto KB) { keep_in_vgprs(S[decltype(KB)::value]); });
    // the next tile of the stream must have landed (from this wave) before the
    // barrier that ends the second phase of this iteration: group 1's MFMA
    // phase, group 0's VALU phase (bf16 mode: group 0's copies of T+1)
    if (!BF && grp == 1) wait_dma(pending);
    phase_barrier();
    valu_step(k);
    if constexpr (BF) {
      static_for<8>([&](auto I) { keep_in_vgprs(Pb[decltype(I)::value]); });
    } else {
      static_for<2>([&](auto I) {
        keep_in_vgprs(Phi[decltype(I)::value]);
        if constexpr (!FAST) keep_in_vgprs(Plo[decltype(I)::value]);
      });
    }
    if (grp == 0) wait_dma(BF ? 0 : pending);
    phase_barrier();
  };
  // the item's last iteration (P·V of tile nt - 1 only): its MFMA phase also
  // requests the next item's query rows, its VALU phase stores this item's
  // rows and switches to item jn
  auto last_iteration = [&](int jn) __attribute__((always_inline)) {
    uint32_t wq[NS][16];
    if (jn < n_items) load_q(jn, wq);
    mfma_step(nt, std::true_type{}, std::false_type{});
    static_for<NDB>([&](auto DB) { keep_in_vgprs(O[decltype(DB)::value]); });
    if constexpr (BF) keep_in_vgprs(Lh); else keep_in_vgprs(L);
    phase_barrier();
    store_rows();
    if (jn < n_items) {
      quantize_q(wq);
      g0 += (uint32_t)nt;
      setup(jn);
      reset_acc();
    }
    phase_barrier();
  };

  // ---- first item: its rows, the stream's first tiles ----
  int cur_i = 0;
  const int cur = seq_item(cur_i);
  setup(cur);
  if (!BF || grp == 0) feed();
  int pending0 = 0;
  if constexpr (!BF) pending0 = feed() ? my_chunks : 0;   // tile 1 stays in flight
  {
    uint32_t wq[NS][16];
    load_q(cur, wq);
    quantize_q(wq);
  }
  reset_acc();
  if constexpr (!BF) {
    if (tid < 256) reinterpret_cast<uint32_t*>(lds + kOnes)[tid] = kFp8Ones;
  }
  wait_dma(pending0);                  // tile 0 (this wave's chunks)
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the ones operand is written
  phase_barrier();
  if (grp == 1) phase_barrier();       // group 1 runs one phase behind
  for (;;) {
    int next_i = cur_i + 1;
    const int jn = seq_item(next_i);
    iteration(0, std::false_type{});
    for (int k = 1; k < nt; ++k) iteration(k, std::true_type{});
    last_iteration(jn);
    if (jn >= n_items) break;
    cur_i = next_i;
  }
  if (grp == 0) phase_barrier();       // matches group 1's initial wait
}

static int gcd_int(int x, int y) {
  while (y) { int t = x % y; x = y; y = t; }
  return x;
}

template <int D, bool BV>
static hipError_t launch_pack_d(const PrefillParams& p, hipStream_t stream) {
  const PrefillLayout L = prefill_layout(p.batch, p.kv_heads, p.seq_k, D, p.v_tile_rows, BV);
  uint8_t* wvt = p.ws + L.off_vtile;
  const int64_t bk = (int64_t)p.batch * p.kv_heads;
  const int64_t total_k = bk * L.n_tiles * kKvTile * (D / 32);
  const int64_t nblk_k = (total_k + 255) / 256;
  if (p.v_tile_rows <= kKvTile) {
    PackKVArgs a;
    a.k = p.k; a.v = p.v;
    a.ks0 = p.ks[0]; a.ks1 = p.ks[1]; a.ks2 = p.ks[2]; a.vs0 = p.vs[0]; a.vs1 = p.vs[1]; a.vs2 = p.vs[2];
    a.kv_heads = p.kv_heads; a.seq_k = p.seq_k; a.R = p.v_tile_rows; a.hadamard = p.hadamard;
    a.n_tiles = L.n_tiles; a.n_vtiles = L.n_vtiles; a.total_k = total_k; a.nblk_k = nblk_k;
    a.vtile = wvt; a.rec = p.ws + L.off_rec;
    hipLaunchKernelGGL((pack_kv_kernel<D, BV>), dim3((unsigned)(nblk_k + bk * L.n_tiles)), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((pack_k_kernel<D, BV>), dim3((unsigned)nblk_k), dim3(256), 0, stream, p.k, p.ks[0], p.ks[1],
                       p.ks[2], p.kv_heads, p.seq_k, L.n_tiles, p.ws + L.off_rec, total_k, p.hadamard);
    hipLaunchKernelGGL((vtile_scale_kernel<D>), dim3((unsigned)(bk * L.n_vtiles)), dim3(256), 0, stream, p.v,
                       p.vs[0], p.vs[1], p.vs[2], p.kv_heads, p.seq_k, p.v_tile_rows, L.n_vtiles, wvt);
    hipLaunchKernelGGL((pack_v_kernel<D, false, BV>), dim3((unsigned)(bk * L.n_tiles)), dim3(256), 0, stream, p.v,
                       p.vs[0], p.vs[1], p.vs[2], p.kv_heads, p.seq_k, p.v_tile_rows, L.n_tiles, L.n_vtiles, wvt,
                       p.ws + L.off_rec);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL, int PM>
static void launch_attn_kernel(dim3 grid, const AttnArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_kernel<D, CAUSAL, PM>), grid, dim3(kWaves * 64), 0, stream, a);
}

template <int D>
static hipError_t launch_attn_d(const PrefillParams& p, hipStream_t stream) {
  const PrefillLayout L = prefill_layout(p.batch, p.kv_heads, p.seq_k, D, p.v_tile_rows, p.p_mode == kPBf16);
  AttnArgs a;
  a.q = p.q; a.o = p.o; a.lse = p.lse;
  a.rec = p.ws + L.off_rec;
  a.qs0 = p.qs[0]; a.qs1 = p.qs[1]; a.qs2 = p.qs[2];
  a.os0 = p.os[0]; a.os1 = p.os[1]; a.os2 = p.os[2];
  a.q_heads = p.q_heads; a.kv_heads = p.kv_heads;
  a.group = p.q_heads / p.kv_heads;
  a.heads_per_wg = gcd_int(a.group, kWaves);
  a.pos_blocks = kWaves / a.heads_per_wg;
  a.seq_q = p.seq_q; a.seq_k = p.seq_k;
  a.n_tiles = L.n_tiles;
  // rotated rows: (H q).(H k) = D (q.k), so the score multiplier is divided
  // by D (exact: a power of two)
  a.c = p.softmax_scale * kLog2e / (p.hadamard ? (float)D : 1.0f);
  a.hadamard = p.hadamard;
  a.window = p.causal && p.window < p.seq_k ? p.window : 0;   // a window of seq_k or more keeps every key
  const int rows_per_wg = a.pos_blocks * kRowsPerWave;
  a.xblocks = p.batch * p.kv_heads * (a.group / a.heads_per_wg);
  a.pos_groups = (p.seq_q + rows_per_wg - 1) / rows_per_wg;
  // persistent: one workgroup per CU (the kernel's LDS and registers allow
  // no more), each walking its share of the work items
  const int64_t items = (int64_t)a.xblocks * a.pos_groups;
  if (items > INT32_MAX) return hipErrorInvalidValue;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)std::min<int64_t>(items, std::max(cus, 1)));
  switch (p.p_mode * 2 + (p.causal ? 1 : 0)) {
    case kPTwoTerm * 2: launch_attn_kernel<D, false, kPTwoTerm>(grid, a, stream); break;
    case kPTwoTerm * 2 + 1: launch_attn_kernel<D, true, kPTwoTerm>(grid, a, stream); break;
    case kPSingle * 2: launch_attn_kernel<D, false, kPSingle>(grid, a, stream); break;
    case kPSingle * 2 + 1: launch_attn_kernel<D, true, kPSingle>(grid, a, stream); break;
    case kPBf16 * 2: launch_attn_kernel<D, false, kPBf16>(grid, a, stream); break;
    default: launch_attn_kernel<D, true, kPBf16>(grid, a, stream); break;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_pack(const PrefillParams& p, hipStream_t stream) {
  const bool bv = p.p_mode == kPBf16;
  if (p.head_dim == 64) return bv ? launch_pack_d<64, true>(p, stream) : launch_pack_d<64, false>(p, stream);
  return bv ? launch_pack_d<128, true>(p, stream) : launch_pack_d<128, false>(p, stream);
}

hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t stream) {
  return p.head_dim == 64 ? launch_attn_d<64>(p, stream) : launch_attn_d<128>(p, stream);
}

}  // namespace qk4v8
