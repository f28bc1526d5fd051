// Grouped GEMM engine for gfx950 MFMA (bf16 and fp32 inputs, fp32 accumulation).
//
//   C[rows of a tile, n] = sum_k A[row, k] * B[group][n, k]
//
// A holds token-side rows (K contiguous); a row is either read directly or
// gathered through the expert permutation (token = perm[row] / top_k), so
// the expert-sorted copy of the tokens is never materialised. B holds
// weight-side rows, also K contiguous (weights are packed [group][N][K]).
// Work items are (row tile, N tile) pairs; row tiles come from the device
// tile list written by the permutation stage (grouped mode) or are cut
// uniformly from M rows (dense mode, the shared expert). The host sizes the
// grid with an upper bound and surplus workgroups exit.
//
// Tiling: 256 threads = 4 waves; each wave owns WM_SUB x WN_SUB MFMA tiles
// of 32x32; a K stage is 128 bytes of every row (64 bf16 or 32 fp32),
// double-buffered in LDS with 16 bytes of row padding so the 16-byte
// fragment reads are bank-conflict free. The MFMA is issued with the
// weight fragment as its first operand, so each lane ends up holding four
// consecutive output columns of one row: 8-byte (bf16) or 16-byte (fp32)
// stores straight from the accumulators.
#pragma once

#include "common.h"

namespace moe {

enum EpiMode {
  kEpiStore = 0,     // c[row][n] = acc
  kEpiSwiglu = 1,    // packed gate|up columns -> c[row][j] = SiLU(gate) * up (+ saved gate, up)
  kEpiSwigluBwd = 2, // acc = dH[row][j]; with saved gate a and up b:
                     // c[row][j] = dH b SiLU'(a), c[row][h + j] = dH SiLU(a)
  kEpiCombine = 3,   // dense rows are tokens t: v = acc rounded to the storage type,
                     // c[t][n] = sum_i gw[t,i] * gy[ginv[t*gk + i]][n] + v
  kEpiStoreRouter = 4  // wide bf16 engine only: c[row][n] = acc + rdl[row] * rw[group][n]
};

// Largest top_k the fused gather-sum epilogue takes.
constexpr int kCombineMaxK = 8;

struct GemmArgs {
  const void* a;          // token-side rows
  int64_t lda;            // elements between rows of a
  const int32_t* perm;    // gather mode: sorted row -> flat slot
  int topk;               // gather mode: token = perm[row] / topk
  const void* b;          // [groups][N][ldb]: row n holds k = 0 .. ksplit-1
  int64_t b_group_stride; // elements between groups of b
  int64_t ldb;            // elements between rows of b (0: K)
  const void* b2;         // optional second half: row n holds k = ksplit .. K-1
  int64_t b2_group_stride;
  int ksplit;             // first k read from b2 (K when b2 is unused); a multiple of the stage
  int N, K;
  const int32_t* tiles;     // grouped mode: (group, first row, rows) triples
  const int32_t* num_tiles; // grouped mode: number of valid triples
  int64_t M;                // dense mode: number of rows
  void* c;                  // output rows, indexed by tile row (sorted row or token)
  int64_t ldc;
  void* sa;                 // SwiGLU: saved gate pre-activations (optional in forward)
  void* sb;                 // SwiGLU: saved up pre-activations
  int64_t lds;              // row stride of sa / sb
  int hsplit;               // SwiGLU backward: column offset of the up gradient in c
  const void* gy;           // fused combine: expert-sorted rows, row stride ldc
  const float* gw;          // fused combine: [M][gk] weights
  const int32_t* ginv;      // fused combine: [M][gk] sorted row of each (token, rank)
  int gk;                   // fused combine: top_k (<= kCombineMaxK)
  const float* rdl;         // kEpiStoreRouter: per-row scale, indexed by tile row
  const float* rw;          // kEpiStoreRouter: [groups][N] rows added, scaled by rdl
};

// Value of v once stored in T and read back.
__device__ __forceinline__ float round_to(float v, const bf16_t*) { return bf16_to_f32(f32_to_bf16(v)); }
__device__ __forceinline__ float round_to(float v, const float*) { return v; }

// Fused gather-sum for four consecutive columns n.. of token t, in the
// combine stage's order: fp32 multiply-adds over ranks 0..k-1 from zero,
// then the (already rounded) dense value v added. idx and wt hold the
// token's sorted rows and weights; a row of -1 (dropped by capacity routing)
// is left out.
template <typename T>
__device__ __forceinline__ void combine4(const GemmArgs& p, int64_t t, int n, const float (&v)[4],
                                         const int (&idx)[kCombineMaxK],
                                         const float (&wt)[kCombineMaxK]) {
  const T* y = static_cast<const T*>(p.gy);
  float yv[kCombineMaxK][4];
#pragma unroll
  for (int i = 0; i < kCombineMaxK; ++i)
    if (i < p.gk && idx[i] >= 0) load4(y + static_cast<int64_t>(idx[i]) * p.ldc + n, yv[i]);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < kCombineMaxK; ++i)
    if (i < p.gk && idx[i] >= 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(wt[i], yv[i][q], acc[q]);
    }
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] += v[q];
  store4(static_cast<T*>(p.c) + t * p.ldc + n, acc[0], acc[1], acc[2], acc[3]);
}

template <int BM_, int WAVES_M_, int WAVES_N_, int WM_SUB_, int WN_SUB_, int PF_ = 2>
struct TileCfg {
  static constexpr int BM = BM_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int WPE = 2;  // waves per SIMD the register budget is sized for
  static constexpr int PF = PF_;  // K stages prefetched into registers (1 or 2)
  static constexpr int WM_SUB = WM_SUB_, WN_SUB = WN_SUB_;
  static constexpr int BN = WAVES_N * WN_SUB * 32;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;  // threads per workgroup
  static_assert(WAVES_M * WM_SUB * 32 == BM, "rows");
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "whole chunks per thread");
};
// Four-wave tiles (BN 128), one per block_m.
using Cfg128 = TileCfg<128, 2, 2, 2, 2>;
using Cfg64 = TileCfg<64, 2, 2, 1, 2>;
using Cfg32 = TileCfg<32, 1, 4, 1, 1>;
// Eight-wave tiles with BN 256: twice the MFMA work per byte staged. Wide
// N (a whole gate|up block of width <= 128, or 256 model columns) per tile.
using Cfg128W = TileCfg<128, 2, 4, 2, 2>;  // 128 x 256, waves 64 x 64
using Cfg64W = TileCfg<64, 2, 4, 1, 2>;    // 64 x 256, waves 32 x 64
// 256 x 256, waves 128 x 64, one stage of register prefetch (registers):
// 128 MFMA flops per staged byte, twice the 128 x 128 tile.
using Cfg256W = TileCfg<256, 2, 4, 4, 2, 1>;
// 256 x 128 for N not a multiple of 256 (four waves, 64 x 128 each).
using Cfg256N = TileCfg<256, 4, 1, 2, 4, 1>;

constexpr int kStageBytes = 128;   // K bytes per row per stage
constexpr int kLdsRowBytes = 144;  // + 16 bytes padding

template <typename T>
struct Mfma;
template <>
struct Mfma<bf16_t> {
  // One 16-byte chunk per lane group: 32x32x16.
  __device__ static void step(const u32x4& w, const u32x4& x, f32x16_t& acc) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w),
                                                  __builtin_bit_cast(bf16x8_t, x), acc, 0, 0, 0);
  }
};
template <>
struct Mfma<float> {
  // One 16-byte chunk per lane group = 4 k values: four 32x32x2 steps, step s
  // taking element s of each lane group's chunk (the same k on both sides).
  __device__ static void step(const u32x4& w, const u32x4& x, f32x16_t& acc) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(w.x), __uint_as_float(x.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(w.y), __uint_as_float(x.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(w.z), __uint_as_float(x.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(w.w), __uint_as_float(x.w), acc, 0, 0, 0);
  }
};

// Pipeline pieces of the GEMM main loop. A stage's staging registers travel
// by value so they stay in VGPRs.
template <int A_CH, int B_CH>
struct StageRegs {
  u32x4 a[A_CH];
  u32x4 b[B_CH];
};

template <int A_CH, int B_CH, int NT>
__device__ __forceinline__ StageRegs<A_CH, B_CH> gemm_gload(const char* const (&a_src)[A_CH],
                                                           const char* b_src, int64_t b_row_bytes,
                                                           int off) {
  StageRegs<A_CH, B_CH> r;
#pragma unroll
  for (int i = 0; i < A_CH; ++i) r.a[i] = *reinterpret_cast<const u32x4*>(a_src[i] + off);
  // b_src already points at this thread's first chunk; chunk i is NT/8 rows further.
#pragma unroll
  for (int i = 0; i < B_CH; ++i)
    r.b[i] = *reinterpret_cast<const u32x4*>(b_src + i * (NT / 8) * b_row_bytes + off);
  return r;
}

// Thread tid stages 16-byte chunk (tid + NT i) of each operand tile: row
// (tid >> 3) + (NT / 8) i, column chunk tid & 7.
template <int A_CH, int B_CH, int A_BYTES, int NT>
__device__ __forceinline__ void gemm_lstore(char* s, const StageRegs<A_CH, B_CH> r, int lds_off) {
#pragma unroll
  for (int i = 0; i < A_CH; ++i)
    *reinterpret_cast<u32x4*>(s + lds_off + i * (NT / 8) * kLdsRowBytes) = r.a[i];
#pragma unroll
  for (int i = 0; i < B_CH; ++i)
    *reinterpret_cast<u32x4*>(s + A_BYTES + lds_off + i * (NT / 8) * kLdsRowBytes) = r.b[i];
}

// One K stage out of LDS: four fragment steps of 32 bytes per row.
template <typename T, int WM_SUB, int WN_SUB>
__device__ __forceinline__ void gemm_compute(const char* s, int a_frag, int b_frag,
                                             f32x16_t (&acc)[WM_SUB][WN_SUB]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    u32x4 xf[WM_SUB], wf[WN_SUB];
#pragma unroll
    for (int i = 0; i < WM_SUB; ++i)
      xf[i] = *reinterpret_cast<const u32x4*>(s + a_frag + i * 32 * kLdsRowBytes + q * 32);
#pragma unroll
    for (int j = 0; j < WN_SUB; ++j)
      wf[j] = *reinterpret_cast<const u32x4*>(s + b_frag + j * 32 * kLdsRowBytes + q * 32);
#pragma unroll
    for (int i = 0; i < WM_SUB; ++i)
#pragma unroll
      for (int j = 0; j < WN_SUB; ++j) Mfma<T>::step(wf[j], xf[i], acc[i][j]);
  }
}

// Epilogue of one tile. Accumulator register q of MFMA tile (i, j) holds row
// m = i*32 + r32 and column n = j*32 + 8*(q/4) + 4*g + q%4 of the wave's
// sub-block, so each lane writes runs of four consecutive columns.
template <typename T, typename Cfg, int kEpi>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& p,
                                              const f32x16_t (&acc)[Cfg::WM_SUB][Cfg::WN_SUB],
                                              int row0, int rows, int nt, int wm, int wn, int g,
                                              int r32) {
  constexpr int WM_SUB = Cfg::WM_SUB, WN_SUB = Cfg::WN_SUB, BN = Cfg::BN;
  T* c = static_cast<T*>(p.c);
#pragma unroll
  for (int i = 0; i < WM_SUB; ++i) {
    const int m = wm * WM_SUB * 32 + i * 32 + r32;
    if (m >= rows) continue;
    const int64_t orow = static_cast<int64_t>(row0) + m;
    int idx[kCombineMaxK];
    float wt[kCombineMaxK];
    if (kEpi == kEpiCombine) {
#pragma unroll
      for (int ii = 0; ii < kCombineMaxK; ++ii) {
        idx[ii] = ii < p.gk ? p.ginv[orow * p.gk + ii] : 0;
        wt[ii] = ii < p.gk ? p.gw[orow * p.gk + ii] : 0.0f;
      }
    }
    if (kEpi == kEpiSwigluBwd) {
      // The saved pre-activations of JB MFMA tiles are all loaded before
      // any result is stored: interleaved, each load would wait behind the
      // previous stores (they may alias as far as the compiler knows),
      // one memory round trip per four columns.
      constexpr int JB = WM_SUB >= 4 ? 1 : (WN_SUB > 2 ? 2 : WN_SUB);
      const T* sa = static_cast<const T*>(p.sa);
      const T* sb = static_cast<const T*>(p.sb);
#pragma unroll
      for (int jb = 0; jb < WN_SUB; jb += JB) {
        float a[JB][4][4], b[JB][4][4];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int n = nt * BN + wn * WN_SUB * 32 + (jb + jj) * 32 + 8 * rr + 4 * g;
            load4(sa + orow * p.lds + n, a[jj][rr]);
            load4(sb + orow * p.lds + n, b[jj][rr]);
          }
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int n = nt * BN + wn * WN_SUB * 32 + (jb + jj) * 32 + 8 * rr + 4 * g;
            float da[4], db[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float dh = acc[i][jb + jj][4 * rr + q];
              const float av = a[jj][rr][q], bv = b[jj][rr][q];
              const float sg = sigmoid_f(av);
              da[q] = dh * bv * sg * (1.0f + av * (1.0f - sg));
              db[q] = dh * av * sg;
            }
            store4(c + orow * p.ldc + n, da[0], da[1], da[2], da[3]);
            store4(c + orow * p.ldc + p.hsplit + n, db[0], db[1], db[2], db[3]);
          }
      }
      continue;
    }
#pragma unroll
    for (int j = 0; j < WN_SUB; ++j) {
      const int n0 = nt * BN + wn * WN_SUB * 32 + j * 32;
      if (kEpi == kEpiCombine) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float v[4] = {round_to(acc[i][j][4 * rr + 0], c), round_to(acc[i][j][4 * rr + 1], c),
                              round_to(acc[i][j][4 * rr + 2], c), round_to(acc[i][j][4 * rr + 3], c)};
          combine4<T>(p, orow, n0 + 8 * rr + 4 * g, v, idx, wt);
        }
      } else if (kEpi == kEpiStore) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int n = n0 + 8 * rr + 4 * g;
          store4(c + orow * p.ldc + n, acc[i][j][4 * rr + 0], acc[i][j][4 * rr + 1],
                 acc[i][j][4 * rr + 2], acc[i][j][4 * rr + 3]);
        }
      } else {
        // Packed columns [n0, n0+16) are gate columns n0/2 + [0,16) and
        // [n0+16, n0+32) the matching up columns: registers 0-7 are gate
        // values, 8-15 the up values of the same hidden columns.
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int hc = n0 / 2 + 8 * rr + 4 * g;
          float a[4], b[4], hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            a[q] = acc[i][j][4 * rr + q];
            b[q] = acc[i][j][4 * (rr + 2) + q];
            hv[q] = silu_f(a[q]) * b[q];
          }
          store4(c + orow * p.ldc + hc, hv[0], hv[1], hv[2], hv[3]);
          if (p.sa) {
            store4(static_cast<T*>(p.sa) + orow * p.lds + hc, a[0], a[1], a[2], a[3]);
            store4(static_cast<T*>(p.sb) + orow * p.lds + hc, b[0], b[1], b[2], b[3]);
          }
        }
      }
    }
  }
}

// Row tile of one work item: its weight group, first output row and rows.
struct TileInfo {
  int group, row0, rows;
};

template <typename Cfg, bool kDense>
__device__ __forceinline__ TileInfo tile_info(const GemmArgs& p, int w, int n_tiles_n) {
  const int mt = w / n_tiles_n;
  TileInfo t;
  if (kDense) {
    t.group = 0;
    t.row0 = mt * Cfg::BM;
    const int64_t left = p.M - t.row0;
    t.rows = left <= 0 ? 0 : static_cast<int>(left < Cfg::BM ? left : Cfg::BM);
  } else if (mt < *p.num_tiles) {
    t.group = p.tiles[3 * mt + 0];
    t.row0 = p.tiles[3 * mt + 1];
    t.rows = p.tiles[3 * mt + 2];
  } else {
    t.group = 0;
    t.row0 = 0;
    t.rows = 0;  // past the last tile
  }
  return t;
}

// Source rows of the A chunks this thread stages for a tile (rows past the
// tile's end repeat its last row; their results are never stored).
template <int A_CH, int NT, bool kGather>
__device__ __forceinline__ void tile_rows(const GemmArgs& p, const TileInfo& t, int tid,
                                          int (&src)[A_CH]) {
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int r = (tid + i * NT) >> 3;
    const int mr = t.rows > 0 ? min(r, t.rows - 1) : 0;
    src[i] = kGather ? (t.rows > 0 ? p.perm[t.row0 + mr] / p.topk : 0) : t.row0 + mr;
  }
}

// Persistent grouped GEMM. Workgroup b runs on XCD b % 8 (round-robin
// dispatch) and walks that XCD's contiguous share of the (row tile, N tile)
// work list, so the tiles of one expert, and its weights, stay in one L2.
// The next item's metadata is fetched at the start of a tile and its
// gathered row indices before this tile's epilogue, off the critical path.
template <typename T, typename Cfg, bool kGather, int kEpi, bool kDense>
__global__ __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::WPE)))
void gemm_kernel(const GemmArgs p, int total_work) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, NT = Cfg::NT;
  constexpr int WM_SUB = Cfg::WM_SUB, WN_SUB = Cfg::WN_SUB;
  constexpr int A_CH = BM * 8 / NT;  // 16-byte chunks per thread per stage
  constexpr int B_CH = BN * 8 / NT;
  constexpr int KT = kStageBytes / static_cast<int>(sizeof(T));
  constexpr int A_BYTES = BM * kLdsRowBytes, B_BYTES = BN * kLdsRowBytes;
  __shared__ __attribute__((aligned(16))) char smem[2 * (A_BYTES + B_BYTES)];

  const int n_tiles_n = p.N / BN;
  const int G = gridDim.x;
  const int nx = G < 8 ? G : 8;
  const int x = blockIdx.x % nx, wi = blockIdx.x / nx;
  const int gx = G / nx + (x < G % nx ? 1 : 0);
  const int per = (total_work + nx - 1) / nx;
  const int w_end = min(total_work, (x + 1) * per);
  int w = x * per + wi;
  if (w >= w_end) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int64_t ldb = p.ldb ? p.ldb : p.K;
  const int ks_split = p.b2 ? p.ksplit / KT : (1 << 30);  // first stage read from b2
  const int nk = p.K / KT;
  const int a_frag = (wm * WM_SUB * 32 + r32) * kLdsRowBytes + g * 16;
  const int b_frag = A_BYTES + (wn * WN_SUB * 32 + r32) * kLdsRowBytes + g * 16;
  const int bufb = A_BYTES + B_BYTES;
  const int lds_off = (tid >> 3) * kLdsRowBytes + (tid & 7) * 16;
  const int64_t b_row_bytes = ldb * static_cast<int64_t>(sizeof(T));
  const int64_t b_thr = (tid >> 3) * b_row_bytes + (tid & 7) * 16;

  TileInfo cur = tile_info<Cfg, kDense>(p, w, n_tiles_n);
  int src_cur[A_CH];
  tile_rows<A_CH, NT, kGather>(p, cur, tid, src_cur);

  while (true) {
    if (cur.rows <= 0) break;  // past the last tile; every later item is too
    const int nt = w % n_tiles_n;
    const int group = cur.group, row0 = cur.row0, rows = cur.rows;
    const char* a_src[A_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i)
      a_src[i] = static_cast<const char*>(p.a) +
                 static_cast<int64_t>(src_cur[i]) * p.lda * static_cast<int64_t>(sizeof(T)) +
                 ((tid + i * NT) & 7) * 16;
    const char* b_base = static_cast<const char*>(p.b) + b_thr +
                         (static_cast<int64_t>(group) * p.b_group_stride +
                          static_cast<int64_t>(nt) * BN * ldb) * static_cast<int64_t>(sizeof(T));
    const char* b2_base = p.b2 ? static_cast<const char*>(p.b2) + b_thr +
                                     (static_cast<int64_t>(group) * p.b2_group_stride +
                                      static_cast<int64_t>(nt) * BN * ldb -
                                      static_cast<int64_t>(p.ksplit)) * static_cast<int64_t>(sizeof(T))
                               : nullptr;
    auto stage_b = [&](int st) { return st < ks_split ? b_base : b2_base; };

    f32x16_t acc[WM_SUB][WN_SUB];
#pragma unroll
    for (int i = 0; i < WM_SUB; ++i)
#pragma unroll
      for (int j = 0; j < WN_SUB; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    // Metadata of the next item (its row indices are fetched after this tile).
    const int w1 = w + gx;
    const TileInfo nxt = (w1 < w_end) ? tile_info<Cfg, kDense>(p, w1, n_tiles_n) : TileInfo{0, 0, 0};
    // Software pipeline with a ring of PF register stages: while stage s is
    // multiplied out of LDS buffer s&1, stages s+1 .. s+PF-1 wait in
    // registers and stage s+PF is in flight from memory, so PF stages of
    // loads cover one memory latency. The scheduling fences keep loads
    // before the MFMAs and the LDS store (which waits for its loads) after
    // them; left alone, the compiler hoists the store and sinks the loads to
    // save registers. The loop is unrolled by PF so ring slots are static.
    constexpr int PF = Cfg::PF;
    StageRegs<A_CH, B_CH> ring[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j)
      if (j < nk) ring[j] = gemm_gload<A_CH, B_CH, NT>(a_src, stage_b(j), b_row_bytes, j * kStageBytes);
    gemm_lstore<A_CH, B_CH, A_BYTES, NT>(smem, ring[0], lds_off);
    __syncthreads();
    for (int s0 = 0; s0 < nk; s0 += PF) {
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        const int s = s0 + j;
        if (s < nk) {
          if (s + PF < nk)
            ring[j] = gemm_gload<A_CH, B_CH, NT>(a_src, stage_b(s + PF), b_row_bytes,
                                                 (s + PF) * kStageBytes);
          __builtin_amdgcn_sched_barrier(0);
          gemm_compute<T, WM_SUB, WN_SUB>(smem + (s & 1) * bufb, a_frag, b_frag, acc);
          __builtin_amdgcn_sched_barrier(0);
          if (s + 1 < nk) {
            gemm_lstore<A_CH, B_CH, A_BYTES, NT>(smem + ((s + 1) & 1) * bufb, ring[(j + 1) % PF],
                                                 lds_off);
            __syncthreads();
          }
        }
      }
    }
    // Row indices of the next item, while this tile's results drain.
    tile_rows<A_CH, NT, kGather>(p, nxt, tid, src_cur);

    gemm_epilogue<T, Cfg, kEpi>(p, acc, row0, rows, nt, wm, wn, g, r32);

    // The last stage's LDS reads finish before the next tile's first store.
    __syncthreads();
    w += gx;
    if (w >= w_end) break;
    cur = nxt;
  }
}

// ------------------------------------------------------------------ wgrad
// Weight-gradient GEMM: the reduction runs over token rows.
//
//   C[g][m][n] = sum over rows r of group g: A[r][m] * B[r][n]     (fp32 out)
//
// Group g covers rows [row_offsets[g], row_offsets[g+1]) (grouped mode: an
// expert's sorted rows, so K varies per expert) or the g-th of `splits`
// equal slices of rows_total (dense mode, a split-K partial reduced later
// in a fixed order). Both operands are row-major with the reduction index
// as the row, so each stage is transposed on its way to LDS: a thread loads
// a V x V block (V = 16 bytes of elements) with V 16-byte loads, transposes
// it in registers and writes V 16-byte LDS rows, giving the same
// K-contiguous LDS tiles as the forward kernel. Rows past the group's end
// load as zeros. One workgroup owns each (group, M tile, N tile) output, so
// the result is deterministic without atomics.
struct WgradArgs {
  const void* a;
  int64_t lda;
  const int32_t* perm;  // gather mode for A: row r reads token perm[r] / topk
  int topk;
  const void* b;
  int64_t ldb;
  int M, N;
  const int32_t* row_offsets;  // grouped mode: [groups + 1]
  int cap;                     // grouped mode: rows per group past which rows are
                               // dropped (capacity routing); 0 = none
  int64_t rows_total;          // dense mode
  int splits;                  // dense mode
  float* c;
  float* c2;       // columns n >= nsplit go to c2 (column n - nsplit)
  int nsplit;
  int64_t ldc;
  int64_t c_group_stride;
  int trans_c;     // bf16 kernel: store C^T, element (m, n) at c + n * ldc + m (no c2)
};

template <typename T>
struct Transpose;
template <>
struct Transpose<bf16_t> {
  static constexpr int V = 8;
  // out[c] = (in[0][c], in[1][c], ..., in[7][c])
  __device__ static void run(const u32x4* in, u32x4* out) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(in);  // w[4*r + c/2]
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = w[4 * (2 * q) + c / 2], hi = w[4 * (2 * q + 1) + c / 2];
        o[q] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      out[c] = (u32x4){o[0], o[1], o[2], o[3]};
    }
  }
};
template <>
struct Transpose<float> {
  static constexpr int V = 4;
  __device__ static void run(const u32x4* in, u32x4* out) {
    out[0] = (u32x4){in[0].x, in[1].x, in[2].x, in[3].x};
    out[1] = (u32x4){in[0].y, in[1].y, in[2].y, in[3].y};
    out[2] = (u32x4){in[0].z, in[1].z, in[2].z, in[3].z};
    out[3] = (u32x4){in[0].w, in[1].w, in[2].w, in[3].w};
  }
};

// Stage loader of the weight-gradient kernel: thread `tid` fetches its
// V x V blocks of A (blocks 0 .. NB-1) and B (NB .. 2NB-1); rows outside
// [r0, r1) read as zeros.
template <typename T, bool kGatherA, int PER, int V, int NB, int KT>
__device__ __forceinline__ void wgrad_gload(const WgradArgs& p, u32x4 (&blk)[PER][V], int64_t r0,
                                            int64_t r1, int ks, int mt, int nt, int tid) {
  constexpr int CB = 128 / V;  // column blocks per operand row
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int b = tid + q * 256;
    const bool is_b = b >= NB;
    const int bb = is_b ? b - NB : b;
    const int rb = bb / CB, cb = bb % CB;
#pragma unroll
    for (int rr = 0; rr < V; ++rr) {
      const int64_t r = r0 + static_cast<int64_t>(ks) * KT + rb * V + rr;
      u32x4 v = (u32x4){0u, 0u, 0u, 0u};
      if (r < r1) {
        const T* src;
        if (is_b) {
          src = static_cast<const T*>(p.b) + r * p.ldb + nt * 128 + cb * V;
        } else {
          const int64_t ar = kGatherA ? static_cast<int64_t>(p.perm[r] / p.topk) : r;
          src = static_cast<const T*>(p.a) + ar * p.lda + mt * 128 + cb * V;
        }
        v = *reinterpret_cast<const u32x4*>(src);
      }
      blk[q][rr] = v;
    }
  }
}

// Transposes the fetched blocks into K-contiguous LDS rows.
template <typename T, int PER, int V, int NB, int A_BYTES>
__device__ __forceinline__ void wgrad_lstore(char* s, const u32x4 (&blk)[PER][V], int tid) {
  constexpr int CB = 128 / V;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int b = tid + q * 256;
    const bool is_b = b >= NB;
    const int bb = is_b ? b - NB : b;
    const int rb = bb / CB, cb = bb % CB;
    u32x4 t[V];
    Transpose<T>::run(blk[q], t);
    char* base = s + (is_b ? A_BYTES : 0) + rb * 16;
#pragma unroll
    for (int cc = 0; cc < V; ++cc) *reinterpret_cast<u32x4*>(base + (cb * V + cc) * kLdsRowBytes) = t[cc];
  }
}

template <typename T, bool kGatherA, bool kDense>
__global__ __launch_bounds__(256, 2) void wgrad_kernel(const WgradArgs p) {
  constexpr int BM = 128, BN = 128, WM_SUB = 2, WN_SUB = 2;
  constexpr int V = Transpose<T>::V;
  constexpr int KT = kStageBytes / static_cast<int>(sizeof(T));  // rows per stage
  constexpr int NB = (KT / V) * (BM / V);                         // blocks per operand
  constexpr int PER = 2 * NB / 256;                               // blocks per thread
  constexpr int A_BYTES = BM * kLdsRowBytes, B_BYTES = BN * kLdsRowBytes;
  __shared__ __attribute__((aligned(16))) char smem[2 * (A_BYTES + B_BYTES)];

  const int tiles_m = p.M / BM, tiles_n = p.N / BN;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = logical / (tiles_m * tiles_n);
  const int rem = logical % (tiles_m * tiles_n);
  const int mt = rem / tiles_n, nt = rem % tiles_n;
  int64_t r0, r1;
  if (kDense) {
    r0 = p.rows_total * grp / p.splits;
    r1 = p.rows_total * (grp + 1) / p.splits;
  } else {
    r0 = p.row_offsets[grp];
    r1 = p.row_offsets[grp + 1];
    if (p.cap > 0 && r1 - r0 > p.cap) r1 = r0 + p.cap;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16_t acc[WM_SUB][WN_SUB];
#pragma unroll
  for (int i = 0; i < WM_SUB; ++i)
#pragma unroll
    for (int j = 0; j < WN_SUB; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  const int nk = static_cast<int>((r1 - r0 + KT - 1) / KT);
  const int a_frag = (wm * WM_SUB * 32 + r32) * kLdsRowBytes + g * 16;
  const int b_frag = A_BYTES + (wn * WN_SUB * 32 + r32) * kLdsRowBytes + g * 16;
  u32x4 blk[PER][V];
  if (nk > 0) {
    wgrad_gload<T, kGatherA, PER, V, NB, KT>(p, blk, r0, r1, 0, mt, nt, tid);
    wgrad_lstore<T, PER, V, NB, A_BYTES>(smem, blk, tid);
    __syncthreads();
    for (int ks = 0; ks + 1 < nk; ++ks) {
      const int buf = ks & 1;
      wgrad_gload<T, kGatherA, PER, V, NB, KT>(p, blk, r0, r1, ks + 1, mt, nt, tid);
      gemm_compute<T, WM_SUB, WN_SUB>(smem + buf * (A_BYTES + B_BYTES), a_frag, b_frag, acc);
      wgrad_lstore<T, PER, V, NB, A_BYTES>(smem + (buf ^ 1) * (A_BYTES + B_BYTES), blk, tid);
      __syncthreads();
    }
    gemm_compute<T, WM_SUB, WN_SUB>(smem + ((nk - 1) & 1) * (A_BYTES + B_BYTES), a_frag, b_frag,
                                    acc);
  }

  float* cg = p.c + grp * p.c_group_stride;
  float* cg2 = p.c2 ? p.c2 + grp * p.c_group_stride : nullptr;
#pragma unroll
  for (int i = 0; i < WM_SUB; ++i) {
    const int64_t m = mt * BM + wm * WM_SUB * 32 + i * 32 + r32;
#pragma unroll
    for (int j = 0; j < WN_SUB; ++j) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int n = nt * BN + wn * WN_SUB * 32 + j * 32 + 8 * rr + 4 * g;
        float* dst = n < p.nsplit ? cg + m * p.ldc + n : cg2 + m * p.ldc + (n - p.nsplit);
        *reinterpret_cast<float4*>(dst) = make_float4(acc[i][j][4 * rr + 0], acc[i][j][4 * rr + 1],
                                                      acc[i][j][4 * rr + 2], acc[i][j][4 * rr + 3]);
      }
    }
  }
}

// Grid size for a GEMM over `row_tiles` row tiles (upper bound in grouped mode).
template <typename Cfg>
inline dim3 gemm_grid(int64_t row_tiles, int N) {
  return dim3(static_cast<unsigned>(row_tiles * (N / Cfg::BN)));
}

}  // namespace moe
