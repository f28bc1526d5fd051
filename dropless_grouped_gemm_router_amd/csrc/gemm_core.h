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
  kEpiSwigluBwd = 2  // acc = dH[row][j]; with saved gate a and up b:
                     // c[row][j] = dH b SiLU'(a), c[row][h + j] = dH SiLU(a)
};

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
};

template <int BM_, int WAVES_M_, int WAVES_N_, int WM_SUB_, int WN_SUB_>
struct TileCfg {
  static constexpr int BM = BM_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int WM_SUB = WM_SUB_, WN_SUB = WN_SUB_;
  static constexpr int BN = WAVES_N * WN_SUB * 32;
  static_assert(WAVES_M * WAVES_N == 4, "four waves");
  static_assert(WAVES_M * WM_SUB * 32 == BM, "rows");
};
using Cfg128 = TileCfg<128, 2, 2, 2, 2>;  // BN 128
using Cfg64 = TileCfg<64, 2, 2, 1, 2>;    // BN 128
using Cfg32 = TileCfg<32, 1, 4, 1, 1>;    // BN 128

constexpr int kStageBytes = 128;   // K bytes per row per stage
constexpr int kLdsRowBytes = 144;  // + 16 bytes padding

template <typename T>
struct Mfma;
template <>
struct Mfma<bf16_t> {
  // One 16-byte chunk per lane group: 32x32x16.
  __device__ static void step(const uint4& w, const uint4& x, f32x16_t& acc) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w),
                                                  __builtin_bit_cast(bf16x8_t, x), acc, 0, 0, 0);
  }
};
template <>
struct Mfma<float> {
  // One 16-byte chunk per lane group = 4 k values: four 32x32x2 steps, step s
  // taking element s of each lane group's chunk (the same k on both sides).
  __device__ static void step(const uint4& w, const uint4& x, f32x16_t& acc) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(w.x), __uint_as_float(x.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(w.y), __uint_as_float(x.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(w.z), __uint_as_float(x.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(w.w), __uint_as_float(x.w), acc, 0, 0, 0);
  }
};

// Pipeline pieces of the GEMM main loop (force-inlined so that the staging
// registers stay in VGPRs).
template <int A_CH, int B_CH>
__device__ __forceinline__ void gemm_gload(uint4 (&ra)[A_CH], uint4 (&rb)[B_CH],
                                           const char* const (&a_src)[A_CH], const char* b_base,
                                           const int (&b_off)[B_CH], int off) {
#pragma unroll
  for (int i = 0; i < A_CH; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + off);
#pragma unroll
  for (int i = 0; i < B_CH; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_base + b_off[i] + off);
}

template <int A_CH, int B_CH>
__device__ __forceinline__ void gemm_lstore(char* s, const uint4 (&ra)[A_CH],
                                            const uint4 (&rb)[B_CH], const int (&a_dst)[A_CH],
                                            const int (&b_dst)[B_CH]) {
#pragma unroll
  for (int i = 0; i < A_CH; ++i) *reinterpret_cast<uint4*>(s + a_dst[i]) = ra[i];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) *reinterpret_cast<uint4*>(s + b_dst[i]) = rb[i];
}

// One K stage out of LDS: four fragment steps of 32 bytes per row.
template <typename T, int WM_SUB, int WN_SUB>
__device__ __forceinline__ void gemm_compute(const char* s, int a_frag, int b_frag,
                                             f32x16_t (&acc)[WM_SUB][WN_SUB]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint4 xf[WM_SUB], wf[WN_SUB];
#pragma unroll
    for (int i = 0; i < WM_SUB; ++i)
      xf[i] = *reinterpret_cast<const uint4*>(s + a_frag + i * 32 * kLdsRowBytes + q * 32);
#pragma unroll
    for (int j = 0; j < WN_SUB; ++j)
      wf[j] = *reinterpret_cast<const uint4*>(s + b_frag + j * 32 * kLdsRowBytes + q * 32);
#pragma unroll
    for (int i = 0; i < WM_SUB; ++i)
#pragma unroll
      for (int j = 0; j < WN_SUB; ++j) Mfma<T>::step(wf[j], xf[i], acc[i][j]);
  }
}

template <typename T, typename Cfg, bool kGather, int kEpi, bool kDense>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const GemmArgs p) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN;
  constexpr int WM_SUB = Cfg::WM_SUB, WN_SUB = Cfg::WN_SUB;
  constexpr int A_CH = BM * 8 / 256;  // 16-byte chunks per thread per stage
  constexpr int B_CH = BN * 8 / 256;
  constexpr int KT = kStageBytes / static_cast<int>(sizeof(T));
  constexpr int A_BYTES = BM * kLdsRowBytes, B_BYTES = BN * kLdsRowBytes;
  __shared__ __attribute__((aligned(16))) char smem[2 * (A_BYTES + B_BYTES)];

  const int n_tiles_n = p.N / BN;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = logical / n_tiles_n, nt = logical % n_tiles_n;
  int group, row0, rows;
  if (kDense) {
    group = 0;
    row0 = mt * BM;
    if (row0 >= p.M) return;
    rows = static_cast<int>(min(static_cast<int64_t>(BM), p.M - row0));
  } else {
    if (mt >= *p.num_tiles) return;
    group = p.tiles[3 * mt + 0];
    row0 = p.tiles[3 * mt + 1];
    rows = p.tiles[3 * mt + 2];
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;

  // Global source of each chunk this thread stages (rows past the tile's end
  // re-read its last row; their results are never stored).
  const char* a_src[A_CH];
  int a_dst[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + i * 256;
    const int r = c >> 3, c16 = c & 7;
    const int mr = min(r, rows - 1);
    int64_t src_row;
    if (kGather) src_row = p.perm[row0 + mr] / p.topk;
    else src_row = static_cast<int64_t>(row0) + mr;
    a_src[i] = static_cast<const char*>(p.a) + (src_row * p.lda) * static_cast<int64_t>(sizeof(T)) + c16 * 16;
    a_dst[i] = r * kLdsRowBytes + c16 * 16;
  }
  const int64_t ldb = p.ldb ? p.ldb : p.K;
  const char* b_base = static_cast<const char*>(p.b) +
                       (static_cast<int64_t>(group) * p.b_group_stride +
                        static_cast<int64_t>(nt) * BN * ldb) * static_cast<int64_t>(sizeof(T));
  const char* b2_base = p.b2 ? static_cast<const char*>(p.b2) +
                                   (static_cast<int64_t>(group) * p.b2_group_stride +
                                    static_cast<int64_t>(nt) * BN * ldb -
                                    static_cast<int64_t>(p.ksplit)) * static_cast<int64_t>(sizeof(T))
                             : nullptr;
  const int ks_split = p.b2 ? p.ksplit / KT : (1 << 30);  // first stage read from b2
  int b_off[B_CH];
  int b_dst[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + i * 256;
    const int r = c >> 3, c16 = c & 7;
    b_off[i] = static_cast<int>(r * ldb * static_cast<int64_t>(sizeof(T))) + c16 * 16;
    b_dst[i] = A_BYTES + r * kLdsRowBytes + c16 * 16;
  }

  f32x16_t acc[WM_SUB][WN_SUB];
#pragma unroll
  for (int i = 0; i < WM_SUB; ++i)
#pragma unroll
    for (int j = 0; j < WN_SUB; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  const int nk = p.K / KT;
  const int a_frag = (wm * WM_SUB * 32 + r32) * kLdsRowBytes + g * 16;
  const int b_frag = A_BYTES + (wn * WN_SUB * 32 + r32) * kLdsRowBytes + g * 16;
  uint4 ra[A_CH], rb[B_CH];
  gemm_gload<A_CH, B_CH>(ra, rb, a_src, b_base, b_off, 0);
  gemm_lstore<A_CH, B_CH>(smem, ra, rb, a_dst, b_dst);
  __syncthreads();
  // Software pipeline: stage ks+1 is fetched into registers while stage ks
  // is multiplied out of LDS; the last stage is peeled.
  for (int ks = 0; ks + 1 < nk; ++ks) {
    const int buf = ks & 1;
    gemm_gload<A_CH, B_CH>(ra, rb, a_src, ks + 1 < ks_split ? b_base : b2_base, b_off,
                           (ks + 1) * kStageBytes);
    gemm_compute<T, WM_SUB, WN_SUB>(smem + buf * (A_BYTES + B_BYTES), a_frag, b_frag, acc);
    gemm_lstore<A_CH, B_CH>(smem + (buf ^ 1) * (A_BYTES + B_BYTES), ra, rb, a_dst, b_dst);
    __syncthreads();
  }
  gemm_compute<T, WM_SUB, WN_SUB>(smem + ((nk - 1) & 1) * (A_BYTES + B_BYTES), a_frag, b_frag, acc);

  // Epilogue. Accumulator register q of MFMA tile (i, j) holds row
  // m = i*32 + r32 and column n = j*32 + 8*(q/4) + 4*g + q%4 of the wave's
  // sub-block.
  T* c = static_cast<T*>(p.c);
#pragma unroll
  for (int i = 0; i < WM_SUB; ++i) {
    const int m = wm * WM_SUB * 32 + i * 32 + r32;
    if (m >= rows) continue;
    const int64_t orow = static_cast<int64_t>(row0) + m;
#pragma unroll
    for (int j = 0; j < WN_SUB; ++j) {
      const int n0 = nt * BN + wn * WN_SUB * 32 + j * 32;
      if (kEpi == kEpiStore) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int n = n0 + 8 * rr + 4 * g;
          store4(c + orow * p.ldc + n, acc[i][j][4 * rr + 0], acc[i][j][4 * rr + 1],
                 acc[i][j][4 * rr + 2], acc[i][j][4 * rr + 3]);
        }
      } else if (kEpi == kEpiSwigluBwd) {
        const T* sa = static_cast<const T*>(p.sa);
        const T* sb = static_cast<const T*>(p.sb);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int n = n0 + 8 * rr + 4 * g;
          float a[4], b[4], da[4], db[4];
          load4(sa + orow * p.lds + n, a);
          load4(sb + orow * p.lds + n, b);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float dh = acc[i][j][4 * rr + q];
            const float sg = sigmoid_f(a[q]);
            da[q] = dh * b[q] * sg * (1.0f + a[q] * (1.0f - sg));
            db[q] = dh * a[q] * sg;
          }
          store4(c + orow * p.ldc + n, da[0], da[1], da[2], da[3]);
          store4(c + orow * p.ldc + p.hsplit + n, db[0], db[1], db[2], db[3]);
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
  int64_t rows_total;          // dense mode
  int splits;                  // dense mode
  float* c;
  float* c2;       // columns n >= nsplit go to c2 (column n - nsplit)
  int nsplit;
  int64_t ldc;
  int64_t c_group_stride;
};

template <typename T>
struct Transpose;
template <>
struct Transpose<bf16_t> {
  static constexpr int V = 8;
  // out[c] = (in[0][c], in[1][c], ..., in[7][c])
  __device__ static void run(const uint4* in, uint4* out) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(in);  // w[4*r + c/2]
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = w[4 * (2 * q) + c / 2], hi = w[4 * (2 * q + 1) + c / 2];
        o[q] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      out[c] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
};
template <>
struct Transpose<float> {
  static constexpr int V = 4;
  __device__ static void run(const uint4* in, uint4* out) {
    out[0] = make_uint4(in[0].x, in[1].x, in[2].x, in[3].x);
    out[1] = make_uint4(in[0].y, in[1].y, in[2].y, in[3].y);
    out[2] = make_uint4(in[0].z, in[1].z, in[2].z, in[3].z);
    out[3] = make_uint4(in[0].w, in[1].w, in[2].w, in[3].w);
  }
};

// Stage loader of the weight-gradient kernel: thread `tid` fetches its
// V x V blocks of A (blocks 0 .. NB-1) and B (NB .. 2NB-1); rows outside
// [r0, r1) read as zeros.
template <typename T, bool kGatherA, int PER, int V, int NB, int KT>
__device__ __forceinline__ void wgrad_gload(const WgradArgs& p, uint4 (&blk)[PER][V], int64_t r0,
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
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r < r1) {
        const T* src;
        if (is_b) {
          src = static_cast<const T*>(p.b) + r * p.ldb + nt * 128 + cb * V;
        } else {
          const int64_t ar = kGatherA ? static_cast<int64_t>(p.perm[r] / p.topk) : r;
          src = static_cast<const T*>(p.a) + ar * p.lda + mt * 128 + cb * V;
        }
        v = *reinterpret_cast<const uint4*>(src);
      }
      blk[q][rr] = v;
    }
  }
}

// Transposes the fetched blocks into K-contiguous LDS rows.
template <typename T, int PER, int V, int NB, int A_BYTES>
__device__ __forceinline__ void wgrad_lstore(char* s, const uint4 (&blk)[PER][V], int tid) {
  constexpr int CB = 128 / V;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int b = tid + q * 256;
    const bool is_b = b >= NB;
    const int bb = is_b ? b - NB : b;
    const int rb = bb / CB, cb = bb % CB;
    uint4 t[V];
    Transpose<T>::run(blk[q], t);
    char* base = s + (is_b ? A_BYTES : 0) + rb * 16;
#pragma unroll
    for (int cc = 0; cc < V; ++cc) *reinterpret_cast<uint4*>(base + (cb * V + cc) * kLdsRowBytes) = t[cc];
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
  uint4 blk[PER][V];
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
