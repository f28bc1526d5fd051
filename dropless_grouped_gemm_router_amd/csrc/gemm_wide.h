// Wide-tile grouped GEMM for bf16 on gfx950: 256 x 256 output tiles.
//
//   C[rows of a tile, n] = sum_k A[row, k] * B[group][n, k]
//
// Same operands, work list, epilogues and argument block as gemm_kernel
// (gemm_core.h); this variant is the one sized for the chip:
//
//  * 512 threads = 8 waves as 4 (rows) x 2 (columns); each wave owns a
//    64 x 128 block of 2 x 4 MFMA 32x32x16 tiles, i.e. 42.7 flops per byte
//    of fragment read from LDS (a 64 x 64 wave block gives 32, which is at
//    the LDS read rate of a CU at full MFMA issue).
//  * The workgroup tile reads 128 flops per byte from L2, twice a 128 x 128
//    tile, which is what keeps the L2-to-CU path off the critical path.
//  * K stages of 64 elements (128 bytes per row) go from global memory
//    straight into LDS with global_load_lds_dwordx4: no staging registers
//    and no LDS store instructions. Two 64 KiB stage buffers, so a stage is
//    in flight while the previous one is multiplied out; the first stage of
//    the next work item is issued while the current item's last stage is
//    multiplied out, so its load overlaps that stage and the epilogue.
//  * A direct-to-LDS load writes 64 consecutive 16-byte pieces, so rows
//    cannot be padded; instead the 16-byte chunk c of LDS row r sits at
//    position c ^ ((r >> 1) & 7) of the row, which spreads the 32 rows one
//    fragment read touches over all banks.
#pragma once

#include "gemm_core.h"

namespace moe {

struct WideCfg {
  static constexpr int BM = 256, BN = 256;
  static constexpr int WAVES_M = 4, WAVES_N = 2;
  static constexpr int WM_SUB = 2, WN_SUB = 4;  // 32 x 32 MFMA tiles per wave
  static constexpr int NT = 512;
};

constexpr int kWideRowBytes = 128;                   // K bytes per row per stage
constexpr int kWideStage = 512 * kWideRowBytes;      // A rows 0..255, B rows 256..511
constexpr int kWideLoads = 4;                        // A (and B) loads per lane per stage

// Byte offset of 16-byte chunk c of LDS row r within a stage buffer.
__device__ __forceinline__ int wide_swizzle(int r, int c) {
  return r * kWideRowBytes + ((c ^ ((r >> 1) & 7)) << 4);
}

// Wait for this wave's outstanding vector-memory operations (the
// direct-to-LDS loads count there) and LDS reads.
__device__ __forceinline__ void wide_wait_all() {
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0x0 << 8));
}

// Every wave's loads for a stage have landed once each wave has waited for
// its own and passed this barrier. The asm form carries no memory fence (a
// fence would make the compiler wait for every outstanding load, including
// the next stage's) and its clobber keeps LDS accesses on their side.
__device__ __forceinline__ void wide_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Issue one K stage into an LDS buffer. Load i of lane l in wave w covers
// tile row r = (4 w + i) * 8 + l / 8, 16-byte position l % 8 of LDS row r
// (and of row 256 + r for B); the lane's global addresses already point at
// the chunk that belongs at that position.
// With with_b false only the A rows are loaded: the B rows of the stage
// are already in the buffer (the same weights as the previous item's).
__device__ __forceinline__ void wide_issue(char* buf, const char* const (&a_row)[kWideLoads],
                                           const char* b_base, const int (&b_off)[2],
                                           int64_t b_step, int koff, int wave,
                                           bool with_b = true) {
#pragma unroll
  for (int i = 0; i < kWideLoads; ++i)
    __builtin_amdgcn_global_load_lds(a_row[i] + koff, buf + (wave * kWideLoads + i) * 1024, 16, 0,
                                     0);
  if (!with_b) return;
#pragma unroll
  for (int i = 0; i < kWideLoads; ++i)
    __builtin_amdgcn_global_load_lds(b_base + koff + b_off[i & 1] + i * b_step,
                                     buf + 256 * kWideRowBytes + (wave * kWideLoads + i) * 1024,
                                     16, 0, 0);
}

// Multiply one stage out of LDS: four 16-element K steps. K step q reads
// chunk 2q + g of its rows at position (2q + g) ^ ((r32 >> 1) & 7), i.e.
// 2q ^ sw_base with sw_base = g ^ ((r32 >> 1) & 7); the positions are formed
// per call (an opaque copy of the base) instead of held in registers.
__device__ __forceinline__ void wide_compute(const char* buf, int a_frag, int b_frag, int sw_base,
                                             f32x16_t (&acc)[WideCfg::WM_SUB][WideCfg::WN_SUB]) {
  int sb = sw_base;
  asm volatile("" : "+v"(sb));
  int sw[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) sw[q] = ((2 * q) ^ sb) << 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    u32x4 xf[WideCfg::WM_SUB], wf[WideCfg::WN_SUB];
#pragma unroll
    for (int i = 0; i < WideCfg::WM_SUB; ++i)
      xf[i] = *reinterpret_cast<const u32x4*>(buf + a_frag + i * 32 * kWideRowBytes + sw[q]);
#pragma unroll
    for (int j = 0; j < WideCfg::WN_SUB; ++j)
      wf[j] = *reinterpret_cast<const u32x4*>(buf + b_frag + j * 32 * kWideRowBytes + sw[q]);
#pragma unroll
    for (int i = 0; i < WideCfg::WM_SUB; ++i)
#pragma unroll
      for (int j = 0; j < WideCfg::WN_SUB; ++j) Mfma<bf16_t>::step(wf[j], xf[i], acc[i][j]);
  }
}

// Row indices behind the A loads of this lane for a work item, as read
// (rows past the tile's end repeat its last row; their results are never
// stored). In gather mode this is the flat slot; the token is slot / top_k,
// taken only when the addresses are formed, so that the load's wait lands
// where the stage loads are waited for anyway.
template <bool kGather>
__device__ __forceinline__ void wide_src_rows(const GemmArgs& p, const TileInfo& t, int lrow,
                                              int (&src)[kWideLoads]) {
#pragma unroll
  for (int i = 0; i < kWideLoads; ++i) {
    // An empty item (t.rows == 0, t.row0 == 0) reads slot 0, which exists
    // whenever the kernel runs; the load is unconditional so that no branch
    // writes its destination register while an older load may target it.
    const int mr = max(0, min(lrow + 8 * i, t.rows - 1));
    src[i] = kGather ? p.perm[t.row0 + mr] : t.row0 + mr;
  }
}

template <bool kGather>
__device__ __forceinline__ void wide_a_rows(const GemmArgs& p, const int (&src)[kWideLoads],
                                            const int (&chunk_off)[2],
                                            const char* (&a_row)[kWideLoads]) {
  const int64_t a_row_bytes = p.lda * 2;
#pragma unroll
  for (int i = 0; i < kWideLoads; ++i) {
    const int r = kGather ? src[i] / p.topk : src[i];
    a_row[i] = static_cast<const char*>(p.a) + r * a_row_bytes + chunk_off[i & 1];
  }
}

// Weight base of a work item (and of its second part, offset so that stage
// s of either reads at s * 128 bytes).
__device__ __forceinline__ void wide_b_bases(const GemmArgs& p, const TileInfo& t, int nt,
                                             int64_t ldb, const char*& b1, const char*& b2) {
  b1 = static_cast<const char*>(p.b) +
       (static_cast<int64_t>(t.group) * p.b_group_stride + static_cast<int64_t>(nt) * 256 * ldb) * 2;
  b2 = p.b2 ? static_cast<const char*>(p.b2) +
                  (static_cast<int64_t>(t.group) * p.b2_group_stride +
                   static_cast<int64_t>(nt) * 256 * ldb - p.ksplit) * 2
            : b1;
}

// Epilogue through LDS. Stored straight from the accumulators, each store
// instruction would touch 32 rows with 8 bytes each; instead each wave
// writes its results as a 64-row x 128-byte block into a private 8 KiB LDS
// region and stores it back as whole 128-byte row pieces (64 lanes x 16
// bytes = 8 rows per instruction). Chunk c of region row r sits at position
// c ^ (r & 7), so the accumulator-layout writes spread over the banks.
// The park writes and the drain's reads are inline assembly: the compiler
// takes any plain LDS access as possibly aliasing the next item's first
// stage, which is in flight by direct-to-LDS loads, and would wait for all
// of it first. (The region is the other stage buffer; the next item's first
// wait covers those loads.)
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ void wide_park(char* region, int row, int byte, float v0, float v1,
                                          float v2, float v3) {
  const int pos = (((byte >> 4) ^ (row & 7)) << 4) | (byte & 15);
  const uint64_t d = static_cast<uint64_t>(pack_bf16x2(v0, v1)) |
                     (static_cast<uint64_t>(pack_bf16x2(v2, v3)) << 32);
  asm volatile("ds_write_b64 %0, %1" : : "v"(lds_addr(region + row * 128 + pos)), "v"(d) : "memory");
}

// A 16-byte row piece, as a nontemporal store when kNT. The SwiGLU outputs
// (H, and the pre-activations a training forward saves) are written that
// way: they are read back only by later kernels, and kept out of L2 they
// leave it to the token rows and weights the GEMM re-reads (the shared
// gate/up GEMM at 131072 tokens reads 1.06x its algorithmic bytes past L2
// instead of 1.63x; forward at 131072 tokens, E=64, top-8: 1.376 -> 1.354
// ms median, same bits). The
// plain-store epilogues measured the same or slower with it (the routed
// down GEMM's y_sorted stores 0.251 -> 0.267 ms).
template <bool kNT>
__device__ __forceinline__ void wide_store16(bf16_t* dst, const u32x4& v) {
  if (kNT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
  else *reinterpret_cast<u32x4*>(dst) = v;
}

// Writes the parked block: region row r goes to dst + r * ld (elements),
// 64 bf16 columns, for rows r < rows; rows may be 0 or negative (a wave
// block past the tile's end), with dst + (rows - 1) * ld then the tile's
// last row. Every lane issues exactly eight stores: a row r >= rows was
// computed from a repeat of the tile's last row (wide_src_rows), so its
// values are that row's, bit for bit, and it is written over that row.
// The fixed store count lets the next item's first wait leave these
// stores in flight (wide_wait_stores).
template <bool kNT>
__device__ __forceinline__ void wide_drain(const char* region, bf16_t* dst, int64_t ld, int rows,
                                           int lane) {
  // All eight LDS reads first (always in bounds), then the stores.
  const int c = lane & 7;
  uint32_t ad[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = k * 8 + (lane >> 3);
    ad[k] = lds_addr(region + r * 128 + ((c ^ (r & 7)) << 4));
  }
  u32x4 v[8];
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\t"
      "ds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
        "v"(ad[7])
      : "memory");
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = k * 8 + (lane >> 3);
    wide_store16<kNT>(dst + min(r, rows - 1) * ld + c * 8, v[k]);
  }
}

// wide_drain for a 32-row block (region rows 0..31, four stores per lane;
// rows >= rows are written over the tile's last row as in wide_drain).
__device__ __forceinline__ void wide_drain32(const char* region, bf16_t* dst, int64_t ld, int rows,
                                             int lane) {
  const int c = lane & 7;
  uint32_t ad[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = k * 8 + (lane >> 3);
    ad[k] = lds_addr(region + r * 128 + ((c ^ (r & 7)) << 4));
  }
  u32x4 v[4];
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
      : "memory");
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = k * 8 + (lane >> 3);
    wide_store16<false>(dst + min(r, rows - 1) * ld + c * 8, v[k]);
  }
}

// Global stores a wave's epilogue issues per item through wide_drain (8
// per call), or 0 where the epilogue's store count varies (the gather-sum
// and SwiGLU-backward drains skip rows past the tile's end).
template <int kEpi>
__device__ __forceinline__ int wide_epilogue_stores(const GemmArgs& p) {
  return (kEpi == kEpiStore || kEpi == kEpiStoreRouter) ? 16 : (kEpi == kEpiSwiglu ? (p.sa ? 24 : 8) : 0);
}

// First wait of an item whose predecessor's epilogue issued n stores after
// this item's first stage loads. vmcnt counts a wave's loads and stores in
// issue order, so vmcnt(n) sees those loads land and leaves the stores in
// flight during the first stage; lgkmcnt(0) as in wide_wait_all.
__device__ __forceinline__ void wide_wait_stores(int n) {
  if (n == 8) __builtin_amdgcn_s_waitcnt(8 | (0x7 << 4));
  else if (n == 16) __builtin_amdgcn_s_waitcnt(0 | (1 << 14) | (0x7 << 4));
  else if (n == 24) __builtin_amdgcn_s_waitcnt(8 | (1 << 14) | (0x7 << 4));
  else wide_wait_all();
}

// Fused gather-sum drain (kEpiCombine, dense rows = tokens): region row r
// holds token orow + r's dense results, already rounded to bf16; the
// wave's comb area holds each row's sorted rows ([64][k] int32) and weights
// ([64][k] fp32 at byte 2048). Each 16-byte output piece is the combine
// stage's sum, in its order: fp32 multiply-adds over ranks 0..k-1 from zero,
// then the dense value; rows of -1 (dropped by capacity routing) are left
// out. All k row loads of a piece are issued before use.
__device__ __forceinline__ void wide_drain_combine(const GemmArgs& p, const char* region,
                                                   const char* comb, int64_t orow, int col,
                                                   int rows, int lane) {
  const bf16_t* y = static_cast<const bf16_t*>(p.gy);
  bf16_t* out = static_cast<bf16_t*>(p.c);
  const int32_t* cidx = reinterpret_cast<const int32_t*>(comb);
  const float* cw = reinterpret_cast<const float*>(comb + 2048);
  const int K = p.gk;
#pragma unroll 1
  for (int k = 0; k < 8; ++k) {
    const int r = k * 8 + (lane >> 3), c = lane & 7;
    if (r >= rows) break;
    const u32x4 sv = *reinterpret_cast<const u32x4*>(region + r * 128 + ((c ^ (r & 7)) << 4));
    int idx[kCombineMaxK];
    float wt[kCombineMaxK];
#pragma unroll
    for (int i = 0; i < kCombineMaxK; ++i) {
      idx[i] = i < K ? cidx[r * K + i] : 0;
      wt[i] = i < K ? cw[r * K + i] : 0.0f;
    }
    u32x4 yv[kCombineMaxK];
#pragma unroll
    for (int i = 0; i < kCombineMaxK; ++i)
      if (i < K && idx[i] >= 0)
        yv[i] = *reinterpret_cast<const u32x4*>(y + static_cast<int64_t>(idx[i]) * p.ldc + col + c * 8);
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < kCombineMaxK; ++i)
      if (i < K && idx[i] >= 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = __builtin_fmaf(wt[i], bf16lo(yv[i][q]), acc[2 * q]);
          acc[2 * q + 1] = __builtin_fmaf(wt[i], bf16hi(yv[i][q]), acc[2 * q + 1]);
        }
      }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = pack_bf16x2(acc[2 * q] + bf16lo(sv[q]), acc[2 * q + 1] + bf16hi(sv[q]));
    *reinterpret_cast<u32x4*>(out + (orow + r) * p.ldc + col + c * 8) = o;
  }
}

// SwiGLU backward through LDS: region row r holds 32 fp32 values of dH
// (16-byte chunk c at c ^ (r & 7)); lane l takes rows l / 8 + 8 k and the
// four columns 4 (l % 8) of the pass, so eight lanes load the saved gate and
// up values and store dA and dB as 64 contiguous bytes of a row. The same
// formulas as the accumulator-layout epilogue.
__device__ __forceinline__ void wide_drain_swiglu_bwd(const GemmArgs& p, const char* region,
                                                      int64_t orow, int col, int rows, int lane) {
  const bf16_t* sa = static_cast<const bf16_t*>(p.sa);
  const bf16_t* sb = static_cast<const bf16_t*>(p.sb);
  bf16_t* c = static_cast<bf16_t*>(p.c);
  const int ch = lane & 7;
  const int n = col + 4 * ch;
#pragma unroll 2
  for (int k = 0; k < 8; ++k) {
    const int r = k * 8 + (lane >> 3);
    if (r >= rows) break;
    const float4 dh = *reinterpret_cast<const float4*>(region + r * 128 + ((ch ^ (r & 7)) << 4));
    float a[4], b[4];
    load4(sa + (orow + r) * p.lds + n, a);
    load4(sb + (orow + r) * p.lds + n, b);
    const float dv[4] = {dh.x, dh.y, dh.z, dh.w};
    float da[4], db[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float sg = sigmoid_f(a[q]);
      da[q] = dv[q] * b[q] * sg * (1.0f + a[q] * (1.0f - sg));
      db[q] = dv[q] * a[q] * sg;
    }
    store4(c + (orow + r) * p.ldc + n, da[0], da[1], da[2], da[3]);
    store4(c + (orow + r) * p.ldc + p.hsplit + n, db[0], db[1], db[2], db[3]);
  }
}

// Parks the wave's 64 x 64 block of SwiGLU results (kWhich 0), gate
// pre-activations (1) or up pre-activations (2). Packed columns j*32 +
// [0,16) are gate columns and j*32 + [16,32) the matching up columns, so
// registers 4rr + q (rr < 2) hold gate and 4(rr + 2) + q the up values of
// hidden column j*16 + 8rr + 4g + q of the block.
template <int kWhich>
__device__ __forceinline__ void wide_park_swiglu(
    const f32x16_t (&acc)[WideCfg::WM_SUB][WideCfg::WN_SUB], char* region, int g, int r32) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a = acc[i][j][4 * rr + q], b = acc[i][j][4 * (rr + 2) + q];
          v[q] = kWhich == 0 ? silu_f(a) * b : (kWhich == 1 ? a : b);
        }
        wide_park(region, i * 32 + r32, j * 32 + rr * 16 + g * 8, v[0], v[1], v[2], v[3]);
      }
}

// Wave epilogue of one wide tile for the plain store, the forward SwiGLU and
// the fused gather-sum (comb: the wave's 4 KiB index area, else unused).
// Accumulator register q of MFMA tile (i, j) holds row i*32 + r32 and
// column j*32 + 8*(q/4) + 4*g + q%4 of the wave's 64 x 128 block.
template <int kEpi>
__device__ __forceinline__ void wide_epilogue(const GemmArgs& p,
                                              const f32x16_t (&acc)[WideCfg::WM_SUB][WideCfg::WN_SUB],
                                              char* region, char* comb, int row0, int rows,
                                              int nt, int wm, int wn, int g, int r32, int lane,
                                              int group) {
  const int wrows = rows - wm * 64;  // rows of this wave's block that exist
  const int64_t orow = static_cast<int64_t>(row0) + wm * 64;
  bf16_t* c = static_cast<bf16_t*>(p.c);
  if (kEpi == kEpiCombine) {
    // Its drain reads the parked rows with plain LDS loads between its row
    // gathers; after this wait the compiler knows the next item's stage
    // loads have landed and keeps the gathers pipelined instead of waiting
    // for all of them before every LDS read.
    wide_wait_all();
    // The block's 64 tokens own 64 k consecutive entries of ginv and gw.
    const int K = p.gk;
    const int valid = (wrows < 64 ? (wrows > 0 ? wrows : 0) : 64) * K;
#pragma unroll
    for (int j = 0; j < kCombineMaxK; ++j) {
      const int e = lane + 64 * j;
      if (j < K && e < valid) {
        reinterpret_cast<int32_t*>(comb)[e] = p.ginv[orow * K + e];
        reinterpret_cast<float*>(comb + 2048)[e] = p.gw[orow * K + e];
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const f32x16_t& a = acc[i][2 * h + jj];
            wide_park(region, i * 32 + r32, jj * 64 + rr * 16 + g * 8, a[4 * rr], a[4 * rr + 1],
                      a[4 * rr + 2], a[4 * rr + 3]);
          }
      wide_drain_combine(p, region, comb, orow, nt * WideCfg::BN + wn * 128 + h * 64, wrows, lane);
    }
  } else if (kEpi == kEpiSwigluBwd) {
    // Four passes of 32 columns (MFMA tile j = h), dH parked as fp32.
#pragma unroll
    for (int h = 0; h < 4; ++h) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int row = i * 32 + r32, chunk = 2 * rr + g;
          *reinterpret_cast<float4*>(region + row * 128 + ((chunk ^ (row & 7)) << 4)) =
              make_float4(acc[i][h][4 * rr], acc[i][h][4 * rr + 1], acc[i][h][4 * rr + 2],
                          acc[i][h][4 * rr + 3]);
        }
      wide_drain_swiglu_bwd(p, region, orow, nt * WideCfg::BN + wn * 128 + h * 32, wrows, lane);
    }
  } else if (kEpi == kEpiStore || kEpi == kEpiStoreRouter) {
    // Four passes of 32 rows x 64 columns (MFMA tile row i, tiles j = 2h,
    // 2h + 1) through the first 4 KiB of the region: the wave's 4 KiB share
    // of the buffer's A half, so a stage buffer's B half survives the
    // epilogue (wide_gemm_kernel keeps the weights of K = 128 GEMMs).
    // kEpiStoreRouter first adds rdl[row] * rw[group][n] in fp32: the
    // lane's two row scales and its 64 columns of rw are loaded before any
    // store (a row past the tile's end takes the last row's scale, so it
    // still repeats that row's bits), so the next item's counted first wait
    // still leaves exactly the 16 stores in flight.
    float rs[2] = {0.0f, 0.0f};
    f32x4_t rwv[2][2][4];
    if (kEpi == kEpiStoreRouter) {
#pragma unroll
      for (int i = 0; i < 2; ++i) rs[i] = p.rdl[row0 + min(wm * 64 + i * 32 + r32, rows - 1)];
      const float* rwg = p.rw + static_cast<int64_t>(group) * p.N + nt * WideCfg::BN + wn * 128;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            rwv[h][jj][rr] = *reinterpret_cast<const f32x4_t*>(rwg + h * 64 + jj * 32 + rr * 8 + g * 4);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const f32x16_t& a = acc[i][2 * h + jj];
            float v[4] = {a[4 * rr], a[4 * rr + 1], a[4 * rr + 2], a[4 * rr + 3]};
            if (kEpi == kEpiStoreRouter) {
#pragma unroll
              for (int q = 0; q < 4; ++q) v[q] = __builtin_fmaf(rs[i], rwv[h][jj][rr][q], v[q]);
            }
            wide_park(region, r32, jj * 64 + rr * 16 + g * 8, v[0], v[1], v[2], v[3]);
          }
        const int col = nt * WideCfg::BN + wn * 128 + h * 64;
        wide_drain32(region, c + (orow + i * 32) * p.ldc + col, p.ldc, wrows - i * 32, lane);
      }
  } else {
    const int hcol = nt * (WideCfg::BN / 2) + wn * 64;
    wide_park_swiglu<0>(acc, region, g, r32);
    wide_drain<true>(region, c + orow * p.ldc + hcol, p.ldc, wrows, lane);
    if (p.sa) {
      wide_park_swiglu<1>(acc, region, g, r32);
      wide_drain<true>(region, static_cast<bf16_t*>(p.sa) + orow * p.lds + hcol, p.lds, wrows, lane);
      wide_park_swiglu<2>(acc, region, g, r32);
      wide_drain<true>(region, static_cast<bf16_t*>(p.sb) + orow * p.lds + hcol, p.lds, wrows, lane);
    }
  }
}

// Row tile of work item w. The tile list arrives as separate restrict
// arguments: nothing the kernel stores can alias it, so its reads compile to
// scalar loads, whose waits do not hold up the in-flight stage loads.
template <bool kDense>
__device__ __forceinline__ TileInfo wide_tile(const GemmArgs& p, const int32_t* __restrict__ tiles,
                                              const int32_t* __restrict__ num_tiles, int w,
                                              int n_tiles_n) {
  const int mt = w / n_tiles_n;
  TileInfo t{0, 0, 0};
  if (kDense) {
    t.row0 = mt * WideCfg::BM;
    const int64_t left = p.M - t.row0;
    t.rows = left <= 0 ? 0 : static_cast<int>(left < WideCfg::BM ? left : WideCfg::BM);
  } else if (mt < *num_tiles) {
    t.group = tiles[3 * mt + 0];
    t.row0 = tiles[3 * mt + 1];
    t.rows = tiles[3 * mt + 2];
  }
  return t;
}

// Persistent wide-tile GEMM (bf16). Work assignment as in gemm_kernel: the
// workgroups of XCD x walk its contiguous share of the (row tile, N tile)
// list, so one expert's tiles, and its weights, stay in one L2. `tiles` and
// `num_tiles` are p.tiles and p.num_tiles (unused in dense mode).
template <bool kGather, int kEpi, bool kDense>
__global__ __launch_bounds__(WideCfg::NT) __attribute__((amdgpu_waves_per_eu(2)))
void wide_gemm_kernel(const GemmArgs p, const int32_t* __restrict__ tiles,
                      const int32_t* __restrict__ num_tiles, int total_work) {
  // The fused gather-sum epilogue adds 4 KiB per wave for its rows' indices
  // and weights (160 KiB in all, the CU's LDS).
  __shared__ __attribute__((aligned(1024))) char smem[2 * kWideStage + (kEpi == kEpiCombine ? 8 * 4096 : 0)];
  const int n_tiles_n = p.N / WideCfg::BN;
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
  const int wm = wave / WideCfg::WAVES_N, wn = wave % WideCfg::WAVES_N;
  const int64_t ldb = p.ldb ? p.ldb : p.K;
  const int64_t b_step = 16 * ldb;  // 8 rows
  const int nk = p.K / 64;
  const int ks_split = p.b2 ? p.ksplit / 64 : (1 << 30);

  // Load side: lane's first row, and the chunk it fetches for even and odd
  // loads ((row >> 1) & 7 of row lrow + 8 i is (lane >> 4) + 4 (i & 1)).
  const int lrow = wave * kWideLoads * 8 + (lane >> 3);
  const int xr = lane >> 4;
  const int chunk_off[2] = {((lane & 7) ^ xr) * 16, ((lane & 7) ^ (xr + 4)) * 16};
  const int b_off[2] = {static_cast<int>(lrow * ldb * 2) + chunk_off[0],
                        static_cast<int>(lrow * ldb * 2) + chunk_off[1]};
  // Fragment side: rows wm * 64 + r32 (A) and 256 + wn * 128 + r32 (B), and
  // the swizzled position of K step q's chunk 2 q + g.
  const int a_frag = (wm * WideCfg::WM_SUB * 32 + r32) * kWideRowBytes;
  const int b_frag = (256 + wn * WideCfg::WN_SUB * 32 + r32) * kWideRowBytes;
  const int sw_base = g ^ ((r32 >> 1) & 7);

  TileInfo cur = wide_tile<kDense>(p, tiles, num_tiles, w, n_tiles_n);
  if (cur.rows <= 0) return;
  int src[kWideLoads];
  wide_src_rows<kGather>(p, cur, lrow, src);
  const char* a_cur[kWideLoads];
  wide_a_rows<kGather>(p, src, chunk_off, a_cur);
  const char *b1_cur, *b2_cur;
  wide_b_bases(p, cur, w % n_tiles_n, ldb, b1_cur, b2_cur);

  int buf = 0;
  wide_issue(smem, a_cur, b1_cur, b_off, b_step, 0, wave);
  int stores_out = 0;  // stores the previous item's epilogue left in flight
  // K = 128 plain-store GEMMs (the routed down projection): each stage
  // always lands in the same buffer, so when the next item has the same
  // weights (same group and N tile, as a workgroup's consecutive items
  // mostly do) only its A rows are loaded; the epilogue parks in the A half.
  const bool keep_b = kEpi == kEpiStore && nk == 2 && p.b2 == nullptr;
  bool b_same = false;       // this item's B rows are already in the buffers
  bool b_same_next = false;  // the same for the next item

  while (true) {
    const int nt = w % n_tiles_n;
    const int w1 = w + gx;
    TileInfo nxt{0, 0, 0};

    f32x16_t acc[WideCfg::WM_SUB][WideCfg::WN_SUB];
#pragma unroll
    for (int i = 0; i < WideCfg::WM_SUB; ++i)
#pragma unroll
      for (int j = 0; j < WideCfg::WN_SUB; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    for (int s = 0; s < nk; ++s) {
      if (s == 0) wide_wait_stores(stores_out);
      else wide_wait_all();
      wide_barrier();
      char* nb = smem + (buf ^ 1) * kWideStage;
      // The next item's metadata and row indices are read during this
      // item's first stage (before its issue only when there is one stage).
      if (s == 0 && nk == 1) {
        nxt = (w1 < w_end) ? wide_tile<kDense>(p, tiles, num_tiles, w1, n_tiles_n) : TileInfo{0, 0, 0};
        wide_src_rows<kGather>(p, nxt, lrow, src);
      }
      if (s + 1 < nk) {
        wide_issue(nb, a_cur, (s + 1) < ks_split ? b1_cur : b2_cur, b_off, b_step, (s + 1) * 128,
                   wave, !b_same);
      } else if (nxt.rows > 0) {
        b_same_next = keep_b && nxt.group == cur.group && w1 % n_tiles_n == nt;
        wide_a_rows<kGather>(p, src, chunk_off, a_cur);
        wide_b_bases(p, nxt, w1 % n_tiles_n, ldb, b1_cur, b2_cur);
        wide_issue(nb, a_cur, b1_cur, b_off, b_step, 0, wave, !b_same_next);
      }
      if (s == 0 && nk > 1) {
        nxt = (w1 < w_end) ? wide_tile<kDense>(p, tiles, num_tiles, w1, n_tiles_n) : TileInfo{0, 0, 0};
        wide_src_rows<kGather>(p, nxt, lrow, src);
      }
      wide_compute(smem + buf * kWideStage, a_frag, b_frag, sw_base, acc);
      buf ^= 1;
    }

    // Every epilogue goes through LDS, whole 128-byte row pieces per store
    // (for the SwiGLU output alone too: 8-byte stores straight from the
    // accumulators touch 32 rows per instruction and were 3-4 % slower).
    // The buffer of the last stage is free once every wave is done with it
    // (the other one is receiving the next item's first stage).
    wide_barrier();
    wide_epilogue<kEpi>(p, acc,
                        smem + (buf ^ 1) * kWideStage +
                            wave * ((kEpi == kEpiStore || kEpi == kEpiStoreRouter) ? 4096 : 8192),
                        kEpi == kEpiCombine ? smem + 2 * kWideStage + wave * 4096 : nullptr,
                        cur.row0, cur.rows, nt, wm, wn, g, r32, lane, cur.group);
    stores_out = wide_epilogue_stores<kEpi>(p);

    if (nxt.rows <= 0) break;
    w = w1;
    cur = nxt;
    b_same = b_same_next;
  }
}

}  // namespace moe
