// Routed down-projection data gradient (bf16), with every other per-row
// quantity the backward needs from the expert's hidden layer, in one pass
// over the expert-sorted rows r (slot s = perm[r], token t = s / top_k,
// expert e, combine weight w_s):
//
//   dHu[r] = G[t] W_down[e]^T        (G = grad_out; K = d_model)
//   H[r]   = silu(A[r]) B[r]         (from the saved gate/up pre-activations)
//   dw[s]  = <dHu[r], H[r]>          (= <G[t], y[r]>, the gradient of w_s)
//   dH[r]  = w_s dHu[r] -> dA[r], dB[r] through SwiGLU
//   Hw[r]  = w_s H[r]                (dW_down[e] = sum_r Hw[r]^T G[t])
//
// (gpu_moe_h100.json header: value and gradient of the layer; the combine
// stage's backward follows from out[t] = sum_i w_i y[slot(t, i)].) Reading
// G by token, as the forward's gate/up GEMM reads x, leaves the per-slot
// upstream gradient w_s G[t] unmaterialised: the combine weight enters after
// the contraction, as the row scale of dH, and as the row scale of Hw for
// the down weight gradient, and dw comes from the same accumulators instead
// of a pass over the expert outputs.
//
// Tile: 256 sorted rows x 128 hidden columns, K = d_model in 64-deep stages
// loaded straight into LDS (the wide engine's row layout and swizzle: A
// rows 0..255, the 128 weight rows at 256..383, 48 KiB per stage). Three
// stage buffers with counted waits keep two stages in flight: a stage holds
// little MFMA work, so one stage in flight left the loop waiting a memory
// round trip per stage. Eight waves each own 32 rows x 128 columns (four
// 32x32x16 MFMA tiles), so a row's slice of dw is summed inside one wave.
// The epilogue's saved pre-activations are loaded before the tile's last
// stage is multiplied out, all 16 per lane at once; the epilogue parks each
// 32-column accumulator pass as fp32 in the wave's 4 KiB of the free stage
// buffer and reads it back as eight-column row pieces (four lanes per
// 64-byte run of a row), stores dA, dB and Hw as 16-byte pieces and keeps
// its piece of the dot product, summed over the row's four lanes at the
// end. d_hidden > 128 runs as 128-column slices, each writing its own dw
// part (summed in slice order by the router step). Persistent grid,
// XCD-aware item order as in the wide engine.
#pragma once

#include "gemm_wide.h"

namespace moe {

struct DgradArgs {
  const bf16_t* g;      // [tokens][d] upstream gradient of the layer output
  const int32_t* perm;  // sorted row -> flat slot
  int topk;
  const bf16_t* w;      // w_down [E][h][d]: row j = hidden unit, K = d contiguous
  const bf16_t* sab;    // saved [rows][2h]: gate pre-activations, then up
  const float* ws;      // [rows] combine weight of each sorted row's slot
  bf16_t* dab;          // [rows][2h] out: dA, then dB
  bf16_t* hw;           // [rows][h] out: w_s H
  float* dwp;           // [h / 128][rows] out: per-slice <dHu, H> by sorted row
  int64_t rows;         // tokens * top_k (dwp's slice stride)
  int d, h;
};

constexpr int kDgRows = 384;                       // LDS rows per stage (256 A + 128 B)
constexpr int kDgStage = kDgRows * kWideRowBytes;  // 48 KiB

// One K stage: lane l of wave w fetches A rows (4 w + i) * 8 + l / 8
// (i < 4) and weight rows (2 w + i) * 8 + l / 8 (i < 2), each the 16-byte
// chunk that belongs at position l % 8 of its swizzled LDS row.
__device__ __forceinline__ void dg_issue(char* buf, const char* const (&a_row)[4],
                                         const char* const (&b_row)[2], int koff, int wave) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_global_load_lds(a_row[i] + koff, buf + (wave * 4 + i) * 1024, 16, 0, 0);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    __builtin_amdgcn_global_load_lds(b_row[i] + koff,
                                     buf + 256 * kWideRowBytes + (wave * 2 + i) * 1024, 16, 0, 0);
}

// Multiply one stage out of LDS: four 16-deep K steps, one A fragment (the
// wave's 32 rows) against four weight fragments.
__device__ __forceinline__ void dg_compute(const char* buf, int a_frag, int b_frag, int sw_base,
                                           f32x16_t (&acc)[4]) {
  int sb = sw_base;
  asm volatile("" : "+v"(sb));
  int sw[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) sw[q] = ((2 * q) ^ sb) << 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 xf = *reinterpret_cast<const u32x4*>(buf + a_frag + sw[q]);
    u32x4 wf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      wf[j] = *reinterpret_cast<const u32x4*>(buf + b_frag + j * 32 * kWideRowBytes + sw[q]);
#pragma unroll
    for (int j = 0; j < 4; ++j) Mfma<bf16_t>::step(wf[j], xf, acc[j]);
  }
}

__device__ __forceinline__ TileInfo dg_tile(const int32_t* __restrict__ tiles,
                                            const int32_t* __restrict__ num_tiles, int w,
                                            int n_slices) {
  const int mt = w / n_slices;
  TileInfo t{0, 0, 0};
  if (mt < *num_tiles) {
    t.group = tiles[3 * mt + 0];
    t.row0 = tiles[3 * mt + 1];
    t.rows = tiles[3 * mt + 2];
  }
  return t;
}

// Flat slots behind this lane's A rows (rows past the tile's end repeat its
// last row; an empty item reads row 0, which exists whenever the kernel
// runs).
__device__ __forceinline__ void dg_src(const DgradArgs& p, const TileInfo& t, int lrow,
                                       int (&src)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) src[i] = p.perm[t.row0 + max(0, min(lrow + 8 * i, t.rows - 1))];
}

__device__ __forceinline__ void dg_rows(const DgradArgs& p, const TileInfo& t, int slice,
                                        const int (&src)[4], const int (&chunk_off)[2], int wave,
                                        int lane, const char* (&a_row)[4],
                                        const char* (&b_row)[2]) {
  const int64_t row_bytes = static_cast<int64_t>(p.d) * 2;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    a_row[i] = reinterpret_cast<const char*>(p.g) + (src[i] / p.topk) * row_bytes + chunk_off[i & 1];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t n = static_cast<int64_t>(t.group) * p.h + slice * 128 + wave * 16 + 8 * i + (lane >> 3);
    b_row[i] = reinterpret_cast<const char*>(p.w) + n * row_bytes + chunk_off[i];
  }
}

// s_waitcnt vmcnt(n) (n < 64) and lgkmcnt(0).
template <int N>
__device__ __forceinline__ void dg_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

constexpr int kDgBufs = 3;
constexpr int kDgLoads = 6;      // direct-to-LDS loads per lane per stage (dg_issue)
constexpr int kDgEpiLoads = 18;  // epilogue operand loads per lane (2 weights, 16 pieces)

// The next item's perm entries for this wave's 32 rows go to LDS by one
// direct-to-LDS load (lane l: row l % 32, entry at byte 4 l of the wave's
// 256-byte slot) and come back by inline-assembly LDS reads when the next
// item's first stage is issued: values carried in registers across
// iterations would make the compiler wait for every load in flight there.
__device__ __forceinline__ void dg_issue_idx(char* slot, const DgradArgs& p, const TileInfo& t,
                                             int wave, int lane) {
  const int r = max(0, min(wave * 32 + (lane & 31), t.rows - 1));
  __builtin_amdgcn_global_load_lds(p.perm + t.row0 + r, slot, 4, 0, 0);
}

__device__ __forceinline__ void dg_read_idx(uint32_t slot_lds, int lane, int (&src)[4]) {
  const uint32_t a0 = slot_lds + 4 * (lane >> 3);
  asm volatile(
      "ds_read_b32 %0, %4\n\t"
      "ds_read_b32 %1, %4 offset:32\n\t"
      "ds_read_b32 %2, %4 offset:64\n\t"
      "ds_read_b32 %3, %4 offset:96\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(src[0]), "=&v"(src[1]), "=&v"(src[2]), "=&v"(src[3])
      : "v"(a0)
      : "memory");
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void down_dgrad_kernel(const DgradArgs p, const int32_t* __restrict__ tiles,
                       const int32_t* __restrict__ num_tiles, int total_work) {
  __shared__ __attribute__((aligned(1024))) char smem[kDgBufs * kDgStage + 8 * 256];
  const int n_slices = p.h / 128;
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
  const int nk = p.d / 64;
  const int lrow = wave * 32 + (lane >> 3);
  const int xr = lane >> 4;
  const int chunk_off[2] = {((lane & 7) ^ xr) * 16, ((lane & 7) ^ (xr + 4)) * 16};
  const int a_frag = (wave * 32 + r32) * kWideRowBytes;
  const int b_frag = (256 + r32) * kWideRowBytes;
  const int sw_base = g ^ ((r32 >> 1) & 7);
  const int h2 = 2 * p.h;
  const int c4 = lane & 3;  // epilogue: 8-column piece of a 32-column pass
  char* idx_slot = smem + kDgBufs * kDgStage + wave * 256;
  const uint32_t idx_lds = lds_addr(idx_slot);

  TileInfo cur = dg_tile(tiles, num_tiles, w, n_slices);
  if (cur.rows <= 0) return;
  const char* a_row[4];
  const char* b_row[2];
  {
    int src[4];
    dg_src(p, cur, lrow, src);
    dg_rows(p, cur, w % n_slices, src, chunk_off, wave, lane, a_row, b_row);
  }

  // Stage q of the workgroup's sequence (items back to back) sits in buffer
  // q % 3; two stages are issued ahead.
  int w1 = w + gx;
  TileInfo nxt = (w1 < w_end) ? dg_tile(tiles, num_tiles, w1, n_slices) : TileInfo{0, 0, 0};
  bool idx_ready = false;  // the next item's perm entries have been requested
  // Stage i of the current item (i < nk), or stage i - nk of the next.
  auto issue = [&](int i, int q) {
    char* b = smem + (q % kDgBufs) * kDgStage;
    if (i < nk) {
      dg_issue(b, a_row, b_row, i * 128, wave);
      return true;
    }
    if (nxt.rows <= 0) return false;
    if (i == nk) {
      if (!idx_ready) {
        dg_issue_idx(idx_slot, p, nxt, wave, lane);
        idx_ready = true;
      }
      // The entries' load was issued before the previous stage's loads and
      // the counted wait covered it, except at d_model 128 (two stages),
      // where it was issued in this same iteration.
      if (nk == 2) wide_wait_all();
      int src[4];
      dg_read_idx(idx_lds, lane, src);
      dg_rows(p, nxt, w1 % n_slices, src, chunk_off, wave, lane, a_row, b_row);
    }
    dg_issue(b, a_row, b_row, (i - nk) * 128, wave);
    return true;
  };
  int gs = 0;      // global index of the stage being multiplied
  int issued = 1;  // stages issued so far
  issue(0, 0);
  if (issue(1, 1)) issued = 2;

  while (true) {
    const int slice = w % n_slices;
    f32x16_t acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[j][q] = 0.0f;

    // epilogue rows of this lane: wave rows kk * 16 + lane / 4 (kk < 2)
    int64_t srow[2];
    bool ok[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int tr = wave * 32 + kk * 16 + (lane >> 2);
      ok[kk] = tr < cur.rows;
      srow[kk] = cur.row0 + min(tr, cur.rows - 1);
    }
    u32x4 sa[2][4], sb[2][4];
    float ws[2];

    // One K stage: wait for stage gs, issue stage gs + 2 into the buffer
    // stage gs - 1 used, multiply stage gs out.
    auto stage = [&](int s) {
      // Stage gs has landed once at most the memory operations issued after
      // it remain (vmcnt retires a wave's loads and stores in issue order):
      // stage gs + 1's loads if it was issued; for an item's first stage
      // after an epilogue also the 18 operand loads of that epilogue (issued
      // unconditionally after stage gs + 1), so its stores stay in flight.
      if (issued <= gs + 1) wide_wait_all();
      else if (s == 0 && gs > 0) dg_wait_vm<kDgLoads + kDgEpiLoads>();
      else dg_wait_vm<kDgLoads>();
      wide_barrier();
      if (s == 0 && nxt.rows > 0 && !idx_ready) {
        // ahead of this iteration's stage loads, so the counted waits of
        // the following stages cover it
        dg_issue_idx(idx_slot, p, nxt, wave, lane);
        idx_ready = true;
      }
      if (issue(s + 2, gs + 2)) ++issued;
    };
    for (int s = 0; s < nk - 1; ++s) {
      stage(s);
      dg_compute(smem + (gs % kDgBufs) * kDgStage, a_frag, b_frag, sw_base, acc);
      ++gs;
    }
    // The last stage, outside the loop: the epilogue's operands are loaded
    // here, in flight while the stage is multiplied (inside the loop their
    // registers would look loop-carried, and the compiler would wait for
    // every load in flight before reusing them).
    stage(nk - 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      ws[kk] = p.ws[srow[kk]];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = slice * 128 + j * 32 + c4 * 8;
        sa[kk][j] = *reinterpret_cast<const u32x4*>(p.sab + srow[kk] * h2 + col);
        sb[kk][j] = *reinterpret_cast<const u32x4*>(p.sab + srow[kk] * h2 + p.h + col);
      }
    }
    dg_compute(smem + (gs % kDgBufs) * kDgStage, a_frag, b_frag, sw_base, acc);
    ++gs;

    // Epilogue in the buffer of the item's last stage, free once every wave
    // is past its compute (the other two receive the next item's stages).
    wide_barrier();
    char* region = smem + ((gs - 1) % kDgBufs) * kDgStage + wave * 4096;
    float dot[2] = {0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // Accumulator register q of tile j: row r32, column j*32 + 8*(q/4) +
      // 4*g + q%4 of the wave's block; chunk 2*(q/4) + g of the pass row.
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        *reinterpret_cast<float4*>(region + r32 * 128 + (((2 * rr + g) ^ (r32 & 7)) << 4)) =
            make_float4(acc[j][4 * rr], acc[j][4 * rr + 1], acc[j][4 * rr + 2], acc[j][4 * rr + 3]);
      const int col = slice * 128 + j * 32 + c4 * 8;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int r = kk * 16 + (lane >> 2);
        const float4 d0 =
            *reinterpret_cast<const float4*>(region + r * 128 + (((2 * c4) ^ (r & 7)) << 4));
        const float4 d1 =
            *reinterpret_cast<const float4*>(region + r * 128 + (((2 * c4 + 1) ^ (r & 7)) << 4));
        if (!ok[kk]) continue;
        const float du[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
        float a[8], b[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a[2 * q] = bf16lo(sa[kk][j][q]);
          a[2 * q + 1] = bf16hi(sa[kk][j][q]);
          b[2 * q] = bf16lo(sb[kk][j][q]);
          b[2 * q + 1] = bf16hi(sb[kk][j][q]);
        }
        float da[8], db[8], hw[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float sg = sigmoid_f(a[q]);
          const float si = a[q] * sg;
          const float hq = si * b[q];
          dot[kk] = __builtin_fmaf(du[q], hq, dot[kk]);
          const float dh = ws[kk] * du[q];
          da[q] = dh * b[q] * sg * (1.0f + a[q] * (1.0f - sg));
          db[q] = dh * si;
          hw[q] = ws[kk] * hq;
        }
        u32x4 oa, ob, oh;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          oa[q] = pack_bf16x2(da[2 * q], da[2 * q + 1]);
          ob[q] = pack_bf16x2(db[2 * q], db[2 * q + 1]);
          oh[q] = pack_bf16x2(hw[2 * q], hw[2 * q + 1]);
        }
        *reinterpret_cast<u32x4*>(p.dab + srow[kk] * h2 + col) = oa;
        *reinterpret_cast<u32x4*>(p.dab + srow[kk] * h2 + p.h + col) = ob;
        *reinterpret_cast<u32x4*>(p.hw + srow[kk] * p.h + col) = oh;
      }
    }
    // Rows past the tile's end skip the arithmetic; their prefetched
    // registers are consumed here all the same, so that no path leaves a
    // load in flight into registers the next item's prefetch reuses (the
    // compiler would otherwise wait for every load before that prefetch).
    asm volatile("" ::"v"(sa[0][0]), "v"(sa[0][1]), "v"(sa[0][2]), "v"(sa[0][3]), "v"(sa[1][0]),
                 "v"(sa[1][1]), "v"(sa[1][2]), "v"(sa[1][3]), "v"(sb[0][0]), "v"(sb[0][1]),
                 "v"(sb[0][2]), "v"(sb[0][3]), "v"(sb[1][0]), "v"(sb[1][1]), "v"(sb[1][2]),
                 "v"(sb[1][3]), "v"(ws[0]), "v"(ws[1]));
    // Sum each row's pieces over its four lanes (a fixed tree order).
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float v = dot[kk];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      if (c4 == 0 && ok[kk]) p.dwp[slice * p.rows + srow[kk]] = v;
    }

    if (nxt.rows <= 0) break;
    w = w1;
    w1 = w + gx;
    cur = nxt;
    nxt = (w1 < w_end) ? dg_tile(tiles, num_tiles, w1, n_slices) : TileInfo{0, 0, 0};
    idx_ready = false;
  }
  // Stages issued past the last item target buffers nobody reads; they must
  // land before the workgroup's LDS is released.
  wide_wait_all();
}

}  // namespace moe
