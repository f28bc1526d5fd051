// Measurement probe (not part of libmoe): the wide GEMM engine's K-stage
// loop on its own, to find what bounds it. Each of `grid` persistent
// workgroups (512 threads, the engine's 8 waves and 256 x 256 tile) runs
// `items` tiles of 8 stages of 64-deep K, multiplying each stage out of LDS
// with the engine's own wide_compute while the next stage is loaded in the
// way `mode` selects:
//   0  nothing loaded (operands stay in LDS: the MFMA and LDS-read rate)
//   1  the token half of each stage only (32 KiB, direct-to-LDS)
//   2  the weight half only (32 KiB, direct-to-LDS)
//   3  both halves (64 KiB, direct-to-LDS): the engine's stage
//   4  the same 64 KiB into registers instead of LDS
//   5  64 KiB of LDS writes from registers, no global loads
//   6  all 64 KiB issued by waves 0-3 only (one per SIMD)
//   7  MFMA only: each wave's fragments are read from LDS once and held in
//      registers; no LDS reads, loads or barriers in the loop
//   8  as 3 with four waves of 128 x 128 blocks (one wave per SIMD, 256
//      threads) instead of eight of 64 x 128
//   9  as 3 with the token half in a ring of three 32 KiB buffers, issued
//      two stages ahead, and the weight half in two (160 KiB of LDS)
//  10  as 8 with the next stage's loads and the next K step's fragment
//      reads spread between the MFMAs by scheduling barriers
// Token rows come from a region of `a_rows` 1 KiB rows, read in order or
// (random != 0) at hashed rows, as gathered expert rows are; weights from a
// 2 MiB region (8 groups of 256 rows x 512 bf16), L2-resident. K = 512.
// Both stage buffers are filled from the first tile's rows before the loop,
// so the modes that load nothing multiply the same data. `data` selects the
// operand values: 0 all zeros, 1 hashed bf16 values of magnitude 0.5 to 2
// with random signs. The MFMA pipes draw more power on the second, and the
// clock the chip sustains under it is what a real GEMM runs at.
#include <hip/hip_runtime.h>

#include "gemm_wide.h"

namespace {

using namespace moe;

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void stage_probe_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bw, int64_t a_rows,
                        int mode, int random, int items, float* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kWideStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int wm = wave / 2, wn = wave % 2;
  constexpr int kStages = 8;
  const int64_t ldb = 64 * kStages;  // weight row = K elements
  const int lrow = wave * kWideLoads * 8 + (lane >> 3);
  const int xr = lane >> 4;
  const int chunk_off[2] = {((lane & 7) ^ xr) * 16, ((lane & 7) ^ (xr + 4)) * 16};
  const int b_off[2] = {static_cast<int>(lrow * ldb * 2) + chunk_off[0],
                        static_cast<int>(lrow * ldb * 2) + chunk_off[1]};
  const int a_frag = (wm * 64 + r32) * kWideRowBytes;
  const int b_frag = (256 + wn * 128 + r32) * kWideRowBytes;
  const int sw_base = g ^ ((r32 >> 1) & 7);
  f32x16_t acc[2][4];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 4; ++j)
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  unsigned sink = 0;
  // Both buffers from the first tile's rows (every mode multiplies data).
  for (int b = 0; b < 2; ++b) {
    for (int i = 0; i < kWideLoads; ++i) {
      int64_t r = static_cast<int64_t>(blockIdx.x) * items * 256 + lrow + 8 * i;
      if (random) r *= 2654435761ll;
      r %= a_rows;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(A) + r * 1024 + chunk_off[i & 1] + b * 128,
                                       smem + b * kWideStage + (wave * kWideLoads + i) * 1024, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(Bw) + b_off[i & 1] + i * 16 * ldb + b * 128,
                                       smem + b * kWideStage + 256 * kWideRowBytes + (wave * kWideLoads + i) * 1024,
                                       16, 0, 0);
    }
  }
  wide_wait_all();
  __syncthreads();
  if (mode == 7) {
    u32x4 xf[2], wf[4];
    for (int i = 0; i < 2; ++i)
      xf[i] = *reinterpret_cast<const u32x4*>(smem + a_frag + i * 32 * kWideRowBytes + (sw_base << 4));
    for (int j = 0; j < 4; ++j)
      wf[j] = *reinterpret_cast<const u32x4*>(smem + b_frag + j * 32 * kWideRowBytes + (sw_base << 4));
    for (int it = 0; it < items * kStages; ++it)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) Mfma<bf16_t>::step(wf[j], xf[i], acc[i][j]);
  }
  int buf = 0;
  for (int it = 0; it < (mode == 7 ? 0 : items); ++it) {
    const int64_t item = static_cast<int64_t>(blockIdx.x) * items + it;
    const char* a_row[kWideLoads];
    for (int i = 0; i < kWideLoads; ++i) {
      int64_t r = item * 256 + lrow + 8 * i;
      if (random) r *= 2654435761ll;
      r %= a_rows;
      a_row[i] = reinterpret_cast<const char*>(A) + r * 1024 + chunk_off[i & 1];
    }
    const char* b_base = reinterpret_cast<const char*>(Bw) + (item % 8) * 256 * ldb * 2;
    const int64_t b_step = 16 * ldb;
    for (int s = 0; s < kStages; ++s) {
      wide_wait_all();
      wide_barrier();
      char* cb = smem + buf * kWideStage;
      const int koff = s * 128;
      if (mode == 1 || mode == 3)
        for (int i = 0; i < kWideLoads; ++i)
          __builtin_amdgcn_global_load_lds(a_row[i] + koff, cb + (wave * kWideLoads + i) * 1024, 16, 0, 0);
      if (mode == 2 || mode == 3)
        for (int i = 0; i < kWideLoads; ++i)
          __builtin_amdgcn_global_load_lds(b_base + koff + b_off[i & 1] + i * b_step,
                                           cb + 256 * kWideRowBytes + (wave * kWideLoads + i) * 1024,
                                           16, 0, 0);
      if (mode == 4)
        for (int i = 0; i < kWideLoads; ++i) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(a_row[i] + koff);
          const u32x4 u = *reinterpret_cast<const u32x4*>(b_base + koff + b_off[i & 1] + i * b_step);
          sink ^= v[0] ^ v[3] ^ u[1] ^ u[2];
        }
      if (mode == 5)
        for (int i = 0; i < 8; ++i)
          *reinterpret_cast<u32x4*>(cb + (wave * 8 + i) * 1024 + lane * 16) = u32x4{sink, 1u, 2u, 3u};
      if (mode == 6 && wave < 4)
        for (int i = 0; i < 4 * kWideLoads; ++i)
          __builtin_amdgcn_global_load_lds(a_row[i & 3] + koff, cb + (wave * 4 * kWideLoads + i) * 1024,
                                           16, 0, 0);
      wide_compute(smem + (buf ^ 1) * kWideStage, a_frag, b_frag, sw_base, acc);
      buf ^= 1;
    }
  }
  float sum = 0.0f;
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 4; ++j)
      for (int q = 0; q < 16; ++q) sum += acc[i][j][q];
  // a test that is practically never true; keeps the work alive
  if (sum == 1234.5f || sink == 0x12345678u) out[blockIdx.x * 512 + tid] = sum;
}

// Weight rows of item `item`: group item % 8 of the 2 MiB weight region.
__device__ __forceinline__ const char* Bw_base(const bf16_t* Bw, int64_t item) {
  return reinterpret_cast<const char*>(Bw) + (item % 8) * 256 * 1024;
}

// Modes 8 and 9: NW waves of WM x WN MFMA tiles each; RING 0 keeps the
// engine's two 64 KiB stage buffers (both halves issued one stage ahead),
// RING 1 a three-deep token ring and a two-deep weight ring. The stage
// loop runs over all items' stages in one sequence, as in the engine.
template <int NW, int WM, int WN, int RING>
__device__ void stage_ring(const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bw,
                           int64_t a_rows, int random, int items, float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(1024))) char dyn[];
  constexpr int kHalfLoads = 32 / NW;  // 1 KiB direct-to-LDS loads per wave per half stage
  constexpr int kWavesN = 256 / (WN * 32);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int a_frag = (wm * WM * 32 + r32) * kWideRowBytes;
  const int b_frag = (wn * WN * 32 + r32) * kWideRowBytes;
  const int sw_base = g ^ ((r32 >> 1) & 7);
  const int xr = lane >> 4;
  const int chunk_off[2] = {((lane & 7) ^ xr) * 16, ((lane & 7) ^ (xr + 4)) * 16};
  f32x16_t acc[WM][WN];
  for (int i = 0; i < WM; ++i)
    for (int j = 0; j < WN; ++j)
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  const int total = items * 8;
  auto a_slot = [&](int s) { return RING ? dyn + (s % 3) * 32768 : dyn + (s & 1) * 65536; };
  auto b_slot = [&](int s) {
    return RING ? dyn + 98304 + (s & 1) * 32768 : dyn + (s & 1) * 65536 + 32768;
  };
  // issue_a runs once per stage in stage order; the row addresses of an
  // item are formed at its first stage, as the engine forms them per item
  const char* a_row[kHalfLoads];
  auto issue_a = [&](int s) {
    if ((s & 7) == 0) {
      const int64_t item = static_cast<int64_t>(blockIdx.x) * items + s / 8;
#pragma unroll
      for (int i = 0; i < kHalfLoads; ++i) {
        int64_t row = item * 256 + (wave * kHalfLoads + i) * 8 + (lane >> 3);
        if (random) row *= 2654435761ll;
        row %= a_rows;
        a_row[i] = reinterpret_cast<const char*>(A) + row * 1024 + chunk_off[i & 1];
      }
    }
    char* dst = a_slot(s);
#pragma unroll
    for (int i = 0; i < kHalfLoads; ++i)
      __builtin_amdgcn_global_load_lds(a_row[i] + (s & 7) * 128, dst + (wave * kHalfLoads + i) * 1024,
                                       16, 0, 0);
  };
  auto issue_b = [&](int s) {
    const int64_t item = static_cast<int64_t>(blockIdx.x) * items + s / 8;
    const char* base = reinterpret_cast<const char*>(Bw) + (item % 8) * 256 * 1024;
    char* dst = b_slot(s);
#pragma unroll
    for (int i = 0; i < kHalfLoads; ++i) {
      const int r = (wave * kHalfLoads + i) * 8 + (lane >> 3);
      __builtin_amdgcn_global_load_lds(base + r * 1024 + chunk_off[i & 1] + (s % 8) * 128,
                                       dst + (wave * kHalfLoads + i) * 1024, 16, 0, 0);
    }
  };
  auto compute = [&](int s) {
    const char* ab = a_slot(s);
    const char* bb = b_slot(s);
    int sb = sw_base;
    asm volatile("" : "+v"(sb));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int sw = ((2 * q) ^ sb) << 4;
      u32x4 xf[WM], wf[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) xf[i] = *reinterpret_cast<const u32x4*>(ab + a_frag + i * 4096 + sw);
#pragma unroll
      for (int j = 0; j < WN; ++j) wf[j] = *reinterpret_cast<const u32x4*>(bb + b_frag + j * 4096 + sw);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) Mfma<bf16_t>::step(wf[j], xf[i], acc[i][j]);
    }
  };
  if (RING == 0) {
    issue_a(0);
    issue_b(0);
    for (int s = 0; s < total; ++s) {
      wide_wait_all();
      wide_barrier();
      if (s + 1 < total) {
        issue_a(s + 1);
        issue_b(s + 1);
      }
      compute(s);
    }
  } else {
    // Per stage the weights of s + 1 are issued before the token rows of
    // s + 2, so waiting for all but the last kHalfLoads loads leaves only
    // the newest token rows in flight.
    issue_a(0);
    issue_b(0);
    issue_a(1);
    for (int s = 0; s < total; ++s) {
      if (s + 2 < total)
        __builtin_amdgcn_s_waitcnt((kHalfLoads & 15) | ((kHalfLoads >> 4) << 14) | (0x7 << 4));
      else
        wide_wait_all();
      wide_barrier();
      if (s + 1 < total) issue_b(s + 1);
      if (s + 2 < total) issue_a(s + 2);
      compute(s);
    }
  }
  wide_wait_all();
  float sum = 0.0f;
  for (int i = 0; i < WM; ++i)
    for (int j = 0; j < WN; ++j)
      for (int q = 0; q < 16; ++q) sum += acc[i][j][q];
  if (sum == 1234.5f) out[blockIdx.x * 512 + tid] = sum;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void stage_four_wave_kernel(const bf16_t* A, const bf16_t* Bw, int64_t a_rows, int random,
                            int items, float* out) {
  stage_ring<4, 4, 4, 0>(A, Bw, a_rows, random, items, out);
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void stage_token_ring_kernel(const bf16_t* A, const bf16_t* Bw, int64_t a_rows, int random,
                             int items, float* out) {
  stage_ring<8, 2, 4, 1>(A, Bw, a_rows, random, items, out);
}

// Mode 10: four waves of 128 x 128 blocks, two 64 KiB stage buffers. Each K
// step reads the next step's fragments and issues a quarter of the next
// stage's 16 loads per wave, and scheduling barriers place them between
// its 16 MFMAs ([MFMA][read][MFMA][read][MFMA][load][MFMA] four times).
// The loads run unconditionally: past the last stage they fetch in-bounds
// rows of a tile past this workgroup's share into the buffer nobody reads.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void stage_four_wave_spread_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bw,
                                   int64_t a_rows, int random, int items, float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(1024))) char dyn[];
  constexpr int kHalf = 8;  // loads per wave per half stage
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int wm = wave / 2, wn = wave % 2;
  const int a_frag = (wm * 128 + r32) * kWideRowBytes;
  const int b_frag = 32768 + (wn * 128 + r32) * kWideRowBytes;
  const int xr = lane >> 4;
  const int chunk_off[2] = {((lane & 7) ^ xr) * 16, ((lane & 7) ^ (xr + 4)) * 16};
  f32x16_t acc[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j)
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  const int total = items * 8;
  const char* a_row[kHalf];
  const char* b_base = Bw_base(Bw, 0);
  auto rows_for = [&](int s) {
    const int64_t item = static_cast<int64_t>(blockIdx.x) * items + s / 8;
#pragma unroll
    for (int i = 0; i < kHalf; ++i) {
      int64_t row = item * 256 + (wave * kHalf + i) * 8 + (lane >> 3);
      if (random) row *= 2654435761ll;
      row %= a_rows;
      a_row[i] = reinterpret_cast<const char*>(A) + row * 1024 + chunk_off[i & 1];
    }
    b_base = Bw_base(Bw, item);
  };
  auto load1 = [&](int s, int u) {  // load u (0..15) of stage s
    char* dst = dyn + (s & 1) * 65536;
    const int koff = (s & 7) * 128;
    if (u < kHalf) {
      __builtin_amdgcn_global_load_lds(a_row[u] + koff, dst + (wave * kHalf + u) * 1024, 16, 0, 0);
    } else {
      const int i = u - kHalf;
      const int r = (wave * kHalf + i) * 8 + (lane >> 3);
      __builtin_amdgcn_global_load_lds(b_base + r * 1024 + chunk_off[i & 1] + koff,
                                       dst + 32768 + (wave * kHalf + i) * 1024, 16, 0, 0);
    }
  };
  rows_for(0);
#pragma unroll
  for (int u = 0; u < 16; ++u) load1(0, u);
  int sb = g ^ ((r32 >> 1) & 7);
  for (int s = 0; s < total; ++s) {
    wide_wait_all();
    wide_barrier();
    if (((s + 1) & 7) == 0) rows_for(s + 1);
    const char* buf = dyn + (s & 1) * 65536;
    asm volatile("" : "+v"(sb));
    u32x4 xf[2][4], wf[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xf[0][i] = *reinterpret_cast<const u32x4*>(buf + a_frag + i * 4096 + (sb << 4));
#pragma unroll
    for (int j = 0; j < 4; ++j) wf[0][j] = *reinterpret_cast<const u32x4*>(buf + b_frag + j * 4096 + (sb << 4));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = q & 1, n = c ^ 1;
      if (q < 3) {
        const int sw = ((2 * (q + 1)) ^ sb) << 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) xf[n][i] = *reinterpret_cast<const u32x4*>(buf + a_frag + i * 4096 + sw);
#pragma unroll
        for (int j = 0; j < 4; ++j) wf[n][j] = *reinterpret_cast<const u32x4*>(buf + b_frag + j * 4096 + sw);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) load1(s + 1, q * 4 + u);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) Mfma<bf16_t>::step(wf[c][j], xf[c][i], acc[i][j]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wide_wait_all();
  float sum = 0.0f;
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j)
      for (int q = 0; q < 16; ++q) sum += acc[i][j][q];
  if (sum == 1234.5f) out[blockIdx.x * 512 + tid] = sum;
}

#define PROBE_EXPORT extern "C" __attribute__((visibility("default")))

// Hashed bf16 values, two per 32-bit word: random sign, exponent 2^-1 or
// 2^0, random mantissa (magnitudes 0.5 to 2); or zeros.
__global__ void probe_fill_kernel(uint32_t* p, int64_t n, int data) {
  for (int64_t i = blockIdx.x * int64_t{256} + threadIdx.x; i < n; i += int64_t{gridDim.x} * 256) {
    uint32_t v = 0;
    if (data) {
      uint32_t h = static_cast<uint32_t>(i) * 2654435761u + 12345u;
      h ^= h >> 15;
      h *= 2246822519u;
      h ^= h >> 13;
      const uint32_t lo = ((h & 1) << 15) | ((126 + ((h >> 1) & 1)) << 7) | ((h >> 2) & 127);
      const uint32_t hi = (((h >> 9) & 1) << 15) | ((126 + ((h >> 10) & 1)) << 7) | ((h >> 11) & 127);
      v = lo | (hi << 16);
    }
    p[i] = v;
  }
}

// Store-pattern probe: 1 GiB of bf16 rows [2^20][512] written by 256
// persistent workgroups of eight waves, each wave a 64 x 128 block as 16
// stores of eight 128-byte row pieces (the engine's drain), in the order of
// `mode`: 0 256 x 256 tiles, tile t = (row block t / 2, column half t % 2),
// so neighbouring workgroups share a row block; 1 whole-row 128 x 512
// tiles; 2 256 x 256 tiles with both column halves of a row block written
// by one workgroup back to back.
__device__ __forceinline__ void store_block(char* y, int64_t row0, int col0, int wr, int wc,
                                            int lane, u32x4 v) {
  for (int h = 0; h < 2; ++h)
    for (int k = 0; k < 8; ++k) {
      const int64_t r = row0 + wr + k * 8 + (lane >> 3);
      *reinterpret_cast<u32x4*>(y + r * 1024 + col0 + wc + h * 128 + (lane & 7) * 16) = v;
    }
}

__global__ __launch_bounds__(512) void store_probe_kernel(char* __restrict__ y, int mode) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = gridDim.x;
  const u32x4 v = {1u + lane, 2u, 3u, 4u};
  if (mode == 0) {
    for (int t = blockIdx.x; t < 8192; t += G)
      store_block(y, static_cast<int64_t>(t / 2) * 256, (t % 2) * 512, (wave / 2) * 64,
                  (wave % 2) * 256, lane, v);
  } else if (mode == 1) {
    for (int t = blockIdx.x; t < 8192; t += G)
      store_block(y, static_cast<int64_t>(t) * 128, 0, (wave / 4) * 64, (wave % 4) * 256, lane, v);
  } else {
    for (int b = blockIdx.x; b < 4096; b += G)
      for (int half = 0; half < 2; ++half)
        store_block(y, static_cast<int64_t>(b) * 256, half * 512, (wave / 2) * 64,
                    (wave % 2) * 256, lane, v);
  }
}

}  // namespace

// Runs one probe configuration `reps` times after two warm-up launches and
// writes the average milliseconds per launch to *ms. Allocates and frees
// its own buffers (1 GiB of token rows at most). Returns 0 or a HIP error.
PROBE_EXPORT int moe_stage_probe(int mode, int64_t a_rows, int random, int data, int grid,
                                 int items, int reps, float* ms) {
  if (mode < 0 || mode > 10 || a_rows < 256 || a_rows > (int64_t{1} << 20) || data < 0 ||
      data > 1 || grid < 1 || items < 1 || reps < 1 || !ms)
    return -1;
  bf16_t *A = nullptr, *Bw = nullptr;
  float* out = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipMalloc(&A, a_rows * 1024);
  if (e == hipSuccess) e = hipMalloc(&Bw, size_t{8} * 256 * 1024);
  if (e == hipSuccess) e = hipMalloc(&out, size_t{4} * 512 * grid);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(probe_fill_kernel, dim3(1024), dim3(256), 0, 0,
                       reinterpret_cast<uint32_t*>(A), a_rows * 256, data);
    hipLaunchKernelGGL(probe_fill_kernel, dim3(1024), dim3(256), 0, 0,
                       reinterpret_cast<uint32_t*>(Bw), int64_t{8} * 256 * 256, data);
    e = hipGetLastError();
  }
  if (e == hipSuccess && mode == 9)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(stage_token_ring_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
  if (e == hipSuccess && mode == 8)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(stage_four_wave_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 131072);
  if (e == hipSuccess && mode == 10)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(stage_four_wave_spread_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 131072);
  auto launch = [&]() {
    if (mode == 8)
      hipLaunchKernelGGL(stage_four_wave_kernel, dim3(grid), dim3(256), 131072, 0, A, Bw, a_rows,
                         random, items, out);
    else if (mode == 10)
      hipLaunchKernelGGL(stage_four_wave_spread_kernel, dim3(grid), dim3(256), 131072, 0, A, Bw,
                         a_rows, random, items, out);
    else if (mode == 9)
      hipLaunchKernelGGL(stage_token_ring_kernel, dim3(grid), dim3(512), 163840, 0, A, Bw, a_rows,
                         random, items, out);
    else
      hipLaunchKernelGGL(stage_probe_kernel, dim3(grid), dim3(512), 0, 0, A, Bw, a_rows, mode,
                         random, items, out);
  };
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) {
    for (int r = 0; r < 2; ++r) launch();
    e = hipEventRecord(e0, 0);
    for (int r = 0; r < reps && e == hipSuccess; ++r) launch();
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) e = hipEventRecord(e1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float t = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, e0, e1);
    *ms = t / reps;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (out) (void)hipFree(out);
  if (Bw) (void)hipFree(Bw);
  if (A) (void)hipFree(A);
  return e == hipSuccess ? 0 : static_cast<int>(e);
}

// Runs the store-pattern probe `reps` times after two warm-up launches and
// writes the average milliseconds per launch to *ms. Allocates and frees
// its own 1 GiB buffer. Returns 0, -1 for a bad argument, or a HIP error.
PROBE_EXPORT int moe_store_probe(int mode, int reps, float* ms) {
  if (mode < 0 || mode > 2 || reps < 1 || !ms) return -1;
  char* y = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipMalloc(&y, size_t{1} << 30);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) {
    for (int r = 0; r < 2; ++r)
      hipLaunchKernelGGL(store_probe_kernel, dim3(256), dim3(512), 0, 0, y, mode);
    e = hipEventRecord(e0, 0);
    for (int r = 0; r < reps && e == hipSuccess; ++r)
      hipLaunchKernelGGL(store_probe_kernel, dim3(256), dim3(512), 0, 0, y, mode);
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) e = hipEventRecord(e1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float t = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, e0, e1);
    *ms = t / reps;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (y) (void)hipFree(y);
  return e == hipSuccess ? 0 : static_cast<int>(e);
}
