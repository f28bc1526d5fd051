// Stage "sort_permute" (kernel_gmm_gpu.json "pieces" suite): a stable
// counting sort of the T*k flat token-slots by expert, and the block_m tile
// schedule of the grouped GEMM.
//
//   1. count:   each block of kSlotsPerBlock consecutive flat slots counts
//               its slots per expert (integer LDS atomics: order-free sums).
//   2. scan:    one workgroup scans the [expert][block] counts (expert-
//               major, block-minor), which yields every block's first row per
//               expert and the expert offsets, then writes the tile list.
//   3. scatter: each block ranks its slots within each expert in flat order
//               (wave ballots give the rank among equal experts in a
//               64-slot step; running per-expert counters carry it across
//               steps and waves) and writes perm / inv_perm.
// The result is unique (stable by flat slot), so it matches a sequential
// counting sort bit for bit. No device-to-host synchronisation: the tile
// count stays on the device and the GEMMs are sized on the host by the
// upper bound ceil(S / block_m) + E.
#include "common.h"

namespace moe {

namespace {

constexpr int kPermThreads = 256;
constexpr int kSlotsPerWave = 1024;
constexpr int kSlotsPerBlock = kSlotsPerWave * (kPermThreads / 64);  // 4096
constexpr int kMaxE = 64;

__global__ __launch_bounds__(kPermThreads) void count_kernel(const int32_t* __restrict__ idx,
                                                             int64_t S, int E, int nblk,
                                                             int32_t* __restrict__ blk_counts) {
  __shared__ int32_t c[kMaxE];
  for (int e = threadIdx.x; e < E; e += kPermThreads) c[e] = 0;
  __syncthreads();
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kSlotsPerBlock;
  // All of a thread's expert indices are loaded first (one memory latency),
  // then counted.
  constexpr int kPer = kSlotsPerBlock / kPermThreads;
  int32_t ev[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int64_t s = s0 + threadIdx.x + q * kPermThreads;
    ev[q] = s < S ? idx[s] : 0;
  }
#pragma unroll
  for (int q = 0; q < kPer; ++q)
    if (s0 + threadIdx.x + q * kPermThreads < S) atomicAdd(&c[ev[q]], 1);
  __syncthreads();
  // Expert-major layout [E][nblk]: a flat exclusive scan of it is, for
  // every (expert, block), the expert's offset plus the rows of that expert
  // in earlier blocks.
  for (int e = threadIdx.x; e < E; e += kPermThreads)
    blk_counts[static_cast<int64_t>(e) * nblk + blockIdx.x] = c[e];
}

constexpr int kScanThreads = 1024;

// Rows of an expert with `count` slots that capacity routing keeps (cap 0:
// all of them).
__device__ __forceinline__ int32_t kept_rows(int32_t count, int cap) {
  return (cap > 0 && count > cap) ? cap : count;
}

// One workgroup: in-place exclusive scan of blk_counts[E * nblk], then the
// expert offsets and the tile list.
// Tile offsets of the experts (E <= 64, so one wave): lane e counts its
// expert's tiles of bm rows over its kept rows (rows_e), an inclusive scan
// over the lanes gives every expert's first tile, and lane 63 holds the
// total. Called by the first wave only.
__device__ __forceinline__ void wave_tile_offsets(int32_t rows_e, int E, int bm,
                                                  int32_t* tile_off, int32_t* num_tiles) {
  const int e = threadIdx.x;
  const int32_t cnt = e < E ? (rows_e + bm - 1) / bm : 0;
  int32_t incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t v = __shfl_up(incl, o, 64);
    if (e >= o) incl += v;
  }
  if (e < E) tile_off[e] = incl - cnt;
  if (e == 63) {
    tile_off[E] = incl;
    *num_tiles = incl;
  }
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(int32_t* __restrict__ blk_counts,
                                                            int nblk, int E, int bm, int cap,
                                                            int64_t S,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ tiles,
                                                            int32_t* __restrict__ num_tiles) {
  __shared__ int32_t wsum[kScanThreads / 64];
  __shared__ int32_t off[kMaxE + 1];
  __shared__ int32_t tile_off[kMaxE + 1];
  const int64_t L = static_cast<int64_t>(E) * nblk;
  const int64_t chunk = (L + kScanThreads - 1) / kScanThreads;
  const int64_t b0 = min(L, chunk * threadIdx.x), b1 = min(L, b0 + chunk);
  // Up to kScanRegs entries per thread are read once, all loads in flight
  // together, and kept in registers for the write-back.
  constexpr int kScanRegs = 16;
  const bool in_regs = chunk <= kScanRegs;
  // A whole chunk of kScanRegs entries (64 bytes, 16-byte aligned since b0
  // is a multiple of chunk) moves as four 16-byte accesses.
  const bool whole = chunk == kScanRegs && b1 - b0 == kScanRegs;
  int32_t vals[kScanRegs];
  int32_t local = 0;
  if (whole) {
#pragma unroll
    for (int q = 0; q < kScanRegs / 4; ++q) {
      const int4 v = *reinterpret_cast<const int4*>(blk_counts + b0 + 4 * q);
      vals[4 * q] = v.x; vals[4 * q + 1] = v.y; vals[4 * q + 2] = v.z; vals[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int q = 0; q < kScanRegs; ++q) local += vals[q];
  } else if (in_regs) {
#pragma unroll
    for (int q = 0; q < kScanRegs; ++q) {
      const int64_t i = b0 + q;
      const int32_t v = blk_counts[i < L ? i : L - 1];
      vals[q] = i < b1 ? v : 0;
      local += vals[q];
    }
  } else {
    for (int64_t i = b0; i < b1; ++i) local += blk_counts[i];
  }
  // Exclusive scan of the per-thread sums: within the wave, then across waves.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t run = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      const int32_t v = wsum[w];
      wsum[w] = run;
      run += v;
    }
  }
  __syncthreads();
  int32_t run = wsum[wave] + incl - local;
  // Entry e * nblk is block 0 of expert e: the first such entry at or after
  // b0, found with one division; later ones follow every nblk entries.
  int e_next = static_cast<int>((b0 + nblk - 1) / nblk);
  int64_t i_next = static_cast<int64_t>(e_next) * nblk;
  if (whole) {
    int32_t ex[kScanRegs];
#pragma unroll
    for (int q = 0; q < kScanRegs; ++q) {
      const int64_t i = b0 + q;
      ex[q] = run;
      if (i == i_next) {
        off[e_next] = run;
        ++e_next;
        i_next += nblk;
      }
      run += vals[q];
    }
#pragma unroll
    for (int q = 0; q < kScanRegs / 4; ++q)
      *reinterpret_cast<int4*>(blk_counts + b0 + 4 * q) =
          make_int4(ex[4 * q], ex[4 * q + 1], ex[4 * q + 2], ex[4 * q + 3]);
  } else if (in_regs) {
#pragma unroll
    for (int q = 0; q < kScanRegs; ++q) {
      const int64_t i = b0 + q;
      if (i < b1) {
        blk_counts[i] = run;
        if (i == i_next) {
          off[e_next] = run;
          ++e_next;
          i_next += nblk;
        }
        run += vals[q];
      }
    }
  } else {
    for (int64_t i = b0; i < b1; ++i) {
      const int32_t v = blk_counts[i];
      blk_counts[i] = run;
      if (i == i_next) {
        off[e_next] = run;
        ++e_next;
        i_next += nblk;
      }
      run += v;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) off[E] = static_cast<int32_t>(S);
  if (threadIdx.x < 64) {
    const int e = threadIdx.x;
    const int32_t hi = e + 1 < E ? off[e + 1] : static_cast<int32_t>(S);
    wave_tile_offsets(e < E ? kept_rows(hi - off[e], cap) : 0, E, bm, tile_off, num_tiles);
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += kScanThreads) offsets[e] = off[e];
  // Tile n of expert e covers rows [off[e] + (n - tile_off[e]) * bm, ...),
  // at most bm of them, within the expert's kept rows.
  const int32_t nt = tile_off[E];
  for (int32_t n = threadIdx.x; n < nt; n += kScanThreads) {
    int lo = 0, hi = E - 1;  // last e with tile_off[e] <= n
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_off[mid] <= n) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int32_t r = (n - tile_off[e]) * bm;
    tiles[3 * n + 0] = e;
    tiles[3 * n + 1] = off[e] + r;
    tiles[3 * n + 2] = min(bm, kept_rows(off[e + 1] - off[e], cap) - r);
  }
}

// Lanes of this wave whose expert equals mine (E <= 64: six ballots on the
// bits of the expert index; lanes past the end carry the value E).
__device__ __forceinline__ uint64_t same_expert_mask(int e) {
  uint64_t m = ~0ull;
#pragma unroll
  for (int b = 0; b < 7; ++b) {
    const uint64_t bal = __ballot((e >> b) & 1);
    m &= ((e >> b) & 1) ? bal : ~bal;
  }
  return m;
}

__global__ __launch_bounds__(kPermThreads) void scatter_kernel(const int32_t* __restrict__ idx,
                                                               int64_t S, int E, int nblk,
                                                               const int32_t* __restrict__ blk_base,
                                                               const int32_t* __restrict__ offsets,
                                                               int cap, int32_t* __restrict__ perm,
                                                               int32_t* __restrict__ inv_perm) {
  __shared__ int32_t wave_cnt[kPermThreads / 64][kMaxE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < (kPermThreads / 64) * kMaxE; i += kPermThreads)
    (&wave_cnt[0][0])[i] = 0;
  __syncthreads();
  const int64_t w0 = static_cast<int64_t>(blockIdx.x) * kSlotsPerBlock +
                     static_cast<int64_t>(wave) * kSlotsPerWave;
  // Pass 1: per-wave counts. Step q of the wave covers slots w0 + 64 q +
  // lane; the wave's expert indices are loaded once, all at a time, and kept
  // for pass 2 (slots past S carry E).
  constexpr int kSteps = kSlotsPerWave / 64;
  int32_t ev[kSteps];
#pragma unroll
  for (int q = 0; q < kSteps; ++q) {
    const int64_t s = w0 + q * 64 + lane;
    ev[q] = s < S ? idx[s] : E;
  }
#pragma unroll
  for (int q = 0; q < kSteps; ++q)
    if (w0 + q * 64 + lane < S) atomicAdd(&wave_cnt[wave][ev[q]], 1);
  __syncthreads();
  // Per-wave running counters start at the block base plus the counts of
  // the earlier waves of the block.
  if (threadIdx.x < E) {
    const int e = threadIdx.x;
    int32_t run = blk_base[static_cast<int64_t>(e) * nblk + blockIdx.x];
    for (int w = 0; w < kPermThreads / 64; ++w) {
      const int32_t c = wave_cnt[w][e];
      wave_cnt[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  // Pass 2: stable ranks, 64 slots per step in flat order.
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int q = 0; q < kSteps; ++q) {
    const int64_t s = w0 + q * 64 + lane;
    const bool ok = s < S;
    const int e = ev[q];
    const uint64_t m = same_expert_mask(e);
    const int rank = __popcll(m & lt);
    const int cnt = __popcll(m);
    if (ok) {
      const int32_t base = wave_cnt[wave][e];
      const int32_t pos = base + rank;
      perm[pos] = static_cast<int32_t>(s);
      // Capacity routing drops every slot past the expert's first cap.
      inv_perm[s] = (cap > 0 && pos - offsets[e] >= cap) ? -1 : pos;
    }
    // All lanes have read their base (the read above precedes this point
    // in the wave's in-order LDS queue); the last lane of each expert group
    // advances its counter.
    __builtin_amdgcn_wave_barrier();
    if (ok && rank == cnt - 1) wave_cnt[wave][e] += cnt;
    __builtin_amdgcn_wave_barrier();
  }
}

// A tile list with another row count bm2 from the expert offsets (the same
// definition as the scan's list: experts ascending, each expert's kept rows
// in pieces of bm2, the last one partial). One workgroup.
__global__ __launch_bounds__(kScanThreads) void retile_kernel(const int32_t* __restrict__ offsets,
                                                              int E, int bm2, int cap,
                                                              int32_t* __restrict__ tiles,
                                                              int32_t* __restrict__ num_tiles) {
  __shared__ int32_t tile_off[kMaxE + 1];
  __shared__ int32_t kept[kMaxE];
  if (threadIdx.x < 64) {
    const int e = threadIdx.x;
    const int32_t rows = e < E ? kept_rows(offsets[e + 1] - offsets[e], cap) : 0;
    if (e < E) kept[e] = rows;
    wave_tile_offsets(rows, E, bm2, tile_off, num_tiles);
  }
  __syncthreads();
  const int32_t nt = tile_off[E];
  for (int32_t n = threadIdx.x; n < nt; n += kScanThreads) {
    int lo = 0, hi = E - 1;  // last e with tile_off[e] <= n
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_off[mid] <= n) lo = mid; else hi = mid - 1;
    }
    const int32_t r = (n - tile_off[lo]) * bm2;
    tiles[3 * n + 0] = lo;
    tiles[3 * n + 1] = offsets[lo] + r;
    tiles[3 * n + 2] = min(bm2, kept[lo] - r);
  }
}

}  // namespace

hipError_t launch_retile(const int32_t* offsets, int E, int bm2, int cap, int32_t* tiles,
                         int32_t* num_tiles, hipStream_t s) {
  MOE_LAUNCH("retile", retile_kernel, dim3(1), dim3(kScanThreads), 0, s, offsets, E, bm2, cap,
             tiles, num_tiles);
  // Called in the middle of a stage: the error stays pending for the
  // stage's own final hipGetLastError().
  return hipPeekAtLastError();
}

// Scratch of moe_permute_static: the per-block expert counts live in this
// fixed device array instead of a caller workspace. Each device holds its
// own copy at its own address, looked up once per device with
// hipGetSymbolAddress (the array's name is not a device address in host
// code). The count kernel writes every entry the scan and scatter read, so
// nothing needs clearing between calls; calls on one device share it.
constexpr size_t kStaticScratchBytes = size_t{1} << 20;
static __device__ __align__(256) int32_t scratch[kStaticScratchBytes / sizeof(int32_t)];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];
}  // namespace

size_t static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t permute_ws_bytes(int64_t S, int E) {
  const int64_t nblk = (S + kSlotsPerBlock - 1) / kSlotsPerBlock;
  return align_up(sizeof(int32_t) * static_cast<size_t>(nblk) * E, 256);
}

hipError_t launch_permute(int64_t T, int k, int E, int bm, int cap, const int32_t* topk_idx,
                          int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* tiles,
                          int32_t* num_tiles, void* ws, hipStream_t s) {
  const int64_t S = T * k;
  const int nblk = static_cast<int>((S + kSlotsPerBlock - 1) / kSlotsPerBlock);
  int32_t* blk = static_cast<int32_t*>(ws);
  MOE_LAUNCH("permute_count", count_kernel, dim3(nblk), dim3(kPermThreads), 0, s, topk_idx, S, E, nblk,
                     blk);
  MOE_LAUNCH("permute_scan", scan_kernel, dim3(1), dim3(kScanThreads), 0, s, blk, nblk, E, bm, cap, S,
             offsets, tiles, num_tiles);
  MOE_LAUNCH("permute_scatter", scatter_kernel, dim3(nblk), dim3(kPermThreads), 0, s, topk_idx, S, E, nblk,
             blk, offsets, cap, perm, inv_perm);
  return hipGetLastError();
}

}  // namespace moe
