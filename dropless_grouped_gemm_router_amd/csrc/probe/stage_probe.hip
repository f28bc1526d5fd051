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
// Token rows come from a region of `a_rows` 1 KiB rows, read in order or
// (random != 0) at hashed rows, as gathered expert rows are; weights from a
// 2 MiB region (8 groups of 256 rows x 512 bf16), L2-resident. K = 512.
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
  int buf = 0;
  for (int it = 0; it < items; ++it) {
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
  // never true for the zero-filled operands; keeps the work alive
  if (sum == 1234.5f || sink == 0x12345678u) out[blockIdx.x * 512 + tid] = sum;
}

}  // namespace

#define PROBE_EXPORT extern "C" __attribute__((visibility("default")))

// Runs one probe configuration `reps` times after two warm-up launches and
// writes the average milliseconds per launch to *ms. Allocates and frees
// its own buffers (1 GiB of token rows at most). Returns 0 or a HIP error.
PROBE_EXPORT int moe_stage_probe(int mode, int64_t a_rows, int random, int grid, int items,
                                 int reps, float* ms) {
  if (mode < 0 || mode > 6 || a_rows < 256 || a_rows > (int64_t{1} << 20) || grid < 1 ||
      items < 1 || reps < 1 || !ms)
    return -1;
  bf16_t *A = nullptr, *Bw = nullptr;
  float* out = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipMalloc(&A, a_rows * 1024);
  if (e == hipSuccess) e = hipMalloc(&Bw, size_t{8} * 256 * 1024);
  if (e == hipSuccess) e = hipMalloc(&out, size_t{4} * 512 * grid);
  if (e == hipSuccess) e = hipMemset(A, 0, a_rows * 1024);
  if (e == hipSuccess) e = hipMemset(Bw, 0, size_t{8} * 256 * 1024);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) {
    for (int r = 0; r < 2; ++r)
      hipLaunchKernelGGL(stage_probe_kernel, dim3(grid), dim3(512), 0, 0, A, Bw, a_rows, mode,
                         random, items, out);
    e = hipEventRecord(e0, 0);
    for (int r = 0; r < reps && e == hipSuccess; ++r)
      hipLaunchKernelGGL(stage_probe_kernel, dim3(grid), dim3(512), 0, 0, A, Bw, a_rows, mode,
                         random, items, out);
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
