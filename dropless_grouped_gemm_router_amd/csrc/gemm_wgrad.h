// Weight-gradient GEMM for bf16 operands with the reduction over rows:
//
//   C[g][m][n] = sum over rows r of group g: A[r][m] * B[r][n]     (fp32 out)
//
// Both operands are row-major with the reduction index r as the row, so the
// MFMA fragments (8 consecutive r per lane) run down columns. Stages of
// KT = 64 rows are copied verbatim into LDS by direct global-to-LDS loads
// (16-byte chunks, rows XOR-swizzled in chunk units), and the fragments are
// read with gfx950's transposing LDS read ds_read_b64_tr_b16: within each
// group of 16 lanes, lane 4a + b receives element b of the 8-byte pieces
// addressed by lanes 4q + a (q = 0..3). When lane s of a group addresses row
// k0 + s / 4, columns c0 + 4 (s % 4) .. + 3, lane j of the group receives
// rows k0 .. k0 + 3 of column c0 + j: half a 32x32x16 MFMA fragment.
//
// The stages form a ring of NS buffers. Every wave issues the same number of
// loads per stage (rows past the group's end read a zero row), and the loop
// holds no other memory operation, so waiting for vmcnt <= loads of NS - 2
// stages leaves the next NS - 2 stages in flight while one is multiplied.
//
// Gathered A (kGather): row r of A is token perm[r] / topk of x. Each wave
// fetches the 64 perm entries of a stage into its own LDS slot by one more
// direct-to-LDS load per stage (so the per-stage load count stays the same
// for every wave and the counted waits stay exact), NS - 1 stages before
// that stage's row loads are issued, and reads them back by inline-assembly
// LDS reads when it forms the row addresses. Tokens are clamped to the
// table, so no address leaves x whatever an entry holds.
//
// Group g covers rows [row_offsets[g], row_offsets[g+1]) (clipped to cap
// rows under capacity routing), or the g-th of `splits` equal slices of
// rows_total (dense split-K partials, reduced later in a fixed order). One
// workgroup owns each (group, M tile, N tile) output: deterministic, no
// atomics.
#pragma once

#include "gemm_core.h"

namespace moe {

typedef short tr_v4i16 __attribute__((ext_vector_type(4)));

constexpr int kTrKT = 64;        // rows per stage
constexpr int kTrBN = 128;       // N tile
constexpr int kTrZeroBytes = 1024;  // zero row read past a group's end (>= 2 * BM bytes)

template <int BM_, int NS_>
struct TrCfg {
  static constexpr int BM = BM_, BN = kTrBN, NS = NS_;
  static constexpr int WAVES_M = BM / 64, WAVES_N = 2;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int A_PITCH = BM * 2, B_PITCH = BN * 2;         // bytes per LDS row
  static constexpr int A_BYTES = kTrKT * A_PITCH, B_BYTES = kTrKT * B_PITCH;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_CPR = A_PITCH / 16, B_CPR = B_PITCH / 16;  // 16-byte chunks per row
  // 64-lane load instructions per wave per stage, for each operand.
  static constexpr int A_LOADS = A_BYTES / 1024 / (NT / 64);
  static constexpr int B_LOADS = B_BYTES / 1024 / (NT / 64);
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static_assert(A_BYTES % (1024 * (NT / 64)) == 0 && B_BYTES % (1024 * (NT / 64)) == 0, "loads");
  static_assert(NS >= 2 && NS * STAGE + NS * (NT / 64) * 256 <= 160 * 1024, "LDS");
};

// Chunk position of logical 16-byte chunk c of LDS row r.
__device__ __forceinline__ int tr_swz(int r, int c) { return c ^ ((r & 7) << 1); }

// s_waitcnt with vmcnt <= n (n < 64), expcnt and lgkmcnt not waited on.
template <int N>
__device__ __forceinline__ void tr_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One operand's loads of one stage: instruction u of this wave covers the
// operand's 64-lane chunk block (wave * LOADS_OP + u), i.e. chunks
// [64 i, 64 i + 63] in LDS order; chunk i at row i / CPR, position i % CPR
// holds logical chunk tr_swz(row, position) of that row.
template <int CPR, int LOADS_OP>
__device__ __forceinline__ void tr_issue(char* lds_op, const bf16_t* base, int64_t ld, int col0,
                                         int64_t row0, int64_t row_end, const bf16_t* zero,
                                         int wave, int lane) {
#pragma unroll
  for (int u = 0; u < LOADS_OP; ++u) {
    const int blk = wave * LOADS_OP + u;
    const int ci = blk * 64 + lane;
    const int r = ci / CPR, pos = ci % CPR;
    const int c = tr_swz(r, pos);
    const int64_t row = row0 + r;
    const bf16_t* src = row < row_end ? base + row * ld + col0 + c * 8 : zero + c * 8;
    __builtin_amdgcn_global_load_lds(src, lds_op + blk * 1024, 16, 0, 0);
  }
}

// One stage's 64 perm entries (rows row_start ..) into a 256-byte LDS slot,
// lane l's entry at byte 4 l; entries past the table repeat its last one.
__device__ __forceinline__ void tr_issue_idx(char* slot, const int32_t* perm, int64_t row_start,
                                             int64_t len, int lane) {
  int64_t r = row_start + lane;
  r = r < len ? r : len - 1;
  __builtin_amdgcn_global_load_lds(perm + r, slot, 4, 0, 0);
}

// A-operand loads of one stage with gathered rows: as tr_issue, the row's
// address taken from token perm[row] / topk (read from the stage's slot at
// LDS byte address idx_lds), clamped to [0, ntok).
template <int CPR, int LOADS_OP>
__device__ __forceinline__ void tr_issue_gather(char* lds_op, const bf16_t* x, int64_t ld,
                                                int col0, int64_t row0, int64_t row_end,
                                                const bf16_t* zero, uint32_t idx_lds, int topk,
                                                int64_t ntok, int wave, int lane) {
  static_assert(LOADS_OP == 4, "four A loads per wave per stage");
  int rr[4], pos[4];
  uint32_t ad[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int ci = (wave * LOADS_OP + u) * 64 + lane;
    rr[u] = ci / CPR;
    pos[u] = ci % CPR;
    ad[u] = idx_lds + 4 * rr[u];
  }
  int v[4];
  asm volatile(
      "ds_read_b32 %0, %4\n\t"
      "ds_read_b32 %1, %5\n\t"
      "ds_read_b32 %2, %6\n\t"
      "ds_read_b32 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
      : "memory");
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int64_t tok = v[u] / topk;
    tok = tok < 0 ? 0 : (tok >= ntok ? ntok - 1 : tok);
    const int c = tr_swz(rr[u], pos[u]);
    const bf16_t* src = row0 + rr[u] < row_end ? x + tok * ld + col0 + c * 8 : zero + c * 8;
    __builtin_amdgcn_global_load_lds(src, lds_op + (wave * LOADS_OP + u) * 1024, 16, 0, 0);
  }
}

// Byte offset (within an operand's stage) of this lane's transposed read of
// 4 rows x 4 columns for the fragment of columns [col0, col0 + 32) at k
// step 0; `second` selects rows + 4. Adding 16 * PITCH moves to the next k
// step (the swizzle repeats every 8 rows).
template <int PITCH>
__device__ __forceinline__ int tr_frag_off(int col0, int lane, int second) {
  const int g = lane >> 4, s = lane & 15;
  const int col = col0 + 16 * (g & 1) + 4 * (s & 3);
  const int row = 8 * (g >> 1) + (s >> 2) + 4 * second;
  return row * PITCH + (tr_swz(row, col >> 3) << 4) + (col & 7) * 2;
}

// The eight transposed reads of one 16-row k step (two halves of two A and
// two B fragments), waited for inside the same statement. Written as inline
// assembly: the compiler treats the builtin as possibly aliasing the
// in-flight direct-to-LDS loads and would wait for all of them first. The
// addresses are LDS byte addresses.
__device__ __forceinline__ void tr_read_kstep(const uint32_t (&ad)[8], tr_v4i16 (&v)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
        "v"(ad[7])
      : "memory");
}

template <typename Cfg, bool kDense, bool kGather>
__global__ __launch_bounds__(Cfg::NT) void wgrad_tr_kernel(const WgradArgs p,
                                                           const bf16_t* __restrict__ zero) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, NS = Cfg::NS;
  constexpr int kIdxSlots = kGather ? NS * (Cfg::NT / 64) : 0;  // NS slots of 256 B per wave
  constexpr int kLoads = Cfg::LOADS + (kGather ? 1 : 0);         // per wave per stage
  __shared__ __attribute__((aligned(1024))) char smem[NS * Cfg::STAGE + kIdxSlots * 256];

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
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const bf16_t* A = static_cast<const bf16_t*>(p.a);
  const bf16_t* B = static_cast<const bf16_t*>(p.b);
  const int a_col = mt * BM, b_col = nt * BN;

  // Fragment offsets: A side (second MFMA operand, the m index), B side
  // (first operand, the n index); [sub-tile][first / second half of k].
  int a_off[2][2], b_off[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      a_off[i][h] = tr_frag_off<Cfg::A_PITCH>(wm * 64 + i * 32, lane, h);
      b_off[i][h] = Cfg::A_BYTES + tr_frag_off<Cfg::B_PITCH>(wn * 64 + i * 32, lane, h);
    }

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // LDS byte address of smem (the low 32 bits of its generic address).
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
  const int nk = static_cast<int>((r1 - r0 + kTrKT - 1) / kTrKT);
  // Gather: this wave's perm slots (slot t % NS holds stage t's entries,
  // fetched with the loads of stage t - NS + 1).
  char* idx_slots = smem + NS * Cfg::STAGE + wave * NS * 256;
  const uint32_t idx_lds = lds_base + NS * Cfg::STAGE + wave * NS * 256;
  const int64_t ntok = kGather ? p.rows_total / p.topk : 0;
  auto issue = [&](int st) {
    char* buf = smem + (st % NS) * Cfg::STAGE;
    const int64_t row0 = r0 + static_cast<int64_t>(st) * kTrKT;
    if (kGather) {
      tr_issue_idx(idx_slots + ((st + NS - 1) % NS) * 256, p.perm,
                   r0 + static_cast<int64_t>(st + NS - 1) * kTrKT, p.rows_total, lane);
      tr_issue_gather<Cfg::A_CPR, Cfg::A_LOADS>(buf, A, p.lda, a_col, row0, r1, zero,
                                                idx_lds + (st % NS) * 256, p.topk, ntok, wave,
                                                lane);
    } else {
      tr_issue<Cfg::A_CPR, Cfg::A_LOADS>(buf, A, p.lda, a_col, row0, r1, zero, wave, lane);
    }
    tr_issue<Cfg::B_CPR, Cfg::B_LOADS>(buf + Cfg::A_BYTES, B, p.ldb, b_col, row0, r1, zero, wave,
                                       lane);
  };
  if (kGather) {
    // the entries of stages 0 .. NS - 2, landed before their row loads
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
      tr_issue_idx(idx_slots + st * 256, p.perm, r0 + static_cast<int64_t>(st) * kTrKT,
                   p.rows_total, lane);
    tr_wait_vm<0>();
  }
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) issue(st);

  for (int s = 0; s < nk; ++s) {
    // This wave's part of stage s has landed once at most NS - 2 stages'
    // loads remain; the barrier makes every wave's part visible and frees
    // the buffer multiplied in iteration s - 1 for stage s + NS - 1. (With
    // a gather, stage s + NS - 1's perm entries came with stage s's loads.)
    tr_wait_vm<kLoads * (NS - 2)>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    issue(s + NS - 1);
    const uint32_t buf = lds_base + (s % NS) * Cfg::STAGE;
#pragma unroll
    for (int ks = 0; ks < kTrKT / 16; ++ks) {
      uint32_t ad[8];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          ad[2 * i + h] = buf + ks * 16 * Cfg::A_PITCH + a_off[i][h];
          ad[4 + 2 * i + h] = buf + ks * 16 * Cfg::B_PITCH + b_off[i][h];
        }
      tr_v4i16 v[8];
      tr_read_kstep(ad, v);
      bf16x8_t af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v[2 * i], v[2 * i + 1], 0, 1, 2, 3, 4, 5, 6, 7));
        bf[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v[4 + 2 * i], v[5 + 2 * i], 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
    }
  }
  // Loads issued for stages past the end target buffers nobody reads, but
  // they must land before the workgroup's LDS is released.
  tr_wait_vm<0>();

  // Lane L holds, for MFMA tile (i, j), row m = i*32 + L%32 of the wave's
  // block and columns n = j*32 + 8*(q/4) + 4*(L/32) + q%4: runs of four.
  const int r32 = lane & 31, g = lane >> 5;
  float* cg = p.c + grp * p.c_group_stride;
  float* cg2 = p.c2 ? p.c2 + grp * p.c_group_stride : nullptr;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = a_col + wm * 64 + i * 32 + r32;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int n = b_col + wn * 64 + j * 32 + 8 * rr + 4 * g;
        if (p.trans_c) {
          // C^T: the 32 lanes of a column n write 32 consecutive floats.
#pragma unroll
          for (int q = 0; q < 4; ++q) cg[static_cast<int64_t>(n + q) * p.ldc + m] = acc[i][j][4 * rr + q];
          continue;
        }
        float* dst = n < p.nsplit ? cg + m * p.ldc + n : cg2 + m * p.ldc + (n - p.nsplit);
        *reinterpret_cast<float4*>(dst) =
            make_float4(acc[i][j][4 * rr], acc[i][j][4 * rr + 1], acc[i][j][4 * rr + 2],
                        acc[i][j][4 * rr + 3]);
      }
  }
}

// Launch over (group, M tile, N tile); M a multiple of 128 (256-row M tiles
// taken when they divide M and still give a workgroup to every CU), N a
// multiple of 128; `zero` a kTrZeroBytes zero buffer.
// kGather: a.perm (a.rows_total entries, at least one) maps rows to slots,
// token = slot / a.topk.
template <bool kDense, bool kGather = false>
void wgrad_tr(const char* name, const WgradArgs& a, int groups, const bf16_t* zero,
              hipStream_t s) {
  if (kGather && a.rows_total < 1) return;
  if (a.M % 256 == 0 &&
      static_cast<int64_t>(groups) * (a.M / 256) * (a.N / 128) >= cu_count()) {
    using Cfg = TrCfg<256, 3>;
    const int64_t blocks = static_cast<int64_t>(groups) * (a.M / 256) * (a.N / 128);
    if (blocks <= 0) return;
    MOE_LAUNCH(name, (wgrad_tr_kernel<Cfg, kDense, kGather>), dim3(static_cast<unsigned>(blocks)),
               dim3(Cfg::NT), 0, s, a, zero);
  } else {
    using Cfg = TrCfg<128, 4>;
    const int64_t blocks = static_cast<int64_t>(groups) * (a.M / 128) * (a.N / 128);
    if (blocks <= 0) return;
    MOE_LAUNCH(name, (wgrad_tr_kernel<Cfg, kDense, kGather>), dim3(static_cast<unsigned>(blocks)),
               dim3(Cfg::NT), 0, s, a, zero);
  }
}

}  // namespace moe
