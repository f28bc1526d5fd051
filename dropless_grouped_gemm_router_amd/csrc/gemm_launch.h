// Host-side launchers of the grouped GEMM engines (gemm_core.h,
// gemm_wide.h), shared by the forward and backward stages.
#pragma once

#include <type_traits>

#include "gemm_wide.h"

namespace moe {

// Persistent launch: one workgroup per resident slot, at most one per item.
template <typename T, typename Cfg, bool kGather, int kEpi, bool kDense>
void gemm(const char* name, const GemmArgs& a, int64_t row_tiles, hipStream_t s) {
  if (kDense) row_tiles = (a.M + Cfg::BM - 1) / Cfg::BM;
  if (row_tiles <= 0) return;
  const int64_t work = row_tiles * (a.N / Cfg::BN);
  const int slots = persistent_slots(
      reinterpret_cast<const void*>(&gemm_kernel<T, Cfg, kGather, kEpi, kDense>), Cfg::NT);
  const unsigned grid = static_cast<unsigned>(work < slots ? work : slots);
  MOE_LAUNCH(name, (gemm_kernel<T, Cfg, kGather, kEpi, kDense>), dim3(grid), dim3(Cfg::NT), 0, s,
             a, static_cast<int>(work));
}

template <bool kGather, int kEpi, bool kDense>
void wide_gemm(const char* name, const GemmArgs& a, int64_t row_tiles, hipStream_t s) {
  if (kDense) row_tiles = (a.M + WideCfg::BM - 1) / WideCfg::BM;
  if (row_tiles <= 0) return;
  const int64_t work = row_tiles * (a.N / WideCfg::BN);
  const int slots = persistent_slots(
      reinterpret_cast<const void*>(&wide_gemm_kernel<kGather, kEpi, kDense>), WideCfg::NT);
  const unsigned grid = static_cast<unsigned>(work < slots ? work : slots);
  MOE_LAUNCH(name, (wide_gemm_kernel<kGather, kEpi, kDense>), dim3(grid), dim3(WideCfg::NT), 0, s,
             a, a.tiles, a.num_tiles, static_cast<int>(work));
}

// The wide engine takes bf16 operands with N a multiple of 256, K (and the
// b2 split) a multiple of 64, and lane offsets of 256 weight rows within
// 32 bits.
template <typename T>
bool wide_fits(const GemmArgs& a) {
  const int64_t ldb = a.ldb ? a.ldb : a.K;
  return std::is_same<T, bf16_t>::value && a.N % 256 == 0 && a.K % 64 == 0 &&
         (a.b2 == nullptr || a.ksplit % 64 == 0) && ldb < (int64_t{1} << 22);
}

// Grouped GEMM over the block_m tile list. block_m 256 in bf16 takes the
// wide engine; otherwise the eight-wave 256-column tile when N allows it,
// else the four-wave 128-column tile.
template <typename T, bool kGather, int kEpi>
void grouped_gemm(const char* name, const GemmArgs& a, int bm, int64_t max_tiles, hipStream_t s) {
  const bool wide = a.N % 256 == 0;
  if (bm == 256) {
    if (wide_fits<T>(a)) wide_gemm<kGather, kEpi, false>(name, a, max_tiles, s);
    else if (wide) gemm<T, Cfg256W, kGather, kEpi, false>(name, a, max_tiles, s);
    else gemm<T, Cfg256N, kGather, kEpi, false>(name, a, max_tiles, s);
  } else if (bm == 128) {
    if (wide) gemm<T, Cfg128W, kGather, kEpi, false>(name, a, max_tiles, s);
    else gemm<T, Cfg128, kGather, kEpi, false>(name, a, max_tiles, s);
  } else if (bm == 64) {
    if (wide) gemm<T, Cfg64W, kGather, kEpi, false>(name, a, max_tiles, s);
    else gemm<T, Cfg64, kGather, kEpi, false>(name, a, max_tiles, s);
  } else {
    gemm<T, Cfg32, kGather, kEpi, false>(name, a, max_tiles, s);
  }
}

// Dense GEMM over all rows (shared expert).
template <typename T, int kEpi>
void dense_gemm(const char* name, const GemmArgs& a, hipStream_t s) {
  if (wide_fits<T>(a)) wide_gemm<false, kEpi, true>(name, a, 1, s);
  else if (a.N % 256 == 0) gemm<T, Cfg128W, false, kEpi, true>(name, a, 1, s);
  else gemm<T, Cfg256N, false, kEpi, true>(name, a, 1, s);
}

}  // namespace moe
