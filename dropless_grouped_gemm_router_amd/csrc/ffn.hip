// Stage "experts_grouped_swiglu" (kernel_gmm_gpu.json "pieces" suite):
// the gated expert FFN over expert-sorted token-slots, and the shared
// expert (gpu_moe_h100.json records, field "shared").
//
//   H[row]        = SiLU(x[tok] W_gate[e]) * (x[tok] W_up[e])   (gather GEMM, fused epilogue)
//   y_sorted[row] = H[row] W_down[e]                            (grouped GEMM)
//   shared: the same two GEMMs over all tokens, with identity row maps.
//
// Weights arrive in the layer's own layout ([E][d][h] and [E][h][d], N
// contiguous) and are first packed K-contiguous for the MFMA operand
// loads; gate and up are interleaved in 16-column groups so that one
// 32-column MFMA tile carries matching gate and up columns and the SwiGLU
// epilogue needs no data exchange.
#include "gemm_launch.h"
#include "sort_rows.h"

namespace moe {

namespace {

constexpr int kPackTile = 64;

// dst[g][p][k] (K contiguous) from src[g][k][n] (N contiguous), one 64 x 64
// tile per workgroup, 16-byte loads and stores around an LDS transpose.
// interleave == 0: p = n of src0. interleave != 0: dst has 2 * nsrc rows;
// row p takes column 16 * (p / 32) + p % 16 of src0 (gate) when p % 32 < 16,
// else the same column of src1 (up). So the 64 rows of a tile come from four
// runs of 16 consecutive source columns: gate, up, gate, up.
template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(const T* __restrict__ src0,
                                                   const T* __restrict__ src1, T* __restrict__ dst,
                                                   int K, int nsrc, int interleave) {
  constexpr int V = 16 / static_cast<int>(sizeof(T));  // elements per 16 bytes
  __shared__ T tile[kPackTile][kPackTile + 2];          // [k][p]
  const int ndst = interleave ? 2 * nsrc : nsrc;
  const int p0 = blockIdx.x * kPackTile, k0 = blockIdx.y * kPackTile;
  const int64_t gs = static_cast<int64_t>(K) * nsrc;
  const T* s0 = src0 + blockIdx.z * gs;
  const T* s1 = interleave ? src1 + blockIdx.z * gs : s0;
  // Load: piece (kk, c) = 16 bytes of row k0 + kk at tile rows c*V .. c*V + V-1.
  constexpr int kPieces = kPackTile / V;
  for (int i = threadIdx.x; i < kPackTile * kPieces; i += 256) {
    const int kk = i / kPieces, c = (i % kPieces) * V;
    const int pr = p0 + c;
    const T* s = s0;
    int col = pr;
    if (interleave) {
      col = 16 * (pr / 32) + pr % 16;
      if (pr % 32 >= 16) s = s1;
    }
    const u32x4 v = *reinterpret_cast<const u32x4*>(s + static_cast<int64_t>(k0 + kk) * nsrc + col);
    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int q = 0; q < V; ++q) tile[kk][c + q] = e[q];
  }
  __syncthreads();
  // Store: piece (pp, c) = 16 bytes of dst row p0 + pp at k0 + c*V.
  T* d = dst + blockIdx.z * static_cast<int64_t>(ndst) * K;
  for (int i = threadIdx.x; i < kPackTile * kPieces; i += 256) {
    const int pp = i / kPieces, c = (i % kPieces) * V;
    u32x4 v;
    T* e = reinterpret_cast<T*>(&v);
#pragma unroll
    for (int q = 0; q < V; ++q) e[q] = tile[c + q][pp];
    *reinterpret_cast<u32x4*>(d + static_cast<int64_t>(p0 + pp) * K + k0 + c) = v;
  }
}

// bf16 variant without LDS: one 64 x 64 tile per wave, lane 8 kb + pb
// transposing the 8 x 8 block of source rows k0 + 8 kb + i and destination
// rows p0 + 8 pb + j in registers. Word m of destination row j pairs rows
// 2m and 2m + 1 of column j, i.e. the low (j even) or high (j odd) halves of
// word j / 2 of those two source rows, one byte-select each. Eight lanes
// read, and eight lanes write, 128 contiguous bytes of one row.
__global__ __launch_bounds__(256) void pack_bf16_kernel(const bf16_t* __restrict__ src0,
                                                        const bf16_t* __restrict__ src1,
                                                        bf16_t* __restrict__ dst, int K, int nsrc,
                                                        int interleave) {
  const int ndst = interleave ? 2 * nsrc : nsrc;
  const int tiles_p = ndst / kPackTile;
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= tiles_p * (K / kPackTile)) return;
  const int lane = threadIdx.x & 63, kb = lane >> 3, pb = lane & 7;
  const int pr = (tile % tiles_p) * kPackTile + 8 * pb;
  const int k0 = (tile / tiles_p) * kPackTile + 8 * kb;
  const int64_t gs = static_cast<int64_t>(K) * nsrc;
  const bf16_t* s = src0 + blockIdx.z * gs;
  int col = pr;
  if (interleave) {
    col = 16 * (pr / 32) + pr % 16;
    if (pr % 32 >= 16) s = src1 + blockIdx.z * gs;
  }
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = *reinterpret_cast<const u32x4*>(s + static_cast<int64_t>(k0 + i) * nsrc + col);
  bf16_t* d = dst + blockIdx.z * static_cast<int64_t>(ndst) * K;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x4 o;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      o[m] = __builtin_amdgcn_perm(v[2 * m + 1][j / 2], v[2 * m][j / 2],
                                   (j & 1) ? 0x07060302u : 0x05040100u);
    *reinterpret_cast<u32x4*>(d + static_cast<int64_t>(pr + j) * K + k0) = o;
  }
}

// Several bf16 packs in one launch (the routed gate|up and down weights and
// the shared expert's, 27 MiB at the measured shape, were four launches of a
// few microseconds each). Job j packs `groups` matrices as pack_bf16_kernel
// does; the flat wave-tile index runs over the jobs in order.
struct PackJob {
  const bf16_t* s0;
  const bf16_t* s1;
  bf16_t* dst;
  int K, nsrc, interleave, groups;
};
constexpr int kMaxPackJobs = 4;
struct PackJobs {
  PackJob job[kMaxPackJobs];
  int end[kMaxPackJobs];  // exclusive end of each job's wave tiles
  int n;
};

__global__ __launch_bounds__(256) void pack_bf16_jobs_kernel(const PackJobs jobs) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  int j = 0;
  while (j < jobs.n && t >= jobs.end[j]) ++j;
  if (j >= jobs.n) return;
  const PackJob& b = jobs.job[j];
  const int local = t - (j ? jobs.end[j - 1] : 0);
  const int ndst = b.interleave ? 2 * b.nsrc : b.nsrc;
  const int tiles_p = ndst / kPackTile;
  const int per_group = tiles_p * (b.K / kPackTile);
  const int grp = local / per_group, tile = local % per_group;
  const int lane = threadIdx.x & 63, kb = lane >> 3, pb = lane & 7;
  const int pr = (tile % tiles_p) * kPackTile + 8 * pb;
  const int k0 = (tile / tiles_p) * kPackTile + 8 * kb;
  const int64_t gs = static_cast<int64_t>(b.K) * b.nsrc;
  const bf16_t* src = b.s0 + grp * gs;
  int col = pr;
  if (b.interleave) {
    col = 16 * (pr / 32) + pr % 16;
    if (pr % 32 >= 16) src = b.s1 + grp * gs;
  }
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(k0 + i) * b.nsrc + col);
  bf16_t* d = b.dst + grp * static_cast<int64_t>(ndst) * b.K;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    u32x4 o;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      o[m] = __builtin_amdgcn_perm(v[2 * m + 1][jj / 2], v[2 * m][jj / 2],
                                   (jj & 1) ? 0x07060302u : 0x05040100u);
    *reinterpret_cast<u32x4*>(d + static_cast<int64_t>(pr + jj) * b.K + k0) = o;
  }
}

void pack_bf16_jobs(PackJobs& jobs, hipStream_t s) {
  int total = 0;
  for (int j = 0; j < jobs.n; ++j) {
    const PackJob& b = jobs.job[j];
    const int ndst = b.interleave ? 2 * b.nsrc : b.nsrc;
    total += (ndst / kPackTile) * (b.K / kPackTile) * b.groups;
    jobs.end[j] = total;
  }
  if (total == 0) return;
  MOE_LAUNCH("pack_weights", pack_bf16_jobs_kernel, dim3((total + 3) / 4), dim3(256), 0, s, jobs);
}

template <typename T>
void pack(const void* s0, const void* s1, void* dst, int groups, int K, int nsrc, bool il,
          hipStream_t s) {
  const int ndst = il ? 2 * nsrc : nsrc;
  if (std::is_same<T, bf16_t>::value) {
    const int tiles = (ndst / kPackTile) * (K / kPackTile);
    MOE_LAUNCH("pack_weights", pack_bf16_kernel, dim3((tiles + 3) / 4, 1, groups), dim3(256), 0, s,
               static_cast<const bf16_t*>(s0), static_cast<const bf16_t*>(s1),
               static_cast<bf16_t*>(dst), K, nsrc, il ? 1 : 0);
    return;
  }
  MOE_LAUNCH("pack_weights", pack_kernel<T>, dim3(ndst / kPackTile, K / kPackTile, groups), dim3(256), 0,
                     s, static_cast<const T*>(s0), static_cast<const T*>(s1),
                     static_cast<T*>(dst), K, nsrc, il ? 1 : 0);
}



// Fused gather-sum: the shared down GEMM writes out[t] = sum_i w y + shared.
struct FuseCombine {
  void* out;
  const void* y_sorted;
  const float* topk_w;
  const int32_t* inv_perm;
};

template <typename T>
void routed_ffn(const moe_problem& p, const void* x, const moe_routing& r, const void* gu,
                const void* dn, void* h_sorted, void* y_sorted, void* sa, void* sb, void* x_sorted,
                void* tiles256, hipStream_t s) {
  const int64_t S = p.tokens * p.top_k;
  const int64_t max_tiles = (S + p.block_m - 1) / p.block_m + p.experts;
  if (x_sorted)
    MOE_LAUNCH("sort_rows", sort_rows_kernel<T>, dim3(sort_rows_blocks(S)), dim3(kSortThreads),
               0, s, static_cast<const T*>(x), r.perm, p.top_k, S, p.d_model,
               static_cast<T*>(x_sorted));
  GemmArgs a{};
  a.a = x_sorted ? x_sorted : x;
  a.lda = p.d_model;
  a.perm = r.perm;
  a.topk = p.top_k;
  a.b = gu;
  a.b_group_stride = static_cast<int64_t>(2) * p.d_hidden * p.d_model;
  a.N = 2 * p.d_hidden;
  a.K = p.d_model;
  a.tiles = r.tiles;
  a.num_tiles = r.num_tiles;
  a.c = h_sorted;
  a.ldc = p.d_hidden;
  a.sa = sa;
  a.sb = sb;
  a.lds = 2 * static_cast<int64_t>(p.d_hidden);
  // 256-row tile list (by expert, from the offsets) when block_m is smaller
  // and the experts are full enough: both GEMMs then run on the wide engine
  // (the gate/up GEMM whenever it gathers its rows).
  int32_t* t256 = static_cast<int32_t*>(tiles256);
  const int64_t mt256 = (S + kRetileBm - 1) / kRetileBm + p.experts;
  const bool retiled = retile_rows(p);
  if (retiled) (void)launch_retile(r.expert_offsets, p.experts, kRetileBm, p.capacity, t256 + 4, t256, s);
  if (retiled && !x_sorted && wide_fits<T>(a)) {
    GemmArgs a256 = a;
    a256.tiles = t256 + 4;
    a256.num_tiles = t256;
    grouped_gemm<T, true, kEpiSwiglu>("gemm_gate_up", a256, kRetileBm, mt256, s);
  } else if (x_sorted) {
    grouped_gemm<T, false, kEpiSwiglu>("gemm_gate_up", a, p.block_m, max_tiles, s);
  } else {
    grouped_gemm<T, true, kEpiSwiglu>("gemm_gate_up", a, p.block_m, max_tiles, s);
  }

  GemmArgs b{};
  b.a = h_sorted;
  b.lda = p.d_hidden;
  b.b = dn;
  b.b_group_stride = static_cast<int64_t>(p.d_model) * p.d_hidden;
  b.N = p.d_model;
  b.K = p.d_hidden;
  b.tiles = r.tiles;
  b.num_tiles = r.num_tiles;
  b.c = y_sorted;
  b.ldc = p.d_model;
  if (retiled && wide_fits<T>(b)) {
    // 256-row tiles on the wide engine for the down GEMM (its output stores
    // dominate, and the wide engine parks them as whole row pieces)
    b.tiles = t256 + 4;
    b.num_tiles = t256;
    grouped_gemm<T, false, kEpiStore>("gemm_down", b, kRetileBm, mt256, s);
  } else {
    grouped_gemm<T, false, kEpiStore>("gemm_down", b, p.block_m, max_tiles, s);
  }
}

template <typename T>
void shared_ffn(const moe_problem& p, const void* x, const void* sgu, const void* sdn, void* hs,
                void* out, void* sa, void* sb, const FuseCombine* fuse, hipStream_t s) {
  GemmArgs a{};
  a.a = x;
  a.lda = p.d_model;
  a.b = sgu;
  a.N = 2 * p.d_shared;
  a.K = p.d_model;
  a.M = p.tokens;
  a.c = hs;
  a.ldc = p.d_shared;
  a.sa = sa;
  a.sb = sb;
  a.lds = 2 * static_cast<int64_t>(p.d_shared);
  dense_gemm<T, kEpiSwiglu>("shared_gate_up", a, s);

  GemmArgs b{};
  b.a = hs;
  b.lda = p.d_shared;
  b.b = sdn;
  b.N = p.d_model;
  b.K = p.d_shared;
  b.M = p.tokens;
  b.c = out;
  b.ldc = p.d_model;
  if (fuse) {
    b.c = fuse->out;
    b.gy = fuse->y_sorted;
    b.gw = fuse->topk_w;
    b.ginv = fuse->inv_perm;
    b.gk = p.top_k;
    dense_gemm<T, kEpiCombine>("shared_down_combine", b, s);
  } else {
    dense_gemm<T, kEpiStore>("shared_down", b, s);
  }
}

// The routed experts' weights (and, with `shared`, the shared expert's) in
// the GEMMs' layout (workspace). Depends on the weights alone, so it may run
// on another stream before the routing. bf16: one launch for all of them.
template <typename T>
void pack_weights_t(const moe_problem& p, const moe_weights& w, void* ws, bool training,
                    bool shared, hipStream_t s) {
  const FfnLayout L = ffn_layout(p, training);
  char* W = static_cast<char*>(ws);
  const int E = p.experts, d = p.d_model, h = p.d_hidden, hs = p.d_shared;
  shared = shared && hs > 0;
  if (std::is_same<T, bf16_t>::value) {
    PackJobs jobs{};
    auto add = [&](const void* a, const void* b, char* dst, int groups, int K, int nsrc, bool il) {
      jobs.job[jobs.n++] = PackJob{static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(b),
                                   reinterpret_cast<bf16_t*>(dst), K, nsrc, il ? 1 : 0, groups};
    };
    add(w.w_gate, w.w_up, W + L.gu_packed, E, d, h, true);
    add(w.w_down, nullptr, W + L.down_packed, E, h, d, false);
    if (shared) {
      add(w.ws_gate, w.ws_up, W + L.sgu_packed, 1, d, hs, true);
      add(w.ws_down, nullptr, W + L.sdown_packed, 1, hs, d, false);
    }
    pack_bf16_jobs(jobs, s);
    return;
  }
  pack<T>(w.w_gate, w.w_up, W + L.gu_packed, E, d, h, true, s);
  pack<T>(w.w_down, nullptr, W + L.down_packed, E, h, d, false, s);
  if (shared) {
    pack<T>(w.ws_gate, w.ws_up, W + L.sgu_packed, 1, d, hs, true, s);
    pack<T>(w.ws_down, nullptr, W + L.sdown_packed, 1, hs, d, false, s);
  }
}

// Routed part: pack the expert weights (unless `packed`: already enqueued,
// possibly on another stream, and ordered before this call's GEMMs by the
// caller), gate/up GEMM with SwiGLU, down GEMM.
template <typename T>
void ffn_routed_t(const moe_problem& p, const void* x, const moe_weights& w,
                  const moe_routing& r, void* y_sorted, void* saved, void* ws, void* x_sorted,
                  hipStream_t s, bool packed = false) {
  const FfnLayout L = ffn_layout(p, saved != nullptr);
  char* W = static_cast<char*>(ws);
  char* SV = static_cast<char*>(saved);
  const int h = p.d_hidden;
  if (!packed) pack_weights_t<T>(p, w, ws, saved != nullptr, false, s);
  T* hbuf = (saved && !std::is_same<T, bf16_t>::value) ? reinterpret_cast<T*>(SV + L.sv_h)
                                                        : reinterpret_cast<T*>(W + L.h_sorted);
  T* sa = saved ? reinterpret_cast<T*>(SV + L.sv_ab) : nullptr;
  T* sb = saved ? sa + h : nullptr;
  routed_ffn<T>(p, x, r, W + L.gu_packed, W + L.down_packed, hbuf, y_sorted, sa, sb, x_sorted,
                W + L.tiles256, s);
}

// Shared part (d_shared > 0): pack its weights, its two GEMMs. It touches
// only its own workspace and saved regions, so it may run beside the
// routed part on another stream.
template <typename T>
void ffn_shared_t(const moe_problem& p, const void* x, const moe_weights& w, void* shared_out,
                  void* saved, void* ws, const FuseCombine* fuse, hipStream_t s,
                  bool packed = false) {
  const FfnLayout L = ffn_layout(p, saved != nullptr);
  char* W = static_cast<char*>(ws);
  char* SV = static_cast<char*>(saved);
  const int d = p.d_model, hs = p.d_shared;
  if (!packed) {
    pack<T>(w.ws_gate, w.ws_up, W + L.sgu_packed, 1, d, hs, true, s);
    pack<T>(w.ws_down, nullptr, W + L.sdown_packed, 1, hs, d, false, s);
  }
  T* hsb = saved ? reinterpret_cast<T*>(SV + L.sv_sh) : reinterpret_cast<T*>(W + L.h_shared);
  T* ssa = saved ? reinterpret_cast<T*>(SV + L.sv_sab) : nullptr;
  T* ssb = saved ? ssa + hs : nullptr;
  shared_ffn<T>(p, x, W + L.sgu_packed, W + L.sdown_packed, hsb, shared_out, ssa, ssb, fuse, s);
}

template <typename T>
hipError_t ffn_fwd_t(const moe_problem& p, const void* x, const moe_weights& w,
                     const moe_routing& r, void* y_sorted, void* shared_out, void* saved,
                     void* ws, void* x_sorted, const FuseCombine* fuse, hipStream_t s) {
  pack_weights_t<T>(p, w, ws, saved != nullptr, true, s);
  ffn_routed_t<T>(p, x, w, r, y_sorted, saved, ws, x_sorted, s, true);
  if (p.d_shared > 0) ffn_shared_t<T>(p, x, w, shared_out, saved, ws, fuse, s, true);
  return hipGetLastError();
}

}  // namespace

FfnLayout ffn_layout(const moe_problem& p, bool training) {
  const size_t es = p.dtype == MOE_BF16 ? 2 : 4;
  const size_t E = p.experts, d = p.d_model, h = p.d_hidden, hs = p.d_shared;
  const size_t T = static_cast<size_t>(p.tokens), S = T * p.top_k;
  FfnLayout L{};
  size_t o = 0;
  L.gu_packed = o;    o = align_up(o + E * 2 * h * d * es, 256);
  L.down_packed = o;  o = align_up(o + E * d * h * es, 256);
  L.sgu_packed = o;   o = align_up(o + 2 * hs * d * es, 256);
  L.sdown_packed = o; o = align_up(o + d * hs * es, 256);
  // The routed H stays in the workspace unless the fp32 backward needs it
  // saved (the bf16 backward recomputes it from the saved pre-activations).
  const bool save_h = training && p.dtype != MOE_BF16;
  L.h_sorted = o;     o = align_up(o + (save_h ? 0 : S * h * es), 256);
  L.h_shared = o;     o = align_up(o + (training ? 0 : T * hs * es), 256);
  L.tiles256 = o;     o = align_up(o + retile_bytes(static_cast<int64_t>(S), p.experts), 256);
  L.total = o;
  size_t v = 0;
  L.sv_ab = v;  v = align_up(v + S * 2 * h * es, 256);
  L.sv_h = v;   v = align_up(v + (p.dtype == MOE_BF16 ? 0 : S * h * es), 256);
  L.sv_sab = v; v = align_up(v + T * 2 * hs * es, 256);
  L.sv_sh = v;  v = align_up(v + T * hs * es, 256);
  L.sv_total = v;
  return L;
}

hipError_t launch_ffn_fwd(const moe_problem& p, const void* x, const moe_weights& w,
                          const moe_routing& r, void* y_sorted, void* shared_out, void* saved,
                          void* ws, hipStream_t s) {
  if (p.dtype == MOE_BF16)
    return ffn_fwd_t<bf16_t>(p, x, w, r, y_sorted, shared_out, saved, ws, nullptr, nullptr, s);
  return ffn_fwd_t<float>(p, x, w, r, y_sorted, shared_out, saved, ws, nullptr, nullptr, s);
}

ForwardLayout forward_layout(const moe_problem& p, int dispatch, bool training) {
  const size_t es = p.dtype == MOE_BF16 ? 2 : 4;
  const size_t T = static_cast<size_t>(p.tokens), S = T * p.top_k;
  ForwardLayout L{};
  L.fused = dispatch == MOE_DISPATCH_FUSED_GSUM && p.d_shared > 0 && p.top_k <= kCombineMaxK;
  // The permute scratch has a region of its own: the shared expert may be
  // packing its weights while the permutation runs.
  size_t o = align_up(ffn_layout(p, training).total, 256);
  L.permute = o;
  o = align_up(o + permute_ws_bytes(static_cast<int64_t>(S), p.experts), 256);
  L.shared_out = o;
  if (p.d_shared > 0 && !L.fused) o = align_up(o + T * p.d_model * es, 256);
  L.x_sorted = o;
  if (dispatch == MOE_DISPATCH_SORTED) o = align_up(o + S * p.d_model * es, 256);
  L.total = o > 256 ? o : 256;
  return L;
}

namespace {

// route -> permute -> routed FFN on s. With a fork, the routed weights were
// packed on its side stream before its mark, which s waits for first.
hipError_t routed_forward(const moe_problem& p, const void* x, const moe_weights& w,
                          const moe_routing& r, void* y_sorted, void* saved, void* ws,
                          void* x_sorted, void* permute_ws, hipStream_t s,
                          StreamFork* fork = nullptr, bool packed = false) {
  hipError_t e = launch_route(p.dtype, x, w.w_router, p.tokens, p.d_model, p.experts, p.top_k,
                              r.topk_idx, r.topk_w, s);
  if (e != hipSuccess) return e;
  e = launch_permute(p.tokens, p.top_k, p.experts, p.block_m, p.capacity, r.topk_idx,
                     r.expert_offsets, r.perm, r.inv_perm, r.tiles, r.num_tiles, permute_ws, s);
  if (e != hipSuccess) return e;
  if (fork) {
    e = fork->wait_mark();
    if (e != hipSuccess) return e;
  }
  packed = packed || fork != nullptr;
  if (p.dtype == MOE_BF16) ffn_routed_t<bf16_t>(p, x, w, r, y_sorted, saved, ws, x_sorted, s, packed);
  else ffn_routed_t<float>(p, x, w, r, y_sorted, saved, ws, x_sorted, s, packed);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const moe_problem& p, int dispatch, const void* x, const moe_weights& w,
                          const moe_routing& r, void* y_sorted, void* saved, void* out, void* ws,
                          hipStream_t s, hipStream_t side) {
  const ForwardLayout L = forward_layout(p, dispatch, saved != nullptr);
  char* W = static_cast<char*>(ws);
  void* shared_out = p.d_shared > 0 && !L.fused ? W + L.shared_out : nullptr;
  void* x_sorted = dispatch == MOE_DISPATCH_SORTED ? W + L.x_sorted : nullptr;
  const bool bf = p.dtype == MOE_BF16;
  // Unfused, the shared expert depends on nothing but the tokens and its
  // weights: with a second stream it runs there beside the routed path, and
  // the combine waits for it. From 65536 tokens on it starts after the
  // permutation: beside route and permute its persistent GEMMs hold the CUs
  // the small permute kernels need (count and scan stretched to tens of
  // times their own duration), and forward steps at 131072 tokens measured
  // 1.45 -> 1.42 ms; at 16384 tokens the early start overlaps more of the
  // shared expert and is the faster one (train step 0.78 vs 0.79 ms).
  if (p.d_shared > 0 && !L.fused && side != nullptr && side != s && p.tokens >= 65536) {
    if (bf) pack_weights_t<bf16_t>(p, w, ws, saved != nullptr, true, s);
    else pack_weights_t<float>(p, w, ws, saved != nullptr, true, s);
    hipError_t e = launch_route(p.dtype, x, w.w_router, p.tokens, p.d_model, p.experts, p.top_k,
                                r.topk_idx, r.topk_w, s);
    if (e != hipSuccess) return e;
    e = launch_permute(p.tokens, p.top_k, p.experts, p.block_m, p.capacity, r.topk_idx,
                       r.expert_offsets, r.perm, r.inv_perm, r.tiles, r.num_tiles, W + L.permute, s);
    if (e != hipSuccess) return e;
    StreamFork fork(s, side);
    e = fork.fork();
    if (e != hipSuccess) return e;
    if (bf) ffn_shared_t<bf16_t>(p, x, w, shared_out, saved, ws, nullptr, fork.side(), true);
    else ffn_shared_t<float>(p, x, w, shared_out, saved, ws, nullptr, fork.side(), true);
    if (bf) ffn_routed_t<bf16_t>(p, x, w, r, y_sorted, saved, ws, x_sorted, s, true);
    else ffn_routed_t<float>(p, x, w, r, y_sorted, saved, ws, x_sorted, s, true);
    e = hipGetLastError();
    if (e == hipSuccess) e = fork.join();
    if (e != hipSuccess) return e;
    return launch_combine(p.dtype, p.tokens, p.top_k, p.d_model, y_sorted, r.topk_w, r.inv_perm,
                          shared_out, out, s);
  }
  if (p.d_shared > 0 && !L.fused && side != nullptr && side != s) {
    // The routed weights are packed first on the side stream too, beside the
    // router kernel (which leaves room on every CU for the pack kernel's
    // workgroups); the routed GEMMs wait for that mark.
    StreamFork fork(s, side);
    hipError_t e = fork.fork();
    if (e != hipSuccess) return e;
    if (bf) pack_weights_t<bf16_t>(p, w, ws, saved != nullptr, true, fork.side());
    else pack_weights_t<float>(p, w, ws, saved != nullptr, true, fork.side());
    e = fork.mark();
    if (e != hipSuccess) return e;
    if (bf) ffn_shared_t<bf16_t>(p, x, w, shared_out, saved, ws, nullptr, fork.side(), true);
    else ffn_shared_t<float>(p, x, w, shared_out, saved, ws, nullptr, fork.side(), true);
    e = routed_forward(p, x, w, r, y_sorted, saved, ws, x_sorted, W + L.permute, s, &fork);
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) e = fork.join();
    if (e != hipSuccess) return e;
    return launch_combine(p.dtype, p.tokens, p.top_k, p.d_model, y_sorted, r.topk_w, r.inv_perm,
                          shared_out, out, s);
  }
  // One stream: every weight pack first (one launch in bf16), then the path.
  if (bf) pack_weights_t<bf16_t>(p, w, ws, saved != nullptr, true, s);
  else pack_weights_t<float>(p, w, ws, saved != nullptr, true, s);
  hipError_t e =
      routed_forward(p, x, w, r, y_sorted, saved, ws, x_sorted, W + L.permute, s, nullptr, true);
  if (e != hipSuccess) return e;
  if (p.d_shared > 0) {
    // fused: the shared down GEMM's epilogue reads the routed outputs
    const FuseCombine fuse{out, y_sorted, r.topk_w, r.inv_perm};
    if (bf) ffn_shared_t<bf16_t>(p, x, w, shared_out, saved, ws, L.fused ? &fuse : nullptr, s, true);
    else ffn_shared_t<float>(p, x, w, shared_out, saved, ws, L.fused ? &fuse : nullptr, s, true);
  }
  e = hipGetLastError();
  if (e != hipSuccess || L.fused) return e;
  return launch_combine(p.dtype, p.tokens, p.top_k, p.d_model, y_sorted, r.topk_w, r.inv_perm,
                        shared_out, out, s);
}

}  // namespace moe
