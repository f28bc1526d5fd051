// Train-step backward of the dropless MoE layer (gpu_moe_h100.json header:
// value and gradient with respect to the parameters and the input) for
// L = sum(out * G), with the top-k selection held fixed.
//
//   combine:  dY[slot(t,i)] = w_i G_t,  dw_i = <G_t, y[slot(t,i)]>
//   router:   dl_i = w_i (dw_i - sum_j w_j dw_j);  dW_r = x^T dl;  dx += dl W_r^T
//   experts:  dH = dY W_down^T -> (dA, dB) through SwiGLU with the saved
//             pre-activations; dX_sorted = dA W_gate^T + dB W_up^T;
//             dW_down = H^T dY, dW_gate = X^T dA, dW_up = X^T dB per expert
//   shared:   the same chain with weight 1 over all tokens
//   dx[t] = sum_i dX_sorted[slot(t,i)] + router term + shared term
//
// In bf16, dY is never formed: the down dgrad reads G by token and applies
// w_i after the contraction (gemm_dgrad.h), dw_i = <G W_down^T, H> comes
// from the same accumulators, and dW_down = sum (w_i H)^T G with G's rows
// gathered. fp32 runs the chain as written above.
//
// Every reduction runs in a fixed order with one writer per output (no
// floating-point atomics), so the gradients are deterministic. In bf16 the
// weight gradients take the transposing-LDS-read kernel (gemm_wgrad.h),
// which reads row ranges and gathers token rows through perm itself.
#include "gemm_dgrad.h"
#include "gemm_launch.h"
#include "gemm_wgrad.h"

namespace moe {

namespace {

constexpr int kRowThreads = 256;

template <typename T>
struct V16;  // one 16-byte piece of a row
template <>
struct V16<bf16_t> {
  static constexpr int N = 8;
  __device__ static void load(const bf16_t* p, float* o) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    o[0] = bf16lo(v.x); o[1] = bf16hi(v.x); o[2] = bf16lo(v.y); o[3] = bf16hi(v.y);
    o[4] = bf16lo(v.z); o[5] = bf16hi(v.z); o[6] = bf16lo(v.w); o[7] = bf16hi(v.w);
  }
  __device__ static void store(bf16_t* p, const float* o) {
    uint4 v;
    v.x = pack_bf16x2(o[0], o[1]); v.y = pack_bf16x2(o[2], o[3]);
    v.z = pack_bf16x2(o[4], o[5]); v.w = pack_bf16x2(o[6], o[7]);
    *reinterpret_cast<uint4*>(p) = v;
  }
  // Nontemporal forms, for rows touched once (gathered expert outputs and
  // input gradients, the final grad_x) that should not evict reused data.
  __device__ static void load_nt(const bf16_t* p, float* o) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    o[0] = bf16lo(v.x); o[1] = bf16hi(v.x); o[2] = bf16lo(v.y); o[3] = bf16hi(v.y);
    o[4] = bf16lo(v.z); o[5] = bf16hi(v.z); o[6] = bf16lo(v.w); o[7] = bf16hi(v.w);
  }
  __device__ static void unpack(const u32x4& v, float* o) {
    o[0] = bf16lo(v.x); o[1] = bf16hi(v.x); o[2] = bf16lo(v.y); o[3] = bf16hi(v.y);
    o[4] = bf16lo(v.z); o[5] = bf16hi(v.z); o[6] = bf16lo(v.w); o[7] = bf16hi(v.w);
  }
  __device__ static void store_nt(bf16_t* p, const float* o) {
    u32x4 v;
    v.x = pack_bf16x2(o[0], o[1]); v.y = pack_bf16x2(o[2], o[3]);
    v.z = pack_bf16x2(o[4], o[5]); v.w = pack_bf16x2(o[6], o[7]);
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  }
};
template <>
struct V16<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* o) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
  __device__ static void store(float* p, const float* o) {
    *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
  }
  __device__ static void load_nt(const float* p, float* o) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
  }
  __device__ static void unpack(const u32x4& v, float* o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
  __device__ static void store_nt(float* p, const float* o) {
    const f32x4_t v = {o[0], o[1], o[2], o[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// One wave per token: dY rows, dw by wave reduction, then dl for the kept
// experts (lane i holds rank i; k <= 64). A slot dropped by capacity
// routing (inv_perm -1) has y = 0: dw = 0 and no dY row, while its dl
// still carries the normalisation term.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void combine_bwd_kernel(
    int64_t ntok, int k, int d, const T* __restrict__ G, const T* __restrict__ y,
    const float* __restrict__ w, const int32_t* __restrict__ inv_perm, T* __restrict__ dY,
    float* __restrict__ dl) {
  constexpr int N = V16<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kRowThreads / 64) + (threadIdx.x >> 6);
  if (t >= ntok) return;
  float my_dw = 0.0f, my_w = 0.0f;
  for (int i = 0; i < k; ++i) {
    const int64_t slot = inv_perm[t * k + i];
    const float wi = w[t * k + i];
    float dot = 0.0f;
    for (int c = lane * N; slot >= 0 && c < d; c += 64 * N) {
      float g[N], yv[N], o[N];
      V16<T>::load(G + t * d + c, g);
      V16<T>::load_nt(y + slot * d + c, yv);
#pragma unroll
      for (int q = 0; q < N; ++q) {
        dot = __builtin_fmaf(g[q], yv[q], dot);
        o[q] = wi * g[q];
      }
      V16<T>::store(dY + slot * d + c, o);
    }
    dot = wave_sum(dot);
    if (lane == i) {
      my_dw = dot;
      my_w = wi;
    }
  }
  const float s = wave_sum(lane < k ? my_w * my_dw : 0.0f);
  if (lane < k) dl[t * k + lane] = my_w * (my_dw - s);
}

// Router weight gradient, stage 1: per block_m piece of an expert's sorted
// rows, partial[piece][j] = sum over the piece's rows, in order, of
// x[tok][j] * dl[slot]. The pieces are those of the dropless tile list
// (experts ascending, block_m rows each, the last partial), derived from
// the expert offsets: under capacity routing the dropped slots still carry
// router gradient, though no GEMM tile covers their rows.
// k = K <= 8: lane i reads slot i's sorted row and weight, the wave
// broadcasts them, the token's G piece is read once and all K expert-row
// loads of a piece are issued together. Each rank's dot product still sums
// over the pieces in order and then over the wave as in combine_bwd_kernel,
// so the results are the same bits.
template <typename T, int K>
__global__ __launch_bounds__(kRowThreads) void combine_bwd_k_kernel(
    int64_t ntok, int d, const T* __restrict__ G, const T* __restrict__ y,
    const float* __restrict__ w, const int32_t* __restrict__ inv_perm, T* __restrict__ dY,
    float* __restrict__ dl) {
  constexpr int N = V16<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kRowThreads / 64) + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int my_slot = lane < K ? inv_perm[t * K + lane] : 0;
  const float my_w = lane < K ? w[t * K + lane] : 0.0f;
  int64_t slot[K];
  float wi[K], dot[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    slot[i] = __builtin_amdgcn_readlane(my_slot, i);
    wi[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), i));
    dot[i] = 0.0f;
  }
  for (int c = lane * N; c < d; c += 64 * N) {
    float g[N], yv[K][N];
    V16<T>::load(G + t * d + c, g);
#pragma unroll
    for (int i = 0; i < K; ++i)
      if (slot[i] >= 0) V16<T>::load_nt(y + slot[i] * d + c, yv[i]);
#pragma unroll
    for (int i = 0; i < K; ++i)
      if (slot[i] >= 0) {
        float o[N];
#pragma unroll
        for (int q = 0; q < N; ++q) {
          dot[i] = __builtin_fmaf(g[q], yv[i][q], dot[i]);
          o[q] = wi[i] * g[q];
        }
        V16<T>::store(dY + slot[i] * d + c, o);
      }
  }
  float my_dw = 0.0f;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const float di = wave_sum(dot[i]);
    if (lane == i) my_dw = di;
  }
  const float s = wave_sum(lane < K ? my_w * my_dw : 0.0f);
  if (lane < K) dl[t * K + lane] = my_w * (my_dw - s);
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void router_partial_kernel(
    const T* __restrict__ x, int d, int topk, const int32_t* __restrict__ perm,
    const float* __restrict__ dl, const int32_t* __restrict__ offsets, int E, int bm,
    float* __restrict__ partial) {
  __shared__ int64_t tok[256];  // rows of one piece (block_m <= 256)
  __shared__ float dv[256];
  __shared__ int piece_row0, piece_rows;
  const int tile = blockIdx.x;
  if (threadIdx.x == 0) {
    int n = 0, r0 = 0, nr = 0;
    for (int e = 0; e < E; ++e) {
      const int cnt = offsets[e + 1] - offsets[e];
      const int np = (cnt + bm - 1) / bm;
      if (tile < n + np) {
        const int r = (tile - n) * bm;
        r0 = offsets[e] + r;
        nr = cnt - r < bm ? cnt - r : bm;
        break;
      }
      n += np;
    }
    piece_row0 = r0;
    piece_rows = nr;
  }
  __syncthreads();
  const int row0 = piece_row0, rows = piece_rows;
  if (rows == 0) return;
  for (int r = threadIdx.x; r < rows; r += kRowThreads) {
    const int32_t s = perm[row0 + r];
    tok[r] = s / topk;
    dv[r] = dl[s];
  }
  __syncthreads();
  // Two adjacent columns per thread (d is even); eight rows' values are
  // loaded before they are multiplied in, row order kept per column.
  constexpr int kBatch = 8;
  auto load2 = [&](int r, int j, float& v0, float& v1) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(x + tok[r] * d + j);
      v0 = bf16lo(u);
      v1 = bf16hi(u);
    } else {
      const float2 u = *reinterpret_cast<const float2*>(x + tok[r] * d + j);
      v0 = u.x;
      v1 = u.y;
    }
  };
  for (int j = 2 * threadIdx.x; j < d; j += 2 * kRowThreads) {
    float a0 = 0.0f, a1 = 0.0f;
    int r = 0;
    for (; r + kBatch <= rows; r += kBatch) {
      float v0[kBatch], v1[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) load2(r + u, j, v0[u], v1[u]);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        a0 = __builtin_fmaf(v0[u], dv[r + u], a0);
        a1 = __builtin_fmaf(v1[u], dv[r + u], a1);
      }
    }
    for (; r < rows; ++r) {
      float v0, v1;
      load2(r, j, v0, v1);
      a0 = __builtin_fmaf(v0, dv[r], a0);
      a1 = __builtin_fmaf(v1, dv[r], a1);
    }
    partial[static_cast<int64_t>(tile) * d + j] = a0;
    partial[static_cast<int64_t>(tile) * d + j + 1] = a1;
  }
}

// Stage 2: dW_r[j][e] = sum of expert e's tile partials, in tile order.
__global__ __launch_bounds__(kRowThreads) void router_reduce_kernel(
    const float* __restrict__ partial, const int32_t* __restrict__ offsets, int E, int bm, int d,
    float* __restrict__ dwr) {
  __shared__ int32_t first, cnt;
  const int e = blockIdx.x;
  if (threadIdx.x == 0) {
    int32_t n = 0;
    for (int q = 0; q < e; ++q) n += (offsets[q + 1] - offsets[q] + bm - 1) / bm;
    first = n;
    cnt = (offsets[e + 1] - offsets[e] + bm - 1) / bm;
  }
  __syncthreads();
  constexpr int kBatch = 8;
  for (int j = threadIdx.x; j < d; j += kRowThreads) {
    float acc = 0.0f;
    int n = 0;
    for (; n + kBatch <= cnt; n += kBatch) {
      float v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = partial[static_cast<int64_t>(first + n + u) * d + j];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) acc += v[u];
    }
    for (; n < cnt; ++n) acc += partial[static_cast<int64_t>(first + n) * d + j];
    dwr[static_cast<int64_t>(j) * E + e] = acc;
  }
}

// bf16 path, before the down dgrad: the combine weight of each sorted
// row's slot (ws[r] = w[perm[r]]), the zero row the weight-gradient loads
// read past a group's end, the router transposed for dx (wrT[e][j] =
// wr[j][e], so that its columns are contiguous rows), and the zeroed dl
// table the router step fills (dlhl_n 16-byte pieces).
__global__ __launch_bounds__(kRowThreads) void bwd_prep_kernel(
    int64_t rows, const int32_t* __restrict__ perm, const float* __restrict__ w,
    float* __restrict__ ws, float* __restrict__ zero_row, int zero_n, const float* __restrict__ wr,
    int d, int E, float* __restrict__ wrT, u32x4* __restrict__ dlhl, int64_t dlhl_n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kRowThreads;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kRowThreads + threadIdx.x;
  for (int64_t i = i0; i < zero_n; i += stride) zero_row[i] = 0.0f;
  for (int64_t i = i0; i < dlhl_n; i += stride) dlhl[i] = u32x4{0u, 0u, 0u, 0u};
  const int64_t dE = static_cast<int64_t>(d) * E;
  for (int64_t i = i0; i < dE; i += stride) {
    const int64_t e = i / d, j = i % d;
    wrT[i] = wr[j * E + e];
  }
  for (int64_t r = i0; r < rows; r += stride) ws[r] = w[perm[r]];
}

// bf16 path: dl per slot from the down dgrad's dw parts (by sorted row),
// written by slot (dl) and, for kept slots, by sorted row (dls, which the
// gate/up dgrad's epilogue scales the router column by).
// One thread per token: dw_i = sum of the d_hidden slices' parts in slice
// order (0 for a slot capacity routing dropped: its y is 0), then dl_i =
// w_i (dw_i - sum_j w_j dw_j) with the sum taken in rank order. K = k <= 8
// issues all of a token's loads of one kind before using them.
// With dlhl, each slot's dl also goes into row t of the table [T][128]
// (bf16) as hi = bf16(dl) at column e and lo = bf16(dl - hi) at column 64 + e
// (e = its expert; a token's experts are distinct), for the router weight
// gradient's GEMM: hi + lo carries dl to about 2^-16 relative.
__device__ __forceinline__ void dl_hilo(bf16_t* row, int e, float v) {
  const bf16_t hi = f32_to_bf16(v);
  row[e] = hi;
  row[64 + e] = f32_to_bf16(v - bf16_to_f32(hi));
}

constexpr int kDlThreads = 64;  // one wave per block: more blocks than CUs at 16384 tokens

template <int K>
__global__ __launch_bounds__(kDlThreads) void router_dl_kernel(
    int64_t ntok, int k, int nparts, int64_t rows, const float* __restrict__ dwp,
    const float* __restrict__ w, const int32_t* __restrict__ inv_perm, float* __restrict__ dl,
    float* __restrict__ dls, const int32_t* __restrict__ topk_idx, bf16_t* __restrict__ dlhl) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kDlThreads + threadIdx.x;
  if (t >= ntok) return;
  if constexpr (K > 0) {
    int64_t r[K];
    float wv[K], dw[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      r[i] = inv_perm[t * K + i];
      wv[i] = w[t * K + i];
      dw[i] = 0.0f;
    }
    for (int q = 0; q < nparts; ++q) {
      float v[K];
#pragma unroll
      for (int i = 0; i < K; ++i) v[i] = r[i] >= 0 ? dwp[q * rows + r[i]] : 0.0f;
#pragma unroll
      for (int i = 0; i < K; ++i) dw[i] += v[i];
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < K; ++i) sum = __builtin_fmaf(wv[i], dw[i], sum);
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const float v = wv[i] * (dw[i] - sum);
      dl[t * K + i] = v;
      if (r[i] >= 0) dls[r[i]] = v;
      if (dlhl) dl_hilo(dlhl + t * 128, topk_idx[t * K + i], v);
    }
  } else {
    auto dw_of = [&](int i) {
      const int64_t r = inv_perm[t * k + i];
      float v = 0.0f;
      if (r >= 0)
        for (int q = 0; q < nparts; ++q) v += dwp[q * rows + r];
      return v;
    };
    float sum = 0.0f;
    for (int i = 0; i < k; ++i) sum = __builtin_fmaf(w[t * k + i], dw_of(i), sum);
    for (int i = 0; i < k; ++i) {
      const float v = w[t * k + i] * (dw_of(i) - sum);
      dl[t * k + i] = v;
      const int64_t r = inv_perm[t * k + i];
      if (r >= 0) dls[r] = v;
      if (dlhl) dl_hilo(dlhl + t * 128, topk_idx[t * k + i], v);
    }
  }
}

// bf16 router weight gradient, stage 2: dW_r[j][e] = sum over the token
// splits, in split order, of part[s][j][e] + part[s][j][64 + e] (the hi and
// lo halves of the dl table multiplied out), eight splits loaded at a time.
__global__ __launch_bounds__(kRowThreads) void router_reduce_hl_kernel(
    const float* __restrict__ part, int splits, int d, int E, float* __restrict__ dwr) {
  constexpr int kBatch = 8;
  const int64_t n = static_cast<int64_t>(d) * E;
  const int64_t sstride = static_cast<int64_t>(d) * 128;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kRowThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kRowThreads) {
    const int64_t j = i / E;
    const int e = static_cast<int>(i % E);
    const float* p0 = part + j * 128 + e;
    float acc = 0.0f;
    int sp = 0;
    for (; sp + kBatch <= splits; sp += kBatch) {
      float hi[kBatch], lo[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        hi[u] = p0[(sp + u) * sstride];
        lo[u] = p0[(sp + u) * sstride + 64];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) acc += hi[u] + lo[u];
    }
    for (; sp < splits; ++sp) acc += p0[sp * sstride] + p0[sp * sstride + 64];
    dwr[i] = acc;
  }
}

// dx[t] = sum_i dX_sorted[slot(t,i)] + sum_i dl_i W_r[:, e_i] + dx_shared[t].
// wrT[e][j] = wr[j][e]: the router columns as contiguous rows, so the
// router term of dx reads 16- or 32-byte pieces instead of strided floats.
__global__ __launch_bounds__(256) void router_transpose_kernel(const float* __restrict__ wr,
                                                               int d, int E,
                                                               float* __restrict__ wrT) {
  __shared__ float tile[32][33];
  const int j0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8) {
    const int j = j0 + r, e = e0 + tx;
    tile[r][tx] = (j < d && e < E) ? wr[static_cast<int64_t>(j) * E + e] : 0.0f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int e = e0 + r, j = j0 + tx;
    if (e < E && j < d) wrT[static_cast<int64_t>(e) * d + j] = tile[tx][r];
  }
}

// kKeptRouter: the gate/up dgrad already added the router term to the rows
// of kept slots, so only dropped slots (capacity routing) add it here.
template <typename T, bool kKeptRouter>
__global__ __launch_bounds__(kRowThreads) void dx_gather_kernel(
    int64_t ntok, int k, int d, int E, const T* __restrict__ dxs, const int32_t* __restrict__ inv_perm,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ dl,
    const float* __restrict__ wrT, const T* __restrict__ dx_shared, T* __restrict__ dx) {
  constexpr int N = V16<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kRowThreads / 64) + (threadIdx.x >> 6);
  if (t >= ntok) return;
  for (int c = lane * N; c < d; c += 64 * N) {
    float acc[N];
#pragma unroll
    for (int q = 0; q < N; ++q) acc[q] = 0.0f;
    for (int i = 0; i < k; ++i) {
      const int64_t slot = inv_perm[t * k + i];
      const int e = topk_idx[t * k + i];
      const float li = dl[t * k + i];
      float v[N], wv[N];
      if (slot >= 0) {
        V16<T>::load_nt(dxs + slot * d + c, v);
      } else {
        // dropped by capacity routing: only the router term
#pragma unroll
        for (int q = 0; q < N; ++q) v[q] = 0.0f;
      }
      if (kKeptRouter && slot >= 0) {
#pragma unroll
        for (int q = 0; q < N; ++q) acc[q] += v[q];
        continue;
      }
#pragma unroll
      for (int q = 0; q < N; q += 4) {
        const float4 w4 = *reinterpret_cast<const float4*>(wrT + static_cast<int64_t>(e) * d + c + q);
        wv[q] = w4.x; wv[q + 1] = w4.y; wv[q + 2] = w4.z; wv[q + 3] = w4.w;
      }
#pragma unroll
      for (int q = 0; q < N; ++q) acc[q] += __builtin_fmaf(li, wv[q], v[q]);
    }
    if (dx_shared) {
      float v[N];
      V16<T>::load_nt(dx_shared + t * d + c, v);
#pragma unroll
      for (int q = 0; q < N; ++q) acc[q] += v[q];
    }
    V16<T>::store_nt(dx + t * d + c, acc);
  }
}

// k = K <= 8: lane i reads slot i's sorted row, expert and router-logit
// gradient (one coalesced load each), the wave broadcasts them, and all K
// expert-row and router-row loads of a piece (and the shared row's) are
// issued before any is used: one memory latency per token instead of 2K
// dependent ones. Same arithmetic and order as dx_gather_kernel.
template <typename T, int K, bool kKeptRouter>
__global__ __launch_bounds__(kRowThreads) void dx_gather_k_kernel(
    int64_t ntok, int d, const T* __restrict__ dxs, const int32_t* __restrict__ inv_perm,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ dl,
    const float* __restrict__ wrT, const T* __restrict__ dx_shared, T* __restrict__ dx) {
  constexpr int N = V16<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kRowThreads / 64) + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int my_slot = lane < K ? inv_perm[t * K + lane] : 0;
  const int my_e = lane < K ? topk_idx[t * K + lane] : 0;
  const float my_l = lane < K ? dl[t * K + lane] : 0.0f;
  int64_t slot[K];
  int e[K];
  float li[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    slot[i] = __builtin_amdgcn_readlane(my_slot, i);
    e[i] = __builtin_amdgcn_readlane(my_e, i);
    li[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_l), i));
  }
  for (int c = lane * N; c < d; c += 64 * N) {
    // The K rows and the shared row are loaded raw, all before any is used
    // (16 bytes = 4 registers each; converted to fp32 they took twice that
    // and held the kernel to 3 waves per SIMD); then the router terms.
    u32x4 raw[K], sraw = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < K; ++i)
      raw[i] = slot[i] >= 0
                   ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dxs + slot[i] * d + c))
                   : u32x4{0u, 0u, 0u, 0u};  // dropped by capacity routing: only the router term
    if (dx_shared) sraw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dx_shared + t * d + c));
    float acc[N];
#pragma unroll
    for (int q = 0; q < N; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      float v[N];
      V16<T>::unpack(raw[i], v);
#pragma unroll
      for (int q = 0; q < N; ++q) acc[q] += v[q];
    }
    auto router_term = [&](int i) {
#pragma unroll
      for (int q = 0; q < N; q += 4) {
        const float4 w4 = *reinterpret_cast<const float4*>(wrT + static_cast<int64_t>(e[i]) * d + c + q);
        acc[q] = __builtin_fmaf(li[i], w4.x, acc[q]);
        acc[q + 1] = __builtin_fmaf(li[i], w4.y, acc[q + 1]);
        acc[q + 2] = __builtin_fmaf(li[i], w4.z, acc[q + 2]);
        acc[q + 3] = __builtin_fmaf(li[i], w4.w, acc[q + 3]);
      }
    };
    if (kKeptRouter) {
      // only slots capacity routing dropped (rare): one at a time
#pragma unroll 1
      for (int i = 0; i < K; ++i)
        if (slot[i] < 0) router_term(i);
    } else {
#pragma unroll
      for (int i = 0; i < K; ++i) router_term(i);
    }
    if (dx_shared) {
      float sv[N];
      V16<T>::unpack(sraw, sv);
#pragma unroll
      for (int q = 0; q < N; ++q) acc[q] += sv[q];
    }
    V16<T>::store_nt(dx + t * d + c, acc);
  }
}

// Fixed-order sum of split-K partials [splits][M][N] (split 0 first, fp32
// adds); columns n >= nsplit go to c2 at column n - nsplit. Four columns per
// thread (N and nsplit are multiples of 4) and eight partials loaded before
// they are added, so a thread waits for memory once per eight splits.
__global__ __launch_bounds__(kRowThreads) void split_reduce_kernel(
    const float* __restrict__ partial, int splits, int64_t M, int N, int nsplit, int64_t ldc,
    float* __restrict__ c, float* __restrict__ c2) {
  constexpr int kBatch = 8;
  const int64_t MN = M * N, MN4 = MN / 4;
  const float4* p4 = reinterpret_cast<const float4*>(partial);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kRowThreads + threadIdx.x; i < MN4;
       i += static_cast<int64_t>(gridDim.x) * kRowThreads) {
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    int s = 0;
    for (; s + kBatch <= splits; s += kBatch) {
      float4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = p4[(s + u) * MN4 + i];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w;
      }
    }
    for (; s < splits; ++s) {
      const float4 v = p4[s * MN4 + i];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    const int64_t m = (4 * i) / N;
    const int n = static_cast<int>((4 * i) % N);
    float* dst = n < nsplit ? c + m * ldc + n : c2 + m * ldc + (n - nsplit);
    *reinterpret_cast<float4*>(dst) = acc;
  }
}

__global__ __launch_bounds__(kRowThreads) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kRowThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kRowThreads)
    p[i] = 0.0f;
}

struct BwdLayout {
  // dY holds dY [S][d] (fp32) or w H [S][h] (bf16); dwp the bf16 dw parts,
  // wsr the bf16 combine weights and dls its router-logit gradients by
  // sorted row
  size_t dY, dl, dls, dwp, wsr, dlhl, rph, dAB, dXs, rpart, dABs, dxs, part_sd, part_sgu, wrT, zero,
      tiles256, total;
  int ks_sd, ks_sgu, ks_r;
};

int split_count(int64_t rows, int tiles) {
  // A shared width under the backward's 128-column tile has no output tile
  // (moe_bwd rejects it); the forward's training workspace is still sized.
  if (tiles < 1) tiles = 1;
  int ks = (512 + tiles - 1) / tiles;
  ks = ks < 1 ? 1 : (ks > 64 ? 64 : ks);
  if (ks > rows) ks = static_cast<int>(rows > 0 ? rows : 1);
  return ks;
}

BwdLayout bwd_layout(const moe_problem& p) {
  const size_t es = p.dtype == MOE_BF16 ? 2 : 4;
  const size_t T = static_cast<size_t>(p.tokens), S = T * p.top_k;
  const size_t d = p.d_model, h = p.d_hidden, hs = p.d_shared;
  const size_t max_tiles = (S + p.block_m - 1) / p.block_m + p.experts;
  BwdLayout L{};
  L.ks_sd = hs ? split_count(p.tokens, static_cast<int>((hs / 128) * (d / 128))) : 0;
  L.ks_sgu = hs ? split_count(p.tokens, static_cast<int>((d / 128) * (2 * hs / 128))) : 0;
  size_t o = 0;
  L.dY = o;       o = align_up(o + S * (p.dtype == MOE_BF16 ? h : d) * es, 256);
  L.dl = o;       o = align_up(o + S * 4, 256);
  L.dwp = o;      o = align_up(o + ((h + 127) / 128) * S * 4, 256);
  L.wsr = o;      o = align_up(o + S * 4, 256);
  L.dls = o;      o = align_up(o + S * 4, 256);
  // bf16 router weight gradient: the dl hi/lo table and the token splits'
  // partials (splits of at least 256 tokens, at most 64)
  const bool bf = p.dtype == MOE_BF16;
  L.ks_r = static_cast<int>(T / 256 < 1 ? 1 : (T / 256 > 64 ? 64 : T / 256));
  L.dlhl = o;     o = align_up(o + (bf ? T * 128 * 2 : 0), 256);
  L.rph = o;      o = align_up(o + (bf ? static_cast<size_t>(L.ks_r) * d * 128 * 4 : 0), 256);
  L.dAB = o;      o = align_up(o + S * 2 * h * es, 256);
  L.dXs = o;      o = align_up(o + S * d * es, 256);
  L.rpart = o;    o = align_up(o + max_tiles * d * 4, 256);
  L.dABs = o;     o = align_up(o + T * 2 * hs * es, 256);
  L.dxs = o;      o = align_up(o + T * d * es, 256);
  L.part_sd = o;  o = align_up(o + static_cast<size_t>(L.ks_sd) * hs * d * 4, 256);
  L.part_sgu = o; o = align_up(o + static_cast<size_t>(L.ks_sgu) * d * 2 * hs * 4, 256);
  L.wrT = o;      o = align_up(o + static_cast<size_t>(p.experts) * d * 4, 256);
  L.zero = o;     o = align_up(o + kTrZeroBytes, 256);
  L.tiles256 = o; o = align_up(o + retile_bytes(static_cast<int64_t>(S), p.experts), 256);
  L.total = o;
  return L;
}

void zero(float* p, int64_t n, hipStream_t s) {
  if (!p || n <= 0) return;
  int64_t blocks = (n + kRowThreads - 1) / kRowThreads;
  if (blocks > 4096) blocks = 4096;
  MOE_LAUNCH("fill_zero", fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kRowThreads),
             0, s, p, n);
}



// Weight gradient: bf16 operands take the transposing-LDS-read kernel
// (gathering A's rows through perm when kGatherA), fp32 the
// register-transposing one.
template <typename T, bool kGatherA, bool kDense>
void wgrad(const char* name, const WgradArgs& a, int groups, const void* zero, hipStream_t s) {
  if (std::is_same<T, bf16_t>::value) {
    wgrad_tr<kDense, kGatherA>(name, a, groups, static_cast<const bf16_t*>(zero), s);
    return;
  }
  const int64_t blocks = static_cast<int64_t>(groups) * (a.M / 128) * (a.N / 128);
  if (blocks <= 0) return;
  MOE_LAUNCH(name, (wgrad_kernel<T, kGatherA, kDense>), dim3(static_cast<unsigned>(blocks)),
             dim3(256), 0, s, a);
}

// a15: dX_sorted = dA W_gate^T + dB W_up^T, on the 256-row tile list
// (built by the caller when retile_rows(p) or when the bf16 down dgrad ran)
// or the caller's block_m list. With dls (dl by sorted row) and wrT (the
// router transposed), the wide engine also adds each row's router term
// dl * W_r[:, e] before rounding; returns whether it did.
template <typename T>
bool gate_up_dgrad(const moe_problem& p, const moe_weights& w, const moe_routing& r,
                   const void* dAB, void* dXs, int32_t* t256, bool t256_built, const float* dls,
                   const float* wrT, hipStream_t s) {
  const int64_t S = p.tokens * p.top_k;
  const int64_t max_tiles = (S + p.block_m - 1) / p.block_m + p.experts;
  const int d = p.d_model, h = p.d_hidden;
  GemmArgs b{};
  b.a = dAB;
  b.lda = 2 * static_cast<int64_t>(h);
  b.b = w.w_gate;  // [E][d][h]: row n = model unit, K = h contiguous
  b.b_group_stride = static_cast<int64_t>(d) * h;
  b.ldb = h;
  b.b2 = w.w_up;
  b.b2_group_stride = static_cast<int64_t>(d) * h;
  b.ksplit = h;
  b.N = d;
  b.K = 2 * h;
  b.tiles = r.tiles;
  b.num_tiles = r.num_tiles;
  b.c = dXs;
  b.ldc = d;
  if ((retile_rows(p) || (t256_built && p.block_m == kRetileBm)) && wide_fits<T>(b)) {
    // 256-row tiles on the wide engine (K = 2h, N = d_model)
    const int64_t mt256 = (S + kRetileBm - 1) / kRetileBm + p.experts;
    if (!t256_built)
      (void)launch_retile(r.expert_offsets, p.experts, kRetileBm, p.capacity, t256 + 4, t256, s);
    b.tiles = t256 + 4;
    b.num_tiles = t256;
    if (dls && wrT) {
      b.rdl = dls;
      b.rw = wrT;
      wide_gemm<false, kEpiStoreRouter, false>("bwd_gate_up_dgrad", b, mt256, s);
      return true;
    }
    grouped_gemm<T, false, kEpiStore>("bwd_gate_up_dgrad", b, kRetileBm, mt256, s);
  } else {
    grouped_gemm<T, false, kEpiStore>("bwd_gate_up_dgrad", b, p.block_m, max_tiles, s);
  }
  return false;
}

// fp32 a13: dH = dY W_down^T and the SwiGLU backward into dA|dB.
template <typename T>
void down_dgrad_dy(const moe_problem& p, const moe_weights& w, const moe_routing& r,
                   const void* saved_ab, const void* dY, void* dAB, hipStream_t s) {
  const int64_t S = p.tokens * p.top_k;
  const int64_t max_tiles = (S + p.block_m - 1) / p.block_m + p.experts;
  const int d = p.d_model, h = p.d_hidden;
  GemmArgs a{};
  a.a = dY;
  a.lda = d;
  a.b = w.w_down;  // [E][h][d]: row n = hidden unit, K = d contiguous
  a.b_group_stride = static_cast<int64_t>(h) * d;
  a.N = h;
  a.K = d;
  a.tiles = r.tiles;
  a.num_tiles = r.num_tiles;
  a.c = dAB;
  a.ldc = 2 * static_cast<int64_t>(h);
  a.hsplit = h;
  a.sa = const_cast<void*>(saved_ab);
  a.sb = const_cast<T*>(static_cast<const T*>(saved_ab) + h);
  a.lds = 2 * static_cast<int64_t>(h);
  grouped_gemm<T, false, kEpiSwigluBwd>("bwd_down_dgrad", a, p.block_m, max_tiles, s);
}

// bf16 a11 + a13 (gemm_dgrad.h) over the 256-row list t256 (mt256 entries
// at most): dA|dB, w H into hw, and the dw parts.
void down_dgrad_fused(const moe_problem& p, const moe_weights& w, const moe_routing& r,
                      const void* saved_ab, const void* grad_out, const float* wsr, bf16_t* hw,
                      void* dAB, float* dwp, const int32_t* t256, int64_t mt256, hipStream_t s) {
  DgradArgs a{};
  a.g = static_cast<const bf16_t*>(grad_out);
  a.perm = r.perm;
  a.topk = p.top_k;
  a.w = static_cast<const bf16_t*>(w.w_down);
  a.sab = static_cast<const bf16_t*>(saved_ab);
  a.ws = wsr;
  a.dab = static_cast<bf16_t*>(dAB);
  a.hw = hw;
  a.dwp = dwp;
  a.rows = p.tokens * p.top_k;
  a.d = p.d_model;
  a.h = p.d_hidden;
  const int64_t work = mt256 * (p.d_hidden / 128);
  if (work <= 0) return;
  const int slots = persistent_slots(reinterpret_cast<const void*>(&down_dgrad_kernel), 512);
  const unsigned grid = static_cast<unsigned>(work < slots ? work : slots);
  MOE_LAUNCH("bwd_down_dgrad", down_dgrad_kernel, dim3(grid), dim3(512), 0, s, a, t256 + 4, t256,
             static_cast<int>(work));
}

template <typename T>
hipError_t bwd_t(const moe_problem& p, const void* x, const moe_weights& w, const moe_routing& r,
                 const void* y_sorted, const void* saved, const void* grad_out, void* grad_x,
                 const moe_grads& g, void* ws, hipStream_t s, hipStream_t side) {
  const int64_t T_ = p.tokens, S = T_ * p.top_k;
  const int E = p.experts, k = p.top_k, d = p.d_model, h = p.d_hidden, hs = p.d_shared;
  const int64_t max_tiles = (S + p.block_m - 1) / p.block_m + E;
  const BwdLayout L = bwd_layout(p);
  const FfnLayout F = ffn_layout(p, true);
  char* W = static_cast<char*>(ws);
  const char* SV = static_cast<const char*>(saved);
  T* dY = reinterpret_cast<T*>(W + L.dY);
  float* dl = reinterpret_cast<float*>(W + L.dl);
  T* dAB = reinterpret_cast<T*>(W + L.dAB);
  T* dXs = reinterpret_cast<T*>(W + L.dXs);
  float* rpart = reinterpret_cast<float*>(W + L.rpart);
  // Zero row the bf16 weight-gradient loads read past a group's end (and,
  // in bf16, the combine weights by sorted row for the down dgrad).
  const void* zero_row = W + L.zero;
  float* wsr = reinterpret_cast<float*>(W + L.wsr);
  bf16_t* dlhl = std::is_same<T, bf16_t>::value ? reinterpret_cast<bf16_t*>(W + L.dlhl) : nullptr;
  float* dls = reinterpret_cast<float*>(W + L.dls);
  float* wrT = reinterpret_cast<float*>(W + L.wrT);
  bool router_folded = false;
  if (std::is_same<T, bf16_t>::value) {
    int64_t blocks = (S + kRowThreads - 1) / kRowThreads;
    blocks = blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks);
    MOE_LAUNCH("bwd_prep", bwd_prep_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kRowThreads),
               0, s, S, r.perm, r.topk_w, wsr, reinterpret_cast<float*>(W + L.zero),
               static_cast<int>(kTrZeroBytes / 4), w.w_router, d, E,
               reinterpret_cast<float*>(W + L.wrT), reinterpret_cast<u32x4*>(W + L.dlhl),
               T_ * 128 * 2 / 16);
  }
  const int64_t row_blocks = (T_ + kRowThreads / 64 - 1) / (kRowThreads / 64);

  T* dxs = nullptr;
  // a11-a14 (routed path) and a16 (shared expert); the shared expert needs
  // only grad_out, the tokens and its own saved activations, so it runs on
  // the side stream beside the routed path (each lambda's stream parameter
  // is the `s` its launches use).
  auto routed_bwd = [&](hipStream_t s) {
    const void* sab = SV + F.sv_ab;
    int32_t* t256 = reinterpret_cast<int32_t*>(W + L.tiles256);
    bool t256_built = false;
    if constexpr (std::is_same<T, bf16_t>::value) {
      // a11 + a13: the down dgrad reads G by token and yields dA|dB, w H
      // and the combine weights' gradient parts; then dl per slot
      const int64_t mt256 = (S + kRetileBm - 1) / kRetileBm + E;
      (void)launch_retile(r.expert_offsets, E, kRetileBm, p.capacity, t256 + 4, t256, s);
      t256_built = true;
      float* dwp = reinterpret_cast<float*>(W + L.dwp);
      down_dgrad_fused(p, w, r, sab, grad_out, wsr, dY, dAB, dwp, t256, mt256, s);
      const dim3 dl_grid(static_cast<unsigned>((T_ + kDlThreads - 1) / kDlThreads));
#define MOE_DL_K(KK)                                                                         \
  case KK:                                                                                   \
    MOE_LAUNCH("bwd_router_dl", router_dl_kernel<KK>, dl_grid, dim3(kDlThreads), 0, s, T_,  \
               k, h / 128, S, dwp, r.topk_w, r.inv_perm, dl, dls, r.topk_idx, dlhl);                                \
    break;
      switch (k) {
        MOE_DL_K(1) MOE_DL_K(2) MOE_DL_K(3) MOE_DL_K(4) MOE_DL_K(5) MOE_DL_K(6) MOE_DL_K(7)
        MOE_DL_K(8)
        default:
          MOE_LAUNCH("bwd_router_dl", router_dl_kernel<0>, dl_grid, dim3(kDlThreads), 0, s, T_, k,
                     h / 128, S, dwp, r.topk_w, r.inv_perm, dl, dls, r.topk_idx, dlhl);
      }
#undef MOE_DL_K
    } else {
      // a11: combine backward and per-slot router gradient
      const T* g_t = static_cast<const T*>(grad_out);
      const T* y_t = static_cast<const T*>(y_sorted);
#define MOE_CB_K(KK)                                                                          \
  case KK:                                                                                    \
    MOE_LAUNCH("bwd_combine", (combine_bwd_k_kernel<T, KK>),                                  \
               dim3(static_cast<unsigned>(row_blocks)), dim3(kRowThreads), 0, s, T_, d, g_t,  \
               y_t, r.topk_w, r.inv_perm, dY, dl);                                            \
    break;
      switch (k) {
        MOE_CB_K(1) MOE_CB_K(2) MOE_CB_K(3) MOE_CB_K(4) MOE_CB_K(5) MOE_CB_K(6) MOE_CB_K(7)
        MOE_CB_K(8)
        default:
          MOE_LAUNCH("bwd_combine", combine_bwd_kernel<T>, dim3(static_cast<unsigned>(row_blocks)),
                     dim3(kRowThreads), 0, s, T_, k, d, g_t, y_t, r.topk_w, r.inv_perm, dY, dl);
      }
#undef MOE_CB_K
      // a13: down dgrad from dY
      down_dgrad_dy<T>(p, w, r, sab, dY, dAB, s);
    }
    // a12: router weight gradient
    if constexpr (std::is_same<T, bf16_t>::value) {
      // dW_r = x^T DL as a GEMM over token splits: DL is the dl table
      // (hi | lo halves, one row per token), then the splits and halves
      // summed in a fixed order
      WgradArgs a{};
      a.a = x;
      a.lda = d;
      a.b = dlhl;
      a.ldb = 128;
      a.M = d;
      a.N = 128;
      a.rows_total = T_;
      a.splits = L.ks_r;
      a.c = reinterpret_cast<float*>(W + L.rph);
      a.nsplit = 128;
      a.ldc = 128;
      a.c_group_stride = static_cast<int64_t>(d) * 128;
      wgrad<T, false, true>("bwd_router_wgrad", a, L.ks_r, zero_row, s);
      MOE_LAUNCH("bwd_router_reduce", router_reduce_hl_kernel,
                 dim3(static_cast<unsigned>((static_cast<int64_t>(d) * E + kRowThreads - 1) / kRowThreads)),
                 dim3(kRowThreads), 0, s,
                 reinterpret_cast<const float*>(W + L.rph), L.ks_r, d, E, g.w_router);
    } else {
      // tile partials, then a per-expert ordered sum
      MOE_LAUNCH("bwd_router_partial", router_partial_kernel<T>, dim3(static_cast<unsigned>(max_tiles)),
                 dim3(kRowThreads), 0, s, static_cast<const T*>(x), d, k, r.perm, dl,
                 r.expert_offsets, E, p.block_m, rpart);
      MOE_LAUNCH("bwd_router_reduce", router_reduce_kernel, dim3(E), dim3(kRowThreads), 0, s, rpart,
                 r.expert_offsets, E, p.block_m, d, g.w_router);
    }
    // a15: gate/up dgrad (bf16: with the router term of each kept slot)
    router_folded = gate_up_dgrad<T>(p, w, r, dAB, dXs, t256, t256_built, t256_built ? dls : nullptr,
                                     t256_built ? wrT : nullptr, s);
    // a14: per-expert weight gradients, K = the expert's rows
    {
      WgradArgs a{};
      a.M = h;
      a.N = d;
      a.row_offsets = r.expert_offsets;
      a.cap = p.capacity;
      a.c = g.w_down;
      a.c_group_stride = static_cast<int64_t>(h) * d;
      if constexpr (std::is_same<T, bf16_t>::value) {
        // dW_down[e]^T = sum over rows of G[token]^T (w H): G gathered as
        // the M side, stored transposed into [h][d]
        a.a = grad_out;
        a.lda = d;
        a.perm = r.perm;
        a.topk = k;
        a.rows_total = S;
        a.b = dY;  // w H
        a.ldb = h;
        a.M = d;
        a.N = h;
        a.nsplit = h;
        a.ldc = d;
        a.trans_c = 1;
        wgrad<T, true, false>("bwd_wgrad_down", a, E, zero_row, s);
      } else {
        a.a = SV + F.sv_h;
        a.lda = h;
        a.b = dY;
        a.ldb = d;
        a.nsplit = d;
        a.ldc = d;
        wgrad<T, false, false>("bwd_wgrad_down", a, E, zero_row, s);
      }
      WgradArgs b{};
      b.a = x;
      b.lda = d;
      b.perm = r.perm;
      b.topk = k;
      b.rows_total = S;  // entries of perm
      b.b = dAB;
      b.ldb = 2 * static_cast<int64_t>(h);
      b.M = d;
      b.N = 2 * h;
      b.row_offsets = r.expert_offsets;
      b.cap = p.capacity;
      b.c = g.w_gate;
      b.c2 = g.w_up;
      b.nsplit = h;
      b.ldc = h;
      b.c_group_stride = static_cast<int64_t>(d) * h;
      wgrad<T, true, false>("bwd_wgrad_gate_up", b, E, zero_row, s);
    }
  };
  auto shared_bwd = [&](hipStream_t s) {
    // a16: shared expert
    if (hs > 0) {
      T* dABs = reinterpret_cast<T*>(W + L.dABs);
      dxs = reinterpret_cast<T*>(W + L.dxs);
      const T* ssab = reinterpret_cast<const T*>(SV + F.sv_sab);
      GemmArgs a{};
      a.a = grad_out;
      a.lda = d;
      a.b = w.ws_down;  // [hs][d]
      a.N = hs;
      a.K = d;
      a.M = T_;
      a.c = dABs;
      a.ldc = 2 * static_cast<int64_t>(hs);
      a.hsplit = hs;
      a.sa = const_cast<T*>(ssab);
      a.sb = const_cast<T*>(ssab + hs);
      a.lds = 2 * static_cast<int64_t>(hs);
      dense_gemm<T, kEpiSwigluBwd>("bwd_shared_down_dgrad", a, s);
      GemmArgs b{};
      b.a = dABs;
      b.lda = 2 * static_cast<int64_t>(hs);
      b.b = w.ws_gate;  // [d][hs]
      b.ldb = hs;
      b.b2 = w.ws_up;
      b.ksplit = hs;
      b.N = d;
      b.K = 2 * hs;
      b.M = T_;
      b.c = dxs;
      b.ldc = d;
      dense_gemm<T, kEpiStore>("bwd_shared_gate_up_dgrad", b, s);

      float* p1 = reinterpret_cast<float*>(W + L.part_sd);
      WgradArgs c{};
      c.a = SV + F.sv_sh;
      c.lda = hs;
      c.b = grad_out;
      c.ldb = d;
      c.M = hs;
      c.N = d;
      c.rows_total = T_;
      c.splits = L.ks_sd;
      c.c = p1;
      c.nsplit = d;
      c.ldc = d;
      c.c_group_stride = static_cast<int64_t>(hs) * d;
      wgrad<T, false, true>("bwd_shared_wgrad_down", c, L.ks_sd, zero_row, s);
      MOE_LAUNCH("bwd_split_reduce", split_reduce_kernel, dim3(2048), dim3(kRowThreads), 0, s, p1,
                 L.ks_sd, static_cast<int64_t>(hs), d, d, static_cast<int64_t>(d), g.ws_down,
                 static_cast<float*>(nullptr));
      float* p2 = reinterpret_cast<float*>(W + L.part_sgu);
      WgradArgs e{};
      e.a = x;
      e.lda = d;
      e.b = dABs;
      e.ldb = 2 * static_cast<int64_t>(hs);
      e.M = d;
      e.N = 2 * hs;
      e.rows_total = T_;
      e.splits = L.ks_sgu;
      e.c = p2;
      e.nsplit = 2 * hs;
      e.ldc = 2 * static_cast<int64_t>(hs);
      e.c_group_stride = static_cast<int64_t>(d) * 2 * hs;
      wgrad<T, false, true>("bwd_shared_wgrad_gate_up", e, L.ks_sgu, zero_row, s);
      MOE_LAUNCH("bwd_split_reduce", split_reduce_kernel, dim3(2048), dim3(kRowThreads), 0, s, p2,
                 L.ks_sgu, static_cast<int64_t>(d), 2 * hs, hs, static_cast<int64_t>(hs), g.ws_gate,
                 g.ws_up);
    }
  };
  if (hs > 0) {
    // The shared expert's backward needs only grad_out, x and its saved
    // activations: with a second stream it runs there beside the routed part.
    StreamFork fork(s, side);
    hipError_t e = fork.fork();
    if (e != hipSuccess) return e;
    shared_bwd(fork.side());
    routed_bwd(s);
    e = hipGetLastError();
    if (e == hipSuccess) e = fork.join();
    if (e != hipSuccess) return e;
  } else {
    routed_bwd(s);
  }
  // dx: gather-sum of the routed input gradients plus the router and shared terms
  if (!std::is_same<T, bf16_t>::value)  // bf16: bwd_prep wrote it
    MOE_LAUNCH("bwd_router_transpose", router_transpose_kernel, dim3((d + 31) / 32, (E + 31) / 32),
               dim3(256), 0, s, w.w_router, d, E, wrT);
  const T* dxs_t = static_cast<const T*>(dxs);
  T* gx = static_cast<T*>(grad_x);
#define MOE_DX_K(KK)                                                                          \
  case KK:                                                                                    \
    if (router_folded)                                                                        \
      MOE_LAUNCH("bwd_dx", (dx_gather_k_kernel<T, KK, true>),                                  \
                 dim3(static_cast<unsigned>(row_blocks)), dim3(kRowThreads), 0, s, T_, d, dXs, \
                 r.inv_perm, r.topk_idx, dl, wrT, dxs_t, gx);                                 \
    else                                                                                      \
      MOE_LAUNCH("bwd_dx", (dx_gather_k_kernel<T, KK, false>),                                 \
                 dim3(static_cast<unsigned>(row_blocks)), dim3(kRowThreads), 0, s, T_, d, dXs, \
                 r.inv_perm, r.topk_idx, dl, wrT, dxs_t, gx);                                 \
    break;
  switch (k) {
    MOE_DX_K(1) MOE_DX_K(2) MOE_DX_K(3) MOE_DX_K(4) MOE_DX_K(5) MOE_DX_K(6) MOE_DX_K(7)
    MOE_DX_K(8)
    default:
      if (router_folded)
        MOE_LAUNCH("bwd_dx", (dx_gather_kernel<T, true>), dim3(static_cast<unsigned>(row_blocks)),
                   dim3(kRowThreads), 0, s, T_, k, d, E, dXs, r.inv_perm, r.topk_idx, dl, wrT,
                   dxs_t, gx);
      else
        MOE_LAUNCH("bwd_dx", (dx_gather_kernel<T, false>), dim3(static_cast<unsigned>(row_blocks)),
                   dim3(kRowThreads), 0, s, T_, k, d, E, dXs, r.inv_perm, r.topk_idx, dl, wrT,
                   dxs_t, gx);
  }
#undef MOE_DX_K
  return hipGetLastError();
}

}  // namespace

size_t bwd_ws_bytes(const moe_problem& p) { return bwd_layout(p).total; }

hipError_t launch_bwd(const moe_problem& p, const void* x, const moe_weights& w,
                      const moe_routing& r, const void* y_sorted, const void* saved,
                      const void* grad_out, void* grad_x, const moe_grads& g, void* ws,
                      hipStream_t s, hipStream_t side) {
  if (p.tokens == 0) {
    const int64_t E = p.experts, d = p.d_model, h = p.d_hidden, hs = p.d_shared;
    zero(g.w_router, d * E, s);
    zero(g.w_gate, E * d * h, s);
    zero(g.w_up, E * d * h, s);
    zero(g.w_down, E * h * d, s);
    if (hs > 0) {
      zero(g.ws_gate, d * hs, s);
      zero(g.ws_up, d * hs, s);
      zero(g.ws_down, hs * d, s);
    }
    return hipGetLastError();
  }
  if (p.dtype == MOE_BF16)
    return bwd_t<bf16_t>(p, x, w, r, y_sorted, saved, grad_out, grad_x, g, ws, s, side);
  return bwd_t<float>(p, x, w, r, y_sorted, saved, grad_out, grad_x, g, ws, s, side);
}

}  // namespace moe
