// Stage "route": router logits, top-k selection and renormalised combine
// weights, one fused kernel (kernel_gmm_gpu.json "pieces" suite, piece
// "route").
//
// Logits are the fixed fp32 chain acc = fma(x[t,j], W[j,e], acc) for j
// ascending from +0.0, evaluated in exactly that order; the blocking below
// only pauses the chain. A token group of L lanes holds one token's
// logits, each lane P experts of R tokens, so every router value read from
// LDS feeds R multiply-adds and every token value P. The selection runs k
// rounds of a butterfly argmax inside the group on (logit descending,
// expert index ascending); no floating-point reduction decides an expert.
// Routers that fit in LDS stay resident for a CU's whole token range
// (route_resident_kernel); larger ones are streamed in row chunks.
#include "common.h"

namespace moe {

namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteChunk = 128;  // router rows (j) staged in LDS per pass
constexpr int kRoutePad = 4;      // LDS row padding (floats): conflict-free 16-byte reads

__device__ __forceinline__ void load8(const bf16_t* p, float* o) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  o[0] = bf16lo(v.x); o[1] = bf16hi(v.x);
  o[2] = bf16lo(v.y); o[3] = bf16hi(v.y);
  o[4] = bf16lo(v.z); o[5] = bf16hi(v.z);
  o[6] = bf16lo(v.w); o[7] = bf16hi(v.w);
}
__device__ __forceinline__ void load8(const float* p, float* o) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// Eight values from their raw 16-byte pieces.
template <typename T>
__device__ __forceinline__ void widen8(const u32x4 (&v)[sizeof(T) / 2], float* o);
template <>
__device__ __forceinline__ void widen8<bf16_t>(const u32x4 (&v)[1], float* o) {
  o[0] = bf16lo(v[0].x); o[1] = bf16hi(v[0].x);
  o[2] = bf16lo(v[0].y); o[3] = bf16hi(v[0].y);
  o[4] = bf16lo(v[0].z); o[5] = bf16hi(v[0].z);
  o[6] = bf16lo(v[0].w); o[7] = bf16hi(v[0].w);
}
template <>
__device__ __forceinline__ void widen8<float>(const u32x4 (&v)[2], float* o) {
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    o[4 * n + 0] = __uint_as_float(v[n].x);
    o[4 * n + 1] = __uint_as_float(v[n].y);
    o[4 * n + 2] = __uint_as_float(v[n].z);
    o[4 * n + 3] = __uint_as_float(v[n].w);
  }
}

// Ranking key of (logit, expert): a larger key ranks first, i.e. the larger
// logit, then the lower expert index. The high half is the logit's bits
// mapped to an unsigned order (-0 taken as +0, so equal logits tie), the
// low half the complement of the index. Valid keys are never 0; 0 marks an
// expert that does not exist or has been selected.
__device__ __forceinline__ uint64_t rank_key(float v, int e) {
  uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<uint64_t>(b) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
}
__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t h = static_cast<uint32_t>(key >> 32);
  return __uint_as_float((h & 0x80000000u) ? (h & 0x7FFFFFFFu) : ~h);
}
__device__ __forceinline__ int key_expert(uint64_t key) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
}

// One exchange step across lanes by DPP (quad_perm [1,0,3,2] = 0xB1 and
// [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140): plain VALU
// moves within rows of 16 lanes, no LDS round trip.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), kCtrl, 0xF, 0xF, true));
}
template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_max_key(uint64_t k) {
  const uint64_t o = (static_cast<uint64_t>(dpp_u32<kCtrl>(static_cast<uint32_t>(k >> 32))) << 32) |
                     dpp_u32<kCtrl>(static_cast<uint32_t>(k));
  return o > k ? o : k;
}
template <int kCtrl>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __uint_as_float(dpp_u32<kCtrl>(__float_as_uint(v)));
}

// Maximum / sum over each aligned group of L lanes (L a power of two <= 16),
// the same value in every lane of the group: after the two quad steps a
// quad holds its result, half_mirror pairs the two quads of 8 lanes and
// row_mirror the two halves of 16.
template <int L>
__device__ __forceinline__ uint64_t group_max_key(uint64_t k) {
  static_assert(L >= 1 && L <= 16 && (L & (L - 1)) == 0, "group width");
  if constexpr (L >= 2) k = dpp_max_key<0xB1>(k);
  if constexpr (L >= 4) k = dpp_max_key<0x4E>(k);
  if constexpr (L >= 8) k = dpp_max_key<0x141>(k);
  if constexpr (L >= 16) k = dpp_max_key<0x140>(k);
  return k;
}
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2) v = dpp_add<0xB1>(v);
  if constexpr (L >= 4) v = dpp_add<0x4E>(v);
  if constexpr (L >= 8) v = dpp_add<0x141>(v);
  if constexpr (L >= 16) v = dpp_add<0x140>(v);
  return v;
}

// Top-k per token from a lane's logits acc[q][r] (expert le + q L, token
// t0 + r): k rounds, each taking the largest remaining key of the lane's P
// experts, then of the group's L lanes, and clearing it where it came from;
// the lane's R tokens go through each round together. Then the renormalised
// weights exp(l_i - l_0) / sum over the k kept ranks.
template <int L, int P, int R>
__device__ __forceinline__ void route_select(const float (&acc)[P][R], int le, int64_t t0,
                                             int64_t ntok, int E, int k,
                                             int32_t* __restrict__ topk_idx,
                                             float* __restrict__ topk_w) {
  uint64_t key[R][P], mine[R][P], first[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const int e = le + q * L;
      key[r][q] = e < E ? rank_key(acc[q][r], e) : 0;
      mine[r][q] = 0;
    }
  // Rank i (< k <= L * P) is kept by lane i % L of the group, in slot i / L.
  for (int i = 0; i < k; ++i) {
    const int owner = i % L, slot = i / L;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint64_t best = key[r][0];
#pragma unroll
      for (int q = 1; q < P; ++q) best = key[r][q] > best ? key[r][q] : best;
      best = group_max_key<L>(best);
      if (i == 0) first[r] = best;
#pragma unroll
      for (int q = 0; q < P; ++q) {
        key[r][q] = key[r][q] == best ? 0 : key[r][q];
        if (q == slot && le == owner) mine[r][q] = best;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t t = t0 + r;
    const float vmax = key_logit(first[r]);
    float u[P], sum = 0.0f;
#pragma unroll
    for (int q = 0; q < P; ++q) {
      u[q] = (q * L + le < k) ? expf(key_logit(mine[r][q]) - vmax) : 0.0f;
      sum += u[q];
    }
    sum = group_sum<L>(sum);
    if (t < ntok) {
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int i = q * L + le;
        if (i < k) {
          topk_idx[t * k + i] = key_expert(mine[r][q]);
          topk_w[t * k + i] = u[q] / sum;
        }
      }
    }
  }
}

// Lane layout: a token group of L lanes covers one token's experts, lane
// le of the group owning experts le, le + L, ..., le + (P-1) L; each lane
// evaluates R tokens for each of its P experts, so every token value read
// (and widened) feeds P multiply-adds and every router value read from LDS
// feeds R. 64 / L token groups per wave.
template <typename T, int L, int P, int R>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const T* __restrict__ x,
                                                              const float* __restrict__ wr,
                                                              int64_t ntok, int d, int E, int k,
                                                              int32_t* __restrict__ topk_idx,
                                                              float* __restrict__ topk_w) {
  constexpr int EPAD = L * P;
  __shared__ __attribute__((aligned(16))) float w_lds[EPAD * (kRouteChunk + kRoutePad)];  // [e][j]
  constexpr int kGroups = 64 / L;  // token groups per wave
  constexpr int kTokPerWave = kGroups * R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int le = lane % L, grp = lane / L;
  const int64_t tok0 = (static_cast<int64_t>(blockIdx.x) * (kRouteThreads / 64) + wave) * kTokPerWave;

  // Token rows this lane evaluates (clamped for the tail; not stored).
  const T* xrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t t = tok0 + grp * R + r;
    if (t >= ntok) t = ntok - 1;
    xrow[r] = x + t * d;
  }
  float acc[P][R];
#pragma unroll
  for (int q = 0; q < P; ++q)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[q][r] = 0.0f;

  constexpr int kStride = kRouteChunk + kRoutePad;
  for (int j0 = 0; j0 < d; j0 += kRouteChunk) {
    const int jn = min(kRouteChunk, d - j0);
    __syncthreads();
    // Stage W[j0 .. j0+jn)[0 .. E) transposed to [e][j], kFill loads in
    // flight per thread before their LDS stores.
    constexpr int kFill = 16;
    const int total = jn * EPAD;
    for (int i0 = threadIdx.x; i0 < total; i0 += kRouteThreads * kFill) {
      float v[kFill];
#pragma unroll
      for (int u = 0; u < kFill; ++u) {
        const int i = i0 + u * kRouteThreads;
        const int jj = i / EPAD, ee = i % EPAD;
        v[u] = (i < total && ee < E) ? wr[static_cast<int64_t>(j0 + jj) * E + ee] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kFill; ++u) {
        const int i = i0 + u * kRouteThreads;
        if (i < total) w_lds[(i % EPAD) * kStride + i / EPAD] = v[u];
      }
    }
    __syncthreads();
    for (int jj = 0; jj < jn; jj += 8) {
      float wv[P][8];
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const float* wl = w_lds + (le + q * L) * kStride + jj;
        const float4 w0 = *reinterpret_cast<const float4*>(wl);
        const float4 w1 = *reinterpret_cast<const float4*>(wl + 4);
        wv[q][0] = w0.x; wv[q][1] = w0.y; wv[q][2] = w0.z; wv[q][3] = w0.w;
        wv[q][4] = w1.x; wv[q][5] = w1.y; wv[q][6] = w1.z; wv[q][7] = w1.w;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float xv[8];
        load8(xrow[r] + j0 + jj, xv);
#pragma unroll
        for (int jq = 0; jq < 8; ++jq)
#pragma unroll
          for (int q = 0; q < P; ++q) acc[q][r] = __builtin_fmaf(xv[jq], wv[q][jq], acc[q][r]);
      }
    }
  }

  route_select<L, P, R>(acc, le, tok0 + grp * R, ntok, E, k, topk_idx, topk_w);
}

// Resident-router variant: one 1024-thread workgroup per CU keeps the whole
// router (all d rows, transposed to [e][j]) in LDS for its lifetime and
// walks token passes of (1024 / L) * R tokens, so W is read from memory
// once per CU. Same lane layout and the same fp32 chain per logit as
// route_kernel; the next 8 token values of each row are loaded while the
// current 8 are multiplied in.
constexpr int kResidentThreads = 1024;  // default workgroup size of the resident kernel

template <typename T, int L, int P, int R, int NT>
__global__ __launch_bounds__(NT) void route_resident_kernel(
    const T* __restrict__ x, const float* __restrict__ wr, int64_t ntok, int d, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  constexpr int EPAD = L * P;
  constexpr int XN = static_cast<int>(sizeof(T)) / 2;  // 16-byte pieces per 8 values
  constexpr int kPerPiece = 16 / static_cast<int>(sizeof(T));
  extern __shared__ __attribute__((aligned(16))) float w_res[];  // [EPAD][d + kRoutePad]
  const int stride = d + kRoutePad;
  // Router fill: kFill loads in flight per thread before their LDS stores
  // (one load at a time would cost an L2 round trip per element).
  constexpr int kFill = 16;
  const int total = d * EPAD;
  for (int i0 = threadIdx.x; i0 < total; i0 += NT * kFill) {
    float v[kFill];
#pragma unroll
    for (int u = 0; u < kFill; ++u) {
      const int i = i0 + u * NT;
      const int jj = i / EPAD, ee = i % EPAD;
      v[u] = (i < total && ee < E) ? wr[static_cast<int64_t>(jj) * E + ee] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kFill; ++u) {
      const int i = i0 + u * NT;
      if (i < total) w_res[(i % EPAD) * stride + i / EPAD] = v[u];
    }
  }
  __syncthreads();
  // Rows are d + 4 floats with d a multiple of 8: indexing whole float4s
  // lets the reads compile to 16-byte LDS loads.
  const float4* w4 = reinterpret_cast<const float4*>(w_res);
  const int stride4 = stride / 4;

  constexpr int kTokPerPass = (NT / 64) * (64 / L) * R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int le = lane % L, grp = lane / L;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kTokPerPass; base < ntok;
       base += static_cast<int64_t>(gridDim.x) * kTokPerPass) {
    const int64_t t0 = base + (wave * (64 / L) + grp) * R;
    const T* xrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int64_t t = t0 + r;
      if (t >= ntok) t = ntok - 1;  // clamped for the tail; not stored
      xrow[r] = x + t * d;
    }
    float acc[P][R];
#pragma unroll
    for (int q = 0; q < P; ++q)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[q][r] = 0.0f;

    // Token values 8 at a time, the next 8 loaded while the current ones are
    // multiplied in (two register sets used alternately, so nothing is
    // copied between steps).
    auto load = [&](u32x4 (&dst)[R][XN], int j) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int n = 0; n < XN; ++n)
          dst[r][n] = *reinterpret_cast<const u32x4*>(xrow[r] + j + n * kPerPiece);
    };
    auto step = [&](const u32x4 (&cur)[R][XN], int j) {
      // Router values four j at a time; each logit still takes j ascending.
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float wv[P][4];
#pragma unroll
        for (int q = 0; q < P; ++q) {
          const float4 w = w4[(le + q * L) * stride4 + (j >> 2) + h];
          wv[q][0] = w.x; wv[q][1] = w.y; wv[q][2] = w.z; wv[q][3] = w.w;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float xv[8];
          widen8<T>(cur[r], xv);
#pragma unroll
          for (int jq = 0; jq < 4; ++jq)
#pragma unroll
            for (int q = 0; q < P; ++q)
              acc[q][r] = __builtin_fmaf(xv[4 * h + jq], wv[q][jq], acc[q][r]);
        }
      }
    };
    u32x4 xa[R][XN], xb[R][XN];
    load(xa, 0);
    for (int jj = 0; jj < d; jj += 16) {
      if (jj + 8 < d) load(xb, jj + 8);
      step(xa, jj);
      if (jj + 8 >= d) break;
      if (jj + 16 < d) load(xa, jj + 16);
      step(xb, jj + 8);
    }
    route_select<L, P, R>(acc, le, t0, ntok, E, k, topk_idx, topk_w);
  }
}

template <typename T, int L, int P, int R>
size_t resident_lds_bytes(int d) {
  return static_cast<size_t>(L) * P * (d + kRoutePad) * sizeof(float);
}

template <typename T, int L, int P, int R, int NT = kResidentThreads>
hipError_t launch_route_resident(const void* x, const float* wr, int64_t T_, int d, int E, int k,
                                 int32_t* idx, float* w, hipStream_t s) {
  const size_t lds = resident_lds_bytes<T, L, P, R>(d);
  auto kern = route_resident_kernel<T, L, P, R, NT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  constexpr int kTokPerPass = (NT / 64) * (64 / L) * R;
  const int64_t passes = (T_ + kTokPerPass - 1) / kTokPerPass;
  const int64_t blocks = passes < cu_count() ? passes : cu_count();
  MOE_LAUNCH("route", kern, dim3(static_cast<unsigned>(blocks)), dim3(NT), lds, s,
             static_cast<const T*>(x), wr, T_, d, E, k, idx, w);
  return hipGetLastError();
}

template <typename T, int L, int P, int R>
hipError_t launch_route_chunked(const void* x, const float* wr, int64_t T_, int d, int E, int k,
                                int32_t* idx, float* w, hipStream_t s) {
  constexpr int kTokPerBlock = (kRouteThreads / 64) * (64 / L) * R;
  const int64_t blocks = (T_ + kTokPerBlock - 1) / kTokPerBlock;
  MOE_LAUNCH("route", (route_kernel<T, L, P, R>), dim3(static_cast<unsigned>(blocks)),
             dim3(kRouteThreads), 0, s, static_cast<const T*>(x), wr, T_, d, E, k, idx, w);
  return hipGetLastError();
}

// The router stays resident in LDS when it fits (E <= 64 at d <= 636, the
// padded expert count times d + 4 floats within 160 KiB); larger routers
// are streamed through LDS in 128-row chunks per 256-thread workgroup.
template <typename T>
hipError_t launch_route_dt(const void* x, const float* wr, int64_t T_, int d, int E, int k,
                           int32_t* idx, float* w, hipStream_t s) {
  const int epad = E <= 4 ? 4 : (E <= 8 ? 8 : (E <= 16 ? 16 : (E <= 32 ? 32 : 64)));
  if (E <= 64 && static_cast<size_t>(epad) * (d + kRoutePad) * sizeof(float) <= 160 * 1024) {
    // Tokens per lane R: the largest of 4, 2, 1 that still gives every CU a
    // workgroup (fewer tokens per pass for small batches).
    const int64_t cus = cu_count();
    auto fits = [&](int L, int R) { return T_ >= cus * (kResidentThreads / L) * R; };
    if (E <= 1) return launch_route_resident<T, 1, 1, 1>(x, wr, T_, d, E, k, idx, w, s);
    if (E <= 2) return launch_route_resident<T, 2, 1, 1>(x, wr, T_, d, E, k, idx, w, s);
    if (E <= 4) return launch_route_resident<T, 4, 1, 2>(x, wr, T_, d, E, k, idx, w, s);
    // One token per lane below 65536 tokens, so that more CUs get a
    // workgroup (E=8: 4096 fp32 tokens 0.037 -> 0.021 ms, 32768 bf16
    // tokens 0.026 -> 0.022 ms).
    if (E <= 8) {
      if (fits(8, 2)) return launch_route_resident<T, 8, 1, 2>(x, wr, T_, d, E, k, idx, w, s);
      return launch_route_resident<T, 8, 1, 1>(x, wr, T_, d, E, k, idx, w, s);
    }
    if (E <= 16) return launch_route_resident<T, 4, 4, 2>(x, wr, T_, d, E, k, idx, w, s);
    if (E <= 32) {
      if (fits(8, 2)) return launch_route_resident<T, 8, 4, 2>(x, wr, T_, d, E, k, idx, w, s);
      return launch_route_resident<T, 8, 4, 1>(x, wr, T_, d, E, k, idx, w, s);
    }
    // Eight experts per lane for large batches: each widened token value
    // feeds eight FMAs instead of four (the 210 registers this takes need
    // 512-thread workgroups; 0.238 -> 0.228 ms at 131072 tokens, E=64).
    if (fits(16, 4))
      return launch_route_resident<T, 8, 8, 4, 512>(x, wr, T_, d, E, k, idx, w, s);
    if (fits(16, 2)) return launch_route_resident<T, 16, 4, 2>(x, wr, T_, d, E, k, idx, w, s);
    return launch_route_resident<T, 16, 4, 1>(x, wr, T_, d, E, k, idx, w, s);
  }
  if (E <= 1) return launch_route_chunked<T, 1, 1, 1>(x, wr, T_, d, E, k, idx, w, s);
  if (E <= 2) return launch_route_chunked<T, 2, 1, 1>(x, wr, T_, d, E, k, idx, w, s);
  if (E <= 4) return launch_route_chunked<T, 4, 1, 1>(x, wr, T_, d, E, k, idx, w, s);
  if (E <= 8) return launch_route_chunked<T, 8, 1, 2>(x, wr, T_, d, E, k, idx, w, s);
  if (E <= 16) return launch_route_chunked<T, 4, 4, 2>(x, wr, T_, d, E, k, idx, w, s);
  if (E <= 32) return launch_route_chunked<T, 8, 4, 4>(x, wr, T_, d, E, k, idx, w, s);
  return launch_route_chunked<T, 16, 4, 8>(x, wr, T_, d, E, k, idx, w, s);
}

}  // namespace

hipError_t launch_route(int dtype, const void* x, const float* w_router, int64_t T, int d, int E,
                        int k, int32_t* topk_idx, float* topk_w, hipStream_t s) {
  if (dtype == MOE_BF16)
    return launch_route_dt<bf16_t>(x, w_router, T, d, E, k, topk_idx, topk_w, s);
  return launch_route_dt<float>(x, w_router, T, d, E, k, topk_idx, topk_w, s);
}

}  // namespace moe
