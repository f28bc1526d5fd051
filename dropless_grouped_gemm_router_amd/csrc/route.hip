// Stage "route": router logits, top-k selection and renormalised combine
// weights, one fused kernel (kernel_gmm_gpu.json "pieces" suite, piece
// "route").
//
// Lane layout: a token group of EP lanes (EP = next power of two >= E)
// holds one token's logits, lane e of the group owning expert e; each lane
// evaluates R tokens for its expert so every router value read from LDS
// feeds R fused multiply-adds. Logits are the fixed fp32 chain
// acc = fma(x[t,j], W[j,e], acc) for j ascending from +0.0, evaluated in
// exactly that order (the chunking over j below only pauses the chain).
// The selection runs k rounds of a butterfly argmax inside the group on
// (logit descending, expert index ascending); no floating-point reduction
// decides an expert.
#include "common.h"

namespace moe {

namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteChunk = 256;  // router rows (j) staged in LDS per pass
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

// a ranks before b: valid before invalid, then larger logit, then lower index.
__device__ __forceinline__ bool ranks_before(float av, int ae, float bv, int be) {
  const bool a_ok = ae < 0x10000, b_ok = be < 0x10000;
  if (a_ok != b_ok) return a_ok;
  return (av > bv) || (av == bv && ae < be);
}

template <typename T, int EP, int R>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const T* __restrict__ x,
                                                              const float* __restrict__ wr,
                                                              int64_t ntok, int d, int E, int k,
                                                              int32_t* __restrict__ topk_idx,
                                                              float* __restrict__ topk_w) {
  __shared__ __attribute__((aligned(16))) float w_lds[EP * (kRouteChunk + kRoutePad)];  // [e][j]
  constexpr int kGroups = 64 / EP;  // token groups per wave
  constexpr int kTokPerWave = kGroups * R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = lane % EP, grp = lane / EP;
  const int64_t tok0 = (static_cast<int64_t>(blockIdx.x) * (kRouteThreads / 64) + wave) * kTokPerWave;

  // Token rows this lane evaluates (clamped for the tail; not stored).
  const T* xrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t t = tok0 + grp * R + r;
    if (t >= ntok) t = ntok - 1;
    xrow[r] = x + t * d;
  }
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;

  constexpr int kStride = kRouteChunk + kRoutePad;
  for (int j0 = 0; j0 < d; j0 += kRouteChunk) {
    const int jn = min(kRouteChunk, d - j0);
    __syncthreads();
    // Stage W[j0 .. j0+jn)[0 .. E) transposed to [e][j].
    for (int i = threadIdx.x; i < jn * EP; i += kRouteThreads) {
      const int jj = i / EP, ee = i % EP;
      w_lds[ee * kStride + jj] = (ee < E) ? wr[static_cast<int64_t>(j0 + jj) * E + ee] : 0.0f;
    }
    __syncthreads();
    const float* wl = w_lds + e * kStride;
    for (int jj = 0; jj < jn; jj += 8) {
      float4 w0 = *reinterpret_cast<const float4*>(wl + jj);
      float4 w1 = *reinterpret_cast<const float4*>(wl + jj + 4);
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float xv[8];
        load8(xrow[r] + j0 + jj, xv);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[r] = __builtin_fmaf(xv[q], wv[q], acc[r]);
      }
    }
  }

  // Top-k per token: k rounds of a butterfly argmax within the EP-lane group.
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t t = tok0 + grp * R + r;
    const float v = acc[r];
    bool taken = (e >= E);
    float my_v = 0.0f, vmax = 0.0f;
    int my_e = 0;
    for (int i = 0; i < k; ++i) {
      float bv = v;
      int be = taken ? (0x10000 + e) : e;
#pragma unroll
      for (int off = EP / 2; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, EP);
        const int oe = __shfl_xor(be, off, EP);
        if (ranks_before(ov, oe, bv, be)) {
          bv = ov;
          be = oe;
        }
      }
      if (i == 0) vmax = bv;
      if (be == e) taken = true;
      if (e == i) {
        my_v = bv;
        my_e = be;
      }
    }
    float u = (e < k) ? expf(my_v - vmax) : 0.0f;
    float sum = u;
#pragma unroll
    for (int off = EP / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, EP);
    if (e < k && t < ntok) {
      topk_idx[t * k + e] = my_e;
      topk_w[t * k + e] = u / sum;
    }
  }
}

template <typename T, int EP, int R>
hipError_t launch_route_t(const void* x, const float* wr, int64_t T_, int d, int E, int k,
                          int32_t* idx, float* w, hipStream_t s) {
  constexpr int kTokPerBlock = (kRouteThreads / 64) * (64 / EP) * R;
  const int64_t blocks = (T_ + kTokPerBlock - 1) / kTokPerBlock;
  MOE_LAUNCH("route", (route_kernel<T, EP, R>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kRouteThreads), 0, s, static_cast<const T*>(x), wr, T_, d, E, k, idx,
                     w);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_route_dt(const void* x, const float* wr, int64_t T_, int d, int E, int k,
                           int32_t* idx, float* w, hipStream_t s) {
  if (E <= 1) return launch_route_t<T, 1, 1>(x, wr, T_, d, E, k, idx, w, s);
  if (E <= 2) return launch_route_t<T, 2, 1>(x, wr, T_, d, E, k, idx, w, s);
  if (E <= 4) return launch_route_t<T, 4, 1>(x, wr, T_, d, E, k, idx, w, s);
  if (E <= 8) return launch_route_t<T, 8, 2>(x, wr, T_, d, E, k, idx, w, s);
  if (E <= 16) return launch_route_t<T, 16, 4>(x, wr, T_, d, E, k, idx, w, s);
  if (E <= 32) return launch_route_t<T, 32, 8>(x, wr, T_, d, E, k, idx, w, s);
  return launch_route_t<T, 64, 8>(x, wr, T_, d, E, k, idx, w, s);
}

}  // namespace

hipError_t launch_route(int dtype, const void* x, const float* w_router, int64_t T, int d, int E,
                        int k, int32_t* topk_idx, float* topk_w, hipStream_t s) {
  if (dtype == MOE_BF16)
    return launch_route_dt<bf16_t>(x, w_router, T, d, E, k, topk_idx, topk_w, s);
  return launch_route_dt<float>(x, w_router, T, d, E, k, topk_idx, topk_w, s);
}

}  // namespace moe
