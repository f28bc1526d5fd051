// Internal definitions shared by the libmoe kernels and host code (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "moe.h"

namespace moe {

typedef uint16_t bf16_t;  // bf16 bit pattern

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
// 16 bytes as a native vector (plain loads/stores and SSA values; HIP's
// uint4 is a struct whose copies can turn into memcpy).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; NaN inputs stay NaN (quiet bit forced). gfx950
// converts in hardware (v_cvt_pk_bf16_f32, two values per instruction):
// over all 2^32 fp32 inputs it gives the same bits as the integer rounding
// (add 0x7fff plus the lowest kept bit, keep the high half; NaN: high half
// with the quiet bit set), which costs about six VALU instructions and two
// exec-mask branches per value.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_hw v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw));
}

// Low / high bf16 of a packed pair, widened exactly.
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// The hardware reciprocal (1 ulp) instead of an IEEE division: a few
// instructions instead of a dozen per element. Large |a| behaves as the
// division: exp(-a) = inf gives 0, exp(-a) = 0 gives 1.
__device__ __forceinline__ float sigmoid_f(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }
__device__ __forceinline__ float silu_f(float a) { return a * sigmoid_f(a); }

// Elements of one storage type per 16-byte chunk.
template <typename T>
struct Elem;
template <>
struct Elem<bf16_t> {
  static constexpr int kPer16B = 8;
};
template <>
struct Elem<float> {
  static constexpr int kPer16B = 4;
};

// Store four consecutive accumulator values as one 8-byte (bf16) or
// 16-byte (fp32) write.
__device__ __forceinline__ void store4(bf16_t* p, float a, float b, float c, float d) {
  uint2 v;
  v.x = pack_bf16x2(a, b);
  v.y = pack_bf16x2(c, d);
  *reinterpret_cast<uint2*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void load4(const bf16_t* p, float* o) {
  uint2 v = *reinterpret_cast<const uint2*>(p);
  o[0] = bf16lo(v.x);
  o[1] = bf16hi(v.x);
  o[2] = bf16lo(v.y);
  o[3] = bf16hi(v.y);
}
__device__ __forceinline__ void load4(const float* p, float* o) {
  float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x;
  o[1] = v.y;
  o[2] = v.z;
  o[3] = v.w;
}

// XCD-aware block order: workgroups are handed to the 8 XCDs round-robin
// (block b runs on XCD b % 8). Give each XCD one contiguous range of
// logical work items so that neighbouring tiles (same expert, same
// weights) share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  const int x = b & 7, i = b >> 3;
  const int q = nblocks >> 3, r = nblocks & 7;
  return x * q + (x < r ? x : r) + i;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workgroups of `kernel` (block size `threads`) the current device keeps
// resident at once: CUs x workgroups per CU (cached per device and kernel).
int persistent_slots(const void* kernel, int threads);
// Compute units of the current device.
int cu_count();

// Runs a call's independent part on a second stream that the caller
// passes (side may be null: no second stream, everything on s). The fork,
// mark and join events are created by fork() and released by the
// destructor, so the library itself keeps no stream or event between calls.
// Work enqueued on side() between fork() and join() runs beside s, after
// everything enqueued on s before the fork, and s waits for it from the
// join on. mark() records a point on the side stream that s waits for at
// wait_mark(). If a call returns between fork() and join() (an error path),
// the destructor still joins, so nothing enqueued on the side stream stays
// unordered against s. While the kernel timer is on, the second stream is s
// itself, so each timed kernel runs alone.
class StreamFork {
 public:
  StreamFork(hipStream_t s, hipStream_t side);
  ~StreamFork();
  StreamFork(const StreamFork&) = delete;
  StreamFork& operator=(const StreamFork&) = delete;
  hipError_t fork();
  hipError_t mark();
  hipError_t wait_mark();
  hipError_t join();
  hipStream_t side() const { return forked_ ? side_ : caller_; }

 private:
  hipStream_t caller_, side_;
  bool forked_ = false, joined_ = false;
  hipEvent_t ev_fork_ = nullptr, ev_mark_ = nullptr, ev_join_ = nullptr;
};

// Per-kernel event timing (trace.cpp); no-ops unless moe_trace_enable(1).
bool trace_on();
void trace_push(hipStream_t s, const char* name);
void trace_pop(hipStream_t s);

#define MOE_LAUNCH(name, kernel, grid, block, lds, stream, ...)          \
  do {                                                                  \
    ::moe::trace_push(stream, name);                                    \
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);  \
    ::moe::trace_pop(stream);                                           \
  } while (0)

// ---------------------------------------------------------------- launches
// Host-side launchers (defined in the .hip files). They assume validated
// arguments and return the hipGetLastError() of their launches.

hipError_t launch_route(int dtype, const void* x, const float* w_router, int64_t T, int d, int E,
                        int k, int32_t* topk_idx, float* topk_w, hipStream_t s);

size_t permute_ws_bytes(int64_t S, int E);
// The fixed device scratch of the allocation-free permute (moe_permute_static):
// its size, and its address on the current device (looked up on the first
// call per device).
size_t static_scratch_bytes();
hipError_t static_scratch(void** out);
hipError_t launch_permute(int64_t T, int k, int E, int bm, int cap, const int32_t* topk_idx,
                          int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* tiles,
                          int32_t* num_tiles, void* ws, hipStream_t s);

// 256-row tile list for the GEMMs that run faster on the wide engine than
// on the caller's block_m (see retile_rows), from the expert offsets.
// Returns hipPeekAtLastError(): a launch error is left pending, not cleared.
hipError_t launch_retile(const int32_t* offsets, int E, int bm2, int cap, int32_t* tiles,
                         int32_t* num_tiles, hipStream_t s);
constexpr int kRetileBm = 256;
// Bytes of a retiled list for S token-slots and E experts (tiles + count).
inline size_t retile_bytes(int64_t S, int E) {
  return static_cast<size_t>((S + kRetileBm - 1) / kRetileBm + E) * 12 + 16;
}
// Whether a bf16 grouped GEMM over block_m-row tiles takes a 256-row list
// instead: the caller's tiles are narrower and experts average at least 512
// rows (fewer padded rows than that make the wider tiles a loss).
inline bool retile_rows(const moe_problem& p) {
  return p.dtype == MOE_BF16 && p.block_m < kRetileBm &&
         p.tokens * p.top_k >= static_cast<int64_t>(512) * p.experts;
}

hipError_t launch_combine(int dtype, int64_t T, int k, int d, const void* y_sorted,
                          const float* topk_w, const int32_t* inv_perm, const void* shared_out,
                          void* out, hipStream_t s);

struct FfnLayout {
  // workspace offsets (bytes) of the packed weights and activations, and of
  // the 256-row tile list (retile_rows)
  size_t gu_packed, down_packed, sgu_packed, sdown_packed, h_sorted, h_shared, tiles256, total;
  // saved-buffer offsets (bytes)
  size_t sv_ab, sv_h, sv_sab, sv_sh, sv_total;
};
FfnLayout ffn_layout(const moe_problem& p, bool training);

hipError_t launch_ffn_fwd(const moe_problem& p, const void* x, const moe_weights& w,
                          const moe_routing& r, void* y_sorted, void* shared_out, void* saved,
                          void* ws, hipStream_t s);

// Whole forward (moe_forward): workspace offsets (bytes) of the permute
// scratch, the staged shared-expert output and the expert-ordered token
// copy, after the FFN area at offset 0.
struct ForwardLayout {
  size_t permute, shared_out, x_sorted, total;
  bool fused;  // the combine runs in the shared down GEMM's epilogue
};
ForwardLayout forward_layout(const moe_problem& p, int dispatch, bool training);
hipError_t launch_forward(const moe_problem& p, int dispatch, const void* x, const moe_weights& w,
                          const moe_routing& r, void* y_sorted, void* saved, void* out, void* ws,
                          hipStream_t s, hipStream_t side);

size_t bwd_ws_bytes(const moe_problem& p);
hipError_t launch_bwd(const moe_problem& p, const void* x, const moe_weights& w,
                      const moe_routing& r, const void* y_sorted, const void* saved,
                      const void* grad_out, void* grad_x, const moe_grads& g, void* ws,
                      hipStream_t s, hipStream_t side);

}  // namespace moe
