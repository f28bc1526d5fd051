// C ABI of libmoe: argument validation, workspace sizing and stage launches.
// Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "common.h"
#include "moe.h"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using moe::align_up;

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// Non-null and aligned.
bool ok_ptr(const void* ptr, size_t a = 16) { return ptr != nullptr && aligned(ptr, a); }

int check(const moe_problem* p) {
  if (!p) return MOE_ERR_INVALID;
  if (p->tokens < 0 || p->experts < 1 || p->top_k < 1 || p->top_k > p->experts ||
      p->d_model < 1 || p->d_hidden < 1 || p->d_shared < 0 || p->capacity < 0)
    return MOE_ERR_INVALID;
  if (p->dtype != MOE_FP32 && p->dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (p->block_m != 32 && p->block_m != 64 && p->block_m != 128 && p->block_m != 256)
    return MOE_ERR_UNSUPPORTED;
  if (p->experts > 64) return MOE_ERR_UNSUPPORTED;
  if (p->d_model % 128 != 0 || p->d_model > 8192) return MOE_ERR_UNSUPPORTED;
  if (p->d_hidden % 64 != 0 || p->d_shared % 64 != 0) return MOE_ERR_UNSUPPORTED;
  // tokens * top_k < 2^31, tested without forming the product (tokens may be
  // anywhere up to INT64_MAX)
  if (p->tokens > ((int64_t{1} << 31) - 1) / p->top_k) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t elem_size(const moe_problem* p) { return p->dtype == MOE_BF16 ? 2 : 4; }

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

MOE_EXPORT const char* moe_version(void) { return "libmoe 0.1 (gfx950)"; }

MOE_EXPORT const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported problem";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_TOO_LARGE: return "problem exceeds the fixed scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

MOE_EXPORT int moe_check_problem(const moe_problem* p) { return check(p); }

MOE_EXPORT int64_t moe_max_tiles(const moe_problem* p) {
  if (check(p) != MOE_OK) return 0;
  const int64_t S = p->tokens * p->top_k;
  return (S + p->block_m - 1) / p->block_m + p->experts;
}

MOE_EXPORT int64_t moe_param_count(const moe_problem* p) {
  if (check(p) != MOE_OK) return -1;
  const int64_t E = p->experts, d = p->d_model, h = p->d_hidden, hs = p->d_shared;
  return 3 * E * d * h + d * E + 3 * d * hs;
}

MOE_EXPORT size_t moe_workspace_bytes(const moe_problem* p, int training) {
  if (check(p) != MOE_OK) return 0;
  size_t b = moe::permute_ws_bytes(p->tokens * p->top_k, p->experts);
  b = std::max(b, moe::ffn_layout(*p, training != 0).total);
  if (training) b = std::max(b, moe::bwd_ws_bytes(*p));
  return std::max<size_t>(b, 256);
}

MOE_EXPORT size_t moe_saved_bytes(const moe_problem* p) {
  if (check(p) != MOE_OK) return 0;
  return moe::ffn_layout(*p, true).sv_total;
}

MOE_EXPORT int moe_route(const moe_problem* p, const void* x, const float* w_router,
                         moe_routing* r, void* stream) {
  int st = check(p);
  if (st != MOE_OK) return st;
  if (p->tokens == 0) return MOE_OK;
  if (!r || !ok_ptr(x) || !ok_ptr(w_router, 4) || !ok_ptr(r->topk_idx, 4) || !ok_ptr(r->topk_w, 4))
    return MOE_ERR_INVALID;
  return hip_status(moe::launch_route(p->dtype, x, w_router, p->tokens, p->d_model, p->experts,
                                      p->top_k, r->topk_idx, r->topk_w, as_stream(stream)));
}

MOE_EXPORT int moe_permute(const moe_problem* p, moe_routing* r, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int st = check(p);
  if (st != MOE_OK) return st;
  if (p->tokens == 0) return MOE_OK;
  if (!r || !ok_ptr(r->topk_idx, 4) || !ok_ptr(r->expert_offsets, 4) || !ok_ptr(r->perm, 4) ||
      !ok_ptr(r->inv_perm, 4) || !ok_ptr(r->tiles, 4) || !ok_ptr(r->num_tiles, 4) ||
      !ok_ptr(workspace, 256))
    return MOE_ERR_INVALID;
  if (workspace_bytes < moe::permute_ws_bytes(p->tokens * p->top_k, p->experts))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_permute(p->tokens, p->top_k, p->experts, p->block_m,
                                        p->capacity, r->topk_idx,
                                        r->expert_offsets, r->perm, r->inv_perm, r->tiles,
                                        r->num_tiles, workspace, as_stream(stream)));
}

MOE_EXPORT int moe_permute_static(const moe_problem* p, moe_routing* r, void* stream) {
  int st = check(p);
  if (st != MOE_OK) return st;
  if (p->tokens == 0) return MOE_OK;
  if (!r || !ok_ptr(r->topk_idx, 4) || !ok_ptr(r->expert_offsets, 4) || !ok_ptr(r->perm, 4) ||
      !ok_ptr(r->inv_perm, 4) || !ok_ptr(r->tiles, 4) || !ok_ptr(r->num_tiles, 4))
    return MOE_ERR_INVALID;
  if (moe::permute_ws_bytes(p->tokens * p->top_k, p->experts) > moe::static_scratch_bytes())
    return MOE_ERR_TOO_LARGE;
  void* scratch = nullptr;
  const hipError_t e = moe::static_scratch(&scratch);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_permute(p->tokens, p->top_k, p->experts, p->block_m,
                                        p->capacity, r->topk_idx, r->expert_offsets, r->perm,
                                        r->inv_perm, r->tiles, r->num_tiles, scratch,
                                        as_stream(stream)));
}

MOE_EXPORT int moe_ffn_fwd(const moe_problem* p, const void* x, const moe_weights* w,
                           const moe_routing* r, void* y_sorted, void* shared_out, void* saved,
                           void* workspace, size_t workspace_bytes, void* stream) {
  int st = check(p);
  if (st != MOE_OK) return st;
  if (p->tokens == 0) return MOE_OK;
  if (!w || !r || !ok_ptr(x) || !ok_ptr(w->w_gate) || !ok_ptr(w->w_up) || !ok_ptr(w->w_down) ||
      !ok_ptr(r->perm, 4) || !ok_ptr(r->tiles, 4) || !ok_ptr(r->num_tiles, 4) ||
      !ok_ptr(y_sorted) || !ok_ptr(workspace, 256))
    return MOE_ERR_INVALID;
  if (p->d_shared > 0 &&
      (!ok_ptr(w->ws_gate) || !ok_ptr(w->ws_up) || !ok_ptr(w->ws_down) || !ok_ptr(shared_out)))
    return MOE_ERR_INVALID;
  if (saved && !aligned(saved, 256)) return MOE_ERR_INVALID;
  if (workspace_bytes < moe::ffn_layout(*p, saved != nullptr).total) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_ffn_fwd(*p, x, *w, *r, y_sorted, p->d_shared > 0 ? shared_out : nullptr,
                                        saved, workspace, as_stream(stream)));
}

MOE_EXPORT int moe_combine(const moe_problem* p, const void* y_sorted, const moe_routing* r,
                           const void* shared_out, void* out, void* stream) {
  int st = check(p);
  if (st != MOE_OK) return st;
  if (p->tokens == 0) return MOE_OK;
  if (!r || !ok_ptr(y_sorted) || !ok_ptr(r->topk_w, 4) || !ok_ptr(r->inv_perm, 4) || !ok_ptr(out) ||
      (shared_out && !aligned(shared_out, 16)))
    return MOE_ERR_INVALID;
  return hip_status(moe::launch_combine(p->dtype, p->tokens, p->top_k, p->d_model, y_sorted,
                                        r->topk_w, r->inv_perm, shared_out, out,
                                        as_stream(stream)));
}

MOE_EXPORT size_t moe_forward_workspace_bytes(const moe_problem* p, int dispatch, int training) {
  if (check(p) != MOE_OK) return 0;
  if (dispatch < MOE_DISPATCH_GATHER || dispatch > MOE_DISPATCH_FUSED_GSUM) return 0;
  return moe::forward_layout(*p, dispatch, training != 0).total;
}

MOE_EXPORT int moe_forward(const moe_problem* p, int dispatch, const void* x, const moe_weights* w,
                           moe_routing* r, void* y_sorted, void* saved, void* out, void* workspace,
                           size_t workspace_bytes, void* stream, void* side_stream) {
  if (dispatch < MOE_DISPATCH_GATHER || dispatch > MOE_DISPATCH_FUSED_GSUM) return MOE_ERR_INVALID;
  int st = check(p);
  if (st != MOE_OK) return st;
  if (p->tokens == 0) return MOE_OK;
  if (!w || !r || !ok_ptr(x) || !ok_ptr(w->w_router, 4) || !ok_ptr(w->w_gate) || !ok_ptr(w->w_up) ||
      !ok_ptr(w->w_down) || !ok_ptr(r->topk_idx, 4) || !ok_ptr(r->topk_w, 4) ||
      !ok_ptr(r->expert_offsets, 4) || !ok_ptr(r->perm, 4) || !ok_ptr(r->inv_perm, 4) ||
      !ok_ptr(r->tiles, 4) || !ok_ptr(r->num_tiles, 4) || !ok_ptr(y_sorted) || !ok_ptr(out) ||
      !ok_ptr(workspace, 256))
    return MOE_ERR_INVALID;
  if (p->d_shared > 0 && (!ok_ptr(w->ws_gate) || !ok_ptr(w->ws_up) || !ok_ptr(w->ws_down)))
    return MOE_ERR_INVALID;
  if (saved && !aligned(saved, 256)) return MOE_ERR_INVALID;
  if (workspace_bytes < moe::forward_layout(*p, dispatch, saved != nullptr).total)
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_forward(*p, dispatch, x, *w, *r, y_sorted, saved, out, workspace,
                                        as_stream(stream), as_stream(side_stream)));
}

MOE_EXPORT int moe_bwd(const moe_problem* p, const void* x, const moe_weights* w,
                       const moe_routing* r, const void* y_sorted, const void* saved,
                       const void* grad_out, void* grad_x, const moe_grads* g, void* workspace,
                       size_t workspace_bytes, void* stream, void* side_stream) {
  int st = check(p);
  if (st != MOE_OK) return st;
  // The backward GEMMs tile the hidden widths by 128.
  if (p->d_hidden % 128 != 0 || p->d_shared % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (!g || !ok_ptr(g->w_router, 4) || !ok_ptr(g->w_gate) || !ok_ptr(g->w_up) ||
      !ok_ptr(g->w_down))
    return MOE_ERR_INVALID;
  if (p->d_shared > 0 && (!ok_ptr(g->ws_gate) || !ok_ptr(g->ws_up) || !ok_ptr(g->ws_down)))
    return MOE_ERR_INVALID;
  if (p->tokens == 0) {
    // Nothing flows back from zero tokens, yet the gradients are defined
    // (zero) and fully overwritten.
    return hip_status(moe::launch_bwd(*p, x, w ? *w : moe_weights{}, r ? *r : moe_routing{},
                                      y_sorted, saved, grad_out, grad_x, *g, workspace,
                                      as_stream(stream), nullptr));
  }
  if (!w || !r || !ok_ptr(x) || !ok_ptr(w->w_router, 4) || !ok_ptr(w->w_gate) || !ok_ptr(w->w_up) ||
      !ok_ptr(w->w_down) || !ok_ptr(r->topk_idx, 4) || !ok_ptr(r->topk_w, 4) ||
      !ok_ptr(r->expert_offsets, 4) || !ok_ptr(r->perm, 4) || !ok_ptr(r->inv_perm, 4) ||
      !ok_ptr(r->tiles, 4) || !ok_ptr(r->num_tiles, 4) ||
      (p->dtype != MOE_BF16 && !ok_ptr(y_sorted)) ||  // the bf16 backward does not read it
      !ok_ptr(saved, 256) || !ok_ptr(grad_out) || !ok_ptr(grad_x) || !ok_ptr(g->w_gate) ||
      !ok_ptr(g->w_up) || !ok_ptr(g->w_down) || !ok_ptr(workspace, 256))
    return MOE_ERR_INVALID;
  if (p->d_shared > 0 && (!ok_ptr(w->ws_gate) || !ok_ptr(w->ws_up) || !ok_ptr(w->ws_down) ||
                          !ok_ptr(g->ws_gate) || !ok_ptr(g->ws_up) || !ok_ptr(g->ws_down)))
    return MOE_ERR_INVALID;
  if (workspace_bytes < moe::bwd_ws_bytes(*p)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_bwd(*p, x, *w, *r, y_sorted, saved, grad_out, grad_x, *g,
                                    workspace, as_stream(stream), as_stream(side_stream)));
}
