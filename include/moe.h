/*
 * moe.h - C ABI of libmoe, the MI355X (gfx950) dropless top-k
 * Mixture-of-Experts layer: forward and train-step backward.
 *
 * The layer (probjax benchmark pages kernel_gmm_gpu.json, gpu_nn.json and
 * gpu_moe_h100.json; stage names from the kernel_gmm_gpu.json "pieces"
 * suite: route -> sort_permute -> experts_grouped_swiglu ->
 * unpermute_combine):
 *
 *   logits[t,e] = sum_j x[t,j] * w_router[j,e]             (no bias)
 *   keep the top_k experts of each token by logit, the lower expert index
 *   winning ties; weights w[t,i] = softmax of the kept logits (the softmax
 *   over all experts renormalised over the kept ones)
 *   out[t] = sum_i w[t,i] * FFN_{e_i}(x[t]) + FFN_shared(x[t])
 *   FFN_e(v) = (SiLU(v W_gate[e]) * (v W_up[e])) W_down[e]
 *
 * "Dropless": every one of the tokens*top_k token-slots is computed (record
 * field "routing": "dropless" on kernel_gmm_gpu.json; the gpu_moe_h100.json
 * header describes the layer as dropless). No biases anywhere (gpu_nn.json
 * "moe" records: params = 3*E*d*h + d*E).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise; every array is
 *     dense row-major and 16-byte aligned.
 *   - The caller owns all memory, including the workspace. The library
 *     never allocates, frees or retains a pointer after the call returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without synchronising. Buffers must stay valid
 *     until the stream has executed the work.
 *   - All argument checks run on the host before anything is enqueued; a
 *     call that returns an error has enqueued nothing (MOE_ERR_HIP aside,
 *     which reports a failed launch).
 *   - tokens == 0 is a successful no-op, except that moe_bwd then zeroes
 *     the weight gradients (the gradient of an empty batch).
 *   - Values inside device buffers are not checked: an out-of-range expert
 *     index passed to moe_permute, or a routing state not produced by
 *     moe_route/moe_permute for the same problem, is undefined behaviour.
 *   - No global mutable state besides the optional kernel timer below (a
 *     diagnostic, off unless enabled) and the device address of
 *     moe_permute_static's fixed scratch, looked up once per device: calls
 *     on distinct streams may run concurrently from several host threads.
 *     No device memory is allocated.
 *   - moe_forward and moe_bwd take an optional second stream, side_stream
 *     (NULL or equal to `stream`: everything runs on `stream`). With one,
 *     a problem with a shared expert runs the shared expert's kernels
 *     there, forked from and joined back to `stream` with events created
 *     for the call and released with it, so the caller sees one stream's
 *     ordering and both streams' work is done once `stream` reaches the
 *     call's end; moe_forward also packs the routed experts' weights there
 *     first, and its routed GEMMs wait for that. The caller owns the side
 *     stream; work it already holds runs before the fork point. The results
 *     are the same bits with or without it.
 *   - Results are deterministic: no floating-point atomics are used, and
 *     repeated calls on the same inputs give identical bits.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,     /* null pointer, bad size, misaligned pointer */
  MOE_ERR_UNSUPPORTED = -2, /* valid problem outside what the kernels implement */
  MOE_ERR_WORKSPACE = -3,   /* workspace smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = -4,         /* a kernel launch failed */
  MOE_ERR_TOO_LARGE = -5    /* beyond the fixed scratch of moe_permute_static */
} moe_status;

typedef enum { MOE_FP32 = 0, MOE_BF16 = 1 } moe_dtype;

/*
 * Problem statement, in the pages' record fields: tokens, experts, top_k,
 * d_model, d_hidden, dtype (kernel_gmm_gpu.json "results" records), the
 * shared expert width (gpu_moe_h100.json records, field "shared") and the
 * grouped-GEMM row tile block_m (kernel_gmm_gpu.json config blocks,
 * "block_m" / "block_ms": 32, 64, 128 on the pages' hardware; 256 is
 * supported too and is the gfx950 choice for large problems).
 *
 * dtype is the storage type of x, the expert and shared weights, the
 * sorted expert outputs, the shared-expert output, out, grad_out, grad_x
 * and the saved activations. Accumulation is always fp32. The router
 * matrix, the combine weights and all weight gradients are fp32 in both
 * modes (kernel_gmm_gpu.json "pieces" records, field "xla_arg_mb": the
 * route piece takes bf16 tokens with an fp32 router and the combine piece
 * bf16 expert outputs with fp32 weights).
 *
 * capacity (kernel_gmm_gpu.json records, field "routing": "capacity"
 * against "dropless"): 0 routes every token-slot (dropless). capacity > 0
 * caps each expert at that many token-slots, the first ones in flat slot
 * order t*top_k + i (ascending token): the rest are dropped, contribute
 * nothing to out and no gradient to their expert's weights, and the kept
 * combine weights are not renormalised. The pages name the variant but give
 * neither the capacity nor the drop rule; this is the rule implemented.
 *
 * Supported (else MOE_ERR_UNSUPPORTED): 1 <= experts <= 64,
 * 1 <= top_k <= experts, d_model a multiple of 128 (at most 8192),
 * d_hidden and d_shared multiples of 64 (d_shared may be 0), block_m in
 * {32, 64, 128, 256}, tokens*top_k < 2^31.
 */
typedef struct {
  int64_t tokens;
  int32_t experts;
  int32_t top_k;
  int32_t d_model;
  int32_t d_hidden;
  int32_t d_shared; /* 0 = no shared expert */
  int32_t dtype;    /* moe_dtype */
  int32_t block_m;
  int32_t capacity; /* max token-slots per expert; 0 = dropless; < 0 is MOE_ERR_INVALID */
} moe_problem;

/* Layer weights (device, caller-owned, read only). */
typedef struct {
  const float* w_router; /* [d_model, experts], fp32 */
  const void* w_gate;    /* [experts, d_model, d_hidden], dtype */
  const void* w_up;      /* [experts, d_model, d_hidden], dtype */
  const void* w_down;    /* [experts, d_hidden, d_model], dtype */
  const void* ws_gate;   /* [d_model, d_shared], dtype; NULL when d_shared == 0 */
  const void* ws_up;     /* [d_model, d_shared], dtype; NULL when d_shared == 0 */
  const void* ws_down;   /* [d_shared, d_model], dtype; NULL when d_shared == 0 */
} moe_weights;

/*
 * Routing state written by moe_route and moe_permute, read by the later
 * stages. S = tokens * top_k token-slots; flat slot s = t*top_k + i.
 */
typedef struct {
  int32_t* topk_idx;       /* [tokens, top_k]: kept experts in rank order (logit desc, index asc) */
  float* topk_w;           /* [tokens, top_k]: renormalised combine weights */
  int32_t* expert_offsets; /* [experts + 1]: first sorted row of each expert; [experts] = S */
  int32_t* perm;           /* [S]: sorted row -> flat slot; rows of one expert in ascending slot order */
  int32_t* inv_perm;       /* [S]: flat slot -> sorted row; -1 if capacity dropped the slot */
  int32_t* tiles;          /* [moe_max_tiles(), 3]: (expert, first sorted row, rows <= block_m),
                              covering each expert's kept rows */
  int32_t* num_tiles;      /* [1]: number of valid entries of tiles */
} moe_routing;

/* Weight gradients (device, fp32, fully overwritten). */
typedef struct {
  float* w_router; /* [d_model, experts] */
  float* w_gate;   /* [experts, d_model, d_hidden] */
  float* w_up;     /* [experts, d_model, d_hidden] */
  float* w_down;   /* [experts, d_hidden, d_model] */
  float* ws_gate;  /* [d_model, d_shared]; ignored when d_shared == 0 */
  float* ws_up;    /* [d_model, d_shared]; ignored when d_shared == 0 */
  float* ws_down;  /* [d_shared, d_model]; ignored when d_shared == 0 */
} moe_grads;

/* Library version string (host). */
const char* moe_version(void);

/* Human-readable name of a moe_status value (host). */
const char* moe_status_string(int status);

/* Checks a problem statement (host). MOE_OK, MOE_ERR_INVALID or MOE_ERR_UNSUPPORTED. */
int moe_check_problem(const moe_problem* p);

/*
 * Upper bound on the number of block_m tiles (host): ceil(S / block_m) +
 * experts, since each expert's last tile may be partial. Size of the tiles
 * array in moe_routing, in (expert, row, rows) triples. 0 for an invalid
 * problem.
 */
int64_t moe_max_tiles(const moe_problem* p);

/*
 * Parameter count (host): 3*E*d*h + d*E + 3*d*hs, i.e. three matrices per
 * expert, a bias-free router and three shared matrices. gpu_nn.json, "moe"
 * suite, field "params" (12,587,008 at E=8, d_model 512, d_hidden 1024).
 * -1 for an invalid problem.
 */
int64_t moe_param_count(const moe_problem* p);

/*
 * Workspace bytes (host) that moe_permute, moe_ffn_fwd (training = 0) and,
 * with training = 1, moe_bwd need; one buffer of this size serves every
 * stage. 0 for an invalid problem.
 */
size_t moe_workspace_bytes(const moe_problem* p, int training);

/*
 * Bytes of the activation buffer that moe_ffn_fwd fills for moe_bwd
 * (host): gate and up pre-activations of every token-slot (and, in fp32,
 * their gated hidden values; the bf16 backward recomputes those), and the
 * shared expert's pre-activations and hidden values; all in dtype.
 */
size_t moe_saved_bytes(const moe_problem* p);

/*
 * Stage "route" (kernel_gmm_gpu.json "pieces" suite, piece "route").
 * Reads x [tokens, d_model] (dtype) and w_router [d_model, experts] (fp32).
 * Writes r->topk_idx and r->topk_w only.
 * Logits are fp32 and evaluated in one fixed order, a sequential fused
 * multiply-add chain over j = 0..d_model-1 starting from +0.0, so that the
 * expert choice is reproducible exactly off the GPU. Ranking is on the
 * logits (logit descending, expert index ascending); the weights are
 * exp(l_i - l_0) / sum_j exp(l_j - l_0) over the kept experts, in fp32.
 */
int moe_route(const moe_problem* p, const void* x, const float* w_router, moe_routing* r,
              void* stream);

/*
 * Stage "sort_permute" (kernel_gmm_gpu.json "pieces" suite, piece
 * "sort_permute"; "block_m" of the config blocks).
 * Reads r->topk_idx. Writes r->expert_offsets, r->perm, r->inv_perm,
 * r->tiles and r->num_tiles: a stable counting sort of the flat slots by
 * expert (within an expert, slots keep ascending flat order, hence
 * ascending token order) and the tile list: for each expert in ascending
 * order, its rows cut into pieces of block_m rows, the last one partial.
 * Empty experts have no tile. With capacity > 0 an expert's sorted rows
 * past its first `capacity` are dropped: no tile covers them, and their
 * slots get inv_perm -1 (perm and expert_offsets still list every slot).
 * workspace: >= moe_workspace_bytes(p, 0).
 */
int moe_permute(const moe_problem* p, moe_routing* r, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * moe_permute without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, results and errors as moe_permute,
 * except that its scratch (the per-block expert counts) lives in a fixed
 * 1 MiB device array that libmoe holds on each GPU it runs on until the
 * process ends: experts * ceil(tokens * top_k / 4096) * 4 bytes must fit
 * in it (up to 16,777,216 token-slots at 64 experts), else
 * MOE_ERR_TOO_LARGE and nothing is enqueued. It allocates nothing (the
 * array's device address is looked up once per device, on the first call
 * there). Every call on one GPU uses that GPU's one array: calls that can
 * overlap on one GPU (different streams, or several host threads) race and
 * must be ordered by the caller. The array needs no clearing between calls.
 */
int moe_permute_static(const moe_problem* p, moe_routing* r, void* stream);

/*
 * Stage "experts_grouped_swiglu" (kernel_gmm_gpu.json "pieces" suite):
 * the grouped gated FFN over the expert-sorted token-slots, plus the
 * shared expert.
 *   y_sorted [S, d_model] (dtype): row j = FFN_e(x[perm[j] / top_k]) for the
 *     expert e owning sorted row j, unweighted.
 *   shared_out [tokens, d_model] (dtype): FFN_shared(x[t]); required iff
 *     d_shared > 0, else ignored.
 *   saved: NULL for inference, or moe_saved_bytes(p) bytes that moe_bwd
 *     reads (gate/up pre-activations and gated hidden values).
 * Reads x, the weights and r->{perm, tiles, num_tiles}.
 * workspace: >= moe_workspace_bytes(p, saved != NULL).
 */
int moe_ffn_fwd(const moe_problem* p, const void* x, const moe_weights* w, const moe_routing* r,
                void* y_sorted, void* shared_out, void* saved, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * Stage "unpermute_combine" (kernel_gmm_gpu.json "pieces" suite):
 *   out[t] = sum_i topk_w[t,i] * y_sorted[inv_perm[t*top_k + i]] + shared_out[t]
 * a gather-sum in fp32 (one writer per output row, no atomics), stored in
 * dtype. shared_out may be NULL (no shared term). Slots with inv_perm -1
 * (dropped by capacity) are left out of the sum.
 */
int moe_combine(const moe_problem* p, const void* y_sorted, const moe_routing* r,
                const void* shared_out, void* out, void* stream);

/*
 * Dispatch variants of the forward (kernel_gmm_gpu.json, "layer" suite
 * records, field "dispatch"; the pages name the variants and time them but
 * do not define them). All give the same out, y_sorted and saved buffers,
 * bit for bit: they differ in where token rows are gathered and where the
 * combine runs, not in any arithmetic.
 *   GATHER     the gate/up GEMM reads token rows through perm (moe_ffn_fwd,
 *              then moe_combine).
 *   SORTED     token rows are first copied into expert order (x_sorted
 *              [S, d_model] in the workspace) and the gate/up GEMM reads
 *              that copy row by row.
 *   FUSED_GSUM the gather-sum combine runs in the epilogue of the shared
 *              expert's down GEMM, whose rows are tokens: each output row is
 *              written once, and the shared output is never stored. Needs
 *              d_shared > 0 and top_k <= 8; otherwise it runs as GATHER.
 * The pages' fourth variant, "fused" (a scatter-add from the expert GEMM
 * into out), needs floating-point atomics and is not offered.
 */
typedef enum {
  MOE_DISPATCH_GATHER = 0,
  MOE_DISPATCH_SORTED = 1,
  MOE_DISPATCH_FUSED_GSUM = 2
} moe_dispatch;

/*
 * Workspace bytes (host) of moe_forward for a dispatch variant, with
 * training = 1 when saved activations are written. 0 for an invalid
 * problem or dispatch.
 */
size_t moe_forward_workspace_bytes(const moe_problem* p, int dispatch, int training);

/*
 * The whole forward in one call: "route", "sort_permute",
 * "experts_grouped_swiglu" and "unpermute_combine" (kernel_gmm_gpu.json
 * "pieces" suite), enqueued in that order on `stream`, with the dispatch
 * variant above. Writes every array of r (as moe_route and moe_permute
 * do), y_sorted [S, d_model], out [tokens, d_model] and, when saved is not
 * NULL, the moe_saved_bytes(p) activations moe_bwd reads. The shared
 * expert's output lives in the workspace (or nowhere, FUSED_GSUM).
 * workspace: >= moe_forward_workspace_bytes(p, dispatch, saved != NULL).
 * MOE_ERR_INVALID for an unknown dispatch value.
 */
int moe_forward(const moe_problem* p, int dispatch, const void* x, const moe_weights* w,
                moe_routing* r, void* y_sorted, void* saved, void* out, void* workspace,
                size_t workspace_bytes, void* stream, void* side_stream);

/*
 * Train-step backward (gpu_moe_h100.json header: value and gradient with
 * respect to the parameters and the input) of L = sum(out * grad_out),
 * with the top-k selection held fixed and the gradient reaching w_router
 * through the renormalised weights:
 *   dy = w * G, dw = <G, y>, dl = w (dw - sum w dw) on the kept experts,
 *   and the chain rule through both expert projections and SiLU.
 * Reads x, the weights, the routing state, saved and (fp32 only) y_sorted
 * from the forward, and grad_out [tokens, d_model] (dtype); in bf16 dw is
 * evaluated as <G W_down^T, H>, which equals <G, y>, so y_sorted is not
 * read and may be NULL. Writes grad_x
 * [tokens, d_model] (dtype) and every array of g (fp32; the shared ones
 * only when d_shared > 0). workspace: >= moe_workspace_bytes(p, 1).
 * saved must be the moe_saved_bytes(p) buffer moe_ffn_fwd filled.
 * Needs d_hidden and d_shared to be multiples of 128 (else
 * MOE_ERR_UNSUPPORTED). With tokens == 0 the weight gradients are zeroed
 * and nothing else is touched.
 */
int moe_bwd(const moe_problem* p, const void* x, const moe_weights* w, const moe_routing* r,
            const void* y_sorted, const void* saved, const void* grad_out, void* grad_x,
            const moe_grads* g, void* workspace, size_t workspace_bytes, void* stream,
            void* side_stream);

/*
 * Kernel timer (host). moe_trace_enable(1) clears the record and starts
 * bracketing every libmoe kernel launch with two hipEvents on its stream;
 * moe_trace_enable(0) stops and clears. Timing adds no device work besides
 * the event records. While it is on, moe_forward and moe_bwd ignore
 * side_stream and run everything on `stream` (the same kernels, in issue
 * order), so every recorded duration is that of a kernel running alone.
 * Returns MOE_OK.
 */
int moe_trace_enable(int on);

/*
 * Writes a JSON object {"<kernel>": {"ms": total, "count": launches}, ...}
 * for the launches recorded since moe_trace_enable(1) into buf (host
 * memory, buf_bytes long, NUL-terminated). Waits for the recorded events.
 * MOE_ERR_INVALID if buf is NULL or too small, MOE_ERR_HIP if an event
 * query fails.
 */
int moe_trace_summary(char* buf, size_t buf_bytes);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
