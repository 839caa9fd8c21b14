/*
 * flint_moe.h -- C ABI of libflint_moe.so, the routed-expert MoE feed-forward
 * layer of Flint on AMD Instinct MI355X (gfx950).
 *
 * The layer (what the pages define): each MoE layer holds 256 routed experts,
 * a router picks 6 of them per token, and one shared expert is always applied
 * on top  [evermx.com, "Recursive Flint: Open-Weight MoE Coding Model, 2.5B
 * Active", Feature Overview, paragraph "Sparse architecture"; swarmz.net,
 * "Recursive Flint: 40B Open Model, 2.5B Active", section "The architecture,
 * in plain terms" and the FAQ entry on active parameters; futurpulse.com,
 * "Flint model: local coding with fewer active parameters", section "How
 * does Flint use 39.8B parameters efficiently?"].  Decoding a token reads only
 * the routed group and the shared expert, so it is bound by weight bandwidth
 * [kongchang.com, "Recursive Open-Sources Flint: A 40B MoE Local Coding Model
 * with 2.5B Active Parameters", section "125+ tokens/s: The Practical
 * Threshold for Local Inference"].  4-bit weights are NVFP4 [evermx.com page,
 * paragraph "Quantization"].
 *
 * Readings taken where the pages are silent (the same ones the CPU oracle
 * uses): experts are SwiGLU without biases, h = SiLU(G x) * (U x), y = D h;
 * router logits l = Wr x (+ b) in fp32; the k largest logits are chosen, ties
 * going to the lower expert index; the chosen weights are the softmax of the
 * chosen logits (= the full softmax renormalised over the chosen k); the
 * shared expert enters with weight 1:
 *     out[t] = y_shared(x_t) + sum_j w[t][j] * y_{idx[t][j]}(x_t)   (+ residual[t])
 *
 * Conventions
 *  - Every pointer argument that names a tensor is DEVICE memory owned by the
 *    caller, row-major, 16-byte aligned.  The library never frees it.
 *  - Calls are asynchronous on the caller's hipStream_t: no host sync, no
 *    device-to-host read, no allocation inside flint_moe_forward.
 *  - Every entry point returns a flint_status; none aborts or throws.  A fault
 *    inside a kernel surfaces at the caller's next synchronisation.
 *  - A handle owns only its workspace (allocated once in flint_moe_create) and
 *    serves any number of layers; one handle must not run two forwards at the
 *    same time (they share the workspace).  Separate handles may.
 */
#ifndef FLINT_MOE_H
#define FLINT_MOE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct flint_moe* flint_moe_t;

typedef enum {
    FLINT_OK = 0,
    FLINT_ERR_INVALID_ARG = 1,  /* bad pointer, size, alignment or config; no HIP call made */
    FLINT_ERR_UNSUPPORTED = 2,  /* valid but not implemented (shape or dtype combination) */
    FLINT_ERR_OUT_OF_MEMORY = 3,/* workspace allocation failed */
    FLINT_ERR_NO_DEVICE = 4,    /* no HIP device, or the current device is not gfx950 */
    FLINT_ERR_HIP = 5           /* a HIP runtime call or kernel launch failed */
} flint_status;

typedef enum {
    FLINT_F32 = 0,   /* IEEE binary32 */
    FLINT_BF16 = 1,  /* bfloat16 */
    FLINT_NVFP4 = 2  /* E2M1 codes + E4M3 per-16 block scales + fp32 tensor scale */
} flint_dtype;

/* flags of flint_moe_config */
#define FLINT_FORCE_DECODE_PATH  0x1u  /* always use the expert-GEMV path */
#define FLINT_FORCE_PREFILL_PATH 0x2u  /* always use the grouped-MFMA path (bf16 activations;
                                          bf16 or NVFP4 weights) */
/* Debug: at create and before every forward, fill the floating-point part of
 * the workspace (logits, weights, partial sums, h, y) with NaN bit patterns,
 * so that a kernel reading a value that no kernel of the same forward wrote
 * makes the output NaN.  The hand-off tickets and the integer routing tables
 * keep their contents.  Adds one fill launch per forward; for tests only. */
#define FLINT_DEBUG_POISON_WORKSPACE 0x4u
/* Run small decode batches as separate route, gate/up and down launches
 * instead of the single-launch decode kernel (for comparison and tests).
 * Without it the single launch takes bf16 activations with bf16 weights up to
 * 5 tokens and with NVFP4 weights up to 4 (where it measured faster); the
 * environment variable FLINT_MOE_FUSED_MAX_T, read at create time, sets that
 * limit for both (0 turns the single launch off, the kernel's own limit is 8). */
#define FLINT_UNFUSED_DECODE 0x8u

typedef struct {
    uint32_t struct_size;   /* = sizeof(flint_moe_config) */
    int32_t d_model;        /* d: hidden size; multiple of 64, <= 16384 */
    int32_t n_experts;      /* E: routed experts; 1..256 */
    int32_t top_k;          /* k: experts chosen per token; 1..8 and <= E */
    int32_t d_ff;           /* f: routed expert width; multiple of 32 */
    int32_t d_ff_shared;    /* f_s: shared expert width; 0 (no shared expert) or a multiple of 32 */
    int32_t act_dtype;      /* flint_dtype of hidden/out: FLINT_F32 or FLINT_BF16 */
    int32_t weight_dtype;   /* flint_dtype of expert and shared weights */
    int32_t max_tokens;     /* largest T a forward may pass; sizes the workspace; 1..65536 */
    uint32_t flags;         /* FLINT_FORCE_*, FLINT_DEBUG_POISON_WORKSPACE, FLINT_UNFUSED_DECODE */
} flint_moe_config;

/*
 * One set of expert weights (the routed set has n = E experts, the shared set
 * n = 1).  Layouts, K contiguous in every matrix:
 *   F32 / BF16:  gate_up [n][2f][d]  rows 0..f-1 = G (gate), rows f..2f-1 = U (up)
 *                down    [n][d][f]
 *   NVFP4:       gate_up [n][2f][d/2] bytes, element k of a row in byte k/2,
 *                         even k in the low nibble (E2M1 codes)
 *                down    [n][d][f/2] bytes, same packing
 *                gate_up_scales [n][2f][d/16], down_scales [n][d][f/16]: E4M3
 *                         codes, one per 16 consecutive elements of a row
 *                tensor_scales  [n][3] fp32 = {gate, up, down}
 *   A dequantised NVFP4 weight is E2M1(code) * E4M3(block scale) * tensor scale.
 * Scale pointers must be NULL unless weight_dtype is FLINT_NVFP4.
 */
typedef struct {
    const void* gate_up;
    const void* down;
    const uint8_t* gate_up_scales;
    const uint8_t* down_scales;
    const float* tensor_scales;
} flint_expert_weights;

/* Validate cfg, check for a gfx950 device (the current HIP device), and
 * allocate the workspace for cfg->max_tokens tokens.  On success *out is a
 * new handle.  Argument errors are reported before any HIP call. */
flint_status flint_moe_create(const flint_moe_config* cfg, flint_moe_t* out);

/*
 * The layer on T tokens, enqueued on `stream`.
 *   hidden      [T][d] act_dtype
 *   router_w    [E][d] fp32
 *   router_bias [E] fp32, or NULL for none (added to the logits before both
 *               selection and softmax)
 *   experts     routed weights (n = E);  shared: shared-expert weights (n = 1),
 *               NULL when d_ff_shared == 0
 *   residual    NULL, or [T][d] fp32 added to the result; then `out` is fp32
 *               [T][d] (it may alias `residual`), otherwise `out` is
 *               [T][d] act_dtype
 *   out         must not overlap hidden
 * T == 0 is a no-op (pointers are not examined).  T > max_tokens, NULL
 * tensors, misalignment, scale
 * pointers that do not match weight_dtype, or aliasing give
 * FLINT_ERR_INVALID_ARG before anything is enqueued.
 */
flint_status flint_moe_forward(flint_moe_t h, int32_t T, const void* hidden,
                               const float* router_w, const float* router_bias,
                               const flint_expert_weights* experts,
                               const flint_expert_weights* shared, const float* residual,
                               void* out, hipStream_t stream);

/*
 * One step of a stack of layers with pre-norm residual blocks:
 *   out[t]      = residual[t] + MoE(hidden)[t]                    (fp32, as flint_moe_forward)
 *   norm_out[t] = bf16(out[t] / sqrt(mean(out[t]^2) + eps))       (unit gain, fp32 arithmetic)
 * norm_out is the next layer's input, bit for bit what flint_rmsnorm_forward
 * gives from out.  The model has 47 MoE layers [evermx.com, "Recursive
 * Flint: Open-Weight MoE Coding Model, 2.5B Active", Feature Overview,
 * "Sparse architecture"]; the residual form with a unit-gain RMSNorm before
 * each layer is the reading taken for running them in sequence.  Where the
 * path sums the layer output in a launch of its own, that launch also
 * normalises it, which saves a launch per layer.
 *   residual: [T][d] fp32, required (may equal out); out: [T][d] fp32;
 *   norm_out: [T][d] bf16 (device, 16-byte aligned, disjoint from hidden,
 *   residual and out); eps in [0, 1].
 * Errors as flint_moe_forward; FLINT_ERR_INVALID_ARG for a NULL residual or
 * norm_out, an eps outside [0, 1] or an overlapping norm_out.
 */
flint_status flint_moe_forward_prenorm(flint_moe_t h, int32_t T, const void* hidden,
                                       const float* router_w, const float* router_bias,
                                       const flint_expert_weights* experts,
                                       const flint_expert_weights* shared, const float* residual,
                                       float* out, float eps, void* norm_out, hipStream_t stream);

/*
 * The same forward without a handle and without allocating, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Arguments as flint_moe_forward,
 * with the configuration passed directly (cfg->max_tokens is ignored; the
 * layout is sized for exactly T tokens).
 *   Scratch: the workspace lives in one static 16 MiB device array per GPU
 *   (loaded with the library, held until the process ends); a call whose
 *   workspace for T tokens would be larger returns FLINT_ERR_INVALID_ARG
 *   (at d = 2048, E = 256, k = 6, f = 512 every T up to 128 fits).
 *   No hipMalloc, hipFree or other allocation; the first call on a device
 *   looks up the array's device address (hipGetSymbolAddress) and checks the
 *   device once.  Each call first clears its hand-off tickets with a small
 *   fill kernel (one extra launch), since the array keeps whatever the
 *   previous call left.
 *   Every call on a GPU shares that GPU's array: calls that overlap on one
 *   GPU (two streams, two threads) race and must be serialised by the caller.
 * Errors as flint_moe_forward, plus FLINT_ERR_NO_DEVICE on a non-gfx950
 * device.  FLINT_FORCE_* and FLINT_DEBUG_POISON_WORKSPACE flags apply.
 */
flint_status flint_moe_forward_noalloc(const flint_moe_config* cfg, int32_t T, const void* hidden,
                                       const float* router_w, const float* router_bias,
                                       const flint_expert_weights* experts,
                                       const flint_expert_weights* shared, const float* residual,
                                       void* out, hipStream_t stream);

/*
 * Device-to-device copies of the routing of the handle's last forward
 * (enqueued on `stream`, after that forward).  Any output may be NULL.
 *   idx         [T][k] int32  chosen experts, slot order = descending logit
 *   weights     [T][k] fp32   their combine weights
 *   sorted_pair [k*T] int32   pair ids p = t*k + j ordered by (expert, p)
 *   counts      [E] int32     tokens routed to each expert
 *   logits      [T][E] fp32   router logits (bias included)
 * *T_out receives that forward's T (host memory; may be NULL).
 */
flint_status flint_moe_get_routing(flint_moe_t h, int32_t* idx, float* weights,
                                   int32_t* sorted_pair, int32_t* counts, float* logits,
                                   int32_t* T_out, hipStream_t stream);

/* Debug: the fault word of the single-launch decode kernel, copied
 * asynchronously on `stream` to the device int32 at fault_out.  0 means every
 * grid-barrier wait of every single-launch forward on this handle ended
 * normally; 1 means some wait gave up after its poll limit (the kernel still
 * ended, but that forward's output is not to be trusted).  The word is sticky
 * for the handle's lifetime.  FLINT_ERR_INVALID_ARG for a NULL handle or
 * fault_out. */
flint_status flint_moe_get_fault(flint_moe_t h, int32_t* fault_out, hipStream_t stream);

/* Kernel timing hook for measurement.  After flint_moe_profile_begin(h, id,
 * n), the next n launches of kernel `id` (see FLINT_KERNEL_*) inside
 * flint_moe_forward are bracketed by HIP events on the forward's stream.
 * flint_moe_profile_end synchronises those events and writes up to `cap`
 * per-launch durations in milliseconds to host array ms_out, the count to
 * *n_out, and stops recording. */
#define FLINT_KERNEL_ROUTE        0  /* router + top-k (+ sort on the decode path) */
#define FLINT_KERNEL_SORT         1  /* prefill counting sort */
#define FLINT_KERNEL_EXPERT_UP    2  /* gate/up + SwiGLU (decode GEMV or prefill MFMA) */
#define FLINT_KERNEL_EXPERT_DOWN  3  /* down projection (with the combine folded in for small
                                        decode batches run as separate launches: bf16
                                        weights up to 8 tokens, NVFP4 up to 4; no combine
                                        launch is then recorded) */
#define FLINT_KERNEL_COMBINE      4  /* weighted unpermute + shared + residual */
#define FLINT_KERNEL_FUSED        5  /* single-launch decode (the whole layer) */
#define FLINT_KERNEL_FORWARD      6  /* a whole forward: before its first launch to after its last */
#define FLINT_KERNEL_COUNT        7
flint_status flint_moe_profile_begin(flint_moe_t h, int32_t kernel_id, int32_t n_launches);
flint_status flint_moe_profile_end(flint_moe_t h, float* ms_out, int32_t cap, int32_t* n_out);

/* Release the handle and its workspace (synchronises the device first). */
flint_status flint_moe_destroy(flint_moe_t h);

/* Static description of a status code. */
const char* flint_status_string(flint_status s);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* flint_last_error(void);

/* Pre-norm of the stacked-layer workload: out[t] = bf16(in[t] / sqrt(mean(in[t]^2) + eps))
 * with unit gain, fp32 arithmetic.  in [T][d] fp32, out [T][d] bf16 (device). */
flint_status flint_rmsnorm_forward(int32_t T, int32_t d, const float* in, float eps,
                                   void* out_bf16, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FLINT_MOE_H */
