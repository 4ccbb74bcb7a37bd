/*
 * vla_expert.h — C ABI of the MI355X (gfx950) flow-matching action-expert
 * denoise loop.
 *
 * The operation ("LingBot-VLA on Thor (sm_110)", §1 Architecture / shapes and
 * §6 Notes; "LingBot-VLA v2 Examples", Configuration / CUDA Graph): a noisy
 * action chunk x (horizon T, action dim A) is integrated from t_0 to t_N by
 * explicit Euler steps, x <- x + (t_{k+1} - t_k) * v(x, t_k), where the
 * velocity v is a transformer of n_layers expert blocks. Each block applies a
 * timestep-conditioned AdaRMSNorm, a QKV projection with rotate-half RoPE,
 * grouped-query attention over the request's cached per-layer prefix K/V plus
 * the chunk's own K/V (no mask), an output projection with a gated residual,
 * a second AdaRMSNorm and a SwiGLU MLP with a gated residual. The prefix K/V
 * is built before the loop and is an input here. Exact conventions:
 *
 *   e   = [sin(time_scale*t*w_j), cos(time_scale*t*w_j)], w_j = 10000^(-j/(E/2))
 *   c   = SiLU(t2_w SiLU(t1_w e + t1_b) + t2_b)
 *   h   = x in_w^T + in_b
 *   per layer: [a1,b1,g1,a2,b2,g2] = mod_w c + mod_b   (six H-chunks)
 *     y = RMSNorm(h)(1+a1)+b1;  q,k,v = y wq^T, y wk^T, y wv^T
 *     q,k rotated (pair m with m+d_h/2, angle (P+i) theta^(-2m/d_h))
 *     o_j = softmax(q_j [Kp;k]^T / sqrt(d_h)) [Vp;v], KV head j/(n_q/n_kv)
 *     h += g1 * (o wo^T);  y = RMSNorm(h)(1+a2)+b2
 *     h += g2 * ((SiLU(y wg^T) * (y wu^T)) wd^T)
 *   [af,bf] = modf_w c + modf_b;  v = (RMSNorm(h)(1+af)+bf) out_w^T + out_b
 *   RMSNorm(h) = h / sqrt(mean(h^2) + rms_eps), no learned weight.
 *
 * Precision: weights bf16 (or E4M3FN block linears with per-row fp32 scales),
 * GEMM/attention inputs bf16, every accumulation fp32, the residual stream
 * and the Euler state fp32.
 *
 * Threading: one context is used by one host thread at a time; its calls are
 * ordered on its stream. Errors: functions return a negative VLA_ERR_* code
 * (or NULL) and set a thread-local message readable with vla_last_error().
 * Nothing falls back silently to another dtype, shape or path.
 */
#ifndef VLA_EXPERT_H
#define VLA_EXPERT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Block-linear weight encodings. */
#define VLA_BF16 0
#define VLA_FP8_E4M3 1 /* OCP E4M3FN codes, one fp32 scale per output row */
/* E4M3 as above for wq, wk, wv, wo, wd; OCP MXFP4 for wg and wu (the expert's
 * "FP8 + FP4 gate_up" of "LingBot-VLA on Thor (sm_110)", section 1, in the
 * FP4 format gfx950 takes natively). batch * horizon <= 64 only. */
#define VLA_FP8_E4M3_MXFP4_GU 2

/* Return codes. */
#define VLA_OK 0
#define VLA_ERR_ARG (-1)   /* null / misaligned pointer, bad n_steps or option */
#define VLA_ERR_SHAPE (-2) /* dims the library does not support */
#define VLA_ERR_OOM (-3)   /* device allocation failed */
#define VLA_ERR_HIP (-4)   /* a HIP runtime call failed */

/* Options for vla_set_option. */
#define VLA_OPT_USE_GRAPH 1 /* 1 (default): replay a captured hipGraph per n_steps; 0: launch kernels eagerly */
#define VLA_OPT_PERSISTENT 2 /* 1: for shapes it supports (batch*horizon <= 64, 8 | n_q_heads, ...),
                                 run the whole loop as one persistent kernel (needs every CU: other work on the GPU
                                 makes its bounded waits expire and the output NaN); 0 (default): kernel-per-stage path */
/* Query for vla_get_option: 1 when the next vla_denoise call uses the persistent kernel. */
#define VLA_OPT_PERSISTENT_ACTIVE 3
/* Query for vla_get_option: waits for the ctx stream, then gives the outcome of the last persistent
 * call: 0 completed, 1 an XCD-local wait expired, 2 a cross-XCD wait expired, 3 the workgroups were
 * not spread 32 per XCD. After 1-3 the call's output holds NaN. */
#define VLA_OPT_PERSISTENT_STATUS 4
/* Tile shape of the tiled GEMM (used where batch*horizon > 64): 0 (default) picks one per linear from
 * a cost model; 1, 2, 3, 4 force 256x256, 128x128, 128x64, 256x128 tiles where they divide the output width, also
 * for batch*horizon <= 64 (in place of the weight-streaming kernel). For testing and tuning; setting it
 * waits for the ctx stream and drops captured graphs. */
#define VLA_OPT_GEMM_TILE 5
/* With batch*horizon <= 64, workgroups appended to the attention and norm kernels (on CUs those leave
 * idle) load the next weight-streaming GEMMs' weights into the L2 of the XCD that will read them. Bits:
 * 1 the attention prefetches O, 2 the attention prefetches gate_up, 4 the norm before a layer prefetches
 * its QKV, 8 the norm before gate_up prefetches down; 0 off. Default 4 for bf16 weights whose largest
 * block linear fits the L2 of all XCDs together, else 0 (measured fastest with the non-temporal weight
 * reads). For measurement; setting it waits for the ctx stream and drops captured graphs. */
#define VLA_OPT_L2_PREFETCH 6
/* Large batches: n = 2..4 runs the requests as n parts at once (request ranges [B i / n, B (i+1) / n)),
 * each part a child context (the same weights, its own buffers, graph and stream) forked from and joined
 * back to the ctx stream with events, so that one part's kernel ramps and tails overlap another's; 0 runs
 * the batch as one. Parts of at most 64 rows are not made (the option then runs the batch as one). The
 * default uses two parts when each half has at least 1024 rows (batch * horizon / 2). A request's result
 * can differ from the unsplit run only by the order of fp32 sums in the modulation GEMM (whose row count
 * is steps * requests, so a part can take the weight-streaming kernel where the whole batch takes the
 * tiled one), i.e. within rounding. vla_get_option gives the number of parts in use (0: none). Setting
 * any option rebuilds the parts at the next call. */
#define VLA_OPT_SPLIT_BATCH 8
/* With batch*horizon <= 64, the weight-streaming GEMMs read bf16 / E4M3 weights with the non-temporal
 * hint (1, the default: measured faster on every batch-1 model) or plainly (0); MXFP4 gate_up weights are
 * read plainly. Results do not depend on it. Setting it waits for the ctx stream and drops captured
 * graphs; vla_get_option gives the setting in use. */
#define VLA_OPT_WEIGHT_NT 9

typedef struct vla_ctx vla_ctx;

/*
 * Sizes and conventions. Supported: head_dim in {64, 128}; hidden and
 * intermediate multiples of 64, hidden <= 2048; n_q_heads a multiple of n_kv_heads;
 * n_q_heads*head_dim a multiple of 64; 1 <= action_dim <= 128;
 * 1 <= horizon <= 256; prefix_len >= 0; batch >= 1; time_emb_dim a positive
 * multiple of 64; rms_eps > 0.
 */
typedef struct vla_dims {
    int32_t n_layers;
    int32_t hidden;        /* H */
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;      /* d_h */
    int32_t intermediate;  /* I, SwiGLU width */
    int32_t action_dim;    /* A */
    int32_t horizon;       /* T, chunk length */
    int32_t prefix_len;    /* P, cached prefix tokens per layer */
    int32_t batch;         /* B, independent requests per call */
    int32_t time_emb_dim;  /* E, sinusoidal embedding width (256) */
    float rope_theta;      /* 1e6 */
    float rms_eps;         /* 1e-6 */
    float time_scale;      /* 1000: the embedding's argument is time_scale * t */
    int32_t weight_dtype;  /* VLA_BF16, VLA_FP8_E4M3 or VLA_FP8_E4M3_MXFP4_GU (block linears only) */
} vla_dims;

/*
 * Weights, all DEVICE pointers, torch nn.Linear layout [out, in] row-major.
 * bf16 tensors hold bfloat16 bits; biases and scales are fp32. The per-layer
 * members are HOST arrays of n_layers device pointers.
 *
 *   in_w  [H, A] bf16      in_b  [H]     out_w [A, H] bf16   out_b [A]
 *   t1_w  [H, E] bf16      t1_b  [H]     t2_w  [H, H] bf16   t2_b  [H]
 *   mod_w[l] [6H, H] bf16  mod_b[l] [6H] modf_w [2H, H] bf16 modf_b [2H]
 *   wq[l] [n_q*d_h, H]   wk[l], wv[l] [n_kv*d_h, H]   wo[l] [H, n_q*d_h]
 *   wg[l], wu[l] [I, H]  wd[l] [H, I]     — bf16, or E4M3FN bytes when
 *   weight_dtype == VLA_FP8_E4M3, then sq..sd[l] hold one fp32 scale per
 *   output row (the dequantized weight is code * scale); NULL for bf16.
 *   With VLA_FP8_E4M3_MXFP4_GU, wg[l] and wu[l] hold OCP E2M1 codes two per
 *   byte (element 2j in the low nibble), [I, H/2] bytes, and sg[l], su[l]
 *   point to one E8M0 scale byte per 32 inputs, [I, H/32] bytes (value
 *   2^(e - 127)); the dequantized weight is E2M1 value * block scale.
 */
typedef struct vla_weights {
    const void* in_w;  const float* in_b;
    const void* out_w; const float* out_b;
    const void* t1_w;  const float* t1_b;
    const void* t2_w;  const float* t2_b;
    const void* const* mod_w; const float* const* mod_b;
    const void* modf_w; const float* modf_b;
    const void* const* wq; const void* const* wk; const void* const* wv;
    const void* const* wo; const void* const* wg; const void* const* wu;
    const void* const* wd;
    const float* const* sq; const float* const* sk; const float* const* sv;
    const float* const* so; const float* const* sg; const float* const* su;
    const float* const* sd;
} vla_weights;

/*
 * Create an expert. Validates dims, repacks and COPIES the weights into
 * library-owned device memory (the caller may free its copies on return),
 * allocates every working buffer for dims->batch, and synchronizes before
 * returning. Runs on the current HIP device. Returns NULL on error.
 */
vla_ctx* vla_expert_create(const vla_weights* weights, const vla_dims* dims);

/*
 * Run the n_steps-step Euler denoise loop for all dims.batch requests.
 * All pointers are DEVICE pointers; prefix_k and prefix_v 16-byte aligned,
 * noise, t_schedule and out_actions 4-byte aligned (VLA_ERR_ARG otherwise):
 *   prefix_k, prefix_v  [B, L, P, n_kv, d_h] bf16 — each request's cached
 *                       prefix keys/values per layer, used as given;
 *   noise               [B, T, A] fp32 — the state x at t_0;
 *   t_schedule          [B, n_steps+1] fp32 — t_{b,0..N}; dt_k = t_{k+1}-t_k;
 *   out_actions         [B, T, A] fp32 — x at t_N; may alias noise.
 * Inputs are borrowed until the ctx stream passes this call. Asynchronous on
 * the ctx stream. The first call with a new n_steps captures a graph.
 * Returns VLA_OK or a VLA_ERR_* code (VLA_ERR_ARG for n_steps outside
 * [1, 100000]); argument errors are found before anything is enqueued.
 */
int vla_denoise(vla_ctx* ctx, const void* prefix_k, const void* prefix_v, const float* noise,
                const float* t_schedule, int n_steps, float* out_actions);

/* vla_denoise with a prefix length per request, for prefixes padded to a fixed
 * P (FlashRT flash_rt/api.py page: fixed-shape mode with a device-side valid
 * length; LingBot-VLA v2 Examples: language padded to a fixed length).
 * prefix_valid: device pointer to int32 [B], 4-byte aligned. Request b uses
 * prefix tokens [0, prefix_valid[b]) of its P-token prefix (values are
 * clamped to [0, P]); tokens past that are padding no query attends to, and
 * the chunk's RoPE positions are prefix_valid[b] .. prefix_valid[b] + T - 1.
 * So request b's result equals vla_denoise on a prefix of exactly
 * prefix_valid[b] tokens. The values are read when the call runs on the GPU:
 * one captured graph serves calls with different values. NULL: every request
 * uses all P tokens (vla_denoise). Same ownership and errors as vla_denoise. */
int vla_denoise_varlen(vla_ctx* ctx, const void* prefix_k, const void* prefix_v, const int32_t* prefix_valid,
                       const float* noise, const float* t_schedule, int n_steps, float* out_actions);

/* For callers that cannot allocate device memory during a call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The same loop as vla_denoise (same arguments, ownership and errors, same
 * kernels, so the same bits), launched kernel by kernel on the ctx stream
 * (no graph of its own, none instantiated), calling no allocator: the call's
 * scratch (the modulation table of every step, the time-MLP intermediates,
 * the split-K partials) lives in one library-wide static device array of
 * VLA_STATIC_SCRATCH_BYTES per device, held until the process ends. Calls
 * needing more than that (roughly n_steps * batch * (6 n_layers + 2) * hidden
 * * 4 bytes plus the partials) fail with VLA_ERR_SHAPE before anything is
 * enqueued; e.g. the 36-layer hidden-1024 expert fits up to about 70 steps
 * at batch 1. Every call on a device shares that device's array: calls
 * that overlap on one device (other streams, other contexts) race and must
 * be serialized by the caller. The persistent path option is ignored. */
#define VLA_STATIC_SCRATCH_BYTES 67108864 /* 64 MiB */
int vla_denoise_static(vla_ctx* ctx, const void* prefix_k, const void* prefix_v, const float* noise,
                       const float* t_schedule, int n_steps, float* out_actions);

/* Use `stream` (a hipStream_t) for every later call on ctx. NULL (also the
 * state after vla_expert_create) selects the legacy default stream. Graphs
 * are captured once on a library-created stream and replayed on this one.
 * A context's working buffers serve all its calls, so when the stream
 * changes, the new stream first waits (an event, no host wait) for the work
 * already enqueued on the previous one. Returns VLA_OK, VLA_ERR_ARG or
 * VLA_ERR_HIP. */
int vla_set_stream(vla_ctx* ctx, void* stream);

/* Set an option (VLA_OPT_*). Returns VLA_OK or VLA_ERR_ARG. */
int vla_set_option(vla_ctx* ctx, int option, int value);

/* Read an option (VLA_OPT_*) into *value. Returns VLA_OK or VLA_ERR_ARG. */
int vla_get_option(const vla_ctx* ctx, int option, int* value);

/* Synchronize, free everything owned by ctx. NULL-safe. */
void vla_expert_destroy(vla_ctx* ctx);

/* Message of the last failing call on this host thread ("" if none). */
const char* vla_last_error(void);

/* Bytes of device memory owned by ctx (weights + buffers). */
int64_t vla_device_bytes(const vla_ctx* ctx);

/* ---------------------------------------------------------------------------
 * Single-stage entry points for parity tests (not part of the product path).
 * They run one stage with the context's kernels on the ctx stream and
 * synchronize before returning.
 * ------------------------------------------------------------------------- */

/* Modulation table for n_steps steps of t_schedule [B, n_steps+1]:
 * mod_out [n_steps, B, 6L+2, H] fp32, chunk order (per layer) a1,b1,g1,a2,b2,g2
 * then af,bf. */
int vla_test_modulation(vla_ctx* ctx, const float* t_schedule, int n_steps, float* mod_out);

/* One expert layer `layer` applied to h_in [B*T, H] fp32 with the modulation of
 * step `step` (computed from t_schedule [B, n_steps+1]); writes h_out
 * [B*T, H] fp32. prefix_k/v as in vla_denoise. */
int vla_test_layer(vla_ctx* ctx, const void* prefix_k, const void* prefix_v, const float* t_schedule,
                   int n_steps, int step, int layer, const float* h_in, float* h_out);

/* Grouped-query attention of layer `layer` alone: q [B, n_q, T, d_h],
 * k_new/v_new [B, n_kv, T, d_h] bf16 (already rotated), prefix as above;
 * o_out [B*T, n_q*d_h] bf16. */
int vla_test_attention(vla_ctx* ctx, const void* prefix_k, const void* prefix_v, int layer,
                       const void* q, const void* k_new, const void* v_new, void* o_out);

/* Kernel timing for roofline figures: runs `iters` expert layers exactly as
 * in the loop (cycling through the layers, so weights stream from HBM; step 0
 * of the last vla_denoise call's modulation table) on the ctx stream, and
 * times the one launch per layer of the chosen kernel family with HIP events
 * recorded at that kernel's own start and end (hipExtLaunchKernelGGL). Writes
 * the mean launch duration in microseconds to *us_per_launch and the
 * algorithmic bytes and flops of one launch to *bytes_per_launch and
 * *flops_per_launch. Overwrites the working buffers (call vla_denoise first).
 * Synchronizes. */
#define VLA_KERNEL_QKV 0
#define VLA_KERNEL_ATTN 1
#define VLA_KERNEL_O 2
#define VLA_KERNEL_GATE_UP 3
#define VLA_KERNEL_DOWN 4
int vla_profile_kernel(vla_ctx* ctx, int kernel, int iters, double* us_per_launch, double* bytes_per_launch,
                       double* flops_per_launch);

#ifdef __cplusplus
}
#endif

#endif /* VLA_EXPERT_H */
