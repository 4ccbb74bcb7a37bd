/*
 * vla_prefill.h — C ABI of the prefix K/V construction on MI355X (gfx950):
 * the backbone prefill that builds, once per request and before the denoise
 * loop, the per-layer prefix keys and values that vla_denoise attends to
 * ("LingBot-VLA on Thor (sm_110)", section 1: the Qwen2.5-VL prefix of 36
 * self-attention layers builds the cache; "LingBot-VLA v2 Examples", section
 * "Configuration / CUDA Graph": the 36-layer KV-cache construction runs per
 * request, outside the captured loop).
 *
 * The pages give no layer equations. Each layer is taken to be the plain
 * pre-norm decoder layer of that backbone family:
 *   y = RMSNorm(x) * n1;  q, k, v = y wq^T, y wk^T, y wv^T   (no biases)
 *   q, k rotated: pair m with m + d_h/2 at angle t * theta^(-2m/d_h), token t
 *   o_j = softmax(q_j k^T / sqrt(d_h) + causal mask) v, KV head j/(n_q/n_kv);
 *         query token t sees tokens 0..t
 *   x += o wo^T;  y = RMSNorm(x) * n2;  x += (SiLU(y wg^T) * (y wu^T)) wd^T
 *   RMSNorm(x) = x / sqrt(mean(x^2) + rms_eps)
 * and layer l's cache is its (rotated) k and v. The input x of layer 0 is the
 * prefix token embeddings (vision patches and text, already embedded).
 * Since attention is causal, the cache of tokens [0, n) does not depend on
 * later tokens: a prefix padded at its end gives exact caches for its valid
 * tokens (vla_denoise_varlen then ignores the rest).
 *
 * Precision: weights and GEMM/attention inputs bf16 (or, with
 * VLA_FP8_E4M3, E4M3 weights and per-token E4M3 linear inputs), every
 * accumulation fp32, the residual stream fp32, keys/values out bf16.
 * Threading and errors as in vla_expert.h (shared VLA_ERR_* codes and
 * vla_last_error()).
 */
#ifndef VLA_PREFILL_H
#define VLA_PREFILL_H

#include <stdint.h>

#include "vla_expert.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct vla_prefill_ctx vla_prefill_ctx;

/*
 * Sizes. Supported: head_dim in {64, 128}; hidden a multiple of 64 and at
 * most 4096; intermediate a multiple of 64; n_q_heads a multiple of
 * n_kv_heads; 1 <= prefix_len <= 8192; batch >= 1 with batch * prefix_len
 * <= 2^24. n_layers, n_kv_heads and head_dim must equal the expert's for the
 * output to feed vla_denoise.
 */
typedef struct vla_backbone_dims {
    int32_t n_layers;
    int32_t hidden;        /* H */
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;      /* d_h */
    int32_t intermediate;  /* I (SwiGLU width) */
    int32_t prefix_len;    /* P tokens per request */
    int32_t batch;         /* B requests per call */
    float rope_theta;
    float rms_eps;
    int32_t weight_dtype;  /* VLA_BF16, or VLA_FP8_E4M3 (hidden, n_q_heads*head_dim and
                              intermediate multiples of 128) */
} vla_backbone_dims;

/*
 * Weights, all DEVICE pointers, one array entry per layer (n_layers each):
 *   norm1, norm2  [H] fp32 RMSNorm weights (4-byte aligned)
 *   wq [n_q*d_h, H], wk, wv [n_kv*d_h, H], wo [H, n_q*d_h],
 *   wg, wu [I, H], wd [H, I]   row-major (out, in), 8-byte aligned: bf16, or
 *                              for VLA_FP8_E4M3 OCP E4M3FN codes with
 *   sq, sk, sv, so, sg, su, sd  fp32 per-output-row scales (weight = code *
 *                              scale; unused and may be NULL for bf16).
 * The E4M3 tier also takes each linear's input per token in E4M3 (codes
 * RNE(x * 448 / max|x_row|), row scale max|x_row| / 448), as the expert's
 * batched E4M3 tier does; accumulation stays fp32.
 */
typedef struct vla_backbone_weights {
    const float* const* norm1;
    const float* const* norm2;
    const void* const* wq; const void* const* wk; const void* const* wv;
    const void* const* wo; const void* const* wg; const void* const* wu;
    const void* const* wd;
    const float* const* sq; const float* const* sk; const float* const* sv;
    const float* const* so; const float* const* sg; const float* const* su;
    const float* const* sd;
} vla_backbone_weights;

/*
 * Create a prefill context. Validates dims, repacks and COPIES the weights
 * into library-owned device memory (the caller may free its copies on
 * return), allocates every working buffer for dims->batch and synchronizes.
 * Runs on the current HIP device. Returns NULL on error (vla_last_error()).
 */
vla_prefill_ctx* vla_prefill_create(const vla_backbone_weights* weights, const vla_backbone_dims* dims);

/*
 * Build the prefix cache of all dims.batch requests. DEVICE pointers,
 * 16-byte aligned:
 *   embeddings          [B, P, H] bf16 — the prefix token embeddings;
 *   prefix_k, prefix_v  [B, L, P, n_kv, d_h] bf16 — written: each layer's
 *                       rotated keys and its values (the layout vla_denoise
 *                       takes). Must not overlap embeddings or each other.
 * Inputs are borrowed and outputs written asynchronously on the ctx stream;
 * the first call captures a graph that later calls replay. Returns VLA_OK or
 * a VLA_ERR_* code.
 */
int vla_prefill(vla_prefill_ctx* ctx, const void* embeddings, void* prefix_k, void* prefix_v);

/* Use `stream` (a hipStream_t) for later calls; NULL selects the legacy
 * default stream (the state after vla_prefill_create). When the stream
 * changes, the new stream first waits (an event, no host wait) for the work
 * already enqueued on the previous one, whose buffers later calls reuse.
 * Returns VLA_OK, VLA_ERR_ARG or VLA_ERR_HIP. */
int vla_prefill_set_stream(vla_prefill_ctx* ctx, void* stream);

/* VLA_OPT_USE_GRAPH (1 replay a captured graph, the default; 0 launch
 * eagerly) and VLA_OPT_GEMM_TILE (as for the expert; drops the graph).
 * Returns VLA_OK or VLA_ERR_ARG. */
int vla_prefill_set_option(vla_prefill_ctx* ctx, int option, int value);

/* Synchronize, free everything owned by ctx. NULL-safe. */
void vla_prefill_destroy(vla_prefill_ctx* ctx);

/* Bytes of device memory owned by ctx. */
int64_t vla_prefill_device_bytes(const vla_prefill_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* VLA_PREFILL_H */
