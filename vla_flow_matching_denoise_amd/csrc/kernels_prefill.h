// HIP kernels of the prefix K/V construction (the backbone prefill that runs
// before the denoise loop; "LingBot-VLA on Thor (sm_110)", section 1: the
// VLM prefix's 36 self-attention layers build the per-layer cache;
// "LingBot-VLA v2 Examples", section "Configuration / CUDA Graph": that build
// runs once per request, before the loop).
//
// Each layer is a pre-norm decoder layer: weighted RMSNorm, bias-free QKV
// with rotate-half RoPE at positions 0..P-1, causal GQA self-attention,
// O-projection + residual, weighted RMSNorm, SwiGLU + residual. The GEMMs,
// the QKV/RoPE and SwiGLU epilogues and the attention are the expert's
// kernels (tiled GEMM with row-major activations; attention with the CAUSAL
// mask); this file holds what only the prefill needs.
#pragma once

#include "kernels_layer.h"

// Pointers of the current prefill call (refreshed by one thread before each
// graph replay).
struct PrefillArgs {
    const uint16_t* emb;  // [B, P, H] bf16 token embeddings
    uint16_t* pk;         // [B, L, P, n_kv, d_h] bf16 keys out
    uint16_t* pv;         // values out, same layout
};

__global__ void set_prefill_args_kernel(PrefillArgs* a, const uint16_t* emb, uint16_t* pk, uint16_t* pv) {
    a->emb = emb;
    a->pk = pk;
    a->pv = pv;
}

// Weighted RMSNorm of one token row per workgroup (256 threads, H <= 4096,
// H % 4 == 0): y = bf16(h / sqrt(mean(h^2) + eps) * w). With `args` (the
// first layer) the row comes from the bf16 embeddings and is also written to
// the fp32 residual stream h. With S > 0 the S split-K partials ws[s][M][H]
// of the preceding residual GEMM are first added to h (and h written back).
// With y8 (the E4M3 tier) the output is instead per-token E4M3: codes
// RNE(y * 448 / max|y|) and the row scale max|y| / 448 (1 for a zero row).
__global__ __launch_bounds__(256) void rmsnorm_w_kernel(const PrefillArgs* args, float* __restrict__ h,
                                                        const float* __restrict__ ws, int S, int M,
                                                        const float* __restrict__ w, uint16_t* __restrict__ y,
                                                        int H, float eps, uint8_t* __restrict__ y8,
                                                        float* __restrict__ y8s) {
    __shared__ float red[4], red8[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    float* hr = h + (size_t)row * H;
    f32x4 v[4];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = (tid + 256 * j) * 4;
        if (c < H) {
            if (args) {
                const u32x2 e = *(const u32x2*)(args->emb + (size_t)row * H + c);
                v[j] = (f32x4){__uint_as_float(e[0] << 16), __uint_as_float(e[0] & 0xffff0000u),
                               __uint_as_float(e[1] << 16), __uint_as_float(e[1] & 0xffff0000u)};
                *(f32x4*)(hr + c) = v[j];
            } else {
                v[j] = *(const f32x4*)(hr + c);
                if (S > 0) {
                    for (int z = 0; z < S; ++z) {
                        const f32x4 t = *(const f32x4*)(ws + ((size_t)z * M + row) * H + c);
                        v[j][0] += t[0]; v[j][1] += t[1]; v[j][2] += t[2]; v[j][3] += t[3];
                    }
                    *(f32x4*)(hr + c) = v[j];
                }
            }
            ss += v[j][0] * v[j][0] + v[j][1] * v[j][1] + v[j][2] * v[j][2] + v[j][3] * v[j][3];
        }
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = (tid + 256 * j) * 4;
        if (c < H) {
            const f32x4 wq = *(const f32x4*)(w + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[j][e] = v[j][e] * inv * wq[e];
                amax = fmaxf(amax, fabsf(v[j][e]));
            }
            if (!y8) {
                u32x2 o;
                o[0] = pack_bf16x2(v[j][0], v[j][1]);
                o[1] = pack_bf16x2(v[j][2], v[j][3]);
                *(u32x2*)(y + (size_t)row * H + c) = o;
            }
        }
    }
    if (y8) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        if ((tid & 63) == 0) red8[tid >> 6] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red8[0], red8[1]), fmaxf(red8[2], red8[3]));
        const float qs = amax > 0.f ? 448.0f / amax : 1.0f;
        if (tid == 0) y8s[row] = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = (tid + 256 * j) * 4;
            if (c < H)
                *(uint32_t*)(y8 + (size_t)row * H + c) =
                    f32x4_to_e4m3x4(v[j][0] * qs, v[j][1] * qs, v[j][2] * qs, v[j][3] * qs);
        }
    }
}

// Every layer's keys and values from the attention layout (kcat rows of d_h,
// vcat in PV-operand order; see KVLayout) to the caller's [B, L, P, n_kv, d_h]:
// one thread per 8 consecutive head dims of one (b, l, token, kv head).
__global__ void prefix_export_kernel(const PrefillArgs* a, const uint16_t* __restrict__ kcat,
                                     const uint16_t* __restrict__ vcat, KVLayout kv, int B, int P) {
    const int c8 = kv.dh / 8;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)B * kv.L * P * kv.nkv * c8) return;
    const int d8 = (int)(idx % c8);
    long r = idx / c8;
    const int g = (int)(r % kv.nkv);
    r /= kv.nkv;
    const int t = (int)(r % P);
    r /= P;
    const int l = (int)(r % kv.L);
    const int b = (int)(r / kv.L);
    const size_t dst = ((((size_t)b * kv.L + l) * P + t) * kv.nkv + g) * kv.dh + d8 * 8;
    *(u32x4*)(a->pk + dst) = *(const u32x4*)(kcat + kv.k_at(b, l, g, t, d8 * 8));
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = (uint32_t)vcat[kv.v_at(b, l, g, t, d8 * 8 + 2 * j)] |
               ((uint32_t)vcat[kv.v_at(b, l, g, t, d8 * 8 + 2 * j + 1)] << 16);
    *(u32x4*)(a->pv + dst) = o;
}
