// Kernels of one expert layer: fused residual + AdaRMSNorm, the two GEMM
// families (skinny weight-streaming for M <= 64 rows, tiled for larger M) with
// their fused epilogues, the per-call prefix K/V repack and GQA attention.
#pragma once

#include "common.h"

// ---------------------------------------------------------------------------
// Cross-kernel L2 prefetch of weight-streaming GEMM weights. Workgroup w of a
// launch runs on XCD w % 8 (workgroups are dealt to the XCDs in dispatch
// order), each XCD has its own L2, and clean lines stay in it across kernel
// boundaries. A skinny GEMM whose grid width is a multiple of 8 reads, on
// XCD x, exactly the 16-column tiles nt with nt % 8 == x (all of their K
// splits). Extra workgroups appended to an earlier kernel that leaves most
// CUs idle (the batch-1 attention, the norms) load those tiles on the same
// XCD, so the GEMM starts with its weights in L2 (a probe: a 16.8 MB gate_up
// 9.6 -> 8.4 us; the same prefetch on the wrong XCDs gains nothing).
// ---------------------------------------------------------------------------
constexpr int PF_MAX = 3;
struct L2Prefetch {
    const uint8_t* w[PF_MAX];  // packed weights (or MXFP4 block scales) per 16-column tile (null: none)
    int tile_bytes[PF_MAX];    // bytes of one 16-column tile over all of K
    int n_tiles[PF_MAX];
    uint32_t* sink;            // 16 bytes no realistic load result is written to
};

// Prefetcher `rank` of the `per_xcd` prefetching workgroups on XCD `xcd`
// (nthreads threads each) loads its share of the XCD's tiles of each target.
VLA_DEV void l2_prefetch(const L2Prefetch& pf, int xcd, int rank, int per_xcd, int nthreads, int tid) {
    u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int g = 0; g < PF_MAX; ++g) {
        if (!pf.w[g] || rank >= per_xcd) continue;
        const int ppt = pf.tile_bytes[g] / 16;  // 16-byte pieces per tile
        const int ntx = (pf.n_tiles[g] - xcd + 7) / 8;
        const long pieces = (long)ntx * ppt;
        const long stride = (long)per_xcd * nthreads;
        // eight loads in flight per thread, then their results folded
        for (long i0 = (long)rank * nthreads + tid; i0 < pieces; i0 += 8 * stride) {
            u32x4 t[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const long i = i0 + u * stride;
                const int tl = (int)(i / ppt), pc = (int)(i - (long)tl * ppt);
                t[u] = i < pieces ? *(const u32x4*)(pf.w[g] + (size_t)(xcd + 8 * tl) * pf.tile_bytes[g] + (size_t)pc * 16)
                                  : (u32x4){0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) acc ^= t[u];
        }
    }
    // keeps the loads (the compiler cannot prove the branch dead)
    if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u && acc[2] == 0x94d049bbu) *(u32x4*)pf.sink = acc;
}

// Rank of workgroup `lin` among the prefetchers of its XCD, and their count,
// when the prefetchers are the linear ids [base, base + n).
VLA_DEV void prefetch_rank(int lin, int base, int n, int* xcd, int* rank, int* per_xcd) {
    const int x = lin & 7, off = (x - (base & 7) + 8) & 7;  // first prefetcher on XCD x: base + off
    *xcd = x;
    *rank = (lin - base - off) >> 3;
    *per_xcd = n > off ? (n - off + 7) >> 3 : 0;
}

// ---------------------------------------------------------------------------
// Fused residual + AdaRMSNorm, one workgroup (256 threads) per token row,
// H <= 2048, any number S of split-K partials:
//   h += gate * sum_z ws[z]        (when S > 0: split-K partials of O or down)
//   y  = h / sqrt(mean(h^2) + eps) * (1 + scale) + shift  -> bf16 y and/or fp32 yf
// Every load of the first RN_MAXS partials is issued before the first use, so
// a row costs one memory round trip plus the reduction; partials past
// RN_MAXS (only very deep or very narrow down projections split that far)
// are added by a second loop.
// ---------------------------------------------------------------------------
constexpr int RN_MAXS = 8;

__global__ __launch_bounds__(256) void resnorm_kernel(float* __restrict__ h, const float* __restrict__ ws, int S,
                                                      const float* __restrict__ mod, int gate_off, int scale_off,
                                                      int shift_off, uint16_t* __restrict__ y, float* __restrict__ yf,
                                                      int M, int H, int T, int B, int step, int mod_ld, float eps,
                                                      int afrag, uint8_t* __restrict__ y8, float* __restrict__ y8s,
                                                      L2Prefetch pf) {
    __shared__ float red[4], red8[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    if (row >= M) {  // workgroups past the rows prefetch the next GEMM's weights
        int xcd, rank, per_xcd;
        prefetch_rank(row, M, gridDim.x - M, &xcd, &rank, &per_xcd);
        l2_prefetch(pf, xcd, rank, per_xcd, 256, tid);
        return;
    }
    const int b = row / T;
    float* hr = h + (size_t)row * H;
    const float* mr = mod + (size_t)(step * B + b) * mod_ld;
    float4 v[2], part[2][RN_MAXS], g[2], sc[2], sh[2];
    const bool norm = y || yf || y8;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = (tid + 256 * j) * 4;
        if (c < H) {
            v[j] = *(const float4*)(hr + c);
#pragma unroll
            for (int z = 0; z < RN_MAXS; ++z)
                if (z < S) part[j][z] = *(const float4*)(ws + ((size_t)z * M + row) * H + c);
            if (S > 0) g[j] = *(const float4*)(mr + gate_off + c);
            if (norm) {
                sc[j] = *(const float4*)(mr + scale_off + c);
                sh[j] = *(const float4*)(mr + shift_off + c);
            }
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = (tid + 256 * j) * 4;
        if (c < H) {
            if (S > 0) {
                float4 acc = part[j][0];
#pragma unroll
                for (int z = 1; z < RN_MAXS; ++z)
                    if (z < S) {
                        acc.x += part[j][z].x; acc.y += part[j][z].y; acc.z += part[j][z].z; acc.w += part[j][z].w;
                    }
                for (int z = RN_MAXS; z < S; ++z) {
                    const float4 t = *(const float4*)(ws + ((size_t)z * M + row) * H + c);
                    acc.x += t.x; acc.y += t.y; acc.z += t.z; acc.w += t.w;
                }
                v[j].x += g[j].x * acc.x; v[j].y += g[j].y * acc.y; v[j].z += g[j].z * acc.z; v[j].w += g[j].w * acc.w;
                *(float4*)(hr + c) = v[j];
            }
            ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
        }
    }
    if (!norm) return;
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
    float4 ov[2];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = (tid + 256 * j) * 4;
        if (c < H) {
            float4& o = ov[j];
            o.x = v[j].x * inv * (1.f + sc[j].x) + sh[j].x;
            o.y = v[j].y * inv * (1.f + sc[j].y) + sh[j].y;
            o.z = v[j].z * inv * (1.f + sc[j].z) + sh[j].z;
            o.w = v[j].w * inv * (1.f + sc[j].w) + sh[j].w;
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(o.x), fabsf(o.y)), fmaxf(fabsf(o.z), fabsf(o.w))));
            if (y) {
                uint2 ob;
                ob.x = pack_bf16x2(o.x, o.y);
                ob.y = pack_bf16x2(o.z, o.w);
                *(uint2*)(y + act_index(row, c, H, afrag)) = ob;
            }
            if (yf) *(float4*)(yf + (size_t)row * H + c) = o;
        }
    }
    if (y8) {
        // per-token E4M3 copy of y (row-major, for the FP8 GEMMs): codes
        // RNE(y * 448 / max|y|), row scale max|y| / 448 (1 for a zero row)
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        if ((tid & 63) == 0) red8[tid >> 6] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red8[0], red8[1]), fmaxf(red8[2], red8[3]));
        const float qs = amax > 0.f ? 448.0f / amax : 1.0f;
        if (tid == 0) y8s[row] = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = (tid + 256 * j) * 4;
            if (c < H)
                *(uint32_t*)(y8 + (size_t)row * H + c) =
                    f32x4_to_e4m3x4(ov[j].x * qs, ov[j].y * qs, ov[j].z * qs, ov[j].w * qs);
        }
    }
}

// The same residual + AdaRMSNorm for many rows (batched workloads, where a
// workgroup per row spends more time starting than working): one wave per
// row, four rows per 256-thread workgroup, NC float4 chunks per lane (H <=
// 256 NC), every load of the row issued before the first use, and the sums
// and the maximum reduced within the wave (no LDS, no barrier).
template <int NC>
__global__ __launch_bounds__(256) void resnorm_rows_kernel(float* __restrict__ h, const float* __restrict__ ws, int S,
                                                           const float* __restrict__ mod, int gate_off, int scale_off,
                                                           int shift_off, uint16_t* __restrict__ y,
                                                           float* __restrict__ yf, int M, int H, int T, int B,
                                                           int step, int mod_ld, float eps, int afrag,
                                                           uint8_t* __restrict__ y8, float* __restrict__ y8s) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    float* hr = h + (size_t)row * H;
    const float* mr = mod + (size_t)(step * B + row / T) * mod_ld;
    const bool norm = y || yf || y8;
    f32x4 v[NC], g[NC], sc[NC], sh[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = (lane + 64 * j) * 4;
        if (c < H) {
            v[j] = *(const f32x4*)(hr + c);
            if (S > 0) g[j] = *(const f32x4*)(mr + gate_off + c);
            if (norm) {
                sc[j] = *(const f32x4*)(mr + scale_off + c);
                sh[j] = *(const f32x4*)(mr + shift_off + c);
            }
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = (lane + 64 * j) * 4;
        if (c < H) {
            if (S > 0) {
                f32x4 acc = *(const f32x4*)(ws + (size_t)row * H + c);
                for (int z = 1; z < S; ++z) acc += *(const f32x4*)(ws + ((size_t)z * M + row) * H + c);
                v[j] += g[j] * acc;
                *(f32x4*)(hr + c) = v[j];
            }
            ss += v[j][0] * v[j][0] + v[j][1] * v[j][1] + v[j][2] * v[j][2] + v[j][3] * v[j][3];
        }
    }
    if (!norm) return;
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)H + eps);
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = (lane + 64 * j) * 4;
        if (c < H) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[j][e] = v[j][e] * inv * (1.f + sc[j][e]) + sh[j][e];
                amax = fmaxf(amax, fabsf(v[j][e]));
            }
            if (y) {
                u32x2 ob;
                ob[0] = pack_bf16x2(v[j][0], v[j][1]);
                ob[1] = pack_bf16x2(v[j][2], v[j][3]);
                *(u32x2*)(y + act_index(row, c, H, afrag)) = ob;
            }
            if (yf) *(f32x4*)(yf + (size_t)row * H + c) = v[j];
        }
    }
    if (y8) {  // per-token E4M3 copy of y, as in resnorm_kernel
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        const float qs = amax > 0.f ? 448.0f / amax : 1.0f;
        if (lane == 0) y8s[row] = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int c = (lane + 64 * j) * 4;
            if (c < H)
                *(uint32_t*)(y8 + (size_t)row * H + c) =
                    f32x4_to_e4m3x4(v[j][0] * qs, v[j][1] * qs, v[j][2] * qs, v[j][3] * qs);
        }
    }
}

// ---------------------------------------------------------------------------
// Per-layer K/V of the attention, [prefix ; chunk] concatenated on the key
// axis and padded to a multiple of 32 keys (S_pad), per (request, layer, KV
// head):
//   kcat [B][L][n_kv][S_pad/32][d_h/16][64][8]  the K operand of the
//                                  transposed scores S^T = K Q^T: lane l of
//                                  fragment f = sb * (d_h/32) + ks of block kb
//                                  holds key kb*32 + 8*((l%16)/4) + 4*sb + l%4
//                                  at d = ks*32 + 8*(l/16) + j (kfrag_off), so
//                                  every fragment is one contiguous 1 KiB
//   vcat [B][L][n_kv][S_pad/32][d_h/16][64][8]  the PV B operand: lane l of
//                                  fragment (kb, dn) holds keys
//                                  kb*32 + 8*(l/16) + j at d = dn*16 + l%16
// The prefix part is copied in once per call; the chunk part is written by
// the QKV epilogue of each layer.
// ---------------------------------------------------------------------------
// Element offset, within a 32-key block of K, of key w (0..31) and the 8 head
// dims 8c .. 8c+7 (kept contiguous), in the fragment order above.
VLA_DEV int kfrag_off(int w, int c, int dh) {
    const int sb = (w >> 2) & 1, ks = c >> 2;
    const int lane = ((c & 3) << 4) | ((w >> 3) << 2) | (w & 3);
    return ((sb * (dh >> 5) + ks) * 64 + lane) * 8;
}

struct KVLayout {
    int L, nkv, dh, S_pad;
    VLA_DEV size_t base(int b, int l, int g) const { return (((size_t)b * L + l) * nkv + g) * (size_t)S_pad * dh; }
    VLA_DEV size_t k_at(int b, int l, int g, int key, int d) const {
        return base(b, l, g) + (size_t)(key >> 5) * 32 * dh + kfrag_off(key & 31, d >> 3, dh) + (d & 7);
    }
    VLA_DEV size_t v_at(int b, int l, int g, int key, int d) const {
        const int kb = key >> 5, w = key & 31;
        return base(b, l, g) + (size_t)kb * 32 * dh +
               ((size_t)((d >> 4) * 64 + (w >> 3) * 16 + (d & 15)) * 8 + (w & 7));
    }
};

__global__ void prefix_repack_kernel(const ArgBlock* ab, const uint16_t* pk_direct, const uint16_t* pv_direct,
                                     uint16_t* __restrict__ kcat, uint16_t* __restrict__ vcat, KVLayout kv, int B,
                                     int P) {
    const uint16_t* pk = pk_direct ? pk_direct : ab->prefix_k;
    const uint16_t* pv = pv_direct ? pv_direct : ab->prefix_v;
    const int c8 = kv.dh / 8;
    long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    long total = (long)B * kv.L * P * kv.nkv * c8;
    if (idx >= total) return;
    int d8 = (int)(idx % c8);
    long r = idx / c8;
    int g = (int)(r % kv.nkv);
    r /= kv.nkv;
    int p = (int)(r % P);
    r /= P;
    int l = (int)(r % kv.L);
    int b = (int)(r / kv.L);
    size_t src = ((((size_t)b * kv.L + l) * P + p) * kv.nkv + g) * kv.dh + d8 * 8;
    *(u32x4*)(kcat + kv.k_at(b, l, g, p, d8 * 8)) = *(const u32x4*)(pk + src);
    u32x4 vv = *(const u32x4*)(pv + src);
    const uint16_t* e = (const uint16_t*)&vv;
#pragma unroll
    for (int j = 0; j < 8; ++j) vcat[kv.v_at(b, l, g, p, d8 * 8 + j)] = e[j];
}

// The chunk's own keys/values [B][n_kv][T][d_h] written into layer `layer` of
// kcat/vcat at keys P..P+T-1 (used by the single-stage attention entry point;
// in the loop the QKV epilogue writes them directly).
__global__ void chunk_kv_store_kernel(const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
                                      uint16_t* __restrict__ kcat, uint16_t* __restrict__ vcat, KVLayout kv,
                                      int layer, int P, int B, int T) {
    const int c8 = kv.dh / 8;
    long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)B * kv.nkv * T * c8) return;
    int d8 = (int)(idx % c8);
    long r = idx / c8;
    int i = (int)(r % T);
    r /= T;
    int g = (int)(r % kv.nkv);
    int b = (int)(r / kv.nkv);
    size_t src = (((size_t)b * kv.nkv + g) * T + i) * kv.dh + d8 * 8;
    *(u32x4*)(kcat + kv.k_at(b, layer, g, P + i, d8 * 8)) = *(const u32x4*)(kn + src);
    u32x4 vv = *(const u32x4*)(vn + src);
    const uint16_t* e = (const uint16_t*)&vv;
#pragma unroll
    for (int j = 0; j < 8; ++j) vcat[kv.v_at(b, layer, g, P + i, d8 * 8 + j)] = e[j];
}

// ---------------------------------------------------------------------------
// GEMM epilogues, shared by the skinny and the tiled kernels
// ---------------------------------------------------------------------------
enum { EPI_BIAS_F32 = 0, EPI_RESID = 1, EPI_QKV_ROPE = 2, EPI_SWIGLU = 3, EPI_PARTIAL = 4, EPI_ADD = 5 };

struct GemmParams {
    const uint16_t* A;   // [M, lda] bf16: row-major (tiled kernel) or A-fragment order (skinny kernel)
    int lda;
    int a_frag;          // A given in A-fragment order (required by the skinny kernel)
    int afrag;           // act (SwiGLU output) written in A-fragment order
    int tile_map;        // tiled kernel: 1 = row tiles split over the XCDs (grid padded to 8 row-tile groups)
    const float* ascale; // FP8 tiled kernel: per-row scales of the E4M3 A operand
    const uint8_t* bscale; // MXFP4 weights: E8M0 scale per (packed row, 32 inputs), [N/16][K/32][16]
    const void* W;       // packed fragments
    const float* wscale; // per packed row (E4M3), else null
    int M, N, K;
    int kw;              // K per split (skinny kernel)
    float* ws;           // EPI_PARTIAL: [ksplit][M][N]
    float* out_f32;      // EPI_BIAS_F32: [M][N]; EPI_RESID, EPI_ADD: h [M][N]
    const float* bias;
    const float* mod;    // EPI_RESID gate source
    int mod_ld, gate_off, step, B, T;
    uint16_t* q;         // EPI_QKV_ROPE: q [B][nq][T][dh]
    uint16_t* kcat;      // chunk keys/values go to key P + i of layer `layer`
    uint16_t* vcat;
    KVLayout kv;
    int layer, P;
    const float2* rope;  // [P + T][dh/2] by absolute position
    const int* pvalid;   // [B] this call's valid prefix lengths: row b*T+i sits at pvalid[b] + i
    int nq, nkv, dh;
    int dh_shift;        // log2(dh)
    float inv_T;         // 1/T, for the row -> request split without a divide
    uint16_t* act;       // EPI_SWIGLU output [M][N/2]
};

// row / T for row >= 0: a float estimate corrected to the exact quotient
// (epilogues run this per element, where an integer divide costs ~40 ops).
VLA_DEV int div_T(int row, const GemmParams& p) {
    int b = (int)((float)row * p.inv_T);
    if (b * p.T > row) --b;
    else if ((b + 1) * p.T <= row) ++b;
    return b;
}

// v: this lane's value of (row, col); partner: the value of (row, col ^ 1).
// RoPE position of chunk row r = b*T + i: pvalid[b] + i (QKV epilogue only).
VLA_DEV int qkv_row_pos(const GemmParams& p, int row) {
    const int b = div_T(row, p);
    return p.pvalid[b] + row - b * p.T;
}

// rpos: qkv_row_pos(p, row) for EPI_QKV_ROPE (callers hoist it per row);
// rope_cs: that row's RoPE factors for this column when already loaded.
template <int EPI>
VLA_DEV void epilogue_store(const GemmParams& p, int row, int col, float v, float partner, int kz, int rpos,
                            const float2* rope_cs = nullptr) {
    if (row >= p.M) return;
    if constexpr (EPI == EPI_PARTIAL) {
        p.ws[((size_t)kz * p.M + row) * p.N + col] = v;
    } else if constexpr (EPI == EPI_BIAS_F32) {
        p.out_f32[(size_t)row * p.N + col] = v + p.bias[col];
    } else if constexpr (EPI == EPI_RESID) {
        const int b = div_T(row, p);
        const float g = p.mod[(size_t)(p.step * p.B + b) * p.mod_ld + p.gate_off + col];
        float* hp = p.out_f32 + (size_t)row * p.N + col;
        *hp = *hp + g * v;
    } else if constexpr (EPI == EPI_QKV_ROPE) {
        // packed columns: per head, rotate-half partners (m, m + d_h/2) are the
        // adjacent columns (2m, 2m + 1)
        const int qd = p.nq * p.dh, kvd = p.nkv * p.dh;
        int sec, local;
        if (col < qd) { sec = 0; local = col; }
        else if (col < qd + kvd) { sec = 1; local = col - qd; }
        else { sec = 2; local = col - qd - kvd; }
        const int head = local >> p.dh_shift, pp = local & (p.dh - 1);
        const int m = pp >> 1, second = pp & 1;
        const int b = div_T(row, p), i = row - b * p.T;
        float outv = v;
        if (sec < 2) {
            const float2 cs = rope_cs ? *rope_cs : p.rope[rpos * (p.dh / 2) + m];
            const float u1 = second ? partner : v;
            const float u2 = second ? v : partner;
            outv = second ? (u2 * cs.x + u1 * cs.y) : (u1 * cs.x - u2 * cs.y);
        }
        const int dim = m + second * (p.dh / 2);
        const uint16_t ob = f32_to_bf16(outv);
        if (sec == 0) p.q[((size_t)(b * p.nq + head) * p.T + i) * p.dh + dim] = ob;
        else if (sec == 1) p.kcat[p.kv.k_at(b, p.layer, head, p.P + i, dim)] = ob;
        else p.vcat[p.kv.v_at(b, p.layer, head, p.P + i, dim)] = ob;
    } else if constexpr (EPI == EPI_SWIGLU) {
        // packed columns alternate gate (even) and up (odd) of one output
        if ((col & 1) == 0) p.act[act_index(row, col >> 1, p.N / 2, p.afrag)] = f32_to_bf16(silu_f(v) * partner);
    }
}

// The epilogue of 16 consecutive columns col0..col0+15 of one row (col0 a
// multiple of 16) for the tiled kernel: the same results as epilogue_store
// column by column, with 16-byte global accesses.
template <int EPI>
VLA_DEV void epilogue16(const GemmParams& p, int row, int col0, const float (&v)[16], int kz = 0) {
    if constexpr (EPI == EPI_PARTIAL) {  // split-K partial kz: ws[kz][row][col]
        float* o = p.ws + ((size_t)kz * p.M + row) * p.N + col0;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *(f32x4*)(o + 4 * q) = (f32x4){v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    } else if constexpr (EPI == EPI_BIAS_F32) {
        float* o = p.out_f32 + (size_t)row * p.N + col0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 bq = *(const f32x4*)(p.bias + col0 + 4 * q);
            *(f32x4*)(o + 4 * q) = (f32x4){v[4 * q] + bq[0], v[4 * q + 1] + bq[1], v[4 * q + 2] + bq[2],
                                           v[4 * q + 3] + bq[3]};
        }
    } else if constexpr (EPI == EPI_RESID) {
        const int b = div_T(row, p);
        const float* g = p.mod + (size_t)(p.step * p.B + b) * p.mod_ld + p.gate_off + col0;
        float* hp = p.out_f32 + (size_t)row * p.N + col0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 gq = *(const f32x4*)(g + 4 * q);
            const f32x4 hq = *(const f32x4*)(hp + 4 * q);
            *(f32x4*)(hp + 4 * q) = (f32x4){hq[0] + gq[0] * v[4 * q], hq[1] + gq[1] * v[4 * q + 1],
                                            hq[2] + gq[2] * v[4 * q + 2], hq[3] + gq[3] * v[4 * q + 3]};
        }
    } else if constexpr (EPI == EPI_ADD) {  // plain residual: h += v
        float* hp = p.out_f32 + (size_t)row * p.N + col0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 hq = *(const f32x4*)(hp + 4 * q);
            *(f32x4*)(hp + 4 * q) = (f32x4){hq[0] + v[4 * q], hq[1] + v[4 * q + 1], hq[2] + v[4 * q + 2],
                                            hq[3] + v[4 * q + 3]};
        }
    } else if constexpr (EPI == EPI_SWIGLU) {
        // columns alternate gate (even) and up (odd) of outputs col0/2 .. col0/2 + 7
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = pack_bf16x2(silu_f(v[4 * j]) * v[4 * j + 1], silu_f(v[4 * j + 2]) * v[4 * j + 3]);
        *(u32x4*)(p.act + act_index(row, col0 >> 1, p.N / 2, p.afrag)) = o;
    } else if constexpr (EPI == EPI_QKV_ROPE) {
        // the 16 columns are 8 rotate-half pairs (m, m + d_h/2), m = m0 .. m0+7, of one head
        const int qd = p.nq * p.dh, kvd = p.nkv * p.dh;
        int sec, local;
        if (col0 < qd) { sec = 0; local = col0; }
        else if (col0 < qd + kvd) { sec = 1; local = col0 - qd; }
        else { sec = 2; local = col0 - qd - kvd; }
        const int head = local >> p.dh_shift, m0 = (local & (p.dh - 1)) >> 1;
        const int b = div_T(row, p), i = row - b * p.T;
        float lo[8], hi[8];
        if (sec < 2) {
            const float2* cs = p.rope + (size_t)(p.pvalid[b] + i) * (p.dh / 2) + m0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float2 c = cs[j];
                lo[j] = v[2 * j] * c.x - v[2 * j + 1] * c.y;
                hi[j] = v[2 * j + 1] * c.x + v[2 * j] * c.y;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) { lo[j] = v[2 * j]; hi[j] = v[2 * j + 1]; }
        }
        if (sec < 2) {
            uint16_t* dlo;
            uint16_t* dhi;
            if (sec == 0) {
                dlo = p.q + ((size_t)(b * p.nq + head) * p.T + i) * p.dh + m0;
                dhi = dlo + p.dh / 2;
            } else {
                dlo = p.kcat + p.kv.k_at(b, p.layer, head, p.P + i, m0);
                dhi = p.kcat + p.kv.k_at(b, p.layer, head, p.P + i, m0 + p.dh / 2);
            }
            u32x4 a, c;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a[j] = pack_bf16x2(lo[2 * j], lo[2 * j + 1]);
                c[j] = pack_bf16x2(hi[2 * j], hi[2 * j + 1]);
            }
            *(u32x4*)dlo = a;
            *(u32x4*)dhi = c;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                p.vcat[p.kv.v_at(b, p.layer, head, p.P + i, m0 + j)] = f32_to_bf16(lo[j]);
                p.vcat[p.kv.v_at(b, p.layer, head, p.P + i, m0 + j + p.dh / 2)] = f32_to_bf16(hi[j]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Skinny GEMM for M <= 64 rows (weight streaming). A workgroup of 8 waves
// owns one K split and a strided set of 16-column tiles (tile = blockIdx.x +
// i * gridDim.x). Each wave takes one eighth of the split: it loads its
// activation fragments (4 row tiles) into registers once, then streams the
// weight fragments of each column tile (contiguous 1 KiB per k-step),
// prefetching the next tile's fragments before computing the current one.
// The eight partial tiles are reduced through LDS (double buffered, one
// barrier per tile). No cross-workgroup synchronisation: with several K
// splits the epilogue writes fp32 partials that the next fused residual +
// norm kernel sums.
// ---------------------------------------------------------------------------
constexpr int SK_WAVES = 8;
constexpr int SK_MAXS = 6;  // k-steps (of 32) per wave: K split <= 8 * 6 * 32 = 1536

// Eight E2M1 codes (element j in bits 4j..4j+3) times the E8M0 block scale
// 2^(e - 127) as bf16, by gfx950's scaled FP4 conversion: each
// v_cvt_scalef32_pk_bf16_fp4 takes the two codes of one byte (the low nibble
// is the lower element) and multiplies them by an fp32 scale. An E2M1 value
// has at most two significant bits, so the product by a power of two is
// exact in bf16 while it stays normal, as for weights of any reasonable size.
VLA_DEV bf16x8 e2m1x8_to_bf16x8(uint32_t w, uint32_t e) {
    const float sc = __uint_as_float(e << 23);  // 2^(e - 127) for e in 1..254
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
    return (bf16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// WF: weight format, 0 bf16, 1 E4M3 (fp32 scale per output row), 2 MXFP4
// (E2M1 codes, E8M0 scale per 32 inputs). WNT: bf16 / E4M3 weights read
// with the non-temporal hint (the host's default at batch 1, measured
// faster on every model there): the streamed weights then do not evict
// the lines that are used again (code, activations, the weights a norm
// reads ahead for the next linear).
template <int WF, int EPI, bool WNT = false>
__global__ __launch_bounds__(512) void skinny_gemm_kernel(GemmParams p) {
    constexpr bool W8 = WF == 1;
    __shared__ __attribute__((aligned(16))) float red[2][SK_WAVES][4][64][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kz = blockIdx.y;
    const int n_tiles = p.N / 16;
    const int Kf = p.K / 32;
    const int kt0 = kz * (p.kw / 32);
    const int steps = p.kw / 32;
    const int per = (steps + SK_WAVES - 1) / SK_WAVES;
    const int s_beg = min(steps, wave * per);
    const int ns = min(steps, s_beg + per) - s_beg;  // k-steps of this wave (<= SK_MAXS)

    // activation fragments of this wave's k-steps, all four 16-row tiles
    // (A is in A-fragment order: one contiguous 1 KiB per (k-step, row tile);
    // rows >= M hold zeros)
    bf16x8 af[SK_MAXS][4];
#pragma unroll
    for (int i = 0; i < SK_MAXS; ++i)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            af[i][mt] = i < ns ? *(const bf16x8*)(p.A + ((size_t)((kt0 + s_beg + i) * 4 + mt) * 64 + lane) * 8)
                               : (bf16x8){};

    constexpr int WREG = WF == 2 ? 1 : (W8 ? 2 : 4);  // dwords of one weight fragment slice per lane
    typedef __attribute__((ext_vector_type(WREG == 1 ? 2 : WREG))) unsigned wvec;
    // MXFP4: the block scale of the lane's row (l%16) rides in the second dword
    auto load_w = [&](int nt, wvec* dst) {
#pragma unroll
        for (int i = 0; i < SK_MAXS; ++i)
            if (i < ns) {
                const size_t frag = (size_t)nt * Kf + kt0 + s_beg + i;
                if constexpr (WF == 2) {
                    dst[i][0] = *(const uint32_t*)((const uint8_t*)p.W + (frag * 64 + lane) * 4);
                    dst[i][1] = p.bscale[frag * 16 + (lane & 15)];
                } else {
                    const wvec* src = (const wvec*)((const uint8_t*)p.W + (frag * 64 + lane) * (W8 ? 8 : 16));
                    if constexpr (WNT) dst[i] = __builtin_nontemporal_load(src);
                    else dst[i] = *src;
                }
            }
    };

    wvec wcur[SK_MAXS], wnext[SK_MAXS];
    int nt = blockIdx.x;
    if (nt < n_tiles) load_w(nt, wcur);

    // epilogue operands of the first tile that do not depend on the sums (the
    // E4M3 column scale; the QKV rows' RoPE positions and factors) are loaded
    // now, so the epilogue does not wait on dependent loads
    const int nt0 = blockIdx.x;
    float wsc0 = 1.0f;
    int rpos0[4] = {0, 0, 0, 0};
    float2 cs0[4];
    if (wave < 4 && nt0 < n_tiles) {
        const int col = nt0 * 16 + (lane & 15);
        if constexpr (W8) wsc0 = p.wscale[col];
        if constexpr (EPI == EPI_QKV_ROPE) {
            const bool roped = col < (p.nq + p.nkv) * p.dh;  // q and k columns
            const int m = (col & (p.dh - 1)) >> 1;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wave * 16 + 4 * (lane >> 4) + r;
                rpos0[r] = row < p.M ? qkv_row_pos(p, row) : 0;
                cs0[r] = roped && row < p.M ? p.rope[rpos0[r] * (p.dh / 2) + m] : make_float2(0.f, 0.f);
            }
        }
    }
    int buf = 0;
    for (; nt < n_tiles; nt += gridDim.x) {
        const int nt_next = nt + gridDim.x;
        if (nt_next < n_tiles) load_w(nt_next, wnext);
        f32x4 acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < SK_MAXS; ++i) {
            if (i < ns) {
                bf16x8 b;
                if constexpr (WF == 2) b = e2m1x8_to_bf16x8(wcur[i][0], wcur[i][1]);
                else if constexpr (W8) b = e4m3x8_to_bf16x8(wcur[i]);
                else b = __builtin_bit_cast(bf16x8, wcur[i]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma_16x16x32(af[i][mt], b, acc[mt]);
            }
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) *(f32x4*)(&red[buf][wave][mt][lane][0]) = acc[mt];
        __syncthreads();
        if (wave < 4) {  // wave w finishes row tile w
            f32x4 sum = *(const f32x4*)(&red[buf][0][wave][lane][0]);
#pragma unroll
            for (int w = 1; w < SK_WAVES; ++w) sum += *(const f32x4*)(&red[buf][w][wave][lane][0]);
            const int col = nt * 16 + (lane & 15);
            const bool first = nt == nt0;
            const float wsc = W8 ? (first ? wsc0 : p.wscale[col]) : 1.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wave * 16 + 4 * (lane >> 4) + r;
                const float v = sum[r] * wsc;
                const float partner = __shfl_xor(v, 1, 64);
                if (EPI == EPI_QKV_ROPE && first)
                    epilogue_store<EPI>(p, row, col, v, partner, kz, rpos0[r], &cs0[r]);
                else
                    epilogue_store<EPI>(p, row, col, v, partner, kz,
                                        EPI == EPI_QKV_ROPE && row < p.M ? qkv_row_pos(p, row) : 0);
            }
        }
        buf ^= 1;
#pragma unroll
        for (int i = 0; i < SK_MAXS; ++i) wcur[i] = wnext[i];
    }
}

// ---------------------------------------------------------------------------
// Tiled GEMM for larger M: an MT x NT tile per workgroup of 8 waves. K
// advances in 64-deep stages through a ring of LDS buffers that global->LDS
// DMA loads fill directly (no register staging): stage kt+S is requested as
// soon as every wave is done with stage kt, so S-1 stages are in flight
// while one is multiplied. Both operands sit in LDS as 1 KiB MFMA fragments
// (lane i's 16 bytes at offset 16 i), so the DMA writes and the fragment
// reads are free of bank conflicts. The 8 waves form a 2 x 4 grid of
// MT/2 x NT/4 wave tiles. (Two k-groups of 2 x 2 waves with 64 x 64 wave
// tiles, for half the LDS bytes per MFMA on 128-row tiles, measured no
// faster: the 128-row tiles are not bound by LDS bandwidth.)
// ---------------------------------------------------------------------------
constexpr int GEMM_WAVES = 8;
constexpr int GEMM_KT = 64;   // K granularity of a tiled GEMM (its loop runs k-steps of 32 in pairs)

// 16 bytes per lane from global memory into LDS: the 64 lanes fill the
// 1 KiB at byte offset `lds` (lane i at lds + 16 i). No register receives
// data; the kernel waits for these loads itself (vm_wait) before the
// barrier that publishes a stage, and before it exits. M0 carries the LDS
// address; it is a register the compiler reserves (a clobber of it would be
// ignored), so the block saves and restores it.
VLA_DEV void lds_dma16(const void* g, uint32_t lds) {
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep)
                 : "v"(g), "s"(lds)
                 : "memory");
}
template <int N>
VLA_DEV void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Stage depth and LDS ring per tile shape. A stage holds A as MT rows of
// RB = 2 KT bytes, each row's 16-byte chunk c at chunk position
// c ^ ((r / RPB) % CPR) (RPB rows per 256 bytes, i.e. per pass over the 64
// banks): one DMA load (1 KiB) fills RPL whole rows, each from contiguous
// global bytes, and the 16 lanes that read one MFMA fragment (16 rows, one
// chunk) meet 16 distinct bank groups. Stages: as many as fit in
// GEMM_LDS_BUDGET, at most GEMM_SMAX (one workgroup per CU). The code takes
// 32- or 64-deep stages; 64 is used (32-deep stages make the A rows 64-byte
// half lines, which the DMA path moves at about 60 % of the rate).
constexpr int GEMM_STAGE_KT = 64, GEMM_SMAX = 3, GEMM_LDS_BUDGET = 147456;
template <int MT, int NT, bool W8>
struct GemmShape {
    static constexpr int KT = W8 ? 64 : GEMM_STAGE_KT;           // inputs per stage
    static constexpr int KS = KT / 32;                           // MFMA k-steps per stage
    static constexpr int RB = KT * 2, CPR = RB / 16, RPL = 64 / CPR, RPB = 256 / RB;
    static constexpr int AF = MT / RPL;                          // A loads per stage (1 KiB each)
    static constexpr int BBYTES = NT / 16 * KS * (W8 ? 512 : 1024);
    static constexpr int BCH = BBYTES / 1024;                    // 1 KiB DMA chunks of B per stage
    static constexpr int STAGE = AF * 1024 + BBYTES;
    static constexpr int S = GEMM_LDS_BUDGET / STAGE >= GEMM_SMAX ? GEMM_SMAX : GEMM_LDS_BUDGET / STAGE;
    static constexpr int LA = (AF + GEMM_WAVES - 1) / GEMM_WAVES;   // DMA loads per wave and stage
    static constexpr int LB = (BCH + GEMM_WAVES - 1) / GEMM_WAVES;
    static constexpr int LPW = LA + LB;
    static_assert(KS == 1 || KS == 2, "stages of one or two k-steps");
    static_assert(S >= 2, "tile too large for two LDS stages");
};

// SwiGLU epilogue of a tiled GEMM straight from the MFMA accumulators (8
// waves as 2 x 4 wave tiles of MT/2 x NT/4). The packed weight rows
// alternate gate (even column) and up (odd column), so lanes l and l ^ 1
// hold the two halves of the same outputs for the same four rows. One swap
// of two values between them leaves each lane two outputs (two rows), and a
// second swap with lane l ^ 2 pairs adjacent outputs of one row as bf16x2,
// which each lane writes into a bf16 output tile in LDS. The row pitch is
// NT + 16 bytes, so the 16 rows one write instruction touches meet distinct
// banks and one row's 16-byte chunks are contiguous; 16-byte chunks then go
// to global memory, row by row. val(fm, fn, r) is accumulator element r of
// fragment (fm, fn) with its scales applied. The LDS ring must be free.
template <int MT, int NT, int FM, int FN, typename Val>
VLA_DEV void swiglu_epilogue_tile(const GemmParams& p, uint8_t* lds, int m0, int n0, int wm, int wn, int lane,
                                  int tid, Val val) {
    constexpr int WM = MT / 2, WN = NT / 4, OP = NT + 16;
    const bool odd = lane & 1, podd = lane & 2;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            float a[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = val(fm, fn, r);
            // even lanes keep rows 0, 1 (their gate), odd lanes rows 2, 3 (their up)
            const float y0 = row_dpp<0xB1>(odd ? a[0] : a[2]), y1 = row_dpp<0xB1>(odd ? a[1] : a[3]);
            const float o0 = silu_f(odd ? y0 : a[0]) * (odd ? a[2] : y0);
            const float o1 = silu_f(odd ? y1 : a[1]) * (odd ? a[3] : y1);
            // lanes with bit 1 clear keep the first row, the others the second
            const float w = row_dpp<0x4E>(podd ? o0 : o1);
            const uint32_t pk = podd ? pack_bf16x2(w, o1) : pack_bf16x2(o0, w);
            const int r = wm * WM + fm * 16 + 4 * (lane >> 4) + (odd ? 2 : 0) + (podd ? 1 : 0);
            const int oc = (wn * WN + fn * 16) / 2 + ((lane & 15) >> 2) * 2;
            *(uint32_t*)(lds + r * OP + oc * 2) = pk;
        }
    __syncthreads();
    constexpr int CPR = NT / 16;   // 16-byte chunks (8 outputs) per output row
    for (int u = tid; u < MT * CPR; u += 64 * GEMM_WAVES) {
        const int r = u / CPR, q = u % CPR;
        if (m0 + r < p.M)
            *(u32x4*)(p.act + act_index(m0 + r, n0 / 2 + 8 * q, p.N / 2, p.afrag)) = *(const u32x4*)(lds + r * OP + 16 * q);
    }
}

template <int MT, int NT, bool W8, int EPI>
__global__ __launch_bounds__(64 * GEMM_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_kernel(GemmParams p) {
    using G = GemmShape<MT, NT, W8>;
    constexpr int S = G::S, AF = G::AF, BCH = G::BCH, LA = G::LA, LB = G::LB, LPW = G::LPW, STAGE = G::STAGE;
    constexpr int KT = G::KT, KS = G::KS, RB = G::RB, CPR = G::CPR, RPL = G::RPL, RPB = G::RPB, WGN = 4;
    constexpr int WM = MT / 2, WN = NT / WGN, FM = WM / 16, FN = WN / 16;
    static_assert(FM >= 1 && FN >= 1, "tile smaller than the wave grid");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[S * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    // Tile of this workgroup. Consecutive workgroups run on consecutive XCDs
    // (workgroup w on XCD w % 8), and each XCD has its own L2, so the larger
    // operand is split over the XCDs: with tile_map 1, XCD x takes the row
    // tiles x, x + 8, ... (every column tile of each), so each XCD reads one
    // eighth of A; otherwise, when the column tiles split evenly over the
    // XCDs, XCD x takes one eighth of them (and of W) for every row tile.
    const int ntn = p.N / NT;
    int mt_i, nt_i;
    if (p.tile_map == 1) {
        const int w = blockIdx.x, s = w >> 3;
        mt_i = (w & 7) + 8 * (s / ntn);
        nt_i = s % ntn;
        if (mt_i * MT >= p.M) return;  // padding of the last group of 8 row tiles
    } else if (ntn % 8 == 0) {
        const int w = blockIdx.x, per = ntn / 8, s = w >> 3;
        mt_i = s / per;
        nt_i = (w & 7) * per + s % per;
    } else {
        mt_i = blockIdx.x / ntn;
        nt_i = blockIdx.x % ntn;
    }
    const int m0 = mt_i * MT, n0 = nt_i * NT;
    // split K (gridDim.y > 1, EPI_PARTIAL): this workgroup sums inputs
    // [kz * kw, (kz + 1) * kw) and writes partial kz
    const int kz = blockIdx.y, kf0 = kz * (p.kw / 32);
    const int nk = p.kw / KT, Kf = p.K / 32;
    const uint32_t lbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;

    // Per-lane source of each DMA load of this wave (stage 0) and the stride
    // per stage. Load j of A covers rows RPL j .. RPL j + RPL - 1 of the
    // stage (whole rows from contiguous global bytes: a load of 16 half
    // lines moves about 40 % fewer bytes per clock); chunk c of B is one
    // 1 KiB weight fragment. Waves with fewer chunks than loads repeat one
    // (same bytes, same place).
    const uint16_t* asrc[LA];
    uint32_t adst[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int j = (wave * LA + i) % AF, r = j * RPL + lane / CPR;
        const int c = (lane % CPR) ^ ((r / RPB) % CPR);
        if (p.a_frag) {
            // A-fragment order of <= 64 rows: fragment (k-step, row block) is
            // 1 KiB, lane l holding row l % 16 at inputs 8 (l / 16) .. + 7
            const int row = min(m0 + r, 63);
            asrc[i] = p.A + ((size_t)((kf0 + (c >> 2)) * 4 + (row >> 4)) * 64 + (row & 15) + 16 * (c & 3)) * 8;
        } else {
            // rows past M read row M-1; their results are never stored
            const int row = min(m0 + r, p.M - 1);
            asrc[i] = p.A + (size_t)row * p.lda + kf0 * 32 + c * 8;
        }
        adst[i] = (uint32_t)j * 1024;
    }
    const size_t astride = p.a_frag ? (size_t)KS * 4 * 512 : (size_t)KT;
    const uint8_t* bsrc[LB];
    uint32_t bdst[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int c = (wave * LB + i) % BCH;
        if constexpr (W8) {
            // one chunk = the 2 k-steps (512 bytes each) of one 16-column tile
            bsrc[i] = (const uint8_t*)p.W + ((size_t)(n0 / 16 + c) * Kf + kf0) * 512 + lane * 16;
        } else {
            const int fn = c / KS, ks = c % KS;
            bsrc[i] = (const uint8_t*)p.W + ((size_t)(n0 / 16 + fn) * Kf + kf0 + ks) * 1024 + lane * 16;
        }
        bdst[i] = (uint32_t)(AF * 1024 + c * 1024);
    }
    constexpr size_t bstride = (size_t)KS * (W8 ? 512 : 1024);
    // Stage kt into ring slot kt % S. Past the last stage the loads repeat it
    // (into a slot no later stage uses), so every wave always has the same
    // number of loads in flight and the waits are constants.
    auto issue = [&](int kt_raw) {
        const uint32_t sb = lbase + (uint32_t)((kt_raw % S) * STAGE);
        const int kt = min(kt_raw, nk - 1);
#pragma unroll
        for (int i = 0; i < LA; ++i) lds_dma16(asrc[i] + kt * astride, sb + adst[i]);
#pragma unroll
        for (int i = 0; i < LB; ++i) lds_dma16(bsrc[i] + kt * bstride, sb + bdst[i]);
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // fragments of k-step ks + 1 are read while k-step ks is multiplied; lane
    // l reads row l % 16 of each row block at chunk 4 ks + l / 16 (swizzled)
    bf16x8 fa[2][FM], fb[2][FN];
    const int arow = (wm * FM * 16 + (lane & 15)) * RB;
    const int aswz = ((lane & 15) / RPB) % CPR;   // the row's chunk permutation (fm * 16 rows keep it)
    auto read_frags = [&](int buf, const uint8_t* st, int ks) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            fa[buf][fm] = *(const bf16x8*)(st + arow + fm * 16 * RB + (((ks * 4 + (lane >> 4)) ^ aswz) << 4));
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int frag = (wn * FN + fn) * KS + ks;
            if constexpr (W8) fb[buf][fn] = e4m3x8_to_bf16x8(*(const u32x2*)(st + AF * 1024 + frag * 512 + lane * 8));
            else fb[buf][fn] = *(const bf16x8*)(st + AF * 1024 + frag * 1024 + lane * 16);
        }
    };
    auto multiply = [&](int buf) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma_16x16x32(fa[buf][fm], fb[buf][fn], acc[fm][fn]);
    };

#pragma unroll
    for (int s = 0; s < S; ++s) issue(s);
    vm_wait<(S - 1) * LPW>();
    __syncthreads();
    read_frags(0, lds, 0);
    // k-step g (32 inputs) of stage g / KS multiplies fragment buffer g % 2;
    // the other buffer takes k-step g + 1 meanwhile. Two k-steps per
    // iteration keep the buffer indexes constant (the k-steps of a split
    // are a multiple of two).
    auto step = [&](int g, auto bufc) {
        constexpr int buf = decltype(bufc)::value, ks = buf % KS;
        const int kt = g / KS;
        if (ks + 1 < KS) {
            read_frags(buf ^ 1, lds + (kt % S) * STAGE, ks + 1);
        } else {
            // stage kt+1 landed (this wave's loads), then every wave's
            // loads landed and every wave is done reading stage kt
            vm_wait<(S - 2) * LPW>();
            __syncthreads();
            issue(kt + S);
            read_frags(buf ^ 1, lds + ((kt + 1) % S) * STAGE, 0);
        }
        // keep the fragment reads ahead of the multiplies they overlap
        __builtin_amdgcn_sched_barrier(0);
        multiply(buf);
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int g = 0; g < nk * KS; g += 2) {
        step(g, std::integral_constant<int, 0>{});
        step(g + 1, std::integral_constant<int, 1>{});
    }
    vm_wait<0>();  // the repeated tail loads land before the LDS is reused
    __syncthreads();    // every wave is done with the ring

    if constexpr (EPI == EPI_SWIGLU) {
        static_assert(MT * (NT + 16) <= S * STAGE, "SwiGLU output tile does not fit the ring");
        float wsc[FN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) wsc[fn] = W8 ? p.wscale[n0 + wn * WN + fn * 16 + (lane & 15)] : 1.0f;
        swiglu_epilogue_tile<MT, NT, FM, FN>(p, lds, m0, n0, wm, wn, lane, tid, [&](int fm, int fn, int r) {
            return W8 ? acc[fm][fn][r] * wsc[fn] : acc[fm][fn][r];
        });
        return;
    }

    // Epilogue through LDS, 64 tile rows per pass: the waves holding those
    // rows write their accumulators (times the E4M3 row scales) as fp32 rows,
    // then all threads apply the epilogue to 16 consecutive columns each, so
    // that global reads and writes are 16-byte vectors.
    constexpr int CLD = NT + 4;    // row pitch in floats: a fragment writes rows r, r+4, r+8, r+12 (16 lanes each), 16 banks apart
    constexpr int PPW = FM / 4;    // passes per wave row
    constexpr int UPR = NT / 16;   // 16-column units per row
    static_assert(FM % 4 == 0 && 64 * CLD * 4 <= S * STAGE, "epilogue pass does not fit the ring");
    float* ct = (float*)lds;
    // Column col of a row sits at col ^ (4 s): s = ((col / 64) * (256 / NT)) % 4
    // permutes the 4-float chunks of each 16-column unit, so that the 16
    // threads reading one unit's chunk q (16 units of one row for NT = 256,
    // 8 units of two rows for NT = 128) meet 16 distinct bank groups; a
    // fragment write (16 consecutive columns) stays within one unit.
    auto swz = [](int col) { return col ^ ((((col >> 6) * (256 / NT)) & 3) << 2); };
    float wsc[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) wsc[fn] = W8 ? p.wscale[n0 + wn * WN + fn * 16 + (lane & 15)] : 1.0f;
#pragma unroll
    for (int pass = 0; pass < MT / 64; ++pass) {
        if (wm == pass / PPW) {
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        ct[(f * 16 + 4 * (lane >> 4) + r) * CLD + swz(wn * WN + fn * 16 + (lane & 15))] =
                            acc[(pass % PPW) * 4 + f][fn][r] * wsc[fn];
        }
        __syncthreads();
        for (int u = tid; u < 64 * UPR; u += 64 * GEMM_WAVES) {
            const int lr = u / UPR, uc = u % UPR;
            const int row = m0 + pass * 64 + lr;
            if (row < p.M) {
                float v[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 t = *(const f32x4*)(ct + lr * CLD + swz(uc * 16 + 4 * q));
                    v[4 * q] = t[0]; v[4 * q + 1] = t[1]; v[4 * q + 2] = t[2]; v[4 * q + 3] = t[3];
                }
                epilogue16<EPI>(p, row, n0 + uc * 16, v, kz);
            }
        }
        __syncthreads();
    }
}

// The epilogue of a split-K tiled GEMM: sums the S partials of 16 columns of
// one row (one thread each) and applies epilogue EPI to them.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_finish_kernel(GemmParams p, int S) {
    const int units = p.N / 16;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)p.M * units) return;
    const int row = (int)(idx / units), col0 = (int)(idx % units) * 16;
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = 0.f;
    for (int z = 0; z < S; ++z) {
        const float* w = p.ws + ((size_t)z * p.M + row) * p.N + col0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 t = *(const f32x4*)(w + 4 * q);
            v[4 * q] += t[0]; v[4 * q + 1] += t[1]; v[4 * q + 2] += t[2]; v[4 * q + 3] += t[3];
        }
    }
    epilogue16<EPI>(p, row, col0, v);
}

// ---------------------------------------------------------------------------
// FP8 tiled GEMM for larger M (E4M3 weights with per-output-channel scales,
// per-token E4M3 activations): the structure of gemm_kernel with 128-deep
// stages and the 16x16x128 FP8 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4 with
// unit block scales, twice the bf16 rate). A (row-major E4M3 [M][K]) and W
// (16 x 128 fragments in two 1 KiB halves) reach LDS as 1 KiB DMA chunks;
// lane l of an MFMA operand holds row (or column) l%16 and inputs
// 32*(l/16) .. +31 of the 128, bytes 0-15 from the first chunk and 16-31
// from the second (the instruction pairs the two operands by lane group and
// byte, checked on the device). out = acc * a_scale[row] * w_scale[col].
// ---------------------------------------------------------------------------
constexpr int GEMM8_KT = 128;

template <int MT, int NT>
struct Gemm8Shape {
    static constexpr int ACH = MT / 8, BCH = NT / 16 * 2;        // 1 KiB DMA loads per stage (A: 8 rows each)
    static constexpr int STAGE = (ACH + BCH) * 1024;
    static constexpr int S = 147456 / STAGE >= 3 ? 3 : 147456 / STAGE;
    static constexpr int LA = (ACH + GEMM_WAVES - 1) / GEMM_WAVES;  // DMA loads per wave and stage
    static constexpr int LB = (BCH + GEMM_WAVES - 1) / GEMM_WAVES;
    static constexpr int LPW = LA + LB;
    static_assert(S >= 2, "tile too large for two LDS stages");
};

// Chunk permutation of an FP8 A row (128 bytes, 8 chunks of 16): chunk c of
// row r sits at c ^ a8_swz(r). Each lane reads chunks 2 (l / 16) and
// 2 (l / 16) + 1 of row l % 16; with the bf16 kernel's (r >> 1) those reads
// ran at half the LDS rate (two-way conflicts, measured); taking row bit 3
// into bit 0 makes both reads conflict-free.
VLA_DEV int a8_swz(int r) { return (r & 6) | ((r >> 3) & 1); }

VLA_DEV i32x8 frag32(const uint8_t* lo, const uint8_t* hi) {
    const u32x4 a = *(const u32x4*)lo, b = *(const u32x4*)hi;
    return (i32x8){(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

template <int MT, int NT, int EPI>
__global__ __launch_bounds__(64 * GEMM_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm8_kernel(GemmParams p) {
    using G = Gemm8Shape<MT, NT>;
    constexpr int S = G::S, ACH = G::ACH, BCH = G::BCH, LA = G::LA, LB = G::LB, LPW = G::LPW, STAGE = G::STAGE;
    constexpr int WGN = 4, WM = MT / 2, WN = NT / WGN, FM = WM / 16, FN = WN / 16;
    static_assert(FM >= 1 && FN >= 1, "tile smaller than the wave grid");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[S * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    // tile of this workgroup: as in gemm_kernel's data-parallel mapping
    const int ntn = p.N / NT;
    int mt_i, nt_i;
    if (p.tile_map == 1) {
        const int w = blockIdx.x, s = w >> 3;
        mt_i = (w & 7) + 8 * (s / ntn);
        nt_i = s % ntn;
        if (mt_i * MT >= p.M) return;  // padding of the last group of 8 row tiles
    } else if (ntn % 8 == 0) {
        const int w = blockIdx.x, per = ntn / 8, s = w >> 3;
        mt_i = s / per;
        nt_i = (w & 7) * per + s % per;
    } else {
        mt_i = blockIdx.x / ntn;
        nt_i = blockIdx.x % ntn;
    }
    const int m0 = mt_i * MT, n0 = nt_i * NT;
    // split K (gridDim.y > 1, EPI_PARTIAL): inputs [kz * kw, (kz + 1) * kw)
    const int kz = blockIdx.y, kt0 = kz * (p.kw / GEMM8_KT);
    const int nk = p.kw / GEMM8_KT, Kt = p.K / GEMM8_KT;
    const uint32_t lbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
    const uint8_t* A = (const uint8_t*)p.A + (size_t)kt0 * GEMM8_KT;

    // A in the stage as MT rows of 128 bytes (128 inputs), chunks permuted by
    // a8_swz: load j fills rows 8j .. 8j + 7 from whole 128-byte lines (rows
    // past M read row M-1, never stored); chunk c of B = half c%2 of the
    // fragment of column block c/2
    const uint8_t* asrc[LA];
    uint32_t adst[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int j = (wave * LA + i) % ACH, r = j * 8 + (lane >> 3);
        const int c = (lane & 7) ^ a8_swz(r & 15);
        const int row = min(m0 + r, p.M - 1);
        asrc[i] = A + (size_t)row * p.lda + c * 16;
        adst[i] = (uint32_t)j * 1024;
    }
    const uint8_t* bsrc[LB];
    uint32_t bdst[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int c = (wave * LB + i) % BCH;
        bsrc[i] = (const uint8_t*)p.W + ((size_t)(n0 / 16 + c / 2) * Kt + kt0) * 2048 + (c % 2) * 1024 + lane * 16;
        bdst[i] = (uint32_t)(ACH + c) * 1024;
    }
    // stage kt into ring slot kt % S; past the last stage the loads repeat it
    auto issue = [&](int kt_raw) {
        const uint32_t sb = lbase + (uint32_t)((kt_raw % S) * STAGE);
        const int kt = min(kt_raw, nk - 1);
#pragma unroll
        for (int i = 0; i < LA; ++i) lds_dma16(asrc[i] + (size_t)kt * GEMM8_KT, sb + adst[i]);
#pragma unroll
        for (int i = 0; i < LB; ++i) lds_dma16(bsrc[i] + (size_t)kt * 2048, sb + bdst[i]);
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < S; ++s) issue(s);
    vm_wait<(S - 1) * LPW>();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const uint8_t* st = lds + (kt % S) * STAGE;
        // the wave's B fragments of the stage, then its A fragments one row
        // block at a time, the next one read while the current multiplies;
        // lane l takes row l % 16 of the block, bytes 32 (l / 16) .. + 31
        // (chunks a_lo, a_lo + 1, swizzled)
        i32x8 bf[FN], af[2];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int cb = 2 * (wn * FN + fn);
            bf[fn] = frag32(st + (ACH + cb) * 1024 + lane * 16, st + (ACH + cb + 1) * 1024 + lane * 16);
        }
        const uint8_t* arow = st + (wm * FM * 16 + (lane & 15)) * 128;
        const int a_lo = ((2 * (lane >> 4)) ^ a8_swz(lane & 15)) << 4;
        const int a_hi = ((2 * (lane >> 4) + 1) ^ a8_swz(lane & 15)) << 4;
        af[0] = frag32(arow + a_lo, arow + a_hi);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            if (fm + 1 < FM) af[(fm + 1) & 1] = frag32(arow + (fm + 1) * 2048 + a_lo, arow + (fm + 1) * 2048 + a_hi);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[fm & 1], bf[fn], acc[fm][fn], 0, 0,
                                                                              0, 127, 0, 127);
            __builtin_amdgcn_sched_barrier(0);
        }
        // stage kt+1 landed (this wave's loads), then every wave's loads
        // landed and every wave is done with stage kt's slot
        vm_wait<(S - 2) * LPW>();
        __syncthreads();
        issue(kt + S);
    }
    vm_wait<0>();      // the repeated tail loads land before the LDS is reused
    __syncthreads();

    if constexpr (EPI == EPI_SWIGLU) {
        static_assert(MT * (NT + 16) <= S * STAGE, "SwiGLU output tile does not fit the ring");
        float wsc[FN], asc[FM][4];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) wsc[fn] = p.wscale[n0 + wn * WN + fn * 16 + (lane & 15)];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                asc[fm][r] = p.ascale[min(m0 + wm * WM + fm * 16 + 4 * (lane >> 4) + r, p.M - 1)];
        swiglu_epilogue_tile<MT, NT, FM, FN>(p, lds, m0, n0, wm, wn, lane, tid, [&](int fm, int fn, int r) {
            return acc[fm][fn][r] * wsc[fn] * asc[fm][r];
        });
        return;
    }

    // epilogue through LDS as in gemm_kernel, with the row and column scales
    constexpr int CLD = NT + 4;
    constexpr int PPW = FM / 4;
    constexpr int UPR = NT / 16;
    static_assert(FM % 4 == 0 && 64 * CLD * 4 <= S * STAGE, "epilogue pass does not fit the ring");
    float* ct = (float*)lds;
    auto swz = [](int col) { return col ^ ((((col >> 6) * (256 / NT)) & 3) << 2); };  // as in gemm_kernel
    float wsc[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) wsc[fn] = p.wscale[n0 + wn * WN + fn * 16 + (lane & 15)];
#pragma unroll
    for (int pass = 0; pass < MT / 64; ++pass) {
        if (wm == pass / PPW) {
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        ct[(f * 16 + 4 * (lane >> 4) + r) * CLD + swz(wn * WN + fn * 16 + (lane & 15))] =
                            acc[(pass % PPW) * 4 + f][fn][r] * wsc[fn];
        }
        __syncthreads();
        for (int u = tid; u < 64 * UPR; u += 64 * GEMM_WAVES) {
            const int lr = u / UPR, uc = u % UPR;
            const int row = m0 + pass * 64 + lr;
            if (row < p.M) {
                const float as = p.ascale[row];
                float v[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 t = *(const f32x4*)(ct + lr * CLD + swz(uc * 16 + 4 * q));
                    v[4 * q] = t[0] * as; v[4 * q + 1] = t[1] * as; v[4 * q + 2] = t[2] * as; v[4 * q + 3] = t[3] * as;
                }
                epilogue16<EPI>(p, row, n0 + uc * 16, v, kz);
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Grouped-query attention, no mask, scale 1/sqrt(d_h), online softmax, for
// few query rows (batch 1). Workgroup = (16 query rows of one KV group, group
// g, request b); the G query heads of a group are packed: group row =
// head_in_group*T + token, so the workgroup's rows are one contiguous run of
// q, loaded once into LDS. Its AT_WAVES waves take interleaved 32-key blocks
// of the layer's concatenated K/V straight from the cache (fragment order:
// 1 KiB loads), prefetch their next block, keep their own running max / sum
// / output, and merge them through LDS at the end.
// ---------------------------------------------------------------------------
struct AttnParams {
    const uint16_t* q;      // [B, nq, T, dh]
    const uint16_t* kcat;
    const uint16_t* vcat;
    uint16_t* o;            // [B*T, nq*dh] (A-fragment order when ofrag)
    KVLayout kv;
    int layer, S, T, nq;
    int ofrag;
    float scale_log2;       // log2(e)/sqrt(dh)
    int P;                  // prefix keys per request (the first valid[b] of them count)
    const int* pvalid;      // [B] valid prefix lengths of this call
    int pf_slices;          // attn_kernel: grid z-slices past the requests that prefetch (L2Prefetch)
    L2Prefetch pf;
};

// The running maximum of a query moves only when a block's maximum exceeds it
// by more than ATT_SLACK (log2 units), so most blocks skip the rescale; the
// unnormalised weights stay below 2^ATT_SLACK, well inside bf16 and fp32.
constexpr float ATT_SLACK = 8.0f;
constexpr int ATT_PF_SLEEPS = 3;   // prefetch slices of attn_kernel: s_sleep(16) rounds before their loads

template <int DH, int AT_WAVES>
__global__ __launch_bounds__(AT_WAVES * 64) void attn_kernel(AttnParams p) {
    // the waves' partial outputs (lane rows padded by 4 floats: a 16-byte read
    // of 16 consecutive lanes meets 64 distinct banks) and per-query maxima
    // and total weights
    __shared__ __attribute__((aligned(16))) float Om[AT_WAVES][64][DH / 16 * 4 + 4];
    __shared__ __attribute__((aligned(16))) float Ml[AT_WAVES][2][16];
    __shared__ __attribute__((aligned(16))) uint8_t Qs[16 * DH * 2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = blockIdx.y, b = blockIdx.z;
    const int nb = gridDim.z - p.pf_slices;
    if (b >= nb) {  // slices past the requests prefetch the next GEMMs' weights
        // after ~1.3 us (3 x 1024 clocks asleep), so that the attention
        // workgroups' own first loads are not queued behind the weight
        // stream (batch-1 call 13.80 -> 13.53 ms; longer delays cost more
        // than they gain)
#pragma unroll
        for (int i = 0; i < ATT_PF_SLEEPS; ++i) __builtin_amdgcn_s_sleep(16);
        const int per_slice = gridDim.x * gridDim.y;
        const int lin = per_slice * b + gridDim.x * g + blockIdx.x;
        int xcd, rank, per_xcd;
        prefetch_rank(lin, per_slice * nb, per_slice * p.pf_slices, &xcd, &rank, &per_xcd);
        l2_prefetch(p.pf, xcd, rank, per_xcd, AT_WAVES * 64, tid);
        return;
    }
    const int G = p.nq / p.kv.nkv;
    const int rows_total = G * p.T;
    const int r0 = blockIdx.x * 16;
    const int nblk = p.kv.S_pad / 32;
    const size_t base = p.kv.base(b, p.layer, g);
    const uint16_t* K = p.kcat + base;
    const uint16_t* V = p.vcat + base;
    const int pvb = p.pvalid[b];  // prefix keys past this are padding

    // the workgroup's 16 query rows are contiguous in q (rows of a KV group
    // are head-major, heads consecutive): one 16-byte chunk per thread into
    // LDS, chunk c of row r at c ^ qswz(r) so the fragment reads below (16
    // rows, one chunk column) meet distinct banks
    constexpr int QCH = DH / 8;  // 16-byte chunks per row
    static_assert(16 * QCH <= AT_WAVES * 64, "one query chunk per thread");
    auto qswz = [](int r) { return (DH == 128 ? r : r >> 1) & (QCH - 1); };
    u32x4 qv = (u32x4){0u, 0u, 0u, 0u};
    const int qr = tid / QCH, qc = tid % QCH;
    if (tid < 16 * QCH && r0 + qr < rows_total)
        qv = *(const u32x4*)(p.q + ((size_t)(b * p.nq + g * G) * p.T + r0 + qr) * DH + qc * 8);

    // scores transposed as in attn_rows_kernel: lane l holds, for its query
    // l % 16, keys 8 (l / 16) + j of a block; mrow / lrow are that query's
    // running maximum and this lane's partial sum; oacc rows are the queries
    // 4 (l / 16) + r
    float mrow = -1e30f, lrow = 0.f;  // finite start: an all-masked block adds weight 0, never NaN
    f32x4 oacc[DH / 16];
#pragma unroll
    for (int dn = 0; dn < DH / 16; ++dn) oacc[dn] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // K and V blocks are stored as MFMA fragments: every load is 1 KiB contiguous
    bf16x8 kf[2][DH / 32], vf[DH / 16], kf_n[2][DH / 32], vf_n[DH / 16];
    auto load_kv = [&](int kb, bf16x8 (*kd)[DH / 32], bf16x8* vd) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int ks = 0; ks < DH / 32; ++ks)
                kd[sb][ks] = *(const bf16x8*)(K + (size_t)kb * 32 * DH + ((size_t)(sb * (DH / 32) + ks) * 64 + lane) * 8);
#pragma unroll
        for (int dn = 0; dn < DH / 16; ++dn)
            vd[dn] = *(const bf16x8*)(V + (size_t)kb * 32 * DH + ((size_t)dn * 64 + lane) * 8);
    };
    if (wave < nblk) load_kv(wave, kf, vf);
    if (tid < 16 * QCH) *(u32x4*)(&Qs[qr * DH * 2 + ((qc ^ qswz(qr)) << 4)]) = qv;
    __syncthreads();
    bf16x8 qf[DH / 32];
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks)
        qf[ks] = *(const bf16x8*)(&Qs[(lane & 15) * DH * 2 + (((ks * 4 + (lane >> 4)) ^ qswz(lane & 15)) << 4)]);
    for (int kb = wave; kb < nblk; kb += AT_WAVES) {
        if (kb + AT_WAVES < nblk) load_kv(kb + AT_WAVES, kf_n, vf_n);   // next block of this wave, in flight
        // s[sb][r]: query lane & 15 against key 8 (lane / 16) + 4 sb + r
        f32x4 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            s[sb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DH / 32; ++ks) s[sb] = mfma_16x16x32(kf[sb][ks], qf[ks], s[sb]);
        }
        // every key of the block real (a uniform test): no per-key mask
        const bool whole = (kb * 32 + 32 <= pvb) || (kb * 32 >= p.P && kb * 32 + 32 <= p.S);
        float v[8], lmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[j] = s[j >> 2][j & 3] * p.scale_log2;
            if (!whole) {  // a block with padded prefix keys or keys past P + T
                const int key = kb * 32 + 8 * (lane >> 4) + j;
                if (key >= p.S || (key < p.P && key >= pvb)) v[j] = -INFINITY;
            }
            lmax = fmaxf(lmax, v[j]);
        }
        if (__builtin_amdgcn_ballot_w64(lmax > mrow + ATT_SLACK) != 0) {  // uniform: move the maxima, rescale
            float bm = fmaxf(lmax, __shfl_xor(lmax, 16, 64));  // over the query's four lanes
            bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
            const float mnew = fmaxf(mrow, bm);
            if (kb != wave) {  // (the wave's first block: oacc and lrow are still zero)
                const float alpha = attn_exp2(mrow - mnew);
                lrow *= alpha;
#pragma unroll
                for (int r = 0; r < 4; ++r) {  // oacc row r is the query 4 (l / 16) + r
                    const float ar = __shfl(alpha, 4 * (lane >> 4) + r, 64);
#pragma unroll
                    for (int dn = 0; dn < DH / 16; ++dn) oacc[dn][r] *= ar;
                }
            }
            mrow = mnew;
        }
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            e[j] = attn_exp2(v[j] - mrow);
            lrow += e[j];
        }
        u32x4 pw;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) pw[q2] = pack_bf16x2(e[2 * q2], e[2 * q2 + 1]);
        const bf16x8 pa = __builtin_bit_cast(bf16x8, pw);  // the PV A operand: keys 8 (l / 16) + j
#pragma unroll
        for (int dn = 0; dn < DH / 16; ++dn) oacc[dn] = mfma_16x16x32(pa, vf[dn], oacc[dn]);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int ks = 0; ks < DH / 32; ++ks) kf[sb][ks] = kf_n[sb][ks];
#pragma unroll
        for (int dn = 0; dn < DH / 16; ++dn) vf[dn] = vf_n[dn];
    }

    // merge the waves' partial results: lanes 0..15 publish their query's
    // maximum and total weight (over the query's four lanes); every lane then
    // reads those of its oacc rows 4 (l / 16) + r (16-lane broadcasts)
    {
        float lt = lrow + __shfl_xor(lrow, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        if (lane < 16) {
            Ml[wave][0][lane] = mrow;
            Ml[wave][1][lane] = lt;
        }
#pragma unroll
        for (int dn = 0; dn < DH / 16; ++dn) *(f32x4*)(&Om[wave][lane][dn * 4]) = oacc[dn];
    }
    __syncthreads();
    // wave w finishes d-column tiles dn = w, w + AT_WAVES, ...
    float mw[AT_WAVES][4], lw[AT_WAVES][4];
#pragma unroll
    for (int w = 0; w < AT_WAVES; ++w) {
        const f32x4 m4 = *(const f32x4*)(&Ml[w][0][4 * (lane >> 4)]);
        const f32x4 l4 = *(const f32x4*)(&Ml[w][1][4 * (lane >> 4)]);
#pragma unroll
        for (int r = 0; r < 4; ++r) { mw[w][r] = m4[r]; lw[w][r] = l4[r]; }
    }
    // per row: the waves' weights exp2(m_w - M) with 1 / L folded in (the
    // total weight L >= 1: the row's maximum key contributes 1)
    float scale[AT_WAVES][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float M = mw[0][r];
#pragma unroll
        for (int w = 1; w < AT_WAVES; ++w) M = fmaxf(M, mw[w][r]);
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < AT_WAVES; ++w) {
            scale[w][r] = attn_exp2(mw[w][r] - M);
            L += scale[w][r] * lw[w][r];
        }
        const float inv = __builtin_amdgcn_rcpf(L);
#pragma unroll
        for (int w = 0; w < AT_WAVES; ++w) scale[w][r] *= inv;
    }
    // (head in group, token) of the lane's first row; the next three follow
    const int row0 = r0 + 4 * (lane >> 4);
    const int hh0 = row0 / p.T, i0 = row0 - hh0 * p.T;
    for (int dn = wave; dn < DH / 16; dn += AT_WAVES) {
        f32x4 o = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < AT_WAVES; ++w) {
            f32x4 t = *(const f32x4*)(&Om[w][lane][dn * 4]);
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] += scale[w][r] * t[r];
        }
        int hh = hh0, i = i0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (row0 + r < rows_total)
                p.o[act_index(b * p.T + i, (g * G + hh) * DH + dn * 16 + (lane & 15), p.nq * DH, p.ofrag)] =
                    f32_to_bf16(o[r]);
            if (++i == p.T) { i = 0; ++hh; }
        }
    }
}

// ---------------------------------------------------------------------------
// The same attention for many query rows (large batches): a workgroup of AW
// waves takes AW * 16 * RT query rows of one (request, KV group), each wave
// owning RT 16-row tiles over the whole key range, and every 32-key K/V block
// is staged once per workgroup through LDS. K/V is then read from L2 once per
// workgroup, each K or V fragment read from LDS serves RT tiles, and the
// waves never merge. The blocks arrive by global->LDS DMA into a ring of
// ATT_RING slots, ATT_RING - 1 blocks ahead of the one being multiplied, so
// the load latency of a block is hidden behind the blocks before it (with
// one block in flight, each block waited out most of a memory round trip).
// The running maximum moves only when a block's maximum exceeds it by more
// than ATT_SLACK (log2 units), so most blocks skip the rescale of the
// accumulators and its exponentials; the unnormalised weights stay below
// 2^ATT_SLACK, well inside bf16 and fp32 range.
// The scores are computed transposed (K as the MFMA's A operand, Q as B), so
// lane l holds, for the query l % 16 of each of its tiles, the scores of the
// keys 8 (l / 16) + j, j = 0..7, of a block: the K fragment of sub-block sb
// takes key rows 8 ((l % 16) / 4) + 4 sb + l % 4. Those eight exponentials
// are then directly the A operand of the PV MFMA (no trip through LDS), the
// row sum stays a per-lane partial until the end, and the row maximum needs
// the other three lanes of the query only when some lane's block maximum
// exceeds the running maximum by ATT_SLACK.
// LDS: K and V blocks copied as they are stored (MFMA fragments, 1 KiB each),
// so every fragment read is 64 lanes x 16 contiguous bytes.
// CAUSAL (prefix self-attention, keys = the T tokens themselves, P = 0):
// query token i sees keys 0..i. The workgroup stops after the block holding
// its last row's token, and only blocks that reach past the smallest token of
// a wave's rows are masked per key.
// ---------------------------------------------------------------------------

constexpr int ATT_RING = 4;   // K/V block slots of attn_rows_kernel

template <int DH, int RT, bool CAUSAL = false, int AW = 4>
__global__ __launch_bounds__(64 * AW) void attn_rows_kernel(AttnParams p) {
    constexpr int BLK = 32 * DH * 2;             // one 32-key block of K (or V), bytes
    constexpr int NCH = 2 * BLK / 1024;          // 1 KiB DMA chunks of a K + V block
    constexpr int LPW = (NCH + AW - 1) / AW;     // DMA loads per wave and block
    constexpr int WROWS = AW * 16 * RT;          // query rows of a workgroup
    static_assert(DH == 64 || DH == 128, "head_dim 64 or 128");
    // slot s: K block at s * 2 BLK, V block after it
    __shared__ __attribute__((aligned(1024))) uint8_t ring[ATT_RING * 2 * BLK];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = p.nq / p.kv.nkv;
    const int rows_total = G * p.T;
    const int g = blockIdx.y, b = blockIdx.z;
    const int r0 = blockIdx.x * WROWS + wave * 16 * RT;
    int nblk = p.kv.S_pad / 32;
    // causal: token of this lane's query in each tile, the smallest token of
    // the wave's rows (0 when they span two heads), and the last block any row
    // of the workgroup needs (rows are head-major: row = head_in_group * T + token)
    int tok[RT], tmin = 0;
    if constexpr (CAUSAL) {
        const int R0 = blockIdx.x * WROWS, R1 = min(R0 + WROWS, rows_total) - 1;
        const int tmax = R0 / p.T == R1 / p.T ? R1 % p.T : p.T - 1;
        nblk = min(nblk, tmax / 32 + 1);
        const int w1 = min(r0 + 16 * RT, rows_total) - 1;
        tmin = r0 <= w1 && r0 / p.T == w1 / p.T ? r0 % p.T : 0;
#pragma unroll
        for (int t = 0; t < RT; ++t) tok[t] = (r0 + t * 16 + (lane & 15)) % p.T;
    }
    const size_t base = p.kv.base(b, p.layer, g);
    const uint8_t* K = (const uint8_t*)(p.kcat + base);
    const uint8_t* V = (const uint8_t*)(p.vcat + base);
    const int pvb = p.pvalid[b];  // prefix keys past this are padding
    const uint32_t rbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)ring;

    // Block kb into slot kb % ATT_RING: chunk j < NCH / 2 of K, the rest of V
    // (a wave with fewer chunks than loads repeats one: same bytes, same
    // place). Past the last block the loads repeat it into a slot no later
    // block uses, so every wave always has the same loads in flight.
    auto issue = [&](int kb_raw) {
        const int kb = min(kb_raw, nblk - 1);
        const uint32_t sb = rbase + (uint32_t)((kb_raw % ATT_RING) * 2 * BLK);
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int j = (wave * LPW + i) % NCH;
            const uint8_t* src = j < NCH / 2 ? K + (size_t)kb * BLK + j * 1024 : V + (size_t)kb * BLK + (j - NCH / 2) * 1024;
            lds_dma16(src + lane * 16, sb + (uint32_t)(j * 1024));
        }
    };
#pragma unroll
    for (int kb = 0; kb < ATT_RING - 1; ++kb) issue(kb);

    bf16x8 qf[RT][DH / 32];
    {
        const uint16_t* qg = p.q + (size_t)(b * p.nq + g * G) * p.T * DH;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int row = r0 + t * 16 + (lane & 15);
            const int rowc = min(row, rows_total - 1);
#pragma unroll
            for (int ks = 0; ks < DH / 32; ++ks) {
                const bf16x8 v = *(const bf16x8*)(qg + (size_t)rowc * DH + ks * 32 + 8 * (lane >> 4));
                qf[t][ks] = row < rows_total ? v : (bf16x8){};
            }
        }
    }
    // The compiler counts only its own loads when it places waits: were the
    // first use of q inside the loop, its wait would also cover the ring
    // loads issued there. Taking q here (behind the first ring blocks, which
    // are older and land first) keeps every later wait on the ring explicit.
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int ks = 0; ks < DH / 32; ++ks) asm volatile("" ::"v"(qf[t][ks]));

    // per lane: the running maximum and the partial sum (over this lane's
    // keys) of its query in each tile; oacc rows are the queries 4 (l / 16) + r
    float mrow[RT], lrow[RT];
    f32x4 oacc[RT][DH / 16];
    // running max starts finite: a block whose keys are all masked (padding)
    // then leaves m finite and adds weight 0, where -inf would give
    // exp2(-inf - -inf) = NaN
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        mrow[t] = -1e30f;
        lrow[t] = 0.f;
#pragma unroll
        for (int dn = 0; dn < DH / 16; ++dn) oacc[t][dn] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }

    for (int kb = 0; kb < nblk; ++kb) {
        // block kb landed (this wave's loads), then every wave's loads landed
        // and every wave is done with block kb - 1, whose slot then takes
        // block kb - 1 + ATT_RING
        vm_wait<(ATT_RING - 2) * LPW>();
        __syncthreads();
        issue(kb - 1 + ATT_RING);
        const uint8_t* Ks = ring + (kb % ATT_RING) * 2 * BLK;
        const uint8_t* Vs = Ks + BLK;
        // s[t][sb][r]: query (tile t, lane & 15) against key 8 (lane / 16) + 4 sb + r
        f32x4 s[RT][2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int t = 0; t < RT; ++t) s[t][sb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DH / 32; ++ks) {
                const bf16x8 kf = *(const bf16x8*)(Ks + ((sb * (DH / 32) + ks) * 64 + lane) * 16);
#pragma unroll
                for (int t = 0; t < RT; ++t) s[t][sb] = mfma_16x16x32(kf, qf[t][ks], s[t][sb]);
            }
        }
        // every key of the block real (a uniform test): no per-key mask
        bool whole = (kb * 32 + 32 <= pvb) || (kb * 32 >= p.P && kb * 32 + 32 <= p.S);
        if constexpr (CAUSAL) whole = whole && kb * 32 + 31 <= tmin;
        float v[RT][8], lmax[RT];
        bool grow = false;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            lmax[t] = -INFINITY;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v[t][j] = s[t][j >> 2][j & 3] * p.scale_log2;
                if (!whole) {  // a block with padded prefix keys or keys past P + T
                    const int key = kb * 32 + 8 * (lane >> 4) + j;
                    if (key >= p.S || (key < p.P && key >= pvb)) v[t][j] = -INFINITY;
                    if constexpr (CAUSAL) {
                        if (key > tok[t]) v[t][j] = -INFINITY;
                    }
                }
                lmax[t] = fmaxf(lmax[t], v[t][j]);
            }
            grow |= lmax[t] > mrow[t] + ATT_SLACK;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // uniform: move the maxima, rescale
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                // the query's block maximum over its four lanes (l, l ^ 16, l ^ 32, l ^ 48)
                float bm = fmaxf(lmax[t], __shfl_xor(lmax[t], 16, 64));
                bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
                const float mnew = fmaxf(mrow[t], bm);
                const float alpha = attn_exp2(mrow[t] - mnew);
                lrow[t] *= alpha;
                mrow[t] = mnew;
                // oacc row r is the query 4 (l / 16) + r: its factor from that query's lane
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ar = __shfl(alpha, 4 * (lane >> 4) + r, 64);
#pragma unroll
                    for (int dn = 0; dn < DH / 16; ++dn) oacc[t][dn][r] *= ar;
                }
            }
        }
        // the eight weights of lane l are the PV A operand: query l % 16, keys
        // 8 (l / 16) + j, which is the row order of V's PV fragments
        bf16x8 pa[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            float e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                e[j] = attn_exp2(v[t][j] - mrow[t]);
                lrow[t] += e[j];
            }
            u32x4 w;
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) w[q2] = pack_bf16x2(e[2 * q2], e[2 * q2 + 1]);
            pa[t] = __builtin_bit_cast(bf16x8, w);
        }
#pragma unroll
        for (int dn = 0; dn < DH / 16; ++dn) {
            const bf16x8 vf = *(const bf16x8*)(Vs + (dn * 64 + lane) * 16);
#pragma unroll
            for (int t = 0; t < RT; ++t) oacc[t][dn] = mfma_16x16x32(pa[t], vf, oacc[t][dn]);
        }
    }
    vm_wait<0>();   // the repeated tail loads land before the workgroup ends

#pragma unroll
    for (int t = 0; t < RT; ++t) {
        // the query's total weight over its four lanes
        float lt = lrow[t] + __shfl_xor(lrow[t], 16, 64);
        lt += __shfl_xor(lt, 32, 64);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = r0 + t * 16 + 4 * (lane >> 4) + r;
            const float inv = 1.0f / __shfl(lt, 4 * (lane >> 4) + r, 64);
            if (row < rows_total) {
                const int hh = row / p.T, i = row % p.T;
#pragma unroll
                for (int dn = 0; dn < DH / 16; ++dn)
                    p.o[act_index(b * p.T + i, (g * G + hh) * DH + dn * 16 + (lane & 15), p.nq * DH, p.ofrag)] =
                        f32_to_bf16(oacc[t][dn][r] * inv);
            }
        }
    }
}
