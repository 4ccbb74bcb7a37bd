// HIP kernels of the action-expert denoise loop (gfx950).
//
// Layout conventions used by every kernel:
//   * token rows r = b*T + i (request b, chunk token i); M = B*T valid rows;
//     GEMM operand loads of rows >= M read zeros instead of memory.
//   * packed weights: fragments of 16 output rows x 32 inputs, 1 KiB each for
//     bf16 (512 B for E4M3), ordered [n/16][k/32][lane][8]; lane l holds
//     rows n = l%16 at inputs 8*(l/16)..+7, i.e. exactly the B operand of one
//     16x16x32 MFMA, so one wave reads a fragment as one contiguous 1 KiB.
//   * the modulation table holds, per (step k, request b), (6L+2) chunks of H
//     floats: layer l uses chunks 6l..6l+5 = scale1, shift1, gate1, scale2,
//     shift2, gate2; the final norm uses chunks 6L, 6L+1 = scale, shift.
#pragma once

#include "common.h"

// ---------------------------------------------------------------------------
// Call-argument refresh (one thread, launched before each graph replay)
// ---------------------------------------------------------------------------
__global__ void set_args_kernel(ArgBlock* ab, const uint16_t* pk, const uint16_t* pv,
                                const float* noise, const float* ts, float* out, const int* pvalid) {
    ab->prefix_k = pk;
    ab->prefix_v = pv;
    ab->noise = noise;
    ab->t_schedule = ts;
    ab->out = out;
    ab->prefix_valid = pvalid;
}

// ---------------------------------------------------------------------------
// Weight packing (create time)
// ---------------------------------------------------------------------------
// Source rows of one linear [R, K] (bf16 or bytes) are scattered into the
// fragment layout of a packed matrix with Kf = K/32 fragment columns.
// row_mode 0: dst row = dst_off + src row
// row_mode 1: rotate-half pairs made adjacent: within each head of `dh` rows,
//             src row m -> 2m and m + dh/2 -> 2m+1 (then + dst_off)
// row_mode 2: dst row = 2*src row + parity (gate/up interleave)
__global__ void pack_weight_kernel(const uint8_t* __restrict__ src, int R, int K, int elem_bytes,
                                   uint8_t* __restrict__ dst, int row_mode, int dst_off, int dh,
                                   int parity, int layout) {
    const int chunks_per_row = K / 8;  // 8 inputs per chunk
    long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)R * chunks_per_row) return;
    int r = (int)(idx / chunks_per_row);
    int kc = (int)(idx % chunks_per_row);
    int drow;
    if (row_mode == 1) {
        int head = r / dh, p = r % dh, half = dh / 2;
        int local = (p < half) ? 2 * p : 2 * (p - half) + 1;
        drow = dst_off + head * dh + local;
    } else if (row_mode == 2) {
        drow = 2 * r + parity;
    } else {
        drow = dst_off + r;
    }
    int k = kc * 8;
    size_t dst_off_b;
    if (layout == 2) {
        // E2M1 codes (two per byte, element 2j low): the 16 x 32 fragments of
        // layout 0 with 4 bytes (8 codes) per lane
        const int Kf = K / 32, lane = (drow % 16) + 16 * ((k % 32) / 8);
        const size_t frag = (size_t)(drow / 16) * Kf + k / 32;
        *(uint32_t*)(dst + (frag * 64 + lane) * 4) = *(const uint32_t*)(src + ((size_t)r * K + k) / 2);
        return;
    }
    if (layout == 1) {
        // E4M3 fragments of the 16x16x128 FP8 MFMA: 16 rows x 128 inputs, two
        // 1 KiB halves; lane l = row%16 + 16*(w/32) holds inputs w%32 of the
        // 128 (w = k%128), bytes 0-15 in half 0 and 16-31 in half 1
        const int Kq = K / 128, w = k % 128, lane = (drow % 16) + 16 * (w / 32), b = w % 32;
        const size_t frag = (size_t)(drow / 16) * Kq + k / 128;
        dst_off_b = ((frag * 2 + b / 16) * 64 + lane) * 16 + (b % 16);
    } else {
        int Kf = K / 32;
        int nt = drow / 16, lane = (drow % 16) + 16 * ((k % 32) / 8), kt = k / 32;
        size_t frag = (size_t)nt * Kf + kt;
        dst_off_b = (frag * 64 + lane) * 8 * elem_bytes;
    }
    size_t src_off_b = ((size_t)r * K + k) * elem_bytes;
    if (elem_bytes == 2) {
        *(u32x4*)(dst + dst_off_b) = *(const u32x4*)(src + src_off_b);
    } else {
        *(u32x2*)(dst + dst_off_b) = *(const u32x2*)(src + src_off_b);
    }
}

// ---------------------------------------------------------------------------
// Per-token E4M3 activations: row r of a bf16 [M][K] matrix (K a multiple of
// 8) becomes codes q = RNE(x * 448 / max|x_r|) with the row scale
// max|x_r| / 448 (1 for an all-zero row), so x ~ q * scale. The first 16384
// inputs of a row stay in registers between the maximum and the conversion;
// inputs past them (longer rows) are read a second time.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ src, int K,
                                                         uint8_t* __restrict__ dst, float* __restrict__ scale) {
    __shared__ float red[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    const uint16_t* sr = src + (size_t)row * K;
    float v[8][8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = (tid + 256 * i) * 8;
        if (c < K) {
            const u32x4 w = *(const u32x4*)(sr + c);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[i][2 * j] = __uint_as_float(w[j] << 16);
                v[i][2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
                amax = fmaxf(amax, fmaxf(fabsf(v[i][2 * j]), fabsf(v[i][2 * j + 1])));
            }
        }
    }
    for (int c = (tid + 2048) * 8; c < K; c += 2048) {
        const u32x4 w = *(const u32x4*)(sr + c);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w[j] << 16)), fabsf(__uint_as_float(w[j] & 0xffff0000u))));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
    if (tid == 0) scale[row] = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = (tid + 256 * i) * 8;
        if (c < K) {
            u32x2 q;
            q[0] = f32x4_to_e4m3x4(v[i][0] * inv, v[i][1] * inv, v[i][2] * inv, v[i][3] * inv);
            q[1] = f32x4_to_e4m3x4(v[i][4] * inv, v[i][5] * inv, v[i][6] * inv, v[i][7] * inv);
            *(u32x2*)(dst + (size_t)row * K + c) = q;
        }
    }
    for (int c = (tid + 2048) * 8; c < K; c += 2048) {
        const u32x4 w = *(const u32x4*)(sr + c);
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(w[j] << 16) * inv;
            x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u) * inv;
        }
        u32x2 q;
        q[0] = f32x4_to_e4m3x4(x[0], x[1], x[2], x[3]);
        q[1] = f32x4_to_e4m3x4(x[4], x[5], x[6], x[7]);
        *(u32x2*)(dst + (size_t)row * K + c) = q;
    }
}

// The same per-token E4M3 conversion with one wave per row (four rows per
// 256-thread workgroup) for K <= 512 NC: the row stays in the wave's
// registers and its maximum is reduced within the wave (no LDS, no barrier),
// which suits many short rows better than a workgroup per row.
template <int NC>
__global__ __launch_bounds__(256) void quant_rows_wave_kernel(const uint16_t* __restrict__ src, int K, int M,
                                                              uint8_t* __restrict__ dst, float* __restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const uint16_t* sr = src + (size_t)row * K;
    float v[NC][8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = (lane + 64 * i) * 8;
        if (c < K) {
            const u32x4 w = *(const u32x4*)(sr + c);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[i][2 * j] = __uint_as_float(w[j] << 16);
                v[i][2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
                amax = fmaxf(amax, fmaxf(fabsf(v[i][2 * j]), fabsf(v[i][2 * j + 1])));
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
    if (lane == 0) scale[row] = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = (lane + 64 * i) * 8;
        if (c < K) {
            u32x2 q;
            q[0] = f32x4_to_e4m3x4(v[i][0] * inv, v[i][1] * inv, v[i][2] * inv, v[i][3] * inv);
            q[1] = f32x4_to_e4m3x4(v[i][4] * inv, v[i][5] * inv, v[i][6] * inv, v[i][7] * inv);
            *(u32x2*)(dst + (size_t)row * K + c) = q;
        }
    }
}

// cos/sin of the rotary angle (P + i) * theta^(-2m/d_h), i < T, m < d_h/2,
// evaluated in double precision once at create time.
// cos/sin of every absolute position 0..npos-1 (the chunk of request b sits
// at positions valid_b .. valid_b + T - 1): tab[pos][m], m < dh/2.
__global__ void rope_table_kernel(float2* tab, int npos, int dh, double theta) {
    int idx = blockIdx.x * blockDim.x + threadIdx.x;
    int half = dh / 2;
    if (idx >= npos * half) return;
    int pos = idx / half, m = idx % half;
    double ang = (double)pos * pow(theta, -2.0 * m / dh);
    tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

// Per call: each request's valid prefix length, clamped to [0, P], read by
// the QKV epilogues (RoPE position pvalid[b] + i) and the attention masks.
__global__ void varlen_setup_kernel(const ArgBlock* ab, int* pv_eff, int B, int P) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) pv_eff[b] = prefix_valid(ab, b, P);
}

// ---------------------------------------------------------------------------
// Prologue: time embedding and time MLP for every (step, request)
// ---------------------------------------------------------------------------
// e[row][j], row = k*B + b: sin(time_scale*t*w_j) for j < E/2, cos for the
// rest, w_j = 10000^(-j/(E/2)); computed in double from the fp32 time.
__global__ void time_embed_kernel(const ArgBlock* ab, const float* ts_direct, float* e, int N,
                                  int B, int E, double time_scale) {
    int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= N * B * E) return;
    const float* ts = ts_direct ? ts_direct : ab->t_schedule;
    int row = idx / E, j = idx % E;
    int k = row / B, b = row % B;
    int half = E / 2;
    int jj = j < half ? j : j - half;
    double t = (double)ts[b * (N + 1) + k];
    double w = exp(-log(10000.0) * (double)jj / (double)half);
    double arg = time_scale * t * w;
    e[idx] = (float)(j < half ? sin(arg) : cos(arg));
}

// out[row][n] = SiLU(sum_j W[n][j] in[row][j] + bias[n]) in fp32 (W bf16 [N, Kin]).
// One wave per output element group: lanes split the reduction.
__global__ void small_linear_silu_kernel(const float* __restrict__ in, const uint16_t* __restrict__ W,
                                         const float* __restrict__ bias, float* __restrict__ out_f32,
                                         uint16_t* __restrict__ out_bf16, int rows, int N, int Kin, int afrag) {
    int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    int lane = threadIdx.x & 63;
    if (wave >= rows * N) return;
    int row = wave / N, n = wave % N;
    const float* x = in + (size_t)row * Kin;
    const uint16_t* w = W + (size_t)n * Kin;
    float acc = 0.f;
    for (int j = lane; j < Kin; j += 64) acc += bf16_to_f32(w[j]) * x[j];
    acc = wave_sum(acc);
    if (lane == 0) {
        float v = silu_f(acc + bias[n]);
        if (out_f32) out_f32[(size_t)row * N + n] = v;
        if (out_bf16) out_bf16[act_index(row, n, N, afrag)] = f32_to_bf16(v);
    }
}

#include "kernels_layer.h"

// ---------------------------------------------------------------------------
// In-projection fused with the first AdaRMSNorm of layer 0, one workgroup
// (256 threads) per token row, H <= 2048:
//   h = x in_w^T + in_b   (fp32; in_w given transposed [A][H] so that the
//                          threads of a row read consecutive columns)
//   y = RMSNorm(h)(1 + scale) + shift  -> bf16
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void inproj_norm_kernel(const ArgBlock* ab, int first, const float* x_direct,
                                                          const uint16_t* __restrict__ WinT,
                                                          const float* __restrict__ bias, float* __restrict__ h,
                                                          uint16_t* __restrict__ y, const float* __restrict__ mod,
                                                          int scale_off, int shift_off, int M, int H, int A, int T,
                                                          int B, int step, int mod_ld, float eps, int afrag) {
    __shared__ float xs[128];
    __shared__ float red[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    const float* x = x_direct ? x_direct : (first ? ab->noise : ab->out);
    if (tid < A) xs[tid] = x[(size_t)row * A + tid];
    __syncthreads();
    float4 v[2];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = (tid + 256 * j) * 4;
        if (c < H) {
            float4 acc = *(const float4*)(bias + c);
#pragma unroll 8
            for (int a = 0; a < A; ++a) {
                const uint2 w = *(const uint2*)(WinT + (size_t)a * H + c);
                const float xa = xs[a];
                acc.x += xa * __uint_as_float(w.x << 16);
                acc.y += xa * __uint_as_float(w.x & 0xffff0000u);
                acc.z += xa * __uint_as_float(w.y << 16);
                acc.w += xa * __uint_as_float(w.y & 0xffff0000u);
            }
            v[j] = acc;
            *(float4*)(h + (size_t)row * H + c) = acc;
            ss += acc.x * acc.x + acc.y * acc.y + acc.z * acc.z + acc.w * acc.w;
        }
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
    const float* mr = mod + (size_t)(step * B + row / T) * mod_ld;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = (tid + 256 * j) * 4;
        if (c < H) {
            const float4 sc = *(const float4*)(mr + scale_off + c);
            const float4 sh = *(const float4*)(mr + shift_off + c);
            uint2 ob;
            ob.x = pack_bf16x2(v[j].x * inv * (1.f + sc.x) + sh.x, v[j].y * inv * (1.f + sc.y) + sh.y);
            ob.y = pack_bf16x2(v[j].z * inv * (1.f + sc.z) + sh.z, v[j].w * inv * (1.f + sc.w) + sh.w);
            *(uint2*)(y + act_index(row, c, H, afrag)) = ob;
        }
    }
}

// ---------------------------------------------------------------------------
// Out-projection + Euler update (all fp32):
//   v = yf out_w^T + out_b,  x_{k+1} = x_k + (t_{k+1} - t_k) v
// where yf is the final AdaRMSNorm output. Workgroup (256 threads) = one row
// x 16 outputs, H <= 2048: every load is issued before the first use, then
// the 16 dot products are reduced over the workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void outproj_euler_kernel(const ArgBlock* ab, int first,
                                                            const float* __restrict__ yf,
                                                            const uint16_t* __restrict__ Wout,
                                                            const float* __restrict__ bout, int M, int H, int A,
                                                            int T, int step, int N) {
    __shared__ float red[4][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.x, a0 = blockIdx.y * 16;
    const float* yr = yf + (size_t)row * H;
    float4 yv[2];
    uint2 w[16][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = (tid + 256 * j) * 4;
        yv[j] = c < H ? *(const float4*)(yr + c) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int o = 0; o < 16; ++o)
            w[o][j] = (c < H && a0 + o < A) ? *(const uint2*)(Wout + (size_t)(a0 + o) * H + c) : make_uint2(0u, 0u);
    }
    float acc[16];
#pragma unroll
    for (int o = 0; o < 16; ++o) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            s += yv[j].x * __uint_as_float(w[o][j].x << 16) + yv[j].y * __uint_as_float(w[o][j].x & 0xffff0000u) +
                 yv[j].z * __uint_as_float(w[o][j].y << 16) + yv[j].w * __uint_as_float(w[o][j].y & 0xffff0000u);
        acc[o] = wave_sum(s);
    }
    if (lane == 0) {
#pragma unroll
        for (int o = 0; o < 16; ++o) red[wave][o] = acc[o];
    }
    __syncthreads();
    if (tid < 16 && a0 + tid < A) {
        const float v = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
        const int b = row / T, a = a0 + tid;
        const float* ts = ab->t_schedule;
        const float dt = ts[b * (N + 1) + step + 1] - ts[b * (N + 1) + step];
        const float* xsrc = first ? ab->noise : ab->out;
        const size_t xi = (size_t)row * A + a;
        ab->out[xi] = xsrc[xi] + dt * (v + bout[a]);
    }
}

// Copy fp32 rows (test entry points).
__global__ void copy_f32_kernel(const float* src, float* dst, long n) {
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

// Zero n 16-byte words (clears scratch memory with a kernel, so that callers
// capturing the launches into a graph record no memset node).
__global__ void zero_u32x4_kernel(u32x4* dst, long n) {
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = (u32x4){0u, 0u, 0u, 0u};
}
