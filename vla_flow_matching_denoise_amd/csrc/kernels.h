// HIP kernels of the action-expert denoise loop (gfx950).
//
// Layout conventions used by every kernel:
//   * token rows r = b*T + i (request b, chunk token i); M = B*T valid rows,
//     activation buffers are allocated with a zero-filled row padding.
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
                                const float* noise, const float* ts, float* out) {
    ab->prefix_k = pk;
    ab->prefix_v = pv;
    ab->noise = noise;
    ab->t_schedule = ts;
    ab->out = out;
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
                                   int parity) {
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
    int Kf = K / 32;
    int nt = drow / 16, lane = (drow % 16) + 16 * ((k % 32) / 8), kt = k / 32;
    size_t frag = (size_t)nt * Kf + kt;
    size_t dst_off_b = (frag * 64 + lane) * 8 * elem_bytes;
    size_t src_off_b = ((size_t)r * K + k) * elem_bytes;
    if (elem_bytes == 2) {
        *(u32x4*)(dst + dst_off_b) = *(const u32x4*)(src + src_off_b);
    } else {
        *(u32x2*)(dst + dst_off_b) = *(const u32x2*)(src + src_off_b);
    }
}

// cos/sin of the rotary angle (P + i) * theta^(-2m/d_h), i < T, m < d_h/2,
// evaluated in double precision once at create time.
__global__ void rope_table_kernel(float2* tab, int T, int P, int dh, double theta) {
    int idx = blockIdx.x * blockDim.x + threadIdx.x;
    int half = dh / 2;
    if (idx >= T * half) return;
    int i = idx / half, m = idx % half;
    double ang = (double)(P + i) * pow(theta, -2.0 * m / dh);
    tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
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
                                         uint16_t* __restrict__ out_bf16, int rows, int N, int Kin) {
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
        if (out_bf16) out_bf16[(size_t)row * N + n] = f32_to_bf16(v);
    }
}

// ---------------------------------------------------------------------------
// AdaRMSNorm: y = h / sqrt(mean(h^2) + eps) * (1 + scale) + shift  -> bf16
// One wave per row; scale/shift are chunks of this (step, request)'s row of
// the modulation table.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void adarms_kernel(const float* __restrict__ h, uint16_t* __restrict__ y,
                                                     const float* __restrict__ mod, int M, int H, int T,
                                                     int B, int step, int mod_ld, int scale_off,
                                                     int shift_off, float eps) {
    int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    int lane = threadIdx.x & 63;
    if (row >= M) return;
    int b = row / T;
    const float* hr = h + (size_t)row * H;
    const float* mr = mod + (size_t)(step * B + b) * mod_ld;
    float ss = 0.f;
    for (int c = lane * 4; c < H; c += 256) {
        float4 v = *(const float4*)(hr + c);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    float inv = 1.0f / sqrtf(ss / (float)H + eps);
    for (int c = lane * 4; c < H; c += 256) {
        float4 v = *(const float4*)(hr + c);
        float4 sc = *(const float4*)(mr + scale_off + c);
        float4 sh = *(const float4*)(mr + shift_off + c);
        uint2 o;
        o.x = pack_bf16x2(v.x * inv * (1.f + sc.x) + sh.x, v.y * inv * (1.f + sc.y) + sh.y);
        o.y = pack_bf16x2(v.z * inv * (1.f + sc.z) + sh.z, v.w * inv * (1.f + sc.w) + sh.w);
        *(uint2*)(y + (size_t)row * H + c) = o;
    }
}

// ---------------------------------------------------------------------------
// GEMM: C[M, N] = A[M, K] (bf16, row-major) x W^T with W packed (bf16 or
// E4M3), fp32 accumulation on 16x16x32 MFMAs, and a fused epilogue.
// Tile MT x NT per workgroup (4 waves as 2x2), K staged through LDS 64 at a
// time with register double buffering. Optional split-K over gridDim.z: each
// split writes its fp32 partial tile, and the last split to arrive (per-tile
// counter) sums all partials in split order — deterministic — and runs the
// epilogue.
// ---------------------------------------------------------------------------
enum { EPI_BIAS_F32 = 0, EPI_RESID = 1, EPI_QKV_ROPE = 2, EPI_SWIGLU = 3 };

struct GemmParams {
    const uint16_t* A;   // [rows, lda] bf16
    int lda;
    const void* W;       // packed
    const float* wscale; // per packed row (E4M3), else null
    int M, N, K;         // valid rows; N % NT == 0; K % 64 == 0
    int kchunk;          // K per split (multiple of 64)
    int ksplit;
    float* ws;           // [ksplit][M][N] partials
    int* counters;       // per output tile, zero between launches
    // epilogue operands
    float* out_f32;      // EPI_BIAS_F32: [M][N] ; EPI_RESID: h [M][N]
    const float* bias;   // EPI_BIAS_F32
    const float* mod;    // EPI_RESID: gate chunk source
    int mod_ld, gate_off, step, B, T;
    uint16_t* q;         // EPI_QKV_ROPE outputs
    uint16_t* kn;
    uint16_t* vn;
    const float2* rope;  // [T][dh/2]
    int nq, nkv, dh;
    uint16_t* act;       // EPI_SWIGLU output [M][N/2]
};

template <int MT, int NT, bool W8, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
    constexpr int KT = 64;
    constexpr int WM = MT / 2, WN = NT / 2;
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int APAD = KT + 8;
    constexpr int A_CH = MT * KT / 8 / 256;               // 16-byte chunks per thread
    constexpr int WFRAG_BYTES = W8 ? 512 : 1024;
    constexpr int B_BYTES = (NT / 16) * (KT / 32) * WFRAG_BYTES;
    constexpr int B_CH = B_BYTES / 16 / 256 > 0 ? B_BYTES / 16 / 256 : 1;
    constexpr int B_THREADS = B_BYTES / 16;               // threads that load a B chunk
    static_assert(A_CH >= 1, "tile too small");

    __shared__ __attribute__((aligned(16))) uint16_t As[2][MT][APAD];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][B_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * MT, n0 = blockIdx.x * NT;
    const int kz = blockIdx.z;
    const int kbeg = kz * p.kchunk;
    const int kend = min(p.K, kbeg + p.kchunk);
    const int nk = (kend - kbeg) / KT;
    const int Kf = p.K / 32;

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    u32x4 ra[A_CH], rb[B_CH];

    auto load_tile = [&](int kt) {
        const int k0 = kbeg + kt * KT;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            int c = tid + i * 256;
            int row = c / (KT / 8), c8 = c % (KT / 8);
            int grow = m0 + row;
            ra[i] = grow < p.M ? *(const u32x4*)(p.A + (size_t)grow * p.lda + k0 + c8 * 8)
                               : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            int c = tid + i * 256;
            if (c < B_THREADS) {
                int byte = c * 16;
                int frag = byte / WFRAG_BYTES, within = byte % WFRAG_BYTES;
                int fn = frag / (KT / 32), fk = frag % (KT / 32);
                size_t g = ((size_t)(n0 / 16 + fn) * Kf + (k0 / 32 + fk)) * WFRAG_BYTES + within;
                rb[i] = *(const u32x4*)((const uint8_t*)p.W + g);
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            int c = tid + i * 256;
            int row = c / (KT / 8), c8 = c % (KT / 8);
            *(u32x4*)(&As[buf][row][c8 * 8]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            int c = tid + i * 256;
            if (c < B_THREADS) *(u32x4*)(&Bs[buf][c * 16]) = rb[i];
        }
    };
    auto compute = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < KT / 32; ++ks) {
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                int row = wm * WM + fm * 16 + (lane & 15);
                af[fm] = *(const bf16x8*)(&As[buf][row][ks * 32 + 8 * (lane >> 4)]);
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                int frag = (wn * FN + fn) * (KT / 32) + ks;
                if constexpr (W8) {
                    u32x2 w = *(const u32x2*)(&Bs[buf][frag * 512 + lane * 8]);
                    bfr[fn] = e4m3x8_to_bf16x8(w);
                } else {
                    bfr[fn] = *(const bf16x8*)(&Bs[buf][frag * 1024 + lane * 16]);
                }
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma_16x16x32(af[fm], bfr[fn], acc[fm][fn]);
        }
    };

    if (nk > 0) {
        load_tile(0);
        store_tile(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            if (kt + 1 < nk) load_tile(kt + 1);
            compute(kt & 1);
            if (kt + 1 < nk) store_tile((kt + 1) & 1);
            __syncthreads();
        }
    }

    // -------- split-K fix-up: the last split of this tile reduces ---------
    if (p.ksplit > 1) {
        float* mine = p.ws + (size_t)kz * p.M * p.N;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    int row = m0 + wm * WM + fm * 16 + 4 * (lane >> 4) + r;
                    int col = n0 + wn * WN + fn * 16 + (lane & 15);
                    if (row < p.M) mine[(size_t)row * p.N + col] = acc[fm][fn][r];
                }
        __threadfence();
        __syncthreads();
        __shared__ int s_last;
        if (tid == 0) {
            int tile = blockIdx.y * gridDim.x + blockIdx.x;
            int old = atomicAdd(&p.counters[tile], 1);
            s_last = (old == p.ksplit - 1);
            if (s_last) atomicExch(&p.counters[tile], 0);
        }
        __syncthreads();
        if (!s_last) return;
        __threadfence();
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    int row = m0 + wm * WM + fm * 16 + 4 * (lane >> 4) + r;
                    int col = n0 + wn * WN + fn * 16 + (lane & 15);
                    float s = 0.f;
                    if (row < p.M) {
                        for (int z = 0; z < p.ksplit; ++z) {
                            float v = (z == kz) ? acc[fm][fn][r]
                                                : __builtin_nontemporal_load(
                                                      &p.ws[((size_t)z * p.M + row) * p.N + col]);
                            s += v;
                        }
                    }
                    acc[fm][fn][r] = s;
                }
    }

    // ------------------------------ epilogue ------------------------------
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int col = n0 + wn * WN + fn * 16 + (lane & 15);
            const float wsc = W8 ? p.wscale[col] : 1.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * WM + fm * 16 + 4 * (lane >> 4) + r;
                const bool ok = row < p.M;
                float v = acc[fm][fn][r] * wsc;
                if constexpr (EPI == EPI_BIAS_F32) {
                    if (ok) p.out_f32[(size_t)row * p.N + col] = v + p.bias[col];
                } else if constexpr (EPI == EPI_RESID) {
                    if (ok) {
                        int b = row / p.T;
                        float g = p.mod[(size_t)(p.step * p.B + b) * p.mod_ld + p.gate_off + col];
                        float* hp = p.out_f32 + (size_t)row * p.N + col;
                        *hp = *hp + g * v;
                    }
                } else if constexpr (EPI == EPI_QKV_ROPE) {
                    float partner = __shfl_xor(v, 1, 64);
                    if (ok) {
                        const int qd = p.nq * p.dh, kvd = p.nkv * p.dh;
                        int sec, local;
                        if (col < qd) { sec = 0; local = col; }
                        else if (col < qd + kvd) { sec = 1; local = col - qd; }
                        else { sec = 2; local = col - qd - kvd; }
                        const int head = local / p.dh, pp = local % p.dh;
                        const int m = pp >> 1, second = pp & 1;
                        const int b = row / p.T, i = row % p.T;
                        float outv;
                        if (sec < 2) {
                            float2 cs = p.rope[i * (p.dh / 2) + m];
                            float u1 = second ? partner : v;
                            float u2 = second ? v : partner;
                            outv = second ? (u2 * cs.x + u1 * cs.y) : (u1 * cs.x - u2 * cs.y);
                        } else {
                            outv = v;
                        }
                        const int dim = m + second * (p.dh / 2);
                        uint16_t ob = f32_to_bf16(outv);
                        if (sec == 0) p.q[((size_t)(b * p.nq + head) * p.T + i) * p.dh + dim] = ob;
                        else if (sec == 1) p.kn[((size_t)(b * p.nkv + head) * p.T + i) * p.dh + dim] = ob;
                        else p.vn[((size_t)(b * p.nkv + head) * p.T + i) * p.dh + dim] = ob;
                    }
                } else if constexpr (EPI == EPI_SWIGLU) {
                    float partner = __shfl_xor(v, 1, 64);
                    if (ok && (col & 1) == 0) {
                        float a = silu_f(v) * partner;
                        p.act[(size_t)row * (p.N / 2) + (col >> 1)] = f32_to_bf16(a);
                    }
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Grouped-query attention, no mask, scale 1/sqrt(d_h), online softmax.
// Workgroup = (64 query rows of one KV group, group g, request b); the G query
// heads of a group are packed: group row = head_in_group*T + token. Keys are
// the layer's P prefix keys followed by the T chunk keys, staged through LDS
// 32 at a time (K row-major, V in B-operand fragment order).
// ---------------------------------------------------------------------------
struct AttnParams {
    const ArgBlock* ab;   // prefix pointers come from here unless direct ones are set
    const uint16_t* pk;
    const uint16_t* pv;
    const uint16_t* q;    // [B, nq, T, dh]
    const uint16_t* kn;   // [B, nkv, T, dh]
    const uint16_t* vn;
    uint16_t* o;          // [B*T, nq*dh]
    int layer, L, P, T, nq, nkv;
    float scale_log2;     // log2(e)/sqrt(dh)
};

template <int DH>
__global__ __launch_bounds__(256) void attn_kernel(AttnParams p) {
    constexpr int KB = 32;
    constexpr int KPAD = DH + 8;
    constexpr int CH = KB * DH / 8;              // 16-byte chunks per K (or V) block
    constexpr int CPT = (CH + 255) / 256;        // chunks per thread
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KB][KPAD];
    __shared__ __attribute__((aligned(16))) uint16_t Vf[2][DH / 16][64][8];
    __shared__ __attribute__((aligned(16))) uint16_t Ps[4][16][KB + 8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = blockIdx.y, b = blockIdx.z;
    const int G = p.nq / p.nkv;
    const int rows_total = G * p.T;
    const int S = p.P + p.T;
    const int nblk = (S + KB - 1) / KB;
    const uint16_t* pk = p.pk ? p.pk : p.ab->prefix_k;
    const uint16_t* pv = p.pv ? p.pv : p.ab->prefix_v;

    const int r0 = blockIdx.x * 64 + wave * 16;
    const uint16_t* qg = p.q + (size_t)(b * p.nq + g * G) * p.T * DH;
    bf16x8 qf[DH / 32];
    {
        int row = r0 + (lane & 15);
#pragma unroll
        for (int ks = 0; ks < DH / 32; ++ks) {
            qf[ks] = row < rows_total ? *(const bf16x8*)(qg + (size_t)row * DH + ks * 32 + 8 * (lane >> 4))
                                      : (bf16x8){};
        }
    }

    u32x4 rk[CPT], rv[CPT];
    auto key_src = [&](int s, const uint16_t* pref, const uint16_t* own) -> const uint16_t* {
        if (s < p.P) return pref + ((((size_t)b * p.L + p.layer) * p.P + s) * p.nkv + g) * DH;
        return own + ((size_t)(b * p.nkv + g) * p.T + (s - p.P)) * DH;
    };
    auto load_kv = [&](int kb) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            int c = tid + i * 256;
            if (c < CH) {
                int sl = c / (DH / 8), d8 = c % (DH / 8);
                int s = kb * KB + sl;
                if (s < S) {
                    rk[i] = *(const u32x4*)(key_src(s, pk, p.kn) + d8 * 8);
                    rv[i] = *(const u32x4*)(key_src(s, pv, p.vn) + d8 * 8);
                } else {
                    rk[i] = (u32x4){0u, 0u, 0u, 0u};
                    rv[i] = (u32x4){0u, 0u, 0u, 0u};
                }
            }
        }
    };
    auto store_kv = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            int c = tid + i * 256;
            if (c < CH) {
                int sl = c / (DH / 8), d8 = c % (DH / 8);
                *(u32x4*)(&Ks[buf][sl][d8 * 8]) = rk[i];
                const uint16_t* vv = (const uint16_t*)&rv[i];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    int d = d8 * 8 + j;
                    Vf[buf][d / 16][(sl / 8) * 16 + (d % 16)][sl % 8] = vv[j];
                }
            }
        }
    };

    float mrow[4], lrow[4];
    f32x4 oacc[DH / 16];
#pragma unroll
    for (int r = 0; r < 4; ++r) { mrow[r] = -INFINITY; lrow[r] = 0.f; }
#pragma unroll
    for (int dn = 0; dn < DH / 16; ++dn) oacc[dn] = (f32x4){0.f, 0.f, 0.f, 0.f};

    load_kv(0);
    store_kv(0);
    __syncthreads();
    for (int kb = 0; kb < nblk; ++kb) {
        const int buf = kb & 1;
        if (kb + 1 < nblk) load_kv(kb + 1);
        f32x4 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            s[sb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DH / 32; ++ks) {
                bf16x8 kf = *(const bf16x8*)(&Ks[buf][sb * 16 + (lane & 15)][ks * 32 + 8 * (lane >> 4)]);
                s[sb] = mfma_16x16x32(qf[ks], kf, s[sb]);
            }
        }
        float alpha[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float s0 = s[0][r] * p.scale_log2, s1 = s[1][r] * p.scale_log2;
            int key0 = kb * KB + (lane & 15), key1 = key0 + 16;
            if (key0 >= S) s0 = -INFINITY;
            if (key1 >= S) s1 = -INFINITY;
            float mx = group16_max(fmaxf(s0, s1));
            float mnew = fmaxf(mrow[r], mx);
            alpha[r] = exp2f(mrow[r] - mnew);
            float p0 = exp2f(s0 - mnew), p1 = exp2f(s1 - mnew);
            lrow[r] = lrow[r] * alpha[r] + group16_sum(p0 + p1);
            mrow[r] = mnew;
            Ps[wave][4 * (lane >> 4) + r][lane & 15] = f32_to_bf16(p0);
            Ps[wave][4 * (lane >> 4) + r][16 + (lane & 15)] = f32_to_bf16(p1);
        }
#pragma unroll
        for (int dn = 0; dn < DH / 16; ++dn)
#pragma unroll
            for (int r = 0; r < 4; ++r) oacc[dn][r] *= alpha[r];
        __syncthreads();
        bf16x8 pa = *(const bf16x8*)(&Ps[wave][lane & 15][8 * (lane >> 4)]);
#pragma unroll
        for (int dn = 0; dn < DH / 16; ++dn) {
            bf16x8 vf = *(const bf16x8*)(&Vf[buf][dn][lane][0]);
            oacc[dn] = mfma_16x16x32(pa, vf, oacc[dn]);
        }
        if (kb + 1 < nblk) store_kv((kb + 1) & 1);
        __syncthreads();
    }

#pragma unroll
    for (int r = 0; r < 4; ++r) {
        int row = r0 + 4 * (lane >> 4) + r;
        if (row < rows_total) {
            int hh = row / p.T, i = row % p.T;
            float inv = 1.0f / lrow[r];
            uint16_t* op = p.o + ((size_t)(b * p.T + i) * p.nq + g * G + hh) * DH;
#pragma unroll
            for (int dn = 0; dn < DH / 16; ++dn) op[dn * 16 + (lane & 15)] = f32_to_bf16(oacc[dn][r] * inv);
        }
    }
}

// ---------------------------------------------------------------------------
// In-projection: h[r][n] = in_b[n] + sum_a x[r][a] in_w[n][a] (fp32 state).
// ---------------------------------------------------------------------------
__global__ void inproj_kernel(const ArgBlock* ab, int first, const float* x_direct, const uint16_t* __restrict__ W,
                              const float* __restrict__ bias, float* __restrict__ h, int M, int H, int A) {
    int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= M * H) return;
    const float* x = x_direct ? x_direct : (first ? ab->noise : ab->out);
    int r = idx / H, n = idx % H;
    const float* xr = x + (size_t)r * A;
    const uint16_t* w = W + (size_t)n * A;
    float acc = bias[n];
    for (int a = 0; a < A; ++a) acc += xr[a] * bf16_to_f32(w[a]);
    h[idx] = acc;
}

// ---------------------------------------------------------------------------
// Final AdaRMSNorm + out-projection + Euler update, 4 rows per workgroup:
//   v = (RMSNorm(h)(1+scale_f)+shift_f) out_w^T + out_b
//   x_{k+1} = x_k + (t_{k+1} - t_k) v          (all fp32)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void final_euler_kernel(const ArgBlock* ab, int first, const float* __restrict__ h,
                                                          const float* __restrict__ mod, const uint16_t* __restrict__ Wout,
                                                          const float* __restrict__ bout, int M, int H, int A, int T,
                                                          int B, int step, int N, int mod_ld, int scale_off,
                                                          int shift_off, float eps) {
    extern __shared__ float ynorm[];  // [4][H]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row0 = blockIdx.x * 4;
    {
        int row = row0 + wave;
        if (row < M) {
            int b = row / T;
            const float* hr = h + (size_t)row * H;
            const float* mr = mod + (size_t)(step * B + b) * mod_ld;
            float ss = 0.f;
            for (int c = lane; c < H; c += 64) ss += hr[c] * hr[c];
            ss = wave_sum(ss);
            float inv = 1.0f / sqrtf(ss / (float)H + eps);
            for (int c = lane; c < H; c += 64)
                ynorm[wave * H + c] = hr[c] * inv * (1.f + mr[scale_off + c]) + mr[shift_off + c];
        }
    }
    __syncthreads();
    const float* xsrc = first ? ab->noise : ab->out;
    float* xdst = ab->out;
    const float* ts = ab->t_schedule;
    for (int a = wave; a < A; a += 4) {
        const uint16_t* w = Wout + (size_t)a * H;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int c = lane; c < H; c += 64) {
            float wv = bf16_to_f32(w[c]);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[rr] += ynorm[rr * H + c] * wv;
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            float s = wave_sum(acc[rr]);
            int row = row0 + rr;
            if (lane == 0 && row < M) {
                int b = row / T;
                float dt = ts[b * (N + 1) + step + 1] - ts[b * (N + 1) + step];
                size_t xi = (size_t)row * A + a;
                xdst[xi] = xsrc[xi] + dt * (s + bout[a]);
            }
        }
    }
}

// Copy fp32 rows (test entry points).
__global__ void copy_f32_kernel(const float* src, float* dst, long n) {
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src[i];
}
