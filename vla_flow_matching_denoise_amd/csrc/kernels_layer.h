// Kernels of one expert layer: fused residual + AdaRMSNorm, the two GEMM
// families (skinny weight-streaming for M <= 64 rows, tiled for larger M) with
// their fused epilogues, the per-call prefix K/V repack and GQA attention.
#pragma once

#include "common.h"

// ---------------------------------------------------------------------------
// Fused residual + AdaRMSNorm, one workgroup (256 threads) per token row,
// H <= 2048, S <= 8:
//   h += gate * sum_z ws[z]        (when S > 0: split-K partials of O or down)
//   y  = h / sqrt(mean(h^2) + eps) * (1 + scale) + shift  -> bf16 y and/or fp32 yf
// Every load is issued before the first use, so a row costs one memory round
// trip plus the reduction.
// ---------------------------------------------------------------------------
constexpr int RN_MAXS = 8;

__global__ __launch_bounds__(256) void resnorm_kernel(float* __restrict__ h, const float* __restrict__ ws, int S,
                                                      const float* __restrict__ mod, int gate_off, int scale_off,
                                                      int shift_off, uint16_t* __restrict__ y, float* __restrict__ yf,
                                                      int M, int H, int T, int B, int step, int mod_ld, float eps,
                                                      int afrag) {
    __shared__ float red[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    const int b = row / T;
    float* hr = h + (size_t)row * H;
    const float* mr = mod + (size_t)(step * B + b) * mod_ld;
    float4 v[2], part[2][RN_MAXS], g[2], sc[2], sh[2];
    const bool norm = y || yf;
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
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = (tid + 256 * j) * 4;
        if (c < H) {
            float4 o;
            o.x = v[j].x * inv * (1.f + sc[j].x) + sh[j].x;
            o.y = v[j].y * inv * (1.f + sc[j].y) + sh[j].y;
            o.z = v[j].z * inv * (1.f + sc[j].z) + sh[j].z;
            o.w = v[j].w * inv * (1.f + sc[j].w) + sh[j].w;
            if (y) {
                uint2 ob;
                ob.x = pack_bf16x2(o.x, o.y);
                ob.y = pack_bf16x2(o.z, o.w);
                *(uint2*)(y + act_index(row, c, H, afrag)) = ob;
            }
            if (yf) *(float4*)(yf + (size_t)row * H + c) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// Per-layer K/V of the attention, [prefix ; chunk] concatenated on the key
// axis and padded to a multiple of 32 keys (S_pad), per (request, layer, KV
// head):
//   kcat [B][L][n_kv][S_pad][d_h]  row-major (the QK^T B operand reads
//                                  16 bytes of one key row per lane)
//   vcat [B][L][n_kv][S_pad/32][d_h/16][64][8]  the PV B operand: lane l of
//                                  fragment (kb, dn) holds keys
//                                  kb*32 + 8*(l/16) + j at d = dn*16 + l%16
// The prefix part is copied in once per call; the chunk part is written by
// the QKV epilogue of each layer.
// ---------------------------------------------------------------------------
struct KVLayout {
    int L, nkv, dh, S_pad;
    VLA_DEV size_t base(int b, int l, int g) const { return (((size_t)b * L + l) * nkv + g) * (size_t)S_pad * dh; }
    VLA_DEV size_t k_at(int b, int l, int g, int key, int d) const { return base(b, l, g) + (size_t)key * dh + d; }
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
enum { EPI_BIAS_F32 = 0, EPI_RESID = 1, EPI_QKV_ROPE = 2, EPI_SWIGLU = 3, EPI_PARTIAL = 4 };

struct GemmParams {
    const uint16_t* A;   // [M, lda] bf16: row-major (tiled kernel) or A-fragment order (skinny kernel)
    int lda;
    int a_frag;          // A given in A-fragment order (required by the skinny kernel)
    int afrag;           // act (SwiGLU output) written in A-fragment order
    const void* W;       // packed fragments
    const float* wscale; // per packed row (E4M3), else null
    int M, N, K;
    int kw;              // K per split (skinny kernel)
    float* ws;           // EPI_PARTIAL: [ksplit][M][N]
    float* out_f32;      // EPI_BIAS_F32: [M][N]; EPI_RESID: h [M][N]
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

// rpos: qkv_row_pos(p, row) for EPI_QKV_ROPE (callers hoist it per row).
template <int EPI>
VLA_DEV void epilogue_store(const GemmParams& p, int row, int col, float v, float partner, int kz, int rpos) {
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
            const float2 cs = p.rope[rpos * (p.dh / 2) + m];
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

template <bool W8, int EPI>
__global__ __launch_bounds__(512) void skinny_gemm_kernel(GemmParams p) {
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

    constexpr int WREG = W8 ? 2 : 4;  // dwords of one weight fragment slice per lane
    typedef __attribute__((ext_vector_type(WREG))) unsigned wvec;
    auto load_w = [&](int nt, wvec* dst) {
#pragma unroll
        for (int i = 0; i < SK_MAXS; ++i)
            if (i < ns)
                dst[i] = *(const wvec*)((const uint8_t*)p.W +
                                        (((size_t)nt * Kf + kt0 + s_beg + i) * 64 + lane) * (W8 ? 8 : 16));
    };

    wvec wcur[SK_MAXS], wnext[SK_MAXS];
    int nt = blockIdx.x;
    if (nt < n_tiles) load_w(nt, wcur);
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
                if constexpr (W8) b = e4m3x8_to_bf16x8(wcur[i]);
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
            const float wsc = W8 ? p.wscale[col] : 1.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wave * 16 + 4 * (lane >> 4) + r;
                const float v = sum[r] * wsc;
                const float partner = __shfl_xor(v, 1, 64);
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
// Tiled GEMM for larger M: tile MT x NT per workgroup (4 waves as 2x2), K
// staged through LDS 64 at a time with register double buffering.
// ---------------------------------------------------------------------------
// Workgroup shape of a tile: 256x256 tiles would run 8 waves (2 x 4, each
// 128x64); the tiles in use (128 x 128 / 64) run 4 waves (2 x 2). Measured at
// M = 3200: 256x256 tiles (one 8-wave workgroup per CU, 1.6 rounds of tiles)
// ran gate_up in 92 us against 85 us for 128x128.
constexpr int gemm_waves(int MT, int NT) { return MT >= 256 && NT >= 256 ? 8 : 4; }

template <int MT, int NT, bool W8, int EPI>
__global__ __launch_bounds__(64 * gemm_waves(MT, NT)) void gemm_kernel(GemmParams p) {
    // k-tile per LDS stage: 128x128 tiles take 32 (36 KiB of LDS: four
    // workgroups per CU hide the load latency); narrower tiles take 64
    constexpr int KT = NT >= 128 ? 32 : 64;
    constexpr int NWAVES = gemm_waves(MT, NT), NTHR = 64 * NWAVES;
    constexpr int WGN = NWAVES / 2;  // waves along N (2 along M)
    constexpr int WM = MT / 2, WN = NT / WGN;
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int APAD = KT + 8;
    constexpr int A_CH = MT * KT / 8 / NTHR;
    constexpr int WFRAG_BYTES = W8 ? 512 : 1024;
    constexpr int B_BYTES = (NT / 16) * (KT / 32) * WFRAG_BYTES;
    constexpr int B_CH = B_BYTES / 16 / NTHR > 0 ? B_BYTES / 16 / NTHR : 1;
    constexpr int B_THREADS = B_BYTES / 16;
    static_assert(A_CH >= 1 && MT * KT / 8 == A_CH * NTHR, "A tile does not split over the threads");

    __shared__ __attribute__((aligned(16))) uint16_t As[2][MT][APAD];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][B_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    // Tile of this workgroup. Consecutive workgroups run on consecutive XCDs,
    // so when the N-tiles split evenly over the 8 XCDs, workgroup w takes an
    // N-tile of XCD group w % 8 for every M-tile: each XCD's L2 then holds one
    // eighth of the weights and reuses each A tile across its N-tiles.
    const int ntn = p.N / NT, ntm = (p.M + MT - 1) / MT;
    int mt_i, nt_i;
    if (ntn % 8 == 0) {
        const int w = blockIdx.x, per = ntn / 8, s = w >> 3;
        mt_i = s / per;
        nt_i = (w & 7) * per + s % per;
    } else {
        mt_i = blockIdx.x / ntn;
        nt_i = blockIdx.x % ntn;
    }
    const int m0 = mt_i * MT, n0 = nt_i * NT;
    const int nk = p.K / KT;
    const int Kf = p.K / 32;

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    u32x4 ra[1][A_CH], rb[1][B_CH];
    // Branch-free loads (rows past M read row M-1 and are zeroed by a select;
    // the A layout is a uniform choice), so the compiler can count the
    // loads in flight instead of draining them at divergent joins.
    auto load_tile = [&](int kt, u32x4 (&sa)[A_CH], u32x4 (&sb)[B_CH]) {
        const int k0 = kt * KT;
        if (p.a_frag) {
#pragma unroll
            for (int i = 0; i < A_CH; ++i) {
                const int c = tid + i * NTHR, row = c / (KT / 8), c8 = c % (KT / 8), grow = m0 + row;
                const u32x4 v = *(const u32x4*)(p.A + act_index(min(grow, p.M - 1), k0 + c8 * 8, p.lda, 1));
                sa[i] = grow < p.M ? v : (u32x4){0u, 0u, 0u, 0u};
            }
        } else {
#pragma unroll
            for (int i = 0; i < A_CH; ++i) {
                const int c = tid + i * NTHR, row = c / (KT / 8), c8 = c % (KT / 8), grow = m0 + row;
                const u32x4 v = *(const u32x4*)(p.A + (size_t)min(grow, p.M - 1) * p.lda + k0 + c8 * 8);
                sa[i] = grow < p.M ? v : (u32x4){0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int c = tid + i * NTHR;
            if (B_THREADS % NTHR == 0 || c < B_THREADS) {
                const int byte = c * 16;
                const int frag = byte / WFRAG_BYTES, within = byte % WFRAG_BYTES;
                const int fn = frag / (KT / 32), fk = frag % (KT / 32);
                const size_t g = ((size_t)(n0 / 16 + fn) * Kf + (k0 / 32 + fk)) * WFRAG_BYTES + within;
                sb[i] = *(const u32x4*)((const uint8_t*)p.W + g);
            }
        }
    };
    auto store_tile = [&](int buf, const u32x4 (&sa)[A_CH], const u32x4 (&sb)[B_CH]) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            int c = tid + i * NTHR;
            int row = c / (KT / 8), c8 = c % (KT / 8);
            *(u32x4*)(&As[buf][row][c8 * 8]) = sa[i];
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int c = tid + i * NTHR;
            if (B_THREADS % NTHR == 0 || c < B_THREADS) *(u32x4*)(&Bs[buf][c * 16]) = sb[i];
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

    // k-tile kt+1 is loaded into registers while k-tile kt is multiplied
    // from LDS, then written to the other LDS buffer.
    load_tile(0, ra[0], rb[0]);
    store_tile(0, ra[0], rb[0]);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) load_tile(kt + 1, ra[0], rb[0]);
        compute(kt & 1);
        if (kt + 1 < nk) store_tile((kt + 1) & 1, ra[0], rb[0]);
        __syncthreads();
    }

    float wsc[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) wsc[fn] = W8 ? p.wscale[n0 + wn * WN + fn * 16 + (lane & 15)] : 1.0f;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m0 + wm * WM + fm * 16 + 4 * (lane >> 4) + r;
            // per-row work (the RoPE position) once, not per column
            const int rpos = EPI == EPI_QKV_ROPE && row < p.M ? qkv_row_pos(p, row) : 0;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int col = n0 + wn * WN + fn * 16 + (lane & 15);
                float v = acc[fm][fn][r] * wsc[fn];
                float partner = __shfl_xor(v, 1, 64);
                epilogue_store<EPI>(p, row, col, v, partner, 0, rpos);
            }
        }
}

// ---------------------------------------------------------------------------
// Grouped-query attention, no mask, scale 1/sqrt(d_h), online softmax.
// Workgroup = (16 query rows of one KV group, group g, request b); the G query
// heads of a group are packed: group row = head_in_group*T + token. The
// AT_WAVES waves (8 for few workgroups, 4 otherwise) take interleaved 32-key blocks of the layer's concatenated K/V
// (prefetching their next block), keep their own running max / sum / output,
// and merge them through LDS at the end.
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
};

template <int DH, int AT_WAVES>
__global__ __launch_bounds__(AT_WAVES * 64) void attn_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t Ps[AT_WAVES][16][40];
    __shared__ __attribute__((aligned(16))) float Om[AT_WAVES][64][DH / 16 * 4 + 8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = blockIdx.y, b = blockIdx.z;
    const int G = p.nq / p.kv.nkv;
    const int rows_total = G * p.T;
    const int r0 = blockIdx.x * 16;
    const int nblk = p.kv.S_pad / 32;
    const size_t base = p.kv.base(b, p.layer, g);
    const uint16_t* K = p.kcat + base;
    const uint16_t* V = p.vcat + base;
    const int pvb = p.pvalid[b];  // prefix keys past this are padding

    bf16x8 qf[DH / 32];
    {
        const uint16_t* qg = p.q + (size_t)(b * p.nq + g * G) * p.T * DH;
        const int row = r0 + (lane & 15);
#pragma unroll
        for (int ks = 0; ks < DH / 32; ++ks)
            qf[ks] = row < rows_total ? *(const bf16x8*)(qg + (size_t)row * DH + ks * 32 + 8 * (lane >> 4))
                                      : (bf16x8){};
    }

    float mrow[4], lrow[4];
    f32x4 oacc[DH / 16];
#pragma unroll
    // running max starts finite: a block whose keys are all masked (padding)
    // then leaves m finite and adds weight 0, where -inf would give
    // exp2(-inf - -inf) = NaN
    for (int r = 0; r < 4; ++r) { mrow[r] = -1e30f; lrow[r] = 0.f; }
#pragma unroll
    for (int dn = 0; dn < DH / 16; ++dn) oacc[dn] = (f32x4){0.f, 0.f, 0.f, 0.f};

    bf16x8 kf[2][DH / 32], vf[DH / 16], kf_n[2][DH / 32], vf_n[DH / 16];
    auto load_kv = [&](int kb, bf16x8 (*kd)[DH / 32], bf16x8* vd) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int ks = 0; ks < DH / 32; ++ks)
                kd[sb][ks] = *(const bf16x8*)(K + (size_t)(kb * 32 + sb * 16 + (lane & 15)) * DH + ks * 32 +
                                              8 * (lane >> 4));
#pragma unroll
        for (int dn = 0; dn < DH / 16; ++dn)
            vd[dn] = *(const bf16x8*)(V + (size_t)kb * 32 * DH + ((size_t)dn * 64 + lane) * 8);
    };
    if (wave < nblk) load_kv(wave, kf, vf);
    for (int kb = wave; kb < nblk; kb += AT_WAVES) {
        if (kb + AT_WAVES < nblk) load_kv(kb + AT_WAVES, kf_n, vf_n);   // next block of this wave, in flight
        f32x4 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            s[sb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DH / 32; ++ks) s[sb] = mfma_16x16x32(qf[ks], kf[sb][ks], s[sb]);
        }
        // every key of the block real (a uniform test): no per-key mask
        const bool whole = (kb * 32 + 32 <= pvb) || (kb * 32 >= p.P && kb * 32 + 32 <= p.S);
        float alpha[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float s0 = s[0][r] * p.scale_log2, s1 = s[1][r] * p.scale_log2;
            if (!whole) {  // a block with padded prefix keys or keys past P + T
                const int key0 = kb * 32 + (lane & 15), key1 = key0 + 16;
                if (key0 >= p.S || (key0 < p.P && key0 >= pvb)) s0 = -INFINITY;
                if (key1 >= p.S || (key1 < p.P && key1 >= pvb)) s1 = -INFINITY;
            }
            const float mx = group16_max(fmaxf(s0, s1));
            const float mnew = fmaxf(mrow[r], mx);
            alpha[r] = attn_exp2(mrow[r] - mnew);
            const float p0 = attn_exp2(s0 - mnew), p1 = attn_exp2(s1 - mnew);
            lrow[r] = lrow[r] * alpha[r] + group16_sum(p0 + p1);
            mrow[r] = mnew;
            Ps[wave][4 * (lane >> 4) + r][lane & 15] = f32_to_bf16(p0);
            Ps[wave][4 * (lane >> 4) + r][16 + (lane & 15)] = f32_to_bf16(p1);
        }
#pragma unroll
        for (int dn = 0; dn < DH / 16; ++dn)
#pragma unroll
            for (int r = 0; r < 4; ++r) oacc[dn][r] *= alpha[r];
        // the P tile is private to this wave: LDS ops of one wave complete in order
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        const bf16x8 pa = *(const bf16x8*)(&Ps[wave][lane & 15][8 * (lane >> 4)]);
#pragma unroll
        for (int dn = 0; dn < DH / 16; ++dn) oacc[dn] = mfma_16x16x32(pa, vf[dn], oacc[dn]);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int ks = 0; ks < DH / 32; ++ks) kf[sb][ks] = kf_n[sb][ks];
#pragma unroll
        for (int dn = 0; dn < DH / 16; ++dn) vf[dn] = vf_n[dn];
    }

    // merge the four waves' partial results
#pragma unroll
    for (int dn = 0; dn < DH / 16; ++dn) *(f32x4*)(&Om[wave][lane][dn * 4]) = oacc[dn];
    *(f32x4*)(&Om[wave][lane][DH / 16 * 4]) = (f32x4){mrow[0], mrow[1], mrow[2], mrow[3]};
    *(f32x4*)(&Om[wave][lane][DH / 16 * 4 + 4]) = (f32x4){lrow[0], lrow[1], lrow[2], lrow[3]};
    __syncthreads();
    // wave w finishes d-column tiles dn = w, w + AT_WAVES, ...
    float mw[AT_WAVES][4], lw[AT_WAVES][4];
#pragma unroll
    for (int w = 0; w < AT_WAVES; ++w) {
        f32x4 m4 = *(const f32x4*)(&Om[w][lane][DH / 16 * 4]);
        f32x4 l4 = *(const f32x4*)(&Om[w][lane][DH / 16 * 4 + 4]);
#pragma unroll
        for (int r = 0; r < 4; ++r) { mw[w][r] = m4[r]; lw[w][r] = l4[r]; }
    }
    float scale[AT_WAVES][4], inv[4];
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
        inv[r] = 1.0f / L;
    }
    for (int dn = wave; dn < DH / 16; dn += AT_WAVES) {
        f32x4 o = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < AT_WAVES; ++w) {
            f32x4 t = *(const f32x4*)(&Om[w][lane][dn * 4]);
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] += scale[w][r] * t[r];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = r0 + 4 * (lane >> 4) + r;
            if (row < rows_total) {
                const int hh = row / p.T, i = row % p.T;
                p.o[act_index(b * p.T + i, (g * G + hh) * DH + dn * 16 + (lane & 15), p.nq * DH, p.ofrag)] =
                    f32_to_bf16(o[r] * inv[r]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The same attention for many query rows (large batches): a workgroup of four
// waves takes 64 query rows of one (request, KV group), each wave owning 16 of
// them over the whole key range, and every 32-key K/V block is staged once
// per workgroup through LDS (double-buffered). K/V is then read from L2 once
// per 64 query rows instead of once per 16, and the waves never merge.
// LDS: K rows padded by 16 bytes so the 16 lanes that read one fragment hit
// distinct banks; V kept in PV-operand order.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void attn_rows_kernel(AttnParams p) {
    constexpr int KROW = DH * 2 + 16;            // padded K row in LDS, bytes
    constexpr int KCH = DH * 2 / 16;             // 16-byte chunks per key row
    constexpr int BLK = 32 * DH * 2;             // one 32-key block of K (or V), bytes
    constexpr int CH = BLK / 16 / 256;           // chunks of a block per thread
    static_assert(CH >= 1, "head too small");
    __shared__ __attribute__((aligned(16))) uint8_t Ks[2][32 * KROW];
    __shared__ __attribute__((aligned(16))) uint8_t Vs[2][BLK];
    __shared__ __attribute__((aligned(16))) uint16_t Ps[4][16][40];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = p.nq / p.kv.nkv;
    const int rows_total = G * p.T;
    const int g = blockIdx.y, b = blockIdx.z;
    const int r0 = blockIdx.x * 64 + wave * 16;
    const int nblk = p.kv.S_pad / 32;
    const size_t base = p.kv.base(b, p.layer, g);
    const uint8_t* K = (const uint8_t*)(p.kcat + base);
    const uint8_t* V = (const uint8_t*)(p.vcat + base);
    const int pvb = p.pvalid[b];  // prefix keys past this are padding

    bf16x8 qf[DH / 32];
    {
        const uint16_t* qg = p.q + (size_t)(b * p.nq + g * G) * p.T * DH;
        const int row = r0 + (lane & 15);
        const int rowc = min(row, rows_total - 1);
#pragma unroll
        for (int ks = 0; ks < DH / 32; ++ks) {
            const bf16x8 v = *(const bf16x8*)(qg + (size_t)rowc * DH + ks * 32 + 8 * (lane >> 4));
            qf[ks] = row < rows_total ? v : (bf16x8){};
        }
    }

    float mrow[4], lrow[4];
    f32x4 oacc[DH / 16];
#pragma unroll
    // running max starts finite: a block whose keys are all masked (padding)
    // then leaves m finite and adds weight 0, where -inf would give
    // exp2(-inf - -inf) = NaN
    for (int r = 0; r < 4; ++r) { mrow[r] = -1e30f; lrow[r] = 0.f; }
#pragma unroll
    for (int dn = 0; dn < DH / 16; ++dn) oacc[dn] = (f32x4){0.f, 0.f, 0.f, 0.f};

    u32x4 rk[CH], rv[CH];
    auto gload = [&](int kb) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * 256;
            rk[i] = *(const u32x4*)(K + (size_t)kb * BLK + (size_t)c * 16);
            rv[i] = *(const u32x4*)(V + (size_t)kb * BLK + (size_t)c * 16);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * 256;
            *(u32x4*)(&Ks[buf][(c / KCH) * KROW + (c % KCH) * 16]) = rk[i];
            *(u32x4*)(&Vs[buf][c * 16]) = rv[i];
        }
    };

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kb = 0; kb < nblk; ++kb) {
        const int buf = kb & 1;
        if (kb + 1 < nblk) gload(kb + 1);   // next block in flight during this one
        f32x4 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            s[sb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DH / 32; ++ks) {
                const bf16x8 kf =
                    *(const bf16x8*)(&Ks[buf][(sb * 16 + (lane & 15)) * KROW + ks * 64 + 16 * (lane >> 4)]);
                s[sb] = mfma_16x16x32(qf[ks], kf, s[sb]);
            }
        }
        // every key of the block real (a uniform test): no per-key mask
        const bool whole = (kb * 32 + 32 <= pvb) || (kb * 32 >= p.P && kb * 32 + 32 <= p.S);
        float alpha[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float s0 = s[0][r] * p.scale_log2, s1 = s[1][r] * p.scale_log2;
            if (!whole) {  // a block with padded prefix keys or keys past P + T
                const int key0 = kb * 32 + (lane & 15), key1 = key0 + 16;
                if (key0 >= p.S || (key0 < p.P && key0 >= pvb)) s0 = -INFINITY;
                if (key1 >= p.S || (key1 < p.P && key1 >= pvb)) s1 = -INFINITY;
            }
            const float mx = group16_max(fmaxf(s0, s1));
            const float mnew = fmaxf(mrow[r], mx);
            alpha[r] = attn_exp2(mrow[r] - mnew);
            const float p0 = attn_exp2(s0 - mnew), p1 = attn_exp2(s1 - mnew);
            lrow[r] = lrow[r] * alpha[r] + group16_sum(p0 + p1);
            mrow[r] = mnew;
            Ps[wave][4 * (lane >> 4) + r][lane & 15] = f32_to_bf16(p0);
            Ps[wave][4 * (lane >> 4) + r][16 + (lane & 15)] = f32_to_bf16(p1);
        }
#pragma unroll
        for (int dn = 0; dn < DH / 16; ++dn)
#pragma unroll
            for (int r = 0; r < 4; ++r) oacc[dn][r] *= alpha[r];
        // the P tile is private to this wave: LDS ops of one wave complete in order
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        const bf16x8 pa = *(const bf16x8*)(&Ps[wave][lane & 15][8 * (lane >> 4)]);
#pragma unroll
        for (int dn = 0; dn < DH / 16; ++dn) {
            const bf16x8 vf = *(const bf16x8*)(&Vs[buf][(dn * 64 + lane) * 16]);
            oacc[dn] = mfma_16x16x32(pa, vf, oacc[dn]);
        }
        __builtin_amdgcn_wave_barrier();
        if (kb + 1 < nblk) sstore(buf ^ 1);  // that buffer was last read before the previous barrier
        __syncthreads();
    }

#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = r0 + 4 * (lane >> 4) + r;
        if (row < rows_total) {
            const float inv = 1.0f / lrow[r];
            const int hh = row / p.T, i = row % p.T;
#pragma unroll
            for (int dn = 0; dn < DH / 16; ++dn)
                p.o[act_index(b * p.T + i, (g * G + hh) * DH + dn * 16 + (lane & 15), p.nq * DH, p.ofrag)] =
                    f32_to_bf16(oacc[dn][r] * inv);
        }
    }
}
