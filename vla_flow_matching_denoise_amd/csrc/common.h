// Device-side helpers shared by the expert kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;

#define VLA_DEV __device__ __forceinline__

VLA_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even float -> bfloat16 bits (the hardware conversion).
VLA_DEV uint16_t f32_to_bf16(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

VLA_DEV uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// D += A * B on one 16x16x32 bf16 tile. Operand layout per lane l (checked on
// gfx950): A[i][k] with i = l%16, k = 8*(l/16)+j; B[k][n] with n = l%16,
// k = 8*(l/16)+j; D[i][n] with n = l%16, i = 4*(l/16)+r.
VLA_DEV f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Eight OCP E4M3FN codes (two 32-bit words) -> eight bf16. Every E4M3 value is
// a bf16 value, so taking the upper half of the exact fp32 is exact.
VLA_DEV bf16x8 e4m3x8_to_bf16x8(u32x2 w) {
    f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w[0], false);
    f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w[0], true);
    f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w[1], false);
    f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(w[1], true);
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x07060302u);
    r[1] = __builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), 0x07060302u);
    r[2] = __builtin_amdgcn_perm(__float_as_uint(c[1]), __float_as_uint(c[0]), 0x07060302u);
    r[3] = __builtin_amdgcn_perm(__float_as_uint(d[1]), __float_as_uint(d[0]), 0x07060302u);
    return __builtin_bit_cast(bf16x8, r);
}

// Four floats -> four OCP E4M3FN codes (v_cvt_pk_fp8_f32: round to nearest
// even), first value in the lowest byte.
VLA_DEV uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

VLA_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// v of another lane of the same 16-lane row, by a DPP lane permutation (a
// VALU operand modifier; all 64 lanes must be active, as around an MFMA).
template <int CTRL>
VLA_DEV float row_dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum / max over the 16 lanes that share l/16 (one MFMA output row group),
// as a butterfly: lane ^ 1 and lane ^ 2 (quad permutations), then lane i
// with 7 - i within each 8 (half-row mirror), then i with 15 - i (row
// mirror). Every lane ends with the reduction of all 16.
VLA_DEV float group16_sum(float v) {
    v += row_dpp<0xB1>(v);
    v += row_dpp<0x4E>(v);
    v += row_dpp<0x141>(v);
    v += row_dpp<0x140>(v);
    return v;
}
VLA_DEV float group16_max(float v) {
    v = fmaxf(v, row_dpp<0xB1>(v));
    v = fmaxf(v, row_dpp<0x4E>(v));
    v = fmaxf(v, row_dpp<0x141>(v));
    v = fmaxf(v, row_dpp<0x140>(v));
    return v;
}

// SiLU z / (1 + e^-z) with the hardware exp2 and reciprocal (about one ulp
// each, far below the bf16 rounding of every result it feeds) in place of an
// IEEE division. z -> -inf: e^-z overflows to inf and the reciprocal to 0.
VLA_DEV float silu_f(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.44269504088896341f));
}

// 2^x for softmax weights: the hardware v_exp_f32 alone. The library exp2f adds
// range scaling for results below 2^-126 (six more instructions); softmax
// weights that small are negligible against the row maximum's weight of 1.
VLA_DEV float attn_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Element index of activation (row, k) of a [rows, K] bf16 matrix. Row-major
// when frag == 0; otherwise "A-fragment" order for at most 64 rows:
// [k/32][row/16][lane][8] with lane = row%16 + 16*((k%32)/8), i.e. each
// 16x32 MFMA A operand is one contiguous 1 KiB run (rows >= M stay zero).
VLA_DEV size_t act_index(int row, int k, int K, int frag) {
    if (!frag) return (size_t)row * K + k;
    return ((size_t)((k >> 5) * 4 + (row >> 4)) * 64 + (row & 15) + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
}

// Pointers of the current call. Graph-captured kernels read them from this
// device block, which a one-thread kernel refreshes before each replay.
struct ArgBlock {
    const uint16_t* prefix_k;  // [B, L, P, n_kv, d_h] bf16
    const uint16_t* prefix_v;
    const float* noise;        // [B, T, A]
    const float* t_schedule;   // [B, N+1]
    float* out;                // [B, T, A]
    const int* prefix_valid;   // [B] valid prefix tokens per request, or null (all P)
};

// Valid prefix tokens of request b (clamped to [0, P]): keys [valid, P) are
// padding, and the chunk's RoPE positions start at `valid`.
VLA_DEV int prefix_valid(const ArgBlock* ab, int b, int P) {
    const int* v = ab->prefix_valid;
    return v ? min(max(v[b], 0), P) : P;
}
