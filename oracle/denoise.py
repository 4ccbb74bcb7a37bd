"""CPU oracle of the flow-matching action-expert denoise loop (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it and
shares no code with it.

What it computes (the method described in "LingBot-VLA on Thor (sm_110)",
section 1 "Architecture / shapes": a flow-matching action expert of 36 layers
run once per denoise step over an action chunk; section 2 names the fused
kernels of one expert layer: AdaRMSNorm, QKV+RoPE and the SwiGLU tail; the
"LingBot-VLA v2 Examples" page, section "Configuration / CUDA Graph", fixes
that the per-layer prefix KV cache is built before the loop and the loop of
fixed-shape denoise steps runs on top of it).  The pages print no equations;
every convention below is the plainest reading, listed with its reason in the
design notes of this repository:

  x_0 = noise;  for k = 0..N-1:  x_{k+1} = x_k + (t_{k+1} - t_k) * v(x_k, t_k)

  v(x, t):
    e   = [sin(s*t*w_j), cos(s*t*w_j)],  w_j = 10000^(-j/half), s = time_scale
    c   = SiLU(W_t2 SiLU(W_t1 e + b_t1) + b_t2)
    h   = x W_in^T + b_in
    per layer l, [a1, b1, g1, a2, b2, g2] = W_mod,l c + b_mod,l:
      y = RMSNorm(h) * (1 + a1) + b1
      q, k, v = y W_q^T, y W_k^T, y W_v^T   (heads of d_h columns)
      q, k <- rotate-half RoPE at positions P + i
      o_j = softmax(q_j [Kp_g; k_g]^T / sqrt(d_h)) [Vp_g; v_g],  g = j // (n_q / n_kv)
      h = h + g1 * (o W_o^T)
      y = RMSNorm(h) * (1 + a2) + b2
      h = h + g2 * ((SiLU(y W_g^T) * (y W_u^T)) W_d^T)
    [af, bf] = W_modf c + b_modf
    v = (RMSNorm(h) * (1 + af) + bf) W_out^T + b_out

Weights arrive as raw encodings (bf16 bit patterns, OCP E4M3FN codes with
per-output-row float32 scales, or OCP MXFP4 blocks: E2M1 codes with one E8M0
scale per 32 inputs); this module decodes them itself.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "ExpertDims", "decode_bf16", "decode_e4m3fn", "decode_weights",
    "sinusoidal_embedding", "silu", "time_condition", "modulation",
    "rms_normalize", "ada_rms_norm", "rope_rotate_half", "softmax",
    "gqa_attention", "expert_layer", "velocity", "denoise", "denoise_varlen", "cosine",
    "quantize_e4m3fn", "quantize_per_token_e4m3", "decode_e2m1", "decode_mxfp4",
    "BackboneDims", "decode_backbone_weights", "rms_norm_weighted", "causal_gqa_attention",
    "backbone_layer", "prefill",
]


@dataclasses.dataclass(frozen=True)
class ExpertDims:
    """Sizes and scalar conventions of the expert (notation of the method)."""
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    action_dim: int
    horizon: int
    prefix_len: int
    time_emb_dim: int = 256
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6
    time_scale: float = 1000.0

    @classmethod
    def from_config(cls, cfg) -> "ExpertDims":
        return cls(cfg.n_layers, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                   cfg.intermediate, cfg.action_dim, cfg.horizon, cfg.prefix_len,
                   cfg.time_emb_dim, cfg.rope_theta, cfg.rms_eps, cfg.time_scale)


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """bfloat16 bit patterns -> floats.

    A bfloat16 is the upper half of an IEEE-754 binary32: shifting its 16 bits
    into the top of a 32-bit word gives the same value as a float32.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(dtype)


def decode_e4m3fn(codes: np.ndarray, dtype=np.float64) -> np.ndarray:
    """OCP 8-bit E4M3FN codes -> floats.

    Format (OCP 8-bit floating point specification): 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
    m/8 * 2^-6; there are no infinities; S.1111.111 is NaN; the largest finite
    magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** (-6)
    val = sign * np.where(e == 0, sub, normal)
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return val.astype(dtype)


def _e4m3fn_table() -> np.ndarray:
    """The 127 finite non-negative E4M3FN values, indexed by code 0x00..0x7E
    (increasing with the code)."""
    return decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))


def quantize_e4m3fn(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN value of each element (the format of ``decode_e4m3fn``),
    as floats.  Ties go to the code with an even mantissa; magnitudes above
    448 saturate to 448 (no infinities in the format); NaN stays NaN.  Written
    as a search over the decoded value table, i.e. straight from the format's
    definition.
    """
    x = np.asarray(x, dtype=np.float64)
    tab = _e4m3fn_table()
    mag = np.minimum(np.abs(x), tab[-1])
    hi = np.clip(np.searchsorted(tab, mag, side="left"), 0, tab.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = mag - tab[lo], tab[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    q = np.where(pick_hi, tab[hi], tab[lo])
    return np.where(np.isnan(x), np.nan, np.copysign(q, x))


def quantize_per_token_e4m3(a: np.ndarray) -> np.ndarray:
    """Per-token FP8 activations ("LingBot-VLA v2 Examples", section
    "Configuration / Online Quantization": the tf-kernel-fp8 profile
    quantizes activations per token and weights per output channel).  The
    page gives no formula; the reading taken: each row r of a GEMM input
    [rows, K] gets the scale s_r = max_k |a[r, k]| / 448 (1 for an all-zero
    row) and the GEMM sees q(a[r, k] / s_r) * s_r, q = ``quantize_e4m3fn``.
    """
    a = np.asarray(a, dtype=np.float64)
    amax = np.max(np.abs(a), axis=-1, keepdims=True)
    s = np.where(amax > 0, amax / 448.0, 1.0)
    return quantize_e4m3fn(a / s) * s


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """OCP 4-bit E2M1 codes (0..15) -> floats.

    Format (OCP Microscaling Formats (MX) specification, FP4 E2M1): 1 sign
    bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent field 0 holds
    the subnormal m * 0.5; no infinities or NaN; largest magnitude 6.
    """
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e.astype(np.float64) - 1.0))
    return sign * mag


def decode_mxfp4(packed: np.ndarray, scales: np.ndarray, dtype=np.float64) -> np.ndarray:
    """MXFP4 weights -> floats [N, K]: E2M1 codes two per byte (element 2j in
    the low nibble) [N, K/2], and one E8M0 scale per 32 inputs [N, K/32]
    (value 2^(e - 127), the MX shared exponent; e = 255 is NaN)."""
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = p & 0xF
    codes[:, 1::2] = p >> 4
    e = np.asarray(scales, dtype=np.int64)
    x = np.where(e == 255, np.nan, np.exp2(e.astype(np.float64) - 127.0))
    vals = decode_e2m1(codes).reshape(codes.shape[0], -1, 32) * x[:, :, None]
    return vals.reshape(codes.shape).astype(dtype)


def _linear(raw: dict, name: str, l: Optional[int], dtype):
    w = raw[name] if l is None else raw[name][l]
    if w.dtype == np.uint16:
        return decode_bf16(w, dtype)
    if w.dtype == np.uint8:
        s = raw["s" + name[1]][l]
        if np.asarray(s).dtype == np.uint8:            # MXFP4: E8M0 scale per 32 inputs
            return decode_mxfp4(w, s, dtype)
        return (decode_e4m3fn(w, np.float64) * np.asarray(s, np.float64)[:, None]).astype(dtype)
    raise TypeError(f"{name}: unsupported encoding {w.dtype}")


def decode_weights(raw: dict, dtype=np.float64) -> Dict[str, object]:
    """Decode every weight of the expert to ``dtype`` (per-layer lists kept)."""
    out: Dict[str, object] = {}
    for name in ("in_w", "out_w", "t1_w", "t2_w", "modf_w"):
        out[name] = decode_bf16(raw[name], dtype)
    for name in ("in_b", "out_b", "t1_b", "t2_b", "modf_b"):
        out[name] = np.asarray(raw[name], dtype=np.float64).astype(dtype)
    L = len(raw["mod_w"])
    out["mod_w"] = [decode_bf16(raw["mod_w"][l], dtype) for l in range(L)]
    out["mod_b"] = [np.asarray(raw["mod_b"][l], np.float64).astype(dtype) for l in range(L)]
    for name in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
        out[name] = [_linear(raw, name, l, dtype) for l in range(L)]
    return out


# ----------------------------------------------------------------------------
# Time conditioning
# ----------------------------------------------------------------------------

def sinusoidal_embedding(t: float, dim: int, time_scale: float, max_period: float = 10000.0,
                         dtype=np.float64) -> np.ndarray:
    """Sinusoidal timestep embedding of width ``dim``: sines, then cosines.

    Frequencies form a geometric ladder w_j = max_period^(-j/half),
    j = 0..half-1, and the argument is time_scale * t * w_j.
    """
    half = dim // 2
    j = np.arange(half, dtype=np.float64)
    w = np.exp(-math.log(max_period) * j / half)
    arg = float(time_scale) * float(t) * w
    return np.concatenate([np.sin(arg), np.cos(arg)]).astype(dtype)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def time_condition(t: float, W: dict, dims: ExpertDims) -> np.ndarray:
    """Conditioning vector c (width H) of one time t: embedding -> 2-layer SiLU MLP."""
    dtype = W["t1_w"].dtype
    e = sinusoidal_embedding(t, dims.time_emb_dim, dims.time_scale, dtype=dtype)
    z1 = W["t1_w"] @ e + W["t1_b"]
    return silu(W["t2_w"] @ silu(z1) + W["t2_b"])


def modulation(c: np.ndarray, w: np.ndarray, b: np.ndarray, n_chunks: int):
    """Split W c + b into ``n_chunks`` H-vectors (scale/shift/gate chunks)."""
    m = w @ c + b
    return np.split(m, n_chunks)


# ----------------------------------------------------------------------------
# Normalisation, RoPE, attention
# ----------------------------------------------------------------------------

def rms_normalize(h: np.ndarray, eps: float) -> np.ndarray:
    """Row-wise h / sqrt(mean(h^2) + eps) (no learned weight)."""
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps)


def ada_rms_norm(h: np.ndarray, scale: np.ndarray, shift: np.ndarray, eps: float) -> np.ndarray:
    """Timestep-adaptive RMSNorm: RMSNorm(h) * (1 + scale) + shift."""
    return rms_normalize(h, eps) * (1.0 + scale) + shift


def rope_rotate_half(u: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary position embedding, rotate-half pairing, on the last axis.

    ``u``: [..., T, d]; ``pos``: [T].  Component m is paired with m + d/2 and the
    pair is turned by the angle pos * theta^(-2m/d).
    """
    d = u.shape[-1]
    half = d // 2
    m = np.arange(half, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * m / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang).astype(u.dtype)
    sin = np.sin(ang).astype(u.dtype)
    u1, u2 = u[..., :half], u[..., half:]
    return np.concatenate([u1 * cos - u2 * sin, u2 * cos + u1 * sin], axis=-1)


def softmax(s: np.ndarray) -> np.ndarray:
    """Row-wise softmax along the last axis (max-shifted for range)."""
    z = s - np.max(s, axis=-1, keepdims=True)
    p = np.exp(z)
    return p / np.sum(p, axis=-1, keepdims=True)


def gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Grouped-query attention with no mask.

    ``q``: [n_q, T, d]; ``k``, ``v``: [n_kv, S, d].  Query head j reads KV head
    j // (n_q / n_kv) (contiguous groups); scores are scaled by 1/sqrt(d).
    Returns [n_q, T, d].
    """
    n_q, _, d = q.shape
    n_kv = k.shape[0]
    group = n_q // n_kv
    out = np.empty_like(q)
    scale = 1.0 / math.sqrt(d)
    for j in range(n_q):
        g = j // group
        p = softmax((q[j] @ k[g].T) * scale)
        out[j] = p @ v[g]
    return out


# ----------------------------------------------------------------------------
# One expert layer, the velocity field and the Euler loop
# ----------------------------------------------------------------------------

def expert_layer(h: np.ndarray, W: dict, l: int, mod, prefix_k_l: np.ndarray,
                 prefix_v_l: np.ndarray, dims: ExpertDims, act_quant: bool = False) -> np.ndarray:
    """One expert block on the chunk's hidden rows ``h`` [T, H].

    ``mod`` = (a1, b1, g1, a2, b2, g2); ``prefix_k_l`` / ``prefix_v_l`` are this
    layer's cached prefix keys/values [P, n_kv, d_h], used as given.  With
    ``act_quant`` the input of each block linear (y before QKV, o before O,
    y before gate_up, the SwiGLU output before down) is replaced by its
    per-token FP8 version (``quantize_per_token_e4m3``).
    """
    aq = quantize_per_token_e4m3 if act_quant else (lambda z: z)
    a1, b1, g1, a2, b2, g2 = mod
    T = h.shape[0]
    nq, nkv, dh = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    y = aq(ada_rms_norm(h, a1, b1, dims.rms_eps))
    q = (y @ W["wq"][l].T).reshape(T, nq, dh).transpose(1, 0, 2)
    k = (y @ W["wk"][l].T).reshape(T, nkv, dh).transpose(1, 0, 2)
    v = (y @ W["wv"][l].T).reshape(T, nkv, dh).transpose(1, 0, 2)
    pos = dims.prefix_len + np.arange(T)
    q = rope_rotate_half(q, pos, dims.rope_theta)
    k = rope_rotate_half(k, pos, dims.rope_theta)
    pk = prefix_k_l.astype(h.dtype).transpose(1, 0, 2)      # [n_kv, P, d_h]
    pv = prefix_v_l.astype(h.dtype).transpose(1, 0, 2)
    K = np.concatenate([pk, k], axis=1)
    V = np.concatenate([pv, v], axis=1)
    o = aq(gqa_attention(q, K, V).transpose(1, 0, 2).reshape(T, nq * dh))
    h = h + g1 * (o @ W["wo"][l].T)
    y = aq(ada_rms_norm(h, a2, b2, dims.rms_eps))
    a = aq(silu(y @ W["wg"][l].T) * (y @ W["wu"][l].T))
    return h + g2 * (a @ W["wd"][l].T)


def velocity(x: np.ndarray, t: float, W: dict, prefix_k_b: np.ndarray, prefix_v_b: np.ndarray,
             dims: ExpertDims, act_quant: bool = False) -> np.ndarray:
    """Velocity v(x, t) of one request: x [T, A] -> [T, A].

    ``prefix_k_b`` / ``prefix_v_b``: this request's cache [L, P, n_kv, d_h].
    """
    c = time_condition(t, W, dims)
    h = x @ W["in_w"].T + W["in_b"]
    for l in range(dims.n_layers):
        mod = modulation(c, W["mod_w"][l], W["mod_b"][l], 6)
        h = expert_layer(h, W, l, mod, prefix_k_b[l], prefix_v_b[l], dims, act_quant)
    af, bf = modulation(c, W["modf_w"], W["modf_b"], 2)
    y = ada_rms_norm(h, af, bf, dims.rms_eps)
    return y @ W["out_w"].T + W["out_b"]


def denoise(W: dict, dims: ExpertDims, prefix_k: np.ndarray, prefix_v: np.ndarray,
            noise: np.ndarray, t_schedule: np.ndarray, act_quant: bool = False) -> np.ndarray:
    """Explicit-Euler integration of the learned velocity field.

    ``W``: decoded weights (``decode_weights``); ``prefix_k``/``prefix_v``:
    decoded floats [B, L, P, n_kv, d_h]; ``noise``: x_0 [B, T, A];
    ``t_schedule``: [B, N+1] times t_0..t_N per request.  Requests are
    independent.  Each step evaluates the field at the left end point t_k and
    advances by dt_k = t_{k+1} - t_k.  Returns x_N [B, T, A] in W's dtype.
    ``act_quant``: per-token FP8 inputs of the block linears (``expert_layer``).
    """
    dtype = W["in_w"].dtype
    B = noise.shape[0]
    N = t_schedule.shape[1] - 1
    out = np.empty(noise.shape, dtype=dtype)
    for b in range(B):
        x = noise[b].astype(dtype)
        ts = np.asarray(t_schedule[b], dtype=np.float64)
        for k in range(N):
            dt = dtype.type(ts[k + 1] - ts[k])
            x = x + dt * velocity(x, ts[k], W, prefix_k[b], prefix_v[b], dims, act_quant)
        out[b] = x
    return out


def denoise_varlen(W: dict, dims: ExpertDims, prefix_k: np.ndarray, prefix_v: np.ndarray,
                   noise: np.ndarray, t_schedule: np.ndarray, prefix_valid) -> np.ndarray:
    """The loop over prefixes padded to a common length P, request b using only
    its first ``prefix_valid[b]`` tokens (the fixed-shape mode with a
    device-side valid length on the FlashRT ``flash_rt/api.py`` page; the
    language part is padded to a fixed length on the "LingBot-VLA v2
    Examples" page).  Reading taken: the padded tokens do not exist for the
    request, so its result is the plain loop on the prefix truncated to those
    tokens, and its chunk tokens sit at positions ``prefix_valid[b] + i``.
    Lengths outside [0, P] are clamped.
    """
    out = np.empty(noise.shape, dtype=W["in_w"].dtype)
    P = prefix_k.shape[2]
    for b in range(noise.shape[0]):
        n = min(max(int(prefix_valid[b]), 0), P)
        d = dataclasses.replace(dims, prefix_len=n)
        out[b] = denoise(W, d, prefix_k[b:b + 1, :, :n], prefix_v[b:b + 1, :, :n], noise[b:b + 1],
                         t_schedule[b:b + 1])[0]
    return out


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    """Cosine similarity of two flattened arrays (fp64)."""
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


# ----------------------------------------------------------------------------
# The step before the loop: prefix K/V construction ("LingBot-VLA on Thor
# (sm_110)", section 1: a 36-layer Qwen2.5-VL prefix whose self-attention
# builds the cache; "LingBot-VLA v2 Examples", section "Configuration / CUDA
# Graph": the 36-layer KV-cache construction runs eagerly per request before
# the denoise loop).  The pages give no layer equations; the reading taken is
# the plain pre-norm decoder layer of that backbone family:
#   y = RMSNorm(x) * n1;  q, k, v = y Wq^T, y Wk^T, y Wv^T (no biases);
#   q, k <- rotate-half RoPE at positions 0..P-1;  o = causal GQA attention;
#   x = x + o Wo^T;  y = RMSNorm(x) * n2;  x = x + (SiLU(y Wg^T) * (y Wu^T)) Wd^T
# and the cache of layer l is (roped k, v) of that layer.
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class BackboneDims:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    prefix_len: int
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6

    @classmethod
    def from_config(cls, cfg) -> "BackboneDims":
        return cls(cfg.n_layers, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate,
                   cfg.prefix_len, cfg.rope_theta, cfg.rms_eps)


def decode_backbone_weights(raw: dict, dtype=np.float64) -> Dict[str, list]:
    """bf16 or per-row E4M3 (codes times row scale) linears, fp32 norm weights."""
    out: Dict[str, list] = {}
    for name in ("n1", "n2"):
        out[name] = [np.asarray(w, np.float64).astype(dtype) for w in raw[name]]
    for name in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
        out[name] = [_linear(raw, name, l, dtype) for l in range(len(raw[name]))]
    return out


def rms_norm_weighted(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm with a learned per-channel weight: x / sqrt(mean(x^2) + eps) * w."""
    return rms_normalize(x, eps) * w


def causal_gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """q [n_q, P, d_h], k/v [n_kv, P, d_h]: query i attends to keys j <= i;
    head j reads KV head j // (n_q / n_kv); scale 1/sqrt(d_h)."""
    nq, P, dh = q.shape
    G = nq // k.shape[0]
    out = np.empty_like(q)
    mask = np.tril(np.ones((P, P), dtype=bool))
    for j in range(nq):
        g = j // G
        s = (q[j] @ k[g].T) / math.sqrt(dh)
        s = np.where(mask, s, -np.inf)
        out[j] = softmax(s) @ v[g]
    return out


def backbone_layer(x: np.ndarray, W: dict, l: int, dims: BackboneDims, act_quant: bool = False):
    """One prefix decoder layer on x [P, H]; returns (x, k, v) with k (roped)
    and v [n_kv, P, d_h]. ``act_quant``: the input of each linear (y before
    QKV and gate_up, the attention output before O, the SwiGLU output before
    down) is taken through per-token E4M3 (``quantize_per_token_e4m3``), as
    the expert's batched E4M3 tier does."""
    P = x.shape[0]
    nq, nkv, dh = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    aq = quantize_per_token_e4m3 if act_quant else (lambda z: z)
    y = aq(rms_norm_weighted(x, W["n1"][l], dims.rms_eps))
    q = (y @ W["wq"][l].T).reshape(P, nq, dh).transpose(1, 0, 2)
    k = (y @ W["wk"][l].T).reshape(P, nkv, dh).transpose(1, 0, 2)
    v = (y @ W["wv"][l].T).reshape(P, nkv, dh).transpose(1, 0, 2)
    pos = np.arange(P)
    q = rope_rotate_half(q, pos, dims.rope_theta)
    k = rope_rotate_half(k, pos, dims.rope_theta)
    o = aq(causal_gqa_attention(q, k, v).transpose(1, 0, 2).reshape(P, nq * dh))
    x = x + o @ W["wo"][l].T
    y = aq(rms_norm_weighted(x, W["n2"][l], dims.rms_eps))
    x = x + aq(silu(y @ W["wg"][l].T) * (y @ W["wu"][l].T)) @ W["wd"][l].T
    return x, k, v


def prefill(W: dict, dims: BackboneDims, emb: np.ndarray, n_layers: Optional[int] = None,
            act_quant: bool = False):
    """Prefix cache of every request: emb [B, P, H] (decoded floats) ->
    (prefix_k, prefix_v) [B, L, P, n_kv, d_h] in W's dtype (the layout
    ``denoise`` takes).  ``n_layers`` limits the layers computed;
    ``act_quant`` as in ``backbone_layer``."""
    L = dims.n_layers if n_layers is None else n_layers
    B, P = emb.shape[0], emb.shape[1]
    dtype = W["wq"][0].dtype
    pk = np.empty((B, L, P, dims.n_kv_heads, dims.head_dim), dtype=dtype)
    pv = np.empty_like(pk)
    for b in range(B):
        x = np.asarray(emb[b], dtype=dtype)
        for l in range(L):
            x, k, v = backbone_layer(x, W, l, dims, act_quant)
            pk[b, l] = k.transpose(1, 0, 2)
            pv[b, l] = v.transpose(1, 0, 2)
    return pk, pv
