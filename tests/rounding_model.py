"""Rounding model of the GPU path: the oracle's arithmetic with bf16 rounding
inserted exactly where the HIP kernels store a bf16 value.

TEST INFRASTRUCTURE ONLY.  It is built from the oracle's own functions and
shares nothing with the HIP library.  Its use is to *derive tolerances*: the
difference between this model and the exact (fp64) oracle is the error that
bf16 storage alone causes, so a GPU result within a small factor of it
carries no error beyond the rounding the design chose.  Accumulation stays
fp64 here; the kernels accumulate in fp32, whose error is orders below
bf16 rounding at these widths.

Where the kernels round (expert loop, "LingBot-VLA on Thor (sm_110)", section
2, the fused layer kernels):

* the conditioning vector c, as the modulation GEMM's input;
* each AdaRMSNorm output y, as the QKV and gate_up input;
* q, k and v after the RoPE epilogue (the cache layout is bf16);
* the softmax weights exp(s - m) as the PV MFMA operand (the row sum stays
  fp32, so normalisation uses the unrounded weights);
* the attention output o (O GEMM input) and the SwiGLU output (down input);
* with E4M3 weights at more than 64 rows (per-token E4M3 linear inputs):
  the norm outputs are quantized from fp32, the attention and SwiGLU
  outputs from their bf16 copies.

The residual stream, the final norm, the out-projection and the Euler state
stay fp32 (here fp64).  The prefix backbone ("LingBot-VLA on Thor (sm_110)",
section 1) rounds at the same kinds of points: the weighted-norm outputs,
q/k/v, the softmax weights, o, the SwiGLU output.

Run as a script it prints, per layer of the LingBot-shaped prefix backbone,
how far the modelled caches sit from the exact oracle (max-abs / RMS and its
ratio to sqrt(l + 1)): the numbers behind the depth-scaled max-abs gate of
the prefill parity tests.
"""
from __future__ import annotations

import dataclasses
import math
import sys

import numpy as np

import oracle

__all__ = ["bf16_round", "expert_layer_r", "velocity_r", "denoise_r", "backbone_layer_r", "prefill_r"]


def bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of each element, as float64.

    The value is first taken to float32 (the kernels round fp32 values), then
    the low 16 bits of the float32 pattern are rounded away."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _ident(x):
    return x


def _attention_r(q, k, v, rnd, causal=False):
    """Grouped-query attention whose PV product takes rounded softmax weights
    and whose normalisation uses the unrounded row sum."""
    nq, T, d = q.shape
    G = nq // k.shape[0]
    out = np.empty_like(q)
    for j in range(nq):
        g = j // G
        s = (q[j] @ k[g].T) / math.sqrt(d)
        if causal:
            s = np.where(np.tril(np.ones(s.shape, dtype=bool)), s, -np.inf)
        p = np.exp(s - np.max(s, axis=-1, keepdims=True))
        out[j] = (rnd(p) @ v[g]) / np.sum(p, axis=-1, keepdims=True)
    return out


def expert_layer_r(h, W, l, mod, prefix_k_l, prefix_v_l, dims, rnd=bf16_round, act_quant=False):
    """``oracle.expert_layer`` with the kernels' bf16 stores (``rnd``).

    ``act_quant``: the batched E4M3 tier, whose linears take per-token E4M3
    inputs. The norm kernels quantize their fp32 output directly; the
    attention and SwiGLU outputs are stored as bf16 first and then quantized
    (the quantization itself is the oracle's ``quantize_per_token_e4m3``)."""
    q8 = oracle.quantize_per_token_e4m3 if act_quant else None
    a1, b1, g1, a2, b2, g2 = mod
    T = h.shape[0]
    nq, nkv, dh = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    y = oracle.ada_rms_norm(h, a1, b1, dims.rms_eps)
    y = q8(y) if q8 else rnd(y)
    q = (y @ W["wq"][l].T).reshape(T, nq, dh).transpose(1, 0, 2)
    k = (y @ W["wk"][l].T).reshape(T, nkv, dh).transpose(1, 0, 2)
    v = (y @ W["wv"][l].T).reshape(T, nkv, dh).transpose(1, 0, 2)
    pos = dims.prefix_len + np.arange(T)
    q = rnd(oracle.rope_rotate_half(q, pos, dims.rope_theta))
    k = rnd(oracle.rope_rotate_half(k, pos, dims.rope_theta))
    v = rnd(v)
    K = np.concatenate([prefix_k_l.transpose(1, 0, 2), k], axis=1)
    V = np.concatenate([prefix_v_l.transpose(1, 0, 2), v], axis=1)
    o = rnd(_attention_r(q, K, V, rnd).transpose(1, 0, 2).reshape(T, nq * dh))
    if q8:
        o = q8(o)
    h = h + g1 * (o @ W["wo"][l].T)
    y = oracle.ada_rms_norm(h, a2, b2, dims.rms_eps)
    y = q8(y) if q8 else rnd(y)
    a = rnd(oracle.silu(y @ W["wg"][l].T) * (y @ W["wu"][l].T))
    if q8:
        a = q8(a)
    return h + g2 * (a @ W["wd"][l].T)


def velocity_r(x, t, W, prefix_k_b, prefix_v_b, dims, rnd=bf16_round, act_quant=False):
    """``oracle.velocity`` with the kernels' bf16 stores."""
    c = rnd(oracle.time_condition(t, W, dims))
    h = x @ W["in_w"].T + W["in_b"]
    for l in range(dims.n_layers):
        mod = oracle.modulation(c, W["mod_w"][l], W["mod_b"][l], 6)
        h = expert_layer_r(h, W, l, mod, prefix_k_b[l], prefix_v_b[l], dims, rnd, act_quant)
    af, bf = oracle.modulation(c, W["modf_w"], W["modf_b"], 2)
    return oracle.ada_rms_norm(h, af, bf, dims.rms_eps) @ W["out_w"].T + W["out_b"]


def denoise_r(W, dims, prefix_k, prefix_v, noise, t_schedule, rnd=bf16_round, act_quant=False):
    """``oracle.denoise`` (explicit Euler at the left end point) on ``velocity_r``."""
    out = np.empty(noise.shape, dtype=np.float64)
    for b in range(noise.shape[0]):
        x = noise[b].astype(np.float64)
        ts = np.asarray(t_schedule[b], dtype=np.float64)
        for k in range(ts.shape[0] - 1):
            x = x + (ts[k + 1] - ts[k]) * velocity_r(x, ts[k], W, prefix_k[b], prefix_v[b], dims, rnd, act_quant)
        out[b] = x
    return out


def backbone_layer_r(x, W, l, dims, rnd=bf16_round):
    """``oracle.backbone_layer`` with the prefill kernels' bf16 stores; returns
    (x, k, v) with k and v rounded as the cache stores them."""
    P = x.shape[0]
    nq, nkv, dh = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    y = rnd(oracle.rms_norm_weighted(x, W["n1"][l], dims.rms_eps))
    q = (y @ W["wq"][l].T).reshape(P, nq, dh).transpose(1, 0, 2)
    k = (y @ W["wk"][l].T).reshape(P, nkv, dh).transpose(1, 0, 2)
    v = rnd((y @ W["wv"][l].T).reshape(P, nkv, dh).transpose(1, 0, 2))
    pos = np.arange(P)
    q = rnd(oracle.rope_rotate_half(q, pos, dims.rope_theta))
    k = rnd(oracle.rope_rotate_half(k, pos, dims.rope_theta))
    o = rnd(_attention_r(q, k, v, rnd, causal=True).transpose(1, 0, 2).reshape(P, nq * dh))
    x = x + o @ W["wo"][l].T
    y = rnd(oracle.rms_norm_weighted(x, W["n2"][l], dims.rms_eps))
    x = x + rnd(oracle.silu(y @ W["wg"][l].T) * (y @ W["wu"][l].T)) @ W["wd"][l].T
    return x, k, v


def prefill_r(W, dims, emb, n_layers=None, rnd=bf16_round):
    """``oracle.prefill`` of one request's embeddings [P, H] on
    ``backbone_layer_r``: per-layer (k, v) lists of [n_kv, P, d_h]."""
    L = dims.n_layers if n_layers is None else n_layers
    x = np.asarray(emb, np.float64)
    ks, vs = [], []
    for l in range(L):
        x, k, v = backbone_layer_r(x, W, l, dims, rnd)
        ks.append(k)
        vs.append(v)
    return ks, vs


def prefill_depth_table(n_layers=8, prefix_len=256, seed=0):
    """Per layer of the LingBot-shaped backbone: max-abs / RMS of the modelled
    cache against the exact oracle, for keys and values, and its ratio to
    sqrt(l + 1).  Rows (l, key max-abs/RMS, value max-abs/RMS, worst / sqrt(l+1))."""
    import synth
    bcfg = synth.backbone(2).replace(n_layers=n_layers, prefix_len=prefix_len, batch=1)
    raw = synth.make_backbone_weights(bcfg, seed=seed)
    W = oracle.decode_backbone_weights(raw)
    d = oracle.BackboneDims.from_config(bcfg)
    emb = oracle.decode_bf16(synth.make_embeddings(bcfg, seed=seed))[0]
    pk, pv = oracle.prefill(W, d, emb[None])
    kr, vr = prefill_r(W, d, emb)
    rows = []
    for l in range(n_layers):
        ke, ve = pk[0, l].transpose(1, 0, 2), pv[0, l].transpose(1, 0, 2)
        mk = float(np.max(np.abs(kr[l] - ke)) / np.sqrt(np.mean(ke ** 2)))
        mv = float(np.max(np.abs(vr[l] - ve)) / np.sqrt(np.mean(ve ** 2)))
        rows.append((l, mk, mv, max(mk, mv) / math.sqrt(l + 1)))
    return rows


if __name__ == "__main__":
    n = int(sys.argv[1]) if len(sys.argv) > 1 else 8
    print("LingBot-shaped prefix backbone (hidden 2048, 16 q / 2 KV heads of 128, SwiGLU 11008, P 256):")
    print("layer  keys max-abs/RMS  values max-abs/RMS  worst/sqrt(l+1)")
    for l, mk, mv, r in prefill_depth_table(n):
        print(f"{l:5d}  {mk:16.4f}  {mv:18.4f}  {r:15.4f}", flush=True)
