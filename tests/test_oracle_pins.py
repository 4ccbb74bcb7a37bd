"""Pins of the CPU oracle: values fixed by something other than the oracle.

Each test names what it pins and the plausible mistake it would catch.  The
pages print no worked numerical example of the action expert, so the pins are
library routines (torch, scipy), closed forms that follow from the method's
structure, invariants and brute force on tiny inputs.
"""
import dataclasses
import math
import sys

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from oracle import ExpertDims

RNG = np.random.default_rng(1234)


def _tiny_dims(**kw):
    base = dict(n_layers=2, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, intermediate=48,
                action_dim=5, horizon=6, prefix_len=7)
    base.update(kw)
    return ExpertDims(**base)


def _tiny_weights(d: ExpertDims, std=0.3, seed=0):
    """Decoded float64 weights with larger std than the workloads, so every
    term of the block moves the output measurably."""
    r = np.random.default_rng(seed)
    H, A, L, I = d.hidden, d.action_dim, d.n_layers, d.intermediate
    qd, kvd = d.n_q_heads * d.head_dim, d.n_kv_heads * d.head_dim
    g = lambda *s: r.standard_normal(s) * std
    W = {"in_w": g(H, A), "in_b": g(H), "out_w": g(A, H), "out_b": g(A),
         "t1_w": g(H, d.time_emb_dim), "t1_b": g(H), "t2_w": g(H, H), "t2_b": g(H),
         "modf_w": g(2 * H, H), "modf_b": g(2 * H)}
    W["mod_w"] = [g(6 * H, H) for _ in range(L)]
    W["mod_b"] = [g(6 * H) for _ in range(L)]
    shapes = {"wq": (qd, H), "wk": (kvd, H), "wv": (kvd, H), "wo": (H, qd), "wg": (I, H),
              "wu": (I, H), "wd": (H, I)}
    for n, s in shapes.items():
        W[n] = [g(*s) for _ in range(L)]
    return W


def _tiny_inputs(d: ExpertDims, B=1, seed=1):
    r = np.random.default_rng(seed)
    pk = r.standard_normal((B, d.n_layers, d.prefix_len, d.n_kv_heads, d.head_dim))
    pv = r.standard_normal((B, d.n_layers, d.prefix_len, d.n_kv_heads, d.head_dim))
    x0 = r.standard_normal((B, d.horizon, d.action_dim))
    return pk, pv, x0


# ---------------------------------------------------------------------------
# Number formats: pinned to torch's own conversions (library routines)
# ---------------------------------------------------------------------------

def test_bf16_decode_matches_torch_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits, np.float64)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(ours[m], ref[m])


def test_e4m3_spec_values():
    # OCP FP8 E4M3: max normal 448, min normal 2^-6, min subnormal 2^-9, NaN at S.1111.111
    d = oracle.decode_e4m3fn(np.array([0x7E, 0x08, 0x01, 0x80, 0x7F, 0xFE, 0x38], np.uint8))
    assert d[0] == 448.0 and d[1] == 2.0 ** -6 and d[2] == 2.0 ** -9
    assert d[3] == 0.0 and np.signbit(d[3])
    assert np.isnan(d[4]) and d[5] == -448.0 and d[6] == 1.0


def test_generator_fp8_rows_hit_448():
    # the per-row scale maps the largest magnitude of each row exactly onto 448
    cfg = synth.config(1)
    w = RNG.standard_normal((16, 64)).astype(np.float32)
    q, s = synth.to_e4m3_rowwise(w)
    deq = oracle.decode_e4m3fn(q) * s[:, None].astype(np.float64)
    assert np.all(np.max(np.abs(oracle.decode_e4m3fn(q)), axis=1) == 448.0)
    # e4m3 keeps 3 mantissa bits: relative error of round-to-nearest <= 2^-4
    big = np.abs(w) > 2.0 ** -6 * s[:, None]
    rel = np.abs(deq - w)[big] / np.abs(w)[big]
    assert rel.max() <= 2.0 ** -4 + 1e-7
    assert cfg.hidden == 256


# ---------------------------------------------------------------------------
# Time conditioning
# ---------------------------------------------------------------------------

def test_sinusoidal_embedding_closed_forms():
    e0 = oracle.sinusoidal_embedding(0.0, 256, 1000.0)
    assert np.array_equal(e0, np.r_[np.zeros(128), np.ones(128)])       # sin 0 | cos 0
    t = 0.37
    e = oracle.sinusoidal_embedding(t, 256, 1000.0)
    assert np.allclose(e[:128] ** 2 + e[128:] ** 2, 1.0, atol=1e-15)
    # first frequency is 1, frequency j = 64 is 10000^(-1/2) = 1/100
    assert e[0] == pytest.approx(math.sin(1000.0 * t), abs=1e-13)
    assert e[128] == pytest.approx(math.cos(1000.0 * t), abs=1e-13)
    assert e[64] == pytest.approx(math.sin(10.0 * t), abs=1e-13)
    assert e[127] == pytest.approx(math.sin(1000.0 * t * 10000.0 ** (-127 / 128)), abs=1e-13)


def test_silu_matches_scipy_expit():
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(oracle.silu(z), z * scipy.special.expit(z), rtol=1e-13, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert oracle.silu(np.array([-800.0]))[0] == 0.0


def test_time_mlp_two_silus_closed_form():
    # W_t1 = 0, W_t2 = identity, b_t2 = 0  =>  c = SiLU(SiLU(b_t1)) elementwise.
    d = _tiny_dims()
    W = _tiny_weights(d)
    W["t1_w"] = np.zeros_like(W["t1_w"])
    W["t2_w"] = np.eye(d.hidden)
    W["t2_b"] = np.zeros(d.hidden)
    b1 = W["t1_b"]
    s1 = b1 * scipy.special.expit(b1)
    expect = s1 * scipy.special.expit(s1)
    assert np.allclose(oracle.time_condition(0.4, W, d), expect, rtol=1e-13, atol=1e-15)
    # W_t2 = 0  =>  c = SiLU(b_t2), whatever the first layer does
    W2 = _tiny_weights(d)
    W2["t2_w"] = np.zeros_like(W2["t2_w"])
    expect2 = W2["t2_b"] * scipy.special.expit(W2["t2_b"])
    assert np.allclose(oracle.time_condition(0.8, W2, d), expect2, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# Normalisation
# ---------------------------------------------------------------------------

def test_rms_normalize_matches_linalg_norm():
    h = RNG.standard_normal((5, 40))
    ref = h / (np.linalg.norm(h, axis=1, keepdims=True) / math.sqrt(40))
    assert np.allclose(oracle.rms_normalize(h, 0.0), ref, rtol=1e-14)
    y = oracle.rms_normalize(h, 1e-6)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=1e-6)


def test_ada_rms_norm_scale_shift_form():
    h = RNG.standard_normal((3, 16)) * 4.0
    sc, sh = RNG.standard_normal(16), RNG.standard_normal(16)
    y = oracle.ada_rms_norm(h, sc, sh, 1e-6)
    # scale = -1 removes the normalised input entirely: output == shift
    assert np.array_equal(oracle.ada_rms_norm(h, -np.ones(16), sh, 1e-6), np.broadcast_to(sh, h.shape))
    # invariance to a positive rescaling of the row (up to eps)
    assert np.allclose(oracle.ada_rms_norm(7.0 * h, sc, sh, 1e-6), y, atol=1e-7)
    # zero modulation gives plain RMSNorm
    assert np.array_equal(oracle.ada_rms_norm(h, np.zeros(16), np.zeros(16), 1e-6),
                          oracle.rms_normalize(h, 1e-6))


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def test_rope_invariants():
    d, T = 16, 9
    u = RNG.standard_normal((3, T, d))
    pos = np.arange(T) + 5
    r = oracle.rope_rotate_half(u, pos, 1e6)
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(u, axis=-1), rtol=1e-14)
    assert np.allclose(oracle.rope_rotate_half(u, np.zeros(T), 1e6), u, atol=0)
    # composition: turning by a then by b equals turning by a + b
    a, b = np.arange(T) * 3, np.arange(T) + 11
    rr = oracle.rope_rotate_half(oracle.rope_rotate_half(u, a, 1e6), b, 1e6)
    assert np.allclose(rr, oracle.rope_rotate_half(u, a + b, 1e6), atol=1e-12)
    # relative position: <rope(q,m), rope(k,n)> depends on n - m only
    q, k = RNG.standard_normal(d), RNG.standard_normal(d)
    for m, n, s in [(3, 10, 100), (0, 0, 57), (300, 2, 17)]:
        l = oracle.rope_rotate_half(q[None, None], np.array([m]), 1e6)[0, 0] @ \
            oracle.rope_rotate_half(k[None, None], np.array([n]), 1e6)[0, 0]
        r2 = oracle.rope_rotate_half(q[None, None], np.array([m + s]), 1e6)[0, 0] @ \
            oracle.rope_rotate_half(k[None, None], np.array([n + s]), 1e6)[0, 0]
        assert l == pytest.approx(r2, rel=1e-11, abs=1e-12)


def test_rope_pairing_and_frequency_ladder():
    # basis vector e_m turns in the (m, m + d/2) plane by pos * theta^(-2m/d)
    d, theta, pos = 8, 1e4, 3.0
    for m in range(d // 2):
        e = np.zeros((1, 1, d))
        e[0, 0, m] = 1.0
        r = oracle.rope_rotate_half(e, np.array([pos]), theta)[0, 0]
        ang = math.atan2(r[m + d // 2], r[m])
        want = math.remainder(pos * theta ** (-2.0 * m / d), 2 * math.pi)
        assert ang == pytest.approx(want, abs=1e-12)
        others = np.delete(r, [m, m + d // 2])
        assert np.all(others == 0)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _attention_brute(q, k, v):
    n_q, T, d = q.shape
    n_kv, S, _ = k.shape
    out = np.zeros_like(q)
    for j in range(n_q):
        g = j // (n_q // n_kv)
        for i in range(T):
            s = [sum(q[j, i, c] * k[g, s_, c] for c in range(d)) / math.sqrt(d) for s_ in range(S)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            z = sum(w)
            for c in range(d):
                out[j, i, c] = sum(w[s_] * v[g, s_, c] for s_ in range(S)) / z
    return out


def test_attention_brute_force():
    q = RNG.standard_normal((4, 3, 4))
    k = RNG.standard_normal((2, 5, 4))
    v = RNG.standard_normal((2, 5, 4))
    assert np.allclose(oracle.gqa_attention(q, k, v), _attention_brute(q, k, v), atol=1e-12, rtol=0)


def test_attention_matches_torch_sdpa_gqa():
    q = RNG.standard_normal((8, 6, 16))
    k = RNG.standard_normal((2, 11, 16))
    v = RNG.standard_normal((2, 11, 16))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        enable_gqa=True)[0].numpy()
    assert np.allclose(oracle.gqa_attention(q, k, v), ref, atol=1e-12, rtol=0)


def test_attention_special_cases():
    v = RNG.standard_normal((2, 1, 4))
    q = RNG.standard_normal((4, 3, 4))
    k = RNG.standard_normal((2, 1, 4))
    o = oracle.gqa_attention(q, k, v)                  # one key: output is that value row
    assert np.allclose(o[0, 0], v[0, 0]) and np.allclose(o[3, 2], v[1, 0])
    k2 = RNG.standard_normal((2, 7, 4))
    v2 = RNG.standard_normal((2, 7, 4))
    o0 = oracle.gqa_attention(np.zeros((4, 3, 4)), k2, v2)   # q = 0: mean of the group's values
    assert np.allclose(o0[1, 0], v2[0].mean(axis=0)) and np.allclose(o0[2, 1], v2[1].mean(axis=0))


def test_softmax_properties():
    s = RNG.standard_normal((3, 9)) * 5
    p = oracle.softmax(s)
    assert np.allclose(p.sum(axis=-1), 1.0)
    assert np.allclose(oracle.softmax(s + 123.0), p)
    assert np.allclose(p, scipy.special.softmax(s, axis=-1), rtol=1e-13)


# ---------------------------------------------------------------------------
# Whole block: closed forms from structured weights
# ---------------------------------------------------------------------------

def test_zeroed_blocks_are_identity():
    d = _tiny_dims()
    W = _tiny_weights(d)
    for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
        W[n] = [np.zeros_like(a) for a in W[n]]
    pk, pv, x0 = _tiny_inputs(d)
    t = 0.3
    v = oracle.velocity(x0[0], t, W, pk[0], pv[0], d)
    # independent recomputation: in-projection, final adaptive norm, out-projection
    e = np.r_[np.sin(1000 * t * 10000.0 ** (-np.arange(128) / 128)),
              np.cos(1000 * t * 10000.0 ** (-np.arange(128) / 128))]
    z = W["t1_w"] @ e + W["t1_b"]
    z = z * scipy.special.expit(z)
    c = W["t2_w"] @ z + W["t2_b"]
    c = c * scipy.special.expit(c)
    mf = W["modf_w"] @ c + W["modf_b"]
    h = x0[0] @ W["in_w"].T + W["in_b"]
    hn = h / np.sqrt((h ** 2).mean(axis=1, keepdims=True) + d.rms_eps)
    expect = (hn * (1 + mf[:d.hidden]) + mf[d.hidden:]) @ W["out_w"].T + W["out_b"]
    assert np.allclose(v, expect, atol=1e-12)


def test_closed_gate_reduces_to_plain_rmsnorm():
    d = _tiny_dims()
    W = _tiny_weights(d)
    W["mod_w"] = [np.zeros_like(a) for a in W["mod_w"]]
    W["mod_b"] = [np.zeros_like(a) for a in W["mod_b"]]
    W["modf_w"] = np.zeros_like(W["modf_w"])
    W["modf_b"] = np.zeros_like(W["modf_b"])
    pk, pv, x0 = _tiny_inputs(d)
    v = oracle.velocity(x0[0], 0.55, W, pk[0], pv[0], d)
    h = x0[0] @ W["in_w"].T + W["in_b"]
    hn = h / (np.linalg.norm(h, axis=1, keepdims=True) / math.sqrt(d.hidden))   # eps negligible
    assert np.allclose(v, hn @ W["out_w"].T + W["out_b"], atol=1e-6)


def _only_bias_chunks(d, W, chunks: dict):
    """Modulation weights zero, bias zero except the given chunk vectors."""
    H = d.hidden
    W["mod_w"] = [np.zeros_like(a) for a in W["mod_w"]]
    bs = []
    for _ in range(d.n_layers):
        b = np.zeros(6 * H)
        for ci, vec in chunks.items():
            b[ci * H:(ci + 1) * H] = vec
        bs.append(b)
    W["mod_b"] = bs


def test_uniform_attention_block_closed_form():
    # W_q = W_k = 0 => every score is 0 => each head outputs the mean of its KV
    # group's values over prefix AND chunk keys.  Only the attention gate (chunk 2)
    # is open; the MLP gate (chunk 5) is closed.
    d = _tiny_dims(n_layers=1)
    W = _tiny_weights(d)
    W["wq"] = [np.zeros_like(W["wq"][0])]
    W["wk"] = [np.zeros_like(W["wk"][0])]
    g1 = RNG.standard_normal(d.hidden)
    _only_bias_chunks(d, W, {2: g1})
    pk, pv, x0 = _tiny_inputs(d)
    h = RNG.standard_normal((d.horizon, d.hidden))
    mod = oracle.modulation(np.ones(d.hidden), W["mod_w"][0], W["mod_b"][0], 6)
    out = oracle.expert_layer(h, W, 0, mod, pk[0, 0], pv[0, 0], d)
    y = h / np.sqrt((h ** 2).mean(axis=1, keepdims=True) + d.rms_eps)
    vnew = (y @ W["wv"][0].T).reshape(d.horizon, d.n_kv_heads, d.head_dim)
    allv = np.concatenate([pv[0, 0], vnew], axis=0)          # [P+T, n_kv, d_h]
    mean_v = allv.mean(axis=0)                                # [n_kv, d_h]
    grp = d.n_q_heads // d.n_kv_heads
    o_row = np.concatenate([mean_v[j // grp] for j in range(d.n_q_heads)])
    expect = h + g1 * (o_row @ W["wo"][0].T)[None, :]
    assert np.allclose(out, expect, atol=1e-12)


def test_mlp_block_closed_form():
    # scale chunk 3 = -1 makes the pre-MLP norm output equal to the shift chunk 4,
    # independent of h; gate chunk 5 opens the MLP; attention gate closed.
    d = _tiny_dims(n_layers=1)
    W = _tiny_weights(d)
    beta, gam = RNG.standard_normal(d.hidden), RNG.standard_normal(d.hidden)
    _only_bias_chunks(d, W, {3: -np.ones(d.hidden), 4: beta, 5: gam})
    pk, pv, _ = _tiny_inputs(d)
    h = RNG.standard_normal((d.horizon, d.hidden))
    mod = oracle.modulation(np.ones(d.hidden), W["mod_w"][0], W["mod_b"][0], 6)
    out = oracle.expert_layer(h, W, 0, mod, pk[0, 0], pv[0, 0], d)
    gz = W["wg"][0] @ beta
    a = gz * scipy.special.expit(gz) * (W["wu"][0] @ beta)
    expect = h + (gam * (W["wd"][0] @ a))[None, :]
    assert np.allclose(out, expect, atol=1e-12)


# ---------------------------------------------------------------------------
# The block's rotary positions: a closed form with one-hot weights
# ("LingBot-VLA on Thor (sm_110)", section 2: the QKV projection with RoPE;
# chunk tokens sit after the cached prefix, at positions P + i)
# ---------------------------------------------------------------------------

def _rope_probe_layer(d: ExpertDims, m: int):
    """One layer whose attention scores can be written out by hand.

    Modulation: scale_1 = -1 and shift_1 = e_0, so every chunk row's normed
    input is exactly e_0; gate_1 = 1; the MLP gate is closed.  W_q and W_k
    send e_0 to e_m in every head, W_v sends it to e_2, W_o is the identity.
    Prefix keys: key 0 = e_m, key 1 = e_{m+d/2}, the rest zero; prefix values
    e_0, e_1, then e_3.  Before the rotation every chunk query and key is e_m,
    so each score is a cosine or sine of the rotation angle."""
    H, dh, nq, nkv = d.hidden, d.head_dim, d.n_q_heads, d.n_kv_heads
    assert nq * dh == H
    W = _tiny_weights(d)
    for name, n_heads, unit in (("wq", nq, m), ("wk", nkv, m), ("wv", nkv, 2)):
        w = RNG.standard_normal((n_heads * dh, H))
        w[:, 0] = 0.0
        w[[h * dh + unit for h in range(n_heads)], 0] = 1.0
        W[name] = [w]
    W["wo"] = [np.eye(H)]
    e0 = np.zeros(H)
    e0[0] = 1.0
    _only_bias_chunks(d, W, {0: -np.ones(H), 1: e0, 2: np.ones(H)})
    P = d.prefix_len
    pk = np.zeros((P, nkv, dh))
    pv = np.zeros((P, nkv, dh))
    pk[0, :, m] = 1.0
    pk[1, :, m + dh // 2] = 1.0
    pv[0, :, 0] = 1.0
    pv[1, :, 1] = 1.0
    pv[2:, :, 3] = 1.0
    return W, pk, pv


def _rope_probe_expect(d: ExpertDims, m: int, h: np.ndarray, positions, chunk_rotated=True):
    """h + o for the probe layer, o written out with math.cos / math.sin: the
    query of chunk token i (at positions[i]) scores cos(phi_i) and sin(phi_i)
    against the two prefix keys, 0 against the other prefix keys, and
    cos(phi_i - phi_j) against chunk key j (its own rotation, phi at that
    key's position), where phi = position * theta^(-2m/d_h)."""
    dh, P, T = d.head_dim, d.prefix_len, h.shape[0]
    w_m = d.rope_theta ** (-2.0 * m / dh)
    phi = [positions[i] * w_m for i in range(T)]
    out = np.empty_like(h)
    for i in range(T):
        s = [math.cos(phi[i]), math.sin(phi[i])] + [0.0] * (P - 2)
        s += [math.cos(phi[i] - phi[j]) if chunk_rotated else math.cos(phi[i]) for j in range(T)]
        s = [x / math.sqrt(dh) for x in s]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        z = sum(e)
        o_head = np.zeros(dh)
        o_head[0] = e[0] / z
        o_head[1] = e[1] / z
        o_head[3] = sum(e[2:P]) / z
        o_head[2] = sum(e[P:]) / z
        out[i] = h[i] + np.tile(o_head, d.n_q_heads)
    return out


@pytest.mark.parametrize("m", [0, 1])
@pytest.mark.parametrize("P", [7, 19])
def test_block_rope_positions_closed_form(m, P):
    """The chunk's queries and keys are rotated at positions P + i: the
    oracle's layer equals the hand-written scores above, and differs from
    the two plausible mistakes (positions 0..T-1, or chunk keys left
    unrotated)."""
    d = _tiny_dims(n_layers=1, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, prefix_len=P)
    W, pk, pv = _rope_probe_layer(d, m)
    h = RNG.standard_normal((d.horizon, d.hidden))
    mod = oracle.modulation(np.ones(d.hidden), W["mod_w"][0], W["mod_b"][0], 6)
    got = oracle.expert_layer(h, W, 0, mod, pk, pv, d)
    T = d.horizon
    want = _rope_probe_expect(d, m, h, [P + i for i in range(T)])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)
    wrong_pos = _rope_probe_expect(d, m, h, list(range(T)))
    unrotated = _rope_probe_expect(d, m, h, [P + i for i in range(T)], chunk_rotated=False)
    assert np.abs(got - wrong_pos).max() > 1e-3
    assert np.abs(got - unrotated).max() > 1e-3


def test_varlen_block_positions_follow_the_valid_length():
    """A prefix padded to P with n valid tokens puts the chunk at positions
    n + i: one Euler step of a one-layer probe model (x-independent input
    rows, output projection reading the probe's attention) through
    denoise_varlen equals the hand-written scores at positions n + i."""
    P, n, m = 19, 7, 0
    d = _tiny_dims(n_layers=1, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, prefix_len=P)
    W, pk, pv = _rope_probe_layer(d, m)
    # x enters only through W_in = 0, so h = b_in for every row; the final
    # norm is the plain RMSNorm (closed final gate) and W_out reads it back
    W["in_w"] = np.zeros_like(W["in_w"])
    W["modf_w"] = np.zeros_like(W["modf_w"])
    W["modf_b"] = np.zeros_like(W["modf_b"])
    A, H = d.action_dim, d.hidden
    W["out_w"] = RNG.standard_normal((A, H))
    W["out_b"] = np.zeros(A)
    x0 = RNG.standard_normal((1, d.horizon, A))
    ts = np.array([[0.0, 1.0]])
    pk_pad = np.concatenate([pk[:n], RNG.standard_normal((P - n, d.n_kv_heads, d.head_dim))])[None, None]
    pv_pad = np.concatenate([pv[:n], RNG.standard_normal((P - n, d.n_kv_heads, d.head_dim))])[None, None]
    got = oracle.denoise_varlen(W, d, pk_pad, pv_pad, x0, ts, [n])[0]
    h0 = np.tile(W["in_b"], (d.horizon, 1))
    hd = dataclasses.replace(d, prefix_len=n)
    h1 = _rope_probe_expect(hd, m, h0, [n + i for i in range(d.horizon)])
    hn = h1 / np.sqrt(np.mean(h1 ** 2, axis=1, keepdims=True) + d.rms_eps)
    np.testing.assert_allclose(got, x0[0] + hn @ W["out_w"].T, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Euler loop
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["uniform", "warped"])
def test_constant_velocity_closed_form(kind):
    cfg = synth.config(1)
    raw = synth.make_weights(cfg)
    u = RNG.standard_normal(cfg.action_dim).astype(np.float32)
    raw = synth.apply_variant(raw, "const_velocity", cfg, velocity_bias=u)
    W = oracle.decode_weights(raw)
    pk, pv = synth.make_prefix(cfg)
    x0 = synth.make_noise(cfg)
    ts = synth.make_schedule(cfg.n_steps, 1, kind)
    out = oracle.denoise(W, ExpertDims.from_config(cfg), oracle.decode_bf16(pk),
                         oracle.decode_bf16(pv), x0, ts)
    span = float(ts[0, -1]) - float(ts[0, 0])
    assert np.allclose(out[0], x0[0] + u.astype(np.float64) * span, atol=1e-12, rtol=0)


def test_time_only_field_uses_left_endpoint():
    # W_in = 0 makes v independent of x, so x_N = x_0 + sum_k dt_k v(t_k) exactly;
    # evaluating at t_{k+1} instead gives a measurably different answer.
    d = _tiny_dims()
    W = _tiny_weights(d)
    W["in_w"] = np.zeros_like(W["in_w"])
    pk, pv, x0 = _tiny_inputs(d)
    ts = synth.make_schedule(6, 1, "warped")
    out = oracle.denoise(W, d, pk, pv, x0, ts)[0]
    t = ts[0].astype(np.float64)
    vs = [oracle.velocity(np.zeros_like(x0[0]), t[k], W, pk[0], pv[0], d) for k in range(7)]
    left = x0[0] + sum((t[k + 1] - t[k]) * vs[k] for k in range(6))
    right = x0[0] + sum((t[k + 1] - t[k]) * vs[k + 1] for k in range(6))
    assert np.allclose(out, left, atol=1e-12)
    assert not np.allclose(out, right, atol=1e-6)


def test_schedule_splitting_is_bitwise():
    cfg = synth.config(1)
    W = oracle.decode_weights(synth.make_weights(cfg))
    d = ExpertDims.from_config(cfg)
    pk, pv = (oracle.decode_bf16(a) for a in synth.make_prefix(cfg))
    x0 = synth.make_noise(cfg)
    ts = synth.make_schedule(10, 1)
    full = oracle.denoise(W, d, pk, pv, x0, ts)
    half = oracle.denoise(W, d, pk, pv, x0, ts[:, :6])
    rest = oracle.denoise(W, d, pk, pv, half, ts[:, 5:])
    assert np.array_equal(full, rest)


def test_euler_first_order_convergence():
    # With a slowly varying field (time_scale 1) the Euler error halves with dt:
    # (x_N - x_2N) / (x_2N - x_4N) -> 2.
    d = _tiny_dims(time_scale=1.0)
    W = _tiny_weights(d, std=0.1)
    pk, pv, x0 = _tiny_inputs(d)
    xs = {}
    for n in (16, 32, 64):
        ts = (np.arange(n + 1, dtype=np.float64) / n)[None]
        xs[n] = oracle.denoise(W, d, pk, pv, x0, ts)
    r = np.linalg.norm(xs[16] - xs[32]) / np.linalg.norm(xs[32] - xs[64])
    assert 1.9 < r < 2.1, r


def test_batch_independence_and_permutation():
    cfg = synth.config(1).replace(batch=3)
    W = oracle.decode_weights(synth.make_weights(cfg))
    d = ExpertDims.from_config(cfg)
    pk, pv = (oracle.decode_bf16(a) for a in synth.make_prefix(cfg))
    x0 = synth.make_noise(cfg)
    ts = synth.make_schedule(4, 3, "warped")
    out = oracle.denoise(W, d, pk, pv, x0, ts)
    for b in range(3):
        one = oracle.denoise(W, d, pk[b:b + 1], pv[b:b + 1], x0[b:b + 1], ts[b:b + 1])
        assert np.array_equal(one[0], out[b])
    perm = [2, 0, 1]
    outp = oracle.denoise(W, d, pk[perm], pv[perm], x0[perm], ts[perm])
    assert np.array_equal(outp, out[perm])
    # the generator's request streams: request b of a batch == batch-1 request b
    pk1, _ = synth.make_prefix(cfg.replace(batch=1), requests=[2])
    assert np.array_equal(oracle.decode_bf16(pk1)[0], pk[2])


def test_fp32_twin_agrees_with_fp64():
    cfg = synth.config(1)
    raw = synth.make_weights(cfg)
    d = ExpertDims.from_config(cfg)
    pk, pv = synth.make_prefix(cfg)
    x0 = synth.make_noise(cfg)
    ts = synth.make_schedule(cfg.n_steps, 1)
    o64 = oracle.denoise(oracle.decode_weights(raw, np.float64), d, oracle.decode_bf16(pk),
                         oracle.decode_bf16(pv), x0, ts)
    o32 = oracle.denoise(oracle.decode_weights(raw, np.float32), d,
                         oracle.decode_bf16(pk, np.float32), oracle.decode_bf16(pv, np.float32),
                         x0, ts)
    assert o32.dtype == np.float32
    assert oracle.cosine(o32, o64) >= 1 - 1e-9


# ---------------------------------------------------------------------------
# Prefixes padded to a common length (per-request valid length)
# ---------------------------------------------------------------------------
def test_padded_prefix_keys_are_masked_keys():
    """Attention over a prefix truncated to n tokens equals attention over all
    P tokens with the padded keys' scores set to -inf (written out here with
    numpy, not through the oracle's attention)."""
    r = np.random.default_rng(5)
    T, P, nq, nkv, dh, n = 6, 9, 4, 2, 8, 4
    q = r.standard_normal((nq, T, dh))
    kp, vp = r.standard_normal((nkv, P, dh)), r.standard_normal((nkv, P, dh))
    kc, vc = r.standard_normal((nkv, T, dh)), r.standard_normal((nkv, T, dh))
    K = np.concatenate([kp, kc], axis=1)
    V = np.concatenate([vp, vc], axis=1)
    want = np.empty((nq, T, dh))
    for j in range(nq):
        g = j // (nq // nkv)
        s = q[j] @ K[g].T / math.sqrt(dh)
        s[:, n:P] = -np.inf
        e = np.exp(s - s.max(axis=1, keepdims=True))
        want[j] = (e / e.sum(axis=1, keepdims=True)) @ V[g]
    got = oracle.gqa_attention(q, np.concatenate([kp[:, :n], kc], axis=1), np.concatenate([vp[:, :n], vc], axis=1))
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_varlen_full_lengths_and_padding_invariance():
    d = _tiny_dims()
    W = _tiny_weights(d)
    pk, pv, x0 = _tiny_inputs(d, B=3)
    ts = np.tile(np.linspace(0.0, 1.0, 4), (3, 1))
    full = oracle.denoise(W, d, pk, pv, x0, ts)
    # every request at the full length (and lengths past P, clamped) is the plain loop, bitwise
    assert np.array_equal(oracle.denoise_varlen(W, d, pk, pv, x0, ts, [d.prefix_len] * 3), full)
    assert np.array_equal(oracle.denoise_varlen(W, d, pk, pv, x0, ts, [99, d.prefix_len, 1000]), full)
    valid = [d.prefix_len, 3, 0]
    a = oracle.denoise_varlen(W, d, pk, pv, x0, ts, valid)
    assert np.array_equal(a[0], full[0])
    assert not np.allclose(a[1], full[1]) and not np.allclose(a[2], full[2])
    # what sits in the padded tokens never matters
    pk2, pv2 = pk.copy(), pv.copy()
    pk2[1, :, 3:] = 1e3
    pv2[1, :, 3:] = -1e3
    pk2[2], pv2[2] = 7.0, -7.0
    assert np.array_equal(oracle.denoise_varlen(W, d, pk2, pv2, x0, ts, valid), a)
    # a length of 0 is the loop without a prefix; negative lengths clamp to 0
    d0 = ExpertDims(**{**d.__dict__, "prefix_len": 0})
    none = oracle.denoise(W, d0, pk[2:3, :, :0], pv[2:3, :, :0], x0[2:3], ts[2:3])
    assert np.array_equal(a[2], none[0])
    assert np.array_equal(oracle.denoise_varlen(W, d, pk, pv, x0, ts, [d.prefix_len, 3, -5]), a)



# ---------------------------------------------------------------------------
# Per-token FP8 activations (the batched E4M3 tier)
# ---------------------------------------------------------------------------

def _e4m3_values():
    return oracle.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))


def test_e4m3_encoder_matches_torch_cast():
    """The E4M3FN encoder against torch's float8_e4m3fn cast (round to nearest
    even) on random in-range values and on every midpoint between adjacent
    representable values. Catches a wrong tie rule, exponent bias or
    subnormal step."""
    tab = _e4m3_values()
    mids = (tab[:-1] + tab[1:]) / 2
    mags = np.exp2(RNG.uniform(-12, np.log2(448.0), 4000))
    x = np.concatenate([mids, -mids, mags * RNG.choice([-1.0, 1.0], mags.size), [0.0, -0.0]])
    want = torch.tensor(x, dtype=torch.float64).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.quantize_e4m3fn(x), want)


def test_e4m3_encoder_fixed_points_and_saturation():
    tab = _e4m3_values()
    np.testing.assert_array_equal(oracle.quantize_e4m3fn(tab), tab)
    np.testing.assert_array_equal(oracle.quantize_e4m3fn(-tab), -tab)
    np.testing.assert_array_equal(oracle.quantize_e4m3fn(np.array([1000.0, -500.0, 448.0, 464.0])),
                                  [448.0, -448.0, 448.0, 448.0])
    assert np.isnan(oracle.quantize_e4m3fn(np.array([np.nan]))[0])


def test_per_token_quantization_properties():
    """Scale = row max / 448: rows are independent, a power-of-two row scaling
    commutes exactly, zero rows stay zero, each row's largest element is kept,
    and the relative error of normal-range elements is at most half an ulp
    (2^-4) of a 3-bit mantissa."""
    a = RNG.standard_normal((7, 96)) * np.exp2(RNG.integers(-8, 8, (7, 1)))
    a[3] = 0.0
    q = oracle.quantize_per_token_e4m3(a)
    np.testing.assert_array_equal(q, np.vstack([oracle.quantize_per_token_e4m3(r[None]) for r in a]))
    np.testing.assert_array_equal(oracle.quantize_per_token_e4m3(a * 2.0 ** 5), q * 2.0 ** 5)
    assert np.all(q[3] == 0.0)
    for r in (0, 1, 2, 4, 5, 6):
        j = np.argmax(np.abs(a[r]))
        assert abs(q[r, j] - a[r, j]) <= 1e-12 * abs(a[r, j])
        s = np.max(np.abs(a[r])) / 448.0
        normal = np.abs(a[r]) >= s * 2.0 ** -6
        assert np.all(np.abs(q[r] - a[r])[normal] <= 2.0 ** -4 * np.abs(a[r])[normal] * (1 + 1e-12))


def test_act_quant_wiring_in_the_layer(monkeypatch):
    """With act_quant the four block-linear inputs, and only they, go through
    the per-token quantizer: y [T, H] before QKV, o [T, n_q d_h] before O,
    y [T, H] before gate_up, the SwiGLU output [T, I] before down. Off by
    default (the layer is then unchanged, bitwise)."""
    d = _tiny_dims()
    W = _tiny_weights(d)
    T, H = d.horizon, d.hidden
    h = RNG.standard_normal((T, H))
    mod = [RNG.standard_normal(H) * 0.2 for _ in range(6)]
    pk = RNG.standard_normal((d.prefix_len, d.n_kv_heads, d.head_dim))
    pv = RNG.standard_normal((d.prefix_len, d.n_kv_heads, d.head_dim))
    base = oracle.expert_layer(h, W, 0, mod, pk, pv, d)
    shapes = []
    real = oracle.quantize_per_token_e4m3

    def counting(z):
        shapes.append(z.shape)
        return real(z)

    import sys
    od = sys.modules["oracle.denoise"]   # the module (the package re-exports its function `denoise`)
    monkeypatch.setattr(od, "quantize_per_token_e4m3", counting)
    np.testing.assert_array_equal(od.expert_layer(h, W, 0, mod, pk, pv, d), base)
    assert shapes == []
    out = od.expert_layer(h, W, 0, mod, pk, pv, d, act_quant=True)
    assert shapes == [(T, H), (T, d.n_q_heads * d.head_dim), (T, H), (T, d.intermediate)]
    rel = np.linalg.norm(out - base) / np.linalg.norm(base - h)
    assert 1e-4 < rel < 0.2, rel


# ---------------------------------------------------------------------------
# MXFP4 gate/up weights (the E4M3 + MXFP4 gate_up tier)
# ---------------------------------------------------------------------------

def test_e2m1_decode_table():
    """The 16 E2M1 codes against the value list of the OCP MX specification
    (0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives). Catches a wrong bias or
    subnormal rule."""
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = oracle.decode_e2m1(np.arange(16))
    np.testing.assert_array_equal(got[:8], want)
    np.testing.assert_array_equal(got[8:], [-v for v in want])


def test_mxfp4_decode_layout_and_scales():
    """Nibble order (element 2j low), one E8M0 scale per 32 inputs (2^(e-127),
    255 = NaN), on a hand-built row."""
    codes = np.zeros((1, 64), dtype=np.uint8)
    codes[0, 0], codes[0, 1], codes[0, 31], codes[0, 32], codes[0, 63] = 2, 7, 9, 5, 15
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    got = oracle.decode_mxfp4(packed, np.array([[127 - 3, 127 + 1]], dtype=np.uint8))
    want = np.zeros((1, 64))
    want[0, 0], want[0, 1], want[0, 31] = 1.0 / 8, 6.0 / 8, -0.5 / 8
    want[0, 32], want[0, 63] = 3.0 * 2, -6.0 * 2
    np.testing.assert_array_equal(got, want)
    assert np.all(np.isnan(oracle.decode_mxfp4(packed, np.array([[255, 127]], dtype=np.uint8))[0, :32]))


def test_mxfp4_generated_weights_within_the_format_bound():
    """The generator's MXFP4 blocks decode to values within one E2M1 step of
    the float draws (half a step where no clamping occurs): per block with
    scale X, |decoded - w| <= X for |w / X| <= 6 (steps are 0.5 X below 2 X,
    X up to 4 X, 2 X above), and the clamped top values decode to +-6 X.
    Catches a wrong scale exponent or a dropped nibble."""
    cfg = synth.config(1).replace(weight_dtype="fp8_mxfp4gu")
    raw = synth.make_weights(cfg, seed=3)
    ref = synth.make_weights(cfg, seed=3, weight_dtype="bf16")
    for name in ("wg", "wu"):
        deq = oracle.decode_mxfp4(raw[name][0], raw["s" + name[1]][0])
        w = oracle.decode_bf16(ref[name][0])
        X = np.repeat(np.exp2(raw["s" + name[1]][0].astype(np.float64) - 127.0), 32, axis=1)
        r = np.abs(w) / X
        step = np.where(r < 2, 0.5, np.where(r < 4, 1.0, 2.0))
        # the bf16 reference rounds the draws; allow its 2^-8 relative error
        err = np.abs(deq - w)
        assert np.all(err[r <= 6] <= (step[r <= 6] / 2 + np.abs(w[r <= 6]) / X[r <= 6] * 2 ** -8) * X[r <= 6] + 1e-12)
        assert np.all(np.abs(deq[r > 6]) == 6 * X[r > 6])
        assert np.corrcoef(deq.ravel(), w.ravel())[0, 1] > 0.98


# ---------------------------------------------------------------------------
# Prefix K/V construction (backbone prefill)
# ---------------------------------------------------------------------------

def test_causal_attention_matches_torch_sdpa():
    """Causal GQA attention against torch's scaled_dot_product_attention with
    is_causal (fp64, KV heads repeated per group). Catches an off-by-one in
    the mask or a wrong group mapping."""
    nq, nkv, P, dh = 6, 2, 9, 8
    q, k, v = (RNG.standard_normal(s) for s in ((nq, P, dh), (nkv, P, dh), (nkv, P, dh)))
    got = oracle.causal_gqa_attention(q, k, v)
    G = nq // nkv
    kt = torch.tensor(k).repeat_interleave(G, dim=0)
    vt = torch.tensor(v).repeat_interleave(G, dim=0)
    want = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q)[None], kt[None], vt[None],
                                                            is_causal=True)[0].numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # the last query sees every key: the unmasked attention's last row
    np.testing.assert_allclose(got[:, -1], oracle.gqa_attention(q, k, v)[:, -1], rtol=1e-12, atol=1e-12)


def test_weighted_rms_norm_matches_torch():
    x = RNG.standard_normal((5, 24))
    w = RNG.standard_normal(24)
    want = torch.nn.functional.rms_norm(torch.tensor(x), (24,), torch.tensor(w), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rms_norm_weighted(x, w, 1e-6), want, rtol=1e-12, atol=1e-12)


def test_prefill_is_causal_in_its_tokens():
    """The cache of the first n tokens does not depend on later tokens (every
    layer): prefill of a truncated prefix equals the first n positions of the
    full one. Also why a prefix padded at its end gives exact caches for its
    valid tokens."""
    bcfg = synth.backbone(1).replace(prefix_len=12, batch=2)
    W = oracle.decode_backbone_weights(synth.make_backbone_weights(bcfg, seed=2))
    d = oracle.BackboneDims.from_config(bcfg)
    emb = oracle.decode_bf16(synth.make_embeddings(bcfg, seed=3))
    pk, pv = oracle.prefill(W, d, emb)
    n = 7
    pk7, pv7 = oracle.prefill(W, dataclasses.replace(d, prefix_len=n), emb[:, :n])
    np.testing.assert_allclose(pk7, pk[:, :, :n], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(pv7, pv[:, :, :n], rtol=1e-12, atol=1e-12)
    # and a later token does change later positions (the mask is not all-blocking)
    emb2 = emb.copy()
    emb2[:, n] += 1.0
    pk2, _ = oracle.prefill(W, d, emb2)
    assert np.abs(pk2[:, 1, n + 1:] - pk[:, 1, n + 1:]).max() > 1e-3


def test_prefill_position_zero_key_is_unrotated():
    """RoPE at position 0 is the identity: layer 0's first key equals the
    normalized first embedding times Wk (a special case of the layer)."""
    bcfg = synth.backbone(1).replace(prefix_len=4)
    W = oracle.decode_backbone_weights(synth.make_backbone_weights(bcfg, seed=1))
    d = oracle.BackboneDims.from_config(bcfg)
    emb = oracle.decode_bf16(synth.make_embeddings(bcfg, seed=1))
    pk, _ = oracle.prefill(W, d, emb, n_layers=1)
    x0 = emb[0, 0]
    y0 = x0 / np.sqrt(np.mean(x0 ** 2) + d.rms_eps) * W["n1"][0]
    np.testing.assert_allclose(pk[0, 0, 0].ravel(), W["wk"][0] @ y0, rtol=1e-10, atol=1e-12)


def test_prefill_act_quant_wiring():
    """act_quant takes exactly the four linear inputs through per-token E4M3:
    with the quantizer replaced by the identity the result is the plain
    prefill bitwise, and with it on the result moves by a rounding-sized
    amount (so the switch is wired)."""
    bcfg = synth.backbone(1).replace(prefix_len=9, batch=1)
    W = oracle.decode_backbone_weights(synth.make_backbone_weights(bcfg, seed=5))
    d = oracle.BackboneDims.from_config(bcfg)
    emb = oracle.decode_bf16(synth.make_embeddings(bcfg, seed=6))
    pk, pv = oracle.prefill(W, d, emb)
    mod = sys.modules["oracle.denoise"]
    calls = []
    orig = mod.quantize_per_token_e4m3
    try:
        mod.quantize_per_token_e4m3 = lambda a: (calls.append(a.shape), a)[1]
        qk, qv = oracle.prefill(W, d, emb, act_quant=True)
    finally:
        mod.quantize_per_token_e4m3 = orig
    assert np.array_equal(qk, pk) and np.array_equal(qv, pv)
    H, I, qd = bcfg.hidden, bcfg.intermediate, bcfg.n_q_heads * bcfg.head_dim
    assert calls == [(9, H), (9, qd), (9, H), (9, I)] * bcfg.n_layers
    qk, qv = oracle.prefill(W, d, emb, act_quant=True)
    rel = np.linalg.norm(qk - pk) / np.linalg.norm(pk)
    assert 1e-4 < rel < 0.1


def test_backbone_fp8_weights_decode_to_row_scaled_codes():
    """The E4M3 backbone linears decode to code value x row scale within one
    E4M3 rounding of the same float32 draws (relative 2^-4 per element, the
    row maximum exact to 2^-4 of itself)."""
    bcfg = synth.backbone(1)
    raw8 = synth.make_backbone_weights(bcfg, seed=2, weight_dtype="fp8_e4m3")
    rawb = synth.make_backbone_weights(bcfg, seed=2)
    W8 = oracle.decode_backbone_weights(raw8)
    Wb = oracle.decode_backbone_weights(rawb)
    for name in ("wq", "wo", "wd"):
        a, b = W8[name][1], Wb[name][1]
        assert a.shape == b.shape
        row_max = np.abs(b).max(axis=1, keepdims=True)
        assert np.all(np.abs(a - b) <= 2.0 ** -4 * np.abs(b) + 2.0 ** -9 * row_max / 448 * 2 + 2.0 ** -8 * row_max)
        np.testing.assert_allclose(np.abs(a).max(axis=1), row_max[:, 0], rtol=2.0 ** -4)


# ---------------------------------------------------------------------------
# The backbone layer's body: closed forms and a composition of torch routines
# ("LingBot-VLA on Thor (sm_110)", section 1: the prefix model whose per-layer
# self-attention builds the cache; the layer reading is the plain pre-norm
# decoder layer)
# ---------------------------------------------------------------------------

def _bb_dims(**kw):
    base = dict(n_layers=1, hidden=24, n_q_heads=4, n_kv_heads=2, head_dim=8, intermediate=40, prefix_len=9)
    base.update(kw)
    return oracle.BackboneDims(**base)


def _bb_weights(d, seed=0, std=0.3):
    r = np.random.default_rng(seed)
    H, I = d.hidden, d.intermediate
    qd, kvd = d.n_q_heads * d.head_dim, d.n_kv_heads * d.head_dim
    g = lambda *s: r.standard_normal(s) * std
    W = {"n1": [1.0 + 0.5 * r.standard_normal(H)], "n2": [1.0 + 0.5 * r.standard_normal(H)],
         "wq": [g(qd, H)], "wk": [g(kvd, H)], "wv": [g(kvd, H)], "wo": [g(H, qd)], "wg": [g(I, H)],
         "wu": [g(I, H)], "wd": [g(H, I)]}
    return W


def _rms_rows(x, w, eps):
    """x / rms(x) * w with the RMS from numpy.linalg.norm."""
    return x / np.sqrt(np.linalg.norm(x, axis=1, keepdims=True) ** 2 / x.shape[1] + eps) * w


def test_backbone_uniform_causal_attention_closed_form():
    """W_q = W_k = 0: every score is 0, so token t's head output is the mean of
    the values of tokens 0..t of its KV group; W_g = 0 closes the MLP (SiLU(0)
    = 0).  The layer adds exactly that mean times W_o, its keys are zero, and
    its values are W_v applied to the first norm (weight n1, not n2)."""
    d = _bb_dims()
    W = _bb_weights(d)
    W["wq"][0][:] = 0.0
    W["wk"][0][:] = 0.0
    W["wg"][0][:] = 0.0
    x = RNG.standard_normal((d.prefix_len, d.hidden)) * 2.0
    xo, k, v = oracle.backbone_layer(x, W, 0, d)
    y = _rms_rows(x, W["n1"][0], d.rms_eps)
    vv = (y @ W["wv"][0].T).reshape(d.prefix_len, d.n_kv_heads, d.head_dim)
    grp = d.n_q_heads // d.n_kv_heads
    o = np.empty((d.prefix_len, d.n_q_heads * d.head_dim))
    for t in range(d.prefix_len):
        mean_t = vv[:t + 1].mean(axis=0)
        o[t] = np.concatenate([mean_t[j // grp] for j in range(d.n_q_heads)])
    np.testing.assert_allclose(xo, x + o @ W["wo"][0].T, rtol=0, atol=1e-12)
    assert np.all(k == 0.0)
    np.testing.assert_allclose(v, vv.transpose(1, 0, 2), rtol=0, atol=1e-13)


def test_backbone_zeroed_outputs_are_identity():
    """W_o = W_d = 0: both residual branches add nothing, x passes unchanged."""
    d = _bb_dims()
    W = _bb_weights(d)
    W["wo"][0][:] = 0.0
    W["wd"][0][:] = 0.0
    x = RNG.standard_normal((d.prefix_len, d.hidden))
    xo, _, _ = oracle.backbone_layer(x, W, 0, d)
    assert np.array_equal(xo, x)


def test_backbone_mlp_reads_the_second_norm_of_the_attention_residual():
    """The MLP branch takes RMSNorm(x + attention) * n2.  With W_q = W_k = 0 the
    attention residual has the closed form of the uniform causal mean, so the
    whole layer is written out here; a mix-up of n1 and n2, or an MLP reading
    x before the attention residual, fails."""
    d = _bb_dims()
    W = _bb_weights(d)
    W["wq"][0][:] = 0.0
    W["wk"][0][:] = 0.0
    x = RNG.standard_normal((d.prefix_len, d.hidden))
    xo, _, _ = oracle.backbone_layer(x, W, 0, d)
    y = _rms_rows(x, W["n1"][0], d.rms_eps)
    vv = (y @ W["wv"][0].T).reshape(d.prefix_len, d.n_kv_heads, d.head_dim)
    grp = d.n_q_heads // d.n_kv_heads
    o = np.stack([np.concatenate([vv[:t + 1].mean(axis=0)[j // grp] for j in range(d.n_q_heads)])
                  for t in range(d.prefix_len)])
    x1 = x + o @ W["wo"][0].T

    def mlp(xin, nw):
        y2 = _rms_rows(xin, nw, d.rms_eps)
        gz = y2 @ W["wg"][0].T
        return (gz * scipy.special.expit(gz) * (y2 @ W["wu"][0].T)) @ W["wd"][0].T

    np.testing.assert_allclose(xo, x1 + mlp(x1, W["n2"][0]), rtol=0, atol=1e-12)
    assert np.abs(xo - (x1 + mlp(x1, W["n1"][0]))).max() > 1e-3       # n1 in the MLP
    assert np.abs(xo - (x1 + mlp(x, W["n2"][0]))).max() > 1e-3         # MLP on pre-attention x


def _torch_rope(u: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    """Rotary embedding written as complex multiplication: the pair
    (u_m, u_{m+d/2}) is the complex number u_m + i u_{m+d/2}, turned by
    exp(i pos theta^(-2m/d))."""
    d = u.shape[-1]
    half = d // 2
    z = torch.complex(u[..., :half], u[..., half:])
    freq = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / d)
    rot = torch.polar(torch.ones(pos.shape[0], half, dtype=torch.float64), pos[:, None].double() * freq[None])
    w = z * rot
    return torch.cat([w.real, w.imag], dim=-1)


def test_backbone_layer_matches_torch_composition():
    """The whole layer against torch's own routines (rms_norm, linear,
    scaled_dot_product_attention with is_causal and grouped KV heads, silu)
    and the complex-number RoPE at positions 0..P-1, for layer 1 of a
    two-layer set of weights."""
    F = torch.nn.functional
    d = _bb_dims(n_layers=2)
    W0, W1 = _bb_weights(d, seed=3), _bb_weights(d, seed=4)
    W = {k: W0[k] + W1[k] for k in W0}
    x = RNG.standard_normal((d.prefix_len, d.hidden))
    xo, k, v = oracle.backbone_layer(x, W, 1, d)
    T = lambda a: torch.tensor(a, dtype=torch.float64)
    P, H, nq, nkv, dh = d.prefix_len, d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim
    xt = T(x)
    y = F.rms_norm(xt, (H,), T(W1["n1"][0]), eps=d.rms_eps)
    q = F.linear(y, T(W1["wq"][0])).reshape(P, nq, dh).transpose(0, 1)
    kt = F.linear(y, T(W1["wk"][0])).reshape(P, nkv, dh).transpose(0, 1)
    vt = F.linear(y, T(W1["wv"][0])).reshape(P, nkv, dh).transpose(0, 1)
    pos = torch.arange(P)
    q, kt = _torch_rope(q, pos, d.rope_theta), _torch_rope(kt, pos, d.rope_theta)
    o = F.scaled_dot_product_attention(q[None], kt[None], vt[None], is_causal=True, enable_gqa=True)[0]
    x1 = xt + F.linear(o.transpose(0, 1).reshape(P, nq * dh), T(W1["wo"][0]))
    y2 = F.rms_norm(x1, (H,), T(W1["n2"][0]), eps=d.rms_eps)
    x2 = x1 + F.linear(F.silu(F.linear(y2, T(W1["wg"][0]))) * F.linear(y2, T(W1["wu"][0])), T(W1["wd"][0]))
    np.testing.assert_allclose(xo, x2.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(k, kt.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(v, vt.numpy(), rtol=0, atol=1e-12)


def test_expert_layer_matches_torch_composition():
    """One expert layer against torch's routines: rms_norm with the (1 +
    scale) / shift modulation, linear, the complex-number RoPE at positions
    P + i, unmasked scaled_dot_product_attention over [prefix ; chunk] keys
    with grouped KV heads, the two gated residuals and the SwiGLU MLP."""
    F = torch.nn.functional
    d = _tiny_dims(n_layers=2)
    W = _tiny_weights(d, seed=5)
    pk, pv, _ = _tiny_inputs(d, seed=6)
    h = RNG.standard_normal((d.horizon, d.hidden))
    l = 1
    mod = oracle.modulation(RNG.standard_normal(d.hidden), W["mod_w"][l], W["mod_b"][l], 6)
    got = oracle.expert_layer(h, W, l, mod, pk[0, l], pv[0, l], d)
    T = lambda a: torch.tensor(a, dtype=torch.float64)
    a1, b1, g1, a2, b2, g2 = (T(z) for z in mod)
    Tn, H, nq, nkv, dh, P = d.horizon, d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim, d.prefix_len
    ht = T(h)
    y = F.rms_norm(ht, (H,), eps=d.rms_eps) * (1 + a1) + b1
    q = F.linear(y, T(W["wq"][l])).reshape(Tn, nq, dh).transpose(0, 1)
    k = F.linear(y, T(W["wk"][l])).reshape(Tn, nkv, dh).transpose(0, 1)
    v = F.linear(y, T(W["wv"][l])).reshape(Tn, nkv, dh).transpose(0, 1)
    pos = P + torch.arange(Tn)
    q, k = _torch_rope(q, pos, d.rope_theta), _torch_rope(k, pos, d.rope_theta)
    K = torch.cat([T(pk[0, l]).transpose(0, 1), k], dim=1)
    V = torch.cat([T(pv[0, l]).transpose(0, 1), v], dim=1)
    o = F.scaled_dot_product_attention(q[None], K[None], V[None], enable_gqa=True)[0]
    h1 = ht + g1 * F.linear(o.transpose(0, 1).reshape(Tn, nq * dh), T(W["wo"][l]))
    y2 = F.rms_norm(h1, (H,), eps=d.rms_eps) * (1 + a2) + b2
    h2 = h1 + g2 * F.linear(F.silu(F.linear(y2, T(W["wg"][l]))) * F.linear(y2, T(W["wu"][l])), T(W["wd"][l]))
    np.testing.assert_allclose(got, h2.numpy(), rtol=0, atol=1e-12)
