"""The synthetic-input recipe (no GPU): every input is a pure function of its
seed and request, with the stated shapes and distributions.

* Weights: float32 N(0, 1) * weight_std per (model, tensor, layer) stream,
  stored as the round-to-nearest-even bf16 of that draw; the LingBot-shaped
  workloads share one model, so they share weights.
* Prefix K/V and noise: N(0, 1) per request stream, so a request's inputs do
  not depend on which batch it sits in.
* Schedules: uniform t_k = k / N in float32; the warped variant is monotone
  with exact end points and t_k = (k / N)^p for one p in [0.5, 2] per request.
* Structured variants change exactly the tensors they name.
"""
import numpy as np
import pytest

import synth


def _bf16(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_weights_are_a_pure_function_of_the_seed():
    cfg = synth.config(1)
    a, b, c = synth.make_weights(cfg, seed=0), synth.make_weights(cfg, seed=0), synth.make_weights(cfg, seed=1)
    for name in ("in_w", "wq", "wd", "mod_w"):
        x, y, z = a[name], b[name], c[name]
        x, y, z = (v[0] if isinstance(v, list) else v for v in (x, y, z))
        assert np.array_equal(x, y)
        assert not np.array_equal(x, z)


def test_weights_are_the_rounded_scaled_normal_draw():
    cfg = synth.config(1)
    W = synth.make_weights(cfg, seed=0)
    draw = synth._draw(cfg, 0, "wg", 1, (cfg.intermediate, cfg.hidden))
    got = _bf16(W["wg"][1])
    assert np.array_equal(W["wg"][1], synth.to_bf16_bits(draw))
    # bf16 keeps 8 significant bits: within half an ulp (2^-8 relative) of the draw
    assert np.all(np.abs(got - draw) <= np.abs(draw) * 2.0 ** -8 + 1e-30)
    assert abs(float(np.mean(got))) < 0.02 * 0.05
    assert float(np.std(got)) == pytest.approx(cfg.weight_std, rel=0.03)


def test_lingbot_workloads_share_one_model():
    c2, c4, c5 = synth.config(2), synth.config(4), synth.config(5)
    assert c2.model_tag == c4.model_tag == c5.model_tag
    shape = (c2.n_q_heads * c2.head_dim, c2.hidden)
    assert np.array_equal(synth._draw(c2, 0, "wq", 7, shape), synth._draw(c5, 0, "wq", 7, shape))
    assert synth.config(3).model_tag != c2.model_tag          # the V2-shaped loop is its own model


def test_prefix_and_noise_follow_the_request_not_the_batch():
    cfg = synth.config(1).replace(batch=3)
    k, v = synth.make_prefix(cfg)
    x = synth.make_noise(cfg)
    assert k.shape == (3, cfg.n_layers, cfg.prefix_len, cfg.n_kv_heads, cfg.head_dim) and k.dtype == np.uint16
    assert v.shape == k.shape and v.dtype == np.uint16
    assert x.shape == (3, cfg.horizon, cfg.action_dim) and x.dtype == np.float32
    k2, v2 = synth.make_prefix(cfg, requests=[2])
    assert np.array_equal(k2[0], k[2]) and np.array_equal(v2[0], v[2])
    assert np.array_equal(synth.make_noise(cfg, requests=[1])[0], x[1])
    assert not np.array_equal(k[0], k[1]) and not np.array_equal(k[0], v[0])


def test_prefix_and_noise_are_standard_normal():
    cfg = synth.config(1).replace(batch=4)
    k, v = synth.make_prefix(cfg)
    x = synth.make_noise(cfg.replace(batch=64))
    for s in (_bf16(k), _bf16(v), x):
        s = s.astype(np.float64).ravel()
        assert s.size > 4000
        assert abs(s.mean()) < 4 / np.sqrt(s.size)
        assert s.std() == pytest.approx(1.0, abs=6 / np.sqrt(s.size))


def test_uniform_schedule():
    ts = synth.make_schedule(10, 3)
    assert ts.shape == (3, 11) and ts.dtype == np.float32
    want = np.arange(11, dtype=np.float32) / np.float32(10)
    assert np.array_equal(ts, np.tile(want, (3, 1)))


def test_warped_schedule():
    n, B = 10, 64
    ts = synth.make_schedule(n, B, "warped").astype(np.float64)
    assert ts.shape == (B, n + 1)
    assert np.all(ts[:, 0] == 0.0) and np.all(ts[:, -1] == 1.0)
    assert np.all(np.diff(ts, axis=1) > 0)
    u = np.arange(1, n) / n
    assert np.all(ts[:, 1:-1] >= u ** 2 - 1e-6) and np.all(ts[:, 1:-1] <= u ** 0.5 + 1e-6)
    # one exponent per request: log t_k / log u_k is the same for every interior k
    p = np.log(ts[:, 1:-1]) / np.log(u)
    assert np.allclose(p, p[:, :1], rtol=1e-5)
    assert np.ptp(p[:, 0]) > 0.5                             # the requests differ
    assert np.array_equal(synth.make_schedule(n, B, "warped"), synth.make_schedule(n, B, "warped"))


def test_structured_variants_touch_only_their_tensors():
    cfg = synth.config(1)
    W = synth.make_weights(cfg, seed=0)
    H = cfg.hidden
    g = synth.apply_variant(W, "gate_open", cfg)
    for b0, b1 in zip(W["mod_b"], g["mod_b"]):
        for lo, hi in ((2 * H, 3 * H), (5 * H, 6 * H)):          # the two gate chunks, + 1 in float32
            assert np.array_equal(b1[lo:hi], b0[lo:hi] + np.float32(1.0))
        for lo, hi in ((0, 2 * H), (3 * H, 5 * H)):
            assert np.array_equal(b1[lo:hi], b0[lo:hi])
    assert all(np.array_equal(a, b) for a, b in zip(W["wq"], g["wq"]))
    u = np.linspace(-1, 1, cfg.action_dim).astype(np.float32)
    cv = synth.apply_variant(W, "const_velocity", cfg, velocity_bias=u)
    assert not np.any(cv["out_w"]) and np.array_equal(cv["out_b"], u)
    assert np.array_equal(cv["in_w"], W["in_w"])
    z = synth.apply_variant(W, "zero_blocks", cfg)
    for name in synth.BLOCK_LINEARS:
        assert all(not np.any(a) for a in z[name])
    assert np.array_equal(z["mod_w"][0], W["mod_w"][0])
    assert all(np.any(a) for a in W["wq"])                    # the source set is left as it was
