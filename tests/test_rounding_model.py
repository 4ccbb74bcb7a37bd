"""The rounding model (tests/rounding_model.py) that derives the depth-scaled
and gate-open tolerances: with its rounding switched off it is the oracle, its
bf16 rounding is torch's, and at the LingBot backbone widths its first layers'
cache error stays inside the depth-scaled gate the prefill tests use."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import rounding_model as rm


def test_bf16_round_matches_torch_cast():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(20000) * 10.0 ** r.integers(-6, 6, 20000),
                        [0.0, -0.0, 1.0, 65504.0, 1e-30, 3.0e38]])
    want = torch.tensor(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(rm.bf16_round(x), want)


def test_model_without_rounding_is_the_oracle():
    cfg = synth.config(1).replace(n_steps=3, batch=2)
    W = oracle.decode_weights(synth.make_weights(cfg))
    d = oracle.ExpertDims.from_config(cfg)
    pk, pv = (oracle.decode_bf16(a) for a in synth.make_prefix(cfg))
    x0 = synth.make_noise(cfg)
    ts = synth.make_schedule(3, 2, "warped")
    ident = lambda z: z
    np.testing.assert_allclose(rm.denoise_r(W, d, pk, pv, x0, ts, rnd=ident),
                               oracle.denoise(W, d, pk, pv, x0, ts), rtol=0, atol=1e-12)
    bcfg = synth.backbone(1).replace(prefix_len=20)
    Wb = oracle.decode_backbone_weights(synth.make_backbone_weights(bcfg, seed=1))
    db = oracle.BackboneDims.from_config(bcfg)
    emb = oracle.decode_bf16(synth.make_embeddings(bcfg, seed=1))
    ks, vs = rm.prefill_r(Wb, db, emb[0], rnd=ident)
    rk, rv = oracle.prefill(Wb, db, emb)
    for l in range(bcfg.n_layers):
        np.testing.assert_allclose(ks[l], rk[0, l].transpose(1, 0, 2), rtol=0, atol=1e-12)
        np.testing.assert_allclose(vs[l], rv[0, l].transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_model_rounding_moves_the_tiny_loop_by_a_bf16_sized_amount():
    cfg = synth.config(1)
    W = oracle.decode_weights(synth.make_weights(cfg))
    d = oracle.ExpertDims.from_config(cfg)
    pk, pv = (oracle.decode_bf16(a) for a in synth.make_prefix(cfg))
    x0 = synth.make_noise(cfg)
    ts = synth.make_schedule(cfg.n_steps, 1)
    exact = oracle.denoise(W, d, pk, pv, x0, ts)
    model = rm.denoise_r(W, d, pk, pv, x0, ts)
    rel = np.linalg.norm(model - exact) / np.linalg.norm(exact)
    assert 1e-7 < rel < 1e-3, rel      # small gates (about 0.05) damp the block errors


@pytest.mark.slow
def test_prefill_depth_gate_holds_for_the_model_at_lingbot_widths():
    """The first two layers of the LingBot-shaped backbone at P = 64: the
    modelled cache error, max-abs / RMS, stays under 2e-2 * sqrt(l + 1)."""
    for l, mk, mv, ratio in rm.prefill_depth_table(n_layers=2, prefix_len=64):
        assert max(mk, mv) <= 2e-2 * math.sqrt(l + 1), (l, mk, mv)
        assert mk > 1e-4 and mv > 1e-4          # the model does round


@pytest.mark.slow
def test_batched_e4m3_gate_covers_the_modelled_code_flips():
    """The batched E4M3 tier's gate (cosine >= 0.999, max-abs <= 0.3 x RMS
    against the oracle with per-token E4M3 inputs, tests/test_gpu_fp8_batched.py)
    derived from arithmetic: the rounding model, which stores bf16 where the
    kernels do before quantizing the attention and SwiGLU outputs, moves the
    gate-open layer of that test (LingBot widths, 8 requests, layer 1, step 3)
    by max-abs ~0.15 x RMS from the exact quantized oracle, because inputs
    near an E4M3 rounding boundary take the neighbouring code. The gate allows
    at least 1.5 times that modelled deviation (and twice its cosine
    distance)."""
    from tests.gpu_util import metrics
    cfg = synth.config(4).replace(n_layers=2, batch=8)
    raw = synth.apply_variant(synth.make_weights(cfg, seed=0), "gate_open", cfg)
    pk, pv = synth.make_prefix(cfg)
    ts = synth.make_schedule(cfg.n_steps, cfg.batch, "warped")
    h_in = np.random.default_rng(7).standard_normal((cfg.m_rows, cfg.hidden)).astype(np.float32)
    layer, step, T = 1, 3, cfg.horizon
    W = oracle.decode_weights(raw)
    d = oracle.ExpertDims.from_config(cfg)
    fpk, fpv = oracle.decode_bf16(pk), oracle.decode_bf16(pv)
    exact = np.empty((cfg.batch, T, cfg.hidden))
    model = np.empty_like(exact)
    for b in range(cfg.batch):
        c = oracle.time_condition(float(ts[b, step]), W, d)
        mod = oracle.modulation(c, W["mod_w"][layer], W["mod_b"][layer], 6)
        mod_r = oracle.modulation(rm.bf16_round(c), W["mod_w"][layer], W["mod_b"][layer], 6)
        hb = h_in[b * T:(b + 1) * T].astype(np.float64)
        exact[b] = oracle.expert_layer(hb, W, layer, mod, fpk[b, layer], fpv[b, layer], d, act_quant=True) - hb
        model[b] = rm.expert_layer_r(hb, W, layer, mod_r, fpk[b, layer], fpv[b, layer], d, act_quant=True) - hb
    m = metrics(model, exact)
    assert 0.05 < m["maxabs_over_rms"] and 1.5 * m["maxabs_over_rms"] <= 0.3, m
    assert 1.0 - 2.0 * (1.0 - m["min_req_cos"]) >= 0.999, m
