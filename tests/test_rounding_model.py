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
