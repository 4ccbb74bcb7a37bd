"""GPU parity of the E4M3 + MXFP4 gate_up tier (weight streaming, batch *
horizon <= 64): gate and up in OCP MXFP4 (E2M1, E8M0 scale per 32 inputs),
the other block linears in E4M3 with per-row scales, activations bf16.

The oracle decodes the same encodings, so against it the bf16 gates apply
(cosine >= 0.9995, max-abs <= 2e-2 * RMS). Against the oracle on the
unquantized bf16 weights the acceptance of the LingBot-VLA on Thor page
(section 5: cosine >= 0.995 against the step-matched BF16 reference, met by
its FP8 + FP4 gate_up expert at 10 steps) is checked at 10 steps.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import BF16_COS, BF16_MAXABS, FP8_COS, GpuCase, metrics, run_oracle, say

pytestmark = pytest.mark.gpu


def _cfg(**kw):
    return synth.config(4).replace(weight_dtype="fp8_mxfp4gu", **kw)


def test_mxfp4_gate_up_lingbot_b1_end_to_end():
    cfg = _cfg(n_steps=10)
    raw = synth.make_weights(cfg, seed=0)
    pk, pv = synth.make_prefix(cfg)
    x0 = synth.make_noise(cfg)
    ts = synth.make_schedule(cfg.n_steps, cfg.batch)
    say("[mxfp4 gate_up] LingBot shapes, 36 layers, 10 steps, batch 1")
    case = GpuCase(cfg, raw, pk, pv, x0, ts)
    try:
        out = case.run()
    finally:
        case.close()
    ref = run_oracle(cfg, oracle.decode_weights(raw), pk, pv, x0, ts)
    m = metrics(out, ref)
    say(f"[mxfp4 gate_up] vs oracle on the same encodings: {m}")
    assert m["cos"] >= BF16_COS and m["maxabs_over_rms"] <= BF16_MAXABS, m
    ref_bf16 = run_oracle(cfg, oracle.decode_weights(synth.make_weights(cfg, seed=0, weight_dtype="bf16")),
                          pk, pv, x0, ts)
    m = metrics(out, ref_bf16)
    say(f"[mxfp4 gate_up] vs bf16-weight oracle: {m}")
    assert m["cos"] >= FP8_COS, m


@pytest.mark.parametrize("batch,horizon", [(1, 50), (3, 21)])
def test_mxfp4_gate_up_single_layer(batch, horizon):
    """One layer with the gates open (block output large against the
    residual), ragged row counts."""
    import torch
    from vla_flow_matching_denoise_amd import binding as B
    from vla_flow_matching_denoise_amd.expert import Expert, dims_from_config, to_device
    cfg = _cfg(n_layers=2, batch=batch, horizon=horizon)
    raw = synth.apply_variant(synth.make_weights(cfg, seed=4), "gate_open", cfg)
    pk, pv = synth.make_prefix(cfg, seed=5)
    ts = synth.make_schedule(cfg.n_steps, batch, "warped")
    h_in = np.random.default_rng(9).standard_normal((cfg.m_rows, cfg.hidden)).astype(np.float32)
    layer, step, T = 1, 2, cfg.horizon
    Wd = oracle.decode_weights(raw)
    d = oracle.ExpertDims.from_config(cfg)
    fpk, fpv = oracle.decode_bf16(pk), oracle.decode_bf16(pv)
    want = np.empty((batch, T, cfg.hidden))
    for b in range(batch):
        c = oracle.time_condition(float(ts[b, step]), Wd, d)
        mod = oracle.modulation(c, Wd["mod_w"][layer], Wd["mod_b"][layer], 6)
        hb = h_in[b * T:(b + 1) * T].astype(np.float64)
        want[b] = oracle.expert_layer(hb, Wd, layer, mod, fpk[b, layer], fpv[b, layer], d) - hb
    ex = Expert(raw, dims_from_config(cfg))
    try:
        dpk, dpv, dts, hi = (to_device(a) for a in (pk, pv, ts, h_in))
        ho = torch.empty_like(hi)
        B.vla_test_layer(ex.ctx, dpk.data_ptr(), dpv.data_ptr(), dts.data_ptr(), cfg.n_steps, step, layer,
                         hi.data_ptr(), ho.data_ptr())
        got = (ho.cpu().numpy() - h_in).reshape(batch, T, -1)
    finally:
        ex.close()
    m = metrics(got, want)
    say(f"[mxfp4 layer b{batch} T{horizon}] {m}")
    assert m["min_req_cos"] >= BF16_COS and m["maxabs_over_rms"] <= BF16_MAXABS, m
