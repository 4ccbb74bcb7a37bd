"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Gates (floating point, fp32 accumulation): cosine >= 0.9995 and
max|gpu - oracle| <= 2e-2 * RMS(oracle) for bf16 weights; cosine >= 0.995
for E4M3 weights against the oracle on the unquantized bf16 weights.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (BF16_COS, BF16_MAXABS, FP8_COS, GpuCase, decoded, metrics, run_oracle, say,
                            weights)

pytestmark = pytest.mark.gpu


def _inputs(cfg, requests=None, schedule="uniform", n_steps=None):
    pk, pv = synth.make_prefix(cfg, requests=requests)
    x0 = synth.make_noise(cfg, requests=requests)
    n = cfg.n_steps if n_steps is None else n_steps
    ts = synth.make_schedule(n, x0.shape[0], schedule)
    return pk, pv, x0, ts


def _gate_bf16(m, tag):
    say(f"[{tag}] cos={m['cos']:.7f} min_req_cos={m['min_req_cos']:.7f} "
        f"maxabs/rms={m['maxabs_over_rms']:.3e} rel_l2={m['rel_l2']:.3e}")
    assert m["cos"] >= BF16_COS, m
    assert m["maxabs_over_rms"] <= BF16_MAXABS, m


# ---------------------------------------------------------------------------
# tiny workload: end to end, graph vs eager, determinism, edge cases
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny():
    cfg = synth.config(1)
    raw = weights(1)
    pk, pv, x0, ts = _inputs(cfg)
    case = GpuCase(cfg, raw, pk, pv, x0, ts)
    ref = run_oracle(cfg, decoded(1), pk, pv, x0, ts)
    yield cfg, case, ref, (pk, pv, x0, ts)
    case.close()


def test_tiny_end_to_end(tiny):
    cfg, case, ref, _ = tiny
    say("[tiny] end to end, 10 steps")
    out = case.run()
    _gate_bf16(metrics(out, ref), "tiny")


def test_tiny_graph_equals_eager_and_replays_bitwise(tiny):
    from vla_flow_matching_denoise_amd import binding as B
    cfg, case, ref, _ = tiny
    a = case.run()
    b = case.run()
    case.expert.set_option(B.VLA_OPT_USE_GRAPH, 0)
    try:
        c = case.run()
    finally:
        case.expert.set_option(B.VLA_OPT_USE_GRAPH, 1)
    assert np.array_equal(a, b), "two graph replays differ"
    assert np.array_equal(a, c), "graph replay differs from eager launch"


def test_tiny_step_counts_and_single_step(tiny):
    cfg, case, _, (pk, pv, x0, _) = tiny
    W = decoded(1)
    for n in (1, 3):
        ts = synth.make_schedule(n, 1)
        import torch
        from vla_flow_matching_denoise_amd.expert import to_device
        tsd = to_device(ts)
        out = case.expert.denoise(case.pk, case.pv, case.x0, tsd, n)
        torch.cuda.synchronize()
        ref = run_oracle(cfg, W, pk, pv, x0, ts)
        _gate_bf16(metrics(out.cpu().numpy(), ref), f"tiny n_steps={n}")


def test_tiny_in_place_output(tiny):
    import torch
    cfg, case, ref, _ = tiny
    x = case.x0.clone()
    case.expert.denoise(case.pk, case.pv, x, case.ts, cfg.n_steps, out=x)
    torch.cuda.synchronize()
    _gate_bf16(metrics(x.cpu().numpy(), ref), "tiny in-place")


def test_tiny_structured_closed_forms():
    """Constant velocity (exact x0 + u) and zeroed blocks, on the GPU."""
    cfg = synth.config(1)
    pk, pv, x0, ts = _inputs(cfg)
    u = np.random.default_rng(7).standard_normal(cfg.action_dim).astype(np.float32)
    raw = synth.apply_variant(weights(1), "const_velocity", cfg, velocity_bias=u)
    case = GpuCase(cfg, raw, pk, pv, x0, ts)
    try:
        out = case.run()
    finally:
        case.close()
    # fp32 Euler sum of 10 steps of a constant field: exact up to fp32 rounding
    assert np.allclose(out, x0 + u[None, None, :], atol=1e-5, rtol=0)
    raw = synth.apply_variant(weights(1), "zero_blocks", cfg)
    case = GpuCase(cfg, raw, pk, pv, x0, ts)
    try:
        out = case.run()
    finally:
        case.close()
    ref = run_oracle(cfg, oracle.decode_weights(raw), pk, pv, x0, ts)
    _gate_bf16(metrics(out, ref), "tiny zero_blocks")


def test_tiny_gate_open_sensitivity():
    """Gate-open weights: block outputs dominate the residual (diagnostic gate)."""
    cfg = synth.config(1)
    pk, pv, x0, ts = _inputs(cfg)
    raw = synth.apply_variant(weights(1), "gate_open", cfg)
    case = GpuCase(cfg, raw, pk, pv, x0, ts)
    try:
        out = case.run()
    finally:
        case.close()
    ref = run_oracle(cfg, oracle.decode_weights(raw), pk, pv, x0, ts)
    m = metrics(out, ref)
    say(f"[tiny gate_open] {m}")
    assert m["cos"] >= 0.999, m


@pytest.mark.parametrize("prefix_len,horizon,batch", [(0, 16, 1), (5, 13, 3), (40, 33, 2)])
def test_ragged_shapes(prefix_len, horizon, batch):
    """No prefix, ragged chunk lengths (not multiples of 16) and batches."""
    cfg = synth.config(1).replace(prefix_len=prefix_len, horizon=horizon, batch=batch, n_steps=4)
    raw = weights(1)
    pk, pv, x0, ts = _inputs(cfg, schedule="warped")
    if prefix_len == 0:
        pk = np.zeros((batch, cfg.n_layers, 1, cfg.n_kv_heads, cfg.head_dim), np.uint16)
        pv = pk.copy()
    case = GpuCase(cfg, raw, pk, pv, x0, ts)
    try:
        out = case.run()
    finally:
        case.close()
    if prefix_len == 0:
        pk = pk[:, :, :0]
        pv = pv[:, :, :0]
    ref = run_oracle(cfg, decoded(1), pk, pv, x0, ts)
    _gate_bf16(metrics(out, ref), f"ragged P={prefix_len} T={horizon} B={batch}")


@pytest.mark.parametrize("hidden,intermediate", [(1536, 6144), (2048, 5632)])
def test_wide_hidden_batched_rows(hidden, intermediate):
    """Hidden above 1024 (up to the 2048 maximum) with more than 64 rows: the
    tiled GEMMs and the wave-per-row residual + norm with 8 float4 chunks per
    lane. Two layers, two requests on warped schedules, three steps."""
    cfg = synth.config(3).replace(n_layers=2, hidden=hidden, intermediate=intermediate, prefix_len=64,
                                  horizon=50, batch=2, n_steps=3)
    raw = synth.make_weights(cfg, seed=5)
    pk, pv, x0, ts = _inputs(cfg, schedule="warped")
    say(f"[wide] hidden {hidden}, SwiGLU {intermediate}, 2 layers, B=2 (M=100), 3 steps")
    case = GpuCase(cfg, raw, pk, pv, x0, ts)
    try:
        out = case.run()
    finally:
        case.close()
    ref = run_oracle(cfg, oracle.decode_weights(raw), pk, pv, x0, ts)
    _gate_bf16(metrics(out, ref), f"wide h{hidden}")


# ---------------------------------------------------------------------------
# stage parity
# ---------------------------------------------------------------------------

def test_modulation_table_stage():
    import torch
    from vla_flow_matching_denoise_amd import binding as B
    from vla_flow_matching_denoise_amd.expert import to_device
    cfg = synth.config(1).replace(batch=2)
    raw = weights(1)
    pk, pv, x0, ts = _inputs(cfg, schedule="warped")
    case = GpuCase(cfg, raw, pk, pv, x0, ts)
    try:
        L, H, N = cfg.n_layers, cfg.hidden, cfg.n_steps
        mod = torch.empty((N, 2, 6 * L + 2, H), dtype=torch.float32, device="cuda")
        B.vla_test_modulation(case.expert.ctx, case.ts.data_ptr(), N, mod.data_ptr())
        got = mod.cpu().numpy()
    finally:
        case.close()
    W = decoded(1)
    d = oracle.ExpertDims.from_config(cfg)
    for k in (0, 5, N - 1):
        for b in range(2):
            c = oracle.time_condition(float(ts[b, k]), W, d)
            want = np.concatenate([np.concatenate(oracle.modulation(c, W["mod_w"][l], W["mod_b"][l], 6))
                                   for l in range(L)] +
                                  [np.concatenate(oracle.modulation(c, W["modf_w"], W["modf_b"], 2))])
            g = got[k, b].ravel()
            rms = np.sqrt(np.mean(want ** 2))
            assert oracle.cosine(g, want) >= 0.99999
            assert np.max(np.abs(g - want)) <= 1e-2 * rms


@pytest.mark.parametrize("cfg_id", [1, 2, 4])
def test_single_layer_stage(cfg_id):
    import torch
    from vla_flow_matching_denoise_amd import binding as B
    from vla_flow_matching_denoise_amd.expert import to_device
    cfg = synth.config(cfg_id)
    raw = weights(cfg_id)
    pk, pv, x0, ts = _inputs(cfg)
    # gate-open weights make the block's own output large against the residual
    raw = synth.apply_variant(raw, "gate_open", cfg)
    case = GpuCase(cfg, raw, pk, pv, x0, ts)
    rng = np.random.default_rng(3)
    h_in = rng.standard_normal((cfg.m_rows, cfg.hidden)).astype(np.float32)
    try:
        hi = to_device(h_in)
        ho = torch.empty_like(hi)
        layer, step = cfg.n_layers - 1, 3
        B.vla_test_layer(case.expert.ctx, case.pk.data_ptr(), case.pv.data_ptr(), case.ts.data_ptr(),
                         cfg.n_steps, step, layer, hi.data_ptr(), ho.data_ptr())
        got = ho.cpu().numpy()
    finally:
        case.close()
    Wd = oracle.decode_weights(raw)
    d = oracle.ExpertDims.from_config(cfg)
    c = oracle.time_condition(float(ts[0, step]), Wd, d)
    mod = oracle.modulation(c, Wd["mod_w"][layer], Wd["mod_b"][layer], 6)
    want = oracle.expert_layer(h_in.astype(np.float64), Wd, layer, mod, oracle.decode_bf16(pk)[0, layer],
                               oracle.decode_bf16(pv)[0, layer], d)
    delta_g, delta_w = got - h_in, want - h_in
    m = metrics(delta_g[None], delta_w[None])
    say(f"[layer cfg{cfg_id}] delta {m}")
    assert m["cos"] >= 0.9995 and m["maxabs_over_rms"] <= 2e-2, m


# small grids take the key-split kernel; (2, 12) and (1, 130) have enough
# 16-row tiles (>= 512) to take the 64-rows-per-workgroup kernel (d_h 128 / 64)
# (cfg, batch, prefix, horizon): few rows take the 8-wave kernel (prefix 280
# with T = 16 and prefix 320 with T = 50 give 10 and 12 key blocks: some
# waves take two, and the last block is partly padding); many rows take the
# row-tile kernels, 8 waves of 16 rows when a KV group has more than 64 rows
# (head dim 128: 12 requests of 400 rows; head dim 64: 64 requests of 100
# rows), else 4 waves (head dim 64: 130 requests of 32 rows; head dim 128:
# 64 requests of T = 8, 64 rows)
@pytest.mark.parametrize("cfg_id,batch,prefix,horizon", [
    (1, 1, None, None), (2, 1, None, None), (3, 1, None, None), (2, 3, None, None), (2, 12, None, None),
    (1, 130, None, None), (1, 1, 280, None), (2, 1, 320, None), (1, 64, None, 50), (2, 64, None, 8)])
def test_attention_stage(cfg_id, batch, prefix, horizon):
    import torch
    from vla_flow_matching_denoise_amd import binding as B
    from vla_flow_matching_denoise_amd.expert import Expert, dims_from_config, to_device
    cfg = synth.config(cfg_id).replace(n_layers=2, batch=batch)
    if prefix is not None:
        cfg = cfg.replace(prefix_len=prefix)
    if horizon is not None:
        cfg = cfg.replace(horizon=horizon)
    raw = synth.make_weights(cfg.replace(n_layers=2), seed=0)
    pk, pv = synth.make_prefix(cfg)
    rng = np.random.default_rng(11)
    T, nq, nkv, dh = cfg.horizon, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    q = synth.to_bf16_bits(rng.standard_normal((batch, nq, T, dh)).astype(np.float32))
    kn = synth.to_bf16_bits(rng.standard_normal((batch, nkv, T, dh)).astype(np.float32))
    vn = synth.to_bf16_bits(rng.standard_normal((batch, nkv, T, dh)).astype(np.float32))
    ex = Expert(raw, dims_from_config(cfg))
    try:
        o = torch.empty((batch * T, nq * dh), dtype=torch.int16, device="cuda")
        dq, dk, dv, dpk, dpv = (to_device(a) for a in (q, kn, vn, pk, pv))
        B.vla_test_attention(ex.ctx, dpk.data_ptr(), dpv.data_ptr(), 1, dq.data_ptr(), dk.data_ptr(),
                             dv.data_ptr(), o.data_ptr())
        got = oracle.decode_bf16(o.cpu().numpy().view(np.uint16))
    finally:
        ex.close()
    fq, fk, fv = (oracle.decode_bf16(a) for a in (q, kn, vn))
    fpk, fpv = oracle.decode_bf16(pk), oracle.decode_bf16(pv)
    for b in range(batch):
        K = np.concatenate([fpk[b, 1].transpose(1, 0, 2), fk[b]], axis=1)
        V = np.concatenate([fpv[b, 1].transpose(1, 0, 2), fv[b]], axis=1)
        want = oracle.gqa_attention(fq[b], K, V).transpose(1, 0, 2).reshape(T, nq * dh)
        g = got[b * T:(b + 1) * T]
        rms = np.sqrt(np.mean(want ** 2))
        assert oracle.cosine(g, want) >= 0.9999
        # The stage output is stored in bf16: each element may be off by half an
        # ulp of its own value (2^-9 relative; doubled here), on top of the
        # accumulation allowance. Peaked softmax rows reach |o| ~ 1.2 while the
        # RMS is ~0.1, so an RMS-only bound would reject correct rounding.
        assert np.all(np.abs(g - want) <= 2.0 ** -8 * np.abs(want) + 2e-2 * rms)


# ---------------------------------------------------------------------------
# full-size workloads
# ---------------------------------------------------------------------------

def test_lingbot_b1_end_to_end():
    cfg = synth.config(2)
    pk, pv, x0, ts = _inputs(cfg)
    say("[cfg2] 36 layers, h1024, chunk 50x75, 10 steps, batch 1")
    case = GpuCase(cfg, weights(2), pk, pv, x0, ts)
    try:
        out = case.run()
    finally:
        case.close()
    ref = run_oracle(cfg, decoded(2), pk, pv, x0, ts)
    _gate_bf16(metrics(out, ref), "cfg2")


@pytest.mark.timeout(600)
def test_v2_b1_end_to_end():
    """The V2-shaped loop: 36 layers, hidden 1536, SwiGLU 6144, prefix 512,
    chunk 50x55, 50 Euler steps, batch 1 (its weights are its own model)."""
    cfg = synth.config(3)
    pk, pv, x0, ts = _inputs(cfg)
    say("[cfg3] 36 layers, h1536, prefix 512, chunk 50x55, 50 steps, batch 1: generating weights")
    raw = synth.make_weights(cfg, seed=0)
    case = GpuCase(cfg, raw, pk, pv, x0, ts)
    try:
        from vla_flow_matching_denoise_amd import binding as B
        # gate_up's 37.7 MB of weights exceed the 32 MB of L2: no L2 read-ahead
        # by default (and, as everywhere, non-temporal weight reads)
        assert case.expert.get_option(B.VLA_OPT_WEIGHT_NT) == 1
        assert case.expert.get_option(B.VLA_OPT_L2_PREFETCH) == 0
        out = case.run()
    finally:
        case.close()
    say("[cfg3] GPU done; oracle")
    ref = run_oracle(cfg, oracle.decode_weights(raw), pk, pv, x0, ts)
    _gate_bf16(metrics(out, ref), "cfg3")


@pytest.mark.parametrize("weight_dtype", ["bf16", "fp8_e4m3"])
def test_weight_nt_option_bitwise(weight_dtype):
    """VLA_OPT_WEIGHT_NT changes only how the weight-streaming GEMMs read
    their weights (the non-temporal hint, or plain loads): on the tiny
    expert with bf16 and with E4M3 weights the output is bitwise the same
    either way. The defaults: non-temporal reads; the QKV read-ahead alone
    for bf16 weights of this size (they fit the L2), none for E4M3."""
    from vla_flow_matching_denoise_amd import binding as B
    cfg = synth.config(1)
    wd = None if weight_dtype == "bf16" else weight_dtype
    if wd:
        cfg = cfg.replace(weight_dtype=wd)
    pk, pv, x0, ts = _inputs(cfg)
    say(f"[weight nt] tiny expert, {weight_dtype} weights")
    case = GpuCase(cfg, weights(1, weight_dtype=wd), pk, pv, x0, ts)
    try:
        ex = case.expert
        assert ex.get_option(B.VLA_OPT_WEIGHT_NT) == 1
        assert ex.get_option(B.VLA_OPT_L2_PREFETCH) == (4 if weight_dtype == "bf16" else 0)
        ex.set_option(B.VLA_OPT_WEIGHT_NT, 0)
        plain = case.run()
        ex.set_option(B.VLA_OPT_WEIGHT_NT, 1)
        assert ex.get_option(B.VLA_OPT_WEIGHT_NT) == 1
        nt = case.run()
        ex.set_option(B.VLA_OPT_WEIGHT_NT, 0)
        again = case.run()
        with pytest.raises(B.VlaError):
            ex.set_option(B.VLA_OPT_WEIGHT_NT, 2)
        assert ex.get_option(B.VLA_OPT_WEIGHT_NT) == 0
    finally:
        case.close()
    assert np.all(np.isfinite(plain))
    assert np.array_equal(plain, nt) and np.array_equal(plain, again)


def test_batch64_sampled_requests_warped():
    """Batch 64, per-request warped schedules; requests sampled for the oracle."""
    cfg = synth.config(5)
    pk, pv, x0, ts = _inputs(cfg, schedule="warped")
    say("[cfg5] batch 64, warped per-request schedules")
    case = GpuCase(cfg, weights(2), pk, pv, x0, ts)
    try:
        out = case.run()
    finally:
        case.close()
    W = decoded(2)
    for b in (0, 37, 63):
        ref = run_oracle(cfg.replace(batch=1), W, pk[b:b + 1], pv[b:b + 1], x0[b:b + 1], ts[b:b + 1])
        _gate_bf16(metrics(out[b:b + 1], ref), f"cfg5 request {b}")


@pytest.mark.parametrize("split", [0, 2])
def test_head_dim_64_many_rows_sampled_requests(split):
    """Head dim 64, 100 query rows per KV group, 64 requests (M = 3200): as one
    batch the attention takes the 8-wave row-tile kernel (896 workgroups); in
    two parts of 32 requests the few-row kernel. Warped per-request
    schedules; requests sampled for the oracle."""
    from vla_flow_matching_denoise_amd import binding as B
    cfg = synth.config(1).replace(horizon=50, batch=64, n_steps=3)
    pk, pv, x0, ts = _inputs(cfg, schedule="warped")
    say(f"[dh64 rows] batch 64, T = 50, parts {split}")
    case = GpuCase(cfg, weights(1), pk, pv, x0, ts)
    try:
        case.expert.set_option(B.VLA_OPT_SPLIT_BATCH, split)
        out = case.run()
    finally:
        case.close()
    W = decoded(1)
    for b in (0, 29, 63):
        ref = run_oracle(cfg.replace(batch=1), W, pk[b:b + 1], pv[b:b + 1], x0[b:b + 1], ts[b:b + 1])
        _gate_bf16(metrics(out[b:b + 1], ref), f"dh64 rows parts {split} request {b}")


def test_fp8_tier_end_to_end():
    cfg = synth.config(4)
    pk, pv, x0, ts = _inputs(cfg)
    say("[cfg4] E4M3 block linears, 25 steps")
    case = GpuCase(cfg, weights(4), pk, pv, x0, ts)
    try:
        out = case.run()
    finally:
        case.close()
    ref_bf16 = run_oracle(cfg, decoded(2), pk, pv, x0, ts)          # unquantized bf16 weights
    m = metrics(out, ref_bf16)
    say(f"[cfg4 vs bf16-weight oracle] {m}")
    assert m["cos"] >= FP8_COS, m
    ref_deq = run_oracle(cfg, oracle.decode_weights(weights(4)), pk, pv, x0, ts)   # dequantized weights
    _gate_bf16(metrics(out, ref_deq), "cfg4 vs dequantized-weight oracle")
