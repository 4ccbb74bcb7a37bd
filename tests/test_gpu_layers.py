"""GPU parity that sees every part of the stack, and the ABI's behaviour on a
live context.

* Gate-open layer stages (gate biases + 1, so each block's own output is as
  large as the residual) at the first, middle and last layer and the first
  and last Euler step, for the LingBot batch-1 workload (weight-streaming
  GEMMs, the key-split attention) and the batch-64 workload (tiled GEMMs, the
  row-tile attention; sampled requests on per-request warped schedules), and
  at batch 32, the shapes of one half of the split batch-64 call.
  Gate: the layer's change to the residual, cosine >= 0.9995 and max-abs <=
  2e-2 x its RMS.
* The whole 36-layer gate-open loop (2 Euler steps).  Its tolerance is
  derived, not chosen: tests/rounding_model.py runs the oracle with bf16
  stored exactly where the kernels store bf16; the GPU must sit within twice
  that model's distance from the exact oracle (relative L2 and max-abs).
* A down projection split 16 ways along K (hidden 256, SwiGLU 4096): the
  residual + norm kernel must sum every partial.
* Switching streams between calls orders the new stream after the old one.
* Misaligned pointers and bad step counts on a live context are rejected;
  50 create / destroy cycles leave device memory where it was.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import rounding_model as rm
from tests.gpu_util import BF16_COS, BF16_MAXABS, GpuCase, decoded, metrics, run_oracle, say, weights

pytestmark = pytest.mark.gpu


def _inputs(cfg, schedule="uniform", n_steps=None, seed=0):
    pk, pv = synth.make_prefix(cfg, seed=seed)
    x0 = synth.make_noise(cfg, seed=seed)
    ts = synth.make_schedule(cfg.n_steps if n_steps is None else n_steps, x0.shape[0], schedule)
    return pk, pv, x0, ts


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg_id,batch,requests", [(2, None, (0,)), (5, None, (0, 37, 63)), (5, 32, (0, 31))])
def test_gate_open_layer_stages_first_middle_last(cfg_id, batch, requests):
    """Batch 32 (1600 rows) is one half of the split batch-64 call: its tile
    shapes (256x128 QKV, 128x64 O and down, the 8-wave row attention) differ
    from those of 3200 rows in one launch."""
    import torch
    from vla_flow_matching_denoise_amd import binding as B
    from vla_flow_matching_denoise_amd.expert import to_device
    cfg = synth.config(cfg_id) if batch is None else synth.config(cfg_id).replace(batch=batch)
    pk, pv, x0, ts = _inputs(cfg, schedule="warped" if cfg.batch > 1 else "uniform")
    raw = synth.apply_variant(weights(2), "gate_open", cfg)
    say(f"[layers cfg{cfg_id}] gate-open stages, batch {cfg.batch}")
    case = GpuCase(cfg, raw, pk, pv, x0, ts)
    rng = np.random.default_rng(21)
    h_in = rng.standard_normal((cfg.m_rows, cfg.hidden)).astype(np.float32)
    L, N = cfg.n_layers, cfg.n_steps
    points = [(l, k) for l in (0, L // 2, L - 1) for k in (0, N - 1)]
    got = {}
    try:
        hi = to_device(h_in)
        ho = torch.empty_like(hi)
        for layer, step in points:
            B.vla_test_layer(case.expert.ctx, case.pk.data_ptr(), case.pv.data_ptr(), case.ts.data_ptr(), N, step,
                             layer, hi.data_ptr(), ho.data_ptr())
            got[(layer, step)] = ho.cpu().numpy()
    finally:
        case.close()
    Wd = oracle.decode_weights(raw)
    d = oracle.ExpertDims.from_config(cfg)
    fpk, fpv = oracle.decode_bf16(pk), oracle.decode_bf16(pv)
    T = cfg.horizon
    for layer, step in points:
        for b in requests:
            c = oracle.time_condition(float(ts[b, step]), Wd, d)
            mod = oracle.modulation(c, Wd["mod_w"][layer], Wd["mod_b"][layer], 6)
            hb = h_in[b * T:(b + 1) * T].astype(np.float64)
            want = oracle.expert_layer(hb, Wd, layer, mod, fpk[b, layer], fpv[b, layer], d)
            m = metrics((got[(layer, step)][b * T:(b + 1) * T] - hb)[None], (want - hb)[None])
            say(f"[layers cfg{cfg_id}] layer {layer} step {step} request {b}: cos {m['cos']:.7f} "
                f"max-abs/RMS {m['maxabs_over_rms']:.2e}")
            assert m["cos"] >= BF16_COS and m["maxabs_over_rms"] <= BF16_MAXABS, (layer, step, b, m)


@pytest.mark.timeout(600)
def test_gate_open_36_layer_loop_within_the_rounding_model():
    cfg = synth.config(2).replace(n_steps=2)
    pk, pv, x0, ts = _inputs(cfg)
    raw = synth.apply_variant(weights(2), "gate_open", cfg)
    say("[gate-open 36L] LingBot shapes, 2 Euler steps")
    case = GpuCase(cfg, raw, pk, pv, x0, ts)
    try:
        out = case.run().astype(np.float64)
    finally:
        case.close()
    W = oracle.decode_weights(raw)
    d = oracle.ExpertDims.from_config(cfg)
    fpk, fpv = oracle.decode_bf16(pk), oracle.decode_bf16(pv)
    say("[gate-open 36L] oracle and rounding model")
    exact = oracle.denoise(W, d, fpk, fpv, x0, ts)
    model = rm.denoise_r(W, d, fpk, fpv, x0, ts)
    e_gpu, e_model = out - exact, model - exact
    l2 = lambda e: float(np.linalg.norm(e) / np.linalg.norm(exact))
    mx = lambda e: float(np.max(np.abs(e)) / np.sqrt(np.mean(exact ** 2)))
    say(f"[gate-open 36L] GPU vs exact: rel-L2 {l2(e_gpu):.3e} max-abs/RMS {mx(e_gpu):.3e} "
        f"cos {oracle.cosine(out, exact):.7f}; model vs exact: rel-L2 {l2(e_model):.3e} "
        f"max-abs/RMS {mx(e_model):.3e}; GPU vs model: rel-L2 {l2(out - model):.3e}")
    assert l2(e_gpu) <= 2.0 * l2(e_model), (l2(e_gpu), l2(e_model))
    assert mx(e_gpu) <= 2.0 * mx(e_model), (mx(e_gpu), mx(e_model))


def test_down_projection_split_sixteen_ways():
    """hidden 256 with SwiGLU 4096 at batch 1: the weight-streaming down GEMM
    splits K 16 ways, past the eight partials the norm keeps in registers."""
    cfg = synth.config(1).replace(intermediate=4096, n_steps=3)
    raw = synth.make_weights(cfg, seed=2)
    pk, pv, x0, ts = _inputs(cfg, schedule="warped")
    raw = synth.apply_variant(raw, "gate_open", cfg)
    case = GpuCase(cfg, raw, pk, pv, x0, ts)
    try:
        out = case.run()
    finally:
        case.close()
    m = metrics(out, run_oracle(cfg, oracle.decode_weights(raw), pk, pv, x0, ts))
    say(f"[split 16] {m}")
    assert m["cos"] >= BF16_COS and m["maxabs_over_rms"] <= BF16_MAXABS, m


def test_stream_switch_orders_the_new_stream_after_the_old():
    """A 36-layer call on stream A, then at once a call with other inputs on
    stream B: both outputs equal the same calls run one at a time, bitwise."""
    import torch
    from vla_flow_matching_denoise_amd.expert import to_device
    cfg = synth.config(2)
    case = GpuCase(cfg, weights(2), *_inputs(cfg, seed=0))
    a_in = (case.pk, case.pv, case.x0, case.ts)
    b_in = tuple(to_device(t) for t in _inputs(cfg, schedule="warped", seed=1))
    ex = case.expert
    try:
        ref_a = ex.denoise(*a_in, cfg.n_steps).clone()
        torch.cuda.synchronize()
        ref_b = ex.denoise(*b_in, cfg.n_steps).clone()
        torch.cuda.synchronize()
        sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
        for _ in range(3):
            with torch.cuda.stream(sa):
                out_a = ex.denoise(*a_in, cfg.n_steps)
            with torch.cuda.stream(sb):
                out_b = ex.denoise(*b_in, cfg.n_steps)
            torch.cuda.synchronize()
            assert torch.equal(out_a, ref_a) and torch.equal(out_b, ref_b)
        assert not torch.equal(ref_a, ref_b)
    finally:
        case.close()


def test_live_context_rejects_misaligned_pointers_and_bad_step_counts():
    import torch
    from vla_flow_matching_denoise_amd import binding as B
    cfg = synth.config(1)
    case = GpuCase(cfg, weights(1), *_inputs(cfg))
    ctx = case.expert.ctx
    out = torch.empty_like(case.x0)
    pk, pv, x0, ts = (t.data_ptr() for t in (case.pk, case.pv, case.x0, case.ts))
    try:
        bad = [
            ((pk + 2, pv, x0, ts, 10, out.data_ptr()), "prefix_k"),
            ((pk, pv + 8, x0, ts, 10, out.data_ptr()), "prefix_v"),
            ((pk, pv, x0 + 2, ts, 10, out.data_ptr()), "noise"),
            ((pk, pv, x0, ts + 1, 10, out.data_ptr()), "t_schedule"),
            ((pk, pv, x0, ts, 10, out.data_ptr() + 2), "out_actions"),
            ((pk, pv, x0, ts, 0, out.data_ptr()), "n_steps"),
            ((pk, pv, x0, ts, -3, out.data_ptr()), "n_steps"),
            ((pk, pv, x0, ts, 100001, out.data_ptr()), "n_steps"),
        ]
        for args, what in bad:
            assert B.vla_denoise(ctx, *args, check=False) == B.VLA_ERR_ARG, what
            assert what in B.vla_last_error(), (what, B.vla_last_error())
        # the context still works after the rejected calls
        got = case.run()
        m = metrics(got, run_oracle(cfg, decoded(1), *_inputs(cfg)))
        assert m["cos"] >= BF16_COS, m
    finally:
        case.close()


def test_create_destroy_cycles_release_device_memory():
    import torch
    from vla_flow_matching_denoise_amd.expert import Expert, dims_from_config
    cfg = synth.config(1)
    raw = weights(1)
    dims = dims_from_config(cfg)

    def cycle():
        ex = Expert(raw, dims)
        assert ex.device_bytes() > 0
        ex.close()

    cycle()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(50):
        cycle()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free1, _ = torch.cuda.mem_get_info()
    say(f"[create/destroy x50] free before {free0 / 2**20:.1f} MiB, after {free1 / 2**20:.1f} MiB")
    assert free1 >= free0 - (16 << 20), (free0, free1)


def test_batch_split_into_concurrent_halves():
    """VLA_OPT_SPLIT_BATCH = n runs the requests as n parts on n streams
    (child contexts borrowing the weights): 43 requests (parts of 21 + 22,
    14 + 14 + 15 and 10 + 11 + 11 + 11), warped per-request schedules and
    padded prefixes with per-request valid lengths. Each mode repeats
    bitwise over two calls; the modes differ only through the fp32 summation
    order of the modulation GEMM (its row count is steps x requests, so a
    small part can take the weight-streaming kernel where the whole batch
    takes the tiled one), far inside the bf16 gates, and sampled requests of
    the two-part run meet the oracle's gates."""
    import torch
    from vla_flow_matching_denoise_amd import binding as B
    from vla_flow_matching_denoise_amd.expert import to_device
    cfg = synth.config(5).replace(n_layers=4, batch=43, n_steps=3)
    raw = synth.make_weights(cfg, seed=6)
    case = GpuCase(cfg, raw, *_inputs(cfg, schedule="warped", seed=3))
    valid = to_device(np.random.default_rng(4).integers(0, cfg.prefix_len + 1, cfg.batch).astype(np.int32))
    try:
        ex = case.expert
        outs = {}
        for mode in (0, 2, 3, 4, 0, 2, 3, 4):
            ex.set_option(B.VLA_OPT_SPLIT_BATCH, mode)
            assert ex.get_option(B.VLA_OPT_SPLIT_BATCH) == mode
            a = ex.denoise(case.pk, case.pv, case.x0, case.ts, cfg.n_steps, prefix_valid=valid).clone()
            b = ex.denoise(case.pk, case.pv, case.x0, case.ts, cfg.n_steps).clone()
            torch.cuda.synchronize()
            if mode in outs:
                assert torch.equal(outs[mode][0], a) and torch.equal(outs[mode][1], b)
            outs[mode] = (a, b)
        for mode in (2, 3, 4):
            for i in (0, 1):
                m = metrics(outs[mode][i].cpu().numpy(), outs[0][i].cpu().numpy())
                say(f"[split] {mode} parts vs one batch, call {i}: {m}")
                assert m["cos"] >= 1 - 1e-8 and m["maxabs_over_rms"] <= 2e-3, m
        assert not torch.equal(outs[0][0], outs[0][1])     # the valid lengths did matter
    finally:
        case.close()
    W = oracle.decode_weights(raw)
    pk, pv, x0, ts = _inputs(cfg, schedule="warped", seed=3)
    for b in (0, 21, 42):
        ref = run_oracle(cfg.replace(batch=1), W, pk[b:b + 1], pv[b:b + 1], x0[b:b + 1], ts[b:b + 1])
        m = metrics(outs[2][1][b:b + 1].cpu().numpy(), ref)
        assert m["cos"] >= BF16_COS and m["maxabs_over_rms"] <= BF16_MAXABS, (b, m)
