"""GPU parity of the persistent single-launch path (small batches) against the
CPU oracle, against the kernel-per-stage path, and across repeated calls.

The persistent kernel runs the whole loop in one resident launch with the
layer split over the eight XCDs; it runs for the shapes it supports when
switched on (VLA_OPT_PERSISTENT). Gates are those of the other bf16 parity
tests: cosine >= 0.9995 and max|gpu - oracle| <= 2e-2 * RMS(oracle).
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import BF16_COS, BF16_MAXABS, GpuCase, decoded, metrics, run_oracle, say, weights

pytestmark = pytest.mark.gpu

# two-layer expert with head_dim 128 and 8 query heads (one per XCD) sharing
# one KV head: the smallest shape class of the persistent kernel
SMALL = synth.ExpertConfig("persist_2L_h512", 6, 2, 512, 8, 1, 128, 1024, 32, 16, 7, 4, 1)


def _inputs(cfg, seed=0, schedule="uniform", n_steps=None):
    pk, pv = synth.make_prefix(cfg, seed=seed)
    x0 = synth.make_noise(cfg, seed=seed)
    ts = synth.make_schedule(cfg.n_steps if n_steps is None else n_steps, cfg.batch, schedule)
    return pk, pv, x0, ts


def _gate(out, ref, tag):
    m = metrics(out, ref)
    say(f"[{tag}] cos={m['cos']:.7f} min_req_cos={m['min_req_cos']:.7f} "
        f"maxabs/rms={m['maxabs_over_rms']:.3e} rel_l2={m['rel_l2']:.3e}")
    assert np.all(np.isfinite(out)), tag
    assert m["cos"] >= BF16_COS, m
    assert m["maxabs_over_rms"] <= BF16_MAXABS, m


def _case(cfg, raw, *ins):
    """A GpuCase with the persistent path switched on."""
    from vla_flow_matching_denoise_amd import binding as B
    case = GpuCase(cfg, raw, *ins)
    case.expert.set_option(B.VLA_OPT_PERSISTENT, 1)
    return case


def _status_ok(case):
    from vla_flow_matching_denoise_amd import binding as B
    st = case.expert.get_option(B.VLA_OPT_PERSISTENT_STATUS)
    assert st == 0, f"persistent kernel reported status {st}"


def _small_raw():
    return synth.make_weights(SMALL, seed=0)


def test_persistent_small_end_to_end_and_vs_stage_path():
    from vla_flow_matching_denoise_amd import binding as B
    cfg = SMALL
    raw = _small_raw()
    pk, pv, x0, ts = _inputs(cfg)
    ref = run_oracle(cfg, __import__("oracle").decode_weights(raw), pk, pv, x0, ts)
    say("[persist small] 2 layers, h512, 8x1x128 heads, chunk 16x7, 4 steps")
    case = _case(cfg, raw, pk, pv, x0, ts)
    try:
        assert case.expert.persistent_active
        out_p = case.run()
        _status_ok(case)
        _gate(out_p, ref, "persist small")
        case.expert.set_option(B.VLA_OPT_PERSISTENT, 0)
        assert not case.expert.persistent_active
        out_s = case.run()
        _gate(out_s, ref, "stage path small")
        case.expert.set_option(B.VLA_OPT_PERSISTENT, 1)
        assert case.expert.persistent_active
    finally:
        case.close()


def test_persistent_repeat_bitwise_and_input_switch():
    """Calls are deterministic and a call never sees data left by an earlier one."""
    import oracle
    from vla_flow_matching_denoise_amd.expert import to_device
    cfg = SMALL
    raw = _small_raw()
    W = oracle.decode_weights(raw)
    ins_a = _inputs(cfg, seed=0)
    ins_b = _inputs(cfg, seed=5, schedule="warped")
    say("[persist small] A, B, A calls with different prefix / noise / schedule")
    case = _case(cfg, raw, *ins_a)
    try:
        a1 = case.run()
        dev_b = [to_device(t) for t in ins_b]
        ob = case.expert.denoise(*dev_b, cfg.n_steps)
        case.torch.cuda.synchronize()
        b1 = ob.cpu().numpy()
        a2 = case.run()
    finally:
        case.close()
    assert np.array_equal(a1, a2), "persistent path is not bitwise repeatable"
    _gate(b1, run_oracle(cfg, W, *ins_b), "persist small, second input")
    assert not np.allclose(a1, b1)


def test_persistent_step_counts():
    """Growing and shrinking n_steps between calls (slot buffers are re-sized)."""
    import oracle
    cfg = SMALL
    raw = _small_raw()
    W = oracle.decode_weights(raw)
    case = None
    try:
        for n in (2, 5, 1, 3):
            pk, pv, x0, ts = _inputs(cfg, n_steps=n)
            say(f"[persist small] n_steps={n}")
            if case is None:
                case = _case(cfg, raw, pk, pv, x0, ts)
            else:
                from vla_flow_matching_denoise_amd.expert import to_device
                case.ts = to_device(ts)
            _gate(case.run(n), run_oracle(cfg, W, pk, pv, x0, ts), f"persist small n={n}")
    finally:
        if case is not None:
            case.close()


@pytest.mark.parametrize("batch,horizon,action_dim,prefix_len", [(2, 13, 5, 64), (4, 16, 3, 0), (3, 21, 9, 32)])
def test_persistent_ragged_batches(batch, horizon, action_dim, prefix_len):
    """Several requests, chunk lengths off the 16/32 tiles, and an empty prefix."""
    import oracle
    cfg = SMALL.replace(batch=batch, horizon=horizon, action_dim=action_dim, prefix_len=prefix_len, n_steps=3)
    raw = synth.make_weights(cfg, seed=1)
    pk, pv, x0, ts = _inputs(cfg, seed=2, schedule="warped")
    say(f"[persist ragged] batch={batch} horizon={horizon} action_dim={action_dim} prefix={prefix_len}")
    case = _case(cfg, raw, pk, pv, x0, ts)
    try:
        assert case.expert.persistent_active
        out = case.run()
        _status_ok(case)
    finally:
        case.close()
    _gate(out, run_oracle(cfg, oracle.decode_weights(raw), pk, pv, x0, ts), "persist ragged")


def test_persistent_lingbot_b1_vs_stage_path():
    """The full 36-layer LingBot-shaped workload on both paths, 3 steps."""
    from vla_flow_matching_denoise_amd import binding as B
    cfg = synth.config(2).replace(n_steps=3)
    pk, pv, x0, ts = _inputs(cfg)
    say("[persist cfg2] 36 layers, h1024, chunk 50x75, 3 steps")
    case = _case(cfg, weights(2), pk, pv, x0, ts)
    try:
        assert case.expert.persistent_active
        out_p = case.run()
        _status_ok(case)
        case.expert.set_option(B.VLA_OPT_PERSISTENT, 0)
        out_s = case.run()
    finally:
        case.close()
    ref = run_oracle(cfg, decoded(2), pk, pv, x0, ts)
    _gate(out_p, ref, "persist cfg2")
    _gate(out_s, ref, "stage path cfg2")


@pytest.mark.parametrize("persistent", [0, 1])
def test_default_stream_ordering(persistent):
    """With no stream set, a call is ordered with torch's default stream: an
    input written by a torch kernel just before the call is seen, and the
    output is complete for a plain .cpu() read, with no device-wide sync."""
    import torch
    from vla_flow_matching_denoise_amd import binding as B
    from vla_flow_matching_denoise_amd.expert import to_device
    cfg = SMALL
    raw = _small_raw()
    pk, pv, x0, ts = _inputs(cfg)
    case = GpuCase(cfg, raw, pk, pv, x0, ts)
    try:
        case.expert.set_option(B.VLA_OPT_PERSISTENT, persistent)
        ref = case.run()                                   # fully synchronised
        for _ in range(3):
            big = torch.randn(1 << 22, device="cuda")      # keep the default stream busy
            for _ in range(4):
                big = big * 1.0001
            noise = (to_device(x0) + big[0] * 0.0) * 1.0   # written by a kernel on the default stream
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            out = case.expert.denoise(case.pk, case.pv, noise, case.ts, cfg.n_steps)
            ev1.record()
            got = out.cpu().numpy()                       # ordered after the call, no global sync
            assert np.array_equal(got, ref)
            ev1.synchronize()
            assert ev0.elapsed_time(ev1) > 0.02            # the events bracket the call's GPU work
    finally:
        case.close()
