"""vla_denoise_static, the allocation-free variant of vla_denoise, through the
C ABI: its output equals vla_denoise's on the same inputs (the same kernels in
the same order, so bit for bit, which is within every floating-point gate),
on two calls in a row, the second with a smaller input (fewer steps, and
another context with a smaller batch); it allocates nothing (the context's
device bytes and the device's free memory do not move, even for a step count
past the context's current table capacity); and it rejects a call whose
scratch would not fit the static array before enqueueing anything."""
import numpy as np
import pytest

import synth
from tests.gpu_util import GpuCase, say, weights

pytestmark = pytest.mark.gpu


def _inputs(cfg, n_steps, schedule="uniform", seed=0):
    pk, pv = synth.make_prefix(cfg, seed=seed)
    x0 = synth.make_noise(cfg, seed=seed)
    return pk, pv, x0, synth.make_schedule(n_steps, cfg.batch, schedule)


def _static(case, ts, n, out):
    from vla_flow_matching_denoise_amd import binding as B
    B.vla_set_stream(case.expert.ctx, None)
    B.vla_denoise_static(case.expert.ctx, case.pk.data_ptr(), case.pv.data_ptr(), case.x0.data_ptr(),
                         ts.data_ptr(), n, out.data_ptr())


@pytest.mark.parametrize("cfg_id,batch_a,steps_a,batch_b,steps_b", [(1, 3, 10, 2, 4), (2, 1, 10, 1, 5)])
def test_static_entry_matches_denoise_twice_second_smaller(cfg_id, batch_a, steps_a, batch_b, steps_b):
    import torch
    from vla_flow_matching_denoise_amd.expert import to_device
    for batch, n, sched in ((batch_a, steps_a, "warped"), (batch_b, steps_b, "uniform")):
        cfg = synth.config(cfg_id).replace(batch=batch)
        say(f"[static] cfg{cfg_id} batch {batch}, {n} steps")
        case = GpuCase(cfg, weights(2 if cfg_id == 2 else cfg_id), *_inputs(cfg, n, sched))
        try:
            ref = case.run()
            out = torch.full_like(case.x0, float("nan"))
            torch.cuda.synchronize()
            _static(case, case.ts, n, out)
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            assert np.array_equal(got, ref), float(np.max(np.abs(got - ref)))
            # and again with fewer steps on the same context (a smaller input)
            m = max(1, n // 3)
            ts_m = to_device(synth.make_schedule(m, batch))
            ref_m = case.expert.denoise(case.pk, case.pv, case.x0, ts_m, m).cpu().numpy()
            out.fill_(float("nan"))
            _static(case, ts_m, m, out)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), ref_m)
        finally:
            case.close()


def test_static_entry_allocates_nothing_and_rejects_oversized_calls():
    """40 steps of the 36-layer hidden-1024 expert need a 36 MB modulation
    table, past the 10-step table the context holds: the static call takes it
    from the static array, so neither the context's device bytes nor the
    device's free memory move (4 MiB of slack for the runtime's own pools)."""
    import torch
    from vla_flow_matching_denoise_amd import binding as B
    from vla_flow_matching_denoise_amd.expert import to_device
    cfg = synth.config(2)
    case = GpuCase(cfg, weights(2), *_inputs(cfg, 10))
    try:
        out = torch.empty_like(case.x0)
        _static(case, case.ts, 10, out)
        torch.cuda.synchronize()
        ts40 = to_device(synth.make_schedule(40, 1))
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        ctx_bytes = case.expert.device_bytes()
        free0, _ = torch.cuda.mem_get_info()
        _static(case, ts40, 40, out)
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        say(f"[static] context bytes {ctx_bytes} -> {case.expert.device_bytes()}, device free "
            f"{free0 / 2**20:.1f} -> {free1 / 2**20:.1f} MiB")
        assert case.expert.device_bytes() == ctx_bytes
        assert abs(free1 - free0) <= (4 << 20), (free0, free1)
        got = out.cpu().numpy()
        ref = case.expert.denoise(case.pk, case.pv, case.x0, ts40, 40).cpu().numpy()
        assert np.array_equal(got, ref)
        # about 0.9 MB of table per step: 100 steps do not fit the 64 MiB array
        ts100 = to_device(synth.make_schedule(100, 1))
        rc = B.vla_denoise_static(case.expert.ctx, case.pk.data_ptr(), case.pv.data_ptr(), case.x0.data_ptr(),
                                  ts100.data_ptr(), 100, out.data_ptr(), check=False)
        assert rc == B.VLA_ERR_SHAPE and "scratch" in B.vla_last_error()
    finally:
        case.close()
