"""GPU parity of vla_denoise_varlen (prefixes padded to a common length, a
valid length per request) against the CPU oracle's denoise_varlen.

Reading under test: request b uses its first prefix_valid[b] prefix tokens;
the rest is padding, and its chunk sits at positions prefix_valid[b] + i, so
its result is the plain loop on the truncated prefix. Gates as for the other
bf16 parity tests: cosine >= 0.9995, max|gpu - oracle| <= 2e-2 * RMS(oracle).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import BF16_COS, BF16_MAXABS, metrics, say

pytestmark = pytest.mark.gpu

SMALL = synth.ExpertConfig("persist_2L_h512", 6, 2, 512, 8, 1, 128, 1024, 32, 16, 7, 3, 2)


def _gate(out, ref, tag):
    m = metrics(out, ref)
    say(f"[{tag}] cos={m['cos']:.7f} min_req_cos={m['min_req_cos']:.7f} maxabs/rms={m['maxabs_over_rms']:.3e}")
    assert np.all(np.isfinite(out)), tag
    assert m["min_req_cos"] >= BF16_COS, m
    assert m["maxabs_over_rms"] <= BF16_MAXABS, m


class _Run:
    """One Expert with device inputs; calls with per-request valid lengths."""

    def __init__(self, cfg, raw, seed=0, schedule="uniform", persistent=0):
        import torch
        from vla_flow_matching_denoise_amd import binding as B
        from vla_flow_matching_denoise_amd.expert import Expert, dims_from_config, to_device
        self.torch, self.to_device = torch, to_device
        self.cfg = cfg
        self.pk, self.pv = synth.make_prefix(cfg, seed=seed)
        self.x0 = synth.make_noise(cfg, seed=seed)
        self.ts = synth.make_schedule(cfg.n_steps, cfg.batch, schedule)
        self.ex = Expert(raw, dims_from_config(cfg))
        self.ex.set_option(B.VLA_OPT_PERSISTENT, persistent)
        self.dev = [to_device(a) for a in (self.pk, self.pv, self.x0, self.ts)]
        self.W = oracle.decode_weights(raw)

    def gpu(self, valid, pk=None, pv=None):
        t = self.torch
        dpk = self.dev[0] if pk is None else self.to_device(pk)
        dpv = self.dev[1] if pv is None else self.to_device(pv)
        pvalid = None if valid is None else t.tensor(valid, dtype=t.int32, device="cuda")
        out = self.ex.denoise(dpk, dpv, self.dev[2], self.dev[3], self.cfg.n_steps, prefix_valid=pvalid)
        t.cuda.synchronize()
        return out.cpu().numpy()

    def ref(self, valid):
        d = oracle.ExpertDims.from_config(self.cfg)
        return oracle.denoise_varlen(self.W, d, oracle.decode_bf16(self.pk), oracle.decode_bf16(self.pv),
                                     self.x0, self.ts, valid)

    def close(self):
        self.ex.close()


def test_varlen_tiny_graph_reuse_and_padding_invariance():
    cfg = synth.config(1).replace(batch=3, n_steps=4)
    run = _Run(cfg, synth.make_weights(cfg, seed=0), schedule="warped")
    try:
        for valid in ([32, 11, 0], [5, 32, 20]):      # the second call replays the same graph
            say(f"[varlen tiny] valid={valid}")
            _gate(run.gpu(valid), run.ref(valid), f"tiny {valid}")
        # every request at full length: identical to vla_denoise
        assert np.array_equal(run.gpu([32, 32, 32]), run.gpu(None))
        assert np.array_equal(run.gpu([99, 32, 1000]), run.gpu(None))   # clamped to P
        # the padded tokens never matter
        valid = [7, 32, 3]
        a = run.gpu(valid)
        pk, pv = run.pk.copy(), run.pv.copy()
        pk[0, :, 7:] = synth.to_bf16_bits(np.full(pk[0, :, 7:].shape, 50.0, np.float32))
        pv[2, :, 3:] = synth.to_bf16_bits(np.full(pv[2, :, 3:].shape, -50.0, np.float32))
        assert np.array_equal(run.gpu(valid, pk, pv), a)
    finally:
        run.close()


def test_varlen_many_rows_takes_row_split_attention():
    """130 requests of the tiny expert: 16-row tiles exceed 512 workgroups, so
    attention runs 64 query rows per workgroup, and the GEMMs are tiled."""
    cfg = synth.config(1).replace(batch=130, n_steps=2)
    run = _Run(cfg, synth.make_weights(cfg, seed=3), seed=4, schedule="warped")
    try:
        valid = list(np.random.default_rng(9).integers(0, cfg.prefix_len + 1, size=cfg.batch))
        say("[varlen b130] random lengths")
        _gate(run.gpu(valid), run.ref(valid), "tiny b130")
    finally:
        run.close()


def test_varlen_persistent_path():
    run = _Run(SMALL, synth.make_weights(SMALL, seed=0), seed=1, persistent=1)
    try:
        assert run.ex.persistent_active
        for valid in ([32, 9], [0, 32]):
            say(f"[varlen persistent] valid={valid}")
            _gate(run.gpu(valid), run.ref(valid), f"persistent {valid}")
    finally:
        run.close()


def test_varlen_lingbot_two_requests():
    cfg = synth.config(2).replace(batch=2, n_steps=2)
    from tests.gpu_util import weights
    run = _Run(cfg, weights(2), seed=2)
    try:
        valid = [256, 137]
        say(f"[varlen cfg2] valid={valid}")
        _gate(run.gpu(valid), run.ref(valid), "cfg2 b2")
    finally:
        run.close()
