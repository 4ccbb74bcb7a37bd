"""Helpers shared by the GPU parity tests: seeded inputs, GPU run, oracle run."""
from __future__ import annotations

import functools
import sys

import numpy as np

import oracle
import synth

BF16_COS = 0.9995        # gate for bf16 weights/activations (fp32 accumulation)
BF16_MAXABS = 2e-2       # x RMS of the oracle output
FP8_COS = 0.995          # gate for the E4M3 weight tier vs the bf16-weight oracle


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=4)
def weights(cfg_id: int, seed: int = 0, weight_dtype=None):
    return synth.make_weights(synth.config(cfg_id), seed=seed, weight_dtype=weight_dtype)


@functools.lru_cache(maxsize=2)
def decoded(cfg_id: int, seed: int = 0, weight_dtype=None):
    return oracle.decode_weights(weights(cfg_id, seed, weight_dtype))


def metrics(gpu: np.ndarray, ref: np.ndarray) -> dict:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    cos = oracle.cosine(gpu, ref)
    per_req = [oracle.cosine(gpu[b], ref[b]) for b in range(gpu.shape[0])] if gpu.ndim == 3 else [cos]
    return {
        "cos": cos,
        "min_req_cos": min(per_req),
        "maxabs_over_rms": float(np.max(np.abs(gpu - ref)) / rms),
        "rel_l2": float(np.linalg.norm(gpu - ref) / np.linalg.norm(ref)),
    }


def run_oracle(cfg, W, pk, pv, x0, ts):
    d = oracle.ExpertDims.from_config(cfg)
    return oracle.denoise(W, d, oracle.decode_bf16(pk), oracle.decode_bf16(pv), x0, ts)


class GpuCase:
    """Uploads one workload's inputs and owns an Expert for it."""

    def __init__(self, cfg, raw, pk, pv, x0, ts):
        import torch
        from vla_flow_matching_denoise_amd.expert import Expert, dims_from_config, to_device
        self.cfg = cfg
        self.expert = Expert(raw, dims_from_config(cfg))
        self.pk = to_device(pk)
        self.pv = to_device(pv)
        self.x0 = to_device(x0)
        self.ts = to_device(ts)
        self.torch = torch

    def run(self, n_steps=None, out=None):
        n = self.ts.shape[1] - 1 if n_steps is None else n_steps
        o = self.expert.denoise(self.pk, self.pv, self.x0, self.ts, n, out=out)
        self.torch.cuda.synchronize()
        return o.cpu().numpy()

    def close(self):
        self.expert.close()
