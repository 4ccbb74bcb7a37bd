"""Write the oracle regression fixture for the tiny workload (calls only oracle/ and synth/)."""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402


def compute():
    cfg = synth.config(1)
    W = oracle.decode_weights(synth.make_weights(cfg, seed=0))
    pk, pv = synth.make_prefix(cfg, seed=0)
    x0 = synth.make_noise(cfg, seed=0)
    ts = synth.make_schedule(cfg.n_steps, cfg.batch)
    return oracle.denoise(W, oracle.ExpertDims.from_config(cfg), oracle.decode_bf16(pk),
                          oracle.decode_bf16(pv), x0, ts)


if __name__ == "__main__":
    out = compute()
    path = os.path.join(HERE, "cfg_tiny_seed0.txt")
    with open(path, "w") as f:
        f.write("# fp64 oracle x_N for the tiny workload, seed 0; shape %s\n" % (out.shape,))
        for v in out.ravel():
            f.write("%.17g\n" % v)
    print("wrote", path)
